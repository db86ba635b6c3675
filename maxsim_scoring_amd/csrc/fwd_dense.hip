// Cross-product MaxSim forward for gfx950: fp16/bf16 (32x32x16 MFMA) and
// int8 (32x32x32 MFMA), with d_mask/q_mask, optional argmax and long queries.
//
// "Flash-MaxSim" Sec. 4.1 (fused forward, online max), Sec. 4.1.1 (-inf
// masking, no rescale), Sec. 4.3.1 (INT8 x INT8 with fused dequantisation);
// late-interaction-kernels design notes "Forward" (strict '>' argmax update,
// finalise with finite(m) & q_active) and "Long-query chunking" (a query is
// split into fixed chunks whose partial scores are summed in a fixed order).
//
// Design. A workgroup of 8 waves is persistent over one block of query
// N-tiles (32 query tokens each) and one contiguous range of docs. The query
// block stays in VGPRs for the whole run (loaded once), and the docs of the
// range stream through LDS as one flat sequence of 128-token tiles, crossing
// doc boundaries without draining the pipeline: direct-to-LDS loads fill a
// 3-stage ring two tiles ahead, and one barrier per tile hands a landed tile
// to all 8 waves, so each doc tile is read once per workgroup. Workgroups
// that share a doc range are placed on the same XCD, so the range is fetched
// from HBM once per XCD and served from that XCD's L2 to the others.
//
// The S tile is computed transposed, S^T = D . Q^T: MFMA rows are doc tokens
// and columns are query tokens, so every lane owns one query token and the
// max over doc tokens stays inside the lane; the two lane halves are merged
// once per doc. The d_mask of a range becomes 128 validity bits per tile,
// built into LDS once (scalar loads per tile when it does not fit): tiles
// whose rows are all valid take a path with no mask work, M-tiles with no
// valid row skip their MFMAs. Per-doc partial sums of the N-tiles of a query
// meet in LDS and are added in slot order, so the result does not depend on
// timing.
//
// Argmax: a lane keeps its running max and the base row of the values it
// last saved; when an M-tile raises the max, the quarter of the lane's 16
// values of that M-tile (4 rows) that holds the first occurrence of the new
// max is stored to a per-lane LDS slot (an exec-masked store, so lanes whose max did not
// change issue nothing). At the end of the doc the lowest saved row holding
// the max is the argmax. Keeping the saved values in LDS rather than
// selecting them into registers takes the 16 selects per value tile off the
// VALU, which shares its issue port with the MFMAs.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace maxsim {

namespace {

constexpr int kWaves = 8;

// 4-bit nonzero flags of the 4 bytes of x (byte b -> bit b)
__device__ __forceinline__ uint32_t byte_flags(uint32_t x)
{
    x |= x >> 4;
    x |= x >> 2;
    x |= x >> 1;
    x &= 0x01010101u;
    return ((x * 0x01020408u) >> 24) & 0xFu;
}

// Validity bits of the 64 doc tokens starting at byte `p` of d_mask (bit r =
// token r is valid), for `nb` (1..64) tokens that exist. Uses scalar loads of
// the aligned dwords that hold those bytes only, so nothing past the last
// valid byte's dword is read.
__device__ __forceinline__ uint64_t mask_bits_scalar(const uint8_t* p, int nb)
{
    const uintptr_t a = (uintptr_t)p;
    const int sh = (int)(a & 3u);
    const __attribute__((address_space(4))) uint32_t* w =
        (const __attribute__((address_space(4))) uint32_t*)(a - (uintptr_t)sh);
    const int ndw = (sh + nb + 3) >> 2;  // dwords that hold a valid byte
    uint64_t lo = 0, hi = 0;             // bits of bytes [a - sh, a - sh + 68)
    if (nb == 64) {
        // all 16 (+1 when unaligned) dwords hold a valid byte: one batch of loads
        typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
        const u32x16 x = *(const __attribute__((address_space(4))) u32x16*)w;
#pragma unroll
        for (int k = 0; k < 16; ++k) lo |= (uint64_t)byte_flags(x[k]) << (4 * k);
        if (sh) hi = byte_flags(w[16]);
    } else {
        for (int k = 0; k < ndw; ++k) {
            const uint64_t f = byte_flags(w[k]);
            if (k < 16) lo |= f << (4 * k);
            else hi |= f;
        }
    }
    uint64_t bits = sh ? ((lo >> sh) | (hi << (64 - sh))) : lo;
    if (nb < 64) bits &= (1ull << nb) - 1ull;
    return bits;
}

// N (2 or 4) 64-bit words at a uniform LDS address, read by every lane
// (broadcast) and returned as scalars.
template <int N>
__device__ __forceinline__ void lds_read_u64_uniform(uint32_t addr, uint64_t (&out)[N])
{
    static_assert(N == 2 || N == 4 || N == 8, "one, two or four 16-byte reads");
#pragma unroll
    for (int r = 0; r < N / 2; ++r) {
        i32x4 v;
        asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(addr + 16 * r) : "memory");
        const uint32_t w0 = __builtin_amdgcn_readfirstlane(v[0]);
        const uint32_t w1 = __builtin_amdgcn_readfirstlane(v[1]);
        const uint32_t w2 = __builtin_amdgcn_readfirstlane(v[2]);
        const uint32_t w3 = __builtin_amdgcn_readfirstlane(v[3]);
        out[2 * r] = ((uint64_t)w1 << 32) | w0;
        out[2 * r + 1] = ((uint64_t)w3 << 32) | w2;
    }
}

// LDS accesses made from inline assembly so that the compiler does not add
// waits for the whole direct-to-LDS ring before them (see lds_read4).
__device__ __forceinline__ void lds_store_b32(uint32_t addr, uint32_t v)
{
    asm volatile("ds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ uint32_t lds_load_b32(uint32_t addr)
{
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(addr) : "memory");
    return v;
}

// Max of scores that are finite or -inf. The kernels are built with IEEE mode
// off and NaNs not honoured, so this is one v_max_f32 (three operands fold to
// v_max3_f32) with no canonicalisation of the operands; being plain code, the
// compiler also keeps the wait states between an MFMA and the first read of
// its result, which it does not do for inline assembly.
template <typename V> __device__ __forceinline__ V vmax(V a, V b) { return a > b ? a : b; }
template <> __device__ __forceinline__ float vmax<float>(float a, float b) { return __builtin_fmaxf(a, b); }
template <typename V> __device__ __forceinline__ V vmax3(V a, V b, V c) { return vmax(vmax(a, b), c); }

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// Scheduling groups for the region that holds the MFMA chain of one unit and
// the max fold of the previous one: one MFMA, then up to two VALU
// instructions of the fold, then one LDS read (the next M-tile's fragment),
// repeated, so that the fold issues in the shadow of the chain instead of
// after it.
__device__ __forceinline__ void interleave_fold_with_chain()
{
    static_for<0, 8>([&](auto) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    });
}

// Running state of one N-tile for the lane's 16 rows of each M-tile: the
// running max and, with argmax, the base row of the values saved when an
// M-tile last raised it (a strict '>' across M-tiles in ascending t keeps the
// earlier one on ties). Those values sit in the lane's LDS slot.
template <typename V, bool ARGMAX> struct RowState;
template <typename V> struct RowState<V, false> {
    V m;
    __device__ __forceinline__ void reset() { m = neg_inf<V>(); }
};
template <typename V> struct RowState<V, true> {
    V m;
    int tbase;
    __device__ __forceinline__ void reset()
    {
        m = neg_inf<V>();
        tbase = 0;
    }
};

template <typename V, typename Acc, bool MASKED>
__device__ __forceinline__ void masked_values(const Acc& acc, uint32_t lbits, V (&v)[16])
{
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int r = 8 * (q >> 2) + (q & 3);  // lane row offset without the 4h term
        v[q] = acc[q];
        if constexpr (MASKED) v[q] = ((lbits >> r) & 1u) ? v[q] : neg_inf<V>();
    }
}

template <typename V>
__device__ __forceinline__ V max16(const V (&v)[16])
{
    const V a = vmax3(v[0], v[1], v[2]);
    const V b = vmax3(v[3], v[4], v[5]);
    const V c = vmax3(v[6], v[7], v[8]);
    const V d = vmax3(v[9], v[10], v[11]);
    const V e = vmax3(v[12], v[13], v[14]);
    return vmax(vmax3(a, b, c), vmax3(d, e, v[15]));
}

// 16-byte chunks of a raised M-tile that a lane saves: the quarter of its
// 16 values (in the lane's row order) that holds the first occurrence of the
// tile max. Against saving all 16 values this costs three compares and 12
// selects per raise and cuts the LDS stores and the slot memory to a quarter,
// which ran the 128 x 128 bf16 ColPali pairs about 4 % faster (half the values:
// about 2 %).
constexpr int kSaveChunks = 1;
static_assert(kSaveChunks == 1 || kSaveChunks == 2 || kSaveChunks == 4, "saved chunks per raise");

// max of v[B .. B+N-1], N in {4, 8, 16}
template <int B, int N, typename V>
__device__ __forceinline__ V max_run(const V (&v)[16])
{
    if constexpr (N == 4) return vmax(vmax3(v[B], v[B + 1], v[B + 2]), v[B + 3]);
    else if constexpr (N == 8) return vmax3(vmax3(v[B], v[B + 1], v[B + 2]), vmax3(v[B + 3], v[B + 4], v[B + 5]), vmax(v[B + 6], v[B + 7]));
    else return max16(v);
}

// Fold one 32x32 accumulator tile (M-tile rows starting at `base`) into the
// state of its N-tile. `lbits` bit r = lane row r (+4h) valid. `save` is the
// lane's LDS slot (kSaveChunks chunks of 16 bytes, 64 lanes apart). On a
// raise the lane keeps only the group of values that holds the first
// occurrence of the new max, and folds the group's row offset into tbase.
// CHAINED: the fold follows an MFMA chain issued at raised priority in the
// same region; its max and compare are interleaved with that chain, and the
// priority drops once they are issued.
template <typename V, bool ARGMAX, bool MASKED, typename Acc, bool CHAINED = false>
__device__ __forceinline__ void fold_one(const Acc& acc, RowState<V, ARGMAX>& st, int base,
                                         uint32_t lbits, u32x4* save)
{
    V v[16];
    masked_values<V, Acc, MASKED>(acc, lbits, v);
    if constexpr (ARGMAX) {
        constexpr int SV = 4 * kSaveChunks;  // values per group
        constexpr int NG = 16 / SV;          // groups
        V g[NG];
        static_for<0, NG>([&](auto k) { g[k] = max_run<decltype(k)::value * SV, SV>(v); });
        V tm = g[0];
#pragma unroll
        for (int k = 1; k < NG; ++k) tm = vmax(tm, g[k]);
        const bool upd = tm > st.m;
        st.m = upd ? tm : st.m;
        if constexpr (CHAINED) {
            interleave_fold_with_chain();
            __builtin_amdgcn_s_setprio(0);
        }
        if (upd) {
            // first group whose max is the tile max; its first chunk is
            // chunk k * kSaveChunks, i.e. rows 8 * k * kSaveChunks (+4h) on
            int sel = NG - 1;
#pragma unroll
            for (int k = NG - 2; k >= 0; --k) sel = g[k] == tm ? k : sel;
            st.tbase = base + 8 * kSaveChunks * sel;
#pragma unroll
            for (int c = 0; c < kSaveChunks; ++c) {
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    V x = v[(NG - 1) * SV + 4 * c + e];
#pragma unroll
                    for (int k = NG - 2; k >= 0; --k) x = g[k] == tm ? v[k * SV + 4 * c + e] : x;
                    w[e] = __builtin_bit_cast(uint32_t, x);
                }
                save[64 * c] = u32x4{w[0], w[1], w[2], w[3]};
            }
        }
    } else {
        (void)save;
        st.m = vmax(st.m, max16(v));
        if constexpr (CHAINED) {
            interleave_fold_with_chain();
            __builtin_amdgcn_s_setprio(0);
        }
    }
}

// Lane-local argmax of the doc: lowest row of the saved group equal to the
// max (row offset without the 4h term); only meaningful when the max is
// finite, i.e. when the slot was written for this doc.
template <typename V>
__device__ __forceinline__ int saved_argmax(const RowState<V, true>& st, const u32x4* save)
{
    // the chunk is copied to a plain array before the compares: indexing the
    // vector value directly inside the unrolled loop was compiled (ROCm 7.2)
    // into a compare of element 0 only
    int qs = 4 * kSaveChunks - 1;
#pragma unroll
    for (int c = kSaveChunks - 1; c >= 0; --c) {
        const u32x4 w = save[64 * c];
        const uint32_t wv[4] = {w[0], w[1], w[2], w[3]};
#pragma unroll
        for (int e = 3; e >= 0; --e) qs = __builtin_bit_cast(V, wv[e]) == st.m ? 4 * c + e : qs;
    }
    return st.tbase + 8 * (qs >> 2) + (qs & 3);
}

}  // namespace

// TOK (int8 only): one scale per token. The doc-token scale multiplies each
// integer dot product before the max (a float per score); the query-token
// scale (positive) is applied to the max. The tile's doc scales are staged in
// LDS with the tile.
template <int E, bool ARGMAX, int NTW, bool TOK, int STAGES, int TR, int W = kWaves>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(2))) void fwd_dense_kernel(DenseArgs a)
{
    static_assert(!TOK || E == kI8, "per-token scales are an int8 mode");
    using T = Traits<E>;
    using V = std::conditional_t<TOK, float, typename T::Scalar>;  // value of the max
    using Acc = typename T::Acc;
    typedef float F16v __attribute__((ext_vector_type(16)));
    constexpr int RB = T::kRowBytes;
    constexpr int NCH = RB / 16;           // 16-byte chunks per row
    constexpr int KS = T::kKSteps;
    constexpr int SLOTS = W * NTW;         // N-tiles per workgroup
    static_assert(TR == 128 || TR == 256 || TR == 512, "doc tokens per pipeline stage");
    constexpr int MT = TR / 32;            // MFMA M-tiles per stage
    constexpr int WPT = TR / 64;           // d_mask words per stage
    constexpr int STAGE_BYTES = TR * RB;
    constexpr int CHUNKS = TR * NCH;
    constexpr int THREADS = W * 64;
    constexpr int kMaskWords = W == 8 ? 2048 : 1024;  // d_mask words of a doc range in LDS
    constexpr int LPS = CHUNKS / THREADS;  // direct-to-LDS loads per thread per stage
    constexpr int LPW = LPS + (TOK ? 1 : 0);  // direct-to-LDS loads per wave per stage
    static_assert(CHUNKS % THREADS == 0, "stage must split evenly over the workgroup");
    static_assert(STAGES >= 2 && STAGES <= 4, "ring depth");

    __shared__ __attribute__((aligned(16))) unsigned char stage_buf[STAGES * STAGE_BYTES];
    __shared__ V part[2][SLOTS];
    // d_mask of the whole doc range as bits, when it fits: 2 words per tile
    __shared__ __attribute__((aligned(16))) uint16_t mask_lds[4 * kMaskWords];
    // tiles streamed per doc of the range when its mask is in LDS: up to the
    // last tile holding a valid token (at least one, so every doc is finished)
    __shared__ uint16_t doc_tiles[kMaskWords / 2];
    // doc-token scales of each stage's tile (TOK)
    __shared__ __attribute__((aligned(16))) float sc_buf[TOK ? STAGES * TR : 4];
    // argmax: each lane's saved values, per (wave, N-tile): kSaveChunks chunks x 64 lanes
    __shared__ __attribute__((aligned(16))) u32x4 save_buf[ARGMAX ? W * NTW * 64 * kSaveChunks : 1];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int h = lane >> 5;    // which K-half this lane feeds; which row-quad it owns
    const int col = lane & 31;  // MFMA column = query token within the N-tile

    // ---- work unit: XCD-aware order (workgroup b runs on XCD b % 8) --------
    const int nblk = gridDim.x;
    const int b = blockIdx.x;
    const int xcd = b & 7, kth = b >> 3;
    const int full = nblk >> 3, rem = nblk & 7;
    const int unit = xcd * full + (xcd < rem ? xcd : rem) + kth;
    const int64_t Nd = a.Nd, Lq = a.Lq, Ld = a.Ld;
    // work unit = (query block, doc range), or with a pair list, pair `unit`:
    // query pair_q[unit] (one query per block) against the one doc pair_d[unit]
    const bool pairs = a.pair_q != nullptr;
    int qb;
    int64_t d0, d1;
    if (pairs) {
        const int32_t pq = a.pair_q[unit], pd = a.pair_d[unit];
        qb = pq < 0 ? 0 : (pq >= a.Nq ? (int)a.Nq - 1 : pq);  // precondition guard
        d0 = pd < 0 ? 0 : (pd >= Nd ? Nd - 1 : pd);
        d1 = d0 + 1;
    } else {
        qb = unit % a.nqb;
        const int64_t r = unit / a.nqb;
        d0 = r * Nd / a.nranges;
        d1 = (r + 1) * Nd / a.nranges;
    }
    // the range is uniform; the 64-bit division above runs on the vector unit,
    // so move the results back to scalar registers, which keeps everything
    // derived from them (cursors, tile pointers, mask words) scalar
    d0 = uniform_i64(d0);
    d1 = uniform_i64(d1);
    if (d0 >= d1) return;  // uniform over the workgroup
    // where the results of (query i, doc j) go
    auto out_pair = [&](int64_t i, int64_t j) -> int64_t { return pairs ? (int64_t)unit : i * Nd + j; };

    const int ntd = Ld > 0 ? (int)((Ld + TR - 1) / TR) : 0;  // tiles per doc
    const int64_t F = (d1 - d0) * ntd;                                     // tiles of the range
    const uint32_t part_base = lds_addr(&part[0][0]);

    // A-fragment offsets of M-tile 0 (row = lane % 32, logical chunk 2s + h);
    // M-tile mt adds mt * 32 rows (the swizzle only depends on row % 16)
    uint32_t frag_off[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) frag_off[s] = (uint32_t)(col * RB + swz_chunk<RB>(col, 2 * s + h) * 16);
    const uint32_t ring_base = lds_addr(stage_buf);
    const uint32_t sc_base = lds_addr(sc_buf);

    const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // wave index as a scalar
    // per-lane byte offset of direct-to-LDS load u: LDS slot p = (row p / NCH,
    // chunk p % NCH) of a stage holds logical chunk swz(row, p % NCH) of that
    // row. Load u covers rows 64 u / NCH further on, and with the lane's row
    // bits below those (row % 16 < 4 for 256-byte rows, and row % 8 for
    // 128-byte rows, whose swizzle also takes bit 3 of the row) the swizzle
    // of load u is that of load 0 with fixed chunk bits flipped: offset u =
    // (offset 0 ^ dma_flip(u)) + 1024 u.
    static_assert(64 * LPS * W == CHUNKS && (RB == 256 || (RB == 128 && LPS % 2 == 0)), "load layout");
    auto dma_flip = [](int u) -> uint32_t { return RB == 256 ? 64u * (uint32_t)(u & 3) : 16u * (uint32_t)(u & 1); };
    const uint32_t dma_off0 = [&] {
        const uint32_t p = (uint32_t)(wave * LPS) * 64 + (uint32_t)lane;
        return (p / NCH) * RB + (uint32_t)swz_chunk<RB>((int)(p / NCH), (int)(p % NCH)) * 16;
    }();

    // stage tile tt of doc `doc` into `stage`: uniform base pointer + 32-bit
    // per-lane offsets (scalar-base addressing), no 64-bit per-lane math
    auto issue = [&](int64_t doc, int tt, int stage) {
        const int64_t t0 = (int64_t)tt * TR;
        const void* Dt = uniform_ptr((const unsigned char*)a.D + (doc * Ld + t0) * RB);
        const int rows = Ld - t0 >= TR ? TR : (int)(Ld - t0);  // >= 1
        const uint32_t lds0 = ring_base + (uint32_t)(stage * STAGE_BYTES + wave_u * LPS * 1024);
        // rows past the doc end read its last row's final chunk instead; they
        // are never folded (their validity bits are 0)
        const uint32_t lim = (uint32_t)(rows * RB - 16);
        // offsets 1 .. LPS - 1 are derived at each issue from a copy of
        // offset 0 that the compiler cannot hoist (it depends on the stage),
        // so that they do not hold LPS registers across the tile loop
        uint32_t o0 = dma_off0;
        asm("" : "+v"(o0) : "s"(stage));
#pragma unroll
        for (int u = 0; u < LPS; ++u) {
            const uint32_t o = (o0 ^ dma_flip(u)) + 1024u * (uint32_t)u;
            dma_lds16(Dt, o < lim ? o : lim, lds0 + u * 1024);
        }
        if constexpr (TOK) {  // rows RPW w .. RPW w + RPW - 1 of the tile's doc scales
            constexpr int RPW = TR / W;
            const void* St = uniform_ptr(a.d_scale_tok + doc * Ld + t0);
            const int row = RPW * wave + lane < rows ? RPW * wave + lane : rows - 1;
            if (lane < RPW)
                dma_lds4(St, (uint32_t)(row * 4), sc_base + (uint32_t)((stage * TR + RPW * wave_u) * 4));
        }
    };

    // ---- d_mask bits of the doc range into LDS (2 words per 128-token tile) --
    const int wpd = WPT * ntd;  // mask words per doc
    const bool mask_in_lds = a.d_mask && (d1 - d0) * (int64_t)wpd <= kMaskWords;
    if (mask_in_lds) {
        // each thread turns 16 consecutive mask bytes of one doc into 16 bits
        // (a quarter of a mask word); all loads of a round are in flight together
        const int spd = 4 * wpd;  // 16-token slots per doc
        const int nslots = (int)((d1 - d0) * spd);
        for (int sl = tid; sl < nslots; sl += THREADS) {
            const int64_t doc = d0 + sl / spd;
            const int64_t t = (int64_t)(sl % spd) * 16;
            uint32_t bits = 0;
            if (t < Ld) {
                const uint8_t* p = a.d_mask + doc * Ld + t;
                const int nb = Ld - t >= 16 ? 16 : (int)(Ld - t);
                if (nb == 16 && ((uintptr_t)p & 15u) == 0) {
                    const i32x4 v = *(const i32x4*)p;
                    bits = byte_flags(v[0]) | (byte_flags(v[1]) << 4) | (byte_flags(v[2]) << 8) |
                           (byte_flags(v[3]) << 12);
                } else {
                    for (int i = 0; i < nb; ++i) bits |= (p[i] != 0 ? 1u : 0u) << i;
                }
            }
            mask_lds[sl] = (uint16_t)bits;
        }
        __builtin_amdgcn_s_waitcnt(0);
        block_barrier();
        // trailing tiles with no valid token (padding) are not streamed
        for (int kk = tid; kk < (int)(d1 - d0); kk += THREADS) {
            int n = 1;
            for (int tt = ntd - 1; tt > 0; --tt) {
                const uint16_t* w = &mask_lds[(kk * wpd + WPT * tt) * 4];
                uint32_t any = 0;
                for (int i = 0; i < 4 * WPT; ++i) any |= w[i];
                if (any != 0) {
                    n = tt + 1;
                    break;
                }
            }
            doc_tiles[kk] = (uint16_t)n;
        }
        block_barrier();
    }
    const uint32_t doc_tiles_base = lds_addr(doc_tiles);
    // tiles streamed for doc ordinal kk (uniform)
    auto tiles_of = [&](int64_t kk) -> int {
        if (!mask_in_lds) return ntd;
        uint32_t v;
        asm volatile("ds_read_u16 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(doc_tiles_base + (uint32_t)(kk * 2)) : "memory");
        return __builtin_amdgcn_readfirstlane(v);
    };
    const uint32_t mask_base = lds_addr(mask_lds);

    for (int pass = 0; pass < a.npass; ++pass) {
        // ---- the N-tiles this wave owns in this pass ------------------------
        int qi[NTW], ntl[NTW];
        float qsc[NTW];  // query-token scale (TOK)
        bool tok_ok[NTW];
        bool keep_row[NTW];  // q_mask of this lane's query token
#pragma unroll
        for (int n = 0; n < NTW; ++n) {
            const int slot = wave * NTW + n;
            bool slot_ok;
            if (a.npass == 1) {
                qi[n] = qb * a.qpw + slot / a.ntq;
                ntl[n] = slot % a.ntq;
                slot_ok = slot < a.qpw * a.ntq && qi[n] < a.Nq;
            } else {
                qi[n] = qb;
                ntl[n] = pass * SLOTS + slot;
                slot_ok = ntl[n] < a.ntq;
            }
            const int64_t s_tok = (int64_t)ntl[n] * 32 + col;
            tok_ok[n] = slot_ok && s_tok < Lq;
            keep_row[n] = tok_ok[n] && (!a.q_mask || a.q_mask[(int64_t)qi[n] * Lq + s_tok] != 0);
            if constexpr (TOK) qsc[n] = tok_ok[n] ? a.q_scale_tok[(int64_t)qi[n] * Lq + s_tok] : 0.f;
        }

        // ---- Q fragments (B operand), kept in VGPRs for the whole range -----
        i32x4 qf[NTW][KS];
#pragma unroll
        for (int n = 0; n < NTW; ++n) {
            const int64_t s_tok = (int64_t)ntl[n] * 32 + col;
            const unsigned char* qrow =
                (const unsigned char*)a.Q + ((int64_t)qi[n] * Lq + (tok_ok[n] ? s_tok : 0)) * RB;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                i32x4 v = {0, 0, 0, 0};
                if (tok_ok[n]) v = *(const i32x4*)(qrow + (2 * s + h) * 16);
                qf[n][s] = v;
            }
        }
        wait_vmcnt<0>();  // Q and the q_mask bytes have landed before the pipeline

        RowState<V, ARGMAX> st[NTW];
        // this lane's LDS slot for the saved values of N-tile n
        auto save_slot = [&](int n) -> u32x4* { return &save_buf[ARGMAX ? (wave * NTW + n) * 64 * kSaveChunks + lane : 0]; };

        // finish doc `doc` (ordinal `k` in the range): merge the lane halves,
        // apply q_mask, write argmax, put per-N-tile sums into part[k & 1]
        auto finish_doc = [&](int64_t doc, int64_t k) {
#pragma unroll
            for (int n = 0; n < NTW; ++n) {
                V mv = st[n].m;
                int iv = 0;
                if constexpr (ARGMAX) iv = saved_argmax(st[n], save_slot(n)) + 4 * h;
                const V om = __builtin_bit_cast(V, shfl_xor_i(__builtin_bit_cast(int, mv), 32));
                if constexpr (ARGMAX) {
                    const int oi = shfl_xor_i(iv, 32);
                    argmax_merge(mv, iv, om, oi);
                    if (!finite_score(mv)) iv = 0;
                    if (h == 0 && tok_ok[n])
                        a.argmax[out_pair(qi[n], doc) * Lq + (int64_t)ntl[n] * 32 + col] = iv;
                } else {
                    mv = mv > om ? mv : om;
                }
                if constexpr (TOK) mv = qsc[n] * mv;  // positive: keeps the max and -inf
                V contrib = (keep_row[n] && finite_score(mv)) ? mv : (V)0;
                // fixed-order sum over the 32 query tokens of the N-tile
                contrib = lanes0_31_sum(contrib);
                if (lane == 0)
                    lds_store_b32(part_base + (uint32_t)(((k & 1) * SLOTS + wave * NTW + n) * 4),
                                  __builtin_bit_cast(uint32_t, contrib));
            }
        };

        // wave 0 adds up part[k & 1] and writes the scores of doc `doc`: the
        // cnt partials of a query sit in a group of P lanes (P = cnt rounded
        // up to a power of two) and are added by a fixed butterfly
        auto write_scores = [&](int64_t doc, int64_t k) {
            if (wave != 0) return;
            const int cnt = a.npass == 1 ? a.ntq : (a.ntq - pass * SLOTS < SLOTS ? a.ntq - pass * SLOTS : SLOTS);
            const int nq = a.npass == 1 ? a.qpw : 1;  // queries of the workgroup
            int P = 1;
            while (P < cnt) P <<= 1;
            const int q = lane / P, n = lane % P;
            V v = 0;
            if (q < nq && n < cnt)
                v = __builtin_bit_cast(V, lds_load_b32(part_base + (uint32_t)(((k & 1) * SLOTS + q * cnt + n) * 4)));
            for (int off = P >> 1; off >= 1; off >>= 1) {
                if constexpr (std::is_integral_v<V>)
                    v += shfl_xor_i(v, off);
                else
                    v += shfl_xor_f(v, off);
            }
            if (n != 0 || q >= nq) return;
            if (a.npass == 1) {
                const int64_t i = (int64_t)qb * a.qpw + q;
                if (i < a.Nq) {
                    const int64_t o = out_pair(i, doc);
                    if constexpr (std::is_integral_v<V>) {
                        if (a.scores_i32) a.scores_i32[o] = v;
                        if (a.scores) a.scores[o] = (float)(((double)v * a.q_scale) * a.d_scale);
                    } else {
                        a.scores[o] = v;
                    }
                }
            } else {
                // one long query: this pass's sum is added to the running sum
                // kept in the output (pass 0 starts it)
                const int64_t o = out_pair(qb, doc);
                const bool last = pass + 1 == a.npass;
                if constexpr (std::is_integral_v<V>) {
                    // the int32 running sum lives in scores_i32 when it exists,
                    // else in the float output's bits until the last pass
                    int32_t* run = a.scores_i32 ? a.scores_i32 : (int32_t*)a.scores;
                    const V tot = (pass == 0 ? 0 : run[o]) + v;
                    if (a.scores_i32) a.scores_i32[o] = tot;
                    if (last && a.scores) a.scores[o] = (float)(((double)tot * a.q_scale) * a.d_scale);
                    else if (!a.scores_i32) run[o] = tot;
                } else {
                    a.scores[o] = (pass == 0 ? 0.f : a.scores[o]) + v;
                }
            }
        };

        if (F == 0) {  // Ld == 0: every doc contributes 0 and keeps argmax 0
#pragma unroll
            for (int n = 0; n < NTW; ++n) st[n].reset();
            for (int64_t k = 0; k < d1 - d0; ++k) {
                finish_doc(d0 + k, k);
                block_barrier();
                write_scores(d0 + k, k);
                block_barrier();
            }
            continue;
        }

        // issue cursor (doc ordinal ik, tile it) runs STAGES - 1 tiles ahead
        // of the compute cursor (k, tt); both advance one tile per iteration
        // over the streamed tiles of each doc
        const int64_t nd = d1 - d0;
        int64_t ik = 0;
        int it = 0, ik_tiles = tiles_of(0);
        int64_t issued = 0;
        auto advance_issue = [&]() {
            if (++it == ik_tiles) {
                it = 0;
                if (++ik < nd) ik_tiles = tiles_of(ik);
            }
        };
#pragma unroll
        for (int q = 0; q < STAGES - 1; ++q) {
            if (ik < nd) {
                issue(d0 + ik, it, q);
                advance_issue();
                ++issued;
            }
        }

        int stage = 0;
        int64_t k = 0;  // doc ordinal in the range
        int tt = 0;     // tile within the doc
        int k_tiles = tiles_of(0);
        for (int64_t f = 0; k < nd; ++f) {
            const int64_t doc = d0 + k;
            const int64_t t0 = (int64_t)tt * TR;

            // validity of the tile's rows; the scalar loads run before the
            // wait below so that their latency hides behind it
            uint64_t vb[WPT];
            if (mask_in_lds) {
                lds_read_u64_uniform<WPT>(mask_base + (uint32_t)((k * wpd + WPT * tt) * 8), vb);
            } else {
#pragma unroll
                for (int hh = 0; hh < WPT; ++hh) {
                    const int64_t left = Ld - t0 - 64 * hh;
                    const int nb = left >= 64 ? 64 : (left > 0 ? (int)left : 0);
                    if (nb == 0) vb[hh] = 0;
                    else if (a.d_mask) vb[hh] = mask_bits_scalar(a.d_mask + doc * Ld + t0 + 64 * hh, nb);
                    else vb[hh] = nb >= 64 ? ~0ull : ((1ull << nb) - 1ull);
                }
            }

            // tile f has landed once at most STAGES - 2 later tiles are in flight
            const int64_t ahead = issued - 1 - f;  // tiles issued after f (capped below)
            if constexpr (STAGES >= 4) {
                if (ahead >= 2) wait_vmcnt<2 * LPW>();
                else if (ahead == 1) wait_vmcnt<LPW>();
                else wait_vmcnt<0>();
            } else if constexpr (STAGES == 3) {
                if (ahead >= 1) wait_vmcnt<LPW>();
                else wait_vmcnt<0>();
            } else {
                wait_vmcnt<0>();
            }
            block_barrier();  // tile f landed for everyone; the stage of tile f - 1 is free
            if (ik < nd) {
                issue(d0 + ik, it, stage == 0 ? STAGES - 1 : stage - 1);
                advance_issue();
                ++issued;
            }

            if (tt == 0) {
                if (k > 0) write_scores(doc - 1, k - 1);  // its part[] is complete
#pragma unroll
                for (int n = 0; n < NTW; ++n) st[n].reset();
            }

            uint64_t vany = 0, vall = ~0ull;
#pragma unroll
            for (int hh = 0; hh < WPT; ++hh) {
                vany |= vb[hh];
                vall &= vb[hh];
            }
            if (vany != 0) {
                // A fragments of M-tile mt: row = doc token 32 mt + lane % 32,
                // 16-byte chunk 2s + lane / 32 of that row (swizzled). Plain
                // LDS loads: the stage was published by the wait + barrier
                // above, and the compiler does not see the ring's loads.
                const unsigned char* sb = stage_buf + stage * STAGE_BYTES;
                auto load_a = [&](int mt, i32x4 (&af)[KS]) {
#pragma unroll
                    for (int s = 0; s < KS; ++s) af[s] = *(const i32x4*)(sb + frag_off[s] + mt * 32 * RB);
                };
                // the MFMAs of (M-tile in af, N-tile n); with next >= 0, each
                // fragment is replaced by that of M-tile `next` as soon as its
                // MFMA has been issued (a rolling prefetch of the next M-tile)
                // The wave issues its MFMA chain at raised priority, so that
                // the SIMD's other wave (folding or reading LDS) yields the
                // issue slots while the chain is being fed (2 % on the 128 x 128 bf16
                // ColPali pairs, 3 % on the 1024-token int8 query). The fold
                // that follows in program order (of the previous unit) is
                // interleaved with the chain and drops the priority when its
                // max is issued (fold_one, CHAINED). Not with per-token
                // scales, whose VALU-heavy fold it slows down.
                auto mma = [&](i32x4 (&af)[KS], int n, int next, const Acc& init) {
                    Acc acc = init;
                    if constexpr (!TOK) __builtin_amdgcn_s_setprio(1);
#pragma unroll
                    for (int s = 0; s < KS; ++s) {
                        acc = mfma32<E>(af[s], qf[n][s], acc);
                        if (next >= 0) af[s] = *(const i32x4*)(sb + frag_off[s] + next * 32 * RB);
                    }
                    return acc;
                };
                // doc-token scales of the lane's 16 rows of M-tile mt (TOK)
                const float* scs = sc_buf + stage * TR;
                auto load_sc = [&](int mt, float (&sc)[16]) {
                    if constexpr (TOK) {
                        typedef float f4 __attribute__((ext_vector_type(4)));
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            const f4 v = *(const f4*)(scs + mt * 32 + 8 * g + 4 * h);
#pragma unroll
                            for (int e = 0; e < 4; ++e) sc[4 * g + e] = v[e];
                        }
                    }
                };
                // fold one accumulator tile; TOK first turns the integer dot
                // products into scaled floats
                auto fold = [&](const Acc& acc, int n, int base, int mt, auto maskedc, uint32_t lbits) {
                    constexpr bool MASKED = decltype(maskedc)::value;
                    if constexpr (TOK) {
                        float sc[16];
                        load_sc(mt, sc);
                        F16v sv;
#pragma unroll
                        for (int q = 0; q < 16; ++q) sv[q] = (float)acc[q] * sc[q];
                        fold_one<V, ARGMAX, MASKED>(sv, st[n], base, lbits, save_slot(n));
                    } else {
                        fold_one<V, ARGMAX, MASKED, Acc, true>(acc, st[n], base, lbits, save_slot(n));
                    }
                };
                // validity bits of the 32 rows of M-tile mt
                uint32_t mb[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) mb[mt] = (uint32_t)(vb[mt >> 1] >> (32 * (mt & 1)));
                // The (M-tile, N-tile) units of the tile in order, software-
                // pipelined: the MFMAs of unit u are issued before the fold of
                // unit u - 1, so the two execute together, and the last unit of
                // an M-tile reads the next M-tile's fragments behind its MFMAs.
                // FULL (every row valid) has no mask work at all; otherwise
                // M-tiles with no valid row skip their MFMAs and fold, and
                // partly valid ones fold with -inf in their invalid rows.
                auto run_tile = [&](auto fullc) {
                    constexpr bool FULL = decltype(fullc)::value;
                    constexpr int U = MT * NTW;
                    i32x4 af[KS];
                    Acc accs[2];
                    load_a(0, af);
                    // 16-bit inputs: the invalid rows of a partly valid M-tile
                    // start their accumulation at -inf (the MFMA adds finite
                    // products to it, so they stay -inf) and need no select in
                    // the fold; int8 and per-token scales select in the fold
                    constexpr bool BIAS = !TOK && E != kI8;
                    Acc binit = Acc{};
                    auto mask_bias = [&](int mt) {
                        Acc b;
                        const uint32_t lb = mb[mt] >> (4 * h);
#pragma unroll
                        for (int q = 0; q < 16; ++q)
                            b[q] = ((lb >> (8 * (q >> 2) + (q & 3))) & 1u) ? 0.f : -__builtin_inff();
                        return b;
                    };
                    auto fold_unit = [&](auto puc) {
                        constexpr int pu = decltype(puc)::value, pmt = pu / NTW;
                        const int base = (int)(t0 + pmt * 32);
                        if constexpr (FULL) {
                            fold(accs[pu & 1], pu % NTW, base, pmt, std::false_type{}, 0u);
                        } else if constexpr (BIAS) {
                            if (mb[pmt] != 0) fold(accs[pu & 1], pu % NTW, base, pmt, std::false_type{}, 0u);
                        } else {
                            if (mb[pmt] == 0xffffffffu)
                                fold(accs[pu & 1], pu % NTW, base, pmt, std::false_type{}, 0u);
                            else if (mb[pmt] != 0)
                                fold(accs[pu & 1], pu % NTW, base, pmt, std::true_type{}, mb[pmt] >> (4 * h));
                        }
                    };
                    static_for<0, U>([&](auto uc) {
                        constexpr int u = decltype(uc)::value;
                        constexpr int mt = u / NTW, n = u % NTW;
                        constexpr int next = (n == NTW - 1 && mt + 1 < MT) ? mt + 1 : -1;
                        if constexpr (!FULL && BIAS && n == 0)
                            if (mb[mt] != 0) binit = mb[mt] == 0xffffffffu ? Acc{} : mask_bias(mt);
                        if (FULL || mb[mt] != 0) accs[u & 1] = mma(af, n, next, (FULL || !BIAS) ? Acc{} : binit);
                        else if constexpr (next >= 0) load_a(next, af);
                        if constexpr (u > 0) fold_unit(std::integral_constant<int, u - 1>{});
                    });
                    fold_unit(std::integral_constant<int, U - 1>{});
                };
                if (vall == ~0ull) run_tile(std::true_type{});
                else run_tile(std::false_type{});
                // a chain whose fold was skipped (no valid row) left it raised
                if constexpr (!TOK) __builtin_amdgcn_s_setprio(0);
            }
            if (tt == k_tiles - 1) finish_doc(doc, k);
            stage = stage == STAGES - 1 ? 0 : stage + 1;
            if (++tt == k_tiles) {
                tt = 0;
                if (++k < nd) k_tiles = tiles_of(k);
            }
        }
        block_barrier();
        write_scores(d1 - 1, d1 - 1 - d0);
        block_barrier();  // part[] and the ring are free for the next pass
    }
}

// ---------------------------------------------------------------------------
// Host-side launch helpers.
// ---------------------------------------------------------------------------
template <int E, bool ARGMAX, int NTW, bool TOK, int STAGES, int TR, int W = kWaves>
static hipError_t launch_dense_t(DenseArgs a, hipStream_t stream)
{
    constexpr int SLOTS = W * NTW;
    a.ntq = (int)((a.Lq + 31) / 32);
    if (a.ntq == 0) a.ntq = 1;
    const bool pairs = a.pair_q != nullptr;
    if (a.ntq <= SLOTS) {
        a.qpw = pairs ? 1 : SLOTS / a.ntq;  // a pair is one query
        a.npass = 1;
    } else {
        a.qpw = 1;
        a.npass = (a.ntq + SLOTS - 1) / SLOTS;
    }
    a.nqb = (int)((a.Nq + a.qpw - 1) / a.qpw);
    int64_t units;
    if (pairs) {
        units = a.npairs;
    } else {
        const int ncu = device_cu_count();
        // doc ranges: enough workgroups to give every CU one (two with 4-wave
        // workgroups, which run two to a CU), each range at least one doc
        const int64_t per_cu = W == 8 ? 1 : 2;
        int64_t R = (per_cu * ncu + a.nqb - 1) / a.nqb;
        if (R > a.Nd) R = a.Nd;
        if (R < 1) R = 1;
        a.nranges = (int)R;
        units = (int64_t)a.nqb * R;
    }
    if (units <= 0) return hipSuccess;
    dim3 grid((unsigned)units), block(W * 64);
    hipLaunchKernelGGL((fwd_dense_kernel<E, ARGMAX, NTW, TOK, STAGES, TR, W>), grid, block, 0, stream, a);
    return hipGetLastError();
}

// Variants: 16-bit inputs use 2 N-tiles per wave (64 query tokens), which
// halves the LDS reads per MFMA against one. Without argmax a stage holds 256
// doc tokens (8 M-tiles per barrier), 512 for int8 with per-tensor scales (two
// 64 KB stages of 128-byte rows; 0.9 % faster at 1024 x 1024 tokens than 256);
// with argmax the saved-value slots (64 KB) leave room for two 128-token
// stages. A 1024-token int8 query fits one workgroup (8 waves x 4 N-tiles), so
// D is read once.
#ifndef MAXSIM_DENSE_TR
#define MAXSIM_DENSE_TR 256
#endif
hipError_t launch_fwd_dense(int elem, DenseArgs a, bool want_argmax, hipStream_t stream)
{
    constexpr int TRN = MAXSIM_DENSE_TR;  // stage rows without argmax
    switch (elem) {
    case kF16:
        return want_argmax ? launch_dense_t<kF16, true, 2, false, 2, 128>(a, stream)
                           : launch_dense_t<kF16, false, 2, false, 2, TRN>(a, stream);
    case kBF16:
        return want_argmax ? launch_dense_t<kBF16, true, 2, false, 2, 128>(a, stream)
                           : launch_dense_t<kBF16, false, 2, false, 2, TRN>(a, stream);
    case kI8:
        if (a.q_scale_tok)
            return want_argmax ? launch_dense_t<kI8, true, 2, true, 2, 128>(a, stream)
                               : launch_dense_t<kI8, false, 4, true, 3, 128>(a, stream);
        return want_argmax ? launch_dense_t<kI8, true, 2, false, 2, TRN>(a, stream)
                           : launch_dense_t<kI8, false, 4, false, 2, 512>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace maxsim
