// MaxSim forward at any embedding width for gfx950: fp16/bf16 or int8 rows
// of d elements (1 <= d <= 1024), uniform or cu_seqlens-packed, cross product
// or pair list, with masks and optional argmax; int8 with per-tensor or
// per-token scales. It serves every width other than 128 (which has its own
// kernels) and, at 128 too, cross-product calls with one or two short queries.
//
// TileMaxSim Sec. 3 (dimension tiling: a row wider than 128 is cut into
// 128-wide chunks whose partial dot products are summed before the max) and
// Sec. 6 "Embedding Dimension Scaling" with Table 9 (d from 64 to 768); the
// TileMaxSim README notes on the embedding-dimension dispatch (a width up to
// 128 is padded and the surplus lanes read as zero, which leaves every score
// unchanged); "Flash-MaxSim" Sec. 4.1 and 4.1.1 (online max, -inf masking,
// strict '>' argmax update), Sec. 4.3.1 (INT8 x INT8 with the scales fused
// into the epilogue; per-token doc scales inside the max) and Sec. 4.3.2
// (cu_seqlens scoring over sum(L_d) rows).
//
// Design. The streaming scheme of the 128-wide padding-free kernel,
// generalised in the width. A row is cut into 256-byte chunks (128 fp16/bf16
// or 256 int8 elements, the last chunk partial), so a 16-row tile of the doc
// stream becomes C chunk tiles of 4 KB (rows of at most 128 bytes instead
// fill a 4 KB stage with 32 rows). A workgroup of 4 waves owns a contiguous,
// token-balanced range of whole docs and splits the range's tiles evenly
// among its waves; each wave pulls its chunk tiles through a private LDS ring
// with direct-to-LDS loads (16 bytes per lane, the pieces XOR-swizzled by row
// so that the MFMA operand reads are conflict free). The 16x16x32 fp16/bf16
// MFMA (16x16x64 for int8, exact int32 sums) consumes a chunk tile in up to
// four 64-byte K-steps and accumulates the S tile over the C chunks; only
// after the last chunk is the tile folded into the running max, so the dot
// products are those of the whole row. Past the row end the query side holds
// zeros (K-steps wholly past it are skipped) and the doc side re-reads a
// piece of the same row, so no load leaves the row and the padded lanes add
// exact zeros. A doc whose rows run on into the next wave's share is finished
// by the wave that holds its first row, after the later waves hand their
// partial maxima over through LDS.
//
// When the query block fits one chunk (d <= 128) its fragments stay in VGPRs
// for the pass. Wider queries are staged once per pass into LDS, shared by the
// workgroup's waves, and read per chunk tile; with a pair list, where each
// wave has its own query, a unit is one wave's pair (and a workgroup a single
// wave when the query is staged). Rows whose byte length is not a multiple of
// 16 cannot take 16-byte loads: their pieces are gathered element by element
// and written to LDS in the same layout (a slower path). With per-token int8
// scales, every chunk tile also brings its doc-token scales into the ring by a
// 4-byte direct-to-LDS load; they turn the tile's integer dot products into
// floats before the max, and the query-token scale (positive) multiplies the
// max.
//
// Queries are the fastest grid axis, so the workgroups that are resident
// together share doc ranges and the repeated reads of a range for different
// queries are served from cache. Scores of a long query are the sum of its
// 32-token passes, added in pass order.
#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace maxsim {

namespace {

constexpr int kNT = 2;                         // 16-token query N-tiles per pass
constexpr int kPassTokens = 16 * kNT;          // query tokens per pass
constexpr int kChunkBytes = 256;               // bytes of a row per chunk tile
constexpr int kCTileBytes = 16 * kChunkBytes;  // chunk tile: 16 rows x 256 bytes
#ifndef MAXSIM_DIM_STAGES
#define MAXSIM_DIM_STAGES 2
#endif
constexpr int kStages = MAXSIM_DIM_STAGES;  // chunk tiles in flight per wave (2..4)
static_assert(kStages >= 2 && kStages <= 4, "vmcnt waits cover up to three later tiles");

// vmcnt(LPI n): the n most recently issued chunk tiles (LPI loads each) may
// still be in flight
template <int LPI>
__device__ __forceinline__ void wait_ctiles_behind(int n)
{
    if (n <= 0) wait_vmcnt<0>();
    else if (n == 1) wait_vmcnt<LPI>();
    else if (n == 2) wait_vmcnt<2 * LPI>();
    else wait_vmcnt<3 * LPI>();
}

// Element traits: a K-step is 64 bytes of a row for every type.
template <int E> struct DimT;
template <> struct DimT<kF16> {
    static constexpr int kES = 2;
    typedef f32x4 Acc;
};
template <> struct DimT<kBF16> {
    static constexpr int kES = 2;
    typedef f32x4 Acc;
};
template <> struct DimT<kI8> {
    static constexpr int kES = 1;
    typedef i32x4 Acc;
};
template <int E>
__device__ __forceinline__ typename DimT<E>::Acc mma(const i32x4& a, const i32x4& b, const typename DimT<E>::Acc& c)
{
    if constexpr (E == kI8) return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
    else return mfma16<E>(a, b, c);
}

// 16 bytes of a row starting at byte `off`; bytes at or past `rb` (the row's
// length in bytes) read as zero. With 16-byte aligned rows (`al`) a piece is
// either whole or past the end; otherwise it is gathered from ES-byte elements.
template <int ES>
__device__ __forceinline__ i32x4 load_piece(const unsigned char* row, int off, int rb, bool al)
{
    if (al) {
        i32x4 v = {0, 0, 0, 0};
        if (off < rb) v = *(const i32x4*)(row + off);
        return v;
    }
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int b = 0; b < 16; b += ES) {
        if (off + b < rb) {
            const uint32_t e = ES == 2 ? (uint32_t)(*(const uint16_t*)(row + off + b)) : (uint32_t)row[off + b];
            w[b >> 2] |= e << (8 * (b & 3));
        }
    }
    return i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
}

// LDS store into the direct-to-LDS ring, in assembly so that the compiler adds
// no wait for the ring's loads in flight
__device__ __forceinline__ void lds_write_b128(uint32_t addr, const i32x4& v)
{
    asm volatile("ds_write_b128 %0, %1" ::"v"(addr), "v"(v) : "memory");
}

// nonzero flags of the 4 bytes of x (byte b -> bit b)
__device__ __forceinline__ uint32_t nz_bytes(uint32_t x)
{
    x |= x >> 4;
    x |= x >> 2;
    x |= x >> 1;
    x &= 0x01010101u;
    return ((x * 0x01020408u) >> 24) & 0xFu;
}

// Validity bits of the `nb` (1..16) doc tokens whose mask bytes start at the
// wave-uniform address `p` (bit r = token r), from scalar loads of the aligned
// dwords that hold those bytes only.
__device__ __forceinline__ uint32_t mask_bits16(const uint8_t* p, int nb)
{
    const uintptr_t addr = (uintptr_t)uniform_ptr(p);
    const int sh = (int)(addr & 3u);
    const __attribute__((address_space(4))) uint32_t* w =
        (const __attribute__((address_space(4))) uint32_t*)(addr - (uintptr_t)sh);
    const int ndw = (sh + nb + 3) >> 2;  // 1 .. 5
    uint32_t bits = 0;
    for (int k = 0; k < ndw; ++k) bits |= nz_bytes(w[k]) << (4 * k);
    bits >>= sh;
    return bits & ((1u << nb) - 1u);
}

}  // namespace

// Three waves per SIMD for the plain register-query kernels (they fit in 168
// VGPRs without spilling; two per SIMD measured slower); the argmax and
// per-token instances keep the compiler's choice, which does not spill.
template <int E, bool ARGMAX, bool QREG, int W, bool TOK, int MT>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(QREG && !ARGMAX && !TOK ? 3 : 1)))
void fwd_dim_kernel(DimArgs a)
{
    static_assert(!TOK || E == kI8, "per-token scales are an int8 mode");
    // MT = 2: rows of at most 128 bytes, so a 4 KB stage holds 32 rows of 128
    // bytes (two MFMA M-tiles) instead of 16 rows of 256
    static_assert(MT == 1 || (MT == 2 && QREG), "two M-tiles per stage only for one-chunk rows");
    constexpr int R = 16 * MT;             // rows per chunk tile
    constexpr int CB = kChunkBytes / MT;   // bytes of a row in a stage
    constexpr int KMAX = CB / 64;          // K-steps a stage row holds
    using Acc = typename DimT<E>::Acc;
    using V = std::conditional_t<E == kI8 && !TOK, int, float>;  // value of the max
    constexpr int ES = DimT<E>::kES;
    constexpr int LPI = TOK ? 5 : 4;  // loads per chunk tile: 4 row loads (+ the doc-token scales)
    constexpr int kStageBytes = kCTileBytes + (TOK ? 256 : 0);
    extern __shared__ __attribute__((aligned(16))) unsigned char dim_lds[];
    const int lane = lane_id();
    const int col = lane & 15;  // query token of an N-tile / doc row of a tile
    const int g = lane >> 4;    // tile rows 4g .. 4g+3 and K-quarter g
    const int wave = threadIdx.x >> 6;
    const int C = uniform(a.nchunk);
    const int RB = uniform(a.row_bytes);
    const bool al = (RB & 15) == 0;
    const int kt_last = (RB - (C - 1) * kChunkBytes + 63) >> 6;  // K-steps of the last chunk
    unsigned char* qbuf = dim_lds;  // staged query block: [kNT][C] chunk tiles
    const uint32_t q_base = lds_addr(qbuf);
    unsigned char* ring = dim_lds + (QREG ? 0 : kNT * C * kCTileBytes) + wave * kStages * kStageBytes;
    const uint32_t ring_base = (uint32_t)uniform((int)lds_addr(ring));
    // hand-over slot of wave w, written once its ring is idle at the end of a
    // pass: the continued doc and the per-lane partial state
    auto slot_of = [&](int w) { return dim_lds + (QREG ? 0 : kNT * C * kCTileBytes) + w * kStages * kStageBytes; };
    static_assert(16 + kNT * 64 * 8 <= kCTileBytes, "a hand-over slot fits one ring stage");

    // ---- the docs of this unit ----------------------------------------------
    // With a pair list a unit is one wave's pair. Otherwise a unit is the
    // workgroup's doc range, whose tiles are split evenly among its waves
    // (`split`): a doc belongs to the wave holding its first row, and the
    // waves that hold later rows of it hand their partial maxima over through
    // LDS at the end of the pass.
    const bool pairs = a.pair_q != nullptr;
    const bool split = !pairs;
    const int64_t unit = pairs ? (int64_t)blockIdx.x * W + wave : (int64_t)blockIdx.y;
    const int64_t U = pairs ? a.npairs : (int64_t)a.units;
    const int Nd = (int)a.Nd;
    int jb = 0, je = 0, iq = 0;
    if (unit < U) {
        if (pairs) {
            const int32_t pq = a.pair_q[unit], pd = a.pair_d[unit];
            iq = uniform(pq < 0 ? 0 : (pq >= a.Nq ? (int)a.Nq - 1 : pq));  // precondition guard
            jb = uniform(pd < 0 ? 0 : (pd >= Nd ? Nd - 1 : pd));
            je = jb + 1;
        } else if (a.cu_d) {
            const int64_t T = a.cu_d[Nd];
            jb = unit == 0 ? 0 : nearest_boundary(a.cu_d, Nd, (T * unit) / U);
            je = unit + 1 == U ? Nd : nearest_boundary(a.cu_d, Nd, (T * (unit + 1)) / U);
        } else {
            jb = uniform((int)(((int64_t)Nd * unit) / U));
            je = uniform((int)(((int64_t)Nd * (unit + 1)) / U));
        }
    }
    // a unit with no docs leaves now unless its workgroup shares a staged query
    // (in split mode every wave of the workgroup has the same range)
    if ((QREG || W == 1) && jb >= je) return;

    auto doc_off = [&](int j) -> int64_t { return a.cu_d ? (int64_t)a.cu_d[j] : (int64_t)j * a.Ld; };
    const int64_t u0 = jb < je ? uniform_i64(doc_off(jb)) : 0;
    const int span = jb < je ? uniform((int)(doc_off(je) - u0)) : 0;
    const int ntile = (span + R - 1) / R;
    const unsigned char* unit_ptr = (const unsigned char*)a.D + u0 * RB;

    // this wave's tiles [t_begin, t_end), rows [r_lo, r_hi), and owned docs
    // [j_own, j_lim): those whose first row is in the rows (the last wave also
    // owns the empty docs at the end of the range); j_own - 1 continues into
    // the rows when it starts before r_lo and ends after it
    int t_begin = 0, t_end = ntile, r_lo = 0, r_hi = span, j_own = jb, j_lim = je;
    bool has_cont = false;
    if (split && jb < je) {
        t_begin = (int)(((int64_t)ntile * wave) / W);
        t_end = (int)(((int64_t)ntile * (wave + 1)) / W);
        r_lo = t_begin * R;
        r_hi = wave == W - 1 ? span : t_end * R;
        // first doc of [jb, je] whose start is at or after row x of the range
        auto first_from = [&](int x) -> int {
            if (a.cu_d) return jb + wave_lower_bound(a.cu_d + jb, je - jb, u0 + x);
            if (a.Ld <= 0) return x > 0 ? je : jb;
            const int64_t k = jb + ((int64_t)x + a.Ld - 1) / a.Ld;
            return uniform((int)(k < je ? k : je));
        };
        j_own = first_from(r_lo);
        j_lim = wave == W - 1 ? je : first_from(r_hi);
        has_cont = j_own > jb && doc_off(j_own) - u0 > r_lo;
    }
    const int nitem = (t_end - t_begin) * C;

    // A-operand reads of M-tile m: row r = 16 m + lane % 16, logical piece
    // 4k + g; 256-byte rows keep piece p at slot p ^ (r % 16), 128-byte rows
    // at slot p ^ ((r / 2) % 8), so the 16 rows a read touches fall in
    // distinct banks either way
    uint32_t frag_off[MT][4];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int r = 16 * m + col;
            frag_off[m][k] = MT == 1 ? (uint32_t)(col * kChunkBytes + (((4 * k + g) ^ col) << 4))
                                     : (uint32_t)(r * CB + (((4 * k + g) ^ ((r >> 1) & 7)) << 4));
        }

    const int64_t i_begin = pairs ? iq : blockIdx.x, i_end = pairs ? iq + 1 : a.Nq;
    const int64_t i_step = pairs ? 1 : gridDim.x;
    for (int64_t i = i_begin; i < i_end; i += i_step) {
        const int64_t q0 = a.cu_q ? (int64_t)a.cu_q[i] : i * a.Lq;
        int64_t lq64 = a.cu_q ? (int64_t)a.cu_q[i + 1] - q0 : a.Lq;
        if (lq64 > a.Lq) lq64 = a.Lq;
        if (lq64 < 0) lq64 = 0;
        const int lq = uniform((int)lq64);
        const int npass = lq == 0 ? 1 : (lq + kPassTokens - 1) / kPassTokens;
        const int j_out = pairs ? jb : 0;  // outputs of doc j are at [j - j_out]
        const int64_t out_row = pairs ? unit : i * a.Nd;
        int32_t* arg_row = ARGMAX ? a.argmax + out_row * a.Lq : nullptr;

        for (int pass = 0; pass < npass; ++pass) {
            // ---- query block: tokens pass*32 + n*16 + col ----------------------
            bool tok_in[kNT], tok_ok[kNT];
            float qsc[kNT];  // query-token scales (TOK)
            i32x4 qf[kNT][4];
#pragma unroll
            for (int n = 0; n < kNT; ++n) {
                const int s = pass * kPassTokens + n * 16 + col;
                tok_in[n] = s < lq;
                tok_ok[n] = tok_in[n] && (a.q_mask == nullptr || a.q_mask[i * a.Lq + s] != 0);
                qsc[n] = 0.f;
                if constexpr (TOK) qsc[n] = tok_in[n] ? a.q_scale_tok[q0 + s] : 0.f;
                if constexpr (QREG) {
                    const unsigned char* qrow = (const unsigned char*)a.Q + (q0 + (tok_in[n] ? s : 0)) * RB;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        i32x4 v = {0, 0, 0, 0};
                        if (tok_in[n]) v = load_piece<ES>(qrow, (4 * k + g) << 4, RB, al);
                        qf[n][k] = v;
                    }
                }
            }
            if constexpr (!QREG) {
                block_barrier();  // every wave is done with the previous block
                for (int it = threadIdx.x; it < kNT * C * 256; it += W * 64) {
                    const int lp = it & 15, row = (it >> 4) & 15, nc = it >> 8;
                    const int n = nc / C, c = nc - n * C;
                    const int s = pass * kPassTokens + n * 16 + row;
                    i32x4 v = {0, 0, 0, 0};
                    if (s < lq)
                        v = load_piece<ES>((const unsigned char*)a.Q + (q0 + s) * RB, c * kChunkBytes + (lp << 4), RB, al);
                    *(i32x4*)(qbuf + nc * kCTileBytes + row * kChunkBytes + ((lp ^ row) << 4)) = v;
                }
                block_barrier();
            }
            if (jb >= je) continue;  // no docs: only here to share the staged query

            // ---- doc cursor ------------------------------------------------------
            bool cont = has_cont;  // folding the doc continued from the previous wave
            int j = cont ? j_own - 1 : j_own;
            int cache_base = j + 1;  // lane k holds cu_d[cache_base + k] - u0 (packed docs)
            int cu_cache = 0;
            if (a.cu_d) cu_cache = (int)((int64_t)a.cu_d[cache_base + lane <= Nd ? cache_base + lane : Nd] - u0);
            wait_vmcnt<0>();  // query fragments, scales, masks and the cache have landed
            auto doc_end_of = [&](int jj) -> int {  // offset of the end of doc jj in the unit
                if (!a.cu_d) return uniform((int)((int64_t)(jj + 1) * a.Ld - u0));
                int off = jj + 1 - cache_base;
                if (off >= 64) {  // once per 64 docs
                    cache_base = jj + 1;
                    cu_cache = (int)((int64_t)a.cu_d[cache_base + lane <= Nd ? cache_base + lane : Nd] - u0);
                    wait_vmcnt<0>();
                    off = 0;
                }
                return uniform(__builtin_amdgcn_readlane(cu_cache, off));
            };
            int doc_start = j < je ? uniform((int)(doc_off(j) - u0)) : span;
            int doc_end = j < je ? doc_end_of(j) : span;

            V m[kNT];
            int idx[kNT];
#pragma unroll
            for (int n = 0; n < kNT; ++n) {
                m[n] = neg_inf<V>();
                idx[n] = 0;
            }

            // finish doc j: merge the 4 row groups, sum the valid query rows, write
            auto finish_doc = [&]() {
                V total = 0;
#pragma unroll
                for (int n = 0; n < kNT; ++n) {
                    V mv = m[n];
                    int iv = idx[n];
#pragma unroll
                    for (int off = 16; off <= 32; off <<= 1) {
                        const V om = __builtin_bit_cast(V, shfl_xor_i(__builtin_bit_cast(int, mv), off));
                        if constexpr (ARGMAX) {
                            const int oi = shfl_xor_i(iv, off);
                            argmax_merge(mv, iv, om, oi);
                        } else {
                            mv = om > mv ? om : mv;
                        }
                    }
                    const bool fin = finite_score(mv);
                    if constexpr (TOK) mv = fin ? qsc[n] * mv : mv;  // positive: keeps the max
                    total += row16_sum((tok_ok[n] && fin) ? mv : (V)0);
                    if constexpr (ARGMAX) {
                        if (g == 0 && tok_in[n]) {
                            const int s = pass * kPassTokens + n * 16 + col;
                            arg_row[(int64_t)(j - j_out) * a.Lq + s] = fin ? iv - doc_start : 0;
                        }
                    }
                    m[n] = neg_inf<V>();
                    idx[n] = 0;
                }
                if constexpr (ARGMAX) {
                    if (pass == 0)  // rows past the query's length are 0
                        for (int s = lq + lane; s < a.Lq; s += 64) arg_row[(int64_t)(j - j_out) * a.Lq + s] = 0;
                }
                if (lane == 0) {
                    const int64_t o = out_row + (j - j_out);
                    if constexpr (std::is_integral_v<V>) {
                        // the int32 running sum lives in scores_i32 when it exists,
                        // else in the bits of scores until the last pass
                        int32_t* run = a.scores_i32 ? a.scores_i32 : (int32_t*)a.scores;
                        const int32_t tot = pass == 0 ? total : run[o] + total;
                        if (a.scores_i32) a.scores_i32[o] = tot;
                        if (pass + 1 == npass && a.scores) a.scores[o] = (float)(((double)tot * a.q_scale) * a.d_scale);
                        else if (!a.scores_i32) run[o] = tot;
                    } else {
                        a.scores[o] = pass == 0 ? total : a.scores[o] + total;
                    }
                }
            };

            // fold tile rows [lo, hi) that are valid in `vb` into the running state
            // (TOK: the integer dot products scaled by the rows' doc-token scales)
            auto fold = [&](const Acc (&acc)[kNT], const float (&sc)[4], int tile0, int lo, int hi, uint32_t vb) {
                const uint32_t bits = ((1u << hi) - 1u) & ~((1u << lo) - 1u) & vb;
                const uint32_t lb = bits >> (4 * g);
                const bool full = bits == 0xFFFFu;
#pragma unroll
                for (int n = 0; n < kNT; ++n) {
                    V v[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if constexpr (TOK) v[r] = (float)acc[n][r] * sc[r];
                        else v[r] = acc[n][r];
                        if (!full) v[r] = ((lb >> r) & 1u) ? v[r] : neg_inf<V>();
                    }
                    if constexpr (ARGMAX) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (v[r] > m[n]) {
                                m[n] = v[r];
                                idx[n] = tile0 + 4 * g + r;
                            }
                    } else {
                        const V a01 = v[0] > v[1] ? v[0] : v[1];
                        const V a23 = v[2] > v[3] ? v[2] : v[3];
                        const V a03 = a01 > a23 ? a01 : a23;
                        m[n] = a03 > m[n] ? a03 : m[n];
                    }
                }
            };

            // the partial state of the continued doc, kept until the hand-over
            V mc[kNT];
            int ic[kNT];
#pragma unroll
            for (int n = 0; n < kNT; ++n) {
                mc[n] = neg_inf<V>();
                ic[n] = 0;
            }
            auto store_cont = [&]() {
#pragma unroll
                for (int n = 0; n < kNT; ++n) {
                    mc[n] = m[n];
                    ic[n] = idx[n];
                    m[n] = neg_inf<V>();
                    idx[n] = 0;
                }
                cont = false;
            };
            // a doc that ends: finished here, or handed over when continued
            auto end_doc = [&]() {
                if (cont) store_cont();
                else finish_doc();
            };

            // leading empty docs
            while (j < j_lim && doc_end <= r_lo) {
                finish_doc();
                ++j;
                if (j < j_lim) {
                    doc_start = doc_end;
                    doc_end = doc_end_of(j);
                }
            }

            // ---- chunk-tile ring ---------------------------------------------------
            int t_next = t_begin, c_next = 0, s_next = 0;  // next chunk tile to fetch, its stage
            auto issue = [&]() {
                const unsigned char* tp = (const unsigned char*)uniform_ptr(unit_ptr + (int64_t)t_next * R * RB);
                const int rows_left = span - t_next * R;  // rows past the unit re-read its last row
                const uint32_t dst = (uint32_t)uniform((int)(ring_base + s_next * kStageBytes));
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    // lane's 16-byte slot of instruction k: row and logical piece (see frag_off)
                    const int row = MT == 1 ? 4 * k + g : 8 * k + (lane >> 3);
                    const int lp = MT == 1 ? col ^ row : (lane & 7) ^ ((row >> 1) & 7);
                    const int r = row < rows_left ? row : rows_left - 1;
                    int off = c_next * kChunkBytes + (lp << 4);
                    if (al) {
                        if (off >= RB) off = c_next * kChunkBytes;  // past the row end: a piece of the same row
                        dma_lds16_nt(tp, (uint32_t)(r * RB + off), dst + k * 1024);
                    } else {
                        lds_write_b128(dst + k * 1024 + lane * 16, load_piece<ES>(tp + r * RB, off, RB, false));
                    }
                }
                if constexpr (TOK) {  // lane l: the scale of tile row l % R, at dst + 4 KB + 4 l
                    const float* sp = (const float*)uniform_ptr(a.d_scale_tok + u0 + (int64_t)t_next * R);
                    const int rl = lane & (R - 1);
                    const int r = rl < rows_left ? rl : rows_left - 1;
                    dma_lds4(sp, (uint32_t)(r * 4), dst + kCTileBytes);
                }
                if (++c_next == C) {
                    c_next = 0;
                    ++t_next;
                }
                s_next = s_next + 1 == kStages ? 0 : s_next + 1;
            };
            for (int q = 0; q < kStages && q < nitem; ++q) issue();

            int stage = 0;
            for (int t = t_begin; t < t_end && j < j_lim; ++t) {
                Acc acc[MT][kNT];
#pragma unroll
                for (int m = 0; m < MT; ++m)
#pragma unroll
                    for (int n = 0; n < kNT; ++n) acc[m][n] = Acc{0, 0, 0, 0};
                float sc[MT][4];  // doc-token scales of rows 16m + 4g .. +3 (TOK)
#pragma unroll
                for (int m = 0; m < MT; ++m) sc[m][0] = sc[m][1] = sc[m][2] = sc[m][3] = 1.f;
                for (int c = 0; c < C; ++c) {
                    const int q = (t - t_begin) * C + c;
                    const int behind = nitem - 1 - q;
                    wait_ctiles_behind<LPI>(behind < kStages - 1 ? behind : kStages - 1);
                    const uint32_t sbase = ring_base + stage * kStageBytes;
                    i32x4 af[MT][4];
                    if constexpr (MT == 1)
                        lds_read4(af[0][0], af[0][1], af[0][2], af[0][3], sbase + frag_off[0][0], sbase + frag_off[0][1],
                                  sbase + frag_off[0][2], sbase + frag_off[0][3]);
                    else  // 128-byte rows hold two K-steps
                        lds_read4(af[0][0], af[0][1], af[1][0], af[1][1], sbase + frag_off[0][0], sbase + frag_off[0][1],
                                  sbase + frag_off[1][0], sbase + frag_off[1][1]);
                    if constexpr (TOK) {
                        if (c == C - 1) {  // before the stage is refilled
                            // a plain LDS load (the ring's direct-to-LDS writes are
                            // inline assembly, so the compiler adds no wait for
                            // them): taking the four values out of an assembly
                            // ds_read_b128 that is skipped on other paths gave
                            // the first value for all four with this compiler
#pragma unroll
                            for (int m = 0; m < MT; ++m) {
                                const f32x4 sv = *(const f32x4*)(ring + stage * kStageBytes + kCTileBytes + 64 * m + 16 * g);
                                sc[m][0] = sv.x;
                                sc[m][1] = sv.y;
                                sc[m][2] = sv.z;
                                sc[m][3] = sv.w;
                            }
                        }
                    }
                    if constexpr (!QREG) {
                        i32x4 qv[8];
                        uint32_t qa[8];
#pragma unroll
                        for (int n = 0; n < kNT; ++n)
#pragma unroll
                            for (int k = 0; k < 4; ++k) qa[n * 4 + k] = q_base + (n * C + c) * kCTileBytes + frag_off[0][k];
                        lds_read8(qv, qa);
#pragma unroll
                        for (int n = 0; n < kNT; ++n)
#pragma unroll
                            for (int k = 0; k < 4; ++k) qf[n][k] = qv[n * 4 + k];
                    }
                    if (q + kStages < nitem) issue();  // refill the stage just read
                    stage = stage + 1 == kStages ? 0 : stage + 1;
                    const int kt = c == C - 1 ? kt_last : 4;
#pragma unroll
                    for (int k = 0; k < KMAX; ++k) {
                        if (k < kt) {
#pragma unroll
                            for (int m = 0; m < MT; ++m)
#pragma unroll
                                for (int n = 0; n < kNT; ++n) acc[m][n] = mma<E>(af[m][k], qf[n][k], acc[m][n]);
                        }
                    }
                }

#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    const int tile0 = t * R + 16 * m;
                    if (j >= j_lim || tile0 >= span) break;
                    uint32_t vb = 0xFFFFu;
                    if (a.d_mask) {
                        const int nb = span - tile0 < 16 ? span - tile0 : 16;
                        vb = mask_bits16(a.d_mask + u0 + tile0, nb);
                    }
                    int lo = 0;
                    while (true) {
                        const int hi = doc_end - tile0 < 16 ? doc_end - tile0 : 16;
                        if (hi > lo) fold(acc[m], sc[m], tile0, lo, hi, vb);
                        if (doc_end - tile0 > 16) break;  // the doc continues in the next tile
                        end_doc();
                        ++j;
                        if (j >= j_lim) break;
                        lo = hi > lo ? hi : lo;
                        doc_start = doc_end;
                        doc_end = doc_end_of(j);
                    }
                }
            }
            // a doc continued through all of this wave's rows (or into an empty
            // range) is handed over whole
            if (cont) {
                store_cont();
                ++j;
                if (j < j_lim) {
                    doc_start = doc_end;
                    doc_end = doc_end_of(j);
                }
            }
            // the last rows' open doc: finished by this wave after the hand-over
            const bool open = split && wave < W - 1 && j < j_lim;
            // docs left with no tokens (the empty docs at the end of the range)
            while (!open && j < j_lim) {
                finish_doc();
                ++j;
                if (j < j_lim) {
                    doc_start = doc_end;
                    doc_end = doc_end_of(j);
                }
            }
            wait_vmcnt<0>();  // nothing of this pass is still in flight
            if (split) {
                {
                    unsigned char* sl = slot_of(wave);
                    if (lane == 0) *(int*)sl = has_cont ? j_own - 1 : -1;
#pragma unroll
                    for (int n = 0; n < kNT; ++n) {
                        ((V*)(sl + 16))[n * 64 + lane] = mc[n];
                        ((int*)(sl + 16 + kNT * 64 * 4))[n * 64 + lane] = ic[n];
                    }
                }
                block_barrier();  // every wave's hand-over is in LDS
                if (open) {
                    // merge the later waves' partial maxima of doc j, in wave
                    // (= row) order, so equal maxima keep the lowest row
                    for (int w2 = wave + 1; w2 < W; ++w2) {
                        const unsigned char* sl = slot_of(w2);
                        if (uniform(*(const int*)sl) != j) break;
#pragma unroll
                        for (int n = 0; n < kNT; ++n) {
                            const V om = ((const V*)(sl + 16))[n * 64 + lane];
                            const int oi = ((const int*)(sl + 16 + kNT * 64 * 4))[n * 64 + lane];
                            if constexpr (ARGMAX) argmax_merge(m[n], idx[n], om, oi);
                            else m[n] = om > m[n] ? om : m[n];
                        }
                    }
                    finish_doc();
                }
                block_barrier();  // the slots (ring stages) are free for the next pass
            }
        }
    }
}

namespace {

template <int E, bool ARGMAX, bool QREG, int W, bool TOK, int MT = 1>
hipError_t launch_dim_t(DimArgs a, hipStream_t stream)
{
    auto kern = fwd_dim_kernel<E, ARGMAX, QREG, W, TOK, MT>;
    constexpr int kStageBytes = kCTileBytes + (TOK ? 256 : 0);
    const size_t lds = (size_t)(QREG ? 0 : kNT * a.nchunk) * kCTileBytes + (size_t)W * kStages * kStageBytes;
    if (a.pair_q) {
        a.units = 0;
        const int64_t blocks = (a.npairs + W - 1) / W;
        hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(W * 64), lds, stream, a);
        return hipGetLastError();
    }
    // resident workgroups per CU, per chunk count (the LDS size depends on it)
    static std::atomic<int> per_cu_cache[9];
    const int key = a.nchunk < 9 ? a.nchunk : 8;  // (one instance per MT: a kernel has one MT)
    int per_cu = per_cu_cache[key].load(std::memory_order_relaxed);
    if (per_cu <= 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, W * 64, lds) != hipSuccess || per_cu <= 0)
            per_cu = 1;
        per_cu_cache[key].store(per_cu, std::memory_order_relaxed);
    }
    // a unit is a workgroup's doc range: about one resident workgroup per unit
    // over all queries, at most one unit per doc (more, shorter units measured
    // slower here: a unit's setup, and for a staged query its LDS copy, is
    // paid per unit)
    const int64_t wg_slots = (int64_t)device_cu_count() * per_cu;
    int64_t units = (wg_slots + a.Nq - 1) / a.Nq;
    if (units > a.Nd) units = a.Nd;
    if (units < 1) units = 1;
    a.units = (int32_t)units;
    const int64_t gq = a.Nq < 65535 ? a.Nq : 65535;
    hipLaunchKernelGGL(kern, dim3((unsigned)gq, (unsigned)units), dim3(W * 64), lds, stream, a);
    return hipGetLastError();
}

template <int E, bool TOK>
hipError_t launch_dim_e(DimArgs a, hipStream_t stream)
{
    const bool am = a.argmax != nullptr;
    if (a.row_bytes <= kChunkBytes / 2)  // two 16-row M-tiles of 128-byte rows per stage
        return am ? launch_dim_t<E, true, true, 4, TOK, 2>(a, stream) : launch_dim_t<E, false, true, 4, TOK, 2>(a, stream);
    if (a.nchunk == 1)
        return am ? launch_dim_t<E, true, true, 4, TOK>(a, stream) : launch_dim_t<E, false, true, 4, TOK>(a, stream);
    if constexpr (E != kI8) {  // pair lists (16-bit types only): one wave per workgroup
        if (a.pair_q)
            return am ? launch_dim_t<E, true, false, 1, TOK>(a, stream)
                      : launch_dim_t<E, false, false, 1, TOK>(a, stream);
    }
    return am ? launch_dim_t<E, true, false, 4, TOK>(a, stream) : launch_dim_t<E, false, false, 4, TOK>(a, stream);
}

}  // namespace

hipError_t launch_fwd_dim(int elem, DimArgs a, hipStream_t stream)
{
    if (a.d < 1 || a.d > 1024) return hipErrorInvalidValue;
    a.row_bytes = elem == kI8 ? a.d : a.d * 2;
    a.nchunk = (a.row_bytes + kChunkBytes - 1) / kChunkBytes;
    switch (elem) {
    case kF16: return launch_dim_e<kF16, false>(a, stream);
    case kBF16: return launch_dim_e<kBF16, false>(a, stream);
    case kI8:
        if (a.pair_q) return hipErrorInvalidValue;
        return a.q_scale_tok ? launch_dim_e<kI8, true>(a, stream) : launch_dim_e<kI8, false>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace maxsim
