// Argmax-driven MaxSim backward for gfx950, atomic-free and deterministic.
//
// "Flash-MaxSim" Sec. 4.2.1 Eqs. (2)-(3) (gradients flow only through the
// forward winner), Sec. 4.2.2 (the saved source->destination argmax map is
// inverted at run time into a CSR: histogram, cumulative sum, stable order of
// sources), Sec. 4.2.3 (one owner per output row, fp32 accumulation, each row
// written once, no atomics); late-interaction-kernels design notes "Backward"
// (the q_mask factor, grad_Q as a row-owned gather over docs).
//
// Launch sequence on one stream:
//   csr+dq  one launch of 16-wave workgroups. The first Nd build the CSR of
//           one doc each: every doc receives exactly Nq*Lq sources, so its
//           CSR segment starts at j*Nq*Lq and no global scan is needed. Each
//           wave holds the destinations of a contiguous block of the doc's
//           sources in registers and counts them into its own LDS histogram;
//           the counts are scanned, and every wave places its block in
//           source order (ranks inside a wave from equal destinations found
//           through LDS, or for docs too large for one pass from ballots
//           over the key bits), so each CSR row lists its sources
//           ascending; a one-pass doc is staged in LDS and written out
//           contiguously. The other
//           workgroups compute dQ, which needs no CSR: one 16-lane group per
//           query row (i,s), 64 rows per workgroup; the argmax entries and
//           weights g[i,j] live(j) of 64 docs at a time are staged in LDS
//           (live(j) = any(d_mask[j,:]) found by the workgroup itself), then
//           each group gathers D[j, argmax[i,j,s]] for j ascending (16 bytes
//           per lane, 8 loads in flight) and accumulates in fp32; a row with
//           q_mask 0 gathers nothing. All workgroups sweep j in the same
//           order, so the D rows they gather are shared in L2;
//   dd      one 16-lane group per destination row (j,t): the group walks the
//           row's sources in CSR order, gathers the Q rows (16 bytes per
//           lane) of those with a nonzero weight and accumulates in fp32;
//           every row is written once.
// The padding-free backward (vbwd_*) and the Chamfer backward (cham_*) below
// follow the same pattern.
#include "common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace maxsim {

namespace {

constexpr int kCsrWaves = 16;
constexpr int kCsrThreads = kCsrWaves * 64;
constexpr int kCsrChunk = 16384;  // sources of one doc held in registers per pass (16 per lane)
constexpr int kCsrBins = 1024;    // destination bins handled per round
constexpr int kPartSteps = 4;     // sources per lane in a chunk of the Chamfer partition
constexpr int kPartChunk = kCsrWaves * 64 * kPartSteps;  // 4,096 sources per partition chunk
constexpr int kDqDocs = 64;                   // docs staged per round of the dq pass
constexpr uint16_t kNoKey = 0xFFFF;
#ifndef MAXSIM_DD_WAVES
#define MAXSIM_DD_WAVES 8
#endif
#ifndef MAXSIM_DD_UNROLL
#define MAXSIM_DD_UNROLL 2
#endif
constexpr int kDdUnroll = MAXSIM_DD_UNROLL;  // gathers in flight per lane
constexpr int kDdThreads = 1024;
constexpr int kWTab = 16384;  // per-(i,s) weights of one doc staged in LDS (64 KB)

// 8 consecutive elements (16 bytes) widened to fp32
template <int E> __device__ __forceinline__ void load8(const void* base, int64_t elem_off, float (&x)[8]);
template <> __device__ __forceinline__ void load8<kF16>(const void* base, int64_t off, float (&x)[8])
{
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    const h8 v = *(const h8*)((const _Float16*)base + off);
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = (float)v[k];
}
template <> __device__ __forceinline__ void load8<kBF16>(const void* base, int64_t off, float (&x)[8])
{
    const i32x4 v = *(const i32x4*)((const __bf16*)base + off);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t u = (uint32_t)v[k];
        x[2 * k] = __builtin_bit_cast(float, u << 16);
        x[2 * k + 1] = __builtin_bit_cast(float, u & 0xffff0000u);
    }
}

// gradient rows are written once and not read again here: streamed past the
// caches so that the gathered rows stay in L2
__device__ __forceinline__ void store8(float* p, const float (&a)[8])
{
    typedef float f4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store((f4){a[0], a[1], a[2], a[3]}, (f4*)p);
    __builtin_nontemporal_store((f4){a[4], a[5], a[6], a[7]}, (f4*)(p + 4));
}

// One lane's share of a row at any width: elements [e0, e0 + n) of a row,
// n in 0..8 (n < 8 only in the last 128-wide chunk of a row whose width is not
// a multiple of 128). `vec`: all 8 wanted and 16-byte aligned, one load.
template <int E> __device__ __forceinline__ float elem_f32(const void* base, int64_t off);
template <> __device__ __forceinline__ float elem_f32<kF16>(const void* base, int64_t off)
{
    return (float)((const _Float16*)base)[off];
}
template <> __device__ __forceinline__ float elem_f32<kBF16>(const void* base, int64_t off)
{
    return __builtin_bit_cast(float, (uint32_t)((const uint16_t*)base)[off] << 16);
}
template <int E>
__device__ __forceinline__ void loadn(const void* base, int64_t off, int n, bool vec, float (&x)[8])
{
    if (vec) {
        load8<E>(base, off, x);
        return;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = k < n ? elem_f32<E>(base, off + k) : 0.f;
}
__device__ __forceinline__ void storen(float* p, int n, bool vec, const float (&a)[8])
{
    if (vec) {
        store8(p, a);
        return;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
        if (k < n) __builtin_nontemporal_store(a[k], p + k);
}

// Lane l16's elements of 128-wide chunk c of a row of width dw.
struct LaneSpan {
    int e0, n;
    bool vec;
    __device__ __forceinline__ LaneSpan(int c, int l16, int64_t dw, bool gen)
    {
        e0 = c * 128 + 8 * l16;
        const int64_t left = dw - e0;
        n = !gen ? 8 : (left <= 0 ? 0 : (left >= 8 ? 8 : (int)left));
        vec = !gen || (n == 8 && (dw & 7) == 0);
    }
};

__device__ __forceinline__ uint64_t lanemask_lt() { return (1ull << lane_id()) - 1ull; }

__device__ __forceinline__ void barrier_lds()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// live(j): doc j has at least one valid token (always, without a d_mask,
// when Ld > 0); with t0 > 0, among tokens t0 and later. Computed by one wave.
__device__ __forceinline__ bool doc_live(const uint8_t* __restrict__ d_mask, int64_t j, int64_t Ld,
                                         int64_t t0 = 0)
{
    if (!d_mask) return Ld > 0;
    bool any = false;
    for (int64_t t = t0 + lane_id(); t < Ld; t += 64) {
        any = any || d_mask[j * Ld + t] != 0;
        if (__ballot(any) != 0) break;
    }
    return __ballot(any) != 0;
}

}  // namespace

// Doc-local sources k = i*Lq + s visited with a fixed stride: (i, s) is kept
// incrementally so that no division runs per source. Every index here is
// below Nq*Lq <= 2^31 - 1.
struct SrcWalk {
    uint32_t i, s, di, ds, Lq;
    __device__ __forceinline__ void init(uint32_t k, uint32_t stride, uint32_t lq)
    {
        Lq = lq;
        i = k / lq;
        s = k - i * lq;
        di = stride / lq;
        ds = stride - di * lq;
    }
    __device__ __forceinline__ void next()
    {
        i += di;
        s += ds;
        if (s >= Lq) {
            s -= Lq;
            ++i;
        }
    }
};

// Lanes of the wave (among those with `active`) whose key equals this lane's,
// from one ballot per key bit (keys < 2^10; bits that are 0 in every key
// leave the result unchanged).
__device__ __forceinline__ uint64_t match_key10(uint32_t key, bool active)
{
    uint64_t peers = __ballot(active);
#pragma unroll
    for (int b = 0; b < 10; ++b) {
        const bool bit = (key >> b) & 1u;
        const uint64_t bb = __ballot(bit);
        peers &= bit ? bb : ~bb;
    }
    return peers;
}

// The inverse map of one segment ("Flash-MaxSim" Sec. 4.2.2): nsrc sources,
// each with a destination in [0, L); row_ptr_seg[t] for t < L and the
// segment's col_idx entries starting at `carry`, each row listing its sources
// in ascending order. Run by a whole workgroup of kCsrWaves waves. Sources
// are taken in chunks of kCsrChunk; wave w owns the contiguous block
// [w*kPerWave, (w+1)*kPerWave) of a chunk and holds its destinations in
// registers (lane l, step m: source m*64 + l of the block), counted into the
// wave's own LDS histogram; the per-bin totals are scanned, and each wave
// scatters its block in source order with ranks from ballots over the key
// bits. Bins are handled in rounds of kCsrBins.
// load(k0, tv, sv) fills, for this lane, the destination tv[m] (any value:
// it is clamped into [0, L)) and the column-index value sv[m] of segment
// source k0 + 64 m (only called with k0 + 64 m < nsrc checked per m inside).
// Modes: kCsrFull builds the whole segment in one workgroup (bins in rounds);
// a segment too large for one workgroup is split over workgroups that each own
// one round [t_begin, t_begin + kCsrBins) of bins: kCsrCount writes that
// round's per-bin counts into row_ptr_seg, a scan over the segment turns them
// into row starts, and kCsrScatter then places the round's sources.
enum CsrMode { kCsrFull = 0, kCsrCount = 1, kCsrScatter = 2 };

// LDS of one CSR-building workgroup
struct CsrLds {
    uint32_t hist[kCsrWaves][kCsrBins];  // per-wave counts, then per-wave slots
    uint32_t run[kCsrBins];              // per-bin totals, then next free slot
    uint32_t wsum[kCsrWaves];
};

template <int MODE = kCsrFull, typename Load>
__device__ __forceinline__ void build_segment_csr(CsrLds& sm, int64_t nsrc, int64_t L, int64_t carry,
                                                  int32_t* __restrict__ row_ptr_seg,
                                                  int32_t* __restrict__ col_idx, Load&& load,
                                                  int64_t t_begin = 0)
{
    constexpr int kPerWave = kCsrChunk / kCsrWaves;  // 1024 sources of a chunk per wave
    constexpr int kSteps = kPerWave / 64;             // 16 per lane
    auto& hist = sm.hist;
    auto& run = sm.run;
    auto& wsum = sm.wsum;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int nchunks = (int)((nsrc + kCsrChunk - 1) / kCsrChunk);

    uint32_t key[kSteps];  // destination relative to the round, kNoKey outside it
    int32_t sv[kSteps];    // column-index value of each held source
    auto load_block = [&](int c, int64_t t_lo, int nb) {
        const int64_t k0 = (int64_t)c * kCsrChunk + (int64_t)wave * kPerWave + lane;
        int32_t tv[kSteps];
        load(k0, tv, sv);  // every load in flight before the first use
#pragma unroll
        for (int m = 0; m < kSteps; ++m) {
            key[m] = kNoKey;
            if (k0 + 64 * m < nsrc) {
                int64_t t = tv[m];
                t = t < 0 ? 0 : (t >= L ? L - 1 : t);  // precondition guard
                if (t >= t_lo && t < t_lo + nb) key[m] = (uint32_t)(t - t_lo);
            }
        }
    };
    // per-wave histogram of the block (counts do not depend on order)
    auto count_block = [&](int nb) {
        for (int k = lane; k < nb; k += 64) hist[wave][k] = 0;
        __builtin_amdgcn_s_waitcnt(0xC07F);
#pragma unroll
        for (int m = 0; m < kSteps; ++m)
            if (key[m] != kNoKey) atomicAdd(&hist[wave][key[m]], 1u);
    };
    const int64_t t_end = MODE == kCsrFull ? L : (t_begin + kCsrBins < L ? t_begin + kCsrBins : L);
    for (int64_t t_lo = t_begin; t_lo < t_end; t_lo += kCsrBins) {
        const int nb = (int)(L - t_lo < kCsrBins ? L - t_lo : kCsrBins);

        if constexpr (MODE == kCsrScatter) {
            // row starts of this round, from the count pass and the scan
            for (int k = tid; k < nb; k += kCsrThreads) run[k] = (uint32_t)row_ptr_seg[t_lo + k];
            if (nchunks == 1) {  // the scatter below expects the block in registers
                barrier_lds();
                load_block(0, t_lo, nb);
                count_block(nb);
            }
        } else {
            // ---- totals per bin over every chunk ----------------------------
            for (int k = tid; k < nb; k += kCsrThreads) run[k] = 0;
            for (int c = 0; c < nchunks; ++c) {
                barrier_lds();
                load_block(c, t_lo, nb);
                count_block(nb);
                barrier_lds();
                for (int k = tid; k < nb; k += kCsrThreads) {
                    uint32_t tot = 0;
                    for (int w = 0; w < kCsrWaves; ++w) tot += hist[w][k];
                    run[k] += tot;
                }
            }
            barrier_lds();
            if constexpr (MODE == kCsrCount) {
                for (int k = tid; k < nb; k += kCsrThreads) row_ptr_seg[t_lo + k] = (int32_t)run[k];
                return;
            }

            // ---- exclusive scan of the totals -> row_ptr, first slot per bin
            // (nb <= kCsrThreads: one bin per thread)
            const uint32_t mine = tid < nb ? run[tid] : 0u;
            uint32_t incl = mine;
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t v = __shfl_up(incl, off, 64);
                if (lane >= off) incl += v;
            }
            if (lane == 63) wsum[wave] = incl;
            barrier_lds();
            uint32_t wave_off = 0, round_tot = 0;
            for (int w = 0; w < kCsrWaves; ++w) {
                if (w < wave) wave_off += wsum[w];
                round_tot += wsum[w];
            }
            if (tid < nb) {
                const int64_t first = carry + wave_off + incl - mine;
                row_ptr_seg[t_lo + tid] = (int32_t)first;
                run[tid] = (uint32_t)first;
            }
            carry += round_tot;
        }

        // ---- stable scatter, chunk by chunk, in source order ----------------
        for (int c = 0; c < nchunks; ++c) {
            if (nchunks > 1) {  // the only chunk's block is still in registers
                barrier_lds();
                load_block(c, t_lo, nb);
                count_block(nb);
            }
            barrier_lds();
            // slots: bin k of wave w starts after the earlier waves' sources of bin k
            for (int k = tid; k < nb; k += kCsrThreads) {
                uint32_t pos = run[k];
                for (int w = 0; w < kCsrWaves; ++w) {
                    const uint32_t h = hist[w][k];
                    hist[w][k] = pos;
                    pos += h;
                }
                run[k] = pos;
            }
            barrier_lds();
#pragma unroll
            for (int m = 0; m < kSteps; ++m) {
                const bool act = key[m] != kNoKey;
                if (__ballot(act) == 0) continue;  // uniform
                const uint64_t peers = match_key10(key[m], act);
                if (act) {
                    const uint64_t before = peers & lanemask_lt();
                    const uint32_t slot = hist[wave][key[m]] + (uint32_t)__builtin_popcountll(before);
                    col_idx[slot] = sv[m];
                    if (before == 0) hist[wave][key[m]] += (uint32_t)__builtin_popcountll(peers);
                }
            }
        }
        barrier_lds();
    }
}

// LDS of a workgroup that builds a small segment's map in one pass
struct CsrSmallLds {
    uint32_t hist[kCsrWaves][kCsrBins];  // per-wave counts, then per-wave slots
    uint32_t wsum[kCsrWaves];
    uint64_t grp[kCsrWaves][64];         // per wave: lanes holding equal keys, by representative lane
    uint8_t owner[kCsrWaves][kCsrBins];  // per wave: representative lane of each key of a step
    int32_t stage[kCsrChunk];            // the segment's col_idx entries, in place
};

// One pass over a block of at most kCsrWaves * 64 * STEPS sources (STEPS per
// lane, one register block per wave) with destinations in [0, L), L <= kCsrBins: loads them, ranks each
// source among the equal destinations of its wave's step, and counts them
// into the waves' LDS histograms. Equal destinations within a step are found
// through LDS instead of ballots over the key bits: every lane writes its
// lane number into owner[key], so each group of equal keys reads back one
// member as its representative, and an atomic OR of the lanes' bits into
// grp[representative] gives each lane the set of its group (OR is order
// free, so the set does not depend on which member won the write). A lane's
// rank is the number of group members below it, and the lowest member adds
// the group's size to the wave's histogram, so a row that receives many
// sources costs no more than any other. On return (after a barrier)
// key[m] = destination | rank << 16 | (group size << 24 in the lowest
// member), or kNoKey past the block's end, and sv[m] is the source's value.
template <int STEPS, typename Load>
__device__ __forceinline__ void rank_block(CsrSmallLds& sm, int64_t nsrc, int64_t L, Load&& load,
                                           uint32_t (&key)[STEPS], int32_t (&sv)[STEPS])
{
    constexpr int kSteps = STEPS;
    constexpr int kPerWave = 64 * STEPS;
    const int tid = (int)threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int64_t k0 = (int64_t)wave * kPerWave + lane;
    int32_t tv[kSteps];
    load(k0, tv, sv);  // every load in flight before the first use
    for (int k = lane; k < L; k += 64) sm.hist[wave][k] = 0;
    sm.grp[wave][lane] = 0;
#pragma unroll
    for (int m = 0; m < kSteps; ++m) {
        key[m] = kNoKey;
        if (k0 + 64 * m < nsrc) {
            int64_t t = tv[m];
            t = t < 0 ? 0 : (t >= L ? L - 1 : t);  // precondition guard
            key[m] = (uint32_t)t;
        }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // the zeroing lands before the counts
    // a wave's LDS operations complete in issue order, so each read below
    // sees the writes issued before it; the owner and group reads are
    // volatile: they must return what the other lanes wrote, not what this
    // lane stored a moment before
    const uint64_t me = 1ull << lane;
    typedef __attribute__((address_space(3))) volatile uint8_t lds_u8;
    typedef __attribute__((address_space(3))) volatile uint64_t lds_u64;
    lds_u8* owner = (lds_u8*)sm.owner[wave];
    lds_u64* grp = (lds_u64*)sm.grp[wave];
#pragma unroll
    for (int m = 0; m < kSteps; ++m) {
        const bool act = key[m] != kNoKey;
        if (__ballot(act) == 0) continue;  // uniform
        if (act) owner[key[m]] = (uint8_t)lane;
        const uint32_t rep = act ? owner[key[m]] : 0u;
        if (act) atomicOr(&sm.grp[wave][rep], me);
        const uint64_t peers = act ? grp[rep] : 0ull;
        const uint32_t rank = (uint32_t)__builtin_popcountll(peers & (me - 1ull));
        const uint32_t n = (uint32_t)__builtin_popcountll(peers);
        const bool lead = act && rank == 0;
        if (lead) {
            atomicAdd(&sm.hist[wave][key[m]], n);  // one lane per key
            grp[rep] = 0;                          // free for the next step
        }
        key[m] |= (rank << 16) | (lead ? n << 24 : 0u);  // 0 for an inactive lane
    }
    barrier_lds();
}

// Exclusive scan of the block's per-row totals (one row per thread, rows
// [0, L)), then per-wave first slots in sm.hist: row r of wave w starts after
// the earlier rows and the earlier waves' sources of row r. Returns this
// thread's row's first slot and total (0 past L); the slots are block-local.
__device__ __forceinline__ void block_slots(CsrSmallLds& sm, int64_t L, uint32_t& first, uint32_t& total)
{
    const int tid = (int)threadIdx.x, wave = tid >> 6, lane = tid & 63;
    uint32_t mine = 0;
    if (tid < L)
        for (int w = 0; w < kCsrWaves; ++w) mine += sm.hist[w][tid];
    uint32_t incl = mine;
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
    }
    if (lane == 63) sm.wsum[wave] = incl;
    barrier_lds();
    uint32_t wave_off = 0;
    for (int w = 0; w < wave; ++w) wave_off += sm.wsum[w];
    first = wave_off + incl - mine;
    total = mine;
    if (tid < L) {
        uint32_t pos = first;
        for (int w = 0; w < kCsrWaves; ++w) {
            const uint32_t h = sm.hist[w][tid];
            sm.hist[w][tid] = pos;
            pos += h;
        }
    }
    barrier_lds();
}

// Each ranked source into sm.stage at its block-local slot, in source order
// within every row.
template <int STEPS>
__device__ __forceinline__ void stage_block(CsrSmallLds& sm, const uint32_t (&key)[STEPS], const int32_t (&sv)[STEPS])
{
    const int wave = (int)threadIdx.x >> 6;
#pragma unroll
    for (int m = 0; m < STEPS; ++m) {
        if (key[m] != kNoKey) {
            const uint32_t t = key[m] & 0xFFFFu, rank = (key[m] >> 16) & 0xFFu;
            sm.stage[sm.hist[wave][t] + rank] = sv[m];
            if (rank == 0) sm.hist[wave][t] += key[m] >> 24;
        }
    }
    barrier_lds();
}

// The inverse map of a segment small enough for one pass (the same map as
// build_segment_csr): nsrc <= kCsrChunk sources and L <= kCsrBins rows. The
// sources are ranked (rank_block), the row totals scanned into row_ptr, the
// sources placed in source order into `stage` (LDS), and the segment written
// out in one contiguous run.
template <typename Load>
__device__ __forceinline__ void build_csr_small(CsrSmallLds& sm, int64_t nsrc, int64_t L, int64_t carry,
                                                int32_t* __restrict__ row_ptr_seg,
                                                int32_t* __restrict__ col_idx, Load&& load)
{
    constexpr int kSteps = kCsrChunk / kCsrWaves / 64;
    const int tid = (int)threadIdx.x;
    uint32_t key[kSteps];
    int32_t sv[kSteps];
    rank_block<kSteps>(sm, nsrc, L, load, key, sv);
    uint32_t first, total;
    block_slots(sm, L, first, total);
    if (tid < L) row_ptr_seg[tid] = (int32_t)(carry + first);
    stage_block<kSteps>(sm, key, sv);
    for (int64_t e = tid; e < nsrc; e += kCsrThreads) col_idx[carry + e] = sm.stage[e];
}

// One chunk of a stable partition by row in one pass: the chunk's sources
// (nsrc <= kCsrWaves * 64 * STEPS) with rows in [0, L), L <= kCsrBins. COUNT writes the
// chunk's per-row counts to row_arr[r]; otherwise row_arr[r] holds the
// absolute first slot of the chunk's run in row r (from the scan over the
// chunks), and each source goes to out at its run's slot in source order,
// every run written contiguously. Slots are kept below out_len for any
// row_arr content.
template <bool COUNT, int STEPS, typename Load>
__device__ __forceinline__ void place_small(CsrSmallLds& sm, int64_t nsrc, int64_t L, int32_t* __restrict__ row_arr,
                                            int32_t* __restrict__ out, int64_t out_len, Load&& load)
{
    const int tid = (int)threadIdx.x, wave = tid >> 6, lane = tid & 63;
    uint32_t key[STEPS];
    int32_t sv[STEPS];
    rank_block<STEPS>(sm, nsrc, L, load, key, sv);
    uint32_t first, total;
    block_slots(sm, L, first, total);
    if constexpr (COUNT) {
        if (tid < L) row_arr[tid] = (int32_t)total;
        return;
    }
    // the rows' block-local starts and sizes, in the owner area (free now)
    uint32_t* rstart = (uint32_t*)&sm.owner[0][0];
    uint32_t* rsize = rstart + kCsrBins;
    if (tid < L) {
        rstart[tid] = first;
        rsize[tid] = total;
    }
    stage_block<STEPS>(sm, key, sv);  // ends with a barrier
    for (int64_t r = wave; r < L; r += kCsrWaves) {
        const uint32_t n = rsize[r], s0 = rstart[r];
        const int64_t d0 = row_arr[r];
        for (uint32_t i = lane; i < n; i += 64) {
            const int64_t d = d0 + i;
            if (d >= 0 && d < out_len) out[d] = sm.stage[s0 + i];
        }
    }
}

// Sources of doc j for the CSR builders: doc-local source k = i*Lq + s is
// the flat source (i*Nd + j)*Lq + s.
struct DocSources {
    const int32_t* argmax;
    uint32_t Lq, nd, j, per_doc;
    __device__ __forceinline__ void operator()(int64_t k0, int32_t (&tv)[16], int32_t (&sv)[16]) const
    {
        SrcWalk w;
        w.init((uint32_t)k0, 64, Lq > 0 ? Lq : 1u);
#pragma unroll
        for (int m = 0; m < 16; ++m, w.next()) {
            const bool ok = k0 + 64 * m < per_doc;
            const uint32_t src = ok ? (w.i * nd + j) * Lq + w.s : 0u;
            sv[m] = (int32_t)src;
            tv[m] = ok ? __builtin_nontemporal_load(argmax + src) : 0;
        }
    }
};

// Inverse map of doc j: row_ptr[j*Ld + t] and the doc's segment
// col_idx[j*Nq*Lq, (j+1)*Nq*Lq). Every doc receives exactly Nq*Lq sources,
// so no global scan is needed.
__device__ __forceinline__ void csr_doc(const BwdArgs& a, CsrLds& sm, uint32_t j)
{
    const uint32_t per_doc = (uint32_t)(a.Nq * a.Lq);
    const DocSources load{a.argmax, (uint32_t)a.Lq, (uint32_t)a.Nd, j, per_doc};
    build_segment_csr(sm, per_doc, a.Ld, (int64_t)j * per_doc, a.row_ptr + (int64_t)j * a.Ld, a.col_idx, load);
}

// The same map for a doc small enough for the one-pass builder
// (Nq*Lq <= kCsrChunk, Ld <= kCsrBins).
__device__ __forceinline__ void csr_doc_small(const BwdArgs& a, CsrSmallLds& sm, uint32_t j)
{
    const uint32_t per_doc = (uint32_t)(a.Nq * a.Lq);
    const DocSources load{a.argmax, (uint32_t)a.Lq, (uint32_t)a.Nd, j, per_doc};
    build_csr_small(sm, per_doc, a.Ld, (int64_t)j * per_doc, a.row_ptr + (int64_t)j * a.Ld, a.col_idx, load);
}

// LDS of a dq workgroup with G row groups
template <int G> struct DqLds {
    int32_t am[kDqDocs][G];  // argmax[i, j0 + jj, s0 + g]
    float wj[kDqDocs];       // g[i, j0 + jj] * live(j0 + jj)
};

// Eq. (2): dQ[i,s] = q_mask[i,s] * sum_j g[i,j] live(j) D[j, argmax[i,j,s]].
// Workgroup `blk` = query i and G rows s; group g owns row s0 + g, lane l16
// owns dims 8*l16 .. 8*l16+7 of each 128-wide chunk of the row (GEN: any
// width, the chunks taken one after another). live(j) = any(d_mask[j,:]) is
// found by the workgroup's waves while it stages the doc's weight (one early-
// exit scan of the mask row per doc).
template <int E, bool GEN, int G>
__device__ __forceinline__ void dq_block(const BwdArgs& a, DqLds<G>& sm, int64_t blk)
{
    constexpr int kThreads = 16 * G, kWavesB = kThreads / 64;
    const int64_t Nd = a.Nd, Lq = a.Lq, Ld = a.Ld;
    const int64_t DW = GEN ? (int64_t)a.d : kD;
    const int nchunk = GEN ? (int)((DW + 127) / 128) : 1;
    // blocks go query-minor: the first G rows of every query come first, so
    // that the row blocks most likely to be unmasked (masks usually cut a
    // query's tail) start before the lighter ones
    const int64_t i = blk % a.Nq;
    const int64_t s0 = (blk / a.Nq) * G;
    const int tid = threadIdx.x, grp = tid >> 4, l16 = tid & 15, wave = tid >> 6;
    const int64_t s = s0 + grp;
    const bool row_ok = s < Lq;
    // a masked row's gradient is 0 (written below); its gathers are skipped
    const bool row_live = row_ok && !(a.q_mask && a.q_mask[i * Lq + s] == 0);
    const bool o32 = !GEN && (uint64_t)kDqDocs * (uint64_t)Ld * (kD * sizeof(uint16_t)) <= 0xFFFFFFFFull;

    for (int c = 0; c < nchunk; ++c) {
        const LaneSpan ls(c, l16, DW, GEN);
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int64_t j0 = 0; j0 < Nd; j0 += kDqDocs) {
            const int nj = (int)(Nd - j0 < kDqDocs ? Nd - j0 : kDqDocs);
            barrier_lds();
            // the argmax entries and weights of the batch, every load issued
            // before any is used (out-of-range slots read entry 0)
            constexpr int kPer = kDqDocs * G / kThreads;
            constexpr int kPerW = (kDqDocs + kWavesB - 1) / kWavesB;
            const int lane = tid & 63;
            int32_t tv[kPer];
#pragma unroll
            for (int u = 0; u < kPer; ++u) {
                const int e = tid + u * kThreads, jj = e / G, gg = e % G;
                const bool ok = jj < nj && s0 + gg < Lq;
                tv[u] = a.argmax[ok ? (i * Nd + j0 + jj) * Lq + s0 + gg : 0];
            }
            float gv[kPerW];
            uint8_t m0[kPerW];
            // the mask test sits outside the loads (a branch between two
            // loads makes the second wait for the first)
            auto load_w = [&](auto has_mask) {
#pragma unroll
                for (int u = 0; u < kPerW; ++u) {
                    const int jj = wave + u * kWavesB;
                    const int64_t j = j0 + (jj < nj ? jj : 0);
                    gv[u] = a.g[i * Nd + j];
                    if constexpr (decltype(has_mask)::value) m0[u] = a.d_mask[j * Ld + (lane < Ld ? lane : 0)];
                    else m0[u] = 1;
                }
            };
            if (a.d_mask) load_w(std::true_type{});
            else load_w(std::false_type{});
#pragma unroll
            for (int u = 0; u < kPer; ++u) {
                const int e = tid + u * kThreads, jj = e / G, gg = e % G;
                int32_t t = 0;
                if (jj < nj && s0 + gg < Lq) {
                    t = tv[u];
                    t = t < 0 ? 0 : (t >= Ld ? (int32_t)(Ld - 1) : t);  // precondition guard
                }
                sm.am[jj][gg] = t;
            }
#pragma unroll
            for (int u = 0; u < kPerW; ++u) {
                const int jj = wave + u * kWavesB;  // uniform over the wave
                if (jj < nj) {
                    bool live = Ld > 0;
                    if (a.d_mask) {
                        live = __ballot(lane < Ld && m0[u] != 0) != 0;  // the first 64 tokens
                        if (!live && Ld > 64) live = doc_live(a.d_mask, j0 + jj, Ld, 64);
                    }
                    if (lane == 0) sm.wj[jj] = gv[u] * (live ? 1.f : 0.f);
                }
            }
            barrier_lds();
            if (!row_live || ls.n == 0) continue;
            const int64_t dbase = (j0 * Ld) * DW + ls.e0;
            // d = 128 and a batch's docs under 4 GiB: a gather is the batch's
            // uniform base plus a 32-bit byte offset
            const unsigned char* batch = (const unsigned char*)a.D + (size_t)(j0 * Ld) * (kD * sizeof(uint16_t));
            const uint32_t lane_b = (uint32_t)ls.e0 * (uint32_t)sizeof(uint16_t);
            auto gather = [&](int jr, int t, float (&x)[8]) {
                if (!GEN && o32)
                    load8<E>(batch + (((uint32_t)jr * (uint32_t)Ld + (uint32_t)t) * (uint32_t)(kD * sizeof(uint16_t)) + lane_b), 0, x);
                else
                    loadn<E>(a.D, dbase + ((int64_t)jr * Ld + t) * DW, ls.n, ls.vec, x);
            };
            int jj = 0;
            for (; jj + 8 <= nj; jj += 8) {
                float x[8][8];
#pragma unroll
                for (int u = 0; u < 8; ++u) gather(jj + u, sm.am[jj + u][grp], x[u]);
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float w = sm.wj[jj + u];
#pragma unroll
                    for (int k = 0; k < 8; ++k) acc[k] = __builtin_fmaf(w, x[u][k], acc[k]);
                }
            }
            for (; jj < nj; ++jj) {
                float x[8];
                gather(jj, sm.am[jj][grp], x);
                const float w = sm.wj[jj];
#pragma unroll
                for (int k = 0; k < 8; ++k) acc[k] = __builtin_fmaf(w, x[k], acc[k]);
            }
        }
        if (row_ok && ls.n > 0) storen(a.dQ + (i * Lq + s) * DW + ls.e0, ls.n, ls.vec, acc);
    }
}

// The CSR and the dQ gathers in one launch (neither needs the other):
// workgroups [0, Nd) build doc blockIdx's CSR, the rest are dq workgroups of
// 64 query rows, which fill the CUs the Nd CSR workgroups leave idle. The two
// kinds share one LDS allocation.
template <int E, bool GEN>
__global__ __launch_bounds__(kCsrThreads) void csr_dq_kernel(BwdArgs a, int64_t csr_blocks)
{
    // the general-width instances keep the ballot builder only: with their
    // wider dq state the one-pass builder's larger LDS block made their
    // registers spill
    __shared__ union {
        CsrLds csr;
        typename std::conditional<GEN, CsrLds, CsrSmallLds>::type small;
        DqLds<kCsrThreads / 16> dq;
    } sm;
    const int64_t b = blockIdx.x;
    if (b < csr_blocks) {
        bool done = false;
        if constexpr (!GEN) {
            if (a.Nq * a.Lq <= kCsrChunk && a.Ld <= kCsrBins) {
                csr_doc_small(a, sm.small, (uint32_t)b);
                done = true;
            }
        }
        if (!done) csr_doc(a, sm.csr, (uint32_t)b);
        if (b == a.Nd - 1 && threadIdx.x == 0) a.row_ptr[a.Nd * a.Ld] = (int32_t)(a.Nq * a.Nd * a.Lq);
    } else {
        dq_block<E, GEN, kCsrThreads / 16>(a, sm.dq, b - csr_blocks);
    }
}

// Eq. (3): dD[j,t] = sum over the CSR row of (j,t), in order, of
// w(i,j,s) Q[i,s] with w = g[i,j] q_mask[i,s] live(j). Workgroup = doc j and
// a block of its rows; group g owns rows t_begin + g + 64*k, lane l16 owns
// dims 8*l16 .. 8*l16+7. TAB: the doc's weights w for every (i,s) are staged
// in LDS first (Nq*Lq <= kWTab), so a source costs one CSR read and one
// gather; otherwise w is read from g and q_mask per source. O32 (d = 128 and
// Q under 4 GiB): a source is handed from its decoding lane to its group as
// the 32-bit byte offset of its Q row, and each lane adds its own 16 bytes,
// so a gather needs no 64-bit address arithmetic.
template <int E, bool TAB, bool GEN, bool O32>
__global__ __launch_bounds__(kDdThreads) __attribute__((amdgpu_waves_per_eu(MAXSIM_DD_WAVES))) void dd_kernel(
    BwdArgs a, int rows_per_block)
{
    static_assert(!(O32 && GEN), "32-bit offsets only for 128-wide rows");
    __shared__ float wtab[TAB ? kWTab : 1];
    // per 16-lane group: the current batch's sources of nonzero weight, in order
    struct SrcEntry {
        int q;    // Q row, or (O32) its byte offset
        float w;
    };
    __shared__ SrcEntry srcq[kDdThreads / 16][16];
    const int64_t Nd = a.Nd, Lq = a.Lq, Ld = a.Ld;
    const int64_t DW = GEN ? (int64_t)a.d : kD;
    const int nchunk = GEN ? (int)((DW + 127) / 128) : 1;
    const int64_t blocks_per_doc = (Ld + rows_per_block - 1) / rows_per_block;
    const int64_t j = blockIdx.x / blocks_per_doc;
    const int64_t t_begin = (blockIdx.x % blocks_per_doc) * rows_per_block;
    const int64_t t_end = t_begin + rows_per_block < Ld ? t_begin + rows_per_block : Ld;
    const int tid = threadIdx.x, grp = tid >> 4, l16 = tid & 15;
    const int gbase = tid & 63 & ~15;  // first lane of the group within the wave
    const bool live = doc_live(a.d_mask, j, Ld);
    constexpr int kDdGroups = kDdThreads / 16;

    if constexpr (TAB) {
        const int64_t nqr = a.Nq * Lq;
        // kWTab / kDdThreads entries per thread, every load issued before any
        // is used (indices past the end read entry 0); the mask test sits
        // outside the loads, since a branch between two loads makes the
        // second wait for the first
        auto stage = [&](auto has_mask) {
            constexpr bool kMask = decltype(has_mask)::value;
            constexpr int kW = kWTab / kDdThreads;
            SrcWalk w;
            w.init(tid, kDdThreads, Lq);
            float gk[kW];
            uint8_t qm[kW];
#pragma unroll
            for (int u = 0; u < kW; ++u, w.next()) {
                const int64_t k = tid + (int64_t)u * kDdThreads;
                const bool ok = k < nqr;
                gk[u] = a.g[(ok ? (int64_t)w.i : 0) * Nd + j];
                if constexpr (kMask) qm[u] = a.q_mask[ok ? k : 0];
            }
#pragma unroll
            for (int u = 0; u < kW; ++u) {
                const int64_t k = tid + (int64_t)u * kDdThreads;
                if (k < nqr) wtab[k] = kMask && qm[u] == 0 ? 0.f : gk[u];
            }
        };
        if (live && nqr > 0) {
            if (a.q_mask) stage(std::true_type{});
            else stage(std::false_type{});
        }
        barrier_lds();
    }

    // a source index src = (i*Nd + j)*Lq + s of this doc gives
    // src - j*Lq = i*(Nd*Lq) + s
    const uint32_t ndlq = (uint32_t)(Nd * Lq), jlq = (uint32_t)(j * Lq);
    const uint32_t nq = (uint32_t)a.Nq, lq = (uint32_t)Lq;
    for (int64_t t = t_begin + grp; t < t_end; t += kDdGroups)
    for (int c = 0; c < nchunk; ++c) {
        const LaneSpan ls(c, l16, DW, GEN);
        const int64_t row = j * Ld + t;
        const uint32_t e0b = (uint32_t)ls.e0 * (uint32_t)sizeof(uint16_t);  // this lane's bytes of a row (O32)
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        // the source handed to the group: Q row index, or its byte offset (O32)
        auto gather = [&](int qr, float (&xv)[8]) {
            if constexpr (O32) load8<E>((const unsigned char*)a.Q + ((uint32_t)qr + e0b), 0, xv);
            else loadn<E>(a.Q, (int64_t)qr * DW + ls.e0, ls.n, ls.vec, xv);
        };
        if (live) {
            const int e0 = a.row_ptr[row], e1 = a.row_ptr[row + 1];
            for (int e = e0; e < e1; e += 16) {
                const int cnt = e1 - e < 16 ? e1 - e : 16;
                int qrow = 0;
                float w = 0.f;
                if (l16 < cnt) {
                    const uint32_t x = (uint32_t)a.col_idx[e + l16] - jlq;
                    uint32_t i = x / ndlq;
                    uint32_t s = x - i * ndlq;
                    // in range for any CSR content (guards the gathers)
                    i = i < nq ? i : nq - 1;
                    s = s < lq ? s : lq - 1;
                    qrow = (int)(i * lq + s);
                    if constexpr (TAB) {
                        w = wtab[qrow];
                    } else {
                        w = a.g[(int64_t)i * Nd + j];
                        if (a.q_mask && a.q_mask[qrow] == 0) w = 0.f;
                    }
                }
                // only the sources with a nonzero weight are gathered, in
                // CSR order (a zero-weight term adds an exact zero, the
                // inputs being finite): each such lane puts its source at its
                // rank among them into the group's LDS list, which the group
                // then reads in order (a lane's own slot is the only one it
                // writes; LDS operations of a wave are in order)
                if constexpr (O32) qrow = (int)((uint32_t)qrow * (uint32_t)(kD * sizeof(uint16_t)));
                const bool keep = l16 < cnt && w != 0.f;
                const uint32_t gm = (uint32_t)(__ballot(keep) >> gbase) & 0xffffu;
                const int nz = __builtin_popcount(gm);
                if (keep) srcq[grp][__builtin_popcount(gm & ((1u << l16) - 1u))] = SrcEntry{qrow, w};
                int k = 0;
                for (; k + kDdUnroll <= nz; k += kDdUnroll) {
                    float xv[kDdUnroll][8];
                    float ww[kDdUnroll];
#pragma unroll
                    for (int u = 0; u < kDdUnroll; ++u) {
                        const SrcEntry se = srcq[grp][k + u];
                        ww[u] = se.w;
                        gather(se.q, xv[u]);
                    }
#pragma unroll
                    for (int u = 0; u < kDdUnroll; ++u)
#pragma unroll
                        for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(ww[u], xv[u][q], acc[q]);
                }
                for (; k < nz; ++k) {
                    const SrcEntry se = srcq[grp][k];
                    float xv[8];
                    gather(se.q, xv);
#pragma unroll
                    for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(se.w, xv[q], acc[q]);
                }
            }
        }
        if (ls.n > 0) storen(a.dD + row * DW + ls.e0, ls.n, ls.vec, acc);
    }
}

template <int E, bool GEN>
static hipError_t launch_bwd_t(BwdArgs a, hipStream_t stream)
{
    hipError_t err;
    // CSR of every doc and dQ (zeros when there are no docs) in one launch
    constexpr int64_t kDqRows = kCsrThreads / 16;
    const int64_t csr_blocks = a.Nd;
    const int64_t dq_blocks = a.Nq * a.Lq > 0 ? a.Nq * ((a.Lq + kDqRows - 1) / kDqRows) : 0;
    if (csr_blocks + dq_blocks > 0) {
        hipLaunchKernelGGL((csr_dq_kernel<E, GEN>), dim3((unsigned)(csr_blocks + dq_blocks)), dim3(kCsrThreads), 0,
                           stream, a, csr_blocks);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (a.Nd > 0 && a.Ld > 0) {
        // about two workgroups per CU, whole 64-row steps, within one doc
        const int64_t rows = a.Nd * a.Ld;
        int64_t rpb = (rows + 2 * (int64_t)device_cu_count() - 1) / (2 * (int64_t)device_cu_count());
        rpb = (rpb + 63) / 64 * 64;
        if (rpb > a.Ld) rpb = (a.Ld + 63) / 64 * 64;
        if (rpb > 4096) rpb = 4096;
        const int64_t blocks = a.Nd * ((a.Ld + rpb - 1) / rpb);
        // Q rows addressed by 32-bit byte offsets when Q is under 4 GiB
        constexpr bool kO32 = !GEN;
        const bool o32 = kO32 && a.Nq * a.Lq <= (int64_t)(0xFFFFFFFFu / (kD * sizeof(uint16_t)));
        const dim3 grid((unsigned)blocks), block(kDdThreads);
        if (a.Nq * a.Lq <= kWTab) {
            if (o32) hipLaunchKernelGGL((dd_kernel<E, true, GEN, kO32>), grid, block, 0, stream, a, (int)rpb);
            else hipLaunchKernelGGL((dd_kernel<E, true, GEN, false>), grid, block, 0, stream, a, (int)rpb);
        } else {
            if (o32) hipLaunchKernelGGL((dd_kernel<E, false, GEN, kO32>), grid, block, 0, stream, a, (int)rpb);
            else hipLaunchKernelGGL((dd_kernel<E, false, GEN, false>), grid, block, 0, stream, a, (int)rpb);
        }
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    return hipSuccess;
}

hipError_t launch_bwd(int elem, BwdArgs a, hipStream_t stream)
{
    const bool gen = a.d != kD;
    switch (elem) {
    case kF16: return gen ? launch_bwd_t<kF16, true>(a, stream) : launch_bwd_t<kF16, false>(a, stream);
    case kBF16: return gen ? launch_bwd_t<kBF16, true>(a, stream) : launch_bwd_t<kBF16, false>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

// ===========================================================================
// Padding-free backward ("Flash-MaxSim" Sec. 4.2.1-4.2.3 on the cu_seqlens
// layout of Sec. 4.3.2; design notes "Varlen / packed path"). Query i is
// packed rows [cu_q[i], cu_q[i+1]) and doc j rows [cu_d[j], cu_d[j+1]); the
// argmax is the packed forward's [Nq, Nd, max_lq] doc-relative map. The
// sources are the Tq packed query rows for every doc that has a token (an
// empty doc has no destination and no gradient), so every such doc's CSR
// segment holds Tq entries and starts at Tq * (docs with a token before it).
//
//   prep  one workgroup: that segment start for every doc with a token,
//         parked in the first element of the doc's first dD row (dD is
//         written last), and row_ptr[Td];
//   csr   one workgroup per doc, as the padded kernel: destinations of a
//         block of sources per wave in registers, per-wave LDS histograms,
//         scan, stable scatter with ballot ranks. Source p (a packed query
//         row) belongs to the query found by a search of cu_q once per lane,
//         then by walking forward as p grows;
//   dq    16 packed query rows per workgroup, a 16-lane group per row; the
//         argmax entries, doc offsets and weights of 64 docs at a time are
//         staged in LDS, then each group gathers its D rows in doc order;
//   dd    a 16-lane group per packed doc row walks its CSR row in order and
//         gathers Q rows; every row is written once.
// No atomics on results; results are bitwise reproducible.
// ===========================================================================

namespace {

// largest b in [0, n) with cu[b] <= p (cu non-decreasing, cu[0] = 0 <= p)
__device__ __forceinline__ int seg_of(const int32_t* __restrict__ cu, int n, int64_t p)
{
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)cu[mid] <= p) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

constexpr int kPrepThreads = 1024;

}  // namespace

__global__ __launch_bounds__(kPrepThreads) void vbwd_prep_kernel(VarBwdArgs a)
{
    __shared__ uint32_t part[kPrepThreads];
    const int tid = threadIdx.x;
    const int64_t Nd = a.Nd, Td = a.Td;
    const int64_t chunk = (Nd + kPrepThreads - 1) / kPrepThreads;
    const int64_t j0 = tid * chunk, j1 = j0 + chunk < Nd ? j0 + chunk : Nd;
    uint32_t live = 0;
    for (int64_t j = j0; j < j1; ++j) live += a.cu_d[j + 1] > a.cu_d[j] ? 1u : 0u;
    part[tid] = live;
    barrier_lds();
    // exclusive scan of the per-thread counts (Hillis-Steele in LDS)
    for (int off = 1; off < kPrepThreads; off <<= 1) {
        const uint32_t v = tid >= off ? part[tid - off] : 0u;
        barrier_lds();
        part[tid] += v;
        barrier_lds();
    }
    uint32_t before = part[tid] - live;
    for (int64_t j = j0; j < j1; ++j) {
        const int64_t r = a.cu_d[j];
        if (a.cu_d[j + 1] > r) {
            if (r >= 0 && r < Td) a.dD[r * a.d] = __builtin_bit_cast(float, (uint32_t)((int64_t)before * a.Tq));
            ++before;
        }
    }
    if (tid == kPrepThreads - 1) a.row_ptr[Td] = (int32_t)((int64_t)part[tid] * a.Tq);
}

// CSR of doc j: row_ptr[cu_d[j] + t] and the doc's col_idx segment, whose
// start the prep pass parked in dD. Source p (a packed query row) belongs to
// the query found by a search of cu_q once per lane, then by walking forward
// as p grows.
// SMALL: a doc with at most kCsrBins rows is built by the one-pass builder
// when the segment has at most kCsrChunk sources.
template <bool SMALL, typename SmallLds>
__device__ __forceinline__ void vbwd_csr_doc(const VarBwdArgs& a, CsrLds& sm, SmallLds& small, int64_t j)
{
    const int64_t Nd = a.Nd, Tq = a.Tq;
    const int64_t d0 = a.cu_d[j];
    int64_t L = (int64_t)a.cu_d[j + 1] - d0;
    if (d0 < 0 || d0 >= a.Td) return;  // empty doc (or broken offsets)
    if (L > a.Td - d0) L = a.Td - d0;
    if (L <= 0) return;
    const uint32_t mlq = (uint32_t)a.max_lq, nd = (uint32_t)Nd;
    const int nq = (int)a.Nq;
    auto load = [&](int64_t p0, int32_t (&tv)[16], int32_t (&sv)[16]) {
        int i = p0 < Tq ? seg_of(a.cu_q, nq + 1, p0) : 0;
        i = i < nq ? i : nq - 1;  // precondition guard (cu_q[Nq] == Tq)
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int64_t p = p0 + 64 * m;
            sv[m] = 0;
            tv[m] = 0;
            if (p < Tq) {
                while (i + 1 < nq && (int64_t)a.cu_q[i + 1] <= p) ++i;
                int64_t s = p - a.cu_q[i];
                s = s < 0 ? 0 : (s >= mlq ? mlq - 1 : s);  // precondition guard
                const uint32_t src = ((uint32_t)i * nd + (uint32_t)j) * mlq + (uint32_t)s;
                sv[m] = (int32_t)src;
                tv[m] = __builtin_nontemporal_load(a.argmax + src);
            }
        }
    };
    const int64_t carry = (int64_t)__builtin_bit_cast(uint32_t, a.dD[d0 * a.d]);  // parked by prep
    if constexpr (SMALL) {
        if (Tq <= kCsrChunk && L <= kCsrBins) {
            build_csr_small(small, Tq, L, carry, a.row_ptr + d0, a.col_idx, load);
            return;
        }
    }
    build_segment_csr(sm, Tq, L, carry, a.row_ptr + d0, a.col_idx, load);
}

// Eq. (2) per packed query row p = cu_q[i] + s:
// dQ[p] = sum over docs j with a token, ascending, of g[i,j] D[cu_d[j] + argmax[i,j,s]].
template <int G> struct VdqLds {
    int64_t dbase[kDqDocs];
    int32_t dlen[kDqDocs];
    int32_t am[kDqDocs][G];
    float wq[kDqDocs][G];
    int32_t qi[G], qs[G];
};

template <int E, bool GEN, int G>
__device__ __forceinline__ void vbwd_dq_block(const VarBwdArgs& a, VdqLds<G>& sm, int64_t blk)
{
    constexpr int kThreads = 16 * G;
    auto& dbase = sm.dbase;
    auto& dlen = sm.dlen;
    auto& am = sm.am;
    auto& wq = sm.wq;
    auto& qi = sm.qi;
    auto& qs = sm.qs;
    const int64_t Nd = a.Nd, Tq = a.Tq;
    const int64_t DW = GEN ? (int64_t)a.d : kD;
    const int nchunk = GEN ? (int)((DW + 127) / 128) : 1;
    const int64_t p0 = blk * G;
    const int tid = threadIdx.x, grp = tid >> 4, l16 = tid & 15;
    const int64_t p = p0 + grp;
    const bool row_ok = p < Tq;
    if (tid < G) {
        int i = 0, s = 0;
        if (p0 + tid < Tq) {
            i = seg_of(a.cu_q, (int)a.Nq + 1, p0 + tid);
            i = i < (int)a.Nq ? i : (int)a.Nq - 1;  // precondition guard
            int64_t sv = p0 + tid - a.cu_q[i];
            s = (int)(sv < 0 ? 0 : (sv >= a.max_lq ? a.max_lq - 1 : sv));  // precondition guard
        }
        qi[tid] = i;
        qs[tid] = s;
    }
    for (int c = 0; c < nchunk; ++c) {
        const LaneSpan ls(c, l16, DW, GEN);
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        // with no doc token at all there is no D row to gather (dQ = 0)
        for (int64_t j0 = 0; j0 < (a.Td > 0 ? Nd : 0); j0 += kDqDocs) {
            const int nj = (int)(Nd - j0 < kDqDocs ? Nd - j0 : kDqDocs);
            barrier_lds();
            if (tid < nj) {
                const int64_t b = a.cu_d[j0 + tid];
                int64_t l = (int64_t)a.cu_d[j0 + tid + 1] - b;
                if (b < 0 || b >= a.Td) l = 0;
                else if (l > a.Td - b) l = a.Td - b;
                dbase[tid] = b;
                dlen[tid] = (int32_t)(l < 0 ? 0 : l);
            }
            barrier_lds();
            // every load of the batch issued before any is used
            // (out-of-range slots read entry 0)
            constexpr int kPer = kDqDocs * G / kThreads;
            int32_t tv[kPer];
            float wv[kPer];
#pragma unroll
            for (int u = 0; u < kPer; ++u) {
                const int e = tid + u * kThreads, jj = e / G, gg = e % G;
                const bool ok = jj < nj && p0 + gg < Tq && dlen[jj] > 0;
                const int64_t ij = ok ? (int64_t)qi[gg] * Nd + j0 + jj : 0;
                tv[u] = a.argmax[ok ? ij * a.max_lq + qs[gg] : 0];
                wv[u] = a.g[ij];
            }
#pragma unroll
            for (int u = 0; u < kPer; ++u) {
                const int e = tid + u * kThreads, jj = e / G, gg = e % G;
                int32_t t = 0;
                float w = 0.f;
                if (jj < nj && p0 + gg < Tq && dlen[jj] > 0) {
                    t = tv[u];
                    t = t < 0 ? 0 : (t >= dlen[jj] ? dlen[jj] - 1 : t);  // precondition guard
                    w = wv[u];
                }
                am[jj][gg] = t;
                wq[jj][gg] = w;
            }
            barrier_lds();
            if (!row_ok || ls.n == 0) continue;
            int jj = 0;
            for (; jj + 8 <= nj; jj += 8) {
                float x[8][8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int64_t row = dlen[jj + u] > 0 ? dbase[jj + u] + am[jj + u][grp] : 0;
                    loadn<E>(a.D, row * DW + ls.e0, ls.n, ls.vec, x[u]);
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float w = wq[jj + u][grp];
#pragma unroll
                    for (int k = 0; k < 8; ++k) acc[k] = __builtin_fmaf(w, x[u][k], acc[k]);
                }
            }
            for (; jj < nj; ++jj) {
                float x[8];
                const int64_t row = dlen[jj] > 0 ? dbase[jj] + am[jj][grp] : 0;
                loadn<E>(a.D, row * DW + ls.e0, ls.n, ls.vec, x);
                const float w = wq[jj][grp];
#pragma unroll
                for (int k = 0; k < 8; ++k) acc[k] = __builtin_fmaf(w, x[k], acc[k]);
            }
        }
        if (row_ok && ls.n > 0) storen(a.dQ + p * DW + ls.e0, ls.n, ls.vec, acc);
    }
}

// The packed CSR and the packed dQ gathers in one launch: workgroups
// [0, Nd) build doc blockIdx's CSR (its segment start parked by the prep
// pass), the rest are dq workgroups of 64 packed query rows.
template <int E, bool GEN>
__global__ __launch_bounds__(kCsrThreads) void vbwd_csr_dq_kernel(VarBwdArgs a, int64_t csr_blocks)
{
    // one-pass CSR builder for the 128-wide instances only, as in csr_dq_kernel
    __shared__ union {
        CsrLds csr;
        typename std::conditional<GEN, CsrLds, CsrSmallLds>::type small;
        VdqLds<kCsrThreads / 16> dq;
    } sm;
    if ((int64_t)blockIdx.x < csr_blocks) vbwd_csr_doc<!GEN>(a, sm.csr, sm.small, blockIdx.x);
    else vbwd_dq_block<E, GEN, kCsrThreads / 16>(a, sm.dq, (int64_t)blockIdx.x - csr_blocks);
}

// Eq. (3) per packed doc row r: the sources of CSR row r, in order, each
// g[i,j] Q[cu_q[i] + s]. Workgroup = a block of rows; group g owns rows
// r_begin + g + 64 k. O32 (d = 128, packed Q under 4 GiB): a source is
// handed to its group as the 32-bit byte offset of its Q row.
template <int E, bool GEN, bool O32>
__global__ __launch_bounds__(kDdThreads) __attribute__((amdgpu_waves_per_eu(MAXSIM_DD_WAVES))) void vbwd_dd_kernel(
    VarBwdArgs a, int rows_per_block)
{
    static_assert(!(O32 && GEN), "32-bit offsets only for 128-wide rows");
    constexpr int kDdGroups = kDdThreads / 16;
    const int64_t DW = GEN ? (int64_t)a.d : kD;
    const int nchunk = GEN ? (int)((DW + 127) / 128) : 1;
    const int64_t Nd = a.Nd, Nq = a.Nq, Tq = a.Tq;
    const int64_t r_begin = (int64_t)blockIdx.x * rows_per_block;
    const int64_t r_end = r_begin + rows_per_block < a.Td ? r_begin + rows_per_block : a.Td;
    const int tid = threadIdx.x, grp = tid >> 4, l16 = tid & 15;
    const int gbase = tid & 63 & ~15;
    const uint32_t mlq = (uint32_t)a.max_lq, ndm = (uint32_t)(Nd * a.max_lq);
    for (int64_t r = r_begin + grp; r < r_end; r += kDdGroups)
    for (int c = 0; c < nchunk; ++c) {
        const LaneSpan ls(c, l16, DW, GEN);
        const uint32_t e0b = (uint32_t)ls.e0 * (uint32_t)sizeof(uint16_t);  // this lane's bytes of a row (O32)
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        // a valid row lists at most Tq sources inside col_idx; the bounds
        // also hold for any row_ptr content
        int64_t e0 = a.row_ptr[r], e1 = a.row_ptr[r + 1];
        e0 = e0 < 0 ? 0 : (e0 > a.nnz_cap ? a.nnz_cap : e0);
        e1 = e1 < e0 ? e0 : (e1 > a.nnz_cap ? a.nnz_cap : e1);
        e1 = e1 - e0 > Tq ? e0 + Tq : e1;
        for (int64_t e = e0; e < e1; e += 16) {
            const int cnt = (int)(e1 - e < 16 ? e1 - e : 16);
            int64_t qrow = 0;
            float w = 0.f;
            if (l16 < cnt) {
                const uint32_t x = (uint32_t)a.col_idx[e + l16];
                uint32_t i = x / ndm;
                const uint32_t rem = x - i * ndm;
                uint32_t jd = rem / mlq;
                const uint32_t s = rem - jd * mlq;
                // in range for any CSR content (guards the gathers)
                i = i < (uint32_t)Nq ? i : (uint32_t)Nq - 1;
                jd = jd < (uint32_t)Nd ? jd : (uint32_t)Nd - 1;
                qrow = (int64_t)a.cu_q[i] + s;
                qrow = qrow < 0 ? 0 : (qrow < Tq ? qrow : Tq - 1);
                w = a.g[(int64_t)i * Nd + jd];
            }
            // what the group broadcasts per source: the Q row, or (O32) its
            // 32-bit byte offset
            using Src = typename std::conditional<O32, uint32_t, int64_t>::type;
            const Src hand = O32 ? (Src)((uint64_t)qrow * (kD * sizeof(uint16_t))) : (Src)qrow;
            auto gather = [&](Src qr, float (&xv)[8]) {
                if constexpr (O32) load8<E>((const unsigned char*)a.Q + ((uint32_t)qr + e0b), 0, xv);
                else loadn<E>(a.Q, (int64_t)qr * DW + ls.e0, ls.n, ls.vec, xv);
            };
            int k = 0;
            for (; k + kDdUnroll <= cnt; k += kDdUnroll) {
                float xv[kDdUnroll][8];
                float ww[kDdUnroll];
#pragma unroll
                for (int u = 0; u < kDdUnroll; ++u) {
                    const Src qr = __shfl(hand, gbase + k + u, 64);
                    ww[u] = __shfl(w, gbase + k + u, 64);
                    gather(qr, xv[u]);
                }
#pragma unroll
                for (int u = 0; u < kDdUnroll; ++u)
#pragma unroll
                    for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(ww[u], xv[u][q], acc[q]);
            }
            for (; k < cnt; ++k) {
                const Src qr = __shfl(hand, gbase + k, 64);
                const float wk = __shfl(w, gbase + k, 64);
                float xv[8];
                gather(qr, xv);
#pragma unroll
                for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(wk, xv[q], acc[q]);
            }
        }
        if (ls.n > 0) storen(a.dD + r * DW + ls.e0, ls.n, ls.vec, acc);
    }
}

template <int E, bool GEN>
static hipError_t launch_bwd_varlen_t(VarBwdArgs a, hipStream_t stream)
{
    hipError_t err;
    // segment starts and row_ptr[Td] (always: row_ptr has Td + 1 entries),
    // then the CSR (only docs with a token have rows)
    hipLaunchKernelGGL(vbwd_prep_kernel, dim3(1), dim3(kPrepThreads), 0, stream, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    // the CSR (only docs with a token have rows; with no query rows every
    // row_ptr entry is 0) and dQ in one launch
    constexpr int64_t kDqRows = kCsrThreads / 16;
    const int64_t csr_blocks = a.Td > 0 ? a.Nd : 0;
    const int64_t dq_blocks = (a.Tq + kDqRows - 1) / kDqRows;
    if (csr_blocks + dq_blocks > 0) {
        hipLaunchKernelGGL((vbwd_csr_dq_kernel<E, GEN>), dim3((unsigned)(csr_blocks + dq_blocks)), dim3(kCsrThreads),
                           0, stream, a, csr_blocks);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (a.Td > 0) {
        // about two workgroups per CU, whole 64-row steps
        int64_t rpb = (a.Td + 2 * (int64_t)device_cu_count() - 1) / (2 * (int64_t)device_cu_count());
        rpb = (rpb + 63) / 64 * 64;
        if (rpb > 4096) rpb = 4096;
        const int64_t blocks = (a.Td + rpb - 1) / rpb;
        // Q rows addressed by 32-bit byte offsets when packed Q is under 4 GiB
        const bool o32 = !GEN && a.Tq <= (int64_t)(0xFFFFFFFFu / (kD * sizeof(uint16_t)));
        if (o32)
            hipLaunchKernelGGL((vbwd_dd_kernel<E, GEN, !GEN>), dim3((unsigned)blocks), dim3(kDdThreads), 0, stream, a,
                               (int)rpb);
        else
            hipLaunchKernelGGL((vbwd_dd_kernel<E, GEN, false>), dim3((unsigned)blocks), dim3(kDdThreads), 0, stream, a,
                               (int)rpb);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    return hipSuccess;
}

hipError_t launch_bwd_varlen(int elem, VarBwdArgs a, hipStream_t stream)
{
    const bool gen = a.d != kD;
    switch (elem) {
    case kF16: return gen ? launch_bwd_varlen_t<kF16, true>(a, stream) : launch_bwd_varlen_t<kF16, false>(a, stream);
    case kBF16: return gen ? launch_bwd_varlen_t<kBF16, true>(a, stream) : launch_bwd_varlen_t<kBF16, false>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

// ===========================================================================
// Chamfer backward ("Flash-MaxSim" Sec. 4.2.4: the saved argmin, the
// nearest-neighbour index, drives the same inverse-grid CSR). For the
// weighted sum of distances with upstream gradients g1 [B,N], g2 [B,M]:
//   dP[b,p] = 2 g1[b,p] (P[b,p] - Q[b,idx1]) + sum over CSR2 row (b,p) of
//             2 g2[b,q] (P[b,p] - Q[b,q])
//   dQ[b,q] = 2 g2[b,q] (Q[b,q] - P[b,idx2]) + sum over CSR1 row (b,q) of
//             2 g1[b,p] (Q[b,q] - P[b,p])
// CSR1 inverts idx1 (rows = Q points, sources = P points), CSR2 inverts idx2.
// Each batch is a segment with a fixed number of sources, so segment b of
// CSR1 starts at b*N (of CSR2 at b*M): no global scan. One workgroup builds
// one segment; then one thread per point walks its CSR row in order and
// writes its gradient once. No atomics; results are bitwise reproducible.
// ===========================================================================

// Segment g in [0, 2B): g < B is batch g of CSR1 (sources P, rows Q), else
// batch g - B of CSR2. A segment's rows are split into rounds of kCsrBins,
// one workgroup per (segment, round): a count pass, a scan per segment, a
// scatter pass (every workgroup reads all of its segment's sources).
struct ChamSeg {
    int64_t b, ns, nr;
    const int32_t* idx;
    int32_t* row_ptr;
    int32_t* col_idx;
};

__device__ __forceinline__ ChamSeg cham_seg(const ChamferArgs& a, int64_t g)
{
    const bool second = g >= a.B;
    ChamSeg c;
    c.b = second ? g - a.B : g;
    c.ns = second ? a.M : a.N;
    c.nr = second ? a.N : a.M;
    c.idx = second ? a.idx2 : a.idx1;
    c.row_ptr = second ? a.row_ptr2 : a.row_ptr1;
    c.col_idx = second ? a.col_idx2 : a.col_idx1;
    return c;
}

template <int MODE>
__global__ __launch_bounds__(kCsrThreads) void cham_csr_kernel(ChamferArgs a, int rounds1, int rounds2)
{
    // workgroup -> (segment, round): CSR1 segments first, then CSR2
    const int64_t w = blockIdx.x;
    const int64_t n1 = a.B * rounds1;
    const int64_t g = w < n1 ? w / rounds1 : a.B + (w - n1) / rounds2;
    const int64_t r = w < n1 ? w % rounds1 : (w - n1) % rounds2;
    const ChamSeg c = cham_seg(a, g);
    auto load = [&](int64_t k0, int32_t (&tv)[16], int32_t (&sv)[16]) {
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int64_t k = k0 + 64 * m;
            const int64_t src = c.b * c.ns + (k < c.ns ? k : 0);
            sv[m] = (int32_t)src;
            tv[m] = k < c.ns ? __builtin_nontemporal_load(c.idx + src) : 0;
        }
    };
    __shared__ CsrLds sm;
    build_segment_csr<MODE>(sm, c.ns, c.nr, 0, c.row_ptr + c.b * c.nr, c.col_idx, load, r * (int64_t)kCsrBins);
}

// The two CSRs in two steps, when the scratch fits (see the launcher):
// 1. a stable partition of each segment's sources by bucket of kCsrBins rows
//    (destination / 1024), over chunks of kPartChunk sources: per chunk the
//    bucket counts (cham_part_kernel<kCsrCount>), per segment the scan that
//    turns them into each chunk's first slot per bucket and the bucket starts
//    (cham_part_scan_kernel), per chunk the stable scatter of the local
//    source indices in bucket order (cham_part_kernel<kCsrScatter>), each
//    chunk pass ranked through LDS in one pass (place_small) and the scatter
//    written run by run;
// 2. cham_bucket_kernel, one workgroup per (segment, bucket): the CSR rows of
//    the bucket from the bucket's own sources, in source order (one pass when
//    the bucket has at most kCsrChunk sources).
// Scratch of a segment with ns sources, nchunk chunks and R buckets, in its
// share of dP (the first CSR's sources are P points) or dQ (second CSR) as
// ints, which the gradient kernel writes last: the partition [0, ns), the
// bucket starts [ns, ns + R], the chunk counts, then slots,
// [ns + R + 1, ns + R + 1 + nchunk * R) chunk-major. Every round of the
// three-pass build below reads the whole segment; here each source is read
// three times in all.
struct ChamPart {
    int32_t* part;   // [ns] local source indices in bucket order
    int32_t* start;  // [R + 1] bucket starts
    int32_t* cnt;    // [nchunk][R] counts, then first slots
    int64_t R, nchunk;
};
__device__ __forceinline__ ChamPart cham_part(const ChamferArgs& a, const ChamSeg& c, bool second)
{
    ChamPart p;
    p.part = (int32_t*)(second ? a.dQ : a.dP) + c.b * c.ns * 3;
    p.R = (c.nr + kCsrBins - 1) / kCsrBins;
    p.nchunk = (c.ns + kPartChunk - 1) / kPartChunk;
    p.start = p.part + c.ns;
    p.cnt = p.start + p.R + 1;
    return p;
}

template <int MODE>
__global__ __launch_bounds__(kCsrThreads) void cham_part_kernel(ChamferArgs a, int nch1, int nch2)
{
    // workgroup -> (segment, chunk): CSR1 segments first, then CSR2
    const int64_t w = blockIdx.x;
    const int64_t n1 = a.B * nch1;
    const int64_t g = w < n1 ? w / nch1 : a.B + (w - n1) / nch2;
    const int64_t ch = w < n1 ? w % nch1 : (w - n1) % nch2;
    const bool second = g >= a.B;
    const ChamSeg c = cham_seg(a, g);
    const ChamPart p = cham_part(a, c, second);
    const int64_t k_lo = ch * kPartChunk;
    const int64_t n = c.ns - k_lo < kPartChunk ? c.ns - k_lo : kPartChunk;
    const int32_t last = (int32_t)(c.nr - 1);
    const int32_t* idx = c.idx + c.b * c.ns + k_lo;
    auto load = [&](int64_t k0, int32_t (&tv)[kPartSteps], int32_t (&sv)[kPartSteps]) {
#pragma unroll
        for (int m = 0; m < kPartSteps; ++m) {
            const int64_t k = k0 + 64 * m;
            const bool ok = k < n;
            sv[m] = (int32_t)(ok ? k_lo + k : 0);
            int32_t t = ok ? __builtin_nontemporal_load(idx + k) : 0;
            t = t < 0 ? 0 : (t > last ? last : t);  // precondition guard
            tv[m] = t / kCsrBins;
        }
    };
    // one pass per chunk of kPartChunk sources (this path runs only with
    // R <= kCsrBins buckets); short chunks give the few segments many workgroups
    __shared__ CsrSmallLds sm;
    place_small<MODE == kCsrCount, kPartSteps>(sm, n, p.R, p.cnt + ch * p.R, p.part, c.ns, load);
}

// per segment: bucket totals over the chunks, their exclusive scan (the
// bucket starts), and each chunk's first slot per bucket in place of its count
__global__ __launch_bounds__(kCsrBins) void cham_part_scan_kernel(ChamferArgs a)
{
    __shared__ uint32_t wsum[kCsrBins / 64];
    const int64_t g = blockIdx.x;
    const bool second = g >= a.B;
    const ChamSeg c = cham_seg(a, g);
    const ChamPart p = cham_part(a, c, second);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // the chunk counts of this bucket, 8 loads in flight at a time
    constexpr int kB = 8;
    uint32_t tot = 0;
    if (tid < p.R)
        for (int64_t c0 = 0; c0 < p.nchunk; c0 += kB) {
            uint32_t v[kB];
#pragma unroll
            for (int u = 0; u < kB; ++u) v[u] = c0 + u < p.nchunk ? (uint32_t)p.cnt[(c0 + u) * p.R + tid] : 0u;
#pragma unroll
            for (int u = 0; u < kB; ++u) tot += v[u];
        }
    uint32_t incl = tot;
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
    }
    if (lane == 63) wsum[wave] = incl;
    barrier_lds();
    uint32_t base = 0;
    for (int k = 0; k < wave; ++k) base += wsum[k];
    if (tid < p.R) {
        uint32_t run = base + incl - tot;
        p.start[tid] = (int32_t)run;
        for (int64_t c0 = 0; c0 < p.nchunk; c0 += kB) {
            uint32_t v[kB];
#pragma unroll
            for (int u = 0; u < kB; ++u) v[u] = c0 + u < p.nchunk ? (uint32_t)p.cnt[(c0 + u) * p.R + tid] : 0u;
#pragma unroll
            for (int u = 0; u < kB; ++u)
                if (c0 + u < p.nchunk) {
                    p.cnt[(c0 + u) * p.R + tid] = (int32_t)run;
                    run += v[u];
                }
        }
    }
    if (tid == 0) p.start[p.R] = (int32_t)c.ns;
}

__global__ __launch_bounds__(kCsrThreads) void cham_bucket_kernel(ChamferArgs a, int R1, int R2)
{
    // workgroup -> (segment, bucket): CSR1 segments first, then CSR2
    const int64_t w = blockIdx.x;
    const int64_t n1 = a.B * R1;
    const int64_t g = w < n1 ? w / R1 : a.B + (w - n1) / R2;
    const int64_t r = w < n1 ? w % R1 : (w - n1) % R2;
    const bool second = g >= a.B;
    const ChamSeg c = cham_seg(a, g);
    const ChamPart p = cham_part(a, c, second);
    const int64_t R = second ? R2 : R1;
    const int32_t* part = p.part;
    // the bucket's sources, bounded for any scratch content
    int64_t k_beg = p.start[r], k_end = p.start[r + 1];
    k_beg = k_beg < 0 ? 0 : (k_beg > c.ns ? c.ns : k_beg);
    k_end = k_end < k_beg ? k_beg : (k_end > c.ns ? c.ns : k_end);
    const int64_t cnt = k_end - k_beg;
    const int64_t t0 = r * kCsrBins;
    const int64_t L = c.nr - t0 < kCsrBins ? c.nr - t0 : kCsrBins;
    const int32_t last = (int32_t)(c.nr - 1);
    const int64_t sbase = c.b * c.ns;
    // local source indices are below ns < 2^31 (the entry point bounds B*N and B*M)
    const int32_t ns_last = (int32_t)(c.ns - 1);
    auto load = [&](int64_t k0, int32_t (&tv)[16], int32_t (&sv)[16]) {
        int32_t loc[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int64_t k = k0 + 64 * m;
            const int32_t v = k < cnt ? part[k_beg + k] : 0;
            loc[m] = v < 0 ? 0 : (v > ns_last ? ns_last : v);
        }
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int64_t k = k0 + 64 * m;
            sv[m] = (int32_t)(sbase + loc[m]);
            int32_t t = k < cnt ? c.idx[sbase + loc[m]] : 0;
            t = t < 0 ? 0 : (t > last ? last : t);
            tv[m] = (int32_t)(t - t0);  // in [0, L) for a bucket's own sources
        }
    };
    __shared__ union {
        CsrLds csr;
        CsrSmallLds small;
    } sm;
    if (cnt <= kCsrChunk)  // one pass (L <= kCsrBins always)
        build_csr_small(sm.small, cnt, L, sbase + k_beg, c.row_ptr + c.b * c.nr + t0, c.col_idx, load);
    else
        build_segment_csr<kCsrFull>(sm.csr, cnt, L, sbase + k_beg, c.row_ptr + c.b * c.nr + t0, c.col_idx, load);
    if (c.b == a.B - 1 && r == R - 1 && threadIdx.x == 0) c.row_ptr[a.B * c.nr] = (int32_t)(a.B * c.ns);
}

// per segment: the counts in row_ptr become exclusive row starts (plus the
// segment base b*ns); the last segment of each CSR also writes its end entry
__global__ __launch_bounds__(1024) void cham_scan_kernel(ChamferArgs a)
{
    __shared__ uint32_t part[1024];
    const ChamSeg c = cham_seg(a, blockIdx.x);
    int32_t* rp = c.row_ptr + c.b * c.nr;
    const int tid = threadIdx.x;
    const int64_t chunk = (c.nr + 1023) / 1024;
    const int64_t t0 = tid * chunk, t1 = t0 + chunk < c.nr ? t0 + chunk : c.nr;
    // 16 loads in flight per step (integer sums: the grouping does not matter)
    uint32_t sum = 0;
    int64_t t = t0;
    for (; t + 16 <= t1; t += 16) {
        uint32_t v[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = (uint32_t)rp[t + k];
#pragma unroll
        for (int k = 0; k < 16; ++k) sum += v[k];
    }
    for (; t < t1; ++t) sum += (uint32_t)rp[t];
    part[tid] = sum;
    barrier_lds();
    for (int off = 1; off < 1024; off <<= 1) {  // inclusive scan of the chunk sums
        const uint32_t v = tid >= off ? part[tid - off] : 0u;
        barrier_lds();
        part[tid] += v;
        barrier_lds();
    }
    uint32_t run = (uint32_t)(c.b * c.ns) + part[tid] - sum;
    for (t = t0; t + 16 <= t1; t += 16) {
        uint32_t v[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = (uint32_t)rp[t + k];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            rp[t + k] = (int32_t)run;
            run += v[k];
        }
    }
    for (; t < t1; ++t) {
        const uint32_t cnt = (uint32_t)rp[t];
        rp[t] = (int32_t)run;
        run += cnt;
    }
    if (c.b == a.B - 1 && tid == 0) c.row_ptr[a.B * c.nr] = (int32_t)(a.B * c.ns);
}

// one thread per point; threads [0, B*N) produce dP, [B*N, B*N + B*M) dQ
__global__ __launch_bounds__(256) void cham_grad_kernel(ChamferArgs a)
{
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t nP = a.B * a.N, nQ = a.B * a.M;
    if (t >= nP + nQ) return;
    const bool second = t >= nP;  // a point of Q
    const int64_t r = second ? t - nP : t;
    const int64_t nown = second ? a.M : a.N, nother = second ? a.N : a.M;
    const float* X = second ? a.Q : a.P;      // the point's own set
    const float* Y = second ? a.P : a.Q;      // the other set
    const float* g_own = second ? a.g2 : a.g1;
    const float* g_oth = second ? a.g1 : a.g2;
    const int32_t* idx_own = second ? a.idx2 : a.idx1;
    const int32_t* rp = second ? a.row_ptr1 : a.row_ptr2;  // rows over this set
    const int32_t* ci = second ? a.col_idx1 : a.col_idx2;
    const int64_t b = r / nown;
    const float x0 = X[r * 3], x1 = X[r * 3 + 1], x2 = X[r * 3 + 2];
    int64_t nn = idx_own[r];
    nn = nn < 0 ? 0 : (nn >= nother ? nother - 1 : nn);  // precondition guard
    const float* y = Y + (b * nother + nn) * 3;
    const float w = 2.f * g_own[r];
    float acc0 = w * (x0 - y[0]), acc1 = w * (x1 - y[1]), acc2 = w * (x2 - y[2]);
    // sources of this row: points of the other set whose nearest neighbour is
    // this point, ascending; bounded for any row_ptr content
    const int64_t cap = a.B * nother;
    int64_t e0 = rp[r], e1 = rp[r + 1];
    e0 = e0 < 0 ? 0 : (e0 > cap ? cap : e0);
    e1 = e1 < e0 ? e0 : (e1 > cap ? cap : e1);
    e1 = e1 - e0 > nother ? e0 + nother : e1;
    for (int64_t e = e0; e < e1; ++e) {
        int64_t src = ci[e];
        src = src < 0 ? 0 : (src >= cap ? cap - 1 : src);
        const float* z = Y + src * 3;
        const float v = 2.f * g_oth[src];
        acc0 = __builtin_fmaf(v, x0 - z[0], acc0);
        acc1 = __builtin_fmaf(v, x1 - z[1], acc1);
        acc2 = __builtin_fmaf(v, x2 - z[2], acc2);
    }
    float* out = (second ? a.dQ : a.dP) + r * 3;
    out[0] = acc0;
    out[1] = acc1;
    out[2] = acc2;
}

hipError_t launch_chamfer_bwd(ChamferArgs a, hipStream_t stream)
{
    if (a.B == 0) return hipSuccess;
    hipError_t err;
    const int r1 = (int)((a.M + kCsrBins - 1) / kCsrBins), r2 = (int)((a.N + kCsrBins - 1) / kCsrBins);
    const unsigned wgs = (unsigned)(a.B * (r1 + r2));
    // the two-step build keeps ns + R + 1 + nchunk * R ints in a segment's
    // 3 * ns floats of dP (or dQ), and its partition passes handle up to
    // kCsrBins buckets (segments of at most about 1 M rows)
    const int64_t c1 = (a.N + kPartChunk - 1) / kPartChunk, c2 = (a.M + kPartChunk - 1) / kPartChunk;
    if (r1 <= kCsrBins && r2 <= kCsrBins && r1 + 1 + c1 * r1 <= 2 * a.N && r2 + 1 + c2 * r2 <= 2 * a.M) {
        const unsigned pw = (unsigned)(a.B * (c1 + c2));
        hipLaunchKernelGGL(cham_part_kernel<kCsrCount>, dim3(pw), dim3(kCsrThreads), 0, stream, a, (int)c1, (int)c2);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        hipLaunchKernelGGL(cham_part_scan_kernel, dim3((unsigned)(2 * a.B)), dim3(kCsrBins), 0, stream, a);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        hipLaunchKernelGGL(cham_part_kernel<kCsrScatter>, dim3(pw), dim3(kCsrThreads), 0, stream, a, (int)c1, (int)c2);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        hipLaunchKernelGGL(cham_bucket_kernel, dim3(wgs), dim3(kCsrThreads), 0, stream, a, r1, r2);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    } else {
        hipLaunchKernelGGL(cham_csr_kernel<kCsrCount>, dim3(wgs), dim3(kCsrThreads), 0, stream, a, r1, r2);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        hipLaunchKernelGGL(cham_scan_kernel, dim3((unsigned)(2 * a.B)), dim3(1024), 0, stream, a);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        hipLaunchKernelGGL(cham_csr_kernel<kCsrScatter>, dim3(wgs), dim3(kCsrThreads), 0, stream, a, r1, r2);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    const int64_t n = a.B * (a.N + a.M);
    hipLaunchKernelGGL(cham_grad_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace maxsim
