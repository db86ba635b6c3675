// Top-k after scoring: for each query row of a score matrix, the k largest
// scores in decreasing order, equal scores in increasing doc order (the
// retrieval step that follows the scores in the TileMaxSim paper, Sec. 6.8
// "End-to-End Retrieval Latency").
//
// One workgroup of 16 waves per row. Scores map to 32-bit keys whose
// unsigned order is the float order (-0 and +0 share a key). A four-pass
// radix select (8 bits per pass, per-wave LDS histograms) finds the k-th
// largest key T and how many of the k must have key T. One more pass gathers
// every score above T (in any order) and the first ones equal to T in doc
// order (a workgroup-wide ordered count), and a bitonic sort in LDS puts the
// k candidates into (key descending, doc ascending) order. Output values are
// re-read from the scores, so they are the input bits exactly.
#include "common.hpp"
#include "kernels.hpp"

namespace maxsim {

namespace {

constexpr int kTkWaves = 16;
constexpr int kTkThreads = kTkWaves * 64;
constexpr int kBins = 256;

__device__ __forceinline__ uint32_t order_key(float v)
{
    uint32_t b = __builtin_bit_cast(uint32_t, v);
    if ((b & 0x7fffffffu) == 0) b = 0;  // -0 ranks with +0
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ void tk_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// (key, doc) a comes before b in the output order
__device__ __forceinline__ bool before(uint32_t ka, int32_t ia, uint32_t kb, int32_t ib)
{
    return ka > kb || (ka == kb && ia < ib);
}

}  // namespace

__global__ __launch_bounds__(kTkThreads) void topk_kernel(TopkArgs a)
{
    __shared__ uint32_t hist[kTkWaves][kBins];
    __shared__ uint32_t sel_key[kTopkMaxK];
    __shared__ int32_t sel_idx[kTopkMaxK];
    __shared__ uint32_t wcount[kTkWaves];
    __shared__ uint32_t sh[4];  // digit, count above it, number above T collected

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int64_t i = blockIdx.x;
    const int64_t Nd = a.Nd;
    const int K = a.K;
    const float* row = a.scores + i * Nd;

    // ---- radix select of the K-th largest key --------------------------------
    uint32_t prefix = 0, pmask = 0;
    uint32_t need = (uint32_t)K;  // rank of T among the keys that match the prefix
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int b = lane; b < kBins; b += 64) hist[wave][b] = 0;
        __builtin_amdgcn_s_waitcnt(0xC07F);
        for (int64_t j = tid; j < Nd; j += kTkThreads) {
            const uint32_t k = order_key(row[j]);
            if ((k & pmask) == prefix) atomicAdd(&hist[wave][(k >> shift) & 0xffu], 1u);
        }
        tk_barrier();
        // wave 0: per-bin totals, then the bin where the count from the top reaches `need`
        if (wave == 0) {
            uint32_t c[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int b = 255 - (4 * lane + e);  // lane 0 holds the top bins
                uint32_t t = 0;
                for (int w = 0; w < kTkWaves; ++w) t += hist[w][b];
                c[e] = t;
            }
            const uint32_t mine = c[0] + c[1] + c[2] + c[3];
            uint32_t incl = mine;  // inclusive scan from the top bin down
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t v = __shfl_up(incl, off, 64);
                if (lane >= off) incl += v;
            }
            uint32_t above = incl - mine;  // keys in higher bins than this lane's first
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (above < need && need <= above + c[e]) {
                    sh[0] = (uint32_t)(255 - (4 * lane + e));
                    sh[1] = above;
                }
                above += c[e];
            }
        }
        tk_barrier();
        prefix |= sh[0] << shift;
        pmask |= 0xffu << shift;
        need -= sh[1];
        tk_barrier();  // sh[] and hist[] are reused
    }
    const uint32_t T = prefix;
    const uint32_t n_gt = (uint32_t)K - need;  // keys above T, all selected

    // ---- gather: every key above T, and the first `need` keys equal to T ----
    if (tid == 0) sh[2] = 0;
    tk_barrier();
    uint32_t eq_base = 0;  // keys equal to T in earlier chunks
    for (int64_t j0 = 0; j0 < Nd; j0 += kTkThreads) {
        const int64_t j = j0 + tid;
        uint32_t k = 0;
        if (j < Nd) k = order_key(row[j]);
        const bool gt = j < Nd && k > T;
        const bool eq = j < Nd && k == T;
        if (gt) {
            const uint32_t pos = atomicAdd(&sh[2], 1u);
            sel_key[pos] = k;
            sel_idx[pos] = (int32_t)j;
        }
        // ordered rank of the equal keys: within the wave by ballot, across
        // waves by the per-wave counts
        const uint64_t bal = __ballot(eq);
        if (lane == 0) wcount[wave] = (uint32_t)__builtin_popcountll(bal);
        tk_barrier();
        uint32_t before_w = 0, chunk_eq = 0;
        for (int w = 0; w < kTkWaves; ++w) {
            if (w < wave) before_w += wcount[w];
            chunk_eq += wcount[w];
        }
        if (eq) {
            const uint32_t r = eq_base + before_w + (uint32_t)__builtin_popcountll(bal & ((1ull << lane) - 1ull));
            if (r < need) {
                sel_key[n_gt + r] = k;
                sel_idx[n_gt + r] = (int32_t)j;
            }
        }
        eq_base += chunk_eq;
        tk_barrier();  // wcount is reused
    }

    // ---- bitonic sort of the K candidates (padding sorts last) ---------------
    int n = 1;
    while (n < K) n <<= 1;
    for (int e = tid; e < n; e += kTkThreads)
        if (e >= K) {
            sel_key[e] = 0;
            sel_idx[e] = 0x7fffffff;
        }
    for (int size = 2; size <= n; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            tk_barrier();
            for (int t = tid; t < n; t += kTkThreads) {
                const int p = t ^ stride;
                if (p > t) {
                    const uint32_t kt = sel_key[t], kp = sel_key[p];
                    const int32_t it = sel_idx[t], ip = sel_idx[p];
                    const bool fwd = (t & size) == 0;  // this block runs in output order
                    if (fwd ? before(kp, ip, kt, it) : before(kt, it, kp, ip)) {
                        sel_key[t] = kp;
                        sel_idx[t] = ip;
                        sel_key[p] = kt;
                        sel_idx[p] = it;
                    }
                }
            }
        }
    }
    tk_barrier();
    for (int r = tid; r < K; r += kTkThreads) {
        const int32_t j = sel_idx[r];
        a.idx[i * K + r] = a.ids ? a.ids[i * Nd + j] : j;
        a.val[i * K + r] = row[j];
        if (a.rows) a.rows[i * K + r] = (int32_t)i;
    }
}

hipError_t launch_topk(TopkArgs a, hipStream_t stream)
{
    if (a.Nq <= 0 || a.K <= 0) return hipSuccess;
    hipLaunchKernelGGL(topk_kernel, dim3((unsigned)a.Nq), dim3(kTkThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace maxsim
