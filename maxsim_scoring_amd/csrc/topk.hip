// Top-k after scoring: for each query row of a score matrix, the k largest
// scores in decreasing order, equal scores in increasing doc order (the
// retrieval step that follows the scores in the TileMaxSim paper, Sec. 6.8
// "End-to-End Retrieval Latency").
//
// One workgroup of 16 waves per row. Scores map to 32-bit keys whose
// unsigned order is the float order (-0 and +0 share a key). A four-pass
// radix select (8 bits per pass, per-wave LDS histograms) over a leading
// sample of the row gives a threshold with at least k scores at or above it
// (with few columns, no threshold). One pass over the row, each wave over its
// own contiguous run of columns, collects the scores at or above it into LDS
// in column order; every score equal to the k-th largest is among them. If
// there are at most 1024 candidates they are sorted into (key descending,
// doc ascending) order and the first k kept; otherwise a radix select over
// the candidates finds the k-th largest key T, and the keys above T plus the
// first ones equal to T in doc order are sorted. If the candidates do not fit
// in LDS, the same select-and-gather runs over the whole row. Output values
// are re-read from the scores, so they are the input bits exactly.
#include "common.hpp"
#include "kernels.hpp"

namespace maxsim {

namespace {

constexpr int kTkWaves = 16;
constexpr int kTkThreads = kTkWaves * 64;
constexpr int kBins = 256;
constexpr int kCand = 8192;    // candidates sorted in LDS
constexpr int kSample = 4096;  // smallest leading sample that sets the threshold
constexpr int kBatch = 8;      // row loads in flight per thread

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

// float with order key k (order_key maps -0 and +0 to the key of +0)
__device__ __forceinline__ float key_float(uint32_t k)
{
    return __builtin_bit_cast(float, (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Key T of the `need`-th largest key of a set (radix select, four 8-bit
// passes with per-wave LDS histograms); `need` becomes the number of keys
// equal to T that belong to the selection. fill(f) calls f(key) for each of
// this thread's keys.
template <typename Fill>
__device__ __forceinline__ uint32_t radix_select(Fill fill, uint32_t& need, uint32_t (*hist)[kBins], uint32_t* sh)
{
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    uint32_t prefix = 0, pmask = 0;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int b = lane; b < kBins; b += 64) hist[wave][b] = 0;
        __builtin_amdgcn_s_waitcnt(0xC07F);
        fill([&](uint32_t k) {
            if ((k & pmask) == prefix) atomicAdd(&hist[wave][(k >> shift) & 0xffu], 1u);
        });
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
    return prefix;
}

// Bitonic sort of key/idx[0, n) into output order, n a power of two: per
// stage every thread takes whole compare-exchange pairs (n/2 per stage).
__device__ __forceinline__ void bitonic_sort(uint32_t* key, int32_t* idx, int n)
{
    for (int size = 2, ls = 1; size <= n; size <<= 1, ++ls) {
        for (int stride = size >> 1, lt = ls - 1; stride > 0; stride >>= 1, --lt) {
            tk_barrier();
            for (int q = threadIdx.x; q < (n >> 1); q += kTkThreads) {
                const int t = ((q >> lt) << (lt + 1)) | (q & (stride - 1));
                const int p = t + stride;
                const uint32_t kt = key[t], kp = key[p];
                const int32_t it = idx[t], ip = idx[p];
                const bool fwd = (t & size) == 0;  // this block runs in output order
                if (fwd ? before(kp, ip, kt, it) : before(kt, it, kp, ip)) {
                    key[t] = kp;
                    idx[t] = ip;
                    key[p] = kt;
                    idx[p] = it;
                }
            }
        }
    }
    tk_barrier();
}

// From a set given in increasing column order (chunk by chunk through
// get(e) -> (key, column) for e < n), write into sel[0, K): every key above T
// (in any order) and the first `need` keys equal to T, with n_gt = K - need.
template <typename Get>
__device__ __forceinline__ void gather_top(Get get, int64_t n, uint32_t T, uint32_t need, uint32_t* sel_key,
                                           int32_t* sel_idx, uint32_t* wcount, uint32_t* sh, int K)
{
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const uint32_t n_gt = (uint32_t)K - need;
    if (tid == 0) sh[2] = 0;
    tk_barrier();
    uint32_t eq_base = 0;  // keys equal to T in earlier chunks
    for (int64_t e0 = 0; e0 < n; e0 += kTkThreads) {
        const int64_t e = e0 + tid;
        uint32_t k = 0;
        int32_t j = 0;
        if (e < n) get(e, k, j);
        const bool gt = e < n && k > T;
        const bool eq = e < n && k == T;
        if (gt) {
            const uint32_t pos = atomicAdd(&sh[2], 1u);
            sel_key[pos] = k;
            sel_idx[pos] = j;
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
                sel_idx[n_gt + r] = j;
            }
        }
        eq_base += chunk_eq;
        tk_barrier();  // wcount is reused
    }
}

__global__ __launch_bounds__(kTkThreads) void topk_kernel(TopkArgs a)
{
    __shared__ uint32_t hist[kTkWaves][kBins];
    __shared__ uint32_t cand_key[kCand];  // per-wave slices, later the selection
    __shared__ int32_t cand_idx[kCand];
    __shared__ uint32_t comp_key[kCand];  // the candidates, compacted in column order
    __shared__ int32_t comp_idx[kCand];
    __shared__ uint32_t wcount[kTkWaves];
    __shared__ uint32_t sh[4];  // digit, count above it, gathered count

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int64_t i = blockIdx.x;
    const int64_t Nd = a.Nd;
    const int K = a.K;
    const float* row = a.scores + i * Nd;
    uint32_t* sel_key = cand_key;
    int32_t* sel_idx = cand_idx;

    // ---- threshold: a value with at least K scores at or above it. With few
    // columns every column qualifies; else the K-th largest of a leading
    // sample (a lower bound of the final K-th largest).
    float theta = -__builtin_inff();
    if (Nd > kCand) {
        int64_t S = (2 * (int64_t)K * Nd + kCand - 1) / kCand;  // expect about kCand / 2 candidates
        if (S < kSample) S = kSample;
        if (S > Nd) S = Nd;
        uint32_t need = (uint32_t)K;
        const uint32_t tk = radix_select(
            [&](auto f) {
                for (int64_t j0 = tid; j0 < S; j0 += (int64_t)kBatch * kTkThreads) {
                    float v[kBatch];
#pragma unroll
                    for (int u = 0; u < kBatch; ++u) {
                        const int64_t j = j0 + (int64_t)u * kTkThreads;
                        v[u] = j < S ? row[j] : 0.f;
                    }
#pragma unroll
                    for (int u = 0; u < kBatch; ++u)
                        if (j0 + (int64_t)u * kTkThreads < S) f(order_key(v[u]));
                }
            },
            need, hist, sh);
        theta = key_float(tk);
    }

    // ---- candidates: wave w scans its own contiguous run of columns and
    // appends the scores >= theta to its slice in column order -------------
    constexpr int kPerWave = kCand / kTkWaves;
    const int64_t per = (Nd + kTkWaves - 1) / kTkWaves;
    const int64_t c_lo = per * wave < Nd ? per * wave : Nd;
    const int64_t c_hi = c_lo + per < Nd ? c_lo + per : Nd;
    uint32_t wn = 0;  // this wave's candidates so far (wave-uniform)
    for (int64_t c0 = c_lo; c0 < c_hi; c0 += 64 * kBatch) {
        float v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int64_t j = c0 + 64 * u + lane;
            v[u] = j < c_hi ? row[j] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int64_t j = c0 + 64 * u + lane;
            const bool take = j < c_hi && v[u] >= theta;
            const uint64_t bal = __ballot(take);
            if (bal == 0) continue;  // uniform: the common case
            if (take) {
                const uint32_t pos = wn + (uint32_t)__builtin_popcountll(bal & ((1ull << lane) - 1ull));
                if (pos < (uint32_t)kPerWave) {
                    cand_key[wave * kPerWave + pos] = order_key(v[u]);
                    cand_idx[wave * kPerWave + pos] = (int32_t)j;
                }
            }
            wn += (uint32_t)__builtin_popcountll(bal);
        }
    }
    if (lane == 0) wcount[wave] = wn;
    tk_barrier();
    bool fits = true;
    uint32_t off = 0, ncand = 0;
    for (int w = 0; w < kTkWaves; ++w) {
        fits = fits && wcount[w] <= (uint32_t)kPerWave;
        if (w < wave) off += wcount[w];
        ncand += wcount[w];
    }

    int nsort;  // entries of sel_key/sel_idx to sort
    if (fits) {
        // ---- compact the slices (column order is kept) ----------------------
        for (uint32_t e = lane; e < wcount[wave]; e += 64) {
            comp_key[off + e] = cand_key[wave * kPerWave + e];
            comp_idx[off + e] = cand_idx[wave * kPerWave + e];
        }
        tk_barrier();
        if (ncand <= (uint32_t)kTopkMaxK) {
            // few candidates: sort them all
            for (int e = tid; e < (int)ncand; e += kTkThreads) {
                sel_key[e] = comp_key[e];
                sel_idx[e] = comp_idx[e];
            }
            nsort = (int)ncand;
        } else {
            // the exact K-th largest among the candidates, then the selection
            uint32_t need = (uint32_t)K;
            const uint32_t T = radix_select(
                [&](auto f) {
                    for (int e = tid; e < (int)ncand; e += kTkThreads) f(comp_key[e]);
                },
                need, hist, sh);
            gather_top(
                [&](int64_t e, uint32_t& k, int32_t& j) {
                    k = comp_key[e];
                    j = comp_idx[e];
                },
                (int64_t)ncand, T, need, sel_key, sel_idx, wcount, sh, K);
            nsort = K;
        }
    } else {
        // ---- too many candidates: exact radix select over the whole row ----
        uint32_t need = (uint32_t)K;
        const uint32_t T = radix_select(
            [&](auto f) {
                for (int64_t j0 = tid; j0 < Nd; j0 += (int64_t)kBatch * kTkThreads) {
                    float v[kBatch];
#pragma unroll
                    for (int u = 0; u < kBatch; ++u) {
                        const int64_t j = j0 + (int64_t)u * kTkThreads;
                        v[u] = j < Nd ? row[j] : 0.f;
                    }
#pragma unroll
                    for (int u = 0; u < kBatch; ++u)
                        if (j0 + (int64_t)u * kTkThreads < Nd) f(order_key(v[u]));
                }
            },
            need, hist, sh);
        gather_top(
            [&](int64_t e, uint32_t& k, int32_t& j) {
                k = order_key(row[e]);
                j = (int32_t)e;
            },
            Nd, T, need, sel_key, sel_idx, wcount, sh, K);
        nsort = K;
    }

    // ---- sort the selection (padding sorts last) and write the first K -------
    int n = 1;
    while (n < nsort) n <<= 1;
    for (int e = nsort + tid; e < n; e += kTkThreads) {
        sel_key[e] = 0;
        sel_idx[e] = 0x7fffffff;
    }
    bitonic_sort(sel_key, sel_idx, n);
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
