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
//   live    one wave per doc: live(j) = any(d_mask[j,:]) parked in col_idx[0..Nd)
//           (col_idx is caller-owned and is only filled by the CSR pass later);
//   dq      one wave per query row (i,s): sum over j ascending of
//           g[i,j] * live(j) * D[j, argmax[i,j,s]], times q_mask[i,s];
//   csr     one workgroup per doc: the doc's Nq*Lq sources go into Ld bins.
//           Every doc receives exactly Nq*Lq sources, so its CSR segment starts
//           at j*Nq*Lq and no global scan is needed. Counting and the stable
//           scatter use wave-level key matching (ballots over the key bits):
//           a bin is only ever updated by one lane at a time, in source order;
//   dd      one wave per destination row (j,t): walk the row's sources in CSR
//           order, fp32 accumulation, one write.
#include "common.hpp"
#include "kernels.hpp"

namespace maxsim {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kCsrBins = 2048;  // destination bins handled per round of the CSR pass

template <int E> __device__ __forceinline__ float2 load2(const void* base, int64_t elem_off);
template <> __device__ __forceinline__ float2 load2<kF16>(const void* base, int64_t off)
{
    const _Float16* p = (const _Float16*)base + off;
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    h2 v = *(const h2*)p;
    return make_float2((float)v[0], (float)v[1]);
}
template <> __device__ __forceinline__ float2 load2<kBF16>(const void* base, int64_t off)
{
    const uint32_t u = *(const uint32_t*)((const __bf16*)base + off);
    return make_float2(__builtin_bit_cast(float, u << 16), __builtin_bit_cast(float, u & 0xffff0000u));
}

__device__ __forceinline__ uint64_t lanemask_lt() { return (1ull << lane_id()) - 1ull; }

// Lanes of the wave (among those with `active`) whose key equals this lane's.
__device__ __forceinline__ uint64_t match_key(uint32_t key, bool active, int nbits)
{
    uint64_t peers = __ballot(active);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1u;
        const uint64_t bb = __ballot(active && bit);
        peers &= bit ? bb : ~bb;
    }
    return peers;
}

__device__ __forceinline__ void barrier_lds()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace

// live(j) -> scratch[j] (1 or 0), one wave per doc
__global__ __launch_bounds__(kThreads) void doc_live_kernel(const uint8_t* __restrict__ d_mask,
                                                            int64_t Nd, int64_t Ld,
                                                            int32_t* __restrict__ scratch)
{
    const int64_t j = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (j >= Nd) return;
    const int lane = lane_id();
    bool any = false;
    for (int64_t t = lane; t < Ld && !any; t += 64) any = d_mask[j * Ld + t] != 0;
    const bool live = __ballot(any) != 0;
    if (lane == 0) scratch[j] = live ? 1 : 0;
}

// Eq. (2): one wave per query row r = i*Lq + s; lane l owns dims 2l, 2l+1.
template <int E>
__global__ __launch_bounds__(kThreads) void dq_kernel(BwdArgs a, const int32_t* __restrict__ live)
{
    const int64_t r = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    const int64_t Nq = a.Nq, Nd = a.Nd, Lq = a.Lq, Ld = a.Ld;
    if (r >= Nq * Lq) return;
    const int lane = lane_id();
    const int64_t i = r / Lq, s = r % Lq;
    float ax = 0.f, ay = 0.f;
    const bool qkeep = a.q_mask ? a.q_mask[r] != 0 : true;
    if (qkeep && Ld > 0) {
        for (int64_t j0 = 0; j0 < Nd; j0 += 64) {
            const int64_t jj = j0 + lane;
            int t = 0;
            float w = 0.f;
            if (jj < Nd) {
                t = a.argmax[(i * Nd + jj) * Lq + s];
                t = t < 0 ? 0 : (t >= Ld ? (int)(Ld - 1) : t);  // precondition guard
                w = a.g[i * Nd + jj];
                if (live && live[jj] == 0) w = 0.f;
            }
            const int cnt = Nd - j0 < 64 ? (int)(Nd - j0) : 64;
            int k = 0;
            for (; k + 8 <= cnt; k += 8) {
                float2 x[8];
                float ww[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int tk = __builtin_amdgcn_readlane(t, k + u);
                    ww[u] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), k + u));
                    x[u] = load2<E>(a.D, ((j0 + k + u) * Ld + tk) * kD + 2 * lane);
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    ax = __builtin_fmaf(ww[u], x[u].x, ax);
                    ay = __builtin_fmaf(ww[u], x[u].y, ay);
                }
            }
            for (; k < cnt; ++k) {
                const int tk = __builtin_amdgcn_readlane(t, k);
                const float wk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), k));
                const float2 x = load2<E>(a.D, ((j0 + k) * Ld + tk) * kD + 2 * lane);
                ax = __builtin_fmaf(wk, x.x, ax);
                ay = __builtin_fmaf(wk, x.y, ay);
            }
        }
    }
    *(float2*)(a.dQ + r * kD + 2 * lane) = make_float2(ax, ay);
}

// Inverse map of doc j: row_ptr[j*Ld + t], col_idx[j*Nq*Lq ...] (stable).
__global__ __launch_bounds__(kThreads) void csr_kernel(BwdArgs a)
{
    __shared__ int32_t hist[kWaves][kCsrBins];
    __shared__ int32_t wsum[kWaves];
    const int64_t j = blockIdx.x;
    const int64_t Nq = a.Nq, Nd = a.Nd, Lq = a.Lq, Ld = a.Ld;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int64_t per_doc = Nq * Lq;
    const int64_t base = j * per_doc;
    const int64_t i_lo = Nq * wave / kWaves, i_hi = Nq * (wave + 1) / kWaves;
    int64_t carry = 0;

    for (int64_t t_lo = 0; t_lo < Ld; t_lo += kCsrBins) {
        const int nb = (int)(Ld - t_lo < kCsrBins ? Ld - t_lo : kCsrBins);
        int nbits = 0;
        while ((1 << nbits) < nb) ++nbits;
        for (int k = tid; k < kWaves * kCsrBins; k += kThreads) (&hist[0][0])[k] = 0;
        barrier_lds();

        // pass 1: per-wave histogram of this bin range
        for (int64_t i = i_lo; i < i_hi; ++i) {
            const int32_t* arow = a.argmax + (i * Nd + j) * Lq;
            for (int64_t s0 = 0; s0 < Lq; s0 += 64) {
                const int64_t s = s0 + lane;
                const int t = s < Lq ? arow[s] : -1;
                const bool inr = s < Lq && t >= t_lo && t < t_lo + nb;
                const uint32_t key = inr ? (uint32_t)(t - t_lo) : 0u;
                const uint64_t peers = match_key(key, inr, nbits);
                if (inr && (peers & lanemask_lt()) == 0) hist[wave][key] += __builtin_popcountll(peers);
            }
        }
        barrier_lds();

        // exclusive scan over bins of the per-bin totals; each thread owns a run of bins
        const int per = (nb + kThreads - 1) / kThreads;
        const int k0 = tid * per;
        const int k1 = k0 + per < nb ? k0 + per : nb;
        int run = 0;
        for (int k = k0; k < k1; ++k)
            for (int w = 0; w < kWaves; ++w) run += hist[w][k];
        int incl = run;  // inclusive scan of `run` across the wave
        for (int off = 1; off < 64; off <<= 1) {
            const int v = __shfl_up(incl, off, 64);
            if (lane >= off) incl += v;
        }
        if (lane == 63) wsum[wave] = incl;
        barrier_lds();
        int wave_off = 0;
        for (int w = 0; w < wave; ++w) wave_off += wsum[w];
        int pos = (int)(base + carry) + wave_off + incl - run;  // first CSR slot of bin k0
        for (int k = k0; k < k1; ++k) {
            a.row_ptr[j * Ld + t_lo + k] = pos;
            for (int w = 0; w < kWaves; ++w) {
                const int c = hist[w][k];
                hist[w][k] = pos;  // where wave w's sources of bin k start
                pos += c;
            }
        }
        int tot = 0;
        for (int w = 0; w < kWaves; ++w) tot += wsum[w];
        barrier_lds();

        // pass 2: stable scatter, same traversal order as pass 1
        for (int64_t i = i_lo; i < i_hi; ++i) {
            const int32_t* arow = a.argmax + (i * Nd + j) * Lq;
            for (int64_t s0 = 0; s0 < Lq; s0 += 64) {
                const int64_t s = s0 + lane;
                const int t = s < Lq ? arow[s] : -1;
                const bool inr = s < Lq && t >= t_lo && t < t_lo + nb;
                const uint32_t key = inr ? (uint32_t)(t - t_lo) : 0u;
                const uint64_t peers = match_key(key, inr, nbits);
                if (inr) {
                    const int slot = hist[wave][key] + __builtin_popcountll(peers & lanemask_lt());
                    a.col_idx[slot] = (int32_t)((i * Nd + j) * Lq + s);
                    if ((peers & lanemask_lt()) == 0) hist[wave][key] += __builtin_popcountll(peers);
                }
            }
        }
        carry += tot;
        barrier_lds();
    }
    if (j == Nd - 1 && tid == 0) a.row_ptr[Nd * Ld] = (int32_t)(Nq * Nd * Lq);
}

// Eq. (3): one wave per destination row (j,t), sources in CSR order.
template <int E>
__global__ __launch_bounds__(kThreads) void dd_kernel(BwdArgs a)
{
    const int64_t Nd = a.Nd, Lq = a.Lq, Ld = a.Ld;
    const int64_t blocks_per_doc = (Ld + 63) / 64;
    const int64_t j = blockIdx.x / blocks_per_doc;
    const int64_t tb = (blockIdx.x % blocks_per_doc) * 64;
    const int wave = threadIdx.x >> 6, lane = lane_id();
    bool live = Ld > 0;
    if (a.d_mask) {
        bool any = false;
        for (int64_t t = lane; t < Ld && !any; t += 64) any = a.d_mask[j * Ld + t] != 0;
        live = __ballot(any) != 0;
    }
    for (int rr = 0; rr < 16; ++rr) {
        const int64_t t = tb + wave * 16 + rr;
        if (t >= Ld) break;
        const int64_t row = j * Ld + t;
        float ax = 0.f, ay = 0.f;
        if (live) {
            const int e0 = a.row_ptr[row], e1 = a.row_ptr[row + 1];
            for (int e = e0; e < e1; e += 64) {
                const int cnt = e1 - e < 64 ? e1 - e : 64;
                int qrow = 0;
                float w = 0.f;
                if (lane < cnt) {
                    const uint32_t src = (uint32_t)a.col_idx[e + lane];
                    const uint32_t s = src % (uint32_t)Lq;
                    const uint32_t i = (src / (uint32_t)Lq) / (uint32_t)Nd;
                    qrow = (int)(i * (uint32_t)Lq + s);
                    w = a.g[(int64_t)i * Nd + j];
                    if (a.q_mask && a.q_mask[qrow] == 0) w = 0.f;
                }
                int k = 0;
                for (; k + 8 <= cnt; k += 8) {
                    float2 x[8];
                    float ww[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const int qr = __builtin_amdgcn_readlane(qrow, k + u);
                        ww[u] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), k + u));
                        x[u] = load2<E>(a.Q, (int64_t)qr * kD + 2 * lane);
                    }
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        ax = __builtin_fmaf(ww[u], x[u].x, ax);
                        ay = __builtin_fmaf(ww[u], x[u].y, ay);
                    }
                }
                for (; k < cnt; ++k) {
                    const int qr = __builtin_amdgcn_readlane(qrow, k);
                    const float wk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), k));
                    const float2 x = load2<E>(a.Q, (int64_t)qr * kD + 2 * lane);
                    ax = __builtin_fmaf(wk, x.x, ax);
                    ay = __builtin_fmaf(wk, x.y, ay);
                }
            }
        }
        *(float2*)(a.dD + row * kD + 2 * lane) = make_float2(ax, ay);
    }
}

template <int E>
static hipError_t launch_bwd_t(BwdArgs a, hipStream_t stream)
{
    const int64_t nsrc = a.Nq * a.Nd * a.Lq;
    hipError_t err;
    // live flags parked in col_idx[0..Nd) when there is a d_mask and col_idx can hold them
    const int32_t* live = nullptr;
    if (a.d_mask && nsrc >= a.Nd && a.Nd > 0) {
        hipLaunchKernelGGL(doc_live_kernel, dim3((unsigned)((a.Nd + kWaves - 1) / kWaves)),
                           dim3(kThreads), 0, stream, a.d_mask, a.Nd, a.Ld, a.col_idx);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        live = a.col_idx;
    }
    const int64_t qrows = a.Nq * a.Lq;
    if (qrows > 0) {
        hipLaunchKernelGGL(dq_kernel<E>, dim3((unsigned)((qrows + kWaves - 1) / kWaves)),
                           dim3(kThreads), 0, stream, a, live);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (a.Nd > 0) {
        hipLaunchKernelGGL(csr_kernel, dim3((unsigned)a.Nd), dim3(kThreads), 0, stream, a);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        if (a.Ld > 0) {
            const int64_t blocks = a.Nd * ((a.Ld + 63) / 64);
            hipLaunchKernelGGL(dd_kernel<E>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
            if ((err = hipGetLastError()) != hipSuccess) return err;
        }
    }
    return hipSuccess;
}

hipError_t launch_bwd(int elem, BwdArgs a, hipStream_t stream)
{
    switch (elem) {
    case kF16: return launch_bwd_t<kF16>(a, stream);
    case kBF16: return launch_bwd_t<kBF16>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace maxsim
