// Padding-free MaxSim forward for gfx950 (fp16/bf16, 16x16x32 MFMA).
//
// "Flash-MaxSim" Sec. 4.3.2 / Sec. 5.5 (cu_seqlens scoring does sum(L_d) work
// instead of B * L_d^max, with identical scores); late-interaction-kernels
// design notes "Varlen / packed path" (offsets from cu_seqlens, empty
// sequences contribute zero); TileMaxSim Sec. 3.4 Theorem 1 (the memory-bound
// regime is the time spent reading D, optimal when every embedding is read
// once) and the TileMaxSim README note on 64-bit offsets.
//
// Design: the reranking regime is bound by HBM reads of the packed D, so each
// wave is a persistent streaming unit that owns a token-balanced, contiguous
// range of whole docs and walks it as one flat stream of 16-token tiles,
// regardless of doc boundaries. Each 4 KB tile is fetched with fully
// coalesced, non-temporal direct-to-LDS loads (every instruction reads four
// whole rows) into a per-wave ring of kStages tiles; the 16-byte chunks are
// XOR-swizzled on the way in so that the MFMA A-operand reads back from LDS
// (lane l takes token l % 16) are bank-conflict free. Loads that match the
// MFMA layout directly (16 rows x 64 bytes per instruction) measured slower.
// The query (B operand) stays in VGPRs. Per tile each lane folds 4 doc rows
// into its running max; a doc boundary inside a tile splits the fold with
// -inf masks, and a finished doc is reduced across the 4 row groups and 16
// query columns in a fixed order and written once. The ring is private to the
// wave, so there are no barriers, and there are no atomics.
#include "common.hpp"
#include "kernels.hpp"

namespace maxsim {

namespace {

#ifndef MAXSIM_VARLEN_STAGES
#define MAXSIM_VARLEN_STAGES 3
#endif
constexpr int kStages = MAXSIM_VARLEN_STAGES;  // 4 KB tiles in flight per wave
constexpr int kUnitsPerBlock = 4;
constexpr int kTileBytes = 16 * kD * 2;
constexpr int kNonTemporal = 2;  // cache-policy bit of the load: streamed once

// vmcnt(4 * n) for the number n of later tiles still in flight
__device__ __forceinline__ void wait_tiles_behind(int n)
{
    if (n <= 0) wait_vmcnt<0>();
    else if (n == 1) wait_vmcnt<4>();
    else if (n == 2) wait_vmcnt<8>();
    else wait_vmcnt<12>();
}

// Smallest j in [0, n] with cu[j] >= target, found by the whole wave with
// 64 probes per round (cu is non-decreasing and cu[n] >= target).
__device__ int wave_lower_bound(const int32_t* __restrict__ cu, int n, int64_t target)
{
    const int lane = lane_id();
    int lo = 0, hi = n;  // the answer stays in [lo, hi]
    while (lo < hi) {
        const int step = (hi - lo + 63) / 64;
        const int pos = lo + (lane + 1) * step - 1;
        const bool pred = pos < hi ? ((int64_t)cu[pos] >= target) : true;
        const uint64_t bal = __ballot(pred);
        const int k = bal ? __builtin_ctzll(bal) : 64;  // first probe at or above target
        const int nlo = lo + k * step;
        const int nhi = lo + (k + 1) * step - 1;
        lo = nlo < hi ? nlo : hi;
        hi = nhi < hi ? nhi : hi;
    }
    return lo;
}

}  // namespace

template <int E, bool ARGMAX, int NTQ>
__global__ __launch_bounds__(kUnitsPerBlock * 64) void fwd_varlen_kernel(VarlenArgs a)
{
    constexpr int RB = kD * 2;   // bytes per token row
    constexpr int KS = kD / 32;  // 16x16x32: 4 K-steps
    static_assert(KS == 4, "one lds_read4 per tile");
    __shared__ __attribute__((aligned(16))) unsigned char ring_lds[kUnitsPerBlock][kStages][kTileBytes];
    const int lane = lane_id();
    const int col = lane & 15;   // query token within an N-tile / doc row within a tile
    const int g = lane >> 4;     // row group: this lane owns tile rows 4g .. 4g+3

    const int unit = blockIdx.x * kUnitsPerBlock + (threadIdx.x >> 6);
    const int U = a.units;
    if (unit >= U) return;

    const int Nd = (int)a.Nd;
    const int64_t T = a.cu_d[Nd];
    const int64_t tgt0 = (T * unit) / U;
    const int64_t tgt1 = (T * (unit + 1)) / U;
    const int jb = wave_lower_bound(a.cu_d, Nd, tgt0);
    const int je = unit + 1 == U ? Nd : wave_lower_bound(a.cu_d, Nd, tgt1);
    if (jb >= je) return;

  for (int64_t i = blockIdx.y; i < a.Nq; i += gridDim.y) {
    const int64_t q0 = a.cu_q[i];
    int64_t lq = (int64_t)a.cu_q[i + 1] - q0;
    if (lq > a.max_lq) lq = a.max_lq;
    if (lq < 0) lq = 0;
    const int64_t u0 = a.cu_d[jb];
    const int64_t u1 = a.cu_d[je];
    const int64_t ntile = (u1 - u0 + 15) >> 4;
    const unsigned char* Dbase = (const unsigned char*)a.D;
    const int npass = lq == 0 ? 1 : (int)((lq + 16 * NTQ - 1) / (16 * NTQ));

    for (int pass = 0; pass < npass; ++pass) {
        // ---- query fragments for this pass (B operand: col = token, k-quarter g)
        i32x4 qf[NTQ][KS];
        bool tok_ok[NTQ];
#pragma unroll
        for (int n = 0; n < NTQ; ++n) {
            const int64_t s = (int64_t)pass * 16 * NTQ + n * 16 + col;
            tok_ok[n] = s < lq;
            const unsigned char* qrow = (const unsigned char*)a.Q + (q0 + (tok_ok[n] ? s : 0)) * RB;
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                i32x4 v = {0, 0, 0, 0};
                if (tok_ok[n]) v = *(const i32x4*)(qrow + (4 * k + g) * 16);
                qf[n][k] = v;
            }
        }

        // ---- doc cursor: cu_d values cached one per lane, read with readlane
        int j = jb;
        int cache_base = jb + 1;  // lane k holds cu_d[cache_base + k]
        int cu_cache = a.cu_d[cache_base + lane <= Nd ? cache_base + lane : Nd];
        auto cu_next = [&](int jj) -> int64_t {  // cu_d[jj + 1]
            int off = jj + 1 - cache_base;
            if (off >= 64) {  // once per 64 docs
                cache_base = jj + 1;
                cu_cache = a.cu_d[cache_base + lane <= Nd ? cache_base + lane : Nd];
                // wait here, on the rare refill path, so that the compiler does
                // not keep cu_cache "in flight" and wait for the whole tile ring
                // at every doc boundary
                wait_vmcnt<0>();
                off = 0;
            }
            return (int64_t)__builtin_amdgcn_readlane(cu_cache, off);
        };
        int64_t doc_start = u0;
        int64_t doc_end = cu_next(j);

        float m[NTQ];
        int idx[NTQ];
#pragma unroll
        for (int n = 0; n < NTQ; ++n) {
            m[n] = -__builtin_inff();
            idx[n] = 0;
        }

        // finish doc j: merge the 4 row groups, mask, sum, write
        auto finish_doc = [&]() {
            float total = 0.f;
#pragma unroll
            for (int n = 0; n < NTQ; ++n) {
                float mv = m[n];
                int iv = idx[n];
#pragma unroll
                for (int off = 16; off <= 32; off <<= 1) {
                    const float om = shfl_xor_f(mv, off);
                    const int oi = shfl_xor_i(iv, off);
                    if constexpr (ARGMAX)
                        argmax_merge(mv, iv, om, oi);
                    else
                        mv = mv > om ? mv : om;
                }
                const bool fin = __builtin_isfinite(mv);
                float c = (tok_ok[n] && fin) ? mv : 0.f;
#pragma unroll
                for (int off = 8; off >= 1; off >>= 1) c += shfl_xor_f(c, off);
                total += c;
                if constexpr (ARGMAX) {
                    if (g == 0 && tok_ok[n]) {
                        const int64_t s = (int64_t)pass * 16 * NTQ + n * 16 + col;
                        a.argmax[(i * a.Nd + j) * a.max_lq + s] = fin ? (int)(iv - doc_start) : 0;
                    }
                }
                m[n] = -__builtin_inff();
                idx[n] = 0;
            }
            if constexpr (ARGMAX) {
                if (pass == 0) {  // rows past the query's length are 0
                    for (int64_t s = lq + lane; s < a.max_lq; s += 64)
                        a.argmax[(i * a.Nd + j) * a.max_lq + s] = 0;
                }
            }
            if (lane == 0) {
                float* out = a.scores + i * a.Nd + j;
                *out = pass == 0 ? total : *out + total;
            }
        };

        // fold rows [lo, hi) of the tile starting at token ts into the state
        auto fold = [&](const f32x4 (&acc)[NTQ], int64_t ts, int64_t lo, int64_t hi) {
            const int64_t rbase = ts + 4 * g;
            if (lo <= ts && hi >= ts + 16) {
#pragma unroll
                for (int n = 0; n < NTQ; ++n) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float v = acc[n][r];
                        if constexpr (ARGMAX) {
                            if (v > m[n]) {
                                m[n] = v;
                                idx[n] = (int)(rbase + r);
                            }
                        } else {
                            m[n] = m[n] > v ? m[n] : v;
                        }
                    }
                }
            } else {
#pragma unroll
                for (int n = 0; n < NTQ; ++n) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int64_t row = rbase + r;
                        const float v = (row >= lo && row < hi) ? acc[n][r] : -__builtin_inff();
                        if constexpr (ARGMAX) {
                            if (v > m[n]) {
                                m[n] = v;
                                idx[n] = (int)row;
                            }
                        } else {
                            m[n] = m[n] > v ? m[n] : v;
                        }
                    }
                }
            }
        };

        bool done = false;
        // leading empty docs
        while (!done && doc_end <= u0) {
            finish_doc();
            ++j;
            if (j >= je) done = true;
            else {
                doc_start = doc_end;
                doc_end = cu_next(j);
            }
        }

        // ---- per-wave LDS ring of prefetched tiles ----------------------------
        unsigned char* ring = &ring_lds[threadIdx.x >> 6][0][0];
        auto issue_tile = [&](int64_t t, int stage) {
            unsigned char* sb = ring + stage * kTileBytes;
#pragma unroll
            for (int k = 0; k < 4; ++k) {  // instruction k fills rows 4k .. 4k+3
                const int row = 4 * k + (lane >> 4);
                const int lc = (lane & 15) ^ row;  // logical chunk stored at slot lane & 15
                int64_t grow = u0 + t * 16 + row;
                if (grow >= u1) grow = u1 - 1;  // rows past the range are never folded
                __builtin_amdgcn_global_load_lds((const void*)(Dbase + grow * RB + lc * 16),
                                                 LDS_PTR(sb + k * 1024), 16, 0, kNonTemporal);
            }
        };
        // A-operand read offsets: row = lane % 16, logical chunk 4k + g
        uint32_t frag_off[KS];
#pragma unroll
        for (int k = 0; k < KS; ++k) frag_off[k] = col * RB + (((4 * k + g) ^ col) * 16);
        const uint32_t ring_base = lds_addr(ring);

        wait_vmcnt<0>();  // query fragments have landed before the pipeline starts
#pragma unroll
        for (int q = 0; q < kStages; ++q)
            if (q < ntile) issue_tile(q, q);

        int stage = 0;
        for (int64_t t = 0; t < ntile && !done; ++t) {
            {
                const int64_t behind = ntile - 1 - t;
                wait_tiles_behind(behind < kStages - 1 ? (int)behind : kStages - 1);
            }
            i32x4 af[KS];
            const uint32_t sbase = ring_base + stage * kTileBytes;
            lds_read4(af[0], af[1], af[2], af[3], sbase + frag_off[0], sbase + frag_off[1],
                      sbase + frag_off[2], sbase + frag_off[3]);
            if (t + kStages < ntile) issue_tile(t + kStages, stage);
            stage = stage + 1 == kStages ? 0 : stage + 1;
            {
                f32x4 acc[NTQ];
#pragma unroll
                for (int n = 0; n < NTQ; ++n) {
                    acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int k = 0; k < KS; ++k) acc[n] = mfma16<E>(af[k], qf[n][k], acc[n]);
                }

                const int64_t ts = u0 + t * 16;
                int64_t lo = ts;
                while (true) {
                    const int64_t hi = doc_end < ts + 16 ? doc_end : ts + 16;
                    if (hi > lo) fold(acc, ts, lo, hi);
                    if (doc_end > ts + 16) break;
                    finish_doc();
                    ++j;
                    if (j >= je) {
                        done = true;
                        break;
                    }
                    lo = doc_end;
                    doc_start = doc_end;
                    doc_end = cu_next(j);
                }
            }
        }
        wait_vmcnt<0>();  // nothing of this unit's ring is still in flight
        // docs left with no tokens after the last tile (only when ntile == 0)
        while (!done) {
            finish_doc();
            ++j;
            if (j >= je) done = true;
            else {
                doc_start = doc_end;
                doc_end = cu_next(j);
            }
        }
    }
  }
}

template <int E, int NTQ>
static hipError_t launch_varlen_t(VarlenArgs a, hipStream_t stream)
{
    const bool am = a.argmax != nullptr;
    auto kern = am ? fwd_varlen_kernel<E, true, NTQ> : fwd_varlen_kernel<E, false, NTQ>;
    static int max_units_cache[2] = {0, 0};
    int& max_units = max_units_cache[am ? 1 : 0];
    if (max_units == 0) {
        int dev = 0, ncu = 0, per_cu = 0;
        (void)hipGetDevice(&dev);
        (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
        (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kUnitsPerBlock * 64, 0);
        if (ncu <= 0) ncu = 256;
        if (per_cu <= 0) per_cu = 1;
        max_units = ncu * per_cu * kUnitsPerBlock;
    }
    int64_t units = a.Nd / 8;  // about 8+ docs per unit keeps the per-unit setup amortised
    if (units < 1) units = 1;
    if (units > max_units) units = max_units;
    a.units = (int32_t)units;
    const int64_t gy = a.Nq < 65535 ? a.Nq : 65535;
    dim3 grid((unsigned)((units + kUnitsPerBlock - 1) / kUnitsPerBlock), (unsigned)gy);
    hipLaunchKernelGGL(kern, grid, dim3(kUnitsPerBlock * 64), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_fwd_varlen(int elem, VarlenArgs a, hipStream_t stream)
{
    const bool short_q = a.max_lq <= 32;
    switch (elem) {
    case kF16: return short_q ? launch_varlen_t<kF16, 2>(a, stream) : launch_varlen_t<kF16, 4>(a, stream);
    case kBF16: return short_q ? launch_varlen_t<kBF16, 2>(a, stream) : launch_varlen_t<kBF16, 4>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace maxsim
