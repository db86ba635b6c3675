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
// wave is a streaming unit that owns a token-balanced, contiguous range of
// whole docs and walks it as one flat stream of 16-token tiles, regardless of
// doc boundaries; the units come in a whole number of rounds of the resident
// wave slots, so waves that finish early take units off the tail. Each 4 KB tile is fetched with fully
// coalesced, non-temporal direct-to-LDS loads (every instruction reads four
// whole rows) into a per-wave ring of kStages tiles; the 16-byte chunks are
// XOR-swizzled on the way in so that the MFMA A-operand reads back from LDS
// (lane l takes token l % 16) are bank-conflict free. Loads that match the
// MFMA layout directly (16 rows x 64 bytes per instruction) measured slower.
// The query (B operand) stays in VGPRs. Per tile each lane folds 4 doc rows
// into its running max; a doc boundary inside a tile splits the fold with
// -inf masks, and a finished doc is reduced across the 4 row groups and 16
// query columns in a fixed order and written once. All cursor state is
// wave-uniform (scalar registers). The ring is private to the wave, so there
// are no barriers, and there are no atomics.
#include <atomic>

#include "common.hpp"
#include "kernels.hpp"

namespace maxsim {

namespace {

#ifndef MAXSIM_VARLEN_STAGES
#define MAXSIM_VARLEN_STAGES 2
#endif
constexpr int kStages = MAXSIM_VARLEN_STAGES;  // 4 KB tiles in flight per wave
constexpr int kUnitsPerBlock = 4;
constexpr int kRowBytes = kD * 2;
constexpr int kTileBytes = 16 * kRowBytes;
constexpr int kNonTemporal = 2;  // cache-policy bit of the load: streamed once

// vmcnt(4 * n) for the number n of later tiles still in flight
__device__ __forceinline__ void wait_tiles_behind(int n)
{
    if (n <= 0) wait_vmcnt<0>();
    else if (n == 1) wait_vmcnt<4>();
    else if (n == 2) wait_vmcnt<8>();
    else wait_vmcnt<12>();
}

}  // namespace

// Three waves per SIMD (at most 168 VGPRs) with two ring stages measured
// fastest (6.81 TB/s); two waves with four stages and four waves with two
// stages were slower.
#ifndef MAXSIM_VARLEN_WAVES_PER_EU
#define MAXSIM_VARLEN_WAVES_PER_EU 3
#endif
template <int E, bool ARGMAX, int NTQ>
__global__ __launch_bounds__(kUnitsPerBlock * 64)
__attribute__((amdgpu_waves_per_eu(MAXSIM_VARLEN_WAVES_PER_EU))) void fwd_varlen_kernel(VarlenArgs a)
{
    constexpr int KS = kD / 32;  // 16x16x32: 4 K-steps
    static_assert(KS == 4, "one lds_read4 per tile");
    __shared__ __attribute__((aligned(16))) unsigned char ring_lds[kUnitsPerBlock][kStages][kTileBytes];
    const int lane = lane_id();
    const int col = lane & 15;  // query token within an N-tile / doc row within a tile
    const int g = lane >> 4;    // row group: this lane owns tile rows 4g .. 4g+3

    const int unit = blockIdx.x * kUnitsPerBlock + (threadIdx.x >> 6);
    const int U = a.units;
    if (unit >= U) return;

    // a unit is a range of whole docs scored against every query, or with a
    // pair list the one listed (query, doc) pair `unit`
    const bool pairs = a.pair_q != nullptr;
    const int Nd = (int)a.Nd;
    int jb, je, iq = 0;
    if (pairs) {
        const int32_t pq = a.pair_q[unit], pd = a.pair_d[unit];
        iq = uniform(pq < 0 ? 0 : (pq >= a.Nq ? (int)a.Nq - 1 : pq));  // precondition guard
        jb = uniform(pd < 0 ? 0 : (pd >= Nd ? Nd - 1 : pd));
        je = jb + 1;
    } else {
        const int64_t T = a.cu_d[Nd];
        jb = unit == 0 ? 0 : nearest_boundary(a.cu_d, Nd, (T * unit) / U);
        je = unit + 1 == U ? Nd : nearest_boundary(a.cu_d, Nd, (T * (unit + 1)) / U);
    }
    if (jb >= je) return;

    // token range of the unit; offsets below are relative to u0 and fit int32
    const int64_t u0 = a.cu_d[jb];
    const int span = uniform((int)((int64_t)a.cu_d[je] - u0));
    const int ntile = (span + 15) >> 4;
    const unsigned char* unit_ptr = (const unsigned char*)a.D + u0 * kRowBytes;

    // per-lane byte offsets inside a tile for the 4 load instructions: slot
    // (row 4k + lane/16, chunk lane%16) holds logical chunk (lane%16) ^ row
    int load_row[4], load_off[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        load_row[k] = 4 * k + g;
        load_off[k] = load_row[k] * kRowBytes + ((col ^ load_row[k]) * 16);
    }
    unsigned char* ring = &ring_lds[threadIdx.x >> 6][0][0];
    const uint32_t ring_base = lds_addr(ring);
    // A-operand read offsets: row = lane % 16, logical chunk 4k + g
    uint32_t frag_off[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k) frag_off[k] = col * kRowBytes + (((4 * k + g) ^ col) * 16);

    auto issue_tile = [&](int t, int stage) {
        const unsigned char* tp = unit_ptr + (int64_t)t * kTileBytes;
        unsigned char* sb = ring + stage * kTileBytes;
        const int rows_left = span - t * 16;  // rows of this tile inside the unit
        if (rows_left >= 16) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                __builtin_amdgcn_global_load_lds((const void*)(tp + load_off[k]),
                                                 LDS_PTR(sb + k * 1024), 16, 0, kNonTemporal);
        } else {  // last tile: rows past the unit re-read its last row (never folded)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int r = load_row[k] < rows_left ? load_row[k] : rows_left - 1;
                __builtin_amdgcn_global_load_lds(
                    (const void*)(tp + r * kRowBytes + ((col ^ load_row[k]) * 16)),
                    LDS_PTR(sb + k * 1024), 16, 0, kNonTemporal);
            }
        }
    };

    const int64_t i_begin = pairs ? iq : blockIdx.y, i_end = pairs ? iq + 1 : a.Nq;
    const int64_t i_step = pairs ? 1 : gridDim.y;
    for (int64_t i = i_begin; i < i_end; i += i_step) {
        const int64_t q0 = a.cu_q[i];
        int64_t lq64 = (int64_t)a.cu_q[i + 1] - q0;
        if (lq64 > a.max_lq) lq64 = a.max_lq;
        if (lq64 < 0) lq64 = 0;
        const int lq = uniform((int)lq64);
        const int npass = lq == 0 ? 1 : (lq + 16 * NTQ - 1) / (16 * NTQ);
        // outputs of doc j are at [j - j_out] of these rows
        const int j_out = pairs ? jb : 0;
        float* score_row = a.scores + (pairs ? (int64_t)unit : i * a.Nd);
        int32_t* arg_row = ARGMAX ? a.argmax + (pairs ? (int64_t)unit : i * a.Nd) * (int64_t)a.max_lq : nullptr;

        for (int pass = 0; pass < npass; ++pass) {
            // ---- query fragments (B operand: col = token, k-quarter g) --------
            i32x4 qf[NTQ][KS];
            bool tok_ok[NTQ];
#pragma unroll
            for (int n = 0; n < NTQ; ++n) {
                const int s = pass * 16 * NTQ + n * 16 + col;
                tok_ok[n] = s < lq;
                const unsigned char* qrow = (const unsigned char*)a.Q + (q0 + (tok_ok[n] ? s : 0)) * kRowBytes;
#pragma unroll
                for (int k = 0; k < KS; ++k) {
                    i32x4 v = {0, 0, 0, 0};
                    if (tok_ok[n]) v = *(const i32x4*)(qrow + (4 * k + g) * 16);
                    qf[n][k] = v;
                }
            }

            // ---- doc cursor: cu_d cached one value per lane, read with readlane
            int j = jb;
            int cache_base = jb + 1;  // lane k holds cu_d[cache_base + k] - u0
            int cu_cache = (int)((int64_t)a.cu_d[cache_base + lane <= Nd ? cache_base + lane : Nd] - u0);
            wait_vmcnt<0>();  // query fragments and the cache have landed
            auto doc_end_of = [&](int jj) -> int {  // cu_d[jj + 1] - u0
                int off = jj + 1 - cache_base;
                if (off >= 64) {  // once per 64 docs
                    cache_base = jj + 1;
                    cu_cache = (int)((int64_t)a.cu_d[cache_base + lane <= Nd ? cache_base + lane : Nd] - u0);
                    wait_vmcnt<0>();  // keep the cache out of the tile ring's waits
                    off = 0;
                }
                return uniform(__builtin_amdgcn_readlane(cu_cache, off));
            };
            int doc_start = 0;
            int doc_end = doc_end_of(j);

            float m[NTQ];
            int idx[NTQ];
#pragma unroll
            for (int n = 0; n < NTQ; ++n) {
                m[n] = -__builtin_inff();
                idx[n] = 0;
            }

            // finish doc j: merge the 4 row groups, drop padding lanes, sum, write
            auto finish_doc = [&]() {
                float total = 0.f;
#pragma unroll
                for (int n = 0; n < NTQ; ++n) {
                    float mv = m[n];
                    int iv = idx[n];
#pragma unroll
                    for (int off = 16; off <= 32; off <<= 1) {
                        const float om = shfl_xor_f(mv, off);
                        if constexpr (ARGMAX) {
                            const int oi = shfl_xor_i(iv, off);
                            argmax_merge(mv, iv, om, oi);
                        } else {
                            mv = __builtin_fmaxf(mv, om);
                        }
                    }
                    const bool fin = __builtin_isfinite(mv);
                    total += row16_sum((tok_ok[n] && fin) ? mv : 0.f);
                    if constexpr (ARGMAX) {
                        if (g == 0 && tok_ok[n]) {
                            const int s = pass * 16 * NTQ + n * 16 + col;
                            arg_row[(int64_t)(j - j_out) * a.max_lq + s] = fin ? iv - doc_start : 0;
                        }
                    }
                    m[n] = -__builtin_inff();
                    idx[n] = 0;
                }
                if constexpr (ARGMAX) {
                    if (pass == 0)  // rows past the query's length are 0
                        for (int s = lq + lane; s < a.max_lq; s += 64) arg_row[(int64_t)(j - j_out) * a.max_lq + s] = 0;
                }
                if (lane == 0) score_row[j - j_out] = pass == 0 ? total : score_row[j - j_out] + total;
            };

            // fold tile rows [lo, hi) (tile-relative, uniform) into the state
            auto fold = [&](const f32x4 (&acc)[NTQ], int tile0, int lo, int hi) {
                if (lo == 0 && hi == 16) {
#pragma unroll
                    for (int n = 0; n < NTQ; ++n) {
                        if constexpr (ARGMAX) {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                if (acc[n][r] > m[n]) {
                                    m[n] = acc[n][r];
                                    idx[n] = tile0 + 4 * g + r;
                                }
                        } else {
                            m[n] = __builtin_fmaxf(__builtin_fmaxf(m[n], acc[n][0]),
                                                   __builtin_fmaxf(__builtin_fmaxf(acc[n][1], acc[n][2]), acc[n][3]));
                        }
                    }
                } else {
                    const uint32_t bits = ((1u << hi) - 1u) & ~((1u << lo) - 1u);
                    const uint32_t lb = bits >> (4 * g);
#pragma unroll
                    for (int n = 0; n < NTQ; ++n) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float v = ((lb >> r) & 1u) ? acc[n][r] : -__builtin_inff();
                            if constexpr (ARGMAX) {
                                if (v > m[n]) {
                                    m[n] = v;
                                    idx[n] = tile0 + 4 * g + r;
                                }
                            } else {
                                m[n] = __builtin_fmaxf(m[n], v);
                            }
                        }
                    }
                }
            };

            // leading empty docs
            while (j < je && doc_end <= 0) {
                finish_doc();
                ++j;
                if (j < je) {
                    doc_start = doc_end;
                    doc_end = doc_end_of(j);
                }
            }

#pragma unroll
            for (int q = 0; q < kStages; ++q)
                if (q < ntile) issue_tile(q, q);

            int stage = 0;
            for (int t = 0; t < ntile && j < je; ++t) {
                const int behind = ntile - 1 - t;
                wait_tiles_behind(behind < kStages - 1 ? behind : kStages - 1);
                i32x4 af[KS];
                const uint32_t sbase = ring_base + stage * kTileBytes;
                lds_read4(af[0], af[1], af[2], af[3], sbase + frag_off[0], sbase + frag_off[1],
                          sbase + frag_off[2], sbase + frag_off[3]);
                if (t + kStages < ntile) issue_tile(t + kStages, stage);
                stage = stage + 1 == kStages ? 0 : stage + 1;

                f32x4 acc[NTQ];
#pragma unroll
                for (int n = 0; n < NTQ; ++n) {
                    acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int k = 0; k < KS; ++k) acc[n] = mfma16<E>(af[k], qf[n][k], acc[n]);
                }

                const int tile0 = t * 16;
                int lo = 0;
                while (true) {
                    const int hi = doc_end - tile0 < 16 ? doc_end - tile0 : 16;
                    if (hi > lo) fold(acc, tile0, lo, hi);
                    if (doc_end - tile0 > 16) break;  // the doc continues in the next tile
                    finish_doc();
                    ++j;
                    if (j >= je) break;
                    lo = hi > lo ? hi : lo;
                    doc_start = doc_end;
                    doc_end = doc_end_of(j);
                }
            }
            // docs left with no tokens (only when the unit has no tiles)
            while (j < je) {
                finish_doc();
                ++j;
                if (j < je) {
                    doc_start = doc_end;
                    doc_end = doc_end_of(j);
                }
            }
            wait_vmcnt<0>();  // nothing of this pass is still in flight
        }
    }
}

template <int E, int NTQ>
static hipError_t launch_varlen_t(VarlenArgs a, hipStream_t stream)
{
    const bool am = a.argmax != nullptr;
    auto kern = am ? fwd_varlen_kernel<E, true, NTQ> : fwd_varlen_kernel<E, false, NTQ>;
    static std::atomic<int> per_cu_cache[2];  // resident workgroups per CU, by argmax
    int per_cu = per_cu_cache[am ? 1 : 0].load(std::memory_order_relaxed);
    if (per_cu <= 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kUnitsPerBlock * 64, 0) != hipSuccess ||
            per_cu <= 0)
            per_cu = 1;
        per_cu_cache[am ? 1 : 0].store(per_cu, std::memory_order_relaxed);
    }
    // Units of at least kMinDocsPerUnit docs (the per-unit setup stays
    // amortised); given enough docs, a whole number (up to kMaxRounds) of
    // rounds of the resident slots, so that no round runs part-empty and the
    // workgroups that finish early take the next units off the tail. At the
    // 100,000-doc reranking shape 16 rounds of ~2.5-doc units measured 3.5 %
    // faster than one round of ~33-doc units; a round count that leaves a
    // part-filled last round lost that gain.
    constexpr int64_t kMinDocsPerUnit = 2, kMaxRounds = 16;
    const int64_t slots = (int64_t)device_cu_count() * per_cu * kUnitsPerBlock;
    int64_t units = a.Nd / kMinDocsPerUnit;
    if (units >= slots) {
        const int64_t rounds = units / slots < kMaxRounds ? units / slots : kMaxRounds;
        units = rounds * slots;
    }
    if (units < 1) units = 1;
    int64_t gy = a.Nq < 65535 ? a.Nq : 65535;
    if (a.pair_q) {  // one unit per listed pair
        units = a.npairs;
        gy = 1;
    }
    a.units = (int32_t)units;
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
