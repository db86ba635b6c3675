// Chamfer distance forward for gfx950 ("Flash-MaxSim" Sec. 4.2.4): for every
// point of one set, the squared Euclidean distance to the nearest point of the
// other set and its index (lowest index on ties), streamed with an online
// min instead of the materialised [N, M] distance matrix; then the per-batch
// loss (1/N) sum dist1 + (1/M) sum dist2 in a fixed order.
//
// Design: the search for the nearest point runs on the matrix cores. The pages
// obtain Chamfer from MaxSim by putting a squared distance where the inner
// product was, so the distance tile is formed as a contraction: ||s - t||^2 =
// ||s||^2 + (||t||^2 - 2 <s, t>), where the bracket is one
// v_mfma_f32_16x16x4_f32 per 16 x 16 tile with the targets (tx, ty, tz,
// ||t||^2) as rows of A and the sources (-2 sx, -2 sy, -2 sz, 1) as columns of
// B (K = 4, fp32 in and out). Coordinates are first taken relative to the
// mean of the target set's first 64 points, so the rounding scales with the
// sets' extent rather than their offset from the origin.
//
// The expanded form cancels: its rounding error is of the order of u |s'|^2,
// far above that of the direct form sum_k (s_k - t_k)^2 when the nearest
// distance is small. So the matrix-core pass only finds candidates, and the
// answer is decided in the direct form: a lane owns one source column and 4
// target rows of each tile, and per 256-target tile it folds its 64 values
// into the tile's min. Two slots keep the tiles whose min lies within the
// expanded form's rounding bound tau(b) of the running min b (the best tile
// and one more); a third tile inside the window while both slots are still
// inside it marks the source as overflowed. At the end every kept tile whose
// min is within tau of the source's overall min (over the 4 lanes of the
// column) is re-evaluated row by row in the direct form from the raw fp32
// coordinates, and the smallest direct value wins, lowest index on ties. The
// exact nearest point is always among the re-evaluated rows, so the returned
// index is one a direct-form fp32 evaluation could return, and the distance
// written is that evaluation. An overflowed source is written with index -1,
// and chamfer_fix_kernel then scans its whole target set in the direct form.
//
// Every wave is its own workgroup and streams its own copy of the target set
// through LDS in 256-point tiles (coalesced loads, prepared as
// (x, y, z, ||t||^2), double-buffered), so no barriers are needed. The
// sources of all batches and both directions form one list of 16-point
// blocks; wave w takes a contiguous run of blocks (the runs differ by at most
// one block), cut where a (batch, direction) segment ends, and holds up to
// kChMaxBlocks blocks in registers, so every target tile feeds that many
// MFMAs per LDS read.
#include <atomic>

#include "common.hpp"
#include "kernels.hpp"

namespace maxsim {

namespace {

constexpr int kChTileT = 256;    // target points per LDS tile
constexpr int kChMaxBlocks = 5;  // 16-point source blocks a wave holds at once
typedef float f4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void cham_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// LDS of one wave: two prepared tiles and the raw coordinates being prepared
struct ChamLds {
    f4v tile[2][kChTileT];
    float raw[kChTileT * 3];
};

// Coordinates [t0*3, t0*3 + 768) of a target set with nt points, one float
// per (lane, m) at 64*m + lane: every load instruction reads 256 contiguous
// bytes. Past the set's end the value is 0.
__device__ __forceinline__ void cham_load_raw(const float* __restrict__ T, int64_t nt, int64_t t0, int lane,
                                              float (&r)[12])
{
    const int64_t lim = nt * 3, base = t0 * 3;
#pragma unroll
    for (int m = 0; m < 12; ++m) {
        const int64_t f = base + 64 * m + lane;
        r[m] = f < lim ? T[f] : 0.f;
    }
}

// Raw coordinates -> tile entries (x, y, z, ||t||^2); points past the set's
// end get ||t||^2 = +inf, so their distance is +inf and never wins.
__device__ __forceinline__ void cham_prepare(ChamLds& sm, int buf, const float (&r)[12], int64_t nt, int64_t t0,
                                             int lane, float cx, float cy, float cz)
{
#pragma unroll
    for (int m = 0; m < 12; ++m) sm.raw[64 * m + lane] = r[m];
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's writes are visible to its reads
    // lane l prepares points l, l+64, l+128, l+192 (odd word stride between
    // lanes: no LDS bank conflicts)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int p = lane + 64 * u;  // point of the tile
        const float x = sm.raw[3 * p] - cx, y = sm.raw[3 * p + 1] - cy, z = sm.raw[3 * p + 2] - cz;
        const float n2 = t0 + p < nt ? __builtin_fmaf(z, z, __builtin_fmaf(y, y, x * x)) : __builtin_inff();
        sm.tile[buf][p] = f4v{x, y, z, n2};
    }
}

}  // namespace

// Near-tie window of the matrix-core pass. For a source s' (coordinates
// relative to the centring point) whose running min of the bracket
// ||t'||^2 - 2 <s', t'> is b, a target t can still be the exact nearest point
// only if its bracket is at most thr(b) = b + 2^-18 (18 |s'|^2 + 12 b). This
// holds for any rounding with unit u <= 2^-23 of: the centring differences,
// ||t'||^2 (two fused steps), and a 4-term fp32 dot product with any order of
// its products and sums. For such a t the error of the bracket is at most
// gamma_12 ((|s'| + |t'|)^2 + |s - t|^2) with |t'| <= |s'| + |s - t|, and the
// window is twice that bound for both the true and the found minimum, written
// with b + |s'|^2 in place of the distance.
constexpr float kTauK = 1.0f + 12.0f * 0x1p-18f;
constexpr float kTau0 = 18.0f * 0x1p-18f;

// 4 consecutive points (12 floats), read with one 48-byte copy
struct __attribute__((aligned(4))) ChRows4 {
    float v[12];
};

// KN source blocks of one (batch, direction) segment against its whole
// target set: A [na, 3] holds the sources, blocks k0 .. k0+KN-1; T [nt, 3]
// the targets. Writes dist[sp] and idx[sp] for the blocks' points, or
// idx[sp] = -1 when the source's near-tie candidates overflowed.
template <int KN>
__device__ __forceinline__ void cham_piece(ChamLds& sm, const float* __restrict__ A, int64_t na,
                                           const float* __restrict__ T, int64_t nt, int64_t k0,
                                           float* __restrict__ dist, int32_t* __restrict__ idx)
{
    const int lane = threadIdx.x;
    const int col = lane & 15, rg = lane >> 4;  // source column, target row group (= K index of A, B)
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    // centring point: the mean of the target set's first (up to) 64 points.
    // The butterfly sum gives every lane the same bits; the distances do not
    // depend on it, only the expanded form's rounding does.
    float cx, cy, cz;
    {
        const int m = (int)(nt < 64 ? nt : 64);
        float x = 0.f, y = 0.f, z = 0.f;
        if (lane < m) {
            x = T[lane * 3];
            y = T[lane * 3 + 1];
            z = T[lane * 3 + 2];
        }
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            x += __shfl_xor(x, o, 64);
            y += __shfl_xor(y, o, 64);
            z += __shfl_xor(z, o, 64);
        }
        const float inv = 1.0f / (float)m;
        cx = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x * inv)));
        cy = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(y * inv)));
        cz = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(z * inv)));
    }

    // per source of each block (clamped copies past the end): the B operand,
    // the window constant, the running min and its tile, the second kept tile
    float bop[KN], tau0[KN], best[KN], v1[KN];
    int s0[KN], s1[KN];
    bool ovf[KN];
#pragma unroll
    for (int u = 0; u < KN; ++u) {
        int64_t sp = (k0 + u) * 16 + col;
        sp = sp < na ? sp : na - 1;
        const float sx = A[sp * 3] - cx, sy = A[sp * 3 + 1] - cy, sz = A[sp * 3 + 2] - cz;
        const float comp = rg == 0 ? sx : (rg == 1 ? sy : sz);
        bop[u] = rg < 3 ? -2.f * comp : 1.f;
        tau0[u] = kTau0 * __builtin_fmaf(sz, sz, __builtin_fmaf(sy, sy, sx * sx));
        best[u] = __builtin_inff();
        v1[u] = __builtin_inff();
        s0[u] = 0;
        s1[u] = 0;
        ovf[u] = false;
    }

    const int64_t ntiles = (nt + kChTileT - 1) / kChTileT;
    float raw[12];
    cham_load_raw(T, nt, 0, lane, raw);
    cham_prepare(sm, 0, raw, nt, 0, lane, cx, cy, cz);
    for (int64_t it = 0; it < ntiles; ++it) {
        const int64_t t0 = it * kChTileT;
        const int buf = (int)(it & 1);
        if (it + 1 < ntiles) cham_load_raw(T, nt, t0 + kChTileT, lane, raw);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the tile is prepared
        const int64_t left = nt - t0;
        const int tbs = __builtin_amdgcn_readfirstlane(left >= kChTileT ? kChTileT / 16 : (int)((left + 15) / 16));
        const float* tf = (const float*)&sm.tile[buf][0] + col * 4 + rg;  // A[row col][k rg] of block 0
        // mp: this tile's min of the lane's rows, per source
        float mp[KN];
        if (tbs == kChTileT / 16) {
            // a full tile: every block's operand is read up front, and the
            // blocks go in pairs, the MFMAs issued at raised priority (the
            // SIMD's other waves yield the issue slots to the MFMA stream)
            float av[kChTileT / 16];
#pragma unroll
            for (int tb = 0; tb < kChTileT / 16; ++tb) av[tb] = tf[tb * 64];
#pragma unroll
            for (int tb = 0; tb < kChTileT / 16; tb += 2) {
                f32x4 d[KN], e[KN];
                __builtin_amdgcn_s_setprio(1);
#pragma unroll
                for (int u = 0; u < KN; ++u) d[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[tb], bop[u], zero, 0, 0, 0);
#pragma unroll
                for (int u = 0; u < KN; ++u) e[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[tb + 1], bop[u], zero, 0, 0, 0);
                __builtin_amdgcn_s_setprio(0);
#pragma unroll
                for (int u = 0; u < KN; ++u) {
                    const float x = __builtin_fminf(__builtin_fminf(d[u][0], d[u][1]), d[u][2]);
                    const float y = __builtin_fminf(__builtin_fminf(d[u][3], e[u][0]), e[u][1]);
                    if (tb == 0) {
                        mp[u] = __builtin_fminf(__builtin_fminf(__builtin_fminf(e[u][2], e[u][3]), x), y);
                    } else {
                        const float z = __builtin_fminf(__builtin_fminf(e[u][2], e[u][3]), mp[u]);
                        mp[u] = __builtin_fminf(__builtin_fminf(x, y), z);
                    }
                }
            }
        } else {
#pragma unroll
            for (int u = 0; u < KN; ++u) mp[u] = __builtin_inff();
            for (int tb = 0; tb < tbs; ++tb) {
                const float aop = tf[tb * 64];
#pragma unroll
                for (int u = 0; u < KN; ++u) {
                    const f32x4 d = __builtin_amdgcn_mfma_f32_16x16x4f32(aop, bop[u], zero, 0, 0, 0);
                    mp[u] = __builtin_fminf(__builtin_fminf(__builtin_fminf(d[0], d[1]), __builtin_fminf(d[2], d[3])),
                                            mp[u]);
                }
            }
        }
        // the two kept tiles: a tile inside the window of the running min is
        // kept; a lower tile becomes the best and the old best the second; a
        // third tile inside the window while the second is still inside it
        // overflows. Equal mins keep the earlier tile as the best.
        const int step = (int)it;
#pragma unroll
        for (int u = 0; u < KN; ++u) {
            const float thr_old = __builtin_fmaf(best[u], kTauK, tau0[u]);
            const bool near = mp[u] <= thr_old;
            const bool lower = mp[u] < best[u];
            const float bn = __builtin_fminf(best[u], mp[u]);
            const float thr_new = __builtin_fmaf(bn, kTauK, tau0[u]);
            ovf[u] = ovf[u] | (near & (v1[u] <= thr_new));  // bitwise: no branches
            v1[u] = near ? __builtin_fmaxf(best[u], mp[u]) : v1[u];
            s1[u] = near ? (lower ? s0[u] : step) : s1[u];
            s0[u] = lower ? step : s0[u];
            best[u] = bn;
        }
        if (it + 1 < ntiles) cham_prepare(sm, buf ^ 1, raw, nt, t0 + kChTileT, lane, cx, cy, cz);
    }

    // the answer in the direct form: the kept tiles inside the window of the
    // source's overall min are re-evaluated on this lane's rows from the raw
    // coordinates; the smallest value wins, the lowest index on ties, then
    // the 4 row groups of the column are merged the same way
#pragma unroll
    for (int u = 0; u < KN; ++u) {
        int64_t sp = (k0 + u) * 16 + col;
        const bool own = sp < na;
        sp = own ? sp : na - 1;
        const float px = A[sp * 3], py = A[sp * 3 + 1], pz = A[sp * 3 + 2];
        float bs = best[u];
        bs = __builtin_fminf(bs, __shfl_xor(bs, 16, 64));
        bs = __builtin_fminf(bs, __shfl_xor(bs, 32, 64));
        const float thr = __builtin_fmaf(bs, kTauK, tau0[u]);
        int lost = (ovf[u] & (best[u] <= thr)) ? 1 : 0;
        lost |= __shfl_xor(lost, 16, 64);
        lost |= __shfl_xor(lost, 32, 64);
        float dv = __builtin_inff();
        int di = 0x7fffffff;
        // The column's tasks are the kept tiles of its 4 lanes: bit 2j + slot
        // is set when lane j keeps that slot (j = the lane's row group). Each
        // task's 64 rows (rows 4j .. 4j+3 of the tile's 16 blocks) are split
        // over the column's 4 lanes, lane rg taking blocks 4rg .. 4rg+3, so a
        // wave makes one pass of 16 rows per task of its busiest column.
        const int mine = ((best[u] <= thr) ? 1 : 0) | ((v1[u] <= thr) ? 2 : 0);
        int mask = mine << (2 * rg);
        mask |= __shfl_xor(mask, 16, 64);
        mask |= __shfl_xor(mask, 32, 64);
        int tile[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            tile[2 * j] = __shfl(s0[u], col + 16 * j, 64);
            tile[2 * j + 1] = __shfl(s1[u], col + 16 * j, 64);
        }
        while (__any(mask != 0)) {
            if (mask != 0) {
                const int q = __builtin_ctz(mask);
                mask &= mask - 1;
                int tq = tile[0];
#pragma unroll
                for (int k = 1; k < 8; ++k) tq = q == k ? tile[k] : tq;
                const int64_t tb = (int64_t)tq * kChTileT + 4 * (q >> 1) + 64 * rg;
                ChRows4 x[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int64_t t = tb + 16 * k;
                    if (t + 3 < nt) __builtin_memcpy(&x[k], T + t * 3, sizeof(ChRows4));
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int64_t t = tb + 16 * k;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float tx, ty, tz;
                        if (t + 3 < nt) {
                            tx = x[k].v[3 * r];
                            ty = x[k].v[3 * r + 1];
                            tz = x[k].v[3 * r + 2];
                        } else if (t + r < nt) {
                            tx = T[(t + r) * 3];
                            ty = T[(t + r) * 3 + 1];
                            tz = T[(t + r) * 3 + 2];
                        } else {
                            continue;
                        }
                        const float dx = px - tx, dy = py - ty, dz = pz - tz;
                        const float v = __builtin_fmaf(dz, dz, __builtin_fmaf(dy, dy, dx * dx));
                        if (v < dv || (v == dv && (int)(t + r) < di)) {
                            dv = v;
                            di = (int)(t + r);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int x = 16; x <= 32; x <<= 1) {
            const float ov = __shfl_xor(dv, x, 64);
            const int oi = __shfl_xor(di, x, 64);
            if (ov < dv || (ov == dv && oi < di)) {
                dv = ov;
                di = oi;
            }
        }
        if (rg == 0 && own) {
            if (lost) {
                idx[sp] = -1;
            } else {
                dist[sp] = dv;
                idx[sp] = di;
            }
        }
    }
}

// Sources whose near-tie candidates overflowed (index -1): the whole target
// set in the direct form, the smallest value and the lowest index among equal
// ones. A workgroup checks kFixThreads consecutive sources of the list
// [dist1 | dist2], lists the overflowed ones in order, and takes them in
// groups of up to kFixGroup that share a target set (one batch and
// direction): one pass over the set serves the whole group. Wave w takes
// every 16th run of kFixRun points, reads the run's coordinates with
// consecutive-dword loads (each instruction 256 contiguous bytes) into its own
// LDS stage, and its lanes evaluate the run's points in ascending order.
constexpr int kFixThreads = 1024, kFixRun = 512, kFixGroup = 8;
__global__ __launch_bounds__(kFixThreads) void chamfer_fix_kernel(ChamferArgs a)
{
    constexpr int kWavesFix = kFixThreads / 64;
    __shared__ int list[kFixThreads];
    __shared__ int wcount[kWavesFix];
    __shared__ float stage[kWavesFix][kFixRun * 3];
    __shared__ float wv[kFixGroup][kWavesFix];
    __shared__ int wi[kFixGroup][kWavesFix];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t n1 = a.B * a.N, ntot = n1 + a.B * a.M;
    const int64_t g0 = (int64_t)blockIdx.x * kFixThreads;
    // the overflowed sources of this workgroup, in order
    const int64_t g = g0 + tid;
    bool flagged = false;
    if (g < ntot) flagged = (g < n1 ? a.idx1[g] : a.idx2[g - n1]) < 0;
    const uint64_t bal = __ballot(flagged);
    if (lane == 0) wcount[w] = __builtin_popcountll(bal);
    cham_barrier();
    int nlist = 0, off = 0;
    for (int k = 0; k < kWavesFix; ++k) {
        off += k < w ? wcount[k] : 0;
        nlist += wcount[k];
    }
    if (flagged) list[off + __builtin_popcountll(bal & ((1ull << lane) - 1ull))] = tid;
    cham_barrier();
    float* st = &stage[w][0];
    for (int i0 = 0; i0 < nlist;) {
        // a group: consecutive listed sources of one (batch, direction)
        const int64_t gf = g0 + list[i0];
        const bool second = gf >= n1;
        const int64_t na = second ? a.M : a.N, nt = second ? a.N : a.M;
        const int64_t seg = (second ? gf - n1 : gf) / na;
        int ng = 1;
        while (ng < kFixGroup && i0 + ng < nlist) {
            const int64_t gn = g0 + list[i0 + ng];
            if ((gn >= n1) != second || ((second ? gn - n1 : gn) / na) != seg) break;
            ++ng;
        }
        const float* T = (second ? a.P : a.Q) + seg * nt * 3;
        float px[kFixGroup], py[kFixGroup], pz[kFixGroup], dv[kFixGroup];
        int di[kFixGroup];
#pragma unroll
        for (int k = 0; k < kFixGroup; ++k) {
            const int64_t gk = g0 + list[i0 + (k < ng ? k : 0)];
            const float* S = (second ? a.Q + (gk - n1) * 3 : a.P + gk * 3);
            px[k] = S[0];
            py[k] = S[1];
            pz[k] = S[2];
            dv[k] = __builtin_inff();
            di[k] = 0x7fffffff;
        }
        // ascending targets per lane with a strict '<': the lowest index of a
        // tie stays
        for (int64_t p0 = (int64_t)w * kFixRun; p0 < nt; p0 += (int64_t)kWavesFix * kFixRun) {
            const int64_t lim = nt * 3;
            float v[kFixRun * 3 / 64];
#pragma unroll
            for (int m = 0; m < kFixRun * 3 / 64; ++m) {
                const int64_t f = p0 * 3 + 64 * m + lane;
                v[m] = f < lim ? T[f] : 0.f;
            }
#pragma unroll
            for (int m = 0; m < kFixRun * 3 / 64; ++m) st[64 * m + lane] = v[m];
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's writes are visible to its reads
#pragma unroll 2
            for (int kk = 0; kk < kFixRun / 64; ++kk) {
                const int pl = 64 * kk + lane;  // odd word stride between lanes: no bank conflicts
                const float tx = st[3 * pl], ty = st[3 * pl + 1], tz = st[3 * pl + 2];
                const bool in = p0 + pl < nt;
#pragma unroll
                for (int k = 0; k < kFixGroup; ++k) {
                    if (k < ng) {  // the same for every thread
                        const float dx = px[k] - tx, dy = py[k] - ty, dz = pz[k] - tz;
                        const float d = __builtin_fmaf(dz, dz, __builtin_fmaf(dy, dy, dx * dx));
                        if (in && d < dv[k]) {
                            dv[k] = d;
                            di[k] = (int)(p0 + pl);
                        }
                    }
                }
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // the reads are done before the stage is refilled
        }
#pragma unroll
        for (int k = 0; k < kFixGroup; ++k) {
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) {
                const float ov = __shfl_xor(dv[k], o, 64);
                const int oi = __shfl_xor(di[k], o, 64);
                if (ov < dv[k] || (ov == dv[k] && oi < di[k])) {
                    dv[k] = ov;
                    di[k] = oi;
                }
            }
            if (lane == 0) {
                wv[k][w] = dv[k];
                wi[k][w] = di[k];
            }
        }
        cham_barrier();
        if (tid < ng) {
            float bv = wv[tid][0];
            int bi = wi[tid][0];
            for (int k = 1; k < kWavesFix; ++k)
                if (wv[tid][k] < bv || (wv[tid][k] == bv && wi[tid][k] < bi)) {
                    bv = wv[tid][k];
                    bi = wi[tid][k];
                }
            const int64_t gk = g0 + list[i0 + tid];
            if (second) {
                a.dist2[gk - n1] = bv;
                a.idx2[gk - n1] = bi;
            } else {
                a.dist1[gk] = bv;
                a.idx1[gk] = bi;
            }
        }
        cham_barrier();
        i0 += ng;
    }
}

// One wave per workgroup; see the file comment. Block g of the list is
// source block g of direction 1 (P against Q) for g < B*nb1, else of
// direction 2 (Q against P); each direction is batch-major.
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3))) void chamfer_nn_kernel(ChamferArgs a, int64_t nblocks)
{
    __shared__ ChamLds sm;
    const int64_t nw = gridDim.x, w = blockIdx.x;
    const int64_t nb1 = (a.N + 15) / 16, nb2 = (a.M + 15) / 16;
    const int64_t g_first = w * nblocks / nw, g_last = (w + 1) * nblocks / nw;

    for (int64_t g0 = g_first; g0 < g_last;) {
        // the segment (batch, direction) holding g0 and the piece of it taken now
        const bool second = g0 >= a.B * nb1;
        const int64_t nb = second ? nb2 : nb1;
        const int64_t gl = second ? g0 - a.B * nb1 : g0;
        const int64_t b = gl / nb, k0 = gl % nb;
        int64_t nk = nb - k0;
        if (nk > g_last - g0) nk = g_last - g0;
        if (nk > kChMaxBlocks) nk = kChMaxBlocks;
        g0 += nk;
        const int64_t na = second ? a.M : a.N, nt = second ? a.N : a.M;
        const float* A = (second ? a.Q : a.P) + b * na * 3;
        const float* T = (second ? a.P : a.Q) + b * nt * 3;
        float* dist = (second ? a.dist2 : a.dist1) + b * na;
        int32_t* idx = (second ? a.idx2 : a.idx1) + b * na;
        switch (__builtin_amdgcn_readfirstlane((int)nk)) {
        case 1: cham_piece<1>(sm, A, na, T, nt, k0, dist, idx); break;
        case 2: cham_piece<2>(sm, A, na, T, nt, k0, dist, idx); break;
        case 3: cham_piece<3>(sm, A, na, T, nt, k0, dist, idx); break;
        case 4: cham_piece<4>(sm, A, na, T, nt, k0, dist, idx); break;
        default: cham_piece<5>(sm, A, na, T, nt, k0, dist, idx); break;
        }
    }
}

// loss[b] = (1/N) sum_p dist1[b,p] + (1/M) sum_q dist2[b,q] in a fixed order:
// thread t keeps kLossUnroll partial sums, partial j over the elements
// t + kLossThreads*(kLossUnroll*k + j) for k ascending (so kLossUnroll loads
// are in flight), adds them in j order, then a fixed tree over the workgroup.
constexpr int kLossThreads = 1024, kLossUnroll = 16;
__device__ __forceinline__ float cham_sum(const float* __restrict__ x, int64_t n, int tid)
{
    float part[kLossUnroll];
#pragma unroll
    for (int j = 0; j < kLossUnroll; ++j) part[j] = 0.f;
    for (int64_t p = tid; p < n; p += (int64_t)kLossThreads * kLossUnroll) {
        // every load is issued (clamped in range) before any is used
        float v[kLossUnroll];
#pragma unroll
        for (int j = 0; j < kLossUnroll; ++j) {
            const int64_t q = p + (int64_t)j * kLossThreads;
            v[j] = x[q < n ? q : n - 1];
        }
#pragma unroll
        for (int j = 0; j < kLossUnroll; ++j)
            if (p + (int64_t)j * kLossThreads < n) part[j] += v[j];
    }
    float s = part[0];
#pragma unroll
    for (int j = 1; j < kLossUnroll; ++j) s += part[j];
    return s;
}
__global__ __launch_bounds__(kLossThreads) void chamfer_loss_kernel(const float* __restrict__ dist1,
                                                                    const float* __restrict__ dist2,
                                                                    int64_t N, int64_t M, float* __restrict__ loss)
{
    __shared__ float red[2][kLossThreads];
    const int64_t b = blockIdx.x;
    const int tid = threadIdx.x;
    red[0][tid] = cham_sum(dist1 + b * N, N, tid);
    red[1][tid] = cham_sum(dist2 + b * M, M, tid);
    cham_barrier();
    for (int off = kLossThreads / 2; off > 0; off >>= 1) {
        if (tid < off) {
            red[0][tid] += red[0][tid + off];
            red[1][tid] += red[1][tid + off];
        }
        cham_barrier();
    }
    if (tid == 0) loss[b] = red[0][0] / (float)N + red[1][0] / (float)M;
}

hipError_t launch_chamfer_fwd(ChamferArgs a, hipStream_t stream)
{
    if (a.B == 0) return hipSuccess;
    hipError_t err;
    // one wave per workgroup and as many waves as are resident at once (the
    // runs of blocks then end together); each wave holds at most
    // kChMaxBlocks source blocks, so larger inputs get more waves
    static std::atomic<int> per_cu{0};
    int occ = per_cu.load(std::memory_order_relaxed);
    if (occ <= 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, chamfer_nn_kernel, 64, 0) != hipSuccess || occ <= 0)
            occ = 8;
        per_cu.store(occ, std::memory_order_relaxed);
    }
    const int64_t nblocks = a.B * ((a.N + 15) / 16 + (a.M + 15) / 16);
    int64_t waves = (int64_t)occ * device_cu_count();
    if (waves * kChMaxBlocks < nblocks) waves = (nblocks + kChMaxBlocks - 1) / kChMaxBlocks;
    if (waves > nblocks) waves = nblocks;
    if (waves > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(chamfer_nn_kernel, dim3((unsigned)waves), dim3(64), 0, stream, a, nblocks);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const int64_t nsrc = a.B * (a.N + a.M);
    hipLaunchKernelGGL(chamfer_fix_kernel, dim3((unsigned)((nsrc + kFixThreads - 1) / kFixThreads)),
                       dim3(kFixThreads), 0, stream, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (a.loss) {
        hipLaunchKernelGGL(chamfer_loss_kernel, dim3((unsigned)a.B), dim3(kLossThreads), 0, stream, a.dist1,
                           a.dist2, a.N, a.M, a.loss);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace maxsim
