// Chamfer distance forward for gfx950 ("Flash-MaxSim" Sec. 4.2.4): for every
// point of one set, the squared Euclidean distance to the nearest point of the
// other set and its index (lowest index on ties), streamed with an online
// min instead of the materialised [N, M] distance matrix; then the per-batch
// loss (1/N) sum dist1 + (1/M) sum dist2 in a fixed order.
//
// Design: the search for the nearest point runs on the matrix cores. The pages
// obtain Chamfer from MaxSim by putting a squared distance where the inner
// product was, so the distance tile is formed as a contraction: ||s - t||^2 =
// ||s||^2 + (||t||^2 - 2 <s, t>). Coordinates are first taken relative to the
// mean of the target set's first 64 points (so the rounding scales with the
// sets' extent rather than their offset from the origin), and each of the
// target's x, y, z, ||t||^2 and the source's -2x, -2y, -2z is split into two
// bf16 parts, hi = bf16(v) and lo = bf16(v - hi). One
// v_mfma_f32_32x32x16_bf16 then gives the bracket of a 32 x 32 tile (targets
// as rows of A, sources as columns of B) from the hi x hi, lo x hi and
// hi x lo products of the coordinates and the two parts of ||t||^2, 11 of its
// 16 K slots: four times the values per matrix-core cycle of an fp32
// 16x16x4 MFMA, with a rounding bound of order 2^-14 |s'|^2 (the dropped
// lo x lo products and the parts' own rounding) instead of 2^-21 |s'|^2.
//
// That search form cancels: its rounding error is far above that of the
// direct form sum_k (s_k - t_k)^2 when the nearest distance is small. So the
// matrix-core pass only finds candidates, and the answer is decided in the
// direct form: a lane owns one source column and 16 target rows of each
// 32-row block (rows 8 g + 4 h + r, h = lane / 32), and per 256-target tile
// it folds its 128 values into the tile's min. Three slots keep the tiles
// whose min lies within the search form's rounding window thr(b) of the
// running min b (the best tile and two more); a fourth tile inside the window
// while the oldest kept one is still inside it marks the source as
// overflowed. At the end every kept tile whose min is within the window of
// the source's overall min (over the column's 2 lanes) is re-evaluated row by
// row in the direct form from the raw fp32 coordinates, and the smallest
// direct value wins, lowest index on ties. The exact nearest point is always
// among the re-evaluated rows, so the returned index is one a direct-form
// fp32 evaluation could return, and the distance written is that evaluation.
// An overflowed source is written with index -1, and chamfer_fix_kernel then
// scans its whole target set in the direct form.
//
// A workgroup of kChWaves waves streams its segment's target set through LDS
// in 256-point tiles (coalesced loads, prepared as two planes of bf16 A rows,
// double-buffered): each wave prepares a quarter of every tile, one tile
// ahead, and one barrier per tile publishes it, so the splitting work is
// shared by the four waves. The sources of all batches and both directions
// form one list of 32-point blocks; workgroup w takes a contiguous run of
// blocks (the runs differ by at most one block) in pieces cut where a (batch,
// direction) segment ends, and each wave holds up to kChMaxBlocks of a
// piece's blocks in registers, so every A row read from LDS feeds that many
// MFMAs.
#include <atomic>

#include "common.hpp"
#include "kernels.hpp"

namespace maxsim {

namespace {

#ifndef MAXSIM_CH_TILE
#define MAXSIM_CH_TILE 256
#endif
#ifndef MAXSIM_CH_BLOCKS
#define MAXSIM_CH_BLOCKS 4
#endif
#ifndef MAXSIM_CH_WAVES
#define MAXSIM_CH_WAVES 2
#endif
constexpr int kChTileT = MAXSIM_CH_TILE;      // target points per LDS tile
constexpr int kChBlk = 32;                    // source points per block (one MFMA column block)
constexpr int kChMaxBlocks = MAXSIM_CH_BLOCKS;  // source blocks a wave holds at once
constexpr int kChRB = kChTileT / 32;          // 32-row blocks per tile
constexpr int kChWaves = 4;                   // waves per workgroup, sharing the target tiles
constexpr int kChQuarter = kChTileT / kChWaves;  // targets each wave prepares per tile
constexpr int kChRaw = kChQuarter * 3 / 64;   // raw coordinates per lane per tile
static_assert(kChQuarter % 64 == 0, "whole targets per lane per tile");
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void cham_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// bits of (__bf16)x | (__bf16)y << 16, both rounded to nearest even
__device__ __forceinline__ uint32_t pk_bf16(float x, float y)
{
    const bf16x2 v = {(__bf16)x, (__bf16)y};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __builtin_bit_cast(float, v & 0xffff0000u); }

// LDS of a workgroup: two prepared tiles, each as two planes of 16-byte
// rows (plane h holds the 8 bf16 of K-half h of every target's A row), and
// each wave's raw coordinates being prepared.
struct ChamLds {
    i32x4 tile[2][2][kChTileT];
    float raw[kChWaves][kChQuarter * 3];
};

// Coordinates of targets [t0, t0 + kChQuarter) of a set with nt points, one float per
// (lane, m) at 64*m + lane: every load instruction reads 256 contiguous
// bytes. Past the set's end the value is 0.
__device__ __forceinline__ void cham_load_raw(const float* __restrict__ T, int64_t nt, int64_t t0, int lane,
                                              float (&r)[kChRaw])
{
    const int64_t lim = nt * 3, base = t0 * 3;
#pragma unroll
    for (int m = 0; m < kChRaw; ++m) {
        const int64_t f = base + 64 * m + lane;
        r[m] = f < lim ? T[f] : 0.f;
    }
}

// Raw coordinates -> A rows. With t' = t - c (fp32) and n = |t'|^2 (fp32),
// each of tx', ty', tz', n is split into bf16 parts hi = bf16(v) and
// lo = bf16(v - hi) (v - hi is exact in fp32), and the row holds
//   K 0..7  (plane 0): hx hy hz lx ly lz hx hy
//   K 8..15 (plane 1): hz nh nl 0 0 0 0 0
// against the source columns' -2 hi / -2 lo parts (cham_piece), so one
// bf16 MFMA gives nh + nl - 2 (<th, sh> + <tl, sh> + <th, sl>). Points past
// the set's end get hi = lo = 0 and nh = +inf: their value is +inf.
// Wave `wave` prepares targets [t0 + q wave, t0 + q wave + q) of the tile at
// t0 (q = kChQuarter) into buffer `buf`, from its coordinates r.
__device__ __forceinline__ void cham_prepare(ChamLds& sm, int buf, const float (&r)[kChRaw], int64_t nt,
                                             int64_t t0, int wave, int lane, float cx, float cy, float cz)
{
    float* raw = sm.raw[wave];
#pragma unroll
    for (int m = 0; m < kChRaw; ++m) raw[64 * m + lane] = r[m];
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's writes are visible to its reads
    // lane l prepares points l, l + 64, ... of the quarter (odd word stride
    // between lanes: no LDS bank conflicts)
#pragma unroll
    for (int v = 0; v < kChQuarter / 64; ++v) {
        const int ql = lane + 64 * v;            // point of the quarter
        const int p = kChQuarter * wave + ql;    // point of the tile
        const bool in = t0 + p < nt;
        const float x = raw[3 * ql] - cx, y = raw[3 * ql + 1] - cy, z = raw[3 * ql + 2] - cz;
        const float n = in ? __builtin_fmaf(z, z, __builtin_fmaf(y, y, x * x)) : 0.f;
        const uint32_t hxy = pk_bf16(x, y), hzn = pk_bf16(z, n);
        const uint32_t lxy = pk_bf16(x - bf16_lo(hxy), y - bf16_hi(hxy));
        const uint32_t lzn = pk_bf16(z - bf16_lo(hzn), n - bf16_hi(hzn));
        const i32x4 p0 = {(int)hxy, (int)((hzn & 0xffffu) | (lxy << 16)), (int)((lxy >> 16) | (lzn << 16)), (int)hxy};
        const i32x4 p1 = {in ? (int)hzn : (int)0x7f800000, in ? (int)(lzn >> 16) : 0, 0, 0};
        sm.tile[buf][0][p] = p0;
        sm.tile[buf][1][p] = p1;
    }
}

}  // namespace

// Near-tie window of the matrix-core pass. For a source s' (coordinates
// relative to the centring point) whose running min of the computed bracket
// b~(t) = |t'|^2 - 2 <s', t'> is b, a target t can still be the exact nearest
// point only if b~(t) <= thr(b) = b + tau (2 |s'|^2 + b). The split form
// above drops the lo x lo products and the parts' rounding (each part
// within 2^-9 of its remainder), and sums 11 exact products in fp32 in any
// order (u <= 2^-23); with the centring differences and the fp32 |t'|^2 this
// puts the computed |s'|^2 + b~(t) within E(t) = 2^-14 (|s'|^2 + |s - t|^2)
// of the exact squared distance, using |t'| <= |s'| + |s - t|. For the exact
// nearest point t* and the found minimum t_f, b~(t*) <= b + 2 E(t_f), and
// E(t_f) <= 2^-14 (2 |s'|^2 + b) / (1 - 2^-14), so tau = 2^-13 / (1 - 2^-14),
// taken 1 % larger for the fp32 rounding of thr itself.
constexpr float kTau = 0x1.03p-13f;
constexpr float kTauK = 1.0f + kTau;

// KN source blocks of one (batch, direction) segment against its whole
// target set: A [na, 3] holds the sources, this wave's blocks are
// k0, k0 + kChWaves, ... (KN of them; KN = 0 for a wave that only helps
// prepare the tiles); T [nt, 3] the targets, streamed by the whole workgroup
// (every wave calls this with the same T, nt, and passes the same number of
// barriers). Writes dist[sp] and idx[sp] for the blocks' points, or
// idx[sp] = -1 when the source's near-tie candidates overflowed.
template <int KN>
__device__ __forceinline__ void cham_piece(ChamLds& sm, const float* __restrict__ A, int64_t na,
                                           const float* __restrict__ T, int64_t nt, int64_t k0,
                                           float* __restrict__ dist, int32_t* __restrict__ idx)
{
    constexpr int KA = KN > 0 ? KN : 1;  // array extent (a KN = 0 wave only prepares tiles)
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int col = lane & 31, h = lane >> 5;  // source column; K-half of the operands, row half of the results
    const f32x16 zero = {};
    // centring point: the mean of the target set's first (up to) 64 points.
    // The butterfly sum gives every lane the same bits; the distances do not
    // depend on it, only the search's rounding does.
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

    // per source of each block (clamped copies past the end): the B operand
    // (K-half h of -2 s' split into bf16 parts: hx hy hz hx hy hz lx ly | lz 1 1 0 ...),
    // the window constant, the running min and its tile, two more kept tiles
    i32x4 bop[KA];
    float tau0[KA], best[KA], v1[KA], v2[KA];
    int s0[KA], s1[KA], s2[KA];
    bool ovf[KA];
#pragma unroll
    for (int u = 0; u < KN; ++u) {
        int64_t sp = (k0 + wave + kChWaves * u) * kChBlk + col;
        sp = sp < na ? sp : na - 1;
        const float sx = A[sp * 3] - cx, sy = A[sp * 3 + 1] - cy, sz = A[sp * 3 + 2] - cz;
        const uint32_t hxy = pk_bf16(-2.f * sx, -2.f * sy), hz1 = pk_bf16(-2.f * sz, 1.f);
        const uint32_t lxy = pk_bf16(-2.f * sx - bf16_lo(hxy), -2.f * sy - bf16_hi(hxy));
        const uint32_t lz = pk_bf16(-2.f * sz - bf16_lo(hz1), 0.f);
        if (h == 0)
            bop[u] = i32x4{(int)hxy, (int)((hz1 & 0xffffu) | (hxy << 16)), (int)((hxy >> 16) | (hz1 << 16)), (int)lxy};
        else
            bop[u] = i32x4{(int)((lz & 0xffffu) | 0x3f800000u), 0x3f80, 0, 0};
        tau0[u] = 2.f * kTau * __builtin_fmaf(sz, sz, __builtin_fmaf(sy, sy, sx * sx));
        best[u] = __builtin_inff();
        v1[u] = __builtin_inff();
        v2[u] = __builtin_inff();
        s0[u] = 0;
        s1[u] = 0;
        s2[u] = 0;
        ovf[u] = false;
    }

    // tile it sits in buffer it & 1; each wave prepares a quarter of every
    // tile, one tile ahead, and one barrier per tile publishes it (a wave
    // reaches that barrier only after its reads of the other buffer)
    const int64_t ntiles = (nt + kChTileT - 1) / kChTileT;
    float raw[kChRaw];
    cham_load_raw(T, nt, kChQuarter * wave, lane, raw);
    cham_prepare(sm, 0, raw, nt, 0, wave, lane, cx, cy, cz);
    cham_barrier();
    for (int64_t it = 0; it < ntiles; ++it) {
        const int64_t t0 = it * kChTileT;
        const int buf = (int)(it & 1);
        // A rows of the tile's row blocks: lane l reads row 32 rb + l % 32 of plane l / 32
        i32x4 av[kChRB];
#pragma unroll
        for (int rb = 0; rb < kChRB; ++rb) av[rb] = sm.tile[buf][h][32 * rb + col];
        // the next tile's coordinates (past the last tile: all padding, the
        // preparation below is then unused; no branch in the loop body)
        cham_load_raw(T, nt, t0 + kChTileT + kChQuarter * wave, lane, raw);
        // mp: this tile's min of the lane's rows, per source. The MFMAs of
        // row block rb + 1 are issued before the fold of row block rb, and
        // no later block's MFMAs move above that fold (two blocks' results
        // live at a time)
        float mp[KA];
        auto mfmas = [&](int rb, f32x16 (&d)[KA]) {
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int u = 0; u < KN; ++u)
                d[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[rb]),
                                                               __builtin_bit_cast(bf16x8, bop[u]), zero, 0, 0, 0);
            __builtin_amdgcn_s_setprio(0);
        };
        f32x16 dc[KA], dn[KA];
        mfmas(0, dc);
#pragma unroll
        for (int rb = 0; rb < kChRB; ++rb) {
            if (rb + 1 < kChRB) mfmas(rb + 1, dn);
#pragma unroll
            for (int u = 0; u < KN; ++u) {
                const f32x16& d = dc[u];
                const float a0 = __builtin_fminf(__builtin_fminf(d[0], d[1]), d[2]);
                const float a1 = __builtin_fminf(__builtin_fminf(d[3], d[4]), d[5]);
                const float a2 = __builtin_fminf(__builtin_fminf(d[6], d[7]), d[8]);
                const float a3 = __builtin_fminf(__builtin_fminf(d[9], d[10]), d[11]);
                const float a4 = __builtin_fminf(__builtin_fminf(d[12], d[13]), d[14]);
                const float b0 = __builtin_fminf(__builtin_fminf(a0, a1), a2);
                const float b1 = __builtin_fminf(__builtin_fminf(a3, a4), d[15]);
                mp[u] = rb == 0 ? __builtin_fminf(b0, b1) : __builtin_fminf(__builtin_fminf(b0, b1), mp[u]);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (rb + 1 < kChRB) {
#pragma unroll
                for (int u = 0; u < KN; ++u) dc[u] = dn[u];
            }
        }
        // the three kept tiles: a tile inside the window of the running min
        // is kept; a lower tile becomes the best and the old best the
        // second; the other kept tiles move down one slot, and the one moved
        // out of the third slot overflows the source when it is still inside
        // the window. Equal mins keep the earlier tile as the best.
        const int step = (int)it;
#pragma unroll
        for (int u = 0; u < KN; ++u) {
            const float thr_old = __builtin_fmaf(best[u], kTauK, tau0[u]);
            const bool near = mp[u] <= thr_old;
            const bool lower = mp[u] < best[u];
            const float bn = __builtin_fminf(best[u], mp[u]);
            const float thr_new = __builtin_fmaf(bn, kTauK, tau0[u]);
            ovf[u] = ovf[u] | (near & (v2[u] <= thr_new));  // bitwise: no branches
            v2[u] = near ? v1[u] : v2[u];
            s2[u] = near ? s1[u] : s2[u];
            v1[u] = near ? __builtin_fmaxf(best[u], mp[u]) : v1[u];
            s1[u] = near ? (lower ? s0[u] : step) : s1[u];
            s0[u] = lower ? step : s0[u];
            best[u] = bn;
        }
        cham_prepare(sm, buf ^ 1, raw, nt, t0 + kChTileT, wave, lane, cx, cy, cz);
        cham_barrier();
    }

    // the answer in the direct form: the kept tiles inside the window of the
    // source's overall min are re-evaluated on their rows from the raw
    // coordinates; the smallest value wins, the lowest index on ties, then
    // the two row halves of the column are merged the same way
#pragma unroll
    for (int u = 0; u < KN; ++u) {
        int64_t sp = (k0 + wave + kChWaves * u) * kChBlk + col;
        const bool own = sp < na;
        sp = own ? sp : na - 1;
        const float px = A[sp * 3], py = A[sp * 3 + 1], pz = A[sp * 3 + 2];
        float bs = best[u];
        bs = __builtin_fminf(bs, __shfl_xor(bs, 32, 64));
        const float thr = __builtin_fmaf(bs, kTauK, tau0[u]);
        int lost = (ovf[u] & (best[u] <= thr)) ? 1 : 0;
        lost |= __shfl_xor(lost, 32, 64);
        float dv = __builtin_inff();
        int di = 0x7fffffff;
        // The column's tasks are the kept tiles of its 2 lanes: bit 3j + slot
        // is set when lane half j keeps that slot. A task's rows (rows
        // 32 rb + 8 g + 4 j + r of the tile, g, r < 4) are split over the
        // column's 2 lanes, lane h taking the first or second half of the row
        // blocks, as runs of 4 consecutive points, 8 runs at a time.
        const int mine = ((best[u] <= thr) ? 1 : 0) | ((v1[u] <= thr) ? 2 : 0) | ((v2[u] <= thr) ? 4 : 0);
        int mask = mine << (3 * h);
        mask |= __shfl_xor(mask, 32, 64);
        int tile[6];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            tile[3 * j] = __shfl(s0[u], col + 32 * j, 64);
            tile[3 * j + 1] = __shfl(s1[u], col + 32 * j, 64);
            tile[3 * j + 2] = __shfl(s2[u], col + 32 * j, 64);
        }
        constexpr int kRuns = 4 * kChRB / 2;  // runs of 4 points per lane per task
        while (__any(mask != 0)) {
            if (mask != 0) {
                const int q = __builtin_ctz(mask);
                mask &= mask - 1;
                int tq = tile[0];
#pragma unroll
                for (int k = 1; k < 6; ++k) tq = q == k ? tile[k] : tq;
                const int64_t tb = (int64_t)tq * kChTileT + 4 * (q >= 3 ? 1 : 0) + 32 * (kChRB / 2) * h;
                const int64_t lim = nt * 3 - 1;
                for (int k0 = 0; k0 < kRuns; k0 += 8) {
                    // every load of 8 runs in flight at once (flat indices
                    // clamped into the set; rows past its end are not evaluated)
                    float x[8][12];
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        const int kk = k0 + k;
                        const int64_t f = (tb + 32 * (kk >> 2) + 8 * (kk & 3)) * 3;
#pragma unroll
                        for (int e = 0; e < 12; ++e) x[k][e] = T[f + e < lim ? f + e : lim];
                    }
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        const int kk = k0 + k;
                        const int64_t t = tb + 32 * (kk >> 2) + 8 * (kk & 3);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            if (t + r >= nt) continue;
                            const float dx = px - x[k][3 * r], dy = py - x[k][3 * r + 1], dz = pz - x[k][3 * r + 2];
                            const float v = __builtin_fmaf(dz, dz, __builtin_fmaf(dy, dy, dx * dx));
                            if (v < dv || (v == dv && (int)(t + r) < di)) {
                                dv = v;
                                di = (int)(t + r);
                            }
                        }
                    }
                }
            }
        }
        {
            const float ov = __shfl_xor(dv, 32, 64);
            const int oi = __shfl_xor(di, 32, 64);
            if (ov < dv || (ov == dv && oi < di)) {
                dv = ov;
                di = oi;
            }
        }
        if (h == 0 && own) {
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

// Workgroups of kChWaves waves; see the file comment. Block g of the list
// is source block g of direction 1 (P against Q) for g < B*nb1, else of
// direction 2 (Q against P); each direction is batch-major. A workgroup takes
// a contiguous run of blocks in pieces of at most kChWaves * kChMaxBlocks
// blocks of one segment; wave v of a piece takes its blocks v, v + kChWaves, ...
__global__ __launch_bounds__(kChWaves * 64) __attribute__((amdgpu_waves_per_eu(MAXSIM_CH_WAVES))) void chamfer_nn_kernel(ChamferArgs a, int64_t nblocks)
{
    __shared__ ChamLds sm;
    const int64_t nw = gridDim.x, w = blockIdx.x;
    const int wave = (int)(threadIdx.x >> 6);
    const int64_t nb1 = (a.N + kChBlk - 1) / kChBlk, nb2 = (a.M + kChBlk - 1) / kChBlk;
    const int64_t g_first = w * nblocks / nw, g_last = (w + 1) * nblocks / nw;

    for (int64_t g0 = g_first; g0 < g_last;) {
        // the segment (batch, direction) holding g0 and the piece of it taken now
        const bool second = g0 >= a.B * nb1;
        const int64_t nb = second ? nb2 : nb1;
        const int64_t gl = second ? g0 - a.B * nb1 : g0;
        const int64_t b = gl / nb, k0 = gl % nb;
        int64_t nk = nb - k0;
        if (nk > g_last - g0) nk = g_last - g0;
        if (nk > kChWaves * kChMaxBlocks) nk = kChWaves * kChMaxBlocks;
        g0 += nk;
        const int64_t na = second ? a.M : a.N, nt = second ? a.N : a.M;
        const float* A = (second ? a.Q : a.P) + b * na * 3;
        const float* T = (second ? a.P : a.Q) + b * nt * 3;
        float* dist = (second ? a.dist2 : a.dist1) + b * na;
        int32_t* idx = (second ? a.idx2 : a.idx1) + b * na;
        // this wave's blocks of the piece (0 .. kChMaxBlocks)
        const int kn = nk > wave ? (int)((nk - wave + kChWaves - 1) / kChWaves) : 0;
        switch (__builtin_amdgcn_readfirstlane(kn)) {
        case 0: cham_piece<0>(sm, A, na, T, nt, k0, dist, idx); break;
        case 1: cham_piece<1>(sm, A, na, T, nt, k0, dist, idx); break;
        case 2: if constexpr (kChMaxBlocks >= 2) cham_piece<2>(sm, A, na, T, nt, k0, dist, idx); break;
        case 3: if constexpr (kChMaxBlocks >= 3) cham_piece<3>(sm, A, na, T, nt, k0, dist, idx); break;
        default: if constexpr (kChMaxBlocks >= 4) cham_piece<4>(sm, A, na, T, nt, k0, dist, idx); break;
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
    // as many workgroups as are resident at once (the runs of blocks then end
    // together); a workgroup holds at most kChWaves * kChMaxBlocks source
    // blocks at a time, so larger inputs get more workgroups
    static std::atomic<int> per_cu{0};
    int occ = per_cu.load(std::memory_order_relaxed);
    if (occ <= 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, chamfer_nn_kernel, kChWaves * 64, 0) != hipSuccess ||
            occ <= 0)
            occ = 2;
        per_cu.store(occ, std::memory_order_relaxed);
    }
    const int64_t nblocks = a.B * ((a.N + kChBlk - 1) / kChBlk + (a.M + kChBlk - 1) / kChBlk);
    constexpr int64_t kPiece = kChWaves * kChMaxBlocks;
    int64_t wgs = (int64_t)occ * device_cu_count();
    if (wgs * kPiece < nblocks) wgs = (nblocks + kPiece - 1) / kPiece;
    if (wgs > nblocks) wgs = nblocks;
    if (wgs > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(chamfer_nn_kernel, dim3((unsigned)wgs), dim3(kChWaves * 64), 0, stream, a, nblocks);
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
