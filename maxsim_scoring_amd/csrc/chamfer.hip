// Chamfer distance forward for gfx950 ("Flash-MaxSim" Sec. 4.2.4): for every
// point of one set, the squared Euclidean distance to the nearest point of the
// other set and its index (lowest index on ties), streamed with an online
// min instead of the materialised [N, M] distance matrix; then the per-batch
// loss (1/N) sum dist1 + (1/M) sum dist2 in a fixed order.
//
// Design: the pages obtain Chamfer from MaxSim by putting a squared distance
// where the inner product was, so the distance tile is formed the same way,
// as a contraction on the matrix cores: ||s - t||^2 = ||s||^2 + (||t||^2 -
// 2 <s, t>), where the bracket is one v_mfma_f32_16x16x4_f32 per 16 x 16 tile
// with the targets (tx, ty, tz, ||t||^2) as rows of A and the sources
// (-2 sx, -2 sy, -2 sz, 1) as columns of B (K = 4, fp32 in and out). A lane
// owns one source column and 4 target rows of each tile. Tiles go in pairs of
// 16-target blocks; the lane folds its 8 values of a pair into its running
// min and records, with a strict '<', the pair that last lowered it, so the
// earliest pair keeps a tie. At the end it re-evaluates its 8 rows of that
// pair and takes the lowest index with the smallest value. The 4 row groups
// of a column are then merged by (value, index). ||s||^2 is added once at the
// end (adding the same value to every candidate keeps their order); the
// result is clamped at 0, since the expanded form can round a zero distance
// slightly negative. All coordinates are first taken relative to the target
// set's first point, so that rounding scales with the sets' extent.
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

// KN source blocks of one (batch, direction) segment against its whole
// target set: A [na, 3] holds the sources, blocks k0 .. k0+KN-1; T [nt, 3]
// the targets. Writes dist[sp] and idx[sp] for the blocks' points.
template <int KN>
__device__ __forceinline__ void cham_piece(ChamLds& sm, const float* __restrict__ A, int64_t na,
                                           const float* __restrict__ T, int64_t nt, int64_t k0,
                                           float* __restrict__ dist, int32_t* __restrict__ idx)
{
    const int lane = threadIdx.x;
    const int col = lane & 15, rg = lane >> 4;  // source column, target row group (= K index of A, B)
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    // both sets are taken relative to the target set's first point: the
    // distances do not change, and the expanded form's rounding then scales
    // with the sets' extent rather than their distance from the origin
    const float cx = T[0], cy = T[1], cz = T[2];
    const float crg = rg == 0 ? cx : (rg == 1 ? cy : cz);  // this lane's K component

    // this lane's source point of each block (clamped copies past the end)
    float bop[KN], best[KN];
    int bstep[KN];  // the 16-target block where best was last lowered
#pragma unroll
    for (int u = 0; u < KN; ++u) {
        int64_t sp = (k0 + u) * 16 + col;
        sp = sp < na ? sp : na - 1;
        bop[u] = rg < 3 ? -2.f * (A[sp * 3 + (rg < 3 ? rg : 0)] - crg) : 1.f;
        best[u] = __builtin_inff();
        bstep[u] = 0;
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
        const int step0 = (int)(t0 / 16);
        // one 16-target block (or two): KN MFMAs per block sharing the A
        // operand, then the running min of this lane's 4 rows per block and
        // the first block of the step that last lowered it (strict '<': the
        // earliest step keeps a tie)
        auto block = [&](float aop, int step) {
            f32x4 d[KN];
#pragma unroll
            for (int u = 0; u < KN; ++u) d[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(aop, bop[u], zero, 0, 0, 0);
#pragma unroll
            for (int u = 0; u < KN; ++u) {
                const float m = __builtin_fminf(
                    __builtin_fminf(__builtin_fminf(__builtin_fminf(d[u][0], d[u][1]), d[u][2]), d[u][3]), best[u]);
                bstep[u] = m < best[u] ? step : bstep[u];
                best[u] = m;
            }
        };
        auto block2 = [&](float a0, float a1, int step) {
            f32x4 d[KN], e[KN];
            // MFMAs issued at raised priority (the SIMD's other waves yield
            // the issue slots to the MFMA stream; about 6 % here)
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int u = 0; u < KN; ++u) d[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, bop[u], zero, 0, 0, 0);
#pragma unroll
            for (int u = 0; u < KN; ++u) e[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, bop[u], zero, 0, 0, 0);
            __builtin_amdgcn_s_setprio(0);
#pragma unroll
            for (int u = 0; u < KN; ++u) {
                const float x = __builtin_fminf(__builtin_fminf(d[u][0], d[u][1]), d[u][2]);
                const float y = __builtin_fminf(__builtin_fminf(d[u][3], e[u][0]), e[u][1]);
                const float z = __builtin_fminf(__builtin_fminf(e[u][2], e[u][3]), best[u]);
                const float m = __builtin_fminf(__builtin_fminf(x, y), z);
                bstep[u] = m < best[u] ? step : bstep[u];
                best[u] = m;
            }
        };
        if (tbs == kChTileT / 16) {
            // a full tile: every block's operand is read up front, and the
            // blocks go in pairs (one min update per pair)
            float av[kChTileT / 16];
#pragma unroll
            for (int tb = 0; tb < kChTileT / 16; ++tb) av[tb] = tf[tb * 64];
#pragma unroll
            for (int tb = 0; tb < kChTileT / 16; tb += 2) block2(av[tb], av[tb + 1], step0 + tb);
        } else {
            for (int tb = 0; tb < tbs; ++tb) block(tf[tb * 64], step0 + tb);
        }
        if (it + 1 < ntiles) cham_prepare(sm, buf ^ 1, raw, nt, t0 + kChTileT, lane, cx, cy, cz);
    }

    // the row of the recorded step: among this lane's rows of the step's
    // first block and the block after it (8 targets), the lowest index whose
    // value, evaluated again in the same form on the VALU, is smallest. A row
    // of the later block can only tie the recorded min (a smaller value would
    // have been recorded as a later step), and since the MFMA's own rounding
    // is not reproduced, a row inside a near tie may be taken, within the
    // evaluation bound. Then the 4 row groups of each column are merged by
    // (value, index) and written
#pragma unroll
    for (int u = 0; u < KN; ++u) {
        int64_t sp = (k0 + u) * 16 + col;
        const bool own = sp < na;
        sp = own ? sp : na - 1;
        const float sx = A[sp * 3] - cx, sy = A[sp * 3 + 1] - cy, sz = A[sp * 3 + 2] - cz;
        const int64_t tbase = (int64_t)bstep[u] * 16 + 4 * rg;
        int i = (int)(tbase < nt ? tbase : nt - 1);
        float rv = __builtin_inff();
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int64_t t = tbase + (r < 4 ? r : 12 + r);
            if (t < nt) {
                const float tx = T[t * 3] - cx, ty = T[t * 3 + 1] - cy, tz = T[t * 3 + 2] - cz;
                const float n2 = __builtin_fmaf(tz, tz, __builtin_fmaf(ty, ty, tx * tx));
                const float v =
                    __builtin_fmaf(-2.f * sz, tz, __builtin_fmaf(-2.f * sy, ty, __builtin_fmaf(-2.f * sx, tx, n2)));
                if (v < rv) {
                    rv = v;
                    i = (int)t;
                }
            }
        }
        float v = best[u];
#pragma unroll
        for (int x = 16; x <= 32; x <<= 1) {
            const float ov = __shfl_xor(v, x, 64);
            const int oi = __shfl_xor(i, x, 64);
            if (ov < v || (ov == v && oi < i)) {
                v = ov;
                i = oi;
            }
        }
        if (rg == 0 && own) {
            const float dd = __builtin_fmaf(sz, sz, __builtin_fmaf(sy, sy, sx * sx)) + v;
            dist[sp] = dd > 0.f ? dd : 0.f;
            idx[sp] = i;
        }
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
    if (a.loss) {
        hipLaunchKernelGGL(chamfer_loss_kernel, dim3((unsigned)a.B), dim3(kLossThreads), 0, stream, a.dist1,
                           a.dist2, a.N, a.M, a.loss);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace maxsim
