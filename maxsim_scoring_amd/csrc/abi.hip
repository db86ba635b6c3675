// The C ABI declared in include/maxsim.h: host-side validation (before
// anything is enqueued), then one launcher per entry point.
#include "maxsim.h"

#include <atomic>
#include <climits>

#include "common.hpp"
#include "kernels.hpp"

using namespace maxsim;

int maxsim::device_cu_count()
{
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    int n = dev < kMaxDevices ? cache[dev].load(std::memory_order_relaxed) : 0;
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    if (dev < kMaxDevices) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

namespace {

constexpr int64_t kI32Max = INT32_MAX;

maxsim_status_t launch_status(hipError_t e) { return e == hipSuccess ? MAXSIM_OK : MAXSIM_ERR_LAUNCH; }

bool dtype_ok(maxsim_dtype_t t) { return t == MAXSIM_F16 || t == MAXSIM_BF16; }

// Embedding widths of the entry points: 128 has its own forward kernels,
// every other width up to kMaxDim takes the general-width forward; the
// backward gathers handle any width in 128-wide chunks.
constexpr int64_t kMaxDim = 1024;
bool width_ok(int64_t d) { return d >= 1 && d <= kMaxDim; }

// At most two 32-token query passes in all (one or two short queries, the
// reranking shape): the cross-product kernel would run one N-tile per 8-wave
// workgroup, so these calls take the streaming general-width kernel at any
// width (one 32-token query against 10,000 docs of 128 tokens: 68 us instead
// of 208 us; from four such passes on the cross-product kernel is faster).
bool small_query(int64_t Nq, int64_t Lq) { return Nq <= 2 && Nq * ((Lq + 31) / 32) <= 2; }

int elem_of(maxsim_dtype_t t) { return t == MAXSIM_F16 ? kF16 : kBF16; }

// The product of non-negative sizes, or -1 when it exceeds int64.
int64_t mul_sat(int64_t a, int64_t b)
{
    if (a == 0 || b == 0) return 0;
    if (a > INT64_MAX / b) return -1;
    return a * b;
}

// Row tensors are read and written 16 bytes at a time; every other array
// needs its natural alignment. NULL passes (it is checked separately).
bool aligned(const void* p, uintptr_t n) { return ((uintptr_t)p & (n - 1)) == 0; }

}  // namespace

extern "C" {

maxsim_status_t maxsim_fwd(maxsim_dtype_t dtype, const void* Q, const void* D, int64_t Nq,
                           int64_t Nd, int64_t Lq, int64_t Ld, int64_t d, const uint8_t* q_mask,
                           const uint8_t* d_mask, float* scores, int32_t* argmax,
                           maxsim_stream_t stream)
{
    if (Nq < 0 || Nd < 0 || Lq < 0 || Ld < 0 || d < 0) return MAXSIM_ERR_SHAPE;
    if (!dtype_ok(dtype) || !width_ok(d)) return MAXSIM_ERR_UNSUPPORTED;
    if (Nq == 0 || Nd == 0) return MAXSIM_OK;
    if (!scores) return MAXSIM_ERR_NULL;
    if ((Lq > 0 && !Q) || (Ld > 0 && !D)) return MAXSIM_ERR_NULL;
    if (!aligned(Q, 16) || !aligned(D, 16) || !aligned(scores, 4) || !aligned(argmax, 4))
        return MAXSIM_ERR_UNSUPPORTED;
    const int64_t pairs = mul_sat(Nq, Nd);
    if (pairs < 0 || pairs > kI32Max) return MAXSIM_ERR_OVERFLOW;  // one workgroup per pair group
    if (argmax) {
        const int64_t n = mul_sat(pairs, Lq);
        if (n < 0 || n > kI32Max) return MAXSIM_ERR_OVERFLOW;
    }
    const int64_t rows = mul_sat(Nd, Ld);
    if (d != kD || (small_query(Nq, Lq) && rows >= 0 && rows <= kI32Max)) {
        if (rows < 0 || rows > kI32Max || Lq > kI32Max) return MAXSIM_ERR_OVERFLOW;
        DimArgs g{};
        g.Q = Q;
        g.D = D;
        g.q_mask = q_mask;
        g.d_mask = d_mask;
        g.scores = scores;
        g.argmax = argmax;
        g.Nq = Nq;
        g.Nd = Nd;
        g.Lq = Lq;
        g.Ld = Ld;
        g.d = (int32_t)d;
        return launch_status(launch_fwd_dim(elem_of(dtype), g, (hipStream_t)stream));
    }
    DenseArgs a{};
    a.Q = Q;
    a.D = D;
    a.q_mask = q_mask;
    a.d_mask = d_mask;
    a.scores = scores;
    a.argmax = argmax;
    a.Nq = Nq;
    a.Nd = Nd;
    a.Lq = Lq;
    a.Ld = Ld;
    return launch_status(launch_fwd_dense(elem_of(dtype), a, argmax != nullptr, (hipStream_t)stream));
}

maxsim_status_t maxsim_fwd_varlen(maxsim_dtype_t dtype, const void* Q, const int32_t* cu_q,
                                  int64_t Nq, int32_t max_lq, const void* D, const int32_t* cu_d,
                                  int64_t Nd, int64_t d, float* scores, int32_t* argmax,
                                  maxsim_stream_t stream)
{
    if (Nq < 0 || Nd < 0 || d < 0 || max_lq < 0) return MAXSIM_ERR_SHAPE;
    if (!dtype_ok(dtype) || !width_ok(d)) return MAXSIM_ERR_UNSUPPORTED;
    if (Nq == 0 || Nd == 0) return MAXSIM_OK;
    // Q or D may be NULL only when that packed tensor holds no tokens (an
    // empty torch tensor has no storage); the kernels then never read it.
    if (!cu_q || !cu_d || !scores) return MAXSIM_ERR_NULL;
    if (!aligned(Q, 16) || !aligned(D, 16) || !aligned(cu_q, 4) || !aligned(cu_d, 4) ||
        !aligned(scores, 4) || !aligned(argmax, 4))
        return MAXSIM_ERR_UNSUPPORTED;
    if (Nd > kI32Max - 1) return MAXSIM_ERR_OVERFLOW;
    const int64_t pairs = mul_sat(Nq, Nd);
    if (pairs < 0 || pairs > kI32Max) return MAXSIM_ERR_OVERFLOW;
    if (argmax) {
        const int64_t n = mul_sat(pairs, max_lq);
        if (n < 0 || n > kI32Max) return MAXSIM_ERR_OVERFLOW;
    }
    if (d != kD) {
        DimArgs g{};
        g.Q = Q;
        g.cu_q = cu_q;
        g.D = D;
        g.cu_d = cu_d;
        g.scores = scores;
        g.argmax = argmax;
        g.Nq = Nq;
        g.Nd = Nd;
        g.Lq = max_lq;
        g.d = (int32_t)d;
        return launch_status(launch_fwd_dim(elem_of(dtype), g, (hipStream_t)stream));
    }
    VarlenArgs a{};
    a.Q = Q;
    a.cu_q = cu_q;
    a.D = D;
    a.cu_d = cu_d;
    a.scores = scores;
    a.argmax = argmax;
    a.Nq = Nq;
    a.Nd = Nd;
    a.max_lq = max_lq;
    return launch_status(launch_fwd_varlen(elem_of(dtype), a, (hipStream_t)stream));
}

maxsim_status_t maxsim_fwd_i8(const int8_t* Q, float q_scale, const int8_t* D, float d_scale,
                              int64_t Nq, int64_t Nd, int64_t Lq, int64_t Ld, int64_t d,
                              const uint8_t* q_mask, const uint8_t* d_mask, int32_t* scores_i32,
                              float* scores, int32_t* argmax, maxsim_stream_t stream)
{
    if (Nq < 0 || Nd < 0 || Lq < 0 || Ld < 0 || d < 0) return MAXSIM_ERR_SHAPE;
    if (!width_ok(d)) return MAXSIM_ERR_UNSUPPORTED;
    if (Nq == 0 || Nd == 0) return MAXSIM_OK;
    if (!scores_i32 && !scores) return MAXSIM_ERR_NULL;
    if ((Lq > 0 && !Q) || (Ld > 0 && !D)) return MAXSIM_ERR_NULL;
    if (!aligned(Q, 16) || !aligned(D, 16) || !aligned(scores_i32, 4) || !aligned(scores, 4) ||
        !aligned(argmax, 4))
        return MAXSIM_ERR_UNSUPPORTED;
    // worst case |sum| = Lq * d * 127^2 must stay inside int32
    const int64_t worst = mul_sat(mul_sat(Lq, d), 127 * 127);
    if (worst < 0 || worst > kI32Max) return MAXSIM_ERR_OVERFLOW;
    const int64_t pairs = mul_sat(Nq, Nd);
    if (pairs < 0 || pairs > kI32Max) return MAXSIM_ERR_OVERFLOW;
    if (argmax) {
        const int64_t n = mul_sat(pairs, Lq);
        if (n < 0 || n > kI32Max) return MAXSIM_ERR_OVERFLOW;
    }
    const int64_t rows = mul_sat(Nd, Ld);
    if (d != kD || (small_query(Nq, Lq) && rows >= 0 && rows <= kI32Max)) {
        if (rows < 0 || rows > kI32Max || Lq > kI32Max) return MAXSIM_ERR_OVERFLOW;
        DimArgs g{};
        g.Q = Q;
        g.D = D;
        g.q_mask = q_mask;
        g.d_mask = d_mask;
        g.scores = scores;
        g.scores_i32 = scores_i32;
        g.argmax = argmax;
        g.q_scale = (double)q_scale;
        g.d_scale = (double)d_scale;
        g.Nq = Nq;
        g.Nd = Nd;
        g.Lq = Lq;
        g.Ld = Ld;
        g.d = (int32_t)d;
        return launch_status(launch_fwd_dim(kI8, g, (hipStream_t)stream));
    }
    DenseArgs a{};
    a.Q = Q;
    a.D = D;
    a.q_mask = q_mask;
    a.d_mask = d_mask;
    a.scores = scores;
    a.scores_i32 = scores_i32;
    a.argmax = argmax;
    a.q_scale = (double)q_scale;
    a.d_scale = (double)d_scale;
    a.Nq = Nq;
    a.Nd = Nd;
    a.Lq = Lq;
    a.Ld = Ld;
    return launch_status(launch_fwd_dense(kI8, a, argmax != nullptr, (hipStream_t)stream));
}

maxsim_status_t maxsim_fwd_i8_tok(const int8_t* Q, const float* q_scale, const int8_t* D,
                                  const float* d_scale, int64_t Nq, int64_t Nd, int64_t Lq,
                                  int64_t Ld, int64_t d, const uint8_t* q_mask,
                                  const uint8_t* d_mask, float* scores, int32_t* argmax,
                                  maxsim_stream_t stream)
{
    if (Nq < 0 || Nd < 0 || Lq < 0 || Ld < 0 || d < 0) return MAXSIM_ERR_SHAPE;
    if (!width_ok(d)) return MAXSIM_ERR_UNSUPPORTED;
    if (Nq == 0 || Nd == 0) return MAXSIM_OK;
    if (!scores) return MAXSIM_ERR_NULL;
    if ((Lq > 0 && (!Q || !q_scale)) || (Ld > 0 && (!D || !d_scale))) return MAXSIM_ERR_NULL;
    if (!aligned(Q, 16) || !aligned(D, 16) || !aligned(q_scale, 4) || !aligned(d_scale, 4) ||
        !aligned(scores, 4) || !aligned(argmax, 4))
        return MAXSIM_ERR_UNSUPPORTED;
    const int64_t pairs = mul_sat(Nq, Nd);
    if (pairs < 0 || pairs > kI32Max) return MAXSIM_ERR_OVERFLOW;
    if (argmax) {
        const int64_t n = mul_sat(pairs, Lq);
        if (n < 0 || n > kI32Max) return MAXSIM_ERR_OVERFLOW;
    }
    const int64_t rows = mul_sat(Nd, Ld);
    if (d != kD || (small_query(Nq, Lq) && rows >= 0 && rows <= kI32Max)) {
        if (rows < 0 || rows > kI32Max || Lq > kI32Max) return MAXSIM_ERR_OVERFLOW;
        DimArgs g{};
        g.Q = Q;
        g.D = D;
        g.q_mask = q_mask;
        g.d_mask = d_mask;
        g.scores = scores;
        g.argmax = argmax;
        g.q_scale_tok = q_scale;
        g.d_scale_tok = d_scale;
        g.Nq = Nq;
        g.Nd = Nd;
        g.Lq = Lq;
        g.Ld = Ld;
        g.d = (int32_t)d;
        return launch_status(launch_fwd_dim(kI8, g, (hipStream_t)stream));
    }
    DenseArgs a{};
    a.Q = Q;
    a.D = D;
    a.q_mask = q_mask;
    a.d_mask = d_mask;
    a.scores = scores;
    a.argmax = argmax;
    a.q_scale_tok = q_scale;
    a.d_scale_tok = d_scale;
    a.Nq = Nq;
    a.Nd = Nd;
    a.Lq = Lq;
    a.Ld = Ld;
    return launch_status(launch_fwd_dense(kI8, a, argmax != nullptr, (hipStream_t)stream));
}

maxsim_status_t maxsim_fwd_pairs(maxsim_dtype_t dtype, const void* Q, const void* D, int64_t Nq,
                                 int64_t Nd, int64_t Lq, int64_t Ld, int64_t d,
                                 const uint8_t* q_mask, const uint8_t* d_mask,
                                 const int32_t* pair_q, const int32_t* pair_d, int64_t P,
                                 float* scores, int32_t* argmax, maxsim_stream_t stream)
{
    if (Nq < 0 || Nd < 0 || Lq < 0 || Ld < 0 || d < 0 || P < 0) return MAXSIM_ERR_SHAPE;
    if (!dtype_ok(dtype) || !width_ok(d)) return MAXSIM_ERR_UNSUPPORTED;
    if (P == 0) return MAXSIM_OK;
    if (Nq == 0 || Nd == 0) return MAXSIM_ERR_SHAPE;  // a pair needs a query and a doc
    if (!scores || !pair_q || !pair_d) return MAXSIM_ERR_NULL;
    if ((Lq > 0 && !Q) || (Ld > 0 && !D)) return MAXSIM_ERR_NULL;
    if (!aligned(Q, 16) || !aligned(D, 16) || !aligned(pair_q, 4) || !aligned(pair_d, 4) ||
        !aligned(scores, 4) || !aligned(argmax, 4))
        return MAXSIM_ERR_UNSUPPORTED;
    if (P > kI32Max) return MAXSIM_ERR_OVERFLOW;  // one workgroup per pair
    if (argmax) {
        const int64_t n = mul_sat(P, Lq);
        if (n < 0 || n > kI32Max) return MAXSIM_ERR_OVERFLOW;
    }
    if (d != kD) {
        const int64_t rows = mul_sat(Nd, Ld);
        if (rows < 0 || rows > kI32Max || Lq > kI32Max) return MAXSIM_ERR_OVERFLOW;
        DimArgs g{};
        g.Q = Q;
        g.D = D;
        g.q_mask = q_mask;
        g.d_mask = d_mask;
        g.scores = scores;
        g.argmax = argmax;
        g.pair_q = pair_q;
        g.pair_d = pair_d;
        g.npairs = P;
        g.Nq = Nq;
        g.Nd = Nd;
        g.Lq = Lq;
        g.Ld = Ld;
        g.d = (int32_t)d;
        return launch_status(launch_fwd_dim(elem_of(dtype), g, (hipStream_t)stream));
    }
    DenseArgs a{};
    a.Q = Q;
    a.D = D;
    a.q_mask = q_mask;
    a.d_mask = d_mask;
    a.scores = scores;
    a.argmax = argmax;
    a.pair_q = pair_q;
    a.pair_d = pair_d;
    a.npairs = P;
    a.Nq = Nq;
    a.Nd = Nd;
    a.Lq = Lq;
    a.Ld = Ld;
    return launch_status(launch_fwd_dense(elem_of(dtype), a, argmax != nullptr, (hipStream_t)stream));
}

maxsim_status_t maxsim_topk(const float* scores, int64_t Nq, int64_t Nd, int64_t K,
                            const int32_t* ids, int32_t* idx, float* val, int32_t* rows,
                            maxsim_stream_t stream)
{
    if (Nq < 0 || Nd < 0 || K < 0 || K > Nd) return MAXSIM_ERR_SHAPE;
    if (K > kTopkMaxK) return MAXSIM_ERR_UNSUPPORTED;
    if (Nq == 0 || K == 0) return MAXSIM_OK;
    if (!scores || !idx || !val) return MAXSIM_ERR_NULL;
    if (!aligned(scores, 4) || !aligned(idx, 4) || !aligned(val, 4) || !aligned(ids, 4) ||
        !aligned(rows, 4))
        return MAXSIM_ERR_UNSUPPORTED;
    if (Nd > kI32Max || Nq > kI32Max) return MAXSIM_ERR_OVERFLOW;
    TopkArgs a{};
    a.scores = scores;
    a.Nq = Nq;
    a.Nd = Nd;
    a.K = (int)K;
    a.ids = ids;
    a.idx = idx;
    a.val = val;
    a.rows = rows;
    return launch_status(launch_topk(a, (hipStream_t)stream));
}

maxsim_status_t maxsim_fwd_pairs_varlen(maxsim_dtype_t dtype, const void* Q, const int32_t* cu_q,
                                        int64_t Nq, int32_t max_lq, const void* D,
                                        const int32_t* cu_d, int64_t Nd, int64_t d,
                                        const int32_t* pair_q, const int32_t* pair_d, int64_t P,
                                        float* scores, int32_t* argmax, maxsim_stream_t stream)
{
    if (Nq < 0 || Nd < 0 || d < 0 || max_lq < 0 || P < 0) return MAXSIM_ERR_SHAPE;
    if (!dtype_ok(dtype) || !width_ok(d)) return MAXSIM_ERR_UNSUPPORTED;
    if (P == 0) return MAXSIM_OK;
    if (Nq == 0 || Nd == 0) return MAXSIM_ERR_SHAPE;  // a pair needs a query and a doc
    if (!cu_q || !cu_d || !pair_q || !pair_d || !scores) return MAXSIM_ERR_NULL;
    if (!aligned(Q, 16) || !aligned(D, 16) || !aligned(cu_q, 4) || !aligned(cu_d, 4) ||
        !aligned(pair_q, 4) || !aligned(pair_d, 4) || !aligned(scores, 4) || !aligned(argmax, 4))
        return MAXSIM_ERR_UNSUPPORTED;
    if (Nq > kI32Max - 1 || Nd > kI32Max - 1 || P > kI32Max) return MAXSIM_ERR_OVERFLOW;
    if (argmax) {
        const int64_t n = mul_sat(P, max_lq);
        if (n < 0 || n > kI32Max) return MAXSIM_ERR_OVERFLOW;
    }
    if (d != kD) {
        DimArgs g{};
        g.Q = Q;
        g.cu_q = cu_q;
        g.D = D;
        g.cu_d = cu_d;
        g.scores = scores;
        g.argmax = argmax;
        g.pair_q = pair_q;
        g.pair_d = pair_d;
        g.npairs = P;
        g.Nq = Nq;
        g.Nd = Nd;
        g.Lq = max_lq;
        g.d = (int32_t)d;
        return launch_status(launch_fwd_dim(elem_of(dtype), g, (hipStream_t)stream));
    }
    VarlenArgs a{};
    a.Q = Q;
    a.cu_q = cu_q;
    a.D = D;
    a.cu_d = cu_d;
    a.scores = scores;
    a.argmax = argmax;
    a.Nq = Nq;
    a.Nd = Nd;
    a.max_lq = max_lq;
    a.pair_q = pair_q;
    a.pair_d = pair_d;
    a.npairs = P;
    return launch_status(launch_fwd_varlen(elem_of(dtype), a, (hipStream_t)stream));
}

maxsim_status_t maxsim_bwd_varlen(maxsim_dtype_t dtype, const void* Q, const int32_t* cu_q,
                                  int64_t Nq, int64_t total_q, int32_t max_lq, const void* D,
                                  const int32_t* cu_d, int64_t Nd, int64_t total_d, int64_t d,
                                  const int32_t* argmax, const float* grad_scores, float* dQ,
                                  float* dD, int32_t* csr_row_ptr, int32_t* csr_col_idx,
                                  maxsim_stream_t stream)
{
    if (Nq < 0 || Nd < 0 || total_q < 0 || total_d < 0 || d < 0 || max_lq < 0) return MAXSIM_ERR_SHAPE;
    if (!dtype_ok(dtype) || !width_ok(d)) return MAXSIM_ERR_UNSUPPORTED;
    // packed rows need a sequence to belong to, and a query row a max_lq slot
    if ((Nq == 0 && total_q > 0) || (Nd == 0 && total_d > 0) || (total_q > 0 && max_lq == 0))
        return MAXSIM_ERR_SHAPE;
    const int64_t nsrc = mul_sat(mul_sat(Nq, Nd), max_lq);
    const int64_t nnz = mul_sat(total_q, Nd);
    if (nsrc < 0 || nsrc > kI32Max || nnz < 0 || nnz > kI32Max) return MAXSIM_ERR_OVERFLOW;
    if (total_d + 1 > kI32Max || Nq > kI32Max - 1 || Nd > kI32Max - 1) return MAXSIM_ERR_OVERFLOW;
    if (!cu_q || !cu_d || !csr_row_ptr) return MAXSIM_ERR_NULL;
    if (total_q > 0 && (!Q || !dQ)) return MAXSIM_ERR_NULL;
    if (total_d > 0 && (!D || !dD || (total_q > 0 && !csr_col_idx))) return MAXSIM_ERR_NULL;
    if (Nq * Nd > 0 && (!argmax || !grad_scores)) return MAXSIM_ERR_NULL;
    if (!aligned(Q, 16) || !aligned(D, 16) || !aligned(dQ, 16) || !aligned(dD, 16) ||
        !aligned(cu_q, 4) || !aligned(cu_d, 4) || !aligned(argmax, 4) || !aligned(grad_scores, 4) ||
        !aligned(csr_row_ptr, 4) || !aligned(csr_col_idx, 4))
        return MAXSIM_ERR_UNSUPPORTED;
    VarBwdArgs a{};
    a.Q = Q;
    a.cu_q = cu_q;
    a.D = D;
    a.cu_d = cu_d;
    a.argmax = argmax;
    a.g = grad_scores;
    a.dQ = dQ;
    a.dD = dD;
    a.row_ptr = csr_row_ptr;
    a.col_idx = csr_col_idx;
    a.Nq = Nq;
    a.Nd = Nd;
    a.Tq = total_q;
    a.Td = total_d;
    a.nnz_cap = nnz;
    a.max_lq = max_lq;
    a.d = (int32_t)d;
    return launch_status(launch_bwd_varlen(elem_of(dtype), a, (hipStream_t)stream));
}

maxsim_status_t maxsim_chamfer_fwd(const float* P, const float* Q, int64_t B, int64_t N, int64_t M,
                                   float* dist1, int32_t* idx1, float* dist2, int32_t* idx2,
                                   float* loss, maxsim_stream_t stream)
{
    if (B < 0 || N < 0 || M < 0) return MAXSIM_ERR_SHAPE;
    if (B == 0) return MAXSIM_OK;
    if (N == 0 || M == 0) return MAXSIM_ERR_SHAPE;  // a min over an empty set
    const int64_t nP = mul_sat(B, N), nQ = mul_sat(B, M);
    if (nP < 0 || nP > kI32Max || nQ < 0 || nQ > kI32Max) return MAXSIM_ERR_OVERFLOW;
    if (!P || !Q || !dist1 || !idx1 || !dist2 || !idx2) return MAXSIM_ERR_NULL;
    if (!aligned(P, 4) || !aligned(Q, 4) || !aligned(dist1, 4) || !aligned(idx1, 4) ||
        !aligned(dist2, 4) || !aligned(idx2, 4) || !aligned(loss, 4))
        return MAXSIM_ERR_UNSUPPORTED;
    ChamferArgs a{};
    a.P = P;
    a.Q = Q;
    a.B = B;
    a.N = N;
    a.M = M;
    a.dist1 = dist1;
    a.idx1 = idx1;
    a.dist2 = dist2;
    a.idx2 = idx2;
    a.loss = loss;
    return launch_status(launch_chamfer_fwd(a, (hipStream_t)stream));
}

maxsim_status_t maxsim_chamfer_bwd(const float* P, const float* Q, int64_t B, int64_t N, int64_t M,
                                   const int32_t* idx1, const int32_t* idx2, const float* grad_dist1,
                                   const float* grad_dist2, float* dP, float* dQ,
                                   int32_t* csr_row_ptr1, int32_t* csr_col_idx1,
                                   int32_t* csr_row_ptr2, int32_t* csr_col_idx2,
                                   maxsim_stream_t stream)
{
    if (B < 0 || N < 0 || M < 0) return MAXSIM_ERR_SHAPE;
    if (B == 0) return MAXSIM_OK;
    if (N == 0 || M == 0) return MAXSIM_ERR_SHAPE;
    const int64_t nP = mul_sat(B, N), nQ = mul_sat(B, M);
    if (nP < 0 || nP + 1 > kI32Max || nQ < 0 || nQ + 1 > kI32Max) return MAXSIM_ERR_OVERFLOW;
    if (!P || !Q || !idx1 || !idx2 || !grad_dist1 || !grad_dist2 || !dP || !dQ || !csr_row_ptr1 ||
        !csr_col_idx1 || !csr_row_ptr2 || !csr_col_idx2)
        return MAXSIM_ERR_NULL;
    for (const void* p : {(const void*)P, (const void*)Q, (const void*)idx1, (const void*)idx2,
                          (const void*)grad_dist1, (const void*)grad_dist2, (const void*)dP,
                          (const void*)dQ, (const void*)csr_row_ptr1, (const void*)csr_col_idx1,
                          (const void*)csr_row_ptr2, (const void*)csr_col_idx2})
        if (!aligned(p, 4)) return MAXSIM_ERR_UNSUPPORTED;
    ChamferArgs a{};
    a.P = P;
    a.Q = Q;
    a.B = B;
    a.N = N;
    a.M = M;
    a.idx1 = const_cast<int32_t*>(idx1);
    a.idx2 = const_cast<int32_t*>(idx2);
    a.g1 = grad_dist1;
    a.g2 = grad_dist2;
    a.dP = dP;
    a.dQ = dQ;
    a.row_ptr1 = csr_row_ptr1;
    a.col_idx1 = csr_col_idx1;
    a.row_ptr2 = csr_row_ptr2;
    a.col_idx2 = csr_col_idx2;
    return launch_status(launch_chamfer_bwd(a, (hipStream_t)stream));
}

maxsim_status_t maxsim_bwd(maxsim_dtype_t dtype, const void* Q, const void* D, int64_t Nq,
                           int64_t Nd, int64_t Lq, int64_t Ld, int64_t d, const uint8_t* q_mask,
                           const uint8_t* d_mask, const int32_t* argmax, const float* grad_scores,
                           float* dQ, float* dD, int32_t* csr_row_ptr, int32_t* csr_col_idx,
                           maxsim_stream_t stream)
{
    if (Nq < 0 || Nd < 0 || Lq < 0 || Ld < 0 || d < 0) return MAXSIM_ERR_SHAPE;
    if (!dtype_ok(dtype) || !width_ok(d)) return MAXSIM_ERR_UNSUPPORTED;
    const int64_t nsrc = mul_sat(mul_sat(Nq, Nd), Lq);
    const int64_t nrows = mul_sat(Nd, Ld);
    if (nsrc < 0 || nsrc > kI32Max) return MAXSIM_ERR_OVERFLOW;
    if (nrows < 0 || nrows + 1 > kI32Max) return MAXSIM_ERR_OVERFLOW;
    if (mul_sat(Nq, Lq) > kI32Max) return MAXSIM_ERR_OVERFLOW;
    if (nsrc > 0 && Ld == 0) return MAXSIM_ERR_SHAPE;  // no destination for the sources
    if (Nd > 0 && !csr_row_ptr) return MAXSIM_ERR_NULL;
    if (nsrc > 0 && (!Q || !D || !argmax || !grad_scores || !csr_col_idx)) return MAXSIM_ERR_NULL;
    if (Nq * Lq > 0 && !dQ) return MAXSIM_ERR_NULL;
    if (nrows > 0 && !dD) return MAXSIM_ERR_NULL;
    if (!aligned(Q, 16) || !aligned(D, 16) || !aligned(dQ, 16) || !aligned(dD, 16) ||
        !aligned(argmax, 4) || !aligned(grad_scores, 4) || !aligned(csr_row_ptr, 4) ||
        !aligned(csr_col_idx, 4))
        return MAXSIM_ERR_UNSUPPORTED;
    if (Nq * Lq == 0 && nrows == 0 && Nd == 0) return MAXSIM_OK;
    BwdArgs a{};
    a.Q = Q;
    a.D = D;
    a.q_mask = q_mask;
    a.d_mask = d_mask;
    a.argmax = argmax;
    a.g = grad_scores;
    a.dQ = dQ;
    a.dD = dD;
    a.row_ptr = csr_row_ptr;
    a.col_idx = csr_col_idx;
    a.Nq = Nq;
    a.Nd = Nd;
    a.Lq = Lq;
    a.Ld = Ld;
    a.d = (int32_t)d;
    return launch_status(launch_bwd(elem_of(dtype), a, (hipStream_t)stream));
}

const char* maxsim_status_string(maxsim_status_t s)
{
    switch (s) {
    case MAXSIM_OK: return "ok";
    case MAXSIM_ERR_NULL: return "a required pointer is NULL";
    case MAXSIM_ERR_SHAPE: return "negative or inconsistent sizes";
    case MAXSIM_ERR_UNSUPPORTED: return "unsupported: d outside 1..1024, an unknown dtype, or a misaligned pointer";
    case MAXSIM_ERR_OVERFLOW: return "sizes overflow the int32 index range or the int32 sum";
    case MAXSIM_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
    }
}

int maxsim_abi_version(void) { return MAXSIM_ABI_VERSION; }

}  // extern "C"
