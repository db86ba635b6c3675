// Argument blocks and launchers shared by the host ABI and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace maxsim {

struct DenseArgs {
    const void* Q;
    const void* D;
    const uint8_t* q_mask;  // [Nq, Lq] or null
    const uint8_t* d_mask;  // [Nd, Ld] or null
    float* scores;          // [Nq, Nd] ([npairs] with a pair list) or null (int8 only)
    int32_t* scores_i32;    // [Nq, Nd] or null (int8 per-tensor only)
    int32_t* argmax;        // [Nq, Nd, Lq] ([npairs, Lq] with a pair list) or null
    double q_scale, d_scale;  // int8 only
    const float* q_scale_tok;  // [Nq, Lq] per-token scales (int8) or null
    const float* d_scale_tok;  // [Nd, Ld]
    const int32_t* pair_q;     // [npairs] pair list or null (score listed pairs only)
    const int32_t* pair_d;
    int64_t npairs;
    int64_t Nq, Nd, Lq, Ld;
    // filled by the launcher
    int ntq;      // 32-token N-tiles per query
    int qpw;      // whole queries per workgroup (single pass)
    int npass;    // passes over the docs when one query has more N-tiles than a workgroup holds
    int nqb;      // query blocks
    int nranges;  // doc ranges; workgroup = (query block, doc range)
};

struct VarlenArgs {
    const void* Q;
    const int32_t* cu_q;
    const void* D;
    const int32_t* cu_d;
    float* scores;    // [Nq, Nd]
    int32_t* argmax;  // [Nq, Nd, max_lq] or null
    int64_t Nq, Nd;
    int32_t max_lq;
    int32_t units;           // streaming units (waves) per query
    const int32_t* pair_q;   // [npairs] pair list or null (score listed pairs only)
    const int32_t* pair_d;
    int64_t npairs;
};

// Forward at any embedding width d (rows of d elements, d * element size
// bytes), for uniform or cu_seqlens-packed queries and docs, with or without a
// pair list.
struct DimArgs {
    const void* Q;
    const void* D;
    const int32_t* cu_q;    // [Nq + 1] offsets, or null: query i is rows [i Lq, (i + 1) Lq)
    const int32_t* cu_d;    // [Nd + 1] offsets, or null: doc j is rows [j Ld, (j + 1) Ld)
    const uint8_t* q_mask;  // [Nq, Lq] or null (uniform queries only)
    const uint8_t* d_mask;  // [Nd, Ld] or null (uniform docs only)
    const int32_t* pair_q;  // [npairs] pair list or null (score listed pairs only)
    const int32_t* pair_d;
    int64_t npairs;
    float* scores;    // [Nq, Nd] ([npairs] with a pair list); int8: or null
    int32_t* argmax;  // [Nq, Nd, Lq] ([npairs, Lq] with a pair list) or null
    int32_t* scores_i32;        // int8 per-tensor: [Nq, Nd] exact sums or null
    double q_scale, d_scale;    // int8 per-tensor scales
    const float* q_scale_tok;   // int8 per-token scales: [rows of Q] or null
    const float* d_scale_tok;   // [rows of D]
    int64_t Nq, Nd;
    int64_t Lq;  // uniform query length, or the max_lq bound of packed queries
    int64_t Ld;  // uniform doc length (unused with cu_d)
    int32_t d;
    // filled by the launcher
    int32_t row_bytes;  // d * element size
    int32_t nchunk;     // 256-byte chunks per row
    int32_t units;      // streaming units per query (or pairs)
};

struct BwdArgs {
    const void* Q;
    const void* D;
    const uint8_t* q_mask;
    const uint8_t* d_mask;
    const int32_t* argmax;
    const float* g;
    float* dQ;
    float* dD;
    int32_t* row_ptr;
    int32_t* col_idx;
    int64_t Nq, Nd, Lq, Ld;
    int32_t d;  // embedding width (rows of d elements)
};

struct VarBwdArgs {
    const void* Q;
    const int32_t* cu_q;  // [Nq + 1]
    const void* D;
    const int32_t* cu_d;  // [Nd + 1]
    const int32_t* argmax;  // [Nq, Nd, max_lq] doc-relative
    const float* g;         // [Nq, Nd]
    float* dQ;              // [Tq, d]
    float* dD;              // [Td, d]
    int32_t* row_ptr;       // [Td + 1]
    int32_t* col_idx;       // [Tq * (docs with a token)]
    int64_t Nq, Nd, Tq, Td;
    int64_t nnz_cap;  // entries of col_idx (Tq * Nd)
    int32_t max_lq;
    int32_t d;  // embedding width (rows of d elements)
};

struct ChamferArgs {
    const float* P;  // [B, N, 3]
    const float* Q;  // [B, M, 3]
    int64_t B, N, M;
    float* dist1;    // [B, N]
    int32_t* idx1;
    float* dist2;    // [B, M]
    int32_t* idx2;
    float* loss;     // [B] or null
    // backward
    const float* g1;  // [B, N]
    const float* g2;  // [B, M]
    float* dP;        // [B, N, 3]
    float* dQ;        // [B, M, 3]
    int32_t* row_ptr1;  // [B*M + 1]: rows = Q points, sources = P points
    int32_t* col_idx1;  // [B*N]
    int32_t* row_ptr2;  // [B*N + 1]: rows = P points, sources = Q points
    int32_t* col_idx2;  // [B*M]
};

struct TopkArgs {
    const float* scores;  // [Nq, Nd]
    int64_t Nq, Nd;
    int K;
    const int32_t* ids;  // [Nq, Nd] ids reported for each column, or null (the column)
    int32_t* idx;        // [Nq, K]
    float* val;          // [Nq, K]
    int32_t* rows;       // [Nq, K] row index of each entry, or null
};

constexpr int kTopkMaxK = 1024;  // largest k of one top-k call

// Compute units of the current device (queried once per device, thread-safe).
int device_cu_count();

hipError_t launch_fwd_dense(int elem, DenseArgs a, bool want_argmax, hipStream_t stream);
hipError_t launch_fwd_varlen(int elem, VarlenArgs a, hipStream_t stream);
hipError_t launch_fwd_dim(int elem, DimArgs a, hipStream_t stream);
hipError_t launch_bwd(int elem, BwdArgs a, hipStream_t stream);
hipError_t launch_topk(TopkArgs a, hipStream_t stream);
hipError_t launch_bwd_varlen(int elem, VarBwdArgs a, hipStream_t stream);
hipError_t launch_chamfer_fwd(ChamferArgs a, hipStream_t stream);
hipError_t launch_chamfer_bwd(ChamferArgs a, hipStream_t stream);

}  // namespace maxsim
