// Cross-product MaxSim forward for gfx950: fp16/bf16 (32x32x16 MFMA) and
// int8 (32x32x32 MFMA), with d_mask/q_mask, optional argmax and long queries.
//
// "Flash-MaxSim" Sec. 4.1 (fused forward, online max), Sec. 4.1.1 (-inf
// masking, no rescale), Sec. 4.3.1 (INT8 x INT8 with fused dequantisation);
// late-interaction-kernels design notes "Forward" (strict '>' argmax update,
// finalise with finite(m) & q_active) and "Long-query chunking" (a query is
// split into fixed chunks whose partial scores are summed in a fixed order).
//
// Work unit = one workgroup = (doc j, group of query N-tiles). The S tile is
// computed transposed, S^T = D . Q^T: MFMA rows are doc tokens and columns are
// query tokens, so every lane owns one query token and the max over doc
// tokens stays inside the lane; only the two lane halves are merged, once per
// doc. D is streamed HBM/L2 -> LDS with direct-to-LDS loads into a 3-stage
// ring (prefetch distance 2), shared by every wave of the workgroup, so a doc
// tile is read once per workgroup. Q stays in VGPRs for the whole doc.
#include "common.hpp"
#include "kernels.hpp"

namespace maxsim {

namespace {

constexpr int kTileRows = 64;  // doc tokens per pipeline stage (2 MFMA M-tiles)
constexpr int kStages = 3;
constexpr int kMaxMaskTokens = 32768;  // d_mask bits kept in LDS per segment

// Fold one 32x32 accumulator tile into the running (max, argmax) of each
// N-tile. Lane rows are 8*(q/4) + 4*h + q%4; q ascends with the row, so a
// strict '>' keeps the lowest index on ties. `lbits` bit r = row r + 4h valid.
template <typename V, bool ARGMAX, int NTW, bool MASKED, typename Acc>
__device__ __forceinline__ void update_rows(const Acc (&acc)[NTW], V (&m)[NTW], int (&idx)[NTW],
                                            int base, uint32_t lbits)
{
#pragma unroll
    for (int n = 0; n < NTW; ++n) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int r = 8 * (q >> 2) + (q & 3);
            V v = acc[n][q];
            if constexpr (MASKED) v = ((lbits >> r) & 1u) ? v : neg_inf<V>();
            if constexpr (ARGMAX) {
                if (v > m[n]) {
                    m[n] = v;
                    idx[n] = base + r;
                }
            } else {
                m[n] = m[n] > v ? m[n] : v;
            }
        }
    }
}

}  // namespace

template <int E, bool ARGMAX, int WAVES, int NTW>
__global__ __launch_bounds__(WAVES * 64) void fwd_dense_kernel(DenseArgs a)
{
    using T = Traits<E>;
    using V = typename T::Scalar;
    using Acc = typename T::Acc;
    constexpr int RB = T::kRowBytes;
    constexpr int NCH = RB / 16;                   // 16-byte chunks per row
    constexpr int KS = T::kKSteps;
    constexpr int SLOTS = WAVES * NTW;             // N-tiles per workgroup
    constexpr int STAGE_BYTES = kTileRows * RB;
    constexpr int CHUNKS = kTileRows * NCH;
    constexpr int THREADS = WAVES * 64;
    constexpr int LPS = CHUNKS / THREADS;          // direct-to-LDS loads per thread per stage
    static_assert(CHUNKS % THREADS == 0, "stage must split evenly over the workgroup");

    __shared__ __attribute__((aligned(16))) unsigned char stage_buf[kStages * STAGE_BYTES];
    __shared__ uint64_t mask_bits[kMaxMaskTokens / 64];
    __shared__ V part[SLOTS];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int h = lane >> 5;   // which K-half this lane feeds; which row-quad it owns
    const int col = lane & 31; // MFMA column = query token within the N-tile

    // ---- work unit: XCD-aware order (workgroup b runs on XCD b % 8) --------
    const int nblk = gridDim.x;
    const int b = blockIdx.x;
    const int xcd = b & 7, kth = b >> 3;
    const int full = nblk >> 3, rem = nblk & 7;
    const int unit = xcd * full + (xcd < rem ? xcd : rem) + kth;
    const int64_t j = unit / a.nqg;
    const int qg = unit % a.nqg;

    const int64_t Lq = a.Lq, Ld = a.Ld, Nd = a.Nd;
    const unsigned char* Dj = (const unsigned char*)a.D + j * Ld * RB;
    const uint8_t* dmj = a.d_mask ? a.d_mask + j * Ld : nullptr;

    V qsum = 0;  // running per-query sum across passes (multi-pass long queries)

    for (int pass = 0; pass < a.npass; ++pass) {
        // ---- the N-tiles this wave owns in this pass ------------------------
        int qi[NTW], nt_idx[NTW];
        bool slot_ok[NTW];
#pragma unroll
        for (int n = 0; n < NTW; ++n) {
            const int slot = wave * NTW + n;
            if (a.npass == 1) {
                qi[n] = qg * a.qpw + slot / a.ntq;
                nt_idx[n] = slot % a.ntq;
                slot_ok[n] = slot < a.qpw * a.ntq && qi[n] < a.Nq;
            } else {
                qi[n] = qg;
                nt_idx[n] = pass * SLOTS + slot;
                slot_ok[n] = nt_idx[n] < a.ntq;
            }
        }

        // ---- Q fragments (B operand), kept in VGPRs for the whole doc -------
        i32x4 qf[NTW][KS];
#pragma unroll
        for (int n = 0; n < NTW; ++n) {
            const int64_t s_tok = (int64_t)nt_idx[n] * 32 + col;
            const bool ok = slot_ok[n] && s_tok < Lq;
            const unsigned char* qrow =
                (const unsigned char*)a.Q + ((int64_t)qi[n] * Lq + (ok ? s_tok : 0)) * RB;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                i32x4 v = {0, 0, 0, 0};
                if (ok) v = *(const i32x4*)(qrow + (2 * s + h) * 16);
                qf[n][s] = v;
            }
        }

        // Q must have landed before the pipeline starts: the compiler cannot
        // count direct-to-LDS loads per stage and would otherwise wait for all
        // of them inside the loop before the first use of qf.
        wait_vmcnt<0>();

        // ---- d_mask bits of this doc into LDS (first segment) ---------------
        // Tokens are processed in segments of kMaxMaskTokens so the bitmask
        // always fits LDS; typical docs have a single segment.
        V m[NTW];
        int idx[NTW];
#pragma unroll
        for (int n = 0; n < NTW; ++n) {
            m[n] = neg_inf<V>();
            idx[n] = 0;
        }

        for (int64_t seg0 = 0; seg0 < Ld; seg0 += kMaxMaskTokens) {
            const int64_t seg_len = Ld - seg0 < kMaxMaskTokens ? Ld - seg0 : kMaxMaskTokens;
            if (dmj) {
                block_barrier();  // previous users of mask_bits are done
                const int nwords = (int)((seg_len + 63) >> 6);
                for (int w = wave; w < nwords; w += WAVES) {
                    const int64_t t = seg0 + (int64_t)w * 64 + lane;
                    const bool v = t < Ld && dmj[t] != 0;
                    const uint64_t bits = __ballot(v);
                    if (lane == 0) mask_bits[w] = bits;
                }
                __builtin_amdgcn_s_waitcnt(0);
                block_barrier();
            }
            const int ntiles = (int)((seg_len + kTileRows - 1) / kTileRows);

            // ---- direct-to-LDS staging of one 64-token tile ------------------
            auto issue = [&](int tile, int stage) {
                const int64_t t0 = seg0 + (int64_t)tile * kTileRows;
                unsigned char* sb = stage_buf + stage * STAGE_BYTES;
#pragma unroll
                for (int u = 0; u < LPS; ++u) {
                    const int p0 = (wave * LPS + u) * 64;  // first LDS chunk of this instruction
                    const int p = p0 + lane;
                    const int row = p / NCH;
                    const int pc = p % NCH;
                    const int lc = swz_chunk<RB>(row, pc);
                    int64_t grow = t0 + row;
                    if (grow >= Ld) grow = Ld - 1;  // clamped rows are masked out below
                    const unsigned char* g = Dj + grow * RB + lc * 16;
                    __builtin_amdgcn_global_load_lds((const void*)g, LDS_PTR(sb + p0 * 16), 16, 0, 0);
                }
            };

            issue(0, 0);
            if (ntiles > 1) issue(1, 1);

            for (int it = 0; it < ntiles; ++it) {
                if (it + 1 < ntiles) wait_vmcnt<LPS>();
                else wait_vmcnt<0>();
                block_barrier();
                if (it + 2 < ntiles) issue(it + 2, (it + 2) % kStages);

                // validity of the 64 rows of this tile
                const int64_t t0 = seg0 + (int64_t)it * kTileRows;
                const int64_t left = Ld - t0;
                uint64_t vbits = left >= 64 ? ~0ull : ((1ull << left) - 1ull);
                if (dmj) vbits &= lds_read_u64_uniform(&mask_bits[it]);
                if (vbits == 0) continue;  // no valid token: nothing to reduce
                const bool all_valid = vbits == ~0ull;
                const unsigned char* sb = stage_buf + (it % kStages) * STAGE_BYTES;

#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    const uint32_t mbits = (uint32_t)(vbits >> (mt * 32));
                    if (mbits == 0) continue;
                    // A fragments: row = doc token (lane % 32), k-half = lane / 32
                    i32x4 af[KS];
                    const int row = mt * 32 + col;
                    uint32_t ad[KS];
#pragma unroll
                    for (int s = 0; s < KS; ++s)
                        ad[s] = lds_addr(sb + row * RB + swz_chunk<RB>(row, 2 * s + h) * 16);
                    if constexpr (KS == 8)
                        lds_read8(af, ad);
                    else
                        lds_read4(af[0], af[1], af[2], af[3], ad[0], ad[1], ad[2], ad[3]);
                    Acc acc[NTW];
#pragma unroll
                    for (int n = 0; n < NTW; ++n) acc[n] = Acc{};
#pragma unroll
                    for (int s = 0; s < KS; ++s)
#pragma unroll
                        for (int n = 0; n < NTW; ++n) acc[n] = mfma32<E>(af[s], qf[n][s], acc[n]);

                    // online max (+argmax) over this lane's 16 rows, ascending t;
                    // masked rows become -inf before the max
                    const int base = (int)(t0 + mt * 32);
                    if (all_valid || mbits == 0xffffffffu) {
                        update_rows<V, ARGMAX, NTW, false>(acc, m, idx, base, 0u);
                    } else {
                        update_rows<V, ARGMAX, NTW, true>(acc, m, idx, base, mbits >> (4 * h));
                    }
                }
            }
            // all waves must be done reading the ring before it is reused
            block_barrier();
        }

        // ---- finalise: merge lane halves, q_mask, row sums --------------------
#pragma unroll
        for (int n = 0; n < NTW; ++n) {
            V mv = m[n];
            int iv = idx[n] + 4 * h;
            if constexpr (ARGMAX) {
                const V om = __builtin_bit_cast(V, shfl_xor_i(__builtin_bit_cast(int, mv), 32));
                const int oi = shfl_xor_i(iv, 32);
                argmax_merge(mv, iv, om, oi);
                if (!finite_score(mv)) iv = 0;
            } else {
                const V om = __builtin_bit_cast(V, shfl_xor_i(__builtin_bit_cast(int, mv), 32));
                mv = mv > om ? mv : om;
            }
            const int64_t s_tok = (int64_t)nt_idx[n] * 32 + col;
            const bool tok_ok = slot_ok[n] && s_tok < Lq;
            bool keep = tok_ok && finite_score(mv);
            if (keep && a.q_mask) keep = a.q_mask[(int64_t)qi[n] * Lq + s_tok] != 0;
            V contrib = keep ? mv : (V)0;
            if constexpr (ARGMAX) {
                if (h == 0 && tok_ok)
                    a.argmax[((int64_t)qi[n] * Nd + j) * Lq + s_tok] = iv;
            }
            // fixed-order butterfly over the 32 query tokens of the N-tile
#pragma unroll
            for (int off = 16; off >= 1; off >>= 1) {
                if constexpr (E == kI8)
                    contrib += shfl_xor_i(contrib, off);
                else
                    contrib += shfl_xor_f(contrib, off);
            }
            if (lane == 0) part[wave * NTW + n] = contrib;
        }
        block_barrier();
        if (a.npass == 1) {
            if (tid < a.qpw) {
                const int64_t i = (int64_t)qg * a.qpw + tid;
                if (i < a.Nq) {
                    V sum = 0;
                    for (int n = 0; n < a.ntq; ++n) sum += part[tid * a.ntq + n];
                    if constexpr (E == kI8) {
                        if (a.scores_i32) a.scores_i32[i * Nd + j] = sum;
                        if (a.scores) a.scores[i * Nd + j] = (float)(((double)sum * a.q_scale) * a.d_scale);
                    } else {
                        a.scores[i * Nd + j] = sum;
                    }
                }
            }
        } else if (tid == 0) {
            const int nslots = a.ntq - pass * SLOTS < SLOTS ? a.ntq - pass * SLOTS : SLOTS;
            for (int n = 0; n < nslots; ++n) qsum += part[n];
        }
        block_barrier();
    }

    if (a.npass > 1 && tid == 0) {
        const int64_t i = qg;
        if constexpr (E == kI8) {
            if (a.scores_i32) a.scores_i32[i * Nd + j] = qsum;
            if (a.scores) a.scores[i * Nd + j] = (float)(((double)qsum * a.q_scale) * a.d_scale);
        } else {
            a.scores[i * Nd + j] = qsum;
        }
    }
}

// ---------------------------------------------------------------------------
// Host-side launch helpers.
// ---------------------------------------------------------------------------
template <int E, int WAVES, int NTW>
static hipError_t launch_dense_t(DenseArgs a, bool want_argmax, hipStream_t stream)
{
    constexpr int SLOTS = WAVES * NTW;
    a.ntq = (int)((a.Lq + 31) / 32);
    if (a.ntq == 0) a.ntq = 1;
    if (a.ntq <= SLOTS) {
        a.qpw = SLOTS / a.ntq;
        a.npass = 1;
    } else {
        a.qpw = 1;
        a.npass = (a.ntq + SLOTS - 1) / SLOTS;
    }
    a.nqg = (int)((a.Nq + a.qpw - 1) / a.qpw);
    const int64_t units = (int64_t)a.nqg * a.Nd;
    if (units <= 0) return hipSuccess;
    dim3 grid((unsigned)units), block(WAVES * 64);
    if (want_argmax)
        hipLaunchKernelGGL((fwd_dense_kernel<E, true, WAVES, NTW>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((fwd_dense_kernel<E, false, WAVES, NTW>), grid, block, 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_fwd_dense(int elem, DenseArgs a, bool want_argmax, hipStream_t stream)
{
    switch (elem) {
    case kF16: return launch_dense_t<kF16, 4, 2>(a, want_argmax, stream);
    case kBF16: return launch_dense_t<kBF16, 4, 2>(a, want_argmax, stream);
    case kI8: return launch_dense_t<kI8, 8, 4>(a, want_argmax, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace maxsim
