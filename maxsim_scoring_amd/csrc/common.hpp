// Shared device helpers for the gfx950 MaxSim kernels: vector types, MFMA
// wrappers, wave64 cross-lane helpers and the LDS swizzle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace maxsim {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

constexpr int kD = 128;     // embedding width handled by every kernel
constexpr int kWave = 64;

enum Elem : int { kF16 = 0, kBF16 = 1, kI8 = 2 };

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// ---------------------------------------------------------------------------
// Element traits. A "fragment" is the 16 bytes one lane feeds into one MFMA
// K-step (8 fp16/bf16 values or 16 int8 values).
// ---------------------------------------------------------------------------
template <int E> struct Traits;
template <> struct Traits<kF16> {
    static constexpr int kElemBytes = 2;
    static constexpr int kRowBytes = kD * 2;      // 256
    static constexpr int kKSteps = kD / 16;       // 32x32x16: 8 steps
    typedef f32x16 Acc;
    typedef float Scalar;
};
template <> struct Traits<kBF16> {
    static constexpr int kElemBytes = 2;
    static constexpr int kRowBytes = kD * 2;
    static constexpr int kKSteps = kD / 16;
    typedef f32x16 Acc;
    typedef float Scalar;
};
template <> struct Traits<kI8> {
    static constexpr int kElemBytes = 1;
    static constexpr int kRowBytes = kD;          // 128
    static constexpr int kKSteps = kD / 32;       // 32x32x32: 4 steps
    typedef i32x16 Acc;
    typedef int Scalar;
};

// One 32x32 output tile step: acc += A(32 x K) * B(K x 32), operands given as
// the 16-byte per-lane fragments (lane l holds row/col l % 32, k-half l / 32).
template <int E>
__device__ __forceinline__ typename Traits<E>::Acc mfma32(const i32x4& a, const i32x4& b,
                                                          const typename Traits<E>::Acc& c);
template <>
__device__ __forceinline__ f32x16 mfma32<kF16>(const i32x4& a, const i32x4& b, const f32x16& c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mfma32<kBF16>(const i32x4& a, const i32x4& b, const f32x16& c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ i32x16 mfma32<kI8>(const i32x4& a, const i32x4& b, const i32x16& c)
{
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// 16x16x32 fp16/bf16 step used by the streaming kernel: lane l holds row/col
// l % 16 and k-quarter l / 16.
template <int E> __device__ __forceinline__ f32x4 mfma16(const i32x4& a, const i32x4& b, const f32x4& c);
template <>
__device__ __forceinline__ f32x4 mfma16<kF16>(const i32x4& a, const i32x4& b, const f32x4& c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma16<kBF16>(const i32x4& a, const i32x4& b, const f32x4& c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Cross-lane helpers (wave64).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

__device__ __forceinline__ float shfl_xor_f(float v, int m)
{
    return __builtin_bit_cast(float, __shfl_xor(__builtin_bit_cast(int, v), m, 64));
}
__device__ __forceinline__ int shfl_xor_i(int v, int m) { return __shfl_xor(v, m, 64); }

// Sum over the 16 lanes of each DPP row; every lane of the row receives the
// same bits (each step adds a value and its mirror image, and addition is
// commutative, so the order is fixed).
template <int CTRL, typename V>
__device__ __forceinline__ V dpp_add(V x)
{
    const int o = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false);
    return x + __builtin_bit_cast(V, o);
}
template <typename V>
__device__ __forceinline__ V row16_sum(V v)
{
    v = dpp_add<0xB1>(v);   // quad_perm [1,0,3,2]
    v = dpp_add<0x4E>(v);   // quad_perm [2,3,0,1]
    v = dpp_add<0x141>(v);  // row_half_mirror
    v = dpp_add<0x140>(v);  // row_mirror
    return v;
}

// Sum of lanes 0-31 (DPP row sums, then row 0 + row 1), the same in every
// lane. (The permlane swap builtins are avoided here: with both operands the
// same value, ROCm 7.2 compiled the two swap results as one.)
template <typename V>
__device__ __forceinline__ V lanes0_31_sum(V v)
{
    const uint32_t b = __builtin_bit_cast(uint32_t, row16_sum(v));
    return __builtin_bit_cast(V, __builtin_amdgcn_readlane(b, 0)) +
           __builtin_bit_cast(V, __builtin_amdgcn_readlane(b, 16));
}

// Max with lowest-index tie-break across two (value, index) candidates.
template <typename V>
__device__ __forceinline__ void argmax_merge(V& m, int& idx, V om, int oidx)
{
    if (om > m || (om == m && oidx < idx)) {
        m = om;
        idx = oidx;
    }
}

// Negative infinity / smallest value of the score type.
template <typename V> __device__ __forceinline__ V neg_inf();
template <> __device__ __forceinline__ float neg_inf<float>() { return -__builtin_inff(); }
template <> __device__ __forceinline__ int neg_inf<int>() { return (int)0x80000000; }

__device__ __forceinline__ bool finite_score(float v) { return __builtin_isfinite(v); }
__device__ __forceinline__ bool finite_score(int v) { return v != (int)0x80000000; }

// ---------------------------------------------------------------------------
// LDS swizzle: a row of `kRowBytes` is stored as 16-byte chunks whose position
// is XOR-ed with a function of the row, so that 16 lanes reading the same
// logical chunk of 16 consecutive rows hit distinct banks.
// ---------------------------------------------------------------------------
template <int kRowBytes>
__device__ __forceinline__ int swz_chunk(int row, int chunk)
{
    if constexpr (kRowBytes == 256) {
        return chunk ^ (row & 15);
    } else {  // 128-byte rows: two rows share one 256-byte bank line
        return chunk ^ ((row & 7) ^ ((row >> 3) & 1));
    }
}

// ---------------------------------------------------------------------------
// Synchronisation and LDS access around direct-to-LDS loads.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void lds_fence() { asm volatile("" ::: "memory"); }

// Barrier without the implicit vmcnt(0) of __syncthreads(): loads that are
// still in flight for later pipeline stages keep flying across it. LDS writes
// made before it are waited for (lgkmcnt(0)) so every wave sees them after.
__device__ __forceinline__ void block_barrier()
{
    lds_fence();
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    lds_fence();
}

// One 16-byte-per-lane direct-to-LDS load: lane l reads base + voff[l] and
// the wave's 1 KB lands at LDS byte address `lds` (+ 16 * lane). `base` and
// `lds` must be wave-uniform. Written in assembly to use the scalar-base
// addressing form (32-bit per-lane offsets) and to keep the compiler from
// treating the load as an LDS write it must wait for before every later LDS
// access; callers synchronise explicitly with wait_vmcnt. M0 is set here; no
// compiler-generated code in these kernels keeps a value in M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_lds16(const void* base, uint32_t voff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds), "v"(voff), "s"(base)
                 : "memory", "m0");
}
// the same with the non-temporal hint, for data that is streamed once
__device__ __forceinline__ void dma_lds16_nt(const void* base, uint32_t voff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                 :
                 : "s"(lds), "v"(voff), "s"(base)
                 : "memory", "m0");
}
// One 4-byte-per-lane direct-to-LDS load: lane l's dword lands at `lds` + 4 l
// (active lanes only).
__device__ __forceinline__ void dma_lds4(const void* base, uint32_t voff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
                 :
                 : "s"(lds), "v"(voff), "s"(base)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ const void* uniform_ptr(const void* p)
{
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int64_t uniform_i64(int64_t v)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// ---------------------------------------------------------------------------
// Wave-uniform searches over cu_seqlens offsets.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Smallest j in [0, n] with cu[j] >= target, found by the whole wave with
// 64 probes per round (cu is non-decreasing and cu[n] >= target).
__device__ inline int wave_lower_bound(const int32_t* __restrict__ cu, int n, int64_t target)
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
    return uniform(lo);
}

// The doc boundary j whose offset cu[j] is nearest to `target` (ties to the
// lower one). Units end where the next one starts, so every doc is owned once;
// rounding to the nearest boundary halves the worst token imbalance compared
// with always rounding up.
__device__ inline int nearest_boundary(const int32_t* __restrict__ cu, int n, int64_t target)
{
    const int j1 = wave_lower_bound(cu, n, target);  // first boundary at or above
    if (j1 == 0) return 0;
    const int64_t above = (int64_t)cu[j1] - target;
    const int64_t below = target - (int64_t)cu[j1 - 1];
    return uniform(below <= above ? j1 - 1 : j1);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// LDS reads of direct-to-LDS data. They are issued from inline assembly on
// purpose: the compiler cannot tell which ring stage an outstanding
// direct-to-LDS load targets, so for a plain LDS load it would wait for every
// load in flight (vmcnt(0)) and collapse the prefetch pipeline. The explicit
// vmcnt wait + barrier at the top of each iteration already guarantees that
// the stage being read has landed. Each helper waits for its own reads.
__device__ __forceinline__ uint32_t lds_addr(const void* p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ void lds_read4(i32x4& a0, i32x4& a1, i32x4& a2, i32x4& a3,
                                          uint32_t p0, uint32_t p1, uint32_t p2, uint32_t p3)
{
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3)
        : "v"(p0), "v"(p1), "v"(p2), "v"(p3)
        : "memory");
}

__device__ __forceinline__ void lds_read8(i32x4 (&a)[8], const uint32_t (&p)[8])
{
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %9\n\t"
        "ds_read_b128 %2, %10\n\t"
        "ds_read_b128 %3, %11\n\t"
        "ds_read_b128 %4, %12\n\t"
        "ds_read_b128 %5, %13\n\t"
        "ds_read_b128 %6, %14\n\t"
        "ds_read_b128 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4]), "=&v"(a[5]),
          "=&v"(a[6]), "=&v"(a[7])
        : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "v"(p[5]), "v"(p[6]), "v"(p[7])
        : "memory");
}

// The same reads without the wait, so that later work can overlap their
// latency; lds_wait_regs() waits and ties the destination registers to the
// wait so that no use of them can be scheduled before it.
__device__ __forceinline__ void lds_read8_async(i32x4 (&a)[8], const uint32_t (&p)[8])
{
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %9\n\t"
        "ds_read_b128 %2, %10\n\t"
        "ds_read_b128 %3, %11\n\t"
        "ds_read_b128 %4, %12\n\t"
        "ds_read_b128 %5, %13\n\t"
        "ds_read_b128 %6, %14\n\t"
        "ds_read_b128 %7, %15"
        : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4]), "=&v"(a[5]),
          "=&v"(a[6]), "=&v"(a[7])
        : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "v"(p[5]), "v"(p[6]), "v"(p[7])
        : "memory");
}
__device__ __forceinline__ void lds_read4_async(i32x4 (&a)[4], const uint32_t (&p)[4])
{
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7"
        : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3])
        : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3])
        : "memory");
}
// As above with a compile-time byte offset added to every address (the
// instruction's immediate offset field, so no address registers per offset).
template <int OFF>
__device__ __forceinline__ void lds_read8_async_off(i32x4 (&a)[8], const uint32_t (&p)[8])
{
    static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
    asm volatile(
        "ds_read_b128 %0, %8 offset:%16\n\t"
        "ds_read_b128 %1, %9 offset:%16\n\t"
        "ds_read_b128 %2, %10 offset:%16\n\t"
        "ds_read_b128 %3, %11 offset:%16\n\t"
        "ds_read_b128 %4, %12 offset:%16\n\t"
        "ds_read_b128 %5, %13 offset:%16\n\t"
        "ds_read_b128 %6, %14 offset:%16\n\t"
        "ds_read_b128 %7, %15 offset:%16"
        : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4]), "=&v"(a[5]),
          "=&v"(a[6]), "=&v"(a[7])
        : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "v"(p[5]), "v"(p[6]), "v"(p[7]),
          "i"(OFF)
        : "memory");
}
template <int OFF>
__device__ __forceinline__ void lds_read4_async_off(i32x4 (&a)[4], const uint32_t (&p)[4])
{
    static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
    asm volatile(
        "ds_read_b128 %0, %4 offset:%8\n\t"
        "ds_read_b128 %1, %5 offset:%8\n\t"
        "ds_read_b128 %2, %6 offset:%8\n\t"
        "ds_read_b128 %3, %7 offset:%8"
        : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3])
        : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "i"(OFF)
        : "memory");
}

__device__ __forceinline__ void lds_wait_regs(i32x4 (&a)[8])
{
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]),
                   "+v"(a[6]), "+v"(a[7])
                 :
                 : "memory");
}
__device__ __forceinline__ void lds_wait_regs(i32x4 (&a)[4])
{
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]) : : "memory");
}

__device__ __forceinline__ uint64_t lds_read_u64_uniform(const uint64_t* p)
{
    uint64_t v;
    asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(lds_addr(p)) : "memory");
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

}  // namespace maxsim
