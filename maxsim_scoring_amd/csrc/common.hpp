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

}  // namespace maxsim
