// Device helpers shared by the libkda kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 is carried as raw 16-bit storage; conversions are explicit.
struct bf16 {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest even (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}

// exp(x) through the hardware base-2 exponential.
__device__ __forceinline__ float exp_f(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

constexpr float kLog2e = 1.4426950408889634f;

// Gate activation from raw inputs: the decay factor exp(g) for
// g = -A softplus(z), A = exp(A_log), given zl = z log2(e) (z = x + dt_bias):
//     exp(g) = 2^(-A sp),  sp = softplus(z) log2(e) = max(zl, 0) + log2(1 + 2^-|zl|).
// Three hardware transcendentals.  log2 of the rounded 1 + 2^-|zl| costs at
// most ~1e-7 of sp in absolute terms (relative accuracy is lost only where sp
// itself is tiny), i.e. |error of g| <= ~1e-7 A: far below the rounding of a
// bf16 x (2^-9 relative).
__device__ __forceinline__ float gate_decay(float zl, float A) {
    const float sp = __builtin_fmaxf(zl, 0.f) +
                     __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(-__builtin_fabsf(zl)));
    return __builtin_amdgcn_exp2f(-A * sp);
}

// beta = sigmoid(b) = 1 / (1 + e^-b); e^-b overflowing to +inf gives 0.
__device__ __forceinline__ float sigmoid_f(float b) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-b * kLog2e));
}

// Word 3 of a raw buffer resource on gfx9-family parts: 32-bit data format,
// no swizzle; untyped 16-byte accesses with a byte range check.
constexpr int kBufferWord3 = 0x00020000;

// Element type traits for io / state tensors.
template <typename T> struct io_traits;
template <> struct io_traits<float> {
    static constexpr int bytes = 4;
    __device__ static __forceinline__ float load(const float *p, long i) { return p[i]; }
    __device__ static __forceinline__ void store(float *p, long i, float x) { p[i] = x; }
};
template <> struct io_traits<bf16> {
    static constexpr int bytes = 2;
    __device__ static __forceinline__ float load(const bf16 *p, long i) { return bf16_to_f32(p[i].bits); }
    __device__ static __forceinline__ void store(bf16 *p, long i, float x) { p[i].bits = f32_to_bf16(x); }
};

// Load 4 consecutive elements as floats (16 B for f32, 8 B for bf16).
__device__ __forceinline__ f32x4 load4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ f32x4 load4(const bf16 *p) {
    u32x2 w = *reinterpret_cast<const u32x2 *>(p);
    f32x4 r;
    r[0] = __uint_as_float(w[0] << 16);
    r[1] = __uint_as_float(w[0] & 0xffff0000u);
    r[2] = __uint_as_float(w[1] << 16);
    r[3] = __uint_as_float(w[1] & 0xffff0000u);
    return r;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

template <int W> __device__ __forceinline__ float group_sum(float x) {
    // Sum over W consecutive lanes (W a power of two <= 64).
#pragma unroll
    for (int m = W / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
    return x;
}

}  // namespace kda
