// Device-side helpers shared by the Nectar HIP kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nectar {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 16x16x32 bf16 matrix FMA, fp32 accumulate.  Operand lanes: lane l supplies
// row (A) / column (B) l % 16 and eight contraction slots owned by lane group
// l / 16 (the same slot assignment for A and B).  Result lane l holds column
// l % 16, rows 4 * (l / 16) + 0..3.
__device__ __forceinline__ f32x4 mfma16(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Loads of data streamed once per call (document cache, module weights):
// non-temporal, so the stream does not evict data that is reused.
template <typename T> __device__ __forceinline__ T stream_load(const T *p) {
    return __builtin_nontemporal_load(p);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return (uint16_t)(pack_bf16(f, 0.0f) & 0xffffu);
}

// Element loads of the storage type, widened to fp32.
template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float ld(const float *p, size_t i) { return p[i]; }
};
template <> struct Elem<uint16_t> {
    static __device__ __forceinline__ float ld(const uint16_t *p, size_t i) { return bf16_to_f32(p[i]); }
};

template <typename T> __device__ __forceinline__ void st_out(T *p, size_t i, float v);
template <> __device__ __forceinline__ void st_out<float>(float *p, size_t i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void st_out<uint16_t>(uint16_t *p, size_t i, float v) {
    p[i] = f32_to_bf16(v);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Sum / max over the four 16-lane groups (lanes c, c+16, c+32, c+48).
__device__ __forceinline__ float group4_sum(float v) {
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}
__device__ __forceinline__ float group4_max(float v) {
    v = fmaxf(v, __shfl_xor(v, 16, 64));
    v = fmaxf(v, __shfl_xor(v, 32, 64));
    return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// GELU in the erf form, x * Phi(x) (HIP device erff).
__device__ __forceinline__ float gelu_erf(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }
__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

__device__ __forceinline__ float activation(int act, float x) { return act == 1 ? silu(x) : gelu_erf(x); }

}  // namespace nectar
