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
typedef float f32x16 __attribute__((ext_vector_type(16)));

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

// 32x32x16 bf16 matrix FMA, fp32 accumulate.  Operand lane l supplies row (A)
// / column (B) l % 32 and contraction slots 8 * (l / 32) .. + 7.  Result
// register i of lane l holds column l % 32, row 8 * (i / 4) + 4 * (l / 32) + i % 4.
__device__ __forceinline__ f32x16 mfma32(const u32x4 &a, const u32x4 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
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

// Block -> (row, slice) of a split reduction with NB waves per row: the NB
// slices of a row share blockIdx % 8, which the dispatcher sends to one XCD
// (block ids go round-robin over the eight), so the cache lines the slices
// split are fetched into a single L2.  The grid covers the rows rounded up to
// a multiple of 8; `row` may pass the last row.
template <int NB> __device__ __forceinline__ void slice_of_block(int &row, int &cb) {
    if (NB == 1) {
        row = blockIdx.x;
        cb = 0;
    } else {
        const int x = blockIdx.x & 7, y = blockIdx.x >> 3;
        cb = y % NB;
        row = (y / NB) * 8 + x;
    }
}
static inline long slice_grid(long rows, int nb) { return nb == 1 ? rows : (rows + 7) / 8 * 8 * nb; }

// Folds over the split groups of a wave whose lane (g, c) = (lane / NC, lane %
// NC) holds column c of the splits of group g: lanes that differ only in the
// bits from NC up are combined, N independent values at a time, and every lane
// ends with the total of its column.  The steps inside a row of 16 lanes are
// DPP row rotations (a rotation by o, then by 2o, ..., sums each lane with every
// lane of its row that agrees with it modulo o); the steps across rows are
// lane exchanges.  The order is fixed, so the totals are reproducible and equal
// in every lane of a column.
template <int OFF> __device__ __forceinline__ float row_rotate(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x120 + OFF, 0xf, 0xf, false));
}
template <int NC, bool MAX, int N> __device__ __forceinline__ void splits_fold(float (&v)[N]) {
    auto fold = [&](auto get) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const float o = get(v[i]);
            v[i] = MAX ? fmaxf(v[i], o) : v[i] + o;
        }
    };
    if constexpr (NC <= 1) fold([](float x) { return row_rotate<1>(x); });
    if constexpr (NC <= 2) fold([](float x) { return row_rotate<2>(x); });
    if constexpr (NC <= 4) fold([](float x) { return row_rotate<4>(x); });
    if constexpr (NC <= 8) fold([](float x) { return row_rotate<8>(x); });
    if constexpr (NC <= 16) fold([](float x) { return __shfl_xor(x, 16, 64); });
    if constexpr (NC <= 32) fold([](float x) { return __shfl_xor(x, 32, 64); });
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// GELU in the erf form, x * Phi(x) with Phi(x) = (1 + erf(x / sqrt 2)) / 2 and
// erf from Abramowitz & Stegun, Handbook of Mathematical Functions, 7.1.26
// (|error| <= 1.5e-7): erf(z) = 1 - (a1 t + ... + a5 t^5) exp(-z^2),
// t = 1 / (1 + p z), z >= 0, odd extension.  Branch-free: one reciprocal, one
// exponential and nine arithmetic operations.
__device__ __forceinline__ float gelu_erf(float x) {
    const float z = fabsf(x) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.3275911f, z, 1.0f));
    float p = __builtin_fmaf(1.061405429f, t, -1.453152027f);
    p = __builtin_fmaf(p, t, 1.421413741f);
    p = __builtin_fmaf(p, t, -0.284496736f);
    p = __builtin_fmaf(p, t, 0.254829592f);
    const float e = __builtin_amdgcn_exp2f(-z * z * 1.4426950408889634f);
    const float erfc_half = 0.5f * (p * t) * e;                  // (1 - erf(z)) / 2
    return x * (x >= 0.f ? 1.0f - erfc_half : erfc_half);        // x * Phi(x)
}
// SiLU, x * sigmoid(x) = x / (1 + e^-x) (hardware exp2 and reciprocal).
__device__ __forceinline__ float silu(float x) {
    return x * __builtin_amdgcn_rcpf(1.0f + fast_exp2(-x * kLog2e));
}

// GELU in the tanh form, 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) =
// x * sigmoid(1.5957691 x (1 + 0.044715 x^2)) (Hendrycks & Gimpel's
// approximation); it differs from the erf form by at most 4.8e-4.
__device__ __forceinline__ float gelu_tanh(float x) {
    const float v = x * __builtin_fmaf(x * x, -0.0713548162726f * kLog2e, -1.5957691216057308f * kLog2e);
    return x * __builtin_amdgcn_rcpf(1.0f + fast_exp2(v));
}

// erf-form GELU for the VALU-bound batched and decode MLP kernels: x * Phi(x)
// with Phi(x) = 0.5 + c P(c^2), c = x clamped to [-3.71875, 3.71875], P of
// degree 6 fitted to the odd part of Phi (fit_gelu_erf.py): max |Phi error|
// 5.2e-5, so |GELU error| <= 5.2e-5 |x|.  Ten multiply-add-class operations, no
// exponential or reciprocal (four issue slots each on this part).
__device__ __forceinline__ float gelu_erf_poly(float x) {
    const float c = __builtin_amdgcn_fmed3f(x, -3.71875f, 3.71875f);
    const float u = c * c;
    float p = __builtin_fmaf(u, 4.07418810e-08f, -2.44288435e-06f);
    p = __builtin_fmaf(p, u, 6.33929594e-05f);
    p = __builtin_fmaf(p, u, -9.51952359e-04f);
    p = __builtin_fmaf(p, u, 9.39021632e-03f);
    p = __builtin_fmaf(p, u, -6.58312142e-02f);
    p = __builtin_fmaf(p, u, 3.98723632e-01f);
    return x * __builtin_fmaf(c, p, 0.5f);
}

// Derivatives of the activations (the backward pass of the training step):
//   GELU erf form: Phi(x) + x phi(x), Phi with the same 7.1.26 erf as gelu_erf;
//   SiLU: s (1 + x (1 - s)), s = sigmoid(x);
//   tanh form x sigmoid(v), v = 1.5957691 (x + 0.044715 x^3):
//       sigmoid(v) + x sigmoid(v) (1 - sigmoid(v)) 1.5957691 (1 + 0.134145 x^2).
__device__ __forceinline__ float gelu_erf_grad(float x) {
    const float z = fabsf(x) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.3275911f, z, 1.0f));
    float p = __builtin_fmaf(1.061405429f, t, -1.453152027f);
    p = __builtin_fmaf(p, t, 1.421413741f);
    p = __builtin_fmaf(p, t, -0.284496736f);
    p = __builtin_fmaf(p, t, 0.254829592f);
    const float e = __builtin_amdgcn_exp2f(-z * z * 1.4426950408889634f);   // exp(-x^2 / 2)
    const float erfc_half = 0.5f * (p * t) * e;
    const float Phi = x >= 0.f ? 1.0f - erfc_half : erfc_half;
    return Phi + x * e * 0.3989422804014327f;
}
__device__ __forceinline__ float silu_grad(float x) {
    const float sg = __builtin_amdgcn_rcpf(1.0f + fast_exp2(-x * kLog2e));
    return sg * (1.0f + x * (1.0f - sg));
}
__device__ __forceinline__ float gelu_tanh_grad(float x) {
    const float v = 1.5957691216057308f * x * __builtin_fmaf(0.044715f, x * x, 1.0f);
    const float sg = __builtin_amdgcn_rcpf(1.0f + fast_exp2(-v * kLog2e));
    return sg + x * sg * (1.0f - sg) * 1.5957691216057308f * __builtin_fmaf(0.134145f, x * x, 1.0f);
}
template <int ACT> __device__ __forceinline__ float act_grad_fn(float x) {
    return ACT == 1 ? silu_grad(x) : (ACT == 2 ? gelu_tanh_grad(x) : gelu_erf_grad(x));
}

// Activation fixed at compile time (0: GELU erf form, 1: SiLU, 2: GELU tanh
// form, the values of nectar_act), so only one is evaluated.
template <int ACT> __device__ __forceinline__ float act_fn(float x) {
    return ACT == 1 ? silu(x) : (ACT == 2 ? gelu_tanh(x) : gelu_erf(x));
}
__device__ __forceinline__ float activation(int act, float x) {
    return act == 1 ? silu(x) : (act == 2 ? gelu_tanh(x) : gelu_erf(x));
}

}  // namespace nectar
