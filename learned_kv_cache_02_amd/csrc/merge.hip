// Log-sum-exp merges of (log-normaliser, read-out) pairs, Eqs. (3.4)-(3.5) of
// the Nectar notes: the two-way merge of a document-side pair with the local
// one, and its K-way form over several document-side pairs.
#include "device_common.hpp"
#include "kernels.hpp"

namespace nectar {

// Standalone merge of two (lse, A) pairs, one wave per row.
template <int D, typename OutT>
__global__ __launch_bounds__(256) void merge_pairs(MergeParams a) {
    constexpr int NPL = D / 64;
    const long r = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= a.rows) return;
    const int lane = threadIdx.x & 63;
    const float x = a.a[r], y = a.lam[r];
    float va[NPL], vl[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const size_t e = (size_t)r * D + lane + 64 * i;
        va[i] = a.A[e];
        vl[i] = a.A_loc[e];
    }
    const float M = fmaxf(x, y);
    if (M == -INFINITY) {
#pragma unroll
        for (int i = 0; i < NPL; ++i) st_out<OutT>((OutT *)a.out, r * D + lane + 64 * i, 0.f);
        if (a.lse_out && lane == 0) a.lse_out[r] = -INFINITY;
        return;
    }
    const float wa = expf(x - M), wl = expf(y - M), den = wa + wl;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
        st_out<OutT>((OutT *)a.out, (size_t)r * D + lane + 64 * i, (wa * va[i] + wl * vl[i]) / den);
    if (a.lse_out && lane == 0) a.lse_out[r] = M + logf(den);
}

// K-way merge (the closing section's composition of several context modules):
// one wave per two rows, lane l owning the D/64 contiguous dimensions from
// l * D/64, so each pair's read-out row is one coalesced wave load.  Every
// pair's logit and read-out of both rows are loaded before the first common
// maximum is taken, and the pairs are folded in index order, the local pair last.
template <int NPL> struct RowVec;
template <> struct RowVec<1> {
    static __device__ __forceinline__ void load(const float *p, float *v) { v[0] = *p; }
    static __device__ __forceinline__ void store(float *p, const float *v) { *p = v[0]; }
    static __device__ __forceinline__ void store(uint16_t *p, const float *v) { *p = f32_to_bf16(v[0]); }
};
template <> struct RowVec<2> {
    static __device__ __forceinline__ void load(const float *p, float *v) {
        const float2 t = *(const float2 *)p;
        v[0] = t.x;
        v[1] = t.y;
    }
    static __device__ __forceinline__ void store(float *p, const float *v) { *(float2 *)p = make_float2(v[0], v[1]); }
    static __device__ __forceinline__ void store(uint16_t *p, const float *v) {
        *(uint32_t *)p = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    }
};

template <int D, typename OutT, int RPW>
__global__ __launch_bounds__(256) void merge_k_pairs(MergeKParams a) {
    constexpr int NPL = D / 64;
    using RV = RowVec<NPL>;
    const long r0 = ((long)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW;
    if (r0 >= a.rows) return;
    const bool lane0 = (threadIdx.x & 63) == 0;
    // RPW rows per wave: every pair of all of them loaded before the first maximum
    float x[RPW][kMergeKMax + 1], v[RPW][kMergeKMax + 1][NPL];
#pragma unroll
    for (int u = 0; u < RPW; ++u) {
        const long r = min(r0 + u, a.rows - 1);
        const size_t e = (size_t)r * D + (threadIdx.x & 63) * NPL;
#pragma unroll
        for (int k = 0; k <= kMergeKMax; ++k) {
            const bool loc = (k == kMergeKMax);
            const float *ps = loc ? a.lam : (k < a.K ? a.a[k] : nullptr);
            const float *pv = loc ? a.A_loc : (k < a.K ? a.A[k] : nullptr);
            x[u][k] = ps ? ps[r] : -INFINITY;
#pragma unroll
            for (int i = 0; i < NPL; ++i) v[u][k][i] = 0.f;
            if (pv) RV::load(pv + e, v[u][k]);
        }
    }
#pragma unroll
    for (int u = 0; u < RPW; ++u) {
        const long r = r0 + u;
        if (r >= a.rows) break;
        const size_t e = (size_t)r * D + (threadIdx.x & 63) * NPL;
        float M = -INFINITY;
#pragma unroll
        for (int k = 0; k <= kMergeKMax; ++k) M = fmaxf(M, x[u][k]);
        float acc[NPL];
#pragma unroll
        for (int i = 0; i < NPL; ++i) acc[i] = 0.f;
        if (M == -INFINITY) {
            RV::store((OutT *)a.out + e, acc);
            if (a.lse_out && lane0) a.lse_out[r] = -INFINITY;
            continue;
        }
        float den = 0.f;
#pragma unroll
        for (int k = 0; k <= kMergeKMax; ++k) {
            const float w = x[u][k] == -INFINITY ? 0.f : expf(x[u][k] - M);
            den += w;
#pragma unroll
            for (int i = 0; i < NPL; ++i) acc[i] += w * v[u][k][i];
        }
        const float inv = 1.0f / den;
#pragma unroll
        for (int i = 0; i < NPL; ++i) acc[i] *= inv;
        RV::store((OutT *)a.out + e, acc);
        if (a.lse_out && lane0) a.lse_out[r] = M + logf(den);
    }
}

static inline unsigned blocks_for_waves(long waves) { return (unsigned)((waves + 3) / 4); }

hipError_t launch_merge(const MergeParams &p, int dtype, int d, hipStream_t st) {
    dim3 grid(blocks_for_waves(p.rows)), block(256);
    if (d == 128 && dtype == 1) hipLaunchKernelGGL((merge_pairs<128, uint16_t>), grid, block, 0, st, p);
    else if (d == 128) hipLaunchKernelGGL((merge_pairs<128, float>), grid, block, 0, st, p);
    else if (d == 64 && dtype == 1) hipLaunchKernelGGL((merge_pairs<64, uint16_t>), grid, block, 0, st, p);
    else if (d == 64) hipLaunchKernelGGL((merge_pairs<64, float>), grid, block, 0, st, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_merge_k(const MergeKParams &p, int dtype, int d, hipStream_t st) {
    constexpr int kRows = 2;   // rows per wave
    dim3 grid(blocks_for_waves((p.rows + kRows - 1) / kRows)), block(256);
    if (d == 128 && dtype == 1) hipLaunchKernelGGL((merge_k_pairs<128, uint16_t, kRows>), grid, block, 0, st, p);
    else if (d == 128) hipLaunchKernelGGL((merge_k_pairs<128, float, kRows>), grid, block, 0, st, p);
    else if (d == 64 && dtype == 1) hipLaunchKernelGGL((merge_k_pairs<64, uint16_t, kRows>), grid, block, 0, st, p);
    else if (d == 64) hipLaunchKernelGGL((merge_k_pairs<64, float, kRows>), grid, block, 0, st, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace nectar
