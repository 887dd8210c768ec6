// Device helpers shared by the attention kernels: the P-slot key order of a
// 32-key tile, output row addressing and the in-place row finish (log-sum-exp,
// normalised read-out, optional merge with an extra pair, Eq. (3.5) of the
// Nectar notes).
#pragma once

#include "device_common.hpp"
#include "kernels.hpp"

namespace nectar {

// Key held by P slot j of lane group g within a 32-key tile.
__device__ __forceinline__ int slot_key(int g, int j) { return 16 * (j >> 2) + 4 * g + (j & 3); }

// Output row index of row rho of problem p.
__device__ __forceinline__ size_t out_row(int p, int rho, int Hkv, int G, int Tq, int Hq) {
    const int b = p / Hkv, h = p - b * Hkv;
    const int t = rho / G, gg = rho - t * G;
    return (size_t)(b * Tq + t) * Hq + h * G + gg;
}

// Finish one row held in lane layout: lane (g, c) owns dims DV*(4g+r)+mm of the
// row; m (log2 units) and l are the row's folded statistics.
template <int D, typename OutT>
__device__ __forceinline__ void finish_row_lanes(const AttnParams &a, size_t o, int g, float m, float l,
                                                 const f32x4 (&O)[D / 16]) {
    constexpr int DV = D / 16;
    const bool empty = (m == -INFINITY);
    const float inv = empty ? 0.f : 1.0f / l;
    if (a.lse_out && g == 0) a.lse_out[o] = empty ? -INFINITY : (m + log2f(l)) * kLn2;
    if (a.A_out) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int m4 = 0; m4 < DV; m4 += 4) {
                f32x4 v = {O[m4][r] * inv, O[m4 + 1][r] * inv, O[m4 + 2][r] * inv, O[m4 + 3][r] * inv};
                *(f32x4 *)(a.A_out + o * D + DV * (4 * g + r) + m4) = v;
            }
    }
    if (a.x_lse) {
        const float mx = a.x_lse[o] * kLog2e;
        const float Mt = fmaxf(m, mx);
        const bool none = (Mt == -INFINITY);
        const float wl = (none || empty) ? 0.f : exp2f(m - Mt);
        const float wx = none ? 0.f : exp2f(mx - Mt);
        const float Lt = wl * l + wx;
        const float it = none ? 0.f : 1.0f / Lt;
        if (a.out_lse && g == 0) a.out_lse[o] = none ? -INFINITY : (Mt + log2f(Lt)) * kLn2;
        if (a.out) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float ov[DV];
                const float *xa = a.x_A + o * D + DV * (4 * g + r);
#pragma unroll
                for (int mm = 0; mm < DV; ++mm) ov[mm] = none ? 0.f : (wl * O[mm][r] + wx * xa[mm]) * it;
#pragma unroll
                for (int mm = 0; mm < DV; ++mm) st_out<OutT>((OutT *)a.out, o * D + DV * (4 * g + r) + mm, ov[mm]);
            }
        }
    }
}

}  // namespace nectar
