// Fit metrics of a module against the exact pair: the squared errors of the
// regression losses, Eqs. (3.2)-(3.3) of the Nectar notes, and the summand of
// the relative target error of Eq. (C.1), log(||A_theta - A||^2 / ||q - A||^2).
//
// Pass 1: one wave per four (token, query head) rows; lane l owns the D/64
// consecutive dimensions from l * D/64, so each of the three d-vectors is one
// coalesced wave load; the two squared norms are wave sums.  Passes 2 and 3:
// the per-KV-head sums in fp64, each head's rows cut into kFitParts contiguous
// ranges summed by one block each (every thread a fixed strided subset, then a
// fixed tree), then the parts in index order -- the result does not depend on
// scheduling.
#include "device_common.hpp"
#include "kernels.hpp"

namespace nectar {

// RPW rows per wave, every load of all of them issued before the first sum.
template <int D, typename T, int RPW>
__global__ __launch_bounds__(256) void fit_rows(FitParams a) {
    constexpr int NPL = D / 64;
    const long i0 = ((long)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW;
    if (i0 >= a.rows) return;
    const int lane = threadIdx.x & 63;
    float ex[RPW][NPL], av[RPW][NPL], qv[RPW][NPL], sa[RPW], sb[RPW];
#pragma unroll
    for (int u = 0; u < RPW; ++u) {
        const long i = min(i0 + u, a.rows - 1);
        const size_t e = (size_t)i * D + lane * NPL;
#pragma unroll
        for (int k = 0; k < NPL; ++k) {
            ex[u][k] = a.Aex[e + k];
            av[u][k] = a.A[e + k];
            qv[u][k] = Elem<T>::ld((const T *)a.q, e + k);
        }
        sa[u] = a.a[i];
        sb[u] = a.alpha[i];
    }
#pragma unroll
    for (int u = 0; u < RPW; ++u) {
        const long i = i0 + u;
        float et = 0.f, eq = 0.f;
#pragma unroll
        for (int k = 0; k < NPL; ++k) {
            const float x = av[u][k] - ex[u][k];
            const float y = qv[u][k] - ex[u][k];
            et = __builtin_fmaf(x, x, et);
            eq = __builtin_fmaf(y, y, eq);
        }
        et = wave_sum(et);
        eq = wave_sum(eq);
        if (lane == 0 && i < a.rows) {
            const float ds = sa[u] - sb[u];
            float *o = a.row + 3 * (size_t)i;
            o[0] = ds * ds;
            o[1] = et;
            o[2] = logf(et / eq);
        }
    }
}

// Pass 2: block b of KV head h sums the contiguous range b of the head's rows
// (enumerated token-major, then query head of the group) into part[h][b][3].
__global__ __launch_bounds__(256) void fit_head_parts(FitParams a) {
    const int h = blockIdx.x / kFitParts, b = blockIdx.x - h * kFitParts, G = a.Hq / a.Hkv;
    const long n = a.rows / a.Hq * G;          // rows of this KV head
    const long lo = n * b / kFitParts, hi = n * (b + 1) / kFitParts;
    double s[3] = {0.0, 0.0, 0.0};
    for (long j = lo + threadIdx.x; j < hi; j += 256) {
        const long t = j / G;
        const int g = (int)(j - t * G);
        const float *o = a.row + 3 * ((size_t)t * a.Hq + h * G + g);
        s[0] += o[0];
        s[1] += o[1];
        s[2] += o[2];
    }
    __shared__ double red[3][256];
#pragma unroll
    for (int k = 0; k < 3; ++k) red[k][threadIdx.x] = s[k];
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
        if ((int)threadIdx.x < w)
#pragma unroll
            for (int k = 0; k < 3; ++k) red[k][threadIdx.x] += red[k][threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x < 3) a.part[(size_t)blockIdx.x * 3 + threadIdx.x] = red[threadIdx.x][0];
}

// Pass 3: the parts of each head in index order.
__global__ __launch_bounds__(64) void fit_head_sums(FitParams a) {
    const int h = blockIdx.x, k = threadIdx.x;
    if (k >= 3) return;
    double s = 0.0;
    for (int b = 0; b < kFitParts; ++b) s += a.part[((size_t)h * kFitParts + b) * 3 + k];
    a.head[3 * h + k] = s;
}

hipError_t launch_fit_metrics(const FitParams &p, int dtype, int d, hipStream_t st) {
    constexpr int kRows = 4;   // rows per wave
    dim3 grid((unsigned)((p.rows + 4 * kRows - 1) / (4 * kRows))), block(256);
    if (d == 128 && dtype == 1) hipLaunchKernelGGL((fit_rows<128, uint16_t, kRows>), grid, block, 0, st, p);
    else if (d == 128) hipLaunchKernelGGL((fit_rows<128, float, kRows>), grid, block, 0, st, p);
    else if (d == 64 && dtype == 1) hipLaunchKernelGGL((fit_rows<64, uint16_t, kRows>), grid, block, 0, st, p);
    else if (d == 64) hipLaunchKernelGGL((fit_rows<64, float, kRows>), grid, block, 0, st, p);
    else return hipErrorInvalidValue;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !p.head) return e;
    hipLaunchKernelGGL(fit_head_parts, dim3(p.Hkv * kFitParts), block, 0, st, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(fit_head_sums, dim3(p.Hkv), dim3(64), 0, st, p);
    return hipGetLastError();
}

}  // namespace nectar
