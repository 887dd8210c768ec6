// Finishing pass of a whole layer step (sections 2.1-2.2 of the Nectar notes):
// per query row, the local part's split partials are folded by log-sum-exp into
// (lambda, A_local); each document-side part -- the exact document attention
// or a Quadrature module (log-sum-exp partials) or an MLP module (plain sums
// plus output biases) -- is folded into its pair (alpha, A) or (a, A); and each
// pair is merged with the local one as the virtual logit of Eqs. (3.4)-(3.5).
//
// One block per local row.  Thread (sg, dq) owns four dimensions of the splits
// sg, sg + NSG, ... of every part and issues all of its loads (statistics,
// read-outs, of all parts) before the first reduction, so a row costs one
// memory round trip; the splits are folded in a fixed order.
#include "attn_common.hpp"

namespace nectar {

namespace {

constexpr int kMaxSets = 3;   // local part + two document-side parts

// Block-wide reductions of one value per thread over the four waves.
__device__ __forceinline__ float block_max(float v, float *red) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ float block_sum(float v, float *red) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

}  // namespace

template <int D, typename OutT, int MAXI>
__global__ __launch_bounds__(256) void attn_finish(FinishParams a) {
    constexpr int DQ = D / 4;          // float4 columns
    constexpr int NSG = 256 / DQ;      // split groups
    __shared__ float red[kMaxSets][2][4];
    __shared__ f32x4 accs[kMaxSets][NSG][DQ];

    const int idx = blockIdx.x;
    const int p = idx / a.Rp, rho = idx - p * a.Rp;
    const int b = p / a.Hkv, h = p - b * a.Hkv;
    const size_t o = out_row(p, rho, a.Hkv, a.G, a.Tq, a.Hq);
    const int rho_doc = b * a.Tq * a.G + rho;      // the same query row in the document problems
    const int tid = threadIdx.x, sg = tid / DQ, dq = tid - sg * DQ;
    const int nparts = 1 + a.nsets;

    // part k: base pointers with split stride `stride` rows
    const float *pO[kMaxSets];
    const float2 *pml[kMaxSets];
    const float *ps[kMaxSets];
    int S[kMaxSets];
    size_t stride[kMaxSets];
    pO[0] = a.loc_O + ((size_t)p * a.S_loc * a.Rp + rho) * D;
    pml[0] = a.loc_ml + (size_t)p * a.S_loc * a.Rp + rho;
    ps[0] = nullptr;
    S[0] = a.S_loc;
    stride[0] = a.Rp;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const FinishSet &f = a.set[k];
        const size_t base = (size_t)h * (k < a.nsets ? f.S : 0) * a.Rp_doc + rho_doc;
        pO[k + 1] = k < a.nsets ? f.O + base * D : nullptr;
        pml[k + 1] = k < a.nsets && f.ml ? f.ml + base : nullptr;
        ps[k + 1] = k < a.nsets && f.s ? f.s + base : nullptr;
        S[k + 1] = k < a.nsets ? f.S : 0;
        stride[k + 1] = a.Rp_doc;
    }

    // every load first
    float2 st[kMaxSets][MAXI];
    f32x4 ov[kMaxSets][MAXI];
#pragma unroll
    for (int k = 0; k < kMaxSets; ++k)
#pragma unroll
        for (int i = 0; i < MAXI; ++i) {
            const int s = sg + i * NSG;
            // absent splits: an empty log-sum-exp partial, or a zero sum
            st[k][i] = make_float2(pml[k] ? -INFINITY : 0.f, 0.f);
            ov[k][i] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (k < nparts && s < S[k]) {
                if (pml[k]) st[k][i] = pml[k][s * stride[k]];
                else st[k][i] = make_float2(ps[k][s * stride[k]], 0.f);
                ov[k][i] = *(const f32x4 *)(pO[k] + s * stride[k] * D + 4 * dq);
            }
        }

    // per part: (M in log2 units, L, O) with the read-out unnormalised by L
    float M[kMaxSets], L[kMaxSets];
#pragma unroll
    for (int k = 0; k < kMaxSets; ++k) {
        M[k] = -INFINITY;
        L[k] = 0.f;
        if (k >= nparts) continue;             // uniform
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (pml[k]) {
            float mloc = -INFINITY;
#pragma unroll
            for (int i = 0; i < MAXI; ++i) mloc = fmaxf(mloc, st[k][i].x);
            for (int s = sg + MAXI * NSG; s < S[k]; s += NSG) mloc = fmaxf(mloc, pml[k][s * stride[k]].x);
            const float Mk = block_max(mloc, red[k][0]);
            float lloc = 0.f;
            if (Mk != -INFINITY) {
#pragma unroll
                for (int i = 0; i < MAXI; ++i) {
                    const float w = exp2f(st[k][i].x - Mk);
                    lloc += w * st[k][i].y;
                    acc += w * ov[k][i];
                }
                for (int s = sg + MAXI * NSG; s < S[k]; s += NSG) {
                    const float2 v = pml[k][s * stride[k]];
                    const float w = exp2f(v.x - Mk);
                    lloc += w * v.y;
                    acc += w * *(const f32x4 *)(pO[k] + s * stride[k] * D + 4 * dq);
                }
            }
            // each split's l counted once: only the dq == 0 thread of a group adds it
            L[k] = block_sum(dq == 0 ? lloc : 0.f, red[k][1]);
            M[k] = Mk;
        } else {
            // MLP module: a = bs2 + sum of score partials, A = b2 + sum of read-out partials
            float sloc = 0.f;
#pragma unroll
            for (int i = 0; i < MAXI; ++i) {
                sloc += st[k][i].x;
                acc += ov[k][i];
            }
            for (int s = sg + MAXI * NSG; s < S[k]; s += NSG) {
                sloc += ps[k][s * stride[k]];
                acc += *(const f32x4 *)(pO[k] + s * stride[k] * D + 4 * dq);
            }
            const float asum = block_sum(dq == 0 ? sloc : 0.f, red[k][1]);
            M[k] = (a.set[k - 1].bs2[h] + asum) * kLog2e;   // the pair's log-normaliser, log2 units
            L[k] = 1.f;
        }
        accs[k][sg][dq] = acc;
    }
    __syncthreads();
    if (tid >= DQ) return;

    f32x4 O[kMaxSets];
#pragma unroll
    for (int k = 0; k < kMaxSets; ++k) {
        O[k] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (k >= nparts) continue;
#pragma unroll
        for (int j = 0; j < NSG; ++j) O[k] += accs[k][j][tid];
        if (k > 0 && !pml[k]) O[k] += *(const f32x4 *)(a.set[k - 1].b2 + (size_t)h * D + 4 * tid);
    }

    // the pairs
    auto write_pair = [&](int k, float *lse_out, float *A_out) {
        const bool empty = (M[k] == -INFINITY);
        if (lse_out && tid == 0) lse_out[o] = empty ? -INFINITY : (M[k] + log2f(L[k])) * kLn2;
        if (A_out) *(f32x4 *)(A_out + o * D + 4 * tid) = empty ? f32x4{0.f, 0.f, 0.f, 0.f} : O[k] * (1.0f / L[k]);
    };
    write_pair(0, a.lam_out, a.Aloc_out);
#pragma unroll
    for (int k = 1; k < kMaxSets; ++k) {
        if (k >= nparts) continue;
        const FinishSet &f = a.set[k - 1];
        write_pair(k, f.lse_out, f.A_out);
        // merge with the local part: common maximum, weights, one normaliser
        const float Mt = fmaxf(M[0], M[k]);
        const bool none = (Mt == -INFINITY);
        const float wl = (none || M[0] == -INFINITY) ? 0.f : exp2f(M[0] - Mt);
        const float wk = (none || M[k] == -INFINITY) ? 0.f : exp2f(M[k] - Mt);
        const float Lt = wl * L[0] + wk * L[k];
        const float it = none ? 0.f : 1.0f / Lt;
        if (f.out_lse && tid == 0) f.out_lse[o] = none ? -INFINITY : (Mt + log2f(Lt)) * kLn2;
        if (f.out) {
            const f32x4 r = (wl * O[0] + wk * O[k]) * it;
#pragma unroll
            for (int i = 0; i < 4; ++i) st_out<OutT>((OutT *)f.out, o * D + 4 * tid + i, none ? 0.f : r[i]);
        }
    }
}

hipError_t launch_finish(const FinishParams &p, int dtype, int d, hipStream_t st) {
    dim3 grid((unsigned)((long)p.P * p.Rp)), block(256);
    if (d == 128 && dtype == 1) hipLaunchKernelGGL((attn_finish<128, uint16_t, 8>), grid, block, 0, st, p);
    else if (d == 128) hipLaunchKernelGGL((attn_finish<128, float, 8>), grid, block, 0, st, p);
    else if (d == 64 && dtype == 1) hipLaunchKernelGGL((attn_finish<64, uint16_t, 4>), grid, block, 0, st, p);
    else if (d == 64) hipLaunchKernelGGL((attn_finish<64, float, 4>), grid, block, 0, st, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace nectar
