// Finishing pass of a whole layer step (sections 2.1-2.2 of the Nectar notes):
// per query row, the local part's split partials are folded by log-sum-exp into
// (lambda, A_local); each document-side part -- the exact document attention
// or a Quadrature module (log-sum-exp partials) or an MLP module (plain sums
// plus output biases) -- is folded into its pair (alpha, A) or (a, A); and each
// pair is merged with the local one as the virtual logit of Eqs. (3.4)-(3.5).
//
// One wave per (local row, slice of NC float4 columns): lane (g, c) owns column
// c of the slice for the splits g, g + NG, ... of every part (NG = 64 / NC) and
// issues all of its loads (statistics, read-outs, of all parts) before the
// first reduction, so a row costs one memory round trip; the split groups are
// folded by butterfly exchanges within the wave (no barriers), in a fixed
// order, so every lane ends with the same totals.
#include "attn_common.hpp"

namespace nectar {

namespace {

constexpr int kMaxSets = 3;   // local part + two document-side parts

}  // namespace

template <int D, typename OutT, int NC>
__global__ __launch_bounds__(64) void attn_finish(FinishParams a) {
    constexpr int NB = D / 4 / NC;     // waves per row
    constexpr int NG = 64 / NC;        // split groups
    constexpr int MAXI = 64 / NG;      // splits per lane loaded up front (64 per part)

    int row, cb;
    slice_of_block<NB>(row, cb);
    if (row >= a.P * a.Rp) return;
    const int p = row / a.Rp, rho = row - p * a.Rp;
    const int b = p / a.Hkv, h = p - b * a.Hkv;
    const size_t o = out_row(p, rho, a.Hkv, a.G, a.Tq, a.Hq);
    const int rho_doc = b * a.Tq * a.G + rho;      // the same query row in the document problems
    const int lane = threadIdx.x, sg = lane / NC;
    const int dc = 4 * (cb * NC + (lane - sg * NC));  // first of this lane's four dims
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
            const int s = sg + i * NG;
            // absent splits: an empty log-sum-exp partial, or a zero sum
            st[k][i] = make_float2(pml[k] ? -INFINITY : 0.f, 0.f);
            ov[k][i] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (k < nparts && s < S[k]) {
                if (pml[k]) st[k][i] = pml[k][s * stride[k]];
                else st[k][i] = make_float2(ps[k][s * stride[k]], 0.f);
                ov[k][i] = *(const f32x4 *)(pO[k] + s * stride[k] * D + dc);
            }
        }

    // per part: (M in log2 units, L, O) with the read-out unnormalised by L.
    // The maxima of all parts are folded together, then every sum of all parts.
    float mx[kMaxSets];
#pragma unroll
    for (int k = 0; k < kMaxSets; ++k) {
        mx[k] = -INFINITY;
        if (k >= nparts || !pml[k]) continue;   // uniform
#pragma unroll
        for (int i = 0; i < MAXI; ++i) mx[k] = fmaxf(mx[k], st[k][i].x);
        for (int s = sg + MAXI * NG; s < S[k]; s += NG) mx[k] = fmaxf(mx[k], pml[k][s * stride[k]].x);
    }
    splits_fold<NC, true>(mx);
    float red[kMaxSets * 5];                    // per part: the scalar sum, then four read-out sums
#pragma unroll
    for (int i = 0; i < kMaxSets * 5; ++i) red[i] = 0.f;
#pragma unroll
    for (int k = 0; k < kMaxSets; ++k) {
        if (k >= nparts) continue;             // uniform
        float lloc = 0.f;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (pml[k]) {
            const float Mk = mx[k];
            if (Mk != -INFINITY) {
#pragma unroll
                for (int i = 0; i < MAXI; ++i) {
                    const float w = exp2f(st[k][i].x - Mk);
                    lloc += w * st[k][i].y;
                    acc += w * ov[k][i];
                }
                for (int s = sg + MAXI * NG; s < S[k]; s += NG) {
                    const float2 v = pml[k][s * stride[k]];
                    const float w = exp2f(v.x - Mk);
                    lloc += w * v.y;
                    acc += w * *(const f32x4 *)(pO[k] + s * stride[k] * D + dc);
                }
            }
        } else {
            // MLP module: a = bs2 + sum of score partials, A = b2 + sum of read-out partials
#pragma unroll
            for (int i = 0; i < MAXI; ++i) {
                lloc += st[k][i].x;
                acc += ov[k][i];
            }
            for (int s = sg + MAXI * NG; s < S[k]; s += NG) {
                lloc += ps[k][s * stride[k]];
                acc += *(const f32x4 *)(pO[k] + s * stride[k] * D + dc);
            }
        }
        red[5 * k] = lloc;
#pragma unroll
        for (int e = 0; e < 4; ++e) red[5 * k + 1 + e] = acc[e];
    }
    splits_fold<NC, false>(red);
    float M[kMaxSets], L[kMaxSets];
    f32x4 O[kMaxSets];
#pragma unroll
    for (int k = 0; k < kMaxSets; ++k) {
        O[k] = f32x4{red[5 * k + 1], red[5 * k + 2], red[5 * k + 3], red[5 * k + 4]};
        if (k >= nparts) {
            M[k] = -INFINITY;
            L[k] = 0.f;
        } else if (pml[k]) {
            M[k] = mx[k];
            L[k] = red[5 * k];
        } else {
            M[k] = (a.set[k - 1].bs2[h] + red[5 * k]) * kLog2e;   // the pair's log-normaliser, log2 units
            L[k] = 1.f;
            O[k] += *(const f32x4 *)(a.set[k - 1].b2 + (size_t)h * D + dc);
        }
    }
    if (sg != 0) return;
    const bool lead = (cb == 0 && lane == 0);   // writes the row's scalars

    // the pairs
    auto write_pair = [&](int k, float *lse_out, float *A_out) {
        const bool empty = (M[k] == -INFINITY);
        if (lse_out && lead) lse_out[o] = empty ? -INFINITY : (M[k] + log2f(L[k])) * kLn2;
        if (A_out) *(f32x4 *)(A_out + o * D + dc) = empty ? f32x4{0.f, 0.f, 0.f, 0.f} : O[k] * (1.0f / L[k]);
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
        if (f.out_lse && lead) f.out_lse[o] = none ? -INFINITY : (Mt + log2f(Lt)) * kLn2;
        if (f.out) {
            const f32x4 r = (wl * O[0] + wk * O[k]) * it;
#pragma unroll
            for (int i = 0; i < 4; ++i) st_out<OutT>((OutT *)f.out, o * D + dc + i, none ? 0.f : r[i]);
        }
    }
}

hipError_t launch_finish(const FinishParams &p, int dtype, int d, hipStream_t st) {
    // float4 columns per wave: 2 (16 waves per row at d = 128) for few rows; from
    // 128 rows on, 4 (1M-token decode stack with 224 rows per layer: 6.6 -> 5.9 us
    // per layer; the 4B decode step with the batched folds is flat, 54.5-54.8 us)
#ifndef NECTAR_FINISH_COLS_MANY
#define NECTAR_FINISH_COLS_MANY 4
#endif
#ifndef NECTAR_FINISH_MANY_ROWS
#define NECTAR_FINISH_MANY_ROWS 128
#endif
    constexpr int kCols = 2;
    const long rows = (long)p.P * p.Rp;
    const int nc = rows >= NECTAR_FINISH_MANY_ROWS ? NECTAR_FINISH_COLS_MANY : kCols;
    dim3 grid((unsigned)slice_grid(rows, d / 4 / nc)), block(64);
#define NECTAR_FINISH_CASE(NC) \
    if (nc == NC) { \
        if (d == 128 && dtype == 1) hipLaunchKernelGGL((attn_finish<128, uint16_t, NC>), grid, block, 0, st, p); \
        else if (d == 128) hipLaunchKernelGGL((attn_finish<128, float, NC>), grid, block, 0, st, p); \
        else if (d == 64 && dtype == 1) hipLaunchKernelGGL((attn_finish<64, uint16_t, NC>), grid, block, 0, st, p); \
        else if (d == 64) hipLaunchKernelGGL((attn_finish<64, float, NC>), grid, block, 0, st, p); \
        else return hipErrorInvalidValue; \
        return hipGetLastError(); }
    NECTAR_FINISH_CASE(2) NECTAR_FINISH_CASE(4) NECTAR_FINISH_CASE(8)
#undef NECTAR_FINISH_CASE
    return hipErrorInvalidValue;
}

}  // namespace nectar
