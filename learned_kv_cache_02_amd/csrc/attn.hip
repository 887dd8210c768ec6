// Split-K softmax attention with log-sum-exp partials and its combine: the
// exact document path (Eq. (3.1) of the Nectar notes),
// the Quadrature module (exact attention over p pairs) and the causal local
// part (section 2.2), all as one kernel family.
//
// bf16 path (attn_partial_mfma): every wave owns RT tiles of 16 query rows and
// one contiguous key range, and streams 32-key tiles of K and V straight from
// HBM into registers (no LDS):
//   S^T (32 keys x 16 rows) = K_tile . Q^T   -- K rows are MFMA A operands as
//       loaded: lane (g, c) holds 16 bytes of key c, so four consecutive lanes'
//       loads cover 64 contiguous bytes of one key row;
//   online max/sum per row in fp32, P = exp2(S * scale * log2e - m) -> bf16;
//   O^T (d x 16 rows) += V_tile^T . P^T -- lane (g, c) loads dims 8c..8c+7 of
//       the eight keys its P slots hold (one 256-byte key row per 16 lanes) and
//       transposes the 8x8 bf16 block inside its own registers, so each wave
//       load instruction reads four whole key rows.
// The S^T layout puts one query row per lane column, so every row statistic
// (max, sum, rescale) stays in the lane; only the tile max crosses the four
// 16-lane groups.  A wave issues the loads of a batch of SUB tiles before it
// uses any of them, and at RT == 1 two waves share each SIMD, so one wave's
// loads are in flight while the other computes.
//
// This register-direct form serves a few rows per KV head (decode); with more
// rows (RT > 1 here) every row group re-streams the cache, which the
// LDS-staged kernel in attn_lds.hip avoids for d = 128.
//
// A block's four waves cover WR row groups x WS key splits; the WS splits of a
// row group are folded in LDS (log-sum-exp rescale, then a sum), so each block
// leaves one partial per row.  When one block spans the whole key range the
// block finishes the rows itself (lse, read-out, optional merge); otherwise
// attn_combine folds the per-block partials.  (A last-arriving-block fold was
// measured slower: the agent-scope fences it needs write back and invalidate
// the XCD's L2 on every block.)
#include "attn_body.hpp"

namespace nectar {

// RT == 1: two waves per SIMD (8 per CU), each with a 32 KB batch in flight;
// blocks [0, nb0) serve the first problem set, the rest the second.
template <int D, int RT, int SUB, typename OutT>
__global__ __launch_bounds__(256, RT == 1 ? NECTAR_RT1_WAVES_PER_SIMD : 1) void attn_partial_mfma(AttnGroup gr) {
    const int set = group_set(gr, (int)blockIdx.x);
    attn_partial_body<D, RT, SUB, OutT>(gr.p[set], (int)blockIdx.x - (set ? gr.nb0 : 0));
}

// fp32 path: one wave per (problem, row, split); lanes own head dimensions,
// keys are visited in order with a wave-wide dot product.
template <int D, typename T>
__global__ __launch_bounds__(256) void attn_partial_valu(AttnParams a) {
    constexpr int NPL = D / 64;
    const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wave >= a.P * a.S * a.Rp) return;
    const int s = wave % a.S;
    const int rho = (wave / a.S) % a.Rp;
    const int p = wave / (a.S * a.Rp);
    const int b = p / a.Hkv, h = p - b * a.Hkv;
    const int lane = threadIdx.x & 63;
    const int t = rho / a.G, gg = rho - t * a.G;
    const T *qp = (const T *)a.q + ((size_t)(b * a.Tq + t) * a.Hq + h * a.G + gg) * D;
    const T *kb = (const T *)a.k + b * a.kv_bstride + h * a.kv_hstride;
    const T *vb = (const T *)a.v + b * a.kv_bstride + h * a.kv_hstride;
    float qf[NPL], acc[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) { qf[i] = Elem<T>::ld(qp, lane + 64 * i); acc[i] = 0.f; }
    int L = a.T_kv;
    if (a.causal) L = min(L, a.q_offset + t + 1);
    const int k_lo = s * a.chunk, k_hi = min(k_lo + a.chunk, L);
    float m = -INFINITY, l = 0.f;
    for (int j = k_lo; j < k_hi; ++j) {
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < NPL; ++i) part += qf[i] * Elem<T>::ld(kb, (size_t)j * a.kv_row + lane + 64 * i);
        const float s2 = wave_sum(part) * a.sl2;
        const float mnew = fmaxf(m, s2);
        const float alpha = exp2f(m - mnew);
        const float pj = exp2f(s2 - mnew);
        l = l * alpha + pj;
#pragma unroll
        for (int i = 0; i < NPL; ++i) acc[i] = acc[i] * alpha + pj * Elem<T>::ld(vb, (size_t)j * a.kv_row + lane + 64 * i);
        m = mnew;
    }
    const size_t row = (size_t)(p * a.S + s) * a.Rp + rho;
    if (lane == 0) a.part_ml[row] = make_float2(m, l);
#pragma unroll
    for (int i = 0; i < NPL; ++i) a.part_O[row * D + lane + 64 * i] = acc[i];
}

// One wave per (problem, row, slice of NC float4 columns): log-sum-exp fold of
// the S partials in a fixed order, then the optional merge with an extra
// (lse, A) pair (Eq. (3.5)).  Lane (g, c) owns four dims of the splits g,
// g + NG, ... (NG = 64 / NC) and issues every load it needs (statistics,
// read-outs, the extra pair) before the first reduction, so a row costs one
// memory round trip; the split groups are folded within the wave.
template <int D, typename OutT, int NC, int MAXI>
__global__ __launch_bounds__(64) void attn_combine(CombineParams a) {
    constexpr int NB = D / 4 / NC;       // waves per row
    constexpr int NG = 64 / NC;          // split groups
    int row, cb;
    slice_of_block<NB>(row, cb);
    if (row >= a.P * a.Rp) return;
    const int p = row / a.Rp, rho = row - p * a.Rp;
    const int lane = threadIdx.x, sg = lane / NC;
    const int dc = 4 * (cb * NC + (lane - sg * NC));
    const size_t o = out_row(p, rho, a.Hkv, a.G, a.Tq, a.Hq);
    const float2 *ml = a.part_ml + (size_t)p * a.S * a.Rp + rho;   // stride Rp over splits
    const float *po = a.part_O + ((size_t)p * a.S * a.Rp + rho) * D;

    float2 st[MAXI];
    f32x4 ov[MAXI];
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
        const int s = sg + i * NG;
        if (s < a.S) {
            st[i] = ml[(size_t)s * a.Rp];
            ov[i] = *(const f32x4 *)(po + (size_t)s * a.Rp * D + dc);
        } else {
            st[i] = make_float2(-INFINITY, 0.f);
            ov[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    float mx = -INFINITY;
    f32x4 xa = {0.f, 0.f, 0.f, 0.f};
    if (a.x_lse) {
        mx = a.x_lse[o] * kLog2e;
        if (a.out && sg == 0) xa = *(const f32x4 *)(a.x_A + o * D + dc);
    }
    // splits beyond MAXI * NG (very long split lists) are folded serially
    float mloc = -INFINITY;
#pragma unroll
    for (int i = 0; i < MAXI; ++i) mloc = fmaxf(mloc, st[i].x);
    for (int s = sg + MAXI * NG; s < a.S; s += NG) mloc = fmaxf(mloc, ml[(size_t)s * a.Rp].x);
    float mred[1] = {mloc};
    splits_fold<NC, true>(mred);
    const float M = mred[0];
    const bool empty = (M == -INFINITY);
    float lloc = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (!empty) {
#pragma unroll
        for (int i = 0; i < MAXI; ++i) {
            const float w = exp2f(st[i].x - M);
            lloc += w * st[i].y;
            acc += w * ov[i];
        }
        for (int s = sg + MAXI * NG; s < a.S; s += NG) {
            const float2 v = ml[(size_t)s * a.Rp];
            const float w = exp2f(v.x - M);
            lloc += w * v.y;
            acc += w * *(const f32x4 *)(po + (size_t)s * a.Rp * D + dc);
        }
    }
    float red[5] = {lloc, acc[0], acc[1], acc[2], acc[3]};
    splits_fold<NC, false>(red);
    const float L = red[0];
    const f32x4 O = {red[1], red[2], red[3], red[4]};
    if (sg != 0) return;
    const bool lead = (cb == 0 && lane == 0);   // writes the row's scalars

    const float inv = empty ? 0.f : 1.0f / L;
    if (a.lse_out && lead) a.lse_out[o] = empty ? -INFINITY : (M + log2f(L)) * kLn2;
    if (a.A_out) *(f32x4 *)(a.A_out + o * D + dc) = O * inv;
    if (a.x_lse) {
        const float Mt = fmaxf(M, mx);
        const bool none = (Mt == -INFINITY);
        const float wl = (none || empty) ? 0.f : exp2f(M - Mt);
        const float wx = none ? 0.f : exp2f(mx - Mt);
        const float Lt = wl * L + wx;
        const float it = none ? 0.f : 1.0f / Lt;
        if (a.out_lse && lead) a.out_lse[o] = none ? -INFINITY : (Mt + log2f(Lt)) * kLn2;
        if (a.out) {
            const f32x4 r = (wl * O + wx * xa) * it;
#pragma unroll
            for (int i = 0; i < 4; ++i) st_out<OutT>((OutT *)a.out, o * D + dc + i, none ? 0.f : r[i]);
        }
    }
}

__global__ __launch_bounds__(256) void fill_zero(uint32_t *p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t st) {
    const size_t n = bytes / 4;
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(fill_zero, dim3((unsigned)blocks), dim3(256), 0, st, (uint32_t *)p, n);
    return hipGetLastError();
}

int row_tiles_for(int Rp) { return Rp <= 16 ? 1 : 2; }

static inline unsigned blocks_for_waves(long waves) { return (unsigned)((waves + 3) / 4); }

static hipError_t launch_mfma_group(const AttnGroup &gr, long blocks, int d, int rt, hipStream_t st) {
    dim3 grid((unsigned)blocks), block(256);
#define NECTAR_ATTN_CASE(DD, RR) \
    if (d == DD && rt == RR) { hipLaunchKernelGGL((attn_partial_mfma<DD, RR, (RR == 1 ? NECTAR_RT1_SUB : 1), uint16_t>), grid, block, 0, st, gr); return hipGetLastError(); }
    NECTAR_ATTN_CASE(128, 1) NECTAR_ATTN_CASE(128, 2)
    NECTAR_ATTN_CASE(64, 1) NECTAR_ATTN_CASE(64, 2)
#undef NECTAR_ATTN_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_attn_partial_pair(const AttnParams &p0, const AttnParams &p1, int d, int rt, hipStream_t st) {
    AttnGroup gr;
    gr.p[0] = p0;
    gr.p[1] = p1;
    gr.nb0 = (int)((long)p0.P * p0.RB * p0.SB);
    return launch_mfma_group(gr, gr.nb0 + (long)p1.P * p1.RB * p1.SB, d, rt, st);
}

hipError_t launch_attn_partial(const AttnParams &p, int dtype, int d, int rt, hipStream_t st) {
    if (dtype == 1) {
        AttnGroup gr;
        gr.p[0] = p;
        gr.p[1] = p;
        const long blocks = (long)p.P * p.RB * p.SB;
        gr.nb0 = (int)blocks;
        return launch_mfma_group(gr, blocks, d, rt, st);
    }
    const long waves = (long)p.P * p.S * p.Rp;
    dim3 grid(blocks_for_waves(waves)), block(256);
    if (d == 128) hipLaunchKernelGGL((attn_partial_valu<128, float>), grid, block, 0, st, p);
    else if (d == 64) hipLaunchKernelGGL((attn_partial_valu<64, float>), grid, block, 0, st, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_attn_combine(const CombineParams &p, int dtype, int d, hipStream_t st) {
    const long rows = (long)p.P * p.Rp;
    // 8-dim slices for the fewest rows (4B exact entry point, 32 rows: 48.0 ->
    // 47.4 us; at 224 rows 16-dim slices stay faster, 10.7 against 11.0 us)
    const int nc0 = reduce_cols(rows, d, false);
    const int nc = (nc0 == 4 && rows <= 64) ? 2 : nc0;
    dim3 grid((unsigned)slice_grid(rows, d / 4 / nc)), block(64);
    // splits loaded up front: 64 for 16-dim slices, 8 (d = 128) or 32 (d = 64) for whole rows
#define NECTAR_COMBINE_CASE(DD, T) \
    if (d == DD) { \
        if (nc == 2) hipLaunchKernelGGL((attn_combine<DD, T, 2, 2>), grid, block, 0, st, p); \
        else if (nc == 4) hipLaunchKernelGGL((attn_combine<DD, T, 4, 4>), grid, block, 0, st, p); \
        else hipLaunchKernelGGL((attn_combine<DD, T, DD / 4, 64 * 8 / DD>), grid, block, 0, st, p); \
        return hipGetLastError(); }
    if (dtype == 1) { NECTAR_COMBINE_CASE(128, uint16_t) NECTAR_COMBINE_CASE(64, uint16_t) }
    else { NECTAR_COMBINE_CASE(128, float) NECTAR_COMBINE_CASE(64, float) }
#undef NECTAR_COMBINE_CASE
    return hipErrorInvalidValue;
}

}  // namespace nectar
