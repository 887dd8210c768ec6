// Nectar MLP module forward (Eq. (3.6) of the Nectar notes with one hidden
// layer, the workloads' depth): per KV head h and query row,
//   target A = sum_j W2t[h][j] * act(W1[h][j] . q + b1[h][j]) + b2[h]
//   score  a = sum_j ws2[h][j] * act(Ws[h][j] . q + bs[h][j]) + bs2[h]
// batched over all query heads of the KV group and all query tokens.
//
// bf16 path (mlp_partial_mfma): the attention kernel's register-direct MFMA
// skeleton with the hidden units in place of keys.  Z^T = W1_tile . Q^T on
// MFMA, bias + activation on the fp32 accumulators, the hidden tile is
// rounded to bf16 and fed straight back as the B operand of
// O^T += W2t_tile^T . H^T (W2t rows transposed inside each lane), so the hidden
// activations never leave registers.  The score net keeps its hidden values in
// fp32 and dots them with ws2 on the VALU.  Each wave walks its target tiles
// and then its score tiles as one double-buffered stream, so every weight load
// of the wave is issued before the previous tile's math.  A block folds its WS
// hidden splits in LDS; with one block per row group the block adds the output
// biases and writes (a, A) itself, otherwise mlp_reduce adds the partials in
// split order.
#include "mlp_body.hpp"
#include "mlp_decode.hpp"

namespace nectar {

// Decode shapes (up to 64 rows per KV head): target and score waves, every
// tile load issued up front, block fold through LDS (mlp_decode.hpp).
template <int D, int RT, int ACT>
__global__ __launch_bounds__((dec_threads(D, RT)), (dec_min_blocks(D, RT))) void mlp_decode_mfma(MlpParams a) {
    mlp_decode_body<D, RT, ACT, kDecTiles>(a, (int)blockIdx.x);
}

// Two weight tiles in registers (4B decode module: 13.4 us; three 13.4 us, four
// 13.7 us).
template <int D, int RT, int ACT>
__global__ __launch_bounds__(256) void mlp_partial_mfma(MlpParams a) {
    mlp_partial_body<D, RT, ACT, 2>(a, (int)blockIdx.x);
}

// fp32 path: one wave per (KV head, row, split); lanes own output dimensions.
template <int D, typename T>
__global__ __launch_bounds__(256) void mlp_partial_valu(MlpParams a) {
    constexpr int NPL = D / 64;
    const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wave >= a.Hkv * a.S * a.Rp) return;
    const int s = wave % a.S;
    const int rho = (wave / a.S) % a.Rp;
    const int h = wave / (a.S * a.Rp);
    const int lane = threadIdx.x & 63;
    const int t = rho / a.G, gg = rho - t * a.G;
    const T *qp = (const T *)a.q + ((size_t)t * a.Hq + h * a.G + gg) * D;
    float qf[NPL], acc[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) { qf[i] = Elem<T>::ld(qp, lane + 64 * i); acc[i] = 0.f; }
    const T *W1 = (const T *)a.W1 + (size_t)h * a.Ht * D;
    const T *W2t = (const T *)a.W2t + (size_t)h * a.Ht * D;
    const int j_lo = s * a.chunk_t, j_hi = min(j_lo + a.chunk_t, a.Ht);
    for (int j = j_lo; j < j_hi; ++j) {
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < NPL; ++i) part += Elem<T>::ld(W1, (size_t)j * D + lane + 64 * i) * qf[i];
        const float y = activation(a.act, wave_sum(part) + a.b1[(size_t)h * a.Ht + j]);
#pragma unroll
        for (int i = 0; i < NPL; ++i) acc[i] += Elem<T>::ld(W2t, (size_t)j * D + lane + 64 * i) * y;
    }
    const T *Ws = (const T *)a.Ws + (size_t)h * a.Hs * D;
    const T *ws2 = (const T *)a.ws2 + (size_t)h * a.Hs;
    const int js_lo = s * a.chunk_s, js_hi = min(js_lo + a.chunk_s, a.Hs);
    float sc = 0.f;
    for (int j = js_lo; j < js_hi; ++j) {
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < NPL; ++i) part += Elem<T>::ld(Ws, (size_t)j * D + lane + 64 * i) * qf[i];
        sc += Elem<T>::ld(ws2, j) * activation(a.act, wave_sum(part) + a.bs[(size_t)h * a.Hs + j]);
    }
    const size_t row = (size_t)(h * a.S + s) * a.Rp + rho;
    if (lane == 0) a.part_s[row] = sc;
#pragma unroll
    for (int i = 0; i < NPL; ++i) a.part_O[row * D + lane + 64 * i] = acc[i];
}

// One wave per (KV head, row, slice of NC float4 columns): output bias plus the
// split partials, folded in a fixed order.  Lane (g, c) owns four dims of the
// splits g, g + NG, ... (NG = 64 / NC); every load is issued before the first
// reduction.
template <int D, int NC, int MAXI>
__global__ __launch_bounds__(64) void mlp_reduce(MlpReduceParams a) {
    constexpr int NB = D / 4 / NC;       // waves per row
    constexpr int NG = 64 / NC;          // split groups
    int row, cb;
    slice_of_block<NB>(row, cb);
    if (row >= a.Hkv * a.Rp) return;
    const int h = row / a.Rp, rho = row - h * a.Rp;
    const int lane = threadIdx.x, sg = lane / NC;
    const int dc = 4 * (cb * NC + (lane - sg * NC));
    const int t = rho / a.G, gg = rho - t * a.G;
    const size_t o = (size_t)t * a.Hq + h * a.G + gg;
    const size_t base = (size_t)h * a.S * a.Rp + rho;      // row of split 0; stride Rp per split

    f32x4 ov[MAXI];
    float sv[MAXI];
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
        const int s = sg + i * NG;
        const bool in = s < a.S;
        ov[i] = in ? *(const f32x4 *)(a.part_O + (base + (size_t)s * a.Rp) * D + dc) : f32x4{0.f, 0.f, 0.f, 0.f};
        sv[i] = in ? a.part_s[base + (size_t)s * a.Rp] : 0.f;
    }
    f32x4 acc = ov[0];
    float sacc = sv[0];
#pragma unroll
    for (int i = 1; i < MAXI; ++i) { acc += ov[i]; sacc += sv[i]; }
    for (int s = sg + MAXI * NG; s < a.S; s += NG) {
        acc += *(const f32x4 *)(a.part_O + (base + (size_t)s * a.Rp) * D + dc);
        sacc += a.part_s[base + (size_t)s * a.Rp];
    }
    float red[5] = {sacc, acc[0], acc[1], acc[2], acc[3]};
    splits_fold<NC, false>(red);
    const float ssum = red[0];
    const f32x4 O = {red[1], red[2], red[3], red[4]};
    if (sg != 0) return;
    *(f32x4 *)(a.A_out + o * D + dc) = O + *(const f32x4 *)(a.b2 + (size_t)h * D + dc);
    if (cb == 0 && lane == 0) a.a_out[o] = a.bs2[h] + ssum;
}

static inline unsigned blocks_for_waves(long waves) { return (unsigned)((waves + 3) / 4); }

int mlp_row_tiles(int Rp) { return Rp <= 16 ? 1 : (Rp <= 32 ? 2 : 4); }

hipError_t launch_mlp_partial(const MlpParams &p, int dtype, int d, int rt, hipStream_t st) {
    if (dtype == 1) {
        dim3 grid((unsigned)((long)p.Hkv * p.RB * p.SB)), block(256);
#define NECTAR_MLP_CASE(DD, RR) \
        if (d == DD && rt == RR) { \
            if (p.act == 1) hipLaunchKernelGGL((mlp_partial_mfma<DD, RR, 1>), grid, block, 0, st, p); \
            else if (p.act == 2) hipLaunchKernelGGL((mlp_partial_mfma<DD, RR, 2>), grid, block, 0, st, p); \
            else hipLaunchKernelGGL((mlp_partial_mfma<DD, RR, 0>), grid, block, 0, st, p); \
            return hipGetLastError(); }
        NECTAR_MLP_CASE(128, 1) NECTAR_MLP_CASE(128, 2)
        NECTAR_MLP_CASE(64, 1) NECTAR_MLP_CASE(64, 2)
#undef NECTAR_MLP_CASE
        return hipErrorInvalidValue;
    }
    const long waves = (long)p.Hkv * p.S * p.Rp;
    dim3 grid(blocks_for_waves(waves)), block(256);
    if (d == 128) hipLaunchKernelGGL((mlp_partial_valu<128, float>), grid, block, 0, st, p);
    else if (d == 64) hipLaunchKernelGGL((mlp_partial_valu<64, float>), grid, block, 0, st, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_mlp_decode(const MlpParams &p, int d, int rt, hipStream_t st) {
    dim3 grid((unsigned)((long)p.Hkv * p.RG * p.SB));
#define NECTAR_DEC_CASE(DD, RR) \
    if (d == DD && rt == RR) { \
        const dim3 block((dec_threads(DD, RR))); \
        if (p.act == 1) hipLaunchKernelGGL((mlp_decode_mfma<DD, RR, 1>), grid, block, 0, st, p); \
        else if (p.act == 2) hipLaunchKernelGGL((mlp_decode_mfma<DD, RR, 2>), grid, block, 0, st, p); \
        else hipLaunchKernelGGL((mlp_decode_mfma<DD, RR, 0>), grid, block, 0, st, p); \
        return hipGetLastError(); }
    NECTAR_DEC_CASE(128, 1) NECTAR_DEC_CASE(128, 2) NECTAR_DEC_CASE(128, 4)
    NECTAR_DEC_CASE(64, 1) NECTAR_DEC_CASE(64, 2) NECTAR_DEC_CASE(64, 4)
#undef NECTAR_DEC_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_mlp_reduce(const MlpReduceParams &p, int d, hipStream_t st) {
    const long rows = (long)p.Hkv * p.Rp;
    const int nc = reduce_cols(rows, d, true);
    dim3 grid((unsigned)slice_grid(rows, d / 4 / nc)), block(64);
#define NECTAR_REDUCE_CASE(DD) \
    if (d == DD) { \
        if (nc == 4) hipLaunchKernelGGL((mlp_reduce<DD, 4, 4>), grid, block, 0, st, p); \
        else if (nc == 8) hipLaunchKernelGGL((mlp_reduce<DD, 8, 8>), grid, block, 0, st, p); \
        else hipLaunchKernelGGL((mlp_reduce<DD, DD / 4, 64 * 8 / DD>), grid, block, 0, st, p); \
        return hipGetLastError(); }
    NECTAR_REDUCE_CASE(128) NECTAR_REDUCE_CASE(64)
#undef NECTAR_REDUCE_CASE
    return hipErrorInvalidValue;
}

}  // namespace nectar
