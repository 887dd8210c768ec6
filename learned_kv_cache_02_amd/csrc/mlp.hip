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
#include "device_common.hpp"
#include "kernels.hpp"

namespace nectar {

template <int D> struct WRow;
template <> struct WRow<128> { typedef u32x4 T; };
template <> struct WRow<64> { typedef u32x2 T; };

// One 32-unit tile of either net: first-layer rows (A operand as loaded),
// the target read-out rows (target tiles only), biases, score read-out weights.
template <int D> struct MTile {
    static constexpr int KS = D / 32;
    u32x4 w1[2][KS];
    typename WRow<D>::T w2[8];
    float bias[8];
    float ws[8];
};

__device__ __forceinline__ int hslot(int g, int j) { return 16 * (j >> 2) + 4 * g + (j & 3); }

template <int D>
__device__ __forceinline__ void load_rows(MTile<D> &T, const uint16_t *W, int j0, int jmax, int g, int c) {
    constexpr int KS = D / 32;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const uint16_t *wp = W + (size_t)min(j0 + 16 * hh + c, jmax) * D;
#pragma unroll
        for (int kt = 0; kt < KS; ++kt) T.w1[hh][kt] = stream_load((const u32x4 *)(wp + (4 * kt + g) * 8));
    }
}

template <int D>
__device__ __forceinline__ void load_tgt(MTile<D> &T, const uint16_t *W1, const uint16_t *W2t,
                                         const float *b1, int j0, int jmax, int g, int c) {
    constexpr int DV = D / 16;
    load_rows<D>(T, W1, j0, jmax, g, c);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int u = min(j0 + hslot(g, j), jmax);
        T.w2[j] = stream_load((const typename WRow<D>::T *)(W2t + (size_t)u * D + c * DV));
        T.bias[j] = b1[u];
    }
}

template <int D>
__device__ __forceinline__ void load_score(MTile<D> &T, const uint16_t *Ws, const uint16_t *ws2,
                                           const float *bs, int j0, int jmax, int g, int c) {
    load_rows<D>(T, Ws, j0, jmax, g, c);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int u = min(j0 + hslot(g, j), jmax);
        T.bias[j] = bs[u];
        T.ws[j] = bf16_to_f32(ws2[u]);
    }
}

template <int D>
__device__ __forceinline__ void transpose_w(const MTile<D> &T, u32x4 (&vt)[D / 16]) {
    constexpr int DV = D / 16;
#pragma unroll
    for (int mm = 0; mm < DV; ++mm) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t a0 = T.w2[2 * w][mm >> 1], a1 = T.w2[2 * w + 1][mm >> 1];
            vt[mm][w] = (mm & 1) ? ((a0 >> 16) | (a1 & 0xffff0000u)) : ((a0 & 0xffffu) | (a1 << 16));
        }
    }
}

template <int D, int RT, int ACT>
__device__ __forceinline__ void tgt_tile(const MTile<D> &T, int j0, int Ht,
                                         const u32x4 (&qv)[RT][D / 32], int g, f32x4 (&O)[RT][D / 16]) {
    constexpr int KS = D / 32, DV = D / 16;
    u32x4 vt[DV];
    transpose_w<D>(T, vt);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        f32x4 z0 = {0.f, 0.f, 0.f, 0.f}, z1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < KS; ++kt) {
            z0 = mfma16(T.w1[0][kt], qv[rt][kt], z0);
            z1 = mfma16(T.w1[1][kt], qv[rt][kt], z1);
        }
        float hv[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            hv[r] = act_fn<ACT>(z0[r] + T.bias[r]);
            hv[4 + r] = act_fn<ACT>(z1[r] + T.bias[4 + r]);
        }
        if (j0 + 32 > Ht) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (j0 + hslot(g, j) >= Ht) hv[j] = 0.f;
        }
        const u32x4 H = {pack_bf16(hv[0], hv[1]), pack_bf16(hv[2], hv[3]), pack_bf16(hv[4], hv[5]),
                         pack_bf16(hv[6], hv[7])};
#pragma unroll
        for (int mm = 0; mm < DV; ++mm) O[rt][mm] = mfma16(vt[mm], H, O[rt][mm]);
    }
}

template <int D, int RT, int ACT>
__device__ __forceinline__ void score_tile(const MTile<D> &T, int j0, int Hs,
                                           const u32x4 (&qv)[RT][D / 32], int g, float (&sc)[RT]) {
    constexpr int KS = D / 32;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        f32x4 z0 = {0.f, 0.f, 0.f, 0.f}, z1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < KS; ++kt) {
            z0 = mfma16(T.w1[0][kt], qv[rt][kt], z0);
            z1 = mfma16(T.w1[1][kt], qv[rt][kt], z1);
        }
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float z = (j < 4 ? z0[j] : z1[j - 4]) + T.bias[j];
            float y = act_fn<ACT>(z) * T.ws[j];
            if (j0 + hslot(g, j) >= Hs) y = 0.f;
            acc += y;
        }
        sc[rt] += acc;
    }
}

template <int D, int RT, int ACT>
__global__ __launch_bounds__(256) void mlp_partial_mfma(MlpParams a) {
    constexpr int KS = D / 32, DV = D / 16;
    __shared__ f32x4 fold_O[2][RT * DV][64];
    __shared__ float fold_s[2][RT][64];

    const int w = threadIdx.x >> 6;
    const int wr = w % a.WR, ws = w / a.WR;
    int blk = blockIdx.x;
    const int sb = blk % a.SB;
    blk /= a.SB;
    const int rb = blk % a.RB;
    const int h = blk / a.RB;
    const int rg = rb * a.WR + wr;
    const int s = sb * a.WS + ws;
    const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;

    u32x4 qv[RT][KS];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int rho = (rg * RT + rt) * 16 + c;
        if (rg < a.RG && rho < a.Rp) {
            const int t = rho / a.G, gg = rho - t * a.G;
            const uint16_t *qp = (const uint16_t *)a.q + ((size_t)t * a.Hq + h * a.G + gg) * D;
#pragma unroll
            for (int kt = 0; kt < KS; ++kt) qv[rt][kt] = *(const u32x4 *)(qp + (4 * kt + g) * 8);
        } else {
#pragma unroll
            for (int kt = 0; kt < KS; ++kt) qv[rt][kt] = u32x4{0u, 0u, 0u, 0u};
        }
    }

    f32x4 O[RT][DV];
    float sc[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        sc[rt] = 0.f;
#pragma unroll
        for (int mm = 0; mm < DV; ++mm) O[rt][mm] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const uint16_t *W1 = (const uint16_t *)a.W1 + (size_t)h * a.Ht * D;
    const uint16_t *W2t = (const uint16_t *)a.W2t + (size_t)h * a.Ht * D;
    const float *b1 = a.b1 + (size_t)h * a.Ht;
    const uint16_t *Ws = (const uint16_t *)a.Ws + (size_t)h * a.Hs * D;
    const uint16_t *ws2 = (const uint16_t *)a.ws2 + (size_t)h * a.Hs;
    const float *bs = a.bs + (size_t)h * a.Hs;
    const int jt_lo = s * a.chunk_t, jt_hi = min(jt_lo + a.chunk_t, a.Ht);
    const int js_lo = s * a.chunk_s, js_hi = min(js_lo + a.chunk_s, a.Hs);
    const int ntt = jt_lo < jt_hi ? (jt_hi - jt_lo + 31) / 32 : 0;
    const int nts = js_lo < js_hi ? (js_hi - js_lo + 31) / 32 : 0;
    const int ntiles = rg < a.RG ? ntt + nts : 0;

    auto load = [&](MTile<D> &T, int i) {
        if (i < ntt) load_tgt<D>(T, W1, W2t, b1, jt_lo + 32 * i, a.Ht - 1, g, c);
        else load_score<D>(T, Ws, ws2, bs, js_lo + 32 * (i - ntt), a.Hs - 1, g, c);
    };
    auto run = [&](const MTile<D> &T, int i) {
        if (i < ntt) tgt_tile<D, RT, ACT>(T, jt_lo + 32 * i, a.Ht, qv, g, O);
        else score_tile<D, RT, ACT>(T, js_lo + 32 * (i - ntt), a.Hs, qv, g, sc);
    };
    if (ntiles > 0) {
        MTile<D> t0, t1;
        load(t0, 0);
        for (int i = 0; i < ntiles; i += 2) {
            const bool has1 = i + 1 < ntiles;
            if (has1) load(t1, i + 1);
            run(t0, i);
            if (!has1) break;
            if (i + 2 < ntiles) load(t0, i + 2);
            run(t1, i + 1);
        }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) sc[rt] = group4_sum(sc[rt]);

    if (a.WS > 1) {
        for (int k = a.WS - 1; k >= 1; --k) {
            if (ws == k) {
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    fold_s[wr][rt][lane] = (k == a.WS - 1) ? sc[rt] : fold_s[wr][rt][lane] + sc[rt];
#pragma unroll
                    for (int mm = 0; mm < DV; ++mm)
                        fold_O[wr][rt * DV + mm][lane] =
                            (k == a.WS - 1) ? O[rt][mm] : fold_O[wr][rt * DV + mm][lane] + O[rt][mm];
                }
            }
            __syncthreads();
        }
        if (ws != 0) return;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            sc[rt] += fold_s[wr][rt][lane];
#pragma unroll
            for (int mm = 0; mm < DV; ++mm) O[rt][mm] += fold_O[wr][rt * DV + mm][lane];
        }
    }
    if (rg >= a.RG) return;

#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int rho = (rg * RT + rt) * 16 + c;
        if (rho >= a.Rp) continue;
        if (a.SB == 1 && !a.defer) {
            const int t = rho / a.G, gg = rho - t * a.G;
            const size_t o = (size_t)t * a.Hq + h * a.G + gg;
            if (g == 0) a.a_out[o] = a.bs2[h] + sc[rt];
            const float *b2 = a.b2 + (size_t)h * D;
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int m4 = 0; m4 < DV; m4 += 4) {
                    const int dc = DV * (4 * g + r) + m4;
                    f32x4 v = {b2[dc] + O[rt][m4][r], b2[dc + 1] + O[rt][m4 + 1][r],
                               b2[dc + 2] + O[rt][m4 + 2][r], b2[dc + 3] + O[rt][m4 + 3][r]};
                    *(f32x4 *)(a.A_out + o * D + dc) = v;
                }
        } else {
            const size_t row = (size_t)(h * a.SB + sb) * a.Rp + rho;
            if (g == 0) a.part_s[row] = sc[rt];
            float *op = a.part_O + row * D;
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int m4 = 0; m4 < DV; m4 += 4) {
                    f32x4 v = {O[rt][m4][r], O[rt][m4 + 1][r], O[rt][m4 + 2][r], O[rt][m4 + 3][r]};
                    *(f32x4 *)(op + DV * (4 * g + r) + m4) = v;
                }
        }
    }
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

// One block per (KV head, row): output bias plus the split partials, summed in
// a fixed order.  Every load is issued before the first reduction.
template <int D, int MAXI>
__global__ __launch_bounds__(256) void mlp_reduce(MlpReduceParams a) {
    constexpr int DQ = D / 4;
    constexpr int NSG = 256 / DQ;
    __shared__ f32x4 accs[NSG][DQ];
    __shared__ float red[4];
    const int idx = blockIdx.x;
    const int h = idx / a.Rp, rho = idx - h * a.Rp;
    const int tid = threadIdx.x;
    const int t = rho / a.G, gg = rho - t * a.G;
    const size_t o = (size_t)t * a.Hq + h * a.G + gg;
    const size_t base = (size_t)h * a.S * a.Rp + rho;      // row of split 0; stride Rp per split
    const int sg = tid / DQ, dq = tid - sg * DQ;

    f32x4 ov[MAXI];
    float sv[MAXI];
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
        const int s = sg + i * NSG;
        const bool in = s < a.S;
        ov[i] = in ? *(const f32x4 *)(a.part_O + (base + (size_t)s * a.Rp) * D + 4 * dq) : f32x4{0.f, 0.f, 0.f, 0.f};
        sv[i] = (in && dq == 0) ? a.part_s[base + (size_t)s * a.Rp] : 0.f;
    }
    f32x4 acc = ov[0];
    float sacc = sv[0];
#pragma unroll
    for (int i = 1; i < MAXI; ++i) { acc += ov[i]; sacc += sv[i]; }
    for (int s = sg + MAXI * NSG; s < a.S; s += NSG) {
        acc += *(const f32x4 *)(a.part_O + (base + (size_t)s * a.Rp) * D + 4 * dq);
        if (dq == 0) sacc += a.part_s[base + (size_t)s * a.Rp];
    }
    accs[sg][dq] = acc;
#pragma unroll
    for (int o2 = 32; o2 >= 1; o2 >>= 1) sacc += __shfl_xor(sacc, o2, 64);
    if ((tid & 63) == 0) red[tid >> 6] = sacc;
    __syncthreads();
    if (tid >= DQ) return;
    f32x4 O = *(const f32x4 *)(a.b2 + (size_t)h * D + 4 * tid);
    for (int k = 0; k < NSG; ++k) O += accs[k][tid];
    *(f32x4 *)(a.A_out + o * D + 4 * tid) = O;
    if (tid == 0) a.a_out[o] = a.bs2[h] + ((red[0] + red[1]) + (red[2] + red[3]));
}

static inline unsigned blocks_for_waves(long waves) { return (unsigned)((waves + 3) / 4); }

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

hipError_t launch_mlp_reduce(const MlpReduceParams &p, int d, hipStream_t st) {
    dim3 grid((unsigned)((long)p.Hkv * p.Rp)), block(256);
    if (d == 128) hipLaunchKernelGGL((mlp_reduce<128, 8>), grid, block, 0, st, p);
    else if (d == 64) hipLaunchKernelGGL((mlp_reduce<64, 4>), grid, block, 0, st, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace nectar
