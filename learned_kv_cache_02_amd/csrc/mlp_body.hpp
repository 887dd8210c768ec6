// Device code of the register-direct MFMA MLP partial kernel (see mlp.hip),
// shared with the fused decode-step launch.
#pragma once

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

// Block blk_id of the MLP partial grid (Hkv x RB x SB blocks of 4 waves).
// NBUF: weight tiles held in registers at once -- NBUF - 1 tiles in flight while
// one is computed (about 80 registers per tile); 1 loads each tile just before
// its use.
template <int D, int RT, int ACT, int NBUF = 2>
__device__ __forceinline__ void mlp_partial_body(const MlpParams &a, int blk_id) {
    constexpr int KS = D / 32, DV = D / 16;
    __shared__ f32x4 fold_O[2][RT * DV][64];
    __shared__ float fold_s[2][RT][64];

    const int w = threadIdx.x >> 6;
    const int wr = w % a.WR, ws = w / a.WR;
    int blk = blk_id;
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
    if (NBUF == 1) {
        for (int i = 0; i < ntiles; ++i) {
            MTile<D> t0;
            load(t0, i);
            run(t0, i);
        }
    } else if (ntiles > 0) {
        // ring of NBUF tiles: before tile i is computed, tile i + NBUF - 1 is
        // issued into the slot tile i - 1 has just left (static slot indices)
        MTile<D> t[NBUF];
#pragma unroll
        for (int k = 0; k < NBUF - 1; ++k)
            if (k < ntiles) load(t[k], k);
        for (int i0 = 0; i0 < ntiles; i0 += NBUF) {
#pragma unroll
            for (int k = 0; k < NBUF; ++k) {
                const int i = i0 + k;
                if (i >= ntiles) break;
                if (i + NBUF - 1 < ntiles) load(t[(k + NBUF - 1) % NBUF], i + NBUF - 1);
                run(t[k], i);
            }
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

}  // namespace nectar
