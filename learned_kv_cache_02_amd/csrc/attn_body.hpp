// Device code of the register-direct MFMA attention partial kernel (see
// attn.hip), shared with the fused decode-step launch.
#pragma once

#include "attn_common.hpp"

namespace nectar {

template <int D> struct VRow;
template <> struct VRow<128> { typedef u32x4 T; };   // 8 bf16 per lane per key
template <> struct VRow<64> { typedef u32x2 T; };    // 4 bf16 per lane per key

template <int D> struct KVTile {
    static constexpr int KS = D / 32;
    u32x4 k[2][KS];
    typename VRow<D>::T v[8];
};

template <int D>
__device__ __forceinline__ void load_kv_tile(KVTile<D> &T, const uint16_t *kb, const uint16_t *vb,
                                             int64_t row, int k0, int kmax, int g, int c) {
    constexpr int KS = D / 32, DV = D / 16;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int key = min(k0 + 16 * hh + c, kmax);
        const uint16_t *kp = kb + (size_t)key * row;
#pragma unroll
        for (int kt = 0; kt < KS; ++kt) T.k[hh][kt] = stream_load((const u32x4 *)(kp + (4 * kt + g) * 8));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int key = min(k0 + slot_key(g, j), kmax);
        T.v[j] = stream_load((const typename VRow<D>::T *)(vb + (size_t)key * row + c * DV));
    }
}

// vt[mm] slot j = V[key(g, j)][c * DV + mm]: in-lane 8 x DV transpose of bf16.
template <int D>
__device__ __forceinline__ void transpose_v(const KVTile<D> &T, u32x4 (&vt)[D / 16]) {
    constexpr int DV = D / 16;
#pragma unroll
    for (int mm = 0; mm < DV; ++mm) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t a0 = T.v[2 * w][mm >> 1], a1 = T.v[2 * w + 1][mm >> 1];
            vt[mm][w] = (mm & 1) ? ((a0 >> 16) | (a1 & 0xffff0000u)) : ((a0 & 0xffffu) | (a1 << 16));
        }
    }
}

template <int D, int RT>
__device__ __forceinline__ void attend_tile(const KVTile<D> &T, int k0, const u32x4 (&qv)[RT][D / 32],
                                            const int (&lim)[RT], float sl2, int g,
                                            f32x4 (&O)[RT][D / 16], float (&m)[RT], float (&l)[RT]) {
    constexpr int KS = D / 32, DV = D / 16;
    u32x4 vt[DV];
    transpose_v<D>(T, vt);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < KS; ++kt) {
            s0 = mfma16(T.k[0][kt], qv[rt][kt], s0);
            s1 = mfma16(T.k[1][kt], qv[rt][kt], s1);
        }
        float sv[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) { sv[r] = s0[r]; sv[4 + r] = s1[r]; }
        if (k0 + 32 > lim[rt]) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (k0 + slot_key(g, j) >= lim[rt]) sv[j] = -INFINITY;
        }
        // Lazy reference: the tile's weights against the row's current
        // reference m first; the reference moves to the running maximum (and
        // O and l are rescaled) only when a lane's weights sum past 2^8 -- which
        // every weight above 2^8 makes them do -- or the row has none yet and
        // sees a key of the tile (rows masked to nothing keep none).  The
        // same reference enters numerator and denominator, so the function is
        // unchanged, and the common tile skips the max reduction and the
        // rescale of O.
        float nm = (m[rt] == -INFINITY) ? 0.f : -m[rt];
        float pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) pv[j] = fast_exp2(__builtin_fmaf(sv[j], sl2, nm));
        float ps = ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
        if (__ballot((m[rt] == -INFINITY && k0 < lim[rt]) || !(ps <= 256.f)) != 0) {
            float mt = sv[0];
#pragma unroll
            for (int j = 1; j < 8; ++j) mt = fmaxf(mt, sv[j]);
            const float mnew = fmaxf(m[rt], group4_max(mt * sl2));
            const float sc = (m[rt] == -INFINITY) ? 0.f : fast_exp2(m[rt] - mnew);
            l[rt] *= sc;
#pragma unroll
            for (int mm = 0; mm < DV; ++mm) O[rt][mm] *= sc;
            m[rt] = mnew;
            nm = (mnew == -INFINITY) ? 0.f : -mnew;
#pragma unroll
            for (int j = 0; j < 8; ++j) pv[j] = fast_exp2(__builtin_fmaf(sv[j], sl2, nm));
            ps = ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
        }
        l[rt] += ps;
        const u32x4 P = {pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3]), pack_bf16(pv[4], pv[5]),
                         pack_bf16(pv[6], pv[7])};
#pragma unroll
        for (int mm = 0; mm < DV; ++mm) O[rt][mm] = mfma16(vt[mm], P, O[rt][mm]);
    }
}

#ifndef NECTAR_RT1_WAVES_PER_SIMD
#define NECTAR_RT1_WAVES_PER_SIMD 2
#endif
#ifndef NECTAR_RT1_SUB
#define NECTAR_RT1_SUB 2
#endif
// Fold buffers of a block (used when WS > 1, hence WR <= 2): per row group
// one f32x4 per (register, lane), lane-major so each wave access is
// conflict-free.
template <int D, int RT> struct AttnFoldLds {
    f32x4 O[2][RT * (D / 16)][64];
    float l[2][RT][64];
    float m[4][RT][16];
};

// RT == 1: two waves per SIMD (8 per CU), each with a 32 KB batch in flight.
// Block blk_id of one problem set's grid (P x RB x SB blocks of 4 waves); fl
// is the block's fold buffer (a kernel that also runs other bodies shares it).
template <int D, int RT, int SUB, typename OutT>
__device__ __forceinline__ void attn_partial_body_lds(const AttnParams &a, int blk_id, AttnFoldLds<D, RT> &fl) {
    constexpr int KS = D / 32, DV = D / 16;

    const int w = threadIdx.x >> 6;
    const int wr = w % a.WR, ws = w / a.WR;
    int blk = blk_id;
    const int sb = blk % a.SB;
    blk /= a.SB;
    const int rb = blk % a.RB;
    const int p = blk / a.RB;
    const int rg = rb * a.WR + wr;
    const int s = sb * a.WS + ws;
    const int b = p / a.Hkv, h = p - b * a.Hkv;
    const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
    const uint16_t *kb = (const uint16_t *)a.k + b * a.kv_bstride + h * a.kv_hstride;
    const uint16_t *vb = (const uint16_t *)a.v + b * a.kv_bstride + h * a.kv_hstride;

    u32x4 qv[RT][KS];
    int lim[RT];
    int wlim = 0;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int rho = (rg * RT + rt) * 16 + c;
        if (rg < a.RG && rho < a.Rp) {
            const int t = rho / a.G, gg = rho - t * a.G;
            const uint16_t *qp = (const uint16_t *)a.q + ((size_t)(b * a.Tq + t) * a.Hq + h * a.G + gg) * D;
#pragma unroll
            for (int kt = 0; kt < KS; ++kt) qv[rt][kt] = *(const u32x4 *)(qp + (4 * kt + g) * 8);
            int L = a.T_kv;
            if (a.causal) L = min(L, a.q_offset + t + 1);
            lim[rt] = max(L, 0);
        } else {
#pragma unroll
            for (int kt = 0; kt < KS; ++kt) qv[rt][kt] = u32x4{0u, 0u, 0u, 0u};
            lim[rt] = 0;
        }
        wlim = max(wlim, lim[rt]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) wlim = max(wlim, __shfl_xor(wlim, o, 64));
    // a negative scale is carried by the query's sign (exact for bf16), so the
    // tile code works with sl2 > 0 (masked scores stay -inf)
    float sl2 = a.sl2;
    if (sl2 < 0.f) {
        sl2 = -sl2;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int kt = 0; kt < KS; ++kt) qv[rt][kt] ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
    }

    f32x4 O[RT][DV];
    float m[RT], l[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        m[rt] = -INFINITY;
        l[rt] = 0.f;
#pragma unroll
        for (int mm = 0; mm < DV; ++mm) O[rt][mm] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    int k_lo, k_hi;
    if (a.tiles > 0) {
        k_lo = (int)((long)s * a.tiles / a.S) * a.chunk;
        k_hi = min((int)((long)(s + 1) * a.tiles / a.S) * a.chunk, wlim);
    } else {
        k_lo = s * a.chunk;
        k_hi = min(k_lo + a.chunk, wlim);
    }
    if (k_lo < k_hi) {
        // Batches of SUB 32-key tiles: every load of a batch (SUB x 16 KB) is
        // issued before its first use, and the two waves sharing each SIMD keep
        // the memory system busy while the other one computes.
        const int kmax = a.T_kv - 1;
        int limw[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) limw[rt] = min(lim[rt], k_hi);
        for (int k0 = k_lo; k0 < k_hi; k0 += 32 * SUB) {
            KVTile<D> tl[SUB];
#pragma unroll
            for (int u = 0; u < SUB; ++u) load_kv_tile<D>(tl[u], kb, vb, a.kv_row, min(k0 + 32 * u, kmax), kmax, g, c);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < SUB; ++u) attend_tile<D, RT>(tl[u], k0 + 32 * u, qv, limw, sl2, g, O, m, l);
        }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) l[rt] = group4_sum(l[rt]);

    if (a.WS > 1) {
        // Fold the WS splits of this row group: common max, rescale, sum.
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
            if (g == 0) fl.m[w][rt][c] = m[rt];
        __syncthreads();
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float M = -INFINITY;
            for (int k = 0; k < a.WS; ++k) M = fmaxf(M, fl.m[k * a.WR + wr][rt][c]);
            const float sc = (m[rt] == -INFINITY) ? 0.f : exp2f(m[rt] - M);
            l[rt] *= sc;
#pragma unroll
            for (int mm = 0; mm < DV; ++mm) O[rt][mm] *= sc;
            m[rt] = M;
        }
        for (int k = a.WS - 1; k >= 1; --k) {
            if (ws == k) {
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    fl.l[wr][rt][lane] = (k == a.WS - 1) ? l[rt] : fl.l[wr][rt][lane] + l[rt];
#pragma unroll
                    for (int mm = 0; mm < DV; ++mm)
                        fl.O[wr][rt * DV + mm][lane] =
                            (k == a.WS - 1) ? O[rt][mm] : fl.O[wr][rt * DV + mm][lane] + O[rt][mm];
                }
            }
            __syncthreads();
        }
        if (ws == 0) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                l[rt] += fl.l[wr][rt][lane];
#pragma unroll
                for (int mm = 0; mm < DV; ++mm) O[rt][mm] += fl.O[wr][rt * DV + mm][lane];
            }
        }
    }
    const bool owner = (a.WS == 1 || ws == 0) && rg < a.RG;

#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int rho = (rg * RT + rt) * 16 + c;
        if (!owner || rho >= a.Rp) continue;
        if (a.SB == 1 && !a.defer) {
            finish_row_lanes<D, OutT>(a, out_row(p, rho, a.Hkv, a.G, a.Tq, a.Hq), g, m[rt], l[rt], O[rt]);
        } else {
            const size_t row = (size_t)(p * a.SB + sb) * a.Rp + rho;
            if (g == 0) a.part_ml[row] = make_float2(m[rt], l[rt]);
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

template <int D, int RT, int SUB, typename OutT>
__device__ __forceinline__ void attn_partial_body(const AttnParams &a, int blk_id) {
    __shared__ AttnFoldLds<D, RT> fl;
    attn_partial_body_lds<D, RT, SUB, OutT>(a, blk_id, fl);
}

// Problem set of block b of a two-set grid and the block's index within it.
__device__ __forceinline__ int group_set(const AttnGroup &gr, int b) { return b >= gr.nb0 ? 1 : 0; }

}  // namespace nectar
