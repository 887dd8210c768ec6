// Device code of the decode-shape MLP module kernel (up to 64 query rows per
// KV head per wave), shared by the standalone module launch and the fused
// decode-step launch.
//
// At decode the module forward streams every weight of the module once
// (|theta| * 2 bytes per KV head) and does little arithmetic per byte, so the
// kernel is built around one memory round trip per wave:
//  * a wave is either a target wave (the 32-unit target tiles
//    [t0, t1): W1 and W2t rows) or a score wave (32-unit score tiles: Ws rows
//    and ws2); the host sizes both wave sets so every wave reads about the
//    same number of bytes (a target tile is 16 KB at d = 128, a score tile
//    8 KB, so score waves take up to twice as many tiles);
//  * a wave issues the loads of all its tiles (at most NT target or
//    dec_score_tiles(RT) score tiles, indices clamped to its range) before its
//    first product, in straight-line code;
//  * products as in the register-direct kernel: Z^T = W1_tile . Q^T on the
//    16x16x32 MFMA with the query rows as B columns, bias + activation on the
//    fp32 accumulators, the hidden tile rounded to bf16 and fed back as the B
//    operand of O^T += W2t_tile^T . H^T (W2t rows transposed inside the lane);
//    score hidden values stay fp32 and are dotted with ws2 on the VALU;
//  * a block has four tile slots; at d = 128 with up to 64 rows two waves share
//    a slot's tiles (staged in LDS) and take 32 rows each (eight waves, two per
//    SIMD); the slots fold through LDS (one barrier) and the block writes one
//    partial per row as whole rows (coalesced), or -- when one block covers
//    every tile -- the outputs with their biases.
#pragma once

#include "lds_common.hpp"
#include "mlp_body.hpp"

namespace nectar {

// GELU (erf form) evaluated without transcendentals in the decode kernels too:
// the degree-6 polynomial of gelu_erf_poly (|GELU error| <= 5.2e-5 |x|).
template <int ACT> __device__ __forceinline__ float act_dec(float x) {
    return ACT == 1 ? silu(x) : (ACT == 2 ? gelu_tanh(x) : gelu_erf_poly(x));
}

template <int D, int RT, int ACT>
__device__ __forceinline__ void dec_tgt_tile(const MTile<D> &T, int j0, int Ht, const u32x4 (&qv)[RT][D / 32],
                                             int g, f32x4 (&O)[RT][D / 16]) {
    constexpr int KS = D / 32, DV = D / 16;
    u32x4 vt[DV];
    transpose_w<D>(T, vt);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        f32x4 z0 = {T.bias[0], T.bias[1], T.bias[2], T.bias[3]};
        f32x4 z1 = {T.bias[4], T.bias[5], T.bias[6], T.bias[7]};
#pragma unroll
        for (int kt = 0; kt < KS; ++kt) {
            z0 = mfma16(T.w1[0][kt], qv[rt][kt], z0);
            z1 = mfma16(T.w1[1][kt], qv[rt][kt], z1);
        }
        float hv[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            hv[r] = act_dec<ACT>(z0[r]);
            hv[4 + r] = act_dec<ACT>(z1[r]);
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
__device__ __forceinline__ void dec_score_tile(const MTile<D> &T, int j0, int Hs, const u32x4 (&qv)[RT][D / 32],
                                               int g, float (&sc)[RT]) {
    constexpr int KS = D / 32;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        f32x4 z0 = {T.bias[0], T.bias[1], T.bias[2], T.bias[3]};
        f32x4 z1 = {T.bias[4], T.bias[5], T.bias[6], T.bias[7]};
#pragma unroll
        for (int kt = 0; kt < KS; ++kt) {
            z0 = mfma16(T.w1[0][kt], qv[rt][kt], z0);
            z1 = mfma16(T.w1[1][kt], qv[rt][kt], z1);
        }
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float y = act_dec<ACT>(j < 4 ? z0[j] : z1[j - 4]) * T.ws[j];
            if (j0 + hslot(g, j) >= Hs) y = 0.f;
            acc += y;
        }
        sc[rt] += acc;
    }
}

// LDS of the block fold: per wave, its rows' read-outs [16 RT][D + 4] (rows
// padded by four floats so the sixteen rows of one store land in different
// banks) and score sums [16 RT].
template <int D, int RT, int SL> struct DecFold {
    static constexpr int ROWS = 16 * RT, LD = D + 4;
    float O[SL][ROWS * LD];
    float s[SL][ROWS];
};

// d = 128: a wave's weight rows are copied HBM -> LDS (global_load_lds, whole
// 256-byte rows, four rows per copy) into its own region -- NT target tiles of
// [W1 rows | W2t rows] or up to 2 NT score tiles of Ws rows, 16 KB per target tile --
// with the sixteen 16-byte pieces of row r stored at piece ^ (r % 16), so the
// operand reads of sixteen rows fall in distinct banks.  The fold reuses the
// same LDS after a barrier.
template <int D, int RT, int NT, int SL> union DecLds {
    u32x4 tiles[SL][NT * 2 * 32 * (D / 8)];
    DecFold<D, RT, SL> fold;
};

// Swizzle of the W2t stages of the paired kernel, read by transposing operand
// reads: piece j of unit row r sits at j ^ pair_swizzle(r).  One 16-lane
// group's read touches rows 8G + 4h + 0..3 and two adjacent pieces (an even
// one and the next); bits 1-2 of the swizzle separate the four rows and bit 3
// the two groups that share a half-wave, so the sixteen 16-byte slots a
// half-wave reads fall on distinct banks (and any 16 lanes' eight slots on
// distinct banks of a 32-bank model).
__device__ __forceinline__ int pair_swizzle(int r) { return ((r & 3) << 1) | (((r >> 3) & 1) << 3); }

// LDS of the paired kernel (d = 128, 33..64 rows per KV head, 160 KB): per
// slot two tiles of [32 W1 rows | 32 W2t rows] (score slots: two tiles of 32
// Ws rows), the block's query rows (their region later holds the score sums),
// and the hidden values of one tile round of every slot, [slot][group of 8
// units][row][8 units] in bf16.
struct DecPairLds {
    u32x4 tiles[4][2 * 2 * 32 * 16];
    u32x4 q[64 * 16];
    u32x4 H[4 * 4 * 64];
};

// Copy rows u0 .. u0 + 31 (clamped to umax) of W into LDS rows 0..31 at dst:
// eight copies of four rows; the wave takes copies i0, i0 + 1, ..., i0 + n - 1.
// PSW: pieces at pair_swizzle positions instead of piece ^ (r % 16).
template <bool PSW = false>
__device__ __forceinline__ void stage_rows128(u32x4 *dst, const uint16_t *W, int u0, int umax, int lane, int i0 = 0,
                                              int n = 8) {
#pragma unroll
    for (int i = i0; i < i0 + n; ++i) {
        const int rr = 4 * i + (lane >> 4);
        const int piece = (lane & 15) ^ (PSW ? pair_swizzle(rr) : (rr & 15));
        const uint16_t *src = W + (size_t)min(u0 + rr, umax) * 128 + piece * 8;
        __builtin_amdgcn_global_load_lds((const void *)src, (lds_void *)(dst + 64 * i), 16, 0, 0);
    }
}

// Copy the query rows rg * 16 RT + 0 .. 16 RT - 1 of KV head h (clamped to the
// last row: rows past it feed only results that are never written) into LDS
// rows at dst, pieces swizzled as in stage_rows128; the wave takes copies
// i0 .. i0 + n - 1 of four rows each.
template <int RT>
__device__ __forceinline__ void stage_q128(u32x4 *dst, const uint16_t *q, int Rp, int G, int Hq, int h, int rg,
                                           int lane, int i0, int n) {
#pragma unroll
    for (int i = i0; i < i0 + n; ++i) {
        const int rr = 4 * i + (lane >> 4);
        const int piece = (lane & 15) ^ (rr & 15);
        const int rho = min(rg * 16 * RT + rr, Rp - 1);
        const int t = rho / G, gg = rho - t * G;
        const uint16_t *src = q + ((size_t)t * Hq + h * G + gg) * 128 + piece * 8;
        __builtin_amdgcn_global_load_lds((const void *)src, (lds_void *)(dst + 64 * i), 16, 0, 0);
    }
}

// MFMA operands of one tile from its LDS rows (the layout of load_rows /
// load_tgt); d = 128 only (the d = 64 kernels load tiles into registers).
template <int D> __device__ __forceinline__ void lds_rows128(MTile<D> &T, const u32x4 *rows, int g, int c) {
    if constexpr (D == 128) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                const int r = 16 * hh + c;
                T.w1[hh][kt] = rows[r * 16 + ((4 * kt + g) ^ (r & 15))];
            }
    }
}
template <int D> __device__ __forceinline__ void lds_w2_128(MTile<D> &T, const u32x4 *rows, int g, int c) {
    if constexpr (D == 128) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = hslot(g, j);
            T.w2[j] = rows[r * 16 + (c ^ (r & 15))];
        }
    }
}

// Block blk_id of the grid Hkv x RG x SB: blocks of SL = dec_slots(D, RT) tile
// slots of WPS = dec_wps(D, RT) waves each (wave v takes slot v % SL and row
// tiles (v / SL) * RT / WPS ...).  Slot w of block sb of (KV head h, row group
// rg) is slot i = SL sb + w of that group: target slot i < nwt, score slot
// i - nwt < nws, idle otherwise.
// lds is the block's LDS (a kernel that also runs other bodies shares it).
template <int D, int RT, int ACT, int NT>
__device__ __forceinline__ void mlp_decode_slots(const MlpParams &a, int blk_id,
                                                 DecLds<D, RT, NT, dec_slots(D, RT)> &lds) {
    static_assert(dec_wps(D, RT) == 1, "one wave per slot");
    constexpr int KS = D / 32, DV = D / 16;
    constexpr int WPS = dec_wps(D, RT), SL = dec_slots(D, RT), RTW = RT / WPS;   // waves per slot, slots, row tiles per wave
    constexpr int NS = dec_score_tiles(RT);                 // score tiles per score slot
    DecFold<D, RT, SL> &fold = lds.fold;

    const int v = threadIdx.x >> 6;
    const int w = v % SL, part = v / SL;      // tile slot, row part of this wave
    int blk = blk_id;
    const int sb = blk % a.SB;
    blk /= a.SB;
    const int rg = blk % a.RG;
    const int h = blk / a.RG;
    const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
    const int wi = SL * sb + w;
    const int rt0 = part * RTW;                // first row tile of this wave within the block's RT

    f32x4 O[RTW][DV];
    float sc[RTW];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
        sc[rt] = 0.f;
#pragma unroll
        for (int mm = 0; mm < DV; ++mm) O[rt][mm] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const bool tgt = wi < a.nwt, scw = !tgt && wi < a.nwt + a.nws;
    u32x4 qv[RTW][KS];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
        const int rho = (rg * RT + rt0 + rt) * 16 + c;
        if ((tgt || scw) && rho < a.Rp) {
            const int t = rho / a.G, gg = rho - t * a.G;
            const uint16_t *qp = (const uint16_t *)a.q + ((size_t)t * a.Hq + h * a.G + gg) * D;
#pragma unroll
            for (int kt = 0; kt < KS; ++kt) qv[rt][kt] = *(const u32x4 *)(qp + (4 * kt + g) * 8);
        } else {
#pragma unroll
            for (int kt = 0; kt < KS; ++kt) qv[rt][kt] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    // this slot's tile range
    const int Tt = (a.Ht + 31) / 32, Ts = (a.Hs + 31) / 32;
    const int si = wi - a.nwt;
    const int t0 = tgt ? (int)((long)wi * Tt / a.nwt) : (scw ? (int)((long)si * Ts / a.nws) : 0);
    const int n = tgt ? (int)((long)(wi + 1) * Tt / a.nwt) - t0 : (scw ? (int)((long)(si + 1) * Ts / a.nws) - t0 : 0);
    const uint16_t *W1 = (const uint16_t *)a.W1 + (size_t)h * a.Ht * D;
    const uint16_t *W2t = (const uint16_t *)a.W2t + (size_t)h * a.Ht * D;
    const float *b1 = a.b1 + (size_t)h * a.Ht;
    const uint16_t *Ws = (const uint16_t *)a.Ws + (size_t)h * a.Hs * D;
    const uint16_t *ws2 = (const uint16_t *)a.ws2 + (size_t)h * a.Hs;
    const float *bs = a.bs + (size_t)h * a.Hs;

    // d = 128: the slot's weight rows are staged in LDS (lds.tiles[w]), every
    // copy and bias load first, then one wait before the first product.
    u32x4 *buf = lds.tiles[w];
    // Biases (and score read-out weights): one load per lane and pair of
    // tiles -- lane l holds unit l % 32 of tile 2 i + l / 32 -- handed to the
    // lanes that use them (hidden slots hslot(g, j)) when the tile's products
    // start, instead of eight loads per lane and tile.
    auto tile_unit = [&](int k) { return 32 * (t0 + max(min(k, n - 1), 0)); };
    auto bias_lane = [&](int i) { return tile_unit(2 * i + (lane >> 5)) + (lane & 31); };
    auto from_lane = [&](float v, int k, int j) { return __shfl(v, 32 * (k & 1) + hslot(g, j), 64); };
    auto tgt_bias = [&](auto &bias) {
#pragma unroll
        for (int i = 0; i < (NT + 1) / 2; ++i) bias[i] = b1[min(bias_lane(i), a.Ht - 1)];
    };
    auto tgt_copies = [&](int i0, int ni) {
#pragma unroll
        for (int k = 0; k < NT; ++k) {
            const int u0 = 32 * (t0 + max(min(k, n - 1), 0));
            stage_rows128(buf + k * 1024, W1, u0, a.Ht - 1, lane, i0, ni);
            stage_rows128(buf + k * 1024 + 512, W2t, u0, a.Ht - 1, lane, i0, ni);
        }
    };
    auto tgt_tile = [&](const auto &bias, int k) {
        MTile<D> T;
        lds_rows128(T, buf + k * 1024, g, c);
        lds_w2_128(T, buf + k * 1024 + 512, g, c);
#pragma unroll
        for (int j = 0; j < 8; ++j) T.bias[j] = from_lane(bias[k >> 1], k, j);
        dec_tgt_tile<D, RTW, ACT>(T, 32 * (t0 + k), a.Ht, qv, g, O);
    };
    auto sc_bias = [&](auto &bias, auto &wsv) {
#pragma unroll
        for (int i = 0; i < (NS + 1) / 2; ++i) {
            const int u = min(bias_lane(i), a.Hs - 1);
            bias[i] = bs[u];
            wsv[i] = ws2[u];                   // bf16 bits, widened at use
        }
    };
    auto sc_copies = [&](int i0, int ni) {
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            const int u0 = 32 * (t0 + max(min(k, n - 1), 0));
            stage_rows128(buf + k * 512, Ws, u0, a.Hs - 1, lane, i0, ni);
        }
    };
    auto sc_tile = [&](const auto &bias, const auto &wsv, int k) {
        MTile<D> T;
        lds_rows128(T, buf + k * 512, g, c);
        const float wsk = __uint_as_float((uint32_t)wsv[k >> 1] << 16);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            T.bias[j] = from_lane(bias[k >> 1], k, j);
            T.ws[j] = from_lane(wsk, k, j);
        }
        dec_score_tile<D, RTW, ACT>(T, 32 * (t0 + k), a.Hs, qv, g, sc);
    };
    if constexpr (D == 128) {
        // Loads complete in issue order (biases, then the tiles' copies tile by
        // tile): each tile's products start once its own copies have landed,
        // while the later tiles' are still in flight.  The wave reads only the
        // stage it copied itself, so no barrier is needed.
        static_assert(NT == 2 && (NS == 2 || NS == 4), "tile counts of the staged waits");
        if (tgt) {
            float tb[(NT + 1) / 2];
            tgt_bias(tb);
            asm volatile("" ::: "memory");   // the bias loads stay ahead of the copies
            tgt_copies(0, 8);
            wait_vmcnt<16>();                // tile 1's 16 copies may be pending
            asm volatile("" ::: "memory");   // LDS reads stay below
            if (n > 0) tgt_tile(tb, 0);
            wait_vmcnt<0>();
            asm volatile("" ::: "memory");
            if (n > 1) tgt_tile(tb, 1);
        } else if (scw) {
            float sbias[(NS + 1) / 2];
            uint16_t swsv[(NS + 1) / 2];
            sc_bias(sbias, swsv);
            asm volatile("" ::: "memory");
            sc_copies(0, 8);
            wait_vmcnt<8 * (NS - 1)>();      // tiles 1.. may be pending
            asm volatile("" ::: "memory");
            if (n > 0) sc_tile(sbias, swsv, 0);
            if constexpr (NS == 4) {
                wait_vmcnt<16>();
                asm volatile("" ::: "memory");
                if (n > 1) sc_tile(sbias, swsv, 1);
                wait_vmcnt<8>();
                asm volatile("" ::: "memory");
                if (n > 2) sc_tile(sbias, swsv, 2);
                wait_vmcnt<0>();
                asm volatile("" ::: "memory");
                if (n > 3) sc_tile(sbias, swsv, 3);
            } else {
                wait_vmcnt<0>();
                asm volatile("" ::: "memory");
                if (n > 1) sc_tile(sbias, swsv, 1);
            }
        }
    } else {
        if (tgt) {
            MTile<D> T[NT];
#pragma unroll
            for (int k = 0; k < NT; ++k)
                load_tgt<D>(T[k], W1, W2t, b1, 32 * (t0 + max(min(k, n - 1), 0)), a.Ht - 1, g, c);
#pragma unroll
            for (int k = 0; k < NT; ++k)
                if (k < n) dec_tgt_tile<D, RTW, ACT>(T[k], 32 * (t0 + k), a.Ht, qv, g, O);
        } else if (scw) {
            MTile<D> T[NS];
#pragma unroll
            for (int k = 0; k < NS; ++k)
                load_score<D>(T[k], Ws, ws2, bs, 32 * (t0 + max(min(k, n - 1), 0)), a.Hs - 1, g, c);
#pragma unroll
            for (int k = 0; k < NS; ++k)
                if (k < n) dec_score_tile<D, RTW, ACT>(T[k], 32 * (t0 + k), a.Hs, qv, g, sc);
        }
    }
    if (scw) {
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) sc[rt] = group4_sum(sc[rt]);
    }

    // fold the slots: every wave stores its rows (in the LDS the tiles
    // used, once every wave is past them), one barrier, then the block's
    // threads sum the slots and write whole rows
    constexpr int LD = DecFold<D, RT, SL>::LD, ROWS = DecFold<D, RT, SL>::ROWS;
    if constexpr (D == 128) stage_barrier();
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
        float *op = fold.O[w] + ((rt0 + rt) * 16 + c) * LD;
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int m4 = 0; m4 < DV; m4 += 4)
                *(f32x4 *)(op + DV * (4 * g + r) + m4) = f32x4{O[rt][m4][r], O[rt][m4 + 1][r], O[rt][m4 + 2][r],
                                                              O[rt][m4 + 3][r]};
        if (g == 0) fold.s[w][(rt0 + rt) * 16 + c] = sc[rt];
    }
    __syncthreads();
    const bool direct = a.SB == 1 && !a.defer;
    constexpr int CPR = D / 4;                       // float4 columns per row
    constexpr int RPI = dec_threads(D, RT) / CPR;   // rows per pass of the block
    const int col = (threadIdx.x % CPR) * 4;
#pragma unroll
    for (int r0 = 0; r0 < ROWS; r0 += RPI) {
        const int rr = r0 + (int)threadIdx.x / CPR;
        const int rho = rg * ROWS + rr;
        if (rr >= ROWS || rho >= a.Rp) continue;
        f32x4 v4 = *(const f32x4 *)(fold.O[0] + rr * LD + col);
#pragma unroll
        for (int k = 1; k < SL; ++k) v4 += *(const f32x4 *)(fold.O[k] + rr * LD + col);
        const bool lead = col == 0;
        float s = 0.f;
        if (lead) {
            if constexpr (SL == 4) s = (fold.s[0][rr] + fold.s[1][rr]) + (fold.s[2][rr] + fold.s[3][rr]);
            else {
#pragma unroll
                for (int k = 0; k < SL; ++k) s += fold.s[k][rr];
            }
        }
        if (direct) {
            const int t = rho / a.G, gg = rho - t * a.G;
            const size_t o = (size_t)t * a.Hq + h * a.G + gg;
            *(f32x4 *)(a.A_out + o * D + col) = v4 + *(const f32x4 *)(a.b2 + (size_t)h * D + col);
            if (lead) a.a_out[o] = a.bs2[h] + s;
        } else {
            const size_t row = (size_t)(h * a.SB + sb) * a.Rp + rho;
            *(f32x4 *)(a.part_O + row * D + col) = v4;
            if (lead) a.part_s[row] = s;
        }
    }
}

// d = 128 with 33..64 rows per KV head: a block of four slots of two waves.
// Wave v = 4 part + w stages slot w's weights (with the other wave of the
// slot: four of the eight copies per 32-row table each) and computes, for the
// rows 32 part .. 32 part + 31 of the block's 64,
//   phase 1 (its slot's tile k): Z^T = W1 . Q^T + b1 on the 16x16x32 MFMA,
//     H = act(Z) rounded to bf16 into LDS -- or, in a score slot, the score
//     terms ws2 . act(Ws . q + bs) summed in fp32;
//   phase 2 (every target slot's tile k): O^T += W2t^T . H^T for the output
//     dims 32 w .. 32 w + 31, the W2t operands from the unit-major stage by
//     transposing reads, the hidden values from LDS,
// so each wave ends with its own 32 dims x 32 rows of the block's read-out
// sum, written straight from its accumulators: no fold of slot partials.
// Two tile rounds, four block barriers: tile 0 landed; round 0's hidden
// values written; tile 1 landed (round 0's reads done); round 1's hidden
// values and the score sums written.  Loads complete in issue order: query
// rows, biases, tile 0's copies, tile 1's copies, so round 0 runs while tile
// 1 is in flight.  A target slot with one tile writes zero hidden values in
// round 1 (its second stage holds the first tile's rows again: finite).
template <int ACT>
__device__ __forceinline__ void mlp_decode_pair128(const MlpParams &a, int blk_id, DecPairLds &lds) {
    constexpr int D = 128, SL = 4, NT = 2, CI = 4;
    // the planner's slots per block (dec_slots) must be the four this kernel's
    // dim split over its eight waves assumes
    static_assert(dec_slots(D, 4) == SL && dec_wps(D, 4) == 2, "four paired slots per block");
    const int v = threadIdx.x >> 6;
    const int w = v & 3, part = v >> 2;
    int blk = blk_id;
    const int sb = blk % a.SB;
    blk /= a.SB;
    const int rg = blk % a.RG;
    const int h = blk / a.RG;
    const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
    const int wi = SL * sb + w;
    const bool tgt = wi < a.nwt, scw = !tgt && wi < a.nwt + a.nws;
    const int nto = min(max(a.nwt - SL * sb, 0), SL);   // target slots of the block: the first nto
    const int Tt = (a.Ht + 31) / 32, Ts = (a.Hs + 31) / 32;
    const int si = wi - a.nwt;
    const int t0 = tgt ? (int)((long)wi * Tt / a.nwt) : (scw ? (int)((long)si * Ts / a.nws) : 0);
    const int n = tgt ? (int)((long)(wi + 1) * Tt / a.nwt) - t0 : (scw ? (int)((long)(si + 1) * Ts / a.nws) - t0 : 0);
    const uint16_t *W1 = (const uint16_t *)a.W1 + (size_t)h * a.Ht * D;
    const uint16_t *W2t = (const uint16_t *)a.W2t + (size_t)h * a.Ht * D;
    const float *b1 = a.b1 + (size_t)h * a.Ht;
    const uint16_t *Ws = (const uint16_t *)a.Ws + (size_t)h * a.Hs * D;
    const uint16_t *ws2 = (const uint16_t *)a.ws2 + (size_t)h * a.Hs;
    const float *bs = a.bs + (size_t)h * a.Hs;
    u32x4 *buf = lds.tiles[w];
    float *fs = (float *)lds.q;   // score sums [slot][64 rows], once the query rows are in registers

    auto tile_unit = [&](int k) { return 32 * (t0 + max(min(k, n - 1), 0)); };
    // biases: lane l loads unit l % 32 of tile l / 32; the lanes that use a
    // unit (hidden slots hslot(g, j)) take it by a wave shuffle
    const int ulane = tile_unit(lane >> 5) + (lane & 31);
    auto from_lane = [&](float x, int k, int j) { return __shfl(x, 32 * (k & 1) + hslot(g, j), 64); };

    u32x4 qv[2][4];
    auto q_from_lds = [&]() {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int r = 32 * part + 16 * rt + c;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) qv[rt][kt] = lds.q[r * 16 + ((4 * kt + g) ^ (r & 15))];
        }
    };
    // Z^T of this wave's rows for tile k of the slot (rows of W1 or Ws at rows)
    auto zt = [&](const u32x4 *rows, const float (&bias)[8], int rt, f32x4 &z0, f32x4 &z1) {
        z0 = f32x4{bias[0], bias[1], bias[2], bias[3]};
        z1 = f32x4{bias[4], bias[5], bias[6], bias[7]};
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            const int r0 = c, r1 = 16 + c;
            z0 = mfma16(rows[r0 * 16 + ((4 * kt + g) ^ (r0 & 15))], qv[rt][kt], z0);
            z1 = mfma16(rows[r1 * 16 + ((4 * kt + g) ^ (r1 & 15))], qv[rt][kt], z1);
        }
    };
    // phase 1 of a target slot: H of tile k (zero past the slot's tiles)
    auto tgt_phase1 = [&](float bv, int k) {
        uint32_t hw[2][4];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) hw[rt][i] = 0u;
        if (k < n) {
            float bias[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) bias[j] = from_lane(bv, k, j);
            const int j0 = 32 * (t0 + k);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                f32x4 z0, z1;
                zt(buf + k * 1024, bias, rt, z0, z1);
                float hv[8];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    hv[r] = act_dec<ACT>(z0[r]);
                    hv[4 + r] = act_dec<ACT>(z1[r]);
                }
                if (j0 + 32 > a.Ht) {
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        if (j0 + hslot(g, j) >= a.Ht) hv[j] = 0.f;
                }
                hw[rt][0] = pack_bf16(hv[0], hv[1]);
                hw[rt][1] = pack_bf16(hv[2], hv[3]);
                hw[rt][2] = pack_bf16(hv[4], hv[5]);
                hw[rt][3] = pack_bf16(hv[6], hv[7]);
            }
        }
        // lane (g, c) holds units 16 hh + 4 g .. + 3 of row 32 part + 16 rt + c:
        // half (g & 1) of the 8-unit group 2 hh + g / 2
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                u32x4 *e = lds.H + (w * 4 + 2 * hh + (g >> 1)) * 64 + 32 * part + 16 * rt + c;
                *(u32x2 *)((char *)e + 8 * (g & 1)) = u32x2{hw[rt][2 * hh], hw[rt][2 * hh + 1]};
            }
    };
    // phase 1 of a score slot: the score terms of tile k
    float sc[2] = {0.f, 0.f};
    auto sc_phase1 = [&](float bv, float wsv, int k) {
        if (k >= n) return;                  // uniform
        float bias[8], wsj[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            bias[j] = from_lane(bv, k, j);
            wsj[j] = from_lane(wsv, k, j);
        }
        const int j0 = 32 * (t0 + k);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            f32x4 z0, z1;
            zt(buf + k * 512, bias, rt, z0, z1);
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float y = act_dec<ACT>(j < 4 ? z0[j] : z1[j - 4]) * wsj[j];
                if (j0 + hslot(g, j) >= a.Hs) y = 0.f;
                acc += y;
            }
            sc[rt] += acc;
        }
    };
    // phase 2: O^T (dims 32 w + 16 mb + ., rows 32 part + 16 nt + .) over the
    // target slots' tile k.  A operand of lane (G, x): dim 32 w + 16 mb + x and
    // units 8 G .. 8 G + 7, by two transposing reads of four units each (lane
    // x = a + 4 j names the 8 bytes of unit row 8 G + 4 i + j at dims
    // 32 w + 16 mb + 4 a .. + 3); B operand: units 8 G .. 8 G + 7 of row x.
    f32x4 acc[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mb][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto phase2 = [&](int k) {
#pragma unroll
        for (int s2 = 0; s2 < SL; ++s2) {
            if (s2 >= nto) break;             // uniform
            const u32x4 *wt = lds.tiles[s2] + k * 1024 + 512;
            u32x4 A[2], B[2];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                u32x2 half[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int row = 8 * g + 4 * i + (c >> 2);
                    const int p = 4 * w + 2 * mb + ((c & 3) >> 1);
                    half[i] = lds_read_tr16(wt, (uint32_t)(row * 256 + ((p ^ pair_swizzle(row)) * 16) + (c & 1) * 8));
                }
                A[mb] = u32x4{half[0][0], half[0][1], half[1][0], half[1][1]};
            }
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) B[nt] = lds.H[(s2 * 4 + g) * 64 + 32 * part + 16 * nt + c];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) acc[mb][nt] = mfma16(A[mb], B[nt], acc[mb][nt]);
        }
    };
    auto store_sc = [&]() {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const float t = scw ? group4_sum(sc[rt]) : 0.f;
            if (g == 0) fs[w * 64 + 32 * part + 16 * rt + c] = t;
        }
    };

    // every wave first copies its share of the block's query rows
    stage_q128<4>(lds.q, (const uint16_t *)a.q, a.Rp, a.G, a.Hq, h, rg, lane, 2 * v, 2);
    asm volatile("" ::: "memory");   // ... ahead of every other load
    // each role runs its whole sequence in its own branch, so the compiler's
    // wait analysis sees straight-line code (a join before the products
    // would make it wait for every load)
    if (tgt) {
        const float bv = b1[min(ulane, a.Ht - 1)];
        asm volatile("" ::: "memory");
#pragma unroll
        for (int k = 0; k < NT; ++k) {
            stage_rows128(buf + k * 1024, W1, tile_unit(k), a.Ht - 1, lane, part * CI, CI);
            stage_rows128<true>(buf + k * 1024 + 512, W2t, tile_unit(k), a.Ht - 1, lane, part * CI, CI);
        }
        wait_vmcnt<2 * CI>();            // tile 1's copies may be pending
        stage_barrier();
        asm volatile("" ::: "memory");
        q_from_lds();
        tgt_phase1(bv, 0);
        lds_barrier();
        phase2(0);
        wait_vmcnt<0>();
        stage_barrier();
        asm volatile("" ::: "memory");
        tgt_phase1(bv, 1);
        store_sc();
        lds_barrier();
        phase2(1);
    } else if (scw) {
        const float bv = bs[min(ulane, a.Hs - 1)];
        const uint16_t wv = ws2[min(ulane, a.Hs - 1)];
        asm volatile("" ::: "memory");
#pragma unroll
        for (int k = 0; k < NT; ++k) stage_rows128(buf + k * 512, Ws, tile_unit(k), a.Hs - 1, lane, part * CI, CI);
        wait_vmcnt<CI>();                // tile 1's copies may be pending
        stage_barrier();
        asm volatile("" ::: "memory");
        q_from_lds();
        const float wsv = __uint_as_float((uint32_t)wv << 16);
        sc_phase1(bv, wsv, 0);
        lds_barrier();
        phase2(0);
        wait_vmcnt<0>();
        stage_barrier();
        asm volatile("" ::: "memory");
        sc_phase1(bv, wsv, 1);
        store_sc();
        lds_barrier();
        phase2(1);
    } else {
        wait_vmcnt<0>();
        stage_barrier();
        lds_barrier();
        phase2(0);
        stage_barrier();
        store_sc();
        lds_barrier();
        phase2(1);
    }

    // the block's read-out sums (each wave its dims and rows) and score sums
    const bool direct = a.SB == 1 && !a.defer;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int r = 32 * part + 16 * nt + c;
        const int rho = rg * 64 + r;
        if (rho >= a.Rp) continue;
        const int t = rho / a.G, gg = rho - t * a.G;
        const size_t o = (size_t)t * a.Hq + h * a.G + gg;
        const size_t row = (size_t)(h * a.SB + sb) * a.Rp + rho;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int dc = 32 * w + 16 * mb + 4 * g;
            if (direct) *(f32x4 *)(a.A_out + o * D + dc) = acc[mb][nt] + *(const f32x4 *)(a.b2 + (size_t)h * D + dc);
            else *(f32x4 *)(a.part_O + row * D + dc) = acc[mb][nt];
        }
        if (w == 0 && g == 0) {
            const float ssum = (fs[r] + fs[64 + r]) + (fs[128 + r] + fs[192 + r]);
            if (direct) a.a_out[o] = a.bs2[h] + ssum;
            else a.part_s[row] = ssum;
        }
    }
}

// The LDS a decode block of (D, RT) uses.
template <int D, int RT, int NT>
using DecLdsOf = typename std::conditional<(D == 128 && dec_wps(D, RT) > 1), DecPairLds,
                                           DecLds<D, RT, NT, dec_slots(D, RT)>>::type;

template <int D, int RT, int ACT, int NT>
__device__ __forceinline__ void mlp_decode_body_lds(const MlpParams &a, int blk_id, DecLdsOf<D, RT, NT> &lds) {
    if constexpr (D == 128 && dec_wps(D, RT) > 1) mlp_decode_pair128<ACT>(a, blk_id, lds);
    else mlp_decode_slots<D, RT, ACT, NT>(a, blk_id, lds);
}

template <int D, int RT, int ACT, int NT>
__device__ __forceinline__ void mlp_decode_body(const MlpParams &a, int blk_id) {
    __shared__ DecLdsOf<D, RT, NT> lds;
    mlp_decode_body_lds<D, RT, ACT, NT>(a, blk_id, lds);
}

}  // namespace nectar
