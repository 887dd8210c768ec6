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
    // the block's query rows (16 RT rows, same swizzle) where two waves share a
    // slot: staged once instead of loaded by every slot's waves
    static constexpr int QROWS = (D == 128 && dec_wps(D, RT) > 1) ? 16 * RT : 1;
    struct {
        u32x4 tiles[SL][NT * 2 * 32 * (D / 8)];
        u32x4 q[QROWS * (D / 8)];
    } st;
    DecFold<D, RT, SL> fold;
};

// Copy rows u0 .. u0 + 31 (clamped to umax) of W into LDS rows 0..31 at dst:
// eight copies of four rows; the wave takes copies i0, i0 + 1, ..., i0 + n - 1.
__device__ __forceinline__ void stage_rows128(u32x4 *dst, const uint16_t *W, int u0, int umax, int lane, int i0 = 0,
                                              int n = 8) {
#pragma unroll
    for (int i = i0; i < i0 + n; ++i) {
        const int rr = 4 * i + (lane >> 4);
        const int piece = (lane & 15) ^ (rr & 15);
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
__device__ __forceinline__ void mlp_decode_body_lds(const MlpParams &a, int blk_id,
                                                    DecLds<D, RT, NT, dec_slots(D, RT)> &lds) {
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
    constexpr bool QLDS = D == 128 && WPS > 1;   // query rows staged in LDS (lds.st.q)
    u32x4 qv[RTW][KS];
    if constexpr (!QLDS) {
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
    }
    // the query operands from the staged rows (after the barrier that follows
    // every wave's wait for its own copies)
    auto q_from_lds = [&]() {
        if constexpr (QLDS) {
#pragma unroll
            for (int rt = 0; rt < RTW; ++rt) {
                const int r = (rt0 + rt) * 16 + c;
#pragma unroll
                for (int kt = 0; kt < KS; ++kt) qv[rt][kt] = lds.st.q[r * 16 + ((4 * kt + g) ^ (r & 15))];
            }
        }
    };
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
    u32x4 *buf = lds.st.tiles[w];
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
    if constexpr (D == 128 && WPS > 1) {
        // Two waves per slot share the copies (four of the eight per 32-row
        // table each).  Loads complete in the order issued.  Target slots load
        // their biases, then tile 0's copies, then tile 1's: once at most tile
        // 1's copies are pending, tile 0 has landed, and its products run while
        // tile 1 is still in flight.  Score slots issue their copies first and
        // their biases and read-out weights after (those are widened from bf16
        // as they arrive, which waits for everything issued before): at most CI
        // pending operations are then bias loads, every copy has landed.  A
        // block barrier per tile (every wave takes the same two, idle ones too)
        // makes the other wave's half of the copies visible.
        static_assert(NT == 2 && NS == 2, "two tiles per slot, one barrier each");
        constexpr int CI = 8 / WPS;
        constexpr int QC = 16 * RT / 4 / (SL * WPS);   // query-row copies per wave
        static_assert(QC * 4 * SL * WPS == 16 * RT, "query rows split evenly over the waves");
        // every wave first copies its share of the block's query rows
        stage_q128<RT>(lds.st.q, (const uint16_t *)a.q, a.Rp, a.G, a.Hq, h, rg, lane, v * QC, QC);
        asm volatile("" ::: "memory");       // ... ahead of every other load
        // each role runs its whole sequence in its own branch, so the
        // compiler's wait analysis sees straight-line code (a join before the
        // products would make it wait for every load).  Loads complete in
        // issue order: query rows, biases, tile 0's copies, tile 1's copies.
        if (tgt) {
            float tb[(NT + 1) / 2];
            tgt_bias(tb);
            asm volatile("" ::: "memory");   // the bias loads stay ahead of the copies
            tgt_copies(part * CI, CI);
            wait_vmcnt<2 * CI>();            // tile 1's copies of both tables may be pending
            stage_barrier();
            asm volatile("" ::: "memory");   // the LDS reads stay below
            q_from_lds();
            if (n > 0) tgt_tile(tb, 0);
            wait_vmcnt<0>();
            stage_barrier();
            asm volatile("" ::: "memory");
            if (n > 1) tgt_tile(tb, 1);
        } else if (scw) {
            float sbias[(NS + 1) / 2];
            uint16_t swsv[(NS + 1) / 2];
            sc_bias(sbias, swsv);
            asm volatile("" ::: "memory");
            sc_copies(part * CI, CI);
            wait_vmcnt<CI>();                // tile 1's copies may be pending
            stage_barrier();
            asm volatile("" ::: "memory");
            q_from_lds();
            if (n > 0) sc_tile(sbias, swsv, 0);
            wait_vmcnt<0>();
            stage_barrier();
            asm volatile("" ::: "memory");
            if (n > 1) sc_tile(sbias, swsv, 1);
        } else {
            wait_vmcnt<0>();
            stage_barrier();
            stage_barrier();
        }
    } else if constexpr (D == 128) {
        if (tgt) {
            float tb[(NT + 1) / 2];
            tgt_bias(tb);
            tgt_copies(0, 8);
            wait_vmcnt<0>();
            asm volatile("" ::: "memory");   // the copies landed: LDS reads stay below
#pragma unroll
            for (int k = 0; k < NT; ++k)
                if (k < n) tgt_tile(tb, k);
        } else if (scw) {
            float sbias[(NS + 1) / 2];
            uint16_t swsv[(NS + 1) / 2];
            sc_bias(sbias, swsv);
            sc_copies(0, 8);
            wait_vmcnt<0>();
            asm volatile("" ::: "memory");
#pragma unroll
            for (int k = 0; k < NS; ++k)
                if (k < n) sc_tile(sbias, swsv, k);
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

template <int D, int RT, int ACT, int NT>
__device__ __forceinline__ void mlp_decode_body(const MlpParams &a, int blk_id) {
    __shared__ DecLds<D, RT, NT, dec_slots(D, RT)> lds;
    mlp_decode_body_lds<D, RT, ACT, NT>(a, blk_id, lds);
}

}  // namespace nectar
