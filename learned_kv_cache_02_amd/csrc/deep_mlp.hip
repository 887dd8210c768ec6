// Deep MLP module with input re-injection, Eq. (3.6) of the Nectar notes
// (section 2.4): every layer of a network reads the query again beside the
// previous layer's state, h_{k+1} = act(V_k q + U_k h_k + b_k), and each head
// ends in a linear read-out of its last state.  A layer is one contraction
// over the concatenated input [q | h_k] for all rows of all KV heads; layers
// run as consecutive launches (each needs the whole previous state), the score
// and target heads of one depth side by side in one launch.
//
// bf16, few rows (decode): a block owns 16 rows x 16 outputs of one KV head.
// Its four waves split the contraction into four contiguous ranges of 32-wide
// steps; lane (g, c) loads 16 bytes of weight row n0 + c and of input row
// rho0 + c at offset 8 g of each step (the 16x16x32 MFMA operand layout, both
// operands straight from their row-major arrays), the four partial tiles are
// folded in LDS in a fixed order, and wave 0 adds the bias, applies the
// activation and stores the tile: hidden states as bf16 (round to nearest
// even), read-outs as fp32.
// bf16, many rows (batched decode, prefill): a block of eight waves owns 256
// rows x 128 outputs; 32-wide contraction stages of both tiles stream through
// a three-stage LDS ring (72 KB, two blocks per CU, so one block's activations
// overlap the other's products) by direct HBM -> LDS copies issued two ahead,
// each stored slice-major ([16-wide slice][row][two 16-byte halves], the halves
// swapped on every other group of 8 rows) so that the 32x32x16 MFMA operand
// reads of 16 consecutive lanes touch distinct banks.  Wave (wr, wc) computes
// 64 rows x 64 outputs as 2 x 2 tiles; blocks of one row group are dispatched
// to one XCD (its L2 then serves the input tile to every output tile).
// fp32: one thread per output, a plain sequential dot product.
#include "attn_common.hpp"
#include "lds_common.hpp"

namespace nectar {

namespace {

// The layer a block belongs to, as a reference into the kernel arguments (a
// copy of a runtime-selected struct would be placed in scratch memory).
__device__ __forceinline__ const DeepLayer &pick_layer(const DeepParams &a, long &blk) {
    const bool second = a.nl > 1 && blk >= a.L0.blocks;
    if (second) blk -= a.L0.blocks;
    return second ? a.L1 : a.L0;
}

}  // namespace

template <int D>
__global__ __launch_bounds__(256) void deep_layer_mfma(DeepParams a) {
    long blk = blockIdx.x;
    const DeepLayer &L = pick_layer(a, blk);
    const int NT = (L.N + 15) / 16, RT = (a.Rp + 15) / 16;
    // output tiles fastest: blocks sharing a weight tile are NT ids apart
    const int nt = (int)(blk % NT);
    const long rest = blk / NT;
    const int rt = (int)(rest % RT), p = (int)(rest / RT);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
    const int n0 = nt * 16, rho0 = rt * 16;
    const int nl = min(n0 + c, L.N - 1), rl = min(rho0 + c, a.Rp - 1);   // loads stay in bounds
    const int Dq = L.Wq ? D : 0;
    const int steps = (Dq + L.Kh) / 32;
    const int s0 = wave * steps / 4, s1 = (wave + 1) * steps / 4;

    const uint16_t *wq = (const uint16_t *)L.Wq + ((size_t)p * L.N + nl) * D + 8 * g;
    const uint16_t *xq = (const uint16_t *)a.q + out_row(p, rl, a.Hkv, a.G, 0, a.Hq) * D + 8 * g;
    const uint16_t *wh = (const uint16_t *)L.Wh + ((size_t)p * L.N + nl) * L.Kh + 8 * g;
    const uint16_t *xh = (const uint16_t *)L.X + ((size_t)p * a.Rp + rl) * L.Kh + 8 * g;

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = s0; s < s1; s += 4) {
        u32x4 wa[4], xb[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int k = (s + u) * 32;
            wa[u] = u32x4{0u, 0u, 0u, 0u};
            xb[u] = u32x4{0u, 0u, 0u, 0u};
            if (s + u < s1) {
                if (k < Dq) {
                    wa[u] = *(const u32x4 *)(wq + k);
                    xb[u] = *(const u32x4 *)(xq + k);
                } else {
                    wa[u] = *(const u32x4 *)(wh + (k - Dq));
                    xb[u] = *(const u32x4 *)(xh + (k - Dq));
                }
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) acc = mfma16(wa[u], xb[u], acc);
    }

    __shared__ f32x4 red[3][64];
    if (wave > 0) red[wave - 1][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    acc += red[0][lane];
    acc += red[1][lane];
    acc += red[2][lane];

    // lane (g, c): outputs n0 + 4 g + r of row rho0 + c
    const int rho = rho0 + c;
    if (rho >= a.Rp) return;
    float y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int n = n0 + 4 * g + r;
        y[r] = acc[r] + (n < L.N ? L.b[(size_t)p * L.N + n] : 0.f);
        if (L.act >= 0) y[r] = activation(L.act, y[r]);
    }
    if (L.Y) {
        // hidden widths are multiples of 32: the four outputs are in range
        uint16_t *dst = (uint16_t *)L.Y + ((size_t)p * a.Rp + rho) * L.N + n0 + 4 * g;
        *(u32x2 *)dst = u32x2{pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3])};
    } else {
        const size_t o = out_row(p, rho, a.Hkv, a.G, 0, a.Hq);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int n = n0 + 4 * g + r;
            if (n < L.N) L.Yf[o * L.N + n] = y[r];
        }
    }
}

namespace {

constexpr int kBM = 256, kBN = 128, kBK = 32, kSl = kBK / 16, kLdsWaves = 8, kXcd = 8;

struct DeepStage {
    u32x4 x[kSl * kBM * 2];   // [slice][row][half]: input rows (query or state)
    u32x4 w[kSl * kBN * 2];   // [slice][row][half]: weight rows (outputs)
};
// the bf16 epilogue stages three waves' 32 x 64 tiles (8 KB each) in one stage buffer
static_assert(sizeof(DeepStage) >= 3 * 8192, "epilogue staging");

}  // namespace

template <int D, int ACT>
__global__ __launch_bounds__(64 * kLdsWaves, 4) void deep_layer_lds32(DeepParams a) {
    __shared__ DeepStage st_a, st_b, st_c;

    long blk = blockIdx.x;
    const DeepLayer &L = pick_layer(a, blk);
    // blk = 8 k + xcd; k = g * NT + nt; row group = 8 g + xcd
    const int NT = (L.N + kBN - 1) / kBN;
    const int xcd = (int)(blk % kXcd);
    const long k = blk / kXcd;
    const int nt = (int)(k % NT);
    const int rgi = (int)(k / NT) * kXcd + xcd;
    const int nrb = (a.Rp + kBM - 1) / kBM;
    if (rgi >= a.Hkv * nrb) return;
    const int p = rgi / nrb, rho0 = (rgi - p * nrb) * kBM, n0 = nt * kBN;

    const int t = threadIdx.x, w = t >> 6, lane = t & 63;
    const int wr = w & 3, wc = w >> 2;
    const int Dq = L.Wq ? D : 0, K = Dq + L.Kh;
    const int nst = (K + kBK - 1) / kBK;

    // Copies (three per wave per stage): wave w fills slice w / 4 of every
    // stage -- input rows (2 (w & 3) + jj) * 32 + lane / 2 (jj < 2) and weight
    // rows (w & 3) * 32 + lane / 2, the 16-byte half (lane & 1) ^ ((lane >> 4) & 1)
    // of each row's 32 bytes in that slice.
    const int cs = w >> 2, half = (lane & 1) ^ ((lane >> 4) & 1);
    // per-lane source offsets of the query part and of the state part (plain
    // scalars: a runtime choice between two arrays would live in scratch)
    const int rA = min(rho0 + (2 * (w & 3)) * 32 + (lane >> 1), a.Rp - 1);
    const int rB = min(rho0 + (2 * (w & 3) + 1) * 32 + (lane >> 1), a.Rp - 1);
    const int nW = min(n0 + (w & 3) * 32 + (lane >> 1), L.N - 1);
    const size_t lo = 16 * cs + 8 * half;
    const uint16_t *xqA = (const uint16_t *)a.q + out_row(p, rA, a.Hkv, a.G, 0, a.Hq) * D + lo;
    const uint16_t *xqB = (const uint16_t *)a.q + out_row(p, rB, a.Hkv, a.G, 0, a.Hq) * D + lo;
    const uint16_t *xhA = (const uint16_t *)L.X + ((size_t)p * a.Rp + rA) * L.Kh + lo;
    const uint16_t *xhB = (const uint16_t *)L.X + ((size_t)p * a.Rp + rB) * L.Kh + lo;
    const uint16_t *wqR = (const uint16_t *)L.Wq + ((size_t)p * L.N + nW) * D + lo;
    const uint16_t *whR = (const uint16_t *)L.Wh + ((size_t)p * L.N + nW) * L.Kh + lo;
    auto issue = [&](int i, DeepStage &dst) __attribute__((always_inline)) {
        const int k0 = i * kBK;
        const bool inq = k0 < Dq;
        // a slice past the end of the contraction copies slice 0 again (never used)
        const int kk = (k0 + 16 * cs < K) ? (inq ? k0 : k0 - Dq) : -16 * cs;
        const uint16_t *sA = (inq ? xqA : xhA) + kk;
        const uint16_t *sB = (inq ? xqB : xhB) + kk;
        const uint16_t *sW = (inq ? wqR : whR) + kk;
        __builtin_amdgcn_global_load_lds((const void *)sA, (lds_void *)&dst.x[(cs * kBM + (2 * (w & 3)) * 32) * 2],
                                         16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void *)sB,
                                         (lds_void *)&dst.x[(cs * kBM + (2 * (w & 3) + 1) * 32) * 2], 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void *)sW, (lds_void *)&dst.w[(cs * kBN + (w & 3) * 32) * 2], 16,
                                         0, 0);
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    const int r32 = lane & 31, hsel = (lane >> 5) ^ ((r32 >> 3) & 1);

    auto step = [&](int i, const DeepStage &cur, DeepStage &ahead) __attribute__((always_inline)) {
        if (i + 1 < nst) wait_vmcnt<3>();
        else wait_vmcnt<0>();
        stage_barrier();
        if (i + 2 < nst) issue(i + 2, ahead);
        const int k0 = i * kBK;
#pragma unroll
        for (int s = 0; s < kSl; ++s) {
            if (k0 + 16 * s >= K) break;                   // uniform: the ragged last stage
            u32x4 A[2], B[2];
#pragma unroll
            for (int ti = 0; ti < 2; ++ti) A[ti] = cur.w[(s * kBN + wc * 64 + 32 * ti + r32) * 2 + hsel];
#pragma unroll
            for (int tj = 0; tj < 2; ++tj) B[tj] = cur.x[(s * kBM + wr * 64 + 32 * tj + r32) * 2 + hsel];
#pragma unroll
            for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                for (int tj = 0; tj < 2; ++tj) acc[ti][tj] = mfma32(A[ti], B[tj], acc[ti][tj]);
        }
    };
    issue(0, st_a);
    if (nst > 1) issue(1, st_b);
    for (int i = 0; i < nst; i += 3) {
        step(i, st_a, st_c);
        if (i + 1 >= nst) break;
        step(i + 1, st_b, st_a);
        if (i + 2 >= nst) break;
        step(i + 2, st_c, st_b);
    }

    // register 4 qq + r of tile (ti, tj): output n0 + 64 wc + 32 ti + 8 qq + 4 (lane / 32) + r,
    // row rho0 + 64 wr + 32 tj + lane % 32
    if (!L.Y) {
        // the linear read-outs: fp32 rows of the output layout
#pragma unroll
        for (int tj = 0; tj < 2; ++tj) {
            const int rho = rho0 + wr * 64 + 32 * tj + r32;
            if (rho >= a.Rp) continue;
            const size_t o = out_row(p, rho, a.Hkv, a.G, 0, a.Hq) * L.N;
#pragma unroll
            for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                    const int nb = n0 + wc * 64 + 32 * ti + 8 * qq + 4 * (lane >> 5);
                    float y[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        y[r] = acc[ti][tj][4 * qq + r] + (nb + r < L.N ? L.b[(size_t)p * L.N + nb + r] : 0.f);
                        if (ACT >= 0) y[r] = act_fn<ACT>(y[r]);
                    }
                    if (nb + 3 < L.N) {
                        *(f32x4 *)(L.Yf + o + nb) = f32x4{y[0], y[1], y[2], y[3]};
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (nb + r < L.N) L.Yf[o + nb + r] = y[r];
                    }
                }
        }
        return;
    }
    // hidden states (bf16; widths are multiples of 32): each wave stages its
    // 32 x 64 tiles through the free stage ring so the stores write whole
    // 128-byte row segments (a lane holds four columns of one row)
    __syncthreads();
    uint16_t *ys = (uint16_t *)((w < 3 ? (char *)&st_a : (w < 6 ? (char *)&st_b : (char *)&st_c)) + (w % 3) * 8192);
    const int hh = lane >> 5;
#pragma unroll
    for (int tj = 0; tj < 2; ++tj) {
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const int nb = n0 + wc * 64 + 32 * ti + 8 * qq + 4 * hh;
                float y[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    y[r] = acc[ti][tj][4 * qq + r] + (nb + r < L.N ? L.b[(size_t)p * L.N + nb + r] : 0.f);
                    if (ACT >= 0) y[r] = act_fn<ACT>(y[r]);
                }
                *(u32x2 *)(ys + r32 * 64 + (((4 * ti + qq) ^ (r32 & 7)) * 8) + 4 * hh) =
                    u32x2{pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3])};
            }
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int idx = 64 * it + lane, rr = idx >> 3, pc = idx & 7;
            const int rho = rho0 + wr * 64 + 32 * tj + rr, col = n0 + wc * 64 + 8 * pc;
            const u32x4 yv = *(const u32x4 *)(ys + rr * 64 + ((pc ^ (rr & 7)) * 8));
            if (rho < a.Rp && col < L.N) *(u32x4 *)((uint16_t *)L.Y + ((size_t)p * a.Rp + rho) * L.N + col) = yv;
        }
    }
}

template <int D>
__global__ __launch_bounds__(256) void deep_layer_valu(DeepParams a) {
    long blk = blockIdx.x;
    const DeepLayer &L = pick_layer(a, blk);
    const long idx = blk * 256 + threadIdx.x;
    if (idx >= (long)a.Hkv * a.Rp * L.N) return;
    const int n = (int)(idx % L.N);
    const long pr = idx / L.N;
    const int rho = (int)(pr % a.Rp), p = (int)(pr / a.Rp);
    float z = L.b[(size_t)p * L.N + n];
    if (L.Wq) {
        const float *w = (const float *)L.Wq + ((size_t)p * L.N + n) * D;
        const float *x = (const float *)a.q + out_row(p, rho, a.Hkv, a.G, 0, a.Hq) * D;
        for (int k = 0; k < D; ++k) z += w[k] * x[k];
    }
    if (L.Wh) {
        const float *w = (const float *)L.Wh + ((size_t)p * L.N + n) * L.Kh;
        const float *x = (const float *)L.X + ((size_t)p * a.Rp + rho) * L.Kh;
        for (int k = 0; k < L.Kh; ++k) z += w[k] * x[k];
    }
    if (L.act >= 0) z = activation(L.act, z);
    if (L.Y) ((float *)L.Y)[((size_t)p * a.Rp + rho) * L.N + n] = z;
    else L.Yf[out_row(p, rho, a.Hkv, a.G, 0, a.Hq) * L.N + n] = z;
}

long deep_layer_blocks(int dtype, int lds, int Hkv, int Rp, int N) {
    if (dtype == 1 && lds) {
        const long rg = (long)Hkv * ((Rp + kBM - 1) / kBM);
        return (rg + kXcd - 1) / kXcd * kXcd * ((N + kBN - 1) / kBN);
    }
    if (dtype == 1) return (long)Hkv * ((Rp + 15) / 16) * ((N + 15) / 16);
    return ((long)Hkv * Rp * N + 255) / 256;
}

hipError_t launch_deep_layers(const DeepParams &p, int dtype, int d, int lds, hipStream_t st) {
    const long blocks = p.L0.blocks + (p.nl > 1 ? p.L1.blocks : 0);
    if (blocks <= 0) return hipSuccess;
    dim3 grid((unsigned)blocks);
    if (dtype == 1 && lds) {
        const dim3 block(64 * kLdsWaves);
        const int act = p.L0.act;      // both layers of a launch share it
#define NECTAR_DEEP_LDS(DD, AA) hipLaunchKernelGGL((deep_layer_lds32<DD, AA>), grid, block, 0, st, p)
        if (d == 128) {
            if (act < 0) NECTAR_DEEP_LDS(128, -1);
            else if (act == 1) NECTAR_DEEP_LDS(128, 1);
            else if (act == 2) NECTAR_DEEP_LDS(128, 2);
            else NECTAR_DEEP_LDS(128, 0);
        } else if (d == 64) {
            if (act < 0) NECTAR_DEEP_LDS(64, -1);
            else if (act == 1) NECTAR_DEEP_LDS(64, 1);
            else if (act == 2) NECTAR_DEEP_LDS(64, 2);
            else NECTAR_DEEP_LDS(64, 0);
        } else {
            return hipErrorInvalidValue;
        }
#undef NECTAR_DEEP_LDS
    } else if (dtype == 1 && d == 128) hipLaunchKernelGGL(deep_layer_mfma<128>, grid, dim3(256), 0, st, p);
    else if (dtype == 1 && d == 64) hipLaunchKernelGGL(deep_layer_mfma<64>, grid, dim3(256), 0, st, p);
    else if (d == 128) hipLaunchKernelGGL(deep_layer_valu<128>, grid, dim3(256), 0, st, p);
    else if (d == 64) hipLaunchKernelGGL(deep_layer_valu<64>, grid, dim3(256), 0, st, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace nectar
