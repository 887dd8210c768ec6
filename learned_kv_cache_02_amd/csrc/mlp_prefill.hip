// Nectar MLP module forward for many query rows (batched prefill): the same
// one-hidden-layer score/target networks as mlp.hip (Eq. (3.6) of the Nectar
// notes with one hidden layer), tiled for the MFMA-bound regime.  This kernel
// serves hidden widths that are not multiples of 64; mlp_lds.hip serves the rest.
//
// A block of 8 waves (two per SIMD, so one wave's activations overlap the
// other's matrix work) owns 256 query rows of one KV head -- all G query heads
// of the group, consecutive tokens; each wave holds 32 rows (two 16-row tiles).
// The block walks the hidden units in chunks of 32 and stages each chunk's
// weights once in LDS, double-buffered, with the global loads issued two chunks
// ahead of use:
//   first-layer rows are stored in MFMA A-operand order (one 16-byte read per
//   lane per operand), read-out rows are stored transposed and slot-ordered so
//   a lane reads its W2t^T operand with one 16-byte read per 16 dimensions.
// Per chunk and 16-row tile a wave runs
//   Z^T = b1 + W1_chunk . Q^T (8 MFMAs, the bias is the accumulator's initial
//   value) -> act -> bf16 -> O^T += W2t^T . H^T (8 MFMAs)
// so the hidden activations never leave registers; score chunks run
//   Zs^T = bs + Ws_chunk . Q^T -> act -> fp32 dot with ws2.
//
// The erf-form GELU is evaluated as x * (0.5 + c P(c^2)), c = x clamped to
// [-3.71875, 3.71875], P of degree 6 (gelu_erf_poly).
// With one split (SB == 1) the block adds the output biases and writes (a, A);
// with SB > 1 splits of the hidden units, block (h, row block, split) writes its
// partial sums and mlp_reduce adds them in split order with the biases.
#include "device_common.hpp"
#include "kernels.hpp"

namespace nectar {

namespace {

constexpr int kD = 128, kKS = 4, kDV = 8, kRTW = 2, kThreads = 512, kRows = kThreads / 64 * kRTW * 16;
__device__ __forceinline__ int unit_of_slot(int g, int j) { return 16 * (j >> 2) + 4 * g + (j & 3); }

// One chunk's share of thread t: piece t of the 32 x 128 first-layer tile and
// of the read-out tile (16 pieces of 16 bytes per 256-byte row), one bias or
// score read-out weight.
struct Stage {
    u32x4 w1, w2;
    float b;
};

struct Smem {
    u32x4 w1[2][8][64];             // [buf][hh * 4 + kt][lane]
    uint16_t w2t[2][4][8][16][8];   // [buf][g][mm][c][slot j]: W2t[unit(g, j)][8c + mm]
    float b[2][32];
    float s[2][32];
};

__device__ __forceinline__ void stage_load(Stage &S, const uint16_t *W, const uint16_t *W2, const float *bias,
                                           const uint16_t *ws2, int j0, int H, bool target, int t) {
    const int u = t >> 4, k = t & 15;
    const size_t row = (size_t)min(j0 + u, H - 1) * kD + k * 8;
    S.w1 = stream_load((const u32x4 *)(W + row));
    if (target) S.w2 = stream_load((const u32x4 *)(W2 + row));
    S.b = 0.f;
    if (t < 32) S.b = (j0 + t < H) ? bias[j0 + t] : 0.f;
    else if (t < 64 && !target) S.b = (j0 + t - 32 < H) ? bf16_to_f32(ws2[j0 + t - 32]) : 0.f;
}

__device__ __forceinline__ void stage_store(Smem &sm, const Stage &S, int buf, bool target, int t) {
    const int u = t >> 4, k = t & 15;
    sm.w1[buf][(u >> 4) * 4 + (k >> 2)][(k & 3) * 16 + (u & 15)] = S.w1;
    if (target) {
        // piece (unit u, dims 8k .. 8k+7) -> lane column c = k, slot j of group g
        const int g = (u & 15) >> 2, j = 4 * (u >> 4) + (u & 3);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t wv = S.w2[e >> 1];
            sm.w2t[buf][g][e][k][j] = (uint16_t)((e & 1) ? (wv >> 16) : (wv & 0xffffu));
        }
    }
    if (t < 32) sm.b[buf][t] = S.b;
    else if (t < 64 && !target) sm.s[buf][t - 32] = S.b;
}

}  // namespace

template <int ACT>
__global__ __launch_bounds__(kThreads) void mlp_prefill_mfma(MlpParams a) {
    __shared__ Smem sm;
    const int nrb = (a.Rp + kRows - 1) / kRows;
    const int sb = blockIdx.x % a.SB, hr = blockIdx.x / a.SB;
    const int h = hr / nrb, rb = hr - h * nrb;
    const int t = threadIdx.x, w = t >> 6, lane = t & 63, g = lane >> 4, c = lane & 15;
    auto act = [&](float x) { return ACT == 0 ? gelu_erf_poly(x) : act_fn<ACT>(x); };

    u32x4 qv[kRTW][kKS];
#pragma unroll
    for (int rt = 0; rt < kRTW; ++rt) {
        const int rho = rb * kRows + (w * kRTW + rt) * 16 + c;
        if (rho < a.Rp) {
            const int tk = rho / a.G, gg = rho - tk * a.G;
            const uint16_t *qp = (const uint16_t *)a.q + ((size_t)tk * a.Hq + h * a.G + gg) * kD;
#pragma unroll
            for (int kt = 0; kt < kKS; ++kt) qv[rt][kt] = *(const u32x4 *)(qp + (4 * kt + g) * 8);
        } else {
#pragma unroll
            for (int kt = 0; kt < kKS; ++kt) qv[rt][kt] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    f32x4 O[kRTW][kDV];
    float sc[kRTW];
#pragma unroll
    for (int rt = 0; rt < kRTW; ++rt) {
        sc[rt] = 0.f;
#pragma unroll
        for (int mm = 0; mm < kDV; ++mm) O[rt][mm] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const uint16_t *W1 = (const uint16_t *)a.W1 + (size_t)h * a.Ht * kD;
    const uint16_t *W2t = (const uint16_t *)a.W2t + (size_t)h * a.Ht * kD;
    const float *b1 = a.b1 + (size_t)h * a.Ht;
    const uint16_t *Ws = (const uint16_t *)a.Ws + (size_t)h * a.Hs * kD;
    const uint16_t *ws2 = (const uint16_t *)a.ws2 + (size_t)h * a.Hs;
    const float *bs = a.bs + (size_t)h * a.Hs;
    // this split's chunks: target chunks [t0, t0 + ntc), then score chunks [s0, s0 + nsc)
    const int ttot = (a.Ht + 31) / 32, stot = (a.Hs + 31) / 32;
    const int ctc = a.chunk_t / 32, csc = a.chunk_s / 32;
    const int t0 = min(sb * ctc, ttot), s0 = min(sb * csc, stot);
    const int ntc = min(ctc, ttot - t0), nch = ntc + min(csc, stot - s0);

    auto load_chunk = [&](Stage &S, int i) {
        if (i < ntc) stage_load(S, W1, W2t, b1, nullptr, 32 * (t0 + i), a.Ht, true, t);
        else stage_load(S, Ws, nullptr, bs, ws2, 32 * (s0 + i - ntc), a.Hs, false, t);
    };

    auto compute = [&](int i) {
        const int buf = i & 1;
        u32x4 w1op[2][kKS];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int kt = 0; kt < kKS; ++kt) w1op[hh][kt] = sm.w1[buf][hh * 4 + kt][lane];
        float bias[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) bias[j] = sm.b[buf][unit_of_slot(g, j)];
        if (i < ntc) {
            const int j0 = 32 * (t0 + i);
            u32x4 vt[kDV];
#pragma unroll
            for (int mm = 0; mm < kDV; ++mm) vt[mm] = *(const u32x4 *)&sm.w2t[buf][g][mm][c][0];
#pragma unroll
            for (int rt = 0; rt < kRTW; ++rt) {
                f32x4 z0 = {bias[0], bias[1], bias[2], bias[3]}, z1 = {bias[4], bias[5], bias[6], bias[7]};
#pragma unroll
                for (int kt = 0; kt < kKS; ++kt) {
                    z0 = mfma16(w1op[0][kt], qv[rt][kt], z0);
                    z1 = mfma16(w1op[1][kt], qv[rt][kt], z1);
                }
                float hv[8];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    hv[r] = act(z0[r]);
                    hv[4 + r] = act(z1[r]);
                }
                if (j0 + 32 > a.Ht) {
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        if (j0 + unit_of_slot(g, j) >= a.Ht) hv[j] = 0.f;
                }
                const u32x4 H = {pack_bf16(hv[0], hv[1]), pack_bf16(hv[2], hv[3]), pack_bf16(hv[4], hv[5]),
                                 pack_bf16(hv[6], hv[7])};
#pragma unroll
                for (int mm = 0; mm < kDV; ++mm) O[rt][mm] = mfma16(vt[mm], H, O[rt][mm]);
            }
        } else {
            float wsv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) wsv[j] = sm.s[buf][unit_of_slot(g, j)];
#pragma unroll
            for (int rt = 0; rt < kRTW; ++rt) {
                f32x4 z0 = {bias[0], bias[1], bias[2], bias[3]}, z1 = {bias[4], bias[5], bias[6], bias[7]};
#pragma unroll
                for (int kt = 0; kt < kKS; ++kt) {
                    z0 = mfma16(w1op[0][kt], qv[rt][kt], z0);
                    z1 = mfma16(w1op[1][kt], qv[rt][kt], z1);
                }
                float acc = 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j)      // units past Hs carry ws2 = 0
                    acc += wsv[j] * act(j < 4 ? z0[j] : z1[j - 4]);
                sc[rt] += acc;
            }
        }
    };

    // chunk i is computed from LDS buffer i & 1; its global loads were issued
    // while chunk i - 2 was computed (staging set i & 1), and it is written to
    // LDS after chunk i - 1 is computed.
    if (nch > 0) {
        Stage S0, S1;
        load_chunk(S0, 0);
        if (nch > 1) load_chunk(S1, 1);
        stage_store(sm, S0, 0, 0 < ntc, t);
        __syncthreads();
        for (int i = 0; i < nch; i += 2) {
            if (i + 2 < nch) load_chunk(S0, i + 2);
            compute(i);
            if (i + 1 < nch) stage_store(sm, S1, 1, i + 1 < ntc, t);
            __syncthreads();
            if (i + 1 >= nch) break;
            if (i + 3 < nch) load_chunk(S1, i + 3);
            compute(i + 1);
            if (i + 2 < nch) stage_store(sm, S0, 0, i + 2 < ntc, t);
            __syncthreads();
        }
    }

#pragma unroll
    for (int rt = 0; rt < kRTW; ++rt) {
        const float ssum = group4_sum(sc[rt]);
        const int rho = rb * kRows + (w * kRTW + rt) * 16 + c;
        if (rho >= a.Rp) continue;
        if (a.SB > 1 || a.defer) {
            const size_t row = (size_t)(h * a.SB + sb) * a.Rp + rho;
            if (g == 0) a.part_s[row] = ssum;
            float *op = a.part_O + row * kD;
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int m4 = 0; m4 < kDV; m4 += 4) {
                    f32x4 v = {O[rt][m4][r], O[rt][m4 + 1][r], O[rt][m4 + 2][r], O[rt][m4 + 3][r]};
                    *(f32x4 *)(op + kDV * (4 * g + r) + m4) = v;
                }
            continue;
        }
        const int tk = rho / a.G, gg = rho - tk * a.G;
        const size_t o = (size_t)tk * a.Hq + h * a.G + gg;
        if (g == 0) a.a_out[o] = a.bs2[h] + ssum;
        const float *b2 = a.b2 + (size_t)h * kD;
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int m4 = 0; m4 < kDV; m4 += 4) {
                const int dc = kDV * (4 * g + r) + m4;
                f32x4 v = {b2[dc] + O[rt][m4][r], b2[dc + 1] + O[rt][m4 + 1][r], b2[dc + 2] + O[rt][m4 + 2][r],
                           b2[dc + 3] + O[rt][m4 + 3][r]};
                *(f32x4 *)(a.A_out + o * kD + dc) = v;
            }
    }
}

hipError_t launch_mlp_prefill(const MlpParams &p, hipStream_t st) {
    const long nrb = (p.Rp + kRows - 1) / kRows;
    dim3 grid((unsigned)(p.Hkv * nrb * p.SB)), block(kThreads);
    if (p.act == 1) hipLaunchKernelGGL(mlp_prefill_mfma<1>, grid, block, 0, st, p);
    else if (p.act == 2) hipLaunchKernelGGL(mlp_prefill_mfma<2>, grid, block, 0, st, p);
    else hipLaunchKernelGGL(mlp_prefill_mfma<0>, grid, block, 0, st, p);
    return hipGetLastError();
}

}  // namespace nectar
