// Regression training step of the one-hidden-layer module (section 2.3 of the
// Nectar notes, Eqs. (3.2)-(3.3)): the forward with its pre-activations kept,
// the loss lambda_alpha L_alpha + lambda_A L_A, the backward, global-norm
// gradient clipping and AdamW on fp32 master parameters.
//
// The dense contractions run on the 32x32x16 bf16 MFMA in two batched forms:
// the two first layers, the target read-out and the back-propagation through
// it are "NT" products
//   C[p][m][n] = sum_k X[p][m][k] W[p][n][k] (+ bias[p][n])   (gemm_nt_lds32)
// with both operands row-major and the contraction innermost (the read-out's
// weights go through one small transposed copy, transpose_bf16); the three
// weight gradients, whose contraction runs over the query rows, are "TN"
// products C[p][m][n] = sum_k X[p][k][m] W[p][k][n] (gemm_tn_lds32) that read
// the row-major hidden values and gradients as they are, their MFMA operands
// formed by transposing LDS reads.  The elementwise passes (activation, its
// derivative, the per-row score net and loss terms) and the bias gradients
// (fixed-order column sums) are plain VALU kernels; sums that feed the loss and
// the clipping norm are fixed-order, so a step is reproducible.
#include "attn_common.hpp"
#include "lds_common.hpp"

namespace nectar {

namespace {

constexpr int kBM = 256, kBN = 128, kBK = 32, kSl = kBK / 16, kWaves = 8, kXcd = 8;

struct GemmStage {
    u32x4 x[kSl * kBM * 2];   // [slice][row][half]
    u32x4 w[kSl * kBN * 2];
};
// the bf16 epilogue stages three waves' 32 x 64 tiles (8 KB each) in one stage buffer
static_assert(sizeof(GemmStage) >= 3 * 8192, "epilogue staging");

}  // namespace

// Tile: 256 rows of X x 128 rows of W per block of eight waves, 32-wide
// contraction stages in a three-stage LDS ring filled by direct copies two
// stages ahead (the layout and copy pattern of the deep-MLP layer kernel).
template <int EPI, int ACT>
__global__ __launch_bounds__(64 * kWaves, 4) void gemm_nt_lds32(GemmParams g) {
    __shared__ GemmStage st_a, st_b, st_c;

    const int NT = (g.N + kBN - 1) / kBN, nrb = (g.M + kBM - 1) / kBM;
    const long per_split = (long)((g.P * nrb + kXcd - 1) / kXcd * kXcd) * NT;
    const int ks = (int)(blockIdx.x / per_split);
    const long blk = blockIdx.x - (long)ks * per_split;
    const int xcd = (int)(blk % kXcd);
    const long kq = blk / kXcd;
    const int nt = (int)(kq % NT);
    const int rgi = (int)(kq / NT) * kXcd + xcd;
    if (rgi >= g.P * nrb) return;
    const int p = rgi / nrb, m0 = (rgi - p * nrb) * kBM, n0 = nt * kBN;

    const int t = threadIdx.x, w = t >> 6, lane = t & 63;
    const int wr = w & 3, wc = w >> 2;
    // this block's contraction range [kb, kb + Kc)
    const int kb = ks * g.kchunk, Kc = min(g.K - kb, g.kchunk);
    const int nst = (Kc + kBK - 1) / kBK;
    const int cs = w >> 2, half = (lane & 1) ^ ((lane >> 4) & 1);
    const size_t lo = kb + 16 * cs + 8 * half;
    const int rA = min(m0 + (2 * (w & 3)) * 32 + (lane >> 1), g.M - 1);
    const int rB = min(m0 + (2 * (w & 3) + 1) * 32 + (lane >> 1), g.M - 1);
    const int rW = min(n0 + (w & 3) * 32 + (lane >> 1), g.N - 1);
    const uint16_t *xA = g.X + p * g.sx + (size_t)rA * g.ldx + lo;
    const uint16_t *xB = g.X + p * g.sx + (size_t)rB * g.ldx + lo;
    const uint16_t *wR = g.W + p * g.sw + (size_t)rW * g.ldw + lo;

    auto issue = [&](int i, GemmStage &dst) __attribute__((always_inline)) {
        const int k0 = i * kBK;
        const int kk = (k0 + 16 * cs < Kc) ? k0 : -16 * cs;    // past the end: slice 0 again (unused)
        __builtin_amdgcn_global_load_lds((const void *)(xA + kk),
                                         (lds_void *)&dst.x[(cs * kBM + (2 * (w & 3)) * 32) * 2], 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void *)(xB + kk),
                                         (lds_void *)&dst.x[(cs * kBM + (2 * (w & 3) + 1) * 32) * 2], 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void *)(wR + kk), (lds_void *)&dst.w[(cs * kBN + (w & 3) * 32) * 2],
                                         16, 0, 0);
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    const int r32 = lane & 31, hsel = (lane >> 5) ^ ((r32 >> 3) & 1);

    auto step = [&](int i, const GemmStage &cur, GemmStage &ahead) __attribute__((always_inline)) {
        if (i + 1 < nst) wait_vmcnt<3>();
        else wait_vmcnt<0>();
        stage_barrier();
        if (i + 2 < nst) issue(i + 2, ahead);
        const int k0 = i * kBK;
#pragma unroll
        for (int s = 0; s < kSl; ++s) {
            if (k0 + 16 * s >= Kc) break;
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

    // register 4 qq + r of tile (ti, tj): column n0 + 64 wc + 32 ti + 8 qq + 4 (lane / 32) + r,
    // row m0 + 64 wr + 32 tj + lane % 32.  Every load the epilogue needs (the
    // lane's 32 biases, epilogue 2's pre-activations) is issued before the first use.
    const bool part = g.ksplit > 1;
    f32x4 bq[2][4];
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            const int nb = n0 + wc * 64 + 32 * ti + 8 * qq + 4 * (lane >> 5);
            bq[ti][qq] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (!part && EPI != 2 && g.bias) {
                if (nb + 3 < g.N) {
                    bq[ti][qq] = *(const f32x4 *)(g.bias + p * g.sb + nb);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (nb + r < g.N) bq[ti][qq][r] = g.bias[p * g.sb + nb + r];
                }
            }
        }
    // epilogue 2's pre-activations: whole 128-byte row segments of the wave's
    // 32 x 64 tiles (eight lanes per row), staged through LDS below
    u32x4 zin[2][4];
    if (EPI == 2) {
#pragma unroll
        for (int tj = 0; tj < 2; ++tj)
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int idx = 64 * it + lane, rr = idx >> 3, pc = idx & 7;
                const int m = min(m0 + wr * 64 + 32 * tj + rr, g.M - 1);
                const int col = min(n0 + wc * 64 + 8 * pc, g.N - 8);
                zin[tj][it] = *(const u32x4 *)(g.Zi + p * g.sc + (size_t)m * g.ldc + col);
            }
    }
    // Outputs go through the stage ring (free after the loop): each wave
    // stages its 32 x 64 tiles in its own 8 KB so the stores write whole
    // row segments (a lane holds four columns of one row per register group).
    __syncthreads();
    char *reg = (w < 3 ? (char *)&st_a : (w < 6 ? (char *)&st_b : (char *)&st_c)) + (w % 3) * 8192;
    const int hh = lane >> 5;
    if (EPI == 0) {
        // fp32 (or split partials): [32 rows][16 pieces of four columns], swizzled
        float *cs = (float *)reg;
#pragma unroll
        for (int tj = 0; tj < 2; ++tj) {
#pragma unroll
            for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                    const int pc = 8 * ti + 2 * qq + hh;
                    *(f32x4 *)(cs + r32 * 64 + ((pc ^ (r32 & 15)) * 4)) =
                        f32x4{acc[ti][tj][4 * qq] + bq[ti][qq][0], acc[ti][tj][4 * qq + 1] + bq[ti][qq][1],
                              acc[ti][tj][4 * qq + 2] + bq[ti][qq][2], acc[ti][tj][4 * qq + 3] + bq[ti][qq][3]};
                }
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                const int idx = 64 * it + lane, rr = idx >> 4, pc = idx & 15;
                const int m = m0 + wr * 64 + 32 * tj + rr, col = n0 + wc * 64 + 4 * pc;
                const f32x4 v = *(const f32x4 *)(cs + rr * 64 + ((pc ^ (rr & 15)) * 4));
                if (m >= g.M || col >= g.N) continue;
                float *c = (part ? g.Cpart + (((size_t)ks * g.P + p) * g.M + m) * g.N
                                 : g.C + p * g.sc + (size_t)m * g.ldc) + col;
                if (col + 3 < g.N) {
                    *(f32x4 *)c = v;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (col + r < g.N) c[r] = v[r];
                }
            }
        }
        return;
    }

    // bf16 outputs (EPI 1: pre-activation and activation; EPI 2: the gradient
    // times act'), 128-byte row segments.  Widths are multiples of 32.
    uint16_t *zs = (uint16_t *)reg, *ys = (uint16_t *)(reg + 4096);   // [32 rows][8 pieces][8], swizzled
#pragma unroll
    for (int tj = 0; tj < 2; ++tj) {
        if (EPI == 2) {
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int idx = 64 * it + lane, rr = idx >> 3, pc = idx & 7;
                *(u32x4 *)(zs + rr * 64 + ((pc ^ (rr & 7)) * 8)) = zin[tj][it];
            }
        }
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                float y[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) y[r] = acc[ti][tj][4 * qq + r] + bq[ti][qq][r];
                const int off = r32 * 64 + (((4 * ti + qq) ^ (r32 & 7)) * 8) + 4 * hh;
                if (EPI == 1) {
                    *(u32x2 *)(zs + off) = u32x2{pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3])};
#pragma unroll
                    for (int r = 0; r < 4; ++r) y[r] = act_fn<ACT>(y[r]);
                } else {
                    const u32x2 zz = *(const u32x2 *)(zs + off);
                    y[0] *= act_grad_fn<ACT>(bf16lo(zz.x));
                    y[1] *= act_grad_fn<ACT>(bf16hi(zz.x));
                    y[2] *= act_grad_fn<ACT>(bf16lo(zz.y));
                    y[3] *= act_grad_fn<ACT>(bf16hi(zz.y));
                }
                *(u32x2 *)(ys + off) = u32x2{pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3])};
            }
        // 32 rows x 8 pieces of 16 bytes, four per lane, eight lanes per row
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int idx = 64 * it + lane, rr = idx >> 3, pc = idx & 7;
            const int m = m0 + wr * 64 + 32 * tj + rr, col = n0 + wc * 64 + 8 * pc;
            const int src = rr * 64 + ((pc ^ (rr & 7)) * 8);
            const u32x4 yv = *(const u32x4 *)(ys + src);
            u32x4 zv;
            if (EPI == 1) zv = *(const u32x4 *)(zs + src);
            if (m < g.M && col < g.N) {
                const size_t o = p * g.sc + (size_t)m * g.ldc + col;
                if (EPI == 1) *(u32x4 *)(g.Zo + o) = zv;
                *(u32x4 *)(g.Y + o) = yv;
            }
        }
    }
}

// "TN" product for the contractions over the query rows (the weight
// gradients): C[p][m][n] = sum_k X[p][k][m] W[p][k][n], both operands stored
// row-major with the contraction OUTERMOST (the hidden values or gradients
// [rows][units], the queries or output gradients [rows][d]), fp32 out (or
// split partials).  The same tiling and three-stage ring as gemm_nt_lds32, but
// a stage holds 32 contraction rows of each operand as they lie in memory and
// the MFMA operands (eight consecutive contraction indices of one column per
// lane) come out of it by gfx950's transposing LDS read, so no transposed copy
// is ever written.  Each 16-byte piece p of a stage row k sits at position
// p ^ 2 (k % 4): the four rows one transposing read touches then fill distinct
// banks.  Rows past the contraction end are zeroed in LDS before use.
__global__ __launch_bounds__(64 * kWaves, 4) void gemm_tn_lds32(GemmParams g) {
    struct Stage {
        u32x4 x[kBK * kBM / 8];   // [k][256 columns]: 32 pieces per row
        u32x4 w[kBK * kBN / 8];   // [k][128 columns]: 16 pieces per row
    };
    __shared__ Stage st_a, st_b, st_c;

    const int NT = (g.N + kBN - 1) / kBN, nrb = (g.M + kBM - 1) / kBM;
    const long per_split = (long)((g.P * nrb + kXcd - 1) / kXcd * kXcd) * NT;
    const int ks = (int)(blockIdx.x / per_split);
    const long blk = blockIdx.x - (long)ks * per_split;
    const int xcd = (int)(blk % kXcd);
    const long kq = blk / kXcd;
    const int nt = (int)(kq % NT);
    const int rgi = (int)(kq / NT) * kXcd + xcd;
    if (rgi >= g.P * nrb) return;
    const int p = rgi / nrb, m0 = (rgi - p * nrb) * kBM, n0 = nt * kBN;

    const int t = threadIdx.x, w = t >> 6, lane = t & 63;
    const int wr = w & 3, wc = w >> 2;
    const int kb = ks * g.kchunk, Kc = min(g.K - kb, g.kchunk);
    const int nst = (Kc + kBK - 1) / kBK;
    const uint16_t *X = g.X + p * g.sx, *W = g.W + p * g.sw;

    // copies: wave w fills X rows 2w, 2w + 1 and 2w + 16, 2w + 17 (32 pieces
    // each, one row per 32 lanes) and W rows 4w .. 4w + 3 (16 pieces each)
    auto issue = [&](int i, Stage &dst) __attribute__((always_inline)) {
        const int k0 = kb + i * kBK;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int r = 2 * w + 16 * c + (lane >> 5), pos = lane & 31;
            const int k = min(k0 + r, g.K - 1);
            const int col = min(m0 + 8 * (pos ^ (2 * (r & 3))), g.M - 8);
            __builtin_amdgcn_global_load_lds((const void *)(X + (size_t)k * g.ldx + col),
                                             (lds_void *)&dst.x[(2 * w + 16 * c) * 32], 16, 0, 0);
        }
        const int r = 4 * w + (lane >> 4), pos = lane & 15;
        const int k = min(k0 + r, g.K - 1);
        const int col = min(n0 + 8 * (pos ^ (2 * (r & 3))), g.N - 8);
        __builtin_amdgcn_global_load_lds((const void *)(W + (size_t)k * g.ldw + col),
                                         (lds_void *)&dst.w[(4 * w) * 16], 16, 0, 0);
    };

    // per-lane byte offsets (within a 16-row slice) of the slot this lane names
    // for the transposing reads: rows 8 (lane / 32) + 4 h + (lane / 4) % 4,
    // columns 16 ((lane / 16) % 2) + 4 (lane % 4) .. + 3 of the wave's tiles
    const int G = lane >> 4, aa = lane & 3, e = (lane >> 2) & 3;
    uint32_t wo[2][2], xo[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int r = 8 * (G >> 1) + 4 * h + e;
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) {
            const int pw = 8 * wc + ((4 * ti + 2 * (G & 1) + (aa >> 1)) ^ (2 * e));
            wo[ti][h] = (uint32_t)(r * 256 + pw * 16 + (aa & 1) * 8);
            const int px = 8 * wr + ((4 * ti + 2 * (G & 1) + (aa >> 1)) ^ (2 * e));
            xo[ti][h] = (uint32_t)(r * 512 + px * 16 + (aa & 1) * 8);
        }
    }

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    // optional column sums of X over this block's contraction range (the bias
    // gradient of the same product): the waves of the first column half add
    // up the eight contraction values of each of their X operands
    const bool xs_on = g.xsum != nullptr && wc == 0;
    float xs[2] = {0.f, 0.f};

    auto step = [&](int i, Stage &cur, Stage &ahead) __attribute__((always_inline)) {
        if (i + 1 < nst) wait_vmcnt<3>();
        else wait_vmcnt<0>();
        stage_barrier();
        const int k0 = i * kBK;
        if (k0 + kBK > Kc) {
            // rows past the contraction end: zero in both operands
            const int kv = Kc - k0;
            for (int u = t; u < kBK * 48; u += 64 * kWaves) {
                const int r = u / 48, pc = u - r * 48;
                if (r < kv) continue;
                if (pc < 32) cur.x[r * 32 + pc] = u32x4{0u, 0u, 0u, 0u};
                else cur.w[r * 16 + pc - 32] = u32x4{0u, 0u, 0u, 0u};
            }
            __syncthreads();
        }
        if (i + 2 < nst) issue(i + 2, ahead);
#pragma unroll
        for (int sl = 0; sl < kBK / 16; ++sl) {
            if (k0 + 16 * sl >= Kc) break;
            u32x4 A[2], B[2];
#pragma unroll
            for (int ti = 0; ti < 2; ++ti) {
                const u32x2 a0 = lds_read_tr16(cur.w, sl * 16 * 256 + wo[ti][0]);
                const u32x2 a1 = lds_read_tr16(cur.w, sl * 16 * 256 + wo[ti][1]);
                A[ti] = u32x4{a0.x, a0.y, a1.x, a1.y};
                const u32x2 b0 = lds_read_tr16(cur.x, sl * 16 * 512 + xo[ti][0]);
                const u32x2 b1 = lds_read_tr16(cur.x, sl * 16 * 512 + xo[ti][1]);
                B[ti] = u32x4{b0.x, b0.y, b1.x, b1.y};
            }
#pragma unroll
            for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                for (int tj = 0; tj < 2; ++tj) acc[ti][tj] = mfma32(A[ti], B[tj], acc[ti][tj]);
            if (xs_on) {
#pragma unroll
                for (int tj = 0; tj < 2; ++tj)
#pragma unroll
                    for (int u = 0; u < 4; ++u) xs[tj] += bf16lo(B[tj][u]) + bf16hi(B[tj][u]);
            }
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

    // register 4 qq + r of tile (ti, tj): column n0 + 64 wc + 32 ti + 8 qq + 4 (lane / 32) + r,
    // row m0 + 64 wr + 32 tj + lane % 32 (the layout of gemm_nt_lds32)
    const bool part = g.ksplit > 1;
    const int r32 = lane & 31;
    if (g.xsum != nullptr && nt == 0) {
        // lanes l and l ^ 32 hold the two contraction halves of column l % 32
#pragma unroll
        for (int tj = 0; tj < 2; ++tj) xs[tj] += __shfl_xor(xs[tj], 32, 64);
        const int m = m0 + wr * 64 + 32 * (lane >> 5) + r32;     // lane half h writes tile tj = h
        const float v = (lane >> 5) ? xs[1] : xs[0];
        if (wc == 0 && m < g.M) {
            if (part) g.xsum_part[((size_t)ks * g.P + p) * g.M + m] = v;
            else g.xsum[p * g.sxs + m] = v;
        }
    }
#pragma unroll
    for (int tj = 0; tj < 2; ++tj) {
        const int m = m0 + wr * 64 + 32 * tj + r32;
        if (m >= g.M) continue;
        const size_t row = part ? (((size_t)ks * g.P + p) * g.M + m) * g.N : p * g.sc + (size_t)m * g.ldc;
        float *c = (part ? g.Cpart : g.C) + row;
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const int nb = n0 + wc * 64 + 32 * ti + 8 * qq + 4 * (lane >> 5);
                if (nb >= g.N) continue;
                *(f32x4 *)(c + nb) = f32x4{acc[ti][tj][4 * qq], acc[ti][tj][4 * qq + 1], acc[ti][tj][4 * qq + 2],
                                           acc[ti][tj][4 * qq + 3]};
            }
    }
}

// Column sums over the rows, fixed order: parts[p][c][col] = the sum of rows
// [64 c, 64 c + 64) of X[p][row][col] * (v ? v[p][row] : 1) (four columns per
// thread, 16 rows' loads in flight), then out[p][col] = the parts summed in
// chunk order.
__global__ __launch_bounds__(256) void col_sum_parts(ColSumParams a) {
    const int nch = (a.rows + 63) / 64, cq = a.cols / 4;
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= (long)a.P * nch * cq) return;
    const int q = (int)(i % cq);
    const long pc = i / cq;
    const int c = (int)(pc % nch), p = (int)(pc / nch);
    const int r0 = 64 * c, r1 = min(r0 + 64, a.rows);
    const uint16_t *x = a.X + p * a.sx + 4 * q;
    const float *v = a.v ? a.v + p * a.sv : nullptr;
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    for (int rb = r0; rb < r1; rb += 16) {
        u32x2 xv[16];
        float vr[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int r = min(rb + u, r1 - 1);
            xv[u] = *(const u32x2 *)(x + (size_t)r * a.ldx);
            vr[u] = (rb + u < r1) ? (v ? v[r] : 1.f) : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            s[0] = __builtin_fmaf(bf16lo(xv[u].x), vr[u], s[0]);
            s[1] = __builtin_fmaf(bf16hi(xv[u].x), vr[u], s[1]);
            s[2] = __builtin_fmaf(bf16lo(xv[u].y), vr[u], s[2]);
            s[3] = __builtin_fmaf(bf16hi(xv[u].y), vr[u], s[3]);
        }
    }
    *(f32x4 *)(a.parts + ((size_t)p * nch + c) * a.cols + 4 * q) = s;
}

__global__ __launch_bounds__(256) void col_sum_final(ColSumParams a) {
    const int nch = (a.rows + 63) / 64, cq = a.cols / 4;
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= (long)a.P * cq) return;
    const int q = (int)(i % cq), p = (int)(i / cq);
    const float *pp = a.parts + (size_t)p * nch * a.cols + 4 * q;
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < nch; c0 += 16) {
        f32x4 pv[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)
            pv[u] = (c0 + u < nch) ? *(const f32x4 *)(pp + (size_t)(c0 + u) * a.cols) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 16; ++u) s += pv[u];
    }
    *(f32x4 *)(a.out + p * a.so + 4 * q) = s;
}

// C[p][m][n] = sum over the splits of the partial tiles + bias (fixed order);
// with xsum, also xsum[p][m] = the sum over the splits of its partials.
__global__ __launch_bounds__(256) void gemm_reduce(GemmParams g) {
    if (g.xsum) {
        for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < (long)g.P * g.M; i += (long)gridDim.x * 256) {
            const int m = (int)(i % g.M), p = (int)(i / g.M);
            float s = 0.f;
            for (int ks = 0; ks < g.ksplit; ++ks) s += g.xsum_part[((size_t)ks * g.P + p) * g.M + m];
            g.xsum[p * g.sxs + m] = s;
        }
    }
    const long n4 = (long)g.P * g.M * (g.N / 4);
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n4; i += (long)gridDim.x * 256) {
        const int nq = (int)(i % (g.N / 4));
        const long pm = i / (g.N / 4);
        const int m = (int)(pm % g.M), p = (int)(pm / g.M);
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
        for (int ks = 0; ks < g.ksplit; ++ks)
            s += *(const f32x4 *)(g.Cpart + (((size_t)ks * g.P + p) * g.M + m) * g.N + 4 * nq);
        if (g.bias) s += *(const f32x4 *)(g.bias + p * g.sb + 4 * nq);
        *(f32x4 *)(g.C + p * g.sc + (size_t)m * g.ldc + 4 * nq) = s;
    }
}

// out[p][c][r] = in[p][r][c] for r < rows, 0 for rows <= r < ldo (64 x 64
// tiles through LDS; four elements per thread and access on both sides).
// cols, ldi and ldo are multiples of 4.
__global__ __launch_bounds__(256) void transpose_bf16(TransposeParams a) {
    __shared__ uint16_t tile[64][68];
    const int tc = (a.cols + 63) / 64, tr = (a.ldo + 63) / 64;
    long b = blockIdx.x;
    const int bc = (int)(b % tc);
    b /= tc;
    const int br = (int)(b % tr), p = (int)(b / tr);
    const int r0 = br * 64, c0 = bc * 64;
    const uint16_t *in = a.in + p * a.si;
    uint16_t *out = a.out + p * a.so;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int e = threadIdx.x + 256 * it;            // 64 rows x 16 four-column groups
        const int rr = e >> 4, cq = (e & 15) * 4;
        const int r = r0 + rr, c = c0 + cq;
        u32x2 v = {0u, 0u};
        if (r < a.rows && c < a.cols) v = *(const u32x2 *)(in + (size_t)r * a.ldi + c);
        tile[rr][cq + 0] = (uint16_t)(v.x & 0xffffu);
        tile[rr][cq + 1] = (uint16_t)(v.x >> 16);
        tile[rr][cq + 2] = (uint16_t)(v.y & 0xffffu);
        tile[rr][cq + 3] = (uint16_t)(v.y >> 16);
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int e = threadIdx.x + 256 * it;            // 64 columns x 16 four-row groups
        const int cc = e >> 4, rq = (e & 15) * 4;
        const int r = r0 + rq, c = c0 + cc;
        if (c < a.cols && r < a.ldo) {
            const u32x2 v = {(uint32_t)tile[rq][cc] | ((uint32_t)tile[rq + 1][cc] << 16),
                             (uint32_t)tile[rq + 2][cc] | ((uint32_t)tile[rq + 3][cc] << 16)};
            *(u32x2 *)(out + (size_t)c * a.ldo + r) = v;
        }
    }
}

// Q[p][rho][:] = q row of (token rho / G, query head p G + rho % G).
__global__ __launch_bounds__(256) void gather_q(GatherParams a) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;       // one 16-byte piece
    const int pieces = a.d / 8;
    const int Rs = a.Rpad > 0 ? a.Rpad : a.Rp;
    const long n = (long)a.Hkv * Rs * pieces;
    if (i >= n) return;
    const int pc = (int)(i % pieces);
    const long pr = i / pieces;
    const int rho = (int)(pr % Rs), p = (int)(pr / Rs);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (rho < a.Rp) v = *(const u32x4 *)(a.q + out_row(p, rho, a.Hkv, a.G, 0, a.Hq) * a.d + 8 * pc);
    *(u32x4 *)(a.Q + (size_t)pr * a.d + 8 * pc) = v;
}

// One wave per score row: hidden values, a, the score error and its gradient,
// and the score net's back-propagated pre-activation gradient.
template <int ACT>
__global__ __launch_bounds__(256) void score_rows(ScoreRowParams a) {
    const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= (long)a.Hkv * a.Rp) return;
    const int lane = threadIdx.x & 63;
    const int p = (int)(row / a.Rp), rho = (int)(row - (long)p * a.Rp);
    const float *z = a.Zs + (size_t)row * a.Hs;
    const uint16_t *ws2 = a.ws2 + (size_t)p * a.Hs;
    // lane l owns units 4 l .. 4 l + 3 of every 256 (Hs is a multiple of 32: whole
    // groups of four), loads issued four groups at a time
    float s = 0.f;
    for (int j0 = 4 * lane; j0 < a.Hs; j0 += 1024) {
        f32x4 zv[4];
        u32x2 wv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = j0 + 256 * u;
            if (j < a.Hs) {
                zv[u] = *(const f32x4 *)(z + j);
                wv[u] = *(const u32x2 *)(ws2 + j);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = j0 + 256 * u;
            if (j >= a.Hs) break;
            float y[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) y[r] = act_fn<ACT>(zv[u][r]);
            *(u32x2 *)(a.Ys + (size_t)row * a.Hs + j) = u32x2{pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3])};
            s = __builtin_fmaf(bf16lo(wv[u].x), y[0], s);
            s = __builtin_fmaf(bf16hi(wv[u].x), y[1], s);
            s = __builtin_fmaf(bf16lo(wv[u].y), y[2], s);
            s = __builtin_fmaf(bf16hi(wv[u].y), y[3], s);
        }
    }
    s = wave_sum(s);
    const size_t o = out_row(p, rho, a.Hkv, a.G, 0, a.Hq);
    const float e = a.bs2[p] + s - a.alpha[o];
    const float ga = a.coef * e;                   // 2 lambda_alpha e / R
    for (int j0 = 4 * lane; j0 < a.Hs; j0 += 1024) {
        f32x4 zv[4];
        u32x2 wv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = j0 + 256 * u;
            if (j < a.Hs) {
                zv[u] = *(const f32x4 *)(z + j);
                wv[u] = *(const u32x2 *)(ws2 + j);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = j0 + 256 * u;
            if (j >= a.Hs) break;
            const float g0 = ga * bf16lo(wv[u].x) * act_grad_fn<ACT>(zv[u][0]);
            const float g1 = ga * bf16hi(wv[u].x) * act_grad_fn<ACT>(zv[u][1]);
            const float g2 = ga * bf16lo(wv[u].y) * act_grad_fn<ACT>(zv[u][2]);
            const float g3 = ga * bf16hi(wv[u].y) * act_grad_fn<ACT>(zv[u][3]);
            *(u32x2 *)(a.dZs + (size_t)row * a.Hs + j) = u32x2{pack_bf16(g0, g1), pack_bf16(g2, g3)};
        }
    }
    if (lane == 0) {
        a.ga[row] = ga;
        a.err[row] = e * e;
    }
}

// The same with the row's pre-activations and score weights held in registers
// (Hs <= 256 * MAXG): Zs is read once instead of twice.  Lane l owns units
// 4 l .. 4 l + 3 of every 256; the sums run in the order of score_rows.
template <int ACT, int MAXG>
__global__ __launch_bounds__(256) void score_rows_reg(ScoreRowParams a) {
    const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= (long)a.Hkv * a.Rp) return;
    const int lane = threadIdx.x & 63;
    const int p = (int)(row / a.Rp), rho = (int)(row - (long)p * a.Rp);
    const float *z = a.Zs + (size_t)row * a.Hs;
    const uint16_t *ws2 = a.ws2 + (size_t)p * a.Hs;
    f32x4 zv[MAXG];
    u32x2 wv[MAXG];
#pragma unroll
    for (int u = 0; u < MAXG; ++u) {
        const int j = 4 * lane + 256 * u;
        if (j < a.Hs) {
            zv[u] = *(const f32x4 *)(z + j);
            wv[u] = *(const u32x2 *)(ws2 + j);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < MAXG; ++u) {
        const int j = 4 * lane + 256 * u;
        if (j >= a.Hs) break;
        float y[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = act_fn<ACT>(zv[u][r]);
        *(u32x2 *)(a.Ys + (size_t)row * a.Hs + j) = u32x2{pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3])};
        s = __builtin_fmaf(bf16lo(wv[u].x), y[0], s);
        s = __builtin_fmaf(bf16hi(wv[u].x), y[1], s);
        s = __builtin_fmaf(bf16lo(wv[u].y), y[2], s);
        s = __builtin_fmaf(bf16hi(wv[u].y), y[3], s);
    }
    s = wave_sum(s);
    const size_t o = out_row(p, rho, a.Hkv, a.G, 0, a.Hq);
    const float e = a.bs2[p] + s - a.alpha[o];
    const float ga = a.coef * e;                   // 2 lambda_alpha e / R
#pragma unroll
    for (int u = 0; u < MAXG; ++u) {
        const int j = 4 * lane + 256 * u;
        if (j >= a.Hs) break;
        const float g0 = ga * bf16lo(wv[u].x) * act_grad_fn<ACT>(zv[u][0]);
        const float g1 = ga * bf16hi(wv[u].x) * act_grad_fn<ACT>(zv[u][1]);
        const float g2 = ga * bf16lo(wv[u].y) * act_grad_fn<ACT>(zv[u][2]);
        const float g3 = ga * bf16hi(wv[u].y) * act_grad_fn<ACT>(zv[u][3]);
        *(u32x2 *)(a.dZs + (size_t)row * a.Hs + j) = u32x2{pack_bf16(g0, g1), pack_bf16(g2, g3)};
    }
    if (lane == 0) {
        a.ga[row] = ga;
        a.err[row] = e * e;
    }
}

// One wave per target row: e = A - A_target, ||e||^2 and gA = 2 lambda_A e / R (bf16).
template <int D>
__global__ __launch_bounds__(256) void target_rows(TargetRowParams a) {
    constexpr int NPL = D / 64;
    const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= (long)a.Hkv * a.Rp) return;
    const int lane = threadIdx.x & 63;
    const int p = (int)(row / a.Rp), rho = (int)(row - (long)p * a.Rp);
    const size_t o = out_row(p, rho, a.Hkv, a.G, 0, a.Hq);
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
        const int c = lane * NPL + k;
        const float e = a.A[(size_t)row * D + c] - a.Atgt[o * D + c];
        s = __builtin_fmaf(e, e, s);
        a.gA[(size_t)row * D + c] = f32_to_bf16(a.coef * e);
    }
    s = wave_sum(s);
    if (lane == 0) a.err[row] = s;
}

// out[p * so + j] = sum_k X[p][j][k] * (v ? v[p][k] : 1), one wave per (p, j),
// lane-strided partial sums then a fixed tree.
template <typename T>
__global__ __launch_bounds__(256) void row_dot(RowDotParams a) {
    const long idx = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (idx >= (long)a.P * a.J) return;
    const int lane = threadIdx.x & 63;
    const int p = (int)(idx / a.J), j = (int)(idx - (long)p * a.J);
    const T *x = (const T *)a.X + p * a.sx + (size_t)j * a.ldx;
    const float *v = a.v ? a.v + p * a.sv : nullptr;
    float s = 0.f;
    if (sizeof(T) == 2 && a.K % 8 == 0 && a.ldx % 8 == 0) {
        // eight bf16 per lane per iteration (16-byte loads)
        for (int k = 8 * lane; k < a.K; k += 512) {
            const u32x4 xv = *(const u32x4 *)((const uint16_t *)x + k);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float x0 = bf16lo(xv[u]), x1 = bf16hi(xv[u]);
                if (v) {
                    s = __builtin_fmaf(x0, v[k + 2 * u], s);
                    s = __builtin_fmaf(x1, v[k + 2 * u + 1], s);
                } else {
                    s += x0 + x1;
                }
            }
        }
    } else {
        for (int k = lane; k < a.K; k += 64) {
            const float xv = Elem<T>::ld(x, k);
            s = v ? __builtin_fmaf(xv, v[k], s) : s + xv;
        }
    }
    s = wave_sum(s);
    if (lane == 0) a.out[p * a.so + j] = s;
}

// Fixed-order fp64 sum of n floats (optionally squared) into parts[blockIdx.x].
__global__ __launch_bounds__(256) void sum_parts(SumParams a) {
    const long lo = a.n * blockIdx.x / gridDim.x, hi = a.n * (blockIdx.x + 1) / gridDim.x;
    double s = 0.0;
    for (long i = lo + threadIdx.x; i < hi; i += 256) {
        const double x = a.x[i];
        s += a.square ? x * x : x;
    }
    __shared__ double red[256];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) a.parts[a.part0 + blockIdx.x] = red[0];
}

// The loss and the clipping factor from the part sums (one thread).
// One wave: lane l sums parts l, l + 64, ... of each array in order, then a
// fixed butterfly folds the lanes (every lane ends with the same totals).
__global__ __launch_bounds__(64) void train_scalars(TrainScalars a) {
    const int lane = threadIdx.x;
    double s[3] = {0.0, 0.0, 0.0};
    for (int k = 0; k < 2; ++k)
        for (int b = lane; b < a.nparts; b += 64) s[k] += a.parts[k * a.nparts + b];
    if (a.scale)
        for (int b = lane; b < kNormParts; b += 64) s[2] += a.parts[2 * a.nparts + b];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
#pragma unroll
        for (int k = 0; k < 3; ++k) s[k] += __shfl_xor(s[k], o, 64);
    if (lane != 0) return;
    if (a.loss) {
        a.loss[1] = (float)(s[0] / a.R);
        a.loss[2] = (float)(s[1] / a.R);
        a.loss[0] = (float)(a.lam_alpha * (s[0] / a.R) + a.lam_A * (s[1] / a.R));
    }
    if (a.scale) {
        const double norm = sqrt(s[2]);
        a.scale[0] = (a.clip > 0.f && norm > 0.0) ? (float)fmin(1.0, a.clip / (norm + 1e-6)) : 1.0f;
        a.scale[1] = (float)norm;
        if (a.gnorm) {
            a.gnorm[0] = a.scale[0];
            a.gnorm[1] = a.scale[1];
        }
    }
}
__global__ __launch_bounds__(256) void adamw_kernel(AdamParams a) {
    const float scale = a.scale ? a.scale[0] : 1.0f;
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < a.n; i += (long)gridDim.x * 256) {
        const float gi = scale * a.g[i];
        float th = a.theta[i] * (1.0f - a.lr * a.wd);
        const float m = a.b1 * a.m[i] + (1.0f - a.b1) * gi;
        const float v = a.b2 * a.v[i] + (1.0f - a.b2) * gi * gi;
        a.m[i] = m;
        a.v[i] = v;
        th -= a.lr * (m * a.ic1) / (sqrtf(v * a.ic2) + a.eps);
        a.theta[i] = th;
        if (a.nseg > 0) {
            int k = 0;
            while (k + 1 < a.nseg && i >= a.off[k + 1]) ++k;
            const long j = i - a.off[k];
            if ((a.bf16 >> k) & 1) ((uint16_t *)a.dst[k])[j] = f32_to_bf16(th);
            else ((float *)a.dst[k])[j] = th;
        }
    }
}

// Module arrays from the fp32 master parameters: weights to bf16 (RNE), biases copied.
// ---------------------------------------------------------------------------

static unsigned grid_for(long n, long per_block, long cap) {
    long b = (n + per_block - 1) / per_block;
    if (b > cap) b = cap;
    return (unsigned)(b < 1 ? 1 : b);
}

long gemm_blocks(const GemmParams &g) {
    const long rg = (long)g.P * ((g.M + kBM - 1) / kBM);
    return (rg + kXcd - 1) / kXcd * kXcd * ((g.N + kBN - 1) / kBN);
}

hipError_t launch_gemm_nt(const GemmParams &g, hipStream_t st) {
    if (g.M <= 0 || g.N <= 0 || g.P <= 0) return hipSuccess;
    const dim3 grid((unsigned)(gemm_blocks(g) * (g.ksplit > 1 ? g.ksplit : 1))), block(64 * kWaves);
#define NECTAR_GEMM(E, A) hipLaunchKernelGGL((gemm_nt_lds32<E, A>), grid, block, 0, st, g)
    if (g.epi == 0) NECTAR_GEMM(0, 0);
    else if (g.epi == 1 && g.act == 1) NECTAR_GEMM(1, 1);
    else if (g.epi == 1 && g.act == 2) NECTAR_GEMM(1, 2);
    else if (g.epi == 1) NECTAR_GEMM(1, 0);
    else if (g.act == 1) NECTAR_GEMM(2, 1);
    else if (g.act == 2) NECTAR_GEMM(2, 2);
    else NECTAR_GEMM(2, 0);
#undef NECTAR_GEMM
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || g.ksplit <= 1) return e;
    hipLaunchKernelGGL(gemm_reduce, dim3(grid_for((long)g.P * g.M * (g.N / 4), 256, 8192)), dim3(256), 0, st, g);
    return hipGetLastError();
}

hipError_t launch_gemm_tn(const GemmParams &g, hipStream_t st) {
    if (g.M <= 0 || g.N <= 0 || g.P <= 0) return hipSuccess;
    if (g.M % 8 || g.N % 8 || g.ldx % 8 || g.ldw % 8 || g.K <= 0) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(gemm_blocks(g) * (g.ksplit > 1 ? g.ksplit : 1))), block(64 * kWaves);
    hipLaunchKernelGGL(gemm_tn_lds32, grid, block, 0, st, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || g.ksplit <= 1) return e;
    hipLaunchKernelGGL(gemm_reduce, dim3(grid_for((long)g.P * g.M * (g.N / 4), 256, 8192)), dim3(256), 0, st, g);
    return hipGetLastError();
}

hipError_t launch_col_sum(const ColSumParams &a, hipStream_t st) {
    if (a.P <= 0 || a.cols <= 0) return hipSuccess;
    if (a.cols % 4 || a.ldx % 4 || a.rows <= 0) return hipErrorInvalidValue;
    const long nch = (a.rows + 63) / 64, cq = a.cols / 4;
    hipLaunchKernelGGL(col_sum_parts, dim3(grid_for((long)a.P * nch * cq, 256, 1L << 30)), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(col_sum_final, dim3(grid_for((long)a.P * cq, 256, 1L << 30)), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_transpose_bf16(const TransposeParams &t, hipStream_t st) {
    const long blocks = (long)t.P * ((t.ldo + 63) / 64) * ((t.cols + 63) / 64);
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(transpose_bf16, dim3((unsigned)blocks), dim3(256), 0, st, t);
    return hipGetLastError();
}

hipError_t launch_gather_q(const GatherParams &a, hipStream_t st) {
    const long n = (long)a.Hkv * (a.Rpad > 0 ? a.Rpad : a.Rp) * (a.d / 8);
    hipLaunchKernelGGL(gather_q, dim3(grid_for(n, 256, 1L << 30)), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_score_rows(const ScoreRowParams &a, int act, hipStream_t st) {
    const dim3 grid(grid_for((long)a.Hkv * a.Rp, 4, 1L << 30)), block(256);
    if (a.Hs <= 256 * 16) {
        if (act == 1) hipLaunchKernelGGL((score_rows_reg<1, 16>), grid, block, 0, st, a);
        else if (act == 2) hipLaunchKernelGGL((score_rows_reg<2, 16>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((score_rows_reg<0, 16>), grid, block, 0, st, a);
        return hipGetLastError();
    }
    if (act == 1) hipLaunchKernelGGL(score_rows<1>, grid, block, 0, st, a);
    else if (act == 2) hipLaunchKernelGGL(score_rows<2>, grid, block, 0, st, a);
    else hipLaunchKernelGGL(score_rows<0>, grid, block, 0, st, a);
    return hipGetLastError();
}

hipError_t launch_target_rows(const TargetRowParams &a, int d, hipStream_t st) {
    const dim3 grid(grid_for((long)a.Hkv * a.Rp, 4, 1L << 30)), block(256);
    if (d == 128) hipLaunchKernelGGL(target_rows<128>, grid, block, 0, st, a);
    else if (d == 64) hipLaunchKernelGGL(target_rows<64>, grid, block, 0, st, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_row_dot(const RowDotParams &a, int fp32_in, hipStream_t st) {
    const dim3 grid(grid_for((long)a.P * a.J, 4, 1L << 30)), block(256);
    if (fp32_in) hipLaunchKernelGGL(row_dot<float>, grid, block, 0, st, a);
    else hipLaunchKernelGGL(row_dot<uint16_t>, grid, block, 0, st, a);
    return hipGetLastError();
}

hipError_t launch_sum_parts(const SumParams &a, int nparts, hipStream_t st) {
    hipLaunchKernelGGL(sum_parts, dim3(nparts), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_train_scalars(const TrainScalars &a, hipStream_t st) {
    hipLaunchKernelGGL(train_scalars, dim3(1), dim3(64), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_adamw(const AdamParams &a, hipStream_t st) {
    if (a.n <= 0) return hipSuccess;
    hipLaunchKernelGGL(adamw_kernel, dim3(grid_for(a.n, 256, 8192)), dim3(256), 0, st, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fused loss and backward (d = 128): the forward outputs come from the module's
// own forward kernels; the backward recomputes every pre-activation from the
// staged query rows instead of storing hidden-sized arrays.

// One wave per padded row: residuals, their squared norms, and the gradients
// the backward contracts (zero on padding rows).
__global__ __launch_bounds__(256) void loss_rows128(LossRowParams a) {
    const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= (long)a.Hkv * a.Rpad) return;
    const int lane = threadIdx.x & 63;
    const int p = (int)(row / a.Rpad), rho = (int)(row - (long)p * a.Rpad);
    uint32_t *gA = (uint32_t *)(a.gA + (size_t)row * 128);      // lane: dims 2 lane, 2 lane + 1
    if (rho >= a.Rp) {
        gA[lane] = 0u;
        if (lane == 0) a.ga[row] = 0.f;
        return;
    }
    const size_t o = out_row(p, rho, a.Hkv, a.G, 0, a.Hq);
    const float2 Av = *(const float2 *)(a.A + o * 128 + 2 * lane);
    const float2 Tv = *(const float2 *)(a.Atgt + o * 128 + 2 * lane);
    const float e0 = Av.x - Tv.x, e1 = Av.y - Tv.y;
    gA[lane] = pack_bf16(a.coefA * e0, a.coefA * e1);
    const float s = wave_sum(__builtin_fmaf(e1, e1, e0 * e0));
    if (lane == 0) {
        const long fr = (long)p * a.Rp + rho;
        const float es = a.a[o] - a.alpha[o];
        a.et[fr] = s;
        a.es[fr] = es * es;
        a.ga[row] = a.coefa * es;
    }
}

namespace {

constexpr int kBwdRows = 64;                  // query rows per stage (two halves of 32)
constexpr int kBwdWaves = 8;                  // 4 unit groups of 32 x 2 row halves
constexpr int kBwdUnits = 128;                // units per item

struct BwdStage {
    u32x4 q[kBwdRows * 16];     // query rows: piece j of row r at j ^ tr_swizzle(r)
    u32x4 g[kBwdRows * 16];     // read-out gradient rows (target items), same layout
};
// 160 KB: the item's first-layer rows, its read-out rows (target) or the
// stages' row gradients (score), and a three-stage ring of 64 query rows
struct BwdLds {
    u32x4 w1[kBwdUnits * 16];   // W1[u] (target) or Ws[u] (score): piece j at j ^ (u & 15)
    union {
        u32x4 w2[kBwdUnits * 16];   // W2t[u], same layout
        float ga[3][kBwdRows];
    } x;
    BwdStage st[3];
};
// the final fold of the two row halves reuses the LDS: four waves' 16 f32x4 per
// lane, then their two scalar sums per unit
static_assert(sizeof(BwdLds) >= 4 * 16 * 64 * 16 + (4 * 2 * 32 + 1) * 4, "fold space");
static_assert(sizeof(BwdLds) <= 160 * 1024, "LDS of one workgroup");

}  // namespace

// act(x) and act'(x) together.  Erf form: Phi by the polynomial of
// gelu_erf_poly (|Phi error| <= 5.2e-5, the module forward's own), phi(x) =
// exp(-x^2 / 2) / sqrt(2 pi), GELU' = Phi + x phi.
template <int ACT> __device__ __forceinline__ void act_pair(float x, float &y, float &dy) {
    if constexpr (ACT == 0) {
        const float c = __builtin_amdgcn_fmed3f(x, -3.71875f, 3.71875f);
        const float u = c * c;
        float p = __builtin_fmaf(u, 4.07418810e-08f, -2.44288435e-06f);
        p = __builtin_fmaf(p, u, 6.33929594e-05f);
        p = __builtin_fmaf(p, u, -9.51952359e-04f);
        p = __builtin_fmaf(p, u, 9.39021632e-03f);
        p = __builtin_fmaf(p, u, -6.58312142e-02f);
        p = __builtin_fmaf(p, u, 3.98723632e-01f);
        const float Phi = __builtin_fmaf(c, p, 0.5f);
        const float e = __builtin_amdgcn_exp2f(x * x * -0.72134752044448170f);   // exp(-x^2 / 2)
        y = x * Phi;
        dy = __builtin_fmaf(x * e, 0.3989422804014327f, Phi);
    } else {
        y = act_fn<ACT>(x);
        dy = act_grad_fn<ACT>(x);
    }
}

// One item: the 128 units [u0, u0 + 128) of group h, target (TGT) or score,
// over all the group's rows.  Wave w owns units u0 + 32 (w % 4) + 0..31 and the
// row half w / 4 of every 64-row stage (two waves per SIMD, one per half).
// Lane (n, half) = (lane % 32, lane / 32) holds unit n's first-layer weights as
// the B operand of the 32x32x16 MFMA and, per stage, computes on its 32 rows
//   Z (32 rows x 32 units) = Q . W^T + b               (A: query rows from LDS)
//   target: dH = gA . W2t^T, dZ = dH act'(Z), H = act(Z),
//           dW2t^T (128 x 32) += gA^T . H,  dW1^T += Q^T . dZ,  db1 += sum dZ
//   score:  dZ = ga ws2 act'(Z),  dWs^T += Q^T . dZ,  dbs += sum dZ,
//           dws2 += sum ga act(Z)
// The accumulator of Z holds unit n in every lane and rows 8 (i / 4) + 4 half
// + i % 4 in register i, so registers 8 t .. 8 t + 7 of H or dZ are the B
// operand of row step t as they stand, provided the transposed A operands
// (gA^T, Q^T: dims x rows) take their rows in that order: transposing LDS
// reads (ds_read_b64_tr_b16) of the row-major stage give it.  At the end the
// second half's sums are added to the first's through LDS (fixed order).
template <int ACT, bool TGT>
__device__ __forceinline__ void train_bwd_item(const TrainBwdParams &a, int h, int u0, BwdLds &L) {
    // the wave index as a scalar: the copies' LDS destinations stay in scalar registers
    const int t = threadIdx.x, w = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63, hf = lane >> 5, r = lane & 31;
    const int ug = w & 3, rh = w >> 2;
    const int H = TGT ? a.Ht : a.Hs;
    const bool live = u0 + 32 * ug < H;       // H is a multiple of 32: whole waves
    const int n = min(u0 + 32 * ug + r, H - 1);
    const size_t un = (size_t)h * H + n;

    const float bias = TGT ? a.b1[un] : a.bs[un];
    const float wsc = TGT ? 0.f : bf16_to_f32(a.ws2[un]);

    // transposing-read offsets in a 16-row block of a stage: lane 32 hf + m
    // receives dim 32 mi + m of rows 8 hh + 4 hf + 0..3
    uint32_t woff[2][4];
    {
        const int G = lane >> 4, aa = lane & 3, e = (lane >> 2) & 3;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                const int u = 8 * hh + 4 * (G >> 1) + e;
                const int piece = 4 * mi + 2 * (G & 1) + (aa >> 1);
                woff[hh][mi] = (uint32_t)(u * 256 + ((piece ^ tr_swizzle(u)) * 16) + (aa & 1) * 8);
            }
    }
    const int rr0 = 32 * rh + r;              // this lane's row (A operands) within a stage
    const int trs = tr_swizzle(rr0);
    const int wrow = 32 * ug + r;             // this lane's unit row of the staged weight rows

    f32x16 gX[4], gY[4];          // target: dW2t^T, dW1^T; score: dWs^T (gX unused)
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        gX[mi] = f32x16{};
        gY[mi] = f32x16{};
    }
    float db = 0.f, dw = 0.f, gs = 0.f;

    const uint16_t *Qh = a.Q + (size_t)h * a.Rpad * 128;
    const uint16_t *Gh = a.gA + (size_t)h * a.Rpad * 128;
    const float *gah = a.ga + (size_t)h * a.Rpad;
    const int nst = a.Rpad / kBwdRows;

    // the item's 128 first-layer rows (and read-out rows) once: four 1 KB
    // copies per wave and table
    auto stage_units = [&](const uint16_t *W, u32x4 *dst) {
        const int umax = H - 1 - u0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int r0 = 16 * w + 4 * c, uu = r0 + (lane >> 4);
            const size_t off = (size_t)min(uu, umax) * 128 + ((lane & 15) ^ (uu & 15)) * 8;
            __builtin_amdgcn_global_load_lds((const void *)(W + off), (lds_void *)&dst[r0 * 16], 16, 0, 0);
        }
    };
    stage_units((TGT ? a.W1 : a.Ws) + ((size_t)h * H + u0) * 128, L.w1);
    if constexpr (TGT) stage_units(a.W2t + ((size_t)h * H + u0) * 128, L.x.w2);
    // Stage i: rows 64 i .. 64 i + 63 into ring slot b; every wave copies 8 rows
    // of each table (two 1 KB copies per table), score items' wave 0 also the
    // 64 gradients.
    auto issue = [&](int i, int b) {
        const int row0 = kBwdRows * i;
        BwdStage &dst = L.st[b];
        int lv = lane;                        // addresses formed here, not held across the loop
        asm volatile("" : "+v"(lv));
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int r0 = 8 * w + 4 * c, rr = r0 + (lv >> 4);
            const size_t off = (size_t)(row0 + rr) * 128 + ((lv & 15) ^ tr_swizzle(rr)) * 8;
            __builtin_amdgcn_global_load_lds((const void *)(Qh + off), (lds_void *)&dst.q[r0 * 16], 16, 0, 0);
            if constexpr (TGT)
                __builtin_amdgcn_global_load_lds((const void *)(Gh + off), (lds_void *)&dst.g[r0 * 16], 16, 0, 0);
        }
        if constexpr (!TGT) {
            if (w == 0 && lv < 16)
                __builtin_amdgcn_global_load_lds((const void *)(gah + row0 + 4 * lv), (lds_void *)L.x.ga[b], 16, 0, 0);
        }
    };

    auto compute = [&](int b) {
        const BwdStage &cur = L.st[b];
        // the operand offsets pass through an empty asm each stage, so the
        // compiler forms the per-read addresses at their use instead of
        // holding every (ring slot, step) combination in registers across
        // the loop
        int sq = trs, sw = wrow & 15;
        uint32_t wo[2][4];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) wo[hh][mi] = woff[hh][mi];
        asm volatile("" : "+v"(sq), "+v"(sw), "+v"(wo[0][0]), "+v"(wo[0][1]), "+v"(wo[0][2]), "+v"(wo[0][3]),
                     "+v"(wo[1][0]), "+v"(wo[1][1]), "+v"(wo[1][2]), "+v"(wo[1][3]));
        f32x16 Z, dH;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            Z[i] = bias;
            dH[i] = 0.f;
        }
        // operands one contraction step ahead of their products; the scheduling
        // barriers keep the compiler from hoisting every operand read of the
        // stage (two waves per SIMD leave 256 registers a wave)
        auto ops = [&](int kt, u32x4 (&o)[4]) {
            const int pos = rr0 * 16 + ((2 * kt + hf) ^ sq);
            const int wpos = wrow * 16 + ((2 * kt + hf) ^ sw);
            o[0] = cur.q[pos];
            o[1] = L.w1[wpos];
            if constexpr (TGT) {
                o[2] = cur.g[pos];
                o[3] = L.x.w2[wpos];
            }
        };
        u32x4 op[3][4];
        ops(0, op[0]);
        ops(1, op[1]);
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) {
            if (kt + 2 < 8) ops(kt + 2, op[(kt + 2) % 3]);
            Z = mfma32(op[kt % 3][0], op[kt % 3][1], Z);
            if constexpr (TGT) dH = mfma32(op[kt % 3][2], op[kt % 3][3], dH);
            __builtin_amdgcn_sched_barrier(0);
        }
        float hv[16], dz[16];
        if constexpr (TGT) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float y, dy;
                act_pair<ACT>(Z[i], y, dy);
                hv[i] = y;
                dz[i] = dH[i] * dy;
                db += dz[i];
            }
        } else {
            float gr[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 g4 = *(const f32x4 *)&L.x.ga[b][32 * rh + 8 * q + 4 * hf];
#pragma unroll
                for (int j = 0; j < 4; ++j) gr[4 * q + j] = g4[j];
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float y, dy;
                act_pair<ACT>(Z[i], y, dy);
                dw = __builtin_fmaf(gr[i], y, dw);
                dz[i] = gr[i] * wsc * dy;
                db += dz[i];
            }
            if (u0 == 0 && ug == 0) {
                // the group's sum of ga (the score output-bias gradient), fixed order
#pragma unroll
                for (int i = 0; i < 16; ++i) gs += gr[i];
            }
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const u32x4 Db = {pack_bf16(dz[8 * tt + 0], dz[8 * tt + 1]), pack_bf16(dz[8 * tt + 2], dz[8 * tt + 3]),
                              pack_bf16(dz[8 * tt + 4], dz[8 * tt + 5]), pack_bf16(dz[8 * tt + 6], dz[8 * tt + 7])};
            const char *qb = (const char *)cur.q + (32 * rh + 16 * tt) * 256;
            if constexpr (TGT) {
                const u32x4 Hb = {pack_bf16(hv[8 * tt + 0], hv[8 * tt + 1]), pack_bf16(hv[8 * tt + 2], hv[8 * tt + 3]),
                                  pack_bf16(hv[8 * tt + 4], hv[8 * tt + 5]), pack_bf16(hv[8 * tt + 6], hv[8 * tt + 7])};
                const char *gb = (const char *)cur.g + (32 * rh + 16 * tt) * 256;
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) {
                    const u32x2 g0 = lds_read_tr16(gb, wo[0][mi]), g1 = lds_read_tr16(gb, wo[1][mi]);
                    gX[mi] = mfma32(u32x4{g0.x, g0.y, g1.x, g1.y}, Hb, gX[mi]);
                }
            }
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                const u32x2 q0 = lds_read_tr16(qb, wo[0][mi]), q1 = lds_read_tr16(qb, wo[1][mi]);
                gY[mi] = mfma32(u32x4{q0.x, q0.y, q1.x, q1.y}, Db, gY[mi]);
            }
        }
    };

    // stage i has landed once at most the next stage's copies are pending (the
    // weight rows, issued first, have landed with stage 0)
    auto step = [&](int i, int b) {
        if (i + 1 < nst) {
            if constexpr (TGT) wait_vmcnt<4>();
            else {
                if (w == 0) wait_vmcnt<3>();
                else wait_vmcnt<2>();
            }
        } else {
            wait_vmcnt<0>();
        }
        stage_barrier();
        if (i + 2 < nst) issue(i + 2, (b + 2) % 3);
        if (live) compute(b);
    };
    if (nst > 0) issue(0, 0);
    if (nst > 1) issue(1, 1);
    for (int i = 0; i < nst; i += 3) {
        step(i, 0);
        if (i + 1 >= nst) break;
        step(i + 1, 1);
        if (i + 2 >= nst) break;
        step(i + 2, 2);
    }

    // unit n's sums: both lane halves, then the second row half's waves hand
    // theirs to the first's through LDS (every stage read is done after the
    // barrier), one accumulator array at a time
    db += __shfl_xor(db, 32, 64);
    dw += __shfl_xor(dw, 32, 64);
    f32x4 *fold = (f32x4 *)&L;                // [unit group][16 x f32x4][64 lanes]
    float *fs = (float *)&L + 4 * 64 * 64;    // [unit group][2][32]
    auto hand_over = [&](f32x16 (&acc)[4]) {
        __syncthreads();
        if (rh == 1) {
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    fold[(ug * 16 + 4 * mi + q) * 64 + lane] =
                        f32x4{acc[mi][4 * q], acc[mi][4 * q + 1], acc[mi][4 * q + 2], acc[mi][4 * q + 3]};
        }
        __syncthreads();
        if (rh == 0) {
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 o = fold[(ug * 16 + 4 * mi + q) * 64 + lane];
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[mi][4 * q + j] += o[j];
                }
        }
    };
    hand_over(gY);
    if constexpr (TGT) hand_over(gX);
    // ga sums: the lanes of one half hold the same 16 rows of each stage
    gs += __shfl_xor(gs, 32, 64);
    if (rh == 1 && hf == 0) {
        fs[(ug * 2 + 0) * 32 + r] = db;
        fs[(ug * 2 + 1) * 32 + r] = dw;
        if (ug == 0 && r == 0) fs[8 * 32] = gs;
    }
    __syncthreads();
    if (rh == 1 || !live) return;
    db += fs[(ug * 2 + 0) * 32 + r];
    dw += fs[(ug * 2 + 1) * 32 + r];
    if constexpr (!TGT) {
        if (u0 == 0 && ug == 0 && lane == 0) a.gbs2[h] = gs + fs[8 * 32];
    }

    // register i of block mi is dim 32 mi + 8 (i / 4) + 4 hf + i % 4
    float *gy = (TGT ? a.gW1 : a.gWs) + un * 128;
    float *gx = a.gW2t + un * 128;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int dc = 32 * mi + 8 * q + 4 * hf;
            *(f32x4 *)(gy + dc) = f32x4{gY[mi][4 * q], gY[mi][4 * q + 1], gY[mi][4 * q + 2], gY[mi][4 * q + 3]};
            if constexpr (TGT)
                *(f32x4 *)(gx + dc) = f32x4{gX[mi][4 * q], gX[mi][4 * q + 1], gX[mi][4 * q + 2], gX[mi][4 * q + 3]};
        }
    if (hf == 0) {
        if constexpr (TGT) {
            a.gb1[un] = db;
        } else {
            a.gbs[un] = db;
            a.gws2[un] = dw;
        }
    }
}

// Items (group, role, unit block) in group-major order, a contiguous range per
// XCD (block ids go round-robin over the eight), so each XCD's L2 holds few
// groups' staged rows.
template <int ACT>
__global__ __launch_bounds__(64 * kBwdWaves, 1) void train_bwd_lds32(TrainBwdParams a) {
    __shared__ BwdLds L;
    const int per = (a.items + 7) / 8;
    const int item = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    if (item >= a.items) return;
    const int ipg = a.nut + a.nus;
    const int h = item / ipg, ri = item - h * ipg;
    if (ri < a.nut) train_bwd_item<ACT, true>(a, h, kBwdUnits * ri, L);
    else train_bwd_item<ACT, false>(a, h, kBwdUnits * (ri - a.nut), L);
}

hipError_t launch_loss_rows(const LossRowParams &a, hipStream_t st) {
    const long rows = (long)a.Hkv * a.Rpad;
    if (rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(loss_rows128, dim3(grid_for(rows, 4, 1L << 30)), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_train_bwd(const TrainBwdParams &a, int act, hipStream_t st) {
    if (a.items <= 0) return hipSuccess;
    if (a.Rpad % kBwdRows || a.Ht % 32 || a.Hs % 32) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(8 * ((a.items + 7) / 8))), block(64 * kBwdWaves);
    if (act == 1) hipLaunchKernelGGL(train_bwd_lds32<1>, grid, block, 0, st, a);
    else if (act == 2) hipLaunchKernelGGL(train_bwd_lds32<2>, grid, block, 0, st, a);
    else hipLaunchKernelGGL(train_bwd_lds32<0>, grid, block, 0, st, a);
    return hipGetLastError();
}

}  // namespace nectar
