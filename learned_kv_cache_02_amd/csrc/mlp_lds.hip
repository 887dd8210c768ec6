// Nectar MLP module forward for many query rows (batched decode and prefill):
// the one-hidden-layer score/target networks of Eq. (3.6) of the Nectar notes,
//   target A = sum_j W2t[h][j] * act(W1[h][j] . q + b1[h][j]) + b2[h]
//   score  a = sum_j ws2[h][j] * act(Ws[h][j] . q + bs[h][j]) + bs2[h],
// on the 32x32x16 MFMA with the weights staged through LDS by direct copies.
//
// A block of eight waves (two per SIMD) owns 256 query rows of one KV head, 32
// per wave, and one range of hidden units; the units stream through a
// three-stage LDS ring of 64-unit stages (first-layer rows, read-out rows,
// biases and score weights), copied HBM -> LDS two stages ahead with every
// 256-byte row's 16-byte pieces XOR-swizzled by the unit (first-layer rows:
// by unit & 15; read-out rows: by tr_swizzle), so the operand reads are
// conflict-free.  Per 32-unit chunk a wave runs
//   Z^T (32 units x 32 rows) = b + sum over 8 slices of 16 dims of W1 . Q^T
//       (the bias is the accumulator's initial value),
//   H = act(Z), and for target chunks O^T (128 x 32) += W2t^T . H^T as
//       4 dim blocks x 2 unit groups: H's accumulator registers 8t .. 8t + 7
//       are the B operand of unit group t as they stand, and the read-out
//       operand, in the same unit order, comes from the unit-major read-out
//       stage by transposing LDS reads (ds_read_b64_tr_b16);
//   for score chunks, a dot of H with ws2 in fp32.
// The erf-form GELU is evaluated as x * (0.5 + c P(c^2)), c = x clamped to
// [-3.71875, 3.71875], P of degree 6 (gelu_erf_poly).  (The bias as a ninth
// product of the chain instead of the accumulator's start -- sixteen vector
// moves fewer per chunk -- measured 3.6 % slower: the longer dependent chain
// delays the activations.)
// The unit counts of both nets must be multiples of 64 (every workload's are;
// other widths use mlp_prefill.hip).
#include "lds_common.hpp"
#include "kernels.hpp"

namespace nectar {

namespace {

constexpr int kD = 128, kNW = 8, kThreads = 64 * kNW, kRows = 32 * kNW, kSU = 64, kPieces = 16;
constexpr int kStages = 3;

struct UnitStage {
    u32x4 w1[kSU * kPieces];      // first-layer (or score first-layer) rows
    u32x4 w2[kSU * kPieces];      // read-out rows (target stages)
    float b[kSU];                 // b1 or bs
    uint16_t ws2[kSU];            // score read-out weights (score stages)
};

}  // namespace

template <int ACT>
__global__ __launch_bounds__(kThreads, 1) void mlp_rows_lds32(MlpParams a) {
    // separate variables, so the compiler tells copies into one stage from reads of another
    __shared__ UnitStage st_a, st_b, st_c;

    const int t = threadIdx.x, w = t >> 6, lane = t & 63, hf = lane >> 5, r = lane & 31;
    const int nrb = (a.Rp + kRows - 1) / kRows;
    const int sb = blockIdx.x % a.SB, hr = blockIdx.x / a.SB;
    const int h = hr / nrb, rb = hr - h * nrb;

    auto act = [&](float x) { return ACT == 0 ? gelu_erf_poly(x) : act_fn<ACT>(x); };

    const int rho = rb * kRows + w * 32 + r;
    u32x4 qv[8];
    if (rho < a.Rp) {
        const int tk = rho / a.G, gg = rho - tk * a.G;
        const uint16_t *qp = (const uint16_t *)a.q + ((size_t)tk * a.Hq + h * a.G + gg) * kD;
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) qv[kt] = *(const u32x4 *)(qp + 16 * kt + 8 * hf);
    } else {
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) qv[kt] = u32x4{0u, 0u, 0u, 0u};
    }

    const uint16_t *W1 = (const uint16_t *)a.W1 + (size_t)h * a.Ht * kD;
    const uint16_t *W2t = (const uint16_t *)a.W2t + (size_t)h * a.Ht * kD;
    const float *b1 = a.b1 + (size_t)h * a.Ht;
    const uint16_t *Ws = (const uint16_t *)a.Ws + (size_t)h * a.Hs * kD;
    const uint16_t *ws2 = (const uint16_t *)a.ws2 + (size_t)h * a.Hs;
    const float *bs = a.bs + (size_t)h * a.Hs;
    // this split's stages: target stages [t0, t0 + ntg), then score stages [s0, s0 + nsc)
    const int ttot = a.Ht / kSU, stot = a.Hs / kSU;
    const int cts = a.chunk_t / kSU, css = a.chunk_s / kSU;
    const int t0 = min(sb * cts, ttot), s0 = min(sb * css, stot);
    const int ntg = min(cts, ttot - t0), nst = ntg + min(css, stot - s0);

    // Stage i: every wave copies 8 rows of each row table (two 1 KB copies
    // each; score stages copy their first-layer rows twice so every wave issues
    // the same count), wave 0 also the biases and score weights.
    auto issue = [&](int i, UnitStage &dst) {
        const bool tgt = i < ntg;
        const int u0 = kSU * (tgt ? t0 + i : s0 + i - ntg);
        const uint16_t *Wa = tgt ? W1 : Ws;
        const uint16_t *Wb = tgt ? W2t : Ws;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int r0 = 8 * w + 4 * c, rr = r0 + (lane >> 4);
            // first-layer rows swizzled by the unit (16-byte reads), read-out rows
            // by tr_swizzle (transposing reads)
            const size_t row = (size_t)(u0 + rr) * kD;
            const int piece1 = (lane & 15) ^ (rr & 15), piece2 = (lane & 15) ^ tr_swizzle(rr);
            __builtin_amdgcn_global_load_lds((const void *)(Wa + row + piece1 * 8), (lds_void *)&dst.w1[r0 * kPieces], 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void *)(Wb + row + piece2 * 8), (lds_void *)&dst.w2[r0 * kPieces], 16, 0, 0);
        }
        if (w == 0) {
            // 64 biases = 16 pieces, 64 score weights = 8 pieces (score stages)
            const float *bp = (tgt ? b1 : bs) + u0;
            if (lane < 16)
                __builtin_amdgcn_global_load_lds((const void *)(bp + 4 * lane), (lds_void *)dst.b, 16, 0, 0);
            // target stages copy any valid 128 bytes (unused), so wave 0 always issues 6 copies
            const void *sp = (!tgt) ? (const void *)(ws2 + u0 + 8 * lane)
                                    : (a.Hs > 0 ? (const void *)(ws2 + 8 * lane) : (const void *)(bp + 4 * lane));
            if (lane < 8) __builtin_amdgcn_global_load_lds(sp, (lds_void *)dst.ws2, 16, 0, 0);
        }
    };

    // Byte offsets, within a 16-unit block of a read-out stage, of the 8-byte
    // slot this lane names for the transposing read of unit half `hh` and dim
    // block mi: unit 8 hh + 4 (lane / 32) + (lane / 4) % 4, dims 32 mi + 16
    // ((lane / 16) % 2) + 4 (lane % 4) .. + 3.  Lane 32 h + m then receives dim
    // 32 mi + m of units 8 hh + 4 h + 0..3, the contraction order of H^T.
    uint32_t woff[2][4];
    {
        const int G = lane >> 4, aa = lane & 3, e = (lane >> 2) & 3;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                const int u = 8 * hh + 4 * (G >> 1) + e;
                const int piece = 4 * mi + 2 * (G & 1) + (aa >> 1);
                woff[hh][mi] = (uint32_t)(u * kPieces * 16 + ((piece ^ tr_swizzle(u)) * 16) + (aa & 1) * 8);
            }
    }

    f32x16 O[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) O[mi] = f32x16{};
    float sc = 0.f;

    // Chunk c of a stage: Z^T = b + W1 . Q^T (the bias as the accumulator's start) ...
    auto preact = [&](const UnitStage &cur, int c) {
        f32x16 Z;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            // bias of the lane's 16 units 32c + 8q + 4hf + (0..3)
            const f32x4 bq = *(const f32x4 *)&cur.b[32 * c + 8 * q + 4 * hf];
#pragma unroll
            for (int j = 0; j < 4; ++j) Z[4 * q + j] = bq[j];
        }
        const int ur = 32 * c + r;
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) Z = mfma32(cur.w1[ur * kPieces + ((2 * kt + hf) ^ (ur & 15))], qv[kt], Z);
        return Z;
    };
    // ... then H = act(Z) and its read-out
    auto readout = [&](const UnitStage &cur, bool tgt, int c, const f32x16 &Z) {
        float hv[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) hv[j] = act(Z[j]);
        if (tgt) {
#pragma unroll
            for (int tg = 0; tg < 2; ++tg) {
                const u32x4 H = {pack_bf16(hv[8 * tg + 0], hv[8 * tg + 1]), pack_bf16(hv[8 * tg + 2], hv[8 * tg + 3]),
                                 pack_bf16(hv[8 * tg + 4], hv[8 * tg + 5]), pack_bf16(hv[8 * tg + 6], hv[8 * tg + 7])};
                // W2^T operand of dim block mi, straight from LDS by transposing reads
                const char *ublk = (const char *)cur.w2 + (32 * c + 16 * tg) * (kPieces * 16);
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) {
                    const u32x2 h0 = lds_read_tr16(ublk, woff[0][mi]), h1 = lds_read_tr16(ublk, woff[1][mi]);
                    O[mi] = mfma32(u32x4{h0.x, h0.y, h1.x, h1.y}, H, O[mi]);
                }
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint2 wq = *(const uint2 *)&cur.ws2[32 * c + 8 * q + 4 * hf];
                sc = __builtin_fmaf(bf16lo(wq.x), hv[4 * q + 0], sc);
                sc = __builtin_fmaf(bf16hi(wq.x), hv[4 * q + 1], sc);
                sc = __builtin_fmaf(bf16lo(wq.y), hv[4 * q + 2], sc);
                sc = __builtin_fmaf(bf16hi(wq.y), hv[4 * q + 3], sc);
            }
        }
    };
    // The two waves of a SIMD (w and w + 4) take a stage's chunks in different
    // orders -- the first half chunk by chunk, the second half both chunks'
    // first-layer products first -- so one wave's activations (vector work)
    // tend to meet the other's matrix products rather than both waves issuing
    // the same kind of work after every barrier (rho = 10 % prefill MLP: 3.11
    // -> 3.05 ms).  The sums run in the same order either way.
    const bool skew = w >= kNW / 2;

    auto step = [&](int i, const UnitStage &cur, UnitStage &ahead) {
        // stage i has landed once at most the next stage's copies are pending
        if (i + 1 < nst) {
            if (w == 0) wait_vmcnt<6>();
            else wait_vmcnt<4>();
        } else {
            wait_vmcnt<0>();
        }
        stage_barrier();
        if (i + 2 < nst) issue(i + 2, ahead);
        const bool tgt = i < ntg;
        if (skew) {
            const f32x16 Z0 = preact(cur, 0), Z1 = preact(cur, 1);
            readout(cur, tgt, 0, Z0);
            readout(cur, tgt, 1, Z1);
        } else {
            readout(cur, tgt, 0, preact(cur, 0));
            readout(cur, tgt, 1, preact(cur, 1));
        }
    };
    if (nst > 0) issue(0, st_a);
    if (nst > 1) issue(1, st_b);
    for (int i = 0; i < nst; i += kStages) {
        step(i, st_a, st_c);
        if (i + 1 >= nst) break;
        step(i + 1, st_b, st_a);
        if (i + 2 >= nst) break;
        step(i + 2, st_c, st_b);
    }
    sc += __shfl_xor(sc, 32, 64);
    if (rho >= a.Rp) return;

    // registers 4q .. 4q + 3 of block mi hold dims 32 mi + 8 q + 4 hf + 0..3
    if (a.SB > 1 || a.defer) {
        const size_t row = (size_t)(h * a.SB + sb) * a.Rp + rho;
        if (hf == 0) a.part_s[row] = sc;
        float *op = a.part_O + row * kD;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int mi = i >> 2, q = i & 3;
            *(f32x4 *)(op + 32 * mi + 8 * q + 4 * hf) = f32x4{O[mi][4 * q], O[mi][4 * q + 1], O[mi][4 * q + 2], O[mi][4 * q + 3]};
        }
        return;
    }
    const int tk = rho / a.G, gg = rho - tk * a.G;
    const size_t o = (size_t)tk * a.Hq + h * a.G + gg;
    if (hf == 0) a.a_out[o] = a.bs2[h] + sc;
    const float *b2 = a.b2 + (size_t)h * kD;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int mi = i >> 2, q = i & 3;
        const int dc = 32 * mi + 8 * q + 4 * hf;
        const f32x4 bb = *(const f32x4 *)(b2 + dc);
        *(f32x4 *)(a.A_out + o * kD + dc) = bb + f32x4{O[mi][4 * q], O[mi][4 * q + 1], O[mi][4 * q + 2], O[mi][4 * q + 3]};
    }
}

hipError_t launch_mlp_rows_lds32(const MlpParams &p, hipStream_t st) {
    const long nrb = (p.Rp + kRows - 1) / kRows;
    dim3 grid((unsigned)(p.Hkv * nrb * p.SB)), block(kThreads);
    if (p.act == 1) hipLaunchKernelGGL(mlp_rows_lds32<1>, grid, block, 0, st, p);
    else if (p.act == 2) hipLaunchKernelGGL(mlp_rows_lds32<2>, grid, block, 0, st, p);
    else hipLaunchKernelGGL(mlp_rows_lds32<0>, grid, block, 0, st, p);
    return hipGetLastError();
}

}  // namespace nectar
