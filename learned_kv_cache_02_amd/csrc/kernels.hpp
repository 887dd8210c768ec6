// Internal launch interface between the C ABI (nectar_abi.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nectar {

// One batched attention problem set: problem p = b * Hkv + h attends query rows
// rho = t * G + g (query token b * Tq + t, query head h * G + g) over the keys
// 0 .. T_kv - 1 of the cache at k/v + b * kv_bstride + h * kv_hstride (elements,
// rows of d).  With causal != 0 row t only sees keys < q_offset + t + 1.
struct AttnParams {
    const void *q, *k, *v;
    int64_t kv_bstride, kv_hstride;
    int64_t kv_row;      // elements from one key's K (or V) row to the next's (d: dense rows)
    int Hq, G, Hkv, Tq, B, Rp, T_kv, causal, q_offset;
    float sl2;           // score scale * log2(e)
    // split plan: S key splits of `chunk` keys; RG row groups of 16*RT rows.
    // MFMA path: a block of 4 waves covers WR row groups x WS splits and folds
    // its WS splits together, leaving SB = ceil(S / WS) partials per row;
    // RB = ceil(RG / WR).  fp32 path: one wave per (row, split), SB = S.
    int P, S, chunk, RG, WR, WS, RB, SB;
    // > 0 (register-direct kernel): balanced splits, split s covering key tiles
    // [s * tiles / S, (s + 1) * tiles / S) of `chunk` keys each
    int tiles;
    int xcd_group;       // LDS-staged kernel: row blocks of a split share an XCD
    int defer;           // write partials even when SB == 1 (a later pass finishes)
    float *part_O;       // [P][SB][Rp][d]    unnormalised read-out
    float2 *part_ml;     // [P][SB][Rp]       (running max in log2 units, sum)
    // Row finishing in place when SB == 1 (same meaning as in CombineParams).
    float *lse_out, *A_out;
    const float *x_lse, *x_A;
    void *out;
    float *out_lse;
};

// Two problem sets served by one launch of the register-direct attention
// kernel (blocks [0, nb0) the first set); a single set repeats it.
struct AttnGroup {
    AttnParams p[2];
    int nb0;
};

// Finishing pass over the split partials of AttnParams: writes the pair
// (lse, A) and/or its merge with an extra (lse_x, A_x) pair.
// Split reductions (combine, MLP reduce): one wave per slice of a row, of
// reduce_cols(...) float4 columns -- 16 dims (the most waves: the decode shapes
// are latency-bound), 32 dims (whole 128-byte lines per split) for the plain
// sums of the MLP reduce past kReduceFewRows rows, or the whole row when
// slices would take more than kReduceSliceWaves waves.  Batch-64 decode
// (2,048 rows, 32 splits), 32-dim against 16-dim slices: MLP module forward
// 45.2 against 46.5 us, exact document pass with its combine 360.4 against
// 356.6 us, so only the MLP reduce takes the wider slices.
constexpr long kReduceSliceWaves = 65536;
constexpr long kReduceFewRows = 512;
inline int reduce_cols(long rows, int d, bool lines) {
    if (rows * (d / 16) <= kReduceSliceWaves && (!lines || rows <= kReduceFewRows)) return 4;
    if (lines && rows * (d / 32) <= kReduceSliceWaves) return 8;
    return d / 4;
}

struct CombineParams {
    const float *part_O;
    const float2 *part_ml;
    int Hq, G, Hkv, Tq, P, S, Rp;
    float *lse_out, *A_out;              // nullable
    const float *x_lse, *x_A;            // nullable (extra pair)
    void *out;                           // nullable, typed by dtype
    float *out_lse;                      // nullable
};

struct MlpParams {
    const void *q, *W1, *W2t, *Ws, *ws2;
    const float *b1, *bs, *b2, *bs2;
    int Hq, G, Hkv, Rp, Ht, Hs, act;
    // S hidden splits (chunk_t target units and chunk_s score units each);
    // blocks of WR row groups x WS splits as in AttnParams; SB partials per row.
    int S, chunk_t, chunk_s, RG, WR, WS, RB, SB;
    float *part_O;   // [Hkv][SB][Rp][d]
    float *part_s;   // [Hkv][SB][Rp]
    float *a_out, *A_out;   // written directly when SB == 1 and !defer
    int defer;              // write partials even when SB == 1 (a later pass finishes)
    // decode kernel (mlp_decode.hpp): per (KV head, row group) nwt target waves
    // and nws score waves, in SB blocks of four waves (RB == RG, WS == 4)
    int nwt, nws;
};

// Largest number of 32-unit target tiles a wave (tile slot) of the decode MLP
// kernel holds; a score slot holds up to dec_score_tiles(rt) score tiles (a
// score tile streams half the bytes of a target tile: twice as many with one
// 16-row tile, as many with more rows, where the activations dominate).
constexpr int kDecTiles = 2;
constexpr int dec_score_tiles(int rt) { return kDecTiles * (rt > 1 ? 1 : 2); }
// Waves per tile slot and tile slots per block of the decode MLP kernel: at
// d = 128 with four 16-row tiles (up to 64 rows per KV head) two waves share a
// slot's weight tiles in LDS and take 32 rows each, and a block holds
// NECTAR_DEC_SLOTS_PAIRED slots; otherwise one wave per slot and four slots.
// (Two paired slots per block -- 256 blocks at the 1M-token layer -- measured
// slower: twice the partials, and beside the local blocks a second round of
// blocks; 1M-token Nectar path 17.55 -> 23.4 us.)
// The paired kernel splits the output dims over the eight waves of four slots,
// so four is the only value it compiles with.
#ifndef NECTAR_DEC_SLOTS_PAIRED
#define NECTAR_DEC_SLOTS_PAIRED 4
#endif
constexpr int dec_wps(int d, int rt) { return d == 128 && rt == 4 ? 2 : 1; }
constexpr int dec_slots(int d, int rt) { return dec_wps(d, rt) > 1 ? NECTAR_DEC_SLOTS_PAIRED : 4; }
constexpr int dec_threads(int d, int rt) { return 64 * dec_slots(d, rt) * dec_wps(d, rt); }
// blocks per compute unit the paired kernels are compiled for (two waves per SIMD)
constexpr int dec_min_blocks(int d, int rt) { return dec_wps(d, rt) > 1 ? 8 / (dec_slots(d, rt) * dec_wps(d, rt)) : 1; }

// One layer of the deep MLP module (Eq. (3.6)) for every KV head p and row rho
// of its Rp = R * G query rows:
//   Y[p][rho][n] = act(Wq[p][n] . q_row(p, rho) + Wh[p][n] . X[p][rho] + b[p][n]).
// Wq == nullptr: the layer reads only the state (the linear read-outs);
// Wh == nullptr: it reads only the query.  The result goes to the hidden-state
// buffer Y ([Hkv][Rp][N], storage type) or, for a read-out, to the fp32 output
// rows Yf[out_row * N + n].
struct DeepLayer {
    const void *Wq, *Wh, *X;
    const float *b;
    void *Y;
    float *Yf;
    int N, Kh, act;          // act < 0: none
    long blocks;             // blocks of this layer in its launch
};

// One launch: one or two independent layers (the score and target heads run
// side by side).
struct DeepParams {
    const void *q;
    int Hq, G, Hkv, Rp, nl;
    DeepLayer L0, L1;
};

// Fit metrics: per row (R * Hq rows) the score squared error, the target
// squared error and the log RTE ratio, [rows][3]; per KV head their fp64 sums.
constexpr int kFitParts = 64;      // partial sums per KV head
struct FitParams {
    const void *q;
    const float *a, *A, *alpha, *Aex;
    float *row;
    double *head;      // nullable
    double *part;      // [Hkv][kFitParts][3] workspace when head != nullptr
    long rows;
    int Hq, Hkv;
};

// --- training step of the one-hidden-layer module ---
// C[p][m][n] = sum_k X[p][m][k] W[p][n][k] (+ bias[p * sb + n]); bf16 operands,
// fp32 result; K a multiple of 16, leading dimensions multiples of 8.
// Epilogues: 0 C = acc + bias (fp32); 1 Zo = bf16(acc + bias) and
// Y = bf16(act(acc + bias)); 2 Y = bf16(acc * act'(Zi)), Zi bf16 in C's layout.
// ksplit > 1 (epilogue 0 only): block ks sums K range ks and writes its partial
// tile to Cpart[ks][p][m][n]; gemm_reduce then forms C = sum_ks + bias.
struct GemmParams {
    const uint16_t *X, *W;
    const float *bias;       // nullable
    float *C;
    uint16_t *Zo, *Y;
    const uint16_t *Zi;
    float *Cpart;
    long sx, sw, sb, sc;     // per-batch strides (elements)
    int ldx, ldw, ldc;
    int M, N, K, P;
    int epi, act, ksplit, kchunk;
    // TN products only (nullable): xsum[p * sxs + m] = sum_k X[p][k][m], with
    // per-split partials in xsum_part [ksplit][P][M] when the contraction is split
    float *xsum, *xsum_part;
    long sxs;
};
// out[p][c][r] = in[p][r][c] for r < rows, zero for rows <= r < ldo.
struct TransposeParams {
    const uint16_t *in;
    uint16_t *out;
    long si, so;
    int rows, cols, ldi, ldo, P;
};
struct GatherParams {        // Q[p][rho][:] = q row of rho in KV group p; zero for Rp <= rho < Rpad
    const uint16_t *q;
    uint16_t *Q;
    int Hq, G, Hkv, Rp, d;
    int Rpad;                // rows per group in Q (0: Rp)
};
// Per query row of the fused training pass (d = 128): the loss residuals of the
// module's forward outputs and the gradients that the backward contracts, in
// row-padded group layout (rows Rp <= rho < Rpad zero).
struct LossRowParams {
    const float *a, *A;      // module forward [R][Hq], [R][Hq][d] (output biases included)
    const float *alpha, *Atgt;
    uint16_t *gA;            // [Hkv][Rpad][d] bf16: coefA (A - Atgt)
    float *ga;               // [Hkv][Rpad]: coefa (a - alpha)
    float *es, *et;          // [Hkv][Rp]: (a - alpha)^2, ||A - Atgt||^2
    float coefa, coefA;      // 2 lambda_alpha / R, 2 lambda_A / R
    int Hq, G, Hkv, Rp, Rpad;
};
// Fused backward of the one-hidden-layer module (d = 128): blocks of four waves
// own 128 target or score units of one KV group and run over all its rows,
// recomputing the pre-activations; the weight, bias and score read-out
// gradients of their units are written once, with no partial sums.
struct TrainBwdParams {
    const uint16_t *Q, *gA;  // [Hkv][Rpad][d] bf16 (padding rows zero)
    const float *ga;         // [Hkv][Rpad] (padding rows zero)
    const uint16_t *W1, *W2t, *Ws, *ws2;
    const float *b1, *bs;
    float *gW1, *gb1, *gW2t, *gWs, *gbs, *gws2;
    float *gbs2;             // [Hkv]: sum of ga (each group's first score item)
    int Hkv, Rpad, Ht, Hs;
    int nut, nus, items;     // target / score unit blocks per group, items = Hkv (nut + nus)
};
struct ScoreRowParams {
    const float *Zs;         // [Hkv][Rp][Hs] pre-activations (bias included)
    const uint16_t *ws2;     // [Hkv][Hs]
    const float *bs2, *alpha;
    uint16_t *Ys, *dZs;      // [Hkv][Rp][Hs] bf16
    float *ga, *err;         // [Hkv][Rp]
    float coef;              // 2 lambda_alpha / R
    int Hq, G, Hkv, Rp, Hs;
};
struct TargetRowParams {
    const float *A, *Atgt;   // [Hkv][Rp][d] (bias included), [R][Hq][d]
    uint16_t *gA;            // [Hkv][Rp][d]
    float *err;              // [Hkv][Rp]
    float coef;              // 2 lambda_A / R
    int Hq, G, Hkv, Rp;
};
struct RowDotParams {        // out[p * so + j] = sum_k X[p][j][k] * (v ? v[p][k] : 1)
    const void *X;
    const float *v;
    float *out;
    long sx, sv, so;
    int ldx, J, K, P;
};
struct ColSumParams {         // out[p * so + col] = sum_row X[p][row][col] * (v ? v[p][row] : 1)
    const uint16_t *X;
    const float *v;
    float *parts;            // [P][ceil(rows / 64)][cols] fixed-order partial sums
    float *out;
    long sx, sv, so;
    int ldx, rows, cols, P;
};
constexpr int kNormParts = 1024;   // blocks of the gradient-norm sum
struct SumParams {           // parts[part0 + b] = fixed-order fp64 sum of block b's range
    const float *x;
    double *parts;
    long n;
    int part0, square;
};
struct TrainScalars {
    const double *parts;     // [2][nparts] score and target errors, then [kNormParts] squared gradients
    int nparts;
    double R, lam_alpha, lam_A;
    float clip;
    float *loss;             // [3] or null
    float *scale;            // [2]: clipping factor, gradient norm; or null
    float *gnorm;            // caller's copy of scale (nullable)
};
struct AdamParams {
    float *theta, *m, *v;
    const float *g;
    const float *scale;      // device clipping factor or null
    long n;
    float lr, b1, b2, eps, wd, ic1, ic2;   // ic = 1 / (1 - beta^t)
    // optional copies of the updated theta: elements [off[k], off[k + 1]) to
    // dst[k] (bf16 where bit k of bf16 is set, else fp32); nseg = 0: none
    int nseg, bf16;
    long off[9];
    void *dst[8];
};
long gemm_blocks(const GemmParams &g);
hipError_t launch_gemm_nt(const GemmParams &g, hipStream_t st);
hipError_t launch_gemm_tn(const GemmParams &g, hipStream_t st);
hipError_t launch_col_sum(const ColSumParams &a, hipStream_t st);
hipError_t launch_transpose_bf16(const TransposeParams &t, hipStream_t st);
hipError_t launch_gather_q(const GatherParams &a, hipStream_t st);
hipError_t launch_score_rows(const ScoreRowParams &a, int act, hipStream_t st);
hipError_t launch_target_rows(const TargetRowParams &a, int d, hipStream_t st);
hipError_t launch_row_dot(const RowDotParams &a, int fp32_in, hipStream_t st);
hipError_t launch_loss_rows(const LossRowParams &a, hipStream_t st);
hipError_t launch_train_bwd(const TrainBwdParams &a, int act, hipStream_t st);
hipError_t launch_sum_parts(const SumParams &a, int nparts, hipStream_t st);
hipError_t launch_train_scalars(const TrainScalars &a, hipStream_t st);
hipError_t launch_adamw(const AdamParams &a, hipStream_t st);

// One document-side part of a layer step, finished together with the local
// part: split partials of the exact document attention or of a Quadrature
// module (log-sum-exp form: ml != NULL) or of an MLP module (plain sums:
// s != NULL, plus the output biases).  Rows are those of the document problems
// ([Hkv][S][R * G]).
struct FinishSet {
    const float *O;          // [Hkv][S][Rp_doc][d]
    const float2 *ml;        // [Hkv][S][Rp_doc] (max in log2 units, sum) or NULL
    const float *s;          // [Hkv][S][Rp_doc] score partials or NULL
    const float *b2, *bs2;   // MLP output biases (sum form)
    int S;
    float *lse_out, *A_out;  // the part's pair (nullable)
    void *out;               // merge with the local pair, typed by dtype (nullable)
    float *out_lse;          // (nullable)
};

// Finishing pass of a layer step: per local row, fold the local partials
// ([P][S_loc][Rp] over problems p = b * Hkv + h) and up to two document-side
// parts, write the pairs and the merged outputs.
struct FinishParams {
    const float *loc_O;
    const float2 *loc_ml;
    int S_loc;
    float *lam_out, *Aloc_out;   // local pair (nullable)
    FinishSet set[2];
    int nsets;
    int Hq, G, Hkv, Tq, P, Rp, Rp_doc;
};

struct MlpReduceParams {
    const float *part_O, *part_s, *b2, *bs2;
    int Hq, G, Hkv, Rp, S;
    float *a_out, *A_out;
};

struct MergeParams {
    const float *a, *A, *lam, *A_loc;
    void *out;
    float *lse_out;
    long rows;
};

// K-way merge: up to kMergeKMax document-side pairs and an optional local pair.
constexpr int kMergeKMax = 8;
struct MergeKParams {
    const float *a[kMergeKMax], *A[kMergeKMax];
    const float *lam, *A_loc;       // both null: no local pair
    void *out;
    float *lse_out;
    long rows;
    int K;
};

// Row tiling of the MFMA kernels: rows per wave = 16 * rt.
int row_tiles_for(int Rp);
// ... of the register-direct MLP kernel (up to 64 rows per wave).
int mlp_row_tiles(int Rp);

hipError_t launch_attn_partial(const AttnParams &p, int dtype, int d, int rt, hipStream_t st);
// LDS-staged attention for many rows per KV head (bf16, d = 128): NW waves of
// RT row tiles per block, 16 * NW * RT rows, keys staged SK at a time.
struct LdsShape {
    int NW, RT, SK;
    int BPC;   // blocks per compute unit the kernel of this shape is built for
};
// Blocks per compute unit of the LDS-staged kernel with kStageKeys-key stages:
// two with 32-key stages (48 KB of LDS each), else one.
constexpr int lds_blocks_per_cu(int stage_keys) { return stage_keys == 32 ? 2 : 1; }
LdsShape lds_shape_for(int Rp);
hipError_t launch_attn_rows_lds(const AttnParams &p, LdsShape sh, hipStream_t st);
// Two problem sets of the same shape in one launch (shape {4, 1, 96} only).
hipError_t launch_attn_rows_lds_pair(const AttnParams &p0, const AttnParams &p1, LdsShape sh, hipStream_t st);
// One launch for two bf16 problem sets of the register-direct kernel with the same
// head dimension and row tiling (independent blocks side by side).
hipError_t launch_attn_partial_pair(const AttnParams &p0, const AttnParams &p1, int d, int rt, hipStream_t st);
// One launch of register-direct bf16 attention blocks (one or two problem sets,
// row tiling 1) and MLP module blocks (row tiling 1, decode kernel).
hipError_t launch_step_partials(const AttnParams &p0, const AttnParams *p1, const MlpParams &m, int d, int mlp_rt,
                                hipStream_t st);
hipError_t launch_attn_combine(const CombineParams &p, int dtype, int d, hipStream_t st);
hipError_t launch_mlp_partial(const MlpParams &p, int dtype, int d, int rt, hipStream_t st);
hipError_t launch_mlp_reduce(const MlpReduceParams &p, int d, hipStream_t st);
// Decode-shape MLP (bf16, up to 16 * rt rows per wave): grid Hkv x RG x SB.
hipError_t launch_mlp_decode(const MlpParams &p, int d, int rt, hipStream_t st);
// MLP on the 32x32 MFMA with LDS-staged weights (bf16, d = 128, Ht and Hs
// multiples of 64); grid Hkv x ceil(Rp / 256) x SB, 64-unit split granularity.
hipError_t launch_mlp_rows_lds32(const MlpParams &p, hipStream_t st);
// Batched-prefill MLP (bf16, d = 128): one pass, no workspace.
hipError_t launch_mlp_prefill(const MlpParams &p, hipStream_t st);
hipError_t launch_merge(const MergeParams &p, int dtype, int d, hipStream_t st);
hipError_t launch_merge_k(const MergeKParams &p, int dtype, int d, hipStream_t st);
hipError_t launch_fit_metrics(const FitParams &p, int dtype, int d, hipStream_t st);
// Blocks of one deep-MLP layer for the launch shape of the given dtype (lds:
// the LDS-staged kernel for many rows per KV head).
long deep_layer_blocks(int dtype, int lds, int Hkv, int Rp, int N);
hipError_t launch_deep_layers(const DeepParams &p, int dtype, int d, int lds, hipStream_t st);
hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t st);
hipError_t launch_finish(const FinishParams &p, int dtype, int d, hipStream_t st);

}  // namespace nectar
