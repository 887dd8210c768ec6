/*
 * nectar.h -- C ABI of the MI355X (gfx950) Nectar attention hot path.
 *
 * Nectar ("Nectar: Neural Estimation of Cached-Token Attention via
 * Regression"; reading notes at cc.laoqi.cc/papers/2605.09778/v2/r1) replaces,
 * per layer and KV head, softmax attention over a fixed document's cached keys
 * and values by two small networks of the RoPE'd query: a score net a(q) for
 * the document log-normalizer and a target net A(q) for the document-normalized
 * read-out.  Their pair is merged by log-sum-exp with exact causal attention
 * over the question's own tokens.  This library computes, on one GPU:
 *
 *   nectar_doc_attn_exact   exact (alpha, A) over the document cache, Eq. (3.1)
 *   nectar_doc_attn_partials / nectar_doc_attn_combine   the same as two passes
 *   nectar_module_forward   (a, A) from the MLP form (Eq. (3.6), one hidden
 *                           layer, or the deep re-injection form) or the
 *                           Quadrature KV-pair form (section 2.4)
 *   nectar_local_attn_lse   causal local attention (log Z_local, A_local),
 *                           section 2.2, optionally merged with a document pair
 *   nectar_merge            the log-sum-exp merge of Eqs. (3.4)-(3.5)
 *   nectar_merge_k          the same over K document-side pairs
 *   nectar_fit_metrics      squared errors and the RTE of a module against the
 *                           exact pair (Eqs. (3.2)-(3.3), (C.1))
 *   nectar_mlp_loss_grad / nectar_adamw_step / nectar_mlp_train_step
 *                           the module's regression training step (section 2.3)
 *   nectar_layer_step       all of the above for one layer step, fused
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are caller-owned DEVICE memory, contiguous, row-major
 *   (innermost index last), 16-byte aligned.  The library never allocates,
 *   frees or synchronizes; every call is asynchronous on `stream` (a
 *   hipStream_t; NULL = the null stream).  Outputs are complete when later work
 *   on that stream runs.  No global mutable state (the one exception is the
 *   device scratch of nectar_layer_step_static): calls are thread-safe;
 *   concurrent calls must use distinct workspaces.
 * - Query layout q[R][Hq][d] (token-major).  Query head h' reads KV head
 *   h = h' / (Hq / Hkv) (contiguous GQA groups; the group's query heads share
 *   K, V and the module, section 2.1).  Per-query outputs are [R][Hq] (scalars)
 *   and [R][Hq][d] (vectors).
 * - Element type of q, caches and module weights is desc->dtype (fp32 or bf16);
 *   biases are fp32; log-normalizers and read-outs are returned in fp32
 *   (section 3.2 of the notes caches its regression targets in fp32).
 *   Log-normalizers use the natural logarithm.
 * - Scores are s_j = scale * q.k_j with scale = desc->scale, or 1/sqrt(d) when
 *   desc->scale == 0 (Eq. (3.1)).
 * - Errors: every argument is checked on the host before any HIP call; a non-OK
 *   status is returned synchronously and nothing is launched.  NECTAR_EHIP
 *   reports a launch failure (hipGetLastError); faults inside kernels surface at
 *   the caller's next synchronization.  With NECTAR_SYNC_CHECK=1 in the
 *   environment each call synchronizes its stream and reports such faults as
 *   NECTAR_EHIP.  Outputs are undefined after a non-OK return.  NaN/Inf inputs
 *   are propagated, not checked.
 * - Workspaces: the *_workspace_size functions return the exact number of
 *   bytes (0 allowed) the matching call needs for the same arguments; they
 *   need no GPU.  The workspace is caller-owned device scratch: its contents
 *   need no initialisation and are undefined after a call.  Calls that may run
 *   concurrently (different streams) need distinct workspaces.
 */
#ifndef NECTAR_H
#define NECTAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NECTAR_ABI_VERSION 3

#if defined(__GNUC__) || defined(__clang__)
#define NECTAR_API __attribute__((visibility("default")))
#else
#define NECTAR_API
#endif

typedef enum {
    NECTAR_OK = 0,
    NECTAR_EINVAL = 1,        /* null pointer, bad shape, misalignment, bad enum */
    NECTAR_EUNSUPPORTED = 2,  /* well-formed but not implemented (d not 64/128, ...) */
    NECTAR_EWORKSPACE = 3,    /* ws_bytes smaller than the size query returns */
    NECTAR_EHIP = 4           /* HIP launch (or, with NECTAR_SYNC_CHECK, execution) error */
} nectar_status;

typedef enum { NECTAR_F32 = 0, NECTAR_BF16 = 1 } nectar_dtype;

/* Shape of the query side of one call. */
typedef struct {
    int32_t R;       /* query tokens (rows of q); R == 0 is a valid no-op */
    int32_t Hq;      /* query heads, > 0 */
    int32_t Hkv;     /* KV heads, > 0, Hq % Hkv == 0 */
    int32_t d;       /* head dimension: 64 or 128 */
    int32_t dtype;   /* nectar_dtype of q, caches and module weights */
    float scale;     /* score scale; 0 selects 1/sqrt(d) */
    int32_t splits;  /* 0: automatic; > 0: requested number of key (or hidden)
                        splits per head, clamped to [1, number of key tiles]
                        (64 keys per tile for bf16, 32 for fp32; 32 hidden units).
                        Results agree across split counts up to rounding. */
    int32_t kv_stride; /* document cache rows (the k, v arguments of the exact
                        document attention and of the layer step; not the local
                        cache, not module tensors): elements from one key's row
                        to the next's, the KV head's rows starting n of these
                        apart.  0 (or d): dense [Hkv][n][d] arrays.  2d with
                        v = k + d: K and V interleaved by key in one
                        [Hkv][n][2][d] array, which streams as one contiguous
                        range per key range.  Otherwise a multiple of 8, d or
                        more, at most 2^20; anything else is NECTAR_EINVAL. */
} nectar_attn_desc;

/* The local (question + generated tokens) cache of nectar_local_attn_lse. */
typedef struct {
    int32_t B;         /* questions; R == B * Tq */
    int32_t Tq;        /* query tokens per question in this call */
    int32_t T_loc;     /* valid local keys per (question, KV head), >= 0 */
    int32_t T_cap;     /* allocated rows per (question, KV head), >= T_loc */
    int32_t q_offset;  /* query token t of a question sees local keys
                          0 .. min(q_offset + t, T_loc - 1) (section 2.2: the
                          same causal set i <= t as full attention, including
                          the token itself).  Decode: Tq = 1, q_offset = T_loc - 1.
                          Prefill of the whole local chunk: Tq = T_loc, 0. */
} nectar_local_desc;

typedef enum { NECTAR_MODULE_MLP = 0, NECTAR_MODULE_KVPAIR = 1, NECTAR_MODULE_DEEP_MLP = 2 } nectar_module_kind;
typedef enum { NECTAR_ACT_GELU = 0, NECTAR_ACT_SILU = 1, NECTAR_ACT_GELU_TANH = 2 } nectar_act;

/*
 * A Nectar module for one layer: per KV head h (section 2.4 of the notes).
 *
 * MLP (Eq. (3.6) with one hidden layer, the workloads' depth):
 *   target  A(q) = sum_j W2t[h][j][:] * act(W1[h][j] . q + b1[h][j]) + b2[h]
 *   score   a(q) = sum_j ws2[h][j]   * act(Ws[h][j] . q + bs[h][j]) + bs2[h]
 *   W1, W2t [Hkv][Ht][d] (W2t[h][j] holds hidden unit j's outgoing weights),
 *   Ws [Hkv][Hs][d], ws2 [Hkv][Hs] (dtype); b1 [Hkv][Ht], b2 [Hkv][d],
 *   bs [Hkv][Hs], bs2 [Hkv] (fp32).  act: GELU(x) = x * Phi(x) (erf form),
 *   SiLU(x) = x * sigmoid(x) (the activation Eq. (3.6) names), or the tanh form
 *   of GELU, 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) (within 4.8e-4 of
 *   the erf form and about twice as fast on the batched-prefill kernel).
 *   Ht, Hs >= 0 (any value; 0 leaves the bias).
 * KVPAIR (Quadrature): exact attention over p learnable pairs,
 *   a(q) = log sum_j exp(scale * W[h][j] . q),  A(q) = softmax(scale * W q)^T Z,
 *   W, Z [Hkv][p][d] (dtype), p >= 0 (p == 0 gives a = -inf, A = 0).
 * DEEP_MLP: the deep form of Eq. (3.6), described by *deep (below).
 */
typedef struct nectar_deep_mlp nectar_deep_mlp;
typedef struct {
    int32_t kind;      /* nectar_module_kind */
    int32_t act;       /* nectar_act (MLP only) */
    int32_t Ht, Hs;    /* MLP hidden widths */
    const void *W1;  const float *b1;
    const void *W2t; const float *b2;
    const void *Ws;  const float *bs;
    const void *ws2; const float *bs2;
    int64_t p;         /* KVPAIR pair count */
    const void *W;   const void *Z;
    const nectar_deep_mlp *deep;   /* DEEP_MLP only */
} nectar_module;

/*
 * Deep MLP module with input re-injection, Eq. (3.6) (section 2.4): a network's
 * first layer reads the query, h_0 = act(U_0 q + b_0); each later layer reads
 * the query again beside the previous state, h_{k+1} = act(V_k q + U_k h_k + b_k).
 * The depth triple (D_b, D_s, D_t) of the notes: an optional shared backbone of
 * D_b layers of width H_b, then a score head of D_s layers (width H_s) and a
 * target head of D_t layers (width H_t).  A head's first layer reads the
 * backbone's last state when D_b > 0 (so it has the re-injection form) and only
 * the query otherwise.  Each head ends in a linear read-out of its last state
 * (the backbone's when the head has no layer):
 *   a = ws_out[h] . h_s + bs_out[h],   A[c] = Wt_out[h][c] . h_t + bt_out[h][c].
 * Layers are listed backbone first, then score, then target (l < D_b + D_s + D_t):
 *   Wq[l] [Hkv][H_l][d]     query weights (U_0, or V_k)            (dtype)
 *   Wh[l] [Hkv][H_l][H_in]  state weights U_k; NULL exactly when the layer
 *                           reads only the query                   (dtype)
 *   b[l]  [Hkv][H_l]        bias                                   (fp32)
 *   ws_out [Hkv][H_s last], Wt_out [Hkv][d][H_t last] (dtype); bs_out [Hkv],
 *   bt_out [Hkv][d] (fp32).
 * Constraints: D_b + D_s >= 1, D_b + D_t >= 1, D_b + D_s + D_t <=
 * NECTAR_DEEP_MAX_LAYERS; the width of every part with layers is a positive
 * multiple of 32 (NECTAR_EUNSUPPORTED otherwise).  On the bf16 path hidden
 * states are stored in bf16 (round to nearest even) between layers, as the
 * one-hidden-layer kernels round their hidden layer before the second product.
 * The workspace (nectar_module_workspace_size) holds the hidden states:
 * 2 * (H_b + H_s + H_t) * Hkv * R * (Hq / Hkv) elements of the storage type.
 */
#define NECTAR_DEEP_MAX_LAYERS 16
struct nectar_deep_mlp {
    int32_t depth[3];  /* D_b, D_s, D_t */
    int32_t width[3];  /* H_b, H_s, H_t (ignored for a part with no layer) */
    int32_t act;       /* nectar_act; NECTAR_ACT_SILU is the one Eq. (3.6) names */
    const void *Wq[NECTAR_DEEP_MAX_LAYERS];
    const void *Wh[NECTAR_DEEP_MAX_LAYERS];
    const float *b[NECTAR_DEEP_MAX_LAYERS];
    const void *ws_out; const float *bs_out;
    const void *Wt_out; const float *bt_out;
};

/*
 * Exact document attention, Eq. (3.1) with GQA sharing (section 2.1):
 *   alpha_out[r][h'] = log sum_{j<n} exp(s_j),  A_out[r][h'][:] = sum_j e^{s_j} v_j / sum_j e^{s_j}
 * over the document cache k, v [Hkv][n][d] (keys already RoPE'd).  Split-K over
 * the keys with a log-sum-exp combine (the regrouping of Eq. (3.4)); n == 0
 * gives alpha = -inf and A = 0.  The same call produces the fp32 regression
 * targets of section 2.3.
 */
NECTAR_API size_t nectar_doc_attn_workspace_size(const nectar_attn_desc *desc, int64_t n);
NECTAR_API nectar_status nectar_doc_attn_exact(const nectar_attn_desc *desc, int64_t n,
                                    const void *q, const void *k, const void *v,
                                    float *alpha_out, float *A_out,
                                    void *ws, size_t ws_bytes, void *stream);

/*
 * The same exact document attention as its two passes (the split-K partials
 * and their log-sum-exp combine, Eq. (3.4) regrouped), for callers that place
 * the passes themselves -- e.g. combining partials computed over several key
 * ranges.  partials: caller-owned device buffer of nectar_doc_attn_partials_size
 * bytes (16-byte aligned), written by the first call and read by the second
 * with the same desc and n; its layout is private to the library.
 * nectar_doc_attn_partials followed by nectar_doc_attn_combine writes the same
 * (alpha_out, A_out) as nectar_doc_attn_exact up to rounding (bitwise the same
 * whenever the plan splits the keys, i.e. whenever its workspace size is > 0).
 */
NECTAR_API size_t nectar_doc_attn_partials_size(const nectar_attn_desc *desc, int64_t n);
NECTAR_API nectar_status nectar_doc_attn_partials(const nectar_attn_desc *desc, int64_t n,
                                       const void *q, const void *k, const void *v,
                                       void *partials, size_t bytes, void *stream);
NECTAR_API nectar_status nectar_doc_attn_combine(const nectar_attn_desc *desc, int64_t n,
                                      const void *partials, size_t bytes,
                                      float *alpha_out, float *A_out, void *stream);

/* Module forward: (a_out [R][Hq], A_out [R][Hq][d]) for every query row. */
NECTAR_API size_t nectar_module_workspace_size(const nectar_attn_desc *desc, const nectar_module *m);
NECTAR_API nectar_status nectar_module_forward(const nectar_attn_desc *desc, const nectar_module *m,
                                    const void *q, float *a_out, float *A_out,
                                    void *ws, size_t ws_bytes, void *stream);

/*
 * Causal local attention (section 2.2): for query row r = b * Tq + t and query
 * head h', lse = log Z_local and A_local = N_local / Z_local over the visible
 * keys of k_loc, v_loc [B][Hkv][T_cap][d]; no visible key gives lse = -inf and
 * A_local = 0.
 * Outputs (each group optional, at least one requested):
 *   lse_out [R][Hq], A_out [R][Hq][d] (fp32): the local pair;
 *   out [R][Hq][d] (dtype) and out_lse [R][Hq] (fp32, may be NULL when out is
 *   given): the merge (Eqs. (3.4)-(3.5)) of the local part with the document
 *   pair doc_lse [R][Hq], doc_A [R][Hq][d] (fp32) -- exact (alpha, A) or a
 *   module's (a, A), the "virtual logit".  doc_lse/doc_A are required iff out
 *   or out_lse is given.
 */
NECTAR_API size_t nectar_local_workspace_size(const nectar_attn_desc *desc, const nectar_local_desc *loc);
NECTAR_API nectar_status nectar_local_attn_lse(const nectar_attn_desc *desc, const nectar_local_desc *loc,
                                    const void *q, const void *k_loc, const void *v_loc,
                                    float *lse_out, float *A_out,
                                    const float *doc_lse, const float *doc_A,
                                    void *out, float *out_lse,
                                    void *ws, size_t ws_bytes, void *stream);

/*
 * Log-sum-exp merge, Eqs. (3.4)-(3.5): per row (R * Hq rows),
 *   M = max(a, lam);  out = (e^{a-M} A + e^{lam-M} A_loc) / (e^{a-M} + e^{lam-M});
 *   lse_out = M + log(e^{a-M} + e^{lam-M});   a = lam = -inf gives out = 0, lse = -inf.
 * a, lam: [R][Hq] fp32; A, A_loc: [R][Hq][d] fp32; out [R][Hq][d] in desc->dtype;
 * lse_out nullable.
 */
NECTAR_API nectar_status nectar_merge(const nectar_attn_desc *desc, const float *a, const float *A,
                           const float *lam, const float *A_loc, void *out, float *lse_out,
                           void *stream);

/*
 * K-way log-sum-exp merge: the closing section of the Nectar notes proposes
 * composing several context modules (documents, or pieces of one) by one more
 * softmax grouping over their (score, target) pairs, the virtual-logit form of
 * Eqs. (3.4)-(3.5) with K virtual logits.  Per row (R * Hq rows), with M the
 * largest of a_0..a_{K-1} and lam:
 *   out = (sum_k e^{a_k-M} A_k + e^{lam-M} A_loc) / (sum_k e^{a_k-M} + e^{lam-M}),
 *   lse_out = M + log(sum_k e^{a_k-M} + e^{lam-M});
 * every logit -inf gives out = 0, lse_out = -inf.  When the pairs are exact
 * (alpha, A) over disjoint key ranges of one document, out is attention over
 * their union (with the local keys when the local pair is given).
 *   K          number of document-side pairs, 0..NECTAR_MERGE_K_MAX;
 *   a, A       host arrays of K device pointers: a[k] [R][Hq] fp32 logits,
 *              A[k] [R][Hq][d] fp32 read-outs; the host arrays are read during
 *              the call only;
 *   lam, A_loc the local pair ([R][Hq], [R][Hq][d] fp32), both or neither;
 *   out        [R][Hq][d] in desc->dtype; lse_out [R][Hq] fp32, nullable.
 * NECTAR_EINVAL for K out of range, lam without A_loc (or the reverse), no pair
 * at all, or a misaligned pointer.
 */
#define NECTAR_MERGE_K_MAX 8
NECTAR_API nectar_status nectar_merge_k(const nectar_attn_desc *desc, int K, const float *const *a,
                             const float *const *A, const float *lam, const float *A_loc,
                             void *out, float *lse_out, void *stream);

/*
 * Fit metrics of a module pair (a, A_theta) against the exact pair (alpha, A):
 * the squared errors whose sums over heads and tokens are the regression losses
 * of Eqs. (3.2)-(3.3) (section 2.3 of the notes), and the summand of the
 * relative target error of Eq. (C.1) (App. C.4), which measures the target
 * error against the error of using the query itself as the target.  Per row
 * (token r, query head h'):
 *   row_out[r][h'][0] = (a - alpha)^2
 *   row_out[r][h'][1] = ||A_theta - A||^2             (a sum over the d dimensions)
 *   row_out[r][h'][2] = log(||A_theta - A||^2 / ||q - A||^2)
 * (IEEE semantics: a zero target error gives -inf, q == A gives +inf).
 * head_out[h][k] (fp64, nullable) = the sum of row_out[.][.][k] over the rows of
 * KV head h (every token, every query head of its group), summed in a fixed
 * order; the score and target MSE of a layer are these sums over the heads
 * divided by the row count R * Hq, its RTE term is sum_h head_out[h][2] / (R * G).
 *   q [R][Hq][d] (desc->dtype); a, alpha [R][Hq], A, A_exact [R][Hq][d] (fp32);
 *   row_out [R][Hq][3] fp32: caller-owned, required (it also carries the
 *   per-row values to the head sums);
 *   ws: nectar_fit_metrics_workspace_size bytes (16-byte aligned) when head_out
 *   is given, else unused.
 */
NECTAR_API size_t nectar_fit_metrics_workspace_size(const nectar_attn_desc *desc);
NECTAR_API nectar_status nectar_fit_metrics(const nectar_attn_desc *desc, const void *q, const float *a,
                                 const float *A, const float *alpha, const float *A_exact,
                                 float *row_out, double *head_out, void *ws, size_t ws_bytes,
                                 void *stream);

/*
 * Regression training of the one-hidden-layer MLP module (section 2.3 of the
 * notes, Eqs. (3.2)-(3.3); App. A.2-A.5 for the optimizer).  Over the R query
 * tokens of one layer, with targets (alpha, A_target) from the exact document
 * attention (nectar_doc_attn_exact emits them in fp32, as the notes cache them):
 *   L_alpha = (1/R) sum_r sum_h' (a(q) - alpha)^2,
 *   L_A     = (1/R) sum_r sum_h' ||A(q) - A_target||^2,
 *   L       = lambda_alpha L_alpha + lambda_A L_A     ((0.1, 1) for the MLP).
 * The parameters are handled as one flat fp32 vector theta in the order
 *   W1 [Hkv][Ht][d], b1 [Hkv][Ht], W2t [Hkv][Ht][d], b2 [Hkv][d],
 *   Ws [Hkv][Hs][d], bs [Hkv][Hs], ws2 [Hkv][Hs], bs2 [Hkv]
 * (nectar_mlp_param_count elements); gradients use the same layout.
 * Supported: bf16 modules (desc->dtype == NECTAR_BF16), Ht and Hs positive
 * multiples of 32, R >= 1.  The products run on bf16 operands with fp32
 * accumulation (hidden values and back-propagated gradients rounded to bf16
 * between products, as in the forward kernels); reductions are fixed-order, so
 * a call is reproducible.
 *
 * nectar_mlp_loss_grad: grad (flat fp32) and loss[3] = (L, L_alpha, L_A) of the
 *   module m (its bf16 weights and fp32 biases) on q [R][Hq][d] (bf16), alpha
 *   [R][Hq], A_target [R][Hq][d] (fp32).
 * nectar_adamw_step: one AdamW step on n fp32 parameters (decoupled weight
 *   decay: theta *= 1 - lr wd; m = b1 m + (1 - b1) g; v = b2 v + (1 - b2) g^2;
 *   theta -= lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)).
 * nectar_mlp_train_step: the loss and gradient as above (grad is overwritten),
 *   the global gradient norm, clipping by min(1, clip_norm / (norm + 1e-6))
 *   when clip_norm > 0, the AdamW step on theta, adam_m, adam_v, and the
 *   module's own arrays rewritten from theta (weights rounded to bf16, biases
 *   copied) -- m's arrays are written although the struct declares them const.
 *   loss [3] and gnorm [2] = (clipping factor, norm before clipping) are
 *   optional fp32 device outputs.  theta must hold the module's current values
 *   (the caller initialises it and the moments, zero, once).
 * The learning-rate schedule (warm-up and cosine decay in the notes) is the
 * caller's: pass each step's lr in hp.
 */
typedef struct {
    float lambda_alpha, lambda_A;     /* loss weights */
    float lr, beta1, beta2, eps, weight_decay;
    float clip_norm;                  /* global gradient-norm clip; <= 0: none */
    int32_t step;                     /* Adam step t >= 1 */
} nectar_train_hparams;

NECTAR_API int64_t nectar_mlp_param_count(const nectar_attn_desc *desc, const nectar_module *m);
NECTAR_API size_t nectar_mlp_train_workspace_size(const nectar_attn_desc *desc, const nectar_module *m);
NECTAR_API nectar_status nectar_mlp_loss_grad(const nectar_attn_desc *desc, const nectar_module *m,
                                   const void *q, const float *alpha, const float *A_target,
                                   float lambda_alpha, float lambda_A, float *grad, float *loss,
                                   void *ws, size_t ws_bytes, void *stream);
NECTAR_API nectar_status nectar_adamw_step(int64_t n, float *theta, const float *grad, float *adam_m,
                                float *adam_v, const nectar_train_hparams *hp, void *stream);
NECTAR_API nectar_status nectar_mlp_train_step(const nectar_attn_desc *desc, const nectar_module *m,
                                    const void *q, const float *alpha, const float *A_target,
                                    const nectar_train_hparams *hp, float *theta, float *adam_m,
                                    float *adam_v, float *grad, float *loss, float *gnorm,
                                    void *ws, size_t ws_bytes, void *stream);

/*
 * One layer step of both paths, fused (sections 2.1-2.2; the step loop of a
 * decode or prefill pass).  For every query row it computes the local pair over
 * the causal local set (as nectar_local_attn_lse), the exact document pair
 * (alpha, A) over k, v [Hkv][n][d] (as nectar_doc_attn_exact) when any exact
 * output is requested, and the module pair (a, A) (as nectar_module_forward)
 * when `module` is given, and merges each document-side pair with the local
 * pair (Eqs. (3.4)-(3.5)).  On fp32, and on bf16 at decode shapes (at most 16
 * query rows per KV head, one-hidden-layer or KV-pair module), every part's
 * split partials come from one launch and one finishing launch folds them all
 * and writes every pair and merged output (two launches); otherwise (more rows,
 * or a deep module) each part runs its own kernels and the local pass merges
 * in place.
 * Outputs (all optional; NULL skips, at least one given):
 *   out_exact [R][Hq][d] (dtype), lse_exact [R][Hq]: exact path output;
 *   alpha_out, A_out: the exact document pair (the regression targets);
 *   out_nectar, lse_nectar: Nectar path output; a_out, Am_out: the module pair
 *   (given iff module != NULL);
 *   lam_out, Aloc_out: the local pair.
 * k, v may be NULL when n == 0 or no exact output is requested.  `exact` of the
 * size query says whether exact outputs will be requested.
 */
typedef struct {
    void *out_exact;  float *lse_exact;
    float *alpha_out; float *A_out;
    void *out_nectar; float *lse_nectar;
    float *a_out;     float *Am_out;
    float *lam_out;   float *Aloc_out;
} nectar_step_outputs;

NECTAR_API size_t nectar_layer_step_workspace_size(const nectar_attn_desc *desc, int64_t n,
                                                   const nectar_local_desc *loc, const nectar_module *module,
                                                   int exact);
NECTAR_API nectar_status nectar_layer_step(const nectar_attn_desc *desc, int64_t n, const nectar_local_desc *loc,
                                           const void *q, const void *k, const void *v, const void *k_loc,
                                           const void *v_loc, const nectar_module *module,
                                           const nectar_step_outputs *outs, void *ws, size_t ws_bytes,
                                           void *stream);

/*
 * nectar_layer_step without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Arguments, outputs and results are those
 * of nectar_layer_step (the same plan and kernels, so the same bits).  The
 * split partials go to a scratch array the library holds in device memory, one
 * copy per GPU it runs on, NECTAR_STATIC_SCRATCH_BYTES long, kept until the
 * process ends; its address is looked up on the first call on each device.
 * The call allocates nothing, and nothing in the scratch needs to start at zero.
 * Errors: NECTAR_EWORKSPACE (nothing launched) when the plan needs more scratch
 * than NECTAR_STATIC_SCRATCH_BYTES (nectar_layer_step_workspace_size gives the
 * need: every decode shape of the 4B, 8B and 1M-token layers fits; the
 * 16 x 1,024-token prefill does not); NECTAR_EHIP when the scratch address
 * cannot be obtained.  Every call on one GPU uses that GPU's one scratch array:
 * calls that may overlap on the same GPU (other streams, other threads) race,
 * and must be ordered by the caller.
 */
#define NECTAR_STATIC_SCRATCH_BYTES (64u << 20)
NECTAR_API nectar_status nectar_layer_step_static(const nectar_attn_desc *desc, int64_t n,
                                                  const nectar_local_desc *loc, const void *q, const void *k,
                                                  const void *v, const void *k_loc, const void *v_loc,
                                                  const nectar_module *module, const nectar_step_outputs *outs,
                                                  void *stream);

/* Zero-fills ws_bytes of device memory on `stream` with a fill kernel (no
 * memset node, so it can be captured in a graph); ws must be 16-byte aligned.
 * Workspaces need no initialisation; this is a convenience for callers that
 * want deterministic scratch contents. */
NECTAR_API nectar_status nectar_workspace_init(void *ws, size_t ws_bytes, void *stream);

NECTAR_API const char *nectar_status_string(nectar_status s);
NECTAR_API int nectar_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NECTAR_H */
