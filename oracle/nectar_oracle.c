/*
 * Nectar CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct fp64 implementation of what the Nectar
 * attention hot path computes.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library; the product path never
 * does.  It shares no code, header, table or helper with the HIP library.
 *
 * Source of every definition: the reading notes "Nectar: Neural Estimation of
 * Cached-Token Attention via Regression" (cc.laoqi.cc/papers/2605.09778/v2/r1),
 * section 2 ("method"):
 *   - section 2.1, Eq. (3.1): s_j = q.k_j / sqrt(d),
 *       alpha(q) = log sum_j exp(s_j),
 *       A(q)     = sum_j exp(s_j) v_j / sum_j exp(s_j);
 *     GQA: the query heads of one KV group share K, V and the module pair.
 *   - section 2.2, Eqs. (3.4)-(3.5): Z_local, N_local over the causally visible
 *     local tokens (index i <= t), and the log-sum-exp merge of the document
 *     pair with the local part (the "virtual logit").
 *   - section 2.4, Quadrature form: a = log sum_j exp((W q)_j / sqrt(d)),
 *     A = softmax(W q / sqrt(d))^T Z  -- exact attention over (W, Z, p).
 *   - section 2.4, Eq. (3.6): MLP form.  The workloads fix one hidden layer
 *     with GELU: A = W2 GELU(W1 q + b1) + b2, a = w2 . GELU(Ws q + bs) + bs2.
 *     SiLU is provided as the activation Eq. (3.6) itself names, and the tanh
 *     form of GELU as the common faster variant.  The deep form of Eq. (3.6)
 *     (the query re-injected into every layer, optional shared backbone) is
 *     oracle_deep_mlp.
 *   - closing section: several context modules composed by one more softmax
 *     grouping over their pairs (oracle_merge_k).
 *
 * Precision: every input element is widened exactly to double (bf16 bits are
 * shifted into an fp32 pattern; fp32 widens exactly); every sum is a plain
 * sequential double sum in index order.  The log-sum-exp is evaluated as
 * m + log(sum_j exp(s_j - m)) with m = max_j s_j, which is the same number as
 * log(sum_j exp(s_j)) in exact arithmetic and does not overflow.
 *
 * Parallelism: independent (token, query head) rows are spread over OpenMP
 * threads; each row is computed exactly as written, so the result does not
 * depend on the thread count.
 *
 * Layouts (row-major, innermost last):
 *   q      [R][Hq][d]             R = query tokens
 *   K, V   [Hkv][n][d]            document cache (keys already RoPE'd)
 *   Kl, Vl [B][Hkv][Tloc][d]      local cache per question
 *   W1, W2t[Hkv][Ht][d]           W2t[h][j][c] = weight from hidden j to output c
 *   Ws     [Hkv][Hs][d], ws2 [Hkv][Hs]
 *   b1 [Hkv][Ht], b2 [Hkv][d], bs [Hkv][Hs], bs2 [Hkv]  (double)
 *   query head hq reads KV head hq / (Hq / Hkv).
 */
#define _DEFAULT_SOURCE
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

enum { OR_F32 = 0, OR_BF16 = 1, OR_F64 = 2 };
enum { OR_GELU = 0, OR_SILU = 1, OR_GELU_TANH = 2 };

/* Read element i of an array of the given element type, widened to double. */
static double ld(const void *p, int dt, size_t i)
{
    if (dt == OR_F64) return ((const double *)p)[i];
    if (dt == OR_F32) return (double)((const float *)p)[i];
    uint32_t bits = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static int valid_dt(int dt) { return dt == OR_F32 || dt == OR_BF16 || dt == OR_F64; }

static void set_threads(int nthreads)
{
    if (nthreads > 0) omp_set_num_threads(nthreads);
}

double oracle_gelu(double x) { return x * 0.5 * (1.0 + erf(x / sqrt(2.0))); }
double oracle_silu(double x) { return x / (1.0 + exp(-x)); }
/* tanh form of GELU: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) */
double oracle_gelu_tanh(double x)
{
    return 0.5 * x * (1.0 + tanh(sqrt(2.0 / M_PI) * (x + 0.044715 * x * x * x)));
}

static double act_fn(int act, double x)
{
    if (act == OR_SILU) return oracle_silu(x);
    if (act == OR_GELU_TANH) return oracle_gelu_tanh(x);
    return oracle_gelu(x);
}

/* Derivatives of the activations, written from their definitions:
 *   GELU(x) = x Phi(x):           Phi(x) + x phi(x)
 *   SiLU(x) = x s(x), s sigmoid:  s(x) (1 + x (1 - s(x)))
 *   tanh form 0.5 x (1 + tanh u), u = c (x + k x^3):
 *                                  0.5 (1 + tanh u) + 0.5 x (1 - tanh^2 u) c (1 + 3 k x^2) */
double oracle_act_grad(int act, double x)
{
    if (act == OR_SILU) {
        double sg = 1.0 / (1.0 + exp(-x));
        return sg * (1.0 + x * (1.0 - sg));
    }
    if (act == OR_GELU_TANH) {
        const double c = sqrt(2.0 / M_PI), k = 0.044715;
        double t = tanh(c * (x + k * x * x * x));
        return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * c * (1.0 + 3.0 * k * x * x);
    }
    return 0.5 * (1.0 + erf(x / sqrt(2.0))) + x * exp(-0.5 * x * x) / sqrt(2.0 * M_PI);
}

/*
 * Attention of one query vector over a set of key/value rows, returning the
 * log of the sum of exponentiated scores and the normalized read-out.
 * keys: row j at K + (koff + j * d) elements, j = 0..nk-1.
 * An empty set gives lse = -inf and a zero read-out.
 */
static void attend(int dt, int d, long nk, double scale,
                   const void *q, size_t qoff,
                   const void *K, const void *V, size_t koff,
                   double *s /* scratch, nk */, double *lse, double *out)
{
    for (int c = 0; c < d; ++c) out[c] = 0.0;
    if (nk <= 0) { *lse = -INFINITY; return; }
    double m = -INFINITY;
    for (long j = 0; j < nk; ++j) {
        double dot = 0.0;
        for (int c = 0; c < d; ++c)
            dot += ld(q, dt, qoff + c) * ld(K, dt, koff + (size_t)j * d + c);
        s[j] = dot * scale;
        if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (long j = 0; j < nk; ++j) {
        double w = exp(s[j] - m);
        l += w;
        for (int c = 0; c < d; ++c) out[c] += w * ld(V, dt, koff + (size_t)j * d + c);
    }
    for (int c = 0; c < d; ++c) out[c] /= l;
    *lse = m + log(l);
}

static int shape_ok(int R, int Hq, int Hkv, int d)
{
    return R >= 0 && Hq > 0 && Hkv > 0 && d > 0 && Hq % Hkv == 0;
}

/*
 * Exact document attention, Eq. (3.1), for the listed tokens (toks == NULL:
 * all R tokens).  alpha_out[i][hq], A_out[i][hq][c] for i = 0..ntok-1.
 */
int oracle_doc_attn(int dt, int R, int Hq, int Hkv, int d, long n, double scale,
                    const void *q, const void *K, const void *V,
                    const int32_t *toks, int ntok,
                    double *alpha_out, double *A_out, int nthreads)
{
    if (!valid_dt(dt) || !shape_ok(R, Hq, Hkv, d) || n < 0) return 1;
    if (!toks) ntok = R;
    const int G = Hq / Hkv;
    set_threads(nthreads);
    int err = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        if (!s) {
#pragma omp atomic write
            err = 2;
        }
#pragma omp for schedule(dynamic, 1)
        for (long row = 0; row < (long)ntok * Hq; ++row) {
            if (!s) continue;
            int i = (int)(row / Hq), hq = (int)(row % Hq);
            int r = toks ? toks[i] : i;
            int h = hq / G;
            attend(dt, d, n, scale, q, ((size_t)r * Hq + hq) * d,
                   K, V, (size_t)h * n * d, s,
                   &alpha_out[(size_t)i * Hq + hq], &A_out[((size_t)i * Hq + hq) * d]);
        }
        free(s);
    }
    return err;
}

/*
 * Quadrature (learnable KV pair) module, section 2.4: exact attention over the
 * p parameter pairs (W, Z) with the same 1/sqrt(d) scaling.
 */
int oracle_kvpair(int dt, int R, int Hq, int Hkv, int d, long p, double scale,
                  const void *q, const void *W, const void *Z,
                  const int32_t *toks, int ntok,
                  double *a_out, double *A_out, int nthreads)
{
    return oracle_doc_attn(dt, R, Hq, Hkv, d, p, scale, q, W, Z, toks, ntok, a_out, A_out, nthreads);
}

/*
 * Local causal attention, section 2.2: token t of question b (query row
 * r = b*Tq + t) sees local keys i = 0 .. min(q_offset + t, Tloc - 1) of its
 * own question's cache.  Returns lse = log Z_local and A_local = N_local / Z_local;
 * an empty visible set gives lse = -inf and A_local = 0.
 */
int oracle_local_attn(int dt, int B, int Tq, int Hq, int Hkv, int d, int Tloc, int q_offset,
                      double scale, const void *q, const void *Kl, const void *Vl,
                      const int32_t *toks, int ntok, double *lse_out, double *A_out, int nthreads)
{
    if (!valid_dt(dt) || B < 0 || Tq < 0 || !shape_ok(B * Tq, Hq, Hkv, d) || Tloc < 0) return 1;
    const int R = B * Tq;
    if (!toks) ntok = R;
    const int G = Hq / Hkv;
    set_threads(nthreads);
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(Tloc > 0 ? Tloc : 1));
#pragma omp for schedule(dynamic, 1)
        for (long row = 0; row < (long)ntok * Hq; ++row) {
            int i = (int)(row / Hq), hq = (int)(row % Hq);
            int r = toks ? toks[i] : i;
            int b = r / Tq, t = r % Tq, h = hq / G;
            long vis = (long)q_offset + t + 1;
            if (vis > Tloc) vis = Tloc;
            if (vis < 0) vis = 0;
            attend(dt, d, vis, scale, q, ((size_t)r * Hq + hq) * d,
                   Kl, Vl, ((size_t)b * Hkv + h) * (size_t)Tloc * d, s,
                   &lse_out[(size_t)i * Hq + hq], &A_out[((size_t)i * Hq + hq) * d]);
        }
        free(s);
    }
    return 0;
}

/*
 * Full attention over the concatenated [document; local] cache with the causal
 * mask on the local part only (the left-hand side of Eq. (3.4)).
 */
int oracle_full_attn(int dt, int B, int Tq, int Hq, int Hkv, int d, long n, int Tloc, int q_offset,
                     double scale, const void *q, const void *K, const void *V,
                     const void *Kl, const void *Vl,
                     const int32_t *toks, int ntok, double *lse_out, double *out, int nthreads)
{
    if (!valid_dt(dt) || B < 0 || Tq < 0 || !shape_ok(B * Tq, Hq, Hkv, d) || n < 0 || Tloc < 0) return 1;
    const int R = B * Tq;
    if (!toks) ntok = R;
    const int G = Hq / Hkv;
    set_threads(nthreads);
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(n + Tloc + 1));
#pragma omp for schedule(dynamic, 1)
        for (long row = 0; row < (long)ntok * Hq; ++row) {
            int i = (int)(row / Hq), hq = (int)(row % Hq);
            int r = toks ? toks[i] : i;
            int b = r / Tq, t = r % Tq, h = hq / G;
            long vis = (long)q_offset + t + 1;
            if (vis > Tloc) vis = Tloc;
            if (vis < 0) vis = 0;
            size_t qo = ((size_t)r * Hq + hq) * d;
            size_t dko = (size_t)h * n * d;
            size_t lko = ((size_t)b * Hkv + h) * (size_t)Tloc * d;
            long nk = n + vis;
            double *o = &out[((size_t)i * Hq + hq) * d];
            for (int c = 0; c < d; ++c) o[c] = 0.0;
            if (nk == 0) { lse_out[(size_t)i * Hq + hq] = -INFINITY; continue; }
            double m = -INFINITY;
            for (long j = 0; j < nk; ++j) {
                const void *Kp = j < n ? K : Kl;
                size_t ko = j < n ? dko + (size_t)j * d : lko + (size_t)(j - n) * d;
                double dot = 0.0;
                for (int c = 0; c < d; ++c) dot += ld(q, dt, qo + c) * ld(Kp, dt, ko + c);
                s[j] = dot * scale;
                if (s[j] > m) m = s[j];
            }
            double l = 0.0;
            for (long j = 0; j < nk; ++j) {
                const void *Vp = j < n ? V : Vl;
                size_t vo = j < n ? dko + (size_t)j * d : lko + (size_t)(j - n) * d;
                double w = exp(s[j] - m);
                l += w;
                for (int c = 0; c < d; ++c) o[c] += w * ld(Vp, dt, vo + c);
            }
            for (int c = 0; c < d; ++c) o[c] /= l;
            lse_out[(size_t)i * Hq + hq] = m + log(l);
        }
        free(s);
    }
    return 0;
}

/*
 * One-hidden-layer MLP module (Eq. (3.6) with only h_0), for the listed tokens:
 *   z_j   = sum_c W1[h][j][c] q_c + b1[h][j],     A_c = sum_j W2t[h][j][c] act(z_j) + b2[h][c]
 *   zs_j  = sum_c Ws[h][j][c] q_c + bs[h][j],     a   = sum_j ws2[h][j] act(zs_j) + bs2[h]
 */
int oracle_mlp(int dt, int R, int Hq, int Hkv, int d, int Ht, int Hs, int act,
               const void *W1, const double *b1, const void *W2t, const double *b2,
               const void *Ws, const double *bs, const void *ws2, const double *bs2,
               const void *q, const int32_t *toks, int ntok,
               double *a_out, double *A_out, int nthreads)
{
    if (!valid_dt(dt) || !shape_ok(R, Hq, Hkv, d) || Ht < 0 || Hs < 0) return 1;
    if (act != OR_GELU && act != OR_SILU && act != OR_GELU_TANH) return 1;
    if (!toks) ntok = R;
    const int G = Hq / Hkv;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (long row = 0; row < (long)ntok * Hq; ++row) {
        int i = (int)(row / Hq), hq = (int)(row % Hq);
        int r = toks ? toks[i] : i;
        int h = hq / G;
        size_t qo = ((size_t)r * Hq + hq) * d;
        double *A = &A_out[((size_t)i * Hq + hq) * d];
        for (int c = 0; c < d; ++c) A[c] = b2[(size_t)h * d + c];
        for (int j = 0; j < Ht; ++j) {
            size_t wo = ((size_t)h * Ht + j) * d;
            double z = 0.0;
            for (int c = 0; c < d; ++c) z += ld(W1, dt, wo + c) * ld(q, dt, qo + c);
            double y = act_fn(act, z + b1[(size_t)h * Ht + j]);
            for (int c = 0; c < d; ++c) A[c] += ld(W2t, dt, wo + c) * y;
        }
        double a = bs2[h];
        for (int j = 0; j < Hs; ++j) {
            size_t wo = ((size_t)h * Hs + j) * d;
            double z = 0.0;
            for (int c = 0; c < d; ++c) z += ld(Ws, dt, wo + c) * ld(q, dt, qo + c);
            a += ld(ws2, dt, (size_t)h * Hs + j) * act_fn(act, z + bs[(size_t)h * Hs + j]);
        }
        a_out[(size_t)i * Hq + hq] = a;
    }
    return 0;
}

/*
 * Deep MLP module with input re-injection, Eq. (3.6) of section 2.4: the first
 * layer of a network reads only the query, h_0 = act(U_0 q + b_0); every later
 * layer reads the query again beside the previous layer's state,
 * h_{k+1} = act(V_k q + U_k h_k + b_k).  Reading of the depth triple
 * (D_b, D_s, D_t): an optional shared backbone of D_b such layers (width H_b)
 * is followed by a score head of D_s layers (width H_s) and a target head of
 * D_t layers (width H_t); a head's first layer reads the backbone's last state
 * when there is a backbone (so it too has the re-injection form), else only the
 * query.  Each head ends in a linear read-out of its last state (the
 * backbone's when the head has no layer of its own):
 *   a = ws_out . h_s + bs_out,      A_c = sum_j Wt_out[c][j] h_t,j + bt_out[c].
 *
 * Layers are listed backbone first, then score, then target.  Layer l has
 *   Wq[l] [Hkv][H_l][d]        query weights (U_0 or V_k),
 *   Wh[l] [Hkv][H_l][H_in]     state weights (U_k; NULL for a layer that reads
 *                              only the query),
 *   b[l]  [Hkv][H_l]           bias;
 * ws_out [Hkv][H_s_last], bs_out [Hkv], Wt_out [Hkv][d][H_t_last], bt_out [Hkv][d].
 * Every sum is plain fp64 in index order; hidden states are kept in fp64.
 */
#define OR_DEEP_MAX_LAYERS 64
int oracle_deep_mlp(int dt, int R, int Hq, int Hkv, int d, int act,
                    const int32_t *depth, const int32_t *width,
                    const void *const *Wq, const void *const *Wh, const double *const *b,
                    const void *ws_out, const double *bs_out, const void *Wt_out, const double *bt_out,
                    const void *q, const int32_t *toks, int ntok,
                    double *a_out, double *A_out, int nthreads)
{
    if (!valid_dt(dt) || !shape_ok(R, Hq, Hkv, d)) return 1;
    if (act != OR_GELU && act != OR_SILU && act != OR_GELU_TANH) return 1;
    for (int part = 0; part < 3; ++part)
        if (depth[part] < 0 || (depth[part] > 0 && width[part] <= 0)) return 1;
    const int Db = depth[0], Ds = depth[1], Dt = depth[2];
    if (Db + Ds + Dt > OR_DEEP_MAX_LAYERS || Db + Ds < 1 || Db + Dt < 1) return 1;
    /* width of the state each layer reads (0: the query only) */
    int in_w[OR_DEEP_MAX_LAYERS], out_w[OR_DEEP_MAX_LAYERS];
    int Hmax = 1;
    for (int l = 0; l < Db + Ds + Dt; ++l) {
        int part = l < Db ? 0 : (l < Db + Ds ? 1 : 2);
        int first = part == 0 ? 0 : (part == 1 ? Db : Db + Ds);
        out_w[l] = width[part];
        in_w[l] = l > first ? width[part] : (part > 0 && Db > 0 ? width[0] : 0);
        if ((in_w[l] > 0) != (Wh[l] != NULL) || !Wq[l] || !b[l]) return 1;
        if (out_w[l] > Hmax) Hmax = out_w[l];
    }
    const int Hs_last = Ds > 0 ? width[1] : width[0];
    const int Ht_last = Dt > 0 ? width[2] : width[0];
    if (!toks) ntok = R;
    const int G = Hq / Hkv;
    set_threads(nthreads);
#pragma omp parallel
    {
        double *bb = (double *)calloc((size_t)Hmax, sizeof(double));
        double *s0 = (double *)calloc((size_t)Hmax, sizeof(double));
        double *s1 = (double *)calloc((size_t)Hmax, sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (long row = 0; row < (long)ntok * Hq; ++row) {
            int i = (int)(row / Hq), hq = (int)(row % Hq);
            int r = toks ? toks[i] : i;
            int h = hq / G;
            size_t qo = ((size_t)r * Hq + hq) * d;
            /* run layers [l0, l1) starting from state `init` (width in_w[l0]); result in *res */
            double *cur = s0, *nxt = s1;
            for (int part = 0; part < 3; ++part) {
                int l0 = part == 0 ? 0 : (part == 1 ? Db : Db + Ds);
                int l1 = l0 + depth[part];
                const double *state = part > 0 && Db > 0 ? bb : NULL;
                for (int l = l0; l < l1; ++l) {
                    for (int j = 0; j < out_w[l]; ++j) {
                        size_t wo = ((size_t)h * out_w[l] + j) * d;
                        double z = b[l][(size_t)h * out_w[l] + j];
                        for (int c = 0; c < d; ++c) z += ld(Wq[l], dt, wo + c) * ld(q, dt, qo + c);
                        if (in_w[l] > 0) {
                            size_t ho = ((size_t)h * out_w[l] + j) * in_w[l];
                            for (int k = 0; k < in_w[l]; ++k) z += ld(Wh[l], dt, ho + k) * state[k];
                        }
                        nxt[j] = act_fn(act, z);
                    }
                    double *t = cur; cur = nxt; nxt = t;
                    state = cur;
                }
                if (part == 0) {
                    for (int j = 0; j < width[0] && Db > 0; ++j) bb[j] = cur[j];
                } else if (part == 1) {
                    double a = bs_out[h];
                    for (int j = 0; j < Hs_last; ++j) a += ld(ws_out, dt, (size_t)h * Hs_last + j) * state[j];
                    a_out[(size_t)i * Hq + hq] = a;
                } else {
                    double *A = &A_out[((size_t)i * Hq + hq) * d];
                    for (int c = 0; c < d; ++c) {
                        double v = bt_out[(size_t)h * d + c];
                        size_t wo = ((size_t)h * d + c) * Ht_last;
                        for (int j = 0; j < Ht_last; ++j) v += ld(Wt_out, dt, wo + j) * state[j];
                        A[c] = v;
                    }
                }
            }
        }
        free(bb); free(s0); free(s1);
    }
    return 0;
}

/*
 * Fit metrics of a module against the exact pair (the regression losses of
 * Eqs. (3.2)-(3.3) and the RTE of Eq. (C.1), section 3.3 and App. C.4 of the
 * notes).  For every token row r and query head h' (KV head h = h' / G):
 *   row[0] = (a - alpha)^2                           score squared error
 *   row[1] = || A_theta - A ||^2                     target squared error
 *   row[2] = log( ||A_theta - A||^2 / ||q - A||^2 )  the RTE summand
 * and per KV head the sums of each over its rows (all tokens, all its query
 * heads): head[h][k] = sum row[k].  row [R][Hq][3], head [Hkv][3].  q is read in
 * its storage type; the pairs are fp64.
 */
int oracle_fit_metrics(int dt, int R, int Hq, int Hkv, int d, const void *q,
                       const double *a, const double *A, const double *alpha, const double *Aex,
                       double *row, double *head)
{
    if (!valid_dt(dt) || !shape_ok(R, Hq, Hkv, d)) return 1;
    const int G = Hq / Hkv;
    for (int h = 0; h < Hkv; ++h) head[3 * h] = head[3 * h + 1] = head[3 * h + 2] = 0.0;
    for (long r = 0; r < R; ++r)
        for (int hq = 0; hq < Hq; ++hq) {
            size_t i = (size_t)r * Hq + hq;
            double es = (a[i] - alpha[i]) * (a[i] - alpha[i]);
            double et = 0.0, eq = 0.0;
            for (int c = 0; c < d; ++c) {
                double x = A[i * d + c] - Aex[i * d + c];
                double y = ld(q, dt, i * d + c) - Aex[i * d + c];
                et += x * x;
                eq += y * y;
            }
            double lr = log(et / eq);
            row[3 * i] = es; row[3 * i + 1] = et; row[3 * i + 2] = lr;
            int h = hq / G;
            head[3 * h] += es; head[3 * h + 1] += et; head[3 * h + 2] += lr;
        }
    return 0;
}

/*
 * Regression loss of the one-hidden-layer module and its gradient (section 2.3,
 * Eqs. (3.2)-(3.3)): over the R token rows of one layer,
 *   L_alpha = (1/R) sum_r sum_h' (a(q) - alpha)^2,
 *   L_A     = (1/R) sum_r sum_h' ||A(q) - A_target||^2,
 *   L       = lambda_alpha L_alpha + lambda_A L_A
 * (the expectation over samples is the mean over tokens; the sum runs over the
 * query heads).  loss[0..2] = L, L_alpha, L_A.  The gradient of L with respect
 * to each parameter array (same layouts as oracle_mlp) is written to the fp64
 * arrays gW1 .. gbs2, by the chain rule written out per row:
 *   gA = 2 lambda_A (A - A_target) / R,  ga = 2 lambda_alpha (a - alpha) / R,
 *   target unit j: dz_j = act'(z_j) sum_c W2t[j][c] gA_c; dW2t[j][c] += act(z_j) gA_c,
 *                  dW1[j][c] += dz_j q_c, db1[j] += dz_j; db2 += gA;
 *   score unit j:  dzs_j = act'(zs_j) ws2[j] ga; dws2[j] += act(zs_j) ga,
 *                  dWs[j][c] += dzs_j q_c, dbs[j] += dzs_j; dbs2 += ga.
 * Rows are accumulated in order (single thread), so the result is reproducible.
 */
int oracle_mlp_loss_grad(int dt, int R, int Hq, int Hkv, int d, int Ht, int Hs, int act,
                         const void *W1, const double *b1, const void *W2t, const double *b2,
                         const void *Ws, const double *bs, const void *ws2, const double *bs2,
                         const void *q, const double *alpha, const double *Atgt,
                         double lam_alpha, double lam_A,
                         double *gW1, double *gb1, double *gW2t, double *gb2,
                         double *gWs, double *gbs, double *gws2, double *gbs2, double *loss)
{
    if (!valid_dt(dt) || !shape_ok(R, Hq, Hkv, d) || Ht < 0 || Hs < 0 || R <= 0) return 1;
    if (act != OR_GELU && act != OR_SILU && act != OR_GELU_TANH) return 1;
    const int G = Hq / Hkv;
    memset(gW1, 0, sizeof(double) * (size_t)Hkv * Ht * d);
    memset(gb1, 0, sizeof(double) * (size_t)Hkv * Ht);
    memset(gW2t, 0, sizeof(double) * (size_t)Hkv * Ht * d);
    memset(gb2, 0, sizeof(double) * (size_t)Hkv * d);
    memset(gWs, 0, sizeof(double) * (size_t)Hkv * Hs * d);
    memset(gbs, 0, sizeof(double) * (size_t)Hkv * Hs);
    memset(gws2, 0, sizeof(double) * (size_t)Hkv * Hs);
    memset(gbs2, 0, sizeof(double) * (size_t)Hkv);
    double *z = (double *)malloc(sizeof(double) * (size_t)(Ht > Hs ? Ht : Hs) + 8);
    double *A = (double *)malloc(sizeof(double) * (size_t)d);
    double *gA = (double *)malloc(sizeof(double) * (size_t)d);
    double La = 0.0, LA = 0.0;
    for (long r = 0; r < R; ++r)
        for (int hq = 0; hq < Hq; ++hq) {
            const int h = hq / G;
            const size_t qo = ((size_t)r * Hq + hq) * d, i = (size_t)r * Hq + hq;
            /* forward */
            for (int c = 0; c < d; ++c) A[c] = b2[(size_t)h * d + c];
            for (int j = 0; j < Ht; ++j) {
                size_t wo = ((size_t)h * Ht + j) * d;
                double zz = b1[(size_t)h * Ht + j];
                for (int c = 0; c < d; ++c) zz += ld(W1, dt, wo + c) * ld(q, dt, qo + c);
                z[j] = zz;
                double y = act_fn(act, zz);
                for (int c = 0; c < d; ++c) A[c] += ld(W2t, dt, wo + c) * y;
            }
            for (int c = 0; c < d; ++c) {
                double e = A[c] - Atgt[i * d + c];
                LA += e * e;
                gA[c] = 2.0 * lam_A * e / R;
            }
            /* target backward */
            for (int c = 0; c < d; ++c) gb2[(size_t)h * d + c] += gA[c];
            for (int j = 0; j < Ht; ++j) {
                size_t wo = ((size_t)h * Ht + j) * d;
                double y = act_fn(act, z[j]), dy = 0.0;
                for (int c = 0; c < d; ++c) {
                    dy += ld(W2t, dt, wo + c) * gA[c];
                    gW2t[wo + c] += y * gA[c];
                }
                double dz = dy * oracle_act_grad(act, z[j]);
                gb1[(size_t)h * Ht + j] += dz;
                for (int c = 0; c < d; ++c) gW1[wo + c] += dz * ld(q, dt, qo + c);
            }
            /* score forward and backward */
            double a = bs2[h];
            for (int j = 0; j < Hs; ++j) {
                size_t wo = ((size_t)h * Hs + j) * d;
                double zz = bs[(size_t)h * Hs + j];
                for (int c = 0; c < d; ++c) zz += ld(Ws, dt, wo + c) * ld(q, dt, qo + c);
                z[j] = zz;
                a += ld(ws2, dt, (size_t)h * Hs + j) * act_fn(act, zz);
            }
            double e = a - alpha[i];
            La += e * e;
            double ga = 2.0 * lam_alpha * e / R;
            gbs2[h] += ga;
            for (int j = 0; j < Hs; ++j) {
                size_t wo = ((size_t)h * Hs + j) * d;
                gws2[(size_t)h * Hs + j] += act_fn(act, z[j]) * ga;
                double dz = ld(ws2, dt, (size_t)h * Hs + j) * ga * oracle_act_grad(act, z[j]);
                gbs[(size_t)h * Hs + j] += dz;
                for (int c = 0; c < d; ++c) gWs[wo + c] += dz * ld(q, dt, qo + c);
            }
        }
    free(z); free(A); free(gA);
    loss[1] = La / R;
    loss[2] = LA / R;
    loss[0] = lam_alpha * loss[1] + lam_A * loss[2];
    return 0;
}

/*
 * One AdamW step (Loshchilov & Hutter's decoupled weight decay; the notes'
 * optimizer, App. A.2-A.5) on n parameters with the gradient scaled by `scale`
 * (the global-norm clipping factor):
 *   theta <- theta (1 - lr wd);  g' = scale g;
 *   m <- b1 m + (1 - b1) g';  v <- b2 v + (1 - b2) g'^2;
 *   theta <- theta - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps),  t = step >= 1.
 */
void oracle_adamw(long n, double *theta, const double *g, double *m, double *v, double lr, double b1,
                  double b2, double eps, double wd, int step, double scale)
{
    const double c1 = 1.0 - pow(b1, step), c2 = 1.0 - pow(b2, step);
    for (long i = 0; i < n; ++i) {
        const double gi = scale * g[i];
        theta[i] *= 1.0 - lr * wd;
        m[i] = b1 * m[i] + (1.0 - b1) * gi;
        v[i] = b2 * v[i] + (1.0 - b2) * gi * gi;
        theta[i] -= lr * (m[i] / c1) / (sqrt(v[i] / c2) + eps);
    }
}

/*
 * Log-sum-exp merge of two (lse, read-out) pairs, Eqs. (3.4)-(3.5): the first
 * pair is the document part (exact alpha, A or the module's a, A), used as one
 * extra "virtual logit" with value A beside the local part (lse_loc, A_loc):
 *   out = (e^a A + e^lam A_loc) / (e^a + e^lam),   lse = log(e^a + e^lam),
 * evaluated with M = max(a, lam).  Both sides -inf gives out = 0, lse = -inf.
 */
void oracle_merge(long rows, int d, const double *a, const double *A,
                  const double *lam, const double *Aloc, double *out, double *lse)
{
    for (long r = 0; r < rows; ++r) {
        double M = a[r] > lam[r] ? a[r] : lam[r];
        double *o = &out[(size_t)r * d];
        if (M == -INFINITY) {
            for (int c = 0; c < d; ++c) o[c] = 0.0;
            lse[r] = -INFINITY;
            continue;
        }
        double wa = exp(a[r] - M), wl = exp(lam[r] - M);
        for (int c = 0; c < d; ++c)
            o[c] = (wa * A[(size_t)r * d + c] + wl * Aloc[(size_t)r * d + c]) / (wa + wl);
        lse[r] = M + log(wa + wl);
    }
}

/*
 * K-way composition of document-side pairs with the local part: the pages'
 * closing section proposes merging several context modules by one more
 * softmax grouping over their (score, target) outputs, the virtual-logit form
 * of Eqs. (3.4)-(3.5) with K virtual logits.  Per row:
 *   out = (sum_k e^{a_k} A_k + e^{lam} A_loc) / (sum_k e^{a_k} + e^{lam}),
 *   lse = log(sum_k e^{a_k} + e^{lam}),
 * evaluated with the common maximum M of all logits; lam == NULL drops the local
 * part; every logit -inf gives out = 0, lse = -inf.  a [K][rows], A [K][rows][d].
 */
void oracle_merge_k(long rows, int d, int K, const double *a, const double *A,
                    const double *lam, const double *Aloc, double *out, double *lse)
{
    for (long r = 0; r < rows; ++r) {
        double M = lam ? lam[r] : -INFINITY;
        for (int k = 0; k < K; ++k)
            if (a[(size_t)k * rows + r] > M) M = a[(size_t)k * rows + r];
        double *o = &out[(size_t)r * d];
        for (int c = 0; c < d; ++c) o[c] = 0.0;
        if (M == -INFINITY) {
            lse[r] = -INFINITY;
            continue;
        }
        double den = 0.0;
        for (int k = 0; k < K; ++k) {
            const double w = exp(a[(size_t)k * rows + r] - M);
            den += w;
            for (int c = 0; c < d; ++c) o[c] += w * A[((size_t)k * rows + r) * d + c];
        }
        if (lam) {
            const double w = exp(lam[r] - M);
            den += w;
            for (int c = 0; c < d; ++c) o[c] += w * Aloc[(size_t)r * d + c];
        }
        for (int c = 0; c < d; ++c) o[c] /= den;
        lse[r] = M + log(den);
    }
}
