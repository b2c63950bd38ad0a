/*
 * oracle.c -- plain, slow, fp64 CPU oracle for scaled dot-product
 * multi-head attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load it.  It shares no code, header, table or constant with the HIP
 * library, and it never touches a GPU.
 *
 * Sources (three web pages on "Attention Is All You Need"):
 *   [Slides]     "Attention Is All You Need -- A Revolutionary Architecture
 *                for Sequence Transduction" (slide deck).
 *   [Deep]       "Paper Deep Reading: Attention Is All You Need", sections
 *                01-12.
 *   [Paperglide] "Attention Is All You Need" explainer (paperglide).
 *
 * What is computed.  The method is exactly its definition, so the oracle is
 * that definition written out, in fp64, with no blocking, fusion or
 * reordering:
 *   Attention(Q,K,V) = softmax(Q K^T / sqrt(d_k) + M) V
 *       [Deep] section 04 "Attention mechanics", the attention equation
 *       (with M); [Slides] slide "Attention Mechanism" (without M).
 *       Operation order MatMul -> Scale -> Mask -> SoftMax -> MatMul:
 *       [Deep] section 04, Figure 2 (left) caption.
 *   M is -infinity at illegal connections, 0 elsewhere: [Deep] section 03,
 *       "Decoder layer"; the encoder masks padding and the decoder also masks
 *       future positions: [Deep] section 04, text under the attention
 *       equation.
 *   MultiHead = Concat(head_1..head_h) W^O, head_i = Attention(Q W_i^Q,
 *       K W_i^K, V W_i^V): [Slides] slide "Multi-Head Attention";
 *       [Deep] section 04, MultiHead equations.  Head i owns column block i
 *       of the projected matrix and the concat is head_1 || head_2 || ...:
 *       [Paperglide] two-head toy example under "Multi-Head Attention".
 *
 * Readings taken where the pages are silent (each is listed with its reason
 * in the design notes):
 *   - causal: key j is legal for query i iff j <= i (the diagonal is kept);
 *   - restricted (windowed) self-attention with half-width w: key j is legal
 *     for query i iff |i - j| <= w, a neighbourhood of r = 2w + 1 positions
 *     centred on the query, so a layer costs O(r n d) and a signal crosses n
 *     positions in O(n / r) layers ([Deep] section 05, the complexity table,
 *     "Restricted self-attention"; [Slides] slide "Limitations and Future
 *     Work").  It combines with the other masks as their union, and needs
 *     Lq == Lk (query and key positions on one axis);
 *   - key padding: key j is legal iff j < len_b, with len_b clamped to
 *     [0, Lk];
 *   - a query row with no legal key outputs 0 (softmax of all -inf is 0/0);
 *   - an illegal key's logit is -inf whatever K holds there, so K and V rows
 *     of illegal keys are never read (padding may hold any bits);
 *   - softmax(x) is evaluated as exp(x - max x) / sum exp(x - max x), the
 *     exact identity softmax(x) = softmax(x - c), so fp64 exp stays finite
 *     for logits far from 0;
 *   - projections have no bias; X W with W in [d_model, h*d] (row-vector
 *     convention of the head_i formula).
 *
 * Layouts (row-major, C order):
 *   q [B, Lq, h, d_k]   k [B, Lk, h, d_k]   v [B, Lk, h, d_v]
 *   o [B, Lq, h, d_v]   -- the same bytes as Concat(heads) [B*Lq, h*d_v]
 *   p (optional)  [B, h, Lq, Lk]  attention weights softmax(...)
 *   s (optional)  [B, h, Lq, Lk]  scaled logits q.k/sqrt(d_k), -inf where
 *                                 masked
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_MASK_KEY_PADDING 1
#define ORACLE_MASK_CAUSAL 2

/* Number of threads the OpenMP loops below use. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Is key j legal for query i of batch row b?  [Deep] section 03 "Decoder
 * layer" (future connections are illegal), section 04 (padding), section 05
 * (restricted self-attention: window >= 0 is the half-width, -1 none). */
static int key_is_legal(int mask_flags, long len_b, long window, long i, long j)
{
    if ((mask_flags & ORACLE_MASK_KEY_PADDING) && j >= len_b) return 0;
    if ((mask_flags & ORACLE_MASK_CAUSAL) && j > i) return 0;
    if (window >= 0 && (j < i - window || j > i + window)) return 0;
    return 1;
}

static long clamped_len(int mask_flags, const int32_t* kv_lens, long b, long Lk)
{
    if (!(mask_flags & ORACLE_MASK_KEY_PADDING)) return Lk;
    long len = kv_lens[b];
    if (len < 0) len = 0;
    if (len > Lk) len = Lk;
    return len;
}

/*
 * One output row: o[b, i, t, :] for query i of head t in batch row b.
 * logits/weights are scratch arrays of length Lk owned by the caller.
 * p_row / s_row, when not NULL, receive this row of P and of the scaled
 * logits.
 */
static void attention_row(long B, long h, long Lq, long Lk, long d_k, long d_v,
                          const double* q, const double* k, const double* v,
                          int mask_flags, const int32_t* kv_lens, long window,
                          long b, long t, long i,
                          double* o_row, double* p_row, double* s_row,
                          double* logits, double* weights)
{
    (void)B; (void)Lq;
    const long len_b = clamped_len(mask_flags, kv_lens, b, Lk);
    const double scale = 1.0 / sqrt((double)d_k);
    const double* qi = q + ((b * Lq + i) * h + t) * d_k;

    /* MatMul, then Scale, then Mask ([Deep] section 04, Figure 2 left). */
    int any_legal = 0;
    for (long j = 0; j < Lk; ++j) {
        if (!key_is_legal(mask_flags, len_b, window, i, j)) {
            logits[j] = -INFINITY;
            continue;
        }
        const double* kj = k + ((b * Lk + j) * h + t) * d_k;
        double dot = 0.0;
        for (long c = 0; c < d_k; ++c) dot += qi[c] * kj[c];
        logits[j] = dot * scale;
        any_legal = 1;
    }
    if (s_row)
        for (long j = 0; j < Lk; ++j) s_row[j] = logits[j];

    if (!any_legal) {
        /* softmax over an all -inf row is 0/0; the output is defined as 0. */
        for (long e = 0; e < d_v; ++e) o_row[e] = 0.0;
        if (p_row)
            for (long j = 0; j < Lk; ++j) p_row[j] = 0.0;
        return;
    }

    /* SoftMax: exp(x - max) / sum.  exp(-inf - max) = 0 exactly. */
    double mx = -INFINITY;
    for (long j = 0; j < Lk; ++j)
        if (logits[j] > mx) mx = logits[j];
    double total = 0.0;
    for (long j = 0; j < Lk; ++j) {
        weights[j] = (logits[j] == -INFINITY) ? 0.0 : exp(logits[j] - mx);
        total += weights[j];
    }
    for (long j = 0; j < Lk; ++j) weights[j] /= total;
    if (p_row)
        for (long j = 0; j < Lk; ++j) p_row[j] = weights[j];

    /* MatMul with V: a weighted sum of the value rows ([Slides] slide
     * "Attention Mechanism").  Keys with weight exactly 0 are illegal keys
     * and their V rows are not read. */
    for (long e = 0; e < d_v; ++e) o_row[e] = 0.0;
    for (long j = 0; j < Lk; ++j) {
        if (!key_is_legal(mask_flags, len_b, window, i, j)) continue;
        const double* vj = v + ((b * Lk + j) * h + t) * d_v;
        for (long e = 0; e < d_v; ++e) o_row[e] += weights[j] * vj[e];
    }
}

/*
 * O = softmax(Q K^T / sqrt(d_k) + M) V for every (b, t).
 * kv_lens: [B] int32, read only when KEY_PADDING is set (may be NULL
 * otherwise).  window: the restricted-attention half-width, or -1 for none.
 * p and s may be NULL.  Returns 0, or -1 on bad arguments.
 */
int oracle_attention(long B, long h, long Lq, long Lk, long d_k, long d_v,
                     const double* q, const double* k, const double* v,
                     int mask_flags, const int32_t* kv_lens, long window,
                     double* o, double* p, double* s)
{
    if (B < 0 || h < 1 || Lq < 0 || Lk < 0 || d_k < 1 || d_v < 1 || window < -1) return -1;
    if ((mask_flags & ORACLE_MASK_KEY_PADDING) && !kv_lens && B > 0) return -1;
    if ((mask_flags & ORACLE_MASK_CAUSAL) && Lq != Lk) return -1;
    if (window >= 0 && Lq != Lk) return -1;
    const long rows = B * h * Lq;
    int failed = 0;
#pragma omp parallel
    {
        double* logits = (double*)malloc(sizeof(double) * (size_t)(Lk > 0 ? Lk : 1));
        double* weights = (double*)malloc(sizeof(double) * (size_t)(Lk > 0 ? Lk : 1));
        if (!logits || !weights) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (long r = 0; r < rows; ++r) {
                const long b = r / (h * Lq);
                const long t = (r / Lq) % h;
                const long i = r % Lq;
                double* o_row = o + ((b * Lq + i) * h + t) * d_v;
                double* p_row = p ? p + ((b * h + t) * Lq + i) * Lk : NULL;
                double* s_row = s ? s + ((b * h + t) * Lq + i) * Lk : NULL;
                attention_row(B, h, Lq, Lk, d_k, d_v, q, k, v, mask_flags, kv_lens, window,
                              b, t, i, o_row, p_row, s_row, logits, weights);
            }
        }
        free(logits);
        free(weights);
    }
    return failed ? -1 : 0;
}

/*
 * The same definition evaluated for a chosen list of output rows only:
 * rows[3*n + 0..2] = (b, t, i); o_rows[n, d_v] receives o[b, i, t, :].
 * Used to check large problems one sampled row at a time.
 */
int oracle_attention_rows(long B, long h, long Lq, long Lk, long d_k, long d_v,
                          const double* q, const double* k, const double* v,
                          int mask_flags, const int32_t* kv_lens, long window,
                          long n_rows, const int64_t* rows, double* o_rows)
{
    if (B < 0 || h < 1 || Lq < 0 || Lk < 0 || d_k < 1 || d_v < 1 || n_rows < 0 || window < -1)
        return -1;
    if ((mask_flags & ORACLE_MASK_KEY_PADDING) && !kv_lens && B > 0) return -1;
    if ((mask_flags & ORACLE_MASK_CAUSAL) && Lq != Lk) return -1;
    if (window >= 0 && Lq != Lk) return -1;
    for (long n = 0; n < n_rows; ++n) {
        const int64_t b = rows[3 * n], t = rows[3 * n + 1], i = rows[3 * n + 2];
        if (b < 0 || b >= B || t < 0 || t >= h || i < 0 || i >= Lq) return -1;
    }
    int failed = 0;
#pragma omp parallel
    {
        double* logits = (double*)malloc(sizeof(double) * (size_t)(Lk > 0 ? Lk : 1));
        double* weights = (double*)malloc(sizeof(double) * (size_t)(Lk > 0 ? Lk : 1));
        if (!logits || !weights) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (long n = 0; n < n_rows; ++n)
                attention_row(B, h, Lq, Lk, d_k, d_v, q, k, v, mask_flags, kv_lens, window,
                              rows[3 * n], rows[3 * n + 1], rows[3 * n + 2],
                              o_rows + n * d_v, NULL, NULL, logits, weights);
        }
        free(logits);
        free(weights);
    }
    return failed ? -1 : 0;
}

/*
 * The sub-layer's post-norm output LayerNorm(x + Sublayer(x)), applied to a
 * residual sum z = x + y already formed: for each row of z [M, N],
 *   mu = (1/N) sum_n z_n,  var = (1/N) sum_n (z_n - mu)^2,
 *   out_n = gamma_n (z_n - mu) / sqrt(var + eps) + beta_n.
 * ([Deep] section 03, "Residual + LayerNorm", post-norm order; [Slides]
 * slide "Encoder Architecture".  The pages name layer normalisation without
 * writing it out: this is its standard per-row form over the d_model
 * features, population variance, learnable gain and bias, eps inside the
 * square root.)  Two passes over the row, left to right.
 */
int oracle_layer_norm(long M, long N, const double* z, const double* gamma,
                      const double* beta, double eps, double* out)
{
    if (M < 0 || N < 1 || !(eps >= 0.0)) return -1;
#pragma omp parallel for schedule(static)
    for (long m = 0; m < M; ++m) {
        const double* zm = z + m * N;
        double mu = 0.0;
        for (long n = 0; n < N; ++n) mu += zm[n];
        mu /= (double)N;
        double var = 0.0;
        for (long n = 0; n < N; ++n) var += (zm[n] - mu) * (zm[n] - mu);
        var /= (double)N;
        const double inv = 1.0 / sqrt(var + eps);
        for (long n = 0; n < N; ++n) out[m * N + n] = gamma[n] * (zm[n] - mu) * inv + beta[n];
    }
    return 0;
}

/*
 * Y = A W, A [M, K], W [K, N], Y [M, N], all row-major fp64; a plain triple
 * loop.  This is every linear map of the multi-head block: the per-head
 * projections Q W^Q, K W^K, V W^V (all heads at once, W = [W_1 || ... ||
 * W_h]) and Concat(heads) W^O ([Deep] section 04, MultiHead equations;
 * [Slides] slide "Multi-Head Attention").  No bias appears in those
 * formulas, so none is added.
 */
int oracle_matmul(long M, long K, long N, const double* a, const double* w, double* y)
{
    if (M < 0 || K < 0 || N < 0) return -1;
#pragma omp parallel for schedule(static)
    for (long m = 0; m < M; ++m) {
        double* ym = y + m * N;
        for (long n = 0; n < N; ++n) ym[n] = 0.0;
        for (long kk = 0; kk < K; ++kk) {
            const double amk = a[m * K + kk];
            const double* wk = w + kk * N;
            for (long n = 0; n < N; ++n) ym[n] += amk * wk[n];
        }
    }
    return 0;
}
