/*
 * sparse_attn_oracle.c -- plain fp64 CPU oracle for causal structured-sparse
 * attention (forward, its log-sum-exp, backward, and single-token decode).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or constant with
 * the HIP library; it is written from the method's definition, not from the
 * GPU kernels.
 *
 * What it computes.  For one query position i the method forms an explicit
 * key set and takes ONE softmax over it:
 *
 *   - pi-Attention ("pi-Attention: Periodic Sparse Transformers for
 *     Efficient Long-Context Modeling", section 2, items 1-3): a causal
 *     local window j in [i-k, i] plus the periodic skip keys j = i - m*pi,
 *     m = 1..M, j >= 0.  The page gives the window as i-k..i+k; causal
 *     decoding restricts it to earlier positions, so the causal reading
 *     [i-k, i] is used.  The union is a set: a skip key that already lies in
 *     the window is the window's key (it gets the local prior once).  A
 *     per-token, per-head gate alpha in (0, 1] enters as a log-prior:
 *     log(alpha) is added to the scores of local keys and log(1 - alpha) to
 *     the scores of skip keys before the single softmax.
 *   - Window-only attention ("LT2: Linear-Time Looped Transformers",
 *     section 2.1, sparse variant): the window alone, no prior.
 *   - ECP paired-half-segment attention ("Efficient Context Propagating
 *     Perceiver Architectures for Auto-Regressive Language Modeling",
 *     section 2, PAR block): a query in half-segment c = floor(i/s) sees the
 *     keys of half-segments c-1 and c, causally masked, i.e.
 *     j in [max(0, (c-1)*s), i].  No prior.
 *   - Further masks on the same machinery (no prior, N = sequence length):
 *       window_bidir: j in [max(0, i-k), min(N-1, i+k)] -- the local window
 *         exactly as the pi-Attention page states it, i-k..i+k (encoder use);
 *       ssplit: j in [floor(i/s)*s, i] -- the s-Split variant of the ECP page
 *         (section 2): the history cut into disjoint segments, causal inside;
 *       ecp_full: j in [max(0, (c-1)*s), min(N-1, (c+1)*s - 1)] -- the PAR
 *         block of the ECP page without the causal restriction (queries of
 *         half-segment c see all of half-segments c-1 and c).
 *
 *   score(i, j) = <q_i, k_j> / sqrt(d) + prior(i, j)
 *
 * Options of the *_ex entry points (the fused gate and epilogue variants):
 *   - a score scale other than 1/sqrt(d);
 *   - scaled cosine scores (the attention branch of the hybrid
 *     GSS-Transformer page, methodology item 1):
 *       score(i, j) = scale * <q_i, k_j> / (|q_i| |k_j|) + prior(i, j);
 *   - the gate computed from the query (pi-Attention section 2 item 3: a
 *     light per-token, per-head network -- an MLP -- produces alpha), on the
 *     query row as that network's input:
 *       two layers (hidden width H > 0, ReLU hidden layer):
 *         alpha_i = sigmoid( sum_u w2_hu * relu(<w1_hu, q_i> + b1_hu) + b2_h );
 *       or one linear layer (H = 0): alpha_i = sigmoid(<w1_h, q_i> + b1_h).
 *   The output gate o * sigmoid(g) of the LT2 page (section 3) is elementwise
 *   on the output and applied by the Python wrapper.
 *   o_i        = sum_j exp(score(i,j) - max) v_j / sum_j exp(score(i,j) - max)
 *
 * Everything is evaluated in double precision with libm exp/log.  Inputs are
 * fp32 arrays (bf16 inputs are widened exactly by the caller).  Grouped-query
 * attention ("Long-context modelling with a hybrid GSS-Transformer",
 * methodology item 1): query head h reads key/value head h / (Hq / Hkv).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_MODE_PI 0
#define ORC_MODE_WINDOW 1
#define ORC_MODE_ECP 2
#define ORC_MODE_WINDOW_BIDIR 3
#define ORC_MODE_SSPLIT 4
#define ORC_MODE_ECP_FULL 5

#define ORC_LOCAL 0
#define ORC_SKIP 1

#define ORC_OK 0
#define ORC_ERR_ARGS -1
#define ORC_ERR_ALPHA -2
#define ORC_ERR_NOMEM -3

static int64_t orc_max64(int64_t a, int64_t b) { return a > b ? a : b; }
static int64_t orc_min64(int64_t a, int64_t b) { return a < b ? a : b; }

/* Number of keys the key set of any query can hold (upper bound). */
int64_t orc_key_capacity(int mode, int64_t k_win, int64_t M, int64_t seg)
{
    if (mode == ORC_MODE_ECP || mode == ORC_MODE_ECP_FULL) return 2 * seg;
    if (mode == ORC_MODE_SSPLIT) return seg;
    if (mode == ORC_MODE_WINDOW) return k_win + 1;
    if (mode == ORC_MODE_WINDOW_BIDIR) return 2 * k_win + 1;
    return k_win + 1 + (M > 0 ? M : 0);
}

/*
 * Key set of query position i of a sequence of N positions, in ascending
 * order of position, with the label ORC_LOCAL or ORC_SKIP for each key.
 * Returns the number of keys, or -1 when cap is too small or the parameters
 * are invalid.
 *   PI / WINDOW: pi-Attention section 2 items 1-2; LT2 section 2.1.
 *   ECP: ECP section 2 (queries of the current half-segment, keys and values
 *   of the current and the previous half-segment), causal.
 *   WINDOW_BIDIR, SSPLIT, ECP_FULL: see the header comment.
 */
int64_t orc_key_set(int64_t i, int64_t N, int mode, int64_t k_win, int64_t pi, int64_t M,
                    int64_t seg, int64_t *keys, int32_t *labels, int64_t cap)
{
    int64_t n = 0, lo, hi = i, j, m;
    if (i < 0 || i >= N) return -1;
    if (mode == ORC_MODE_ECP || mode == ORC_MODE_ECP_FULL) {
        if (seg <= 0) return -1;
        lo = orc_max64(0, (i / seg - 1) * seg);
        if (mode == ORC_MODE_ECP_FULL) hi = orc_min64(N - 1, (i / seg + 1) * seg - 1);
    } else if (mode == ORC_MODE_SSPLIT) {
        if (seg <= 0) return -1;
        lo = (i / seg) * seg;
    } else if (mode == ORC_MODE_PI || mode == ORC_MODE_WINDOW || mode == ORC_MODE_WINDOW_BIDIR) {
        if (k_win < 0) return -1;
        lo = orc_max64(0, i - k_win);
        if (mode == ORC_MODE_WINDOW_BIDIR) hi = orc_min64(N - 1, i + k_win);
    } else {
        return -1;
    }
    /* Skip keys lie below the window: i - m*pi for m = M down to 1, keeping
       those at or above position 0 and strictly below the window start (a
       key inside the window belongs to the window). */
    if (mode == ORC_MODE_PI && M > 0) {
        if (pi <= 0) return -1;
        for (m = M; m >= 1; --m) {
            j = i - m * pi;
            if (j < 0 || j >= lo) continue;
            if (n >= cap) return -1;
            keys[n] = j;
            labels[n] = ORC_SKIP;
            ++n;
        }
    }
    for (j = lo; j <= hi; ++j) {
        if (n >= cap) return -1;
        keys[n] = j;
        labels[n] = ORC_LOCAL;
        ++n;
    }
    return n;
}

/*
 * One query row: softmax over the explicit key set with the log-prior, then
 * the weighted sum of value rows.  qrow has d entries; kmat/vmat point at row
 * 0 of the key/value head (row stride d).  log_local/log_skip are the priors
 * (0 for modes without a gate).  Writes d doubles to out.
 */
/* <q, k>, or the cosine <q, k> / (|q| |k|) when cosine is set. */
static double orc_dot(const float *qrow, const float *krow, int64_t d, int cosine)
{
    double dot = 0.0, qq = 0.0, kk = 0.0;
    int64_t c;
    for (c = 0; c < d; ++c) dot += (double)qrow[c] * (double)krow[c];
    if (!cosine) return dot;
    for (c = 0; c < d; ++c) {
        qq += (double)qrow[c] * (double)qrow[c];
        kk += (double)krow[c] * (double)krow[c];
    }
    return dot / (sqrt(qq) * sqrt(kk));
}

static void orc_row(const float *qrow, const float *kmat, const float *vmat,
                    int64_t d, double scale, int cosine, double log_local, double log_skip,
                    const int64_t *keys, const int32_t *labels, int64_t n,
                    double *score, double *out)
{
    double mx = -INFINITY, denom = 0.0;
    int64_t t, c;
    for (t = 0; t < n; ++t) {
        const float *krow = kmat + keys[t] * d;
        score[t] = orc_dot(qrow, krow, d, cosine) * scale + (labels[t] == ORC_LOCAL ? log_local : log_skip);
        if (score[t] > mx) mx = score[t];
    }
    for (c = 0; c < d; ++c) out[c] = 0.0;
    for (t = 0; t < n; ++t) {
        const float *vrow = vmat + keys[t] * d;
        double w = exp(score[t] - mx);
        denom += w;
        for (c = 0; c < d; ++c) out[c] += w * (double)vrow[c];
    }
    for (c = 0; c < d; ++c) out[c] /= denom;
}

static int orc_check_common(int64_t B, int64_t Hq, int64_t Hkv, int64_t d, int mode,
                            int64_t k_win, int64_t pi, int64_t M, int64_t seg)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || Hq % Hkv != 0) return ORC_ERR_ARGS;
    if (mode == ORC_MODE_ECP || mode == ORC_MODE_SSPLIT || mode == ORC_MODE_ECP_FULL)
        return seg > 0 ? ORC_OK : ORC_ERR_ARGS;
    if (mode != ORC_MODE_PI && mode != ORC_MODE_WINDOW && mode != ORC_MODE_WINDOW_BIDIR) return ORC_ERR_ARGS;
    if (k_win < 0) return ORC_ERR_ARGS;
    if (mode == ORC_MODE_PI && (M < 0 || (M > 0 && pi <= 0))) return ORC_ERR_ARGS;
    return ORC_OK;
}

/* Gate network of one query head (see the header): w1 [H][d] (or [d] when
   H = 0), b1 [H] (or one bias), w2 [H], b2 one bias.  NULL w1: no gate. */
typedef struct {
    const float *w1, *b1, *w2, *b2;
    int64_t hidden;
} orc_gate;

static orc_gate orc_gate_of_head(const float *gate_w, const float *gate_b, const float *gate_w2,
                                 const float *gate_b2, int64_t hidden, int64_t h, int64_t d)
{
    orc_gate g;
    g.hidden = hidden;
    if (gate_w == NULL) {
        g.w1 = g.b1 = g.w2 = g.b2 = NULL;
        return g;
    }
    if (hidden > 0) {
        g.w1 = gate_w + h * hidden * d;
        g.b1 = gate_b + h * hidden;
        g.w2 = gate_w2 + h * hidden;
        g.b2 = gate_b2 + h;
    } else {
        g.w1 = gate_w + h * d;
        g.b1 = gate_b + h;
        g.w2 = g.b2 = NULL;
    }
    return g;
}

/* Gate output z (before the sigmoid) for one query row. */
static double orc_gate_logit(const orc_gate *g, const float *qrow, int64_t d)
{
    int64_t c, u;
    if (g->hidden <= 0) {
        double z = (double)*g->b1;
        for (c = 0; c < d; ++c) z += (double)g->w1[c] * (double)qrow[c];
        return z;
    }
    {
        double z = (double)*g->b2;
        for (u = 0; u < g->hidden; ++u) {
            double a = (double)g->b1[u];
            for (c = 0; c < d; ++c) a += (double)g->w1[u * d + c] * (double)qrow[c];
            if (a > 0.0) z += (double)g->w2[u] * a; /* relu */
        }
        return z;
    }
}

/* Priors of one row.  alpha must lie in (0, 1]; alpha = 1 makes the skip
   prior log(0) = -inf, which removes the skip keys from the softmax.  With a
   gate network alpha comes from the query row instead (see orc_gate_logit). */
static int orc_priors_q(int mode, const float *alpha, int64_t at, const float *qrow, const orc_gate *gate,
                        int64_t d, double *lp, double *ls)
{
    double a;
    *lp = 0.0;
    *ls = 0.0;
    if (mode != ORC_MODE_PI) return ORC_OK;
    if (gate != NULL && gate->w1 != NULL) {
        const double z = orc_gate_logit(gate, qrow, d);
        a = 1.0 / (1.0 + exp(-z));
        *lp = log(a);
        *ls = log(1.0 - a);
        return ORC_OK;
    }
    if (alpha == NULL) return ORC_ERR_ALPHA;
    a = (double)alpha[at];
    if (!(a > 0.0 && a <= 1.0)) return ORC_ERR_ALPHA;
    *lp = log(a);
    *ls = log(1.0 - a); /* -inf at a == 1 */
    return ORC_OK;
}

static int orc_priors(int mode, const float *alpha, int64_t at, double *lp, double *ls)
{
    return orc_priors_q(mode, alpha, at, NULL, NULL, 0, lp, ls);
}

/*
 * Forward attention for a selection of query rows.
 *   q     [B, Hq, N, d]  fp32      k, v [B, Hkv, N, d] fp32
 *   alpha [B, Hq, N]     fp32 (PI only; may be NULL otherwise)
 *   sel   nsel flat row ids (b*Hq + h)*N + i, or NULL for every row in order
 *   out   [nsel, d] doubles (or [B, Hq, N, d] when sel is NULL)
 * Returns ORC_OK or a negative error code.
 */
int orc_fwd_rows_ex(const float *q, const float *k, const float *v, const float *alpha,
                    int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                    int mode, int64_t k_win, int64_t pi, int64_t M, int64_t seg,
                    double scale, int cosine, const float *gate_w, const float *gate_b,
                    const float *gate_w2, const float *gate_b2, int64_t gate_hidden,
                    const int64_t *sel, int64_t nsel, double *out)
{
    int64_t cap, total, r;
    int err = orc_check_common(B, Hq, Hkv, d, mode, k_win, pi, M, seg);
    if (err != ORC_OK || N <= 0) return ORC_ERR_ARGS;
    total = B * Hq * N;
    if (sel == NULL) nsel = total;
    cap = orc_key_capacity(mode, k_win, M, seg);
    err = ORC_OK;
#pragma omp parallel
    {
        int64_t *keys = (int64_t *)malloc((size_t)cap * sizeof(int64_t));
        int32_t *labels = (int32_t *)malloc((size_t)cap * sizeof(int32_t));
        double *score = (double *)malloc((size_t)cap * sizeof(double));
        int local_err = (keys && labels && score) ? ORC_OK : ORC_ERR_NOMEM;
#pragma omp for schedule(dynamic, 64)
        for (r = 0; r < nsel; ++r) {
            int64_t row = sel ? sel[r] : r, b, h, i, g, n;
            double lp, ls;
            orc_gate gate;
            if (local_err != ORC_OK) continue;
            if (row < 0 || row >= total) { local_err = ORC_ERR_ARGS; continue; }
            i = row % N;
            h = (row / N) % Hq;
            b = row / (N * Hq);
            g = h / (Hq / Hkv);
            gate = orc_gate_of_head(gate_w, gate_b, gate_w2, gate_b2, gate_hidden, h, d);
            if ((local_err = orc_priors_q(mode, alpha, row, q + row * d, &gate, d, &lp, &ls)) != ORC_OK) continue;
            n = orc_key_set(i, N, mode, k_win, pi, M, seg, keys, labels, cap);
            if (n <= 0) { local_err = ORC_ERR_ARGS; continue; }
            orc_row(q + row * d, k + (b * Hkv + g) * N * d, v + (b * Hkv + g) * N * d,
                    d, scale, cosine, lp, ls, keys, labels, n, score, out + r * d);
        }
        if (local_err != ORC_OK) {
#pragma omp critical
            err = local_err;
        }
        free(keys);
        free(labels);
        free(score);
    }
    return err;
}

int orc_fwd_rows(const float *q, const float *k, const float *v, const float *alpha,
                 int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                 int mode, int64_t k_win, int64_t pi, int64_t M, int64_t seg,
                 const int64_t *sel, int64_t nsel, double *out)
{
    return orc_fwd_rows_ex(q, k, v, alpha, B, Hq, Hkv, N, d, mode, k_win, pi, M, seg,
                           1.0 / sqrt((double)d), 0, NULL, NULL, NULL, NULL, 0, sel, nsel, out);
}

/*
 * Single-token decode over a KV cache: for every sequence b and query head h
 * the query sits at position i = lens[b] - 1 and attends the key set of i,
 * read from the cache rows [b, g, j, :] (the cache already holds the new
 * token's key and value).
 *   q     [B, Hq, d]          kc, vc [B, Hkv, Lmax, d]     lens [B] int32
 *   alpha [B, Hq] (PI only)   out    [B, Hq, d] doubles
 */
int orc_decode_ex(const float *q, const float *kc, const float *vc, const int32_t *lens,
                  const float *alpha, int64_t B, int64_t Hq, int64_t Hkv, int64_t Lmax,
                  int64_t d, int mode, int64_t k_win, int64_t pi, int64_t M, int64_t seg,
                  double scale, int cosine, const float *gate_w, const float *gate_b,
                    const float *gate_w2, const float *gate_b2, int64_t gate_hidden, double *out)
{
    int64_t cap, r;
    int err = orc_check_common(B, Hq, Hkv, d, mode, k_win, pi, M, seg);
    if (err != ORC_OK || Lmax <= 0) return ORC_ERR_ARGS;
    /* a decoded token has no later keys: the non-causal masks do not apply */
    if (mode == ORC_MODE_WINDOW_BIDIR || mode == ORC_MODE_ECP_FULL) return ORC_ERR_ARGS;
    for (r = 0; r < B; ++r)
        if (lens[r] < 1 || lens[r] > Lmax) return ORC_ERR_ARGS;
    cap = orc_key_capacity(mode, k_win, M, seg);
    err = ORC_OK;
#pragma omp parallel
    {
        int64_t *keys = (int64_t *)malloc((size_t)cap * sizeof(int64_t));
        int32_t *labels = (int32_t *)malloc((size_t)cap * sizeof(int32_t));
        double *score = (double *)malloc((size_t)cap * sizeof(double));
        int local_err = (keys && labels && score) ? ORC_OK : ORC_ERR_NOMEM;
#pragma omp for schedule(dynamic, 1)
        for (r = 0; r < B * Hq; ++r) {
            int64_t b = r / Hq, h = r % Hq, g = h / (Hq / Hkv), i = lens[b] - 1, n;
            double lp, ls;
            orc_gate gate;
            if (local_err != ORC_OK) continue;
            gate = orc_gate_of_head(gate_w, gate_b, gate_w2, gate_b2, gate_hidden, h, d);
            if ((local_err = orc_priors_q(mode, alpha, r, q + r * d, &gate, d, &lp, &ls)) != ORC_OK) continue;
            n = orc_key_set(i, i + 1, mode, k_win, pi, M, seg, keys, labels, cap);
            if (n <= 0) { local_err = ORC_ERR_ARGS; continue; }
            orc_row(q + r * d, kc + (b * Hkv + g) * Lmax * d, vc + (b * Hkv + g) * Lmax * d,
                    d, scale, cosine, lp, ls, keys, labels, n, score, out + r * d);
        }
        if (local_err != ORC_OK) {
#pragma omp critical
            err = local_err;
        }
        free(keys);
        free(labels);
        free(score);
    }
    return err;
}

int orc_decode(const float *q, const float *kc, const float *vc, const int32_t *lens,
               const float *alpha, int64_t B, int64_t Hq, int64_t Hkv, int64_t Lmax,
               int64_t d, int mode, int64_t k_win, int64_t pi, int64_t M, int64_t seg,
               double *out)
{
    return orc_decode_ex(q, kc, vc, lens, alpha, B, Hq, Hkv, Lmax, d, mode, k_win, pi, M, seg,
                         1.0 / sqrt((double)d), 0, NULL, NULL, NULL, NULL, 0, out);
}

/*
 * Log-sum-exp of the scores of selected rows (natural log units): the
 * softmax normaliser a training forward keeps for the backward pass,
 *   lse_i = log sum_{j in K(i)} exp(score(i, j)).
 *   sel/nsel as for orc_fwd_rows; out[nsel] doubles.
 */
int orc_lse_rows_ex(const float *q, const float *k, const float *alpha,
                    int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                    int mode, int64_t k_win, int64_t pi, int64_t M, int64_t seg,
                    double scale, int cosine, const float *gate_w, const float *gate_b,
                    const float *gate_w2, const float *gate_b2, int64_t gate_hidden,
                    const int64_t *sel, int64_t nsel, double *out)
{
    int64_t cap, total, r;
    int err = orc_check_common(B, Hq, Hkv, d, mode, k_win, pi, M, seg);
    if (err != ORC_OK || N <= 0) return ORC_ERR_ARGS;
    total = B * Hq * N;
    if (sel == NULL) nsel = total;
    cap = orc_key_capacity(mode, k_win, M, seg);
    err = ORC_OK;
#pragma omp parallel
    {
        int64_t *keys = (int64_t *)malloc((size_t)cap * sizeof(int64_t));
        int32_t *labels = (int32_t *)malloc((size_t)cap * sizeof(int32_t));
        int local_err = (keys && labels) ? ORC_OK : ORC_ERR_NOMEM;
#pragma omp for schedule(dynamic, 64)
        for (r = 0; r < nsel; ++r) {
            int64_t row = sel ? sel[r] : r, b, h, i, g, n, t;
            double lp, ls, mx = -INFINITY, sum = 0.0;
            orc_gate gate;
            const float *qrow, *kmat;
            if (local_err != ORC_OK) continue;
            if (row < 0 || row >= total) { local_err = ORC_ERR_ARGS; continue; }
            i = row % N;
            h = (row / N) % Hq;
            b = row / (N * Hq);
            g = h / (Hq / Hkv);
            gate = orc_gate_of_head(gate_w, gate_b, gate_w2, gate_b2, gate_hidden, h, d);
            if ((local_err = orc_priors_q(mode, alpha, row, q + row * d, &gate, d, &lp, &ls)) != ORC_OK) continue;
            n = orc_key_set(i, N, mode, k_win, pi, M, seg, keys, labels, cap);
            if (n <= 0) { local_err = ORC_ERR_ARGS; continue; }
            qrow = q + row * d;
            kmat = k + (b * Hkv + g) * N * d;
            for (t = 0; t < n; ++t) {
                const double sc = orc_dot(qrow, kmat + keys[t] * d, d, cosine) * scale +
                                  (labels[t] == ORC_LOCAL ? lp : ls);
                if (sc > mx) mx = sc;
            }
            for (t = 0; t < n; ++t)
                sum += exp(orc_dot(qrow, kmat + keys[t] * d, d, cosine) * scale +
                           (labels[t] == ORC_LOCAL ? lp : ls) - mx);
            out[r] = mx + log(sum);
        }
        if (local_err != ORC_OK) {
#pragma omp critical
            err = local_err;
        }
        free(keys);
        free(labels);
    }
    return err;
}

int orc_lse_rows(const float *q, const float *k, const float *alpha,
                 int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                 int mode, int64_t k_win, int64_t pi, int64_t M, int64_t seg,
                 const int64_t *sel, int64_t nsel, double *out)
{
    return orc_lse_rows_ex(q, k, alpha, B, Hq, Hkv, N, d, mode, k_win, pi, M, seg,
                           1.0 / sqrt((double)d), 0, NULL, NULL, NULL, NULL, 0, sel, nsel, out);
}

/*
 * Backward pass: gradients of a scalar loss L given dO = dL/dO, by the chain
 * rule through the definition above.  For every row (b, h, i), with
 * P_ij = softmax over K(i) of score(i, j):
 *   dP_ij   = <dO_i, v_j>
 *   D_i     = sum_j P_ij dP_ij
 *   dS_ij   = P_ij (dP_ij - D_i)              (dL / d score(i, j))
 *   dq_i    = sum_j dS_ij k_j / sqrt(d)
 *   dk_j   += dS_ij q_i / sqrt(d)             (over all rows and the GQA group)
 *   dv_j   += P_ij dO_i
 *   dalpha_i = sum_{j local} dS_ij / alpha_i - sum_{j skip} dS_ij / (1 - alpha_i)
 * (d score / d alpha is 1/alpha on local keys and -1/(1-alpha) on skip keys,
 * pi-Attention section 2 item 3).  The skip term is formed as
 * exp(score without prior - lse_i) (dP_ij - D_i), which equals
 * dS_ij / (1 - alpha_i) and stays finite at alpha = 1.
 * scale is the score scale (1/sqrt(d) for the method as defined; the
 * formulas above use it in place of 1/sqrt(d)).
 *   dO [B, Hq, N, d] doubles;  dq [B, Hq, N, d], dk, dv [B, Hkv, N, d] doubles;
 *   dalpha [B, Hq, N] doubles or NULL (PI only).
 * Work is split over (batch, KV head): one thread owns the dk/dv rows of a
 * KV head and every query row of its group.
 */
int orc_bwd(const float *q, const float *k, const float *v, const float *alpha, const double *dO,
            int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
            int mode, int64_t k_win, int64_t pi, int64_t M, int64_t seg, double scale,
            double *dq, double *dk, double *dv, double *dalpha)
{
    int64_t cap, u;
    int err = orc_check_common(B, Hq, Hkv, d, mode, k_win, pi, M, seg);
    if (err != ORC_OK || N <= 0) return ORC_ERR_ARGS;
    cap = orc_key_capacity(mode, k_win, M, seg);
    err = ORC_OK;
#pragma omp parallel
    {
        int64_t *keys = (int64_t *)malloc((size_t)cap * sizeof(int64_t));
        int32_t *labels = (int32_t *)malloc((size_t)cap * sizeof(int32_t));
        double *sc = (double *)malloc((size_t)cap * sizeof(double));
        double *pr = (double *)malloc((size_t)cap * sizeof(double));
        double *dp = (double *)malloc((size_t)cap * sizeof(double));
        int local_err = (keys && labels && sc && pr && dp) ? ORC_OK : ORC_ERR_NOMEM;
#pragma omp for schedule(dynamic, 1)
        for (u = 0; u < B * Hkv; ++u) {
            const int64_t b = u / Hkv, g = u % Hkv, grp = Hq / Hkv;
            const float *kmat = k + u * N * d, *vmat = v + u * N * d;
            double *dkm = dk + u * N * d, *dvm = dv + u * N * d;
            int64_t hh, i, t, c, n;
            if (local_err != ORC_OK) continue;
            for (t = 0; t < N * d; ++t) { dkm[t] = 0.0; dvm[t] = 0.0; }
            for (hh = 0; hh < grp && local_err == ORC_OK; ++hh) {
                const int64_t h = g * grp + hh;
                for (i = 0; i < N; ++i) {
                    const int64_t row = (b * Hq + h) * N + i;
                    const float *qrow = q + row * d;
                    const double *dorow = dO + row * d;
                    double lp, ls, mx = -INFINITY, sum = 0.0, lse, D = 0.0, da = 0.0;
                    if ((local_err = orc_priors(mode, alpha, row, &lp, &ls)) != ORC_OK) break;
                    n = orc_key_set(i, N, mode, k_win, pi, M, seg, keys, labels, cap);
                    if (n <= 0) { local_err = ORC_ERR_ARGS; break; }
                    for (t = 0; t < n; ++t) {
                        double dot = 0.0;
                        for (c = 0; c < d; ++c) dot += (double)qrow[c] * (double)kmat[keys[t] * d + c];
                        sc[t] = dot * scale;   /* without prior */
                        {
                            const double full = sc[t] + (labels[t] == ORC_LOCAL ? lp : ls);
                            if (full > mx) mx = full;
                        }
                    }
                    for (t = 0; t < n; ++t) sum += exp(sc[t] + (labels[t] == ORC_LOCAL ? lp : ls) - mx);
                    lse = mx + log(sum);
                    for (t = 0; t < n; ++t) {
                        double dot = 0.0;
                        pr[t] = exp(sc[t] + (labels[t] == ORC_LOCAL ? lp : ls) - lse);
                        for (c = 0; c < d; ++c) dot += dorow[c] * (double)vmat[keys[t] * d + c];
                        dp[t] = dot;
                        D += pr[t] * dot;
                    }
                    for (c = 0; c < d; ++c) dq[row * d + c] = 0.0;
                    for (t = 0; t < n; ++t) {
                        const double ds = pr[t] * (dp[t] - D);
                        const int64_t j = keys[t];
                        for (c = 0; c < d; ++c) {
                            dq[row * d + c] += ds * (double)kmat[j * d + c] * scale;
                            dkm[j * d + c] += ds * (double)qrow[c] * scale;
                            dvm[j * d + c] += pr[t] * dorow[c];
                        }
                        if (mode == ORC_MODE_PI) {
                            if (labels[t] == ORC_LOCAL) da += ds / (double)alpha[row];
                            else da -= exp(sc[t] - lse) * (dp[t] - D);
                        }
                    }
                    if (dalpha != NULL) dalpha[row] = da;
                }
            }
        }
        if (local_err != ORC_OK) {
#pragma omp critical
            err = local_err;
        }
        free(keys);
        free(labels);
        free(sc);
        free(pr);
        free(dp);
    }
    return err;
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
