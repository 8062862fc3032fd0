/*
 * spkv_oracle.c -- plain, slow, fp64 CPU oracle for Self-Pruned Key-Value
 * attention (SP-KV).  TEST INFRASTRUCTURE ONLY: it is loaded by the tests,
 * by the package's smoke check and by the benchmark's CPU-baseline leg, and
 * by nothing on the product path.  It shares no code, header or constant
 * with the HIP library.
 *
 * Source of every formula: "Self-Pruned Key-Value Attention: learning when to
 * write by predicting future utility" (arXiv 2605.14037), section 2.1,
 * equations (1)-(4), the paragraph "efficient implementation at
 * deployment" at the end of section 2.1, the post-hoc threshold of
 * section 3.3 (hybrids paragraph), the per-head statistics of Table 1
 * and section 4, and the soft relaxation of Eq. (5)-(6).
 *
 * Precision: every input is a float32 array whose values are exact (bf16
 * values are a subset of float32); each value is widened to double on use and
 * all arithmetic is done in double, in fixed index order.
 *
 * Parity status of each function is stated in its comment; every one is
 * pinned by tests that do not call this file's arithmetic a second time
 * (closed forms, library routines, brute force, worked examples).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define SPKV_ORACLE_VERSION 1

int spkv_oracle_version(void) { return SPKV_ORACLE_VERSION; }

int spkv_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * O1 -- utility gate, SP-KV section 2.1, Eq. (1) and Eq. (2).
 *
 *   a_j     = max(0, sum_i W1[j,i] * h_i + b1[j])        (first MLP layer, ReLU)
 *   logit_k = sum_j W2[k,j] * a_j + b2[k]                 (second layer: one
 *                                                         output per key head)
 *   u_k     = 1 / (1 + exp(-logit_k))                     Eq. (1)
 *   z_k     = 1 if u_k >= tau else 0                      Eq. (2)
 *
 * The page leaves the predictor as "a 2-layer MLP" per layer and key head;
 * the shared d_model -> d_hidden (ReLU) -> n_kv form with biases is the
 * reading used throughout (a bank of per-head MLPs is the case of a
 * block-diagonal W2).  A NaN utility compares false, so it gives z = 0.
 *
 * H  [n_rows, ld_h] (row r at H + r*ld_h, first d_model entries used)
 * W1 [d_hidden, d_model], b1 [d_hidden], W2 [n_kv, d_hidden], b2 [n_kv]
 * u_out / logit_out [n_rows, n_kv] doubles (either may be NULL),
 * z_out [n_rows, n_kv] bytes (may be NULL).
 */
int spkv_oracle_gate(int64_t n_rows, int64_t d_model, int64_t d_hidden,
                     int64_t n_kv, const float *H, int64_t ld_h,
                     const float *W1, const float *b1, const float *W2,
                     const float *b2, double tau, double *u_out,
                     double *logit_out, uint8_t *z_out, int n_threads)
{
    if (n_rows < 0 || d_model <= 0 || d_hidden <= 0 || n_kv <= 0 || ld_h < d_model)
        return -1;
    if (d_hidden > 1024)
        return -2; /* the activations of one row live in a stack buffer */
    if (n_threads < 1)
        n_threads = 1;
    int64_t r;
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(n_threads)
#endif
    for (r = 0; r < n_rows; ++r) {
        const float *h = H + r * ld_h;
        double act[1024];
        for (int64_t j = 0; j < d_hidden; ++j) {
            double acc = 0.0;
            for (int64_t i = 0; i < d_model; ++i)
                acc += (double)W1[j * d_model + i] * (double)h[i];
            acc += (double)b1[j];
            /* ReLU; a NaN is passed on (NaN < 0 is false), so a corrupted
             * hidden state yields u = NaN and therefore z = 0 */
            act[j] = (acc < 0.0) ? 0.0 : acc;
        }
        for (int64_t k = 0; k < n_kv; ++k) {
            double logit = 0.0;
            for (int64_t j = 0; j < d_hidden; ++j)
                logit += (double)W2[k * d_hidden + j] * act[j];
            logit += (double)b2[k];
            double u = 1.0 / (1.0 + exp(-logit));
            if (logit_out)
                logit_out[r * n_kv + k] = logit;
            if (u_out)
                u_out[r * n_kv + k] = u;
            if (z_out)
                z_out[r * n_kv + k] = (uint8_t)(u >= tau ? 1 : 0);
        }
    }
    return 0;
}

/*
 * O2 -- the sparse persistent cache of SP-KV (section 2.1, deployment
 * paragraph): only pairs with z = 1 are kept, in token order.  For one
 * sequence whose rows sit at positions pos0, pos0+1, ..., this is the stable
 * filter of the rows with z[s,g] = 1, for each key head g:
 *
 *   pos_out[g * n_rows + i] = pos0 + s_i   where s_0 < s_1 < ... are the rows
 *                                          with z[s, g] = 1
 *   len_out[g]              = number of such rows
 *
 * The cached key and value of entry i are the input rows s_i, unchanged.
 */
int spkv_oracle_compact(int64_t n_rows, int64_t n_kv, const uint8_t *z,
                        int64_t pos0, int64_t *pos_out, int64_t *len_out)
{
    if (n_rows < 0 || n_kv <= 0)
        return -1;
    for (int64_t g = 0; g < n_kv; ++g) {
        int64_t n = 0;
        for (int64_t s = 0; s < n_rows; ++s) {
            if (z[s * n_kv + g]) {
                pos_out[g * n_rows + n] = pos0 + s;
                ++n;
            }
        }
        len_out[g] = n;
    }
    return 0;
}

/*
 * O5 -- re-thresholding a persistent cache.  SP-KV section 2.1 (deployment
 * paragraph) lets the sparse cache be rebuilt from time to time, and section
 * 3.3 (hybrids paragraph) notes that sparsity can be changed after training
 * by moving the threshold.  An entry kept at threshold tau carries its
 * utility u (Eq. 1); at a new threshold tau2 the keep decision of Eq. (2) is
 * taken again on that stored value.  For one (sequence, key head) list of n
 * entries in logical (token) order this is the stable filter
 *
 *   idx_out[j] = i_j   where i_0 < i_1 < ... are the entries with u[i] >= tau2
 *   *len_out   = number of such entries
 *
 * A NaN utility fails the comparison and is dropped, as in Eq. (2) for the
 * gate.  The rebuilt entry j is entry i_j unchanged (key, value, position,
 * utility).  The comparison is made in double on the exactly converted float
 * values, which decides the same way as a float comparison.
 */
int spkv_oracle_rethreshold(int64_t n, const float *u, double tau2,
                            int64_t *idx_out, int64_t *len_out)
{
    if (n < 0)
        return -1;
    int64_t kept = 0;
    for (int64_t i = 0; i < n; ++i) {
        const double ui = (double)u[i];
        if (ui >= tau2) {
            idx_out[kept] = i;
            ++kept;
        }
    }
    *len_out = kept;
    return 0;
}

/*
 * O7 -- the training-time soft relaxation of the gate, SP-KV section 2.1,
 * Eq. (5)-(6).  Each pair gets alpha_s = sigmoid((u_s - tau) / beta)
 * (Eq. 5) and the hard mask of Eq. (4) is replaced by an additive score
 *
 *   M_soft(t, s) = 0                    if 0 <= t - s < w   (window)
 *                = c * (alpha_s - 1)    otherwise, for s <= t
 *
 * (Eq. 6; positions after t stay excluded, as in Eq. 4), so that for query
 * row t, query head h and key head g = h / group:
 *
 *   x_s = scale * q . k_s + M_soft(t, s)   over s in [0, t]
 *   out = sum_s softmax(x)_s v_s,   lse = log sum_s exp(x_s)
 *
 * u is [T, n_kv] float (the utilities of Eq. 1).  Written literally: alpha is
 * formed first and 1 is subtracted (in double).  Same layouts and row rules
 * as O3.
 */
int spkv_oracle_soft_attention(int64_t T, int64_t n_q, int64_t n_kv, int64_t hd,
                               int64_t w, const float *Q, const int64_t *t_rows,
                               int64_t n_rows, const float *K, const float *V,
                               int64_t ld_kv, const float *u, double tau,
                               double beta, double c, double scale,
                               double *out, double *lse, int n_threads)
{
    if (T < 0 || n_q <= 0 || n_kv <= 0 || hd <= 0 || w < 1 || n_q % n_kv || !(beta > 0.0))
        return -1;
    for (int64_t i = 0; i < n_rows; ++i)
        if (t_rows[i] < 0 || t_rows[i] >= T)
            return -1;
    if (n_threads < 1)
        n_threads = 1;
    const int64_t group = n_q / n_kv;
    int64_t job;
    const int64_t n_jobs = n_rows * n_q;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads)
#endif
    for (job = 0; job < n_jobs; ++job) {
        const int64_t i = job / n_q;
        const int64_t h = job % n_q;
        const int64_t t = t_rows[i];
        const int64_t g = h / group;
        const float *q = Q + (i * n_q + h) * hd;
        double *o = out + (i * n_q + h) * hd;
        /* every causal key takes part; the scores carry the mask of Eq. (6) */
        double m = -INFINITY;
        for (int64_t s = 0; s <= t; ++s) {
            const float *k = K + s * ld_kv + g * hd;
            double x = 0.0;
            for (int64_t e = 0; e < hd; ++e)
                x += (double)q[e] * (double)k[e];
            x *= scale;
            if (t - s >= w) {
                const double alpha = 1.0 / (1.0 + exp(-((double)u[s * n_kv + g] - tau) / beta));
                x += c * (alpha - 1.0);
            }
            if (x > m)
                m = x;
        }
        for (int64_t e = 0; e < hd; ++e)
            o[e] = 0.0;
        double l = 0.0;
        for (int64_t s = 0; s <= t; ++s) {
            const float *k = K + s * ld_kv + g * hd;
            const float *v = V + s * ld_kv + g * hd;
            double x = 0.0;
            for (int64_t e = 0; e < hd; ++e)
                x += (double)q[e] * (double)k[e];
            x *= scale;
            if (t - s >= w) {
                const double alpha = 1.0 / (1.0 + exp(-((double)u[s * n_kv + g] - tau) / beta));
                x += c * (alpha - 1.0);
            }
            const double p = exp(x - m);
            l += p;
            for (int64_t e = 0; e < hd; ++e)
                o[e] += p * (double)v[e];
        }
        for (int64_t e = 0; e < hd; ++e)
            o[e] /= l;
        if (lse)
            lse[i * n_q + h] = m + log(l);
    }
    return 0;
}

/*
 * O6 -- per-head utility statistics.  SP-KV reports the density of a model
 * as the fraction of the pairs outside the local window that the gate keeps
 * (Table 1 caption), and uses the mean learned utility of each head to pick
 * the heads that stay global in a local/global hybrid (section 1,
 * contribution 2; section 4).  Over a set of n_rows gate outputs
 * (u[s, g], z[s, g]) this is, for each key head g,
 *
 *   u_sum[g] += sum over s of u[s, g]     (in row order, in double)
 *   kept[g]  += number of s with z[s, g] != 0
 *
 * accumulated into the outputs so that a long sequence can be fed in parts;
 * mean utility = u_sum / rows, density = kept / rows.  A NaN utility makes
 * its head's sum NaN.  u or z may be NULL (that half is skipped).
 */
int spkv_oracle_head_stats(int64_t n_rows, int64_t n_kv, const float *u,
                           const uint8_t *z, double *u_sum, int64_t *kept)
{
    if (n_rows < 0 || n_kv <= 0)
        return -1;
    for (int64_t g = 0; g < n_kv; ++g) {
        double acc = 0.0;
        int64_t cnt = 0;
        for (int64_t s = 0; s < n_rows; ++s) {
            if (u)
                acc += (double)u[s * n_kv + g];
            if (z && z[s * n_kv + g])
                ++cnt;
        }
        if (u)
            u_sum[g] += acc;
        if (z)
            kept[g] += cnt;
    }
    return 0;
}

/*
 * O3 -- windowed-plus-gated softmax attention, SP-KV section 2.1, Eq. (3)-(4),
 * evaluated directly on the full, uncompacted sequence.
 *
 * For query row i at position t = t_rows[i] and query head h, key head
 * g = h / (n_q / n_kv) (contiguous grouped-query heads):
 *
 *   visible(s) = (0 <= t - s < w)  or  (z[s,g] = 1 and s <= t),  s in [0, t]
 *   x_s        = scale * sum_e q[e] * k_s[e]          (scale = 1/sqrt(d_k))
 *   m          = max over visible s of x_s
 *   p_s        = exp(x_s - m),   l = sum p_s
 *   out        = sum p_s v_s / l,  lse = m + log(l)
 *
 * Q   [n_rows, n_q, hd] (float), t_rows [n_rows]
 * K,V row s, head g at  K + s*ld_kv + g*hd  (so [T, n_kv, hd] has ld_kv = n_kv*hd)
 * z   [T, n_kv] bytes, row s at z + s*n_kv
 * out [n_rows, n_q, hd] doubles, lse [n_rows, n_q] doubles (lse may be NULL)
 * Rows whose t is outside [0, T) are rejected (return -1, nothing written).
 */
int spkv_oracle_attention(int64_t T, int64_t n_q, int64_t n_kv, int64_t hd,
                          int64_t w, const float *Q, const int64_t *t_rows,
                          int64_t n_rows, const float *K, const float *V,
                          int64_t ld_kv, const uint8_t *z, double scale,
                          double *out, double *lse, int n_threads)
{
    if (T < 0 || n_q <= 0 || n_kv <= 0 || hd <= 0 || w < 1 || n_q % n_kv)
        return -1;
    for (int64_t i = 0; i < n_rows; ++i)
        if (t_rows[i] < 0 || t_rows[i] >= T)
            return -1;
    if (n_threads < 1)
        n_threads = 1;
    const int64_t group = n_q / n_kv;
    int64_t job;
    const int64_t n_jobs = n_rows * n_q;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads)
#endif
    for (job = 0; job < n_jobs; ++job) {
        const int64_t i = job / n_q;
        const int64_t h = job % n_q;
        const int64_t t = t_rows[i];
        const int64_t g = h / group;
        const float *q = Q + (i * n_q + h) * hd;
        double *o = out + (i * n_q + h) * hd;

        /* pass 1: the largest visible score */
        double m = -INFINITY;
        for (int64_t s = 0; s <= t; ++s) {
            int in_window = (t - s) < w;
            int kept = z[s * n_kv + g] != 0;
            if (!(in_window || kept))
                continue;
            const float *k = K + s * ld_kv + g * hd;
            double x = 0.0;
            for (int64_t e = 0; e < hd; ++e)
                x += (double)q[e] * (double)k[e];
            x *= scale;
            if (x > m)
                m = x;
        }
        /* pass 2: normaliser and weighted sum of values */
        for (int64_t e = 0; e < hd; ++e)
            o[e] = 0.0;
        double l = 0.0;
        for (int64_t s = 0; s <= t; ++s) {
            int in_window = (t - s) < w;
            int kept = z[s * n_kv + g] != 0;
            if (!(in_window || kept))
                continue;
            const float *k = K + s * ld_kv + g * hd;
            const float *v = V + s * ld_kv + g * hd;
            double x = 0.0;
            for (int64_t e = 0; e < hd; ++e)
                x += (double)q[e] * (double)k[e];
            x *= scale;
            double p = exp(x - m);
            l += p;
            for (int64_t e = 0; e < hd; ++e)
                o[e] += p * (double)v[e];
        }
        for (int64_t e = 0; e < hd; ++e)
            o[e] /= l;
        if (lse)
            lse[i * n_q + h] = m + log(l);
    }
    return 0;
}

/*
 * Row counts of the visible set of O3, |visible(t)| for head g, for each
 * query row -- the same predicate as O3, counted.  Used to state the
 * expected log-normaliser when every key is zero (then lse = log |visible|).
 */
int spkv_oracle_visible_count(int64_t T, int64_t n_kv, int64_t w,
                              const uint8_t *z, const int64_t *t_rows,
                              int64_t n_rows, int64_t g, int64_t *count_out)
{
    if (T < 0 || n_kv <= 0 || w < 1 || g < 0 || g >= n_kv)
        return -1;
    for (int64_t i = 0; i < n_rows; ++i) {
        const int64_t t = t_rows[i];
        if (t < 0 || t >= T)
            return -1;
        int64_t c = 0;
        for (int64_t s = 0; s <= t; ++s)
            if ((t - s) < w || z[s * n_kv + g])
                ++c;
        count_out[i] = c;
    }
    return 0;
}

/*
 * O8 -- the low-rank sink-attention gate of Fast KVzip, an alternative
 * utility predictor f behind the same keep decision, from the page
 * "Fast KVzip: efficient and accurate LLM inference with gated KV eviction"
 * (a summary of arXiv 2601.17668), section "core method" (the gate paragraph)
 * and section "reproduction" (S = 16, D' = 16).  The page describes it in
 * words only; the reading written out here (every step is a reading):
 *
 *   for key head h, with G = query heads per key head and D' = d_key:
 *     q_{h,g} = Wq_{h,g} x      (D' values, g = 0 .. G-1)   linear, no bias
 *     k_h     = Wk_h x          (D' values)                  linear, no bias
 *     s_{h,j}                   (S learned sink keys, D' values each)
 *     a_{h,g} = exp(q.k / sqrt(D')) / (exp(q.k / sqrt(D')) + sum_j exp(q.s_j / sqrt(D')))
 *               -- the attention the token's own key receives against the
 *               sinks, a softmax over 1 + S keys
 *     u_h     = max_g a_{h,g}  -- the page's training target is the largest
 *               attention a pair receives, so the G query heads of a group
 *               are combined by their maximum
 *     z_h     = 1 if u_h >= tau else 0   (Eq. (2) of SP-KV, unchanged)
 *
 * W [n_kv, (G + 1) * d_key, d_model]: per head, the G * d_key query rows
 * (g-major) then the d_key key rows.  sinks [n_kv, n_sinks, d_key].
 * Evaluated as written, in double; the softmax is formed with its maximum
 * subtracted (the same value).  A NaN gives z = 0.
 * u_out [n_rows, n_kv] doubles (may be NULL), z_out bytes (may be NULL).
 * Parity pins: zero hidden state -> 1 / (1 + S); no sinks -> 1; sinks far
 * against q -> 1; G = S = 1 -> the logistic of the score difference; sink
 * and query-head permutations; the bilinear rescaling of q against k and
 * the sinks.  Parity against Fast KVzip itself is unpinned: the page prints
 * no formula and no worked example.
 */
int spkv_oracle_sink_gate(int64_t n_rows, int64_t d_model, int64_t n_kv, int64_t G,
                          int64_t d_key, int64_t n_sinks, const float *H, int64_t ld_h,
                          const float *W, const float *sinks, double tau, double *u_out,
                          uint8_t *z_out, int n_threads)
{
    if (n_rows < 0 || d_model <= 0 || n_kv <= 0 || G <= 0 || d_key <= 0 || n_sinks < 0 ||
        ld_h < d_model || d_key > 256 || G > 64 || n_sinks > 1024)
        return -1;
    if (n_threads < 1)
        n_threads = 1;
    const int64_t per_head = (G + 1) * d_key;
    const double inv_sqrt = 1.0 / sqrt((double)d_key);
    int64_t r;
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(n_threads)
#endif
    for (r = 0; r < n_rows; ++r) {
        const float *x = H + r * ld_h;
        double proj[65 * 256]; /* (G + 1) * d_key values of one head */
        for (int64_t h = 0; h < n_kv; ++h) {
            const float *Wh = W + h * per_head * d_model;
            for (int64_t o = 0; o < per_head; ++o) {
                double acc = 0.0;
                for (int64_t i = 0; i < d_model; ++i)
                    acc += (double)Wh[o * d_model + i] * (double)x[i];
                proj[o] = acc;
            }
            const double *k = proj + G * d_key;
            double u = -1.0;
            int nan = 0;
            for (int64_t g = 0; g < G; ++g) {
                const double *q = proj + g * d_key;
                double own = 0.0;
                for (int64_t e = 0; e < d_key; ++e)
                    own += q[e] * k[e];
                own *= inv_sqrt;
                double m = own;
                double sc[1024];
                for (int64_t j = 0; j < n_sinks; ++j) {
                    const float *s = sinks + (h * n_sinks + j) * d_key;
                    double d = 0.0;
                    for (int64_t e = 0; e < d_key; ++e)
                        d += q[e] * (double)s[e];
                    sc[j] = d * inv_sqrt;
                    if (sc[j] > m)
                        m = sc[j];
                }
                double den = exp(own - m);
                const double num = den;
                for (int64_t j = 0; j < n_sinks; ++j)
                    den += exp(sc[j] - m);
                const double a = num / den;
                if (a != a)
                    nan = 1;
                if (a > u)
                    u = a;
            }
            if (nan)
                u = NAN;
            if (u_out)
                u_out[r * n_kv + h] = u;
            if (z_out)
                z_out[r * n_kv + h] = (uint8_t)(u >= tau ? 1 : 0);
        }
    }
    return 0;
}
