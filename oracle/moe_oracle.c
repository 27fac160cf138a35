/*
 * Plain CPU oracle of the sparse Mixture-of-Experts FFN layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg use it.  It shares no code with the HIP
 * library and is written to be read against the pages, not to be fast.
 *
 * Sources (page title, then section):
 *   [SKILL]  "AI-Research-SKILLs MoE training guide" (discosf.com):
 *            sec. 3.1 basic MoE layer, sec. 4.1 data-flow figure,
 *            sec. 4.2 routing mechanisms, sec. 4.3 auxiliary loss and
 *            router z-loss, sec. 6.1 Mixtral block, sec. 7.1 DeepSeekMoE,
 *            sec. 8.2 capacity factor, sec. 10.1 monitoring metrics.
 *   [DIVE]   "MoE architecture deep dive: from routing to production
 *            inference" (juejin.cn): sec. 1.1 dense FFN to sparse MoE,
 *            sec. 1.2 gating network, sec. 1.3 top-K routing,
 *            sec. 2.2 auxiliary load-balancing loss, sec. 2.3 expert
 *            capacity, sec. 2.4 auxiliary-loss-free balancing,
 *            sec. 3 DeepSeek-V3 shared expert.
 *   [GROUP]  "The expert group activated per token" (wmrh.cn):
 *            sec. 3.1 anatomy of an MoE layer (FFN formula, router),
 *            sec. 4.4 routing monitors (entropy).
 *   [DIVE]   also sec. 4 (expert-collapse threshold of 40 percent).
 *
 * Precision: every floating-point step is IEEE double, except the
 * balancing-bias update, which the layer defines on float32 state.
 * Inputs arrive as float32 words (dtype 0) or bfloat16 bit patterns
 * (dtype 1) and are widened exactly to double.
 *
 * Tie rule (the pages give none): among equal probabilities the lower
 * expert index ranks first.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_ERR_ARG -1
#define OR_ERR_MISSING_EXPERT -2

/* Exact widening of one stored element to double: dtype 0 = float32,
 * 1 = bfloat16 bit patterns, 3 = double (dequantised weights). */
static double ld(const void *p, size_t i, int dtype)
{
    if (dtype == 0)
        return (double)((const float *)p)[i];
    if (dtype == 3)
        return ((const double *)p)[i];
    uint32_t bits = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* One OCP 8-bit floating-point E4M3 code as a double (exact): sign bit,
 * four exponent bits with bias 7, three mantissa bits.  Exponent field 0
 * holds the subnormals m/8 * 2^-6; the all-ones exponent is still finite
 * except for mantissa 7, the NaN code; there are no infinities, and the
 * largest magnitude is 1.75 * 2^8 = 448.  The pages name FP8 weights
 * ("MoE inference with vLLM"; "AI-Research-SKILLs MoE training guide",
 * sec. 9) without a format; E4M3 is the OCP format the gfx950 matrix
 * cores read. */
double oracle_fp8_e4m3(uint8_t b)
{
    const int sign = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/* Per-output-channel dequantisation of an [N][K] FP8 matrix:
 * w[n][c] = e4m3(q[n][c]) * scale[n] (exact in double). */
void oracle_fp8_dequant(int N, int K, const uint8_t *q, const float *scale,
                        double *w)
{
    for (int n = 0; n < N; ++n)
        for (int c = 0; c < K; ++c)
            w[(size_t)n * K + c] =
                oracle_fp8_e4m3(q[(size_t)n * K + c]) * (double)scale[n];
}

/* Expert capacity: floor((tokens / experts) * capacity_factor).
 * [DIVE] sec. 2.3; [SKILL] sec. 8.2 (integer truncation of the same
 * quotient).  A negative factor means "no limit" and returns -1. */
int oracle_capacity(int T, int E, double cf)
{
    if (cf < 0.0 || E <= 0)
        return -1;
    return (int)floor(((double)T / (double)E) * cf);
}

/* Router logits and softmax probabilities for every token.
 *   logit[t,e] = sum_c x[t,c] * Wr[e,c] + add[e] - sub[e]
 *   prob[t,:]  = softmax(logit[t,:])
 * [DIVE] sec. 1.2 (gate_weights = Softmax(x . W_g)); [SKILL] sec. 3.1
 * (router nn.Linear, which carries an additive bias); [DIVE] sec. 2.4
 * (adjusted_logits_i = logits_i - b_i).  add and sub may be NULL. */
void oracle_router(int T, int d, int E, int dtype, const void *x,
                   const void *wr, const float *add, const float *sub,
                   double *logits, double *probs)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        double *lg = logits + (size_t)t * E;
        double *pr = probs + (size_t)t * E;
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int c = 0; c < d; ++c)
                acc += ld(x, (size_t)t * d + c, dtype) *
                       ld(wr, (size_t)e * d + c, dtype);
            if (add)
                acc += (double)add[e];
            if (sub)
                acc -= (double)sub[e];
            lg[e] = acc;
        }
        double m = lg[0];
        for (int e = 1; e < E; ++e)
            if (lg[e] > m)
                m = lg[e];
        double s = 0.0;
        for (int e = 0; e < E; ++e)
            s += exp(lg[e] - m);
        for (int e = 0; e < E; ++e)
            pr[e] = exp(lg[e] - m) / s;
    }
}

/* Top-k selection and renormalisation.
 * The k largest probabilities in descending order (ties: lower index),
 * then w_j = p_j / sum of the k selected, so the weights sum to one.
 * [DIVE] sec. 1.3 steps 2-3; [SKILL] sec. 3.1 and sec. 4.2 (top-2 with
 * renormalisation).  margin[t] = p_(k) - p_(k+1), +inf when k == E. */
void oracle_topk(int T, int E, int k, const double *probs, int32_t *idx,
                 double *w, double *margin)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const double *pr = probs + (size_t)t * E;
        char *taken = (char *)calloc((size_t)E, 1);
        double sum = 0.0;
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || pr[e] > pr[best]))
                    best = e;
            taken[best] = 1;
            idx[(size_t)t * k + j] = best;
            sum += pr[best];
        }
        for (int j = 0; j < k; ++j)
            w[(size_t)t * k + j] = pr[idx[(size_t)t * k + j]] / sum;
        if (margin) {
            if (k >= E) {
                margin[t] = INFINITY;
            } else {
                int next = -1;
                for (int e = 0; e < E; ++e)
                    if (!taken[e] && (next < 0 || pr[e] > pr[next]))
                        next = e;
                margin[t] = pr[idx[(size_t)t * k + k - 1]] - pr[next];
            }
        }
        free(taken);
    }
}

/* Renormalised weights of a given selection (used when a checker adopts a
 * different but equally valid choice at a near-tie): w_j = p[sel_j] / sum. */
void oracle_renorm_selection(int T, int E, int k, const double *probs,
                             const int32_t *idx, double *w)
{
    for (int t = 0; t < T; ++t) {
        double sum = 0.0;
        for (int j = 0; j < k; ++j)
            sum += probs[(size_t)t * E + idx[(size_t)t * k + j]];
        for (int j = 0; j < k; ++j)
            w[(size_t)t * k + j] =
                probs[(size_t)t * E + idx[(size_t)t * k + j]] / sum;
    }
}

/* Counting, capacity and dispatch.
 *   count[e]  = number of (t, j) with idx[t,j] == e        ([SKILL] 4.3,
 *               the bincount of the selected indices)
 *   kept[e]   = min(count[e], C), C = capacity or unlimited ([DIVE] 2.3)
 *   offset[e] = sum of kept[e'] over e' < e; offset[E] = total kept
 * Assignments are visited in token order, then slot order.  The r-th
 * assignment to expert e (r counted from 0) is kept when r < C and is
 * given slot offset[e] + r; otherwise it overflows: slot_of = -1, and the
 * token skips that expert (its residual passes through, [DIVE] 2.3).
 * slot_token[s] is the token of slot s; unused slots hold -1. */
int oracle_dispatch(int T, int E, int k, int capacity, const int32_t *idx,
                    int32_t *counts, int32_t *kept, int32_t *offsets,
                    int32_t *slot_token, int32_t *slot_of)
{
    for (int e = 0; e < E; ++e)
        counts[e] = 0;
    for (size_t a = 0; a < (size_t)T * k; ++a) {
        int e = idx[a];
        if (e < 0 || e >= E)
            return OR_ERR_ARG;
        counts[e] += 1;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) {
        kept[e] = (capacity >= 0 && counts[e] > capacity) ? capacity
                                                          : counts[e];
        offsets[e + 1] = offsets[e] + kept[e];
    }
    for (size_t s = 0; s < (size_t)T * k; ++s)
        slot_token[s] = -1;
    int32_t *seen = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            int e = idx[(size_t)t * k + j];
            int r = seen[e]++;
            if (capacity < 0 || r < capacity) {
                int s = offsets[e] + r;
                slot_token[s] = t;
                slot_of[(size_t)t * k + j] = s;
            } else {
                slot_of[(size_t)t * k + j] = -1;
            }
        }
    }
    free(seen);
    return OR_OK;
}

/* Load-balance statistics.
 *   p_i   = mean over tokens of prob[t,i]         ([DIVE] 2.2; [SKILL] 4.3)
 *   f_i   = count_i / (T * k), before capacity     ([SKILL] 4.3: bincount
 *           divided by the number of selected indices)
 *   L_aux = alpha * E * sum_i f_i * p_i            ([DIVE] 2.2)
 * With T == 0 everything is 0. */
void oracle_stats(int T, int E, int k, const double *probs,
                  const int32_t *counts, double alpha, double *f, double *p,
                  double *l_aux)
{
    double acc = 0.0;
    for (int e = 0; e < E; ++e) {
        double s = 0.0;
        for (int t = 0; t < T; ++t)
            s += probs[(size_t)t * E + e];
        p[e] = T > 0 ? s / (double)T : 0.0;
        f[e] = T > 0 ? (double)counts[e] / ((double)T * (double)k) : 0.0;
        acc += f[e] * p[e];
    }
    *l_aux = alpha * (double)E * acc;
}

/* Activation of the expert's hidden units.
 *   act 0  GELU(z) = z/2 (1 + erf(z/sqrt 2))  ([GROUP] sec. 3.1; [SKILL]
 *          sec. 3.1 Linear, GELU, Linear)
 *   act 1  SiLU(z) = z / (1 + e^-z)           ([SKILL] sec. 6.1 Mixtral
 *          block code: Linear, SiLU, Linear)
 *   act 2  SwiGLU: SiLU(gate) * up, gate = W1 x + b1, up = W3 x + b3
 *          ([SKILL] sec. 6.1 text: the Mixtral expert uses SwiGLU) */
static double silu(double z) { return z / (1.0 + exp(-z)); }

/* One expert applied to one token:
 *   z = W1 x + b1;  h = GELU(z) | SiLU(z) | SiLU(z) * (W3 x + b3)
 *   out = W2 h + b2
 * W1 and W3 are [d_ff][d], W2 is [d][d_ff] (nn.Linear layout); biases
 * may be NULL; w3 is used only by act 2. */
static void expert_apply(int d, int d_ff, int dtype, int wdtype, int act,
                         const double *xrow, const void *w1, const void *b1,
                         const void *w3, const void *b3, const void *w2,
                         const void *b2, double *h, double *out)
{
    for (int f = 0; f < d_ff; ++f) {
        double z = 0.0;
        for (int c = 0; c < d; ++c)
            z += ld(w1, (size_t)f * d + c, wdtype) * xrow[c];
        if (b1)
            z += ld(b1, (size_t)f, dtype);
        if (act == 0) {
            h[f] = 0.5 * z * (1.0 + erf(z / sqrt(2.0)));
        } else if (act == 1) {
            h[f] = silu(z);
        } else {
            double u = 0.0;
            for (int c = 0; c < d; ++c)
                u += ld(w3, (size_t)f * d + c, wdtype) * xrow[c];
            if (b3)
                u += ld(b3, (size_t)f, dtype);
            h[f] = silu(z) * u;
        }
    }
    for (int c = 0; c < d; ++c) {
        double o = 0.0;
        for (int f = 0; f < d_ff; ++f)
            o += ld(w2, (size_t)c * d_ff + f, wdtype) * h[f];
        if (b2)
            o += ld(b2, (size_t)c, dtype);
        out[c] = o;
    }
}

/* The layer output for a list of tokens, given their routing:
 *   y_t = sum over kept j of w[t,j] * Expert_{idx[t,j]}(x_t)  + Shared(x_t)
 * in slot order j = 0..k-1.  A dropped assignment (slot_of < 0) adds
 * nothing and the remaining weights are not renormalised.
 * [DIVE] sec. 1.1 (Output = sum of normalized_weight_i * Expert_i(x));
 * [DIVE] sec. 3 (Output = Shared_Expert(x) + sum of routed terms);
 * [SKILL] sec. 3.1 (weighted merge); [DIVE] sec. 2.3 (overflow skips the
 * experts).
 * Expert weights come as per-expert pointer tables; an entry may be NULL
 * for an expert that no listed token uses.  The weight matrices are in
 * wdtype (dtype, or 3 for dequantised double weights); x and the biases
 * in dtype.  slot_of may be NULL (no capacity limit: every assignment is
 * kept).  ws1 == NULL means no shared expert.  y is [n][d] double. */
int oracle_layer_rows(int n, const int32_t *tokens, int d, int k, int d_ff,
                      int dtype, int wdtype, int act, const void *x,
                      const int32_t *idx,
                      const double *w, const int32_t *slot_of,
                      const void *const *w1, const void *const *b1,
                      const void *const *w3, const void *const *b3,
                      const void *const *w2, const void *const *b2,
                      const void *ws1, const void *bs1, const void *ws3,
                      const void *bs3, const void *ws2, const void *bs2,
                      double *y)
{
    int status = OR_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < n; ++r) {
        int t = tokens[r];
        double *xrow = (double *)malloc(sizeof(double) * (size_t)d);
        double *h = (double *)malloc(sizeof(double) * (size_t)d_ff);
        double *o = (double *)malloc(sizeof(double) * (size_t)d);
        double *yr = y + (size_t)r * d;
        for (int c = 0; c < d; ++c) {
            xrow[c] = ld(x, (size_t)t * d + c, dtype);
            yr[c] = 0.0;
        }
        for (int j = 0; j < k; ++j) {
            size_t a = (size_t)t * k + j;
            if (slot_of && slot_of[a] < 0)
                continue;
            int e = idx[a];
            if (!w1[e] || !w2[e] || (act == 2 && !w3[e])) {
#pragma omp atomic write
                status = OR_ERR_MISSING_EXPERT;
                continue;
            }
            expert_apply(d, d_ff, dtype, wdtype, act, xrow, w1[e],
                         b1 ? b1[e] : NULL, w3 ? w3[e] : NULL,
                         b3 ? b3[e] : NULL, w2[e], b2 ? b2[e] : NULL, h, o);
            for (int c = 0; c < d; ++c)
                yr[c] += w[a] * o[c];
        }
        if (ws1) {
            expert_apply(d, d_ff, dtype, wdtype, act, xrow, ws1, bs1, ws3,
                         bs3, ws2, bs2, h, o);
            for (int c = 0; c < d; ++c)
                yr[c] += o[c];
        }
        free(xrow);
        free(h);
        free(o);
    }
    return status;
}

/* Expert-Choice routing: every expert picks its own C tokens.
 * [SKILL] sec. 4.2: the expert scores are the router output transposed to
 * (experts, tokens) and each expert takes the top capacity_per_expert
 * tokens; this balances the load exactly.  Readings taken where the page
 * is silent: the score is the router logit of (token, expert) (the page
 * transposes the router output itself, before any softmax); ties go to
 * the lower token index; the combine weight of a pick is the token's
 * softmax gate probability for that expert ([DIVE] sec. 1.2 gate
 * weights), not renormalised.  Slots are expert-major, C per expert, and
 * within an expert in ascending token order.  Outputs:
 *   slot_token[e*C + r]  the r-th picked token of expert e
 *   slot_of[t*E + e]     slot of (t, e), or -1 if e did not pick t
 *   gate[t*E + e]        probs[t,e] if e picked t, else 0
 *   picks[t]             how many experts picked t
 * Requires 0 <= C <= T. */
int oracle_expert_choice(int T, int E, int C, const double *logits,
                         const double *probs, int32_t *slot_token,
                         int32_t *slot_of, double *gate, int32_t *picks)
{
    if (C < 0 || C > T)
        return OR_ERR_ARG;
    for (size_t i = 0; i < (size_t)T * E; ++i) {
        gate[i] = 0.0;
        slot_of[i] = -1;
    }
    for (int t = 0; t < T; ++t)
        picks[t] = 0;
    char *taken = (char *)malloc((size_t)(T > 0 ? T : 1));
    for (int e = 0; e < E; ++e) {
        memset(taken, 0, (size_t)(T > 0 ? T : 1));
        for (int r = 0; r < C; ++r) {           /* C rounds of argmax */
            int best = -1;
            for (int t = 0; t < T; ++t)
                if (!taken[t] && (best < 0 ||
                                  logits[(size_t)t * E + e] >
                                      logits[(size_t)best * E + e]))
                    best = t;
            taken[best] = 1;
        }
        int r = 0;
        for (int t = 0; t < T; ++t)             /* ascending token order */
            if (taken[t]) {
                const int slot = e * C + r;
                slot_token[slot] = t;
                slot_of[(size_t)t * E + e] = slot;
                gate[(size_t)t * E + e] = probs[(size_t)t * E + e];
                picks[t] += 1;
                ++r;
            }
    }
    free(taken);
    return OR_OK;
}

/* Expert-Choice layer output for listed tokens:
 *   y_t = sum over experts e that picked t (ascending e) of
 *         gate[t,e] * Expert_e(x_t)   (+ Shared(x_t))
 * A token no expert picked gets 0 (plus the shared expert). */
int oracle_expert_choice_rows(int n, const int32_t *tokens, int d, int E,
                              int d_ff, int dtype, int wdtype, int act,
                              const void *x, const double *gate,
                              const void *const *w1, const void *const *b1,
                              const void *const *w3, const void *const *b3,
                              const void *const *w2, const void *const *b2,
                              const void *ws1, const void *bs1,
                              const void *ws3, const void *bs3,
                              const void *ws2, const void *bs2, double *y)
{
    int status = OR_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < n; ++r) {
        int t = tokens[r];
        double *xrow = (double *)malloc(sizeof(double) * (size_t)d);
        double *h = (double *)malloc(sizeof(double) * (size_t)d_ff);
        double *o = (double *)malloc(sizeof(double) * (size_t)d);
        double *yr = y + (size_t)r * d;
        for (int c = 0; c < d; ++c) {
            xrow[c] = ld(x, (size_t)t * d + c, dtype);
            yr[c] = 0.0;
        }
        for (int e = 0; e < E; ++e) {
            const double g = gate[(size_t)t * E + e];
            if (g == 0.0)
                continue;
            if (!w1[e] || !w2[e] || (act == 2 && !w3[e])) {
#pragma omp atomic write
                status = OR_ERR_MISSING_EXPERT;
                continue;
            }
            expert_apply(d, d_ff, dtype, wdtype, act, xrow, w1[e],
                         b1 ? b1[e] : NULL, w3 ? w3[e] : NULL,
                         b3 ? b3[e] : NULL, w2[e], b2 ? b2[e] : NULL, h, o);
            for (int c = 0; c < d; ++c)
                yr[c] += g * o[c];
        }
        if (ws1) {
            expert_apply(d, d_ff, dtype, wdtype, act, xrow, ws1, bs1, ws3,
                         bs3, ws2, bs2, h, o);
            for (int c = 0; c < d; ++c)
                yr[c] += o[c];
        }
        free(xrow);
        free(h);
        free(o);
    }
    return status;
}

/* Router and load monitors, six values:
 *   out[0] z-loss   = mean over tokens of (logsumexp_e logit[t,e])^2
 *                     ([SKILL] sec. 4.3, router z-loss)
 *   out[1] entropy  = mean over tokens of -sum_e p log2 p, in bits
 *                     ([GROUP] sec. 4.4, routing entropy vs log2(E))
 *   out[2] imbalance = max count / min count, +inf if an expert is empty
 *   out[3] utilization = experts with a nonzero count / E
 *   out[4] drop rate = assignments over capacity / (T k)
 *                     (out[2..4]: [SKILL] sec. 10.1)
 *   out[5] max share = largest count / T, the fraction of tokens sent to
 *                     the busiest expert ([DIVE] sec. 4, collapse above 0.4)
 * logits and probs are the router's (the adjusted logits actually used). */
void oracle_monitor(int T, int E, int k, const double *logits,
                    const double *probs, const int32_t *counts,
                    const int32_t *kept, double *out)
{
    double z = 0.0, h = 0.0;
    for (int t = 0; t < T; ++t) {
        const double *lg = logits + (size_t)t * E;
        const double *pr = probs + (size_t)t * E;
        double m = lg[0];
        for (int e = 1; e < E; ++e)
            if (lg[e] > m)
                m = lg[e];
        double s = 0.0;
        for (int e = 0; e < E; ++e)
            s += exp(lg[e] - m);
        const double lse = m + log(s);
        z += lse * lse;
        double ht = 0.0;
        for (int e = 0; e < E; ++e)
            if (pr[e] > 0.0)
                ht -= pr[e] * log2(pr[e]);
        h += ht;
    }
    out[0] = T > 0 ? z / T : 0.0;
    out[1] = T > 0 ? h / T : 0.0;
    int cmax = 0, cmin = 0, used = 0;
    long total_kept = 0;
    for (int e = 0; e < E; ++e) {
        if (e == 0 || counts[e] > cmax)
            cmax = counts[e];
        if (e == 0 || counts[e] < cmin)
            cmin = counts[e];
        if (counts[e] > 0)
            used += 1;
        total_kept += kept[e];
    }
    out[2] = cmin > 0 ? (double)cmax / (double)cmin : INFINITY;
    out[3] = (double)used / (double)E;
    const double n = (double)T * (double)k;
    out[4] = n > 0 ? (n - (double)total_kept) / n : 0.0;
    out[5] = T > 0 ? (double)cmax / (double)T : 0.0;
}

/* Auxiliary-loss-free balancing, one step on float32 state:
 *   b_i <- b_i + gamma * sign(count_i - target),  sign(0) = 0
 * An overloaded expert's bias grows, which lowers its adjusted logit
 * (logit - b_i) on the next call.  [DIVE] sec. 2.4; [SKILL] sec. 4.3. */
void oracle_bias_update(int E, const int32_t *counts, float target,
                        float gamma, float *bias)
{
    for (int e = 0; e < E; ++e) {
        float c = (float)counts[e];
        float sgn = c > target ? 1.0f : (c < target ? -1.0f : 0.0f);
        volatile float step = gamma * sgn; /* exactly +-gamma or 0 */
        bias[e] = bias[e] + step;
    }
}
