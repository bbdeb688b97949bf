/*
 * oracle.c -- plain, slow, fp64 CPU reference for batched lossless
 * speculative-sampling verification and the first-order Markov-head draft.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or helper with the HIP
 * library: everything below is written out from the pages.
 *
 * Sources (web pages; cited by title and section / equation):
 *  [DART]   "DART：把草稿并行生成之后，还要补上哪些依赖？" -- reading note on
 *           DART (zhongzhuzhou.org, 2026-10-14).  Sec. 2.2 eq. (2) (expected
 *           accepted count); sec. 2.3 eq. (3)-(4) (accept with probability
 *           min(1, q/p), rejection mass R, residual r = [q-p]_+/R, identity
 *           min(p,q) + R r = q, no residual needed when R = 0); sec. 2.3 last
 *           paragraph (T = 0 means checking the target argmax).
 *  [DSPARK] DSpark paper guide (personal-site-bgy.pages.dev, ai-notes):
 *           "speculative decoding basics" (accept min(1, p^t/p^d), strict
 *           left-to-right prefix survival, bonus token), "Markov head"
 *           (p_k(v|x0,x<k) = softmax(U_k(v) + B(x_{k-1}, v)), B = W1 W2,
 *           rank r = 256, x0 = anchor), "confidence head" (analytic
 *           acceptance rate c* = 1 - 1/2 ||p^d - p^t||_1), "scheduler"
 *           (per-request verify length l_r).
 *  [SURVEY] "投机解码综述" (zhifeiding.github.io, 2026-11-02): sec. 1.2 step 3
 *           (accept the longest prefix, commit one corrected token at the first
 *           rejection), sec. 1.3 (greedy verification degenerates to a
 *           position-wise argmax comparison), sec. 2.1 (tau = N + 1).
 *
 * Notation: q = target distribution, p = draft distribution (the DART note's
 * letters).  Logit rows are [R][gamma+1][V] (target) and [R][gamma][V]
 * (draft), V contiguous; row i holds position i+1.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - temperature divides both logit rows before the softmax; T = 0 is greedy;
 *  - accept  <=>  q(x) >= p(x)  or  u_acc < q(x)/p(x)   (u in [0,1), strict <);
 *  - residual and bonus draws are inverse-CDF draws in ascending token id:
 *    token = min{ v : C(v) > u * W }, C the running sum of the weights, W the
 *    total; if no v qualifies (t rounded up to W) the last positive-weight id;
 *  - a rejection whose residual mass is exactly 0 samples q instead (eq. (3)
 *    says rejection cannot happen when R = 0, so this only arises by rounding);
 *  - the bonus comes from target row l_r; l_r = 0 commits one token from q of
 *    target row 0;
 *  - at T = 0: g_i = argmax (lowest id on ties), accept <=> x == g_i,
 *    c* = [argmax draft == g_i], Res = 1 - c*, committed token g_A, log q = 0;
 *  - per-position outputs beyond l_r (c*, Res) and beyond A (log q) are NaN,
 *    padded tokens are -1; an invalid request gets A = -1, all tokens -1 and
 *    NaN floats.
 *
 * Precision: every probability, sum and decision is fp64.  Inputs are fp32 or
 * bf16 (dtype 0 / 1) and convert exactly.  Each decision records its margin
 * (distance of the uniform from the decision boundary, relative to the total
 * weight for inverse-CDF draws); decisions with margin below tie_eps are near
 * ties and are reported, not graded.
 */
#include <float.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

/* Valid temperatures: 0 (greedy) or a finite value in [T_MIN, T_MAX]. */
#define T_MIN 1e-30
#define T_MAX 1e30

/* ------------------------------------------------------------------ */
/* element access                                                      */
/* ------------------------------------------------------------------ */

static double bf16_bits_to_double(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Logit v of the row starting at element offset `row_off` of `base`. */
static double logit_at(const void *base, int dtype, size_t row_off, int v) {
    if (dtype == ORACLE_BF16)
        return bf16_bits_to_double(((const uint16_t *)base)[row_off + (size_t)v]);
    return (double)((const float *)base)[row_off + (size_t)v];
}

/* A logit is acceptable if it is finite or -inf (a masked token). */
static int logit_ok(double z) { return !isnan(z) && z != INFINITY; }

static int temperature_ok(float t) {
    if (isnan(t) || isinf(t) || t < 0.0f) return 0;
    if (t == 0.0f) return 1;
    return (double)t >= T_MIN && (double)t <= T_MAX;
}

static int uniform_ok(float u) { return !isnan(u) && u >= 0.0f && u < 1.0f; }

/* ------------------------------------------------------------------ */
/* temperature softmax (DART note sec. 2.3: q and p are the two        */
/* distributions; DSpark guide: each position's softmax)               */
/* ------------------------------------------------------------------ */

/* prob[v] = exp(z_v/T - m) / S with m = max_v z_v/T and S = sum_v exp(z_v/T - m).
 * Returns 0 if the row holds a NaN or +inf logit or is entirely -inf.
 * On success *m_out = m and *logS_out = log S, so log prob_v = z_v/T - m - log S. */
static int softmax_row(const void *base, int dtype, size_t row_off, int V, double T,
                       double *prob, double *m_out, double *logS_out) {
    double m = -INFINITY;
    for (int v = 0; v < V; ++v) {
        double z = logit_at(base, dtype, row_off, v);
        if (!logit_ok(z)) return 0;
        double a = z / T;
        if (a > m) m = a;
    }
    if (m == -INFINITY) return 0;
    double S = 0.0;
    for (int v = 0; v < V; ++v) {
        double a = logit_at(base, dtype, row_off, v) / T;
        prob[v] = exp(a - m);
        S += prob[v];
    }
    for (int v = 0; v < V; ++v) prob[v] /= S;
    if (m_out) *m_out = m;
    if (logS_out) *logS_out = log(S);
    return 1;
}

/* argmax with the lowest index on ties; -1 if the row holds a NaN or +inf
 * logit or is entirely -inf. */
static int argmax_row(const void *base, int dtype, size_t row_off, int V) {
    int best = -1;
    double bv = -INFINITY;
    for (int v = 0; v < V; ++v) {
        double z = logit_at(base, dtype, row_off, v);
        if (!logit_ok(z)) return -1;
        if (z > bv) {
            best = v;
            bv = z;
        }
    }
    return best;
}

/* ------------------------------------------------------------------ */
/* inverse-CDF draw in ascending token id                              */
/* ------------------------------------------------------------------ */

/* token = min{v : C(v) > t}, t = u * W, C(v) = sum_{v' <= v} w_v'.  If no v
 * qualifies, the last id with positive weight.  *margin = min(t - C(v-1),
 * C(v) - t) / W, where the lower distance is ignored when C(v-1) == 0 (all
 * earlier weights are exactly zero, so no rounding can move the boundary).
 * Returns -1 if W is not positive. */
static int inverse_cdf(const double *w, int V, double u, double *margin) {
    double W = 0.0;
    for (int v = 0; v < V; ++v) W += w[v];
    if (!(W > 0.0)) return -1;
    double t = u * W;
    double C = 0.0;
    for (int v = 0; v < V; ++v) {
        double prev = C;
        C += w[v];
        if (C > t) {
            double lo = (prev > 0.0) ? (t - prev) : INFINITY;
            double hi = C - t;
            *margin = (lo < hi ? lo : hi) / W;
            return v;
        }
    }
    for (int v = V - 1; v >= 0; --v) {
        if (w[v] > 0.0) {
            *margin = 0.0;
            return v;
        }
    }
    return -1;
}

/* ------------------------------------------------------------------ */
/* batched verification                                                */
/* ------------------------------------------------------------------ */

static void mark_invalid(int r, int gamma, int32_t *out_tokens, int32_t *out_num_accepted,
                         double *out_cstar, double *out_resid, double *out_logq) {
    for (int j = 0; j <= gamma; ++j) {
        out_tokens[(size_t)r * (gamma + 1) + j] = -1;
        if (out_logq) out_logq[(size_t)r * (gamma + 1) + j] = NAN;
    }
    for (int i = 0; i < gamma; ++i) {
        if (out_cstar) out_cstar[(size_t)r * gamma + i] = NAN;
        if (out_resid) out_resid[(size_t)r * gamma + i] = NAN;
    }
    out_num_accepted[r] = -1;
}

/*
 * One request r.  Returns 1 if the request is valid, 0 otherwise.
 *
 * For T > 0 (DART note sec. 2.3, DSpark guide "basics"):
 *   for i < l:  c*_i = sum_v min(p_i, q_i)           (DSpark confidence label;
 *               Res_i = sum_v [q_i - p_i]_+           = 1 - c*_i by eq. (3))
 *   accept_i  <=>  q_i(x) >= p_i(x)  or  u_acc[i] < q_i(x)/p_i(x),  x = x_{i+1}
 *   A = number of leading accepts (strict left-to-right prefix survival)
 *   A < l:  residual draw at row A from [q_A - p_A]_+ (eq. (3)-(4)) with u_smp[A]
 *   A = l:  bonus draw from q_l (target row l) with u_smp[l]
 * For T = 0 (DART note sec. 2.3; survey sec. 1.3): argmax comparison.
 *
 * margin_min: smallest margin over the decisions taken; first_tie: index of the
 * first decision whose margin is below tie_eps (accept decision at row j -> j,
 * the final draw -> gamma + 1), -1 if none.
 */
static int verify_one(const void *zt, int t_dtype, const void *zd, int d_dtype,
                      const int32_t *draft_tokens, const int32_t *verify_len,
                      const float *temperature, const float *u_accept, const float *u_sample,
                      int r, int gamma, int V, double tie_eps,
                      int32_t *out_tokens, int32_t *out_num_accepted, double *out_cstar,
                      double *out_resid, double *out_logq, double *out_margin_min,
                      int32_t *out_first_tie, double *q, double *p, double *w) {
    const int l = verify_len[r];
    const float Tf = temperature[r];
    double margin_min = INFINITY;
    int first_tie = -1;
    out_margin_min[r] = INFINITY;
    out_first_tie[r] = -1;

    if (l < 0 || l > gamma || !temperature_ok(Tf)) return 0;
    for (int i = 0; i < l; ++i) {
        int x = draft_tokens[(size_t)r * gamma + i];
        if (x < 0 || x >= V) return 0;
    }
    const size_t trow0 = (size_t)r * (gamma + 1) * (size_t)V;
    const size_t drow0 = (size_t)r * gamma * (size_t)V;
    int32_t *tok = out_tokens + (size_t)r * (gamma + 1);
    double *cs = out_cstar ? out_cstar + (size_t)r * gamma : NULL;
    double *rs = out_resid ? out_resid + (size_t)r * gamma : NULL;
    double *lq = out_logq ? out_logq + (size_t)r * (gamma + 1) : NULL;

    for (int j = 0; j <= gamma; ++j) {
        tok[j] = -1;
        if (lq) lq[j] = NAN;
    }
    for (int i = 0; i < gamma; ++i) {
        if (cs) cs[i] = NAN;
        if (rs) rs[i] = NAN;
    }

    if (Tf == 0.0f) {
        /* Greedy verification: position-wise argmax comparison. */
        int A = 0, rejected = 0;
        for (int i = 0; i < l; ++i) {
            int g = argmax_row(zt, t_dtype, trow0 + (size_t)i * V, V);
            int gd = argmax_row(zd, d_dtype, drow0 + (size_t)i * V, V);
            if (g < 0 || gd < 0) return 0;
            if (cs) cs[i] = (gd == g) ? 1.0 : 0.0;
            if (rs) rs[i] = (gd == g) ? 0.0 : 1.0;
            if (!rejected) {
                if (draft_tokens[(size_t)r * gamma + i] == g) {
                    tok[A] = g;
                    if (lq) lq[A] = 0.0;
                    ++A;
                } else {
                    rejected = 1;
                }
            }
        }
        int g = argmax_row(zt, t_dtype, trow0 + (size_t)A * V, V);
        if (g < 0) return 0;
        /* bonus row l must be valid even when A < l (it is read by the call) */
        if (A < l && argmax_row(zt, t_dtype, trow0 + (size_t)l * V, V) < 0) return 0;
        tok[A] = g;
        if (lq) lq[A] = 0.0;
        out_num_accepted[r] = A;
        out_margin_min[r] = margin_min;
        out_first_tie[r] = first_tie;
        return 1;
    }

    const double T = (double)Tf;
    /* uniforms that the request may read */
    for (int i = 0; i < l; ++i)
        if (!uniform_ok(u_accept[(size_t)r * gamma + i])) return 0;
    for (int j = 0; j <= l; ++j)
        if (!uniform_ok(u_sample[(size_t)r * (gamma + 1) + j])) return 0;

    /* Rows 0..l-1: c*, Res (DSpark confidence label; DART eq. (3)) and the
     * left-to-right accept tests with prefix survival.  Every row the call
     * reads must be valid, so rows after the first rejection are still read. */
    double mq, lSq;
    int A = 0, alive = 1;
    for (int i = 0; i < l; ++i) {
        if (!softmax_row(zt, t_dtype, trow0 + (size_t)i * V, V, T, q, &mq, &lSq)) return 0;
        if (!softmax_row(zd, d_dtype, drow0 + (size_t)i * V, V, T, p, NULL, NULL)) return 0;
        double smin = 0.0, sres = 0.0;
        for (int v = 0; v < V; ++v) {
            smin += (p[v] < q[v]) ? p[v] : q[v];
            sres += (q[v] > p[v]) ? (q[v] - p[v]) : 0.0;
        }
        if (cs) cs[i] = smin;
        if (rs) rs[i] = sres;
        if (!alive) continue;
        const int x = draft_tokens[(size_t)r * gamma + i];
        const double ratio = q[x] / p[x]; /* +inf when p[x] == 0 */
        const double u = (double)u_accept[(size_t)r * gamma + i];
        const int accept = (q[x] >= p[x]) || (u < ratio);
        const double mg = fabs(u - (ratio < 1.0 ? ratio : 1.0));
        if (mg < margin_min) margin_min = mg;
        if (first_tie < 0 && mg < tie_eps) first_tie = i;
        if (!accept) {
            alive = 0;
            continue;
        }
        tok[A] = x;
        if (lq) lq[A] = logit_at(zt, t_dtype, trow0 + (size_t)i * V, x) / T - mq - lSq;
        ++A;
    }
    /* the bonus row l is read by the call even when a rejection came first */
    if (!softmax_row(zt, t_dtype, trow0 + (size_t)l * V, V, T, q, &mq, &lSq)) return 0;

    /* final draw: residual at row A (A < l) or bonus from target row l */
    const double us = (double)u_sample[(size_t)r * (gamma + 1) + A];
    softmax_row(zt, t_dtype, trow0 + (size_t)A * V, V, T, q, &mq, &lSq);
    int token;
    double mg = INFINITY;
    if (A < l) {
        softmax_row(zd, d_dtype, drow0 + (size_t)A * V, V, T, p, NULL, NULL);
        for (int v = 0; v < V; ++v) w[v] = (q[v] > p[v]) ? (q[v] - p[v]) : 0.0;
        token = inverse_cdf(w, V, us, &mg);
        if (token < 0) token = inverse_cdf(q, V, us, &mg); /* residual mass 0 */
    } else {
        token = inverse_cdf(q, V, us, &mg);
    }
    if (token < 0) return 0;
    if (mg < margin_min) margin_min = mg;
    if (first_tie < 0 && mg < tie_eps) first_tie = gamma + 1;
    tok[A] = token;
    if (lq) lq[A] = logit_at(zt, t_dtype, trow0 + (size_t)A * V, token) / T - mq - lSq;
    out_num_accepted[r] = A;
    out_margin_min[r] = margin_min;
    out_first_tie[r] = first_tie;
    return 1;
}

/* Returns the number of invalid requests; -1 on allocation failure. */
int oracle_verify_batch(const void *zt, int t_dtype, const void *zd, int d_dtype,
                        const int32_t *draft_tokens, const int32_t *verify_len,
                        const float *temperature, const float *u_accept, const float *u_sample,
                        int R, int gamma, int V, double tie_eps,
                        int32_t *out_tokens, int32_t *out_num_accepted, double *out_cstar,
                        double *out_resid, double *out_logq, double *out_margin_min,
                        int32_t *out_first_tie) {
    double *q = (double *)malloc(sizeof(double) * (size_t)V);
    double *p = (double *)malloc(sizeof(double) * (size_t)V);
    double *w = (double *)malloc(sizeof(double) * (size_t)V);
    if (!q || !p || !w) {
        free(q); free(p); free(w);
        return -1;
    }
    int bad = 0;
    for (int r = 0; r < R; ++r) {
        int ok = verify_one(zt, t_dtype, zd, d_dtype, draft_tokens, verify_len, temperature,
                            u_accept, u_sample, r, gamma, V, tie_eps, out_tokens,
                            out_num_accepted, out_cstar, out_resid, out_logq, out_margin_min,
                            out_first_tie, q, p, w);
        if (!ok) {
            mark_invalid(r, gamma, out_tokens, out_num_accepted, out_cstar, out_resid, out_logq);
            out_margin_min[r] = INFINITY;
            out_first_tie[r] = -1;
            ++bad;
        }
    }
    free(q); free(p); free(w);
    return bad;
}

/* ------------------------------------------------------------------ */
/* analytic acceptance rate for arbitrary row pairs                    */
/* ------------------------------------------------------------------ */

/* c*_n = sum_v min(p_n, q_n) = 1 - 1/2 ||p_n - q_n||_1 (DSpark confidence
 * label), Res_n = sum_v [q_n - p_n]_+ (DART eq. (3)).  At T = 0 the one-hot
 * limit: c* = [argmax p == argmax q].  Invalid rows give NaN.  Returns the
 * number of invalid rows. */
int oracle_tv_accept_rate(const void *zd, const void *zt, int dtype, const float *temperature,
                          int N, int V, double *out_cstar, double *out_resid) {
    double *q = (double *)malloc(sizeof(double) * (size_t)V);
    double *p = (double *)malloc(sizeof(double) * (size_t)V);
    if (!q || !p) {
        free(q); free(p);
        return -1;
    }
    int bad = 0;
    for (int n = 0; n < N; ++n) {
        const size_t off = (size_t)n * V;
        const float Tf = temperature[n];
        double c = NAN, res = NAN;
        if (temperature_ok(Tf)) {
            if (Tf == 0.0f) {
                int g = argmax_row(zt, dtype, off, V), gd = argmax_row(zd, dtype, off, V);
                if (g >= 0 && gd >= 0) {
                    c = (g == gd) ? 1.0 : 0.0;
                    res = 1.0 - c;
                }
            } else if (softmax_row(zt, dtype, off, V, (double)Tf, q, NULL, NULL) &&
                       softmax_row(zd, dtype, off, V, (double)Tf, p, NULL, NULL)) {
                c = 0.0;
                res = 0.0;
                for (int v = 0; v < V; ++v) {
                    c += (p[v] < q[v]) ? p[v] : q[v];
                    res += (q[v] > p[v]) ? (q[v] - p[v]) : 0.0;
                }
            }
        }
        if (isnan(c)) ++bad;
        out_cstar[n] = c;
        if (out_resid) out_resid[n] = res;
    }
    free(q); free(p);
    return bad;
}

/* ------------------------------------------------------------------ */
/* first-order Markov-head draft (DSpark guide, "Markov head")          */
/* ------------------------------------------------------------------ */

/*
 * For each request r and k = 1..gamma, serially:
 *   b_v   = sum_{j < rank} W1[x_{k-1}][j] * W2[j][v]   (exact fp64, ascending j)
 *   l_v   = float( U[r][k-1][v] + b_v )                 (stored draft logit)
 *   p     = softmax(l / T)                              (fp64 from the stored l)
 *   x_k   = inverse-CDF draw from p with u_draft[r][k-1]
 * with x_0 = anchor[r].  At T = 0, x_k = argmax l (lowest id on ties).
 * The draft distribution is the softmax of the stored fp32 logits, which is
 * the distribution verification later compares against.
 * U: [R][gamma][V] (u_dtype), W1: [V][rank], W2: [rank][V] (w_dtype).
 * Outputs: out_tokens [R][gamma], out_logits [R][gamma][V] fp32 (nullable),
 * out_margin_min / out_first_tie [R] as in verification (first_tie = k-1 of
 * the first near-tie draw).  Invalid requests get tokens -1.  Returns the
 * number of invalid requests.
 */
int oracle_markov_draft(const void *U, int u_dtype, const void *W1, const void *W2, int w_dtype,
                        const int32_t *anchor, const float *temperature, const float *u_draft,
                        int R, int gamma, int V, int rank, double tie_eps, int32_t *out_tokens,
                        float *out_logits, double *out_margin_min, int32_t *out_first_tie) {
    double *b = (double *)malloc(sizeof(double) * (size_t)V);
    double *p = (double *)malloc(sizeof(double) * (size_t)V);
    float *l32 = (float *)malloc(sizeof(float) * (size_t)V);
    if (!b || !p || !l32) {
        free(b); free(p); free(l32);
        return -1;
    }
    int bad = 0;
    for (int r = 0; r < R; ++r) {
        const float Tf = temperature[r];
        int x_prev = anchor[r];
        int ok = temperature_ok(Tf) && x_prev >= 0 && x_prev < V;
        double margin_min = INFINITY;
        int first_tie = -1;
        for (int k = 1; k <= gamma && ok; ++k) {
            for (int v = 0; v < V; ++v) b[v] = 0.0;
            for (int j = 0; j < rank; ++j) {
                double a = logit_at(W1, w_dtype, (size_t)x_prev * rank, j);
                for (int v = 0; v < V; ++v) b[v] += a * logit_at(W2, w_dtype, (size_t)j * V, v);
            }
            const size_t uoff = ((size_t)r * gamma + (k - 1)) * (size_t)V;
            for (int v = 0; v < V; ++v) {
                double uv = logit_at(U, u_dtype, uoff, v);
                l32[v] = (float)(uv + b[v]);
                if (!logit_ok((double)l32[v])) ok = 0;
            }
            if (!ok) break;
            if (out_logits)
                memcpy(out_logits + uoff, l32, sizeof(float) * (size_t)V);
            int x;
            if (Tf == 0.0f) {
                x = argmax_row(l32, ORACLE_F32, 0, V);
            } else {
                const float uu = u_draft[(size_t)r * gamma + (k - 1)];
                if (!uniform_ok(uu) ||
                    !softmax_row(l32, ORACLE_F32, 0, V, (double)Tf, p, NULL, NULL)) {
                    ok = 0;
                    break;
                }
                double mg = INFINITY;
                x = inverse_cdf(p, V, (double)uu, &mg);
                if (mg < margin_min) margin_min = mg;
                if (first_tie < 0 && mg < tie_eps) first_tie = k - 1;
            }
            if (x < 0) {
                ok = 0;
                break;
            }
            out_tokens[(size_t)r * gamma + (k - 1)] = x;
            x_prev = x;
        }
        if (!ok) {
            for (int k = 0; k < gamma; ++k) out_tokens[(size_t)r * gamma + k] = -1;
            margin_min = INFINITY;
            first_tie = -1;
            ++bad;
        }
        out_margin_min[r] = margin_min;
        out_first_tie[r] = first_tie;
    }
    free(b); free(p); free(l32);
    return bad;
}

/* Inverse-CDF helper exposed for the pins: token for weights w at uniform u. */
int oracle_inverse_cdf(const double *w, int V, double u, double *margin) {
    return inverse_cdf(w, V, u, margin);
}
