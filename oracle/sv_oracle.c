/*
 * sv_oracle.c -- plain CPU oracle for batched speculative-decoding verification.
 *
 * TEST INFRASTRUCTURE.  This file is the definition the HIP library is checked
 * against.  Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load it; the product path never calls it.  It shares no code,
 * header, table or constant with the HIP library.
 *
 * Style: scalar C11, every floating-point quantity in double, no SIMD, no
 * fast-math, requests processed independently (OpenMP over requests only).
 *
 * Sources (the pages this follows):
 *   [SD]  "推测解码：先猜几个 token，为什么答案仍然没变" (speculative decoding
 *         tutorial): section "一轮推测解码究竟发生什么" (one round: accept x_i with
 *         probability min(1, p_i(x_i)/q_i(x_i)), stop at the first rejection,
 *         sample the corrected residual there, or one extra token from the next
 *         position when all drafts pass; 1..gamma+1 tokens per round), section
 *         "为什么“猜错再改”不会偏离目标分布" (the identity q*min(1,p/q) = min(p,q),
 *         the residual p' = norm(max(0, p - q)), and the greedy rule: accept while
 *         the draft equals the target argmax, emit the target token at the first
 *         mismatch).
 *   [ADA] "AdaPLD: 面向高效无模型推测解码的自适应检索与重用", section 3.3
 *         (draft tree of a main copy path, branches and successors, verified
 *         with the standard tree-verification framework) and Algorithm 1
 *         (BuildDraftTree, VerifyAndAccept; an empty acceptance falls back to
 *         one autoregressive step; the bonus token is the last emitted one).
 *
 * Readings where the pages leave a step open (each is a choice, stated once):
 *   - p = softmax(Lp / T), q = softmax(Lq / T) with the same temperature T.
 *   - Acceptance draw u in [0,1): accept iff u < p/q; q(x) = 0 counts as r = +inf.
 *     A draft id outside [0, V) has r = 0 (always rejected).
 *   - Inverse CDF in ascending vocabulary order: with C(v) the running sum of
 *     the (unnormalised) mass d and Z = C(V-1), the token is the smallest v with
 *     d(v) > 0 and C(v) > u*Z; if none, the largest v with d(v) > 0.
 *   - If the residual mass Z is 0 (rounding only), the token is drawn from p_j
 *     itself with the same draw.
 *   - Every round emits n+1 tokens: the n accepted drafts and one target token
 *     (residual or bonus); AdaPLD's "empty acceptance => autoregressive step" is
 *     the n = 0 case.
 *   - Argmax ties go to the lowest index; values compare as doubles.
 *   - Tree: node j (j >= 1) is accepted iff its parent is accepted and its
 *     token equals argmax(parent row); the answer is the deepest accepted node,
 *     lowest index on ties; the bonus is argmax(row of that node); the root's
 *     own token is not verified.
 *
 * Margins: each consumed draw records its distance to the decision boundary it
 * was compared with (|u - r| for an acceptance test; for the sample draw the
 * distance from u to the two ends, C(v-1)/Z and C(v)/Z, of the chosen token's
 * cell).  The caller flags a request whose smallest margin is <= some epsilon.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1

/* ---- input decoding -------------------------------------------------------- */

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
static double orc_load(const void *base, int dtype, size_t idx) {
    if (dtype == ORC_BF16) {
        uint16_t h = ((const uint16_t *)base)[idx];
        uint32_t w = ((uint32_t)h) << 16;
        float f;
        memcpy(&f, &w, sizeof f);
        return (double)f;
    }
    return (double)((const float *)base)[idx];
}

/* ---- one distribution row ---------------------------------------------------- */

typedef struct {
    const void *base; /* tensor base */
    size_t off;       /* element offset of the row */
    int dtype;
    int V;
    double T;
    double m; /* max logit */
    double s; /* sum_v exp((L[v] - m) / T) */
} orc_row;

/* Softmax normaliser of L/T, written the plain two-pass way: max, then sum. */
static void orc_row_init(orc_row *r, const void *base, size_t off, int dtype, int V, double T) {
    r->base = base;
    r->off = off;
    r->dtype = dtype;
    r->V = V;
    r->T = T;
    double m = -INFINITY;
    for (int v = 0; v < V; ++v) {
        double x = orc_load(base, dtype, off + (size_t)v);
        if (x > m) m = x;
    }
    double s = 0.0;
    for (int v = 0; v < V; ++v) s += exp((orc_load(base, dtype, off + (size_t)v) - m) / T);
    r->m = m;
    r->s = s;
}

/* probability of token v under softmax(L/T) */
static double orc_prob(const orc_row *r, int v) {
    return exp((orc_load(r->base, r->dtype, r->off + (size_t)v) - r->m) / r->T) / r->s;
}

/* log sum_v exp(L[v]/T) */
static double orc_lse(const orc_row *r) { return r->m / r->T + log(r->s); }

/* Lowest index of the row maximum (strictly greater replaces). */
static int orc_argmax(const void *base, size_t off, int dtype, int V) {
    int best = 0;
    double bv = orc_load(base, dtype, off);
    for (int v = 1; v < V; ++v) {
        double x = orc_load(base, dtype, off + (size_t)v);
        if (x > bv) {
            bv = x;
            best = v;
        }
    }
    return best;
}

/* ---- inverse-CDF draw over an unnormalised mass -------------------------------- */

/* Mass of token v: the residual max(0, p(v) - q(v)) when q is given, else p(v). */
static double orc_mass(const orc_row *p, const orc_row *q, int v) {
    double pv = orc_prob(p, v);
    if (!q) return pv;
    double d = pv - orc_prob(q, v);
    return d > 0.0 ? d : 0.0;
}

/* Returns the chosen token; *margin receives the cell-edge distance of u.
 * *Z_out receives the total mass. */
static int orc_inverse_cdf(const orc_row *p, const orc_row *q, double u, double *margin,
                           double *Z_out) {
    int V = p->V;
    double Z = 0.0;
    for (int v = 0; v < V; ++v) Z += orc_mass(p, q, v);
    *Z_out = Z;
    if (!(Z > 0.0)) {
        *margin = 0.0;
        return -1;
    }
    double t = u * Z;
    double C = 0.0;
    int last_pos = -1;
    for (int v = 0; v < V; ++v) {
        double d = orc_mass(p, q, v);
        double Cprev = C;
        C += d;
        if (d > 0.0) {
            last_pos = v;
            if (C > t) {
                double a = fabs(u - Cprev / Z), b = fabs(u - C / Z);
                *margin = a < b ? a : b;
                return v;
            }
        }
    }
    *margin = 0.0; /* u*Z at or past the end: the clamp case is a boundary */
    return last_pos;
}

/* ---- stochastic chain ([SD] one round) ------------------------------------------ */

/*
 * target [B][K+1][V], draft [B][K][V] (dtype), draft_tokens [B][K],
 * u_accept [B][K], u_sample [B][K+1].  Row i of the target is the distribution
 * after the prefix and drafts 1..i (it scores draft i+1); row K is the bonus
 * row; draft row i is the q that proposed draft i+1.
 * Outputs: accept_len [B], out_tokens [B][K+1] (n+1 valid, -1 pad),
 * lse_target [B][K+1], lse_draft [B][K] (may be NULL), req_status [B]
 * (0 ok, 1 a draft id outside [0,V)), margin [B] (smallest margin over the
 * consumed draws), margin_accept [B] (smallest margin over the consumed
 * acceptance draws alone, +inf when there is none: these draws alone decide
 * accept_len), margin_sample [B] (the margin of the one sample draw), Z [B]
 * (mass of the distribution that was sampled).  Every margin output may be NULL.
 */
int sv_oracle_sample(const void *target, const void *draft, int dtype, const int32_t *draft_tokens,
                     const float *u_accept, const float *u_sample, int B, int K, int V, double T,
                     int32_t *accept_len, int32_t *out_tokens, double *lse_target,
                     double *lse_draft, int32_t *req_status, double *margin,
                     double *margin_accept, double *margin_sample, double *Zout, int nthreads) {
    if (B < 0 || K < 0 || V <= 0 || !(T > 0.0)) return 1;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int b = 0; b < B; ++b) {
        size_t tbase = (size_t)b * (size_t)(K + 1) * (size_t)V;
        size_t dbase = (size_t)b * (size_t)K * (size_t)V;
        const int32_t *x = draft_tokens + (size_t)b * K;
        int32_t *tok = out_tokens + (size_t)b * (K + 1);
        int status = 0;
        for (int i = 0; i < K; ++i)
            if (x[i] < 0 || x[i] >= V) status = 1;

        /* row log-sum-exp of every row, reported for all 2K+1 rows */
        if (lse_target)
            for (int i = 0; i <= K; ++i) {
                orc_row r;
                orc_row_init(&r, target, tbase + (size_t)i * V, dtype, V, T);
                lse_target[(size_t)b * (K + 1) + i] = orc_lse(&r);
            }
        if (lse_draft)
            for (int i = 0; i < K; ++i) {
                orc_row r;
                orc_row_init(&r, draft, dbase + (size_t)i * V, dtype, V, T);
                lse_draft[(size_t)b * K + i] = orc_lse(&r);
            }

        /* left-to-right acceptance; later drafts are discarded at the first rejection */
        double mg = INFINITY;
        int n = K;
        for (int i = 0; i < K; ++i) {
            double r;
            if (x[i] < 0 || x[i] >= V) {
                r = 0.0;
            } else {
                orc_row p, q;
                orc_row_init(&p, target, tbase + (size_t)i * V, dtype, V, T);
                orc_row_init(&q, draft, dbase + (size_t)i * V, dtype, V, T);
                double px = orc_prob(&p, x[i]), qx = orc_prob(&q, x[i]);
                r = (qx == 0.0) ? INFINITY : px / qx;
            }
            double u = (double)u_accept[(size_t)b * K + i];
            if (isfinite(r)) {
                double d = fabs(u - r);
                if (d < mg) mg = d;
            }
            if (!(u < r)) {
                n = i;
                break;
            }
        }

        /* one target token: residual at the rejected row, else the bonus row */
        orc_row p, q;
        orc_row_init(&p, target, tbase + (size_t)n * V, dtype, V, T);
        double us = (double)u_sample[(size_t)b * (K + 1) + n];
        double m2 = 0.0, Z = 0.0;
        int t;
        if (n < K) {
            orc_row_init(&q, draft, dbase + (size_t)n * V, dtype, V, T);
            t = orc_inverse_cdf(&p, &q, us, &m2, &Z);
            if (t < 0) { /* empty residual (rounding): draw from p_n with the same u */
                t = orc_inverse_cdf(&p, NULL, us, &m2, &Z);
                m2 = 0.0;
            }
        } else {
            t = orc_inverse_cdf(&p, NULL, us, &m2, &Z);
        }
        double ma = mg;
        if (m2 < mg) mg = m2;

        for (int i = 0; i < n; ++i) tok[i] = x[i];
        tok[n] = t;
        for (int i = n + 1; i <= K; ++i) tok[i] = -1;
        accept_len[b] = n;
        if (req_status) req_status[b] = status;
        if (margin) margin[b] = mg;
        if (margin_accept) margin_accept[b] = ma;
        if (margin_sample) margin_sample[b] = m2;
        if (Zout) Zout[b] = Z;
    }
    return 0;
}

/* ---- greedy chain ([SD] greedy rule) --------------------------------------------- */

/* target [B][K+1][V]; outputs as in sv_oracle_sample.  Rows after the first
 * mismatch are never read. */
int sv_oracle_greedy(const void *target, int dtype, const int32_t *draft_tokens, int B, int K,
                     int V, int32_t *accept_len, int32_t *out_tokens, int32_t *req_status,
                     int nthreads) {
    if (B < 0 || K < 0 || V <= 0) return 1;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int b = 0; b < B; ++b) {
        size_t tbase = (size_t)b * (size_t)(K + 1) * (size_t)V;
        const int32_t *x = draft_tokens + (size_t)b * K;
        int32_t *tok = out_tokens + (size_t)b * (K + 1);
        int status = 0;
        for (int i = 0; i < K; ++i)
            if (x[i] < 0 || x[i] >= V) status = 1;
        int n = K, a = -1;
        for (int i = 0; i <= K; ++i) {
            a = orc_argmax(target, tbase + (size_t)i * V, dtype, V);
            if (i == K || x[i] != a) {
                n = i;
                break;
            }
        }
        for (int i = 0; i < n; ++i) tok[i] = x[i];
        tok[n] = a;
        for (int i = n + 1; i <= K; ++i) tok[i] = -1;
        accept_len[b] = n;
        if (req_status) req_status[b] = status;
    }
    return 0;
}

/* ---- greedy tree ([ADA] section 3.3, Algorithm 1) ---------------------------------- */

/*
 * target [B][N][V]: row j is the target's prediction after the path ending at
 * node j.  node_tokens [B][N], parents [B][N] (parents[0] = -1,
 * 0 <= parents[j] < j).  Outputs: accept_len [B] = depth of the chosen node
 * (-1 for a malformed parent array), path_nodes [B][N] (node ids from depth 1
 * down to the chosen node, -1 pad), out_tokens [B][N] (their tokens, then the
 * bonus argmax of the chosen node's row, -1 pad), req_status [B] (0 ok, 1 a
 * node id outside [0,V), 2 malformed parents).
 */
int sv_oracle_tree(const void *target, int dtype, const int32_t *node_tokens,
                   const int32_t *parents, int B, int N, int V, int32_t *accept_len,
                   int32_t *path_nodes, int32_t *out_tokens, int32_t *req_status, int nthreads) {
    if (B < 0 || N < 1 || V <= 0) return 1;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int b = 0; b < B; ++b) {
        const int32_t *par = parents + (size_t)b * N;
        const int32_t *tk = node_tokens + (size_t)b * N;
        int32_t *pth = path_nodes + (size_t)b * N;
        int32_t *out = out_tokens + (size_t)b * N;
        for (int j = 0; j < N; ++j) pth[j] = out[j] = -1;

        int bad = (par[0] != -1);
        for (int j = 1; j < N && !bad; ++j)
            if (par[j] < 0 || par[j] >= j) bad = 1;
        if (bad) {
            accept_len[b] = -1;
            if (req_status) req_status[b] = 2;
            continue;
        }
        int status = 0;
        for (int j = 1; j < N; ++j)
            if (tk[j] < 0 || tk[j] >= V) status = 1;

        int *ok = (int *)malloc(sizeof(int) * (size_t)N);
        int *depth = (int *)malloc(sizeof(int) * (size_t)N);
        int *am = (int *)malloc(sizeof(int) * (size_t)N);
        size_t tbase = (size_t)b * (size_t)N * (size_t)V;
        for (int j = 0; j < N; ++j) am[j] = orc_argmax(target, tbase + (size_t)j * V, dtype, V);
        ok[0] = 1;
        depth[0] = 0;
        for (int j = 1; j < N; ++j) {
            int p = par[j];
            ok[j] = ok[p] && tk[j] == am[p];
            depth[j] = depth[p] + 1;
        }
        int best = 0;
        for (int j = 1; j < N; ++j)
            if (ok[j] && depth[j] > depth[best]) best = j;
        int d = depth[best];
        for (int j = best, k = d - 1; j != 0; j = par[j], --k) pth[k] = j;
        for (int k = 0; k < d; ++k) out[k] = tk[pth[k]];
        out[d] = am[best];
        accept_len[b] = d;
        if (req_status) req_status[b] = status;
        free(ok);
        free(depth);
        free(am);
    }
    return 0;
}

/* ---- per-row statistics, exposed for checks ---------------------------------------- */

/* For `rows` consecutive rows of length V: max, softmax normaliser s and lse. */
int sv_oracle_row_stats(const void *logits, int dtype, int rows, int V, double T, double *m,
                        double *s, double *lse) {
    if (rows < 0 || V <= 0 || !(T > 0.0)) return 1;
    for (int i = 0; i < rows; ++i) {
        orc_row r;
        orc_row_init(&r, logits, (size_t)i * V, dtype, V, T);
        if (m) m[i] = r.m;
        if (s) s[i] = r.s;
        if (lse) lse[i] = orc_lse(&r);
    }
    return 0;
}

/* Lowest-index argmax of `rows` consecutive rows. */
int sv_oracle_argmax(const void *logits, int dtype, int rows, int V, int32_t *out) {
    if (rows < 0 || V <= 0) return 1;
    for (int i = 0; i < rows; ++i) out[i] = orc_argmax(logits, (size_t)i * V, dtype, V);
    return 0;
}
