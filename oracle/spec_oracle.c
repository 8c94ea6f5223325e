/*
 * spec_oracle.c -- CPU oracle for batched draft-token verification.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * statement of what the verification path computes.  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load it.  The GPU
 * library shares no code, header, table or helper with it.
 *
 * Sources (cited by page and section; the pages are HTML text, operators were
 * dropped in extraction and are restored as noted):
 *   [Ling tutorial]  "Ling-3.0-flash-dspark" draft-model tutorial, mlqm.cn/news/1205650
 *                    sec. 3.1 (algorithm), sec. 4.2 (SpeculativeDecoder.generate and
 *                    _apply_top_p), sec. 6.2 (batching, same temperature/top-p),
 *                    sec. 6.4 (draft length 0).
 *   [SSD guide]      SSD inference-engine guide, lpnh.cn/news/2716086, sec. 6 (EAGLE3
 *                    reduced draft vocabulary, d2t scatter in compute_logits) and
 *                    sec. 7 (temperature-0 benchmark runs).
 *   [Eagle blog]     "基于1层Llama草稿模型实现2.16推测解码加速", sec. 5 (draft tree:
 *                    32 nodes, depth 5, top-k 8) and the speed-up table (Match = True).
 *
 * Arithmetic: every floating-point step is float64.  Logits arrive as float32 or
 * bfloat16 bit patterns and are widened exactly.  Sums are sequential, in the
 * order stated next to each one.  No blocking, fusion or reordering.
 *
 * Parity pins: see tests/test_oracle_pins.py.  Every function below is pinned.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Per-sequence status bits (documented meaning, defined independently of the
 * GPU library's header). */
#define ORC_ST_TOKEN_RANGE 1  /* a draft / node token id outside [0, V)        */
#define ORC_ST_D2T         2  /* d2t not strictly increasing, or an entry outside [0, Vt) */
#define ORC_ST_NO_MASS     4  /* a row whose maximum logit is not finite       */
#define ORC_ST_BAD_PARENT  8  /* tree parent outside [0, k) for node k >= 1    */

/* Boundary flags returned next to the outputs (oracle-only diagnostics). */
#define ORC_FL_ACCEPT_EDGE 1  /* |u_i - p/q| < band at an evaluated decision, q > 0 */
#define ORC_FL_CDF_EDGE    2  /* u_s within band of an interior CDF edge of the sample */
#define ORC_FL_ZERO_RESID  4  /* residual mass was exactly 0: sampled from p instead */

/* Return codes. */
#define ORC_OK   0
#define ORC_EARG 1
#define ORC_EMEM 2

/* dtype codes of the raw logits: 0 = float32, 1 = bfloat16 bit patterns,
 * 2 = float64 (logits the oracle computed itself, e.g. from an lm_head).
 * Any other code is an argument error. */
static int dtype_ok(int dtype) { return dtype == 0 || dtype == 1 || dtype == 2; }

static double logit_at(const void *base, int dtype, size_t i)
{
    if (dtype == 0) {
        return (double)((const float *)base)[i];
    }
    if (dtype == 2) {
        return ((const double *)base)[i];
    }
    /* bfloat16 is the high half of a float32: widening is exact. */
    uint32_t u = (uint32_t)((const uint16_t *)base)[i] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------------- */
/* D1: the distribution of one logits row.                                   */
/* ------------------------------------------------------------------------- */

typedef struct {
    double y;
    int32_t id;
} yid_t;

/* Descending logit, then ascending token id: a total order, so the sort is the
 * stable sort of the page's torch.sort(descending) with ties broken by id. */
static int cmp_desc_stable(const void *a, const void *b)
{
    const yid_t *x = (const yid_t *)a, *y = (const yid_t *)b;
    if (x->y > y->y) return -1;
    if (x->y < y->y) return 1;
    return (x->id < y->id) ? -1 : (x->id > y->id);
}

typedef struct {
    int32_t k;          /* tokens kept by top-p (V when top-p is off)             */
    double margin_lo;   /* rho - cum_incl(k-2): how close token k-1 came to removal */
    double margin_hi;   /* cum_incl(k-1) - rho: how close token k came to being kept */
} topp_info_t;

/*
 * Row distribution, [Ling tutorial] sec. 4.2 (generate: logits / temperature,
 * _apply_top_p, F.softmax) and sec. 3.1:
 *   1. y_j = z_j / T.
 *   2. top-p (only when rho < 1): order the ids by y descending, ties by lower
 *      id first; pi = softmax(y) over all V; cum_incl(s) = sum_{t<=s} pi_(t).
 *      Sorted position s is removed when cum_incl(s) > rho, shifted right by
 *      one, and position 0 is never removed -- i.e. position s >= 1 is kept iff
 *      cum_incl(s-1) <= rho.
 *   3. p = softmax over the kept logits (removed ones are -inf).
 * k_delta (tests only) moves the kept count to k + k_delta, to enumerate the
 * admissible alternatives when cum_incl lands within a rounding band of rho.
 * top_k (the draft-side sampler; 0 elsewhere): [Ling tutorial] sec. 3.1 names
 * top-k beside top-p for drawing draft tokens and gives no rule for combining
 * them.  Read plainly, both filters cut the same stable order of step 2: top-k
 * keeps its first top_k positions, top-p its first k, so together they keep
 * the first min(top_k, k) positions.  top_k <= 0 or >= V is off.
 * Returns 0, or ORC_ST_NO_MASS when max y is not finite (p is then all zero).
 */
static int row_dist(const void *base, int dtype, size_t off, int V, double T,
                    double rho, int top_k, int k_delta, double *p, yid_t *scratch,
                    topp_info_t *info)
{
    int j;
    double m = -INFINITY;
    for (j = 0; j < V; ++j) {
        p[j] = logit_at(base, dtype, off + (size_t)j) / T;   /* p holds y for now */
        if (p[j] > m) m = p[j];
    }
    info->k = V;
    info->margin_lo = INFINITY;
    info->margin_hi = INFINITY;
    if (!(m > -INFINITY) || m != m || m == INFINITY) {
        for (j = 0; j < V; ++j) p[j] = 0.0;
        return ORC_ST_NO_MASS;
    }
    const int topk_on = top_k > 0 && top_k < V;

    if (rho < 1.0 || topk_on) {
        /* softmax over all V, sum in id order */
        double Z = 0.0;
        for (j = 0; j < V; ++j) Z += exp(p[j] - m);
        for (j = 0; j < V; ++j) {
            scratch[j].y = p[j];
            scratch[j].id = j;
        }
        qsort(scratch, (size_t)V, sizeof(yid_t), cmp_desc_stable);
        /* cumulative softmax in sorted order; find the first s >= 1 whose
         * predecessor's inclusive cum exceeds rho */
        int k = V;
        double cum = 0.0, cum_prev_prev = 0.0;
        for (int s = 0; s < V && rho < 1.0; ++s) {
            double pi = exp(scratch[s].y - m) / Z;
            cum_prev_prev = cum;          /* cum_incl(s-1) */
            cum += pi;                    /* cum_incl(s)   */
            if (s + 1 < V && cum > rho) { /* position s+1 is the first removed */
                k = s + 1;
                info->margin_hi = cum - rho;
                info->margin_lo = (k >= 2) ? rho - cum_prev_prev : INFINITY;
                break;
            }
        }
        if (k == V && V >= 2 && rho < 1.0) {
            /* everything kept: the last kept position's predecessor margin */
            double c = 0.0;
            for (int s = 0; s < V - 1; ++s) c += exp(scratch[s].y - m) / Z;
            info->margin_lo = rho - c;
        }
        info->k = k;
        int kk = k + k_delta;
        if (kk < 1) kk = 1;
        if (kk > V) kk = V;
        if (topk_on && kk > top_k) kk = top_k;       /* top-k cuts the same order */
        /* removed ids become -inf, as the page's filter writes them */
        for (int s = kk; s < V; ++s) p[scratch[s].id] = -INFINITY;
    }

    /* softmax of the (filtered) logits, sum in id order */
    double Zk = 0.0;
    for (j = 0; j < V; ++j)
        if (p[j] > -INFINITY) Zk += exp(p[j] - m);
    for (j = 0; j < V; ++j)
        p[j] = (p[j] > -INFINITY) ? exp(p[j] - m) / Zk : 0.0;
    return 0;
}

/* ------------------------------------------------------------------------- */
/* D3-D6: one sequence of sampling verification.                             */
/* ------------------------------------------------------------------------- */

typedef struct {
    const void *tl; int tdt;
    const void *dl; int ddt;
    const int32_t *tokens;
    const int32_t *d2t;
    const float *u_acc, *u_s;
    int B, gamma, Vt, Vd;
    double T, rho, band;
    const int8_t *k_delta;
    int32_t *out_tokens, *out_len, *out_status, *out_flags;
    double *out_p, *out_q, *out_margin;
    int nthreads, tid;
    int err;
} sample_job_t;

/*
 * Inverse-CDF draw over the nonnegative weights w[0..V-1], ascending token id,
 * [Ling tutorial] sec. 4.2 (torch.multinomial over the normalised weights).
 * Returns min{ j : sum_{t<=j} w_t > u * S } (strict, so zero-weight ids are
 * never drawn); if rounding leaves no such j, the last j with w_j > 0.
 * Sets *edge when u lies within band of an interior edge of the chosen
 * interval: its lower edge when an id before the pick has positive weight,
 * its upper edge when an id after it does.  The outer edges 0 and 1 are not
 * decision boundaries (no other token lies beyond them), so they are never
 * flagged.
 */
static int32_t inverse_cdf(const double *w, int V, double u, double band, int *edge)
{
    double S = 0.0;
    int j;
    for (j = 0; j < V; ++j) S += w[j];
    double target = u * S;
    double cum = 0.0, before = 0.0;
    int32_t pick = -1, last_pos = -1;
    for (j = 0; j < V; ++j) {
        if (w[j] > 0.0) last_pos = j;
        before = cum;
        cum += w[j];
        if (cum > target) {
            pick = j;
            break;
        }
    }
    if (pick < 0) {
        pick = last_pos;
        before = S - (pick >= 0 ? w[pick] : 0.0);
        cum = S;
    }
    int pos_before = 0, pos_after = 0;
    for (j = 0; j < pick; ++j)
        if (w[j] > 0.0) pos_before = 1;
    for (j = pick + 1; pick >= 0 && j < V; ++j)
        if (w[j] > 0.0) pos_after = 1;
    *edge = (S > 0.0) && ((pos_before && fabs(u - before / S) < band) ||
                          (pos_after && fabs(u - cum / S) < band));
    return pick;
}

static void verify_sample_seq(sample_job_t *J, int b, double *P, double *Q,
                              double *qc, double *r, yid_t *scr)
{
    const int g = J->gamma, Vt = J->Vt, Vd = J->Vd;
    const int nrows = 2 * g + 1;
    int32_t status = 0, flags = 0;
    int i;
    /* Every row's distribution: target rows 0..g are p_0..p_g (row i scores
     * draft token i, row g is the bonus position), draft rows 0..g-1 are
     * q_0..q_{g-1}, with the same temperature and top-p for both
     * ([Ling tutorial] sec. 4.2 and sec. 6.2). */
    for (i = 0; i <= g; ++i) {
        topp_info_t info;
        int kd = J->k_delta ? J->k_delta[(size_t)b * nrows + i] : 0;
        size_t off = ((size_t)b * (g + 1) + i) * (size_t)Vt;
        status |= row_dist(J->tl, J->tdt, off, Vt, J->T, J->rho, 0, kd, P + (size_t)i * Vt, scr, &info);
        if (J->out_margin) {
            J->out_margin[((size_t)b * nrows + i) * 2 + 0] = info.margin_lo;
            J->out_margin[((size_t)b * nrows + i) * 2 + 1] = info.margin_hi;
        }
    }
    for (i = 0; i < g; ++i) {
        topp_info_t info;
        int kd = J->k_delta ? J->k_delta[(size_t)b * nrows + g + 1 + i] : 0;
        size_t off = ((size_t)b * g + i) * (size_t)Vd;
        double *q = Q + (size_t)i * Vt;
        if (J->d2t == NULL) {
            status |= row_dist(J->dl, J->ddt, off, Vd, J->T, J->rho, 0, kd, q, scr, &info);
        } else {
            /* [SSD guide] sec. 6: the draft head covers a reduced vocabulary and
             * d2t scatters it into the target vocabulary; ids off the map get
             * probability 0. */
            status |= row_dist(J->dl, J->ddt, off, Vd, J->T, J->rho, 0, kd, qc, scr, &info);
            for (int t = 0; t < Vt; ++t) q[t] = 0.0;
            for (int jd = 0; jd < Vd; ++jd) q[J->d2t[jd]] = qc[jd];
        }
        if (J->out_margin) {
            J->out_margin[((size_t)b * nrows + g + 1 + i) * 2 + 0] = info.margin_lo;
            J->out_margin[((size_t)b * nrows + g + 1 + i) * 2 + 1] = info.margin_hi;
        }
    }

    /* Accept chain, [Ling tutorial] sec. 3.1: accept draft token i with
     * probability min(1, p_i(x_i)/q_i(x_i)); the page draws u ~ U[0,1) and
     * accepts when u is below the ratio.  Written as u*q < p it is the same
     * test for q > 0 and its limit (accept iff p > 0) for q = 0. */
    int n = g;
    for (i = 0; i < g; ++i) {
        int32_t x = J->tokens[(size_t)b * g + i];
        double a = 0.0, c = 0.0;
        if (x < 0 || x >= Vt) {
            status |= ORC_ST_TOKEN_RANGE;
        } else {
            a = P[(size_t)i * Vt + x];
            c = Q[(size_t)i * Vt + x];
        }
        if (J->out_p) J->out_p[(size_t)b * g + i] = a;
        if (J->out_q) J->out_q[(size_t)b * g + i] = c;
        if (n == g) {   /* still in the chain: this decision is evaluated */
            double u = (double)J->u_acc[(size_t)b * g + i];
            if (c > 0.0 && fabs(u - a / c) < J->band) flags |= ORC_FL_ACCEPT_EDGE;
            if (!(u * c < a)) n = i;   /* first rejection */
        }
    }

    /* Replacement or bonus draw with the single sampling uniform.
     * Rejection at n < g: p'(x) = norm(max(0, p_n(x) - q_n(x))) ([Ling tutorial]
     * sec. 3.1 and the F.relu / normalise / multinomial step of sec. 4.2).
     * All accepted: draw from p_g ([Ling tutorial] sec. 3.1, last step). */
    double us = (double)J->u_s[b];
    int edge = 0;
    int32_t pick;
    const double *pn = P + (size_t)n * Vt;
    if (n < g) {
        const double *qn = Q + (size_t)n * Vt;
        double S = 0.0;
        for (int t = 0; t < Vt; ++t) {
            double d = pn[t] - qn[t];
            r[t] = d > 0.0 ? d : 0.0;
            S += r[t];
        }
        if (S > 0.0) {
            pick = inverse_cdf(r, Vt, us, J->band, &edge);
        } else {
            flags |= ORC_FL_ZERO_RESID;
            pick = inverse_cdf(pn, Vt, us, J->band, &edge);
        }
    } else {
        pick = inverse_cdf(pn, Vt, us, J->band, &edge);
    }
    if (edge) flags |= ORC_FL_CDF_EDGE;

    int32_t *ot = J->out_tokens + (size_t)b * (g + 1);
    for (i = 0; i <= g; ++i) ot[i] = -1;
    for (i = 0; i < n; ++i) ot[i] = J->tokens[(size_t)b * g + i];
    ot[n] = pick;
    J->out_len[b] = n;
    if (J->out_status) J->out_status[b] = status;
    if (J->out_flags) J->out_flags[b] = flags;
}

static void *sample_worker(void *arg)
{
    sample_job_t *J = (sample_job_t *)arg;
    size_t Vt = (size_t)J->Vt, Vd = (size_t)J->Vd;
    size_t rows = (size_t)J->gamma + 1;
    double *P = malloc(sizeof(double) * Vt * rows);
    double *Q = malloc(sizeof(double) * Vt * (J->gamma > 0 ? (size_t)J->gamma : 1));
    double *qc = malloc(sizeof(double) * Vd);
    double *r = malloc(sizeof(double) * Vt);
    size_t sv = Vt > Vd ? Vt : Vd;
    yid_t *scr = malloc(sizeof(yid_t) * sv);
    if (!P || !Q || !qc || !r || !scr) {
        J->err = ORC_EMEM;
    } else {
        for (int b = J->tid; b < J->B; b += J->nthreads)
            verify_sample_seq(J, b, P, Q, qc, r, scr);
    }
    free(P); free(Q); free(qc); free(r); free(scr);
    return NULL;
}

/*
 * Sampling verification for a batch (sequences are independent,
 * [Ling tutorial] sec. 6.2).  Layouts are row-major and contiguous:
 *   target logits [B, gamma+1, Vt], draft logits [B, gamma, Vd],
 *   tokens [B, gamma] (target-vocabulary ids), d2t [Vd] or NULL (then Vd == Vt),
 *   u_acc [B, gamma], u_s [B].
 * Outputs: out_tokens [B, gamma+1] (-1 padded), out_len [B],
 *   out_p / out_q [B, gamma] (p_i(x_i), q_i(x_i) for every i; may be NULL),
 *   out_status [B] (ORC_ST_*; may be NULL), out_flags [B] (ORC_FL_*; may be NULL),
 *   (a d2t map that is not strictly increasing inside [0, Vt) gives ORC_ST_D2T
 *   on every sequence when gamma > 0, see above),
 *   out_margin [B, 2*gamma+1, 2] top-p margins per row, target rows first
 *   (may be NULL).  k_delta [B, 2*gamma+1] or NULL: per-row kept-count shifts.
 * band: the half-width of the boundary band for the flags (1e-5 in the tests).
 */
int oracle_verify_sample(const void *tl, int tdt, const void *dl, int ddt,
                         const int32_t *tokens, const int32_t *d2t,
                         const float *u_acc, const float *u_s,
                         int B, int gamma, int Vt, int Vd, double T, double rho,
                         double band, const int8_t *k_delta,
                         int32_t *out_tokens, int32_t *out_len,
                         double *out_p, double *out_q,
                         int32_t *out_status, int32_t *out_flags, double *out_margin,
                         int nthreads)
{
    if (B < 0 || gamma < 0 || Vt < 1 || Vd < 1 || !(T > 0.0) || !(rho > 0.0)) return ORC_EARG;
    if (!dtype_ok(tdt) || (gamma > 0 && !dtype_ok(ddt))) return ORC_EARG;
    if (d2t == NULL && Vd != Vt) return ORC_EARG;
    if (B == 0) return ORC_OK;
    if (d2t && gamma > 0) {
        /* [SSD guide] sec. 6: d2t maps each draft id to a distinct target id;
         * this library takes it sorted.  A map that is not strictly increasing
         * or leaves [0, Vt) is reported, not used: every sequence gets
         * ORC_ST_D2T, no token (-1), length 0 and zero probabilities. */
        int bad = 0;
        for (int j = 0; j < Vd; ++j) {
            if (d2t[j] < 0 || d2t[j] >= Vt) bad = 1;
            if (j > 0 && d2t[j] <= d2t[j - 1]) bad = 1;
        }
        if (bad) {
            for (int b = 0; b < B; ++b) {
                for (int i = 0; i <= gamma; ++i) out_tokens[(size_t)b * (gamma + 1) + i] = -1;
                out_len[b] = 0;
                for (int i = 0; i < gamma; ++i) {
                    if (out_p) out_p[(size_t)b * gamma + i] = 0.0;
                    if (out_q) out_q[(size_t)b * gamma + i] = 0.0;
                }
                if (out_status) out_status[b] = ORC_ST_D2T;
                if (out_flags) out_flags[b] = 0;
                if (out_margin)
                    for (int r = 0; r < 2 * (2 * gamma + 1); ++r)
                        out_margin[(size_t)b * 2 * (2 * gamma + 1) + r] = INFINITY;
            }
            return ORC_OK;
        }
    }
    if (nthreads < 1) nthreads = 1;
    if (nthreads > B) nthreads = B;
    sample_job_t *jobs = calloc((size_t)nthreads, sizeof(sample_job_t));
    pthread_t *th = calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); return ORC_EMEM; }
    for (int t = 0; t < nthreads; ++t) {
        sample_job_t *J = &jobs[t];
        J->tl = tl; J->tdt = tdt; J->dl = dl; J->ddt = ddt;
        J->tokens = tokens; J->d2t = d2t; J->u_acc = u_acc; J->u_s = u_s;
        J->B = B; J->gamma = gamma; J->Vt = Vt; J->Vd = Vd;
        J->T = T; J->rho = rho; J->band = band; J->k_delta = k_delta;
        J->out_tokens = out_tokens; J->out_len = out_len;
        J->out_status = out_status; J->out_flags = out_flags;
        J->out_p = out_p; J->out_q = out_q; J->out_margin = out_margin;
        J->nthreads = nthreads; J->tid = t; J->err = 0;
    }
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, sample_worker, &jobs[t]);
    sample_worker(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
    int err = 0;
    for (int t = 0; t < nthreads; ++t) if (jobs[t].err) err = jobs[t].err;
    free(jobs); free(th);
    return err;
}

/*
 * One row's distribution, exposed for the pins: p [V] receives D1's output
 * (with the top_k cap of the draft-side sampler; 0 = off).
 * Returns the status bits; *k, *margin_lo, *margin_hi as in topp_info_t
 * (k is the top-p count before the top-k cap).
 */
int oracle_row_dist(const void *z, int dtype, int V, double T, double rho, int top_k, int k_delta,
                    double *p, int32_t *k, double *margin_lo, double *margin_hi)
{
    if (V < 1 || !(T > 0.0) || !(rho > 0.0) || !dtype_ok(dtype)) return -ORC_EARG;
    yid_t *scr = malloc(sizeof(yid_t) * (size_t)V);
    if (!scr) return -ORC_EMEM;
    topp_info_t info;
    int st = row_dist(z, dtype, 0, V, T, rho, top_k, k_delta, p, scr, &info);
    free(scr);
    if (k) *k = info.k;
    if (margin_lo) *margin_lo = info.margin_lo;
    if (margin_hi) *margin_hi = info.margin_hi;
    return st;
}

/*
 * The chain and draw alone (D3-D6) on caller-provided distributions, for the
 * pins that integrate over the uniforms and for parity accounting over many
 * uniform sets: P [gamma+1, V], Q [gamma, V].  Writes out_tokens [gamma+1],
 * returns n (accepted count).  When out_flags is not NULL it receives the
 * boundary flags of verify_sample_seq with the same band: an evaluated
 * decision with q > 0 and |u_i - p/q| < band, a draw with u_s within band of
 * either edge of its CDF interval, a zero residual.
 */
int oracle_chain_from_dists(const double *P, const double *Q, const int32_t *tokens,
                            const float *u_acc, float u_s, int gamma, int V,
                            double band, int32_t *out_tokens, int32_t *out_flags)
{
    int n = gamma, i;
    int32_t flags = 0;
    for (i = 0; i < gamma; ++i) {
        int32_t x = tokens[i];
        double a = 0.0, c = 0.0;
        if (x >= 0 && x < V) { a = P[(size_t)i * V + x]; c = Q[(size_t)i * V + x]; }
        if (c > 0.0 && fabs((double)u_acc[i] - a / c) < band) flags |= ORC_FL_ACCEPT_EDGE;
        if (!((double)u_acc[i] * c < a)) { n = i; break; }
    }
    double *r = malloc(sizeof(double) * (size_t)V);
    if (!r) return -ORC_EMEM;
    const double *pn = P + (size_t)n * V;
    int edge = 0;
    int32_t pick;
    if (n < gamma) {
        double S = 0.0;
        for (int t = 0; t < V; ++t) {
            double d = pn[t] - Q[(size_t)n * V + t];
            r[t] = d > 0.0 ? d : 0.0;
            S += r[t];
        }
        if (S > 0.0) {
            pick = inverse_cdf(r, V, (double)u_s, band, &edge);
        } else {
            flags |= ORC_FL_ZERO_RESID;
            pick = inverse_cdf(pn, V, (double)u_s, band, &edge);
        }
    } else {
        pick = inverse_cdf(pn, V, (double)u_s, band, &edge);
    }
    if (edge) flags |= ORC_FL_CDF_EDGE;
    free(r);
    for (i = 0; i <= gamma; ++i) out_tokens[i] = -1;
    for (i = 0; i < n; ++i) out_tokens[i] = tokens[i];
    out_tokens[n] = pick;
    if (out_flags) *out_flags = flags;
    return n;
}

/* ------------------------------------------------------------------------- */
/* D9: the draft-side sampler and the acceptance counters.                   */
/* ------------------------------------------------------------------------- */

/*
 * One draft token per row, [Ling tutorial] sec. 4.2 (the draft loop of
 * generate(): logits / temperature, _apply_top_p, F.softmax,
 * torch.multinomial) and sec. 3.1 (drafting by argmax or top-p/top-k):
 *   p = row_dist(z / T, top-p rho, top-k cap) as in D1 with the top_k reading
 *   above; the token is the inverse-CDF draw of D4 with the caller's uniform
 *   u[b] (ascending id, strict >).  With d2t (a reduced draft vocabulary,
 *   [SSD guide] sec. 6) the drawn draft id j is reported as target id d2t[j].
 * logits [B, V]; u [B]; out_tokens [B]; out_prob [B] = p of the drawn id;
 * out_status [B] (ORC_ST_NO_MASS; may be NULL); out_flags [B] (ORC_FL_CDF_EDGE
 * when u is within band of an interior edge; may be NULL); out_margin [B, 2]
 * top-p margins and out_k [B] the top-p count before the top-k cap (may be
 * NULL); k_delta [B] or NULL moves the top-p count (tests only).
 */
int oracle_draft_sample(const void *logits, int dtype, const int32_t *d2t, const float *u,
                        int B, int V, double T, double rho, int top_k, double band,
                        const int8_t *k_delta, int32_t *out_tokens, double *out_prob,
                        int32_t *out_status, int32_t *out_flags, double *out_margin,
                        int32_t *out_k)
{
    if (B < 0 || V < 1 || !(T > 0.0) || !(rho > 0.0) || !dtype_ok(dtype)) return ORC_EARG;
    double *p = malloc(sizeof(double) * (size_t)V);
    yid_t *scr = malloc(sizeof(yid_t) * (size_t)V);
    if (!p || !scr) { free(p); free(scr); return ORC_EMEM; }
    for (int b = 0; b < B; ++b) {
        topp_info_t info;
        int kd = k_delta ? k_delta[b] : 0;
        int st = row_dist(logits, dtype, (size_t)b * (size_t)V, V, T, rho, top_k, kd, p, scr, &info);
        int edge = 0;
        int32_t pick = st ? -1 : inverse_cdf(p, V, (double)u[b], band, &edge);
        out_tokens[b] = (pick >= 0 && d2t) ? d2t[pick] : pick;
        out_prob[b] = pick >= 0 ? p[pick] : 0.0;
        if (out_status) out_status[b] = st;
        if (out_flags) out_flags[b] = edge ? ORC_FL_CDF_EDGE : 0;
        if (out_margin) { out_margin[2 * b] = info.margin_lo; out_margin[2 * b + 1] = info.margin_hi; }
        if (out_k) out_k[b] = info.k;
    }
    free(p); free(scr);
    return ORC_OK;
}

/*
 * Acceptance counters over one verification call, [Ling tutorial] sec. 4.2
 * (the statistics of generate(): total_tokens, total_target_calls,
 * total_draft_calls, avg_acceptance_rate = sum of accepted counts /
 * (rounds * draft_length), speedup_estimate = tokens / target calls):
 *   counters[0] += B            target calls (one verification pass per sequence)
 *   counters[1] += B * gamma    draft tokens proposed (gamma draft calls each)
 *   counters[2] += sum n_b      draft tokens accepted
 *   counters[3] += sum (n_b+1)  tokens emitted (accepted drafts plus the drawn one)
 *   counters[4] += #{b : n_b outside [0, gamma]}  (such entries add to no other counter)
 */
int oracle_count(const int32_t *accept_len, int B, int gamma, uint64_t *counters)
{
    if (B < 0 || gamma < 0) return ORC_EARG;
    for (int b = 0; b < B; ++b) {
        int32_t n = accept_len[b];
        if (n < 0 || n > gamma) { counters[4] += 1; continue; }
        counters[0] += 1;
        counters[1] += (uint64_t)gamma;
        counters[2] += (uint64_t)n;
        counters[3] += (uint64_t)n + 1;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* D10: the SSD fan-out lookup.                                              */
/* ------------------------------------------------------------------------- */

/*
 * [SSD guide] sec. 1: while the target verifies, the draft pre-speculates the
 * possible verification outcomes and drafts every branch at once; a branch
 * that matches the outcome makes the next round's drafting free.  sec. 7
 * runs it with a fan-out of 3 (--f 3).  Here an outcome is the accepted length
 * n and the token emitted after the accepted drafts, out_tokens[b, n]; for
 * every n in [0, gamma] the table holds f candidate tokens cand[b, n, j], and
 * branch n * f + j carries L pre-drafted tokens.
 *   branch[b] = n * f + j for the lowest slot j with cand[b, n, j] equal to
 *   the emitted token (and >= 0); -1 when none matches or n is outside
 *   [0, gamma].  next[b, :] = that branch's drafts, -1 on a miss.
 * counters [2] or NULL: += B lookups, += hits.
 */
int oracle_fanout_lookup(const int32_t *out_tokens, const int32_t *accept_len, const int32_t *cand,
                         const int32_t *drafts, int B, int gamma, int f, int L,
                         int32_t *out_branch, int32_t *out_next, uint64_t *counters)
{
    if (B < 0 || gamma < 0 || f < 1 || L < 0) return ORC_EARG;
    for (int b = 0; b < B; ++b) {
        int32_t n = accept_len[b];
        int32_t br = -1;
        if (n >= 0 && n <= gamma) {
            int32_t t = out_tokens[(size_t)b * (gamma + 1) + n];
            for (int j = 0; j < f && br < 0; ++j) {
                int32_t c = cand[((size_t)b * (gamma + 1) + n) * f + j];
                if (c >= 0 && c == t) br = n * f + j;
            }
        }
        out_branch[b] = br;
        if (out_next)
            for (int i = 0; i < L; ++i)
                out_next[(size_t)b * L + i] =
                    br >= 0 ? drafts[((size_t)b * (gamma + 1) * f + br) * L + i] : -1;
        if (counters) { counters[0] += 1; counters[1] += br >= 0; }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* D11: the vocabulary-trim d2t builder.                                     */
/* ------------------------------------------------------------------------- */

typedef struct {
    int64_t count;
    int32_t id;
} cid_t;

/* Larger count first, then lower id: a total order. */
static int cmp_count_desc(const void *a, const void *b)
{
    const cid_t *x = (const cid_t *)a, *y = (const cid_t *)b;
    if (x->count > y->count) return -1;
    if (x->count < y->count) return 1;
    return (x->id < y->id) ? -1 : (x->id > y->id);
}

/*
 * [Eagle blog] sec. 6: from the token frequencies of a corpus, keep the core
 * vocabulary whose cumulative probability reaches P >= 0.95; the draft head
 * then scores only those ids ([SSD guide] sec. 6 maps them back through d2t).
 *   counts c[t] of the ids t in [0, Vt) in tokens[0..N) (others are invalid);
 *   order the ids by count descending, lower id first on equal counts;
 *   keep the smallest prefix whose count sum reaches P * Nv, Nv = the valid
 *   tokens (P * Nv in float64); ids of count 0 are never kept, so P >= 1
 *   keeps every observed id.
 * out_d2t [Vt]: the kept ids in ascending order in its first *out_vd entries;
 * out_t2d [Vt] or NULL: position of t in d2t, -1 when t is not kept;
 * out_info [3] or NULL: kept count mass, valid tokens, invalid tokens.
 */
int oracle_vocab_trim(const int32_t *tokens, int64_t N, int Vt, double P, int32_t *out_d2t,
                      int32_t *out_t2d, int32_t *out_vd, int64_t *out_info)
{
    if (N < 0 || Vt < 1 || !(P > 0.0)) return ORC_EARG;
    cid_t *c = calloc((size_t)Vt, sizeof(cid_t));
    if (!c) return ORC_EMEM;
    int64_t valid = 0, invalid = 0;
    for (int t = 0; t < Vt; ++t) c[t].id = t;
    for (int64_t i = 0; i < N; ++i) {
        int32_t t = tokens[i];
        if (t < 0 || t >= Vt) { ++invalid; continue; }
        c[t].count += 1;
        ++valid;
    }
    qsort(c, (size_t)Vt, sizeof(cid_t), cmp_count_desc);
    double T = P * (double)valid;
    int k = 0;
    int64_t cum = 0;
    while (k < Vt && c[k].count > 0 && !((double)cum >= T)) {
        cum += c[k].count;
        ++k;
    }
    /* ascending ids of the first k positions */
    unsigned char *keep = calloc((size_t)Vt, 1);
    if (!keep) { free(c); return ORC_EMEM; }
    for (int s = 0; s < k; ++s) keep[c[s].id] = 1;
    int pos = 0;
    for (int t = 0; t < Vt; ++t) {
        if (out_t2d) out_t2d[t] = keep[t] ? pos : -1;
        if (keep[t]) out_d2t[pos++] = t;
    }
    *out_vd = k;
    if (out_info) { out_info[0] = cum; out_info[1] = valid; out_info[2] = invalid; }
    free(keep);
    free(c);
    return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* D7: greedy (temperature 0) verification.                                  */
/* ------------------------------------------------------------------------- */

/* Lowest id attaining the row maximum, values compared as doubles (so -0 and
 * +0 are equal).  A row of -inf everywhere gives id 0 and ORC_ST_NO_MASS. */
static int32_t row_argmax(const void *base, int dtype, size_t off, int V, int *no_mass)
{
    double best = logit_at(base, dtype, off);
    int32_t arg = 0;
    for (int j = 1; j < V; ++j) {
        double v = logit_at(base, dtype, off + (size_t)j);
        if (v > best) { best = v; arg = j; }
    }
    *no_mass = !(best > -INFINITY) || best == INFINITY || best != best;
    return arg;
}

/*
 * Greedy verification: with temperature 0 the draft and the target both take
 * the argmax ([Ling tutorial] sec. 3.1 drafting by argmax; [SSD guide] sec. 7
 * runs at temperature 0), and the output must equal the target's own argmax
 * chain ([Eagle blog] speed-up table, Match = True).
 *   g_i = argmax z[b, i] for i = 0..gamma; n = first i with x_i != g_i, else
 *   gamma; emit x_0..x_{n-1}, then g_n.
 * logits [B, gamma+1, V]; tokens [B, gamma]; out_tokens [B, gamma+1] (-1
 * padded); out_len [B]; out_status [B] or NULL.
 */
/*
 * D7's chain on given row argmaxes g [B, gamma+1] (the fused lm_head path
 * reports its argmaxes; the chain rule is the same): n = first i with
 * x_i != g_i, emit x_0..x_{n-1}, g_n.  status gets ORC_ST_TOKEN_RANGE for a
 * token outside [0, V).
 */
int oracle_greedy_from_argmax(const int32_t *g, const int32_t *tokens, int B, int gamma, int V,
                              int32_t *out_tokens, int32_t *out_len, int32_t *out_status)
{
    if (B < 0 || gamma < 0 || V < 1) return ORC_EARG;
    for (int b = 0; b < B; ++b) {
        int32_t st = 0;
        int n = gamma;
        for (int i = 0; i < gamma; ++i) {
            int32_t x = tokens[(size_t)b * gamma + i];
            if (x < 0 || x >= V) st |= ORC_ST_TOKEN_RANGE;
            if (n == gamma && x != g[(size_t)b * (gamma + 1) + i]) n = i;
        }
        int32_t *ot = out_tokens + (size_t)b * (gamma + 1);
        for (int i = 0; i <= gamma; ++i) ot[i] = -1;
        for (int i = 0; i < n; ++i) ot[i] = tokens[(size_t)b * gamma + i];
        ot[n] = g[(size_t)b * (gamma + 1) + n];
        out_len[b] = n;
        if (out_status) out_status[b] = st;
    }
    return ORC_OK;
}

int oracle_verify_greedy(const void *logits, int dtype, const int32_t *tokens,
                         int B, int gamma, int V, int32_t *out_tokens,
                         int32_t *out_len, int32_t *out_status)
{
    if (B < 0 || gamma < 0 || V < 1 || !dtype_ok(dtype)) return ORC_EARG;
    for (int b = 0; b < B; ++b) {
        int32_t st = 0;
        int n = gamma;
        int32_t g_n = -1;
        for (int i = 0; i <= gamma; ++i) {
            int nm;
            int32_t gi = row_argmax(logits, dtype, ((size_t)b * (gamma + 1) + i) * (size_t)V, V, &nm);
            if (nm) st |= ORC_ST_NO_MASS;
            if (i < gamma) {
                int32_t x = tokens[(size_t)b * gamma + i];
                if (x < 0 || x >= V) st |= ORC_ST_TOKEN_RANGE;
                if (n == gamma && x != gi) { n = i; g_n = gi; }
            } else if (n == gamma) {
                g_n = gi;
            }
        }
        int32_t *ot = out_tokens + (size_t)b * (gamma + 1);
        for (int i = 0; i <= gamma; ++i) ot[i] = -1;
        for (int i = 0; i < n; ++i) ot[i] = tokens[(size_t)b * gamma + i];
        ot[n] = g_n;
        out_len[b] = n;
        if (out_status) out_status[b] = st;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* D8: greedy tree verification.                                             */
/* ------------------------------------------------------------------------- */

/*
 * Greedy verification of a draft tree ([Eagle blog] sec. 5: one target pass
 * scores every node of a 32-node, depth-5, top-k-8 tree).  Node 0 is the root
 * (the last committed token); row k of the logits is the target's distribution
 * after node k.  Node k >= 1 has parent par[k] < k and token tok[k].
 *   acc[0] = true; acc[k] = acc[par[k]] and tok[k] == argmax(row par[k]).
 *   best = the deepest accepted node, ties to the lowest index.
 *   Emit the tokens on the root->best path (root excluded), then argmax(row best).
 * logits [B, N, V]; node_tokens, parents [B, N]; out_path [B, N] node indices
 * of the path (-1 padded); out_tokens [B, N] (path tokens then the bonus, -1
 * padded); out_len [B] = depth of best; out_status [B] or NULL.
 */
/*
 * D8's walk on given row argmaxes g [B, N] (as reported by the fused lm_head
 * path): the same acceptance rule, winner and outputs as
 * oracle_verify_tree_greedy, without the no-mass check (g carries no values).
 */
int oracle_tree_from_argmax(const int32_t *gall, const int32_t *node_tokens, const int32_t *parents,
                            int B, int N, int V, int32_t *out_path, int32_t *out_tokens,
                            int32_t *out_len, int32_t *out_status)
{
    if (B < 0 || N < 1 || V < 1) return ORC_EARG;
    int32_t *depth = malloc(sizeof(int32_t) * (size_t)N);
    unsigned char *acc = malloc((size_t)N);
    int32_t *stack = malloc(sizeof(int32_t) * (size_t)N);
    if (!depth || !acc || !stack) { free(depth); free(acc); free(stack); return ORC_EMEM; }
    for (int b = 0; b < B; ++b) {
        const int32_t *g = gall + (size_t)b * N;
        int32_t st = 0;
        acc[0] = 1;
        depth[0] = 0;
        for (int k = 1; k < N; ++k) {
            int32_t pk = parents[(size_t)b * N + k];
            int32_t tk = node_tokens[(size_t)b * N + k];
            acc[k] = 0;
            depth[k] = 0;
            if (tk < 0 || tk >= V) st |= ORC_ST_TOKEN_RANGE;
            if (pk < 0 || pk >= k) { st |= ORC_ST_BAD_PARENT; continue; }
            depth[k] = depth[pk] + 1;
            acc[k] = acc[pk] && tk == g[pk];
        }
        int best = 0;
        for (int k = 1; k < N; ++k)
            if (acc[k] && depth[k] > depth[best]) best = k;
        int d = 0;
        for (int k = best; k != 0; k = parents[(size_t)b * N + k]) stack[d++] = k;
        int32_t *op = out_path + (size_t)b * N;
        int32_t *ot = out_tokens + (size_t)b * N;
        for (int k = 0; k < N; ++k) { op[k] = -1; ot[k] = -1; }
        for (int s2 = 0; s2 < d; ++s2) {
            op[s2] = stack[d - 1 - s2];
            ot[s2] = node_tokens[(size_t)b * N + op[s2]];
        }
        ot[d] = g[best];
        out_len[b] = d;
        if (out_status) out_status[b] = st;
    }
    free(depth); free(acc); free(stack);
    return ORC_OK;
}

int oracle_verify_tree_greedy(const void *logits, int dtype, const int32_t *node_tokens,
                              const int32_t *parents, int B, int N, int V,
                              int32_t *out_path, int32_t *out_tokens, int32_t *out_len,
                              int32_t *out_status)
{
    if (B < 0 || N < 1 || V < 1 || !dtype_ok(dtype)) return ORC_EARG;
    int32_t *g = malloc(sizeof(int32_t) * (size_t)N);
    int32_t *depth = malloc(sizeof(int32_t) * (size_t)N);
    unsigned char *acc = malloc((size_t)N);
    int32_t *stack = malloc(sizeof(int32_t) * (size_t)N);
    if (!g || !depth || !acc || !stack) { free(g); free(depth); free(acc); free(stack); return ORC_EMEM; }
    for (int b = 0; b < B; ++b) {
        int32_t st = 0;
        for (int k = 0; k < N; ++k) {
            int nm;
            g[k] = row_argmax(logits, dtype, ((size_t)b * N + k) * (size_t)V, V, &nm);
            if (nm) st |= ORC_ST_NO_MASS;
        }
        acc[0] = 1;
        depth[0] = 0;
        for (int k = 1; k < N; ++k) {
            int32_t pk = parents[(size_t)b * N + k];
            int32_t tk = node_tokens[(size_t)b * N + k];
            acc[k] = 0;
            depth[k] = 0;
            if (tk < 0 || tk >= V) st |= ORC_ST_TOKEN_RANGE;
            if (pk < 0 || pk >= k) { st |= ORC_ST_BAD_PARENT; continue; }
            depth[k] = depth[pk] + 1;
            acc[k] = acc[pk] && tk == g[pk];
        }
        int best = 0;
        for (int k = 1; k < N; ++k)
            if (acc[k] && depth[k] > depth[best]) best = k;
        int d = 0;
        for (int k = best; k != 0; k = parents[(size_t)b * N + k]) stack[d++] = k;
        int32_t *op = out_path + (size_t)b * N;
        int32_t *ot = out_tokens + (size_t)b * N;
        for (int k = 0; k < N; ++k) { op[k] = -1; ot[k] = -1; }
        for (int s = 0; s < d; ++s) {
            op[s] = stack[d - 1 - s];
            ot[s] = node_tokens[(size_t)b * N + op[s]];
        }
        ot[d] = g[best];
        out_len[b] = d;
        if (out_status) out_status[b] = st;
    }
    free(g); free(depth); free(acc); free(stack);
    return ORC_OK;
}
