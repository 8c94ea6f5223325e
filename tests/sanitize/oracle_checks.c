/* oracle_checks.c -- every entry point of the CPU oracle (oracle/spec_oracle.c)
 * on small seeded inputs under AddressSanitizer and UndefinedBehaviorSanitizer:
 * float32 and bfloat16 logits, ragged lengths, gamma 0, a d2t map, tokens out
 * of range, rows of -inf, ties, trees, and the argument errors.  The values
 * are not checked here (the oracle pins do that); this driver shows that no
 * path reads or writes out of bounds or hits undefined behaviour.  Prints
 * "oracle ok" and exits 0 when every call returns the expected code. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_verify_sample(const void *tl, int tdt, const void *dl, int ddt, const int32_t *tokens,
                         const int32_t *d2t, const float *u_acc, const float *u_s, int B, int gamma, int Vt,
                         int Vd, double T, double rho, double band, const int8_t *k_delta, int32_t *out_tokens,
                         int32_t *out_len, double *out_p, double *out_q, int32_t *out_status, int32_t *out_flags,
                         double *out_margin, int nthreads);
int oracle_row_dist(const void *z, int dtype, int V, double T, double rho, int top_k, int k_delta, double *p,
                    int32_t *k, double *margin_lo, double *margin_hi);
int oracle_chain_from_dists(const double *P, const double *Q, const int32_t *tokens, const float *u_acc, float u_s,
                            int gamma, int V, double band, int32_t *out_tokens, int32_t *out_flags);
int oracle_draft_sample(const void *logits, int dtype, const int32_t *d2t, const float *u, int B, int V, double T,
                        double rho, int top_k, double band, const int8_t *k_delta, int32_t *out_tokens,
                        double *out_prob, int32_t *out_status, int32_t *out_flags, double *out_margin,
                        int32_t *out_k);
int oracle_count(const int32_t *accept_len, int B, int gamma, uint64_t *counters);
int oracle_fanout_lookup(const int32_t *out_tokens, const int32_t *accept_len, const int32_t *cand,
                         const int32_t *drafts, int B, int gamma, int f, int L, int32_t *out_branch,
                         int32_t *out_next, uint64_t *counters);
int oracle_vocab_trim(const int32_t *tokens, int64_t N, int Vt, double P, int32_t *out_d2t, int32_t *out_t2d,
                      int32_t *out_vd, int64_t *out_info);
int oracle_greedy_from_argmax(const int32_t *g, const int32_t *tokens, int B, int gamma, int V,
                              int32_t *out_tokens, int32_t *out_len, int32_t *out_status);
int oracle_verify_greedy(const void *logits, int dtype, const int32_t *tokens, int B, int gamma, int V,
                         int32_t *out_tokens, int32_t *out_len, int32_t *out_status);
int oracle_tree_from_argmax(const int32_t *gall, const int32_t *node_tokens, const int32_t *parents, int B, int N,
                            int V, int32_t *out_path, int32_t *out_tokens, int32_t *out_len, int32_t *out_status);
int oracle_verify_tree_greedy(const void *logits, int dtype, const int32_t *node_tokens, const int32_t *parents,
                              int B, int N, int V, int32_t *out_path, int32_t *out_tokens, int32_t *out_len,
                              int32_t *out_status);

static int g_fail = 0;
#define EXPECT(c)                                                               \
    do {                                                                        \
        if (!(c)) {                                                             \
            fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #c);        \
            ++g_fail;                                                           \
        }                                                                       \
    } while (0)

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {               /* xorshift64*, high half */
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    return (uint32_t)((g_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static float unif(void) { return (float)(rnd() >> 8) / 16777216.0f; }
static float normal(void) {
    float s = 0.0f;
    for (int i = 0; i < 12; ++i) s += unif();
    return s - 6.0f;
}
static uint16_t bf16(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    return (uint16_t)(u >> 16);
}
/* n float32 logits (scale sd, every 7th -inf when holes) and their bfloat16 form */
static void logits(float *f, uint16_t *h, int n, float sd, int holes) {
    for (int i = 0; i < n; ++i) {
        f[i] = (holes && i % 7 == 3) ? -INFINITY : sd * normal();
        h[i] = bf16(f[i]);
        f[i] = holes && i % 7 == 3 ? -INFINITY : f[i];
    }
}

static void sample_cases(void) {
    enum { B = 3, G = 4, VT = 37, VD = 20 };
    float tl[B * (G + 1) * VT], dl[B * G * VT], dlm[B * G * VD], ua[B * G], us[B];
    uint16_t tlh[B * (G + 1) * VT], dlh[B * G * VT];
    int32_t tok[B * G], d2t[VD], out_tok[B * (G + 1)], len[B], st[B], fl[B];
    double p[B * G], q[B * G], margin[B * (2 * G + 1) * 2];
    int8_t kd[B * (2 * G + 1)];
    logits(tl, tlh, B * (G + 1) * VT, 2.0f, 0);
    logits(dl, dlh, B * G * VT, 2.0f, 0);
    uint16_t tmp[B * G * VD];
    logits(dlm, tmp, B * G * VD, 1.5f, 0);
    for (int i = 0; i < B * G; ++i) {
        tok[i] = (int32_t)(rnd() % VT);
        ua[i] = unif();
    }
    tok[5] = VT + 3;                                        /* out of range */
    for (int b = 0; b < B; ++b) us[b] = unif();
    for (int j = 0; j < VD; ++j) d2t[j] = j + j / 2;        /* strictly increasing, < VT */
    for (int i = 0; i < B * (2 * G + 1); ++i) kd[i] = (int8_t)((int)(rnd() % 3) - 1);
    const double rhos[] = {0.9, 1.0, 0.3};
    for (int r = 0; r < 3; ++r) {
        EXPECT(oracle_verify_sample(tl, 0, dl, 0, tok, NULL, ua, us, B, G, VT, VT, 0.8, rhos[r], 1e-5, NULL, out_tok,
                                    len, p, q, st, fl, margin, 1) == 0);
        EXPECT(oracle_verify_sample(tlh, 1, dlh, 1, tok, NULL, ua, us, B, G, VT, VT, 1.3, rhos[r], 1e-5, kd, out_tok,
                                    len, p, q, st, fl, margin, 3) == 0);
        EXPECT(oracle_verify_sample(tl, 0, dlm, 0, tok, d2t, ua, us, B, G, VT, VD, 1.0, rhos[r], 1e-5, NULL,
                                    out_tok, len, p, q, st, fl, margin, 2) == 0);
    }
    /* gamma 0: the bonus draw alone */
    EXPECT(oracle_verify_sample(tl, 0, dl, 0, tok, NULL, ua, us, B, 0, VT, VT, 0.8, 0.9, 1e-5, NULL, out_tok, len, p,
                                q, st, fl, margin, 1) == 0);
    /* a bad map (not increasing) is reported, not a crash */
    d2t[4] = d2t[3];
    EXPECT(oracle_verify_sample(tl, 0, dlm, 0, tok, d2t, ua, us, B, G, VT, VD, 1.0, 0.9, 1e-5, NULL, out_tok, len, p,
                                q, st, fl, margin, 1) == 0);
    /* argument errors */
    EXPECT(oracle_verify_sample(tl, 0, dl, 0, tok, NULL, ua, us, B, G, VT, VT, 0.0, 0.9, 1e-5, NULL, out_tok, len, p,
                                q, st, fl, margin, 1) != 0);
    EXPECT(oracle_verify_sample(tl, 5, dl, 0, tok, NULL, ua, us, B, G, VT, VT, 1.0, 0.9, 1e-5, NULL, out_tok, len, p,
                                q, st, fl, margin, 1) != 0);
}

static void row_and_chain_cases(void) {
    enum { V = 50 };
    float z[V];
    uint16_t zh[V];
    double p[V], lo, hi;
    int32_t k;
    logits(z, zh, V, 2.0f, 1);
    const int tks[] = {0, 1, 5, 60};
    const double rhos[] = {1.0, 0.5, 1e-9};
    for (int a = 0; a < 4; ++a)
        for (int r = 0; r < 3; ++r)
            for (int d = -1; d <= 1; ++d) {
                EXPECT(oracle_row_dist(z, 0, V, 0.7, rhos[r], tks[a], d, p, &k, &lo, &hi) >= 0);
                EXPECT(oracle_row_dist(zh, 1, V, 1.1, rhos[r], tks[a], d, p, &k, &lo, &hi) >= 0);
            }
    /* every logit -inf, and ties everywhere */
    for (int i = 0; i < V; ++i) z[i] = -INFINITY;
    EXPECT(oracle_row_dist(z, 0, V, 1.0, 0.9, 0, 0, p, &k, &lo, &hi) >= 0);
    for (int i = 0; i < V; ++i) z[i] = 1.5f;
    EXPECT(oracle_row_dist(z, 0, V, 1.0, 0.37, 7, 0, p, &k, &lo, &hi) >= 0);
    EXPECT(oracle_row_dist(z, 0, 1, 1.0, 0.9, 0, 0, p, &k, &lo, &hi) >= 0);

    enum { G = 6 };
    double P[(G + 1) * V], Q[G * V];
    int32_t tok[G], out[G + 1], fl;
    float ua[G];
    for (int i = 0; i < G; ++i) {
        double sp = 0, sq = 0;
        for (int j = 0; j < V; ++j) {
            P[i * V + j] = unif();
            Q[i * V + j] = (j % 5 == 0) ? 0.0 : unif();
            sp += P[i * V + j];
            sq += Q[i * V + j];
        }
        for (int j = 0; j < V; ++j) {
            P[i * V + j] /= sp;
            Q[i * V + j] /= sq;
        }
        tok[i] = (int32_t)(rnd() % V);
        ua[i] = unif();
    }
    for (int j = 0; j < V; ++j) P[G * V + j] = 1.0 / V;
    EXPECT(oracle_chain_from_dists(P, Q, tok, ua, 0.42f, G, V, 1e-5, out, &fl) >= 0);
    EXPECT(oracle_chain_from_dists(P, Q, tok, ua, 0.0f, 0, V, 1e-5, out, &fl) >= 0);
    memcpy(Q, P, sizeof(double) * G * V);                 /* p == q: zero residual */
    EXPECT(oracle_chain_from_dists(P, Q, tok, ua, 0.99f, G, V, 1e-5, out, &fl) >= 0);
}

static void draft_cases(void) {
    enum { B = 4, V = 50 };
    float z[B * V], u[B];
    uint16_t zh[B * V];
    int32_t tok[B], st[B], fl[B], kk[B], d2t[V];
    double prob[B], margin[B * 2];
    int8_t kd[B] = {-1, 0, 1, 0};
    logits(z, zh, B * V, 2.0f, 1);
    for (int b = 0; b < B; ++b) u[b] = unif();
    for (int j = 0; j < V; ++j) d2t[j] = 3 * j;
    const int tks[] = {0, 1, 10, 50, 70};
    for (int a = 0; a < 5; ++a) {
        EXPECT(oracle_draft_sample(z, 0, NULL, u, B, V, 0.8, 0.9, tks[a], 1e-5, NULL, tok, prob, st, fl, margin, kk) ==
               0);
        EXPECT(oracle_draft_sample(zh, 1, d2t, u, B, V, 1.2, 1.0, tks[a], 1e-5, kd, tok, prob, st, fl, margin, kk) ==
               0);
    }
    EXPECT(oracle_draft_sample(z, 0, NULL, u, B, V, -1.0, 0.9, 0, 1e-5, NULL, tok, prob, st, fl, margin, kk) != 0);
    EXPECT(oracle_draft_sample(z, 4, NULL, u, B, V, 1.0, 0.9, 0, 1e-5, NULL, tok, prob, st, fl, margin, kk) != 0);
}

static void count_fanout_trim_cases(void) {
    enum { B = 9, G = 5, F = 3, L = 4 };
    int32_t len[B], out_tok[B * (G + 1)], cand[B * (G + 1) * F], drafts[B * (G + 1) * F * L];
    int32_t branch[B], next[B * L];
    uint64_t ctr[5] = {0}, fctr[2] = {0};
    for (int b = 0; b < B; ++b) len[b] = (int32_t)(rnd() % (G + 1));
    for (int i = 0; i < B * (G + 1); ++i) out_tok[i] = (int32_t)(rnd() % 11);
    for (int i = 0; i < B * (G + 1) * F; ++i) cand[i] = (int32_t)(rnd() % 11);
    for (int i = 0; i < B * (G + 1) * F * L; ++i) drafts[i] = (int32_t)(rnd() % 1000);
    EXPECT(oracle_count(len, B, G, ctr) == 0);
    EXPECT(oracle_count(len, 0, G, ctr) == 0);
    EXPECT(oracle_fanout_lookup(out_tok, len, cand, drafts, B, G, F, L, branch, next, fctr) == 0);
    EXPECT(oracle_fanout_lookup(out_tok, len, cand, NULL, B, G, F, 0, branch, NULL, NULL) == 0);

    enum { N = 5000, VT = 97 };
    static int32_t tk[N], d2t[VT], t2d[VT];
    int32_t vd;
    int64_t info[3];
    for (int i = 0; i < N; ++i) {
        const uint32_t r = rnd() % 1000;
        tk[i] = r < 990 ? (int32_t)((r * r) % VT) : (int32_t)(VT + r % 7) - (r % 2 ? 2 * VT : 0);
    }
    const double Ps[] = {0.95, 0.5, 1e-6, 1.0, 1.5};
    for (int a = 0; a < 5; ++a) EXPECT(oracle_vocab_trim(tk, N, VT, Ps[a], d2t, t2d, &vd, info) == 0);
    EXPECT(oracle_vocab_trim(tk, 0, VT, 0.95, d2t, t2d, &vd, info) == 0);
    EXPECT(oracle_vocab_trim(tk, N, 1, 0.95, d2t, t2d, &vd, info) == 0);
}

static void greedy_tree_cases(void) {
    enum { B = 3, G = 5, V = 41, N = 12 };
    float z[B * (G + 1) * V];
    uint16_t zh[B * (G + 1) * V];
    int32_t tok[B * G], out[B * (G + 1)], len[B], st[B], gmax[B * (G + 1)];
    logits(z, zh, B * (G + 1) * V, 1.0f, 1);
    for (int i = 0; i < B * G; ++i) tok[i] = (int32_t)(rnd() % V);
    tok[2] = -4;
    for (int i = 0; i < B * (G + 1); ++i) gmax[i] = (int32_t)(rnd() % V);
    EXPECT(oracle_verify_greedy(z, 0, tok, B, G, V, out, len, st) == 0);
    EXPECT(oracle_verify_greedy(zh, 1, tok, B, G, V, out, len, st) == 0);
    EXPECT(oracle_verify_greedy(z, 0, tok, B, 0, V, out, len, st) == 0);
    EXPECT(oracle_greedy_from_argmax(gmax, tok, B, G, V, out, len, st) == 0);
    EXPECT(oracle_verify_greedy(z, 3, tok, B, G, V, out, len, st) != 0);

    float zt[B * N * V];
    uint16_t zth[B * N * V];
    int32_t nt[B * N], par[B * N], path[B * N], ttok[B * N], all[B * N];
    logits(zt, zth, B * N * V, 1.0f, 0);
    for (int b = 0; b < B; ++b)
        for (int k = 0; k < N; ++k) {
            nt[b * N + k] = (int32_t)(rnd() % V);
            par[b * N + k] = k == 0 ? -1 : (int32_t)(rnd() % (uint32_t)k);
            all[b * N + k] = (int32_t)(rnd() % V);
        }
    par[N + 5] = 9;                                        /* a parent after its child */
    EXPECT(oracle_verify_tree_greedy(zt, 0, nt, par, B, N, V, path, ttok, len, st) == 0);
    EXPECT(oracle_verify_tree_greedy(zth, 1, nt, par, B, N, V, path, ttok, len, st) == 0);
    EXPECT(oracle_tree_from_argmax(all, nt, par, B, N, V, path, ttok, len, st) == 0);
}

int main(void) {
    sample_cases();
    row_and_chain_cases();
    draft_cases();
    count_fanout_trim_cases();
    greedy_tree_cases();
    if (g_fail) {
        fprintf(stderr, "%d call(s) returned an unexpected code\n", g_fail);
        return 1;
    }
    printf("oracle ok\n");
    return 0;
}
