/*
 * Sanitizer driver for the CPU oracle (test infrastructure): runs every oracle function on small
 * seeded inputs (a ragged batch, a one-token sequence, empty and full budgets) so that a build
 * with AddressSanitizer and UndefinedBehaviorSanitizer checks every array access and every
 * integer operation of the oracle.  Exits 0 when every call returns; the sanitizers abort on
 * the first error.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint16_t qo_bf16_round(double x);
double qo_bf16_widen(uint16_t b);
void qo_index_project(const uint16_t* k, const float* P, int64_t T, int Hkv, uint16_t* k_index, double* exact_out,
                      double* absmag_out);
void qo_score(const uint16_t* q, const float* P, const uint16_t* k_index, const int64_t* offsets, int B, int Hq,
              int Hkv, double* scores);
int64_t qo_theta_rank(int64_t n, int64_t num, int64_t den);
void qo_theta(const double* scores, const int64_t* offsets, int B, int Hq, int64_t num, int64_t den, double* theta);
void qo_votes(const double* scores, const double* theta, const int64_t* offsets, int B, int Hq, int32_t* votes);
int64_t qo_budget_tokens(int64_t n, int64_t bnum, int64_t bden, int64_t sink, int64_t local);
void qo_select_vote(const int32_t* votes, const int64_t* offsets, int B, int64_t bnum, int64_t bden, int64_t sink,
                    int64_t local, int64_t vmin, int32_t* idx, int64_t* count);
void qo_select_per_head(const double* scores, const int64_t* offsets, int B, int Hq, int64_t bnum, int64_t bden,
                        int64_t sink, int64_t local, int32_t* idx, int64_t* count);
void qo_decode(const uint16_t* q, const uint16_t* K, const uint16_t* V, const int64_t* offsets, const int32_t* idx,
               const int64_t* count, int mode, int B, int Hq, int Hkv, double* out);
void qo_dense_decode(const uint16_t* q, const uint16_t* K, const uint16_t* V, const int64_t* offsets, int B, int Hq,
                     int Hkv, double* out);
void qo_snapkv_importance(const uint16_t* q_obs, const uint16_t* K, int64_t n, int w, int Hq, int Hkv,
                          double* importance);
void qo_avg_pool1d(const double* in, int64_t rows, int64_t n, int kernel, double* out);
int64_t qo_topc(const double* pooled, int64_t rows, int64_t n, int64_t c, int32_t* idx);
void qo_gather_rows(const uint16_t* K, const uint16_t* V, int64_t n, int Hkv, const int32_t* idx, int64_t ce,
                    uint16_t* K_out, uint16_t* V_out);
int64_t qo_expand_capacity(int64_t k_prev, int64_t n, int64_t sink, int64_t local, int64_t radius);
void qo_expand_selection(const int32_t* prev, const int64_t* counts_prev, const int64_t* offsets, int B, int L,
                         int64_t sink, int64_t local, int64_t radius, int32_t* out, int64_t* count_out);
int64_t qo_snapkv_retain_clusters(const uint16_t* K, const uint16_t* V, int64_t n, int Hkv, const int32_t* idx,
                                  int64_t ce, int64_t k_cluster, int32_t* idx_out, uint16_t* K_out, uint16_t* V_out,
                                  int64_t* valid_out);

#define D 128
#define DP 32

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static double unif(void) {                    /* xorshift64*, uniform in [-1, 1) */
    rng ^= rng >> 12;
    rng ^= rng << 25;
    rng ^= rng >> 27;
    return (double)((rng * 0x2545f4914f6cdd1dull) >> 11) / (double)(1ull << 52) - 1.0;
}
static void fill_bf16(uint16_t* x, int64_t count) {
    for (int64_t i = 0; i < count; ++i) x[i] = qo_bf16_round(2.0 * unif());
}
static void* xalloc(size_t bytes) {
    void* p = malloc(bytes ? bytes : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}

/* one decode-step pipeline over a ragged batch, in both selection modes */
static void pipeline(const int64_t* offsets, int B, int Hq, int Hkv, int64_t bnum, int64_t bden, int64_t sink,
                     int64_t local) {
    const int64_t ntot = offsets[B];
    uint16_t* K = xalloc(sizeof(uint16_t) * ntot * Hkv * D);
    uint16_t* V = xalloc(sizeof(uint16_t) * ntot * Hkv * D);
    uint16_t* q = xalloc(sizeof(uint16_t) * B * Hq * D);
    float* P = xalloc(sizeof(float) * D * DP);
    fill_bf16(K, ntot * Hkv * D);
    fill_bf16(V, ntot * Hkv * D);
    fill_bf16(q, (int64_t)B * Hq * D);
    for (int i = 0; i < D * DP; ++i) P[i] = (float)(0.1 * unif());
    uint16_t* ki = xalloc(sizeof(uint16_t) * ntot * Hkv * DP);
    double* ex = xalloc(sizeof(double) * ntot * Hkv * DP);
    double* mg = xalloc(sizeof(double) * ntot * Hkv * DP);
    qo_index_project(K, P, ntot, Hkv, ki, ex, mg);
    qo_index_project(K, P, ntot, Hkv, ki, NULL, NULL);
    double* sc = xalloc(sizeof(double) * Hq * ntot);
    qo_score(q, P, ki, offsets, B, Hq, Hkv, sc);
    double* th = xalloc(sizeof(double) * B * Hq);
    qo_theta(sc, offsets, B, Hq, 9, 10, th);
    qo_theta(sc, offsets, B, Hq, 1, 2, th);
    int32_t* vt = xalloc(sizeof(int32_t) * ntot);
    qo_votes(sc, th, offsets, B, Hq, vt);
    int64_t ktot = 0;
    for (int b = 0; b < B; ++b) ktot += qo_budget_tokens(offsets[b + 1] - offsets[b], bnum, bden, sink, local);
    int32_t* iv = xalloc(sizeof(int32_t) * (ktot ? ktot : 1));
    int32_t* ih = xalloc(sizeof(int32_t) * (Hq * ktot ? Hq * ktot : 1));
    int64_t* cv = xalloc(sizeof(int64_t) * B);
    int64_t* ch = xalloc(sizeof(int64_t) * B);
    qo_select_vote(vt, offsets, B, bnum, bden, sink, local, 1, iv, cv);
    qo_select_vote(vt, offsets, B, bnum, bden, sink, local, 3, iv, cv);
    qo_select_per_head(sc, offsets, B, Hq, bnum, bden, sink, local, ih, ch);
    double* out = xalloc(sizeof(double) * B * Hq * D);
    qo_decode(q, K, V, offsets, iv, cv, 0, B, Hq, Hkv, out);
    qo_decode(q, K, V, offsets, ih, ch, 1, B, Hq, Hkv, out);
    qo_dense_decode(q, K, V, offsets, B, Hq, Hkv, out);
    /* selection reuse: the vote lists (one per sequence) and the per-head lists widened */
    for (int mode = 0; mode < 2; ++mode) {
        const int L = mode ? Hq : 1;
        int64_t cap = 0;
        for (int b = 0; b < B; ++b)
            cap += qo_expand_capacity(mode ? ch[b] : cv[b], offsets[b + 1] - offsets[b], sink, local, 1);
        int32_t* xo = xalloc(sizeof(int32_t) * (L * cap ? L * cap : 1));
        int64_t* xc = xalloc(sizeof(int64_t) * B * L);
        qo_expand_selection(mode ? ih : iv, mode ? ch : cv, offsets, B, L, sink, local, 1, xo, xc);
        free(xo);
        free(xc);
    }
    free(K); free(V); free(q); free(P); free(ki); free(ex); free(mg); free(sc); free(th); free(vt);
    free(iv); free(ih); free(cv); free(ch); free(out);
}

static void snapkv(int64_t n, int w, int Hq, int Hkv, int64_t c) {
    uint16_t* qo = xalloc(sizeof(uint16_t) * w * Hq * D);
    uint16_t* K = xalloc(sizeof(uint16_t) * n * Hkv * D);
    uint16_t* V = xalloc(sizeof(uint16_t) * n * Hkv * D);
    fill_bf16(qo, (int64_t)w * Hq * D);
    fill_bf16(K, n * Hkv * D);
    fill_bf16(V, n * Hkv * D);
    double* imp = xalloc(sizeof(double) * Hkv * n);
    double* pooled = xalloc(sizeof(double) * Hkv * n);
    qo_snapkv_importance(qo, K, n, w, Hq, Hkv, imp);
    qo_avg_pool1d(imp, Hkv, n, 3, pooled);
    const int64_t ce = c < n ? c : n;
    int32_t* idx = xalloc(sizeof(int32_t) * Hkv * (ce ? ce : 1));
    qo_topc(pooled, Hkv, n, c, idx);
    uint16_t* Ko = xalloc(sizeof(uint16_t) * (ce ? ce : 1) * Hkv * D);
    uint16_t* Vo = xalloc(sizeof(uint16_t) * (ce ? ce : 1) * Hkv * D);
    qo_gather_rows(K, V, n, Hkv, idx, ce, Ko, Vo);
    for (int64_t k = 0; k <= 2; ++k) {
        const int64_t cap = qo_expand_capacity(ce, n, 0, 0, k);
        int32_t* io = xalloc(sizeof(int32_t) * Hkv * (cap ? cap : 1));
        uint16_t* Kc = xalloc(sizeof(uint16_t) * (cap ? cap : 1) * Hkv * D);
        uint16_t* Vc = xalloc(sizeof(uint16_t) * (cap ? cap : 1) * Hkv * D);
        int64_t* valid = xalloc(sizeof(int64_t) * Hkv);
        qo_snapkv_retain_clusters(K, V, n, Hkv, idx, ce, k, io, Kc, Vc, valid);
        free(io); free(Kc); free(Vc); free(valid);
    }
    free(qo); free(K); free(V); free(imp); free(pooled); free(idx); free(Ko); free(Vo);
}

int main(void) {
    /* rounding helpers at the edges of the bf16 range */
    const double edge[] = {0.0, -0.0, 1e-45, 3.3895313892515355e38, -3.3895313892515355e38, 1.0 + 1.0 / 256.0};
    for (unsigned i = 0; i < sizeof edge / sizeof edge[0]; ++i) (void)qo_bf16_widen(qo_bf16_round(edge[i]));
    for (int64_t n = 1; n < 40; ++n) (void)qo_theta_rank(n, 9, 10);
    (void)qo_budget_tokens(0, 1, 5, 4, 256);
    (void)qo_expand_capacity(0, 0, 4, 256, 1);
    const int64_t off_ragged[] = {0, 300, 337, 338, 600};
    pipeline(off_ragged, 4, 4, 2, 1, 3, 4, 16);           /* ragged, one 1-token sequence */
    pipeline(off_ragged, 4, 8, 2, 1, 1, 4, 16);           /* 100 % budget */
    pipeline(off_ragged, 4, 4, 4, 1, 100, 0, 0);          /* no forced tokens, tiny budget */
    const int64_t off_short[] = {0, 5};
    pipeline(off_short, 1, 2, 1, 1, 5, 4, 256);           /* n below sink + local */
    snapkv(200, 4, 8, 2, 64);
    snapkv(50, 2, 4, 4, 4096);                             /* c past n */
    printf("oracle sanitizer run: ok\n");
    return 0;
}
