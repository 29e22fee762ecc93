/*
 * Plain, slow, fp64 CPU oracle for query-aware sparse KV selection and sparse decode
 * (TokenSelect / TokenButler) and for SnapKV prefill-end compression.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call this
 * file; it is used by the test suite, by the smoke check and by the CPU-baseline leg of
 * the benchmark. It shares no code, header or table with the GPU library.
 *
 * Sources (cited by page title and section):
 *   [TS]  "論文解説: TokenSelect — 動的トークンレベルKVキャッシュ選択による長文推論の高速化"
 *         (blog explainer of arXiv 2411.05159).
 *   [TB]  "Technische Zusammenfassung: TokenButler" (summary of arXiv 2503.07518).
 *   [SK]  "NeurIPS 2024論文解説: SnapKV — 生成前にKVキャッシュの重要トークンを選択する手法"
 *         (blog explainer of arXiv 2402.02938).
 *
 * Conventions shared with the caller (plain data contract, not code):
 *   bf16 values are passed as uint16_t bit patterns and widened exactly to double.
 *   d = 128 (head dim), dp = 32 (index dim).  GQA: query head h reads KV head h / G,
 *   G = Hq / Hkv.  Token-major caches: K[t][g][d], packed over a batch by offsets[B+1].
 *   Every floating-point step is fp64, summed in plain index order.
 *
 * Parity pins for every function live in the CPU test suite; no function here is
 * "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define QO_D 128
#define QO_DP 32

/* ------------------------------------------------------------------ helpers */

static double bf16_widen(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bfloat16 value, ties to even.  The value is scaled so
 * that one bf16 quantum (8 significant bits; subnormal quantum 2^-133) becomes 1, rounded
 * to an integer with nearbyint (nearest-even in the default rounding mode), and scaled
 * back.  The result has at most 8 significant bits, so the final float conversion is
 * exact (or overflows to infinity, which is also the RNE result). */
static uint16_t bf16_round(double x) {
    if (x == 0.0) return signbit(x) ? 0x8000u : 0x0000u;
    double a = fabs(x);
    int e;
    frexp(a, &e);                 /* a in [2^(e-1), 2^e) */
    int q = (e - 1) - 7;          /* exponent of one quantum */
    if (q < -133) q = -133;
    double r = nearbyint(ldexp(a, -q));
    float f = (float)ldexp(r, q);
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint16_t bits = (uint16_t)(u >> 16);
    if (signbit(x)) bits |= 0x8000u;
    return bits;
}

uint16_t qo_bf16_round(double x) { return bf16_round(x); }
double qo_bf16_widen(uint16_t b) { return bf16_widen(b); }

/* ------------------------------------------------------------ index append */

/* [TS] "Query-Key Dot Product Index": the compressed key index K_index has width
 * d' = d/4 and is built incrementally while decoding.  [TB] "Kernarchitektur": keys are
 * projected into the low-dimensional space by a fixed matrix.  Here
 *   k_index[t][g][c] = bf16( sum_j k[t][g][j] * P[j][c] ),  P is fp32 [128][32].
 * exact_out (nullable) receives the fp64 sum, absmag_out (nullable) sum_j |k_j P_jc|. */
void qo_index_project(const uint16_t* k, const float* P, int64_t T, int Hkv,
                      uint16_t* k_index, double* exact_out, double* absmag_out) {
    for (int64_t t = 0; t < T; ++t)
        for (int g = 0; g < Hkv; ++g) {
            const uint16_t* row = k + (t * Hkv + g) * QO_D;
            for (int c = 0; c < QO_DP; ++c) {
                double s = 0.0, m = 0.0;
                for (int j = 0; j < QO_D; ++j) {
                    double p = bf16_widen(row[j]) * (double)P[j * QO_DP + c];
                    s += p;
                    m += fabs(p);
                }
                int64_t o = (t * Hkv + g) * QO_DP + c;
                k_index[o] = bf16_round(s);
                if (exact_out) exact_out[o] = s;
                if (absmag_out) absmag_out[o] = m;
            }
        }
}

/* ------------------------------------------------------------------- score */

/* [TS] "Query-Key Dot Product Index", eq. Score_h(i) = q_h . k_index,h(i) / sqrt(d').
 * The query is projected with the same P (q'_h = P^T q_h, kept in fp64), and head h
 * reads KV head g = h / G.  scores is [Hq][Ntot], head-major over the packed tokens. */
void qo_score(const uint16_t* q, const float* P, const uint16_t* k_index,
              const int64_t* offsets, int B, int Hq, int Hkv, double* scores) {
    int G = Hq / Hkv;
    int64_t Ntot = offsets[B];
    double qp[QO_DP];
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hq; ++h) {
            const uint16_t* qh = q + ((int64_t)b * Hq + h) * QO_D;
            for (int c = 0; c < QO_DP; ++c) {
                double s = 0.0;
                for (int j = 0; j < QO_D; ++j) s += bf16_widen(qh[j]) * (double)P[j * QO_DP + c];
                qp[c] = s;
            }
            int g = h / G;
            for (int64_t t = offsets[b]; t < offsets[b + 1]; ++t) {
                const uint16_t* ki = k_index + (t * Hkv + g) * QO_DP;
                double s = 0.0;
                for (int c = 0; c < QO_DP; ++c) s += qp[c] * bf16_widen(ki[c]);
                scores[(int64_t)h * Ntot + t] = s / sqrt((double)QO_DP);
            }
        }
}

/* ------------------------------------------------------------------- theta */

static int cmp_double_asc(const void* a, const void* b) {
    double x = *(const double*)a, y = *(const double*)b;
    return (x < y) ? -1 : (x > y) ? 1 : 0;
}

/* Rank of the head threshold: r = ceil(n * num / den), clamped to [1, n]. */
int64_t qo_theta_rank(int64_t n, int64_t num, int64_t den) {
    int64_t r = (n * num + den - 1) / den;
    if (r < 1) r = 1;
    if (r > n) r = n;
    return r;
}

/* [TS] "Voting Mechanism": each head h has its own threshold theta_h.  Read here as the
 * nearest-rank order statistic theta_h = s_(r) of the head's n scores (ascending sort,
 * 1-based r = ceil(n*num/den)); num/den = 9/10 is the 90th percentile, 1/2 the median
 * used by the page's code listing.  theta is [B][Hq]. */
void qo_theta(const double* scores, const int64_t* offsets, int B, int Hq,
              int64_t num, int64_t den, double* theta) {
    int64_t Ntot = offsets[B];
    for (int b = 0; b < B; ++b) {
        int64_t n = offsets[b + 1] - offsets[b];
        double* tmp = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
        for (int h = 0; h < Hq; ++h) {
            memcpy(tmp, scores + (int64_t)h * Ntot + offsets[b], (size_t)n * sizeof(double));
            qsort(tmp, (size_t)n, sizeof(double), cmp_double_asc);
            theta[(int64_t)b * Hq + h] = n > 0 ? tmp[qo_theta_rank(n, num, den) - 1] : 0.0;
        }
        free(tmp);
    }
}

/* -------------------------------------------------------------------- vote */

/* [TS] "Voting Mechanism", eq. Vote(i) = sum_h 1[Score_h(i) > theta_h], strict, summed
 * over every query head of the sequence.  votes is [Ntot]. */
void qo_votes(const double* scores, const double* theta, const int64_t* offsets, int B, int Hq,
              int32_t* votes) {
    int64_t Ntot = offsets[B];
    for (int b = 0; b < B; ++b)
        for (int64_t t = offsets[b]; t < offsets[b + 1]; ++t) {
            int32_t v = 0;
            for (int h = 0; h < Hq; ++h)
                if (scores[(int64_t)h * Ntot + t] > theta[(int64_t)b * Hq + h]) ++v;
            votes[t] = v;
        }
}

/* ---------------------------------------------------------------- selection */

/* [TS] "Token-Level Selection と Sparse Attention" and the code listing of
 * "基本的な統合パターン": the budget is k = max(int(n * budget), sink + local), clipped to
 * n here; the first `sink` and the last `local` tokens are always taken. */
int64_t qo_budget_tokens(int64_t n, int64_t bnum, int64_t bden, int64_t sink, int64_t local) {
    int64_t k = (n * bnum) / bden;
    if (k < sink + local) k = sink + local;
    if (k > n) k = n;
    return k;
}

static int is_forced(int64_t i, int64_t n, int64_t sink, int64_t local) {
    return i < sink || i >= n - local;
}

typedef struct { double key; int64_t idx; } qo_item;

/* Higher key first; equal keys (including -0 vs +0) go to the lower index. */
static int cmp_item(const void* a, const void* b) {
    const qo_item* x = (const qo_item*)a;
    const qo_item* y = (const qo_item*)b;
    if (x->key > y->key) return -1;
    if (x->key < y->key) return 1;
    return (x->idx < y->idx) ? -1 : (x->idx > y->idx) ? 1 : 0;
}

/* Take the forced tokens, then the best `k - |F|` non-forced tokens by key (ties to the
 * lower index), and write the chosen positions in ascending order.  Returns k. */
static int64_t select_one(const double* key, int64_t n, int64_t k, int64_t sink, int64_t local,
                          int32_t* out) {
    char* take = (char*)calloc((size_t)(n > 0 ? n : 1), 1);
    qo_item* items = (qo_item*)malloc((size_t)(n > 0 ? n : 1) * sizeof(qo_item));
    int64_t nf = 0, m = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (is_forced(i, n, sink, local)) { take[i] = 1; ++nf; }
        else { items[m].key = key[i]; items[m].idx = i; ++m; }
    }
    qsort(items, (size_t)m, sizeof(qo_item), cmp_item);
    for (int64_t j = 0; j < k - nf && j < m; ++j) take[items[j].idx] = 1;
    int64_t w = 0;
    for (int64_t i = 0; i < n; ++i)
        if (take[i]) out[w++] = (int32_t)i;
    free(items);
    free(take);
    return w;
}

/* Vote mode.  [TS] eq. S = top-K({i : Vote(i) >= V_min}) with the listing's rule that
 * tokens below V_min keep the key -1 (they remain fillable), sink and local tokens
 * forced, and ascending output.  One shared list per sequence: idx[kpre_b + j],
 * kpre_b = sum of the budgets of the earlier sequences; count[b] = budget. */
void qo_select_vote(const int32_t* votes, const int64_t* offsets, int B,
                    int64_t bnum, int64_t bden, int64_t sink, int64_t local, int64_t vmin,
                    int32_t* idx, int64_t* count) {
    int64_t kpre = 0;
    for (int b = 0; b < B; ++b) {
        int64_t n = offsets[b + 1] - offsets[b];
        int64_t k = qo_budget_tokens(n, bnum, bden, sink, local);
        double* key = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
        for (int64_t i = 0; i < n; ++i) {
            int32_t v = votes[offsets[b] + i];
            key[i] = (v >= vmin) ? (double)v : -1.0;
        }
        count[b] = select_one(key, n, k, sink, local, idx + kpre);
        kpre += k;
        free(key);
    }
}

/* Per-head mode ([TS] "主要な貢献" per-head dynamic selection, the "w/o Voting" ablation;
 * [TB] "Kernarchitektur" scoring under a fixed budget): each query head ranks tokens by
 * its own score.  idx[Hq*kpre_b + h*k_b + j]; count[b] = k_b. */
void qo_select_per_head(const double* scores, const int64_t* offsets, int B, int Hq,
                        int64_t bnum, int64_t bden, int64_t sink, int64_t local,
                        int32_t* idx, int64_t* count) {
    int64_t Ntot = offsets[B];
    int64_t kpre = 0;
    for (int b = 0; b < B; ++b) {
        int64_t n = offsets[b + 1] - offsets[b];
        int64_t k = qo_budget_tokens(n, bnum, bden, sink, local);
        for (int h = 0; h < Hq; ++h)
            select_one(scores + (int64_t)h * Ntot + offsets[b], n, k, sink, local,
                       idx + Hq * kpre + (int64_t)h * k);
        count[b] = k;
        kpre += k;
    }
}

/* ------------------------------------------------------------------ decode */

/* [TS] eq. Attention(Q, K_S, V_S) = softmax(Q K_S^T / sqrt(d)) V_S over the selected set,
 * which already holds the sink and local tokens, so the "output merge" of sparse and
 * local attention is one softmax over their disjoint union.  mode 0: one list per
 * sequence (idx[kpre_b + j]); mode 1: one list per query head
 * (idx[Hq*kpre_b + h*count_b + j]).  Negative entries are empty slots (the padding of an
 * expanded list) and are skipped.  out is [B][Hq][128]. */
void qo_decode(const uint16_t* q, const uint16_t* K, const uint16_t* V, const int64_t* offsets,
               const int32_t* idx, const int64_t* count, int mode, int B, int Hq, int Hkv,
               double* out) {
    int G = Hq / Hkv;
    int64_t kpre = 0;
    for (int b = 0; b < B; ++b) {
        int64_t cnt = count[b];
        double* z = (double*)malloc((size_t)(cnt > 0 ? cnt : 1) * sizeof(double));
        for (int h = 0; h < Hq; ++h) {
            int g = h / G;
            const int32_t* list = (mode == 0) ? idx + kpre : idx + Hq * kpre + (int64_t)h * cnt;
            const uint16_t* qh = q + ((int64_t)b * Hq + h) * QO_D;
            double* o = out + ((int64_t)b * Hq + h) * QO_D;
            double m = -INFINITY;
            for (int64_t j = 0; j < cnt; ++j) {
                if (list[j] < 0) continue;
                const uint16_t* kr = K + ((offsets[b] + list[j]) * Hkv + g) * QO_D;
                double s = 0.0;
                for (int e = 0; e < QO_D; ++e) s += bf16_widen(qh[e]) * bf16_widen(kr[e]);
                z[j] = s / sqrt((double)QO_D);
                if (z[j] > m) m = z[j];
            }
            double l = 0.0;
            for (int e = 0; e < QO_D; ++e) o[e] = 0.0;
            for (int64_t j = 0; j < cnt; ++j) {
                if (list[j] < 0) continue;
                double w = exp(z[j] - m);
                l += w;
                const uint16_t* vr = V + ((offsets[b] + list[j]) * Hkv + g) * QO_D;
                for (int e = 0; e < QO_D; ++e) o[e] += w * bf16_widen(vr[e]);
            }
            for (int e = 0; e < QO_D; ++e) o[e] = (cnt > 0) ? o[e] / l : 0.0;
        }
        free(z);
        kpre += cnt;
    }
}

/* Dense softmax attention of the decode query over all n_b cached tokens
 * ([TS] eq. S_i = q . k_i / sqrt(d) for every token, then softmax-weighted V). */
void qo_dense_decode(const uint16_t* q, const uint16_t* K, const uint16_t* V,
                     const int64_t* offsets, int B, int Hq, int Hkv, double* out) {
    int64_t Ntot = offsets[B];
    int32_t* idx = (int32_t*)malloc((size_t)(Ntot > 0 ? Ntot : 1) * sizeof(int32_t));
    int64_t* count = (int64_t*)malloc((size_t)B * sizeof(int64_t));
    for (int b = 0; b < B; ++b) {
        count[b] = offsets[b + 1] - offsets[b];
        for (int64_t i = 0; i < count[b]; ++i) idx[offsets[b] + i] = (int32_t)i;
    }
    qo_decode(q, K, V, offsets, idx, count, 0, B, Hq, Hkv, out);
    free(count);
    free(idx);
}

/* ------------------------------------------------------------------ SnapKV */

/* [SK] "Attention Score計算とPooling": for each KV head g, every observation-window row
 * r = (query head h of group g, window position t) gets A_r = softmax_j(q_r . k_j /
 * sqrt(d_k)) over all n keys (no mask inside the window), and the importance is the mean
 * of A over the window; the pipeline figure averages across the heads that share the
 * KV head as well, so the mean runs over all G*w rows.  q_obs is [w][Hq][128]; K is
 * [n][Hkv][128]; importance is [Hkv][n]. */
void qo_snapkv_importance(const uint16_t* q_obs, const uint16_t* K, int64_t n, int w, int Hq,
                          int Hkv, double* importance) {
    int G = Hq / Hkv;
    double* s = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    double rows = (double)G * (double)w;
    for (int g = 0; g < Hkv; ++g) {
        double* imp = importance + (int64_t)g * n;
        for (int64_t j = 0; j < n; ++j) imp[j] = 0.0;
        for (int h = g * G; h < (g + 1) * G; ++h)
            for (int t = 0; t < w; ++t) {
                const uint16_t* qr = q_obs + ((int64_t)t * Hq + h) * QO_D;
                double m = -INFINITY;
                for (int64_t j = 0; j < n; ++j) {
                    const uint16_t* kr = K + (j * Hkv + g) * QO_D;
                    double acc = 0.0;
                    for (int e = 0; e < QO_D; ++e) acc += bf16_widen(qr[e]) * bf16_widen(kr[e]);
                    s[j] = acc / sqrt((double)QO_D);
                    if (s[j] > m) m = s[j];
                }
                double l = 0.0;
                for (int64_t j = 0; j < n; ++j) l += exp(s[j] - m);
                for (int64_t j = 0; j < n; ++j) imp[j] += exp(s[j] - m) / l;
            }
        for (int64_t j = 0; j < n; ++j) imp[j] /= rows;
    }
    free(s);
}

/* [SK] "アルゴリズム": avg_pool1d(kernel, padding = kernel/2, stride 1) along the
 * tokens, zero padding counted in the divisor (the divisor is always `kernel`).
 * kernel must be odd so the output keeps length n.  in/out are [rows][n]. */
void qo_avg_pool1d(const double* in, int64_t rows, int64_t n, int kernel, double* out) {
    int half = kernel / 2;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < n; ++j) {
            double s = 0.0;
            for (int o = -half; o <= half; ++o) {
                int64_t jj = j + o;
                if (jj >= 0 && jj < n) s += in[r * n + jj];
            }
            out[r * n + j] = s / (double)kernel;
        }
}

/* [SK] "Top-k SelectionとCluster-based Retention" eq. S = top-k(a, c) per KV head, with
 * c clipped to n and the kept positions sorted ascending, as the listing of "アルゴリズム"
 * does; ties go to the lower index.  pooled is [rows][n]; idx is [rows][min(c, n)]. */
int64_t qo_topc(const double* pooled, int64_t rows, int64_t n, int64_t c, int32_t* idx) {
    int64_t ce = c < n ? c : n;
    for (int64_t r = 0; r < rows; ++r) {
        /* no forced tokens here: sink = local = 0 */
        select_one(pooled + r * n, n, ce, 0, 0, idx + r * ce);
    }
    return ce;
}

/* [SK] "アルゴリズム": gather the chosen K and V rows of each KV head into a compacted
 * cache K_out[s][g][128] = K[idx[g][s]][g][128] (bit copies).  An empty slot (idx < 0, the
 * padding of a cluster-widened list) gets a zero row. */
void qo_gather_rows(const uint16_t* K, const uint16_t* V, int64_t n, int Hkv, const int32_t* idx,
                    int64_t ce, uint16_t* K_out, uint16_t* V_out) {
    (void)n;
    for (int g = 0; g < Hkv; ++g)
        for (int64_t s = 0; s < ce; ++s) {
            int64_t t = idx[(int64_t)g * ce + s];
            int64_t dst = (s * Hkv + g) * QO_D;
            if (t < 0) {
                memset(K_out + dst, 0, QO_D * sizeof(uint16_t));
                memset(V_out + dst, 0, QO_D * sizeof(uint16_t));
                continue;
            }
            int64_t src = (t * Hkv + g) * QO_D;
            memcpy(K_out + dst, K + src, QO_D * sizeof(uint16_t));
            memcpy(V_out + dst, V + src, QO_D * sizeof(uint16_t));
        }
}

/* ------------------------------------------------- selection reuse + neighbours */

/* Capacity of an expanded list: min(n, (2 radius + 1) k_prev + sink + local). */
int64_t qo_expand_capacity(int64_t k_prev, int64_t n, int64_t sink, int64_t local, int64_t radius) {
    int64_t c = (2 * radius + 1) * k_prev + sink + local;
    return c < n ? c : n;
}

/* [TB] "Inferenzstrategie", Optimierungen (prediction interval and neighbour fetch): the
 * selector runs every N decode steps; in between, the last selection is reused, widened by the
 * spatial neighbours of every selected token, and the current step's always-kept tokens are
 * added.  For each list (one per sequence, or one per query head of a sequence): the set
 *   { t + d : t in prev, |d| <= radius, 0 <= t + d < n } U [0, min(sink, n)) U [max(0, n - local), n)
 * in ascending order, followed by -1 (empty slots) up to the list's capacity.  Lists are laid
 * out like ts_select's: list l of sequence b at out[L * cpre_b + l * cap_b + j] (L lists per
 * sequence, cpre_b = sum of the earlier sequences' capacities), the previous lists likewise with
 * the previous counts.  count_out[b * L + l] = the number of valid entries. */
void qo_expand_selection(const int32_t* prev, const int64_t* counts_prev, const int64_t* offsets, int B, int L,
                         int64_t sink, int64_t local, int64_t radius, int32_t* out, int64_t* count_out) {
    int64_t ppre = 0, cpre = 0;
    for (int b = 0; b < B; ++b) {
        int64_t n = offsets[b + 1] - offsets[b];
        int64_t kp = counts_prev[b];
        int64_t cap = qo_expand_capacity(kp, n, sink, local, radius);
        char* take = (char*)calloc((size_t)(n > 0 ? n : 1), 1);
        for (int l = 0; l < L; ++l) {
            memset(take, 0, (size_t)(n > 0 ? n : 1));
            const int32_t* p = prev + L * ppre + (int64_t)l * kp;
            for (int64_t j = 0; j < kp; ++j)
                for (int64_t d = -radius; d <= radius; ++d) {
                    int64_t t = (int64_t)p[j] + d;
                    if (t >= 0 && t < n) take[t] = 1;
                }
            for (int64_t t = 0; t < n; ++t)
                if (is_forced(t, n, sink, local)) take[t] = 1;
            int32_t* o = out + L * cpre + (int64_t)l * cap;
            int64_t w = 0;
            for (int64_t t = 0; t < n; ++t)
                if (take[t]) o[w++] = (int32_t)t;
            count_out[(int64_t)b * L + l] = w;
            for (; w < cap; ++w) o[w] = -1;
        }
        free(take);
        ppre += kp;
        cpre += cap;
    }
}

/* [SK] "Top-k SelectionとCluster-based Retention", eq. S_final = U_{j in S} {j - k, ..., j + k}:
 * every KV head's top-c positions widened by their k_cluster neighbours (inside [0, n)),
 * ascending, padded with -1 to min(n, (2 k_cluster + 1) ce); then the rows gathered as
 * qo_gather_rows does.  idx is [Hkv][ce]; idx_out is [Hkv][cap]; valid_out[g] = the number of
 * entries before the padding.  (The neighbour widening of the selection reuse with no
 * always-kept tokens.)  Returns cap. */
int64_t qo_snapkv_retain_clusters(const uint16_t* K, const uint16_t* V, int64_t n, int Hkv, const int32_t* idx,
                                  int64_t ce, int64_t k_cluster, int32_t* idx_out, uint16_t* K_out,
                                  uint16_t* V_out, int64_t* valid_out) {
    int64_t offsets[2] = {0, n};
    int64_t counts[1] = {ce};
    int64_t cap = qo_expand_capacity(ce, n, 0, 0, k_cluster);
    qo_expand_selection(idx, counts, offsets, 1, Hkv, 0, 0, k_cluster, idx_out, valid_out);
    qo_gather_rows(K, V, n, Hkv, idx_out, cap, K_out, V_out);
    return cap;
}

/* Per-KV-group union of the per-head lists (per-head mode's decode input: [TS] "主要な貢献",
 * each head selects its own tokens; the G query heads of a KV head read the same K/V rows, so
 * the decode reads each row of the group's union once and lets every head use the rows it
 * selected).  idx and count are qo_select_per_head's output (idx[Hq*kpre_b + h*k_b + j],
 * count[b] = k_b).  For sequence b and KV head g, in the block of G*k_b entries at
 * uidx[Hq*kpre_b + g*G*k_b ...]: the tokens of the union of lists g*G .. g*G+G-1 in ascending
 * order, then -1; umask (same layout) has bit hh set when head g*G+hh selected the token (0 for
 * the padding); ucount[b*Hkv + g] = the union's size.  Entries outside [0, n_b) are empty slots
 * (the -1 that pads an expanded list, qo_expand_selection) and join no union. */
void qo_union_lists(const int32_t* idx, const int64_t* count, const int64_t* offsets, int B, int Hq, int Hkv,
                    int32_t* uidx, uint8_t* umask, int64_t* ucount) {
    const int G = Hq / Hkv;
    int64_t kpre = 0;
    for (int b = 0; b < B; ++b) {
        const int64_t n = offsets[b + 1] - offsets[b], k = count[b];
        uint8_t* mark = (uint8_t*)calloc((size_t)(n > 0 ? n : 1), 1);
        for (int g = 0; g < Hkv; ++g) {
            memset(mark, 0, (size_t)(n > 0 ? n : 1));
            for (int hh = 0; hh < G; ++hh) {
                const int32_t* list = idx + (int64_t)Hq * kpre + (int64_t)(g * G + hh) * k;
                for (int64_t j = 0; j < k; ++j)     /* entries outside [0, n) are empty slots */
                    if (list[j] >= 0 && list[j] < n) mark[list[j]] |= (uint8_t)(1u << hh);
            }
            int32_t* uo = uidx + (int64_t)Hq * kpre + (int64_t)g * G * k;
            uint8_t* mo = umask + (int64_t)Hq * kpre + (int64_t)g * G * k;
            int64_t w = 0;
            for (int64_t t = 0; t < n; ++t)
                if (mark[t]) {
                    uo[w] = (int32_t)t;
                    mo[w] = mark[t];
                    ++w;
                }
            ucount[(int64_t)b * Hkv + g] = w;
            for (; w < (int64_t)G * k; ++w) {
                uo[w] = -1;
                mo[w] = 0;
            }
        }
        free(mark);
        kpre += k;
    }
}
