/*
 * qasi -- query-aware sparse index for MI355X (gfx950).
 *
 * C ABI of the decode-step hot path shared by TokenSelect and TokenButler (query-aware
 * token-level KV selection followed by sparse attention over the selected tokens, for one
 * attention layer) and of SnapKV prefill-end compression.
 *
 * Sources (cited by page title and section):
 *   [TS] "論文解説: TokenSelect — 動的トークンレベルKVキャッシュ選択による長文推論の高速化"
 *   [TB] "Technische Zusammenfassung: TokenButler"
 *   [SK] "NeurIPS 2024論文解説: SnapKV — 生成前にKVキャッシュの重要トークンを選択する手法"
 *
 * Common conventions
 *   - d = 128 (head dimension) and d' = 32 (index dimension) are fixed; Hkv must be 1, 2,
 *     4 or 8, G = Hq / Hkv must be 1, 2, 4 or 8 (query head h reads KV head h / G) and
 *     Hq <= 64.  Other layouts return QASI_ERR_UNSUPPORTED.
 *   - bf16 tensors are passed as uint16_t bit patterns.  All device pointers must be
 *     16-byte aligned.
 *   - Caches are token-major and packed over a ragged batch: K[t][g][128], V[t][g][128],
 *     K_index[t][g][32], where sequence b owns rows [offsets[b], offsets[b+1]).  Functions
 *     that size launches take the same offsets twice: `offsets_dev` (device, read by the
 *     kernels) and `offsets_host` (host, read synchronously to size grids; no device sync).
 *     For a single sequence (B = 1) the kernels take the bounds, and in the decode calls the
 *     list length, from the host copies as launch arguments, so the two copies must agree.
 *   - Token positions inside index lists are sequence-local (0 .. n_b - 1).
 *   - The caller owns every buffer.  Nothing is allocated or freed by any call; scratch
 *     comes from a caller workspace sized by the *_workspace_bytes queries.  No pointer is
 *     kept after the enqueued work completes.  All work is enqueued asynchronously on the
 *     caller's stream; calls on different streams with different workspaces are independent.
 *   - Return codes: 0 success; QASI_ERR_INVALID (null or misaligned pointer, bad count,
 *     non-monotone offsets, out-of-range parameters); QASI_ERR_UNSUPPORTED (shape outside
 *     the supported set); QASI_ERR_WORKSPACE (workspace too small); QASI_ERR_HIP (a launch
 *     failed).  Validation is synchronous and happens before any HIP call, so a non-zero
 *     return other than QASI_ERR_HIP enqueues nothing.  Device faults are asynchronous and
 *     surface at the caller's next synchronisation.  ts_last_error() returns a
 *     thread-local message for the last failing call.  Inputs are assumed finite.
 */
#ifndef QASI_H
#define QASI_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QASI_OK 0
#define QASI_ERR_INVALID (-1)
#define QASI_ERR_UNSUPPORTED (-2)
#define QASI_ERR_WORKSPACE (-3)
#define QASI_ERR_HIP (-4)

#define QASI_MODE_VOTE 0
#define QASI_MODE_PER_HEAD 1
#define QASI_MODE_UNION 2      /* ts_decode_workspace_bytes only: the workspace of ts_union_decode */
#define QASI_MODE_DENSE 3      /* ts_tiered_decode only: every position of each sequence */

/* Selection parameters ([TS] "基本的な統合パターン", TokenSelectConfig).
 *   budget = budget_num / budget_den of the n_b cached tokens; the list length is
 *            K_b = min(n_b, max(floor(n_b * budget), sink + local)) ([TS] same listing).
 *   sink, local: the first `sink` and last `local` tokens are always selected
 *            ([TS] "Token-Level Selection と Sparse Attention", always-included table).
 *   v_min:   vote mode only; tokens with Vote < v_min rank below every candidate but
 *            remain fillable ([TS] "Voting Mechanism").
 *   theta_num / theta_den: vote mode only; the head threshold is the nearest-rank order
 *            statistic s_(r), r = ceil(n_b * theta_num / theta_den) (9/10: 90th
 *            percentile; 1/2: the median of the page's listing).                       */
typedef struct {
    int32_t mode;          /* QASI_MODE_VOTE or QASI_MODE_PER_HEAD */
    int32_t reserved;
    int64_t budget_num, budget_den;
    int64_t sink, local;
    int64_t v_min;
    int64_t theta_num, theta_den;
} ts_select_params;

/* Thread-local description of the last error (never NULL). */
const char* ts_last_error(void);

/* Row stride S of the score array: offsets[B] rounded up to a multiple of 64 (-1 if invalid). */
int64_t ts_score_stride(const int64_t* offsets_host, int32_t B);

/* K_b for one sequence of n tokens under `p` (host-only helper; -1 if p is invalid or n is
 * outside [0, 2^31]). */
int64_t ts_budget_tokens(int64_t n, const ts_select_params* p);

/* Append T tokens to the compressed key index ([TS] "Query-Key Dot Product Index": the
 * d' = d/4 index is built incrementally during inference; [TB] "Kernarchitektur": keys are
 * projected by a fixed matrix into the low-dimensional space):
 *   k_index[pos + t][g][c] = bf16_rne( sum_j k_new[t][g][j] * P[j][c] )
 * with the sum formed in fp64 and rounded once to bf16 (nearest-even).
 *   k_new   device bf16 [T][Hkv][128]
 *   P       device fp32 [128][32] (one projection shared by all KV heads)
 *   k_index device bf16 [>= pos + T][Hkv][32]; rows pos .. pos+T-1 are written.
 * T = 1 per decode step; T = n rebuilds the index of a whole cache.                   */
int ts_index_append(const uint16_t* k_new, const float* P, uint16_t* k_index, int64_t pos,
                    int64_t T, int32_t Hkv, hipStream_t stream);

/* Workspace for ts_score (the projected queries q'_h, B * Hq * 32 fp32 values). */
size_t ts_score_workspace_bytes(int32_t B, int32_t Hq);

/* Index scores for every query head and cached token ([TS] "Query-Key Dot Product
 * Index", eq. Score_h(i) = q_h . k_index,h(i) / sqrt(d')):  q'_h = P^T q_h (fp32) and
 *   scores[h * S + t] = (q'_h / sqrt(32)) . k_index[t][h / G]   (fp32, t packed over the batch)
 *   q       device bf16 [B][Hq][128] (one decode query per sequence)
 *   k_index device bf16 [Ntot][Hkv][32]
 *   scores  device fp32 [Hq][S]: row stride S = ts_score_stride(offsets_host, B), i.e.
 *           Ntot = offsets[B] rounded up to a multiple of 64 so that rows start on 256-byte
 *           boundaries; entries t >= Ntot of a row are not written.
 *   ws      device workspace of at least ts_score_workspace_bytes(B, Hq) bytes (holds
 *           q'_h / sqrt(32) between the two kernels of the call).                       */
int ts_score(const uint16_t* q, const float* P, const uint16_t* k_index,
             const int64_t* offsets_dev, const int64_t* offsets_host, int32_t B, int32_t Hq,
             int32_t Hkv, float* scores, void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace for ts_select. */
size_t ts_select_workspace_bytes(const int64_t* offsets_host, int32_t B, int32_t Hq,
                                 const ts_select_params* p);

/* Token selection per sequence.
 * Vote mode ([TS] "Voting Mechanism" and "Token-Level Selection", with the listing of
 * "基本的な統合パターン"): theta_h = s_(r) per (sequence, head); Vote(t) = #{h : score_h(t)
 * > theta_h} (strict); key(t) = Vote(t) if Vote(t) >= v_min else -1; the list is the forced
 * tokens F = [0, sink) U [n_b - local, n_b) plus the K_b - |F| non-forced tokens of highest
 * key, ties to the lower position, in ascending order:  idx_out[kpre_b + j], j < K_b, with
 * kpre_b = sum_{b' < b} K_b'.
 * Per-head mode ([TS] "主要な貢献" per-head selection, the "w/o Voting" ablation; [TB]
 * "Kernarchitektur"): the same rule per query head with key = score_h(t); -0 and +0 tie:
 * idx_out[Hq * kpre_b + h * K_b + j].
 *   scores     device fp32 [Hq][S] (as written by ts_score, S = ts_score_stride)
 *   idx_out    device int32 (layout above)
 *   count_out  device int64 [B] (receives K_b)
 *   theta_out  nullable device fp32 [B][Hq] (vote mode: theta_h)
 *   votes_out  nullable device uint8 [Ntot] (vote mode: Vote(t))
 *   ws         device workspace of at least ts_select_workspace_bytes(...) bytes.     */
int ts_select(const float* scores, const int64_t* offsets_dev, const int64_t* offsets_host,
              int32_t B, int32_t Hq, int32_t Hkv, const ts_select_params* p, int32_t* idx_out,
              int64_t* count_out, float* theta_out, uint8_t* votes_out, void* ws,
              size_t ws_bytes, hipStream_t stream);

/* Workspace for ts_score_select. */
size_t ts_score_select_workspace_bytes(const int64_t* offsets_host, int32_t B, int32_t Hq,
                                       const ts_select_params* p);

/* One decode step's index scores and selection in a single call: the same scores as
 * ts_score and the same thresholds, votes and lists as ts_select on them (the outputs are
 * identical), with fewer passes over the score array ([TS] "Query-Key Dot Product Index",
 * "Voting Mechanism", "Token-Level Selection と Sparse Attention"; [TB] "Kernarchitektur").
 * If K_last is non-NULL the call first appends, for every sequence b, the index row of its
 * last token t = offsets[b+1] - 1 from K_last (the K cache, whose row t already holds the
 * step's new key), exactly as ts_index_append(K_last + t*Hkv*128, P, k_index, t, 1, Hkv)
 * would.
 *   q, P, k_index, offsets: as for ts_score (k_index is written only when K_last is given)
 *   K_last    nullable device bf16 [Ntot][Hkv][128]
 *   p, idx_out, count_out, theta_out, votes_out: as for ts_select
 *   scores    device fp32 [Hq][S] (written, S = ts_score_stride)
 *   ws        device workspace of at least ts_score_select_workspace_bytes(...) bytes.
 * Each head's order statistic is found from a key bracket taken from 1024 sampled index
 * scores (rows of more than 16384 candidate keys; shorter rows are ranked whole): the score pass
 * counts, per 64-token tile, the keys below the bracket and keeps the keys inside it; one block
 * per (sequence, head) then ranks the kept keys.  When the target rank falls outside the
 * bracket the whole row is radix-selected instead (same result, tens of microseconds more).   */
int ts_score_select(const uint16_t* q, const float* P, uint16_t* k_index, const uint16_t* K_last,
                    const int64_t* offsets_dev, const int64_t* offsets_host, int32_t B, int32_t Hq,
                    int32_t Hkv, const ts_select_params* p, float* scores, int32_t* idx_out,
                    int64_t* count_out, float* theta_out, uint8_t* votes_out, void* ws,
                    size_t ws_bytes, hipStream_t stream);

/* Diagnostics of ts_score_select's sampled brackets: the byte offset, in its workspace, of the
 * per-instance records that a completed call leaves there (-1 if an argument is invalid; the
 * arguments are those of ts_score_select_workspace_bytes).  Record i = b*Hq + h is 8 int64:
 *   [0] flag (0: order statistic taken, 1: no token taken, 2: every candidate taken)
 *   [1] the answer's order key (the fp32 bits of theta_h mapped to an unsigned order:
 *       negative values bitwise inverted, others with the sign bit set; -0 counts as +0)
 *   [2] the number of candidate keys above it      [3] per-head mode: tokens still to take
 *   [4], [5] the sampled bracket [lo, hi] of order keys (lo > hi: no bracket, the row was ranked
 *       whole because it holds at most 16384 candidates)
 *   [6], [7] the candidate range [begin, end) of token positions.
 * The bracket held, and the whole-row fallback was not taken, when lo <= [1] <= hi.  The records
 * are only read from the workspace: the caller owns it and nothing else there is documented. */
int64_t ts_score_select_state_offset(const int64_t* offsets_host, int32_t B, int32_t Hq,
                                     const ts_select_params* p);

/* Capacity of an expanded list (ts_expand_selection): min(n, (2 radius + 1) k_prev + sink +
 * local); -1 if an argument is out of range (k_prev in [0, n], n, sink and local in [0, 2^31],
 * radius in [0, 2^20]). */
int64_t ts_expand_capacity(int64_t k_prev, int64_t n, int64_t sink, int64_t local, int64_t radius);

/* Workspace for ts_expand_selection (0 if an argument is invalid). */
size_t ts_expand_workspace_bytes(const int64_t* counts_prev_host, int32_t B, int32_t lists);

/* Selection reuse with neighbour fetch ([TB] "Inferenzstrategie", Optimierungen: the selector
 * runs every N decode steps and the steps in between reuse its selection, widened by the
 * spatial neighbours of the selected tokens; sink and local window are the always-kept buffers).
 * For every list l < lists of sequence b (lists = 1 for vote-mode lists, Hq for per-head lists),
 * with the current lengths n_b = offsets[b+1] - offsets[b]:
 *   out = { t + d : t in prev, |d| <= radius, 0 <= t + d < n_b } U [0, min(sink, n_b))
 *         U [max(0, n_b - local), n_b),  ascending,
 * followed by -1 (empty slots, skipped by ts_sparse_decode) up to the list's capacity
 * cap_b = ts_expand_capacity(counts_prev[b], n_b, sink, local, radius).
 *   idx_prev     device int32 lists in the ts_select layout for `lists` lists per sequence with the
 *                lengths counts_prev (sorted ascending, unique; negative entries are ignored)
 *   counts_prev  device (counts_prev_dev) and host (counts_prev_host) int64 [B], the same values,
 *                each at most n_b (an earlier step's lengths)
 *   idx_out      device int32 [lists * sum_b cap_b], list l of b at lists*cpre_b + l*cap_b + j
 *                (cpre_b = sum of the earlier capacities)
 *   caps_out     device int64 [B] (receives cap_b: the list lengths to hand to ts_sparse_decode)
 *   valid_out    device int64 [B][lists] (receives the number of entries before the empty slots)
 *   ws           device workspace of at least ts_expand_workspace_bytes(counts_prev_host, B, lists)
 *                bytes.
 * Pass caps_out and the host capacities as the counts of ts_sparse_decode.                */
int ts_expand_selection(const int32_t* idx_prev, const int64_t* counts_prev_dev, const int64_t* counts_prev_host,
                        const int64_t* offsets_dev, const int64_t* offsets_host, int32_t B, int32_t lists,
                        int64_t sink, int64_t local, int64_t radius, int32_t* idx_out, int64_t* caps_out,
                        int64_t* valid_out, void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace for ts_sparse_decode (mode QASI_MODE_VOTE or QASI_MODE_PER_HEAD, counts_host = the
 * per-sequence list lengths), for ts_union_decode (mode QASI_MODE_UNION, counts_host = the
 * per-head list lengths) and for ts_dense_decode (counts_host = NULL).  0 if an argument is
 * invalid. */
size_t ts_decode_workspace_bytes(const int64_t* offsets_host, const int64_t* counts_host,
                                 int32_t B, int32_t Hq, int32_t Hkv, int32_t mode);

/* Sparse decode attention over the selected tokens ([TS] eq. Attention(Q, K_S, V_S) =
 * softmax(Q K_S^T / sqrt(d)) V_S; the lists already hold the sink and local tokens, so the
 * page's "output merge" of sparse and local attention is one softmax over their union):
 *   out[b][h][:] = sum_{t in S} softmax_t(q[b][h] . K[t][h/G] / sqrt(128)) V[t][h/G]
 * computed as a gathered split-K flash decode (fp32 accumulation) with a log-sum-exp
 * merge of the partial results.
 *   q           device bf16 [B][Hq][128]
 *   K, V        device bf16 [Ntot][Hkv][128]
 *   idx         device int32 lists in the ts_select layout for `mode`; positions must be
 *               in [0, n_b) or negative: a negative entry is an empty slot and is skipped
 *               (positions >= n_b are a caller error; the kernel clamps them into range so
 *               that a bad list cannot read outside the cache)
 *   counts_dev  device int64 [B] and counts_host host int64 [B]: the same list lengths
 *               (0 < count_b <= n_b; e.g. count_out of ts_select and ts_budget_tokens)
 *   out         device fp32 [B][Hq][128].                                             */
int ts_sparse_decode(const uint16_t* q, const uint16_t* K, const uint16_t* V,
                     const int64_t* offsets_dev, const int64_t* offsets_host, const int32_t* idx,
                     const int64_t* counts_dev, const int64_t* counts_host, int32_t mode,
                     int32_t B, int32_t Hq, int32_t Hkv, float* out, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/* For measurement: ts_sparse_decode, then a wait for the call's own work on `stream`, and
 * *gather_us receives the gather kernel's duration in microseconds, taken from its dispatch
 * start and end timestamps (the figure a kernel trace reports for it, without the merge kernel
 * and the launch gaps).  Arguments, validation and results otherwise as for ts_sparse_decode. */
int ts_sparse_decode_timed(const uint16_t* q, const uint16_t* K, const uint16_t* V,
                           const int64_t* offsets_dev, const int64_t* offsets_host, const int32_t* idx,
                           const int64_t* counts_dev, const int64_t* counts_host, int32_t mode,
                           int32_t B, int32_t Hq, int32_t Hkv, float* out, void* ws, size_t ws_bytes,
                           hipStream_t stream, float* gather_us);

/* For callers that cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid device allocation): ts_sparse_decode without a workspace.  The split-K
 * partials live in a static device array of the library (64 MiB on each device it runs on,
 * held until the process ends); arguments, layouts and results are those of ts_sparse_decode.
 * Calls whose ts_decode_workspace_bytes(offsets_host, counts_host, B, Hq, Hkv, mode) exceeds
 * 64 MiB return QASI_ERR_WORKSPACE before anything is enqueued.  Every call on one device shares
 * that array: calls that overlap on one device (other streams or host threads) race, so the
 * caller must order them.  Nothing is allocated or freed by this call.                   */
int ts_sparse_decode_noalloc(const uint16_t* q, const uint16_t* K, const uint16_t* V,
                             const int64_t* offsets_dev, const int64_t* offsets_host, const int32_t* idx,
                             const int64_t* counts_dev, const int64_t* counts_host, int32_t mode, int32_t B,
                             int32_t Hq, int32_t Hkv, float* out, hipStream_t stream);

/* Workspace for ts_union_lists (0 if an argument is invalid). */
size_t ts_union_workspace_bytes(const int64_t* offsets_host, int32_t B, int32_t Hkv);

/* Per-KV-group union of per-head lists with a G-bit head mask ([TS] "主要な貢献": in per-head
 * mode every query head selects its own tokens; the G = Hq/Hkv heads of a KV group read the same
 * K/V rows, so their decode can gather the rows of the group's union once).  For sequence b and
 * KV head g, with K_b = counts[b] and the heads h = g G + hh, hh < G:
 *   U = the set union of the G lists' entries in [0, n_b) (negative entries are empty slots),
 *   uidx[Hq kpre_b + g G K_b + j] = the j-th smallest token of U (j < |U|), then -1 up to G K_b,
 *   umask[same]   = the byte with bit hh set when head g G + hh's list holds that token (0 past U),
 *   ucount[b Hkv + g] = |U|,
 * kpre_b = sum of the earlier counts (the layout of ts_select's per-head lists).
 *   idx        device int32 per-head lists in ts_select's per-head layout, each list ascending
 *              with its negative entries last (ts_select and ts_expand_selection produce such
 *              lists; out-of-order lists give unspecified, in-bounds results)
 *   counts     device (counts_dev) and host (counts_host) int64 [B], the same per-head lengths,
 *              0 < count_b <= n_b
 *   uidx       device int32 [Hq sum_b K_b];  umask device uint8, same shape;
 *   ucount     device int64 [B][Hkv]
 *   ws         device workspace of at least ts_union_workspace_bytes(offsets_host, B, Hkv) bytes.
 * Hq/Hkv in {1, 2, 4, 8} (at most 8 mask bits).                                             */
int ts_union_lists(const int32_t* idx, const int64_t* counts_dev, const int64_t* counts_host,
                   const int64_t* offsets_dev, const int64_t* offsets_host, int32_t B, int32_t Hq,
                   int32_t Hkv, int32_t* uidx, uint8_t* umask, int64_t* ucount, void* ws,
                   size_t ws_bytes, hipStream_t stream);

/* Decode attention of per-head selections read through their per-KV-group union (ts_union_lists'
 * output): the result of ts_sparse_decode in per-head mode on the lists the union was built from
 * (the same sets per head, summed in another order), with every K/V row of a group's union
 * gathered once for the group's G heads; a head's score of a token outside its own list is
 * -inf.
 *   q, K, V, out  as for ts_sparse_decode
 *   uidx, umask   device, ts_union_lists' layout; ucount device int64 [B][Hkv], each in
 *                 [0, G count_b] (a larger value is taken as G count_b)
 *   counts        device and host int64 [B]: the per-head list lengths the union was built from
 *   ws            device workspace of at least ts_decode_workspace_bytes(offsets_host,
 *                 counts_host, B, Hq, Hkv, QASI_MODE_UNION) bytes.
 * A head whose list holds no token of [0, n_b) gets NaN (0/0).                           */
int ts_union_decode(const uint16_t* q, const uint16_t* K, const uint16_t* V,
                    const int64_t* offsets_dev, const int64_t* offsets_host, const int32_t* uidx,
                    const uint8_t* umask, const int64_t* ucount, const int64_t* counts_dev,
                    const int64_t* counts_host, int32_t B, int32_t Hq, int32_t Hkv, float* out,
                    void* ws, size_t ws_bytes, hipStream_t stream);

/* Dense decode attention over all n_b tokens of each sequence (the comparison baseline,
 * [TS] eq. S_i = q . k_i / sqrt(d) for every cached token).  Same layouts as above.   */
int ts_dense_decode(const uint16_t* q, const uint16_t* K, const uint16_t* V,
                    const int64_t* offsets_dev, const int64_t* offsets_host, int32_t B,
                    int32_t Hq, int32_t Hkv, float* out, void* ws, size_t ws_bytes,
                    hipStream_t stream);

/* Decode over a tiered KV cache ([TB] "Inferenzstrategie": the sink, a circular buffer of the
 * newest N tokens and the rest of the cache, from which the important tokens are read; [TB]
 * "Hauptbeiträge" 4 and "Latenz": that rest kept in host memory, with the selection on the GPU and
 * only the selected rows read across the host link).  The result of ts_sparse_decode
 * (mode QASI_MODE_VOTE or QASI_MODE_PER_HEAD, same lists and counts) or ts_dense_decode
 * (QASI_MODE_DENSE; idx and counts are not read and may be NULL) on the logical cache in which
 * position t of sequence b is
 *   K_ring[b][t mod N] when t >= n_b - N, else K_main[offsets[b] + t]   (V alike),
 * up to the grouping of the split-K sums.
 *   K_main, V_main  bf16 [Ntot][Hkv][128], the positions older than the ring (rows of the newest
 *                   N positions are never read): device memory, or pinned host memory through the
 *                   address ts_host_device_pointer gives (the offloaded tier)
 *   K_ring, V_ring  device bf16 [B][N][Hkv][128]
 *   ring_len        N, a power of two in [1, 2^20]; a sequence of at most N tokens is read from its
 *                   ring alone
 *   ws              workspace of at least ts_decode_workspace_bytes(offsets_host, counts_host (NULL
 *                   for dense), B, Hq, Hkv, mode (QASI_MODE_VOTE for dense)) bytes.
 * With a ring of N slots, the index rows of the ring's tokens can be appended N at a time ([TB]
 * "Optimierungen", Batching): when position n_b is a multiple of N the ring holds positions
 * [n_b - N, n_b) in slot order, so ts_index_append(K_ring + b*N*Hkv*128, P, k_index,
 * offsets[b] + n_b - N, N, Hkv) appends all of them.                                        */
int ts_tiered_decode(const uint16_t* q, const uint16_t* K_main, const uint16_t* V_main,
                     const uint16_t* K_ring, const uint16_t* V_ring, int64_t ring_len,
                     const int64_t* offsets_dev, const int64_t* offsets_host, const int32_t* idx,
                     const int64_t* counts_dev, const int64_t* counts_host, int32_t mode, int32_t B,
                     int32_t Hq, int32_t Hkv, float* out, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/* The address kernels use for pinned host memory of the caller (hipHostMalloc, or a pinned
 * tensor): hipHostGetDevicePointer.  QASI_ERR_HIP when `host` is not pinned host memory.  The
 * caller keeps the memory alive while work that reads it is in flight.                      */
int ts_host_device_pointer(const void* host, void** dev);

/* Workspace for snapkv_compress. */
size_t snapkv_workspace_bytes(int64_t n, int32_t w, int32_t Hq, int32_t Hkv, int64_t c);

/* SnapKV prefill-end compression of one sequence ([SK] "Attention Score計算とPooling",
 * "Top-k SelectionとCluster-based Retention" and the listing of "アルゴリズム"):
 *   for each KV head g, rows r = (query head h of group g, window position t):
 *     A_r = softmax_j(q_obs[t][h] . K[j][g] / sqrt(128)) over all n keys (no mask),
 *     imp[g][j] = mean over the G*w rows of A_r[j]   (the page's inter-head average),
 *     pooled[g][j] = (imp[g][j-1] + imp[g][j] + imp[g][j+1]) / 3 (zero padding, kernel 3),
 *     idx_out[g][:] = the ce = min(c, n) positions of largest pooled value, ties to the
 *                     lower position, ascending;
 *     K_out[s][g][:] = K[idx_out[g][s]][g][:], V_out likewise (bit copies).
 * QK^T runs on bf16 MFMA with fp32 accumulation; softmax statistics are fp32.
 *   q_obs          device bf16 [w][Hq][128] (the last w prompt queries)
 *   K, V           device bf16 [n][Hkv][128]
 *   n              1 .. 2^24 tokens; G*w (G = Hq/Hkv) a multiple of 16 and at most 256 (the
 *                  MFMA row tiles of a KV head's window rows); otherwise QASI_ERR_UNSUPPORTED
 *   pool_kernel    must be 3 (odd kernels keep the length; only 3 is built)
 *   idx_out        device int32 [Hkv][ce]
 *   K_out, V_out   device bf16 [ce][Hkv][128]
 *   importance_out nullable device fp32 [Hkv][n] (imp)
 *   pooled_out     nullable device fp32 [Hkv][n] (pooled)                             */
int snapkv_compress(const uint16_t* q_obs, const uint16_t* K, const uint16_t* V, int64_t n,
                    int32_t w, int32_t Hq, int32_t Hkv, int64_t c, int32_t pool_kernel,
                    int32_t* idx_out, uint16_t* K_out, uint16_t* V_out, float* importance_out,
                    float* pooled_out, void* ws, size_t ws_bytes, hipStream_t stream);

/* SnapKV cluster-based retention ([SK] "Top-k SelectionとCluster-based Retention", eq.
 * S_final = U_{j in S} {j - k_cluster, ..., j + k_cluster}): every KV head's top-c list, as
 * snapkv_compress writes it, widened by the k_cluster neighbours of its positions (inside
 * [0, n)), ascending, padded with -1 to cap = ts_expand_capacity(ce, n, 0, 0, k_cluster) =
 * min(n, (2 k_cluster + 1) ce), and the rows of the widened lists gathered:
 *   K_out[s][g][:] = K[idx_out[g][s]][g][:] (bit copies), zero rows for the -1 slots.
 *   idx        device int32 [Hkv][ce] (sorted ascending, unique)
 *   K, V       device bf16 [n][Hkv][128]
 *   idx_out    device int32 [Hkv][cap]
 *   K_out, V_out device bf16 [cap][Hkv][128]
 *   valid_out  device int64 [Hkv] (receives each head's number of entries before the padding)
 *   ws         device workspace of at least snapkv_clusters_workspace_bytes(ce, Hkv) bytes.
 * k_cluster = 0 copies the lists unchanged.                                              */
size_t snapkv_clusters_workspace_bytes(int64_t ce, int32_t Hkv);
int snapkv_retain_clusters(const int32_t* idx, int64_t n, int32_t Hkv, int64_t ce, int64_t k_cluster,
                           const uint16_t* K, const uint16_t* V, int32_t* idx_out, uint16_t* K_out,
                           uint16_t* V_out, int64_t* valid_out, void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QASI_H */
