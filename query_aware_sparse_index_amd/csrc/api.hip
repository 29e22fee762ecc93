// C-ABI layer: synchronous host-side validation, workspace sizing and launch orchestration.
// Every check runs before the first HIP call of an entry point, so a validation failure
// enqueues nothing.  No entry point allocates or frees memory.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/qasi.h"
#include "qasi_internal.h"

namespace qasi {
hipError_t init_score_kernels();
hipError_t init_snap_kernels();
hipError_t init_kernels() {
    hipError_t e = init_score_kernels();
    if (e != hipSuccess) return e;
    return init_snap_kernels();
}
}  // namespace qasi

namespace {

thread_local std::string g_last_error = "no error";

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return QASI_OK;
    return fail(QASI_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int init_once() {
    static std::once_flag flag;
    static hipError_t status = hipSuccess;
    std::call_once(flag, [] { status = qasi::init_kernels(); });
    return hip_status(status, "kernel initialisation");
}

bool hkv_ok(int32_t Hkv) { return Hkv == 1 || Hkv == 2 || Hkv == 4 || Hkv == 8; }

int check_heads(int32_t Hq, int32_t Hkv) {
    if (Hq <= 0 || Hkv <= 0) return fail(QASI_ERR_INVALID, "Hq=%d and Hkv=%d must be positive", Hq, Hkv);
    if (!hkv_ok(Hkv)) return fail(QASI_ERR_UNSUPPORTED, "Hkv=%d not in {1,2,4,8}", Hkv);
    if (Hq % Hkv != 0) return fail(QASI_ERR_UNSUPPORTED, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
    int G = Hq / Hkv;
    if (G != 1 && G != 2 && G != 4 && G != 8) return fail(QASI_ERR_UNSUPPORTED, "G=Hq/Hkv=%d not in {1,2,4,8}", G);
    if (Hq > 64) return fail(QASI_ERR_UNSUPPORTED, "Hq=%d exceeds 64", Hq);
    return QASI_OK;
}

// offsets_host: B+1 entries, starts at 0, non-decreasing, each length below 2^31.
int check_offsets(const int64_t* offsets_dev, const int64_t* offsets_host, int32_t B, bool nonempty) {
    if (B <= 0) return fail(QASI_ERR_INVALID, "B=%d must be positive", B);
    if (!offsets_dev || !offsets_host) return fail(QASI_ERR_INVALID, "offsets pointers must be non-null");
    if ((reinterpret_cast<uintptr_t>(offsets_dev) & 7u) != 0) return fail(QASI_ERR_INVALID, "offsets_dev must be 8-byte aligned");
    if (offsets_host[0] != 0) return fail(QASI_ERR_INVALID, "offsets[0]=%lld must be 0", (long long)offsets_host[0]);
    for (int b = 0; b < B; ++b) {
        int64_t n = offsets_host[b + 1] - offsets_host[b];
        if (n < 0) return fail(QASI_ERR_INVALID, "offsets not monotone at %d", b);
        if (nonempty && n == 0) return fail(QASI_ERR_INVALID, "sequence %d is empty", b);
        if (n >= ((int64_t)1 << 31)) return fail(QASI_ERR_UNSUPPORTED, "sequence %d longer than 2^31-1", b);
    }
    return QASI_OK;
}

int to_cfg(const ts_select_params* p, qasi::SelectConfig* c) {
    if (!p) return fail(QASI_ERR_INVALID, "params must be non-null");
    if (p->mode != QASI_MODE_VOTE && p->mode != QASI_MODE_PER_HEAD) return fail(QASI_ERR_INVALID, "mode=%d", p->mode);
    if (p->budget_den <= 0 || p->budget_num < 0 || p->budget_num > ((int64_t)1 << 31) || p->budget_den > ((int64_t)1 << 31))
        return fail(QASI_ERR_INVALID, "budget %lld/%lld invalid", (long long)p->budget_num, (long long)p->budget_den);
    if (p->sink < 0 || p->local < 0 || p->sink > ((int64_t)1 << 31) || p->local > ((int64_t)1 << 31))
        return fail(QASI_ERR_INVALID, "sink/local must be in [0, 2^31]");
    if (p->mode == QASI_MODE_VOTE) {
        if (p->theta_den <= 0 || p->theta_num < 0 || p->theta_num > p->theta_den || p->theta_den > ((int64_t)1 << 31))
            return fail(QASI_ERR_INVALID, "theta %lld/%lld must be in [0, 1] with a denominator of at most 2^31",
                        (long long)p->theta_num, (long long)p->theta_den);
        if (p->v_min < 0) return fail(QASI_ERR_INVALID, "v_min must be >= 0");
    }
    c->mode = p->mode;
    c->bnum = p->budget_num;
    c->bden = p->budget_den;
    c->sink = p->sink;
    c->local = p->local;
    c->vmin = p->v_min < 255 ? p->v_min : 255;
    c->tnum = p->theta_num;
    c->tden = p->theta_den > 0 ? p->theta_den : 1;
    return QASI_OK;
}

}  // namespace

extern "C" {

const char* ts_last_error(void) { return g_last_error.c_str(); }

int64_t ts_score_stride(const int64_t* offsets_host, int32_t B) {
    if (!offsets_host || B <= 0) return -1;
    return ((offsets_host[B] + 63) / 64) * 64;
}

int64_t ts_budget_tokens(int64_t n, const ts_select_params* p) {
    qasi::SelectConfig c;
    // n * budget_num stays below 2^62
    if (n < 0 || n > ((int64_t)1 << 31) || to_cfg(p, &c) != QASI_OK) return -1;
    return qasi::budget_tokens(n, c);
}

int ts_index_append(const uint16_t* k_new, const float* P, uint16_t* k_index, int64_t pos, int64_t T, int32_t Hkv,
                    hipStream_t stream) {
    if (!aligned16(k_new) || !aligned16(P) || !aligned16(k_index))
        return fail(QASI_ERR_INVALID, "k_new, P and k_index must be non-null and 16-byte aligned");
    if (pos < 0 || T < 0) return fail(QASI_ERR_INVALID, "pos=%lld and T=%lld must be >= 0", (long long)pos, (long long)T);
    if (!hkv_ok(Hkv)) return fail(QASI_ERR_UNSUPPORTED, "Hkv=%d not in {1,2,4,8}", Hkv);
    if (T == 0) return QASI_OK;
    if (int r = init_once()) return r;
    return hip_status(qasi::launch_index_append(k_new, P, k_index, pos, T, Hkv, stream), "ts_index_append launch");
}

size_t ts_score_workspace_bytes(int32_t B, int32_t Hq) {
    if (B <= 0 || Hq <= 0 || Hq > 64) return 0;
    return qasi::score_workspace(B, Hq);
}

int ts_score(const uint16_t* q, const float* P, const uint16_t* k_index, const int64_t* offsets_dev,
             const int64_t* offsets_host, int32_t B, int32_t Hq, int32_t Hkv, float* scores, void* ws,
             size_t ws_bytes, hipStream_t stream) {
    if (!aligned16(q) || !aligned16(P) || !aligned16(k_index) || !aligned16(scores) || !aligned16(ws))
        return fail(QASI_ERR_INVALID, "q, P, k_index, scores and ws must be non-null and 16-byte aligned");
    if (int r = check_heads(Hq, Hkv)) return r;
    if (int r = check_offsets(offsets_dev, offsets_host, B, false)) return r;
    size_t need = qasi::score_workspace(B, Hq);
    if (ws_bytes < need) return fail(QASI_ERR_WORKSPACE, "ts_score needs %zu workspace bytes, got %zu", need, ws_bytes);
    if (int r = init_once()) return r;
    return hip_status(qasi::launch_score(q, P, k_index, offsets_dev, offsets_host, B, Hq, Hkv, scores, ws, ws_bytes,
                                         stream),
                      "ts_score launch");
}

size_t ts_select_workspace_bytes(const int64_t* offsets_host, int32_t B, int32_t Hq, const ts_select_params* p) {
    qasi::SelectConfig c;
    if (!offsets_host || B <= 0 || Hq <= 0 || to_cfg(p, &c) != QASI_OK) return 0;
    return qasi::select_workspace(offsets_host, B, Hq, c);
}

int ts_select(const float* scores, const int64_t* offsets_dev, const int64_t* offsets_host, int32_t B, int32_t Hq,
              int32_t Hkv, const ts_select_params* p, int32_t* idx_out, int64_t* count_out, float* theta_out,
              uint8_t* votes_out, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!aligned16(scores) || !aligned16(idx_out) || !aligned16(ws))
        return fail(QASI_ERR_INVALID, "scores, idx_out and ws must be non-null and 16-byte aligned");
    if (!count_out || (reinterpret_cast<uintptr_t>(count_out) & 7u))
        return fail(QASI_ERR_INVALID, "count_out must be non-null and 8-byte aligned");
    if (theta_out && (reinterpret_cast<uintptr_t>(theta_out) & 3u)) return fail(QASI_ERR_INVALID, "theta_out misaligned");
    if (int r = check_heads(Hq, Hkv)) return r;
    if (int r = check_offsets(offsets_dev, offsets_host, B, true)) return r;
    for (int b = 0; b < B; ++b)
        if (offsets_host[b + 1] - offsets_host[b] > ((int64_t)1 << 24))
            return fail(QASI_ERR_UNSUPPORTED, "sequence %d longer than 2^24 tokens (selection limit)", b);
    qasi::SelectConfig c;
    if (int r = to_cfg(p, &c)) return r;
    size_t need = qasi::select_workspace(offsets_host, B, Hq, c);
    if (ws_bytes < need) return fail(QASI_ERR_WORKSPACE, "ts_select needs %zu workspace bytes, got %zu", need, ws_bytes);
    if (int r = init_once()) return r;
    return hip_status(qasi::launch_select(scores, ts_score_stride(offsets_host, B), offsets_dev, offsets_host, B, Hq, c,
                                          idx_out, count_out, theta_out, votes_out, ws, ws_bytes, stream),
                      "ts_select launch");
}

size_t ts_score_select_workspace_bytes(const int64_t* offsets_host, int32_t B, int32_t Hq,
                                       const ts_select_params* p) {
    qasi::SelectConfig c;
    if (!offsets_host || B <= 0 || Hq <= 0 || to_cfg(p, &c) != QASI_OK) return 0;
    return qasi::score_select_workspace(offsets_host, B, Hq, c);
}

int64_t ts_score_select_state_offset(const int64_t* offsets_host, int32_t B, int32_t Hq,
                                     const ts_select_params* p) {
    qasi::SelectConfig c;
    if (!offsets_host || B <= 0 || Hq <= 0 || to_cfg(p, &c) != QASI_OK) return -1;
    return (int64_t)qasi::score_select_state_offset(offsets_host, B, Hq, c);
}

int ts_score_select(const uint16_t* q, const float* P, uint16_t* k_index, const uint16_t* K_last,
                    const int64_t* offsets_dev, const int64_t* offsets_host, int32_t B, int32_t Hq, int32_t Hkv,
                    const ts_select_params* p, float* scores, int32_t* idx_out, int64_t* count_out,
                    float* theta_out, uint8_t* votes_out, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!aligned16(q) || !aligned16(P) || !aligned16(k_index) || !aligned16(scores) || !aligned16(idx_out) ||
        !aligned16(ws))
        return fail(QASI_ERR_INVALID, "q, P, k_index, scores, idx_out and ws must be non-null and 16-byte aligned");
    if (K_last && !aligned16(K_last)) return fail(QASI_ERR_INVALID, "K_last must be 16-byte aligned");
    if (!count_out || (reinterpret_cast<uintptr_t>(count_out) & 7u))
        return fail(QASI_ERR_INVALID, "count_out must be non-null and 8-byte aligned");
    if (theta_out && (reinterpret_cast<uintptr_t>(theta_out) & 3u)) return fail(QASI_ERR_INVALID, "theta_out misaligned");
    if (int r = check_heads(Hq, Hkv)) return r;
    if (int r = check_offsets(offsets_dev, offsets_host, B, true)) return r;
    for (int b = 0; b < B; ++b)
        if (offsets_host[b + 1] - offsets_host[b] > ((int64_t)1 << 24))
            return fail(QASI_ERR_UNSUPPORTED, "sequence %d longer than 2^24 tokens (selection limit)", b);
    qasi::SelectConfig c;
    if (int r = to_cfg(p, &c)) return r;
    size_t need = qasi::score_select_workspace(offsets_host, B, Hq, c);
    if (ws_bytes < need)
        return fail(QASI_ERR_WORKSPACE, "ts_score_select needs %zu workspace bytes, got %zu", need, ws_bytes);
    if (int r = init_once()) return r;
    return hip_status(qasi::launch_score_select(q, P, k_index, K_last, offsets_dev, offsets_host, B, Hq, Hkv, c, scores,
                                                idx_out, count_out, theta_out, votes_out, ws, ws_bytes, stream),
                      "ts_score_select launch");
}

int64_t ts_expand_capacity(int64_t k_prev, int64_t n, int64_t sink, int64_t local, int64_t radius) {
    // (2 radius + 1) k_prev + sink + local stays below 2^62
    const int64_t lim = (int64_t)1 << 31;
    if (k_prev < 0 || n < 0 || n > lim || sink < 0 || sink > lim || local < 0 || local > lim || radius < 0 ||
        radius > (1 << 20) || k_prev > n)
        return -1;
    return qasi::expand_capacity(k_prev, n, sink, local, radius);
}

size_t ts_expand_workspace_bytes(const int64_t* counts_prev_host, int32_t B, int32_t lists) {
    if (!counts_prev_host || B <= 0 || lists < 1 || lists > 64) return 0;
    for (int b = 0; b < B; ++b)
        if (counts_prev_host[b] < 0) return 0;
    return (size_t)qasi::expand_blocks(counts_prev_host, B, lists) * sizeof(uint32_t);
}

int ts_expand_selection(const int32_t* idx_prev, const int64_t* counts_prev_dev, const int64_t* counts_prev_host,
                        const int64_t* offsets_dev, const int64_t* offsets_host, int32_t B, int32_t lists,
                        int64_t sink, int64_t local, int64_t radius, int32_t* idx_out, int64_t* caps_out,
                        int64_t* valid_out, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!idx_prev || (reinterpret_cast<uintptr_t>(idx_prev) & 3u) || !idx_out || (reinterpret_cast<uintptr_t>(idx_out) & 3u))
        return fail(QASI_ERR_INVALID, "idx_prev and idx_out must be non-null and 4-byte aligned");
    if (!counts_prev_dev || !counts_prev_host || (reinterpret_cast<uintptr_t>(counts_prev_dev) & 7u))
        return fail(QASI_ERR_INVALID, "counts_prev_dev / counts_prev_host must be non-null (device copy 8-byte aligned)");
    if (!caps_out || !valid_out || (reinterpret_cast<uintptr_t>(caps_out) & 7u) || (reinterpret_cast<uintptr_t>(valid_out) & 7u))
        return fail(QASI_ERR_INVALID, "caps_out and valid_out must be non-null and 8-byte aligned");
    if (lists < 1 || lists > 64) return fail(QASI_ERR_INVALID, "lists=%d outside [1, 64]", lists);
    if (sink < 0 || local < 0 || sink > ((int64_t)1 << 31) || local > ((int64_t)1 << 31))
        return fail(QASI_ERR_INVALID, "sink/local must be in [0, 2^31]");
    if (radius < 0 || radius > (1 << 20)) return fail(QASI_ERR_INVALID, "radius=%lld outside [0, 2^20]", (long long)radius);
    if (int r = check_offsets(offsets_dev, offsets_host, B, true)) return r;
    for (int b = 0; b < B; ++b) {
        const int64_t n = offsets_host[b + 1] - offsets_host[b];
        if (counts_prev_host[b] < 0 || counts_prev_host[b] > n)
            return fail(QASI_ERR_INVALID, "counts_prev[%d]=%lld outside [0, n_b=%lld]", b, (long long)counts_prev_host[b],
                        (long long)n);
    }
    if (!ws || (reinterpret_cast<uintptr_t>(ws) & 3u)) return fail(QASI_ERR_INVALID, "ws must be non-null and aligned");
    const size_t need = (size_t)qasi::expand_blocks(counts_prev_host, B, lists) * sizeof(uint32_t);
    if (ws_bytes < need) return fail(QASI_ERR_WORKSPACE, "ts_expand_selection needs %zu workspace bytes, got %zu", need, ws_bytes);
    if (int r = init_once()) return r;
    return hip_status(qasi::launch_expand(idx_prev, counts_prev_dev, counts_prev_host, offsets_dev, offsets_host, B,
                                          lists, sink, local, radius, idx_out, caps_out, valid_out,
                                          static_cast<uint32_t*>(ws), stream),
                      "ts_expand_selection launch");
}

size_t ts_decode_workspace_bytes(const int64_t* offsets_host, const int64_t* counts_host, int32_t B, int32_t Hq,
                                 int32_t Hkv, int32_t mode) {
    if (!offsets_host || B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv) return 0;
    if (mode != QASI_MODE_VOTE && mode != QASI_MODE_PER_HEAD && mode != QASI_MODE_UNION) return 0;
    if (mode == QASI_MODE_UNION && !counts_host) return 0;
    return qasi::decode_workspace(offsets_host, counts_host, B, Hq, Hkv, mode == QASI_MODE_UNION ? 3 : mode);
}

// Checks shared by ts_sparse_decode and its timed variant (everything before the first HIP call).
static int sparse_decode_checks(const uint16_t* q, const uint16_t* K, const uint16_t* V, const int64_t* offsets_dev,
                                const int64_t* offsets_host, const int32_t* idx, const int64_t* counts_dev,
                                const int64_t* counts_host, int32_t mode, int32_t B, int32_t Hq, int32_t Hkv,
                                const float* out, const void* ws, size_t ws_bytes, const char* name) {
    if (!aligned16(q) || !aligned16(K) || !aligned16(V) || !aligned16(out) || !aligned16(ws))
        return fail(QASI_ERR_INVALID, "q, K, V, out and ws must be non-null and 16-byte aligned");
    if (!idx || (reinterpret_cast<uintptr_t>(idx) & 3u)) return fail(QASI_ERR_INVALID, "idx must be non-null and aligned");
    if (!counts_dev || !counts_host || (reinterpret_cast<uintptr_t>(counts_dev) & 7u))
        return fail(QASI_ERR_INVALID, "counts_dev / counts_host must be non-null (counts_dev 8-byte aligned)");
    if (mode != QASI_MODE_VOTE && mode != QASI_MODE_PER_HEAD) return fail(QASI_ERR_INVALID, "mode=%d", mode);
    if (int r = check_heads(Hq, Hkv)) return r;
    if (int r = check_offsets(offsets_dev, offsets_host, B, true)) return r;
    for (int b = 0; b < B; ++b) {
        int64_t n = offsets_host[b + 1] - offsets_host[b];
        if (counts_host[b] < 1 || counts_host[b] > n)
            return fail(QASI_ERR_INVALID, "counts[%d]=%lld outside [1, n_b=%lld]", b, (long long)counts_host[b], (long long)n);
    }
    size_t need = qasi::decode_workspace(offsets_host, counts_host, B, Hq, Hkv, mode);
    if (ws_bytes < need) return fail(QASI_ERR_WORKSPACE, "%s needs %zu workspace bytes, got %zu", name, need, ws_bytes);
    return QASI_OK;
}

int ts_sparse_decode(const uint16_t* q, const uint16_t* K, const uint16_t* V, const int64_t* offsets_dev,
                     const int64_t* offsets_host, const int32_t* idx, const int64_t* counts_dev,
                     const int64_t* counts_host, int32_t mode, int32_t B, int32_t Hq, int32_t Hkv, float* out, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
    if (int r = sparse_decode_checks(q, K, V, offsets_dev, offsets_host, idx, counts_dev, counts_host, mode, B, Hq, Hkv,
                                     out, ws, ws_bytes, "ts_sparse_decode"))
        return r;
    if (int r = init_once()) return r;
    return hip_status(qasi::launch_sparse_decode(q, K, V, offsets_dev, offsets_host, idx, counts_dev, counts_host, mode,
                                                 B, Hq, Hkv, out, ws, ws_bytes, stream),
                      "ts_sparse_decode launch");
}

int ts_sparse_decode_timed(const uint16_t* q, const uint16_t* K, const uint16_t* V, const int64_t* offsets_dev,
                           const int64_t* offsets_host, const int32_t* idx, const int64_t* counts_dev,
                           const int64_t* counts_host, int32_t mode, int32_t B, int32_t Hq, int32_t Hkv, float* out,
                           void* ws, size_t ws_bytes, hipStream_t stream, float* gather_us) {
    if (!gather_us) return fail(QASI_ERR_INVALID, "gather_us must be non-null");
    if (int r = sparse_decode_checks(q, K, V, offsets_dev, offsets_host, idx, counts_dev, counts_host, mode, B, Hq, Hkv,
                                     out, ws, ws_bytes, "ts_sparse_decode_timed"))
        return r;
    if (int r = init_once()) return r;
    hipEvent_t t0 = nullptr, t1 = nullptr;
    hipError_t e = hipEventCreate(&t0);
    if (e == hipSuccess) e = hipEventCreate(&t1);
    if (e == hipSuccess)
        e = qasi::launch_sparse_decode(q, K, V, offsets_dev, offsets_host, idx, counts_dev, counts_host, mode, B, Hq, Hkv,
                                       out, ws, ws_bytes, stream, t0, t1);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, t0, t1);
    if (t0) (void)hipEventDestroy(t0);
    if (t1) (void)hipEventDestroy(t1);
    if (e == hipSuccess) *gather_us = ms * 1000.f;
    return hip_status(e, "ts_sparse_decode_timed");
}

int ts_sparse_decode_noalloc(const uint16_t* q, const uint16_t* K, const uint16_t* V, const int64_t* offsets_dev,
                             const int64_t* offsets_host, const int32_t* idx, const int64_t* counts_dev,
                             const int64_t* counts_host, int32_t mode, int32_t B, int32_t Hq, int32_t Hkv, float* out,
                             hipStream_t stream) {
    if (!aligned16(q) || !aligned16(K) || !aligned16(V) || !aligned16(out))
        return fail(QASI_ERR_INVALID, "q, K, V and out must be non-null and 16-byte aligned");
    if (!idx || (reinterpret_cast<uintptr_t>(idx) & 3u)) return fail(QASI_ERR_INVALID, "idx must be non-null and aligned");
    if (!counts_dev || !counts_host || (reinterpret_cast<uintptr_t>(counts_dev) & 7u))
        return fail(QASI_ERR_INVALID, "counts_dev / counts_host must be non-null (counts_dev 8-byte aligned)");
    if (mode != QASI_MODE_VOTE && mode != QASI_MODE_PER_HEAD) return fail(QASI_ERR_INVALID, "mode=%d", mode);
    if (int r = check_heads(Hq, Hkv)) return r;
    if (int r = check_offsets(offsets_dev, offsets_host, B, true)) return r;
    for (int b = 0; b < B; ++b) {
        int64_t n = offsets_host[b + 1] - offsets_host[b];
        if (counts_host[b] < 1 || counts_host[b] > n)
            return fail(QASI_ERR_INVALID, "counts[%d]=%lld outside [1, n_b=%lld]", b, (long long)counts_host[b], (long long)n);
    }
    size_t need = qasi::decode_workspace(offsets_host, counts_host, B, Hq, Hkv, mode);
    if (need > qasi::kNoAllocScratchBytes)
        return fail(QASI_ERR_WORKSPACE, "ts_sparse_decode_noalloc needs %zu scratch bytes; the static scratch holds %zu",
                    need, qasi::kNoAllocScratchBytes);
    if (int r = init_once()) return r;
    return hip_status(qasi::launch_sparse_decode_noalloc(q, K, V, offsets_dev, offsets_host, idx, counts_dev,
                                                         counts_host, mode, B, Hq, Hkv, out, stream),
                      "ts_sparse_decode_noalloc launch");
}

// Shared checks of per-sequence list lengths: host and device copies given, 0 < count_b <= n_b.
static int check_counts(const int64_t* counts_dev, const int64_t* counts_host, const int64_t* offsets_host, int32_t B) {
    if (!counts_dev || !counts_host || (reinterpret_cast<uintptr_t>(counts_dev) & 7u))
        return fail(QASI_ERR_INVALID, "counts_dev / counts_host must be non-null (counts_dev 8-byte aligned)");
    for (int b = 0; b < B; ++b) {
        const int64_t n = offsets_host[b + 1] - offsets_host[b];
        if (counts_host[b] < 1 || counts_host[b] > n)
            return fail(QASI_ERR_INVALID, "counts[%d]=%lld outside [1, n_b=%lld]", b, (long long)counts_host[b], (long long)n);
    }
    return QASI_OK;
}

size_t ts_union_workspace_bytes(const int64_t* offsets_host, int32_t B, int32_t Hkv) {
    if (!offsets_host || B <= 0 || Hkv <= 0) return 0;
    return qasi::union_workspace(offsets_host, B, Hkv);
}

int ts_union_lists(const int32_t* idx, const int64_t* counts_dev, const int64_t* counts_host, const int64_t* offsets_dev,
                   const int64_t* offsets_host, int32_t B, int32_t Hq, int32_t Hkv, int32_t* uidx, uint8_t* umask,
                   int64_t* ucount, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!idx || (reinterpret_cast<uintptr_t>(idx) & 3u) || !uidx || (reinterpret_cast<uintptr_t>(uidx) & 3u))
        return fail(QASI_ERR_INVALID, "idx and uidx must be non-null and 4-byte aligned");
    if (!umask || !ucount || (reinterpret_cast<uintptr_t>(ucount) & 7u) || !aligned16(ws))
        return fail(QASI_ERR_INVALID, "umask, ucount (8-byte aligned) and ws (16-byte aligned) must be non-null");
    if (int r = check_heads(Hq, Hkv)) return r;
    if (int r = check_offsets(offsets_dev, offsets_host, B, true)) return r;
    if (int r = check_counts(counts_dev, counts_host, offsets_host, B)) return r;
    const size_t need = qasi::union_workspace(offsets_host, B, Hkv);
    if (ws_bytes < need) return fail(QASI_ERR_WORKSPACE, "ts_union_lists needs %zu workspace bytes, got %zu", need, ws_bytes);
    if (int r = init_once()) return r;
    return hip_status(qasi::launch_union(idx, counts_dev, counts_host, offsets_dev, offsets_host, B, Hq, Hkv, uidx,
                                         umask, ucount, ws, ws_bytes, stream),
                      "ts_union_lists launch");
}

int ts_union_decode(const uint16_t* q, const uint16_t* K, const uint16_t* V, const int64_t* offsets_dev,
                    const int64_t* offsets_host, const int32_t* uidx, const uint8_t* umask, const int64_t* ucount,
                    const int64_t* counts_dev, const int64_t* counts_host, int32_t B, int32_t Hq, int32_t Hkv,
                    float* out, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!aligned16(q) || !aligned16(K) || !aligned16(V) || !aligned16(out) || !aligned16(ws))
        return fail(QASI_ERR_INVALID, "q, K, V, out and ws must be non-null and 16-byte aligned");
    if (!uidx || (reinterpret_cast<uintptr_t>(uidx) & 3u) || !umask || !ucount ||
        (reinterpret_cast<uintptr_t>(ucount) & 7u))
        return fail(QASI_ERR_INVALID, "uidx (4-byte aligned), umask and ucount (8-byte aligned) must be non-null");
    if (int r = check_heads(Hq, Hkv)) return r;
    if (int r = check_offsets(offsets_dev, offsets_host, B, true)) return r;
    if (int r = check_counts(counts_dev, counts_host, offsets_host, B)) return r;
    const size_t need = qasi::decode_workspace(offsets_host, counts_host, B, Hq, Hkv, 3);
    if (ws_bytes < need) return fail(QASI_ERR_WORKSPACE, "ts_union_decode needs %zu workspace bytes, got %zu", need, ws_bytes);
    if (int r = init_once()) return r;
    return hip_status(qasi::launch_union_decode(q, K, V, offsets_dev, offsets_host, uidx, umask, ucount, counts_dev,
                                                counts_host, B, Hq, Hkv, out, ws, ws_bytes, stream),
                      "ts_union_decode launch");
}

int ts_dense_decode(const uint16_t* q, const uint16_t* K, const uint16_t* V, const int64_t* offsets_dev,
                    const int64_t* offsets_host, int32_t B, int32_t Hq, int32_t Hkv, float* out, void* ws,
                    size_t ws_bytes, hipStream_t stream) {
    if (!aligned16(q) || !aligned16(K) || !aligned16(V) || !aligned16(out) || !aligned16(ws))
        return fail(QASI_ERR_INVALID, "q, K, V, out and ws must be non-null and 16-byte aligned");
    if (int r = check_heads(Hq, Hkv)) return r;
    if (int r = check_offsets(offsets_dev, offsets_host, B, true)) return r;
    size_t need = qasi::decode_workspace(offsets_host, nullptr, B, Hq, Hkv, 2);
    if (ws_bytes < need) return fail(QASI_ERR_WORKSPACE, "ts_dense_decode needs %zu workspace bytes, got %zu", need, ws_bytes);
    if (int r = init_once()) return r;
    return hip_status(qasi::launch_dense_decode(q, K, V, offsets_dev, offsets_host, B, Hq, Hkv, out, ws, ws_bytes, stream),
                      "ts_dense_decode launch");
}

int ts_tiered_decode(const uint16_t* q, const uint16_t* K_main, const uint16_t* V_main, const uint16_t* K_ring,
                     const uint16_t* V_ring, int64_t ring_len, const int64_t* offsets_dev, const int64_t* offsets_host,
                     const int32_t* idx, const int64_t* counts_dev, const int64_t* counts_host, int32_t mode, int32_t B,
                     int32_t Hq, int32_t Hkv, float* out, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!aligned16(q) || !aligned16(K_main) || !aligned16(V_main) || !aligned16(K_ring) || !aligned16(V_ring) ||
        !aligned16(out) || !aligned16(ws))
        return fail(QASI_ERR_INVALID, "q, K_main, V_main, K_ring, V_ring, out and ws must be non-null and 16-byte aligned");
    if (ring_len < 1 || ring_len > ((int64_t)1 << 20) || (ring_len & (ring_len - 1)))
        return fail(QASI_ERR_INVALID, "ring_len=%lld is not a power of two in [1, 2^20]", (long long)ring_len);
    if (mode != QASI_MODE_VOTE && mode != QASI_MODE_PER_HEAD && mode != QASI_MODE_DENSE)
        return fail(QASI_ERR_INVALID, "mode=%d (vote, per-head or dense)", mode);
    if (int r = check_heads(Hq, Hkv)) return r;
    if (int r = check_offsets(offsets_dev, offsets_host, B, true)) return r;
    const bool dense = mode == QASI_MODE_DENSE;
    if (!dense) {
        if (!idx || (reinterpret_cast<uintptr_t>(idx) & 3u)) return fail(QASI_ERR_INVALID, "idx must be non-null and aligned");
        if (int r = check_counts(counts_dev, counts_host, offsets_host, B)) return r;
    }
    const size_t need = qasi::decode_workspace(offsets_host, dense ? nullptr : counts_host, B, Hq, Hkv, dense ? 2 : mode);
    if (ws_bytes < need) return fail(QASI_ERR_WORKSPACE, "ts_tiered_decode needs %zu workspace bytes, got %zu", need, ws_bytes);
    if (int r = init_once()) return r;
    const qasi::DecRing ring{K_ring, V_ring, ring_len};
    return hip_status(qasi::launch_tiered_decode(q, K_main, V_main, ring, offsets_dev, offsets_host, dense ? nullptr : idx,
                                                 dense ? nullptr : counts_dev, dense ? nullptr : counts_host,
                                                 dense ? 2 : mode, B, Hq, Hkv, out, ws, ws_bytes, stream),
                      "ts_tiered_decode launch");
}

int ts_host_device_pointer(const void* host, void** dev) {
    if (!host || !dev) return fail(QASI_ERR_INVALID, "host and dev must be non-null");
    *dev = nullptr;
    void* d = nullptr;
    const hipError_t e = hipHostGetDevicePointer(&d, const_cast<void*>(host), 0);
    if (e != hipSuccess) return hip_status(e, "hipHostGetDevicePointer (not pinned host memory?)");
    *dev = d;
    return QASI_OK;
}

size_t snapkv_workspace_bytes(int64_t n, int32_t w, int32_t Hq, int32_t Hkv, int64_t c) {
    if (n <= 0 || w <= 0 || Hq <= 0 || Hkv <= 0 || c <= 0 || Hq % Hkv) return 0;
    return qasi::snapkv_workspace(n, w, Hq, Hkv, c);
}

int snapkv_compress(const uint16_t* q_obs, const uint16_t* K, const uint16_t* V, int64_t n, int32_t w, int32_t Hq,
                    int32_t Hkv, int64_t c, int32_t pool_kernel, int32_t* idx_out, uint16_t* K_out, uint16_t* V_out,
                    float* importance_out, float* pooled_out, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!aligned16(q_obs) || !aligned16(K) || !aligned16(V) || !aligned16(idx_out) || !aligned16(K_out) ||
        !aligned16(V_out) || !aligned16(ws))
        return fail(QASI_ERR_INVALID, "q_obs, K, V, idx_out, K_out, V_out and ws must be non-null and 16-byte aligned");
    if ((importance_out && (reinterpret_cast<uintptr_t>(importance_out) & 3u)) ||
        (pooled_out && (reinterpret_cast<uintptr_t>(pooled_out) & 3u)))
        return fail(QASI_ERR_INVALID, "importance_out / pooled_out misaligned");
    if (n <= 0 || n >= ((int64_t)1 << 31)) return fail(QASI_ERR_INVALID, "n=%lld outside [1, 2^31)", (long long)n);
    if (n > ((int64_t)1 << 24))
        return fail(QASI_ERR_UNSUPPORTED, "n=%lld longer than 2^24 tokens (selection limit)", (long long)n);
    if (w <= 0 || c <= 0) return fail(QASI_ERR_INVALID, "w=%d and c=%lld must be positive", w, (long long)c);
    if (int r = check_heads(Hq, Hkv)) return r;
    if (pool_kernel != 3) return fail(QASI_ERR_UNSUPPORTED, "pool_kernel=%d (only 3 is built)", pool_kernel);
    const int R = (Hq / Hkv) * w;
    if (R > 256 || R % 16 != 0)
        return fail(QASI_ERR_UNSUPPORTED, "(Hq/Hkv)*w=%d must be a multiple of 16 and at most 256", R);
    size_t need = qasi::snapkv_workspace(n, w, Hq, Hkv, c);
    if (ws_bytes < need) return fail(QASI_ERR_WORKSPACE, "snapkv_compress needs %zu workspace bytes, got %zu", need, ws_bytes);
    if (int r = init_once()) return r;
    return hip_status(qasi::launch_snapkv(q_obs, K, V, n, w, Hq, Hkv, c, idx_out, K_out, V_out, importance_out,
                                          pooled_out, ws, ws_bytes, stream),
                      "snapkv_compress launch");
}

size_t snapkv_clusters_workspace_bytes(int64_t ce, int32_t Hkv) {
    if (ce < 0 || Hkv <= 0 || Hkv > 64) return 0;
    const int64_t c[1] = {ce};
    return (size_t)qasi::expand_blocks(c, 1, Hkv) * sizeof(uint32_t);
}

int snapkv_retain_clusters(const int32_t* idx, int64_t n, int32_t Hkv, int64_t ce, int64_t k_cluster, const uint16_t* K,
                           const uint16_t* V, int32_t* idx_out, uint16_t* K_out, uint16_t* V_out, int64_t* valid_out,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!idx || (reinterpret_cast<uintptr_t>(idx) & 3u) || !idx_out || (reinterpret_cast<uintptr_t>(idx_out) & 3u))
        return fail(QASI_ERR_INVALID, "idx and idx_out must be non-null and 4-byte aligned");
    if (!aligned16(K) || !aligned16(V) || !aligned16(K_out) || !aligned16(V_out))
        return fail(QASI_ERR_INVALID, "K, V, K_out and V_out must be non-null and 16-byte aligned");
    if (!valid_out || (reinterpret_cast<uintptr_t>(valid_out) & 7u))
        return fail(QASI_ERR_INVALID, "valid_out must be non-null and 8-byte aligned");
    if (n <= 0 || n > ((int64_t)1 << 24)) return fail(QASI_ERR_INVALID, "n=%lld outside [1, 2^24]", (long long)n);
    if (!hkv_ok(Hkv)) return fail(QASI_ERR_UNSUPPORTED, "Hkv=%d not in {1,2,4,8}", Hkv);
    if (ce < 0 || ce > n) return fail(QASI_ERR_INVALID, "ce=%lld outside [0, n]", (long long)ce);
    if (k_cluster < 0 || k_cluster > (1 << 20))
        return fail(QASI_ERR_INVALID, "k_cluster=%lld outside [0, 2^20]", (long long)k_cluster);
    if (!ws || (reinterpret_cast<uintptr_t>(ws) & 3u)) return fail(QASI_ERR_INVALID, "ws must be non-null and aligned");
    const int64_t c[1] = {ce};
    const size_t need = (size_t)qasi::expand_blocks(c, 1, Hkv) * sizeof(uint32_t);
    if (ws_bytes < need)
        return fail(QASI_ERR_WORKSPACE, "snapkv_retain_clusters needs %zu workspace bytes, got %zu", need, ws_bytes);
    if (int r = init_once()) return r;
    return hip_status(qasi::launch_snapkv_clusters(idx, n, Hkv, ce, k_cluster, K, V, idx_out, K_out, V_out, valid_out,
                                                   static_cast<uint32_t*>(ws), stream),
                      "snapkv_retain_clusters launch");
}

}  // extern "C"
