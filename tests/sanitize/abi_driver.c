/*
 * Sanitizer driver for the C-ABI boundary (test infrastructure): calls the entry points with
 * invalid or unsupported arguments, each of which the library must reject synchronously, before
 * any HIP call (so no GPU is needed), and the host-side queries with valid and edge-case
 * arguments.  Built with AddressSanitizer and UndefinedBehaviorSanitizer on the host code of the
 * library, it checks the validation code for out-of-bounds reads of the host arrays (offsets,
 * per-sequence counts) and for integer overflow.  Exits 0 when every code is as expected.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "qasi.h"

static int failures = 0;
#define EXPECT(call, code)                                                                   \
    do {                                                                                     \
        const long long got_ = (long long)(call);                                            \
        if (got_ != (long long)(code)) {                                                     \
            fprintf(stderr, "line %d: %s returned %lld, expected %lld (%s)\n", __LINE__, #call, \
                    got_, (long long)(code), ts_last_error());                               \
            ++failures;                                                                      \
        }                                                                                    \
    } while (0)

static ts_select_params params(int32_t mode, int64_t bnum, int64_t bden, int64_t sink, int64_t local, int64_t vmin,
                               int64_t tn, int64_t td) {
    ts_select_params p;
    memset(&p, 0, sizeof p);
    p.mode = mode;
    p.budget_num = bnum;
    p.budget_den = bden;
    p.sink = sink;
    p.local = local;
    p.v_min = vmin;
    p.theta_num = tn;
    p.theta_den = td;
    return p;
}

int main(void) {
    /* aligned and misaligned stand-ins: validation rejects the call before any is dereferenced */
    void* F = (void*)(uintptr_t)4096;
    void* M = (void*)(uintptr_t)4097;
    const int64_t o1[2] = {0, 4096}, obad[3] = {0, 10, 5}, oneg[2] = {1, 100}, o1000[2] = {0, 1000};
    const int64_t c100[1] = {100}, c0[1] = {0}, c1001[1] = {1001};
    const ts_select_params ok = params(0, 1, 5, 4, 256, 1, 9, 10);

    /* host-side queries */
    EXPECT(ts_score_stride(NULL, 1), -1);
    EXPECT(ts_score_stride(o1, 1) >= 4096, 1);
    EXPECT(ts_budget_tokens(100, &ok), 100);
    EXPECT(ts_budget_tokens(100000, &ok), 20000);
    EXPECT(ts_budget_tokens(100, NULL), -1);
    EXPECT(ts_expand_capacity(100, 1000, 4, 256, 1), 560);
    EXPECT(ts_expand_capacity(-1, 1000, 4, 256, 1), -1);
    EXPECT(ts_expand_capacity(INT64_MAX / 2, INT64_MAX / 2, 4, 256, INT64_MAX / 4), -1);
    EXPECT(ts_expand_capacity((int64_t)1 << 40, (int64_t)1 << 40, 0, 0, 1), -1);        /* would overflow */
    EXPECT(ts_expand_capacity((int64_t)1 << 31, (int64_t)1 << 31, 1 << 30, 1 << 30, 1 << 20), (int64_t)1 << 31);
    const ts_select_params wide = params(0, ((int64_t)1 << 31) - 1, (int64_t)1 << 31, 4, 256, 1, 9, 10);
    EXPECT(ts_budget_tokens((int64_t)1 << 40, &wide), -1);                                 /* would overflow */
    EXPECT(ts_budget_tokens((int64_t)1 << 31, &wide), ((int64_t)1 << 31) - 1);

    /* index append */
    EXPECT(ts_index_append(NULL, F, F, 0, 1, 8, NULL), -1);
    EXPECT(ts_index_append(M, F, F, 0, 1, 8, NULL), -1);
    EXPECT(ts_index_append(F, F, F, -1, 1, 8, NULL), -1);
    EXPECT(ts_index_append(F, F, F, 0, 1, 3, NULL), -2);

    /* score: offsets, heads, workspace */
    EXPECT(ts_score(F, F, F, F, oneg, 1, 32, 8, F, F, (size_t)1 << 20, NULL), -1);
    EXPECT(ts_score(F, F, F, F, obad, 2, 32, 8, F, F, (size_t)1 << 20, NULL), -1);
    EXPECT(ts_score(F, F, F, F, o1, 0, 32, 8, F, F, (size_t)1 << 20, NULL), -1);
    EXPECT(ts_score(F, F, F, F, o1, 1, 24, 8, F, F, (size_t)1 << 20, NULL), -2);
    EXPECT(ts_score(F, F, F, F, o1, 1, 32, 8, F, F, ts_score_workspace_bytes(1, 32) - 1, NULL), -3);

    /* select and score_select: parameters and workspace */
    ts_select_params bad[4] = {params(2, 1, 5, 4, 256, 1, 9, 10), params(0, 1, 0, 4, 256, 1, 9, 10),
                               params(0, 1, 5, 4, 256, 1, 11, 10), params(0, 1, 5, -1, 256, 1, 9, 10)};
    for (int i = 0; i < 4; ++i) {
        EXPECT(ts_select(F, F, o1, 1, 8, 2, &bad[i], F, F, NULL, NULL, F, (size_t)1 << 40, NULL), -1);
        EXPECT(ts_score_select(F, F, F, NULL, F, o1, 1, 8, 2, &bad[i], F, F, F, NULL, NULL, F, (size_t)1 << 40, NULL),
               -1);
    }
    const size_t sel = ts_select_workspace_bytes(o1, 1, 8, &ok);
    EXPECT(sel > 0, 1);
    EXPECT(ts_select(F, F, o1, 1, 8, 2, &ok, F, F, NULL, NULL, F, sel - 1, NULL), -3);
    EXPECT(ts_select(F, F, o1, 1, 8, 2, NULL, F, F, NULL, NULL, F, sel, NULL), -1);
    const size_t ssel = ts_score_select_workspace_bytes(o1, 1, 8, &ok);
    EXPECT(ts_score_select_state_offset(o1, 1, 8, &ok) >= 0, 1);
    EXPECT(ts_score_select_state_offset(o1, 1, 8, NULL), -1);
    EXPECT(ts_tiered_decode(F, F, F, F, F, 3, F, o1, F, F, c100, 0, 1, 8, 2, F, F, (size_t)1 << 40, NULL), -1);
    EXPECT(ts_tiered_decode(F, F, F, NULL, F, 64, F, o1, F, F, c100, 0, 1, 8, 2, F, F, (size_t)1 << 40, NULL), -1);
    EXPECT(ts_tiered_decode(F, F, F, F, F, 64, F, o1, NULL, NULL, NULL, 3, 1, 8, 2, F, F, 16, NULL), -3);
    EXPECT(ts_host_device_pointer(NULL, NULL), -1);
    float gus = 0.f;
    EXPECT(ts_sparse_decode_timed(F, F, F, F, o1, F, F, c100, 0, 1, 8, 2, F, F, 16, NULL, &gus), -3);
    EXPECT(ts_sparse_decode_timed(F, F, F, F, o1, F, F, c100, 0, 1, 8, 2, F, F, (size_t)1 << 40, NULL, NULL), -1);
    EXPECT(ts_score_select(F, F, F, M, F, o1, 1, 8, 2, &ok, F, F, F, NULL, NULL, F, ssel, NULL), -1);
    EXPECT(ts_score_select(F, F, F, NULL, F, o1, 1, 8, 2, &ok, F, F, F, NULL, NULL, F, ssel - 1, NULL), -3);
    EXPECT(ts_score_select(F, F, F, NULL, F, o1, 1, 12, 8, &ok, F, F, F, NULL, NULL, F, ssel, NULL), -2);
    EXPECT(ts_score_select(F, F, F, NULL, F, obad, 2, 8, 2, &ok, F, F, F, NULL, NULL, F, ssel, NULL), -1);

    /* selection expansion */
    const int64_t cp[1] = {100};
    const size_t xw = ts_expand_workspace_bytes(cp, 1, 1);
    EXPECT(ts_expand_selection(F, F, cp, F, o1000, 1, 1, 4, 256, 1, F, F, F, F, xw - 1, NULL), -3);
    EXPECT(ts_expand_selection(F, F, cp, F, o1000, 1, 1, -1, 256, 1, F, F, F, F, xw, NULL), -1);

    /* decode */
    const size_t dw = ts_decode_workspace_bytes(o1000, c100, 1, 32, 8, 0);
    EXPECT(ts_sparse_decode(F, F, F, F, o1000, F, F, c0, 0, 1, 32, 8, F, F, dw, NULL), -1);
    EXPECT(ts_sparse_decode(F, F, F, F, o1000, F, F, c1001, 0, 1, 32, 8, F, F, dw, NULL), -1);
    EXPECT(ts_sparse_decode(F, F, F, F, o1000, F, F, c100, 7, 1, 32, 8, F, F, dw, NULL), -1);
    EXPECT(ts_sparse_decode(F, F, F, F, o1000, NULL, F, c100, 0, 1, 32, 8, F, F, dw, NULL), -1);
    EXPECT(ts_sparse_decode(F, F, F, F, o1000, F, F, c100, 0, 1, 32, 8, F, F, dw - 1, NULL), -3);
    EXPECT(ts_sparse_decode_noalloc(M, F, F, F, o1000, F, F, c100, 0, 1, 32, 8, F, NULL), -1);
    EXPECT(ts_sparse_decode_noalloc(F, F, F, F, o1000, F, F, c100, 0, 1, 24, 8, F, NULL), -2);
    EXPECT(ts_dense_decode(F, M, F, F, o1000, 1, 32, 8, F, F, (size_t)1 << 40, NULL), -1);
    EXPECT(ts_dense_decode(F, F, F, F, o1000, 1, 32, 8, F, F, ts_decode_workspace_bytes(o1000, NULL, 1, 32, 8, 0) - 1,
                           NULL), -3);

    /* per-KV-group union and its decode */
    const size_t uw = ts_union_workspace_bytes(o1000, 1, 8);
    EXPECT(ts_union_lists(NULL, F, c100, F, o1000, 1, 32, 8, F, F, F, F, uw, NULL), -1);
    EXPECT(ts_union_lists(F, F, c1001, F, o1000, 1, 32, 8, F, F, F, F, uw, NULL), -1);
    EXPECT(ts_union_lists(F, F, c100, F, o1000, 1, 48, 4, F, F, F, F, uw, NULL), -2);
    EXPECT(ts_union_lists(F, F, c100, F, o1000, 1, 32, 8, F, F, F, F, uw - 1, NULL), -3);
    const size_t udw = ts_decode_workspace_bytes(o1000, c100, 1, 32, 8, QASI_MODE_UNION);
    EXPECT(ts_union_decode(F, F, F, F, o1000, F, F, F, F, c0, 1, 32, 8, F, F, udw, NULL), -1);
    EXPECT(ts_union_decode(F, F, F, F, o1000, F, F, F, F, c100, 1, 24, 8, F, F, udw, NULL), -2);
    EXPECT(ts_union_decode(F, F, F, F, o1000, F, F, F, F, c100, 1, 32, 8, F, F, udw - 1, NULL), -3);

    /* SnapKV */
    EXPECT(snapkv_compress(F, F, F, 1000, 32, 64, 8, 4096, 5, F, F, F, NULL, NULL, F, (size_t)1 << 40, NULL), -2);
    EXPECT(snapkv_compress(F, F, F, 1000, 3, 64, 8, 4096, 3, F, F, F, NULL, NULL, F, (size_t)1 << 40, NULL), -2);
    EXPECT(snapkv_compress(F, F, F, 0, 32, 64, 8, 4096, 3, F, F, F, NULL, NULL, F, (size_t)1 << 40, NULL), -1);
    EXPECT(snapkv_compress(F, F, F, ((int64_t)1 << 24) + 1, 32, 64, 8, 4096, 3, F, F, F, NULL, NULL, F,
                           (size_t)1 << 40, NULL), -2);
    EXPECT(snapkv_compress(F, F, F, 1000, 32, 64, 8, 4096, 3, F, F, F, NULL, NULL, F,
                           snapkv_workspace_bytes(1000, 32, 64, 8, 4096) - 1, NULL), -3);
    EXPECT(snapkv_retain_clusters(F, 1000, 8, 100, -1, F, F, F, F, F, F, F, (size_t)1 << 40, NULL), -1);

    if (failures) {
        fprintf(stderr, "%d unexpected codes\n", failures);
        return 1;
    }
    printf("C-ABI sanitizer run: ok\n");
    return 0;
}
