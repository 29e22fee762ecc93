// Internal launcher interface between the C-ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qasi {

// An int64 array (sequence offsets, list lengths) as a kernel argument.  For a single
// sequence (one length, or the offsets {0, n}) the values travel in the launch arguments, so
// that a kernel knows its bounds without a dependent global load at its start; otherwise the
// kernels read the device copy.  The C ABI requires the host and device copies to agree.
struct I64Arg {
    const int64_t* dev;
    int32_t one;      // 1: a single sequence, values in h0 (and h1)
    int64_t h0, h1;
    __host__ __device__ __forceinline__ int64_t operator[](int64_t i) const {
        return one ? (i == 0 ? h0 : h1) : dev[i];
    }
};
inline I64Arg i64_arg(const int64_t* dev, const int64_t* host, int64_t count) {
    I64Arg a;
    a.dev = dev;
    a.one = (host && (count == 1 || count == 2)) ? 1 : 0;
    a.h0 = a.one ? host[0] : 0;
    a.h1 = (a.one && count == 2) ? host[1] : 0;
    return a;
}

// ---- index and score
hipError_t launch_index_append(const uint16_t* k_new, const float* P, uint16_t* k_index, int64_t pos, int64_t T,
                               int Hkv, hipStream_t stream);
size_t score_workspace(int B, int Hq);
hipError_t launch_score(const uint16_t* q, const float* P, const uint16_t* k_index, const int64_t* offsets_dev,
                        const int64_t* offsets_host, int B, int Hq, int Hkv, float* scores, void* ws,
                        size_t ws_bytes, hipStream_t stream);

// Scores plus the classification of every tile against per-instance key brackets (the fused
// score-and-select path): q' is read from qp; per (head, tile) records, see score_kernel.
hipError_t launch_score_classify(const float* qp, const uint16_t* k_index, const int64_t* offsets_dev,
                                 const int64_t* offsets_host, int B, int Hq, int Hkv, float* scores,
                                 const int64_t* state, uint32_t* tinfo, uint32_t* cand, uint32_t* tcand,
                                 hipStream_t stream);
int64_t score_items(const int64_t* offsets_host, int B);

// ---- selection
// Per-instance state of an order statistic: int64 words at state[(b * Hq + h) * 8 + k].
enum : int { kStFlag = 0, kStKey = 1, kStGt = 2, kStNeed = 3, kStLo = 4, kStHi = 5, kStBeg = 6, kStEnd = 7 };
// Key run of a 64-token tile in the fused path's tile classification: at most 64 in-bracket
// keys for each of at most 64 query heads.
constexpr int kClsTile = 64 * 64;
// In-bracket keys of one (head, tile) kept in the head-major slots of the tile classification;
// the rest go to the tile's key area.
constexpr int kClsSlots = 16;

struct SelectConfig {
    int mode;
    int64_t bnum, bden, sink, local, vmin, tnum, tden;
};
size_t select_workspace(const int64_t* offsets_host, int B, int Hq, const SelectConfig& c);
hipError_t launch_select(const float* scores, int64_t S, const int64_t* offsets_dev, const int64_t* offsets_host,
                         int B, int Hq, const SelectConfig& c, int32_t* idx_out, int64_t* count_out, float* theta_out,
                         uint8_t* votes_out, void* ws, size_t ws_bytes, hipStream_t stream);
int64_t budget_tokens(int64_t n, const SelectConfig& c);
// ts_score followed by ts_select in one pass (and, when K is given, the index row of every
// sequence's last token appended first): identical scores, thresholds and lists.
size_t score_select_workspace(const int64_t* offsets_host, int B, int Hq, const SelectConfig& c);
// byte offset in that workspace of the per-instance records [B * Hq][8] (kSt* fields)
size_t score_select_state_offset(const int64_t* offsets_host, int B, int Hq, const SelectConfig& c);
hipError_t launch_score_select(const uint16_t* q, const float* P, uint16_t* k_index, const uint16_t* K,
                               const int64_t* offsets_dev, const int64_t* offsets_host, int B, int Hq, int Hkv,
                               const SelectConfig& c, float* scores, int32_t* idx_out, int64_t* count_out,
                               float* theta_out, uint8_t* votes_out, void* ws, size_t ws_bytes, hipStream_t stream);
// SnapKV top-c of `rows` importance rows imp[rows][n]: pooled[r * ps + j] (and, when non-null,
// pooled_out[r * n + j]) = avg_pool1d(3) of the row, then the top min(c, n) positions per row,
// ties to the lower position, ascending in idx_out[r * min(c, n) + j].
size_t snap_topc_workspace(int rows, int64_t n);
hipError_t launch_snap_topc(const float* imp, int64_t n, int rows, int64_t c, float* pooled, int64_t ps,
                            float* pooled_out, int32_t* idx_out, void* ws, size_t ws_bytes, hipStream_t stream);

// ---- selection reuse with neighbour fetch
int64_t expand_capacity(int64_t k_prev, int64_t n, int64_t sink, int64_t local, int64_t radius);
// blocks of the two expansion kernels (one u32 of workspace each)
int64_t expand_blocks(const int64_t* counts_prev_host, int B, int L);
hipError_t launch_expand(const int32_t* prev, const int64_t* counts_prev_dev, const int64_t* counts_prev_host,
                         const int64_t* offsets_dev, const int64_t* offsets_host, int B, int L, int64_t sink,
                         int64_t local, int64_t radius, int32_t* out, int64_t* caps_out, int64_t* valid_out,
                         uint32_t* chunk_counts, hipStream_t stream);

// ---- per-KV-group union of per-head lists with head masks
size_t union_workspace(const int64_t* offsets_host, int B, int Hkv);
hipError_t launch_union(const int32_t* idx, const int64_t* counts_dev, const int64_t* counts_host,
                        const int64_t* offsets_dev, const int64_t* offsets_host, int B, int Hq, int Hkv, int32_t* uidx,
                        uint8_t* umask, int64_t* ucount, void* ws, size_t ws_bytes, hipStream_t stream);

// ---- decode
// mode: 0 vote lists, 1 per-head lists, 2 dense (counts_host NULL), 3 union lists (G*count_b slots)
// The newest N positions of every sequence in a ring of N slots: position t of sequence b at slot
// t mod N of K / V [B][N][Hkv][128] (N a power of two); the older positions in the main cache.
struct DecRing {
    const uint16_t* K;
    const uint16_t* V;
    int64_t N;
};
size_t decode_workspace(const int64_t* offsets_host, const int64_t* counts_host, int B, int Hq, int Hkv, int mode);
// gather_start / gather_stop (nullable): events recorded at the gather kernel's dispatch start and end
hipError_t launch_sparse_decode(const uint16_t* q, const uint16_t* K, const uint16_t* V, const int64_t* offsets_dev,
                                const int64_t* offsets_host, const int32_t* idx, const int64_t* counts_dev,
                                const int64_t* counts_host, int mode,
                                int B, int Hq, int Hkv, float* out, void* ws, size_t ws_bytes, hipStream_t stream,
                                hipEvent_t gather_start = nullptr, hipEvent_t gather_stop = nullptr);
// ts_sparse_decode with its partials in the library's static device scratch (no workspace);
// hipErrorInvalidValue when the call needs more than kNoAllocScratchBytes.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;
hipError_t launch_sparse_decode_noalloc(const uint16_t* q, const uint16_t* K, const uint16_t* V,
                                        const int64_t* offsets_dev, const int64_t* offsets_host, const int32_t* idx,
                                        const int64_t* counts_dev, const int64_t* counts_host, int mode, int B, int Hq,
                                        int Hkv, float* out, hipStream_t stream);
// Union decode: per (sequence, KV head) the union list (G*count_b slots) with its per-entry head
// masks and its size on the device (the output of launch_union); mode 3 of decode_workspace.
hipError_t launch_union_decode(const uint16_t* q, const uint16_t* K, const uint16_t* V, const int64_t* offsets_dev,
                               const int64_t* offsets_host, const int32_t* uidx, const uint8_t* umask,
                               const int64_t* ucount, const int64_t* counts_dev, const int64_t* counts_host, int B,
                               int Hq, int Hkv, float* out, void* ws, size_t ws_bytes, hipStream_t stream);
hipError_t launch_dense_decode(const uint16_t* q, const uint16_t* K, const uint16_t* V, const int64_t* offsets_dev,
                               const int64_t* offsets_host, int B, int Hq, int Hkv, float* out, void* ws,
                               size_t ws_bytes, hipStream_t stream);
// Decode over a tiered cache (mode 0, 1 or 2 as above): K / V hold the positions older than the
// ring (device memory, or host memory mapped for the device), `ring` the newest N.
hipError_t launch_tiered_decode(const uint16_t* q, const uint16_t* K, const uint16_t* V, const DecRing& ring,
                                const int64_t* offsets_dev, const int64_t* offsets_host, const int32_t* idx,
                                const int64_t* counts_dev, const int64_t* counts_host, int mode, int B, int Hq,
                                int Hkv, float* out, void* ws, size_t ws_bytes, hipStream_t stream);

// ---- SnapKV
size_t snapkv_workspace(int64_t n, int w, int Hq, int Hkv, int64_t c);
hipError_t launch_snapkv(const uint16_t* q_obs, const uint16_t* K, const uint16_t* V, int64_t n, int w, int Hq,
                         int Hkv, int64_t c, int32_t* idx_out, uint16_t* K_out, uint16_t* V_out, float* imp_out,
                         float* pooled_out, void* ws, size_t ws_bytes, hipStream_t stream);

// SnapKV cluster-based retention: the top-c lists widened by +-k_cluster, rows gathered
hipError_t launch_snapkv_clusters(const int32_t* idx, int64_t n, int Hkv, int64_t ce, int64_t k_cluster,
                                  const uint16_t* K, const uint16_t* V, int32_t* idx_out, uint16_t* K_out,
                                  uint16_t* V_out, int64_t* valid_out, uint32_t* chunk_counts, hipStream_t stream);

// One-time per-process set-up (kernel attributes); returns the first error.
hipError_t init_kernels();

// Workspace carving: 256-byte aligned sub-buffers.
struct WsCarver {
    char* base;
    size_t off = 0;
    explicit WsCarver(void* p) : base(static_cast<char*>(p)) {}
    template <class T>
    T* take(size_t count) {
        off = (off + 255) & ~(size_t)255;
        T* p = reinterpret_cast<T*>(base ? base + off : nullptr);
        off += count * sizeof(T);
        return p;
    }
    size_t size() const { return (off + 255) & ~(size_t)255; }
};

}  // namespace qasi
