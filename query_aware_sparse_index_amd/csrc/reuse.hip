// Selection reuse with neighbour fetch.
//
// [TB] "Inferenzstrategie", Optimierungen: the token selector need not run at every decode step;
// it runs every N steps (the prediction interval) and the steps in between reuse its selection.
// To cover tokens whose importance shifts between two selections, every selected token is widened
// to its spatial neighbours (neighbour fetch).  The sink tokens and the local window of the
// current step are always kept ([TB] the sink and circular local-window buffers).
//
// expand_kernel, one block per list (sequence b, list l: one list per sequence in vote mode, one
// per query head in per-head mode).  The previous list is sorted and unique; the expanded list
//   out = [0, s) U ((U_j [t_j - r, t_j + r]) cut to [s, le)) U [le, n),
//   s = min(sink, n), le = max(s, n - local),
// is written in ascending order.  Because the t_j ascend, the interval of entry j adds the
// positions above both the previous entry's interval end and s - 1:
//   lo_j = max(t_j - r, s, min(t_{j-1} + r, le - 1) + 1),  hi_j = min(t_j + r, le - 1),
// so every entry's count follows from itself and its predecessor, and one block scan over the
// counts places the positions.  Slots past the expanded list's length, up to its capacity, are
// -1 (empty slots that the sparse decode skips).
#include "qasi_device.h"
#include "qasi_internal.h"

namespace qasi {

constexpr int kExThreads = 1024;
constexpr int kExPer = 32;                         // consecutive previous entries per thread per round
constexpr int kExRound = kExThreads * kExPer;

__host__ __device__ inline int64_t expand_cap(int64_t k_prev, int64_t n, int64_t sink, int64_t local, int64_t r) {
    const int64_t c = (2 * r + 1) * k_prev + sink + local;
    return c < n ? c : n;
}

int64_t expand_capacity(int64_t k_prev, int64_t n, int64_t sink, int64_t local, int64_t radius) {
    return expand_cap(k_prev, n, sink, local, radius);
}

__global__ __launch_bounds__(kExThreads) void expand_kernel(const int32_t* __restrict__ prev, I64Arg counts_prev,
                                                           I64Arg offsets, int B, int L, int64_t sink, int64_t local,
                                                           int64_t r, int32_t* __restrict__ out,
                                                           int64_t* __restrict__ caps_out,
                                                           int64_t* __restrict__ valid_out) {
    __shared__ int tmp[kExThreads / 64];
    const int b = blockIdx.x / L, l = blockIdx.x % L, t = threadIdx.x;
    const int64_t n = offsets[b + 1] - offsets[b];
    const int64_t kp = counts_prev[b];
    const int64_t cap = expand_cap(kp, n, sink, local, r);
    // list starts of the sequences before b (every lane of the wave calls these)
    const int64_t ppre = wave_prefix_seq(b, [cd = counts_prev.dev](int i) { return cd[i]; });
    const int64_t cpre = wave_prefix_seq(b, [cd = counts_prev.dev, od = offsets.dev, sink, local, r](int i) {
        return expand_cap(cd[i], od[i + 1] - od[i], sink, local, r);
    });
    const int32_t* p = prev + L * ppre + (int64_t)l * kp;
    int32_t* o = out + L * cpre + (int64_t)l * cap;
    const int64_t s = sink < n ? sink : n;
    const int64_t le = n - local > s ? n - local : s;
    // the sink tokens first
    for (int64_t i = t; i < s; i += kExThreads) o[i] = (int32_t)i;
    int64_t pos0 = s;                                // output position of the round's first entry
    for (int64_t r0 = 0; r0 < kp; r0 += kExRound) {
        const int64_t j0 = r0 + (int64_t)kExPer * t;
        // the thread's entries and their predecessor, all loads in flight at once (entries past
        // the list read its first entry and count nothing)
        int32_t e[kExPer];
#pragma unroll
        for (int u = 0; u < kExPer; ++u) e[u] = p[j0 + u < kp ? j0 + u : 0];
        const int32_t before = (j0 > 0 && j0 - 1 < kp) ? p[j0 - 1] : -1;
        int64_t cov = before < 0 ? s - 1 : (before + r < le - 1 ? before + r : le - 1);
        if (cov < s - 1) cov = s - 1;
        int cnt[kExPer];
        int tot = 0;
#pragma unroll
        for (int u = 0; u < kExPer; ++u) {
            cnt[u] = 0;
            if (j0 + u >= kp || e[u] < 0) continue;   // past the list, or an empty slot
            const int64_t tj = e[u];
            int64_t lo = tj - r;
            if (lo < cov + 1) lo = cov + 1;
            const int64_t hi = tj + r < le - 1 ? tj + r : le - 1;
            if (hi >= lo) cnt[u] = (int)(hi - lo + 1);
            if (hi > cov) cov = hi;
            tot += cnt[u];
        }
        int all;
        const int inc = block_inclusive_scan<kExThreads>(tot, tmp, &all);
        int64_t pos = pos0 + inc - tot;
        // write the positions (the same interval arithmetic again, now with the output offset)
        cov = before < 0 ? s - 1 : (before + r < le - 1 ? before + r : le - 1);
        if (cov < s - 1) cov = s - 1;
#pragma unroll
        for (int u = 0; u < kExPer; ++u) {
            if (cnt[u] == 0) {
                if (j0 + u < kp && e[u] >= 0) {
                    const int64_t hi = (int64_t)e[u] + r < le - 1 ? (int64_t)e[u] + r : le - 1;
                    if (hi > cov) cov = hi;
                }
                continue;
            }
            const int64_t lo = (int64_t)e[u] - r > cov + 1 ? (int64_t)e[u] - r : cov + 1;
            for (int c = 0; c < cnt[u]; ++c) o[pos + c] = (int32_t)(lo + c);
            pos += cnt[u];
            cov = lo + cnt[u] - 1;
        }
        pos0 += all;
        __syncthreads();                               // tmp is reused by the next round's scan
    }
    // the local window, then empty slots up to the capacity
    for (int64_t i = t; i < n - le; i += kExThreads) o[pos0 + i] = (int32_t)(le + i);
    const int64_t valid = pos0 + (n - le);
    for (int64_t i = valid + t; i < cap; i += kExThreads) o[i] = -1;
    if (t == 0) {
        valid_out[(int64_t)b * L + l] = valid;
        if (l == 0 && caps_out) caps_out[b] = cap;
    }
}

hipError_t launch_expand(const int32_t* prev, const int64_t* counts_prev_dev, const int64_t* counts_prev_host,
                         const int64_t* offsets_dev, const int64_t* offsets_host, int B, int L, int64_t sink,
                         int64_t local, int64_t radius, int32_t* out, int64_t* caps_out, int64_t* valid_out,
                         hipStream_t stream) {
    const I64Arg offs = i64_arg(offsets_dev, offsets_host, (int64_t)B + 1);
    const I64Arg cnts = i64_arg(counts_prev_dev, counts_prev_host, B);
    hipLaunchKernelGGL(expand_kernel, dim3((unsigned)(B * L)), dim3(kExThreads), 0, stream, prev, cnts, offs, B, L,
                       sink, local, radius, out, caps_out, valid_out);
    return hipGetLastError();
}

}  // namespace qasi
