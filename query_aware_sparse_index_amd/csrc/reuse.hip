// Selection reuse with neighbour fetch.
//
// [TB] "Inferenzstrategie", Optimierungen: the token selector need not run at every decode step;
// it runs every N steps (the prediction interval) and the steps in between reuse its selection.
// To cover tokens whose importance shifts between two selections, every selected token is widened
// to its spatial neighbours (neighbour fetch).  The sink tokens and the local window of the
// current step are always kept ([TB] the sink and circular local-window buffers).
//
// The expanded list of sequence b, list l (one list per sequence in vote mode, one per query
// head in per-head mode), from its previous list (sorted, unique):
//   out = [0, s) U ((U_j [t_j - r, t_j + r]) cut to [s, le)) U [le, n),
//   s = min(sink, n), le = max(s, n - local),
// in ascending order.  Because the t_j ascend, the interval of entry j adds the positions above
// both the previous entry's interval end and s - 1:
//   lo_j = max(t_j - r, s, min(t_{j-1} + r, le - 1) + 1),  hi_j = min(t_j + r, le - 1),
// so every entry's count follows from itself and its predecessor.  Two kernels over chunks of
// kExChunk previous entries (block = (list, chunk), thread = kExPer consecutive entries read as
// one 16-byte load): expand_count_kernel sums each chunk's counts; expand_write_kernel adds the
// earlier chunks' sums, places its entries with one block scan and writes them.  The first chunk
// also writes the sink tokens, the last one the local window and -1 (empty slots that the sparse
// decode skips) up to the list's capacity.
#include "qasi_device.h"
#include "qasi_internal.h"

namespace qasi {

constexpr int kExThreads = 256;
constexpr int kExPer = 4;                          // consecutive previous entries per thread
constexpr int kExChunk = kExThreads * kExPer;      // previous entries per block

__host__ __device__ inline int64_t expand_cap(int64_t k_prev, int64_t n, int64_t sink, int64_t local, int64_t r) {
    const int64_t c = (2 * r + 1) * k_prev + sink + local;
    return c < n ? c : n;
}

int64_t expand_capacity(int64_t k_prev, int64_t n, int64_t sink, int64_t local, int64_t radius) {
    return expand_cap(k_prev, n, sink, local, radius);
}

__host__ __device__ inline int64_t expand_chunks(int64_t k_prev) {
    const int64_t c = (k_prev + kExChunk - 1) / kExChunk;
    return c > 0 ? c : 1;
}

// Geometry of block (list, chunk): the list and chunk indices, the sequence's bounds and the
// previous / expanded lists' starts.  Blocks are numbered sequence by sequence, L * chunks each.
struct ExBlock {
    int b, l;
    int64_t c, nch, n, kp, cap, s, le;
    const int32_t* p;
    int32_t* o;
    int64_t list;        // global list number b * L + l
};

__device__ __forceinline__ bool ex_block(const int32_t* prev, int32_t* out, const I64Arg& counts_prev,
                                         const I64Arg& offsets, int B, int L, int64_t sink, int64_t local, int64_t r,
                                         ExBlock& x) {
    const SeqPos sp = wave_find_seq(B, blockIdx.x, L * expand_chunks(counts_prev[0]),
                                    [cd = counts_prev.dev, L](int i) { return L * expand_chunks(cd[i]); });
    if (sp.b < 0) return false;
    x.b = sp.b;
    x.nch = sp.cnt / L;
    const int64_t k = blockIdx.x - sp.first;
    x.l = (int)(k / x.nch);
    x.c = k % x.nch;
    x.n = offsets[x.b + 1] - offsets[x.b];
    x.kp = B == 1 ? counts_prev[0] : counts_prev.dev[x.b];
    x.cap = expand_cap(x.kp, x.n, sink, local, r);
    const int64_t ppre = wave_prefix_seq(x.b, [cd = counts_prev.dev](int i) { return cd[i]; });
    const int64_t cpre = wave_prefix_seq(x.b, [cd = counts_prev.dev, od = offsets.dev, sink, local, r](int i) {
        return expand_cap(cd[i], od[i + 1] - od[i], sink, local, r);
    });
    x.p = prev + L * ppre + (int64_t)x.l * x.kp;
    x.o = out + L * cpre + (int64_t)x.l * x.cap;
    x.s = sink < x.n ? sink : x.n;
    x.le = x.n - local > x.s ? x.n - local : x.s;
    x.list = (int64_t)x.b * L + x.l;
    return true;
}

// The thread's entries of the block's chunk with their counts; cov0 = the coverage before them.
__device__ __forceinline__ int ex_counts(const ExBlock& x, int64_t r, int32_t (&e)[kExPer], int (&cnt)[kExPer],
                                         int64_t& cov0) {
    const int64_t j0 = x.c * kExChunk + (int64_t)kExPer * threadIdx.x;
    // the four entries one by one (a list starts on a 16-byte boundary only when the lengths before
    // it are multiples of 4); a wave's loads cover one contiguous run of the list
#pragma unroll
    for (int u = 0; u < kExPer; ++u) e[u] = x.kp > 0 ? x.p[j0 + u < x.kp ? j0 + u : 0] : -1;   // none: no read
    const int32_t before = (j0 > 0 && j0 - 1 < x.kp) ? x.p[j0 - 1] : -1;
    int64_t cov = before < 0 ? x.s - 1 : ((int64_t)before + r < x.le - 1 ? (int64_t)before + r : x.le - 1);
    if (cov < x.s - 1) cov = x.s - 1;
    cov0 = cov;
    int tot = 0;
#pragma unroll
    for (int u = 0; u < kExPer; ++u) {
        cnt[u] = 0;
        if (j0 + u >= x.kp || e[u] < 0) continue;       // past the list, or an empty slot
        int64_t lo = (int64_t)e[u] - r;
        if (lo < cov + 1) lo = cov + 1;
        const int64_t hi = (int64_t)e[u] + r < x.le - 1 ? (int64_t)e[u] + r : x.le - 1;
        if (hi >= lo) cnt[u] = (int)(hi - lo + 1);
        if (hi > cov) cov = hi;
        tot += cnt[u];
    }
    return tot;
}

__global__ __launch_bounds__(kExThreads) void expand_count_kernel(const int32_t* __restrict__ prev, I64Arg counts_prev,
                                                                 I64Arg offsets, int B, int L, int64_t sink,
                                                                 int64_t local, int64_t r,
                                                                 uint32_t* __restrict__ chunk_counts) {
    __shared__ int tmp[kExThreads / 64];
    ExBlock x;
    if (!ex_block(prev, nullptr, counts_prev, offsets, B, L, sink, local, r, x)) return;
    int32_t e[kExPer];
    int cnt[kExPer];
    int64_t cov0;
    const int tot = ex_counts(x, r, e, cnt, cov0);
    int all;
    block_inclusive_scan<kExThreads>(tot, tmp, &all);
    if (threadIdx.x == 0) chunk_counts[blockIdx.x] = (uint32_t)all;
}

__global__ __launch_bounds__(kExThreads) void expand_write_kernel(const int32_t* __restrict__ prev, I64Arg counts_prev,
                                                                 I64Arg offsets, int B, int L, int64_t sink,
                                                                 int64_t local, int64_t r, int32_t* __restrict__ out,
                                                                 const uint32_t* __restrict__ chunk_counts,
                                                                 int64_t* __restrict__ caps_out,
                                                                 int64_t* __restrict__ valid_out) {
    __shared__ int tmp[kExThreads / 64];
    __shared__ int64_t red[kExThreads / 64];
    ExBlock x;
    if (!ex_block(prev, out, counts_prev, offsets, B, L, sink, local, r, x)) return;
    const int t = threadIdx.x;
    const uint32_t* cc = chunk_counts + (blockIdx.x - x.c);    // the list's chunk sums
    // the earlier chunks' entries, and (last chunk) the whole list's
    const int64_t upto = x.c == x.nch - 1 ? x.nch : x.c;
    int64_t before = 0, total = 0;
    for (int64_t i = t; i < upto; i += kExThreads) {
        const int64_t v = cc[i];
        total += v;
        if (i < x.c) before += v;
    }
    for (int o = 32; o > 0; o >>= 1) {
        before += __shfl_xor(before, o, 64);
        total += __shfl_xor(total, o, 64);
    }
    if ((t & 63) == 0) red[t >> 6] = before;
    __syncthreads();
    int64_t bsum = 0;
#pragma unroll
    for (int w = 0; w < kExThreads / 64; ++w) bsum += red[w];
    __syncthreads();
    if ((t & 63) == 0) red[t >> 6] = total;
    __syncthreads();
    int64_t tsum = 0;
#pragma unroll
    for (int w = 0; w < kExThreads / 64; ++w) tsum += red[w];
    int32_t e[kExPer];
    int cnt[kExPer];
    int64_t cov;
    const int tot = ex_counts(x, r, e, cnt, cov);
    int all;
    const int inc = block_inclusive_scan<kExThreads>(tot, tmp, &all);
    int64_t pos = x.s + bsum + inc - tot;
#pragma unroll
    for (int u = 0; u < kExPer; ++u) {
        if (cnt[u] == 0) continue;
        const int64_t lo = (int64_t)e[u] - r > cov + 1 ? (int64_t)e[u] - r : cov + 1;
        for (int k = 0; k < cnt[u]; ++k) x.o[pos + k] = (int32_t)(lo + k);
        pos += cnt[u];
        cov = lo + cnt[u] - 1;
    }
    if (x.c == 0)                                        // the sink tokens
        for (int64_t i = t; i < x.s; i += kExThreads) x.o[i] = (int32_t)i;
    if (x.c == x.nch - 1) {                              // the local window, then the empty slots
        const int64_t mid = x.s + tsum;
        for (int64_t i = t; i < x.n - x.le; i += kExThreads) x.o[mid + i] = (int32_t)(x.le + i);
        const int64_t valid = mid + (x.n - x.le);
        for (int64_t i = valid + t; i < x.cap; i += kExThreads) x.o[i] = -1;
        if (t == 0) {
            valid_out[x.list] = valid;
            if (x.l == 0 && caps_out) caps_out[x.b] = x.cap;
        }
    }
}

int64_t expand_blocks(const int64_t* counts_prev_host, int B, int L) {
    int64_t nb = 0;
    for (int b = 0; b < B; ++b) nb += L * expand_chunks(counts_prev_host[b]);
    return nb;
}

hipError_t launch_expand(const int32_t* prev, const int64_t* counts_prev_dev, const int64_t* counts_prev_host,
                         const int64_t* offsets_dev, const int64_t* offsets_host, int B, int L, int64_t sink,
                         int64_t local, int64_t radius, int32_t* out, int64_t* caps_out, int64_t* valid_out,
                         uint32_t* chunk_counts, hipStream_t stream) {
    const I64Arg offs = i64_arg(offsets_dev, offsets_host, (int64_t)B + 1);
    const I64Arg cnts = i64_arg(counts_prev_dev, counts_prev_host, B);
    const unsigned nb = (unsigned)expand_blocks(counts_prev_host, B, L);
    hipLaunchKernelGGL(expand_count_kernel, dim3(nb), dim3(kExThreads), 0, stream, prev, cnts, offs, B, L, sink, local,
                       radius, chunk_counts);
    hipLaunchKernelGGL(expand_write_kernel, dim3(nb), dim3(kExThreads), 0, stream, prev, cnts, offs, B, L, sink, local,
                       radius, out, chunk_counts, caps_out, valid_out);
    return hipGetLastError();
}

}  // namespace qasi
