// Per-KV-group union of the per-head lists with a G-bit head mask (the union decode's input).
//
// [TS] "主要な貢献": in per-head mode each query head selects its own tokens; the G query heads
// that share a KV head read the same K/V rows, so the decode can read each row of the group's
// union once and let every head use the rows it selected.  Input: per-head lists in ts_select's
// layout (idx[Hq*kpre_b + h*K_b + j]), each ascending with its empty slots (-1) last.  Output,
// for sequence b and KV head g, in the block of G*K_b entries at Hq*kpre_b + g*G*K_b: the union's
// tokens in ascending order, then -1; the mask (same layout) has bit hh set when head g*G + hh
// selected the token (0 past the union); ucount[b*Hkv + g] = the union's size.  Entries outside
// [0, n_b) (the empty slots) are no tokens.
//
// The sequence's tokens go in windows of kUnWin; block = (sequence, KV head, window), numbered
// sequence by sequence, KV head by KV head.  union_mark_kernel: wave hh finds head hh's entries
// of the window (two 64-ary searches of the ascending list: 64 probes per step), the block sets
// their head bits in a mask byte per token in LDS (32-bit atomic OR on the byte's word), then
// stores the window's mask bytes and its count of non-zero bytes to the workspace.
// union_write_kernel: the counts of the group's earlier windows give the window's first output
// position; one block scan places its tokens in order; the group's padding is spread over its
// windows.
#include "qasi_device.h"
#include "qasi_internal.h"

namespace qasi {

constexpr int kUnWin = 4096;                       // tokens per window (mask bytes)
constexpr int kUnMarkThreads = 512;                // a wave per head of the group (G <= 8)
constexpr int kUnWriteThreads = kUnWin / 16;       // 16 mask bytes per thread

__host__ __device__ inline int64_t un_windows(int64_t n) { return (n + kUnWin - 1) / kUnWin; }

// First index j of list[0, k) with (uint32) list[j] >= x, for a list ascending in that order
// (valid entries ascending, the -1 slots after them); the whole wave returns it.
__device__ __forceinline__ int64_t wave_lower_bound(const int32_t* list, int64_t k, uint32_t x) {
    const int lane = threadIdx.x & 63;
    int64_t lo = 0, hi = k;                        // the answer lies in [lo, hi]
    while (hi - lo > 64) {
        // probe j_l = lo + (l+1) s - 1; the first c probes hold keys below x
        const int64_t s = (hi - lo + 63) / 64;
        const int64_t j = lo + (int64_t)(lane + 1) * s - 1;
        const bool below = j < hi && (uint32_t)list[j] < x;
        const int64_t c = __popcll(__ballot(below));
        const int64_t jc = lo + (c + 1) * s - 1;    // first probe at or above x
        lo += c * s;
        hi = jc < hi ? jc : hi;
    }
    const int64_t j = lo + lane;
    const bool below = j < hi && (uint32_t)list[j] < x;
    return lo + __popcll(__ballot(below));
}

// Block -> (sequence, KV head, window) and the group's list pointers.
struct UnBlock {
    int b, g;
    int64_t w, nw, n, K, kpre, w0, w1, first;      // first: block number of the group's window 0
};
__device__ __forceinline__ bool un_block(const I64Arg& counts, const I64Arg& offsets, int B, int Hkv, UnBlock& x) {
    const SeqPos sp = wave_find_seq(B, blockIdx.x, Hkv * un_windows(offsets[1] - offsets[0]),
                                    [od = offsets.dev, Hkv](int i) { return Hkv * un_windows(od[i + 1] - od[i]); });
    if (sp.b < 0) return false;
    x.b = sp.b;
    x.nw = sp.cnt / Hkv;
    const int64_t k = blockIdx.x - sp.first;
    x.g = (int)(k / x.nw);
    x.w = k % x.nw;
    x.first = blockIdx.x - x.w;
    x.n = offsets[x.b + 1] - offsets[x.b];
    x.K = counts[x.b];
    x.kpre = wave_prefix_seq(x.b, [cd = counts.dev](int i) { return cd[i]; });
    x.w0 = x.w * kUnWin;
    x.w1 = x.w0 + kUnWin < x.n ? x.w0 + kUnWin : x.n;
    return true;
}

__global__ __launch_bounds__(kUnMarkThreads) void union_mark_kernel(const int32_t* __restrict__ idx, I64Arg counts,
                                                                   I64Arg offsets, int B, int Hq, int Hkv,
                                                                   uint4* __restrict__ bm, uint32_t* __restrict__ wcnt) {
    __shared__ uint32_t mk[kUnWin / 4];
    __shared__ int64_t rs[8], re[8];
    __shared__ int tmp[kUnMarkThreads / 64];
    UnBlock x;
    if (!un_block(counts, offsets, B, Hkv, x)) return;
    const int t = threadIdx.x, wid = t >> 6, G = Hq / Hkv;
    const int32_t* lists = idx + (int64_t)Hq * x.kpre + (int64_t)x.g * G * x.K;   // head g*G + hh at + hh*K
    for (int i = t; i < kUnWin / 4; i += kUnMarkThreads) mk[i] = 0;
    if (wid < G) {
        const int32_t* l = lists + (int64_t)wid * x.K;
        const int64_t s = x.w0 == 0 ? 0 : wave_lower_bound(l, x.K, (uint32_t)x.w0);
        const int64_t e = wave_lower_bound(l, x.K, (uint32_t)x.w1);
        if ((t & 63) == 0) {
            rs[wid] = s;
            re[wid] = e;
        }
    }
    __syncthreads();
    for (int hh = 0; hh < G; ++hh) {
        const int32_t* l = lists + (int64_t)hh * x.K;
        for (int64_t j = rs[hh] + t; j < re[hh]; j += kUnMarkThreads) {
            const uint32_t r = (uint32_t)l[j] - (uint32_t)x.w0;           // in [0, w1 - w0) for an ascending list
            if (r < (uint32_t)kUnWin) atomicOr(&mk[r >> 2], (1u << hh) << (8 * (r & 3)));
        }
    }
    __syncthreads();
    int c = 0;
    if (t < kUnWin / 16) {
        const uint4 v = reinterpret_cast<const uint4*>(mk)[t];
        bm[blockIdx.x * (int64_t)(kUnWin / 16) + t] = v;
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int u = 0; u < 4; ++u)
            c += ((w4[u] & 0xffu) ? 1 : 0) + ((w4[u] & 0xff00u) ? 1 : 0) + ((w4[u] & 0xff0000u) ? 1 : 0) +
                 ((w4[u] >> 24) ? 1 : 0);
    }
    int tot = 0;
    block_inclusive_scan<kUnMarkThreads>(c, tmp, &tot);
    if (t == 0) wcnt[blockIdx.x] = (uint32_t)tot;
}

__global__ __launch_bounds__(kUnWriteThreads) void union_write_kernel(I64Arg counts, I64Arg offsets, int B, int Hq,
                                                                     int Hkv, const uint4* __restrict__ bm,
                                                                     const uint32_t* __restrict__ wcnt,
                                                                     int32_t* __restrict__ uidx,
                                                                     uint8_t* __restrict__ umask,
                                                                     int64_t* __restrict__ ucount) {
    __shared__ int tmp[kUnWriteThreads / 64];
    __shared__ int64_t red[2][kUnWriteThreads / 64];
    UnBlock x;
    if (!un_block(counts, offsets, B, Hkv, x)) return;
    const int t = threadIdx.x, G = Hq / Hkv;
    const int64_t base = (int64_t)Hq * x.kpre + (int64_t)x.g * G * x.K;
    int32_t* uo = uidx + base;
    uint8_t* mo = umask + base;
    // the earlier windows' counts of the group, and the union's size
    int64_t before = 0, total = 0;
    for (int64_t i = t; i < x.nw; i += kUnWriteThreads) {
        const int64_t v = wcnt[x.first + i];
        total += v;
        if (i < x.w) before += v;
    }
    for (int o = 32; o > 0; o >>= 1) {
        before += __shfl_xor(before, o, 64);
        total += __shfl_xor(total, o, 64);
    }
    if ((t & 63) == 0) {
        red[0][t >> 6] = before;
        red[1][t >> 6] = total;
    }
    __syncthreads();
    int64_t bsum = 0, U = 0;
#pragma unroll
    for (int w = 0; w < kUnWriteThreads / 64; ++w) {
        bsum += red[0][w];
        U += red[1][w];
    }
    // the window's tokens in order: thread t holds tokens w0 + 16t .. w0 + 16t + 15
    const uint4 v = bm[blockIdx.x * (int64_t)(kUnWin / 16) + t];
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
    int c = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u)
        c += ((w4[u] & 0xffu) ? 1 : 0) + ((w4[u] & 0xff00u) ? 1 : 0) + ((w4[u] & 0xff0000u) ? 1 : 0) +
             ((w4[u] >> 24) ? 1 : 0);
    int all = 0;
    const int inc = block_inclusive_scan<kUnWriteThreads>(c, tmp, &all);
    int64_t p = bsum + inc - c;
    // U <= G K for ascending lists; the bound keeps lists out of order from writing past the block
    const int64_t cap = (int64_t)G * x.K;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t m = (w4[u] >> (8 * q)) & 0xffu;
            if (m) {
                if (p < cap) {
                    uo[p] = (int32_t)(x.w0 + 16 * t + 4 * u + q);
                    mo[p] = (uint8_t)m;
                }
                ++p;
            }
        }
    // padding [U, G K): an equal share per window
    const int64_t per = (cap - U + x.nw - 1) / x.nw;
    const int64_t p0 = U + x.w * per, p1 = p0 + per < cap ? p0 + per : cap;
    for (int64_t j = p0 + t; j < p1; j += kUnWriteThreads) {
        uo[j] = -1;
        mo[j] = 0;
    }
    if (x.w == 0 && t == 0) ucount[(int64_t)x.b * Hkv + x.g] = U < cap ? U : cap;
}

static int64_t union_blocks(const int64_t* offsets_host, int B, int Hkv) {
    int64_t nb = 0;
    for (int b = 0; b < B; ++b) nb += Hkv * un_windows(offsets_host[b + 1] - offsets_host[b]);
    return nb;
}

size_t union_workspace(const int64_t* offsets_host, int B, int Hkv) {
    const int64_t nb = union_blocks(offsets_host, B, Hkv);
    WsCarver w(nullptr);
    w.take<uint4>((size_t)nb * (kUnWin / 16));
    w.take<uint32_t>((size_t)nb);
    return w.size();
}

hipError_t launch_union(const int32_t* idx, const int64_t* counts_dev, const int64_t* counts_host,
                        const int64_t* offsets_dev, const int64_t* offsets_host, int B, int Hq, int Hkv, int32_t* uidx,
                        uint8_t* umask, int64_t* ucount, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (union_workspace(offsets_host, B, Hkv) > ws_bytes) return hipErrorInvalidValue;
    const int64_t nb = union_blocks(offsets_host, B, Hkv);
    WsCarver w(ws);
    uint4* bm = w.take<uint4>((size_t)nb * (kUnWin / 16));
    uint32_t* wcnt = w.take<uint32_t>((size_t)nb);
    const I64Arg offs = i64_arg(offsets_dev, offsets_host, (int64_t)B + 1);
    const I64Arg cnts = i64_arg(counts_dev, counts_host, B);
    hipLaunchKernelGGL(union_mark_kernel, dim3((unsigned)nb), dim3(kUnMarkThreads), 0, stream, idx, cnts, offs, B, Hq,
                       Hkv, bm, wcnt);
    hipLaunchKernelGGL(union_write_kernel, dim3((unsigned)nb), dim3(kUnWriteThreads), 0, stream, cnts, offs, B, Hq, Hkv,
                       bm, wcnt, uidx, umask, ucount);
    return hipGetLastError();
}

}  // namespace qasi
