// Token selection: head thresholds (exact order statistics), votes and ordered compaction.
//
// [TS] "Voting Mechanism": each head h has its own threshold theta_h and
//   Vote(i) = sum_h 1[Score_h(i) > theta_h];  tokens with Vote >= V_min are candidates.
// [TS] "Token-Level Selection と Sparse Attention" and the listing of "基本的な統合パターン":
//   the budget is k = max(int(n * budget), sink + local); sink and local tokens are always
//   kept; below-V_min tokens keep the key -1 and stay fillable; the output is sorted.
// [TS] "主要な貢献" / ablation "w/o Voting" and [TB] "Kernarchitektur": per-head selection
//   ranks tokens by each head's own score under the same budget.
//
// Both modes need an exact order statistic per (sequence, head): theta_h = s_(r) for the
// vote, and the boundary score of the per-head top-K.  It is found by a three-digit radix
// select over order-preserving uint32 keys of the fp32 scores (digits 12 / 12 / 8 bits):
//   os_hist    : per (instance, slice) LDS histogram of the top 12 bits;
//   os_collect : sums the slice histograms, finds the top digit of the answer and copies the
//                keys that share it (the "candidates") next to the slice;
//   os_final   : resolves the low 20 bits among the candidates (two more digits).
// Ties resolve to the lowest position in the compaction kernels, which take every token
// above the boundary and the first `need_eq` tokens equal to it in position order.
#include "qasi_device.h"
#include "qasi_internal.h"

namespace qasi {

constexpr int kOsSlice = 16384;     // keys per radix slice
constexpr int kOsThreads = 1024;
constexpr int kOsMaxSL = 1024;      // slices per instance (n up to 16M tokens)
constexpr int kChunk = 1024;        // tokens per vote / compaction block
constexpr int kVoteBins = 72;       // vote keys 0 .. Hq + 1 (Hq <= 64)

enum : int64_t { kFlagActive = 0, kFlagTakeNone = 1, kFlagTakeAll = 2 };

// state[inst * 8 + k]
enum { kStFlag = 0, kStKey = 1, kStGt = 2, kStNeed = 3, kStD1 = 4, kStR1 = 5, kStGtBin = 6 };

struct DevCfg {
    int mode;
    int64_t bnum, bden, sink, local, vmin, tnum, tden;
};

__host__ __device__ inline int64_t budget_k(int64_t n, int64_t bnum, int64_t bden, int64_t sink, int64_t local) {
    int64_t k = (n * bnum) / bden;
    if (k < sink + local) k = sink + local;
    if (k > n) k = n;
    return k;
}

int64_t budget_tokens(int64_t n, const SelectConfig& c) { return budget_k(n, c.bnum, c.bden, c.sink, c.local); }

// Instance (sequence b, head h) of the order statistic.
struct OsInst {
    int64_t n, beg, end, rank, need, flag;
};

__host__ __device__ inline OsInst os_instance(int64_t n, const DevCfg& c) {
    OsInst o;
    o.n = n;
    if (c.mode == 0) {  // vote: theta over all n tokens
        o.beg = 0;
        o.end = n;
        int64_t r = (n * c.tnum + c.tden - 1) / c.tden;
        if (r < 1) r = 1;
        if (r > n) r = n;
        o.rank = r;
        o.need = 0;
        o.flag = n > 0 ? kFlagActive : kFlagTakeNone;
        return o;
    }
    int64_t a = c.sink < n ? c.sink : n;
    int64_t e = n - c.local;
    if (e < a) e = a;
    int64_t m = e - a;
    int64_t K = budget_k(n, c.bnum, c.bden, c.sink, c.local);
    int64_t need = K - (n - m);
    o.beg = a;
    o.end = e;
    o.need = need;
    if (need <= 0) { o.flag = kFlagTakeNone; o.rank = 0; }
    else if (need >= m) { o.flag = kFlagTakeAll; o.rank = 0; }
    else { o.flag = kFlagActive; o.rank = m - need + 1; }
    return o;
}

__device__ __forceinline__ bool is_forced(int64_t t, int64_t n, int64_t sink, int64_t local) {
    return t < sink || t >= n - local;
}
// number of forced positions in [0, x)
__device__ __forceinline__ int64_t forced_before(int64_t x, int64_t n, int64_t sink, int64_t local) {
    int64_t s = sink < n ? sink : n;
    int64_t a = x < s ? x : s;
    int64_t lo = n - local;
    if (lo < s) lo = s;
    int64_t b = x > lo ? x - lo : 0;
    return a + b;
}

// ------------------------------------------------------------------------ os_hist
__global__ __launch_bounds__(kOsThreads) void os_hist_kernel(const float* __restrict__ scores,
                                                            const int64_t* __restrict__ offsets, int B, int Hq,
                                                            DevCfg cfg, int SL, int64_t S, uint32_t* __restrict__ part1) {
    // 4 sub-histograms (one per group of 4 waves), two 16-bit bins per word
    __shared__ uint32_t sub[4][2048];
    const int inst = blockIdx.y, s = blockIdx.x;
    const int b = inst / Hq, h = inst % Hq;
    const int64_t off = offsets[b];
    OsInst oi = os_instance(offsets[b + 1] - off, cfg);
    for (int i = threadIdx.x; i < 4 * 2048; i += kOsThreads) (&sub[0][0])[i] = 0;
    __syncthreads();
    int64_t lo = oi.beg + (int64_t)s * kOsSlice, hi = lo + kOsSlice;
    if (hi > oi.end) hi = oi.end;
    const bool act = oi.flag == kFlagActive && lo < hi;
    if (act) {
        const float* row = scores + (int64_t)h * S + off;
        uint32_t* mine = sub[threadIdx.x >> 8];
        for_each_f32<kOsThreads, 4>(row, lo, hi, [&](int64_t, float v, bool ok) {
            if (ok) {
                const uint32_t d = order_key(v) >> 20;
                atomicAdd(&mine[d >> 1], (d & 1) ? 0x10000u : 1u);
            }
        });
    }
    __syncthreads();
    uint32_t* dst = part1 + ((size_t)inst * SL + s) * 2048;
    for (int i = threadIdx.x; i < 2048; i += kOsThreads) dst[i] = act ? (sub[0][i] + sub[1][i] + sub[2][i] + sub[3][i]) : 0u;
}

// Finds the digit whose cumulative count (ascending) first reaches `rank` in the 4096-bin
// LDS histogram `hist`.  Returns the digit; *below = count of keys in smaller digits.
__device__ int find_digit_4096(const uint32_t* hist, int64_t rank, int64_t* below, int64_t* sbuf, int* tmp) {
    constexpr int PER = 4096 / kOsThreads;   // consecutive bins owned by a thread
    const int tid = threadIdx.x;
    if (tid == 0) { sbuf[0] = 0; sbuf[1] = 0; }
    __syncthreads();
    int64_t local = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) local += hist[tid * PER + i];
    int total;
    const int inc = block_inclusive_scan<kOsThreads>((int)local, tmp, &total);
    const int64_t excl = inc - local;
    if (excl < rank && rank <= inc) {
        int64_t c = excl;
        for (int i = 0; i < PER; ++i) {
            const int64_t nc = c + hist[tid * PER + i];
            if (rank <= nc) { sbuf[0] = tid * PER + i; sbuf[1] = c; break; }
            c = nc;
        }
    }
    __syncthreads();
    const int d = (int)sbuf[0];
    *below = sbuf[1];
    __syncthreads();
    return d;
}

// --------------------------------------------------------------------- os_collect
__global__ __launch_bounds__(kOsThreads) void os_collect_kernel(const float* __restrict__ scores,
                                                               const int64_t* __restrict__ offsets, int B, int Hq,
                                                               DevCfg cfg, int SL, int64_t S, const uint32_t* __restrict__ part1,
                                                               uint32_t* __restrict__ cand, uint32_t* __restrict__ cand_cnt,
                                                               int64_t* __restrict__ state) {
    __shared__ uint32_t hist[4096];
    __shared__ int64_t sbuf[2];
    __shared__ int tmp[kOsThreads / 64];
    __shared__ uint32_t lcnt;
    const int inst = blockIdx.y, s = blockIdx.x;
    const int b = inst / Hq, h = inst % Hq;
    const int64_t off = offsets[b];
    OsInst oi = os_instance(offsets[b + 1] - off, cfg);
    if (oi.flag != kFlagActive) {
        if (s == 0 && threadIdx.x == 0) {
            state[inst * 8 + kStFlag] = oi.flag;
            state[inst * 8 + kStNeed] = oi.need;
        }
        return;
    }
    // sum the slice histograms (two 16-bit bins per word)
    for (int i0 = threadIdx.x; i0 < 2048; i0 += 8 * kOsThreads) {
        uint32_t a[8], c[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) { a[u] = 0; c[u] = 0; }
        for (int k0 = 0; k0 < SL; k0 += 4) {
            uint32_t w[4][8];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int i = i0 + u * kOsThreads;
                    w[kk][u] = (k0 + kk < SL && i < 2048) ? part1[((size_t)inst * SL + k0 + kk) * 2048 + i] : 0u;
                }
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int u = 0; u < 8; ++u) { a[u] += w[kk][u] & 0xffffu; c[u] += w[kk][u] >> 16; }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * kOsThreads;
            if (i < 2048) { hist[2 * i] = a[u]; hist[2 * i + 1] = c[u]; }
        }
    }
    if (threadIdx.x == 0) lcnt = 0;
    __syncthreads();
    int64_t below;
    const int d1 = find_digit_4096(hist, oi.rank, &below, sbuf, tmp);
    if (s == 0 && threadIdx.x == 0) {
        int64_t m = oi.end - oi.beg;
        state[inst * 8 + kStFlag] = kFlagActive;
        state[inst * 8 + kStNeed] = oi.need;
        state[inst * 8 + kStD1] = d1;
        state[inst * 8 + kStR1] = oi.rank - below;
        state[inst * 8 + kStGtBin] = m - below - hist[d1];
    }
    int64_t lo = oi.beg + (int64_t)s * kOsSlice, hi = lo + kOsSlice;
    if (hi > oi.end) hi = oi.end;
    const float* row = scores + (int64_t)h * S + off;
    uint32_t* dst = cand + ((size_t)inst * SL + s) * kOsSlice;
    const int lane = threadIdx.x & 63;
    for_each_f32<kOsThreads, 4>(row, lo, hi, [&](int64_t, float v, bool ok) {
        const uint32_t k = order_key(v);
        const bool hit = ok && (int)(k >> 20) == d1;
        const uint64_t mask = __ballot(hit);
        if (mask) {
            uint32_t basep = 0;
            const int leader = __ffsll((unsigned long long)mask) - 1;
            if (lane == leader) basep = atomicAdd(&lcnt, (uint32_t)__popcll(mask));
            basep = __shfl(basep, leader, 64);
            if (hit) dst[basep + __popcll(mask & ((1ull << lane) - 1ull))] = k;
        }
    });
    __syncthreads();
    if (threadIdx.x == 0) cand_cnt[(size_t)inst * SL + s] = (lo < hi) ? lcnt : 0u;
}

// ----------------------------------------------------------------------- os_final
__global__ __launch_bounds__(kOsThreads) void os_final_kernel(int B, int Hq, int SL, const uint32_t* __restrict__ cand,
                                                             const uint32_t* __restrict__ cand_cnt,
                                                             int64_t* __restrict__ state, float* __restrict__ theta_out) {
    __shared__ uint32_t hist[4096];
    __shared__ int64_t sbuf[2];
    __shared__ int tmp[kOsThreads / 64];
    __shared__ uint32_t scnt[kOsMaxSL], spre[kOsMaxSL + 1];
    const int inst = blockIdx.x;
    int64_t* st = state + inst * 8;
    if (st[kStFlag] != kFlagActive) {
        if (theta_out && threadIdx.x == 0) theta_out[inst] = 0.f;
        return;
    }
    const uint32_t d1 = (uint32_t)st[kStD1];
    int64_t r = st[kStR1];
    int64_t gt = st[kStGtBin];
    // candidate counts of all slices, and their prefix, in LDS
    for (int k = threadIdx.x; k < SL; k += kOsThreads) scnt[k] = cand_cnt[(size_t)inst * SL + k];
    // digit 2: bits 19..8
    for (int i = threadIdx.x; i < 4096; i += kOsThreads) hist[i] = 0;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t acc = 0;
        for (int k = 0; k < SL; ++k) { spre[k] = acc; acc += scnt[k]; }
        spre[SL] = acc;
    }
    __syncthreads();
    const uint32_t total = spre[SL];
    const uint32_t* cbase = cand + (size_t)inst * SL * kOsSlice;
    auto cand_at = [&](uint32_t gi) {   // global candidate index -> key
        int lo2 = 0, hi2 = SL - 1;
        while (lo2 < hi2) {
            const int mid = (lo2 + hi2 + 1) >> 1;
            if (spre[mid] <= gi) lo2 = mid; else hi2 = mid - 1;
        }
        return cbase[(size_t)lo2 * kOsSlice + (gi - spre[lo2])];
    };
    for (uint32_t j0 = threadIdx.x; j0 < total; j0 += 8 * kOsThreads) {
        uint32_t key[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) key[u] = (j0 + u * kOsThreads < total) ? cand_at(j0 + u * kOsThreads) : 0u;
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (j0 + u * kOsThreads < total) atomicAdd(&hist[(key[u] >> 8) & 0xfffu], 1u);
    }
    __syncthreads();
    int64_t below;
    const int d2 = find_digit_4096(hist, r, &below, sbuf, tmp);
    {
        // candidates in digits above d2
        int64_t tot = 0;
        for (int i = threadIdx.x; i < 4096; i += kOsThreads)
            if (i > d2) tot += hist[i];
        int t32 = wave_sum_i((int)tot);
        if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = t32;
        __syncthreads();
        int64_t all = 0;
        for (int w = 0; w < kOsThreads / 64; ++w) all += tmp[w];
        gt += all;
        __syncthreads();
    }
    r -= below;
    // digit 3: bits 7..0 among keys with prefix (d1, d2)
    for (int i = threadIdx.x; i < 4096; i += kOsThreads) hist[i] = 0;
    __syncthreads();
    for (uint32_t j0 = threadIdx.x; j0 < total; j0 += 8 * kOsThreads) {
        uint32_t key[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) key[u] = (j0 + u * kOsThreads < total) ? cand_at(j0 + u * kOsThreads) : 0u;
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (j0 + u * kOsThreads < total && (int)((key[u] >> 8) & 0xfffu) == d2) atomicAdd(&hist[key[u] & 0xffu], 1u);
    }
    __syncthreads();
    const int d3 = find_digit_4096(hist, r, &below, sbuf, tmp);   // bins >= 256 are empty
    {
        int64_t tot = 0;
        for (int i = threadIdx.x; i < 256; i += kOsThreads)
            if (i > d3) tot += hist[i];
        int t32 = wave_sum_i((int)tot);
        if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = t32;
        __syncthreads();
        int64_t all = 0;
        for (int w = 0; w < kOsThreads / 64; ++w) all += tmp[w];
        gt += all;
    }
    if (threadIdx.x == 0) {
        uint32_t key = (d1 << 20) | ((uint32_t)d2 << 8) | (uint32_t)d3;
        st[kStKey] = key;
        st[kStGt] = gt;
        if (theta_out) theta_out[inst] = key_to_float(key);
    }
}

// ----------------------------------------------------------------- chunk lookup
__device__ __forceinline__ bool find_chunk(const int64_t* __restrict__ offsets, int B, int64_t item, int& b,
                                           int64_t& first, int64_t& nch, int64_t& t0, int64_t& len) {
    int64_t acc = 0;
    for (int i = 0; i < B; ++i) {
        int64_t n = offsets[i + 1] - offsets[i];
        int64_t nb = (n + kChunk - 1) / kChunk;
        if (item < acc + nb) {
            b = i;
            first = acc;
            nch = nb;
            t0 = (item - acc) * kChunk;
            len = n - t0 < kChunk ? n - t0 : kChunk;
            return true;
        }
        acc += nb;
    }
    return false;
}

__device__ __forceinline__ int64_t kpre_of(const int64_t* __restrict__ offsets, int b, const DevCfg& c) {
    int64_t k = 0;
    for (int i = 0; i < b; ++i) k += budget_k(offsets[i + 1] - offsets[i], c.bnum, c.bden, c.sink, c.local);
    return k;
}

// -------------------------------------------------------------------------- votes
// One thread per token (1024-token blocks).  Vote(t) = #{h : scores[h][t] > theta_h}
// (strict, IEEE compare so -0 == +0).  The key of a non-forced token is Vote + 1 if
// Vote >= v_min, else 0 (the listing's -1); forced tokens get 255.  Each block also counts
// the keys of its non-forced tokens (one histogram per block).
__global__ __launch_bounds__(kChunk) void vote_kernel(const float* __restrict__ scores,
                                                     const int64_t* __restrict__ offsets, int B, int Hq,
                                                     DevCfg cfg, int64_t S, const int64_t* __restrict__ state,
                                                     uint8_t* __restrict__ votes, uint8_t* __restrict__ keys,
                                                     uint32_t* __restrict__ hist) {
    __shared__ float th[64];
    __shared__ uint32_t lh[kChunk / 64][kVoteBins];
    int b;
    int64_t first, nch, t0, len;
    if (!find_chunk(offsets, B, blockIdx.x, b, first, nch, t0, len)) return;
    const int64_t off = offsets[b], n = offsets[b + 1] - off;
    for (int h = threadIdx.x; h < Hq; h += kChunk) th[h] = key_to_float((uint32_t)state[((int64_t)b * Hq + h) * 8 + kStKey]);
    for (int i = threadIdx.x; i < (kChunk / 64) * kVoteBins; i += kChunk) (&lh[0][0])[i] = 0;
    __syncthreads();
    const int64_t i = threadIdx.x;
    const int64_t t = t0 + i;
    if (i < len) {
        const float* col = scores + off + t;
        int v = 0;
        for (int h0 = 0; h0 < Hq; h0 += 16) {
            float sv[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) sv[u] = (h0 + u < Hq) ? col[(int64_t)(h0 + u) * S] : 0.f;
#pragma unroll
            for (int u = 0; u < 16; ++u) v += (h0 + u < Hq && sv[u] > th[h0 + u]) ? 1 : 0;
        }
        votes[off + t] = (uint8_t)v;
        uint8_t key;
        if (is_forced(t, n, cfg.sink, cfg.local)) key = 255;
        else {
            key = (uint8_t)(v >= cfg.vmin ? v + 1 : 0);
            atomicAdd(&lh[threadIdx.x >> 6][key], 1u);
        }
        keys[off + t] = key;
    }
    __syncthreads();
    for (int k = threadIdx.x; k < kVoteBins; k += kChunk) {
        uint32_t a = 0;
#pragma unroll
        for (int w = 0; w < kChunk / 64; ++w) a += lh[w][k];
        hist[(size_t)blockIdx.x * kVoteBins + k] = a;
    }
}

// Sums the key histograms of the blocks of sequence b into tot[] and those of the blocks
// before block c into bef[] (rows staged through LDS, 128 blocks at a time).
__device__ void sum_block_hists(const uint32_t* __restrict__ hist, int64_t first, int64_t nch, int64_t c,
                                uint32_t (*stage)[kVoteBins], uint32_t* tot, uint32_t* bef) {
    if (threadIdx.x < kVoteBins) { tot[threadIdx.x] = 0; bef[threadIdx.x] = 0; }
    for (int64_t k0 = 0; k0 < nch; k0 += 128) {
        const int64_t rows = nch - k0 < 128 ? nch - k0 : 128;
        __syncthreads();
        const int64_t ne = rows * kVoteBins;
        for (int64_t e0 = threadIdx.x; e0 < ne; e0 += 16 * (int64_t)blockDim.x) {
            uint32_t x[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int64_t e = e0 + (int64_t)u * blockDim.x;
                x[u] = e < ne ? hist[(size_t)(first + k0) * kVoteBins + e] : 0u;
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int64_t e = e0 + (int64_t)u * blockDim.x;
                if (e < ne) stage[e / kVoteBins][e % kVoteBins] = x[u];
            }
        }
        __syncthreads();
        if (threadIdx.x < kVoteBins) {
            uint32_t a = 0, p = 0;
            for (int64_t r = 0; r < rows; ++r) {
                const uint32_t x = stage[r][threadIdx.x];
                a += x;
                if (k0 + r < c) p += x;
            }
            tot[threadIdx.x] += a;
            bef[threadIdx.x] += p;
        }
    }
    __syncthreads();
}

// ------------------------------------------------------------ vote compaction
// One thread per token.  The boundary key v* is the largest key whose suffix count reaches
// need = K - |F|; every non-forced token above v*, the first (need - #above) tokens equal to
// v* in position order and every forced token are written, ascending, at their rank.
__global__ __launch_bounds__(kChunk) void compact_vote_kernel(const int64_t* __restrict__ offsets, int B,
                                                             DevCfg cfg, const uint8_t* __restrict__ keys,
                                                             const uint32_t* __restrict__ hist,
                                                             int32_t* __restrict__ idx_out,
                                                             int64_t* __restrict__ count_out) {
    __shared__ uint32_t stage[128][kVoteBins];
    __shared__ uint32_t tot[kVoteBins], bef[kVoteBins];
    __shared__ int64_t sh[4];
    __shared__ int tmp[kChunk / 64];
    int b;
    int64_t first, nch, t0, len;
    if (!find_chunk(offsets, B, blockIdx.x, b, first, nch, t0, len)) return;
    const int64_t off = offsets[b], n = offsets[b + 1] - off;
    const int64_t c = blockIdx.x - first;
    sum_block_hists(hist, first, nch, c, stage, tot, bef);
    const int64_t K = budget_k(n, cfg.bnum, cfg.bden, cfg.sink, cfg.local);
    const int64_t need = K - forced_before(n, n, cfg.sink, cfg.local);
    // suffix counts over the keys (thread t holds key kVoteBins - 1 - t); v* is the largest
    // key whose suffix count reaches `need` (none when need == 0)
    {
        const int t = threadIdx.x;
        const int v = kVoteBins - 1 - t;
        const int cnt = (t < kVoteBins) ? (int)tot[v] : 0;
        int all;
        const int incl = block_inclusive_scan<kChunk>(cnt, tmp, &all);
        if (t == 0) { sh[0] = kVoteBins; sh[1] = 0; }
        __syncthreads();
        if (need > 0 && t < kVoteBins && incl >= need && incl - cnt < need) { sh[0] = v; sh[1] = incl - cnt; }
        __syncthreads();
    }
    const int vs = (int)sh[0];
    const int64_t gt = sh[1];
    {
        const int t = threadIdx.x;
        const int x = (t < kVoteBins && t > vs) ? (int)bef[t] : 0;
        int gtb;
        block_inclusive_scan<kChunk>(x, tmp, &gtb);
        if (t == 0) {
            const int64_t eqb = vs < kVoteBins ? bef[vs] : 0;
            const int64_t need_eq = need - gt;
            sh[1] = need_eq;
            sh[2] = eqb;
            sh[3] = forced_before(t0, n, cfg.sink, cfg.local) + gtb + (eqb < need_eq ? eqb : need_eq);
            if (c == 0) count_out[b] = K;
        }
    }
    __syncthreads();
    const int64_t need_eq = sh[1], eqb = sh[2], base = sh[3];
    const int64_t i = threadIdx.x;
    const uint8_t kk = i < len ? keys[off + t0 + i] : 0;
    const int eqf = (i < len && kk != 255 && kk == vs) ? 1 : 0;
    int tot_eq;
    const int eq_rank = block_inclusive_scan<kChunk>(eqf, tmp, &tot_eq) - eqf;
    int sel = 0;
    if (i < len) {
        if (kk == 255) sel = 1;
        else if (vs < kVoteBins && kk > vs) sel = 1;
        else if (eqf) sel = (eqb + eq_rank < need_eq) ? 1 : 0;
    }
    int tot_sel;
    const int64_t p = base + block_inclusive_scan<kChunk>(sel, tmp, &tot_sel) - sel;
    const int64_t kpre = kpre_of(offsets, b, cfg);
    if (sel && p < K) idx_out[kpre + p] = (int32_t)(t0 + i);
}

// --------------------------------------------------------- per-head compaction
// cnt[(h * nitems + item) * 2 + {0: above, 1: equal}] for the non-forced tokens of a block.
__global__ __launch_bounds__(kChunk) void ph_count_kernel(const float* __restrict__ scores,
                                                         const int64_t* __restrict__ offsets, int B, int Hq,
                                                         DevCfg cfg, int64_t S, const int64_t* __restrict__ state,
                                                         int64_t nitems, uint32_t* __restrict__ cnt) {
    __shared__ int tmp[kChunk / 64];
    int b;
    int64_t first, nch, t0, len;
    if (!find_chunk(offsets, B, blockIdx.x, b, first, nch, t0, len)) return;
    const int h = blockIdx.y;
    const int64_t off = offsets[b], n = offsets[b + 1] - off;
    const int64_t* st = state + ((int64_t)b * Hq + h) * 8;
    const uint32_t ks = (uint32_t)st[kStKey];
    const bool act = st[kStFlag] == kFlagActive;
    const int64_t i = threadIdx.x, t = t0 + i;
    int gt = 0, eq = 0;
    if (act && i < len && !is_forced(t, n, cfg.sink, cfg.local)) {
        const uint32_t k = order_key(scores[(int64_t)h * S + off + t]);
        gt = k > ks;
        eq = k == ks;
    }
    int tg, te;
    block_inclusive_scan<kChunk>(gt, tmp, &tg);
    block_inclusive_scan<kChunk>(eq, tmp, &te);
    if (threadIdx.x == 0) {
        cnt[((size_t)h * nitems + blockIdx.x) * 2 + 0] = (uint32_t)tg;
        cnt[((size_t)h * nitems + blockIdx.x) * 2 + 1] = (uint32_t)te;
    }
}

__global__ __launch_bounds__(kChunk) void ph_compact_kernel(const float* __restrict__ scores,
                                                           const int64_t* __restrict__ offsets, int B, int Hq,
                                                           DevCfg cfg, int64_t S, const int64_t* __restrict__ state,
                                                           int64_t nitems, const uint32_t* __restrict__ cnt,
                                                           int32_t* __restrict__ idx_out,
                                                           int64_t* __restrict__ count_out) {
    __shared__ int tmp[kChunk / 64];
    int b;
    int64_t first, nch, t0, len;
    if (!find_chunk(offsets, B, blockIdx.x, b, first, nch, t0, len)) return;
    const int h = blockIdx.y;
    const int64_t off = offsets[b], n = offsets[b + 1] - off;
    const int64_t c = blockIdx.x - first;
    const int64_t* st = state + ((int64_t)b * Hq + h) * 8;
    const int64_t flag = st[kStFlag];
    const uint32_t ks = (uint32_t)st[kStKey];
    const int64_t K = budget_k(n, cfg.bnum, cfg.bden, cfg.sink, cfg.local);
    const int64_t need_eq = flag == kFlagActive ? st[kStNeed] - st[kStGt] : 0;
    // counts of the blocks before this one (one block per thread, then a block sum)
    int gtb_i = 0, eqb_i = 0;
    for (int64_t k = threadIdx.x; k < c; k += kChunk) {
        gtb_i += (int)cnt[((size_t)h * nitems + first + k) * 2 + 0];
        eqb_i += (int)cnt[((size_t)h * nitems + first + k) * 2 + 1];
    }
    int gtb, eqb;
    block_inclusive_scan<kChunk>(gtb_i, tmp, &gtb);
    block_inclusive_scan<kChunk>(eqb_i, tmp, &eqb);
    const int64_t fb = forced_before(t0, n, cfg.sink, cfg.local);
    int64_t base;
    if (flag == kFlagTakeAll) base = t0;
    else if (flag == kFlagTakeNone) base = fb;
    else base = fb + gtb + ((int64_t)eqb < need_eq ? (int64_t)eqb : need_eq);
    if (c == 0 && h == 0 && threadIdx.x == 0) count_out[b] = K;

    const int64_t i = threadIdx.x, t = t0 + i;
    const bool in = i < len;
    const bool f = in && is_forced(t, n, cfg.sink, cfg.local);
    const uint32_t kk = (in && !f) ? order_key(scores[(int64_t)h * S + off + t]) : 0u;
    const int eqf = (in && !f && flag == kFlagActive && kk == ks) ? 1 : 0;
    int tot;
    const int eq_rank = block_inclusive_scan<kChunk>(eqf, tmp, &tot) - eqf;
    int sel = in ? (f ? 1 : (flag == kFlagTakeAll ? 1 : (flag == kFlagActive && kk > ks ? 1 : 0))) : 0;
    if (eqf) sel = ((int64_t)eqb + eq_rank < need_eq) ? 1 : 0;
    const int64_t p = base + block_inclusive_scan<kChunk>(sel, tmp, &tot) - sel;
    const int64_t kpre = kpre_of(offsets, b, cfg);
    if (sel && p < K) idx_out[Hq * kpre + (int64_t)h * K + p] = (int32_t)t;
}

// ------------------------------------------------------------------- host side
static DevCfg dev_cfg(const SelectConfig& c) {
    DevCfg d;
    d.mode = c.mode;
    d.bnum = c.bnum;
    d.bden = c.bden;
    d.sink = c.sink;
    d.local = c.local;
    d.vmin = c.vmin;
    d.tnum = c.tnum;
    d.tden = c.tden;
    return d;
}

struct SelectLayout {
    int SL;
    int64_t nitems, Ntot;
    uint32_t *part1, *cand, *cand_cnt, *hist, *phcnt;
    int64_t* state;
    uint8_t *votes, *keys;
    size_t bytes;
};

static SelectLayout select_layout(void* ws, const int64_t* offsets_host, int B, int Hq, const SelectConfig& c) {
    SelectLayout L;
    DevCfg d = dev_cfg(c);
    int64_t maxm = 0, items = 0;
    for (int b = 0; b < B; ++b) {
        int64_t n = offsets_host[b + 1] - offsets_host[b];
        OsInst o = os_instance(n, d);
        if (o.end - o.beg > maxm) maxm = o.end - o.beg;
        items += (n + kChunk - 1) / kChunk;
    }
    L.SL = (int)((maxm + kOsSlice - 1) / kOsSlice);
    if (L.SL < 1) L.SL = 1;
    L.nitems = items;
    L.Ntot = offsets_host[B];
    WsCarver w(ws);
    const size_t inst = (size_t)B * Hq;
    L.part1 = w.take<uint32_t>(inst * L.SL * 2048);
    L.cand = w.take<uint32_t>(inst * L.SL * kOsSlice);
    L.cand_cnt = w.take<uint32_t>(inst * L.SL);
    L.state = w.take<int64_t>(inst * 8);
    L.votes = w.take<uint8_t>((size_t)L.Ntot + 16);
    L.keys = w.take<uint8_t>((size_t)L.Ntot + 16);
    L.hist = w.take<uint32_t>((size_t)items * kVoteBins);
    L.phcnt = c.mode == 1 ? w.take<uint32_t>((size_t)Hq * items * 2) : nullptr;
    L.bytes = w.size();
    return L;
}

size_t select_workspace(const int64_t* offsets_host, int B, int Hq, const SelectConfig& c) {
    return select_layout(nullptr, offsets_host, B, Hq, c).bytes;
}

hipError_t launch_select(const float* scores, int64_t S, const int64_t* offsets_dev, const int64_t* offsets_host,
                         int B, int Hq, const SelectConfig& c, int32_t* idx_out, int64_t* count_out, float* theta_out,
                         uint8_t* votes_out, void* ws, size_t ws_bytes, hipStream_t stream) {
    SelectLayout L = select_layout(ws, offsets_host, B, Hq, c);
    if (L.bytes > ws_bytes) return hipErrorInvalidValue;
    DevCfg d = dev_cfg(c);
    const unsigned inst = (unsigned)(B * Hq);
    hipLaunchKernelGGL(os_hist_kernel, dim3(L.SL, inst), dim3(kOsThreads), 0, stream, scores, offsets_dev, B, Hq, d,
                       L.SL, S, L.part1);
    hipLaunchKernelGGL(os_collect_kernel, dim3(L.SL, inst), dim3(kOsThreads), 0, stream, scores, offsets_dev, B, Hq, d,
                       L.SL, S, L.part1, L.cand, L.cand_cnt, L.state);
    hipLaunchKernelGGL(os_final_kernel, dim3(inst), dim3(kOsThreads), 0, stream, B, Hq, L.SL, L.cand, L.cand_cnt,
                       L.state, c.mode == 0 ? theta_out : nullptr);
    if (L.nitems == 0) return hipGetLastError();
    if (c.mode == 0) {
        uint8_t* votes = votes_out ? votes_out : L.votes;
        hipLaunchKernelGGL(vote_kernel, dim3((unsigned)L.nitems), dim3(kChunk), 0, stream, scores, offsets_dev,
                           B, Hq, d, S, L.state, votes, L.keys, L.hist);
        hipLaunchKernelGGL(compact_vote_kernel, dim3((unsigned)L.nitems), dim3(kChunk), 0, stream, offsets_dev,
                           B, d, L.keys, L.hist, idx_out, count_out);
    } else {
        hipLaunchKernelGGL(ph_count_kernel, dim3((unsigned)L.nitems, Hq), dim3(kChunk), 0, stream, scores,
                           offsets_dev, B, Hq, d, S, L.state, L.nitems, L.phcnt);
        hipLaunchKernelGGL(ph_compact_kernel, dim3((unsigned)L.nitems, Hq), dim3(kChunk), 0, stream, scores,
                           offsets_dev, B, Hq, d, S, L.state, L.nitems, L.phcnt, idx_out, count_out);
    }
    return hipGetLastError();
}

// ------------------------------------------------------------- row-wise top-k
__global__ void set_offsets_kernel(int64_t* o, int64_t n) {
    if (threadIdx.x == 0) { o[0] = 0; o[1] = n; }
}

static SelectConfig rows_cfg(int64_t n, int64_t k) {
    SelectConfig c;
    c.mode = 1;
    c.bnum = k;
    c.bden = n > 0 ? n : 1;
    c.sink = 0;
    c.local = 0;
    c.vmin = 0;
    c.tnum = 1;
    c.tden = 1;
    return c;
}

size_t rows_topk_workspace(int rows, int64_t n, int64_t k) {
    int64_t oh[2] = {0, n};
    WsCarver w(nullptr);
    w.take<int64_t>(4);
    w.take<int64_t>(4);
    w.take<char>(select_workspace(oh, 1, rows, rows_cfg(n, k)));
    return w.size();
}

hipError_t launch_rows_topk(const float* vals, int64_t stride, int rows, int64_t n, int64_t k, int32_t* idx_out,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
    if (rows_topk_workspace(rows, n, k) > ws_bytes) return hipErrorInvalidValue;
    int64_t oh[2] = {0, n};
    SelectConfig c = rows_cfg(n, k);
    WsCarver w(ws);
    int64_t* od = w.take<int64_t>(4);
    int64_t* cnt = w.take<int64_t>(4);
    size_t sb = select_workspace(oh, 1, rows, c);
    void* sws = w.take<char>(sb);
    hipLaunchKernelGGL(set_offsets_kernel, dim3(1), dim3(64), 0, stream, od, n);
    return launch_select(vals, stride, od, oh, 1, rows, c, idx_out, cnt, nullptr, nullptr, sws, sb, stream);
}

}  // namespace qasi
