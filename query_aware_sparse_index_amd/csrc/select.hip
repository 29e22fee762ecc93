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
constexpr int kOsThreads = 256;
constexpr int kChunk = 1024;        // tokens per vote / compaction block
constexpr int kChunkThreads = 256;
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
                                                            DevCfg cfg, int SL, uint32_t* __restrict__ part1) {
    // 4 per-wave sub-histograms, two 16-bit bins per word
    __shared__ uint32_t sub[4][2048];
    const int inst = blockIdx.y, s = blockIdx.x;
    const int b = inst / Hq, h = inst % Hq;
    const int64_t off = offsets[b];
    OsInst oi = os_instance(offsets[b + 1] - off, cfg);
    for (int i = threadIdx.x; i < 4 * 2048; i += kOsThreads) (&sub[0][0])[i] = 0;
    __syncthreads();
    const int64_t Ntot = offsets[B];
    int64_t lo = oi.beg + (int64_t)s * kOsSlice, hi = lo + kOsSlice;
    if (hi > oi.end) hi = oi.end;
    const bool act = oi.flag == kFlagActive && lo < hi;
    if (act) {
        const float* row = scores + (int64_t)h * Ntot + off;
        uint32_t* mine = sub[threadIdx.x >> 6];
        for (int64_t t = lo + threadIdx.x; t < hi; t += kOsThreads) {
            uint32_t d = order_key(row[t]) >> 20;
            atomicAdd(&mine[d >> 1], (d & 1) ? 0x10000u : 1u);
        }
    }
    __syncthreads();
    uint32_t* dst = part1 + ((size_t)inst * SL + s) * 2048;
    for (int i = threadIdx.x; i < 2048; i += kOsThreads) dst[i] = act ? (sub[0][i] + sub[1][i] + sub[2][i] + sub[3][i]) : 0u;
}

// Finds the digit whose cumulative count (ascending) first reaches `rank` in the 4096-bin
// LDS histogram `hist`.  Returns the digit; *below = count of keys in smaller digits.
__device__ int find_digit_4096(const uint32_t* hist, int64_t rank, int64_t* below, int64_t* sbuf, int* tmp) {
    // each thread owns 16 consecutive bins
    const int tid = threadIdx.x;
    if (tid == 0) { sbuf[0] = 0; sbuf[1] = 0; }
    __syncthreads();
    int64_t local = 0;
    for (int i = 0; i < 16; ++i) local += hist[tid * 16 + i];
    // inclusive scan of 64-bit locals through the int scan (counts fit in 31 bits here)
    int total;
    int inc = block_inclusive_scan<kOsThreads>((int)local, tmp, &total);
    int64_t excl = inc - local;
    if (excl < rank && rank <= inc) {
        int64_t c = excl;
        for (int i = 0; i < 16; ++i) {
            int64_t nc = c + hist[tid * 16 + i];
            if (rank <= nc) { sbuf[0] = tid * 16 + i; sbuf[1] = c; break; }
            c = nc;
        }
    }
    __syncthreads();
    int d = (int)sbuf[0];
    *below = sbuf[1];
    __syncthreads();
    return d;
}

// --------------------------------------------------------------------- os_collect
__global__ __launch_bounds__(kOsThreads) void os_collect_kernel(const float* __restrict__ scores,
                                                               const int64_t* __restrict__ offsets, int B, int Hq,
                                                               DevCfg cfg, int SL, const uint32_t* __restrict__ part1,
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
    for (int i = threadIdx.x; i < 2048; i += kOsThreads) {
        uint32_t a = 0, c = 0;
        for (int k = 0; k < SL; ++k) {
            uint32_t w = part1[((size_t)inst * SL + k) * 2048 + i];
            a += w & 0xffffu;
            c += w >> 16;
        }
        hist[2 * i] = a;
        hist[2 * i + 1] = c;
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
    const int64_t Ntot = offsets[B];
    int64_t lo = oi.beg + (int64_t)s * kOsSlice, hi = lo + kOsSlice;
    if (hi > oi.end) hi = oi.end;
    const float* row = scores + (int64_t)h * Ntot + off;
    uint32_t* dst = cand + ((size_t)inst * SL + s) * kOsSlice;
    for (int64_t t = lo + threadIdx.x; t < hi; t += kOsThreads) {
        uint32_t k = order_key(row[t]);
        if ((int)(k >> 20) == d1) {
            uint32_t p = atomicAdd(&lcnt, 1u);
            dst[p] = k;
        }
    }
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
    const int inst = blockIdx.x;
    int64_t* st = state + inst * 8;
    if (st[kStFlag] != kFlagActive) {
        if (theta_out && threadIdx.x == 0) theta_out[inst] = 0.f;
        return;
    }
    const uint32_t d1 = (uint32_t)st[kStD1];
    int64_t r = st[kStR1];
    int64_t gt = st[kStGtBin];
    // digit 2: bits 19..8
    for (int i = threadIdx.x; i < 4096; i += kOsThreads) hist[i] = 0;
    __syncthreads();
    for (int k = 0; k < SL; ++k) {
        const uint32_t* src = cand + ((size_t)inst * SL + k) * kOsSlice;
        uint32_t cnt = cand_cnt[(size_t)inst * SL + k];
        for (uint32_t j = threadIdx.x; j < cnt; j += kOsThreads) atomicAdd(&hist[(src[j] >> 8) & 0xfffu], 1u);
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
    for (int k = 0; k < SL; ++k) {
        const uint32_t* src = cand + ((size_t)inst * SL + k) * kOsSlice;
        uint32_t cnt = cand_cnt[(size_t)inst * SL + k];
        for (uint32_t j = threadIdx.x; j < cnt; j += kOsThreads) {
            uint32_t key = src[j];
            if ((int)((key >> 8) & 0xfffu) == d2) atomicAdd(&hist[key & 0xffu], 1u);
        }
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
// Vote(t) = #{h : scores[h][t] > theta_h} (strict, IEEE compare so -0 == +0); the key of a
// non-forced token is Vote + 1 if Vote >= v_min, else 0 (the listing's -1); forced tokens
// get 255.  Each block also counts the keys of its non-forced tokens.
__global__ __launch_bounds__(kChunkThreads) void vote_kernel(const float* __restrict__ scores,
                                                            const int64_t* __restrict__ offsets, int B, int Hq,
                                                            DevCfg cfg, const int64_t* __restrict__ state,
                                                            uint8_t* __restrict__ votes, uint8_t* __restrict__ keys,
                                                            uint32_t* __restrict__ hist) {
    __shared__ float th[64];
    __shared__ uint32_t lh[kVoteBins];
    int b;
    int64_t first, nch, t0, len;
    if (!find_chunk(offsets, B, blockIdx.x, b, first, nch, t0, len)) return;
    const int64_t off = offsets[b], n = offsets[b + 1] - off, Ntot = offsets[B];
    for (int h = threadIdx.x; h < Hq; h += kChunkThreads) th[h] = key_to_float((uint32_t)state[((int64_t)b * Hq + h) * 8 + kStKey]);
    for (int i = threadIdx.x; i < kVoteBins; i += kChunkThreads) lh[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < len; i += kChunkThreads) {
        int64_t t = t0 + i;
        int v = 0;
        for (int h = 0; h < Hq; ++h) v += scores[(int64_t)h * Ntot + off + t] > th[h] ? 1 : 0;
        votes[off + t] = (uint8_t)v;
        uint8_t key;
        if (is_forced(t, n, cfg.sink, cfg.local)) key = 255;
        else {
            key = (uint8_t)(v >= cfg.vmin ? v + 1 : 0);
            atomicAdd(&lh[key], 1u);
        }
        keys[off + t] = key;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kVoteBins; i += kChunkThreads) hist[(size_t)blockIdx.x * kVoteBins + i] = lh[i];
}

// ------------------------------------------------------------ vote compaction
__global__ __launch_bounds__(kChunkThreads) void compact_vote_kernel(const int64_t* __restrict__ offsets, int B,
                                                                    DevCfg cfg, const uint8_t* __restrict__ keys,
                                                                    const uint32_t* __restrict__ hist,
                                                                    int32_t* __restrict__ idx_out,
                                                                    int64_t* __restrict__ count_out) {
    __shared__ uint32_t tot[kVoteBins], bef[kVoteBins];
    __shared__ int64_t sh[4];
    __shared__ int tmp[kChunkThreads / 64];
    int b;
    int64_t first, nch, t0, len;
    if (!find_chunk(offsets, B, blockIdx.x, b, first, nch, t0, len)) return;
    const int64_t off = offsets[b], n = offsets[b + 1] - off;
    const int64_t c = blockIdx.x - first;
    for (int v = threadIdx.x; v < kVoteBins; v += kChunkThreads) {
        uint32_t a = 0, p = 0;
        for (int64_t k = 0; k < nch; ++k) {
            uint32_t x = hist[(size_t)(first + k) * kVoteBins + v];
            a += x;
            if (k < c) p += x;
        }
        tot[v] = a;
        bef[v] = p;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const int64_t K = budget_k(n, cfg.bnum, cfg.bden, cfg.sink, cfg.local);
        const int64_t fb = forced_before(n, n, cfg.sink, cfg.local);
        const int64_t need = K - fb;
        int vs = kVoteBins;   // no non-forced token is taken when need == 0
        int64_t gt = 0;
        if (need > 0) {
            int64_t cum = 0;
            for (int v = kVoteBins - 1; v >= 0; --v) {
                if (cum + tot[v] >= need) { vs = v; break; }
                cum += tot[v];
            }
            gt = cum;
        }
        int64_t gtb = 0;
        for (int v = vs + 1; v < kVoteBins; ++v) gtb += bef[v];
        int64_t eqb = vs < kVoteBins ? bef[vs] : 0;
        int64_t need_eq = need - gt;
        sh[0] = vs;
        sh[1] = need_eq;
        sh[2] = eqb;
        sh[3] = forced_before(t0, n, cfg.sink, cfg.local) + gtb + (eqb < need_eq ? eqb : need_eq);
        if (c == 0) count_out[b] = K;
    }
    __syncthreads();
    const int vs = (int)sh[0];
    const int64_t need_eq = sh[1], eqb = sh[2], base = sh[3];
    const int64_t kpre = kpre_of(offsets, b, cfg);
    // each thread owns 4 consecutive tokens of the chunk
    uint8_t kk[4];
    int eqf[4];
    int neq = 0;
    for (int j = 0; j < 4; ++j) {
        int64_t i = (int64_t)threadIdx.x * 4 + j;
        kk[j] = i < len ? keys[off + t0 + i] : 0;
        eqf[j] = (i < len && kk[j] != 255 && kk[j] == vs) ? 1 : 0;
        neq += eqf[j];
    }
    int tot_eq;
    int eq_inc = block_inclusive_scan<kChunkThreads>(neq, tmp, &tot_eq);
    int eq_rank = eq_inc - neq;
    int self[4];
    int nsel = 0;
    for (int j = 0; j < 4; ++j) {
        int64_t i = (int64_t)threadIdx.x * 4 + j;
        int s = 0;
        if (i < len) {
            if (kk[j] == 255) s = 1;
            else if (kk[j] > vs && vs < kVoteBins) s = 1;
            else if (eqf[j]) { s = (eqb + eq_rank < need_eq) ? 1 : 0; ++eq_rank; }
        }
        self[j] = s;
        nsel += s;
    }
    int tot_sel;
    int sel_inc = block_inclusive_scan<kChunkThreads>(nsel, tmp, &tot_sel);
    int64_t p = base + sel_inc - nsel;
    const int64_t K = budget_k(n, cfg.bnum, cfg.bden, cfg.sink, cfg.local);
    for (int j = 0; j < 4; ++j) {
        if (self[j] && p < K) idx_out[kpre + p] = (int32_t)(t0 + (int64_t)threadIdx.x * 4 + j);
        p += self[j];
    }
}

// --------------------------------------------------------- per-head compaction
// cnt[(h * nitems + item) * 2 + {0: above, 1: equal}] for the non-forced tokens of a chunk.
__global__ __launch_bounds__(kChunkThreads) void ph_count_kernel(const float* __restrict__ scores,
                                                                const int64_t* __restrict__ offsets, int B, int Hq,
                                                                DevCfg cfg, const int64_t* __restrict__ state,
                                                                int64_t nitems, uint32_t* __restrict__ cnt) {
    __shared__ int tmp[kChunkThreads / 64];
    int b;
    int64_t first, nch, t0, len;
    if (!find_chunk(offsets, B, blockIdx.x, b, first, nch, t0, len)) return;
    const int h = blockIdx.y;
    const int64_t off = offsets[b], n = offsets[b + 1] - off, Ntot = offsets[B];
    const int64_t* st = state + ((int64_t)b * Hq + h) * 8;
    const uint32_t ks = (uint32_t)st[kStKey];
    const bool act = st[kStFlag] == kFlagActive;
    int gt = 0, eq = 0;
    if (act) {
        for (int64_t i = threadIdx.x; i < len; i += kChunkThreads) {
            int64_t t = t0 + i;
            if (is_forced(t, n, cfg.sink, cfg.local)) continue;
            uint32_t k = order_key(scores[(int64_t)h * Ntot + off + t]);
            gt += k > ks;
            eq += k == ks;
        }
    }
    int tg, te;
    block_inclusive_scan<kChunkThreads>(gt, tmp, &tg);
    block_inclusive_scan<kChunkThreads>(eq, tmp, &te);
    if (threadIdx.x == 0) {
        cnt[((size_t)h * nitems + blockIdx.x) * 2 + 0] = (uint32_t)tg;
        cnt[((size_t)h * nitems + blockIdx.x) * 2 + 1] = (uint32_t)te;
    }
}

__global__ __launch_bounds__(kChunkThreads) void ph_compact_kernel(const float* __restrict__ scores,
                                                                  const int64_t* __restrict__ offsets, int B, int Hq,
                                                                  DevCfg cfg, const int64_t* __restrict__ state,
                                                                  int64_t nitems, const uint32_t* __restrict__ cnt,
                                                                  int32_t* __restrict__ idx_out,
                                                                  int64_t* __restrict__ count_out) {
    __shared__ int64_t sh[2];
    __shared__ int tmp[kChunkThreads / 64];
    int b;
    int64_t first, nch, t0, len;
    if (!find_chunk(offsets, B, blockIdx.x, b, first, nch, t0, len)) return;
    const int h = blockIdx.y;
    const int64_t off = offsets[b], n = offsets[b + 1] - off, Ntot = offsets[B];
    const int64_t c = blockIdx.x - first;
    const int64_t* st = state + ((int64_t)b * Hq + h) * 8;
    const int64_t flag = st[kStFlag];
    const uint32_t ks = (uint32_t)st[kStKey];
    const int64_t K = budget_k(n, cfg.bnum, cfg.bden, cfg.sink, cfg.local);
    const int64_t need_eq = flag == kFlagActive ? st[kStNeed] - st[kStGt] : 0;
    if (threadIdx.x == 0) {
        int64_t gtb = 0, eqb = 0;
        for (int64_t k = 0; k < c; ++k) {
            gtb += cnt[((size_t)h * nitems + first + k) * 2 + 0];
            eqb += cnt[((size_t)h * nitems + first + k) * 2 + 1];
        }
        int64_t fb = forced_before(t0, n, cfg.sink, cfg.local);
        int64_t base;
        if (flag == kFlagTakeAll) base = t0;
        else if (flag == kFlagTakeNone) base = fb;
        else base = fb + gtb + (eqb < need_eq ? eqb : need_eq);
        sh[0] = base;
        sh[1] = eqb;
        if (c == 0 && h == 0) count_out[b] = K;
    }
    __syncthreads();
    const int64_t base = sh[0], eqb = sh[1];
    int sel[4], eqf[4];
    uint32_t kk[4];
    int neq = 0;
    for (int j = 0; j < 4; ++j) {
        int64_t i = (int64_t)threadIdx.x * 4 + j;
        int64_t t = t0 + i;
        bool in = i < len;
        bool f = in && is_forced(t, n, cfg.sink, cfg.local);
        kk[j] = (in && !f) ? order_key(scores[(int64_t)h * Ntot + off + t]) : 0u;
        eqf[j] = (in && !f && flag == kFlagActive && kk[j] == ks) ? 1 : 0;
        neq += eqf[j];
        sel[j] = in ? (f ? 1 : (flag == kFlagTakeAll ? 1 : (flag == kFlagActive && kk[j] > ks ? 1 : 0))) : 0;
    }
    int tot;
    int eq_inc = block_inclusive_scan<kChunkThreads>(neq, tmp, &tot);
    int eq_rank = eq_inc - neq;
    int nsel = 0;
    for (int j = 0; j < 4; ++j) {
        if (eqf[j]) { sel[j] = (eqb + eq_rank < need_eq) ? 1 : 0; ++eq_rank; }
        nsel += sel[j];
    }
    int sel_inc = block_inclusive_scan<kChunkThreads>(nsel, tmp, &tot);
    int64_t p = base + sel_inc - nsel;
    const int64_t kpre = kpre_of(offsets, b, cfg);
    int32_t* dst = idx_out + Hq * kpre + (int64_t)h * K;
    for (int j = 0; j < 4; ++j) {
        if (sel[j] && p < K) dst[p] = (int32_t)(t0 + (int64_t)threadIdx.x * 4 + j);
        p += sel[j];
    }
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

hipError_t launch_select(const float* scores, const int64_t* offsets_dev, const int64_t* offsets_host, int B, int Hq,
                         const SelectConfig& c, int32_t* idx_out, int64_t* count_out, float* theta_out,
                         uint8_t* votes_out, void* ws, size_t ws_bytes, hipStream_t stream) {
    SelectLayout L = select_layout(ws, offsets_host, B, Hq, c);
    if (L.bytes > ws_bytes) return hipErrorInvalidValue;
    DevCfg d = dev_cfg(c);
    const unsigned inst = (unsigned)(B * Hq);
    hipLaunchKernelGGL(os_hist_kernel, dim3(L.SL, inst), dim3(kOsThreads), 0, stream, scores, offsets_dev, B, Hq, d,
                       L.SL, L.part1);
    hipLaunchKernelGGL(os_collect_kernel, dim3(L.SL, inst), dim3(kOsThreads), 0, stream, scores, offsets_dev, B, Hq, d,
                       L.SL, L.part1, L.cand, L.cand_cnt, L.state);
    hipLaunchKernelGGL(os_final_kernel, dim3(inst), dim3(kOsThreads), 0, stream, B, Hq, L.SL, L.cand, L.cand_cnt,
                       L.state, c.mode == 0 ? theta_out : nullptr);
    if (L.nitems == 0) return hipGetLastError();
    if (c.mode == 0) {
        uint8_t* votes = votes_out ? votes_out : L.votes;
        hipLaunchKernelGGL(vote_kernel, dim3((unsigned)L.nitems), dim3(kChunkThreads), 0, stream, scores, offsets_dev,
                           B, Hq, d, L.state, votes, L.keys, L.hist);
        hipLaunchKernelGGL(compact_vote_kernel, dim3((unsigned)L.nitems), dim3(kChunkThreads), 0, stream, offsets_dev,
                           B, d, L.keys, L.hist, idx_out, count_out);
    } else {
        hipLaunchKernelGGL(ph_count_kernel, dim3((unsigned)L.nitems, Hq), dim3(kChunkThreads), 0, stream, scores,
                           offsets_dev, B, Hq, d, L.state, L.nitems, L.phcnt);
        hipLaunchKernelGGL(ph_compact_kernel, dim3((unsigned)L.nitems, Hq), dim3(kChunkThreads), 0, stream, scores,
                           offsets_dev, B, Hq, d, L.state, L.nitems, L.phcnt, idx_out, count_out);
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

hipError_t launch_rows_topk(const float* vals, int rows, int64_t n, int64_t k, int32_t* idx_out, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
    if (rows_topk_workspace(rows, n, k) > ws_bytes) return hipErrorInvalidValue;
    int64_t oh[2] = {0, n};
    SelectConfig c = rows_cfg(n, k);
    WsCarver w(ws);
    int64_t* od = w.take<int64_t>(4);
    int64_t* cnt = w.take<int64_t>(4);
    size_t sb = select_workspace(oh, 1, rows, c);
    void* sws = w.take<char>(sb);
    hipLaunchKernelGGL(set_offsets_kernel, dim3(1), dim3(64), 0, stream, od, n);
    return launch_select(vals, od, oh, 1, rows, c, idx_out, cnt, nullptr, nullptr, sws, sb, stream);
}

}  // namespace qasi
