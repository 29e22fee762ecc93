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
// vote, and the boundary score of the per-head top-K.  It is found on order-preserving
// uint32 keys of the fp32 scores in two kernels:
//   th_collect : every block of an instance derives the same key bracket [lo, hi] from a
//                stratified sample of the row (kRuns runs of 16 keys): a histogram over the
//                sample's value range locates the sample order statistics kDelta ranks below
//                and above the target's expected sample rank.  Then, per slice of the row, it
//                counts the keys below lo, compacts the keys inside the bracket (the
//                "candidates") next to the slice grouped by their top kDigit bits of key - lo;
//   th_final   : sums the slice histograms to find the answer's top digit, gathers the
//                candidates of that digit into LDS and finishes with a radix select over
//                the remaining bits.  If the answer's rank is not among the candidates (or
//                its digit holds more than kCap of them) the block runs the radix select
//                over the whole row instead.  The result is exact either way; the sample
//                only decides how much work it takes.
// Ties resolve to the lowest position in the compaction kernels, which take every token
// above the boundary and the first `need_eq` tokens equal to it in position order.
#include "qasi_device.h"
#include "qasi_internal.h"

namespace qasi {

constexpr int kThThreads = 1024;   // final blocks
constexpr int kRuns = 128, kRunLen = 16;
constexpr int kSample = kRuns * kRunLen;   // sampled keys per instance
constexpr int kSampleBins = 2048;
constexpr int kDelta = 96;         // bracket half-width in sample ranks
constexpr int kDigit = 11;         // radix digit width of the final select
constexpr int kDigitBins = 1 << kDigit;
constexpr int kCap = 16384;        // keys of the answer's top digit resolved in LDS
constexpr int kSlice = 8192;       // keys per collect block
constexpr int kColThreads = 512;
constexpr int kMaxSL = 2048;       // slices per instance (n up to 2^24 tokens)
constexpr int kChunk = 1024;       // tokens per vote / compaction block
constexpr int kVoteBins = 72;      // vote keys 0 .. Hq + 1 (Hq <= 64)

enum : int64_t { kFlagActive = 0, kFlagTakeNone = 1, kFlagTakeAll = 2 };


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

// ---------------------------------------------------------------------- th_collect
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

// Shift that leaves the top kDigit bits of a key offset below 2^nbits.
__host__ __device__ __forceinline__ int top_shift(uint32_t span) {
    int nbits = 0;
    while (nbits < 32 && (span >> nbits) != 0u) ++nbits;
    return nbits > kDigit ? nbits - kDigit : 0;
}

// Position (relative to the range start) of sample i of an instance over a range of m keys,
// for a sample of `runs` runs of kRunLen keys: run j = i / kRunLen starts at a hashed position of
// stratum [j m / runs, (j + 1) m / runs), so the runs cover the whole range.  Needs
// m >= runs * kRunLen.
__device__ __forceinline__ int64_t sample_pos(int i, int64_t m, int inst, int runs) {
    const int j = i / kRunLen;
    const int64_t a = (int64_t)j * m / runs, e = (int64_t)(j + 1) * m / runs;
    const uint32_t r = mix32((uint32_t)j * 0x9e3779b9u ^ mix32((uint32_t)inst + 0x632be5abu));
    return a + (int64_t)(r % (uint32_t)(e - a - kRunLen + 1)) + (i % kRunLen);
}

template <int NS, int DELTA, bool KEYBINS = false>
__device__ void bracket_of_sample(const float (&v)[NS / kColThreads], const OsInst& oi, uint32_t* hist,
                                  float* wmin, float* wmax, int* tmp, int* sb, uint32_t& klo, uint32_t& khi);

// Key bracket [lo, hi] of an instance whose row (m keys) is longer than kCap, from the sampled
// scores of the row; every thread of the block calls it and every block of the instance computes
// the same result.
__device__ void sample_bracket(const float* __restrict__ row, const OsInst& oi, int inst, uint32_t* hist,
                               float* wmin, float* wmax, int* tmp, int* sb, uint32_t& klo, uint32_t& khi) {
    constexpr int PER = kSample / kColThreads;
    const int64_t m = oi.end - oi.beg;
    float v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) v[u] = row[oi.beg + sample_pos(threadIdx.x + u * kColThreads, m, inst, kRuns)];
    bracket_of_sample<kSample, kDelta>(v, oi, hist, wmin, wmax, tmp, sb, klo, khi);
}

// The bracket [klo, khi] from the NS sample values v (PER per thread): the sample's [min, max]
// is cut into kSampleBins equal bins; lo is the lower edge of the bin before the one holding
// sample rank ir - DELTA and hi the upper edge of the bin after the one holding ir + DELTA (the
// key range's ends when these leave the sample), ir the target's expected sample rank.  Every
// thread of the block calls it; `hist` (kSampleBins words) is left dirty.
// The sample's ranks il, ih = ir -+ DELTA around the target rank ir are located in kSampleBins
// bins of the sample range: equal-width value bins, or (KEYBINS) equal-width bins of the order
// keys, which spread heavy-tailed positive values (such as mean attention probabilities) over
// their octaves.  With KEYBINS an upper rank past the sample keeps the bin of the sample's maximum
// (keys above the bracket are counted, not ranked).
template <int NS, int DELTA, bool KEYBINS>
__device__ void bracket_of_sample(const float (&v)[NS / kColThreads], const OsInst& oi, uint32_t* hist,
                                  float* wmin, float* wmax, int* tmp, int* sb, uint32_t& klo, uint32_t& khi) {
    constexpr int NW = kColThreads / 64;
    constexpr int PER = NS / kColThreads;
    const int64_t m = oi.end - oi.beg;
    for (int i = threadIdx.x; i < kSampleBins; i += kColThreads) hist[i] = 0;
    float mn = v[0], mx = v[0];
#pragma unroll
    for (int u = 1; u < PER; ++u) { mn = fminf(mn, v[u]); mx = fmaxf(mx, v[u]); }
    for (int o = 32; o > 0; o >>= 1) {
        mn = fminf(mn, __shfl_xor(mn, o, 64));
        mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    }
    if ((threadIdx.x & 63) == 0) { wmin[threadIdx.x >> 6] = mn; wmax[threadIdx.x >> 6] = mx; }
    __syncthreads();
    mn = wmin[0];
    mx = wmax[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) { mn = fminf(mn, wmin[w]); mx = fmaxf(mx, wmax[w]); }
    const int64_t ir = (oi.rank - 1) * NS / m;
    const int64_t il = ir - DELTA, ih = ir + DELTA;
    klo = 0u;
    khi = 0xffffffffu;
    if (KEYBINS && mx > mn) {
        const uint32_t kmn = order_key(mn), kmx = order_key(mx);
        const int sh = top_shift(kmx - kmn);
        const int64_t ihc = ih < NS - 1 ? ih : NS - 1;
#pragma unroll
        for (int u = 0; u < PER; ++u) atomicAdd(&hist[(order_key(v[u]) - kmn) >> sh], 1u);
        __syncthreads();
        constexpr int BPT = kSampleBins / kColThreads;
        int c = 0;
#pragma unroll
        for (int u = 0; u < BPT; ++u) c += (int)hist[threadIdx.x * BPT + u];
        int tot;
        const int inc = block_inclusive_scan<kColThreads>(c, tmp, &tot);
        int acc = inc - c;
#pragma unroll
        for (int u = 0; u < BPT; ++u) {
            const int bin = threadIdx.x * BPT + u;
            const int nx = acc + (int)hist[bin];
            if (acc <= il && il < nx) sb[0] = bin;
            if (acc <= ihc && ihc < nx) sb[1] = bin;
            acc = nx;
        }
        __syncthreads();
        if (il > 0) klo = kmn + ((uint32_t)(sb[0] > 0 ? sb[0] - 1 : 0) << sh);
        const uint64_t hk = (uint64_t)kmn + ((uint64_t)(sb[1] + 2) << sh) - 1;
        khi = hk < 0xffffffffull ? (uint32_t)hk : 0xffffffffu;
    } else if (mx > mn) {
        const float scale = (float)kSampleBins / (mx - mn);
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            int bin = (int)((v[u] - mn) * scale);
            bin = bin < 0 ? 0 : (bin >= kSampleBins ? kSampleBins - 1 : bin);
            atomicAdd(&hist[bin], 1u);
        }
        __syncthreads();
        constexpr int BPT = kSampleBins / kColThreads;
        int c = 0;
#pragma unroll
        for (int u = 0; u < BPT; ++u) c += (int)hist[threadIdx.x * BPT + u];
        int tot;
        const int inc = block_inclusive_scan<kColThreads>(c, tmp, &tot);
        int acc = inc - c;
#pragma unroll
        for (int u = 0; u < BPT; ++u) {
            const int bin = threadIdx.x * BPT + u;
            const int nx = acc + (int)hist[bin];
            if (acc <= il && il < nx) sb[0] = bin;      // bin holding sample rank il (0-based)
            if (acc <= ih && ih < nx) sb[1] = bin;
            acc = nx;
        }
        __syncthreads();
        const float w = (mx - mn) / (float)kSampleBins;
        if (il > 0) klo = order_key(mn + (float)(sb[0] - 1) * w);
        if (ih < NS - 1) khi = order_key(mn + (float)(sb[1] + 2) * w);
    } else {
        klo = khi = order_key(mn);
    }
    if (klo > khi) klo = khi;
    __syncthreads();
}

// Block (slice s, instance).  Every block derives the instance's key bracket (all keys when
// the row has at most kCap of them, else sample_bracket); block 0 stores the flag, need and
// bracket in the state.  Output: cnt[(inst * SL + s) * 2] = #keys < lo, [+1] = #candidates;
// the candidates (keys in [lo, hi]) at cand[(inst * SL + s) * kSlice ...], grouped by their top
// digit (key - lo) >> top_shift(hi - lo) in ascending digit order (any order inside a digit);
// dpre[inst][s]: the number of the slice's candidates with digit < d, d = 0 .. kDigitBins, as
// 16-bit values (kPreWords words), followed by the count of each digit (16-bit, two per word).
constexpr int kPreWords = kDigitBins / 2 + 1;   // 16-bit prefix values 0 .. kDigitBins, two per word
constexpr int kDpWords = kPreWords + kDigitBins / 2 + 1;   // per slice: prefixes, then counts (two per word)
__global__ __launch_bounds__(kColThreads) void th_collect_kernel(const float* __restrict__ scores,
                                                                I64Arg offsets, int Hq,
                                                                DevCfg cfg, int SL, int64_t S,
                                                                int64_t* __restrict__ state,
                                                                uint32_t* __restrict__ cand,
                                                                uint32_t* __restrict__ cnt,
                                                                uint32_t* __restrict__ dpre) {
    constexpr int NW = kColThreads / 64;
    constexpr int PT = kSlice / kColThreads;       // slice keys per thread
    constexpr int BPT = kDigitBins / kColThreads;  // digit bins per thread in the scan
    static_assert(kDigitBins == kSampleBins, "the sample and digit histograms share one array");
    __shared__ int wsum[NW];
    __shared__ int tmp[NW];
    __shared__ float wmin[NW], wmax[NW];
    __shared__ int sb[2];
    __shared__ uint32_t hist[kDigitBins];          // sample bins; then digit counts, then cursors
    const int inst = blockIdx.y, s = blockIdx.x;
    const int b = inst / Hq, h = inst % Hq;
    const int64_t off = offsets[b];
    const OsInst oi = os_instance(offsets[b + 1] - off, cfg);
    int64_t* st = state + (int64_t)inst * 8;
    if (s == 0 && threadIdx.x == 0) {
        st[kStFlag] = oi.flag;
        st[kStNeed] = oi.need;
    }
    if (oi.flag != kFlagActive) return;
    const int64_t lo = oi.beg + (int64_t)s * kSlice;
    const int64_t hi = lo + kSlice < oi.end ? lo + kSlice : oi.end;
    const float* row = scores + (int64_t)h * S + off;
    // the slice and the sample in one memory round trip
    float xv[PT];
#pragma unroll
    for (int j = 0; j < PT; ++j) {
        const int64_t t = lo + threadIdx.x + (int64_t)j * kColThreads;
        xv[j] = t < hi ? row[t] : 0.f;
    }
    uint32_t klo = 0u, khi = 0xffffffffu;
    if (oi.end - oi.beg > kCap) sample_bracket(row, oi, inst, hist, wmin, wmax, tmp, sb, klo, khi);
    if (s == 0 && threadIdx.x == 0) {
        st[kStLo] = klo;
        st[kStHi] = khi;
    }
    for (int i = threadIdx.x; i < kDigitBins; i += kColThreads) hist[i] = 0;
    __syncthreads();
    const int dsh = top_shift(khi - klo);
    // classify: keys below the bracket are counted, candidates are counted per digit
    int below = 0;
    uint32_t hitmask = 0;
#pragma unroll
    for (int j = 0; j < PT; ++j) {
        const bool ok = lo + threadIdx.x + (int64_t)j * kColThreads < hi;
        const uint32_t k = order_key(xv[j]);
        below += (ok && k < klo) ? 1 : 0;
        if (ok && k >= klo && k <= khi) {
            hitmask |= 1u << j;
            atomicAdd(&hist[(k - klo) >> dsh], 1u);
        }
    }
    below = wave_sum_i(below);
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = below;
    __syncthreads();
    // exclusive prefix over the digits (BPT consecutive bins per thread)
    uint32_t c[BPT];
    int csum = 0;
#pragma unroll
    for (int u = 0; u < BPT; ++u) { c[u] = hist[threadIdx.x * BPT + u]; csum += (int)c[u]; }
    int total;
    const int incl = block_inclusive_scan<kColThreads>(csum, tmp, &total);
    uint32_t* dp = dpre + ((size_t)inst * SL + s) * kDpWords;
    {
#pragma unroll
        for (int u = 0; u < BPT; u += 2) dp[kPreWords + (threadIdx.x * BPT + u) / 2] = c[u] | (c[u + 1] << 16);
        uint32_t acc = (uint32_t)(incl - csum);
        uint32_t pre[BPT];
#pragma unroll
        for (int u = 0; u < BPT; ++u) { pre[u] = acc; acc += c[u]; }
        static_assert(BPT % 2 == 0, "prefix values are written in pairs");
#pragma unroll
        for (int u = 0; u < BPT; u += 2) dp[(threadIdx.x * BPT + u) / 2] = pre[u] | (pre[u + 1] << 16);
#pragma unroll
        for (int u = 0; u < BPT; ++u) hist[threadIdx.x * BPT + u] = pre[u];   // cursor
        if (threadIdx.x == 0) dp[kDigitBins / 2] = (uint32_t)total;
    }
    __syncthreads();
    // scatter the candidates to their digit's range
    uint32_t* dst = cand + ((size_t)inst * SL + s) * kSlice;
#pragma unroll
    for (int j = 0; j < PT; ++j) {
        if (hitmask & (1u << j)) {
            const uint32_t k = order_key(xv[j]);
            dst[atomicAdd(&hist[(k - klo) >> dsh], 1u)] = k;
        }
    }
    if (threadIdx.x == 0) {
        int tb = 0;
        for (int w = 0; w < NW; ++w) tb += wsum[w];
        cnt[((size_t)inst * SL + s) * 2 + 0] = (uint32_t)tb;
        cnt[((size_t)inst * SL + s) * 2 + 1] = (uint32_t)total;
    }
}

// ---------------------------------------------------------------------- th_final
// Radix selection over the keys that visit(f) hands to f (f(x) once per key): returns the
// rank-th smallest x (1-based) and adds the number of keys above it to *gt.  Digits of
// kDigit bits from bit nbits - 1 down; every thread of the block calls it.
template <int NT = kThThreads, class Visit>
__device__ uint32_t radix_rank(Visit visit, int nbits, int64_t rank, uint32_t* hist, int* tmp, int64_t* sh,
                               int64_t* gt) {
    constexpr int NB = 1 << kDigit, BPT = NB / NT;
    uint64_t prefix = 0;
    int shift = nbits;
    while (shift > 0) {
        const int d = shift < kDigit ? shift : kDigit;
        shift -= d;
        const int top = shift + d;
        const uint32_t dmask = (1u << d) - 1u;
        for (int i = threadIdx.x; i < NB; i += NT) hist[i] = 0;
        __syncthreads();
        visit([&](uint32_t x) {
            const uint64_t xx = x;
            if ((xx >> top) == (prefix >> top)) atomicAdd(&hist[(uint32_t)(xx >> shift) & dmask], 1u);
        });
        __syncthreads();
        int c = 0;
#pragma unroll
        for (int u = 0; u < BPT; ++u) c += (int)hist[threadIdx.x * BPT + u];
        int total;
        const int inc = block_inclusive_scan<NT>(c, tmp, &total);
        if (inc - c < rank && rank <= inc) {
            int acc = inc - c;
            for (int u = 0; u < BPT; ++u) {
                const int bin = threadIdx.x * BPT + u;
                const int nx = acc + (int)hist[bin];
                if (acc < rank && rank <= nx) {
                    sh[0] = bin;
                    sh[1] = acc;
                    sh[2] = total - nx;
                }
                acc = nx;
            }
        }
        __syncthreads();
        prefix |= (uint64_t)sh[0] << shift;
        rank -= sh[1];
        *gt += sh[2];
        __syncthreads();
    }
    return (uint32_t)prefix;
}

// One block per instance: theta key, #keys above it (state) and theta_out.
__global__ __launch_bounds__(kThThreads) void th_final_kernel(const float* __restrict__ scores,
                                                             I64Arg offsets, int Hq,
                                                             DevCfg cfg, int SL, int64_t S,
                                                             const uint32_t* __restrict__ cand,
                                                             const uint32_t* __restrict__ cnt,
                                                             const uint32_t* __restrict__ dpre,
                                                             int64_t* __restrict__ state, float* __restrict__ theta_out) {
    static_assert(kDigitBins / 2 == kThThreads, "one pair of digit bins per thread");
    __shared__ uint32_t xs[kCap];
    __shared__ int segpre[kMaxSL + 1], sega[kMaxSL];
    __shared__ uint32_t hist[kDigitBins];
    __shared__ int tmp[kThThreads / 64];
    __shared__ int tmp3[3][kThThreads / 64];
    __shared__ int64_t sh[4];
    __shared__ uint32_t nd;
    const int inst = blockIdx.x;
    int64_t* st = state + (int64_t)inst * 8;
    const int b = inst / Hq, h = inst % Hq;
    const int t = threadIdx.x;
    // every global load of the prologue is issued before any is used (one memory round trip):
    // the sequence bounds, the bracket, the slice counts of slices 2t and 2t+1 and the counts of
    // digit pair (2t, 2t+1) in every slice (slices past the row's end hold zeros)
    const int64_t off = offsets[b];
    const int64_t nrow = offsets[b + 1] - off;
    const uint32_t klo = (uint32_t)st[kStLo], khi = (uint32_t)st[kStHi];
    const uint32_t* cs = cnt + (size_t)inst * SL * 2;
    uint2 cp[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int sl = 2 * t + u;
        cp[u] = reinterpret_cast<const uint2*>(cs)[sl < SL ? sl : SL - 1];
    }
    // rows with more than 2 kThThreads slices (of 8192 keys, or 128 tiles: past 2^22 tokens):
    // the counts of the slices past the first 2 kThThreads, one more round trip
    uint32_t more_lo = 0, more_mid = 0;
    for (int sl = 2 * kThThreads + t; sl < SL; sl += kThThreads) {
        const uint2 c = reinterpret_cast<const uint2*>(cs)[sl];
        more_lo += c.x;
        more_mid += c.y;
    }
    uint32_t dlo = 0, dhi = 0;
    {
        constexpr int SLR = 32;
        const uint32_t* dc = dpre + (size_t)inst * SL * kDpWords + kPreWords + t;
        for (int sl0 = 0; sl0 < SL; sl0 += SLR) {
            uint32_t w[SLR];
#pragma unroll
            for (int u = 0; u < SLR; ++u) w[u] = dc[(size_t)(sl0 + u < SL ? sl0 + u : SL - 1) * kDpWords];
            // every load of the batch is issued before the first sum (else the scheduler starts
            // the sums early and the last loads wait a round trip)
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < SLR; ++u) {
                const uint32_t x = sl0 + u < SL ? w[u] : 0u;
                dlo += x & 0xffffu;
                dhi += x >> 16;
            }
        }
    }
    const OsInst oi = os_instance(nrow, cfg);
    if (oi.flag != kFlagActive) {
        if (theta_out && t == 0) theta_out[inst] = 0.f;
        return;
    }
    const int64_t m = oi.end - oi.beg;
    const int nsl = (int)((m + kSlice - 1) / kSlice);   // slices of the key range [beg, end)
    int lsum = (int)more_lo, csum = (int)more_mid;
#pragma unroll
    for (int u = 0; u < 2; ++u)
        if (2 * t + u < SL) { lsum += (int)cp[u].x; csum += (int)cp[u].y; }
    // one block scan gives the keys below the bracket (nlo), the candidates (nmid) and the
    // inclusive digit-count prefix; from them, the answer's digit
    const int cd = (int)(dlo + dhi);
    int nlo, nmid, tot;
    const int inc = block_inclusive_scan3<kThThreads>(lsum, csum, cd, tmp3, &nlo, &nmid, &tot);
    if (t == 0) nd = 0;
    int64_t gt = 0;
    uint32_t key = 0;
    const int64_t r = oi.rank;
    bool whole_row = !(nlo < r && r <= (int64_t)nlo + nmid);
    const int dsh = top_shift(khi - klo);
    if (!whole_row && klo != khi) {
        const int64_t rr0 = r - nlo;
        if (inc - cd < rr0 && rr0 <= inc) {
            const int below = inc - cd;
            const bool first = rr0 <= below + (int)dlo;
            sh[0] = first ? 2 * t : 2 * t + 1;
            sh[1] = first ? below : below + (int)dlo;
            sh[2] = tot - (first ? below + (int)dlo : inc);
            sh[3] = first ? dlo : dhi;
        }
    }
    __syncthreads();
    if (!whole_row) {
        gt = m - nlo - nmid;                       // keys above hi
        int64_t rr = r - nlo;
        if (klo == khi) {
            key = klo;
        } else {
            const uint32_t D = (uint32_t)sh[0];
            rr -= sh[1];
            gt += sh[2];
            const int64_t nD = sh[3];
            if (nD > kCap) {
                whole_row = true;
            } else {
                // copy digit D's candidates of every slice (their low bits) into LDS: the slices'
                // segments [a_s, e_s) of their digit-sorted candidates are laid end to end
                const uint32_t low = dsh ? ((1u << dsh) - 1u) : 0u;
                const uint32_t* dp = dpre + (size_t)inst * SL * kDpWords;
                auto pre_at = [&](int sl, uint32_t d) {
                    return (dp[(size_t)sl * kDpWords + d / 2] >> (16 * (d & 1))) & 0xffffu;
                };
                if (nD <= 1024) {
                    // small bucket: one thread per slice copies its few keys
                    for (int sl = t; sl < nsl; sl += kThThreads) {
                        const uint32_t a = pre_at(sl, D), e = pre_at(sl, D + 1);
                        if (e > a) {
                            const uint32_t base = atomicAdd(&nd, e - a);
                            const uint32_t* src = cand + ((size_t)inst * SL + sl) * kSlice;
                            for (uint32_t q = a; q < e; ++q) xs[base + (q - a)] = (src[q] - klo) & low;
                        }
                    }
                    __syncthreads();
                } else {
                    // large bucket: every thread copies keys, 16 in flight.  The slices' segments
                    // are laid end to end, 2 kThThreads slices per pass.
                    int ntot = 0;
                    for (int sl0 = 0; sl0 < nsl; sl0 += 2 * kThThreads) {
                        int la[2], ll[2];
#pragma unroll
                        for (int u = 0; u < 2; ++u) {
                            const int sl = sl0 + 2 * t + u;
                            la[u] = 0;
                            ll[u] = 0;
                            if (sl < nsl) {
                                la[u] = (int)pre_at(sl, D);
                                ll[u] = (int)pre_at(sl, D + 1) - la[u];
                            }
                        }
                        int npass;
                        const int sinc = block_inclusive_scan<kThThreads>(ll[0] + ll[1], tmp, &npass);
#pragma unroll
                        for (int u = 0; u < 2; ++u) {
                            const int sl = sl0 + 2 * t + u;
                            if (sl < nsl) {
                                segpre[sl] = ntot + sinc - ll[0] - ll[1] + (u ? ll[0] : 0);
                                sega[sl] = la[u];
                            }
                        }
                        ntot += npass;
                    }
                    if (t == 0) segpre[nsl] = ntot;
                    __syncthreads();
                    for (int i0 = t; i0 < ntot; i0 += 16 * kThThreads) {
                        uint32_t v[16];
#pragma unroll
                        for (int u = 0; u < 16; ++u) {
                            const int i = i0 + u * kThThreads;
                            v[u] = klo;
                            if (i < ntot) {
                                int a = 0, z = nsl - 1;          // last slice with segpre[slice] <= i
                                while (a < z) {
                                    const int mid = (a + z + 1) >> 1;
                                    if (segpre[mid] <= i) a = mid; else z = mid - 1;
                                }
                                v[u] = cand[((size_t)inst * SL + a) * kSlice + sega[a] + (i - segpre[a])];
                            }
                        }
#pragma unroll
                        for (int u = 0; u < 16; ++u) {
                            const int i = i0 + u * kThThreads;
                            if (i < ntot) xs[i] = (v[u] - klo) & low;
                        }
                    }
                    if (t == 0) nd = (uint32_t)ntot;
                    __syncthreads();
                }
                const int cntD = (int)nd;
                uint32_t xl;
                if (cntD <= 64) {
                    // one wave ranks the bucket: the answer x has #{< x} < rr <= #{<= x}
                    if (t < 64) {
                        const bool has = t < cntD;
                        const uint32_t x = has ? xs[t] : 0xffffffffu;
                        int less = 0, leq = 0;
                        for (int j = 0; j < cntD; ++j) {
                            const uint32_t y = __shfl(x, j, 64);
                            less += y < x ? 1 : 0;
                            leq += y <= x ? 1 : 0;
                        }
                        if (has && less < rr && rr <= leq) {
                            sh[0] = x;
                            sh[1] = cntD - leq;
                        }
                    }
                    __syncthreads();
                    xl = (uint32_t)sh[0];
                    gt += sh[1];
                } else {
                    xl = radix_rank(
                        [&](auto f) {
                            for (int i = t; i < cntD; i += kThThreads) f(xs[i]);
                        },
                        dsh, rr, hist, tmp, sh, &gt);
                }
                key = klo + ((D << dsh) | xl);
            }
        }
    }
    if (whole_row) {
        // the answer lies outside the bracket or its digit overflows LDS: whole row
        gt = 0;
        const float* row = scores + (int64_t)h * S + off;
        key = radix_rank(
            [&](auto f) {
                for_each_f32<kThThreads, 4>(row, oi.beg, oi.end, [&](int64_t, float v, bool ok) {
                    if (ok) f(order_key(v));
                });
            },
            32, r, hist, tmp, sh, &gt);
    }
    if (t == 0) {
        st[kStKey] = key;
        st[kStGt] = gt;
        if (theta_out) theta_out[inst] = key_to_float(key);
    }
}

// ------------------------------------------------- fused score-and-select: prep, final
// prep_kernel, block (b, h) of the B*Hq instance blocks: q'_{b,h} = P^T q_{b,h} / sqrt(32) in
// the order of qproj_kernel (so the scores equal those of ts_score), then the instance's key
// bracket from kPrepSample sampled index scores (rows longer than kCap; otherwise every key is a
// candidate), and the instance state (flag, need, bracket, range).  When K is given, block
// B*Hq + b first writes the index row of sequence b's last token (the token appended by this
// decode step) exactly as index_append_kernel does; the samples never read that row.
constexpr int kPrepThreads = kColThreads;
constexpr int kPrepSample = 1024;  // sampled index scores per instance (runs of kRunLen tokens)
constexpr int kPrepDelta = 48;     // bracket half-width in sample ranks (about 5 standard deviations)
static_assert(kPrepSample % (kPrepThreads / 4) == 0 && kPrepSample % kColThreads == 0, "whole sample passes");
__global__ __launch_bounds__(kPrepThreads) void prep_kernel(const uint16_t* __restrict__ q, const float* __restrict__ P,
                                                           uint16_t* k_index, const uint16_t* __restrict__ K,
                                                           I64Arg offsets, int B, int Hq, int Hkv, DevCfg cfg,
                                                           float* __restrict__ qp, int64_t* __restrict__ state) {
    constexpr int NW = kPrepThreads / 64;
    constexpr int PASSES = kPrepSample / (kPrepThreads / 4);
    __shared__ float sP[kD * kDP];
    __shared__ float sk[8][kD];
    __shared__ float sq[kD];
    __shared__ float sqp[kDP];
    __shared__ float samp[kPrepSample];
    __shared__ float spart[4][kDP];
    __shared__ uint32_t hist[kSampleBins];
    __shared__ float wmin[NW], wmax[NW];
    __shared__ int tmp[NW];
    __shared__ int sb[2];
    const int ninst = B * Hq;
    const int t = threadIdx.x;
    if ((int)blockIdx.x >= ninst) {
        // index row of the last token of sequence b, (g, c) = (t / 32, t % 32), fp64 sum in order
        const int b = blockIdx.x - ninst;
        const int64_t tok = offsets[b + 1] - 1;
        if (tok < offsets[b]) return;
        for (int i = t; i < kD * kDP / 4; i += kPrepThreads)
            reinterpret_cast<float4*>(sP)[i] = reinterpret_cast<const float4*>(P)[i];
        for (int i = t; i < Hkv * kD; i += kPrepThreads) sk[i / kD][i % kD] = bf16_to_f32(K[tok * Hkv * kD + i]);
        __syncthreads();
        if (t < Hkv * kDP) {
            const int g = t / kDP, c = t % kDP;
            double acc = 0.0;
#pragma unroll 16
            for (int j = 0; j < kD; ++j) acc = fma((double)sk[g][j], (double)sP[j * kDP + c], acc);
            k_index[(tok * Hkv + g) * kDP + c] = f64_to_bf16_rne(acc);
        }
        return;
    }
    const int inst = blockIdx.x, b = inst / Hq, h = inst % Hq, g = h / (Hq / Hkv);
    const int64_t off = offsets[b], n = offsets[b + 1] - off;
    const OsInst oi = os_instance(n, cfg);
    // the sample range leaves out the token appended by this step
    const int64_t send = (K && oi.end == n) ? n - 1 : oi.end;
    const int64_t ms = send - oi.beg;
    const bool sampled = oi.flag == kFlagActive && oi.end - oi.beg > kCap && ms >= kRuns * kRunLen;
    constexpr int kPrepRuns = kPrepSample / kRunLen;   // one stratum of the range per run
    static_assert(kPrepRuns <= kRuns, "a sampled range (>= kRuns kRunLen keys) holds every run");
    const int part = t & 3;
    // P and q first, then the sample rows: staging P and q waits for them alone, and the
    // samples arrive while q' is formed.  The loads and the staging are one basic block: a
    // branch would let the compiler move the P and q loads past the sample loads, to their use.
    // Without a sample every lane reads the start of P (the offset is multiplied by 0).
    static_assert(kD * kDP / 4 == 2 * kPrepThreads && kD <= kPrepThreads && (kD & (kD - 1)) == 0,
                  "two float4 of P and one q value per thread");
    const float4* P4 = reinterpret_cast<const float4*>(P);
    const float4 p0 = P4[t], p1 = P4[t + kPrepThreads];
    const uint16_t qb = q[((int64_t)b * Hq + h) * kD + (t & (kD - 1))];
    __builtin_amdgcn_sched_barrier(0);
    const int64_t use = sampled ? 1 : 0;
    const int64_t ms_pos = sampled ? ms : (int64_t)kRuns * kRunLen;   // a valid range either way
    const uint16_t* sbase = sampled ? k_index : reinterpret_cast<const uint16_t*>(P);
    uint4 kv[PASSES];
#pragma unroll
    for (int u = 0; u < PASSES; ++u) {
        const int i = u * (kPrepThreads / 4) + (t >> 2);
        const int64_t pos = oi.beg + sample_pos(i, ms_pos, inst, kPrepRuns);
        kv[u] = ld16(sbase + (((off + pos) * Hkv + g) * kDP + part * 8) * use);
    }
    __builtin_amdgcn_sched_barrier(0);
    reinterpret_cast<float4*>(sP)[t] = p0;
    reinterpret_cast<float4*>(sP)[t + kPrepThreads] = p1;
    sq[t & (kD - 1)] = bf16_to_f32(qb);     // threads t and t + kD store the same value
    __syncthreads();
    if (t < 4 * kDP) {
        // partial k of q'[c] over j in [32k, 32k + 32), in order (the order of qproj_kernel)
        const int c = t % kDP, k = t / kDP;
        float acc = 0.f;
#pragma unroll
        for (int j = 32 * k; j < 32 * k + 32; ++j) acc = fmaf(sq[j], sP[j * kDP + c], acc);
        spart[k][c] = acc;
    }
    __syncthreads();
    if (t < kDP) {
        const float acc = ((spart[0][t] + spart[1][t]) + (spart[2][t] + spart[3][t])) * 0.17677669529663688f;
        sqp[t] = acc;
        qp[(int64_t)inst * kDP + t] = acc;
    }
    __syncthreads();
    // no sample (rows of at most kCap keys): the empty bracket lo > hi, so that the score kernel
    // classifies nothing and th_final2 ranks the row itself
    uint32_t klo = 1u, khi = 0u;
    if (sampled) {
        float qr[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) qr[e] = sqp[part * 8 + e];
#pragma unroll
        for (int u = 0; u < PASSES; ++u) {
            const uint4 w = kv[u];
            const float kf[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                                 bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
            float sdot = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) sdot = fmaf(qr[e], kf[e], sdot);
            sdot = sum_quad(sdot);
            if (part == 0) samp[u * (kPrepThreads / 4) + (t >> 2)] = sdot;
        }
        __syncthreads();
        float v[kPrepSample / kColThreads];
#pragma unroll
        for (int u = 0; u < kPrepSample / kColThreads; ++u) v[u] = samp[t + u * kColThreads];
        bracket_of_sample<kPrepSample, kPrepDelta>(v, oi, hist, wmin, wmax, tmp, sb, klo, khi);
    }
    if (t == 0) {
        int64_t* st = state + (int64_t)inst * 8;
        st[kStFlag] = oi.flag;
        st[kStNeed] = oi.need;
        st[kStLo] = klo;
        st[kStHi] = khi;
        st[kStBeg] = oi.beg;
        st[kStEnd] = oi.end;
    }
}

// ----------------------------------------------------------------- chunk lookup
// Work item -> (sequence b, its first item, its item count, first token, length) for chunks of CH
// tokens numbered sequence by sequence.
template <int CH = kChunk>
__device__ __forceinline__ bool find_chunk(const I64Arg& offsets, int B, int64_t item, int& b,
                                           int64_t& first, int64_t& nch, int64_t& t0, int64_t& len) {
    const SeqPos sp = wave_find_seq(B, item, (offsets[1] - offsets[0] + CH - 1) / CH,
                                    [od = offsets.dev](int i) { return (od[i + 1] - od[i] + CH - 1) / CH; });
    if (sp.b < 0) return false;
    b = sp.b;
    first = sp.first;
    nch = sp.cnt;
    // one sequence: its length from the launch arguments; more: from device memory
    const int64_t n = B == 1 ? offsets[1] - offsets[0] : offsets.dev[b + 1] - offsets.dev[b];
    t0 = (item - first) * CH;
    len = n - t0 < CH ? n - t0 : CH;
    return true;
}

// list entries of the sequences before b (every lane of the wave calls it)
__device__ __forceinline__ int64_t kpre_of(const I64Arg& offsets, int b, const DevCfg& c) {
    return wave_prefix_seq(b, [od = offsets.dev, c](int i) { return budget_k(od[i + 1] - od[i], c.bnum, c.bden, c.sink, c.local); });
}

// -------------------------------------------------------------------------- votes
// One thread per token (1024-token blocks).  Vote(t) = #{h : scores[h][t] > theta_h}
// (strict, IEEE compare so -0 == +0).  The key of a non-forced token is Vote + 1 if
// Vote >= v_min, else 0 (the listing's -1); forced tokens get 255.  Each block also counts
// the keys of its non-forced tokens (one histogram per block).
__global__ __launch_bounds__(kChunk) void vote_kernel(const float* __restrict__ scores,
                                                     I64Arg offsets, int B, int Hq,
                                                     DevCfg cfg, int64_t S, const int64_t* __restrict__ state,
                                                     uint8_t* __restrict__ votes, uint8_t* __restrict__ keys,
                                                     uint32_t* __restrict__ hist) {
    __shared__ float th[64];
    __shared__ uint32_t lh[kChunk / 64][kVoteBins];
    int b;
    int64_t first, nch, t0, len;
    if (!find_chunk(offsets, B, blockIdx.x, b, first, nch, t0, len)) return;
    const int64_t off = offsets[b], n = offsets[b + 1] - off;
    const int64_t i = threadIdx.x;
    const int64_t t = t0 + i;
    // this token's first 32 scores are requested before the thresholds are staged, so both
    // arrive in one memory round trip
    const float* col = scores + off + (i < len ? t : t0);
    float sv[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) sv[u] = col[(int64_t)(u < Hq ? u : Hq - 1) * S];
    for (int h = threadIdx.x; h < Hq; h += kChunk) th[h] = key_to_float((uint32_t)state[((int64_t)b * Hq + h) * 8 + kStKey]);
    for (int k = threadIdx.x; k < (kChunk / 64) * kVoteBins; k += kChunk) (&lh[0][0])[k] = 0;
    __syncthreads();
    if (i < len) {
        int v = 0;
#pragma unroll
        for (int u = 0; u < 32; ++u) v += (u < Hq && sv[u] > th[u]) ? 1 : 0;
        for (int h0 = 32; h0 < Hq; h0 += 32) {
#pragma unroll
            for (int u = 0; u < 32; ++u) sv[u] = col[(int64_t)(h0 + u < Hq ? h0 + u : Hq - 1) * S];
#pragma unroll
            for (int u = 0; u < 32; ++u) v += (h0 + u < Hq && sv[u] > th[h0 + u]) ? 1 : 0;
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

// ------------------------------------------------------------ vote compaction
// One block per 1024-token chunk c of sequence b.  The block first sums the key histograms of
// all chunks of b (read straight from memory) into the totals and into the counts of the chunks
// before c.  From the totals: need = K - |F|, the boundary key v* (largest
// key whose suffix count reaches need; none when need == 0), gt = #keys above v* and
// need_eq = need - gt.  The chunk's first selected token then has output rank
//   forced_before(first token of c) + #keys above v* before c + min(eqb, need_eq),
// eqb = #keys equal to v* before c.  One wave finds v*, gt and the counts before c from suffix
// sums over the key bins (two bins per lane, from the top key down); one block scan then places
// every forced token, every non-forced token above v* and the first need_eq - eqb tokens equal
// to v* in position order, written ascending.
__global__ __launch_bounds__(kChunk) void compact_vote_kernel(I64Arg offsets, int B,
                                                             DevCfg cfg, const uint8_t* __restrict__ keys,
                                                             const uint32_t* __restrict__ hist,
                                                             int32_t* __restrict__ idx_out,
                                                             int64_t* __restrict__ count_out) {
    constexpr int NG = kChunk / kVoteBins;          // row groups for the column sums
    constexpr int RU = 16;                          // histogram rows in flight per thread
    __shared__ uint32_t part[NG][kVoteBins][2];
    __shared__ uint32_t tot[kVoteBins], bef[kVoteBins];
    __shared__ int tmp[kChunk / 64];
    __shared__ int sh[4];
    int b;
    int64_t first, nch, t0, len;
    if (!find_chunk(offsets, B, blockIdx.x, b, first, nch, t0, len)) return;
    const int t = threadIdx.x;
    const int64_t off = offsets[b], n = offsets[b + 1] - off;
    const int64_t c = blockIdx.x - first;
    const uint8_t kk = t < len ? keys[off + t0 + t] : 0;
    const uint32_t* hrows = hist + (size_t)first * kVoteBins;
    // key totals over the sequence and over the chunks before c: thread (grp, kb) sums column kb
    // of the rows grp, grp + NG, ... straight from the histograms, RU rows in flight (no LDS
    // staging, so the block's LDS stays small and two blocks fit on a CU).  NG * RU = 224 rows
    // per pass: one memory round trip for sequences of up to 224 chunks.  Rows past the end are
    // loaded as the last row and not counted, so the loads need no branch.
    const int grp = t / kVoteBins, kb = t % kVoteBins;
    uint32_t at = 0, ab = 0;
    const int nchi = (int)nch, ci = (int)c;   // chunks of one sequence: < 2^14
    if (grp < NG) {
        for (int r0 = grp; r0 < nchi; r0 += NG * RU) {
            uint32_t x[RU];
#pragma unroll
            for (int u = 0; u < RU; ++u) {
                const int r = r0 + u * NG;
                x[u] = hrows[(size_t)(r < nchi ? r : nchi - 1) * kVoteBins + kb];
            }
#pragma unroll
            for (int u = 0; u < RU; ++u) {
                at += (r0 + u * NG < nchi) ? x[u] : 0u;
                ab += (r0 + u * NG < ci) ? x[u] : 0u;
            }
        }
    }
    if (grp < NG) { part[grp][kb][0] = at; part[grp][kb][1] = ab; }
    __syncthreads();
    if (t < kVoteBins) {
        uint32_t a = 0, p = 0;
#pragma unroll
        for (int g = 0; g < NG; ++g) { a += part[g][t][0]; p += part[g][t][1]; }
        tot[t] = a;
        bef[t] = p;
    }
    __syncthreads();
    const int64_t K = budget_k(n, cfg.bnum, cfg.bden, cfg.sink, cfg.local);
    const int64_t need = K - forced_before(n, n, cfg.sink, cfg.local);
    static_assert(kVoteBins <= 128, "two key bins per lane of one wave");
    if (t < 64) {
        // lane l holds bins b0 = top - 2l and b1 = b0 - 1; inclusive sums over the lanes give the
        // suffix counts of the keys (sequence: x, chunks before c: y) above and at each bin
        const int b0 = kVoteBins - 1 - 2 * t, b1 = b0 - 1;
        const int c0 = b0 >= 0 ? (int)tot[b0] : 0, c1 = b1 >= 0 ? (int)tot[b1] : 0;
        const int e0 = b0 >= 0 ? (int)bef[b0] : 0, e1 = b1 >= 0 ? (int)bef[b1] : 0;
        const int x = wave_inclusive_scan(c0 + c1), y = wave_inclusive_scan(e0 + e1);
        const int xa = x - c0 - c1, ya = y - e0 - e1;        // the keys above bin b0
        // v*: the bin whose suffix count first reaches need (one lane owns it when need > 0)
        const bool own0 = need > 0 && b0 >= 0 && xa < need && need <= xa + c0;
        const bool own1 = need > 0 && b1 >= 0 && xa + c0 < need && need <= xa + c0 + c1;
        const uint64_t m = __ballot(own0 || own1);
        int vs = kVoteBins, gt = 0, gtb = 0, eqb = 0;
        if (m) {
            const int L = __builtin_ctzll(m);
            vs = __builtin_amdgcn_readlane(own0 ? b0 : b1, L);
            gt = __builtin_amdgcn_readlane(own0 ? xa : xa + c0, L);
            gtb = __builtin_amdgcn_readlane(own0 ? ya : ya + e0, L);
            eqb = __builtin_amdgcn_readlane(own0 ? e0 : e1, L);
        }
        if (t == 0) {
            sh[0] = vs;
            sh[1] = gt;
            sh[2] = gtb;
            sh[3] = eqb;
        }
    }
    __syncthreads();
    const int vs = sh[0];
    const int64_t need_eq = need - sh[1];
    const int64_t gtb = sh[2], eqb = sh[3];
    const int64_t base = forced_before(t0, n, cfg.sink, cfg.local) + gtb + (eqb < need_eq ? eqb : need_eq);
    if (c == 0 && t == 0) count_out[b] = K;
    // one scan: the low 16 bits count the tokens taken for sure (forced, or above v*), the high 16
    // bits the tokens equal to v*, of which the chunk takes the first need_eq - eqb
    const bool in = t < len;
    const int sure = (in && (kk == 255 || (vs < kVoteBins && kk > vs))) ? 1 : 0;
    const int eqf = (in && kk != 255 && kk == vs) ? 1 : 0;
    const int packed = sure | (eqf << 16);
    int tot_packed;
    const int exc = block_inclusive_scan<kChunk>(packed, tmp, &tot_packed) - packed;
    const int64_t quota = need_eq - eqb > 0 ? need_eq - eqb : 0;
    const int64_t eq_before = exc >> 16;
    const bool sel = sure || (eqf && eq_before < quota);
    const int64_t p = base + (exc & 0xffff) + (eq_before < quota ? eq_before : quota);
    const int64_t kpre = kpre_of(offsets, b, cfg);
    if (sel && p < K) idx_out[kpre + p] = (int32_t)(t0 + t);
}

// --------------------------------------------------------- per-head compaction
// Three kernels over 64-token chunks, one wave per chunk (four independent waves per block, no
// LDS and no block barriers).  A wave covers every head of its chunk: the heads' score loads
// are issued together, lane u keeps the parameters of head h0 + u, and each head's step reads
// them back as wave-uniform values (readlane), so the per-head work is ballots and popcounts.
//   ph_count   : cnt[(h * nitems + item) * 2 + {0, 1}] = non-forced tokens of the chunk with key
//                above / equal to theta_h;
//   ph_scan    : one wave per (sequence, head): exclusive prefix of those counts over the
//                sequence's chunks, written in place;
//   ph_compact : the chunk's selected tokens of every head, at their ranks: forced tokens, keys
//                above theta_h, and the first need_eq - eqb keys equal to theta_h in position order.
constexpr int kPhHeads = 32;   // heads handled per pass of a wave (Hq <= 64 takes two)
constexpr int kPhChunk = 64;   // tokens per chunk: one per lane of a wave
constexpr int kPhWaves = 4;    // independent chunk waves per block

__device__ __forceinline__ int lane_pick(int v, int u) { return __builtin_amdgcn_readlane(v, u); }
// number of set bits of the wave mask m in the lanes below this one
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__global__ __launch_bounds__(kPhWaves * 64) void ph_count_kernel(const float* __restrict__ scores,
                                                               I64Arg offsets, int B, int Hq,
                                                               DevCfg cfg, int64_t S, const int64_t* __restrict__ state,
                                                               int64_t nitems, uint32_t* __restrict__ cnt) {
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * kPhWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (item >= nitems) return;
    int b;
    int64_t first, nch, t0, len;
    if (!find_chunk<kPhChunk>(offsets, B, item, b, first, nch, t0, len)) return;
    const int64_t off = offsets[b], n = offsets[b + 1] - off;
    const int64_t t = t0 + lane;
    const bool in = lane < len && !is_forced(t, n, cfg.sink, cfg.local);
    const float* col = scores + off + (lane < len ? t : t0);
    for (int h0 = 0; h0 < Hq; h0 += kPhHeads) {
        float sv[kPhHeads];
#pragma unroll
        for (int u = 0; u < kPhHeads; ++u) sv[u] = col[(int64_t)(h0 + u < Hq ? h0 + u : Hq - 1) * S];
        // lane u: flag and theta key of head h0 + u
        const int hl = h0 + (lane < kPhHeads ? lane : 0) < Hq ? h0 + (lane < kPhHeads ? lane : 0) : Hq - 1;
        const int64_t* st = state + ((int64_t)b * Hq + hl) * 8;
        const int lact = st[kStFlag] == kFlagActive ? 1 : 0;
        const int lkey = (int)(uint32_t)st[kStKey];
        uint32_t cg = 0, ce = 0;   // lane u ends with head h0 + u's counts
#pragma unroll
        for (int u = 0; u < kPhHeads; ++u) {
            if (h0 + u >= Hq) break;
            const bool act = lane_pick(lact, u) != 0;
            const uint32_t ks = (uint32_t)lane_pick(lkey, u);
            const uint32_t k = order_key(sv[u]);
            const uint32_t g = (uint32_t)__popcll(__ballot(act && in && k > ks));
            const uint32_t e = (uint32_t)__popcll(__ballot(act && in && k == ks));
            cg = lane == u ? g : cg;
            ce = lane == u ? e : ce;
        }
        if (lane < kPhHeads && h0 + lane < Hq)
            reinterpret_cast<uint2*>(cnt)[(size_t)(h0 + lane) * nitems + item] = make_uint2(cg, ce);
    }
}

// One block per (sequence b, head h): exclusive prefix over the chunks of b of the (above,
// equal) counts, in place.  Thread t sums kPhScanPer consecutive chunks, a block scan places
// the sums, and the block walks the chunks in tiles of kPhScanThreads * kPhScanPer.
constexpr int kPhScanThreads = 256;
constexpr int kPhScanPer = 8;
__global__ __launch_bounds__(kPhScanThreads) void ph_scan_kernel(I64Arg offsets, int B, int Hq,
                                                                int64_t nitems, uint32_t* __restrict__ cnt) {
    constexpr int NW = kPhScanThreads / 64;
    __shared__ uint32_t wt[2][NW];
    const int64_t inst = blockIdx.x;
    if (inst >= (int64_t)B * Hq) return;
    const int b = (int)(inst / Hq), h = (int)(inst % Hq);
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int64_t first = wave_prefix_seq(b, [od = offsets.dev](int i) { return (od[i + 1] - od[i] + kPhChunk - 1) / kPhChunk; });
    const int64_t nch = (offsets[b + 1] - offsets[b] + kPhChunk - 1) / kPhChunk;
    uint2* row = reinterpret_cast<uint2*>(cnt) + (size_t)h * nitems + first;
    uint32_t carry0 = 0, carry1 = 0;
    for (int64_t c0 = 0; c0 < nch; c0 += kPhScanThreads * kPhScanPer) {
        const int64_t cl = c0 + (int64_t)t * kPhScanPer;
        uint2 v[kPhScanPer];
#pragma unroll
        for (int u = 0; u < kPhScanPer; ++u) v[u] = cl + u < nch ? row[cl + u] : make_uint2(0, 0);
        uint32_t s0 = 0, s1 = 0;
#pragma unroll
        for (int u = 0; u < kPhScanPer; ++u) { s0 += v[u].x; s1 += v[u].y; }
        // (two's-complement addition: the same bits as unsigned sums)
        const uint32_t i0 = (uint32_t)wave_inclusive_scan((int)s0), i1 = (uint32_t)wave_inclusive_scan((int)s1);
        if (lane == 63) { wt[0][wid] = i0; wt[1][wid] = i1; }
        __syncthreads();
        uint32_t b0 = 0, b1 = 0, t0 = 0, t1 = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const uint32_t x = wt[0][w], y = wt[1][w];
            if (w < wid) { b0 += x; b1 += y; }
            t0 += x;
            t1 += y;
        }
        __syncthreads();                      // wt is written again by the next tile
        uint32_t a0 = carry0 + b0 + i0 - s0, a1 = carry1 + b1 + i1 - s1;
#pragma unroll
        for (int u = 0; u < kPhScanPer; ++u) {
            if (cl + u < nch) row[cl + u] = make_uint2(a0, a1);
            a0 += v[u].x;
            a1 += v[u].y;
        }
        carry0 += t0;
        carry1 += t1;
    }
}

// ph_compact_kernel: one wave per (64-token chunk, group of HPW heads), the groups of a chunk in
// adjacent waves.  One sequence: 8 heads per wave, so that more waves than chunks keep enough loads
// in flight (at 128K tokens and 32 heads 8192 waves: 11.9 us against 13.2 us with 32 heads per
// wave).  A batch: 32 heads per wave, since every wave repeats the sequence lookup and the list
// prefix of its chunk (16 sequences of 16K-64K tokens: 47.8 us against 64.1 us with 8).
template <int HPW>
__global__ __launch_bounds__(kPhWaves * 64) void ph_compact_kernel(const float* __restrict__ scores,
                                                                 I64Arg offsets, int B, int Hq,
                                                                 DevCfg cfg, int64_t S, const int64_t* __restrict__ state,
                                                                 int64_t nitems, const uint32_t* __restrict__ pre,
                                                                 int32_t* __restrict__ idx_out,
                                                                 int64_t* __restrict__ count_out) {
    const int lane = threadIdx.x & 63;
    const int HG = (Hq + HPW - 1) / HPW;
    const int64_t wv = (int64_t)blockIdx.x * kPhWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (wv >= nitems * HG) return;
    const int64_t item = wv / HG;
    const int h0 = (int)(wv % HG) * HPW;
    int b;
    int64_t first, nch, t0, len;
    if (!find_chunk<kPhChunk>(offsets, B, item, b, first, nch, t0, len)) return;
    const int64_t off = offsets[b], n = offsets[b + 1] - off;
    const int64_t K = budget_k(n, cfg.bnum, cfg.bden, cfg.sink, cfg.local);
    const int64_t kpre = kpre_of(offsets, b, cfg);
    const int64_t fb = forced_before(t0, n, cfg.sink, cfg.local);
    if (item == first && h0 == 0 && lane == 0) count_out[b] = K;
    const int64_t t = t0 + lane;
    const bool inr = lane < len;
    const bool frc = inr && is_forced(t, n, cfg.sink, cfg.local);
    const float* col = scores + off + (inr ? t : t0);
    {
        float sv[HPW];
#pragma unroll
        for (int u = 0; u < HPW; ++u) sv[u] = col[(int64_t)(h0 + u < Hq ? h0 + u : Hq - 1) * S];
        // lane u: the parameters of head h0 + u in this chunk.  A token is taken when it is forced,
        // when its key is above ks, or when it equals ks and is among the first `quota` such
        // tokens of the chunk; base is the list offset of the chunk's first taken token.  Take-all
        // and take-none heads are the same rule with ks = 0 and quota = 64 (every token) or
        // ks = ~0 and quota = 0 (forced tokens only).
        const int hl = h0 + (lane < HPW ? lane : 0) < Hq ? h0 + (lane < HPW ? lane : 0) : Hq - 1;
        const int64_t* st = state + ((int64_t)b * Hq + hl) * 8;
        const int64_t flag = st[kStFlag];
        const uint2 gq = reinterpret_cast<const uint2*>(pre)[(size_t)hl * nitems + item];
        const int64_t gtb = gq.x, eqb = gq.y;
        int64_t base, quota;
        uint32_t ks;
        if (flag == kFlagTakeAll) {
            base = t0;
            ks = 0u;
            quota = kPhChunk;
        } else if (flag == kFlagTakeNone) {
            base = fb;
            ks = ~0u;
            quota = 0;
        } else {
            const int64_t need_eq = st[kStNeed] - st[kStGt];
            base = fb + gtb + (eqb < need_eq ? eqb : need_eq);
            ks = (uint32_t)st[kStKey];
            quota = need_eq - eqb;
            quota = quota < 0 ? 0 : (quota > kPhChunk ? kPhChunk : quota);
        }
        const int lks = (int)ks, lquota = (int)quota, lbase = (int)base;
        const bool cand = inr && !frc;
#pragma unroll
        for (int u = 0; u < HPW; ++u) {
            if (h0 + u >= Hq) break;
            const uint32_t ku = (uint32_t)lane_pick(lks, u);
            const uint32_t k = order_key(sv[u]);
            const bool eqf = cand && k == ku;
            const int erank = lanes_below(__ballot(eqf));
            const bool sel = inr && (frc || k > ku || (eqf && erank < lane_pick(lquota, u)));
            const int64_t p = (int64_t)lane_pick(lbase, u) + lanes_below(__ballot(sel));
            if (sel && p < K) idx_out[Hq * kpre + (int64_t)(h0 + u) * K + p] = (int32_t)t;
        }
    }
}

// ------------------------------------------------------- fused path: order statistic
// th_final2_kernel, one block per instance (sequence b, head h), after prep_kernel and the score
// kernel's tile classification (records [h][tile] of the sequence's tiles):
//   1. loads the records of its tiles with the tiles' first in-bracket keys (head-major slots,
//      when the sequence fits one round; a pair of lanes per tile, eight slots each, so that a
//      wave's loads read consecutive tiles) and sums the counts below and inside the bracket; the
//      target rank r lies inside when #below < r <= #below + #inside;
//   2. counts the in-bracket keys per top digit (kDigit bits of key - lo) in LDS, straight from
//      the registers (the rare keys past a tile's slots are read into LDS first), finds the
//      answer's digit and ranks that digit's keys, picked from the registers again (one wave when
//      there are at most 64, else a radix select).
// A row of at most kCap keys has no bracket and is ranked from the score row itself
// (f2_short_row_rank).  A rank outside the bracket, more overflow keys than LDS holds or a
// sequence of more than one round take the out-of-line paths: an LDS histogram of the digits
// over the keys in memory, or a radix select over the instance's whole score row (same result).
// The state gets the answer's key and the number of keys above it, as th_final_kernel leaves them.
constexpr int kF2Threads = 512;
constexpr int kF2Per = 5;                                  // consecutive tiles per thread per round
constexpr int kF2Round = kF2Threads * kF2Per;              // tiles per round (163840 tokens)
constexpr int kF2Cap = 20480;                              // in-bracket keys held in LDS
constexpr int kF2Batch = 8;                                // LDS keys read per thread before use

struct F2Args {
    const uint32_t* tinfo;   // [Hq][ntiles] below | inside << 8 | offset << 16
    const uint32_t* cand;    // [Hq][ntiles][kClsSlots] first in-bracket keys
    const uint32_t* tcand;   // [ntiles][tstride] the other in-bracket keys
    int64_t ntiles;
    int64_t tstride;         // u32 words per tile in tcand
    uint2* phpre;            // nullable [Hq][ntiles]: per 64-token chunk, the (above, equal) key counts
                             // of the chunks before it in the sequence (the per-head compaction's input)
};

// Per-chunk (above, equal) counts of the keys of a score row at positions [beg, end) against the
// key ks, as exclusive prefixes over the sequence's nt chunks of 64 tokens, into pre[0 .. nt).
// Thread t takes a contiguous run of chunks; the counts go to `pre` first and are turned into
// prefixes in place.  (Out of line: used only after the rare whole-row and from-memory paths.)
__device__ __noinline__ void f2_prefix_from_row(const float* row, int64_t nt, int64_t beg, int64_t end, uint32_t ks,
                                                uint2* pre, int* tmp) {
    const int t = threadIdx.x;
    const int64_t per = (nt + kF2Threads - 1) / kF2Threads;
    const int64_t c0 = (int64_t)t * per, c1 = c0 + per < nt ? c0 + per : nt;
    int sg = 0, se = 0;
    for (int64_t c = c0; c < c1; ++c) {
        const int64_t a = 64 * c > beg ? 64 * c : beg, e = 64 * c + 64 < end ? 64 * c + 64 : end;
        uint32_t g = 0, q = 0;
        for (int64_t i = a; i < e; ++i) {
            const uint32_t k = order_key(row[i]);
            g += k > ks ? 1u : 0u;
            q += k == ks ? 1u : 0u;
        }
        pre[c] = make_uint2(g, q);
        sg += (int)g;
        se += (int)q;
    }
    int tg = 0, te = 0;
    const int ig = block_inclusive_scan<kF2Threads>(sg, tmp, &tg);
    const int ie = block_inclusive_scan<kF2Threads>(se, tmp, &te);
    uint32_t ag = (uint32_t)(ig - sg), ae = (uint32_t)(ie - se);
    for (int64_t c = c0; c < c1; ++c) {
        const uint2 v = pre[c];
        pre[c] = make_uint2(ag, ae);
        ag += v.x;
        ae += v.y;
    }
}

// The rank-r key (1-based) of a score row over [beg, end) by a whole-row radix select; *gt gets
// the number of keys above it.  (Out of line: the common path is register-allocated alone.)
__device__ __noinline__ uint32_t f2_rank_row(const float* row, int64_t beg, int64_t end, int64_t r, uint32_t* hist,
                                             int* tmp, int64_t* sh, int64_t* gt) {
    *gt = 0;
    return radix_rank<kF2Threads>(
        [&](auto f) {
            for_each_f32<kF2Threads, 4>(row, beg, end, [&](int64_t, float v, bool ok) {
                if (ok) f(order_key(v));
            });
        },
        32, r, hist, tmp, sh, gt);
}

// The in-bracket keys of the instance, f(key) once each (every thread of the block calls it).
template <class F>
__device__ __forceinline__ void f2_each_cand(const uint32_t* inf_h, const uint32_t* cand_h, const uint32_t* over,
                                             int64_t nt, int64_t tstride, F f) {
    for (int64_t r0 = 0; r0 < nt; r0 += kF2Round)
        for (int u = 0; u < kF2Per; ++u) {
            const int64_t T = r0 + (int64_t)kF2Per * threadIdx.x + u;
            if (T >= nt) continue;
            const uint32_t w = inf_h[T];
            const int cnt = (int)((w >> 8) & 0xffu);
            for (int j = 0; j < cnt; ++j)
                f(j < kClsSlots ? cand_h[T * kClsSlots + j] : over[(size_t)T * tstride + (w >> 16) + (j - kClsSlots)]);
        }
}

// The answer's digit D among kDigitBins digit counts in `hist` (every thread calls it): sh[0] = D,
// sh[1] = keys below D, sh[2] = keys above D, sh[3] = keys in D.
__device__ __forceinline__ void f2_find_digit(const uint32_t* hist, int64_t rr, int* tmp, int64_t* sh) {
    constexpr int BPT = kDigitBins / kF2Threads;
    const int t = threadIdx.x;
    int c = 0;
#pragma unroll
    for (int u = 0; u < BPT; ++u) c += (int)hist[t * BPT + u];
    int tot;
    const int inc = block_inclusive_scan<kF2Threads>(c, tmp, &tot);
    if (inc - c < rr && rr <= inc) {
        int acc = inc - c;
#pragma unroll
        for (int u = 0; u < BPT; ++u) {
            const int bin = t * BPT + u;
            const int nx = acc + (int)hist[bin];
            if (acc < rr && rr <= nx) {
                sh[0] = bin;
                sh[1] = acc;
                sh[2] = tot - nx;
                sh[3] = hist[bin];
            }
            acc = nx;
        }
    }
    __syncthreads();
}

// Rank rr (1-based) among the nD keys (values below 2^nbits) that visit(f) hands over;
// *gt gets the keys above it.  At most 64 keys: one wave ranks them from `xd`; else a radix select.
template <class Visit>
__device__ __forceinline__ uint32_t f2_rank_keys(Visit visit, int nD, int nbits, int64_t rr, uint32_t* xd,
                                                 uint32_t* cursor, uint32_t* hist, int* tmp, int64_t* sh,
                                                 int64_t* gt) {
    const int t = threadIdx.x;
    if (nD <= 64) {
        visit([&](uint32_t x) { xd[atomicAdd(cursor, 1u)] = x; });
        __syncthreads();
        if (t < 64) {
            const bool has = t < nD;
            const uint32_t x = has ? xd[t] : 0xffffffffu;
            int less = 0, leq = 0;
            for (int j = 0; j < nD; ++j) {
                const uint32_t y = __shfl(x, j, 64);
                less += y < x ? 1 : 0;
                leq += y <= x ? 1 : 0;
            }
            if (has && less < rr && rr <= leq) {       // the answer x: #{< x} < rr <= #{<= x}
                sh[0] = x;
                sh[1] = nD - leq;
            }
        }
        __syncthreads();
        *gt += sh[1];
        return (uint32_t)sh[0];
    }
    int64_t gin = 0;
    const uint32_t xl = radix_rank<kF2Threads>(visit, nbits, rr, hist, tmp, sh, &gin);
    *gt += gin;
    return xl;
}

// Rank rr (1-based) among the nD keys src[0 .. nD) in LDS (values below 2^nbits); *gt gets the
// keys above it.  At most 64 keys: one wave ranks them; else a radix select.
__device__ __forceinline__ uint32_t f2_rank_lds(const uint32_t* src, int nD, int nbits, int64_t rr, uint32_t* hist,
                                                int* tmp, int64_t* sh, int64_t* gt) {
    const int t = threadIdx.x;
    if (nD <= 64) {
        if (t < 64) {
            const bool has = t < nD;
            const uint32_t x = has ? src[t] : 0xffffffffu;
            int less = 0, leq = 0;
            for (int j = 0; j < nD; ++j) {
                const uint32_t y = __shfl(x, j, 64);
                less += y < x ? 1 : 0;
                leq += y <= x ? 1 : 0;
            }
            if (has && less < rr && rr <= leq) {       // the answer x: #{< x} < rr <= #{<= x}
                sh[0] = x;
                sh[1] = nD - leq;
            }
        }
        __syncthreads();
        *gt += sh[1];
        return (uint32_t)sh[0];
    }
    int64_t gin = 0;
    const uint32_t xl = radix_rank<kF2Threads>(
        [&](auto f) {
            for (int i = t; i < nD; i += kF2Threads) f(src[i]);
        },
        nbits, rr, hist, tmp, sh, &gin);
    *gt += gin;
    return xl;
}

// Rank rr of the low dsh bits among the keys x that visit(f) hands over with (x >> dsh) == D.
template <class Visit>
__device__ __forceinline__ uint32_t f2_rank_in_digit(Visit visit, int nD, uint32_t D, int dsh, int64_t rr,
                                                     uint32_t* xd, uint32_t* cursor, uint32_t* hist, int* tmp,
                                                     int64_t* sh, int64_t* gt) {
    const uint32_t low = dsh ? ((1u << dsh) - 1u) : 0u;
    return f2_rank_keys(
        [&](auto f) {
            visit([&](uint32_t x) {
                if ((x >> dsh) == D) f(x & low);
            });
        },
        nD, dsh, rr, xd, cursor, hist, tmp, sh, gt);
}

// The rank-r key (1-based) of a row of at most kCap keys over [beg, end) (rows prep leaves without
// a bracket), the row read once, coalesced, into registers.  The keys are counted in kDigitBins
// equal-width bins of the value range [vmin, vmax]: bin(v) = floor((v - vmin) * kDigitBins /
// (vmax - vmin)), clamped, is non-decreasing in v whatever the fp32 rounding, so every key of a
// lower bin is smaller, and the bins spread the keys evenly where the scores are dense (the top
// bits of the order keys would put a quarter of an octave, hundreds of keys, in one bin).  The
// answer's bin is found from the counts and its keys are ranked exactly.  *gt gets the number of
// keys above the answer.
__device__ __forceinline__ uint32_t f2_short_row_rank(const float* row, int64_t beg, int64_t m, int64_t r,
                                                      uint32_t* hist, float* red, uint32_t* xd, uint32_t* cursor,
                                                      int* tmp, int64_t* sh, int64_t* gt, uint2* pre, int64_t nt) {
    constexpr int KPT = kCap / kF2Threads;
    constexpr int NW = kF2Threads / 64;
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    // slot u of every thread holds key t + u kF2Threads; slots u >= nu (uniform) are not used
    const int nu = (int)((m + kF2Threads - 1) / kF2Threads);
    float v[KPT];
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
        const int64_t i = t + (int64_t)u * kF2Threads;
        v[u] = u < nu ? row[beg + (i < m ? i : 0)] : 0.f;   // past the end: the first value again
    }
    float mn = v[0], mx = v[0];
#pragma unroll
    for (int u = 1; u < KPT; ++u)
        if (u < nu) {
            mn = fminf(mn, v[u]);
            mx = fmaxf(mx, v[u]);
        }
    for (int o = 32; o > 0; o >>= 1) {
        mn = fminf(mn, __shfl_xor(mn, o, 64));
        mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    }
    for (int i = t; i < kDigitBins; i += kF2Threads) hist[i] = 0;
    if (lane == 0) {
        red[wid] = mn;
        red[NW + wid] = mx;
    }
    __syncthreads();
    float vmin = red[0], vmax = red[NW];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
        vmin = fminf(vmin, red[w]);
        vmax = fmaxf(vmax, red[NW + w]);
    }
    const float span = vmax - vmin;
    const float scale = (span > 0.f && span < INFINITY) ? (float)kDigitBins / span : 0.f;
    auto bin_of = [&](float x) {
        const float f = (x - vmin) * scale;
        return f >= (float)(kDigitBins - 1) ? kDigitBins - 1 : (int)f;
    };
#pragma unroll
    for (int u = 0; u < KPT; ++u)
        if (u < nu && t + (int64_t)u * kF2Threads < m) atomicAdd(&hist[bin_of(v[u])], 1u);
    __syncthreads();
    f2_find_digit(hist, r, tmp, sh);
    const int D = (int)sh[0];
    const int64_t rr = r - sh[1];
    const int nD = (int)sh[3];
    *gt = sh[2];
    __syncthreads();
    const uint32_t ks = f2_rank_keys(
        [&](auto f) {
#pragma unroll
            for (int u = 0; u < KPT; ++u)
                if (u < nu && t + (int64_t)u * kF2Threads < m && bin_of(v[u]) == D) f(order_key(v[u]));
        },
        nD, 32, rr, xd, cursor, hist, tmp, sh, gt);
    if (pre) {
        // per-chunk (above, equal) counts of the row's keys against the answer: the row's chunks
        // cb .. cb + nc - 1 (at most 258) counted in LDS (above in hist[c], equal in hist[512 + c]),
        // then exclusive prefixes over the sequence's nt chunks
        const int64_t cb = beg >> 6;
        const int nc = (int)(((beg + m - 1) >> 6) - cb + 1);
        __syncthreads();
        for (int i = t; i < 1024; i += kF2Threads) hist[i] = 0;
        __syncthreads();
#pragma unroll
        for (int u = 0; u < KPT; ++u)
            if (u < nu && t + (int64_t)u * kF2Threads < m) {
                const uint32_t k = order_key(v[u]);
                const int c = (int)(((beg + t + (int64_t)u * kF2Threads) >> 6) - cb);
                if (k > ks) atomicAdd(&hist[c], 1u);
                else if (k == ks) atomicAdd(&hist[512 + c], 1u);
            }
        __syncthreads();
        const int cg = t < nc ? (int)hist[t] : 0, ce = t < nc ? (int)hist[512 + t] : 0;
        int tg = 0, te = 0;
        const int ig = block_inclusive_scan<kF2Threads>(cg, tmp, &tg);
        const int ie = block_inclusive_scan<kF2Threads>(ce, tmp, &te);
        if (t < nc) pre[cb + t] = make_uint2((uint32_t)(ig - cg), (uint32_t)(ie - ce));
        for (int64_t c = t; c < cb; c += kF2Threads) pre[c] = make_uint2(0u, 0u);
        for (int64_t c = cb + nc + t; c < nt; c += kF2Threads) pre[c] = make_uint2((uint32_t)tg, (uint32_t)te);
    }
    return ks;
}

// Rank rr0 among the in-bracket keys [klo, khi] read from memory (keys that do not fit in LDS,
// sequences of more than one round): an LDS histogram of their top digit, then the digit's keys.
// Returns false when that digit holds more than kF2Cap keys.  *gt gets the in-bracket keys above.
__device__ __noinline__ bool f2_rank_digit(const uint32_t* inf_h, const uint32_t* cand_h, const uint32_t* over,
                                           int64_t nt, int64_t tstride, uint32_t klo, uint32_t khi, int64_t rr0, uint32_t* xs,
                                           uint32_t* xd, uint32_t* hist, int* tmp, int64_t* sh, uint32_t* cursor,
                                           uint32_t* key, int64_t* gt) {
    const int t = threadIdx.x;
    const int dsh = top_shift(khi - klo);
    for (int i = t; i < kDigitBins; i += kF2Threads) hist[i] = 0;
    if (t == 0) *cursor = 0;
    __syncthreads();
    f2_each_cand(inf_h, cand_h, over, nt, tstride, [&](uint32_t k) { atomicAdd(&hist[(k - klo) >> dsh], 1u); });
    __syncthreads();
    f2_find_digit(hist, rr0, tmp, sh);
    const uint32_t D = (uint32_t)sh[0];
    const int64_t rr = rr0 - sh[1];
    const int64_t gt_d = sh[2];
    const int64_t nD = sh[3];
    __syncthreads();
    if (nD > kF2Cap) return false;
    // the digit's keys (their low dsh bits) into LDS, then ranked there
    const uint32_t low = dsh ? ((1u << dsh) - 1u) : 0u;
    f2_each_cand(inf_h, cand_h, over, nt, tstride, [&](uint32_t k) {
        if (((k - klo) >> dsh) == D) xs[atomicAdd(cursor, 1u)] = (k - klo) & low;
    });
    __syncthreads();
    if (t == 0) *cursor = 0;
    __syncthreads();
    int64_t g = gt_d;
    const uint32_t xl = f2_rank_in_digit(
        [&](auto f) {
            for (int i = t; i < nD; i += kF2Threads) f(xs[i]);
        },
        (int)nD, 0u, dsh, rr, xd, cursor, hist, tmp, sh, &g);
    *key = klo + ((D << dsh) | xl);
    *gt = g;
    return true;
}

// PRE: also the per-chunk prefixes of the per-head compaction (a.phpre).
template <bool PRE>
__global__ __launch_bounds__(kF2Threads) void th_final2_kernel(const float* __restrict__ scores, I64Arg offsets,
                                                              int Hq, DevCfg cfg, int64_t S, F2Args a,
                                                              int64_t* __restrict__ state,
                                                              float* __restrict__ theta_out) {
    __shared__ uint32_t xs[kF2Cap];                          // the in-bracket keys, in tile order
    __shared__ uint16_t xt[PRE ? kF2Cap : 1];                // PRE: the tile of each key
    __shared__ int tp[kF2Round + 1];                         // tile T's keys: xs[tp[T] .. tp[T + 1])
    __shared__ uint32_t tc[PRE ? kF2Round : 1];              // PRE: per tile, above | equal << 16
    __shared__ uint32_t hist[kDigitBins];
    __shared__ uint32_t dummy[64];                           // spare words of writes that are not needed
    __shared__ uint16_t dummyt[PRE ? 64 : 1];
    __shared__ uint32_t xd[64];
    __shared__ int tmp[kF2Threads / 64];
    __shared__ int tmp3[3][kF2Threads / 64];
    __shared__ int64_t sh[4];
    __shared__ uint32_t cursor;
    const int inst = blockIdx.x, b = inst / Hq, h = inst % Hq, t = threadIdx.x, lane = t & 63;
    int64_t* st = state + (int64_t)inst * 8;
    const int64_t off = offsets[b], n = offsets[b + 1] - off;
    const OsInst oi = os_instance(n, cfg);
    const int64_t m = oi.end - oi.beg;
    const bool active = oi.flag == kFlagActive;
    if (t == 0) cursor = 0;
    if (!active || m <= kCap) {
        // ---- no order statistic, or a row prep leaves without a bracket: ranked from the row itself
        int64_t gt = 0;
        uint32_t key = 0;
        if (active) {
            uint2* pre = nullptr;
            if (PRE)
                pre = a.phpre + (size_t)h * a.ntiles +
                      wave_prefix_seq(b, [od = offsets.dev](int i) { return (od[i + 1] - od[i] + 63) / 64; });
            key = f2_short_row_rank(scores + (int64_t)h * S + off, oi.beg, m, oi.rank, hist,
                                    reinterpret_cast<float*>(tmp3), xd, &cursor, tmp, sh, &gt, pre, (n + 63) / 64);
        }
        if (t == 0) {
            st[kStKey] = key;
            st[kStGt] = gt;
            if (cfg.mode == 0 && theta_out) theta_out[inst] = active ? key_to_float(key) : 0.f;
        }
        return;
    }
    const int64_t tf = wave_prefix_seq(b, [od = offsets.dev](int i) { return (od[i + 1] - od[i] + 63) / 64; });
    const int64_t nt = (n + 63) / 64;
    const size_t hrow = (size_t)h * a.ntiles + tf;
    const uint32_t* inf_h = a.tinfo + hrow;
    const uint32_t* cand_h = a.cand + hrow * kClsSlots;
    const uint32_t* over = a.tcand + (size_t)tf * a.tstride;     // overflow keys of the sequence's tiles
    const bool one = nt <= kF2Round;                   // one round: the keys load with the records

    // ---- 1. records and slot keys: one memory round trip.  Thread t takes the records of the
    // kF2Per consecutive tiles kF2Per t + u; the slot keys are read in 16-byte chunks in a
    // coalesced order (chunk g = r kF2Threads + t holds slots 4 (g % 4) .. of tile g / 4).  Tiles
    // past nt read tile 0 (in bounds) and count nothing; the bracket is read after these loads.
    constexpr int kChunks = kF2Round * (kClsSlots / 4) / kF2Threads;
    uint32_t w[kF2Per];
    uint4 kc[kChunks];
#pragma unroll
    for (int u = 0; u < kF2Per; ++u) {
        const int64_t T = (int64_t)kF2Per * t + u;
        w[u] = inf_h[T < nt ? T : 0];
    }
    if (one) {
#pragma unroll
        for (int r2 = 0; r2 < kChunks; ++r2) {
            const int g = r2 * kF2Threads + t, T = g / (kClsSlots / 4);
            kc[r2] = reinterpret_cast<const uint4*>(cand_h + (int64_t)(T < nt ? T : 0) * kClsSlots)[g % (kClsSlots / 4)];
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t klo = (uint32_t)st[kStLo], khi = (uint32_t)st[kStHi];
    const int dsh = top_shift(khi - klo);
    for (int i = t; i < kDigitBins; i += kF2Threads) hist[i] = 0;
    int lsum = 0, csum = 0, ov0 = 0;
#pragma unroll
    for (int u = 0; u < kF2Per; ++u) {
        if ((int64_t)kF2Per * t + u >= nt) w[u] = 0;
        const int c = (int)((w[u] >> 8) & 0xffu);
        lsum += (int)(w[u] & 0xffu);
        csum += c;
        ov0 += c > kClsSlots ? c - kClsSlots : 0;
    }
    for (int64_t r0 = kF2Round; r0 < nt; r0 += kF2Round)
#pragma unroll
        for (int u = 0; u < kF2Per; ++u) {
            const int64_t T = r0 + (int64_t)kF2Per * t + u;
            const uint32_t x = T < nt ? inf_h[T] : 0u;
            lsum += (int)(x & 0xffu);
            csum += (int)((x >> 8) & 0xffu);
        }
    int nlo = 0, nmid = 0, novf = 0;
    const int cinc = block_inclusive_scan3<kF2Threads>(lsum, ov0, csum, tmp3, &nlo, &novf, &nmid);
    const int64_t r = oi.rank;
    bool whole_row = !(nlo < r && r <= (int64_t)nlo + nmid);
    uint32_t key = 0;
    int64_t gt = 0;
    bool regs = false;                 // the in-bracket keys sit in LDS in tile order (tp), or klo == khi
    if (!whole_row) {
        gt = m - nlo - nmid;                              // keys above the bracket
        const int64_t rr0 = r - nlo;
        if (klo == khi) {
            key = klo;                                    // every in-bracket key is the answer
            regs = one;
        } else {
            bool from_mem = !(one && nmid <= kF2Cap);
            if (!from_mem) {
                // ---- 2. the in-bracket keys (minus klo) into LDS in tile order: tile T's keys at
                // xs[tp[T] .. tp[T + 1]), its slots' keys from the registers, the rest (rare) from
                // memory in batches of 8 loads
                int pos = cinc - csum;
#pragma unroll
                for (int u = 0; u < kF2Per; ++u) {
                    const int64_t T = (int64_t)kF2Per * t + u;
                    if (T < nt) tp[T] = pos;
                    pos += (int)((w[u] >> 8) & 0xffu);
                }
                if (t == 0) tp[nt] = nmid;
                if (PRE)
                    for (int i = t; i < nt; i += kF2Threads) tc[i] = 0u;
                __syncthreads();
                // every chunk's table entries first (one LDS wait), then its keys: slots past the
                // tile's count (and chunks past nt) write to a spare word instead
                int b0[kChunks], c0[kChunks];
#pragma unroll
                for (int r2 = 0; r2 < kChunks; ++r2) {
                    const int T = (r2 * kF2Threads + t) / (kClsSlots / 4);
                    const int Tc = T < nt ? T : (int)nt;
                    b0[r2] = tp[Tc];
                    c0[r2] = T < nt ? tp[Tc + 1] : 0;
                }
#pragma unroll
                for (int r2 = 0; r2 < kChunks; ++r2) {
                    const int g = r2 * kF2Threads + t, T = g / (kClsSlots / 4), j0 = 4 * (g % (kClsSlots / 4));
                    const int c = c0[r2] - b0[r2];
                    const uint32_t x4[4] = {kc[r2].x, kc[r2].y, kc[r2].z, kc[r2].w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const bool ok = j0 + i < c;
                        const int at = b0[r2] + j0 + i;
                        *(ok ? &xs[at] : &dummy[lane]) = x4[i] - klo;
                        if (PRE) *(ok ? &xt[at] : &dummyt[lane]) = (uint16_t)T;
                    }
                }
                if (novf > 0) {
#pragma unroll
                    for (int u = 0; u < kF2Per; ++u) {
                        const int64_t T = (int64_t)kF2Per * t + u;
                        const int cnt = (int)((w[u] >> 8) & 0xffu);
                        if (cnt <= kClsSlots) continue;
                        const uint32_t* ov = over + (size_t)T * a.tstride + (w[u] >> 16);
                        const int tb = tp[T];
                        for (int j0 = kClsSlots; j0 < cnt; j0 += 8) {
                            uint32_t x8[8];
#pragma unroll
                            for (int v = 0; v < 8; ++v) x8[v] = ov[(j0 + v < cnt ? j0 + v : j0) - kClsSlots];
#pragma unroll
                            for (int v = 0; v < 8; ++v)
                                if (j0 + v < cnt) {
                                    xs[tb + j0 + v] = x8[v] - klo;
                                    if (PRE) xt[tb + j0 + v] = (uint16_t)T;
                                }
                        }
                    }
                }
                __syncthreads();
                // ---- 3. the answer's digit, then its keys ranked (the loops over the keys read 8
                // keys per thread before they update LDS, so that the reads overlap)
                for (int i0 = t; i0 < nmid; i0 += kF2Batch * kF2Threads) {
                    uint32_t x[kF2Batch];
#pragma unroll
                    for (int k = 0; k < kF2Batch; ++k) x[k] = xs[min(i0 + k * kF2Threads, kF2Cap - 1)];
#pragma unroll
                    for (int k = 0; k < kF2Batch; ++k)
                        if (i0 + k * kF2Threads < nmid) atomicAdd(&hist[x[k] >> dsh], 1u);
                }
                __syncthreads();
                f2_find_digit(hist, rr0, tmp, sh);
                const uint32_t D = (uint32_t)sh[0];
                const int64_t rr = rr0 - sh[1];
                const int nD = (int)sh[3];
                const int64_t gt_d = sh[2];
                __syncthreads();
                if (nD > 64 && nmid + nD > kF2Cap) {
                    from_mem = true;                      // the digit does not fit beside the keys
                } else {
                    // the digit's keys (low bits) into xd for at most 64, else after the keys
                    const uint32_t low = dsh ? ((1u << dsh) - 1u) : 0u;
                    uint32_t* dst = nD <= 64 ? xd : xs + nmid;
                    for (int i0 = t; i0 < nmid; i0 += kF2Batch * kF2Threads) {
                        uint32_t x[kF2Batch];
#pragma unroll
                        for (int k = 0; k < kF2Batch; ++k) x[k] = xs[min(i0 + k * kF2Threads, kF2Cap - 1)];
#pragma unroll
                        for (int k = 0; k < kF2Batch; ++k)
                            if (i0 + k * kF2Threads < nmid && (x[k] >> dsh) == D) dst[atomicAdd(&cursor, 1u)] = x[k] & low;
                    }
                    __syncthreads();
                    gt += gt_d;
                    const uint32_t xl = f2_rank_lds(dst, nD, dsh, rr, hist, tmp, sh, &gt);
                    key = klo + ((D << dsh) | xl);
                    regs = true;
                }
            }
            if (from_mem) {
                // ---- 2'. from memory: an LDS histogram of the in-bracket keys' digits, then the
                // digit's keys
                uint32_t kd = 0;
                int64_t gd = 0;
                __syncthreads();
                if (f2_rank_digit(inf_h, cand_h, over, nt, a.tstride, klo, khi, rr0, xs, xd, hist, tmp, sh, &cursor, &kd, &gd)) {
                    key = kd;
                    gt += gd;
                } else {
                    whole_row = true;
                }
            }
        }
    }
    if (whole_row)   // the answer lies outside the bracket (or its digit overflows LDS): the whole row
        key = f2_rank_row(scores + (int64_t)h * S + off, oi.beg, oi.end, r, hist, tmp, sh, &gt);
    if (t == 0) {
        st[kStKey] = key;
        st[kStGt] = gt;
        if (cfg.mode == 0 && theta_out) theta_out[inst] = key_to_float(key);
    }
    if (PRE) {
        // per-chunk (above, equal) counts against the answer, as exclusive prefixes
        uint2* pre = a.phpre + hrow;
        if (regs && !whole_row) {
            // from the records: a tile's keys above the bracket are above the answer, those below
            // it below; its in-bracket keys above / equal to the answer are counted per tile with
            // one pass over the keys in LDS (all equal when klo == khi)
            if (klo != khi) {
                const uint32_t xa = key - klo;
                for (int i0 = t; i0 < nmid; i0 += kF2Batch * kF2Threads) {
                    uint32_t x[kF2Batch];
                    uint16_t tt[kF2Batch];
#pragma unroll
                    for (int k = 0; k < kF2Batch; ++k) {
                        const int i = min(i0 + k * kF2Threads, (PRE ? kF2Cap : 1) - 1);   // in bounds
                        x[k] = xs[i];
                        tt[k] = xt[i];
                    }
#pragma unroll
                    for (int k = 0; k < kF2Batch; ++k)
                        if (i0 + k * kF2Threads < nmid && x[k] >= xa) atomicAdd(&tc[tt[k]], x[k] > xa ? 1u : 0x10000u);
                }
                __syncthreads();
            }
            int tg[kF2Per], te[kF2Per];
            int sg = 0, se = 0;
#pragma unroll
            for (int u = 0; u < kF2Per; ++u) {
                const int64_t T = (int64_t)kF2Per * t + u;
                const int cnt = (int)((w[u] >> 8) & 0xffu);
                int g = 0, e = 0;
                if (klo == khi) {
                    e = cnt;
                } else if (T < nt) {
                    const uint32_t v = tc[T];
                    g = (int)(v & 0xffffu);
                    e = (int)(v >> 16);
                }
                const int64_t pa = 64 * T > oi.beg ? 64 * T : oi.beg, pe = 64 * T + 64 < oi.end ? 64 * T + 64 : oi.end;
                const int valid = (T < nt && pe > pa) ? (int)(pe - pa) : 0;
                tg[u] = g + valid - (int)(w[u] & 0xffu) - cnt;
                te[u] = e;
                sg += tg[u];
                se += te[u];
            }
            int tgs = 0, tes = 0;
            const int ig = block_inclusive_scan<kF2Threads>(sg, tmp, &tgs);
            const int ie = block_inclusive_scan<kF2Threads>(se, tmp, &tes);
            uint32_t ag = (uint32_t)(ig - sg), ae = (uint32_t)(ie - se);
#pragma unroll
            for (int u = 0; u < kF2Per; ++u) {
                const int64_t T = (int64_t)kF2Per * t + u;
                if (T < nt) pre[T] = make_uint2(ag, ae);
                ag += (uint32_t)tg[u];
                ae += (uint32_t)te[u];
            }
        } else {
            __syncthreads();
            f2_prefix_from_row(scores + (int64_t)h * S + off, nt, oi.beg, oi.end, key, pre, tmp);
        }
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
    int64_t nitems, ph_items, Ntot, ntiles;
    uint32_t *cand, *cnt, *dhist, *hist, *phcnt;
    int64_t* state;
    size_t state_off;   // byte offset of `state` in the workspace
    uint8_t *votes, *keys;
    float* qp;          // fused path: q' per (sequence, head)
    uint32_t* tinfo;    // fused path: per (head, tile) counts below / inside the bracket, key offset
    uint32_t* hcand;    // fused path: per (head, tile) the first in-bracket keys
    uint32_t* tcand;    // fused path: per tile the heads' keys inside the bracket
    size_t bytes;
};

// fused: the score-and-select path (tile classification instead of the slice candidates).
static SelectLayout select_layout(void* ws, const int64_t* offsets_host, int B, int Hq, const SelectConfig& c,
                                  bool fused = false) {
    SelectLayout L;
    DevCfg d = dev_cfg(c);
    int64_t maxm = 0, items = 0, ph_items = 0, tiles = 0;
    for (int b = 0; b < B; ++b) {
        int64_t n = offsets_host[b + 1] - offsets_host[b];
        OsInst o = os_instance(n, d);
        if (o.end - o.beg > maxm) maxm = o.end - o.beg;
        items += (n + kChunk - 1) / kChunk;
        ph_items += (n + kPhChunk - 1) / kPhChunk;
        tiles += (n + 63) / 64;
    }
    L.ph_items = ph_items;
    L.SL = (int)((maxm + kSlice - 1) / kSlice);
    if (L.SL < 1) L.SL = 1;
    L.nitems = items;
    L.ntiles = tiles;
    L.Ntot = offsets_host[B];
    WsCarver w(ws);
    const size_t inst = (size_t)B * Hq;
    L.cand = L.cnt = L.dhist = L.phcnt = nullptr;
    L.qp = nullptr;
    L.tinfo = nullptr;
    L.hcand = nullptr;
    L.tcand = nullptr;
    if (fused) {
        L.qp = w.take<float>(inst * kDP);
        L.tinfo = w.take<uint32_t>((size_t)Hq * tiles);
        L.hcand = w.take<uint32_t>((size_t)Hq * tiles * kClsSlots);
        L.tcand = w.take<uint32_t>((size_t)tiles * kClsTile);
    } else {
        L.cand = w.take<uint32_t>(inst * L.SL * kSlice);
        L.cnt = w.take<uint32_t>(inst * L.SL * 2);
        L.dhist = w.take<uint32_t>(inst * L.SL * kDpWords);
    }
    L.phcnt = c.mode == 1 ? w.take<uint32_t>((size_t)Hq * ph_items * 2) : nullptr;
    L.state_off = w.size();
    L.state = w.take<int64_t>(inst * 8);
    L.votes = w.take<uint8_t>((size_t)L.Ntot + 16);
    L.keys = w.take<uint8_t>((size_t)L.Ntot + 16);
    L.hist = w.take<uint32_t>((size_t)items * kVoteBins);
    L.bytes = w.size();
    return L;
}

size_t select_workspace(const int64_t* offsets_host, int B, int Hq, const SelectConfig& c) {
    return select_layout(nullptr, offsets_host, B, Hq, c).bytes;
}

size_t score_select_workspace(const int64_t* offsets_host, int B, int Hq, const SelectConfig& c) {
    return select_layout(nullptr, offsets_host, B, Hq, c, true).bytes;
}

size_t score_select_state_offset(const int64_t* offsets_host, int B, int Hq, const SelectConfig& c) {
    return select_layout(nullptr, offsets_host, B, Hq, c, true).state_off;
}

// Votes and the ordered compaction (vote mode) or the per-head compaction, once the order
// statistics are in the state.
// prefixed: the per-head chunk prefixes are already in L.phcnt (th_final2 writes them).
static hipError_t launch_select_tail(const SelectLayout& L, const float* scores, int64_t S, const I64Arg& offs,
                                     int B, int Hq, const SelectConfig& c, int32_t* idx_out, int64_t* count_out,
                                     uint8_t* votes_out, hipStream_t stream, bool prefixed = false) {
    DevCfg d = dev_cfg(c);
    if (L.nitems == 0) return hipGetLastError();
    if (c.mode == 0) {
        uint8_t* votes = votes_out ? votes_out : L.votes;
        hipLaunchKernelGGL(vote_kernel, dim3((unsigned)L.nitems), dim3(kChunk), 0, stream, scores, offs,
                           B, Hq, d, S, L.state, votes, L.keys, L.hist);
        hipLaunchKernelGGL(compact_vote_kernel, dim3((unsigned)L.nitems), dim3(kChunk), 0, stream, offs,
                           B, d, L.keys, L.hist, idx_out, count_out);
    } else {
        const dim3 phg((unsigned)((L.ph_items + kPhWaves - 1) / kPhWaves));
        const int hpw = B == 1 ? 8 : 32;
        const int64_t cw = L.ph_items * ((Hq + hpw - 1) / hpw);
        const dim3 phcg((unsigned)((cw + kPhWaves - 1) / kPhWaves));
        if (!prefixed) {
            hipLaunchKernelGGL(ph_count_kernel, phg, dim3(kPhWaves * 64), 0, stream, scores, offs,
                               B, Hq, d, S, L.state, L.ph_items, L.phcnt);
            hipLaunchKernelGGL(ph_scan_kernel, dim3((unsigned)(B * Hq)), dim3(kPhScanThreads), 0, stream, offs, B,
                               Hq, L.ph_items, L.phcnt);
        }
        if (hpw == 8)
            hipLaunchKernelGGL(ph_compact_kernel<8>, phcg, dim3(kPhWaves * 64), 0, stream, scores,
                               offs, B, Hq, d, S, L.state, L.ph_items, L.phcnt, idx_out, count_out);
        else
            hipLaunchKernelGGL(ph_compact_kernel<32>, phcg, dim3(kPhWaves * 64), 0, stream, scores,
                               offs, B, Hq, d, S, L.state, L.ph_items, L.phcnt, idx_out, count_out);
    }
    return hipGetLastError();
}

hipError_t launch_select(const float* scores, int64_t S, const int64_t* offsets_dev, const int64_t* offsets_host,
                         int B, int Hq, const SelectConfig& c, int32_t* idx_out, int64_t* count_out, float* theta_out,
                         uint8_t* votes_out, void* ws, size_t ws_bytes, hipStream_t stream) {
    SelectLayout L = select_layout(ws, offsets_host, B, Hq, c);
    if (L.bytes > ws_bytes || L.SL > kMaxSL) return hipErrorInvalidValue;
    DevCfg d = dev_cfg(c);
    const unsigned inst = (unsigned)(B * Hq);
    const I64Arg offs = i64_arg(offsets_dev, offsets_host, (int64_t)B + 1);
    hipLaunchKernelGGL(th_collect_kernel, dim3(L.SL, inst), dim3(kColThreads), 0, stream, scores, offs, Hq, d,
                       L.SL, S, L.state, L.cand, L.cnt, L.dhist);
    hipLaunchKernelGGL(th_final_kernel, dim3(inst), dim3(kThThreads), 0, stream, scores, offs, Hq, d, L.SL, S,
                       L.cand, L.cnt, L.dhist, L.state, c.mode == 0 ? theta_out : nullptr);
    return launch_select_tail(L, scores, S, offs, B, Hq, c, idx_out, count_out, votes_out, stream);
}

hipError_t launch_score_select(const uint16_t* q, const float* P, uint16_t* k_index, const uint16_t* K,
                               const int64_t* offsets_dev, const int64_t* offsets_host, int B, int Hq, int Hkv,
                               const SelectConfig& c, float* scores, int32_t* idx_out, int64_t* count_out,
                               float* theta_out, uint8_t* votes_out, void* ws, size_t ws_bytes, hipStream_t stream) {
    SelectLayout L = select_layout(ws, offsets_host, B, Hq, c, true);
    if (L.bytes > ws_bytes) return hipErrorInvalidValue;
    DevCfg d = dev_cfg(c);
    const unsigned inst = (unsigned)(B * Hq);
    const I64Arg offs = i64_arg(offsets_dev, offsets_host, (int64_t)B + 1);
    const int64_t S = score_stride(offsets_host[B]);
    hipLaunchKernelGGL(prep_kernel, dim3(inst + (K ? B : 0)), dim3(kPrepThreads), 0, stream, q, P, k_index, K, offs,
                       B, Hq, Hkv, d, L.qp, L.state);
    hipError_t e = launch_score_classify(L.qp, k_index, offsets_dev, offsets_host, B, Hq, Hkv, scores, L.state, L.tinfo,
                                         L.hcand, L.tcand, stream);
    if (e != hipSuccess) return e;
    // per-head mode: th_final2 also writes the compaction's chunk prefixes (no count and scan kernels)
    const F2Args fa{L.tinfo, L.hcand, L.tcand, L.ntiles, kClsTile,
                    c.mode == 1 ? reinterpret_cast<uint2*>(L.phcnt) : nullptr};
    if (c.mode == 1)
        hipLaunchKernelGGL(th_final2_kernel<true>, dim3(inst), dim3(kF2Threads), 0, stream, scores, offs, Hq, d, S, fa,
                           L.state, theta_out);
    else
        hipLaunchKernelGGL(th_final2_kernel<false>, dim3(inst), dim3(kF2Threads), 0, stream, scores, offs, Hq, d, S, fa,
                           L.state, theta_out);
    return launch_select_tail(L, scores, S, offs, B, Hq, c, idx_out, count_out, votes_out, stream, true);
}

// ------------------------------------------------------------ SnapKV top-c per row
// [SK] "アルゴリズム": the top min(c, n) positions of each KV head's pooled importance, in
// ascending position order; ties at the threshold go to the lower positions.  The rows are few
// (one per KV head) and long, so instead of the general selection:
//   snap_prep_kernel:          per row, a key bracket around the threshold from 4096 sampled
//                              pooled values (rows of more than kCap keys), as prep_kernel does
//                              for index scores from 1024;
//   snap_pool_classify_kernel: pooled[j] = ((imp[j-1] + imp[j]) + imp[j+1]) / 3 (zero outside
//                              [0, n)), written once, and each 64-key tile classified against the
//                              bracket in the score kernel's record layout;
//   th_final2_kernel:          the threshold key, the number of keys above it and each 64-key
//                              chunk's prefix of (above, equal) counts;
//   ph_compact_kernel:         the positions of the keys above the threshold and of the first
//                              (need - #above) keys equal to it, one wave per chunk.
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

// the pooled value at position j of a row of n importances
__device__ __forceinline__ float pooled_at(const float* row, int64_t n, int64_t j) {
    const float a = j > 0 ? row[j - 1] : 0.f;
    const float c = j + 1 < n ? row[j + 1] : 0.f;
    return ((a + row[j]) + c) / 3.0f;
}

constexpr int kSnapSample = 4096;   // sampled pooled values per SnapKV row
constexpr int kSnapDelta = 64;      // bracket half-width in sample ranks
static_assert(kSnapSample % kColThreads == 0 && kSnapSample / kRunLen * kRunLen <= kCap,
              "whole sample passes; a row of more than kCap keys holds every run");
__global__ __launch_bounds__(kPrepThreads) void snap_prep_kernel(const float* __restrict__ imp, int64_t n, DevCfg cfg,
                                                                int64_t* __restrict__ state) {
    constexpr int NW = kPrepThreads / 64;
    __shared__ uint32_t hist[kSampleBins];
    __shared__ float wmin[NW], wmax[NW];
    __shared__ int tmp[NW];
    __shared__ int sb[2];
    const int g = blockIdx.x, t = threadIdx.x;
    const OsInst oi = os_instance(n, cfg);
    const int64_t m = oi.end - oi.beg;
    uint32_t klo = 1u, khi = 0u;                     // no bracket: the empty one (lo > hi)
    if (oi.flag == kFlagActive && m > kCap) {
        // a SnapKV call has few rows (one per KV head), so each row affords 4 times the decode's
        // sample: the bracket (+-64 of 4096 sample ranks, about 6 standard deviations at a 3 %
        // top-c) holds about a third as many keys for the order statistic (at 131072 keys and
        // c = 4096: its kernel 23.3 -> 19.2 us, this one 6.2 -> 8.0 us)
        constexpr int NS = kSnapSample, kSnapRuns = NS / kRunLen;
        const float* row = imp + (int64_t)g * n;
        float v[NS / kColThreads];
#pragma unroll
        for (int u = 0; u < NS / kColThreads; ++u)
            v[u] = pooled_at(row, n, oi.beg + sample_pos(t + u * kColThreads, m, g, kSnapRuns));
        bracket_of_sample<NS, kSnapDelta, true>(v, oi, hist, wmin, wmax, tmp, sb, klo, khi);
    }
    if (t == 0) {
        int64_t* st = state + (int64_t)g * 8;
        st[kStFlag] = oi.flag;
        st[kStNeed] = oi.need;
        st[kStLo] = klo;
        st[kStHi] = khi;
        st[kStBeg] = oi.beg;
        st[kStEnd] = oi.end;
    }
}

// Block = 4 tiles of 64 keys of row g, one wave each; lane = key of the tile.  Records as the
// score kernel's: tinfo[g][tile] = below | inside << 8 | (g * 64) << 16, the first kClsSlots
// in-bracket keys in cand[g][tile][], the rest at tcand[tile * rows * 64 + g * 64 + j - kClsSlots].
constexpr int kSnapTilesPerBlock = 4;
__global__ __launch_bounds__(64 * kSnapTilesPerBlock) void snap_pool_classify_kernel(
    const float* __restrict__ imp, int64_t n, int rows, int64_t ps, const int64_t* __restrict__ state,
    float* __restrict__ pooled, float* __restrict__ pooled_out, uint32_t* __restrict__ tinfo,
    uint32_t* __restrict__ cand, uint32_t* __restrict__ tcand, int64_t ntiles) {
    const int lane = threadIdx.x & 63;
    const int64_t tb = (ntiles + kSnapTilesPerBlock - 1) / kSnapTilesPerBlock;
    const int g = (int)(blockIdx.x / tb);
    const int64_t tile = (blockIdx.x % tb) * kSnapTilesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (tile >= ntiles) return;
    const int64_t* st = state + (int64_t)g * 8;
    const int64_t flag = st[kStFlag];
    const uint32_t lo = (uint32_t)st[kStLo], hi = (uint32_t)st[kStHi];
    const int64_t j = tile * 64 + lane;
    const bool inr = j < n;
    const float v = inr ? pooled_at(imp + (int64_t)g * n, n, j) : 0.f;
    if (inr) {
        pooled[(int64_t)g * ps + j] = v;
        if (pooled_out) pooled_out[(int64_t)g * n + j] = v;
    }
    uint32_t below = 0;
    uint64_t mm = 0;
    const uint32_t key = order_key(v);
    if (flag == kFlagActive && lo <= hi) {
        below = (uint32_t)__popcll(__ballot(inr && key < lo));
        mm = __ballot(inr && key >= lo && key <= hi);
    }
    const uint32_t cnt = (uint32_t)__popcll(mm);
    const size_t r = (size_t)g * ntiles + tile;
    if (lane == 0) tinfo[r] = below | (cnt << 8) | ((uint32_t)(g * 64) << 16);
    if ((mm >> lane) & 1ull) {
        const uint32_t jj = (uint32_t)__popcll(mm & ((1ull << lane) - 1ull));
        if (jj < (uint32_t)kClsSlots) cand[r * kClsSlots + jj] = key;
        else tcand[(size_t)tile * rows * 64 + g * 64 + jj - kClsSlots] = key;
    }
}

struct SnapTopcLayout {
    int64_t ntiles;
    int64_t* state;
    int64_t* count;
    uint32_t *tinfo, *cand, *tcand;
    uint2* pre;
    size_t bytes;
};

static SnapTopcLayout snap_topc_layout(void* ws, int rows, int64_t n) {
    SnapTopcLayout L;
    L.ntiles = (n + 63) / 64;
    WsCarver w(ws);
    L.state = w.take<int64_t>((size_t)rows * 8);
    L.count = w.take<int64_t>(1);
    L.pre = w.take<uint2>((size_t)rows * L.ntiles);
    L.tinfo = w.take<uint32_t>((size_t)rows * L.ntiles);
    L.cand = w.take<uint32_t>((size_t)rows * L.ntiles * kClsSlots);
    L.tcand = w.take<uint32_t>((size_t)L.ntiles * rows * 64);
    L.bytes = w.size();
    return L;
}

size_t snap_topc_workspace(int rows, int64_t n) { return snap_topc_layout(nullptr, rows, n).bytes; }

hipError_t launch_snap_topc(const float* imp, int64_t n, int rows, int64_t c, float* pooled, int64_t ps,
                            float* pooled_out, int32_t* idx_out, void* ws, size_t ws_bytes, hipStream_t stream) {
    SnapTopcLayout L = snap_topc_layout(ws, rows, n);
    if (L.bytes > ws_bytes || n <= 0 || c <= 0) return hipErrorInvalidValue;
    const int64_t ce = c < n ? c : n;
    const DevCfg d = dev_cfg(rows_cfg(n, ce));
    hipLaunchKernelGGL(snap_prep_kernel, dim3(rows), dim3(kPrepThreads), 0, stream, imp, n, d, L.state);
    const int64_t tb = (L.ntiles + kSnapTilesPerBlock - 1) / kSnapTilesPerBlock;
    hipLaunchKernelGGL(snap_pool_classify_kernel, dim3((unsigned)(tb * rows)), dim3(64 * kSnapTilesPerBlock), 0, stream,
                       imp, n, rows, ps, L.state, pooled, pooled_out, L.tinfo, L.cand, L.tcand, L.ntiles);
    // one sequence {0, n} of `rows` instances: the bounds travel as launch arguments
    const int64_t oh[2] = {0, n};
    const I64Arg offs = i64_arg(nullptr, oh, 2);
    const F2Args fa{L.tinfo, L.cand, L.tcand, L.ntiles, (int64_t)rows * 64, L.pre};
    hipLaunchKernelGGL(th_final2_kernel<true>, dim3(rows), dim3(kF2Threads), 0, stream, pooled, offs, rows, d, ps, fa,
                       L.state, nullptr);
    // the per-head compaction: the rows are the heads of one sequence with no forced tokens, so the
    // list of row r is idx_out[r * ce ...]
    const int64_t cw = L.ntiles * ((rows + 7) / 8);
    hipLaunchKernelGGL(ph_compact_kernel<8>, dim3((unsigned)((cw + kPhWaves - 1) / kPhWaves)), dim3(kPhWaves * 64), 0,
                       stream, pooled, offs, 1, rows, d, ps, L.state, L.ntiles, reinterpret_cast<const uint32_t*>(L.pre),
                       idx_out, L.count);
    return hipGetLastError();
}

}  // namespace qasi
