// Sparse (gathered) and dense split-K flash decode with a log-sum-exp merge.
//
// [TS] "Token-Level Selection と Sparse Attention", eq. Attention(Q, K_S, V_S) =
// softmax(Q K_S^T / sqrt(d)) V_S over the selected tokens, which include the sink and local
// tokens; the "output merge" of the five-step integration is the log-sum-exp merge of the
// partial softmax results of disjoint chunks of the list.
//
// Work item (block) = (sequence b, range of EB list entries, KV head g) [vote / dense] or
// (b, range, query head h) [per-head]; blocks of one range are adjacent, so the chip sweeps the
// sorted lists front to back.  EB is chosen on the host so that the grid is about one round of
// resident blocks.  A block has 4 waves; wave w takes the EW = EB / 4 entries
// [w EW, (w+1) EW) of the range and serves the GH query heads that read KV head g (all G heads
// of g in vote / dense mode, one head in per-head mode), so each gathered K/V row is read once
// for the whole GQA group.  A wave works through its entries in sub-batches of 16: a wave is 4
// rows of 16 lanes, row r takes entries 4r .. 4r+3 of the sub-batch and lane p holds dims
// [8p, 8p+8) (one 16-byte load of K and one of V per entry).  A wave issues one sub-batch's K and
// V rows and then computes it; the other waves of the CU (16 resident in the shared-list modes)
// cover the gather latency:
//   z  = q . k * log2(e)/sqrt(128): bf16 pair dot products (exact products, fp32 sums), then a
//        transposed butterfly over the 16 lanes of the row (DPP);
//   online softmax per head over the sub-batches: m, l and acc = sum 2^(z - m) v, rescaled
//        when m grows; the row sums of the accumulators use the gfx950 row swaps;
//   the 4 waves' (m, l, acc) merge in LDS into the block's partial (M, L, A[128]) per head.
// The merge kernel combines the ranges of a sequence: out = sum_c A_c 2^(M_c - M) /
// sum_c L_c 2^(M_c - M).
#include <hip/hip_ext.h>

#include <mutex>

#include "qasi_device.h"
#include "qasi_internal.h"

namespace qasi {

constexpr int kDecWaves = 4;                       // waves per block
constexpr int kDecSub = 16;                        // entries per sub-batch of a wave
constexpr int kDecMaxEW = 512;                     // entries per wave at most
constexpr float kLog2eOverSqrtD = 1.4426950408889634f / 11.313708498984761f;

// query heads served by a wave
__host__ __device__ constexpr int dec_gh(int G, int mode) { return mode == 1 ? 1 : G; }

// lm: list entries per count (the union lists of a KV group hold G * count slots)
__device__ __forceinline__ bool find_list_chunk(const I64Arg& counts, int B, int64_t item, int EB, int lm, int& b,
                                                int64_t& j0, int64_t& len, int64_t& kpre) {
    const SeqPos sp = wave_find_seq(B, item, (lm * counts[0] + EB - 1) / EB,
                                    [cd = counts.dev, EB, lm](int i) { return (lm * cd[i] + EB - 1) / EB; });
    if (sp.b < 0) return false;
    b = sp.b;
    const int64_t n = lm * counts[b];
    j0 = (item - sp.first) * EB;
    len = n - j0 < EB ? n - j0 : EB;
    kpre = wave_prefix_seq(b, [cd = counts.dev](int i) { return cd[i]; });
    return true;
}

// bf16 pair dot product with fp32 accumulation: a.lo*b.lo + a.hi*b.hi + c
typedef __bf16 __attribute__((ext_vector_type(2))) bf16x2_t;
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}

// One step of a transposed butterfly inside a 16-lane row: the lane keeps the half of its N
// values chosen by its lane bit (`upper`) and adds the partner's copy of that half; the
// partner (a DPP lane permutation that flips that bit) keeps the other half.
template <int N, class F>
__device__ __forceinline__ void tstep(const float (&in)[N], float (&out)[N / 2], bool upper, F partner) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
        const float lo = in[i], hi = in[N / 2 + i];
        out[i] = (upper ? hi : lo) + partner(upper ? lo : hi);
    }
}
// Sum over the 16 lanes of a row of NV per-lane values.  NV >= 16: lane p ends with the NV/16
// complete sums of indices p*NV/16 + s; NV < 16: lane p ends with the sum of index p / (16/NV)
// (DUP = 16/NV neighbouring lanes hold the same sum).
template <int NV>
struct RowSum {
    static constexpr int FV = NV >= 16 ? NV / 16 : 1;
    static constexpr int DUP = NV >= 16 ? 1 : 16 / NV;
    __device__ static __forceinline__ void run(float (&v)[NV], float (&o)[FV], int p) {
        if constexpr (NV == 32) {
            float a[16], b[8], c[4];
            tstep<32>(v, a, p & 8, dpp_row_mirror);
            tstep<16>(a, b, p & 4, dpp_row_half_mirror);
            tstep<8>(b, c, p & 2, dpp_quad_xor2);
            tstep<4>(c, o, p & 1, dpp_quad_xor1);
        } else if constexpr (NV == 16) {
            float a[8], b[4], c[2];
            tstep<16>(v, a, p & 8, dpp_row_mirror);
            tstep<8>(a, b, p & 4, dpp_row_half_mirror);
            tstep<4>(b, c, p & 2, dpp_quad_xor2);
            tstep<2>(c, o, p & 1, dpp_quad_xor1);
        } else if constexpr (NV == 8) {
            float a[4], b[2], c[1];
            tstep<8>(v, a, p & 8, dpp_row_mirror);
            tstep<4>(a, b, p & 4, dpp_row_half_mirror);
            tstep<2>(b, c, p & 2, dpp_quad_xor2);
            o[0] = c[0] + dpp_quad_xor1(c[0]);
        } else {
            static_assert(NV == 4, "4, 8, 16 or 32 values per lane");
            float a[2], b[1];
            tstep<4>(v, a, p & 8, dpp_row_mirror);
            tstep<2>(a, b, p & 4, dpp_row_half_mirror);
            const float c = b[0] + dpp_quad_xor2(b[0]);
            o[0] = c + dpp_quad_xor1(c);
        }
    }
};
// Reduction over the lanes of a row that hold one head's values (steps S0 .. S1-1 of the
// partners xor1, xor2, half-mirror, mirror; the steps below S0 would combine duplicate lanes),
// then over the 4 rows with the gfx950 row swaps.
template <bool MAX>
__device__ __forceinline__ float op2(float a, float b) { return MAX ? fmaxf(a, b) : a + b; }
template <bool MAX, int S0, int S1>
__device__ __forceinline__ float head_reduce(float x) {
    if constexpr (S0 <= 0 && S1 > 0) x = op2<MAX>(x, dpp_quad_xor1(x));
    if constexpr (S0 <= 1 && S1 > 1) x = op2<MAX>(x, dpp_quad_xor2(x));
    if constexpr (S0 <= 2 && S1 > 2) x = op2<MAX>(x, dpp_row_half_mirror(x));
    if constexpr (S0 <= 3 && S1 > 3) x = op2<MAX>(x, dpp_row_mirror(x));
    auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = op2<MAX>(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
    auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return op2<MAX>(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
}
__host__ __device__ constexpr int ilog2c(int x) { return x <= 1 ? 0 : 1 + ilog2c(x / 2); }
// Sum over the 4 rows of NA per-lane values, transposed: row r ends with the sums of indices
// r*NA/4 + j, j < NA/4 (one permlane32 swap and one permlane16 swap per value pair).
template <int NA>
__device__ __forceinline__ void rows_tsum(const float (&v)[NA], float (&o)[NA / 4]) {
    float w[NA / 2];
#pragma unroll
    for (int j = 0; j < NA / 2; ++j) {
        auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[j]), __float_as_uint(v[j + NA / 2]), false, false);
        w[j] = __uint_as_float(s[0]) + __uint_as_float(s[1]);
    }
#pragma unroll
    for (int j = 0; j < NA / 4; ++j) {
        auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(w[j]), __float_as_uint(w[j + NA / 4]), false, false);
        o[j] = __uint_as_float(s[0]) + __uint_as_float(s[1]);
    }
}

// MODE 0: shared list per sequence (vote); MODE 1: list per query head; MODE 2: dense
// (the list is implicit: entry j is token j, counts are the sequence lengths); MODE 3: the union
// of a KV group's per-head lists (G * count slots per (sequence, KV head), padded with -1) with a
// per-entry mask of the heads that selected the token: each gathered row is read once for the
// group and a head's score of an entry it did not select is -inf.
// Blocks per CU to keep: 4 (16 waves) for the vote and dense modes with G <= 4, whose registers
// fit in 128 (512 / 4) per lane with one sub-batch in flight per wave; 3 for the union mode with
// G <= 4, which spills at 128 (its head masks); no bound otherwise.  Against 3 blocks with two
// sub-batches in flight per wave: the dense 128K decode 110 -> 102 us, the decode of a
// 16-sequence ragged batch 112 -> 107 us, the 128K vote decode 37.2 -> 36.7 us; the union decode
// at 128K / 20 % 80.1 us with 4 blocks (7 VGPRs spilled) against 73.4 us with 3.
__host__ __device__ constexpr int dec_min_blocks(int G, int mode) {
    return (mode != 1 && G <= 4) ? (mode == 3 ? 3 : 4) : 1;
}

// RING: positions >= n_b - N are read from slot t mod N of the sequence's ring (`ring`), the older
// ones from K / V (a tiered cache: the newest tokens in a device ring, the rest possibly in host
// memory mapped for the device).
template <int G, int MODE, bool RING = false>
__global__ __launch_bounds__(kDecWaves * 64, dec_min_blocks(G, MODE)) void decode_partial_kernel(const uint16_t* __restrict__ q,
                                                                       const uint16_t* __restrict__ K,
                                                                       const uint16_t* __restrict__ V,
                                                                       I64Arg offsets,
                                                                       const int32_t* __restrict__ idx,
                                                                       I64Arg counts, int B, int Hq,
                                                                       int Hkv, int EB, float* __restrict__ part_acc,
                                                                       float2* __restrict__ part_ml,
                                                                       const uint8_t* __restrict__ umask,
                                                                       const int64_t* __restrict__ ucount,
                                                                       DecRing ring) {
    constexpr int GH = dec_gh(G, MODE);
    constexpr int EPR = kDecSub / 4;               // entries per lane row and sub-batch
    constexpr int NV = GH * EPR;                   // (head, entry) scores of a row
    constexpr int FV = RowSum<NV>::FV;             // complete scores per lane
    constexpr int DUP = RowSum<NV>::DUP;           // lanes holding the same score
    constexpr int NA = GH * 8;                     // accumulators per lane
    // reduction steps over the lanes of a row that hold one head's scores
    constexpr int HS0 = ilog2c(DUP);
    constexpr int HS1 = HS0 + ilog2c(EPR / FV);
    __shared__ float s_acc[kDecWaves][GH][kD];
    __shared__ float s_m[kDecWaves][GH], s_l[kDecWaves][GH];
    __shared__ float4 s_p[kDecWaves][4][NV / 4];
    __shared__ int4 s_tok[kDecWaves][kDecMaxEW / 4];
    __shared__ uint32_t s_msk[(MODE == 3) ? kDecWaves : 1][(MODE == 3) ? kDecMaxEW / 4 : 1];   // union: head masks

    const int HW = (MODE == 1) ? Hq : Hkv;
    int64_t item;
    int hw;
    if constexpr (MODE == 1) {
        // The G blocks of one (item, KV head) pair get equal blockIdx % 8: blocks are dealt to
        // the 8 XCDs round-robin, so the pair's heads run on one XCD, whose L2 then serves the
        // rows their lists share.  x = (pair / 8) * 8G + j * 8 + pair % 8 for head j of the group.
        const int64_t x = blockIdx.x;
        const int64_t pair = (x / (8 * G)) * 8 + x % 8;
        item = pair / Hkv;
        hw = (int)(pair % Hkv) * G + (int)((x / 8) % G);
    } else {
        item = blockIdx.x / HW;
        hw = blockIdx.x % HW;
    }
    int b;
    int64_t j0, len, kpre;
    constexpr int LM = (MODE == 3) ? G : 1;
    if (!find_list_chunk(counts, B, item, EB, LM, b, j0, len, kpre)) return;
    const int64_t off = offsets[b];
    const int32_t nmax = (int32_t)(offsets[b + 1] - off - 1);   // list entries are clamped to [0, n_b)
    const int g = (MODE == 1) ? hw / G : hw;
    const int hbase = (MODE == 1) ? hw : hw * G;                 // first query head of the wave
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int row = lane >> 4, p = lane & 15;
    if (MODE == 3) {
        // the union's size is known on the device only: its entries are split evenly over the
        // group's ceil(G K / EB) ranges (at most EB each), so that every block has work
        const int64_t cap = (int64_t)G * counts[b];
        int64_t uc = ucount[(int64_t)b * Hkv + hw];
        uc = uc < 0 ? 0 : (uc > cap ? cap : uc);
        const int64_t nch = (cap + EB - 1) / EB, c = j0 / EB;
        j0 = uc * c / nch;
        len = uc * (c + 1) / nch - j0;
    }
    const int EW = (MODE == 3) ? (int)((len + kDecWaves - 1) / kDecWaves) : EB / kDecWaves;
    const int64_t wb = (int64_t)wid * EW;
    const int wlen = len <= wb ? 0 : (len - wb < EW ? (int)(len - wb) : EW);
    const int nsb = (wlen + kDecSub - 1) / kDecSub;

    // token ids of the wave's entries into LDS (entries past the wave's end repeat its first token,
    // so that every load of a sub-batch is issued and hits a row already requested); negative
    // entries are empty slots (-1): their rows are read at position 0 and their scores are -inf
    int32_t* tok = reinterpret_cast<int32_t*>(&s_tok[wid][0]);
    {
        // the list of this block: the sequence's (vote), the head's (per-head), the KV group's (union)
        const int64_t lbase = (MODE == 1) ? Hq * kpre + (int64_t)hw * counts[b]
                                          : ((MODE == 3) ? Hq * kpre + (int64_t)hw * G * counts[b] : kpre);
        int32_t t0 = 0;
        if (wlen > 0) {
            const int64_t j = j0 + wb;
            t0 = (MODE == 2) ? (int32_t)j : idx[lbase + j];
        }
        uint8_t* msk = (MODE == 3) ? reinterpret_cast<uint8_t*>(&s_msk[wid][0]) : nullptr;
        for (int i = lane; i < nsb * kDecSub; i += 64) {
            int32_t t = t0;
            uint8_t mb = 0;
            if (i < wlen) {
                const int64_t j = j0 + wb + i;
                t = (MODE == 2) ? (int32_t)j : idx[lbase + j];
                if (MODE == 3) mb = umask[lbase + j];
            }
            if (MODE == 3) {
                msk[i] = mb;
                if (i < wlen && mb == 0) t = -1;          // no head selected it: an empty slot
            }
            tok[i] = t < 0 ? -1 : (t > nmax ? nmax : t);
        }
    }
    uint4 qv[GH];
#pragma unroll
    for (int hh = 0; hh < GH; ++hh) qv[hh] = ld16(q + ((int64_t)b * Hq + hbase + hh) * kD + p * 8);
    __builtin_amdgcn_wave_barrier();

    const uint16_t* Kg = K + (off * Hkv + g) * kD + p * 8;
    const uint16_t* Vg = V + (off * Hkv + g) * kD + p * 8;
    const int64_t rstride = (int64_t)Hkv * kD;
    // ring: its first position (negative when the whole sequence fits in it) and slot mask; a
    // ring slot is a row of Hkv * 128 values like a row of the main cache
    const uint16_t* Kr = Kg;
    const uint16_t* Vr = Vg;
    int32_t rfirst = 0, rmask = 0;
    if constexpr (RING) {
        Kr = ring.K + ((int64_t)b * ring.N * Hkv + g) * kD + p * 8;
        Vr = ring.V + ((int64_t)b * ring.N * Hkv + g) * kD + p * 8;
        rfirst = (int32_t)((int64_t)nmax + 1 - ring.N);
        rmask = (int32_t)ring.N - 1;
    }
    // em: bit k set when entry k of the lane's row is an empty slot
    auto issue = [&](int sb, uint4 (&kb)[EPR], uint4 (&vb)[EPR], int& em, uint32_t& hm) {
        const int4 t = s_tok[wid][(sb * kDecSub + row * EPR) / 4];
        if (MODE == 3) hm = s_msk[wid][(sb * kDecSub + row * EPR) / 4];
        const int tt[4] = {t.x < 0 ? 0 : t.x, t.y < 0 ? 0 : t.y, t.z < 0 ? 0 : t.z, t.w < 0 ? 0 : t.w};
        em = (t.x < 0 ? 1 : 0) | (t.y < 0 ? 2 : 0) | (t.z < 0 ? 4 : 0) | (t.w < 0 ? 8 : 0);
        if constexpr (RING) {
            bool inr[EPR];
            int32_t row[EPR];
#pragma unroll
            for (int k = 0; k < EPR; ++k) {
                inr[k] = tt[k] >= rfirst;
                row[k] = inr[k] ? (tt[k] & rmask) : tt[k];
            }
#pragma unroll
            for (int k = 0; k < EPR; ++k) kb[k] = ld16((inr[k] ? Kr : Kg) + row[k] * rstride);
#pragma unroll
            for (int k = 0; k < EPR; ++k) vb[k] = ld16((inr[k] ? Vr : Vg) + row[k] * rstride);
        } else {
#pragma unroll
            for (int k = 0; k < EPR; ++k) kb[k] = ld16(Kg + tt[k] * rstride);
#pragma unroll
            for (int k = 0; k < EPR; ++k) vb[k] = ld16(Vg + tt[k] * rstride);
        }
    };

    float m_run = -INFINITY, l_run = 0.f;         // this lane's head (hh_l)
    float acc[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) acc[i] = 0.f;
    // this lane's scores: index i = p * FV + s (NV >= 16) or p / DUP (NV < 16), head i / EPR,
    // entry 4 row + (i % EPR) of the sub-batch
    const int i0 = NV >= 16 ? p * FV : p / DUP;
    const int hh_l = i0 / EPR;
    float4* sp4 = &s_p[wid][row][0];
    float* sp = reinterpret_cast<float*>(sp4);

    auto compute = [&](int sb, const uint4 (&kb)[EPR], const uint4 (&vb)[EPR], int em, uint32_t hm) {
        float zp[NV];
#pragma unroll
        for (int k = 0; k < EPR; ++k)
#pragma unroll
            for (int hh = 0; hh < GH; ++hh) {
                float s = dot2_bf16(qv[hh].x, kb[k].x, 0.f);
                s = dot2_bf16(qv[hh].y, kb[k].y, s);
                s = dot2_bf16(qv[hh].z, kb[k].z, s);
                zp[hh * EPR + k] = dot2_bf16(qv[hh].w, kb[k].w, s);
            }
        float z[FV];
        RowSum<NV>::run(zp, z, p);
        float mx = -INFINITY;
#pragma unroll
        for (int s = 0; s < FV; ++s) {
            const int ke = (i0 + s) % EPR;
            const int e = sb * kDecSub + row * EPR + ke;
            bool use = e < wlen && !((em >> ke) & 1);
            if (MODE == 3) use = use && ((hm >> (8 * ke + (i0 + s) / EPR)) & 1u);   // the head selected it
            z[s] = use ? z[s] * kLog2eOverSqrtD : -INFINITY;
            mx = fmaxf(mx, z[s]);
        }
        const float m_new = fmaxf(m_run, head_reduce<true, HS0, HS1>(mx));
        const float alpha = m_run == -INFINITY ? 0.f : fast_exp2(m_run - m_new);
        float ls = 0.f;
#pragma unroll
        for (int s = 0; s < FV; ++s) {
            z[s] = m_new == -INFINITY ? 0.f : fast_exp2(z[s] - m_new);
            ls += z[s];
        }
        l_run = l_run * alpha + head_reduce<false, HS0, HS1>(ls);
        m_run = m_new;
        // the row's probabilities to every lane of the row (LDS, one wave: in order)
        if (NV >= 16) {
#pragma unroll
            for (int s = 0; s < FV; ++s) sp[i0 + s] = z[s];
        } else if (p % DUP == 0) {
            sp[i0] = z[0];
        }
        __builtin_amdgcn_wave_barrier();
        float pr[NV];
#pragma unroll
        for (int i = 0; i < NV / 4; ++i) {
            const float4 x = sp4[i];
            pr[4 * i] = x.x; pr[4 * i + 1] = x.y; pr[4 * i + 2] = x.z; pr[4 * i + 3] = x.w;
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int hh = 0; hh < GH; ++hh) {
            // rescale factor of head hh: uniform over the wave, read from its first lane
            const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha),
                                                                    (hh * EPR * DUP) / FV));
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[hh * 8 + e] *= a;
        }
#pragma unroll
        for (int k = 0; k < EPR; ++k) {
            const float vf[8] = {bf16_lo(vb[k].x), bf16_hi(vb[k].x), bf16_lo(vb[k].y), bf16_hi(vb[k].y),
                                 bf16_lo(vb[k].z), bf16_hi(vb[k].z), bf16_lo(vb[k].w), bf16_hi(vb[k].w)};
#pragma unroll
            for (int hh = 0; hh < GH; ++hh)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[hh * 8 + e] = fmaf(pr[hh * EPR + k], vf[e], acc[hh * 8 + e]);
        }
    };

    uint4 ka[EPR], va[EPR];
    int ema = 0;
    uint32_t hma = 0;
    for (int sb = 0; sb < nsb; ++sb) {
        issue(sb, ka, va, ema, hma);
        compute(sb, ka, va, ema, hma);
    }

    // sum over the 4 rows: row r holds accumulator indices r * NA / 4 + j
    float ar[NA / 4];
    rows_tsum<NA>(acc, ar);
#pragma unroll
    for (int j = 0; j < NA / 4; ++j) {
        const int i = row * (NA / 4) + j;
        s_acc[wid][i / 8][p * 8 + (i % 8)] = ar[j];
    }
    if (row == 0 && p == (hh_l * EPR * DUP) / FV) {
        s_m[wid][hh_l] = m_run;
        s_l[wid][hh_l] = l_run;
    }
    __syncthreads();
    // the block's partial: merge of the waves
    for (int o = threadIdx.x; o < GH * kD; o += kDecWaves * 64) {
        const int hh = o / kD, d = o % kD;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, s_m[w][hh]);
        float A = 0.f, L = 0.f;
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w) {
            const float mw = s_m[w][hh];
            const float wt = mw == -INFINITY ? 0.f : fast_exp2(mw - M);
            A = fmaf(s_acc[w][hh][d], wt, A);
            L = fmaf(s_l[w][hh], wt, L);
        }
        const int64_t slot = item * Hq + hbase + hh;
        part_acc[slot * kD + d] = A;
        if (d == 0) part_ml[slot] = make_float2(M, L);
    }
}

// Merge of the chunk partials of each (sequence, head).  One block per (b, h); thread
// (cg, d) = (tid / 128, tid % 128) takes every 8th chunk of the sequence with 16 loads in
// flight and keeps a running (M, A, L) in the log2 domain; the 8 groups then combine in LDS.
constexpr int kMergeThreads = 1024;
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(const float* __restrict__ part_acc,
                                                                    const float2* __restrict__ part_ml,
                                                                    I64Arg counts, int B, int Hq, int EB, int lm,
                                                                    float* __restrict__ out) {
    constexpr int NG = kMergeThreads / kD, U = 16;
    __shared__ float sM[NG], sL[NG];
    __shared__ float sA[NG][kD];
    const int bh = blockIdx.x, b = bh / Hq, h = bh % Hq;
    const int64_t first = wave_prefix_seq(b, [cd = counts.dev, EB, lm](int i) { return (lm * cd[i] + EB - 1) / EB; });
    const int64_t nch = (lm * counts[b] + EB - 1) / EB;
    const int cg = threadIdx.x / kD, d = threadIdx.x % kD;
    float M = -INFINITY, A = 0.f, L = 0.f;
    for (int64_t c0 = cg; c0 < nch; c0 += (int64_t)NG * U) {
        float x[U], mm[U], ll[U];
        float2 ml[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = c0 + (int64_t)NG * u;
            const int64_t slot = (first + (c < nch ? c : c0)) * Hq + h;
            x[u] = part_acc[slot * kD + d];
            ml[u] = part_ml[slot];
        }
        // every load of the batch is issued before the first use
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            mm[u] = c0 + (int64_t)NG * u < nch ? ml[u].x : -INFINITY;
            ll[u] = ml[u].y;
        }
        // no branch on Mn: the compiler would move the x and l loads into it, behind the wait
        // for the maxima.  Slots with m = -inf (the clamped slots past the list's end, and in the
        // union decode the ranges in which the head selected nothing) have weight 0 and A = L = 0;
        // while Mn = -inf, A and L stay 0.
        float Mn = M;
#pragma unroll
        for (int u = 0; u < U; ++u) Mn = fmaxf(Mn, mm[u]);
        const float rs = M == -INFINITY ? 0.f : fast_exp2(M - Mn);
        A *= rs;
        L *= rs;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float w = mm[u] == -INFINITY ? 0.f : fast_exp2(mm[u] - Mn);
            A = fmaf(x[u], w, A);
            L = fmaf(ll[u], w, L);
        }
        M = Mn;
    }
    sA[cg][d] = A;
    if (d == 0) { sM[cg] = M; sL[cg] = L; }
    __syncthreads();
    if (threadIdx.x < kD) {
        float Mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < NG; ++k) Mx = fmaxf(Mx, sM[k]);
        float As = 0.f, Ls = 0.f;
#pragma unroll
        for (int k = 0; k < NG; ++k) {
            const float w = sM[k] == -INFINITY ? 0.f : fast_exp2(sM[k] - Mx);
            As = fmaf(sA[k][threadIdx.x], w, As);
            Ls = fmaf(sL[k], w, Ls);
        }
        out[((int64_t)b * Hq + h) * kD + threadIdx.x] = As / Ls;
    }
}

// ranges of EB entries over the lists (lm entries per count: G for the union lists)
static int64_t list_items(const int64_t* counts_host, int B, int EB, int lm) {
    int64_t it = 0;
    for (int b = 0; b < B; ++b) it += (lm * counts_host[b] + EB - 1) / EB;
    return it;
}

// Compute units of the current device (queried once per device).
static int device_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

template <int MODE, bool RING>
static const void* partial_fn(int G) {
    switch (G) {
        case 1: return reinterpret_cast<const void*>(decode_partial_kernel<1, MODE, RING>);
        case 2: return reinterpret_cast<const void*>(decode_partial_kernel<2, MODE, RING>);
        case 4: return reinterpret_cast<const void*>(decode_partial_kernel<4, MODE, RING>);
        default: return reinterpret_cast<const void*>(decode_partial_kernel<8, MODE, RING>);
    }
}
// Resident blocks per compute unit of an instantiation (queried once).
static int partial_blocks_per_cu(int G, int mode, bool ring) {
    static int cache[2][4][4] = {};
    const int lg = G == 1 ? 0 : (G == 2 ? 1 : (G == 4 ? 2 : 3));
    int& c = cache[ring ? 1 : 0][mode][lg];
    if (c == 0) {
        const void* f = ring ? (mode == 0 ? partial_fn<0, true>(G) : (mode == 1 ? partial_fn<1, true>(G) : partial_fn<2, true>(G)))
                             : (mode == 0 ? partial_fn<0, false>(G)
                                          : (mode == 1 ? partial_fn<1, false>(G)
                                                       : (mode == 2 ? partial_fn<2, false>(G) : partial_fn<3, false>(G))));
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, kDecWaves * 64, 0) != hipSuccess || n <= 0) n = 2;
        c = n;
    }
    return c;
}

// Entries per block: the whole work (entries x HW blocks per range) spread over one round of
// resident blocks; a multiple of 4 and at least one sub-batch per wave.  With a list shared by
// a sequence's heads (vote mode), each sequence's last range is partial, so EB then grows (by
// 1/16 at a time, up to kDecMaxEW entries per wave) until the ranges of all sequences fit in
// that round.  The dense decode keeps EB at most 256 entries per wave and per-head lists at most
// 64: there several rounds of smaller blocks measured faster, the blocks that finish early taking
// the next ones (dense 128K decode 106 against 110 us; per-head lists at 128K tokens and 20 %,
// 69.7 against 80.8 us with 256 entries per wave).  len(b) is the list length (or, for the dense
// decode, the sequence length) of sequence b.
template <class Len>
static int decode_eb(Len len, int B, int HW, int G, int mode, bool ring = false) {
    const int64_t target = (int64_t)partial_blocks_per_cu(G, mode, ring) * device_cus();
    int64_t entries = 0;
    for (int b = 0; b < B; ++b) entries += len(b);
    const int64_t lo = kDecWaves * kDecSub, hi = kDecWaves * (mode == 1 ? 64 : (mode == 2 ? 256 : kDecMaxEW));
    auto clampr = [&](int64_t e) {
        e = (e + 3) / 4 * 4;
        return e < lo ? lo : (e > hi ? hi : e);
    };
    int64_t eb = clampr((entries * HW + target - 1) / target);
    auto blocks = [&](int64_t e) {
        int64_t it = 0;
        for (int b = 0; b < B; ++b) it += (len(b) + e - 1) / e;
        return it * HW;
    };
    if (mode == 0 || mode == 3)
        while (eb < hi && blocks(eb) > target) eb = clampr(eb + (eb + 15) / 16);
    return (int)eb;
}

// Workspace: the partials of at most sum_b ceil(K_b / EB) <= sum_b K_b / (kDecWaves kDecSub) + B
// ranges (EB never falls below kDecWaves kDecSub; K_b is G times the count for the union lists),
// a bound that grows with the list lengths.
size_t decode_workspace(const int64_t* offsets_host, const int64_t* counts_host, int B, int Hq, int Hkv, int mode) {
    const int lm = mode == 3 ? Hq / Hkv : 1;
    int64_t total = 0;
    for (int b = 0; b < B; ++b) total += counts_host ? lm * counts_host[b] : offsets_host[b + 1] - offsets_host[b];
    const int64_t items = (total + kDecWaves * kDecSub - 1) / (kDecWaves * kDecSub) + B;
    WsCarver w(nullptr);
    w.take<int64_t>((size_t)B + 1);   // dense: per-sequence lengths
    w.take<float>((size_t)items * Hq * kD);
    w.take<float2>((size_t)items * Hq);
    return w.size();
}

// t0 / t1: when given, the launch records them at the kernel's start and end (its dispatch
// timestamps), for a duration that matches a kernel trace's.
template <int MODE, bool RING = false>
static hipError_t launch_partial_G(int G, dim3 grid, hipStream_t stream, const uint16_t* q, const uint16_t* K,
                                   const uint16_t* V, const I64Arg& offsets, const int32_t* idx,
                                   const I64Arg& counts, int B, int Hq, int Hkv, int EB, float* part, float2* ml,
                                   const uint8_t* umask = nullptr, const int64_t* ucount = nullptr,
                                   const DecRing& ring = DecRing{nullptr, nullptr, 0}, hipEvent_t t0 = nullptr,
                                   hipEvent_t t1 = nullptr) {
    const dim3 block(kDecWaves * 64);
    if (t0 && t1) {
        switch (G) {
            case 1: hipExtLaunchKernelGGL((decode_partial_kernel<1, MODE, RING>), grid, block, 0, stream, t0, t1, 0, q, K, V, offsets, idx, counts, B, Hq, Hkv, EB, part, ml, umask, ucount, ring); break;
            case 2: hipExtLaunchKernelGGL((decode_partial_kernel<2, MODE, RING>), grid, block, 0, stream, t0, t1, 0, q, K, V, offsets, idx, counts, B, Hq, Hkv, EB, part, ml, umask, ucount, ring); break;
            case 4: hipExtLaunchKernelGGL((decode_partial_kernel<4, MODE, RING>), grid, block, 0, stream, t0, t1, 0, q, K, V, offsets, idx, counts, B, Hq, Hkv, EB, part, ml, umask, ucount, ring); break;
            case 8: hipExtLaunchKernelGGL((decode_partial_kernel<8, MODE, RING>), grid, block, 0, stream, t0, t1, 0, q, K, V, offsets, idx, counts, B, Hq, Hkv, EB, part, ml, umask, ucount, ring); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    switch (G) {
        case 1: hipLaunchKernelGGL((decode_partial_kernel<1, MODE, RING>), grid, block, 0, stream, q, K, V, offsets, idx, counts, B, Hq, Hkv, EB, part, ml, umask, ucount, ring); break;
        case 2: hipLaunchKernelGGL((decode_partial_kernel<2, MODE, RING>), grid, block, 0, stream, q, K, V, offsets, idx, counts, B, Hq, Hkv, EB, part, ml, umask, ucount, ring); break;
        case 4: hipLaunchKernelGGL((decode_partial_kernel<4, MODE, RING>), grid, block, 0, stream, q, K, V, offsets, idx, counts, B, Hq, Hkv, EB, part, ml, umask, ucount, ring); break;
        case 8: hipLaunchKernelGGL((decode_partial_kernel<8, MODE, RING>), grid, block, 0, stream, q, K, V, offsets, idx, counts, B, Hq, Hkv, EB, part, ml, umask, ucount, ring); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// dense decode: counts are the sequence lengths, computed on the device into the workspace
__global__ void lengths_kernel(I64Arg offsets, int B, int64_t* __restrict__ lens) {
    for (int b = threadIdx.x; b < B; b += blockDim.x) lens[b] = offsets[b + 1] - offsets[b];
}

// List decode (vote or per-head lists); ring: the tiered cache's ring, or null; t0 / t1: events
// recorded at the gather kernel's start and end, or null.
static hipError_t sparse_decode(const uint16_t* q, const uint16_t* K, const uint16_t* V, const DecRing* ring,
                                const int64_t* offsets_dev, const int64_t* offsets_host, const int32_t* idx,
                                const int64_t* counts_dev, const int64_t* counts_host, int mode, int B, int Hq, int Hkv,
                                float* out, void* ws, size_t ws_bytes, hipStream_t stream, hipEvent_t t0 = nullptr,
                                hipEvent_t t1 = nullptr) {
    if (decode_workspace(offsets_host, counts_host, B, Hq, Hkv, mode) > ws_bytes) return hipErrorInvalidValue;
    const int G = Hq / Hkv;
    const int EB = decode_eb([&](int b) { return counts_host[b]; }, B, mode == 1 ? Hq : Hkv, G, mode, ring != nullptr);
    WsCarver w(ws);
    w.take<int64_t>((size_t)B + 1);
    const int64_t items = list_items(counts_host, B, EB, 1);
    float* part = w.take<float>((size_t)items * Hq * kD);
    float2* ml = w.take<float2>((size_t)items * Hq);
    const I64Arg offs = i64_arg(offsets_dev, offsets_host, (int64_t)B + 1);
    const I64Arg cnts = i64_arg(counts_dev, counts_host, B);
    if (items == 0) return hipSuccess;
    hipError_t e;
    // blocks of the (item, KV head) pairs in groups of 8, G heads each in per-head mode (see the
    // kernel); the pairs past items * Hkv find no list chunk and return
    const dim3 grid = mode == 0 ? dim3((unsigned)(items * Hkv)) : dim3((unsigned)((items * Hkv + 7) / 8 * 8 * G));
    if (ring) {
        if (mode == 0) e = launch_partial_G<0, true>(G, grid, stream, q, K, V, offs, idx, cnts, B, Hq, Hkv, EB, part, ml, nullptr, nullptr, *ring);
        else e = launch_partial_G<1, true>(G, grid, stream, q, K, V, offs, idx, cnts, B, Hq, Hkv, EB, part, ml, nullptr, nullptr, *ring);
    } else {
        const DecRing none{nullptr, nullptr, 0};
        if (mode == 0) e = launch_partial_G<0>(G, grid, stream, q, K, V, offs, idx, cnts, B, Hq, Hkv, EB, part, ml, nullptr, nullptr, none, t0, t1);
        else e = launch_partial_G<1>(G, grid, stream, q, K, V, offs, idx, cnts, B, Hq, Hkv, EB, part, ml, nullptr, nullptr, none, t0, t1);
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_merge_kernel, dim3(B * Hq), dim3(kMergeThreads), 0, stream, part, ml, cnts, B, Hq, EB, 1, out);
    return hipGetLastError();
}

hipError_t launch_sparse_decode(const uint16_t* q, const uint16_t* K, const uint16_t* V, const int64_t* offsets_dev,
                                const int64_t* offsets_host, const int32_t* idx, const int64_t* counts_dev,
                                const int64_t* counts_host, int mode, int B, int Hq, int Hkv, float* out, void* ws,
                                size_t ws_bytes, hipStream_t stream, hipEvent_t gather_start, hipEvent_t gather_stop) {
    return sparse_decode(q, K, V, nullptr, offsets_dev, offsets_host, idx, counts_dev, counts_host, mode, B, Hq, Hkv,
                         out, ws, ws_bytes, stream, gather_start, gather_stop);
}

hipError_t launch_union_decode(const uint16_t* q, const uint16_t* K, const uint16_t* V, const int64_t* offsets_dev,
                               const int64_t* offsets_host, const int32_t* uidx, const uint8_t* umask,
                               const int64_t* ucount, const int64_t* counts_dev, const int64_t* counts_host, int B,
                               int Hq, int Hkv, float* out, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (decode_workspace(offsets_host, counts_host, B, Hq, Hkv, 3) > ws_bytes) return hipErrorInvalidValue;
    const int G = Hq / Hkv;
    const int EB = decode_eb([&](int b) { return G * counts_host[b]; }, B, Hkv, G, 3);
    WsCarver w(ws);
    w.take<int64_t>((size_t)B + 1);
    const int64_t items = list_items(counts_host, B, EB, G);
    float* part = w.take<float>((size_t)items * Hq * kD);
    float2* ml = w.take<float2>((size_t)items * Hq);
    const I64Arg offs = i64_arg(offsets_dev, offsets_host, (int64_t)B + 1);
    const I64Arg cnts = i64_arg(counts_dev, counts_host, B);
    if (items == 0) return hipSuccess;
    hipError_t e = launch_partial_G<3>(G, dim3((unsigned)(items * Hkv)), stream, q, K, V, offs, uidx, cnts, B, Hq, Hkv,
                                       EB, part, ml, umask, ucount);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_merge_kernel, dim3(B * Hq), dim3(kMergeThreads), 0, stream, part, ml, cnts, B, Hq, EB, G, out);
    return hipGetLastError();
}

// ------------------------------------------------------------- no-allocation variant
// The partials of ts_sparse_decode_noalloc live in this file-scope device array instead of a
// caller workspace.  Each device the library runs on holds its own copy (allocated with the code
// object, kept until the process ends).  On the host the array's name is only a stand-in for the
// device symbol, so its device address is looked up once per device with hipGetSymbolAddress and
// only that address is used.  Every call on one device shares the array: calls that overlap on
// one device (different streams, or host threads) race.  Nothing in it needs to start at zero:
// every partial slot a merge reads is written by its block in the same call.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

static hipError_t scratch_on_current_device(void** out) {
    static std::mutex mu;
    static void* ptr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        ptr[dev] = p;
    }
    *out = ptr[dev];
    return hipSuccess;
}

hipError_t launch_sparse_decode_noalloc(const uint16_t* q, const uint16_t* K, const uint16_t* V,
                                        const int64_t* offsets_dev, const int64_t* offsets_host, const int32_t* idx,
                                        const int64_t* counts_dev, const int64_t* counts_host, int mode, int B, int Hq,
                                        int Hkv, float* out, hipStream_t stream) {
    if (decode_workspace(offsets_host, counts_host, B, Hq, Hkv, mode) > kNoAllocScratchBytes)
        return hipErrorInvalidValue;
    void* ws = nullptr;
    hipError_t e = scratch_on_current_device(&ws);
    if (e != hipSuccess) return e;
    return launch_sparse_decode(q, K, V, offsets_dev, offsets_host, idx, counts_dev, counts_host, mode, B, Hq, Hkv,
                                out, ws, kNoAllocScratchBytes, stream);
}

static hipError_t dense_decode(const uint16_t* q, const uint16_t* K, const uint16_t* V, const DecRing* ring,
                               const int64_t* offsets_dev, const int64_t* offsets_host, int B, int Hq, int Hkv,
                               float* out, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (decode_workspace(offsets_host, nullptr, B, Hq, Hkv, 2) > ws_bytes) return hipErrorInvalidValue;
    const int G = Hq / Hkv;
    const int EB = decode_eb([&](int b) { return offsets_host[b + 1] - offsets_host[b]; }, B, Hkv, G, 2, ring != nullptr);
    int64_t items = 0;
    for (int b = 0; b < B; ++b) items += (offsets_host[b + 1] - offsets_host[b] + EB - 1) / EB;
    WsCarver w(ws);
    int64_t* lens = w.take<int64_t>((size_t)B + 1);
    float* part = w.take<float>((size_t)items * Hq * kD);
    float2* ml = w.take<float2>((size_t)items * Hq);
    const I64Arg offs = i64_arg(offsets_dev, offsets_host, (int64_t)B + 1);
    // one sequence: its length is a launch argument; otherwise the lengths are computed on
    // the device
    const int64_t hl = offsets_host[B] - offsets_host[0];
    const I64Arg lns = i64_arg(lens, B == 1 ? &hl : nullptr, B);
    if (items == 0) return hipSuccess;
    if (B != 1) hipLaunchKernelGGL(lengths_kernel, dim3(1), dim3(256), 0, stream, offs, B, lens);
    const dim3 grid((unsigned)(items * Hkv));
    hipError_t e = ring ? launch_partial_G<2, true>(G, grid, stream, q, K, V, offs, nullptr, lns, B, Hq, Hkv, EB, part,
                                                    ml, nullptr, nullptr, *ring)
                        : launch_partial_G<2>(G, grid, stream, q, K, V, offs, nullptr, lns, B, Hq, Hkv, EB, part, ml);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_merge_kernel, dim3(B * Hq), dim3(kMergeThreads), 0, stream, part, ml, lns, B, Hq, EB, 1, out);
    return hipGetLastError();
}

hipError_t launch_dense_decode(const uint16_t* q, const uint16_t* K, const uint16_t* V, const int64_t* offsets_dev,
                               const int64_t* offsets_host, int B, int Hq, int Hkv, float* out, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
    return dense_decode(q, K, V, nullptr, offsets_dev, offsets_host, B, Hq, Hkv, out, ws, ws_bytes, stream);
}

hipError_t launch_tiered_decode(const uint16_t* q, const uint16_t* K, const uint16_t* V, const DecRing& ring,
                                const int64_t* offsets_dev, const int64_t* offsets_host, const int32_t* idx,
                                const int64_t* counts_dev, const int64_t* counts_host, int mode, int B, int Hq,
                                int Hkv, float* out, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (ring.N < 1 || (ring.N & (ring.N - 1)) || !ring.K || !ring.V) return hipErrorInvalidValue;
    if (mode == 2) return dense_decode(q, K, V, &ring, offsets_dev, offsets_host, B, Hq, Hkv, out, ws, ws_bytes, stream);
    if (mode != 0 && mode != 1) return hipErrorInvalidValue;
    return sparse_decode(q, K, V, &ring, offsets_dev, offsets_host, idx, counts_dev, counts_host, mode, B, Hq, Hkv,
                         out, ws, ws_bytes, stream);
}

}  // namespace qasi
