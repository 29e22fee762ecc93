// Compressed key index: append (projection + one bf16 rounding) and per-head index scores.
//
// [TS] "Query-Key Dot Product Index": the index K_index has width d' = d/4, is built
// incrementally while decoding, and scores tokens by Score_h(i) = q_h . k_index,h(i)/sqrt(d').
// [TB] "Kernarchitektur": keys are projected by a fixed matrix into the low-dimensional space.
#include "qasi_device.h"
#include "qasi_internal.h"

namespace qasi {

// ---------------------------------------------------------------------------------------
// Index append.  A block owns runs of 8 (token, KV head) rows; thread (r, c) = (tid / 32,
// tid % 32) forms the projection of row r onto column c of P: the k row is staged in LDS, the
// 128 entries P[j][c] are loaded up front (fully unrolled), and the sum is formed in fp64 in
// order j = 0..127 with fma (the bf16 x fp32 product is exact in fp64), then rounded once.
// ---------------------------------------------------------------------------------------
constexpr int kAppendThreads = 256;
constexpr int kAppendRows = kAppendThreads / kDP;   // 8 rows per pass

__global__ __launch_bounds__(kAppendThreads) void index_append_kernel(
    const uint16_t* __restrict__ k_new, const float* __restrict__ P, uint16_t* __restrict__ k_index,
    int64_t pos, int64_t rows, int Hkv) {
    __shared__ float sk[kAppendRows][kD];
    const int r = threadIdx.x / kDP, c = threadIdx.x % kDP;
    float pc[kD];
#pragma unroll
    for (int j = 0; j < kD; ++j) pc[j] = P[j * kDP + c];
    for (int64_t base = (int64_t)blockIdx.x * kAppendRows; base < rows; base += (int64_t)gridDim.x * kAppendRows) {
        __syncthreads();
        {   // 8 rows x 128 bf16 = 2 KiB: one 8-byte piece per thread
            const int rr = threadIdx.x / 32, jj = (threadIdx.x % 32) * 4;
            const int64_t row = base + rr;
            uint2 w = make_uint2(0, 0);
            if (row < rows) w = *reinterpret_cast<const uint2*>(k_new + row * kD + jj);
            sk[rr][jj] = bf16_lo(w.x);
            sk[rr][jj + 1] = bf16_hi(w.x);
            sk[rr][jj + 2] = bf16_lo(w.y);
            sk[rr][jj + 3] = bf16_hi(w.y);
        }
        __syncthreads();
        const int64_t row = base + r;
        if (row < rows) {
            double acc = 0.0;
#pragma unroll
            for (int j = 0; j < kD; ++j) acc = fma((double)sk[r][j], (double)pc[j], acc);
            const int64_t t = row / Hkv, g = row % Hkv;
            k_index[((pos + t) * Hkv + g) * kDP + c] = f64_to_bf16_rne(acc);
        }
    }
}

hipError_t launch_index_append(const uint16_t* k_new, const float* P, uint16_t* k_index, int64_t pos,
                               int64_t T, int Hkv, hipStream_t stream) {
    int64_t rows = T * Hkv;
    int64_t blocks = (rows + kAppendRows - 1) / kAppendRows;
    if (blocks > 2048) blocks = 2048;
    hipLaunchKernelGGL(index_append_kernel, dim3((unsigned)blocks), dim3(kAppendThreads), 0, stream, k_new, P,
                       k_index, pos, rows, Hkv);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Index scores, two kernels:
//   qproj_kernel : q'_h = P^T q_h / sqrt(32) in fp32 for every (sequence, query head), into
//                  the workspace (one block per sequence);
//   score_kernel : work item = (sequence b, block of kScoreTB tokens of b), dispatched in
//                  token order.  A token's index row (Hkv x 32 bf16 = Hkv x 64 B) is read by
//                  LPT = 4*Hkv lanes with one 16-byte load each: lane (g, part) holds 8 index
//                  values of KV head g and forms the partial dot products of the G heads of g.
//                  A transposed quad butterfly (DPP) leaves lane `part` with the complete
//                  scores of the heads h = part (mod 4) of its group, so every lane stores
//                  whole scores.  Scores are staged in a padded LDS tile [Hq][kScoreTB + 1]
//                  (conflict-free) and written row by row into scores[h * S + t].
// ---------------------------------------------------------------------------------------
constexpr int kScoreTB = 64;
// block size: at most 512 threads and at least two token rows per lane (4 lanes per KV head)
template <int HKV>
constexpr int score_threads() {
    return kScoreTB * 4 * HKV / 2 < 512 ? kScoreTB * 4 * HKV / 2 : 512;
}
constexpr int kTileLd = kScoreTB + 1;

// item -> (sequence b, first token t0 of the item's block of tb tokens, its length); every lane
// of the wave calls it
__device__ __forceinline__ bool find_item(const I64Arg& offsets, int B, int64_t item, int tb, int& b,
                                          int64_t& t0, int64_t& len) {
    const SeqPos sp = wave_find_seq(B, item, (offsets[1] - offsets[0] + tb - 1) / tb,
                                    [od = offsets.dev, tb](int i) { return (od[i + 1] - od[i] + tb - 1) / tb; });
    if (sp.b < 0) return false;
    b = sp.b;
    // one sequence: its length from the launch arguments; more: from device memory
    const int64_t n = B == 1 ? offsets[1] - offsets[0] : offsets.dev[b + 1] - offsets.dev[b];
    t0 = (item - sp.first) * tb;
    len = n - t0 < tb ? n - t0 : tb;
    return true;
}

// qp[(b * Hq + h) * 32 + c] = sum_j q[b][h][j] P[j][c] / sqrt(32): P and the block's
// queries are staged in LDS with one round trip to memory; the sum is formed as four partial
// sums over j in [32k, 32k + 32) (each in order) combined as ((s0 + s1) + (s2 + s3)), then
// scaled.
__global__ __launch_bounds__(1024) void qproj_kernel(const uint16_t* __restrict__ q, const float* __restrict__ P,
                                                    int Hq, float* __restrict__ qp) {
    __shared__ float sP[kD * kDP];
    __shared__ uint4 sq[64 * kD / 8];
    __shared__ float spart[4][64 * kDP];
    const int b = blockIdx.x;
    const uint4* qb = reinterpret_cast<const uint4*>(q + (int64_t)b * Hq * kD);
    for (int i = threadIdx.x; i < kD * kDP / 4; i += 1024)
        reinterpret_cast<float4*>(sP)[i] = reinterpret_cast<const float4*>(P)[i];
    for (int i = threadIdx.x; i < Hq * kD / 8; i += 1024) sq[i] = qb[i];
    __syncthreads();
    for (int o = threadIdx.x; o < 4 * Hq * kDP; o += 1024) {
        const int k = o / (Hq * kDP), hc = o % (Hq * kDP), h = hc / kDP, c = hc % kDP;
        float acc = 0.f;
#pragma unroll
        for (int j8 = 4 * k; j8 < 4 * k + 4; ++j8) {
            const uint4 w = sq[h * (kD / 8) + j8];
            const float qv[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                                 bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = fmaf(qv[e], sP[(j8 * 8 + e) * kDP + c], acc);
        }
        spart[k][hc] = acc;
    }
    __syncthreads();
    for (int o = threadIdx.x; o < Hq * kDP; o += 1024)
        qp[(int64_t)b * Hq * kDP + o] = ((spart[0][o] + spart[1][o]) + (spart[2][o] + spart[3][o])) * 0.17677669529663688f;
}

// Transposed quad reduction: v[hh] (hh < G) are this lane's partial sums; afterwards
// v[k] of lane `part` holds the full sum of head hh = part + 4k (G >= 4), of head
// hh = part & 1 (G == 2, lanes part and part^2 agree) or of head 0 (G == 1).
template <int G>
__device__ __forceinline__ void quad_transpose_sum(float (&v)[G], int part) {
    if constexpr (G == 1) {
        v[0] = sum_quad(v[0]);
    } else if constexpr (G == 2) {
        const bool odd = part & 1;
        const float send = odd ? v[0] : v[1];
        const float keep = odd ? v[1] : v[0];
        const float r = keep + dpp_quad_xor1(send);
        v[0] = r + dpp_quad_xor2(r);
    } else {
        // step 1 (partner part^1): keep heads with (hh & 1) == (part & 1)
        constexpr int H1 = G / 2;
        float k1[H1];
        const bool odd = part & 1;
#pragma unroll
        for (int i = 0; i < H1; ++i) {
            const float a = v[2 * i], c = v[2 * i + 1];
            const float send = odd ? a : c;
            const float keep = odd ? c : a;
            k1[i] = keep + dpp_quad_xor1(send);     // head 2i + (part & 1)
        }
        // step 2 (partner part^2): keep heads with (hh & 3) == part
        const bool hi2 = part & 2;
#pragma unroll
        for (int i = 0; i < H1 / 2; ++i) {
            const float a = k1[2 * i], c = k1[2 * i + 1];   // heads 4i + (part&1), 4i + 2 + (part&1)
            const float send = hi2 ? a : c;
            const float keep = hi2 ? c : a;
            v[i] = keep + dpp_quad_xor2(send);        // head 4i + part
        }
    }
}

// Tile classification against a key bracket (CLS): for every query head h of the tile's
// sequence b whose instance (b, h) is active, over the tile's positions in [beg, end), with
// records laid out head-major, [h][tile] (tiles numbered sequence by sequence):
//   tinfo[h][tile] = below | inside << 8 | offset << 16 (#keys below lo, #keys in [lo, hi], offset
//                    of the head's keys in the tile's key area);
//   cand[h][tile][j], j < min(inside, kClsSlots): the head's first in-bracket keys (in position
//                    order), so that one head's keys of consecutive tiles are contiguous;
//   tcand[tile * kClsTile + offset + j - kClsSlots], kClsSlots <= j < inside: the rest (rare), the
//                    heads' runs packed one after the other in the order they reserve them.
// Inactive instances, and those without a bracket (lo > hi: rows short enough to be ranked whole),
// write zero records.  The bracket comes from state[(b * Hq + h) * 8 + ...].
struct ClsArgs {
    const int64_t* state;
    uint32_t* tinfo;
    uint32_t* cand;
    uint32_t* tcand;
    int64_t ntiles;
};

template <int HKV, int G, bool CLS>
__global__ __launch_bounds__(score_threads<HKV>()) void score_kernel(const float* __restrict__ qp,
                                                             const uint16_t* __restrict__ k_index,
                                                             I64Arg offsets, int B,
                                                             float* __restrict__ scores,
                                                             const int64_t* __restrict__ cls_state, ClsArgs cls) {
    constexpr int NT = score_threads<HKV>();
    constexpr int Hq = HKV * G;
    constexpr int LPT = 4 * HKV;          // lanes per token
    constexpr int TPW = 64 / LPT;         // tokens per wave per load
    constexpr int TPB = TPW * (NT / 64);  // tokens per block per load
    static_assert(NT % 64 == 0 && kScoreTB % TPB == 0, "whole waves, whole passes over the tile");
    constexpr int ITERS = kScoreTB / TPB;
    static_assert(ITERS <= 4, "the tile's rows are loaded up front");
    constexpr int NOUT = G >= 4 ? G / 4 : 1;          // complete heads per lane
    __shared__ float tile[Hq * kTileLd];
    __shared__ uint32_t s_run;

    int b;
    int64_t t0, len;
    if (!find_item(offsets, B, blockIdx.x, kScoreTB, b, t0, len)) return;
    if (CLS && threadIdx.x == 0) s_run = 0;
    // CLS: the brackets of this wave's heads wid + i NW, requested first as wave-uniform (scalar)
    // loads so they arrive while the tile is computed
    constexpr int NWC = score_threads<HKV>() / 64;
    constexpr int HPW = (HKV * G + NWC - 1) / NWC;
    const int wu = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int64_t c_flag[CLS ? HPW : 1], c_lo[CLS ? HPW : 1], c_hi[CLS ? HPW : 1], c_beg[CLS ? HPW : 1], c_end[CLS ? HPW : 1];
    if constexpr (CLS) {
#pragma unroll
        for (int i = 0; i < HPW; ++i) {
            const int h = wu + i * NWC < HKV * G ? wu + i * NWC : HKV * G - 1;
            const int64_t* st = cls_state + ((int64_t)b * HKV * G + h) * 8;
            c_flag[i] = st[kStFlag];
            c_lo[i] = st[kStLo];
            c_hi[i] = st[kStHi];
            c_beg[i] = st[kStBeg];
            c_end[i] = st[kStEnd];
        }
    }
    const int64_t S = score_stride(offsets[B]);
    const int64_t base_tok = offsets[b] + t0;

    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int lit = lane % LPT, g = lit / 4, part = lit % 4;
    const int slot = wid * TPW + lane / LPT;

    // the tile's index rows, all loads in flight at once: lanes past the tile's end read its
    // first row (their values are never used), so the loads need no branch and no merge copy
    // (a zeroed register merged with a conditional load makes the compiler wait for it)
    uint4 kv[ITERS];
#pragma unroll
    for (int u = 0; u < ITERS; ++u) {
        const int tl = u * TPB + slot;
        kv[u] = ld16(k_index + ((base_tok + (tl < len ? tl : 0)) * HKV + g) * kDP + part * 8);
    }
    float qr[G][8];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        const float4* src = reinterpret_cast<const float4*>(qp + ((int64_t)b * Hq + g * G + hh) * kDP + part * 8);
        const float4 a = src[0], c = src[1];
        qr[hh][0] = a.x; qr[hh][1] = a.y; qr[hh][2] = a.z; qr[hh][3] = a.w;
        qr[hh][4] = c.x; qr[hh][5] = c.y; qr[hh][6] = c.z; qr[hh][7] = c.w;
    }
    // rows of the tile this lane writes: heads g*G + part + 4k (G >= 4), g*G + (part&1) (G == 2), g*G (G == 1)
    const bool writer = (G >= 4) || (G == 2 ? part < 2 : part == 0);
    const int hrow = g * G + (G >= 4 ? part : (G == 2 ? (part & 1) : 0));

    {
#pragma unroll
        for (int u = 0; u < ITERS; ++u) {
            const int tl = u * TPB + slot;
            const uint4 w = kv[u];
            const float kf[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                                 bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
            float v[G];
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                float s = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) s = fmaf(qr[hh][e], kf[e], s);
                v[hh] = s;
            }
            quad_transpose_sum<G>(v, part);
            if (writer && tl < len) {
#pragma unroll
                for (int k = 0; k < NOUT; ++k) tile[(hrow + 4 * k) * kTileLd + tl] = v[k];
            }
        }
    }
    __syncthreads();
    for (int o = threadIdx.x; o < Hq * kScoreTB; o += NT) {
        const int h = o / kScoreTB, tl = o % kScoreTB;
        if (tl < len) scores[(int64_t)h * S + base_tok + tl] = tile[h * kTileLd + tl];
    }
    if constexpr (CLS) {
        static_assert(kScoreTB == 64, "one wave lane per tile token");
        // wave w takes heads w, w + NW, ...; lane = token of the tile; the wave reserves the runs
        // of keys of its heads with one LDS atomic.
        constexpr int NW = NT / 64;
        static_assert(NW == NWC, "one wave count");
        const uint64_t lt = (1ull << lane) - 1ull;
        uint32_t below[HPW], cnt[HPW], key[HPW];
        uint64_t mm[HPW];
#pragma unroll
        for (int i = 0; i < HPW; ++i) {
            const int h = wu + i * NW;
            below[i] = 0;
            key[i] = 0;
            mm[i] = 0;
            const uint32_t lo = (uint32_t)c_lo[i], hi = (uint32_t)c_hi[i];
            if (h < Hq && c_flag[i] == 0 && lo <= hi) {  // an active order statistic with a bracket
                const int64_t t = t0 + lane;
                const bool valid = lane < len && t >= c_beg[i] && t < c_end[i];
                key[i] = order_key(tile[h * kTileLd + lane]);
                below[i] = (uint32_t)__popcll(__ballot(valid && key[i] < lo));
                mm[i] = __ballot(valid && key[i] >= lo && key[i] <= hi);
            }
            cnt[i] = (uint32_t)__popcll(mm[i]);
        }
        // one reservation in the tile's overflow area for the keys past the first kClsSlots of
        // the wave's heads, whose runs follow each other (the heads of the tile in any order)
        uint32_t tot = 0;
#pragma unroll
        for (int i = 0; i < HPW; ++i) tot += cnt[i] > kClsSlots ? cnt[i] - kClsSlots : 0u;
        uint32_t off = 0;
        if (lane == 0 && tot) off = atomicAdd(&s_run, tot);
        off = __builtin_amdgcn_readfirstlane(off);
#pragma unroll
        for (int i = 0; i < HPW; ++i) {
            const int h = wu + i * NW;
            if (h >= Hq) continue;
            const size_t r = (size_t)h * cls.ntiles + blockIdx.x;
            if (lane == 0) cls.tinfo[r] = below[i] | (cnt[i] << 8) | (off << 16);
            if ((mm[i] >> lane) & 1ull) {
                const uint32_t j = (uint32_t)__popcll(mm[i] & lt);
                if (j < (uint32_t)kClsSlots) cls.cand[r * kClsSlots + j] = key[i];
                else cls.tcand[(size_t)blockIdx.x * kClsTile + off + j - kClsSlots] = key[i];
            }
            off += cnt[i] > kClsSlots ? cnt[i] - kClsSlots : 0u;
        }
    }
}

int64_t score_items(const int64_t* offsets_host, int B) {
    int64_t items = 0;
    for (int b = 0; b < B; ++b) items += (offsets_host[b + 1] - offsets_host[b] + kScoreTB - 1) / kScoreTB;
    return items;
}

size_t score_workspace(int B, int Hq) {
    WsCarver w(nullptr);
    w.take<float>((size_t)B * Hq * kDP);
    return w.size();
}

template <int HKV, bool CLS>
static hipError_t launch_score_g(int G, dim3 grid, hipStream_t stream, const float* qp, const uint16_t* k_index,
                                 const I64Arg& offsets, int B, float* scores, const ClsArgs& cls) {
    dim3 block(score_threads<HKV>());
    switch (G) {
        case 1: hipLaunchKernelGGL((score_kernel<HKV, 1, CLS>), grid, block, 0, stream, qp, k_index, offsets, B, scores, cls.state, cls); break;
        case 2: hipLaunchKernelGGL((score_kernel<HKV, 2, CLS>), grid, block, 0, stream, qp, k_index, offsets, B, scores, cls.state, cls); break;
        case 4: hipLaunchKernelGGL((score_kernel<HKV, 4, CLS>), grid, block, 0, stream, qp, k_index, offsets, B, scores, cls.state, cls); break;
        case 8: hipLaunchKernelGGL((score_kernel<HKV, 8, CLS>), grid, block, 0, stream, qp, k_index, offsets, B, scores, cls.state, cls); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <bool CLS>
static hipError_t launch_score_tiles(const float* qp, const uint16_t* k_index, const I64Arg& offs, int64_t items,
                                     int B, int Hq, int Hkv, float* scores, const ClsArgs& cls, hipStream_t stream) {
    const dim3 grid((unsigned)items);
    const int G = Hq / Hkv;
    switch (Hkv) {
        case 1: return launch_score_g<1, CLS>(G, grid, stream, qp, k_index, offs, B, scores, cls);
        case 2: return launch_score_g<2, CLS>(G, grid, stream, qp, k_index, offs, B, scores, cls);
        case 4: return launch_score_g<4, CLS>(G, grid, stream, qp, k_index, offs, B, scores, cls);
        case 8: return launch_score_g<8, CLS>(G, grid, stream, qp, k_index, offs, B, scores, cls);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_score(const uint16_t* q, const float* P, const uint16_t* k_index, const int64_t* offsets_dev,
                        const int64_t* offsets_host, int B, int Hq, int Hkv, float* scores, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
    if (score_workspace(B, Hq) > ws_bytes) return hipErrorInvalidValue;
    float* qp = static_cast<float*>(ws);
    hipLaunchKernelGGL(qproj_kernel, dim3(B), dim3(1024), 0, stream, q, P, Hq, qp);
    const int64_t items = score_items(offsets_host, B);
    if (items == 0) return hipGetLastError();
    const I64Arg offs = i64_arg(offsets_dev, offsets_host, (int64_t)B + 1);
    return launch_score_tiles<false>(qp, k_index, offs, items, B, Hq, Hkv, scores, ClsArgs{}, stream);
}

// Scores plus the tile classification against the brackets in `state` (q' already in qp).
hipError_t launch_score_classify(const float* qp, const uint16_t* k_index, const int64_t* offsets_dev,
                                 const int64_t* offsets_host, int B, int Hq, int Hkv, float* scores,
                                 const int64_t* state, uint32_t* tinfo, uint32_t* cand, uint32_t* tcand,
                                 hipStream_t stream) {
    const int64_t items = score_items(offsets_host, B);
    if (items == 0) return hipSuccess;
    const I64Arg offs = i64_arg(offsets_dev, offsets_host, (int64_t)B + 1);
    return launch_score_tiles<true>(qp, k_index, offs, items, B, Hq, Hkv, scores,
                                    ClsArgs{state, tinfo, cand, tcand, items}, stream);
}

}  // namespace qasi

namespace qasi {
hipError_t init_score_kernels() { return hipSuccess; }
}  // namespace qasi
