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
// Index scores.  Work item = (sequence b, block of kScoreTB tokens of b).  The block first
// issues its first index loads, then projects the sequence's queries (q'_h = P^T q_h /
// sqrt(32), fp32, P and q staged in LDS).  A token's index row (Hkv x 32 bf16 = Hkv x 64 B)
// is read by LPT = 4*Hkv lanes with one 16-byte non-temporal load each: lane (g, part)
// holds 8 index values of KV head g and forms the partial dot products of the G heads of g;
// a quad butterfly (DPP) completes each dot product.  Scores are staged in LDS as an
// [Hq][kScoreTB] tile and written row by row (coalesced) into scores[h][t].
// ---------------------------------------------------------------------------------------
constexpr int kScoreThreads = 512;
constexpr int kScoreTB = 512;

__device__ __forceinline__ bool find_item(const int64_t* __restrict__ offsets, int B, int64_t item, int tb, int& b,
                                          int64_t& t0, int64_t& len) {
    int64_t acc = 0;
    for (int i = 0; i < B; ++i) {
        int64_t n = offsets[i + 1] - offsets[i];
        int64_t nb = (n + tb - 1) / tb;
        if (item < acc + nb) {
            b = i;
            int64_t j = item - acc;
            t0 = j * tb;
            len = n - t0 < tb ? n - t0 : tb;
            return true;
        }
        acc += nb;
    }
    return false;
}

template <int HKV>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(const uint16_t* __restrict__ q, const float* __restrict__ P,
                                                             const uint16_t* __restrict__ k_index,
                                                             const int64_t* __restrict__ offsets, int B, int Hq,
                                                             float* __restrict__ scores) {
    constexpr int LPT = 4 * HKV;          // lanes per token
    constexpr int TPW = 64 / LPT;         // tokens per wave per load
    constexpr int TPB = TPW * (kScoreThreads / 64);  // tokens per block per load
    constexpr int ITERS = kScoreTB / TPB;
    constexpr int UNR = ITERS < 8 ? ITERS : 8;
    extern __shared__ float smem[];
    float* sq = smem;                       // [Hq][32] projected queries
    float* sP = sq + Hq * kDP;              // [128][32]        } staging, dead once q' is formed
    float* sqf = sP + kD * kDP;             // [Hq][128] queries }
    float* tile = sP;                       // [Hq][kScoreTB] score tile, overlays the staging

    int b;
    int64_t t0, len;
    if (!find_item(offsets, B, blockIdx.x, kScoreTB, b, t0, len)) return;
    const int64_t S = score_stride(offsets[B]);
    const int64_t base_tok = offsets[b] + t0;
    const int G = Hq / HKV;

    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int lit = lane % LPT, g = lit / 4, part = lit % 4;
    const int slot = wid * TPW + lane / LPT;

    // first batch of index loads, issued before the query projection
    uint4 kv[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
        int tl = u * TPB + slot;
        kv[u] = make_uint4(0, 0, 0, 0);
        if (tl < len) kv[u] = ld16(k_index + ((base_tok + tl) * HKV + g) * kDP + part * 8);
    }
    // stage P (16 KB) and the queries of sequence b
    for (int i = threadIdx.x; i < kD * kDP / 4; i += kScoreThreads)
        reinterpret_cast<float4*>(sP)[i] = reinterpret_cast<const float4*>(P)[i];
    for (int i = threadIdx.x; i < Hq * kD / 8; i += kScoreThreads) {
        uint4 w = reinterpret_cast<const uint4*>(q + (int64_t)b * Hq * kD)[i];
        float* d = sqf + i * 8;
        d[0] = bf16_lo(w.x); d[1] = bf16_hi(w.x); d[2] = bf16_lo(w.y); d[3] = bf16_hi(w.y);
        d[4] = bf16_lo(w.z); d[5] = bf16_hi(w.z); d[6] = bf16_lo(w.w); d[7] = bf16_hi(w.w);
    }
    __syncthreads();
    // q'_h[c] = sum_j q[b][h][j] P[j][c] / sqrt(32)
    for (int o = threadIdx.x; o < Hq * kDP; o += kScoreThreads) {
        const int h = o / kDP, c = o % kDP;
        const float* qh = sqf + h * kD;
        float acc = 0.f;
#pragma unroll 16
        for (int j = 0; j < kD; ++j) acc = fmaf(qh[j], sP[j * kDP + c], acc);
        sq[o] = acc * 0.17677669529663688f;
    }
    __syncthreads();
    float qr[8][8];   // [head in group][element]
#pragma unroll
    for (int hh = 0; hh < 8; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) qr[hh][e] = (hh < G) ? sq[(g * G + hh) * kDP + part * 8 + e] : 0.f;

    for (int it0 = 0; it0 < ITERS; it0 += UNR) {
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            int tl = (it0 + u) * TPB + slot;
            uint4 w = kv[u];
            // prefetch the next batch into the same register
            int tn = (it0 + UNR + u) * TPB + slot;
            if (it0 + UNR < ITERS) {
                kv[u] = make_uint4(0, 0, 0, 0);
                if (tn < len) kv[u] = ld16(k_index + ((base_tok + tn) * HKV + g) * kDP + part * 8);
            }
            float kf[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                           bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
#pragma unroll
            for (int hh = 0; hh < 8; ++hh) {
                if (hh < G) {
                    float s = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) s = fmaf(qr[hh][e], kf[e], s);
                    s = sum_quad(s);
                    if ((hh & 3) == part && tl < len) tile[(g * G + hh) * kScoreTB + tl] = s;
                }
            }
        }
    }
    __syncthreads();
    for (int o = threadIdx.x; o < Hq * kScoreTB; o += kScoreThreads) {
        int h = o / kScoreTB, tl = o % kScoreTB;
        if (tl < len) scores[(int64_t)h * S + base_tok + tl] = tile[o];
    }
}

static size_t score_shm(int Hq) {
    size_t stage = (size_t)kD * kDP + (size_t)Hq * kD, tile = (size_t)Hq * kScoreTB;
    return ((size_t)Hq * kDP + (stage > tile ? stage : tile)) * sizeof(float);
}

int64_t score_items(const int64_t* offsets_host, int B) {
    int64_t items = 0;
    for (int b = 0; b < B; ++b) items += (offsets_host[b + 1] - offsets_host[b] + kScoreTB - 1) / kScoreTB;
    return items;
}

hipError_t launch_score(const uint16_t* q, const float* P, const uint16_t* k_index, const int64_t* offsets_dev,
                        const int64_t* offsets_host, int B, int Hq, int Hkv, float* scores, hipStream_t stream) {
    int64_t items = score_items(offsets_host, B);
    if (items == 0) return hipSuccess;
    size_t shm = score_shm(Hq);
    dim3 grid((unsigned)items), block(kScoreThreads);
    switch (Hkv) {
        case 1: hipLaunchKernelGGL(score_kernel<1>, grid, block, shm, stream, q, P, k_index, offsets_dev, B, Hq, scores); break;
        case 2: hipLaunchKernelGGL(score_kernel<2>, grid, block, shm, stream, q, P, k_index, offsets_dev, B, Hq, scores); break;
        case 4: hipLaunchKernelGGL(score_kernel<4>, grid, block, shm, stream, q, P, k_index, offsets_dev, B, Hq, scores); break;
        case 8: hipLaunchKernelGGL(score_kernel<8>, grid, block, shm, stream, q, P, k_index, offsets_dev, B, Hq, scores); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace qasi

namespace qasi {
hipError_t init_score_kernels() {
    const int bytes = (int)score_shm(64);
    hipError_t e = hipSuccess;
    if ((e = hipFuncSetAttribute((const void*)score_kernel<1>, hipFuncAttributeMaxDynamicSharedMemorySize, bytes))) return e;
    if ((e = hipFuncSetAttribute((const void*)score_kernel<2>, hipFuncAttributeMaxDynamicSharedMemorySize, bytes))) return e;
    if ((e = hipFuncSetAttribute((const void*)score_kernel<4>, hipFuncAttributeMaxDynamicSharedMemorySize, bytes))) return e;
    return hipFuncSetAttribute((const void*)score_kernel<8>, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}
}  // namespace qasi
