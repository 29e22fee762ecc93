// Compressed key index: append (projection + one bf16 rounding) and per-head index scores.
//
// [TS] "Query-Key Dot Product Index": the index K_index has width d' = d/4, is built
// incrementally while decoding, and scores tokens by Score_h(i) = q_h . k_index,h(i)/sqrt(d').
// [TB] "Kernarchitektur": keys are projected by a fixed matrix into the low-dimensional space.
#include "qasi_device.h"
#include "qasi_internal.h"

namespace qasi {

// ---------------------------------------------------------------------------------------
// Index append.  One block owns a run of (token, KV head) rows; each of its 256 threads is
// (row slot r = tid / 32, output column c = tid % 32).  The k row is staged in LDS and the
// projection is summed in fp64 in order j = 0..127 with fma (the bf16 x fp32 product is
// exact in fp64), then rounded once to bf16.
// ---------------------------------------------------------------------------------------
constexpr int kAppendThreads = 256;
constexpr int kAppendRows = kAppendThreads / kDP;   // 8 rows per pass

__global__ __launch_bounds__(kAppendThreads) void index_append_kernel(
    const uint16_t* __restrict__ k_new, const float* __restrict__ P, uint16_t* __restrict__ k_index,
    int64_t pos, int64_t rows, int Hkv) {
    __shared__ float sP[kD * kDP];
    __shared__ double sk[kAppendRows][kD];
    for (int i = threadIdx.x; i < kD * kDP; i += kAppendThreads) sP[i] = P[i];
    const int r = threadIdx.x / kDP, c = threadIdx.x % kDP;
    for (int64_t base = (int64_t)blockIdx.x * kAppendRows; base < rows; base += (int64_t)gridDim.x * kAppendRows) {
        __syncthreads();
        // 8 rows x 128 bf16 = 512 uint32 pairs; 2 pairs per thread
        for (int i = threadIdx.x; i < kAppendRows * kD / 2; i += kAppendThreads) {
            int rr = i / (kD / 2), jj = (i % (kD / 2)) * 2;
            int64_t row = base + rr;
            uint32_t pr = 0;
            if (row < rows) pr = *reinterpret_cast<const uint32_t*>(k_new + row * kD + jj);
            sk[rr][jj] = (double)bf16_lo(pr);
            sk[rr][jj + 1] = (double)bf16_hi(pr);
        }
        __syncthreads();
        int64_t row = base + r;
        if (row < rows) {
            double acc = 0.0;
#pragma unroll 8
            for (int j = 0; j < kD; ++j) acc = fma(sk[r][j], (double)sP[j * kDP + c], acc);
            int64_t t = row / Hkv, g = row % Hkv;
            k_index[((pos + t) * Hkv + g) * kDP + c] = f64_to_bf16_rne(acc);
        }
    }
}

hipError_t launch_index_append(const uint16_t* k_new, const float* P, uint16_t* k_index, int64_t pos,
                               int64_t T, int Hkv, hipStream_t stream) {
    int64_t rows = T * Hkv;
    int64_t blocks = (rows + kAppendRows - 1) / kAppendRows;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(index_append_kernel, dim3((unsigned)blocks), dim3(kAppendThreads), 0, stream, k_new, P,
                       k_index, pos, rows, Hkv);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Index scores.  Work item = (sequence b, block of kScoreTB tokens of b).  The block first
// projects the sequence's queries (q'_h = P^T q_h / sqrt(32), fp32) into LDS while its first
// index loads are in flight.  A token's index row (Hkv x 32 bf16 = Hkv x 64 B) is read by
// LPT = 4*Hkv lanes with one 16-byte load each: lane (g, part) holds 8 index values of KV
// head g and forms the partial dot products of the G heads of g; a quad butterfly (DPP)
// completes each dot product.  Scores are staged in LDS as an [Hq][kScoreTB] tile and
// written row by row (coalesced) into scores[h][t].
// ---------------------------------------------------------------------------------------
constexpr int kScoreThreads = 256;
constexpr int kScoreTB = 256;

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
    float* tile = smem + Hq * kDP;          // [Hq][kScoreTB]

    int b;
    int64_t t0, len;
    if (!find_item(offsets, B, blockIdx.x, kScoreTB, b, t0, len)) return;
    const int64_t Ntot = offsets[B];
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
        if (tl < len) kv[u] = *reinterpret_cast<const uint4*>(k_index + ((base_tok + tl) * HKV + g) * kDP + part * 8);
    }

    // q'_h[c] = sum_j q[b][h][j] P[j][c] / sqrt(32)
    for (int o = threadIdx.x; o < Hq * kDP; o += kScoreThreads) {
        int h = o / kDP, c = o % kDP;
        const uint16_t* qh = q + ((int64_t)b * Hq + h) * kD;
        float acc = 0.f;
        for (int j = 0; j < kD; j += 2) {
            uint32_t pr = *reinterpret_cast<const uint32_t*>(qh + j);
            acc = fmaf(bf16_lo(pr), P[j * kDP + c], acc);
            acc = fmaf(bf16_hi(pr), P[(j + 1) * kDP + c], acc);
        }
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
                if (tn < len) kv[u] = *reinterpret_cast<const uint4*>(k_index + ((base_tok + tn) * HKV + g) * kDP + part * 8);
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
        if (tl < len) scores[(int64_t)h * Ntot + base_tok + tl] = tile[o];
    }
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
    size_t shm = (size_t)Hq * (kDP + kScoreTB) * sizeof(float);
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
    const int bytes = 64 * (kDP + kScoreTB) * (int)sizeof(float);
    hipError_t e = hipSuccess;
    if ((e = hipFuncSetAttribute((const void*)score_kernel<1>, hipFuncAttributeMaxDynamicSharedMemorySize, bytes))) return e;
    if ((e = hipFuncSetAttribute((const void*)score_kernel<2>, hipFuncAttributeMaxDynamicSharedMemorySize, bytes))) return e;
    if ((e = hipFuncSetAttribute((const void*)score_kernel<4>, hipFuncAttributeMaxDynamicSharedMemorySize, bytes))) return e;
    return hipFuncSetAttribute((const void*)score_kernel<8>, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}
}  // namespace qasi
