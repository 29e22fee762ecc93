// SnapKV prefill-end compression on gfx950 MFMA.
//
// [SK] "Attention Score計算とPooling": for every observation-window query the attention
// over all n prompt keys is A = softmax(Q_obs K^T / sqrt(d_k)); the importance of key j is
// the mean of A[:, j] over the window, and the pipeline figure averages across the query
// heads that share a KV head as well.  [SK] "アルゴリズム": the importance is smoothed by
// avg_pool1d(kernel 3, padding 1, stride 1), the top min(c, n) positions are kept per KV
// head, sorted, and the chosen K/V rows are gathered into a compacted cache.
//
// The contraction S = Q_g K_g^T (R = G*w rows x n keys x 128) runs on
// v_mfma_f32_16x16x32_bf16: the A operand is a 16-key x 32-dim slice of K read straight
// from HBM (one 16-byte load per lane), the B operand a 32-dim x 16-row slice of Q_g from
// LDS.  Lane l of the 16x16 fp32 result holds keys 4*(l/16)+i (i < 4) for row l%16.
//   pass 1 (snap_pass_kernel<1>): per row online max / sum of 2^s over the block's keys
//   snap_lse_kernel:             combines the per-block (m, l) into LSE_r (log2 domain)
//   pass 2 (snap_pass_kernel<2>): p = 2^(s - LSE_r); the column sum over the R rows (a
//                                 16-lane DPP butterfly per 16-row tile) gives imp[j] * R
// Scores are kept in the log2 domain (s = q.k * log2(e)/sqrt(128)) so that exp2 is used.
#include "qasi_device.h"
#include "qasi_internal.h"

namespace qasi {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kSnapThreads = 256;     // 4 waves
constexpr int kSnapNIT = 8;           // 16-key sub-tiles per wave
constexpr int kSnapKT = 4 * 16 * kSnapNIT;   // keys per block (512)
constexpr float kSnapScale = 1.4426950408889634f / 11.313708498984761f;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
    bf16x8_t r;
    __builtin_memcpy(&r, &v, 16);
    return r;
}

// grid: x = KV head g, y = key block.  Q rows of group g: r = hh * w + t  <->  q_obs[t][g*G + hh].
template <int PASS>
__global__ __launch_bounds__(kSnapThreads) void snap_pass_kernel(const uint16_t* __restrict__ q_obs,
                                                                const uint16_t* __restrict__ K, int64_t n, int w,
                                                                int Hq, int Hkv, float2* __restrict__ pstat,
                                                                const float* __restrict__ lse,
                                                                float* __restrict__ imp) {
    extern __shared__ uint4 sQ[];   // [R][16] uint4 (128 bf16 per row), row-swizzled by (row & 15)
    __shared__ float2 wstat[4][256];
    const int g = blockIdx.x;
    const int64_t kb = blockIdx.y;
    const int G = Hq / Hkv, R = G * w, RT = R / 16;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;

    // stage Q_g (R x 128 bf16) in LDS; 16-byte chunk c of row r goes to slot (c ^ (r & 15))
    for (int i = threadIdx.x; i < R * 16; i += kSnapThreads) {
        int r = i / 16, c = i % 16;
        int hh = r / w, t = r % w;
        uint4 v = *reinterpret_cast<const uint4*>(q_obs + ((int64_t)t * Hq + g * G + hh) * kD + c * 8);
        sQ[r * 16 + (c ^ (r & 15))] = v;
    }
    float lrow[16];   // pass 2: LSE of row c*16 + lr
    if (PASS == 2) {
#pragma unroll
        for (int c = 0; c < 16; ++c) lrow[c] = (c < RT) ? lse[(int64_t)g * R + c * 16 + lr] : 0.f;
    }
    __syncthreads();

    float m[16], l[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) { m[c] = -INFINITY; l[c] = 0.f; }

    for (int it = 0; it < kSnapNIT; ++it) {
        const int64_t j0 = kb * kSnapKT + (int64_t)(it * 4 + wid) * 16;
        if (j0 >= n) break;
        // A operands: key j0 + lr, dims 32 s + 8 lg .. +8
        bf16x8_t a[4];
        const int64_t jl = j0 + lr;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (jl < n) v = *reinterpret_cast<const uint4*>(K + (jl * Hkv + g) * kD + s * 32 + lg * 8);
            a[s] = as_bf16x8(v);
        }
        float colsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            if (c < RT) {
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
                const int r = c * 16 + lr;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int chunk = s * 4 + lg;
                    bf16x8_t bq = as_bf16x8(sQ[r * 16 + (chunk ^ (r & 15))]);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], bq, acc, 0, 0, 0);
                }
                float sv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t j = j0 + lg * 4 + i;
                    sv[i] = (j < n) ? acc[i] * kSnapScale : -INFINITY;
                }
                if (PASS == 1) {
                    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
                    float mn = fmaxf(m[c], mx);
                    if (mn != -INFINITY) {
                        float e = exp2f(sv[0] - mn) + exp2f(sv[1] - mn) + exp2f(sv[2] - mn) + exp2f(sv[3] - mn);
                        l[c] = l[c] * exp2f(m[c] - mn) + e;
                        m[c] = mn;
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) colsum[i] += exp2f(sv[i] - lrow[c]);
                }
            }
        }
        if (PASS == 2) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float s = sum_row16(colsum[i]);
                const int64_t j = j0 + lg * 4 + i;
                if (lr == i && j < n) imp[(int64_t)g * n + j] = s / (float)R;
            }
        }
    }
    if (PASS == 1) {
        // combine the 4 lane groups (same rows, different keys), then the 4 waves
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            if (c < RT) {
#pragma unroll
                for (int o = 16; o <= 32; o <<= 1) {
                    float m2 = __shfl_xor(m[c], o, 64), l2 = __shfl_xor(l[c], o, 64);
                    float mn = fmaxf(m[c], m2);
                    if (mn != -INFINITY) {
                        l[c] = l[c] * exp2f(m[c] - mn) + l2 * exp2f(m2 - mn);
                        m[c] = mn;
                    }
                }
                if (lg == 0) wstat[wid][c * 16 + lr] = make_float2(m[c], l[c]);
            }
        }
        __syncthreads();
        for (int r = threadIdx.x; r < R; r += kSnapThreads) {
            float M = -INFINITY, L = 0.f;
            for (int wv = 0; wv < 4; ++wv) {
                float2 v = wstat[wv][r];
                float mn = fmaxf(M, v.x);
                if (mn != -INFINITY) {
                    L = L * exp2f(M - mn) + v.y * exp2f(v.x - mn);
                    M = mn;
                }
            }
            pstat[((int64_t)g * gridDim.y + kb) * R + r] = make_float2(M, L);
        }
    }
}

__global__ void snap_lse_kernel(const float2* __restrict__ pstat, int64_t nblk, int R, int Hkv, float* __restrict__ lse) {
    const int gr = blockIdx.x * blockDim.x + threadIdx.x;
    if (gr >= Hkv * R) return;
    const int g = gr / R, r = gr % R;
    float M = -INFINITY;
    for (int64_t k = 0; k < nblk; ++k) M = fmaxf(M, pstat[((int64_t)g * nblk + k) * R + r].x);
    float L = 0.f;
    for (int64_t k = 0; k < nblk; ++k) {
        float2 v = pstat[((int64_t)g * nblk + k) * R + r];
        if (v.x != -INFINITY) L += v.y * exp2f(v.x - M);
    }
    lse[gr] = M + log2f(L);
}

// pooled[g][j] = ((imp[j-1] + imp[j]) + imp[j+1]) / 3, zero outside [0, n); written with row
// stride `ps` into the workspace and, when requested, densely into pooled_out.
__global__ void snap_pool_kernel(const float* __restrict__ imp, int64_t n, int Hkv, int64_t ps,
                                 float* __restrict__ pooled, float* __restrict__ pooled_out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n * Hkv) return;
    const int64_t g = i / n, j = i % n;
    const float* row = imp + g * n;
    float a = j > 0 ? row[j - 1] : 0.f;
    float c = j + 1 < n ? row[j + 1] : 0.f;
    const float v = ((a + row[j]) + c) / 3.0f;
    pooled[g * ps + j] = v;
    if (pooled_out) pooled_out[i] = v;
}

// K_out[s][g] = K[idx[g][s]][g]; one 16-byte piece per thread
__global__ void snap_gather_kernel(const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                   const int32_t* __restrict__ idx, int64_t n, int64_t ce, int Hkv,
                                   uint16_t* __restrict__ K_out, uint16_t* __restrict__ V_out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= ce * Hkv * 16) return;
    const int64_t piece = i % 16, sg = i / 16;
    const int64_t s = sg / Hkv, g = sg % Hkv;
    int64_t t = idx[g * ce + s];
    t = t < 0 ? 0 : (t >= n ? n - 1 : t);
    const int64_t src = (t * Hkv + g) * kD + piece * 8;
    const int64_t dst = (s * Hkv + g) * kD + piece * 8;
    *reinterpret_cast<uint4*>(K_out + dst) = *reinterpret_cast<const uint4*>(K + src);
    *reinterpret_cast<uint4*>(V_out + dst) = *reinterpret_cast<const uint4*>(V + src);
}

struct SnapLayout {
    int64_t nblk;
    float2* pstat;
    float *lse, *imp, *pooled;
    void* sel_ws;
    size_t sel_bytes, bytes;
};

static SnapLayout snap_layout(void* ws, int64_t n, int w, int Hq, int Hkv, int64_t c) {
    SnapLayout L;
    const int R = (Hq / Hkv) * w;
    L.nblk = (n + kSnapKT - 1) / kSnapKT;
    WsCarver wc(ws);
    L.pstat = wc.take<float2>((size_t)Hkv * L.nblk * R);
    L.lse = wc.take<float>((size_t)Hkv * R);
    L.imp = wc.take<float>((size_t)Hkv * n);
    L.pooled = wc.take<float>((size_t)Hkv * score_stride(n));
    int64_t ce = c < n ? c : n;
    L.sel_bytes = rows_topk_workspace(Hkv, n, ce);
    L.sel_ws = wc.take<char>(L.sel_bytes);
    L.bytes = wc.size();
    return L;
}

size_t snapkv_workspace(int64_t n, int w, int Hq, int Hkv, int64_t c) {
    return snap_layout(nullptr, n, w, Hq, Hkv, c).bytes;
}

hipError_t launch_snapkv(const uint16_t* q_obs, const uint16_t* K, const uint16_t* V, int64_t n, int w, int Hq,
                         int Hkv, int64_t c, int32_t* idx_out, uint16_t* K_out, uint16_t* V_out, float* imp_out,
                         float* pooled_out, void* ws, size_t ws_bytes, hipStream_t stream) {
    SnapLayout L = snap_layout(ws, n, w, Hq, Hkv, c);
    if (L.bytes > ws_bytes) return hipErrorInvalidValue;
    const int R = (Hq / Hkv) * w;
    float* imp = imp_out ? imp_out : L.imp;
    float* pooled = L.pooled;
    const size_t shq = (size_t)R * kD * 2;
    dim3 grid(Hkv, (unsigned)L.nblk);
    hipLaunchKernelGGL(snap_pass_kernel<1>, grid, dim3(kSnapThreads), shq, stream, q_obs, K, n, w, Hq, Hkv, L.pstat,
                       nullptr, nullptr);
    hipLaunchKernelGGL(snap_lse_kernel, dim3((Hkv * R + 255) / 256), dim3(256), 0, stream, L.pstat, L.nblk, R, Hkv,
                       L.lse);
    hipLaunchKernelGGL(snap_pass_kernel<2>, grid, dim3(kSnapThreads), shq, stream, q_obs, K, n, w, Hq, Hkv, nullptr,
                       L.lse, imp);
    const int64_t tot = n * Hkv;
    hipLaunchKernelGGL(snap_pool_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, stream, imp, n, Hkv,
                       score_stride(n), pooled, pooled_out);
    const int64_t ce = c < n ? c : n;
    hipError_t e = launch_rows_topk(pooled, score_stride(n), Hkv, n, ce, idx_out, L.sel_ws, L.sel_bytes, stream);
    if (e != hipSuccess) return e;
    const int64_t pieces = ce * Hkv * 16;
    hipLaunchKernelGGL(snap_gather_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, stream, K, V, idx_out,
                       n, ce, Hkv, K_out, V_out);
    return hipGetLastError();
}

}  // namespace qasi

namespace qasi {
hipError_t init_snap_kernels() {
    const int bytes = 256 * kD * 2;
    hipError_t e = hipFuncSetAttribute((const void*)snap_pass_kernel<1>, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute((const void*)snap_pass_kernel<2>, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}
}  // namespace qasi
