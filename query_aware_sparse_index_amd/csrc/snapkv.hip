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
//   pass 2 (snap_pass_kernel<2>): each block first combines the pass-1 blocks' (m, l) of its
//                                 rows into LSE_r (log2 domain), while its first keys load;
//                                 then p = 2^(s - LSE_r), and the column sum over the R rows (a
//                                 16-lane DPP butterfly per 16-row tile) gives imp[j] * R
// Scores are kept in the log2 domain (s = q.k * log2(e)/sqrt(128)) so that exp2 is used.
#include <type_traits>
#include <utility>

#include "qasi_device.h"
#include "qasi_internal.h"

namespace qasi {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kSnapThreads = 512;     // 8 waves
constexpr int kSnapKTW = 4;           // 16-key tiles per wave, held in registers
constexpr int kSnapKT = 8 * 16 * kSnapKTW;   // keys per block (512)
constexpr float kSnapScale = 1.4426950408889634f / 11.313708498984761f;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
    bf16x8_t r;
    __builtin_memcpy(&r, &v, 16);
    return r;
}

// grid: x = KV head g, y = p < P.  The block stages Q_g in LDS once, then walks the key blocks
// kb = p, p + P, ... of kSnapKT keys (concurrent blocks cover adjacent key ranges).  RT = R / 16
// row tiles, R = G * w rows, row r = hh * w + t  <->  q_obs[t][g*G + hh].  In key block kb,
// wave wid owns the key tiles kb * kSnapKT + (wid * kSnapKTW + kt) * 16, kt < kSnapKTW: their
// A fragments (16 keys x 128 dims) sit in registers while the row tiles' B fragments stream
// from LDS, each used for kSnapKTW MFMAs; the next key block's fragments are loaded into a
// second register set while the current one is consumed.
template <int PASS, int RT>
__global__ __launch_bounds__(kSnapThreads) void snap_pass_kernel(const uint16_t* __restrict__ q_obs,
                                                                const uint16_t* __restrict__ K, int64_t n, int w,
                                                                int Hq, int Hkv, int64_t nblk,
                                                                float2* __restrict__ pstat,
                                                                float* __restrict__ imp) {
    constexpr int R = RT * 16;
    constexpr int NW = kSnapThreads / 64;
    extern __shared__ uint4 sQ[];   // [R][16] uint4 (128 bf16 per row), row-swizzled by (row & 15)
    __shared__ float2 wstat[(PASS == 1) ? NW : 1][(PASS == 1) ? R : 1];
    __shared__ float2 mlst[(PASS == 1) ? NW * RT * 64 : 1];   // pass 1: running (max, sum) per lane
    __shared__ float sL[(PASS == 2) ? R : 1];   // pass 2: LSE (log2 domain) of the rows
    const int g = blockIdx.x;
    const int p = blockIdx.y, P = gridDim.y;
    const int G = Hq / Hkv;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;

    // stage Q_g (R x 128 bf16) in LDS; 16-byte chunk c of row r goes to slot (c ^ (r & 15))
    for (int i = threadIdx.x; i < R * 16; i += kSnapThreads) {
        const int r = i / 16, c = i % 16;
        const int hh = r / w, t = r % w;
        const uint4 v = *reinterpret_cast<const uint4*>(q_obs + ((int64_t)t * Hq + g * G + hh) * kD + c * 8);
        sQ[r * 16 + (c ^ (r & 15))] = v;
    }

    // A fragments of key block kb: key jw(kb) + kt*16 + lr, dims 32 s + 8 lg .. +8
    auto key0 = [&](int64_t kb) { return kb * kSnapKT + (int64_t)wid * kSnapKTW * 16; };
    // keys past the end load key n - 1 (in bounds); their scores are masked in compute
    auto load = [&](bf16x8_t (&a)[kSnapKTW][4], int64_t kb) {
        const int64_t jw = key0(kb);
#pragma unroll
        for (int kt = 0; kt < kSnapKTW; ++kt) {
            const int64_t jl = min(jw + kt * 16 + lr, n - 1);
#pragma unroll
            for (int s = 0; s < 4; ++s)
                a[kt][s] = as_bf16x8(*reinterpret_cast<const uint4*>(K + (jl * Hkv + g) * kD + s * 32 + lg * 8));
        }
    };

    if (PASS == 1)
        for (int c = 0; c < RT; ++c) mlst[(wid * RT + c) * 64 + lane] = make_float2(-INFINITY, 0.f);

    // one key block: pass 1 folds its scores into (m, l), pass 2 writes its keys' importance
    // MASK: the wave's keys reach past n (only in the last key block)
    auto compute = [&](const bf16x8_t (&a)[kSnapKTW][4], int64_t kb, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const int64_t jw = key0(kb);
        float colsum[(PASS == 2) ? kSnapKTW : 1][4];
#pragma unroll
        for (int kt = 0; kt < ((PASS == 2) ? kSnapKTW : 1); ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) colsum[kt][i] = 0.f;

        // (row r = 16 c + lr, so r & 15 = lr: the LDS addresses are a per-lane base plus a
        // constant offset per tile)
        // The per-lane bases pass through an empty register constraint once per key block: the
        // reads of the fully unrolled row-tile loop are then not hoisted out of the key-block loop
        // (they do not change across key blocks), which would pin all 16 tiles' fragments.
        int qa[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            qa[s] = lr * 16 + ((s * 4 + lg) ^ lr);
            asm volatile("" : "+v"(qa[s]));
        }
        int la = lr;
        asm volatile("" : "+v"(la));
        auto tile_b = [&](int c, bf16x8_t (&bq)[4]) {
#pragma unroll
            for (int s = 0; s < 4; ++s) bq[s] = as_bf16x8(sQ[c * 256 + qa[s]]);
        };
        // the MFMAs of a row tile: 4 key tiles x 4 dim slices
        auto tile_mma = [&](const bf16x8_t (&bq)[4], f32x4_t (&acc)[kSnapKTW]) {
#pragma unroll
            for (int kt = 0; kt < kSnapKTW; ++kt) acc[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int kt = 0; kt < kSnapKTW; ++kt)
                    acc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[kt][s], bq[s], acc[kt], 0, 0, 0);
        };
        // the vector work on row tile c's scores; pass 1 folds them into the running (max, sum)
        // ml of the lane's row and returns it
        auto tile_epi = [&](int c, f32x4_t (&acc)[kSnapKTW], float2 ml) {
            if (MASK) {
#pragma unroll
                for (int kt = 0; kt < kSnapKTW; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (jw + kt * 16 + lg * 4 + i >= n) acc[kt][i] = -INFINITY;
            }
            if (PASS == 1) {
                // online (max, sum) of 2^(scale * dot) for row r over this lane's keys
                float mx = acc[0][0];
#pragma unroll
                for (int kt = 0; kt < kSnapKTW; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, acc[kt][i]);
                const float mn = fmaxf(ml.x, mx * kSnapScale);
                // while every score seen is -inf, subtract 0 so that the terms are 0, not NaN
                const float ms = (mn == -INFINITY) ? 0.f : mn;
                float e = 0.f;
#pragma unroll
                for (int kt = 0; kt < kSnapKTW; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) e += fast_exp2(fmaf(acc[kt][i], kSnapScale, -ms));
                ml.y = ml.y * fast_exp2(ml.x - ms) + e;
                ml.x = mn;
            } else {
                const float lr_c = sL[c * 16 + la];
#pragma unroll
                for (int kt = 0; kt < kSnapKTW; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) colsum[kt][i] += fast_exp2(fmaf(acc[kt][i], kSnapScale, -lr_c));
            }
            return ml;
        };
        // Software pipeline over the row tiles, one scheduling region per tile c: the LDS reads
        // of tile c + 1's B fragments and tile c's running (max, sum) or LSE, tile c + 1's MFMAs,
        // and tile c's vector work, with one MFMA issued between every few VALU instructions so
        // that the matrix core and the vector unit of a SIMD work at the same time within one
        // wave.
        auto interleave = [&]() {
            __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);   // LDS reads
#pragma unroll
            for (int k = 0; k < 4 * kSnapKTW; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, (PASS == 1) ? 4 : 3, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        f32x4_t acc[2][kSnapKTW];
        // one region: tile c + 1's MFMAs (when it exists) into acc[nx], tile c's vector work on
        // acc[cu]
        auto region = [&](int c, bool next, f32x4_t (&ac)[kSnapKTW], f32x4_t (&an)[kSnapKTW]) {
            if (next) {
                bf16x8_t bq[4];
                tile_b(c + 1, bq);
                tile_mma(bq, an);
            }
            if constexpr (PASS == 1) {
                float2* mp = &mlst[(wid * RT + c) * 64 + lane];
                *mp = tile_epi(c, ac, *mp);
            } else {
                tile_epi(c, ac, float2{0.f, 0.f});
            }
            interleave();
        };
        {
            bf16x8_t bq[4];
            tile_b(0, bq);
            tile_mma(bq, acc[0]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (PASS == 1) {
#pragma unroll
            for (int c = 0; c < RT; ++c) region(c, c + 1 < RT, acc[c & 1], acc[(c & 1) ^ 1]);
        } else {
            // pass 2 holds 16 more registers (the column sums): with a fully unrolled tile loop
            // the compiler moves the MFMAs away from their vector work and spills, so the tiles
            // run as a loop over pairs with the last one or two peeled
            int c = 0;
#pragma unroll 1
            for (; c + 2 < RT; c += 2) {
                region(c, true, acc[0], acc[1]);
                region(c + 1, true, acc[1], acc[0]);
            }
            if (RT - c == 2) {
                region(c, true, acc[0], acc[1]);
                region(c + 1, false, acc[1], acc[0]);
            } else {
                region(c, false, acc[0], acc[1]);
            }
        }

        if (PASS == 2) {
            // column sums over the 16 rows of each lane group (DPP butterfly); lane lr then keeps
            // the sum of key tile lr / 4, key lg * 4 + lr % 4, so that the wave's 64 keys leave in
            // one store
            float v = 0.f;
#pragma unroll
            for (int kt = 0; kt < kSnapKTW; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float sv = sum_row16(colsum[kt][i]);
                    v = (lr == kt * 4 + i) ? sv : v;
                }
            const int64_t j = jw + (lr >> 2) * 16 + lg * 4 + (lr & 3);
            if (!MASK || j < n) imp[(int64_t)g * n + j] = v / (float)R;
        }
    };

    // the wave index is uniform: read it into a scalar so that the full / masked choice is a
    // scalar branch and the row-tile loop stays one basic block
    const int64_t wkeys = (int64_t)__builtin_amdgcn_readfirstlane(wid) * kSnapKTW * 16 + kSnapKTW * 16;
    auto run = [&](const bf16x8_t (&a)[kSnapKTW][4], int64_t kb) {
        if (kb * kSnapKT + wkeys <= n)
            compute(a, kb, std::false_type{});
        else
            compute(a, kb, std::true_type{});
    };

    // The loads are unconditional: a key block past the end loads key n - 1 (the clamp in
    // load), so that every path through the loop issues the same memory operations and the
    // waits before the MFMAs count the prefetch as still in flight instead of draining it.
    // Pass 2 walks the key blocks from the last one down: the keys pass 1 read last are the
    // ones most likely still held in the last-level cache.  Steps past the end stay unmapped
    // (their loads clamp to key n - 1).
    auto order = [&](int64_t kb) { return (PASS == 2 && kb < nblk) ? nblk - 1 - kb : kb; };
    bf16x8_t a0[kSnapKTW][4], a1[kSnapKTW][4];
    load(a0, order(p));
    if (PASS == 2) {
        // LSE_r = M + log2(L) over the P pass-1 blocks' (M, L) of row r: two lanes per row, each
        // half of the blocks with 8 loads in flight, then the pair combined
        static_assert(2 * R <= kSnapThreads, "two lanes per row");
        const int r = threadIdx.x >> 1, hf = threadIdx.x & 1;
        float M = -INFINITY, L = 0.f;
        if (r < R)
            for (int k0 = hf; k0 < P; k0 += 2 * 8) {
                float2 v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int k = k0 + 2 * u;
                    v[u] = k < P ? pstat[((int64_t)g * P + k) * R + r] : make_float2(-INFINITY, 0.f);
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float mn = fmaxf(M, v[u].x);
                    if (mn != -INFINITY) {
                        L = L * fast_exp2(M - mn) + v[u].y * fast_exp2(v[u].x - mn);
                        M = mn;
                    }
                }
            }
        const float m2 = __shfl_xor(M, 1, 64), l2 = __shfl_xor(L, 1, 64);
        const float mn = fmaxf(M, m2);
        if (mn != -INFINITY) L = L * fast_exp2(M - mn) + l2 * fast_exp2(m2 - mn);
        if (r < R && hf == 0) sL[r] = mn + log2f(L);
    }
    __syncthreads();
    for (int64_t kb = p; kb < nblk; kb += 2 * (int64_t)P) {
        load(a1, order(kb + P));
        run(a0, order(kb));
        if (kb + P >= nblk) break;
        load(a0, order(kb + 2 * (int64_t)P));
        run(a1, order(kb + P));
    }

    if (PASS == 1) {
        // combine the 4 lane groups (same rows, different keys), then the waves
        for (int c = 0; c < RT; ++c) {
            const float2 ml = mlst[(wid * RT + c) * 64 + lane];
            float mc = ml.x, lc = ml.y;
#pragma unroll
            for (int o = 16; o <= 32; o <<= 1) {
                const float m2 = __shfl_xor(mc, o, 64), l2 = __shfl_xor(lc, o, 64);
                const float mn = fmaxf(mc, m2);
                if (mn != -INFINITY) {
                    lc = lc * fast_exp2(mc - mn) + l2 * fast_exp2(m2 - mn);
                    mc = mn;
                }
            }
            if (lg == 0) wstat[wid][c * 16 + lr] = make_float2(mc, lc);
        }
        __syncthreads();
        for (int r = threadIdx.x; r < R; r += kSnapThreads) {
            float M = -INFINITY, L = 0.f;
#pragma unroll
            for (int wv = 0; wv < NW; ++wv) {
                const float2 v = wstat[wv][r];
                const float mn = fmaxf(M, v.x);
                if (mn != -INFINITY) {
                    L = L * fast_exp2(M - mn) + v.y * fast_exp2(v.x - mn);
                    M = mn;
                }
            }
            pstat[((int64_t)g * P + p) * R + r] = make_float2(M, L);
        }
    }
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

// Cluster-based retention ([SK] "Top-k SelectionとCluster-based Retention", eq. S_final): the
// widened lists come from the selection expansion kernel (no always-kept tokens); this gather
// copies their rows and writes zero rows for the empty slots (-1) that pad a head's list to the
// capacity.  K_out[s][g] = idx[g][s] >= 0 ? K[idx[g][s]][g] : 0; one 16-byte piece per thread.
__global__ void snap_gather_padded_kernel(const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                          const int32_t* __restrict__ idx, int64_t n, int64_t cap, int Hkv,
                                          uint16_t* __restrict__ K_out, uint16_t* __restrict__ V_out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= cap * Hkv * 16) return;
    const int64_t piece = i % 16, sg = i / 16;
    const int64_t s = sg / Hkv, g = sg % Hkv;
    const int64_t t = idx[g * cap + s];
    const int64_t dst = (s * Hkv + g) * kD + piece * 8;
    uint4 k = make_uint4(0, 0, 0, 0), v = make_uint4(0, 0, 0, 0);
    if (t >= 0) {
        const int64_t tc = t >= n ? n - 1 : t;
        const int64_t src = (tc * Hkv + g) * kD + piece * 8;
        k = *reinterpret_cast<const uint4*>(K + src);
        v = *reinterpret_cast<const uint4*>(V + src);
    }
    *reinterpret_cast<uint4*>(K_out + dst) = k;
    *reinterpret_cast<uint4*>(V_out + dst) = v;
}

hipError_t launch_snapkv_clusters(const int32_t* idx, int64_t n, int Hkv, int64_t ce, int64_t k_cluster,
                                  const uint16_t* K, const uint16_t* V, int32_t* idx_out, uint16_t* K_out,
                                  uint16_t* V_out, int64_t* valid_out, uint32_t* chunk_counts, hipStream_t stream) {
    // one sequence {0, n} with Hkv lists of ce entries: the bounds travel as launch arguments
    const int64_t offs[2] = {0, n};
    const int64_t cnt[1] = {ce};
    hipError_t e = launch_expand(idx, nullptr, cnt, nullptr, offs, 1, Hkv, 0, 0, k_cluster, idx_out, nullptr,
                                 valid_out, chunk_counts, stream);
    if (e != hipSuccess) return e;
    const int64_t cap = expand_capacity(ce, n, 0, 0, k_cluster);
    const int64_t pieces = cap * Hkv * 16;
    hipLaunchKernelGGL(snap_gather_padded_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, stream, K, V,
                       idx_out, n, cap, Hkv, K_out, V_out);
    return hipGetLastError();
}

// one pass block per CU: 256 / Hkv per KV head, at most one per key block
static int64_t snap_blocks_per_head(int Hkv, int64_t nblk) {
    int64_t p = 256 / Hkv;
    return p < nblk ? p : (nblk > 0 ? nblk : 1);
}

struct SnapLayout {
    int64_t nblk, P;
    float2* pstat;
    float *imp, *pooled;
    void* sel_ws;
    size_t sel_bytes, bytes;
};

static SnapLayout snap_layout(void* ws, int64_t n, int w, int Hq, int Hkv, int64_t c) {
    SnapLayout L;
    const int R = (Hq / Hkv) * w;
    L.nblk = (n + kSnapKT - 1) / kSnapKT;
    L.P = snap_blocks_per_head(Hkv, L.nblk);
    WsCarver wc(ws);
    L.pstat = wc.take<float2>((size_t)Hkv * L.P * R);
    L.imp = wc.take<float>((size_t)Hkv * n);
    L.pooled = wc.take<float>((size_t)Hkv * score_stride(n));
    (void)c;
    L.sel_bytes = snap_topc_workspace(Hkv, n);
    L.sel_ws = wc.take<char>(L.sel_bytes);
    L.bytes = wc.size();
    return L;
}

template <int PASS, int RT>
static hipError_t launch_pass_rt(dim3 grid, size_t shq, hipStream_t stream, const uint16_t* q_obs, const uint16_t* K,
                                 int64_t n, int w, int Hq, int Hkv, int64_t nblk, float2* pstat, float* imp) {
    hipLaunchKernelGGL((snap_pass_kernel<PASS, RT>), grid, dim3(kSnapThreads), shq, stream, q_obs, K, n, w, Hq, Hkv,
                       nblk, pstat, imp);
    return hipGetLastError();
}

template <int PASS, int... RTS>
static hipError_t dispatch_pass(int rt, std::integer_sequence<int, RTS...>, dim3 grid, size_t shq, hipStream_t stream,
                                const uint16_t* q_obs, const uint16_t* K, int64_t n, int w, int Hq, int Hkv,
                                int64_t nblk, float2* pstat, float* imp) {
    hipError_t e = hipErrorInvalidValue;
    ((rt == RTS + 1
          ? (e = launch_pass_rt<PASS, RTS + 1>(grid, shq, stream, q_obs, K, n, w, Hq, Hkv, nblk, pstat, imp), 0)
          : 0),
     ...);
    return e;
}

template <int PASS>
static hipError_t launch_snap_pass(int rt, dim3 grid, size_t shq, hipStream_t stream, const uint16_t* q_obs,
                                   const uint16_t* K, int64_t n, int w, int Hq, int Hkv, int64_t nblk, float2* pstat,
                                   float* imp) {
    return dispatch_pass<PASS>(rt, std::make_integer_sequence<int, 16>{}, grid, shq, stream, q_obs, K, n, w, Hq, Hkv,
                               nblk, pstat, imp);
}

template <int... RTS>
static hipError_t set_lds_all(int bytes, std::integer_sequence<int, RTS...>) {
    hipError_t e = hipSuccess;
    ((e == hipSuccess ? (e = hipFuncSetAttribute((const void*)snap_pass_kernel<1, RTS + 1>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, bytes)) : e), ...);
    ((e == hipSuccess ? (e = hipFuncSetAttribute((const void*)snap_pass_kernel<2, RTS + 1>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, bytes)) : e), ...);
    return e;
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
    dim3 grid(Hkv, (unsigned)L.P);
    hipError_t e = launch_snap_pass<1>(R / 16, grid, shq, stream, q_obs, K, n, w, Hq, Hkv, L.nblk, L.pstat, nullptr);
    if (e != hipSuccess) return e;
    e = launch_snap_pass<2>(R / 16, grid, shq, stream, q_obs, K, n, w, Hq, Hkv, L.nblk, L.pstat, imp);
    if (e != hipSuccess) return e;
    e = launch_snap_topc(imp, n, Hkv, c, pooled, score_stride(n), pooled_out, idx_out, L.sel_ws, L.sel_bytes, stream);
    if (e != hipSuccess) return e;
    const int64_t ce = c < n ? c : n;
    const int64_t pieces = ce * Hkv * 16;
    hipLaunchKernelGGL(snap_gather_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, stream, K, V, idx_out,
                       n, ce, Hkv, K_out, V_out);
    return hipGetLastError();
}

}  // namespace qasi

namespace qasi {
hipError_t init_snap_kernels() { return set_lds_all(256 * kD * 2, std::make_integer_sequence<int, 16>{}); }
}  // namespace qasi
