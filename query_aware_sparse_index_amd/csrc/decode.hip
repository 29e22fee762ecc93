// Sparse (gathered) and dense split-K flash decode with a log-sum-exp merge.
//
// [TS] "Token-Level Selection と Sparse Attention", eq. Attention(Q, K_S, V_S) =
// softmax(Q K_S^T / sqrt(d)) V_S over the selected tokens, which include the sink and local
// tokens; the "output merge" of the five-step integration is the log-sum-exp merge of the
// partial softmax results of disjoint chunks of the list.
//
// Work item = (sequence b, chunk of kDecCH list entries) [vote / dense] or (b, KV head g,
// chunk) [per-head].  Items are dispatched in list order, so the chip sweeps the sorted lists
// front to back.  A block has 8 waves (vote / dense) or G waves (per-head).  In vote mode a
// wave is tied to a KV head g and serves the G query heads of g, so each gathered K/V row is
// read once for the whole GQA group.  A wave is 4 rows of 16 lanes; a row takes one entry at
// a time and lane p holds dims [8p, 8p+8) (one 16-byte load of K or V).
//   phase 1: z = q . k * log2(e)/sqrt(128) for every entry of the chunk (row butterfly)
//   phase 2: per-head chunk max m, p = exp2(z - m), l = sum p (LDS)
//   phase 3: acc += p * v
// The partial (m, l, acc[128]) of every chunk and head goes to the workspace; the merge kernel
// combines the chunks of a sequence: out = sum_c acc_c 2^(m_c - M) / sum_c l_c 2^(m_c - M).
#include "qasi_device.h"
#include "qasi_internal.h"

namespace qasi {

constexpr int kDecCH = 64;            // list entries per chunk
static_assert(kDecCH % 16 == 0, "the softmax phase gives each head slot one 16-lane row");
constexpr float kLog2eOverSqrtD = 1.4426950408889634f / 11.313708498984761f;
__device__ __forceinline__ bool find_list_chunk(const I64Arg& counts, int B, int64_t item, int& b,
                                                int64_t& first, int64_t& nch, int64_t& j0, int64_t& len,
                                                int64_t& kpre) {
    int64_t acc = 0, kp = 0;
    for (int i = 0; i < B; ++i) {
        int64_t n = counts[i];
        int64_t nb = (n + kDecCH - 1) / kDecCH;
        if (item < acc + nb) {
            b = i;
            first = acc;
            nch = nb;
            j0 = (item - acc) * kDecCH;
            len = n - j0 < kDecCH ? n - j0 : kDecCH;
            kpre = kp;
            return true;
        }
        acc += nb;
        kp += n;
    }
    return false;
}

// MODE 0: shared list per sequence (vote); MODE 1: list per query head; MODE 2: dense
// (the list is implicit: entry j is token j, counts are the sequence lengths).
template <int G, int MODE>
__global__ __launch_bounds__(512) void decode_partial_kernel(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ K,
                                                            const uint16_t* __restrict__ V,
                                                            I64Arg offsets,
                                                            const int32_t* __restrict__ idx,
                                                            I64Arg counts, int B, int Hq,
                                                            int Hkv, float* __restrict__ part_acc,
                                                            float2* __restrict__ part_ml) {
    constexpr int GH = (MODE == 1) ? 1 : G;          // query heads per wave
    constexpr int NW = (MODE == 1) ? G : 8;          // waves per block
    __shared__ float zb[((MODE == 1) ? G : 64) * kDecCH];   // [head slot][entry]
    __shared__ float red[NW * GH * kD];
    __shared__ float stat[((MODE == 1) ? G : 64) * 2];
    __shared__ int32_t tok[(MODE == 1) ? G * kDecCH : kDecCH];

    int b;
    int64_t first, nch, j0, len, kpre;
    if (!find_list_chunk(counts, B, blockIdx.x, b, first, nch, j0, len, kpre)) return;
    const int64_t off = offsets[b];
    const int32_t nmax = (int32_t)(offsets[b + 1] - off - 1);   // list entries are clamped to [0, n_b)
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int row = lane >> 4, p = lane & 15;

    // wave role
    int g, sub, nsub, hbase;
    if (MODE == 1) { g = blockIdx.y; sub = 0; nsub = 1; hbase = g * G + wid; }
    else { g = wid % Hkv; sub = wid / Hkv; nsub = 8 / Hkv; hbase = g * G; }
    const bool wave_on = (MODE == 1) ? true : (wid < Hkv * nsub);
    const int hslot0 = (MODE == 1) ? wid : hbase;   // first head slot of this wave in zb/stat

    // token ids of the chunk
    if (MODE == 1) {
        for (int i = threadIdx.x; i < G * kDecCH; i += NW * 64) {
            int w = i / kDecCH, j = i % kDecCH;
            int h = g * G + w;
            int32_t t = (j < len) ? idx[Hq * kpre + (int64_t)h * counts[b] + j0 + j] : 0;
            tok[i] = t < 0 ? 0 : (t > nmax ? nmax : t);
        }
    } else {
        for (int i = threadIdx.x; i < kDecCH; i += NW * 64) {
            int32_t t = (i < len) ? ((MODE == 2) ? (int32_t)(j0 + i) : idx[kpre + j0 + i]) : 0;
            tok[i] = t < 0 ? 0 : (t > nmax ? nmax : t);
        }
    }

    // queries: lane p holds dims [8p, 8p+8) of its heads, scaled into the log2 domain
    float qr[GH][8];
#pragma unroll
    for (int hh = 0; hh < GH; ++hh) {
        const uint16_t* qh = q + ((int64_t)b * Hq + hbase + hh) * kD + p * 8;
        uint4 w = *reinterpret_cast<const uint4*>(qh);
        qr[hh][0] = bf16_lo(w.x) * kLog2eOverSqrtD; qr[hh][1] = bf16_hi(w.x) * kLog2eOverSqrtD;
        qr[hh][2] = bf16_lo(w.y) * kLog2eOverSqrtD; qr[hh][3] = bf16_hi(w.y) * kLog2eOverSqrtD;
        qr[hh][4] = bf16_lo(w.z) * kLog2eOverSqrtD; qr[hh][5] = bf16_hi(w.z) * kLog2eOverSqrtD;
        qr[hh][6] = bf16_lo(w.w) * kLog2eOverSqrtD; qr[hh][7] = bf16_hi(w.w) * kLog2eOverSqrtD;
    }
    __syncthreads();

    // entries handled by this (wave, row): i = sub + nsub * (row + 4 k)
    const int istep = 4 * nsub;
    const int ibeg = sub + nsub * row;
    constexpr int UNR = 4;

    // phase 1: scores
    if (wave_on) {
        for (int i0 = ibeg; i0 < len; i0 += UNR * istep) {
            uint4 kv[UNR];
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                int i = i0 + u * istep;
                kv[u] = make_uint4(0, 0, 0, 0);
                if (i < len) {
                    int t = (MODE == 1) ? tok[wid * kDecCH + i] : tok[i];
                    kv[u] = *reinterpret_cast<const uint4*>(K + ((off + t) * Hkv + g) * kD + p * 8);
                }
            }
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                int i = i0 + u * istep;
                float kf[8] = {bf16_lo(kv[u].x), bf16_hi(kv[u].x), bf16_lo(kv[u].y), bf16_hi(kv[u].y),
                               bf16_lo(kv[u].z), bf16_hi(kv[u].z), bf16_lo(kv[u].w), bf16_hi(kv[u].w)};
#pragma unroll
                for (int hh = 0; hh < GH; ++hh) {
                    float s = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) s = fmaf(qr[hh][e], kf[e], s);
                    s = sum_row16(s);
                    if (p == hh && i < len) zb[(hslot0 + hh) * kDecCH + i] = s;
                }
            }
        }
    }
    __syncthreads();

    // phase 2: per-head max, exponentials and sums; one 16-lane row per head slot, kDecCH / 16
    // entries per lane, row reductions through DPP
    const int nslots = (MODE == 1) ? G : Hq;
    constexpr int EPL = kDecCH / 16;   // entries per lane
    for (int hs = threadIdx.x >> 4; hs < nslots; hs += NW * 4) {
        const int l16 = threadIdx.x & 15;
        float z[EPL];
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const int i = l16 + 16 * e;
            z[e] = i < len ? zb[hs * kDecCH + i] : -INFINITY;
            mx = fmaxf(mx, z[e]);
        }
        const float m = max_row16(mx);
        float l = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const int i = l16 + 16 * e;
            const float ev = i < len ? fast_exp2(z[e] - m) : 0.f;
            zb[hs * kDecCH + i] = ev;
            l += ev;
        }
        l = sum_row16(l);
        if (l16 == 0) { stat[hs * 2] = m; stat[hs * 2 + 1] = l; }
    }
    __syncthreads();

    // phase 3: acc += p * v
    float acc[GH][8];
#pragma unroll
    for (int hh = 0; hh < GH; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;
    if (wave_on) {
        for (int i0 = ibeg; i0 < len; i0 += UNR * istep) {
            uint4 vv[UNR];
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                int i = i0 + u * istep;
                vv[u] = make_uint4(0, 0, 0, 0);
                if (i < len) {
                    int t = (MODE == 1) ? tok[wid * kDecCH + i] : tok[i];
                    vv[u] = *reinterpret_cast<const uint4*>(V + ((off + t) * Hkv + g) * kD + p * 8);
                }
            }
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                int i = i0 + u * istep;
                if (i < len) {
                    float vf[8] = {bf16_lo(vv[u].x), bf16_hi(vv[u].x), bf16_lo(vv[u].y), bf16_hi(vv[u].y),
                                   bf16_lo(vv[u].z), bf16_hi(vv[u].z), bf16_lo(vv[u].w), bf16_hi(vv[u].w)};
#pragma unroll
                    for (int hh = 0; hh < GH; ++hh) {
                        float pw = zb[(hslot0 + hh) * kDecCH + i];
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[hh][e] = fmaf(pw, vf[e], acc[hh][e]);
                    }
                }
            }
        }
    }
    // reduce the 4 rows of the wave
#pragma unroll
    for (int hh = 0; hh < GH; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = acc[hh][e];
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 32, 64);
            acc[hh][e] = v;
        }
    if (row == 0) {
#pragma unroll
        for (int hh = 0; hh < GH; ++hh)
#pragma unroll
            for (int e = 0; e < 8; ++e) red[(wid * GH + hh) * kD + p * 8 + e] = wave_on ? acc[hh][e] : 0.f;
    }
    __syncthreads();

    // write the partials: (m, l, acc) per head of the block
    if (MODE == 1) {
        for (int o = threadIdx.x; o < G * kD; o += NW * 64) {
            int w = o / kD, d = o % kD;
            int h = g * G + w;
            const int64_t slot = (int64_t)blockIdx.x * Hq + h;
            part_acc[slot * kD + d] = red[w * kD + d];
            if (d == 0) part_ml[slot] = make_float2(stat[w * 2], stat[w * 2 + 1]);
        }
    } else {
        for (int o = threadIdx.x; o < Hq * kD; o += NW * 64) {
            int h = o / kD, d = o % kD;
            int gg = h / G, hh = h % G;
            float s = 0.f;
            for (int sb = 0; sb < nsub; ++sb) s += red[((sb * Hkv + gg) * GH + hh) * kD + d];
            const int64_t slot = (int64_t)blockIdx.x * Hq + h;
            part_acc[slot * kD + d] = s;
            if (d == 0) part_ml[slot] = make_float2(stat[h * 2], stat[h * 2 + 1]);
        }
    }
}

// Merge of the chunk partials of each (sequence, head).  Block = (b * Hq + h, 16-dim slice);
// its 1024 threads are (chunk group cg < 64, dim dl < 16).  Every thread first requests its
// chunks' (m, l) and acc values (8 chunks in flight, every 64th chunk of the sequence), then
// the block takes the maximum M of all chunk maxima, and the weighted sums
// sum_c acc_c 2^(m_c - M) and sum_c l_c 2^(m_c - M) are reduced over the 64 groups in LDS.
__global__ __launch_bounds__(1024) void decode_merge_kernel(const float* __restrict__ part_acc,
                                                           const float2* __restrict__ part_ml,
                                                           I64Arg counts, int B, int Hq,
                                                           float* __restrict__ out) {
    constexpr int U = 8;
    __shared__ float sa[64][17];
    __shared__ float sl[64];
    __shared__ float smax[16];
    const int bh = blockIdx.x, b = bh / Hq, h = bh % Hq, ds = blockIdx.y;
    int64_t first = 0;
    for (int i = 0; i < b; ++i) first += (counts[i] + kDecCH - 1) / kDecCH;
    const int64_t nch = (counts[b] + kDecCH - 1) / kDecCH;
    const int cg = threadIdx.x >> 4, dl = threadIdx.x & 15, d = ds * 16 + dl;
    float a = 0.f, l = 0.f;
    float M = -INFINITY;
    for (int64_t c0 = cg; c0 - cg < nch; c0 += 64 * U) {
        float x[U], mm[U], ll[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = c0 + 64 * u;
            const int64_t slot = (first + (c < nch ? c : 0)) * Hq + h;
            x[u] = part_acc[slot * kD + d];
            const float2 ml = part_ml[slot];
            mm[u] = c < nch ? ml.x : -INFINITY;
            ll[u] = ml.y;
        }
        // the block-wide maximum over every chunk seen so far
        float mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u) mx = fmaxf(mx, mm[u]);
        mx = wave_max(mx);
        __syncthreads();
        if ((threadIdx.x & 63) == 0) smax[threadIdx.x >> 6] = mx;
        __syncthreads();
        float Mn = M;
#pragma unroll
        for (int w = 0; w < 16; ++w) Mn = fmaxf(Mn, smax[w]);
        if (Mn != -INFINITY) {
            const float rs = fast_exp2(M - Mn);     // rescale what was summed under M
            a *= rs;
            l *= rs;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (c0 + 64 * u < nch) {
                    const float w = fast_exp2(mm[u] - Mn);
                    a = fmaf(x[u], w, a);
                    l = fmaf(ll[u], w, l);
                }
            }
            M = Mn;
        }
    }
    sa[cg][dl] = a;
    if (dl == 0) sl[cg] = l;
    __syncthreads();
    if (threadIdx.x < 16) {
        float A = 0.f, L = 0.f;
        for (int k = 0; k < 64; ++k) { A += sa[k][threadIdx.x]; L += sl[k]; }
        out[((int64_t)b * Hq + h) * kD + ds * 16 + threadIdx.x] = A / L;
    }
}

static int64_t list_items(const int64_t* counts_host, int B) {
    int64_t it = 0;
    for (int b = 0; b < B; ++b) it += (counts_host[b] + kDecCH - 1) / kDecCH;
    return it;
}

size_t decode_workspace(const int64_t* offsets_host, const int64_t* counts_host, int B, int Hq, int Hkv, int mode) {
    (void)Hkv;
    (void)mode;
    int64_t items = 0;
    if (counts_host) items = list_items(counts_host, B);
    else
        for (int b = 0; b < B; ++b) items += (offsets_host[b + 1] - offsets_host[b] + kDecCH - 1) / kDecCH;
    WsCarver w(nullptr);
    w.take<int64_t>((size_t)B + 1);   // dense: per-sequence lengths
    w.take<float>((size_t)items * Hq * kD);
    w.take<float2>((size_t)items * Hq);
    return w.size();
}

template <int MODE>
static hipError_t launch_partial_G(int G, dim3 grid, hipStream_t stream, const uint16_t* q, const uint16_t* K,
                                   const uint16_t* V, const I64Arg& offsets, const int32_t* idx,
                                   const I64Arg& counts, int B, int Hq, int Hkv, float* part, float2* ml) {
    dim3 block(MODE == 1 ? 64 * G : 512);
    switch (G) {
        case 1: hipLaunchKernelGGL((decode_partial_kernel<1, MODE>), grid, block, 0, stream, q, K, V, offsets, idx, counts, B, Hq, Hkv, part, ml); break;
        case 2: hipLaunchKernelGGL((decode_partial_kernel<2, MODE>), grid, block, 0, stream, q, K, V, offsets, idx, counts, B, Hq, Hkv, part, ml); break;
        case 4: hipLaunchKernelGGL((decode_partial_kernel<4, MODE>), grid, block, 0, stream, q, K, V, offsets, idx, counts, B, Hq, Hkv, part, ml); break;
        case 8: hipLaunchKernelGGL((decode_partial_kernel<8, MODE>), grid, block, 0, stream, q, K, V, offsets, idx, counts, B, Hq, Hkv, part, ml); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// dense decode: counts are the sequence lengths, computed on the device into the workspace
__global__ void lengths_kernel(I64Arg offsets, int B, int64_t* __restrict__ lens) {
    for (int b = threadIdx.x; b < B; b += blockDim.x) lens[b] = offsets[b + 1] - offsets[b];
}

hipError_t launch_sparse_decode(const uint16_t* q, const uint16_t* K, const uint16_t* V, const int64_t* offsets_dev,
                                const int64_t* offsets_host, const int32_t* idx, const int64_t* counts_dev,
                                const int64_t* counts_host, int mode, int B, int Hq, int Hkv, float* out, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
    if (decode_workspace(offsets_host, counts_host, B, Hq, Hkv, mode) > ws_bytes) return hipErrorInvalidValue;
    WsCarver w(ws);
    w.take<int64_t>((size_t)B + 1);
    const int64_t items = list_items(counts_host, B);
    float* part = w.take<float>((size_t)items * Hq * kD);
    float2* ml = w.take<float2>((size_t)items * Hq);
    const int G = Hq / Hkv;
    const I64Arg offs = i64_arg(offsets_dev, offsets_host, (int64_t)B + 1);
    const I64Arg cnts = i64_arg(counts_dev, counts_host, B);
    hipError_t e;
    if (mode == 0) e = launch_partial_G<0>(G, dim3((unsigned)items), stream, q, K, V, offs, idx, cnts, B, Hq, Hkv, part, ml);
    else e = launch_partial_G<1>(G, dim3((unsigned)items, Hkv), stream, q, K, V, offs, idx, cnts, B, Hq, Hkv, part, ml);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_merge_kernel, dim3(B * Hq, kD / 16), dim3(1024), 0, stream, part, ml, cnts, B, Hq, out);
    return hipGetLastError();
}

hipError_t launch_dense_decode(const uint16_t* q, const uint16_t* K, const uint16_t* V, const int64_t* offsets_dev,
                               const int64_t* offsets_host, int B, int Hq, int Hkv, float* out, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
    if (decode_workspace(offsets_host, nullptr, B, Hq, Hkv, 2) > ws_bytes) return hipErrorInvalidValue;
    int64_t items = 0;
    for (int b = 0; b < B; ++b) items += (offsets_host[b + 1] - offsets_host[b] + kDecCH - 1) / kDecCH;
    WsCarver w(ws);
    int64_t* lens = w.take<int64_t>((size_t)B + 1);
    float* part = w.take<float>((size_t)items * Hq * kD);
    float2* ml = w.take<float2>((size_t)items * Hq);
    const I64Arg offs = i64_arg(offsets_dev, offsets_host, (int64_t)B + 1);
    // one sequence: its length is a launch argument; otherwise the lengths are computed on
    // the device
    const int64_t hl = offsets_host[B] - offsets_host[0];
    const I64Arg lns = i64_arg(lens, B == 1 ? &hl : nullptr, B);
    if (B != 1) hipLaunchKernelGGL(lengths_kernel, dim3(1), dim3(256), 0, stream, offs, B, lens);
    hipError_t e = launch_partial_G<2>(Hq / Hkv, dim3((unsigned)items), stream, q, K, V, offs, nullptr, lns,
                                       B, Hq, Hkv, part, ml);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_merge_kernel, dim3(B * Hq, kD / 16), dim3(1024), 0, stream, part, ml, lns, B, Hq, out);
    return hipGetLastError();
}

}  // namespace qasi
