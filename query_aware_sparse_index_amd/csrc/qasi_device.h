// Device-side helpers shared by the gfx950 kernels of the qasi library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qasi {

constexpr int kD = 128;   // head dimension
constexpr int kDP = 32;   // index dimension d' = d / 4

// Row stride of the [Hq][S] score array: the packed token count rounded up to 64 floats, so
// that every row starts on a 256-byte boundary.
__host__ __device__ __forceinline__ int64_t score_stride(int64_t ntot) { return ((ntot + 63) / 64) * 64; }

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp64 -> bf16 with one rounding, nearest-even.  Normal range: drop 45 mantissa bits of the
// double with round-half-even integer arithmetic (a carry into the exponent is the correct
// result).  Below 2^-126: count quanta of the subnormal grid 2^-133 and round that count
// with rint (nearest-even in the default mode); 128 quanta is the smallest normal 0x0080.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
    uint64_t u = (uint64_t)__double_as_longlong(x);
    uint32_t sign = (uint32_t)(u >> 63) << 15;
    uint64_t a = u & 0x7fffffffffffffffull;
    if (a == 0) return (uint16_t)sign;
    uint32_t bexp = (uint32_t)(a >> 52);
    if (bexp >= 1023 - 126) {
        a += 0x00000fffffffffffull + ((a >> 45) & 1ull);
        uint32_t e = (uint32_t)(a >> 52);
        if (e > 1023 + 127) return (uint16_t)(sign | 0x7f80u);
        uint32_t mant = (uint32_t)((a >> 45) & 0x7full);
        return (uint16_t)(sign | ((e - 1023 + 127) << 7) | mant);
    }
    double q = rint(__longlong_as_double((long long)a) * 0x1p133);
    return (uint16_t)(sign | (uint32_t)q);
}

// 16-byte load of streamed data.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Calls f(t, value, ok) for every t in [lo, hi) of a fp32 row, with 16-byte loads for the aligned
// body (U loads in flight per thread) and scalar loads for the unaligned head and tail.  All
// NT threads of the block take part.
template <int NT, int U, class F>
__device__ __forceinline__ void for_each_f32(const float* __restrict__ row, int64_t lo, int64_t hi, F f) {
    if (lo >= hi) return;
    const uintptr_t a = reinterpret_cast<uintptr_t>(row + lo);
    int64_t head = (int64_t)(((16u - (a & 15u)) & 15u) / 4u);
    if (head > hi - lo) head = hi - lo;
    if (threadIdx.x < head) f(lo + threadIdx.x, row[lo + threadIdx.x], true);
    const int64_t b0 = lo + head;
    const int64_t nv = (hi - b0) / 4;
    const float4* body = reinterpret_cast<const float4*>(row + b0);
    for (int64_t v0 = threadIdx.x; v0 - threadIdx.x < nv; v0 += (int64_t)U * NT) {
        float4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t v = v0 + (int64_t)u * NT;
            x[u] = v < nv ? body[v] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t v = v0 + (int64_t)u * NT;
            const bool ok = v < nv;
            const int64_t t = b0 + 4 * v;
            f(t, x[u].x, ok);
            f(t + 1, x[u].y, ok);
            f(t + 2, x[u].z, ok);
            f(t + 3, x[u].w, ok);
        }
    }
    const int64_t tail0 = b0 + 4 * nv;
    if (threadIdx.x < hi - tail0) f(tail0 + threadIdx.x, row[tail0 + threadIdx.x], true);
}

// 2^x with one v_exp_f32 (about 1 ulp; results below 2^-126 flush to zero, exp2(-inf) = 0).
// The library's exp2f adds a denormal rescaling around the same instruction.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Order-preserving map fp32 -> uint32 (ascending keys <=> ascending values); -0 maps to
// the key of +0 so the two tie.
__device__ __forceinline__ uint32_t order_key(float s) {
    uint32_t b = __float_as_uint(s);
    if (b == 0x80000000u) b = 0u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
    uint32_t b = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(b);
}

// Butterfly sums across lanes with DPP (no LDS traffic).  xor1 / xor2 stay inside a quad;
// half-mirror and mirror pair 4-lane and 8-lane groups inside a 16-lane row.
__device__ __forceinline__ float dpp_quad_xor1(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xb1, 0xf, 0xf, true));  // [1,0,3,2]
}
__device__ __forceinline__ float dpp_quad_xor2(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4e, 0xf, 0xf, true));  // [2,3,0,1]
}
__device__ __forceinline__ float dpp_row_half_mirror(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xf, 0xf, true));
}
__device__ __forceinline__ float dpp_row_mirror(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xf, 0xf, true));
}
// Sum over each group of 4 lanes (result in every lane of the quad).
__device__ __forceinline__ float sum_quad(float v) {
    v += dpp_quad_xor1(v);
    v += dpp_quad_xor2(v);
    return v;
}
// Sum over each 16-lane row (result in every lane of the row).
__device__ __forceinline__ float sum_row16(float v) {
    v += dpp_quad_xor1(v);
    v += dpp_quad_xor2(v);
    v += dpp_row_half_mirror(v);
    v += dpp_row_mirror(v);
    return v;
}

// Maximum over each 16-lane row (result in every lane of the row).
__device__ __forceinline__ float max_row16(float v) {
    v = fmaxf(v, dpp_quad_xor1(v));
    v = fmaxf(v, dpp_quad_xor2(v));
    v = fmaxf(v, dpp_row_half_mirror(v));
    v = fmaxf(v, dpp_row_mirror(v));
    return v;
}

// Wave-wide reductions (64 lanes) through shuffles.
__device__ __forceinline__ float wave_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Inclusive prefix sum over the 64 lanes of a wave in registers (DPP, no LDS crossbar): shifts
// by 1, 2, 4 and 8 lanes within each row of 16 (lanes shifted in from outside the row add 0),
// then lane 15 of rows 0 and 2 is added to rows 1 and 3, and lane 31 to rows 2 and 3.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
    return x;
}

// Inclusive prefix sum of one int per thread over a block of NT threads (NT multiple of 64,
// at most 1024).  `tmp` holds NT/64 ints.  Returns the inclusive value; *total the sum.
template <int NT>
__device__ __forceinline__ int block_inclusive_scan(int v, int* tmp, int* total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int x = wave_inclusive_scan(v);
    if (lane == 63) tmp[wid] = x;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        int t = tmp[w];
        if (w < wid) base += t;
        tot += t;
    }
    __syncthreads();
    *total = tot;
    return x + base;
}

// Block-wide: the totals of a and b and the inclusive scan of c (returned, total in *tc), with
// one exchange through LDS.  tmp holds 3 x NT / 64 ints.  Every thread must call it.
template <int NT>
__device__ __forceinline__ int block_inclusive_scan3(int a, int b, int c, int (*tmp)[NT / 64], int* ta, int* tb,
                                                     int* tc) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int x = wave_inclusive_scan(c);
    a = wave_inclusive_scan(a);   // lane 63: the wave's total
    b = wave_inclusive_scan(b);
    if (lane == 63) {
        tmp[0][wid] = a;
        tmp[1][wid] = b;
        tmp[2][wid] = x;
    }
    __syncthreads();
    int sa = 0, sb = 0, base = 0, sc = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        sa += tmp[0][w];
        sb += tmp[1][w];
        const int v = tmp[2][w];
        if (w < wid) base += v;
        sc += v;
    }
    __syncthreads();
    *ta = sa;
    *tb = sb;
    *tc = sc;
    return x + base;
}

// ---- sequence lookups for work items numbered sequence by sequence (ragged batches)
// Every lane of a wave must call these together (converged control flow); each returns the same
// values in every lane.  One sequence: scalar.  More: lane i % 64 loads sequence i's value (one
// round trip for up to 64 sequences), then a wave-uniform loop reads the values back with
// readlane (no memory or LDS round trip per sequence).
__device__ __forceinline__ int64_t readlane_i64(int64_t v, int l) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), l);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}
// The sequence b holding work item `item` when sequence i owns units(i) >= 0 items: first =
// items of the sequences before b, cnt = units(b); b = -1 when item is past the last one.
// units0 is units(0) for a batch of one sequence (its values are launch arguments); for more,
// units(i) is evaluated per lane and must read device memory only (a lane-varying index into
// launch-argument values would go through scratch memory).
struct SeqPos {
    int64_t first, cnt;
    int b;
};
template <class Units>
__device__ __forceinline__ SeqPos wave_find_seq(int B, int64_t item, int64_t units0, Units units) {
    SeqPos r{0, 0, -1};
    if (B == 1) {
        r.cnt = units0;
        if (item < r.cnt) r.b = 0;
        return r;
    }
    const int lane = threadIdx.x & 63;
    int64_t acc = 0;
    for (int base = 0; base < B && r.b < 0; base += 64) {
        const int i = base + lane;
        const int64_t u = i < B ? units(i) : 0;
        const int lim = B - base < 64 ? B - base : 64;
        for (int l = 0; l < lim; ++l) {
            const int64_t ul = readlane_i64(u, l);
            if (item < acc + ul) {
                r.b = base + l;
                r.first = acc;
                r.cnt = ul;
                break;
            }
            acc += ul;
        }
    }
    // the values are wave-uniform: say so, so that the caller indexes with scalars
    r.b = __builtin_amdgcn_readfirstlane(r.b);
    r.first = readlane_i64(r.first, 0);
    r.cnt = readlane_i64(r.cnt, 0);
    return r;
}
// sum of w(i) over the sequences i < b (b > 0 only in batches of several sequences, so w reads
// device memory)
template <class W>
__device__ __forceinline__ int64_t wave_prefix_seq(int b, W w) {
    const int lane = threadIdx.x & 63;
    int64_t acc = 0;
    for (int base = 0; base < b; base += 64) {
        const int i = base + lane;
        const int64_t v = i < b ? w(i) : 0;
        const int lim = b - base < 64 ? b - base : 64;
        for (int l = 0; l < lim; ++l) acc += readlane_i64(v, l);
    }
    return acc;
}

}  // namespace qasi
