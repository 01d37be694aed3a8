// Device helpers of the top-k routing and the per-token activation
// statistics, shared by the router kernels and the decode gate/up kernel
// that routes small batches itself.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "pw_internal.h"
#include "xscale.h"

namespace pw {
namespace rdev {

// ---- 16 lanes per token (E <= 256) ----
// A row of 16 lanes routes one token; lane i of the row holds the logits of
// experts i, i + 16, ... . Reductions across the row use DPP (quad
// permutations, then the half-row and row mirrors), which leaves the row's
// result in every lane of the row without a trip through LDS.
// (every pattern used here reads a valid lane of the same row, so the
// instruction needs no old value: bound_ctrl, and no copy of x to keep)
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
    return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xf, 0xf, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, x)));
}
constexpr int kQuadXor1 = 0xb1;        // quad_perm [1, 0, 3, 2]
constexpr int kQuadXor2 = 0x4e;        // quad_perm [2, 3, 0, 1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

__device__ __forceinline__ float row_sum(float x) {
    x += dpp_f<kQuadXor1>(x);
    x += dpp_f<kQuadXor2>(x);
    x += dpp_f<kRowHalfMirror>(x);
    x += dpp_f<kRowMirror>(x);
    return x;
}

// (logit, expert) as one 64-bit key ordered like better(): the logit's bits
// made order-preserving as an unsigned integer above, the complement of the
// expert id below (equal logits: lower id is larger). 0 is below every key;
// a zero logit decodes as +0.
__device__ __forceinline__ uint64_t route_key(float v, int e) {
    const uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);   // -0 ties with +0, as in better()
    const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)o << 32) | (uint64_t)(0xffffffffu - (uint32_t)e);
}
__device__ __forceinline__ float key_value(uint64_t k) {
    const uint32_t o = (uint32_t)(k >> 32);
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ int key_expert(uint64_t k) { return (int)(0xffffffffu - (uint32_t)k); }

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x) {
    const int lo = dpp_i<CTRL>((int)(uint32_t)x), hi = dpp_i<CTRL>((int)(uint32_t)(x >> 32));
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ __forceinline__ uint64_t row_max_key(uint64_t k) {
    uint64_t o = dpp_u64<kQuadXor1>(k);
    k = o > k ? o : k;
    o = dpp_u64<kQuadXor2>(k);
    k = o > k ? o : k;
    o = dpp_u64<kRowHalfMirror>(k);
    k = o > k ? o : k;
    o = dpp_u64<kRowMirror>(k);
    return o > k ? o : k;
}

// Wave-wide reductions: the row result (DPP, as above), then row 1 takes
// row 0's (row_bcast:15) and row 3 row 2's, then rows 2 and 3 take row 1's
// (row_bcast:31): lane 63 holds the wave's result, read into a scalar.
constexpr int kRowBcast15 = 0x142;
constexpr int kRowBcast31 = 0x143;
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_rows_i(int x) {
    return __builtin_amdgcn_update_dpp(x, x, CTRL, ROWS, 0xf, false);
}
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
    k = row_max_key(k);
    uint64_t o = ((uint64_t)(uint32_t)dpp_rows_i<kRowBcast15, 0xa>((int)(uint32_t)(k >> 32)) << 32) |
                 (uint32_t)dpp_rows_i<kRowBcast15, 0xa>((int)(uint32_t)k);
    k = o > k ? o : k;
    o = ((uint64_t)(uint32_t)dpp_rows_i<kRowBcast31, 0xc>((int)(uint32_t)(k >> 32)) << 32) |
        (uint32_t)dpp_rows_i<kRowBcast31, 0xc>((int)(uint32_t)k);
    k = o > k ? o : k;
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)k, 63);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(k >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ float wave_sum(float x) {
    x = row_sum(x);
    x += __builtin_bit_cast(float, dpp_rows_i<kRowBcast15, 0xa>(__builtin_bit_cast(int, x)));
    x += __builtin_bit_cast(float, dpp_rows_i<kRowBcast31, 0xc>(__builtin_bit_cast(int, x)));
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// Statistics of an activation row (xscale.h) by a group of L lanes (16: a
// row of lanes, reduced with DPP; 64: a wave, the rows then combined with
// shuffles): lane i takes the 16-byte chunks i, i + L, ...; max |x| as bf16
// magnitude bits and sum |x| in fp64 (no overflow or underflow for any row
// of bf16 values). Every reduction step adds two partial results in either
// order, so all lanes of the group end with the same bits.
template <int CTRL>
__device__ __forceinline__ double dpp_d(double x) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const int lo = dpp_i<CTRL>((int)(uint32_t)u), hi = dpp_i<CTRL>((int)(uint32_t)(u >> 32));
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}
template <int L>
__device__ __forceinline__ XStat lanes_stat(const uint16_t* row, int d) {
    const int li = threadIdx.x & (L - 1);
    const uint4* r = reinterpret_cast<const uint4*>(row);
    uint32_t mx = 0;
    // eight independent partial sums (one per activation of a chunk): a
    // single running sum made the fp64 adds one dependent chain per lane,
    // most of the router's time at d_model 4096
    double part[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
#pragma unroll 8
    for (int c = li; c < d / 8; c += L) {
        const uint4 u = r[c];
        const uint32_t ww[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const uint32_t lo = ww[h] & 0x7fffu, hi = (ww[h] >> 16) & 0x7fffu;
            mx = max(mx, max(lo, hi));
            part[2 * h] += (double)__uint_as_float(lo << 16);
            part[2 * h + 1] += (double)__uint_as_float(hi << 16);
        }
    }
    double sum = ((part[0] + part[1]) + (part[2] + part[3])) + ((part[4] + part[5]) + (part[6] + part[7]));
    mx = max(mx, (uint32_t)dpp_i<kQuadXor1>((int)mx));
    sum += dpp_d<kQuadXor1>(sum);
    mx = max(mx, (uint32_t)dpp_i<kQuadXor2>((int)mx));
    sum += dpp_d<kQuadXor2>(sum);
    mx = max(mx, (uint32_t)dpp_i<kRowHalfMirror>((int)mx));
    sum += dpp_d<kRowHalfMirror>(sum);
    mx = max(mx, (uint32_t)dpp_i<kRowMirror>((int)mx));
    sum += dpp_d<kRowMirror>(sum);
    if constexpr (L == 64) {
        for (int o = 16; o < 64; o <<= 1) {
            mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
            sum += __shfl_xor(sum, o);
        }
    }
    const int e = xsc::x_exponent(__uint_as_float(mx << 16));
    return XStat{(float)ldexp(sum, -e), e};
}

// Top-k of one token by its row of 16 lanes (lane l16 holds the logits
// v[i] of experts l16 + 16 i; `valid` false for a row past the batch): k
// rounds of the row's largest key, each removed from its lane; softmax
// weights from the native base-2 exponential of (v - top) log2(e), over all
// E experts or (renorm) over the k chosen. Lane l16 gets choice l16 (id0,
// g0) if l16 < k and choice l16 + 16 (id1, g1) if l16 + 16 < k.
struct RowChoice {
    int id0, id1;
    float g0, g1;
};
template <int PER>
__device__ __forceinline__ RowChoice row_topk(const float (&v)[PER], int E, int k, int renorm, bool valid) {
    const int l16 = threadIdx.x & 15;
    uint64_t key[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = l16 + 16 * i;
        key[i] = (valid && e < E) ? route_key(v[i], e) : 0ull;
    }
    int id0 = 0, id1 = 0;
    float val0 = -INFINITY, val1 = -INFINITY, top = -INFINITY;
    for (int j = 0; j < k; ++j) {
        uint64_t best = key[0];
#pragma unroll
        for (int i = 1; i < PER; ++i) best = key[i] > best ? key[i] : best;
        best = row_max_key(best);
#pragma unroll
        for (int i = 0; i < PER; ++i) key[i] = key[i] == best ? 0ull : key[i];
        const float bv = key_value(best);
        const int be = key_expert(best);
        if (j == 0) top = bv;
        if (j == l16) { id0 = be; val0 = bv; }
        if (j == l16 + 16) { id1 = be; val1 = bv; }
    }
    constexpr float kLog2e = 1.4426950408889634f;
    float sum_all = 0.0f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = l16 + 16 * i;
        if (e < E) sum_all += __builtin_amdgcn_exp2f((v[i] - top) * kLog2e);
    }
    const float m0 = l16 < k ? __builtin_amdgcn_exp2f((val0 - top) * kLog2e) : 0.0f;
    const float m1 = l16 + 16 < k ? __builtin_amdgcn_exp2f((val1 - top) * kLog2e) : 0.0f;
    const float den = row_sum(renorm ? m0 + m1 : sum_all);
    return RowChoice{id0, id1, m0 / den, m1 / den};
}

}  // namespace rdev
}  // namespace pw
