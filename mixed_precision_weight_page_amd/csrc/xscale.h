// Power-of-two scaling of the matrix-core operands into fp16 range.
//
// The layer takes bf16 activations (range up to 2^128) and its SwiGLU rows h
// can be as large as the fp32 products allow, while the matrix cores read
// fp16 (largest finite 65504, normal down to 2^-14). Exact powers of two
// bridge the gap without rounding anything:
//
//   x~ = x 2^-e_t, e_t chosen per token so that max|x~| lies in [2^14, 2^15)
//        (every value of the row down to max|x| 2^-31 stays exact in fp16);
//   with n1_t = sum |x~| over the row and |q| <= qmax, the gate and up sums
//        satisfy |s sum q x~| <= s qmax n1_t < 2^Ea (fp32 accumulation error
//        and the rounding of n1_t are covered by a factor 1.25);
//   a_s = s acc_a 2^-Ea (|a_s| < 1) and c_s = s acc_c 2^(15-Ea) (|c_s| < 2^15)
//        give h~ = a_s sigmoid(a) c_s with |h~| < 2^15, the stored fp16 row,
//        and h = h~ 2^m with m = 2 (Ea + e_t) - 15;
//   the down product's sums are multiplied back by 2^m in fp32.
//
// Every factor is a power of two, so the MFMA products stay exact and only
// the fp32 accumulation rounds, as without scaling. The gate/up and down
// kernels derive Ea and m from the same per-token statistics and the same
// expert scale, so they agree bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "pw_internal.h"

namespace pw {
namespace xsc {

// e with M 2^-e in [2^14, 2^15) for M > 0 (0 for M = 0)
__device__ __forceinline__ int x_exponent(float M) {
    if (!(M > 0.0f)) return 0;
    int e;
    (void)frexpf(M, &e);   // M = f 2^e, f in [0.5, 1)
    return e - 15;
}

// Ea with s qmax n1 1.25 < 2^Ea (0 when s or n1 is 0: the sums are then 0)
__device__ __forceinline__ int a_exponent(float s, int qmax, float n1) {
    if (!(s > 0.0f) || !(n1 > 0.0f)) return 0;
    int es, en, em;
    const float fs = frexpf(s, &es), fn = frexpf(n1, &en);
    (void)frexpf(fs * fn * (float)qmax * 1.25f, &em);   // in [0.15, 159): no overflow
    return es + en + em;
}

// Per-token factors of the gate/up epilogue for an expert whose weights are
// s times integer codes of magnitude at most qmax: a_s = acc_a fa,
// c_s = acc_c fc, a = a_s 2^ea.
struct GateUpScale {
    float fa, fc;
    int ea;
};
__device__ __forceinline__ GateUpScale gate_up_scale(float s, int qmax, XStat xt) {
    const int Ea = a_exponent(s, qmax, xt.n1);
    return GateUpScale{ldexpf(s, -Ea), ldexpf(s, 15 - Ea), Ea + xt.e};
}

// Exponent m of the stored h~ rows (h = h~ 2^m) of a token and expert.
__device__ __forceinline__ int h_exponent(float s, int qmax, XStat xt) {
    return 2 * (a_exponent(s, qmax, xt.n1) + xt.e) - 15;
}

// h~ from the two fp32 sums; sigmoid(a) with a = a_s 2^ea (which may
// overflow to +-inf: the sigmoid is then exactly 1 or 0)
__device__ __forceinline__ float swiglu_scaled(float acc_a, float acc_c, const GateUpScale& g) {
    const float as = acc_a * g.fa;
    const float a = ldexpf(as, g.ea);
    return as / (1.0f + expf(-a)) * (acc_c * g.fc);
}

// The same with the native base-2 exponential and reciprocal (the
// large-batch kernels' epilogue).
__device__ __forceinline__ float swiglu_scaled_fast(float acc_a, float acc_c, const GateUpScale& g) {
    constexpr float kLog2e = 1.4426950408889634f;
    const float as = acc_a * g.fa;
    const float a = ldexpf(as, g.ea);
    return as * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-a * kLog2e)) * (acc_c * g.fc);
}

// One wave: max |x| (as bf16 magnitude bits, in every lane) and sum |x|
// (fp64, which neither overflows nor underflows for a row of bf16 values;
// lane 0 holds the wave's sum) over a row of d bf16 values (d a multiple of
// 8, the row 16-byte aligned), in one pass of 16-byte loads.
__device__ __forceinline__ XStat row_stat(const uint16_t* row, int d) {
    const int lane = threadIdx.x & 63;
    const uint4* r = reinterpret_cast<const uint4*>(row);
    uint32_t mx = 0;
    double sum = 0.0;
    for (int c = lane; c < d / 8; c += 64) {
        const uint4 u = r[c];
        const uint32_t ww[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const uint32_t lo = ww[h] & 0x7fffu, hi = (ww[h] >> 16) & 0x7fffu;
            mx = max(mx, max(lo, hi));
            sum += (double)__uint_as_float(lo << 16) + (double)__uint_as_float(hi << 16);
        }
    }
    for (int o = 32; o > 0; o >>= 1) {
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
        sum += __shfl_xor(sum, o);
    }
    const int e = x_exponent(__uint_as_float(mx << 16));
    return XStat{(float)ldexp(sum, -e), e};
}

// bf16 bits -> x 2^-e as fp32 (exact unless below 2^-149)
__device__ __forceinline__ float bf16_scaled(uint16_t v, int e) {
    return ldexpf(__uint_as_float((uint32_t)v << 16), -e);
}

}  // namespace xsc
}  // namespace pw
