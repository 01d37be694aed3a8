// Packed codes -> exact fp16 integers in registers, shared by the streaming
// (decode) and matrix-core (prefill) expert kernels (PagedWeight page,
// section "Dynamic Paging": pages are dequantized on the fly; Eq. 2:
// W = s_e q, with the scale s_e applied once to the fp32 sums).
//
// A run is 32 consecutive codes of one weight row, LSB-first in B dwords
// (code c at bits B c .. B c + B - 1). Each MFMA operand fragment is 8 fp16
// values; a run gives 4 fragments. The K order in which a run's codes land
// in the fragments (perm_slot) is chosen so that unpacking is cheap; the
// activations are staged in the same order.
//
// Unpacking: a code u placed in the mantissa of fp16 1024 (exponent pattern
// 0x6400) at bit S <= 7 of a 16-bit half is the exact value 1024 + 2^S u.
// One fused multiply-add by 2^-S minus 2^(10-S) + 2^(B-1) then gives the
// signed code q = u - 2^(B-1) exactly (a plain subtract for S = 0). Each pair
// of codes costs one v_and_or_b32 and one packed fp16 operation, plus a
// shift for the codes above bit 7 of their half. Exact q keeps the MFMA sums
// free of the offset 2^(B-1) sum(x), which would otherwise dominate them
// when most codes are 0 (weights far below an expert's largest weight).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pw {
namespace dq {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr uint32_t kMagic = 0x64006400u;   // fp16 1024 in both halves

__device__ __forceinline__ half2_t as_half2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

// A 32-bit constant held in a VGPR. A VOP3 instruction on this target can
// read at most one SGPR or literal: with the exponent pattern in a VGPR,
// (w & mask) | magic is one v_and_or_b32 with the mask as the SGPR operand.
__device__ __forceinline__ uint32_t vgpr_const(uint32_t c) {
    uint32_t r;
    asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
    return r;
}

struct Const {
    uint32_t magic;   // 0x64006400
    uint32_t e8;      // 0x64646464: exponent byte for v_perm_b32
};

__device__ __forceinline__ Const make_const() { return Const{vgpr_const(kMagic), vgpr_const(0x64646464u)}; }

// The two B-bit codes at bit S of each 16-bit half of x, as exact signed
// fp16 values (low half, high half).
template <int B, int S>
__device__ __forceinline__ half2_t code_pair(uint32_t x, const Const& c) {
    static_assert(S >= 0 && S + B <= 10, "the code must stay inside the fp16 mantissa");
    constexpr uint32_t mask = ((1u << B) - 1u) * 0x00010001u << S;
    const half2_t v = as_half2((x & mask) | c.magic);
    if constexpr (S == 0) {
        constexpr _Float16 bias = (_Float16)(1024 + (1 << (B - 1)));
        return v - half2_t{bias, bias};
    } else {
        constexpr _Float16 m = (_Float16)(1.0f / (1 << S));
        constexpr _Float16 bias = (_Float16)(-(float)((1024 >> S) + (1 << (B - 1))));
        return __builtin_elementwise_fma(v, half2_t{m, m}, half2_t{bias, bias});
    }
}

__device__ __forceinline__ half8_t cat(half2_t a, half2_t b, half2_t c, half2_t d) {
    return __builtin_shufflevector(__builtin_shufflevector(a, b, 0, 1, 2, 3),
                                   __builtin_shufflevector(c, d, 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
}

// The 16 signed pairs of a 3-bit run in three dwords; pair p = (K-slot 2p,
// K-slot 2p + 1). Half-words of two dwords are merged so that codes j and
// j + 16 sit at the same offset of the two halves; every code is then taken
// at bit 0, 3 or 6 of its half (two multiply-add constants in registers).
__device__ __forceinline__ void pairs3(const uint32_t* w, half2_t p[16], const Const& c) {
    const uint32_t v01 = (w[0] & 0xffffu) | (w[1] & 0xffff0000u);   // codes 0-4 | 16-20 at 3j
    const uint32_t v02 = (w[2] & 0xffffu) | (w[0] & 0xffff0000u);   // codes 22-25 | 6-9 at 3j-16
    const uint32_t v12 = (w[1] & 0xffffu) | (w[2] & 0xffff0000u);   // codes 11-15 | 27-31 at 3j-32
    const uint32_t t01 = v01 >> 9, t02 = v02 >> 2, u02 = v02 >> 11, t12 = v12 >> 1, u12 = v12 >> 10;
    p[0] = code_pair<3, 0>(v01, c);    // (0, 16)
    p[1] = code_pair<3, 3>(v01, c);    // (1, 17)
    p[2] = code_pair<3, 6>(v01, c);    // (2, 18)
    p[3] = code_pair<3, 0>(t01, c);    // (3, 19)
    p[4] = code_pair<3, 3>(t01, c);    // (4, 20)
    // code 5 (bits 15-17) and code 21 (bits 63-65) straddle dword boundaries
    p[5] = code_pair<3, 0>((w[0] >> 15 & 0xffffu) | (__builtin_amdgcn_alignbit(w[2], w[1], 15) & 0xffff0000u), c);
    p[6] = code_pair<3, 0>(t02, c);    // (22, 6)
    p[7] = code_pair<3, 3>(t02, c);    // (23, 7)
    p[8] = code_pair<3, 6>(t02, c);    // (24, 8)
    p[9] = code_pair<3, 0>(u02, c);    // (25, 9)
    // code 10 (bits 30-32) and code 26 (bits 78-80)
    p[10] = code_pair<3, 0>((__builtin_amdgcn_alignbit(w[1], w[0], 30) & 0xffffu) |
                                (__builtin_amdgcn_alignbit(w[2], w[1], 30) & 0xffff0000u), c);
    p[11] = code_pair<3, 0>(t12, c);   // (11, 27)
    p[12] = code_pair<3, 3>(t12, c);   // (12, 28)
    p[13] = code_pair<3, 6>(t12, c);   // (13, 29)
    p[14] = code_pair<3, 0>(u12, c);   // (14, 30)
    p[15] = code_pair<3, 3>(u12, c);   // (15, 31)
}

// Fragment i (K-slots 8i .. 8i + 7) of a 4- or 8-bit run. 4-bit: nibbles
// (0, 4), (1, 5), (2, 6), (3, 7) of dword i. 8-bit: bytes (0, 2) and (1, 3) of
// dwords 2i and 2i + 1, moved next to the exponent byte by v_perm_b32
// (selector bytes 0-3 pick from the dword, 4 from the exponent pattern).
template <int B>
__device__ __forceinline__ half8_t frag48(const uint32_t* w, int i, const Const& c) {
    static_assert(B == 4 || B == 8, "3-bit runs go through pairs3");
    if constexpr (B == 4) {
        const uint32_t x = w[i], t = x >> 8;
        return cat(code_pair<4, 0>(x, c), code_pair<4, 4>(x, c), code_pair<4, 0>(t, c), code_pair<4, 4>(t, c));
    } else {
        const uint32_t w0 = w[2 * i], w1 = w[2 * i + 1];
        const half2_t bias = {(_Float16)1152.0f, (_Float16)1152.0f};
        return cat(as_half2(__builtin_amdgcn_perm(c.e8, w0, 0x04020400u)) - bias,
                   as_half2(__builtin_amdgcn_perm(c.e8, w0, 0x04030401u)) - bias,
                   as_half2(__builtin_amdgcn_perm(c.e8, w1, 0x04020400u)) - bias,
                   as_half2(__builtin_amdgcn_perm(c.e8, w1, 0x04030401u)) - bias);
    }
}

// Code (within a run) whose activation goes to K-slot s: the order the
// fragments above produce.
template <int B>
__host__ __device__ __forceinline__ constexpr int perm_slot(int s) {
    if constexpr (B == 4) {
        constexpr int p[8] = {0, 4, 1, 5, 2, 6, 3, 7};
        return (s & ~7) + p[s & 7];
    } else if constexpr (B == 8) {
        constexpr int p[8] = {0, 2, 1, 3, 4, 6, 5, 7};
        return (s & ~7) + p[s & 7];
    } else {
        constexpr int p[32] = {0, 16, 1, 17, 2, 18, 3, 19, 4, 20, 5, 21, 22, 6, 23, 7,
                               24, 8, 25, 9, 10, 26, 11, 27, 12, 28, 13, 29, 14, 30, 15, 31};
        return p[s];
    }
}

}  // namespace dq
}  // namespace pw
