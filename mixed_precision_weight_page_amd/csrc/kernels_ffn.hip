// Expert FFN kernels for routed tokens (PagedWeight page, section "Dynamic
// Paging": the routed experts' pages are dequantized on the fly; Eq. 2 gives
// the dequantized weight s_e * q). SwiGLU: h = silu(W1 x) * (W3 x), o = W2 h.
//
// One workgroup = one 16*WR-row tile of one active expert, all of the
// expert's tokens. Four waves: WR along rows, WK along K (partial sums are
// added in LDS in a fixed order). Codes stream from the page with one
// 4B-byte load per lane per 128-code step (B = bits), prefetched PD steps
// ahead; they are turned into exact fp16 integers q in registers
// (magic-exponent OR, then one packed fp16 subtract) and multiplied on the
// matrix cores (v_mfma_f32_16x16x32_f16: 16 weight rows x 16 token columns,
// K = 32), accumulating in fp32. Token rows are staged once per K chunk in
// LDS as fp16, permuted so that each lane's 8 K-slots line up with the
// order in which its codes unpack. The per-expert scale is applied in the
// epilogue, so every product is exact and only fp32 accumulation rounds.
//
// Why matrix cores for a memory-bound skinny product: with T_e tokens per
// expert a VALU dot product costs T_e/2 instructions per weight (packed
// dot2), which exceeds the VALU issue budget at HBM speed (about 2.5
// lane-instructions per 4-bit weight at 8 TB/s) as soon as T_e > 2. The
// MFMA does the multiply-adds for up to 16 tokens at once and leaves the
// VALU only the unpack (about 1.4 instructions per 4-bit weight).
#include <hip/hip_runtime.h>

#include <math.h>

#include "pw_internal.h"

namespace pw {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kStep = 128;   // codes per wave per step (4 K-groups x 32)
constexpr int kPD = 4;       // steps of codes in flight per wave
constexpr uint32_t kMagic = 0x64006400u;   // two fp16 1024.0

template <int B>
struct Codes {
    uint32_t w[B];   // 32 consecutive codes of one row, LSB-first
};

template <int B>
__device__ __forceinline__ Codes<B> load_codes(const uint8_t* p) {
    Codes<B> c;
    if constexpr (B == 4) {
        const uint4 u = *reinterpret_cast<const uint4*>(p);
        c.w[0] = u.x; c.w[1] = u.y; c.w[2] = u.z; c.w[3] = u.w;
    } else if constexpr (B == 8) {
        const uint4 u = *reinterpret_cast<const uint4*>(p);
        const uint4 v = *reinterpret_cast<const uint4*>(p + 16);
        c.w[0] = u.x; c.w[1] = u.y; c.w[2] = u.z; c.w[3] = u.w;
        c.w[4] = v.x; c.w[5] = v.y; c.w[6] = v.z; c.w[7] = v.w;
    } else {
        const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
        c.w[0] = q[0]; c.w[1] = q[1]; c.w[2] = q[2];
    }
    return c;
}

__device__ __forceinline__ half8_t to_frag(uint32_t a, uint32_t b, uint32_t c, uint32_t d,
                                           _Float16 bias) {
    union {
        uint32_t u[4];
        half8_t h;
    } x;
    x.u[0] = a; x.u[1] = b; x.u[2] = c; x.u[3] = d;
    return x.h - bias;   // 1024 + u - (1024 + 2^(B-1)) = q, exact in fp16
}

// The 16 fp16 pairs (each "1024 + code") of a 3-bit group of 32 codes held
// in three dwords; pair p = (slot 2p, slot 2p+1) of the staging permutation.
__device__ __forceinline__ void pairs3(const uint32_t* w, uint32_t p[16]) {
    const uint32_t M3 = 0x00070007u;
    const uint32_t v01 = (w[0] & 0xffffu) | (w[1] & 0xffff0000u);
    const uint32_t v12 = (w[1] & 0xffffu) | (w[2] & 0xffff0000u);
    const uint32_t v02 = (w[2] & 0xffffu) | (w[0] & 0xffff0000u);
#pragma unroll
    for (int j = 0; j < 5; ++j) p[j] = ((v01 >> (3 * j)) & M3) | kMagic;          // (j, j+16)
    p[5] = ((w[0] >> 15) & 7u) | (__builtin_amdgcn_alignbit(w[2], w[1], 15) & 0x70000u) |
           kMagic;                                                                 // (5, 21)
#pragma unroll
    for (int j = 6; j < 10; ++j) p[j] = ((v02 >> (3 * j - 16)) & M3) | kMagic;    // (j+16, j)
    p[10] = (__builtin_amdgcn_alignbit(w[1], w[0], 30) & 7u) | ((w[2] << 2) & 0x70000u) |
            kMagic;                                                                // (10, 26)
#pragma unroll
    for (int j = 11; j < 16; ++j) p[j] = ((v12 >> (3 * j - 32)) & M3) | kMagic;   // (j, j+16)
}

// A fragments (8 fp16 K-slots per lane) for the 4 MFMAs of one step.
template <int B>
__device__ __forceinline__ void unpack(const Codes<B>& c, half8_t f[4]) {
    if constexpr (B == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w = c.w[i];
            f[i] = to_frag((w & 0x000f000fu) | kMagic, ((w >> 4) & 0x000f000fu) | kMagic,
                           ((w >> 8) & 0x000f000fu) | kMagic, ((w >> 12) & 0x000f000fu) | kMagic,
                           (_Float16)1032.0f);
        }
    } else if constexpr (B == 8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w0 = c.w[2 * i], w1 = c.w[2 * i + 1];
            f[i] = to_frag((w0 & 0x00ff00ffu) | kMagic, ((w0 >> 8) & 0x00ff00ffu) | kMagic,
                           (w1 & 0x00ff00ffu) | kMagic, ((w1 >> 8) & 0x00ff00ffu) | kMagic,
                           (_Float16)1152.0f);
        }
    } else {
        uint32_t p[16];
        pairs3(c.w, p);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            f[i] = to_frag(p[4 * i], p[4 * i + 1], p[4 * i + 2], p[4 * i + 3], (_Float16)1028.0f);
    }
}

// Code (within a 32-code group) whose activation goes to LDS slot s.
template <int B>
__device__ __forceinline__ constexpr int perm_slot(int s) {
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

__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// Stage K-chunk [k0, k0 + kc) of nt token rows into LDS as permuted fp16.
// MODE 0 reads bf16 activations of the tokens in tok[]; MODE 1 reads the
// fp16 SwiGLU rows base.. of H.
template <int MODE, int B>
__device__ __forceinline__ void stage(_Float16* xs, int stride, const FfnArgs& a,
                                      const int* tok, int hrow0, int nt, int k0, int kc) {
    const int ngrp = kc / 32;
    for (int idx = threadIdx.x; idx < nt * ngrp; idx += kThreads) {
        const int n = idx / ngrp, grp = idx - n * ngrp;
        _Float16 v[32];
        if constexpr (MODE == 0) {
            const uint4* src = reinterpret_cast<const uint4*>(a.x + (int64_t)tok[n] * a.d + k0 + 32 * grp);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint4 u = src[q];
                const uint32_t ww[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    v[8 * q + 2 * h] = (_Float16)bf16_to_f32((uint16_t)(ww[h] & 0xffffu));
                    v[8 * q + 2 * h + 1] = (_Float16)bf16_to_f32((uint16_t)(ww[h] >> 16));
                }
            }
        } else {
            const uint4* src = reinterpret_cast<const uint4*>(a.w.H + (int64_t)(hrow0 + n) * a.F + k0 + 32 * grp);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                union {
                    uint4 u;
                    _Float16 h[8];
                } t;
                t.u = src[q];
#pragma unroll
                for (int h = 0; h < 8; ++h) v[8 * q + h] = t.h[h];
            }
        }
        union {
            uint4 u[4];
            _Float16 h[32];
        } o;
#pragma unroll
        for (int s = 0; s < 32; ++s) o.h[s] = v[perm_slot<B>(s)];
        uint4* dst = reinterpret_cast<uint4*>(xs + n * stride + 32 * grp);
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[q] = o.u[q];
    }
}

// MODE 0: gate/up + SwiGLU (NMAT = 2: W1, W3); MODE 1: down (NMAT = 1: W2).
template <int MODE, int B, int WR, int WK>
__device__ __forceinline__ void ffn_tile(const FfnArgs& a, const FfnPlan& pl, int e, int rt,
                                         _Float16* xs, int* tok) {
    constexpr int NMAT = MODE == 0 ? 2 : 1;
    const int K = MODE == 0 ? a.d : a.F;
    const int rows_total = MODE == 0 ? a.F : a.d;
    const int64_t mat_bytes = (int64_t)a.F * a.d * B / 8;
    const int64_t row_bytes = (int64_t)K * B / 8;
    const uint8_t* page = a.pool + a.tab.off[e];
    const float s = a.tab.scale[e];
    const int Te = a.w.cnt[e];
    const int base = a.w.off[e];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wr = wave % WR, wk = wave / WR;
    const int r = lane & 15, g = lane >> 4;
    const int row0 = rt * 16 * WR + 16 * wr;
    const uint8_t* ap[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
        ap[m] = page + (MODE == 0 ? m : 2) * mat_bytes + (int64_t)(row0 + r) * row_bytes + 4 * B * g;
    const int stride = pl.kc + 8;
    const int kcp = pl.kc / WK;
    const int nsteps = kcp / kStep;
    const int nchunks = K / pl.kc;

    for (int tb = 0; tb < Te; tb += 16) {
        const int nt = min(16, Te - tb);
        if constexpr (MODE == 0) {
            __syncthreads();
            if (threadIdx.x < nt) tok[threadIdx.x] = a.w.sorted[base + tb + threadIdx.x] / a.k;
        }
        f32x4 acc[NMAT];
#pragma unroll
        for (int m = 0; m < NMAT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        const _Float16* bp = xs + min(r, nt - 1) * stride + 32 * g + wk * kcp;
        for (int c = 0; c < nchunks; ++c) {
            __syncthreads();
            stage<MODE, B>(xs, stride, a, tok, base + tb, nt, c * pl.kc, pl.kc);
            __syncthreads();
            const int64_t kb = (int64_t)(c * pl.kc + wk * kcp) * B / 8;   // byte offset of the part
            Codes<B> buf[NMAT][kPD];
#pragma unroll
            for (int j = 0; j < kPD; ++j)
                if (j < nsteps)
#pragma unroll
                    for (int m = 0; m < NMAT; ++m) buf[m][j] = load_codes<B>(ap[m] + kb + j * kStep * B / 8);
            for (int s0 = 0; s0 < nsteps; s0 += kPD) {
#pragma unroll
                for (int j = 0; j < kPD; ++j) {
                    const int st = s0 + j;
                    if (st < nsteps) {
                        half8_t f[NMAT][4];
#pragma unroll
                        for (int m = 0; m < NMAT; ++m) unpack<B>(buf[m][j], f[m]);
                        if (st + kPD < nsteps)
#pragma unroll
                            for (int m = 0; m < NMAT; ++m)
                                buf[m][j] = load_codes<B>(ap[m] + kb + (int64_t)(st + kPD) * kStep * B / 8);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const half8_t bfr = *reinterpret_cast<const half8_t*>(bp + st * kStep + 8 * i);
#pragma unroll
                            for (int m = 0; m < NMAT; ++m)
                                acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f[m][i], bfr, acc[m], 0, 0, 0);
                        }
                    }
                }
            }
        }
        if constexpr (WK > 1) {
            // add the K-parts in LDS: parts 1..WK-1 store, part 0 adds in order
            __syncthreads();
            float* red = reinterpret_cast<float*>(xs);
            if (wk > 0)
#pragma unroll
                for (int m = 0; m < NMAT; ++m)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        red[((((wk - 1) * WR + wr) * NMAT + m) * 4 + v) * 64 + lane] = acc[m][v];
            __syncthreads();
            if (wk == 0)
                for (int p = 1; p < WK; ++p)
#pragma unroll
                    for (int m = 0; m < NMAT; ++m)
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            acc[m][v] += red[((((p - 1) * WR + wr) * NMAT + m) * 4 + v) * 64 + lane];
        }
        // D layout: lane (n = lane % 16, g = lane / 16) holds rows 4g..4g+3, token n
        if (wk == 0 && r < nt) {
            const int pos = base + tb + r;
            const int orow = row0 + 4 * g;
            if constexpr (MODE == 0) {
                union {
                    uint2 u;
                    _Float16 h[4];
                } hv;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float av = s * acc[0][v];
                    const float cv = s * acc[1][v];
                    hv.h[v] = (_Float16)(av / (1.0f + expf(-av)) * cv);
                }
                *reinterpret_cast<uint2*>(a.w.H + (int64_t)pos * a.F + orow) = hv.u;
            } else {
                float4 o;
                o.x = s * acc[0][0]; o.y = s * acc[0][1]; o.z = s * acc[0][2]; o.w = s * acc[0][3];
                *reinterpret_cast<float4*>(a.w.O + (int64_t)pos * a.d + orow) = o;
            }
        }
    }
    (void)rows_total;
}

template <int MODE, int WR, int WK>
__global__ __launch_bounds__(kThreads) void ffn_kernel(FfnArgs a, FfnPlan pl, int tiles_per_expert) {
    extern __shared__ __attribute__((aligned(16))) _Float16 xs[];
    __shared__ int tok[16];
    const int ai = blockIdx.x / tiles_per_expert;
    if (ai >= a.w.n_act[0]) return;
    const int rt = blockIdx.x - ai * tiles_per_expert;
    const int e = a.w.act[ai];
    const int b = a.tab.bits[e];
    if (b == 4) ffn_tile<MODE, 4, WR, WK>(a, pl, e, rt, xs, tok);
    else if (b == 8) ffn_tile<MODE, 8, WR, WK>(a, pl, e, rt, xs, tok);
    else ffn_tile<MODE, 3, WR, WK>(a, pl, e, rt, xs, tok);
}

template <int MODE>
hipError_t launch_ffn(const FfnArgs& a, const FfnPlan& p, hipStream_t s) {
    const int rows = MODE == 0 ? a.F : a.d;
    const int tpe = rows / (16 * p.wr);
    const dim3 grid((unsigned)(a.max_act * tpe));
    if (p.wr == 4) ffn_kernel<MODE, 4, 1><<<grid, kThreads, p.lds, s>>>(a, p, tpe);
    else if (p.wr == 2) ffn_kernel<MODE, 2, 2><<<grid, kThreads, p.lds, s>>>(a, p, tpe);
    else ffn_kernel<MODE, 1, 4><<<grid, kThreads, p.lds, s>>>(a, p, tpe);
    return hipGetLastError();
}

// y[t] = sum_j g[t,j] * O[pos(t,j)] in slot order; grid (ceil(d/1024), T)
__global__ __launch_bounds__(kThreads) void combine_kernel(FwdWork w, int d, int k, float* y) {
    const int t = blockIdx.y;
    const int col = (blockIdx.x * kThreads + threadIdx.x) * 4;
    if (col >= d) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
        const int p = t * k + j;
        const float gj = w.g[p];
        const float4 o = *reinterpret_cast<const float4*>(w.O + (int64_t)w.pos[p] * d + col);
        acc.x = fmaf(gj, o.x, acc.x);
        acc.y = fmaf(gj, o.y, acc.y);
        acc.z = fmaf(gj, o.z, acc.z);
        acc.w = fmaf(gj, o.w, acc.w);
    }
    *reinterpret_cast<float4*>(y + (int64_t)t * d + col) = acc;
}

}  // namespace

// Pick the wave split and the LDS chunk for a product with K codes, at most
// T tokens per expert and `rows` output rows per expert.
FfnPlan plan_ffn(int K, int T, int rows) {
    FfnPlan p;
    p.nt_alloc = T < 16 ? (T < 1 ? 1 : T) : 16;
    // few tokens: split K across the waves (more waves in flight per
    // expert, little activation staging); many tokens: split rows
    if (T <= 2) { p.wr = 1; p.wk = 4; }
    else if (T <= 8) { p.wr = 2; p.wk = 2; }
    else { p.wr = 4; p.wk = 1; }
    while (p.wr < 4 && (K / kRowAlign) % p.wk != 0) { p.wr *= 2; p.wk /= 2; }
    while (p.wr > 1 && rows % (16 * p.wr) != 0) { p.wr /= 2; p.wk *= 2; }
    // chunk: the largest divisor of K (in 128-code blocks, a multiple of wk)
    // whose fp16 rows fit the LDS budget
    const size_t budget = 40 * 1024;
    const int nblk = K / kRowAlign;
    int best = p.wk;
    for (int c = p.wk; c <= nblk; c += p.wk)
        if (nblk % c == 0 && (size_t)p.nt_alloc * (c * kRowAlign + 8) * 2 <= budget) best = c;
    p.kc = best * kRowAlign;
    const size_t xs = (size_t)p.nt_alloc * (p.kc + 8) * 2;
    const size_t red = (size_t)(p.wk - 1) * p.wr * 2 * 4 * 64 * 4;
    p.lds = xs > red ? xs : red;
    return p;
}

hipError_t launch_gate_up(const FfnArgs& a, const FfnPlan& p, hipStream_t s) {
    return launch_ffn<0>(a, p, s);
}
hipError_t launch_down(const FfnArgs& a, const FfnPlan& p, hipStream_t s) {
    return launch_ffn<1>(a, p, s);
}

hipError_t launch_combine(const FwdWork& w, int T, int d, int k, float* y, hipStream_t s) {
    dim3 grid((unsigned)((d + 4 * kThreads - 1) / (4 * kThreads)), (unsigned)T);
    combine_kernel<<<grid, kThreads, 0, s>>>(w, d, k, y);
    return hipGetLastError();
}

}  // namespace pw
