// Quantizer kernels (PagedWeight page, section "Implementation Details",
// Eq. 2): per-expert max|w|, the per-expert loss table L(b) used by Eq. 1,
// and the pack of codes into the expert's page. Bitplane pages (the
// PagedMoE page's prefix-compatible layout, read as a tree codebook over
// Eq. 2's 8-bit codes u8): plane j holds bit 7 - j of every u8, a depth-b
// page holds planes 0 .. b-1 (each the three matrices' tiles, W_e / 8
// bytes), and a depth-b weight is s8 c / 2 with c = (2p + 1) 2^(8-b) - 257,
// p = u8 >> (8 - b).
//
// Weight space of expert e: its W1 block (M = F*d weights), then W3, then W2,
// each row-major. A page holds the codes u = q + 2^(b-1) of W1, W3, W2, each
// matrix in tiles of 16 rows x 128 codes: tiles in (row block, K step)
// order; in a tile, lane l = 16 g + r holds the LSB-first run of codes
// 32g..32g+31 of row r (4b bytes), split into pieces of at most 16 bytes,
// piece p of all 64 lanes stored together. A wave of the forward kernels
// then reads each tile as contiguous 16-byte (12-byte) lane loads.
#include <hip/hip_runtime.h>

#include "pw_internal.h"

namespace pw {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = kStatChunk / kThreads;  // 64 weights

__device__ __forceinline__ const void* matrix_base(const void* w1, const void* w3,
                                                   const void* w2, int mtx) {
    return mtx == 0 ? w1 : (mtx == 1 ? w3 : w2);
}

// Four consecutive weights of fp16 (F16) or fp32 masters: the raw load and
// its conversion to fp32 (fp16 converts exactly) are separate, so that a
// thread's loads can all be issued before the first is used (the master
// type is a template parameter: no branch between the loads).
template <bool F16>
struct Raw4 {
    typedef uint2 type;
};
template <>
struct Raw4<false> {
    typedef float4 type;
};
template <bool F16>
__device__ __forceinline__ typename Raw4<F16>::type load4_raw(const void* base, int64_t idx) {
    if constexpr (F16) return *reinterpret_cast<const uint2*>(static_cast<const _Float16*>(base) + idx);
    else return *reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
}
template <bool F16>
__device__ __forceinline__ void to_f32(const typename Raw4<F16>::type& u, float v[4]) {
    if constexpr (F16) {
        const _Float16* h = reinterpret_cast<const _Float16*>(&u);
        v[0] = (float)h[0]; v[1] = (float)h[1]; v[2] = (float)h[2]; v[3] = (float)h[3];
    } else {
        v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
    }
}

// s = the fp32 value nearest m / qmax: the fp64 quotient is correctly
// rounded and m / qmax (qmax odd) never lies on an fp32 rounding boundary.
__device__ __forceinline__ float scale_of(float m, int qm) {
    return m == 0.0f ? 0.0f : (float)((double)m / (double)qm);
}

// round-half-to-even of the exact quotient w / s (s > 0), without a
// divide. p = w * (1/s) rounds twice (1/s and the product), so it differs
// from w / s by at most |p| 2^-22; r = rint(p), and p - r is exact (both are
// multiples of p's last place and |p - r| <= 1/2). If p is closer to r than
// 1/2 - |p| 2^-22, so is w / s, and r is its rounding: nearly every weight
// ends there. Otherwise r is within one of the correctly rounded quotient
// and the two neighbouring midpoints are tested exactly: fma(-(r +- 1/2),
// s, w) is w - (r +- 1/2) s rounded once, so its sign (and whether it is
// zero) is that of the exact difference. Scales below 2^-100 take the fp64
// path so that the difference cannot underflow.
__device__ __forceinline__ float round_quotient(float w, float s, float inv_s) {
    if (s < 7.8886091e-31f) return (float)rint((double)w / (double)s);
    const float p = w * inv_s;
    float r = rintf(p);
    if (fabsf(p - r) < fmaf(fabsf(p), -2.384185791015625e-07f, 0.5f)) return r;
    const float hi = fmaf(-(r + 0.5f), s, w);   // sign of w/s - (r + 1/2)
    const float lo = fmaf(-(r - 0.5f), s, w);   // sign of w/s - (r - 1/2)
    const bool odd = ((int)r) & 1;
    if (hi > 0.0f) r += 1.0f;
    else if (lo < 0.0f) r -= 1.0f;
    else if (hi == 0.0f) { if (odd) r += 1.0f; }   // tie at r + 1/2
    else if (lo == 0.0f) { if (odd) r -= 1.0f; }   // tie at r - 1/2
    return r;
}

__device__ __forceinline__ float code_of(float w, float s, float inv_s, float qm) {
    if (s == 0.0f) return 0.0f;
    const float r = round_quotient(w, s, inv_s);
    return fminf(fmaxf(r, -qm), qm);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
    return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// grid (3*M / kStatChunk, E); every load of a thread in flight at once
template <bool F16>
__global__ __launch_bounds__(kThreads) void absmax_kernel(const void* w1, const void* w3,
                                                          const void* w2, int64_t M,
                                                          uint32_t* absmax, uint32_t* flags) {
    const int e = blockIdx.y;
    const int64_t start = (int64_t)blockIdx.x * kStatChunk;
    const int mtx = (int)(start / M);
    const void* base = matrix_base(w1, w3, w2, mtx);
    const int64_t off = (int64_t)e * M + (start - (int64_t)mtx * M);
    uint32_t m = 0, bad = 0;
    typename Raw4<F16>::type raw[kPerThread / 4];
#pragma unroll
    for (int i = 0; i < kPerThread / 4; ++i)
        raw[i] = load4_raw<F16>(base, off + (int64_t)(i * kThreads + threadIdx.x) * 4);
#pragma unroll
    for (int i = 0; i < kPerThread / 4; ++i) {
        float v[4];
        to_f32<F16>(raw[i], v);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t a = __float_as_uint(v[j]) & 0x7fffffffu;
            if (a >= 0x7f800000u) bad = 1;
            else m = max(m, a);
        }
    }
    __shared__ uint32_t red[kThreads / 64];
    m = wave_max_u32(m);
    const uint32_t anybad = __any(bad);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = red[0];
        for (int w = 1; w < kThreads / 64; ++w) r = max(r, red[w]);
        atomicMax(&absmax[e], r);
    }
    if (anybad && (threadIdx.x & 63) == 0) atomicOr(&flags[0], 1u);
}

// grid (3*M / kStatChunk, E): per-block partial sums of (w - s q)^2 for
// b = 3, 4, 8 in fp64 (bitplane pages: of (w - s8 c / 2)^2 at depths 3, 4,
// 8), written in block order (no atomics).
template <bool F16>
__global__ __launch_bounds__(kThreads) void loss_partial_kernel(const void* w1, const void* w3,
                                                                const void* w2,
                                                                int64_t M,
                                                                const uint32_t* absmax,
                                                                double* partial, int planes) {
    const int e = blockIdx.y;
    const int64_t start = (int64_t)blockIdx.x * kStatChunk;
    const int mtx = (int)(start / M);
    const void* base = matrix_base(w1, w3, w2, mtx);
    const int64_t off = (int64_t)e * M + (start - (int64_t)mtx * M);
    const float m = __uint_as_float(absmax[e]);
    float s[3], inv_s[3], qm[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        qm[i] = (float)qmax_of(bits_of_index(i));
        s[i] = scale_of(m, qmax_of(bits_of_index(i)));
        inv_s[i] = s[i] > 0.0f ? 1.0f / s[i] : 0.0f;
    }
    double acc[3] = {0.0, 0.0, 0.0};
    // the loads of four iterations in flight at once
    for (int i0 = 0; i0 < kPerThread / 4; i0 += 4) {
      typename Raw4<F16>::type raw[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
          raw[k] = load4_raw<F16>(base, off + (int64_t)((i0 + k) * kThreads + threadIdx.x) * 4);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float v[4];
        to_f32<F16>(raw[k], v);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (planes) {
                const int u = (int)code_of(v[j], s[2], inv_s[2], qm[2]) + 128;   // u8 (s[2] = s8)
#pragma unroll
                for (int b = 0; b < 3; ++b) {
                    const int depth = bits_of_index(b);
                    const int c = (2 * (u >> (8 - depth)) + 1) * (1 << (8 - depth)) - 257;
                    const double err = (double)v[j] - (double)s[2] * (double)c * 0.5;   // exact
                    acc[b] = fma(err, err, acc[b]);
                }
            } else {
#pragma unroll
                for (int b = 0; b < 3; ++b) {
                    const float q = code_of(v[j], s[b], inv_s[b], qm[b]);
                    const double err = (double)v[j] - (double)s[b] * (double)q;  // exact
                    acc[b] = fma(err, err, acc[b]);
                }
            }
        }
      }
    }
    __shared__ double red[kThreads / 64][3];
#pragma unroll
    for (int b = 0; b < 3; ++b) {
        const double t = wave_sum_f64(acc[b]);
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6][b] = t;
    }
    __syncthreads();
    if (threadIdx.x < 3) {
        double t = 0.0;
        for (int w = 0; w < kThreads / 64; ++w) t += red[w][threadIdx.x];
        partial[((int64_t)e * gridDim.x + blockIdx.x) * 3 + threadIdx.x] = t;
    }
}

// grid E: L[e][b] = (sum of the partials in a fixed order) / W_e.
__global__ __launch_bounds__(kThreads) void loss_final_kernel(const double* partial, int nblk,
                                                              int64_t We, double* loss) {
    const int e = blockIdx.x;
    double acc[3] = {0.0, 0.0, 0.0};
    for (int i = threadIdx.x; i < nblk; i += kThreads)
        for (int b = 0; b < 3; ++b) acc[b] += partial[((int64_t)e * nblk + i) * 3 + b];
    __shared__ double red[kThreads / 64][3];
    for (int b = 0; b < 3; ++b) {
        const double t = wave_sum_f64(acc[b]);
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6][b] = t;
    }
    __syncthreads();
    if (threadIdx.x < 3) {
        double t = 0.0;
        for (int w = 0; w < kThreads / 64; ++w) t += red[w][threadIdx.x];
        loss[e * 3 + threadIdx.x] = t / (double)We;
    }
}

// One wave packs one tile of 16 rows x 128 codes of one matrix. Loads are
// row-contiguous (lanes 0-31 one row, 32-63 the next, four weights each);
// the codes u = q + 2^(b-1) go through LDS as bytes (rows padded to 144
// bytes), and lane l = 16 g + r then packs codes 32g..32g+31 of row r into
// a 32B-bit LSB-first run: 4-bit 16 bytes at 16 l; 8-bit 16 bytes at 16 l
// and 16 bytes at 1024 + 16 l; 3-bit 12 bytes at 12 l.
constexpr int kCodeRow = 144;   // LDS bytes per row of codes

template <int B>
__device__ __forceinline__ void pack_run(const uint8_t* codes, uint8_t* tile) {
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const uint4 c0 = *reinterpret_cast<const uint4*>(codes + r * kCodeRow + 32 * g);
    const uint4 c1 = *reinterpret_cast<const uint4*>(codes + r * kCodeRow + 32 * g + 16);
    const uint32_t c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};   // 4 codes per word
    if constexpr (B == 8) {
        *reinterpret_cast<uint4*>(tile + 16 * lane) = c0;
        *reinterpret_cast<uint4*>(tile + 1024 + 16 * lane) = c1;
    } else if constexpr (B == 4) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // codes 8i..8i+7 from words 2i (bytes 0-3) and 2i+1 (bytes 4-7)
            const uint32_t lo = c[2 * i], hi = c[2 * i + 1];
            const uint32_t a = (lo & 0x0fu) | ((lo >> 4) & 0xf0u) | ((lo >> 8) & 0xf00u) | ((lo >> 12) & 0xf000u);
            const uint32_t b = (hi & 0x0fu) | ((hi >> 4) & 0xf0u) | ((hi >> 8) & 0xf00u) | ((hi >> 12) & 0xf000u);
            w[i] = a | (b << 16);
        }
        *reinterpret_cast<uint4*>(tile + 16 * lane) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
        uint32_t w[3] = {0u, 0u, 0u};
#pragma unroll
        for (int k = 0; k < 32; ++k) {
            const uint32_t u = (c[k >> 2] >> (8 * (k & 3))) & 0xffu;
            const int bit = 3 * k;                    // compile-time after unrolling
            w[bit / 32] |= u << (bit % 32);
            if (bit % 32 + 3 > 32) w[bit / 32 + 1] |= u >> (32 - bit % 32);
        }
        uint32_t* o = reinterpret_cast<uint32_t*>(tile + 12 * lane);
        o[0] = w[0]; o[1] = w[1]; o[2] = w[2];
    }
}

// Bitplane j of a tile: lane l = 16 g + r writes one word, bit i = bit
// 7 - j of code 32 g + i of row r (codes as bytes in LDS, as for pack_run).
__device__ __forceinline__ uint32_t plane_word(const uint8_t* codes, int j) {
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const uint4 c0 = *reinterpret_cast<const uint4*>(codes + r * kCodeRow + 32 * g);
    const uint4 c1 = *reinterpret_cast<const uint4*>(codes + r * kCodeRow + 32 * g + 16);
    const uint32_t c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};   // 4 codes per word
    uint32_t w = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t x = (c[k] >> (7 - j)) & 0x01010101u;   // the bit of each byte, at 0, 8, 16, 24
        w |= ((x | (x >> 7) | (x >> 14) | (x >> 21)) & 0xfu) << (4 * k);
    }
    return w;
}

// grid (3*M / 8192, nlist), 4 waves: wave w of block x packs tile 4x + w of
// the listed expert (tiles of W1, then W3, then W2; in each matrix in
// (16-row block, 128-code step) order). Bitplane pages (planes != 0): the
// codes are u8 of Eq. 2 at 8 bits with scale s8 (the table's scale), and
// planes first[i] .. depth - 1 of the i-th listed expert are written.
template <bool F16>
__global__ __launch_bounds__(kThreads) void pack_kernel(const void* w1, const void* w3,
                                                        const void* w2, int d, int F,
                                                        DevTable tab, const int32_t* list,
                                                        const int32_t* first, int planes,
                                                        uint8_t* pool) {
    __shared__ __attribute__((aligned(16))) uint8_t s_codes[kThreads / 64][16 * kCodeRow];
    const int e = list[blockIdx.y];
    const int b = tab.bits[e];            // bit-width, or the depth of a bitplane page
    const int cb = planes ? 8 : b;         // bits of the codes computed
    const float s = tab.scale[e];
    const float inv_s = s > 0.0f ? 1.0f / s : 0.0f;
    const float qm = (float)qmax_of(cb);
    const int bias = 1 << (cb - 1);
    const int64_t M = (int64_t)F * d;
    const int64_t tpm = M / 2048;                         // tiles per matrix
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + wave;
    const int mtx = (int)(t / tpm);
    const int64_t tt = t - mtx * tpm;
    const int K = mtx == 2 ? F : d;
    const int steps = K / 128;
    const int64_t rb = tt / steps;
    const int st = (int)(tt - rb * steps);
    const void* base = matrix_base(w1, w3, w2, mtx);
    uint8_t* codes = s_codes[wave];
    // rows 2i + lane / 32 of the tile, weights 4 (lane % 32) .. +4; all
    // eight loads in flight before the first is used
    const int half = lane >> 5, c4 = 4 * (lane & 31);
    typename Raw4<F16>::type raw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        raw[i] = load4_raw<F16>(base, (int64_t)e * M + (rb * 16 + 2 * i + half) * K + st * 128 + c4);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = 2 * i + half;
        float v[4];
        to_f32<F16>(raw[i], v);
        uint32_t packed = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            packed |= (uint32_t)((int)code_of(v[j], s, inv_s, qm) + bias) << (8 * j);
        *reinterpret_cast<uint32_t*>(codes + row * kCodeRow + c4) = packed;
    }
    __syncthreads();   // (the wave's own rows; a block barrier keeps it simple)
    if (planes) {
        const int64_t plane = 3 * M / 8;
        uint8_t* tile = pool + tab.off[e] + mtx * (M / 8) + tt * 256 + 4 * lane;
        for (int j = first[blockIdx.y]; j < b; ++j)
            *reinterpret_cast<uint32_t*>(tile + j * plane) = plane_word(codes, j);
        return;
    }
    uint8_t* tile = pool + tab.off[e] + mtx * (M * b / 8) + tt * (256 * b);
    if (b == 3) pack_run<3>(codes, tile);
    else if (b == 4) pack_run<4>(codes, tile);
    else pack_run<8>(codes, tile);
}

}  // namespace

hipError_t launch_absmax(const void* w1, const void* w3, const void* w2, int f16, int E,
                         int64_t M, uint32_t* absmax, uint32_t* flags, hipStream_t s) {
    dim3 grid((unsigned)(3 * M / kStatChunk), (unsigned)E);
    if (f16) absmax_kernel<true><<<grid, kThreads, 0, s>>>(w1, w3, w2, M, absmax, flags);
    else absmax_kernel<false><<<grid, kThreads, 0, s>>>(w1, w3, w2, M, absmax, flags);
    return hipGetLastError();
}

hipError_t launch_loss(const void* w1, const void* w3, const void* w2, int f16, int E,
                       int64_t M, const uint32_t* absmax, double* partial, double* loss, int planes,
                       hipStream_t s) {
    const int nblk = (int)(3 * M / kStatChunk);
    if (f16) loss_partial_kernel<true><<<dim3(nblk, E), kThreads, 0, s>>>(w1, w3, w2, M, absmax, partial, planes);
    else loss_partial_kernel<false><<<dim3(nblk, E), kThreads, 0, s>>>(w1, w3, w2, M, absmax, partial, planes);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    loss_final_kernel<<<E, kThreads, 0, s>>>(partial, nblk, 3 * M, loss);
    return hipGetLastError();
}

hipError_t launch_pack(const void* w1, const void* w3, const void* w2, int f16, int d, int F,
                       DevTable tab, const int32_t* list, const int32_t* first, int nlist, int planes,
                       uint8_t* pool, hipStream_t s) {
    if (nlist == 0) return hipSuccess;
    const int64_t M = (int64_t)F * d;
    dim3 grid((unsigned)(3 * M / 8192), (unsigned)nlist);
    if (f16) pack_kernel<true><<<grid, kThreads, 0, s>>>(w1, w3, w2, d, F, tab, list, first, planes, pool);
    else pack_kernel<false><<<grid, kThreads, 0, s>>>(w1, w3, w2, d, F, tab, list, first, planes, pool);
    return hipGetLastError();
}

}  // namespace pw
