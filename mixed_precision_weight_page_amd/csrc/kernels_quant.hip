// Quantizer kernels (PagedWeight page, section "Implementation Details",
// Eq. 2): per-expert max|w|, the per-expert loss table L(b) used by Eq. 1,
// and the pack of codes into the expert's page.
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

// Four consecutive weights as fp32 (fp16 masters convert exactly).
__device__ __forceinline__ void load4(const void* base, int64_t idx, int f16, float v[4]) {
    if (f16) {
        const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const _Float16*>(base) + idx);
        const _Float16* h = reinterpret_cast<const _Float16*>(&u);
        v[0] = (float)h[0]; v[1] = (float)h[1]; v[2] = (float)h[2]; v[3] = (float)h[3];
    } else {
        const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
        v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
    }
}

// s = the fp32 value nearest m / qmax: the fp64 quotient is correctly
// rounded and m / qmax (qmax odd) never lies on an fp32 rounding boundary.
__device__ __forceinline__ float scale_of(float m, int qm) {
    return m == 0.0f ? 0.0f : (float)((double)m / (double)qm);
}

// round-half-to-even of the exact quotient w / s (s > 0), without a
// double-precision divide: take the rounded fp32 quotient, then test it
// against the two neighbouring midpoints exactly. fma(-(r +- 1/2), s, w)
// is w - (r +- 1/2) s rounded once, so its sign (and whether it is zero) is
// that of the exact difference. Scales below 2^-100 take the fp64 path so
// that the difference cannot underflow.
__device__ __forceinline__ float round_quotient(float w, float s) {
    if (s < 7.8886091e-31f) return (float)rint((double)w / (double)s);
    float r = rintf(w / s);
    const float hi = fmaf(-(r + 0.5f), s, w);   // sign of w/s - (r + 1/2)
    const float lo = fmaf(-(r - 0.5f), s, w);   // sign of w/s - (r - 1/2)
    const bool odd = ((int)r) & 1;
    if (hi > 0.0f) r += 1.0f;
    else if (lo < 0.0f) r -= 1.0f;
    else if (hi == 0.0f) { if (odd) r += 1.0f; }   // tie at r + 1/2
    else if (lo == 0.0f) { if (odd) r -= 1.0f; }   // tie at r - 1/2
    return r;
}

__device__ __forceinline__ float code_of(float w, float s, float qm) {
    if (s == 0.0f) return 0.0f;
    const float r = round_quotient(w, s);
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

// grid (3*M / kStatChunk, E)
__global__ __launch_bounds__(kThreads) void absmax_kernel(const void* w1, const void* w3,
                                                          const void* w2, int f16, int64_t M,
                                                          uint32_t* absmax, uint32_t* flags) {
    const int e = blockIdx.y;
    const int64_t start = (int64_t)blockIdx.x * kStatChunk;
    const int mtx = (int)(start / M);
    const void* base = matrix_base(w1, w3, w2, mtx);
    const int64_t off = (int64_t)e * M + (start - (int64_t)mtx * M);
    uint32_t m = 0, bad = 0;
#pragma unroll 4
    for (int i = 0; i < kPerThread / 4; ++i) {
        float v[4];
        load4(base, off + (int64_t)(i * kThreads + threadIdx.x) * 4, f16, v);
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
// b = 3, 4, 8 in fp64, written in block order (no atomics).
__global__ __launch_bounds__(kThreads) void loss_partial_kernel(const void* w1, const void* w3,
                                                                const void* w2, int f16,
                                                                int64_t M,
                                                                const uint32_t* absmax,
                                                                double* partial) {
    const int e = blockIdx.y;
    const int64_t start = (int64_t)blockIdx.x * kStatChunk;
    const int mtx = (int)(start / M);
    const void* base = matrix_base(w1, w3, w2, mtx);
    const int64_t off = (int64_t)e * M + (start - (int64_t)mtx * M);
    const float m = __uint_as_float(absmax[e]);
    float s[3], qm[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        qm[i] = (float)qmax_of(bits_of_index(i));
        s[i] = scale_of(m, qmax_of(bits_of_index(i)));
    }
    double acc[3] = {0.0, 0.0, 0.0};
    for (int i = 0; i < kPerThread / 4; ++i) {
        float v[4];
        load4(base, off + (int64_t)(i * kThreads + threadIdx.x) * 4, f16, v);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int b = 0; b < 3; ++b) {
                const float q = code_of(v[j], s[b], qm[b]);
                const double err = (double)v[j] - (double)s[b] * (double)q;  // exact
                acc[b] = fma(err, err, acc[b]);
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

// One wave packs one tile of 16 rows x 128 codes. Lane l = 16 g + r
// quantizes codes 32g..32g+31 of row r into a 32B-bit LSB-first run and
// stores it in the tile: 4-bit 16 bytes at 16 l; 8-bit 16 bytes at 16 l and
// 16 bytes at 1024 + 16 l; 3-bit 12 bytes at 12 l.
template <int B>
__device__ __forceinline__ void pack_lane(const void* base, int64_t src, int f16, float s,
                                          uint8_t* tile) {
    const int lane = threadIdx.x & 63;
    const float qm = (float)qmax_of(B);
    uint32_t w[B];
#pragma unroll
    for (int i = 0; i < B; ++i) w[i] = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float v[4];
        load4(base, src + 4 * i, f16, v);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t u = (uint32_t)((int)code_of(v[j], s, qm) + (1 << (B - 1)));
            const int bit = B * (4 * i + j);          // compile-time after unrolling
            w[bit / 32] |= u << (bit % 32);
            if (bit % 32 + B > 32) w[bit / 32 + 1] |= u >> (32 - bit % 32);
        }
    }
    if constexpr (B == 4) {
        *reinterpret_cast<uint4*>(tile + 16 * lane) = make_uint4(w[0], w[1], w[2], w[3]);
    } else if constexpr (B == 8) {
        *reinterpret_cast<uint4*>(tile + 16 * lane) = make_uint4(w[0], w[1], w[2], w[3]);
        *reinterpret_cast<uint4*>(tile + 1024 + 16 * lane) = make_uint4(w[4], w[5], w[6], w[7]);
    } else {
        uint32_t* o = reinterpret_cast<uint32_t*>(tile + 12 * lane);
        o[0] = w[0]; o[1] = w[1]; o[2] = w[2];
    }
}

// grid (3*M / 8192, nlist), 4 waves: wave w of block x packs tile 4x + w of
// the listed expert (tiles of W1, then W3, then W2; in each matrix in
// (16-row block, 128-code step) order).
__global__ __launch_bounds__(kThreads) void pack_kernel(const void* w1, const void* w3,
                                                        const void* w2, int f16, int d, int F,
                                                        DevTable tab, const int32_t* list,
                                                        uint8_t* pool) {
    const int e = list[blockIdx.y];
    const int b = tab.bits[e];
    const float s = tab.scale[e];
    const int64_t M = (int64_t)F * d;
    const int64_t tpm = M / 2048;                         // tiles per matrix
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int mtx = (int)(t / tpm);
    const int64_t tt = t - mtx * tpm;
    const int K = mtx == 2 ? F : d;
    const int steps = K / 128;
    const int64_t rb = tt / steps;
    const int st = (int)(tt - rb * steps);
    const int lane = threadIdx.x & 63;
    const int64_t row = rb * 16 + (lane & 15);
    const int64_t src = (int64_t)e * M + row * K + st * 128 + 32 * (lane >> 4);
    const void* base = matrix_base(w1, w3, w2, mtx);
    uint8_t* tile = pool + tab.off[e] + mtx * (M * b / 8) + tt * (256 * b);
    if (b == 3) pack_lane<3>(base, src, f16, s, tile);
    else if (b == 4) pack_lane<4>(base, src, f16, s, tile);
    else pack_lane<8>(base, src, f16, s, tile);
}

}  // namespace

hipError_t launch_absmax(const void* w1, const void* w3, const void* w2, int f16, int E,
                         int64_t M, uint32_t* absmax, uint32_t* flags, hipStream_t s) {
    dim3 grid((unsigned)(3 * M / kStatChunk), (unsigned)E);
    absmax_kernel<<<grid, kThreads, 0, s>>>(w1, w3, w2, f16, M, absmax, flags);
    return hipGetLastError();
}

hipError_t launch_loss(const void* w1, const void* w3, const void* w2, int f16, int E,
                       int64_t M, const uint32_t* absmax, double* partial, double* loss,
                       hipStream_t s) {
    const int nblk = (int)(3 * M / kStatChunk);
    loss_partial_kernel<<<dim3(nblk, E), kThreads, 0, s>>>(w1, w3, w2, f16, M, absmax, partial);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    loss_final_kernel<<<E, kThreads, 0, s>>>(partial, nblk, 3 * M, loss);
    return hipGetLastError();
}

hipError_t launch_pack(const void* w1, const void* w3, const void* w2, int f16, int d, int F,
                       DevTable tab, const int32_t* list, int nlist, uint8_t* pool,
                       hipStream_t s) {
    if (nlist == 0) return hipSuccess;
    const int64_t M = (int64_t)F * d;
    dim3 grid((unsigned)(3 * M / 8192), (unsigned)nlist);
    pack_kernel<<<grid, kThreads, 0, s>>>(w1, w3, w2, f16, d, F, tab, list, pool);
    return hipGetLastError();
}

}  // namespace pw
