// Expert FFN kernels for routed tokens (PagedWeight page, section "Dynamic
// Paging": the routed experts' pages are dequantized on the fly; Eq. 2 gives
// the dequantized weight s_e * q). SwiGLU: h = silu(W1 x) * (W3 x), o = W2 h.
//
// One workgroup = 64 rows of one active expert, all of the expert's tokens;
// each of its four waves streams one 16-row block, whose tiles (16 rows x
// 128 codes) are contiguous in the page, so every load instruction of a
// wave reads one contiguous run. One 4B-byte load per lane per tile
// (B = bits), prefetched several steps ahead; they are turned into exact
// fp16 integers q in registers (dequant.h: magic-exponent OR, then one
// packed fp16 subtract or multiply-add per pair) and multiplied on the
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
// VALU only the unpack (about 1.1 instructions per 4-bit weight).
#include <hip/hip_runtime.h>

#include <math.h>

#include "dequant.h"
#include "pw_internal.h"

namespace pw {
namespace {

using dq::half8_t;
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kStep = 128;   // codes per wave per step (4 K-groups x 32)

template <int B>
struct Codes {
    uint32_t w[B];   // 32 consecutive codes of one row, LSB-first
};

// byte offset of lane l's run inside a 16-row x 128-code tile (the 8-bit
// run's second half lies 1024 bytes further)
template <int B>
__device__ __forceinline__ constexpr int lane_offset(int l) { return (B == 3 ? 12 : 16) * l; }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Codes are read once per forward: non-temporal loads keep them from
// displacing the activations and partial outputs in the caches.
__device__ __forceinline__ u32x4 stream_load16(const uint8_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

template <int B>
__device__ __forceinline__ Codes<B> load_codes(const uint8_t* p) {
    Codes<B> c;
    if constexpr (B == 4) {
        const u32x4 u = stream_load16(p);
        c.w[0] = u.x; c.w[1] = u.y; c.w[2] = u.z; c.w[3] = u.w;
    } else if constexpr (B == 8) {
        const u32x4 u = stream_load16(p);
        const u32x4 v = stream_load16(p + 1024);
        c.w[0] = u.x; c.w[1] = u.y; c.w[2] = u.z; c.w[3] = u.w;
        c.w[4] = v.x; c.w[5] = v.y; c.w[6] = v.z; c.w[7] = v.w;
    } else {
        const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
        c.w[0] = __builtin_nontemporal_load(q);
        c.w[1] = __builtin_nontemporal_load(q + 1);
        c.w[2] = __builtin_nontemporal_load(q + 2);
    }
    return c;
}

using dq::half2_t;
using dq::perm_slot;

__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// Stage K-chunk [k0, k0 + kc) of nt token rows into LDS as permuted fp16.
// MODE 0 reads bf16 activations of the tokens in tok[]; MODE 1 reads the
// fp16 SwiGLU rows base.. of H.
template <int MODE, int B>
__device__ __forceinline__ void stage(_Float16* xs, int stride, const FfnArgs& a,
                                      const int* tok, int hrow0, int nt, int k0, int kc) {
    if constexpr (B == 3) {
        // the 3-bit order permutes across all 32 codes of a run
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
    } else {
        // 4- and 8-bit orders permute within groups of 8: one 16-byte chunk
        // of 8 activations per thread and iteration
        const int nch = kc / 8;
        for (int idx = threadIdx.x; idx < nt * nch; idx += kThreads) {
            const int n = idx / nch, ch = idx - n * nch;
            _Float16 v[8];
            if constexpr (MODE == 0) {
                const uint4 u = *reinterpret_cast<const uint4*>(a.x + (int64_t)tok[n] * a.d + k0 + 8 * ch);
                const uint32_t ww[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    v[2 * h] = (_Float16)bf16_to_f32((uint16_t)(ww[h] & 0xffffu));
                    v[2 * h + 1] = (_Float16)bf16_to_f32((uint16_t)(ww[h] >> 16));
                }
            } else {
                union {
                    uint4 u;
                    _Float16 h[8];
                } t;
                t.u = *reinterpret_cast<const uint4*>(a.w.H + (int64_t)(hrow0 + n) * a.F + k0 + 8 * ch);
#pragma unroll
                for (int h = 0; h < 8; ++h) v[h] = t.h[h];
            }
            union {
                uint4 u;
                _Float16 h[8];
            } o;
#pragma unroll
            for (int s = 0; s < 8; ++s) o.h[s] = v[perm_slot<B>(s)];
            *reinterpret_cast<uint4*>(xs + n * stride + 8 * ch) = o.u;
        }
    }
}

// Steps of codes in flight per wave: 8 x 16 B (4-bit), 8 x 12 B (3-bit),
// 4 x 32 B (8-bit) per matrix and lane.
template <int B>
__device__ __forceinline__ constexpr int prefetch_depth() { return B == 8 ? 4 : 8; }

// The four MFMAs of one 128-code step for each matrix; bp points at the
// step's 128 staged activations of this lane's token row and K-group.
template <int B, int NMAT>
__device__ __forceinline__ void step_mma(const Codes<B> (&cur)[NMAT], const _Float16* bp,
                                         f32x4 (&acc)[NMAT], const dq::Const& dc) {
    if constexpr (B == 3) {
        half2_t pr[NMAT][16];
#pragma unroll
        for (int m = 0; m < NMAT; ++m) dq::pairs3(cur[m].w, pr[m], dc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const half8_t bfr = *reinterpret_cast<const half8_t*>(bp + 8 * i);
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
                acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    dq::cat(pr[m][4 * i], pr[m][4 * i + 1], pr[m][4 * i + 2], pr[m][4 * i + 3]), bfr, acc[m], 0,
                    0, 0);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const half8_t bfr = *reinterpret_cast<const half8_t*>(bp + 8 * i);
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
                acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dq::frag48<B>(cur[m].w, i, dc), bfr, acc[m], 0, 0, 0);
        }
    }
}

// MODE 0: gate/up + SwiGLU (NMAT = 2: W1, W3); MODE 1: down (NMAT = 1: W2),
// over K-steps [ks0, ks0 + nsteps) (the down product may be split along K
// across workgroups; split `sp` writes its own partial output).
// The workgroup covers rows [64 rt, 64 rt + 64) of expert e; wave w owns 16
// of them. Codes are prefetched PD steps ahead in a register ring; the main
// loop issues its loads unconditionally so the ring stays full, and LDS
// chunks of the token rows are staged before the first load when K fits.
// The expert's page-table entry and token range, read by the kernel in one
// round of independent loads before its first code load.
struct ExpertRef {
    const uint8_t* page;
    float s;
    int Te, base;
};

template <int MODE, int B>
__device__ __forceinline__ void ffn_tile(const FfnArgs& a, int lds_bytes, const ExpertRef& ex, int rt, int sp,
                                         int ks0, int nsteps, _Float16* xs, int* tok) {
    constexpr int NMAT = MODE == 0 ? 2 : 1;
    constexpr int PD = prefetch_depth<B>();
    constexpr int SB = 16 * kStep * B / 8;   // bytes of one tile: 16 rows x 128 codes
    const int K = MODE == 0 ? a.d : a.F;
    const int64_t mat_bytes = (int64_t)a.F * a.d * B / 8;
    const uint8_t* page = ex.page;
    const float s = ex.s;
    const int Te = ex.Te;
    const int base = ex.base;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int row0 = rt * 64 + 16 * wave;
    const dq::Const dc = dq::make_const();
    // this wave's 16-row block is one contiguous run of K/128 tiles
    const uint8_t* ap[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
        ap[m] = page + (MODE == 0 ? m : 2) * mat_bytes + ((int64_t)(row0 / 16) * (K / kStep) + ks0) * SB +
                lane_offset<B>(lane);

    for (int tb = 0; tb < Te; tb += 16) {
        const int nt = min(16, Te - tb);
        // steps per LDS chunk: all of them if nt rows fit, else a multiple of
        // PD (the host sizes the LDS for at least PD steps of 16 rows)
        int spc = nsteps;
        if (nt * (nsteps * kStep + 8) * 2 > lds_bytes)
            spc = ((lds_bytes / (2 * nt) - 8) / (kStep * PD)) * PD;
        const int stride = spc * kStep + 8;
        // the first PD steps of codes: the down product issues them before
        // its token rows are staged (their round trips overlap), gate/up
        // after (its token-id and token-row loads, which the first step
        // waits for, are then not queued behind the codes): measured best
        // for each
        Codes<B> buf[NMAT][PD];
        auto issue_codes = [&]() {
#pragma unroll
            for (int j = 0; j < PD; ++j)
#pragma unroll
                for (int m = 0; m < NMAT; ++m) buf[m][j] = load_codes<B>(ap[m] + min(j, nsteps - 1) * SB);
        };
        if constexpr (MODE == 1) issue_codes();
        __syncthreads();   // previous token block done with tok and xs
        if constexpr (MODE == 0) {
            if ((int)threadIdx.x < nt) tok[threadIdx.x] = a.w.sorted[base + tb + threadIdx.x] / a.k;
        }
        __syncthreads();
        // the down product writes this lane's token row of O at its pair index
        int my_pair = 0;
        if constexpr (MODE == 1) my_pair = a.w.sorted[base + tb + min(r, nt - 1)];
        stage<MODE, B>(xs, stride, a, tok, base + tb, nt, ks0 * kStep, min(spc, nsteps) * kStep);
        if constexpr (MODE == 0) issue_codes();
        __syncthreads();
        f32x4 acc[NMAT];
#pragma unroll
        for (int m = 0; m < NMAT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        // B-fragment row of this lane's token (columns past nt repeat a real row)
        const _Float16* bp0 = xs + min(r, nt - 1) * stride + 32 * g;
        int s0 = 0;
        for (; s0 + 2 * PD <= nsteps; s0 += PD) {
            if (s0 != 0 && s0 % spc == 0) {
                __syncthreads();
                stage<MODE, B>(xs, stride, a, tok, base + tb, nt, (ks0 + s0) * kStep,
                               min(spc, nsteps - s0) * kStep);
                __syncthreads();
            }
            const _Float16* bp = bp0 + (s0 % spc) * kStep;
#pragma unroll
            for (int j = 0; j < PD; ++j) {
                Codes<B> cur[NMAT];
#pragma unroll
                for (int m = 0; m < NMAT; ++m) {
                    cur[m] = buf[m][j];
                    buf[m][j] = load_codes<B>(ap[m] + (int64_t)(s0 + j + PD) * SB);
                }
                step_mma<B, NMAT>(cur, bp + j * kStep, acc, dc);
            }
        }
        // The last one or two groups. A group that still has loads to issue
        // clamps their addresses to the last tile (the loads past the end
        // are never used; a conditional load would make the ring slot's old
        // value need a copy while it is still being consumed). The final
        // group issues no loads.
        if (nsteps - s0 > PD) {
            if (s0 != 0 && s0 % spc == 0) {
                __syncthreads();
                stage<MODE, B>(xs, stride, a, tok, base + tb, nt, (ks0 + s0) * kStep,
                               min(spc, nsteps - s0) * kStep);
                __syncthreads();
            }
            const _Float16* bp = bp0 + (s0 % spc) * kStep;
#pragma unroll
            for (int j = 0; j < PD; ++j) {
                Codes<B> cur[NMAT];
#pragma unroll
                for (int m = 0; m < NMAT; ++m) {
                    cur[m] = buf[m][j];
                    buf[m][j] = load_codes<B>(ap[m] + (int64_t)min(s0 + j + PD, nsteps - 1) * SB);
                }
                step_mma<B, NMAT>(cur, bp + j * kStep, acc, dc);
            }
            s0 += PD;
        }
        if (s0 < nsteps) {
            if (s0 != 0 && s0 % spc == 0) {
                __syncthreads();
                stage<MODE, B>(xs, stride, a, tok, base + tb, nt, (ks0 + s0) * kStep,
                               min(spc, nsteps - s0) * kStep);
                __syncthreads();
            }
            const _Float16* bp = bp0 + (s0 % spc) * kStep;
#pragma unroll
            for (int j = 0; j < PD; ++j) {
                if (s0 + j < nsteps) {
                    Codes<B> cur[NMAT];
#pragma unroll
                    for (int m = 0; m < NMAT; ++m) cur[m] = buf[m][j];
                    step_mma<B, NMAT>(cur, bp + j * kStep, acc, dc);
                }
            }
        }
        // D layout: lane (n = lane % 16, g = lane / 16) holds rows 4g..4g+3, token n
        if (r < nt) {
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
                o.x = s * acc[0][0];
                o.y = s * acc[0][1];
                o.z = s * acc[0][2];
                o.w = s * acc[0][3];
                *reinterpret_cast<float4*>(a.w.O + ((int64_t)sp * a.P + my_pair) * a.d + orow) = o;
            }
        }
    }
}

// grid: (active expert, 64-row tile, K split) flattened; experts beyond the
// device-side active count exit at once.
template <int MODE>
__global__ __launch_bounds__(kThreads, MODE == 0 ? 3 : 5) void ffn_kernel(FfnArgs a, int lds_bytes, int tiles, int nsplit) {
    extern __shared__ __attribute__((aligned(16))) _Float16 xs[];
    __shared__ int tok[16];
    const int per_expert = tiles * nsplit;
    const int ai = blockIdx.x / per_expert;
    const SlotDesc sd = a.w.slots[ai];   // stale past the active count, not used then
    if (ai >= a.w.n_act[0]) return;
    const int rem = blockIdx.x - ai * per_expert;
    const int rt = rem / nsplit, sp = rem - rt * nsplit;
    const int b = sd.bits;
    const ExpertRef ex{a.pool + sd.page, sd.scale, sd.cnt, sd.off};
    const int total = (MODE == 0 ? a.d : a.F) / kStep;
    const int nsteps = total / nsplit;
    if (b == 4) ffn_tile<MODE, 4>(a, lds_bytes, ex, rt, sp, sp * nsteps, nsteps, xs, tok);
    else if (b == 8) ffn_tile<MODE, 8>(a, lds_bytes, ex, rt, sp, sp * nsteps, nsteps, xs, tok);
    else ffn_tile<MODE, 3>(a, lds_bytes, ex, rt, sp, sp * nsteps, nsteps, xs, tok);
}

template <int MODE>
hipError_t launch_ffn(const FfnArgs& a, const FfnPlan& p, hipStream_t s, KTimer t) {
    const int rows = MODE == 0 ? a.F : a.d;
    const int tiles = rows / 64;
    const dim3 grid((unsigned)(a.max_act * tiles * p.nsplit));
    return launch_timed(ffn_kernel<MODE>, grid, dim3(kThreads), p.lds, s, t.start, t.stop, a,
                        (int)p.lds, tiles, p.nsplit);
}

// Partial outputs are read once: non-temporal loads (17% faster for 4096
// tokens x top-6 than plain ones).
__device__ __forceinline__ float4 load_partial(const float* p) {
    return __builtin_bit_cast(float4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}

// y[t] = sum_j g[t,j] * (sum_s O[s][t k + j]) in slot and split order;
// grid (ceil(d/1024), T). A token's k partial rows are consecutive in O;
// the loads of up to 8 slots (and of two further splits of each) are issued
// before any of them is used, and the sums keep the slot and split order.
__global__ __launch_bounds__(kThreads) void combine_kernel(FwdWork w, int d, int k, int P, int nsplit,
                                                           float* y) {
    const int t = blockIdx.y;
    const int col = (blockIdx.x * kThreads + threadIdx.x) * 4;
    if (col >= d) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = 0; j0 < k; j0 += 8) {
        float4 o[8];
        float gj[8];
        const float* src[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (j0 + u < k) {
                const int p = t * k + j0 + u;
                gj[u] = w.g[p];
                src[u] = w.O + (int64_t)p * d + col;
                o[u] = load_partial(src[u]);
            }
        }
        // the other K splits, two at a time: the loads of both splits for
        // every slot are issued before any is added (one round trip per two
        // splits, not one per slot and split); sums in split order
        for (int sp = 1; sp < nsplit; sp += 2) {
            const bool two = sp + 1 < nsplit;
            float4 qa[8], qb[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (j0 + u < k) {
                    qa[u] = load_partial(src[u] + (int64_t)sp * P * d);
                    if (two) qb[u] = load_partial(src[u] + (int64_t)(sp + 1) * P * d);
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (j0 + u < k) {
                    o[u].x += qa[u].x; o[u].y += qa[u].y; o[u].z += qa[u].z; o[u].w += qa[u].w;
                    if (two) {
                        o[u].x += qb[u].x; o[u].y += qb[u].y; o[u].z += qb[u].z; o[u].w += qb[u].w;
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (j0 + u < k) {
                acc.x = fmaf(gj[u], o[u].x, acc.x);
                acc.y = fmaf(gj[u], o[u].y, acc.y);
                acc.z = fmaf(gj[u], o[u].z, acc.z);
                acc.w = fmaf(gj[u], o[u].w, acc.w);
            }
        }
    }
    *reinterpret_cast<float4*>(y + (int64_t)t * d + col) = acc;
}

}  // namespace

// LDS for the staged token rows: all of the K range for up to min(T, 16)
// tokens if that fits 34 KB, else 34 KB (the kernel then stages K in chunks
// sized by the expert's actual token count).
FfnPlan plan_ffn(int K, int T, int nsplit) {
    FfnPlan p;
    p.nt_alloc = T < 16 ? (T < 1 ? 1 : T) : 16;
    p.nsplit = nsplit;
    const size_t full = (size_t)p.nt_alloc * (K / nsplit + 8) * 2;
    // at least 8 steps (the deepest prefetch) of 16 token rows, so a chunk of
    // staged rows always covers whole prefetch groups; 34 KB lets four
    // workgroups share a CU's LDS
    const size_t floor_bytes = (size_t)16 * (8 * kStep + 8) * 2;
    const size_t cap = 34 * 1024 > floor_bytes ? 34 * 1024 : floor_bytes;
    p.lds = full < cap ? full : cap;
    return p;
}

// The down product of a small batch splits K so that the workgroups still
// fill the GPU: the fewest splits (each workgroup streaming the longest run
// of K steps) that give at least kFillWorkgroups workgroups for max_act
// routed experts. Splits divide the d_ff/128 steps; at most max_splits.
int down_splits(int F, int d, int max_act, int max_splits) {
    constexpr int kFillWorkgroups = 1024;
    const int nblk = F / kStep;
    const int64_t per_split = (int64_t)(max_act > 0 ? max_act : 1) * (d / 64);
    int best = 1;
    for (int n = 1; n <= nblk && n <= max_splits; ++n) {
        if (nblk % n) continue;
        best = n;
        // with at most two routed experts (one token) half the workgroups:
        // fewer partial outputs for the combine, and each workgroup's start-up
        // serves twice the bytes (2% faster at one token, measured)
        if (per_split * n >= (max_act <= 2 ? kFillWorkgroups / 2 : kFillWorkgroups)) break;
    }
    return best;
}

hipError_t launch_gate_up(const FfnArgs& a, const FfnPlan& p, hipStream_t s, KTimer t) {
    return launch_ffn<0>(a, p, s, t);
}
hipError_t launch_down(const FfnArgs& a, const FfnPlan& p, hipStream_t s, KTimer t) {
    return launch_ffn<1>(a, p, s, t);
}

hipError_t launch_combine(const FwdWork& w, int T, int d, int k, int P, int nsplit, float* y,
                          hipStream_t s, KTimer t) {
    dim3 grid((unsigned)((d + 4 * kThreads - 1) / (4 * kThreads)), (unsigned)T);
    return launch_timed(combine_kernel, grid, dim3(kThreads), 0, s, t.start, t.stop, w, d, k, P,
                        nsplit, y);
}

}  // namespace pw
