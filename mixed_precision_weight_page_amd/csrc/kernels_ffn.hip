// Expert FFN kernels for routed tokens (PagedWeight page, section "Dynamic
// Paging": the routed experts' pages are dequantized on the fly; Eq. 2 gives
// the dequantized weight s_e * q). SwiGLU: h = silu(W1 x) * (W3 x), o = W2 h.
//
// One workgroup = 64 rows of one routed expert (64 rpw rows when the down
// product walks row-block sequences), all of the expert's tokens, 16 per
// pass (64 for an expert with more than 16 tokens: wide passes); each of
// its four waves streams one 16-row block at a time, whose tiles (16 rows x
// 128 codes) are contiguous in the page, so every load instruction of a
// wave reads one contiguous run. One 4B-byte load per lane per tile
// (B = bits; a bitplane page: one 4-byte word per plane), prefetched
// several steps ahead; they are turned into exact
// fp16 integers q in registers (dequant.h: magic-exponent OR, then one
// packed fp16 subtract or multiply-add per pair) and multiplied on the
// matrix cores (v_mfma_f32_16x16x32_f16: 16 weight rows x 16 token columns,
// K = 32), accumulating in fp32. Token rows are staged once per K chunk in
// LDS as fp16, permuted so that each lane's 8 K-slots line up with the
// order in which its codes unpack. The per-expert scale is applied in the
// epilogue, so every product is exact and only fp32 accumulation rounds.
// Token rows enter as x 2^-e_t and the SwiGLU rows are stored as h 2^-m
// (exact powers of two, xscale.h), so any finite bf16 input and any h
// representable in fp32 fit the fp16 operands; the epilogues multiply the
// powers back.
//
// Batches of at most 16 tokens over at most 64 experts are grouped by the
// gate/up kernel itself (gate_up_own_route_kernel), which up to 4 tokens
// also routes them (no router launch).
//
// Why matrix cores for a memory-bound skinny product: with T_e tokens per
// expert a VALU dot product costs T_e/2 instructions per weight (packed
// dot2), which exceeds the VALU issue budget at HBM speed (about 2.5
// lane-instructions per 4-bit weight at 8 TB/s) as soon as T_e > 2. The
// MFMA does the multiply-adds for up to 16 tokens at once and leaves the
// VALU only the unpack (about 1.1 instructions per 4-bit weight).
#include <hip/hip_runtime.h>

#include <math.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <utility>

#include "dequant.h"
#include "pw_internal.h"
#include "route_dev.h"
#include "xscale.h"

namespace pw {
namespace {

using dq::half8_t;
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kCUs = 256;     // compute units of the GPU
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


// Stage K-chunk [k0, k0 + kc) of nt token rows into LDS as permuted fp16.
// MODE 0 reads bf16 activations of the tokens in tok[], each row scaled by
// its token's 2^-e; MODE 1 reads the (already scaled) fp16 SwiGLU rows of
// the pairs in prs[] from H.
// Loads per thread issued together before any is used: the row chunks of
// a batch are in flight at once (one round trip per batch, not per chunk).
template <int MODE, class C>
__host__ __device__ constexpr int stage_batch() { return C::kPermSpan == 32 ? 1 : (MODE == 0 ? 4 : 2); }

template <int MODE, class C>
__device__ __forceinline__ void stage(_Float16* xs, int stride, const FfnArgs& a,
                                      const int* tok, const int* prs, int nt, int k0, int kc, int tid) {
    constexpr int NBT = stage_batch<MODE, C>();
    if constexpr (C::kPermSpan == 32) {
        // the order permutes across all 32 codes of a run: 64 bytes (a
        // group) per thread and item
        const int ngrp = kc / 32;
        const int total = nt * ngrp;
        for (int base = tid; base < total; base += NBT * kThreads) {
            uint4 u[NBT][4];
            int ex[NBT];
#pragma unroll
            for (int j = 0; j < NBT; ++j) {
                const int idx = base + j * kThreads;
                if (idx < total) {
                    const int n = idx / ngrp, grp = idx - n * ngrp;
                    const uint4* src = MODE == 0
                        ? reinterpret_cast<const uint4*>(a.x + (int64_t)tok[n] * a.d + k0 + 32 * grp)
                        : reinterpret_cast<const uint4*>(a.w.H + (int64_t)prs[n] * a.F + k0 + 32 * grp);
#pragma unroll
                    for (int q = 0; q < 4; ++q) u[j][q] = src[q];
                    ex[j] = MODE == 0 ? a.w.xst[tok[n]].e : 0;
                }
            }
#pragma unroll
            for (int j = 0; j < NBT; ++j) {
                const int idx = base + j * kThreads;
                if (idx >= total) continue;
                const int n = idx / ngrp, grp = idx - n * ngrp;
                _Float16 v[32];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if constexpr (MODE == 0) {
                        const uint32_t ww[4] = {u[j][q].x, u[j][q].y, u[j][q].z, u[j][q].w};
#pragma unroll
                        for (int h = 0; h < 4; ++h) {
                            v[8 * q + 2 * h] = (_Float16)xsc::bf16_scaled((uint16_t)(ww[h] & 0xffffu), ex[j]);
                            v[8 * q + 2 * h + 1] = (_Float16)xsc::bf16_scaled((uint16_t)(ww[h] >> 16), ex[j]);
                        }
                    } else {
                        union {
                            uint4 u;
                            _Float16 h[8];
                        } t;
                        t.u = u[j][q];
#pragma unroll
                        for (int h = 0; h < 8; ++h) v[8 * q + h] = t.h[h];
                    }
                }
                union {
                    uint4 u[4];
                    _Float16 h[32];
                } o;
#pragma unroll
                for (int s = 0; s < 32; ++s) o.h[s] = v[C::perm(s)];
                uint4* dst = reinterpret_cast<uint4*>(xs + n * stride + 32 * grp);
#pragma unroll
                for (int q = 0; q < 4; ++q) dst[q] = o.u[q];
            }
        }
    } else {
        // 4- and 8-bit orders permute within groups of 8: one 16-byte chunk
        // of 8 activations per thread and item
        const int nch = kc / 8;
        const int total = nt * nch;
        for (int base = tid; base < total; base += NBT * kThreads) {
            uint4 u[NBT];
            int ex[NBT];
#pragma unroll
            for (int j = 0; j < NBT; ++j) {
                const int idx = base + j * kThreads;
                if (idx < total) {
                    const int n = idx / nch, ch = idx - n * nch;
                    u[j] = MODE == 0 ? *reinterpret_cast<const uint4*>(a.x + (int64_t)tok[n] * a.d + k0 + 8 * ch)
                                     : *reinterpret_cast<const uint4*>(a.w.H + (int64_t)prs[n] * a.F + k0 + 8 * ch);
                    ex[j] = MODE == 0 ? a.w.xst[tok[n]].e : 0;
                }
            }
#pragma unroll
            for (int j = 0; j < NBT; ++j) {
                const int idx = base + j * kThreads;
                if (idx >= total) continue;
                const int n = idx / nch, ch = idx - n * nch;
                _Float16 v[8];
                if constexpr (MODE == 0) {
                    const uint32_t ww[4] = {u[j].x, u[j].y, u[j].z, u[j].w};
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        v[2 * h] = (_Float16)xsc::bf16_scaled((uint16_t)(ww[h] & 0xffffu), ex[j]);
                        v[2 * h + 1] = (_Float16)xsc::bf16_scaled((uint16_t)(ww[h] >> 16), ex[j]);
                    }
                } else {
                    union {
                        uint4 u;
                        _Float16 h[8];
                    } t;
                    t.u = u[j];
#pragma unroll
                    for (int h = 0; h < 8; ++h) v[h] = t.h[h];
                }
                union {
                    uint4 u;
                    _Float16 h[8];
                } o;
#pragma unroll
                for (int s = 0; s < 8; ++s) o.h[s] = v[C::perm(s)];
                *reinterpret_cast<uint4*>(xs + n * stride + 8 * ch) = o.u;
            }
        }
    }
}

// Steps of codes in flight per wave: 8 x 16 B (4-bit), 8 x 12 B (3-bit),
// 4 x 32 B (8-bit) per matrix and lane.
template <int B>
__host__ __device__ constexpr int prefetch_depth() { return B == 8 ? 4 : 8; }

// The MFMAs of one 128-code step: for each matrix and each of the nblk
// (<= NB) blocks of 16 tokens, four K-groups; bp[nb] points at the step's
// 128 staged activations of this lane's token row of block nb and K-group.
// Each dequantized code fragment feeds every block.
template <int NB>
__device__ __forceinline__ void mma_blocks(const half8_t& af, const _Float16* const (&bp)[NB], int i,
                                           f32x4 (&acc)[NB], int nblk) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        if (NB == 1 || nb < nblk) {
            const half8_t bfr = *reinterpret_cast<const half8_t*>(bp[nb] + 8 * i);
            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bfr, acc[nb], 0, 0, 0);
        }
    }
}

template <int B, int NMAT, int NB>
__device__ __forceinline__ void step_mma(const Codes<B> (&cur)[NMAT], const _Float16* const (&bp)[NB],
                                         f32x4 (&acc)[NMAT][NB], int nblk, const dq::Const& dc) {
    if constexpr (B == 3) {
        half2_t pr[NMAT][16];
#pragma unroll
        for (int m = 0; m < NMAT; ++m) dq::pairs3(cur[m].w, pr[m], dc);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
                mma_blocks<NB>(dq::cat(pr[m][4 * i], pr[m][4 * i + 1], pr[m][4 * i + 2], pr[m][4 * i + 3]), bp, i,
                               acc[m], nblk);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int m = 0; m < NMAT; ++m) mma_blocks<NB>(dq::frag48<B>(cur[m].w, i, dc), bp, i, acc[m], nblk);
    }
}

// How the codes of a page reach the matrix cores. Eq2Codec<B>: Eq. 2 pages;
// a lane's 32-code run of a tile is 4B contiguous bytes. PlaneCodec<NP>:
// bitplane pages at depth NP (planes 0 .. NP-1 of the expert, W_e / 8 bytes
// apart; each plane of a 16 x 128 tile is 256 bytes, lane l = 16 g + r holding
// the bits of codes 32g .. 32g+31 of row r as one 32-bit word).
template <int B>
struct Eq2Codec {
    static constexpr int kWords = B;
    static constexpr int PD = prefetch_depth<B>();
    static constexpr int kStepBytes = 16 * kStep * B / 8;
    static constexpr int kPermSpan = B == 3 ? 32 : 8;
    static constexpr int kQmax = qmax_of(B);                       // largest |code| the MFMA sees
    __device__ static float eff_scale(float s) { return s; }        // weight = eff_scale(s) code
    __device__ static int lane_offset(int l) { return (B == 3 ? 12 : 16) * l; }
    __device__ static int64_t mat_bytes(int64_t M) { return M * B / 8; }
    using Src = const uint8_t*;
    __device__ static Src source(const uint8_t* base) { return base; }
    __device__ static Codes<B> load(Src p, int64_t off, int lane_off, int64_t) { return load_codes<B>(p + off + lane_off); }
    __host__ __device__ static constexpr int perm(int s) { return perm_slot<B>(s); }
    template <int NMAT, int NB>
    __device__ static void mma(const Codes<B> (&cur)[NMAT], const _Float16* const (&bp)[NB],
                               f32x4 (&acc)[NMAT][NB], int nblk, const dq::Const& dc) {
        step_mma<B, NMAT, NB>(cur, bp, acc, nblk, dc);
    }
};

// Bitplane decoding (the nested quantizer read from the PagedMoE page's
// abstract: a depth-NP weight is the centre of the node named by the first
// NP bits of Eq. 2's 8-bit code; twice its code is the integer
// c = (2p + 1) 2^(8-NP) - 257 for the prefix p, so the MFMA products stay
// exact and the epilogue scales by s8 / 2). The NP plane words of a step are
// transposed in groups of four with two rounds of masked block swaps (four
// words hold a 4 x 32 bit matrix; afterwards word i holds, in nibble g, the
// four plane bits of code i + 4 g), so every code's prefix bits sit in one
// nibble; then each pair of codes (at bit S = 0 or 4 of both 16-bit halves)
// becomes exact fp16 c with a magic-exponent OR, one subtract and one or two
// fma. Word i gives MFMA fragment i, K-slots 8i .. 8i+7 holding codes
// i, i+16, i+4, i+20, i+8, i+24, i+12, i+28.
__device__ __forceinline__ void transpose4(uint32_t& x0, uint32_t& x1, uint32_t& x2, uint32_t& x3) {
    uint32_t t = ((x0 >> 2) ^ x2) & 0x33333333u;
    x2 ^= t;
    x0 ^= t << 2;
    t = ((x1 >> 2) ^ x3) & 0x33333333u;
    x3 ^= t;
    x1 ^= t << 2;
    t = ((x0 >> 1) ^ x1) & 0x55555555u;
    x1 ^= t;
    x0 ^= t << 1;
    t = ((x2 >> 1) ^ x3) & 0x55555555u;
    x3 ^= t;
    x2 ^= t << 1;
}

// the nibbles at bit S of both halves of t, times 2^S, as fp16
template <int S>
__device__ __forceinline__ half2_t nibbles(uint32_t t, const dq::Const& c) {
    constexpr uint32_t mask = 0x000F000Fu << S;
    const half2_t k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
    return dq::as_half2((t & mask) | c.magic) - k1024;
}

template <int NP>
struct PlaneCodec {
    static constexpr int kWords = NP;
    static constexpr int PD = NP <= 4 ? 8 : (NP <= 6 ? 5 : 4);   // at most 64 plane words per lane in flight
    static constexpr int kStepBytes = 256;
    static constexpr int kPermSpan = 32;
    static constexpr int kQmax = 257;                               // |c| <= 257
    __device__ static float eff_scale(float s8) { return 0.5f * s8; }   // weight = s8 c / 2
    __device__ static int lane_offset(int l) { return 4 * l; }
    __device__ static int64_t mat_bytes(int64_t M) { return M / 8; }
    // A buffer descriptor over the wave's (uniform) stream base, in scalar
    // registers: each plane word is one non-temporal buffer load with the
    // lane's offset in a vector register and the plane's in a scalar one, so
    // the NP planes cost no per-plane address registers.
    struct Src {
        __amdgpu_buffer_rsrc_t r;
    };
    __device__ static Src source(const uint8_t* base) {
        const uint64_t a = reinterpret_cast<uint64_t>(base);
        const uint64_t u = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(a >> 32)) << 32) |
                           (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
        return Src{__builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(u), (short)0, 0x7fffffff, 0x00020000)};
    }
    __device__ static Codes<NP> load(const Src& p, int64_t off, int lane_off, int64_t plane) {
        Codes<NP> c;
#pragma unroll
        for (int j = 0; j < NP; ++j)
            c.w[j] = __builtin_amdgcn_raw_buffer_load_b32(p.r, lane_off, (int)(j * plane + off), 2 /* nt */);
        return c;
    }
    __host__ __device__ static constexpr int perm(int s) { return (s >> 3) + 4 * ((s >> 1) & 3) + 16 * (s & 1); }

    // fragment of word pair (hi: nibble of planes 0-3, or of all NP <= 4
    // planes; lo: planes 4-7, zero-padded)
    __device__ static half8_t frag(uint32_t hi, uint32_t lo, const dq::Const& dc) {
        constexpr float K = (float)((1 << (8 - NP)) - 257);
        const half2_t k2 = {(_Float16)K, (_Float16)K};
        half2_t p[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t th = (q & 2) ? hi >> 8 : hi;
            const uint32_t tl = (q & 2) ? lo >> 8 : lo;
            const half2_t h = (q & 1) ? nibbles<4>(th, dc) : nibbles<0>(th, dc);
            if constexpr (NP <= 4) {
                // c = p 2^(9-NP) + K
                const float m = (float)(1 << (9 - NP)) / ((q & 1) ? 16.0f : 1.0f);
                p[q] = __builtin_elementwise_fma(h, half2_t{(_Float16)m, (_Float16)m}, k2);
            } else {
                // c = 32 H + 2 L + K
                const half2_t l = (q & 1) ? nibbles<4>(tl, dc) : nibbles<0>(tl, dc);
                const float mh = (q & 1) ? 2.0f : 32.0f, ml = (q & 1) ? 0.125f : 2.0f;
                p[q] = __builtin_elementwise_fma(h, half2_t{(_Float16)mh, (_Float16)mh},
                                                 __builtin_elementwise_fma(l, half2_t{(_Float16)ml, (_Float16)ml}, k2));
            }
        }
        return dq::cat(p[0], p[1], p[2], p[3]);
    }

    template <int NMAT, int NB>
    __device__ static void mma(const Codes<NP> (&cur)[NMAT], const _Float16* const (&bp)[NB],
                               f32x4 (&acc)[NMAT][NB], int nblk, const dq::Const& dc) {
        uint32_t hi[NMAT][4], lo[NMAT][4];
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
            // row r of the high group is plane (min(NP, 4) - 1 - r); of the
            // low group plane 7 - r (zero past the depth)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int jh = (NP < 4 ? NP : 4) - 1 - r;
                hi[m][r] = jh >= 0 ? cur[m].w[jh < 0 ? 0 : jh] : 0u;
                const int jl = 7 - r;
                lo[m][r] = (NP > 4 && jl < NP) ? cur[m].w[jl < NP ? jl : 0] : 0u;
            }
            transpose4(hi[m][0], hi[m][1], hi[m][2], hi[m][3]);
            if constexpr (NP > 4) transpose4(lo[m][0], lo[m][1], lo[m][2], lo[m][3]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int m = 0; m < NMAT; ++m) mma_blocks<NB>(frag(hi[m][i], lo[m][i], dc), bp, i, acc[m], nblk);
    }
};

// MODE 0: gate/up + SwiGLU (NMAT = 2: W1, W3); MODE 1: down (NMAT = 1: W2),
// over K-steps [ks0, ks0 + nsteps) (the down product may be split along K
// across workgroups; split `sp` writes its own partial output).
// The workgroup covers rows [64 rpw rt, 64 rpw (rt + 1)) of expert e; wave
// w owns rpw consecutive 16-row blocks of them. Codes are prefetched PD
// steps ahead in a register ring; the main loop issues a load for every step
// (the last steps' loads repeat the last tile), so the ring stays full, and
// LDS chunks of the token rows are staged before the first load when K fits.
// The expert's page-table entry, pair count and pair list, read by the
// kernel in one round of independent loads before its first code load
// (with the first 16 entries of the list: p0 is this thread's).
struct ExpertRef {
    const uint8_t* page;
    float s;
    int Te;
    const int32_t* list;
    int p0;
    int tb0 = 0;     // first token of the workgroup's passes
    int tstep = 0;   // tokens between its passes (0: one pass after another)
};

// NB: blocks of 16 tokens per pass over the codes (1, or 4 for the experts
// that receive more than 16 tokens, whose passes prefetch two steps, the
// most of 64 token rows the LDS holds).
// SEQ: 0, one 16-row block per wave (rpw = 1); 1, rpw row blocks of 16 per
// wave (the down product's NB = 1 passes, picked when the LDS holds every
// step of the pass's token rows), walked as one sequence of steps so that
// the prefetch ring runs on across block boundaries; a block's output is
// written right after its last step. (A compile-time choice: the sequence's
// per-step bookkeeping costs the single-block case about 4%. Gate/up
// sequences, their sums kept in LDS until after the loop, ran 10% slower on
// the 128-expert decode layer: one round of longer workgroups, all starting
// at once, against two rounds that overlap.)
template <int MODE, class C, int NB, int SEQ>
__device__ __forceinline__ void ffn_tile(const FfnArgs& a, int lds_bytes, const ExpertRef& ex, int rt, int sp,
                                         int ks0, int nsteps, int rpw, _Float16* xs, int* tok, int* prs) {
    constexpr int NMAT = MODE == 0 ? 2 : 1;
    constexpr int PD = NB == 1 ? C::PD : 2;   // a wide pass stages two steps of its rows at a time
    constexpr int SB = C::kStepBytes;   // bytes of one tile (of one plane): 16 rows x 128 codes
    constexpr int NW = C::kWords;
    const int K = MODE == 0 ? a.d : a.F;
    const int KS = K / kStep;   // tiles of one 16-row block in a matrix
    const int64_t mat_bytes = C::mat_bytes((int64_t)a.F * a.d);
    const int64_t plane = 3 * (int64_t)a.F * a.d / 8;   // bitplane pages: bytes per plane
    const uint8_t* page = ex.page;
    const float s = C::eff_scale(ex.s);
    const int Te = ex.Te;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int r = lane & 15, g = lane >> 4;
    static_assert(SEQ == 0 || (MODE == 1 && NB == 1), "row-block sequences: the down product's NB = 1 passes");
    constexpr bool kSeq = SEQ != 0;   // several row blocks per wave
    const int R = kSeq ? rpw : 1;
    const int total = R * nsteps;   // steps of the wave's sequence
    const int row0 = (rt * 4 + wave) * R * 16;
    const dq::Const dc = dq::make_const();
    // this wave's 16-row blocks are consecutive runs of K/128 tiles: a
    // wave-uniform base per matrix, plus the lane's offset
    typename C::Src ap[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
        ap[m] = C::source(page + (MODE == 0 ? m : 2) * mat_bytes + ((int64_t)(row0 / 16) * KS + ks0) * SB);
    const int loff = C::lane_offset(lane);

    const int tstep = ex.tstep ? ex.tstep : 16 * NB;
    for (int tb = ex.tb0; tb < Te; tb += tstep) {
        const int nt = min(16 * NB, Te - tb);
        const int nblk = (nt + 15) >> 4;
        // steps per LDS chunk: all of them if nt rows fit, else a multiple of
        // PD (the host sizes the LDS for at least PD steps of 16 rows)
        int spc = nsteps;
        if (nt * (nsteps * kStep + 8) * 2 > lds_bytes)
            spc = ((lds_bytes / (2 * nt) - 8) / (kStep * PD)) * PD;
        const int stride = spc * kStep + 8;
        // the load cursor: sequence index, step within its block and tile
        // index of the next code load (it stays on the last step once there:
        // the ring's loads past the end are never used, and a conditional
        // load would make the ring slot's old value need a copy while it is
        // still being consumed)
        int lf = 0, ls = 0, la = 0;
        auto load_step = [&](Codes<NW> (&dst)[NMAT]) {
            if constexpr (kSeq) {
#pragma unroll
                for (int m = 0; m < NMAT; ++m) dst[m] = C::load(ap[m], (int64_t)la * SB, loff, plane);
                const int adv = lf < total - 1 ? 1 : 0;
                lf += adv;
                la += adv;
                ls += adv;
                const bool wrap = ls == nsteps;
                la += wrap ? KS - nsteps : 0;
                ls = wrap ? 0 : ls;
            } else {
                // one row block: the tile index is the sequence index
#pragma unroll
                for (int m = 0; m < NMAT; ++m) dst[m] = C::load(ap[m], (int64_t)min(lf, total - 1) * SB, loff, plane);
                ++lf;
            }
        };
        // the first PD steps of codes: the down product issues them before
        // its token rows are staged (their round trips overlap), gate/up
        // after (its token-id and token-row loads, which the first step
        // waits for, are then not queued behind the codes): measured best
        // for each
        Codes<NW> buf[PD][NMAT];
        auto issue_codes = [&]() {
#pragma unroll
            for (int j = 0; j < PD; ++j) load_step(buf[j]);
        };
        if constexpr (MODE == 1) issue_codes();
        // this pass's pairs (the first 16 came with the expert's entry)
        const int p = (tb == 0 && tid < 16) ? ex.p0 : (tid < nt ? ex.list[tb + tid] : 0);
        __syncthreads();   // previous token block done with tok, prs and xs
        if (tid < nt) {
            prs[tid] = p;
            tok[tid] = p / a.k;
        }
        __syncthreads();
        // this lane's pair in each block (its row of H, or of O for the
        // down product)
        int my_pair[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) my_pair[nb] = prs[min(16 * nb + r, nt - 1)];
        stage<MODE, C>(xs, stride, a, tok, prs, nt, ks0 * kStep, min(spc, nsteps) * kStep, tid);
        // the statistics of this lane's tokens, for the epilogue (issued
        // after the staging loads, which the barrier below waits for)
        XStat my_xs[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) my_xs[nb] = a.w.xst[my_pair[nb] / a.k];
        if constexpr (MODE == 0) issue_codes();
        __syncthreads();
        f32x4 acc[NMAT][NB];
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[m][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        // B-fragment row of this lane's token in each block (columns past nt
        // repeat a real row)
        const _Float16* bp0[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) bp0[nb] = xs + min(16 * nb + r, nt - 1) * stride + 32 * g;
        // the output of row block i, from the accumulators
        // D layout: lane (n = lane % 16, g = lane / 16) holds rows 4g..4g+3, token n
        auto write_out = [&](int i) {
            const int orow = row0 + 16 * i + 4 * g;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                if (16 * nb + r >= nt) continue;
                if constexpr (MODE == 0) {
                    union {
                        uint2 u;
                        _Float16 h[4];
                    } hv;
                    const xsc::GateUpScale gs = xsc::gate_up_scale(s, C::kQmax, my_xs[nb]);
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        hv.h[v] = (_Float16)xsc::swiglu_scaled(acc[0][nb][v], acc[1][nb][v], gs);
                    *reinterpret_cast<uint2*>(a.w.H + (int64_t)my_pair[nb] * a.F + orow) = hv.u;
                } else {
                    const int m = xsc::h_exponent(s, C::kQmax, my_xs[nb]);
                    float4 o;
                    o.x = ldexpf(s * acc[0][nb][0], m);
                    o.y = ldexpf(s * acc[0][nb][1], m);
                    o.z = ldexpf(s * acc[0][nb][2], m);
                    o.w = ldexpf(s * acc[0][nb][3], m);
                    *reinterpret_cast<float4*>(a.w.O + ((int64_t)sp * a.P + my_pair[nb]) * a.d + orow) = o;
                }
            }
        };
        // the compute cursor: step within its row block, the block, and the
        // step's offset in the staged chunk (without row-block sequences a
        // group's steps sit at fixed offsets from the group's: immediate
        // offsets of its LDS reads)
        int cs = 0, ci = 0, cbo = 0;
        auto compute_step = [&](const Codes<NW> (&cur)[NMAT], int j) {
            const int off = kSeq ? cbo : cbo + j * kStep;
            const _Float16* bq[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) bq[nb] = bp0[nb] + off;
            C::template mma<NMAT, NB>(cur, bq, acc, nblk, dc);
            if constexpr (kSeq) {
                if (cs == nsteps - 1) {
                    write_out(ci);
                    acc[0][0] = f32x4{0.f, 0.f, 0.f, 0.f};
                    ++ci;
                    cs = 0;
                    cbo = 0;
                } else {
                    ++cs;
                    cbo += kStep;
                    if (cbo == spc * kStep) cbo = 0;   // next LDS chunk (one row block)
                }
            }
        };
        // after a group of PD steps, in a single row block
        auto next_group = [&]() {
            if constexpr (!kSeq) {
                cs += PD;
                cbo += PD * kStep;
                if (cbo == spc * kStep) cbo = 0;
            }
        };
        // a new LDS chunk of the token rows at a group's start (rpw is 1 when
        // K is staged in chunks, and chunks hold whole groups)
        auto restage = [&](int f0) {
            if (spc < nsteps && f0 != 0 && cbo == 0) {
                __syncthreads();
                stage<MODE, C>(xs, stride, a, tok, prs, nt, (ks0 + cs) * kStep, min(spc, nsteps - cs) * kStep, tid);
                __syncthreads();
            }
        };
        int f0 = 0;
        for (; total - f0 > PD; f0 += PD) {
            restage(f0);
            // each slot's codes are consumed before its next load is issued
            // into the same registers (a load issued first would need
            // registers of its own, and the ring copied between them, after
            // a wait for every load in flight, at the loop's end)
#pragma unroll
            for (int j = 0; j < PD; ++j) {
                compute_step(buf[j], j);
                load_step(buf[j]);
            }
            next_group();
        }
        // the final group issues no loads
        restage(f0);
#pragma unroll
        for (int j = 0; j < PD; ++j)
            if (f0 + j < total) compute_step(buf[j], j);
        if constexpr (!kSeq) write_out(0);
    }
}

// One workgroup's share of an expert: row tile rt, K split sp. PLANES:
// bitplane pages (a kernel of its own, so that the Eq. 2 kernel's register
// allocation does not depend on the bitplane decoding).
template <int MODE, bool PLANES, int NB, int SEQ>
__device__ __forceinline__ void ffn_width(const FfnArgs& a, int lds_bytes, int nsplit, int rpw, const ExpertRef& ex,
                                          int b, int rt, int sp, _Float16* xs, int* tok, int* prs) {
    const int total = (MODE == 0 ? a.d : a.F) / kStep;
    const int nsteps = total / nsplit;
    if constexpr (PLANES) {
        // bitplane pages: b is the depth, 1 .. 8 planes
        switch (b) {
            case 1: ffn_tile<MODE, PlaneCodec<1>, NB, SEQ>(a, lds_bytes, ex, rt, sp, sp * nsteps, nsteps, rpw, xs, tok, prs); break;
            case 2: ffn_tile<MODE, PlaneCodec<2>, NB, SEQ>(a, lds_bytes, ex, rt, sp, sp * nsteps, nsteps, rpw, xs, tok, prs); break;
            case 3: ffn_tile<MODE, PlaneCodec<3>, NB, SEQ>(a, lds_bytes, ex, rt, sp, sp * nsteps, nsteps, rpw, xs, tok, prs); break;
            case 4: ffn_tile<MODE, PlaneCodec<4>, NB, SEQ>(a, lds_bytes, ex, rt, sp, sp * nsteps, nsteps, rpw, xs, tok, prs); break;
            case 5: ffn_tile<MODE, PlaneCodec<5>, NB, SEQ>(a, lds_bytes, ex, rt, sp, sp * nsteps, nsteps, rpw, xs, tok, prs); break;
            case 6: ffn_tile<MODE, PlaneCodec<6>, NB, SEQ>(a, lds_bytes, ex, rt, sp, sp * nsteps, nsteps, rpw, xs, tok, prs); break;
            case 7: ffn_tile<MODE, PlaneCodec<7>, NB, SEQ>(a, lds_bytes, ex, rt, sp, sp * nsteps, nsteps, rpw, xs, tok, prs); break;
            default: ffn_tile<MODE, PlaneCodec<8>, NB, SEQ>(a, lds_bytes, ex, rt, sp, sp * nsteps, nsteps, rpw, xs, tok, prs); break;
        }
    } else {
        if (b == 4) ffn_tile<MODE, Eq2Codec<4>, NB, SEQ>(a, lds_bytes, ex, rt, sp, sp * nsteps, nsteps, rpw, xs, tok, prs);
        else if (b == 8) ffn_tile<MODE, Eq2Codec<8>, NB, SEQ>(a, lds_bytes, ex, rt, sp, sp * nsteps, nsteps, rpw, xs, tok, prs);
        else ffn_tile<MODE, Eq2Codec<3>, NB, SEQ>(a, lds_bytes, ex, rt, sp, sp * nsteps, nsteps, rpw, xs, tok, prs);
    }
}

template <int MODE, bool PLANES, int NB, int SEQ>
__device__ __forceinline__ void ffn_role(const FfnArgs& a, int lds_bytes, int nsplit, int rpw, int e, int rem,
                                         _Float16* xs, int* tok, int* prs, int tb0 = 0, int tstep = 0) {
    const DecodeGroup& dg = a.w.dg;
    const int rt = rem / nsplit, sp = rem - rt * nsplit;
    const int32_t* list = dg.list + (int64_t)e * a.w.tcap;
    const int b = a.tab.bits[e];
    const ExpertRef ex{a.pool + a.tab.off[e], a.tab.scale[e], dg.cnt[e], list, list[threadIdx.x & 15], tb0, tstep};
    ffn_width<MODE, PLANES, NB, SEQ>(a, lds_bytes, nsplit, rpw, ex, b, rt, sp, xs, tok, prs);
}

// Experts that receive more than 16 tokens are served by wide passes,
// kWideNB blocks of 16 tokens per pass over their codes: every code is read
// once per 16 kWideNB tokens instead of once per 16. Both kinds share the
// launch's LDS; a wide pass holds its token rows two steps at a time.
constexpr int kWideNB = 4;

// Experts with more than 16 tokens ("hot") among the routed ones, found by
// one wave scanning the m routed slots in order with ballots; every lane
// gets the same answer.
// hot_expert: the h-th hot expert (0-based), or -1 if there are fewer.
__device__ __forceinline__ int hot_expert(const DecodeGroup& dg, int m, int h) {
    const int lane = threadIdx.x & 63;
    const int nf = dg.n_act[0], nb = dg.n_act[1];
    int seen = 0;
    for (int base = 0; base < m; base += 64) {
        const int idx = base + lane;
        const int e = idx < m ? slot_expert(dg, m, idx, nf, nb) : -1;
        const bool hot = e >= 0 && dg.cnt[e] > 16;
        const uint64_t m = __ballot(hot);
        const int c = __popcll(m);
        if (seen + c > h) {
            // the (h - seen)-th set bit of m
            uint64_t mm = m;
            for (int i = 0; i < h - seen; ++i) mm &= mm - 1;
            return __shfl(e, __ffsll((unsigned long long)mm) - 1);
        }
        seen += c;
    }
    return -1;
}

// hot_rank: how many hot experts come before routed slot ai.
__device__ __forceinline__ int hot_rank(const DecodeGroup& dg, int m, int nf, int nb, int ai) {
    const int lane = threadIdx.x & 63;
    int seen = 0;
    for (int base = 0; base < ai; base += 64) {
        const int idx = base + lane;
        const int e = idx < ai ? slot_expert(dg, m, idx, nf, nb) : -1;
        const bool hot = e >= 0 && dg.cnt[e] > 16;
        seen += __popcll(__ballot(hot));
    }
    return seen;
}

// Hot experts whose tiles beyond the routed slot's own get workgroups of
// their own when a workgroup covers several row tiles.
constexpr int kHotExtra = 16;

// Gate/up: the first kHotSplit hot experts have each 64-row tile served by
// kHotShares workgroups, share j taking the passes of 16 tokens that start
// at 16 j, 16 (j + kHotShares), ... (one wide pass of 64 tokens costs about
// three passes of 16 on one workgroup, so a hot expert's tiles would
// otherwise outlast the rest of the launch). Each share streams the tile's
// codes; the extra shares of one tile sit 8 workgroups apart, so that they
// run on one XCD and its L2 serves the repeated reads.
constexpr int kHotSplit = 16;
constexpr int kHotShares = 4;

// extra workgroup i -> (unit u = hot expert h x row tiles + tile, share j
// in 1 .. kHotShares - 1); u past the units launched: none
__device__ __forceinline__ void split_unit(int i, int& u, int& j) {
    constexpr int G = 8 * (kHotShares - 1);
    const int q = i / G, r = i - q * G;
    j = 1 + r / 8;
    u = q * 8 + (r & 7);
}

// grid: `extra` workgroups for hot experts (gate/up: the token shares of
// the first kHotSplit; down: tiles beyond the routed workgroups' own), then
// (routed expert slot, 64 rpw-row tile, K split) flattened; slots past the
// device-side routed count exit at once. The slot's expert comes from the
// router's list (with bitplane pages the deeper experts first, so the
// longest workgroups are dispatched first); its page-table entry, pair count
// and first 16 pairs are then read in one round of independent loads (the
// pair list has room for at least 16 entries). wide (set when the batch has
// more than 16 tokens): an expert may be hot. Gate/up: the tiles of the
// first kHotSplit hot experts are shared by token passes as above, those of
// later hot experts take wide passes. Down: a hot expert's 64-row tiles take
// wide passes, one tile per workgroup. With rpw = 1 that is its routed
// workgroups; with rpw > 1 its routed workgroups take its first tiles/rpw
// tiles and, for the first kHotExtra hot experts, the extra workgroups the
// rest; a later hot expert keeps the passes of 16 tokens over its
// workgroups' rpw-tile sequences.
template <int MODE, bool PLANES, int SEQ>
__global__ __launch_bounds__(kThreads, MODE == 0 ? 3 : 4) void ffn_kernel(FfnArgs a, int lds_bytes, int tiles,
                                                                          int nsplit, int rpw, int extra) {
    extern __shared__ __attribute__((aligned(16))) _Float16 xs[];
    __shared__ int tok[16 * kWideNB];   // token of each pair of the current pass
    __shared__ int prs[16 * kWideNB];   // the pairs t k + j of the current pass
    const DecodeGroup& dg = a.w.dg;
    const int own = tiles / rpw;   // 64-row tiles of a hot expert its routed workgroups take
    // the workgroup's expert, share of it (row tile and K split), token
    // passes and pass width; one call site per width
    int e, rem, tb0 = 0, tstep = 0;
    bool wide = false;
    if (MODE == 0 && (int)blockIdx.x < extra) {
        int u, j;
        split_unit(blockIdx.x, u, j);
        const int h = u / (tiles * nsplit);
        if (h >= kHotSplit) return;
        // the same on every lane: kept in a scalar register
        e = __builtin_amdgcn_readfirstlane(hot_expert(dg, a.max_act, h));
        if (e < 0) return;
        rem = u - h * tiles * nsplit;
        tb0 = 16 * j;
        tstep = 16 * kHotShares;
    } else if ((int)blockIdx.x < extra) {
        const int per = (tiles - own) * nsplit;
        const int h = blockIdx.x / per;
        e = hot_expert(dg, a.max_act, h);
        if (e < 0) return;
        rem = own * nsplit + (blockIdx.x - h * per);
        wide = true;
    } else {
        const int blk = blockIdx.x - extra;
        const int per_expert = own * nsplit;
        const int ai = blk / per_expert;
        // the counts and both candidates of the slot in one round of loads
        const int nf = dg.n_act[0], nb = dg.n_act[1];
        e = slot_expert(ai, a.max_act, nf, nb, dg.act[ai], dg.act[dg.E - a.max_act + ai]);
        if (e < 0) return;
        rem = blk - ai * per_expert;
        if (a.wide && dg.cnt[e] > 16) {
            if constexpr (MODE == 0) {
                if (hot_rank(dg, a.max_act, nf, nb, ai) < kHotSplit) tstep = 16 * kHotShares;
                else wide = true;
            } else {
                wide = rpw == 1 || hot_rank(dg, a.max_act, nf, nb, ai) < kHotExtra;
            }
        }
    }
    if (wide)
        ffn_role<MODE, PLANES, kWideNB, 0>(a, lds_bytes, nsplit, 1, e, rem, xs, tok, prs);
    else
        ffn_role<MODE, PLANES, 1, SEQ>(a, lds_bytes, nsplit, rpw, e, rem, xs, tok, prs, tb0, tstep);
}

// Small batches skip the routed-list round trip. Up to kOwnRouteTokens
// tokens (at most kOwnRouteExperts experts, top-kOwnRouteTopK) there is no
// router launch: every gate/up workgroup routes the whole batch itself (a
// row of 16 lanes per token, the router's top-k and weights, route_dev.h)
// and takes every token's statistics (a wave per token, its loads in flight
// with the logits'). Up to kOwnGroupTokens tokens the router only routes
// (ids, weights, statistics, no grouping atomics) and every gate/up
// workgroup groups the pairs of its ids itself. Either way the workgroup
// orders the routed experts by class, then id (Eq. 2 pages: those of at
// most 4 bits first; bitplane pages: those deeper than 4 planes first, as
// the router orders them), serves the ai-th, and keeps its pairs (in pair
// order) in LDS: its page-table entry, token ids and token rows then come in
// one round of loads. What the later kernels read is written by the
// workgroups that own it: row tile 0 of each expert its list (and, routing
// itself, its pairs' ids and weights); the first workgroup every expert's
// count and the routed list (and the tokens' statistics), and it clears the
// next forward's counters, as the router does. Every workgroup derives the
// same grouping from the same logits or ids, so they agree on the order.
constexpr int kOwnRouteTokens = 4;
constexpr int kOwnGroupTokens = 16;
constexpr int kOwnRouteExperts = 64;
constexpr int kOwnRouteTopK = 16;
static_assert(kOwnRouteTokens <= kThreads / 64, "a wave per token for the statistics");
static_assert(kOwnGroupTokens * kOwnRouteTopK <= kThreads, "a thread per pair");

template <int PER>
__device__ __forceinline__ rdev::RowChoice own_topk(const FfnArgs& a, int t, bool valid, XStat* s_xst) {
    const int l16 = threadIdx.x & 15;
    const float* row = a.logits + (int64_t)t * a.E;
    float v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = l16 + 16 * i;
        v[i] = (valid && e < a.E) ? row[e] : -INFINITY;
    }
    // wave w takes token w's statistics meanwhile
    const int wave = threadIdx.x >> 6;
    if (wave < a.T) {
        const XStat st = rdev::lanes_stat<64>(a.x + (int64_t)wave * a.d, a.d);
        if ((threadIdx.x & 63) == 0) s_xst[wave] = st;
    }
    return rdev::row_topk<PER>(v, a.E, a.k, a.renorm, valid);
}

__device__ __forceinline__ int lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// grid: (routed expert in class and id order, 64-row tile); positions past
// the routed count exit once the grouping is known. ROUTE: route the batch
// (else group the router's ids).
template <bool PLANES, bool ROUTE>
__global__ __launch_bounds__(kThreads, 3) void gate_up_own_route_kernel(FfnArgs a, int lds_bytes, int tiles) {
    extern __shared__ __attribute__((aligned(16))) _Float16 xs[];
    __shared__ int tok[16 * kWideNB];
    __shared__ int prs[16 * kWideNB];
    __shared__ int s_ids[kOwnGroupTokens * kOwnRouteTopK];   // expert of each pair
    __shared__ int s_cnt[kOwnRouteExperts];                   // pairs per expert
    __shared__ int s_list[kOwnGroupTokens];                   // this expert's pairs (Te <= T)
    __shared__ int s_wcnt[kThreads / 64];
    __shared__ XStat s_xst[kOwnRouteTokens];                  // by token (routing here)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ai = blockIdx.x / tiles, rt = blockIdx.x - ai * tiles;
    const int my_bits = lane < a.E ? a.tab.bits[lane] : 0;   // the class of expert `lane`
    const int P = a.T * a.k;
    if (tid < kOwnRouteExperts) s_cnt[tid] = 0;
    // pair p of this thread and its expert: routing here, token t = tid / 16
    // by its row of lanes, lane l16 < k holding choice l16; else pair tid
    rdev::RowChoice c{0, 0, 0.0f, 0.0f};
    int p = tid, pe = 0;
    bool chosen;
    if constexpr (ROUTE) {
        const int t = tid >> 4, l16 = tid & 15;
        const bool valid = t < a.T;
        const int tc = valid ? t : 0;
        if (a.E <= 16) c = own_topk<1>(a, tc, valid, s_xst);
        else if (a.E <= 32) c = own_topk<2>(a, tc, valid, s_xst);
        else c = own_topk<4>(a, tc, valid, s_xst);
        chosen = valid && l16 < a.k;
        p = t * a.k + l16;
        pe = c.id0;
    } else {
        chosen = tid < P;
        if (chosen) pe = a.w.ids[tid];
    }
    __syncthreads();   // s_cnt cleared
    if (chosen) {
        s_ids[p] = pe;
        atomicAdd(&s_cnt[pe], 1);
    }
    __syncthreads();
    // the routed experts by class, then id (every wave finds the same);
    // this workgroup's expert is the ai-th
    const bool act = lane < a.E && s_cnt[lane] > 0;
    const bool first = (my_bits > 4) == (a.bitplane != 0);
    const uint64_t m0 = __ballot(act && first), m1 = __ballot(act && !first);
    const int n0 = __popcll(m0), n_act = n0 + __popcll(m1);
    if (ai >= n_act) return;
    const int arank = (act && first) ? lanes_below(m0) : n0 + lanes_below(m1);
    const int e = __ffsll((unsigned long long)__ballot(act && arank == ai)) - 1;
    // its pairs in pair order (at most one per token)
    const int Te = s_cnt[e];
    const bool mine = tid < P && s_ids[tid] == e;
    const uint64_t mm = __ballot(mine);
    if (lane == 0) s_wcnt[wave] = __popcll(mm);
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += s_wcnt[w];
    if (mine) s_list[base + lanes_below(mm)] = tid;
    if (rt == 0) {
        if (ROUTE && chosen && pe == e) {
            a.w.ids[p] = e;
            a.w.g[p] = c.g0;
        }
        if (ai == 0) {
            if (ROUTE && tid < a.T) a.w.xst[tid] = s_xst[tid];
            if (tid < a.E) {
                a.w.dg.cnt[tid] = s_cnt[tid];
                a.w.dg_next.cnt[tid] = 0;
            }
            if (tid < 64 && act) a.w.dg.act[arank] = lane;
            if (tid < 2) {
                a.w.dg.n_act[tid] = tid == 0 ? n_act : 0;
                a.w.dg_next.n_act[tid] = 0;
            }
        }
    }
    __syncthreads();   // s_list complete
    if (rt == 0 && tid < Te) a.w.dg.list[(int64_t)e * a.w.tcap + tid] = s_list[tid];
    FfnArgs b = a;
    if (ROUTE) b.w.xst = s_xst;
    const ExpertRef ex{a.pool + a.tab.off[e], a.tab.scale[e], Te, s_list, s_list[tid & 15]};
    ffn_width<0, PLANES, 1, 0>(b, lds_bytes, 1, 1, ex, a.tab.bits[e], rt, 0, xs, tok, prs);
}

// Resident workgroups of a kernel per CU at an LDS size, and the CU count
// (cached: the occupancy query is host arithmetic, but not free).
int resident_blocks(const void* kernel, size_t lds) {
    static std::mutex mu;
    static std::map<std::pair<const void*, size_t>, int> cache;
    std::lock_guard<std::mutex> lk(mu);
    auto it = cache.find({kernel, lds});
    if (it != cache.end()) return it->second;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kThreads, lds) != hipSuccess || n < 1) n = 1;
    cache[{kernel, lds}] = n;
    return n;
}

int cu_count() {
    static std::mutex mu;
    static std::map<int, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return kCUs;
    std::lock_guard<std::mutex> lk(mu);
    auto it = cache.find(dev);
    if (it != cache.end()) return it->second;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = kCUs;
    cache[dev] = n;
    return n;
}

template <int MODE, bool PLANES>
hipError_t launch_ffn_k(const FfnArgs& a, const FfnPlan& p, hipStream_t s, KTimer t) {
    const int rows = MODE == 0 ? a.F : a.d;
    const int tiles = rows / 64;
    // a wide pass stages 64 token rows of at least two steps (or of the
    // whole K range if shorter): 33,792 bytes at most
    size_t lds = p.lds;
    if (a.wide) {
        const int k = (MODE == 0 ? a.d : a.F) / p.nsplit;
        lds = std::max(lds, (size_t)16 * kWideNB * (std::min(k, 2 * kStep) + 8) * 2);
    }
    // rpw = 1: one row block per wave; rpw > 1 (the down product, when the
    // LDS holds all of K): the sequence variant. Among 1, 2, 4, 8 the one
    // whose grid (all max_act experts routed) fills its last round of
    // resident workgroups best, ties to the most rows per wave (fewer
    // workgroup start-ups for the same bytes)
    auto kernel_for = [](int r) { return r > 1 ? ffn_kernel<MODE, PLANES, MODE> : ffn_kernel<MODE, PLANES, 0>; };
    int rpw = 1;
    if (MODE == 1 && p.whole_k) {
        double best = -1.0;
        for (int r = 1; r <= 8; r *= 2) {
            if (tiles % r) break;
            const int64_t slots =
                (int64_t)resident_blocks(reinterpret_cast<const void*>(kernel_for(r)), lds) * cu_count();
            const int64_t blocks = (int64_t)a.max_act * (tiles / r) * p.nsplit;
            const int64_t rounds = (blocks + slots - 1) / slots;
            const double fill = (double)blocks / (double)(rounds * slots);
            if (fill >= best - 1e-9) {
                best = fill;
                rpw = r;
            }
        }
    }
    auto kernel = kernel_for(rpw);
    // gate/up: the hot experts' extra token shares, in whole groups of 8
    // units; down: the hot experts' tiles beyond their routed workgroups'
    const int units = kHotSplit * tiles * p.nsplit;
    const int extra = MODE == 0 ? (a.wide ? (units + 7) / 8 * 8 * (kHotShares - 1) : 0)
                                : ((a.wide && rpw > 1) ? kHotExtra * (tiles - tiles / rpw) * p.nsplit : 0);
    const dim3 grid((unsigned)((int64_t)a.max_act * (tiles / rpw) * p.nsplit + extra));
    return launch_timed(kernel, grid, dim3(kThreads), lds, s, t.start, t.stop, a, (int)lds, tiles, p.nsplit, rpw,
                        extra);
}

template <int MODE>
hipError_t launch_ffn(const FfnArgs& a, const FfnPlan& p, hipStream_t s, KTimer t) {
    if (MODE == 0 && a.own_route) {
        const int tiles = a.F / 64;
        const dim3 grid((unsigned)((int64_t)a.max_act * tiles));
        auto kernel = a.own_route == 1 ? (a.bitplane ? gate_up_own_route_kernel<true, true>
                                                     : gate_up_own_route_kernel<false, true>)
                                       : (a.bitplane ? gate_up_own_route_kernel<true, false>
                                                     : gate_up_own_route_kernel<false, false>);
        return launch_timed(kernel, grid, dim3(kThreads), p.lds, s, t.start, t.stop, a, (int)p.lds, tiles);
    }
    return a.bitplane ? launch_ffn_k<MODE, true>(a, p, s, t) : launch_ffn_k<MODE, false>(a, p, s, t);
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

int own_route_mode(int T, int E, int k) {
    if (E > kOwnRouteExperts || k > kOwnRouteTopK) return 0;
    return T <= kOwnRouteTokens ? 1 : (T <= kOwnGroupTokens ? 2 : 0);
}

// LDS for the staged token rows: all of the K range for up to min(T, 16)
// tokens if that fits 34 KB, else 34 KB (the kernel then stages K in chunks
// sized by the pass's actual token count; a wide pass of 64 tokens holds at
// least two steps: 64 x 264 halves fit).
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
    p.whole_k = full <= cap;
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
