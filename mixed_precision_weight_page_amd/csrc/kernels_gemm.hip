// Expert FFN for large batches (prefill): per active expert, a dense
// product of its T_e routed tokens with its dequantized weights on the
// matrix cores (PagedWeight page, section "Dynamic Paging": pages are
// dequantized on the fly; Eq. 2: W = s_e q). SwiGLU as in the decode path:
// h = silu(W1 x) * (W3 x) (MODE 0), o = W2 h (MODE 1).
//
// Workgroup tile: 64 tokens of one expert x 128 rows of W1 and of W3
// (MODE 0) or 256 rows of W2 (MODE 1); two workgroups per CU, so each SIMD
// interleaves two waves. Each of the four waves streams four 16-row blocks
// of the page's tiles straight from the page into registers (a two-step
// ring, each slot reloaded as soon as its last fragment is dequantized) and
// turns them into exact fp16 integers q in registers: no LDS for weights,
// each code read once per workgroup. The token rows (fp16, in the same
// per-32 K permutation as the codes unpack, prepared once per forward) go
// through double-buffered LDS one 128-code step at a time, one step ahead
// in registers; each lane's MFMA operand is one 16-byte LDS read, and the
// next K group's operands are read while the current ones are in use.
// Per step and wave: 4 K groups x 4 code streams x 4 token blocks of
// v_mfma_f32_16x16x32_f16, fp32 accumulate. Token rows are x 2^-e_t and
// the SwiGLU rows h 2^-m (exact powers of two, xscale.h), so every finite
// bf16 input and every h representable in fp32 fits the fp16 operands.
//
// Tile order: expert (in the active list, 8-bit first), row tile, token
// tile; with N tiles in this forward, workgroup b runs tile
// (b % 8) * ceil(N/8) + b / 8, so each XCD (which receives every eighth
// workgroup) walks one contiguous eighth: the workgroups resident on an XCD
// share weight tiles and token rows through its L2.
#include <hip/hip_runtime.h>

#include <math.h>

#include <algorithm>

#include "dequant.h"
#include "pw_internal.h"
#include "xscale.h"

namespace pw {
namespace {

using dq::half8_t;
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
// Weight rows per tile: 128 of W1 and of W3 (MODE 0), 256 of W2 (MODE 1).
// Either way a wave streams four 16-row blocks, so each token fragment read
// from LDS feeds four MFMAs.
template <int MODE>
constexpr int tile_rows() { return MODE == 0 ? 128 : 256; }
constexpr int BN = kGemmTokens;  // tokens per tile
// LDS row (floats) of the down tile's output staging: 256 rows + padding
// against bank conflicts; 32 tokens at a time
constexpr int kOutStride = 256 + 4;

template <int B>
struct Run {
    uint32_t w[B];   // 32 consecutive codes of one row, LSB-first
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// One 32-code run at p (lane offset applied): 16 bytes (4-bit), 16 + 16
// bytes 1 KB apart (8-bit), 12 bytes (3-bit). Plain loads: the workgroups of
// the expert's other token tiles read the same runs at about the same time,
// and those hits in L2 are what keeps the matrix cores fed.
template <int B>
__device__ __forceinline__ Run<B> load_run_at(const uint8_t* p) {
    Run<B> r;
    if constexpr (B == 4) {
        const u32x4 u = *reinterpret_cast<const u32x4*>(p);
        r.w[0] = u.x; r.w[1] = u.y; r.w[2] = u.z; r.w[3] = u.w;
    } else if constexpr (B == 8) {
        const u32x4 u = *reinterpret_cast<const u32x4*>(p);
        const u32x4 v = *reinterpret_cast<const u32x4*>(p + 1024);
        r.w[0] = u.x; r.w[1] = u.y; r.w[2] = u.z; r.w[3] = u.w;
        r.w[4] = v.x; r.w[5] = v.y; r.w[6] = v.z; r.w[7] = v.w;
    } else {
        const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
        r.w[0] = q[0];
        r.w[1] = q[1];
        r.w[2] = q[2];
    }
    return r;
}

using dq::perm_slot;

// K-slot that code c (within a 32-code run) takes in the K order of B-bit
// codes: the inverse of perm_slot.
template <int B>
__device__ __forceinline__ int slot_of(int c) {
    int slot = 0;
#pragma unroll
    for (int s = 0; s < 32; ++s)
        if (perm_slot<B>(s) == c) slot = s;
    return slot;
}

// 32 consecutive bf16 activations scaled by 2^-e (xscale.h) as fp16 in the
// K-slot order of B-bit codes.
template <int B>
__device__ __forceinline__ void permute32(const uint4 (&in)[4], uint4 out[4], int e) {
    _Float16 v[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t ww[4] = {in[q].x, in[q].y, in[q].z, in[q].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            v[8 * q + 2 * h] = (_Float16)xsc::bf16_scaled((uint16_t)(ww[h] & 0xffffu), e);
            v[8 * q + 2 * h + 1] = (_Float16)xsc::bf16_scaled((uint16_t)(ww[h] >> 16), e);
        }
    }
    union {
        uint4 u[4];
        _Float16 h[32];
    } o;
#pragma unroll
    for (int s = 0; s < 32; ++s) o.h[s] = v[perm_slot<B>(s)];
#pragma unroll
    for (int q = 0; q < 4; ++q) out[q] = o.u[q];
}

// 8 consecutive bf16 activations scaled by 2^-e as fp16 in the K-slot
// order of B-bit codes (B = 4 or 8: the order permutes within groups of 8).
template <int B>
__device__ __forceinline__ uint4 permute8(const uint4& in, int e) {
    static_assert(B == 4 || B == 8, "orders within groups of 8");
    const uint32_t ww[4] = {in.x, in.y, in.z, in.w};
    _Float16 v[8];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        v[2 * h] = (_Float16)xsc::bf16_scaled((uint16_t)(ww[h] & 0xffffu), e);
        v[2 * h + 1] = (_Float16)xsc::bf16_scaled((uint16_t)(ww[h] >> 16), e);
    }
    union {
        uint4 u;
        _Float16 h[8];
    } o;
#pragma unroll
    for (int s = 0; s < 8; ++s) o.h[s] = v[perm_slot<B>(s)];
    return o.u;
}

// Token rows for the gate/up tiles, once per forward. One wave per token:
// the token's statistics (xscale.h) into xst[t], then xp[i][t] = x[t] 2^-e
// as fp16 in the K order of the codes of bit-width kBits[i], for each
// bit-width some expert uses (bit i of mask). Up to 64 C 16-byte chunks
// (d_model up to 512 C) the wave reads the row once, lane l holding chunks
// l, l + 64, ... (each load and store instruction of the wave covers 1 KB
// of consecutive bytes), and writes the 4- and 8-bit orders from those
// registers; the 3-bit order, which permutes across 32 activations, reads
// its 64-byte groups again (from the cache). Longer rows: statistics, then
// every plane from a second read.
template <int C>
__global__ __launch_bounds__(kThreads) void prep_x_kernel(const uint16_t* x, int T, int d, int mask,
                                                          _Float16* xp, int64_t plane, XStat* xst) {
    const int t = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (t >= T) return;
    const int lane = threadIdx.x & 63;
    const uint16_t* row = x + (int64_t)t * d;
    const int64_t base = (int64_t)t * d;
    const int nch = d / 8;
    XStat st;
    if (nch <= 64 * C) {
        const uint4* src = reinterpret_cast<const uint4*>(row);
        uint4 in[C];
#pragma unroll
        for (int j = 0; j < C; ++j) {
            const int ch = lane + 64 * j;
            in[j] = ch < nch ? src[ch] : uint4{0u, 0u, 0u, 0u};
        }
        // max |x| and sum |x| (eight partial sums per lane, fp64; the zero
        // chunks past the row add nothing)
        uint32_t mx = 0;
        double part[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int j = 0; j < C; ++j) {
            const uint32_t ww[4] = {in[j].x, in[j].y, in[j].z, in[j].w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const uint32_t lo = ww[h] & 0x7fffu, hi = (ww[h] >> 16) & 0x7fffu;
                mx = max(mx, max(lo, hi));
                part[2 * h] += (double)__uint_as_float(lo << 16);
                part[2 * h + 1] += (double)__uint_as_float(hi << 16);
            }
        }
        double sum = ((part[0] + part[1]) + (part[2] + part[3])) + ((part[4] + part[5]) + (part[6] + part[7]));
        for (int o = 32; o > 0; o >>= 1) {
            mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
            sum += __shfl_xor(sum, o);
        }
        const int e = xsc::x_exponent(__uint_as_float(mx << 16));
        st = XStat{(float)ldexp(sum, -e), e};
#pragma unroll
        for (int i = 1; i < 3; ++i) {
            if (!((mask >> i) & 1)) continue;
            uint4* dst = reinterpret_cast<uint4*>(xp + i * plane + base);
#pragma unroll
            for (int j = 0; j < C; ++j) {
                const int ch = lane + 64 * j;
                if (ch < nch) dst[ch] = i == 1 ? permute8<4>(in[j], e) : permute8<8>(in[j], e);
            }
        }
        mask &= 1;   // the 3-bit order below, if in use
    } else {
        st = xsc::row_stat(row, d);
    }
    if (lane == 0) xst[t] = st;
    for (int grp = lane; grp < d / 32; grp += 64) {
        if (!mask) break;
        const uint4* src = reinterpret_cast<const uint4*>(row + 32 * grp);
        const uint4 in[4] = {src[0], src[1], src[2], src[3]};
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            if (!((mask >> i) & 1)) continue;
            uint4 o[4];
            if (i == 0) permute32<3>(in, o, st.e);
            else if (i == 1) permute32<4>(in, o, st.e);
            else permute32<8>(in, o, st.e);
            uint4* dst = reinterpret_cast<uint4*>(xp + i * plane + base + 32 * grp);
#pragma unroll
            for (int q = 0; q < 4; ++q) dst[q] = o[q];
        }
    }
}

constexpr int SK = 128;            // K codes per step (one page tile)
constexpr int LDX = SK;            // LDS row of staged tokens (halves): 256 B, no padding
// 16-byte chunk c of token row n lives at chunk position c ^ (c / 8 % 2) ^ f(n)
// of its row, f(n) = n % 16 with its two low bits swapped. Any 8 consecutive
// lanes then touch 8 different 16-byte bank groups of a 128-byte window (and
// any 16 lanes 16 groups of 256 bytes), both for the MFMA operand reads (one
// chunk of consecutive rows) and for the staging stores (two rows, chunks q,
// q + 4, q + 8, q + 12). A plain c ^ (n % 16) leaves chunks q and q + 8 of a
// row in the same group: the stores took two passes.
__device__ __forceinline__ int swz(int n, int c) {
    const int f = (n & 12) | ((n & 1) << 1) | ((n >> 1) & 1);
    return n * (LDX / 8) + (c ^ ((c >> 3) & 1) ^ f);
}

// Steps of codes in flight per wave.
template <int B>
__device__ __forceinline__ constexpr int gemm_depth() { return 2; }  // even

// Fragment i (K-slots 8i .. 8i + 7) of a run as exact fp16 q.
template <int B>
__device__ __forceinline__ half8_t frag_of(const Run<B>& r, int i, const dq::Const& c) {
    if constexpr (B == 3) {
        dq::half2_t p[16];
        dq::pairs3(r.w, p, c);   // the compiler keeps only fragment i's pairs
        return dq::cat(p[4 * i], p[4 * i + 1], p[4 * i + 2], p[4 * i + 3]);
    } else {
        return dq::frag48<B>(r.w, i, c);
    }
}

// Token rows of one step (already fp16 in the codes' K order): thread t
// copies chunks 4 (t % 4) .. +4 (32 codes) of token t / 4.
constexpr int XR = BN * SK * 2 / 16 / kThreads;   // 16-byte chunks per thread and step
static_assert(XR == 4, "staging assumes 4 chunks per thread");
__device__ __forceinline__ void load_act(u32x4 (&xr)[XR], const _Float16* act_row, int step, int tid) {
    const u32x4* src = reinterpret_cast<const u32x4*>(act_row + step * SK + 32 * (tid & 3));
#pragma unroll
    for (int q = 0; q < XR; ++q) xr[q] = src[q];
}

__device__ __forceinline__ void store_act(const u32x4 (&xr)[XR], _Float16* xs, int tid) {
    u32x4* dst = reinterpret_cast<u32x4*>(xs);
    const int n = tid >> 2;
#pragma unroll
    for (int q = 0; q < XR; ++q) dst[swz(n, 4 * (tid & 3) + q)] = xr[q];
}

// Scheduling groups for one step (64 MFMAs, 16 LDS reads, 16 fragments of
// dequantization): masks 0x8 MFMA, 0x2 VALU, 0x100 LDS read.
template <int B, int NA>
__device__ __forceinline__ void sched_step() {
    constexpr int kMfma = 16 * NA;                          // 4 K groups x 4 code streams x NA
    constexpr int kValuPerMfma = (B == 8 ? 8 : 12) / NA;    // the dequantization spread over them
    __builtin_amdgcn_sched_group_barrier(0x100, NA, 0);
    __builtin_amdgcn_sched_group_barrier(0x2, B == 8 ? 32 : 44, 0);
#pragma unroll
    for (int i = 0; i < kMfma; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x8, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x2, kValuPerMfma, 0);
        if (i % 4 == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
}

// Per-token scaling of the epilogue (xscale.h): the gate/up factors, or the
// exponent of the token's stored SwiGLU row for the down product.
struct TokScale {
    xsc::GateUpScale gu;
    int m;
};

template <int MODE, int B, int NA>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, int e, int Te, int base, int tt, int rt,
                                          _Float16* smem, int* tok, int* pair, TokScale* tsc) {
    constexpr int NMAT = 2;   // stream pairs: W1 / W3 (MODE 0), two 32-row halves of W2 (MODE 1)
    constexpr int PD = gemm_depth<B>();
    constexpr int TB = 256 * B;                  // bytes of one 16-row x 128-code tile
    const int K = MODE == 0 ? a.d : a.F;
    const int S = K / SK;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int t0 = tt * BN;
    const int nt = min(BN, Te - t0);
    const float s = a.tab.scale[e];
    const uint8_t* page = a.pool + a.tab.off[e];
    const int64_t mat_bytes = (int64_t)a.F * a.d * B / 8;
    const int loff = (B == 3 ? 12 : 16) * lane;
    // this wave's four code streams (m, blk), all K steps: row block
    // 8 rt + 2 wave + blk of matrix m (W1, W3), or row block
    // 16 rt + 4 wave + 2 m + blk of W2
    const uint8_t* ap[NMAT][2];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const int rb = MODE == 0 ? 8 * rt + 2 * wave + blk : 16 * rt + 4 * wave + 2 * m + blk;
            ap[m][blk] = page + (MODE == 0 ? m : 2) * mat_bytes + (int64_t)rb * S * TB + loff;
        }

    // the token statistics are loaded here and used after the loop
    XStat my_xs{0.0f, 0};
    if (tid < BN) {
        const int n = tid < nt ? tid : 0;   // past nt: repeat the first row, outputs dropped
        const int p = a.w.sorted[base + t0 + n];
        tok[tid] = MODE == 0 ? p / a.k : base + t0 + n;
        // the down product writes each token's rows of O at its pair index
        if constexpr (MODE == 1) pair[tid] = p;
        my_xs = a.w.xst[p / a.k];
    }
    __syncthreads();
    const int my_tok = tok[tid >> 2];
    const _Float16* act_row = MODE == 0 ? a.xp + (int64_t)bits_index(B) * a.xp_plane + (int64_t)my_tok * a.d
                                        : a.w.H + (int64_t)my_tok * a.F;
    _Float16* xs[2] = {smem, smem + BN * LDX};
    const dq::Const dc = dq::make_const();

    // prologue: codes for steps 0..PD-1 in flight, token rows of step 0 staged
    Run<B> ring[PD][NMAT][2];
#pragma unroll
    for (int j = 0; j < PD; ++j)
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
                ring[j][m][blk] = load_run_at<B>(ap[m][blk] + (int64_t)min(j, S - 1) * TB);
    // token rows travel one step ahead through registers
    u32x4 xr[XR];
    load_act(xr, act_row, 0, tid);
    store_act(xr, xs[0], tid);
    __syncthreads();

    f32x4 acc[NMAT][2][NA];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int j = 0; j < NA; ++j) acc[m][blk][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // one step: token rows of step st + 1 into registers; the MFMAs of step
    // st, with the token fragments of K-group kc + 1 read from LDS while
    // those of kc are in use, and the codes of ring slot j, reloaded with
    // step st + PD as soon as their last fragment is in registers (old and
    // new never live together, so the slot keeps its registers across the
    // loop and nothing waits on the load); then the token rows of step
    // st + 1 into the other LDS buffer
    auto step = [&](int st, auto& ring_j, const _Float16* cur, _Float16* nxt) {
        load_act(xr, act_row, min(st + 1, S - 1), tid);
        // keep the loads here: the scheduler would otherwise sink them to
        // their LDS stores at the end of the step and expose their latency
        __builtin_amdgcn_sched_barrier(0);
        // lane (r, g): its run holds codes 32g..32g+31 of the step and MFMA
        // kc uses codes 32g + 8kc..+8, so the token fragment is the same 8
        // K-slots of token row 16 jt + r
        const u32x4* xl = reinterpret_cast<const u32x4*>(cur);
        half8_t bq[2][NA];
#pragma unroll
        for (int jt = 0; jt < NA; ++jt) bq[0][jt] = __builtin_bit_cast(half8_t, xl[swz(16 * jt + r, 4 * g)]);
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            if (kc < 3) {
#pragma unroll
                for (int jt = 0; jt < NA; ++jt)
                    bq[(kc + 1) & 1][jt] = __builtin_bit_cast(half8_t, xl[swz(16 * jt + r, 4 * g + kc + 1)]);
            }
            half8_t af[NMAT][2];
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int blk = 0; blk < 2; ++blk) af[m][blk] = frag_of<B>(ring_j[m][blk], kc, dc);
            if (kc == 3) {
#pragma unroll
                for (int m = 0; m < NMAT; ++m)
#pragma unroll
                    for (int blk = 0; blk < 2; ++blk)
                        ring_j[m][blk] = load_run_at<B>(ap[m][blk] + (int64_t)min(st + PD, S - 1) * TB);
            }
#pragma unroll
            for (int jt = 0; jt < NA; ++jt)
#pragma unroll
                for (int m = 0; m < NMAT; ++m)
#pragma unroll
                    for (int blk = 0; blk < 2; ++blk)
                        acc[m][blk][jt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[m][blk], bq[kc & 1][jt],
                                                                                 acc[m][blk][jt], 0, 0, 0);
        }
        // issue order for the step: the first K group's token fragments and
        // codes, then each MFMA followed by a few VALU instructions (the next
        // groups' dequantization) and, every fourth MFMA, one LDS read
        sched_step<B, NA>();
        if (st + 1 < S) store_act(xr, nxt, tid);
        __syncthreads();
    };

    // whole ring cycles without guards (the prefetch stays in flight across
    // iterations), then the last S % PD steps; PD is even, so step s0 + j
    // reads LDS buffer j % 2
    int s0 = 0;
    for (; s0 + PD <= S; s0 += PD) {
#pragma unroll
        for (int j = 0; j < PD; ++j) step(s0 + j, ring[j], xs[j & 1], xs[(j + 1) & 1]);
    }
#pragma unroll
    for (int j = 0; j < PD; ++j)
        if (s0 + j < S) step(s0 + j, ring[j], xs[j & 1], xs[(j + 1) & 1]);
    // epilogue: lane (n = lane % 16, g) holds rows 4g..4g+3 of each 16 x 16 tile
    if (tid < BN) {
        if constexpr (MODE == 0) tsc[tid].gu = xsc::gate_up_scale(s, qmax_of(B), my_xs);
        else tsc[tid].m = xsc::h_exponent(s, qmax_of(B), my_xs);
    }
    if constexpr (MODE == 0) {
        // SwiGLU rows h = silu(s W1 x) * (s W3 x) of the tile's 64 tokens x
        // 128 rows go through LDS (the token buffers are free after the last
        // step's barrier), already at the K-slots the down projection's
        // B-bit codes expect, then to H in coalesced 16-byte chunks. silu with
        // the native base-2 exponential and reciprocal; h is stored as fp16
        // scaled by the token's 2^-m (xscale.h).
        constexpr int HS = tile_rows<0>() + 8;   // LDS row (halves), padded against bank conflicts
        _Float16* hs = smem;
        __syncthreads();   // the token scales are in LDS
#pragma unroll
        for (int jt = 0; jt < NA; ++jt) {
            const int n = 16 * jt + r;
            const xsc::GateUpScale gs = tsc[n].gu;
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float h = xsc::swiglu_scaled_fast(acc[0][blk][jt][v], acc[1][blk][jt][v], gs);
                    hs[n * HS + 32 * wave + slot_of<B>(16 * blk + 4 * g + v)] = (_Float16)h;
                }
        }
        __syncthreads();
        const int col0 = rt * tile_rows<0>();
        for (int c = tid; c < nt * (tile_rows<0>() / 8); c += kThreads) {
            const int n = c / (tile_rows<0>() / 8), ch = c % (tile_rows<0>() / 8);
            *reinterpret_cast<u32x4*>(a.w.H + (int64_t)(base + t0 + n) * a.F + col0 + 8 * ch) =
                *reinterpret_cast<const u32x4*>(hs + n * HS + 8 * ch);
        }
    } else {
        // the tile's 256 output rows of each token are contiguous in O: 32
        // tokens at a time go through LDS, then out as whole rows of 16-byte
        // chunks
        float* os = reinterpret_cast<float*>(smem);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            if (2 * half >= NA) break;
            if (half) __syncthreads();   // the previous half's rows are out
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int jt = 2 * half + q;
                if (jt < NA) {
                    const int n = 16 * q + r;
#pragma unroll
                    for (int m = 0; m < NMAT; ++m)
#pragma unroll
                        for (int blk = 0; blk < 2; ++blk) {
                            const int row = 64 * wave + 32 * m + 16 * blk + 4 * g;
                            *reinterpret_cast<f32x4*>(os + n * kOutStride + row) = s * acc[m][blk][jt];
                        }
                }
            }
            __syncthreads();
            const int n0 = 32 * half;
            const int rows = min(32, nt - n0);
            constexpr int kChunks = tile_rows<1>() / 4;   // 16-byte chunks per token row
            for (int c = tid; c < rows * kChunks; c += kThreads) {
                const int n = c / kChunks, ch = c % kChunks;
                const int m = tsc[n0 + n].m;   // the token's SwiGLU rows were stored as h 2^-m
                const f32x4 v = *reinterpret_cast<const f32x4*>(os + n * kOutStride + 4 * ch);
                *reinterpret_cast<f32x4*>(a.w.O + (int64_t)pair[n0 + n] * a.d + rt * tile_rows<1>() + 4 * ch) =
                    f32x4{ldexpf(v.x, m), ldexpf(v.y, m), ldexpf(v.z, m), ldexpf(v.w, m)};
            }
        }
    }
}

template <int MODE, int B>
__device__ __forceinline__ void dispatch_na(int na, const GemmArgs& a, const TileDesc& td, int tt, int rt,
                                            _Float16* smem, int* tok, int* pair, TokScale* tsc) {
    if (na >= 4) gemm_tile<MODE, B, 4>(a, td.e, td.cnt, td.off, tt, rt, smem, tok, pair, tsc);
    else if (na == 3) gemm_tile<MODE, B, 3>(a, td.e, td.cnt, td.off, tt, rt, smem, tok, pair, tsc);
    else if (na == 2) gemm_tile<MODE, B, 2>(a, td.e, td.cnt, td.off, tt, rt, smem, tok, pair, tsc);
    else gemm_tile<MODE, B, 1>(a, td.e, td.cnt, td.off, tt, rt, smem, tok, pair, tsc);
}

template <int MODE>
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(GemmArgs a, int row_tiles) {
    extern __shared__ __attribute__((aligned(16))) _Float16 smem[];
    __shared__ int tok[BN];
    __shared__ int pair[MODE == 1 ? BN : 1];
    __shared__ TokScale tsc[BN];
    // XCD swizzle: the eighth of this forward's tiles (the grid is sized for
    // the most a batch can have) that this workgroup's XCD walks, so the
    // XCDs get equal shares and the unused workgroups are spread over them
    const int used = a.w.n_act[1] * row_tiles;
    const int share = (used + 7) >> 3;
    const int i = blockIdx.x >> 3;
    const int L = (blockIdx.x & 7) * share + i;
    if (i >= share || L >= used) return;
    // L lies in the range of token tile L / row_tiles's expert; within an
    // expert's range, row tile major and token tile minor: the workgroups
    // that stream the same codes are neighbours in dispatch order and run
    // side by side on one XCD, so the codes come from its L2
    const TileDesc td = a.w.tiles[L / row_tiles];
    const int ntt = (td.cnt + BN - 1) / BN;
    const int l = L - td.first * row_tiles;
    const int rt = l / ntt;
    const int tt = l - rt * ntt;
    const int b = a.tab.bits[td.e];
    // 16-token blocks holding real tokens (fewer than four only in an
    // expert's last token tile): the MFMAs of the empty ones are skipped
    const int nblk = (min(BN, td.cnt - tt * BN) + 15) >> 4;
    if (b == 4) dispatch_na<MODE, 4>(nblk, a, td, tt, rt, smem, tok, pair, tsc);
    else if (b == 8) dispatch_na<MODE, 8>(nblk, a, td, tt, rt, smem, tok, pair, tsc);
    else dispatch_na<MODE, 3>(nblk, a, td, tt, rt, smem, tok, pair, tsc);
}

template <int MODE>
hipError_t launch_gemm(const GemmArgs& a, hipStream_t s, KTimer t) {
    const int rows = MODE == 0 ? a.F : a.d;
    const int row_tiles = rows / tile_rows<MODE>();
    // token tiles over all experts: at most ceil(P / BN) + (active experts)
    const int64_t tt_max = (a.P_used + BN - 1) / BN + a.max_act;
    int64_t ntiles = tt_max * row_tiles;
    ntiles = (ntiles + 7) / 8 * 8;
    // two token-row buffers; the down tile's output staging may need more
    const size_t lds = std::max<size_t>(2 * (size_t)BN * LDX * 2, MODE == 1 ? 32 * kOutStride * 4 : 0);
    return launch_timed(gemm_kernel<MODE>, dim3((unsigned)ntiles), dim3(kThreads), lds, s, t.start,
                        t.stop, a, row_tiles);
}

}  // namespace

bool gemm_supported(int d, int F) { return d % tile_rows<1>() == 0 && F % tile_rows<0>() == 0; }

hipError_t launch_prep_x(const GemmArgs& a, hipStream_t s) {
    const int per_block = kThreads / 64;
    auto kernel = a.d <= 8 * 64 * 8 ? prep_x_kernel<8> : prep_x_kernel<16>;
    return launch_timed(kernel, dim3((unsigned)((a.T + per_block - 1) / per_block)), dim3(kThreads), 0, s,
                        (hipEvent_t) nullptr, (hipEvent_t) nullptr, a.x, a.T, a.d, a.bits_mask,
                        const_cast<_Float16*>(a.xp), a.xp_plane, a.w.xst);
}
hipError_t launch_gate_up_gemm(const GemmArgs& a, hipStream_t s, KTimer t) { return launch_gemm<0>(a, s, t); }
hipError_t launch_down_gemm(const GemmArgs& a, hipStream_t s, KTimer t) { return launch_gemm<1>(a, s, t); }

}  // namespace pw
