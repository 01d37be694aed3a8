// Router and grouping (PagedWeight page, section "Dynamic Paging": the
// router determines which experts each token needs, and those experts'
// pages are fetched through the page table).
//
// Per token: the k largest logits (equal values -> lower expert index) and
// softmax weights g. Then a stable counting sort of the (token, slot) pairs
// by expert: rank of a pair = number of earlier tokens routed to the same
// expert; offsets = exclusive prefix of the per-expert counts. The list of
// active experts is ordered 8-bit pages first, then 4-bit, then 3-bit (each
// by expert id), so the longest tiles are dispatched first.
//
// Top-k per token: with at most 256 experts a row of 16 lanes routes one
// token (DPP reductions within the row), else a wave (shuffles).
//
// The streaming (decode) kernels need per expert only its set of pairs, in
// any order (each token is its own column of the expert's products, their
// SwiGLU rows and outputs are addressed by pair index, and the combine sums
// in slot order), so their router groups the pairs with atomic adds in the
// same launch as the top-k: one kernel over many small workgroups, which
// also takes each token's activation statistics (xscale.h). Batches of at
// most 16 tokens over at most 64 experts are grouped by the decode gate/up
// kernel itself (kernels_ffn.hip; this router then skips its atomics), and
// up to 4 tokens routed there too, with the same top-k (route_dev.h).
//
// The matrix-core kernels work on token tiles of a stable counting sort.
// Up to 64 tokens (16 with more than 256 experts): one workgroup does
// everything. Up to kFusedMaxPairs pairs: a router kernel over many
// workgroups, then one workgroup ranks and offsets. Larger batches: router; ranks per expert and
// chunk of kRankChunk tokens; counts, chunk prefixes and offsets in one
// workgroup; pair positions over many workgroups. Kernel boundaries carry
// the results between workgroups (a device-scope handshake inside one kernel
// would have to write back and invalidate the per-XCD L2 caches). No host
// synchronisation.
#include <hip/hip_runtime.h>

#include <math.h>

#include <algorithm>

#include "pw_internal.h"
#include "route_dev.h"
#include "xscale.h"

namespace pw {
namespace {

using namespace rdev;

constexpr int kBlock = 1024;
constexpr int kWaves = kBlock / 64;
constexpr int kRowMaxExperts = 256;             // 16 lanes per token up to this many experts
// The streaming router takes the 16-lane rows only up to this many experts
// (a wave per token beyond: fewer keys per lane, shorter rounds; 128 experts
// x top-8 routed 2 us faster)
constexpr int kRowDecodeMaxExperts = 64;
// One workgroup routes and groups up to this many tokens (one pass of its
// 64 rows of 16 lanes with at most 256 experts, one token per wave else);
// beyond, the top-k is spread over many workgroups and only the grouping
// stays in one.
constexpr int kFusedMaxTokensRow = 64;
constexpr int kFusedMaxTokens = 16;

__device__ __forceinline__ bool better(float v, int e, float v2, int e2) {
    return v > v2 || (v == v2 && e < e2);
}

// The decode grouping of pair p = t k + j routed to expert e: the next
// position of e's list; the expert's first pair enters it in the active
// list, from the front (without widths, or if it is wider than 4 bits),
// else from the back.
__device__ __forceinline__ void group_pair(const DecodeGroup& g, int tcap, const int32_t* bits, int e, int p) {
    const int slot = atomicAdd(&g.cnt[e], 1);
    g.list[(int64_t)e * tcap + slot] = p;
    if (slot == 0) {
        if (!bits || bits[e] > 4) g.act[atomicAdd(&g.n_act[0], 1)] = e;
        else g.act[g.E - 1 - atomicAdd(&g.n_act[1], 1)] = e;
    }
}

// ---- 16 lanes per token (E <= 256): route_dev.h ----

// One wave routes token t (lane l holds the logits of experts l, l + 64,
// ...): k rounds of the wave's largest (logit, expert) key, each removed from
// its lane; the wave-wide results are scalars. Writes ids/g (and the ids to
// s_ids if given); k <= 64. pre() runs after the logits loads are issued.
template <int PER, class Pre>
__device__ __forceinline__ void route_token_t(const RouteArgs& a, const FwdWork& w, int t, int* s_ids,
                                              bool group, Pre&& pre) {
    const int lane = threadIdx.x & 63;
    const float* row = a.logits + (int64_t)t * a.E;
    float v[PER];
    uint64_t key[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < a.E ? row[e] : -INFINITY;
    }
    pre();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + 64 * i;
        key[i] = e < a.E ? route_key(v[i], e) : 0ull;
    }
    int my_id = 0;
    float my_val = -INFINITY, top = -INFINITY;
    for (int j = 0; j < a.k; ++j) {
        // this lane's largest key (a tree over its keys), then the wave's
        uint64_t m[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) m[i] = key[i];
#pragma unroll
        for (int h = 1; h < PER; h *= 2)
#pragma unroll
            for (int i = 0; i + h < PER; i += 2 * h) m[i] = m[i + h] > m[i] ? m[i + h] : m[i];
        const uint64_t best = wave_max_key(m[0]);
#pragma unroll
        for (int i = 0; i < PER; ++i) key[i] = key[i] == best ? 0ull : key[i];
        const float bv = key_value(best);
        if (j == 0) top = bv;
        if (lane == j) { my_id = key_expert(best); my_val = bv; }
    }
    constexpr float kLog2e = 1.4426950408889634f;
    float sum_all = 0.0f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + 64 * i;
        if (e < a.E) sum_all += __builtin_amdgcn_exp2f((v[i] - top) * kLog2e);
    }
    const float mine = lane < a.k ? __builtin_amdgcn_exp2f((my_val - top) * kLog2e) : 0.0f;
    const float den = wave_sum(a.renorm ? mine : sum_all);
    if (lane < a.k) {
        w.ids[(int64_t)t * a.k + lane] = my_id;
        w.g[(int64_t)t * a.k + lane] = mine / den;
        if (s_ids) s_ids[t * a.k + lane] = my_id;
        if (group) group_pair(w.dg, w.tcap, a.bits, my_id, t * a.k + lane);
    }
}

// The row of 16 lanes containing this thread routes token t (all lanes of
// the row call it with the same t; `valid` false for a row past the batch):
// top-k and weights by row_topk (route_dev.h). pre() runs after the logits loads are issued and before they are used
// (the streaming router takes the token's activation statistics there, so
// that both rows' loads are in flight together).
template <int PER, class Pre>
__device__ __forceinline__ void route_row_t(const RouteArgs& a, const FwdWork& w, int t, bool valid,
                                            int* s_ids, bool group, Pre&& pre) {
    const int l16 = threadIdx.x & 15;
    const float* row = a.logits + (int64_t)t * a.E;
    float v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = l16 + 16 * i;
        v[i] = (valid && e < a.E) ? row[e] : -INFINITY;
    }
    pre();
    const RowChoice c = row_topk<PER>(v, a.E, a.k, a.renorm, valid);
    if (!valid) return;
    if (l16 < a.k) {
        w.ids[(int64_t)t * a.k + l16] = c.id0;
        w.g[(int64_t)t * a.k + l16] = c.g0;
        if (s_ids) s_ids[t * a.k + l16] = c.id0;
        if (group) group_pair(w.dg, w.tcap, a.bits, c.id0, t * a.k + l16);
    }
    if (l16 + 16 < a.k) {
        w.ids[(int64_t)t * a.k + l16 + 16] = c.id1;
        w.g[(int64_t)t * a.k + l16 + 16] = c.g1;
        if (s_ids) s_ids[t * a.k + l16 + 16] = c.id1;
        if (group) group_pair(w.dg, w.tcap, a.bits, c.id1, t * a.k + l16 + 16);
    }
}

struct NoPre {
    __device__ void operator()() const {}
};

template <class Pre = NoPre>
__device__ __forceinline__ void route_row(const RouteArgs& a, const FwdWork& w, int t, bool valid, int* s_ids,
                                          bool group = false, Pre&& pre = Pre{}) {
    const int per = (a.E + 15) / 16;
    if (per == 1) route_row_t<1>(a, w, t, valid, s_ids, group, pre);
    else if (per == 2) route_row_t<2>(a, w, t, valid, s_ids, group, pre);
    else if (per <= 4) route_row_t<4>(a, w, t, valid, s_ids, group, pre);
    else if (per <= 8) route_row_t<8>(a, w, t, valid, s_ids, group, pre);
    else route_row_t<16>(a, w, t, valid, s_ids, group, pre);
}

template <class Pre = NoPre>
__device__ __forceinline__ void route_token(const RouteArgs& a, const FwdWork& w, int t, int* s_ids,
                                            bool group = false, Pre&& pre = Pre{}) {
    const int per = (a.E + 63) / 64;
    if (per == 1) route_token_t<1>(a, w, t, s_ids, group, pre);
    else if (per == 2) route_token_t<2>(a, w, t, s_ids, group, pre);
    else if (per <= 4) route_token_t<4>(a, w, t, s_ids, group, pre);
    else if (per <= 8) route_token_t<8>(a, w, t, s_ids, group, pre);
    else route_token_t<16>(a, w, t, s_ids, group, pre);
}

// Inclusive scan over the 1024 threads of the block (every thread calls it).
template <typename T>
__device__ __forceinline__ T block_scan(T v, T* s_wave, T* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int o = 1; o < 64; o <<= 1) {
        const T n = __shfl_up(v, o);
        if (lane >= o) v += n;
    }
    __syncthreads();
    if (lane == 63) s_wave[wave] = v;
    __syncthreads();
    if (wave == 0) {
        T x = lane < kWaves ? s_wave[lane] : T(0);
        for (int o = 1; o < kWaves; o <<= 1) {
            const T n = __shfl_up(x, o);
            if (lane >= o) x += n;
        }
        if (lane < kWaves) s_wave[lane] = x;
    }
    __syncthreads();
    *total = s_wave[kWaves - 1];
    return v + (wave > 0 ? s_wave[wave - 1] : T(0));
}

// Inclusive scans of two values at once over the 1024 threads (one set of
// barriers for both).
__device__ __forceinline__ void block_scan2(int& a, long long& b, int* sa, long long* sb, int* ta, long long* tb) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int o = 1; o < 64; o <<= 1) {
        const int na = __shfl_up(a, o);
        const long long nb = __shfl_up(b, o);
        if (lane >= o) {
            a += na;
            b += nb;
        }
    }
    __syncthreads();
    if (lane == 63) {
        sa[wave] = a;
        sb[wave] = b;
    }
    __syncthreads();
    if (wave == 0) {
        int x = lane < kWaves ? sa[lane] : 0;
        long long y = lane < kWaves ? sb[lane] : 0ll;
        for (int o = 1; o < kWaves; o <<= 1) {
            const int nx = __shfl_up(x, o);
            const long long ny = __shfl_up(y, o);
            if (lane >= o) {
                x += nx;
                y += ny;
            }
        }
        if (lane < kWaves) {
            sa[lane] = x;
            sb[lane] = y;
        }
    }
    __syncthreads();
    *ta = sa[kWaves - 1];
    *tb = sb[kWaves - 1];
    if (wave > 0) {
        a += sa[wave - 1];
        b += sb[wave - 1];
    }
}

// Page-table entry of expert threadIdx.x, read at kernel entry.
struct ExpertPage {
    uint64_t off;
    float scale;
    int bits;
};
__device__ __forceinline__ ExpertPage load_page(const DevTable& tab, int E) {
    const int e = threadIdx.x;
    return e < E ? ExpertPage{tab.off[e], tab.scale[e], tab.bits[e]} : ExpertPage{0, 0.0f, 0};
}

// Offsets, bit-ordered active list and the token tiles; cnt_of(e) gives the
// count of expert e. Leaves the offsets in s_off.
template <class CntF>
__device__ __forceinline__ void finalize_offsets(int E, const FwdWork& w, const ExpertPage& my, int tiles,
                                                 CntF cnt_of, int* s_off) {
    __shared__ int s_wave_i[kWaves];
    __shared__ long long s_wave_l[kWaves];
    const int tid = threadIdx.x;
    const int c = tid < E ? cnt_of(tid) : 0;
    // classes: 0 = 8-bit, 1 = 4-bit, 2 = 3-bit; 21-bit counters per class
    const int b = my.bits;   // bit-width of expert tid (loaded by the caller at kernel entry)
    const int cls = b == 8 ? 0 : (b == 4 ? 1 : 2);
    const long long flag = (tid < E && c > 0) ? (1ll << (21 * cls)) : 0ll;
    // the offsets' scan and the class counters' scan together
    int inc = c, tot;
    long long linc = flag, ltot;
    block_scan2(inc, linc, s_wave_i, s_wave_l, &tot, &ltot);
    if (tid < E) {
        s_off[tid] = inc - c;
        w.off[tid] = inc - c;
    }
    if (tid == 0) w.off[E] = tot;
    const int n8 = (int)(ltot & 0x1fffff), n4 = (int)((ltot >> 21) & 0x1fffff),
              n3 = (int)((ltot >> 42) & 0x1fffff);
    // token tiles of the large-batch kernels, in active-list order
    __shared__ int s_slot_cnt[kMaxExperts];
    __shared__ int s_slot_exp[kMaxExperts];
    if (flag) {
        const int before = (int)((linc >> (21 * cls)) & 0x1fffff) - 1;
        const int base = cls == 0 ? 0 : (cls == 1 ? n8 : n8 + n4);
        w.act[base + before] = tid;
        s_slot_cnt[base + before] = c;
        s_slot_exp[base + before] = tid;
    }
    if (tid == 0) w.n_act[0] = n8 + n4 + n3;
    __syncthreads();
    if (!tiles) return;   // only the large-batch kernels read the token tiles
    const int na = n8 + n4 + n3;
    const int ntt = tid < na ? (s_slot_cnt[tid] + kGemmTokens - 1) / kGemmTokens : 0;
    __shared__ int s_first[kMaxExperts];
    int ttot;
    const int tinc = block_scan<int>(ntt, s_wave_i, &ttot);
    if (tid < na) s_first[tid] = tinc - ntt;
    if (tid == 0) w.n_act[1] = ttot;
    __syncthreads();
    // one descriptor per token tile: the slot whose range holds tile j is
    // the last one starting at or before j (every slot has at least one tile)
    for (int j = tid; j < ttot; j += kBlock) {
        int lo = 0, hi = na;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_first[mid] <= j) lo = mid; else hi = mid;
        }
        const int e = s_slot_exp[lo];
        w.tiles[j] = TileDesc{e, s_first[lo], s_slot_cnt[lo], s_off[e]};
    }
    __syncthreads();
}

// Offsets and pair positions in one workgroup; rank_of(p) gives the rank of
// pair p, id_of(p) its expert.
template <class CntF, class RankF, class IdF>
__device__ __forceinline__ void finalize(int T, int E, int k, const FwdWork& w, const ExpertPage& my, int tiles,
                                         CntF cnt_of, RankF rank_of, IdF id_of) {
    __shared__ int s_off[kMaxExperts];
    finalize_offsets(E, w, my, tiles, cnt_of, s_off);
    const int P = T * k;
    for (int p = threadIdx.x; p < P; p += kBlock) {
        const int e = id_of(p);
        w.sorted[s_off[e] + rank_of(p)] = p;
    }
}

// Stable rank of every pair from ids in LDS: for each chunk of 64 tokens,
// lane = token, holding its KMAX (>= k) expert ids in registers; wave w
// handles experts w, w + 16, ... and keeps their running counts in s_cnt.
// Writes s_rank, s_cnt and w.cnt.
template <int KMAX>
__device__ __forceinline__ void rank_small_t(int T, int E, int k, const int* s_ids, int* s_rank, int* s_cnt,
                                             const FwdWork& w) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (T <= 64) {
        // one chunk: ranks and counts straight from the ballots, no running
        // counts to read back
        int my[KMAX];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) my[j] = (j < k && lane < T) ? s_ids[lane * k + j] : -1;
        for (int e = wave; e < E; e += kWaves) {
            int slot = -1;
#pragma unroll
            for (int j = 0; j < KMAX; ++j)
                if (my[j] == e) slot = j;
            const uint64_t m = __ballot(slot >= 0);
            if (slot >= 0) s_rank[lane * k + slot] = __popcll(m & ((1ull << lane) - 1ull));
            if (lane == 0) {
                s_cnt[e] = __popcll(m);
                w.cnt[e] = __popcll(m);
            }
        }
        return;
    }
    for (int e = wave; e < E; e += kWaves)
        if (lane == 0) s_cnt[e] = 0;
    for (int t0 = 0; t0 < T; t0 += 64) {
        const int tt = t0 + lane;
        int my[KMAX];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) my[j] = (j < k && tt < T) ? s_ids[tt * k + j] : -1;
        for (int e = wave; e < E; e += kWaves) {
            int slot = -1;
#pragma unroll
            for (int j = 0; j < KMAX; ++j)
                if (my[j] == e) slot = j;
            const uint64_t m = __ballot(slot >= 0);
            const int base = s_cnt[e];
            if (slot >= 0) s_rank[tt * k + slot] = base + __popcll(m & ((1ull << lane) - 1ull));
            if (lane == 0) s_cnt[e] = base + __popcll(m);
        }
    }
    for (int e = wave; e < E; e += kWaves)
        if (lane == 0) w.cnt[e] = s_cnt[e];
}

__device__ __forceinline__ void rank_small(int T, int E, int k, const int* s_ids, int* s_rank, int* s_cnt,
                                           const FwdWork& w) {
    if (k <= 2) rank_small_t<2>(T, E, k, s_ids, s_rank, s_cnt, w);
    else if (k <= 4) rank_small_t<4>(T, E, k, s_ids, s_rank, s_cnt, w);
    else if (k <= 8) rank_small_t<8>(T, E, k, s_ids, s_rank, s_cnt, w);
    else if (k <= 16) rank_small_t<16>(T, E, k, s_ids, s_rank, s_cnt, w);
    else rank_small_t<32>(T, E, k, s_ids, s_rank, s_cnt, w);
}

// ---- small batches (up to one pass of rows or waves): everything in one workgroup ----
__global__ __launch_bounds__(kBlock) void route_fused_kernel(RouteArgs a, FwdWork w,
                                                             DevTable tab) {
    __shared__ int s_ids[kFusedMaxPairs];
    __shared__ int s_rank[kFusedMaxPairs];
    __shared__ int s_cnt[kMaxExperts];
    const ExpertPage my = load_page(tab, a.E);
    if (a.E <= kRowMaxExperts) {
        const int r16 = threadIdx.x >> 4;          // 64 rows of 16 lanes
        for (int t0 = 0; t0 < a.T; t0 += kBlock / 16)
            route_row(a, w, t0 + r16, t0 + r16 < a.T, s_ids);
    } else {
        const int wave = threadIdx.x >> 6;
        for (int t = wave; t < a.T; t += kWaves) route_token(a, w, t, s_ids);
    }
    __syncthreads();
    rank_small(a.T, a.E, a.k, s_ids, s_rank, s_cnt, w);
    __syncthreads();
    finalize(a.T, a.E, a.k, w, my, a.tiles, [&](int e) { return s_cnt[e]; },
             [&](int p) { return s_rank[p]; }, [&](int p) { return s_ids[p]; });
}

// ---- small batches: ranking and offsets of routed pairs in one workgroup ----
__global__ __launch_bounds__(kBlock) void group_small_kernel(int T, int E, int k, int tiles, FwdWork w,
                                                             DevTable tab) {
    __shared__ int s_ids[kFusedMaxPairs];
    __shared__ int s_rank[kFusedMaxPairs];
    __shared__ int s_cnt[kMaxExperts];
    const ExpertPage my = load_page(tab, E);
    const int P = T * k;
    for (int p = threadIdx.x; p < P; p += kBlock) s_ids[p] = w.ids[p];
    __syncthreads();
    rank_small(T, E, k, s_ids, s_rank, s_cnt, w);
    __syncthreads();
    finalize(T, E, k, w, my, tiles, [&](int e) { return s_cnt[e]; },
             [&](int p) { return s_rank[p]; }, [&](int p) { return s_ids[p]; });
}

// ---- large batches: route, rank, finalize ----
// grid ceil(T / 16) (E <= 256: row r of block b handles token 16b + r) or
// ceil(T / 4) (wave w of block b handles token 4b + w), 256 threads.
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a, FwdWork w) {
    if (a.E <= kRowMaxExperts) {
        const int t = blockIdx.x * 16 + (threadIdx.x >> 4);
        route_row(a, w, t < a.T ? t : a.T - 1, t < a.T, nullptr);
    } else {
        const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
        if (t < a.T) route_token(a, w, t, nullptr);
    }
}

// ---- streaming kernels: top-k, grouping by atomics, token statistics ----
// grid T, 128 threads: one token per workgroup (no workgroup barriers, so
// the tokens spread over as many CUs). Wave 0 routes token t (up to 64
// experts with its first row of 16 lanes, beyond with the whole wave) while
// wave 1 takes the token's statistics. Block 0 also clears
// the other counter set for the next forward (every kernel of the previous
// forward, which used it, has finished).
__global__ __launch_bounds__(128) void route_decode_kernel(RouteArgs a, FwdWork w) {
    if (blockIdx.x == 0) {
        for (int e = threadIdx.x; e < a.E; e += blockDim.x) w.dg_next.cnt[e] = 0;
        if (threadIdx.x < 2) w.dg_next.n_act[threadIdx.x] = 0;
    }
    const int t = blockIdx.x;
    auto stats = [&]() {
        if (a.x) {
            const XStat st = lanes_stat<64>(a.x + (int64_t)t * a.d, a.d);
            if ((threadIdx.x & 63) == 0) w.xst[t] = st;
        }
    };
    if (threadIdx.x >= 64) stats();
    else if (a.E > kRowDecodeMaxExperts) route_token(a, w, t, nullptr, a.group != 0);
    else route_row(a, w, t, threadIdx.x < 16, nullptr, a.group != 0);
}

// grid (E, C), 256 threads: rank of expert e's pairs in token order among
// the tokens of chunk c, and their count.
__global__ __launch_bounds__(256) void rank_kernel(int T, int k, int C, FwdWork w) {
    const int e = blockIdx.x, c = blockIdx.y;
    __shared__ int wave_tot[4];
    int running = 0;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t_end = min(T, (c + 1) * kRankChunk);
    for (int t0 = c * kRankChunk; t0 < t_end; t0 += 256) {
        const int t = t0 + threadIdx.x;
        int slot = -1;
        if (t < t_end)
            for (int j = 0; j < k; ++j)
                if (w.ids[(int64_t)t * k + j] == e) slot = j;
        const uint64_t m = __ballot(slot >= 0);
        const int before = __popcll(m & ((1ull << lane) - 1ull));
        __syncthreads();
        if (lane == 0) wave_tot[wave] = __popcll(m);
        __syncthreads();
        int base = running;
        for (int i = 0; i < wave; ++i) base += wave_tot[i];
        if (slot >= 0) w.rank[(int64_t)t * k + slot] = base + before;
        running += wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
    }
    if (threadIdx.x == 0) w.ccnt[e * C + c] = running;
}

// One workgroup: per-expert counts and chunk prefixes, then offsets, the
// active list and the token tiles.
__global__ __launch_bounds__(kBlock) void offsets_kernel(int E, int C, int tiles, FwdWork w, DevTable tab) {
    __shared__ int s_cnt[kMaxExperts];
    __shared__ int s_off[kMaxExperts];
    const ExpertPage my = load_page(tab, E);
    for (int e = threadIdx.x; e < E; e += kBlock) {
        int run = 0;
        for (int c = 0; c < C; ++c) {
            w.cpre[e * C + c] = run;
            run += w.ccnt[e * C + c];
        }
        s_cnt[e] = run;
        w.cnt[e] = run;
    }
    __syncthreads();
    finalize_offsets(E, w, my, tiles, [&](int e) { return s_cnt[e]; }, s_off);
}

// grid ceil(P / 256): position of every pair in expert-sorted order.
__global__ __launch_bounds__(256) void scatter_kernel(int P, int k, int C, FwdWork w) {
    const int p = blockIdx.x * 256 + threadIdx.x;
    if (p >= P) return;
    const int e = w.ids[p];
    const int c = (p / k) / kRankChunk;
    w.sorted[w.off[e] + w.cpre[e * C + c] + w.rank[p]] = p;
}

__global__ __launch_bounds__(256) void zero_kernel(int32_t* p, uint64_t n) {
    for (uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (uint64_t)gridDim.x * 256) p[i] = 0;
}

}  // namespace

hipError_t launch_zero_i32(int32_t* p, uint64_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    zero_kernel<<<(unsigned)std::min<uint64_t>((n + 255) / 256, 1024), 256, 0, s>>>(p, n);
    return hipGetLastError();
}

hipError_t launch_route_decode(const RouteArgs& a, const FwdWork& w, hipStream_t s, KTimer t) {
    // one token per workgroup, two waves (routing, statistics)
    return launch_timed(route_decode_kernel, dim3((unsigned)a.T), dim3(128), 0, s, t.start, t.stop, a, w);
}

hipError_t launch_route(const RouteArgs& a, const FwdWork& w, const DevTable& tab, hipStream_t s,
                        KTimer t) {
    const hipEvent_t none = nullptr;
    if (a.T <= (a.E <= kRowMaxExperts ? kFusedMaxTokensRow : kFusedMaxTokens) && a.T * a.k <= kFusedMaxPairs)
        return launch_timed(route_fused_kernel, dim3(1), dim3(kBlock), 0, s, t.start, t.stop, a, w, tab);
    const int per_block = a.E <= kRowMaxExperts ? 16 : 4;
    hipError_t err = launch_timed(route_kernel, dim3((a.T + per_block - 1) / per_block), dim3(256), 0, s, t.start,
                                  none, a, w);
    if (err != hipSuccess) return err;
    if (a.T * a.k <= kFusedMaxPairs)
        return launch_timed(group_small_kernel, dim3(1), dim3(kBlock), 0, s, none, t.stop, a.T, a.E, a.k,
                            a.tiles, w, tab);
    const int C = (a.T + kRankChunk - 1) / kRankChunk;
    err = launch_timed(rank_kernel, dim3(a.E, C), dim3(256), 0, s, none, none, a.T, a.k, C, w);
    if (err != hipSuccess) return err;
    err = launch_timed(offsets_kernel, dim3(1), dim3(kBlock), 0, s, none, none, a.E, C, a.tiles, w, tab);
    if (err != hipSuccess) return err;
    const int P = a.T * a.k;
    return launch_timed(scatter_kernel, dim3((P + 255) / 256), dim3(256), 0, s, none, t.stop, P, a.k, C, w);
}

}  // namespace pw
