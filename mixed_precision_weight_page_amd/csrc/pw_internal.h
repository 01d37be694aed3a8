// Internal interface between the C-ABI host code and the HIP kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/pagedweight.h"

namespace pw {

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int kRowAlign = 128;         // codes per row are a multiple of this
constexpr int kPageAlign = 256;        // page offsets and sizes
constexpr int64_t kStatChunk = 16384;  // weights per block in the stats kernels
constexpr int kFusedMaxPairs = 4096;   // (token, slot) pairs ranked by one workgroup
constexpr int kRankChunk = 1024;      // tokens per ranking workgroup of the large-batch router
constexpr int kGemmTokens = 64;        // tokens per tile of the large-batch kernels
constexpr int kGemmMinTokens = 64;     // mean tokens per active expert for those kernels

// supported bit-widths, in loss-table order
__host__ __device__ constexpr int bits_of_index(int i) { return i == 0 ? 3 : i == 1 ? 4 : 8; }
__host__ __device__ constexpr int bits_index(int b) { return b == 3 ? 0 : b == 4 ? 1 : b == 8 ? 2 : -1; }
__host__ __device__ constexpr int qmax_of(int b) { return (1 << (b - 1)) - 1; }

// Device page table (structure of arrays, one entry per expert).
struct DevTable {
    uint64_t* off;
    float* scale;
    int32_t* bits;
};

// One token tile (kGemmTokens sorted pairs of one expert) of the
// large-batch kernels: its expert, the index of that expert's first token
// tile, the expert's pair count and its first sorted position.
struct __attribute__((aligned(16))) TileDesc {
    int32_t e, first, cnt, off;
};

// Grouping of the streaming (decode) kernels: per expert the list of its
// (token, slot) pairs t k + j, filled by atomic adds (capacity tcap per
// expert: a token routes to an expert at most once), and the list of routed
// experts. The counters come in two sets that alternate between forwards:
// the router of one forward clears the set of the next.
struct DecodeGroup {
    int32_t* cnt;     // [E] pairs routed to each expert
    int32_t* n_act;   // [2] routed experts at the front of act, and at its back
    int32_t* act;     // [E] routed experts in arrival order, from the front (all
                      // of them, or those wider than 4 bits) and from the back;
                      // in class and id order, from the front, when the gate/up
                      // kernel groups the pairs
    int32_t* list;    // [E, tcap] pair indices of each expert, in arrival order
                      // (in pair order when the gate/up kernel groups them)
    int E;            // entries of act
};

// The decode kernels' routed slots: m = min(E, pairs) slots, the first
// n_act[0] holding the front of the router's list (act[i]), the last
// n_act[1] its back (act[E - m + i]), none in between. When the router
// orders by width, the wider experts are at the front: their workgroups
// run longest and are dispatched first, the narrow ones fill in behind
// them. Both candidates of a slot can be read before the counts arrive.
__device__ __forceinline__ int slot_expert(int i, int m, int nf, int nb, int front, int back) {
    return i < nf ? front : (i >= m - nb ? back : -1);
}
__device__ __forceinline__ int slot_expert(const DecodeGroup& g, int m, int i, int nf, int nb) {
    return slot_expert(i, m, nf, nb, g.act[i], g.act[g.E - m + i]);
}

// Per-token statistics of the activations (xscale.h): e with max|x| 2^-e in
// [2^14, 2^15) and n1 = sum |x| 2^-e over the row.
struct __attribute__((aligned(8))) XStat {
    float n1;
    int32_t e;
};

// Forward-pass scratch carved out of the bound workspace.
struct FwdWork {
    int32_t* ids;      // [P] expert of pair p = t*k + j
    float* g;          // [P] routing weight
    int32_t* rank;     // [P] rank of the pair among its expert's pairs
    int32_t* sorted;   // [P] pair at each sorted position
    int32_t* cnt;      // [E] tokens per expert
    int32_t* off;      // [E+1] exclusive prefix of cnt
    int32_t* act;      // [E] experts with cnt > 0, ascending
    int32_t* n_act;    // [2] active experts; token tiles of the large-batch kernels
    TileDesc* tiles;   // [ceil(P / kGemmTokens) + E] token tiles in active-list order
    DecodeGroup dg;    // grouping of this forward (streaming kernels)
    DecodeGroup dg_next;   // the other counter set, cleared for the next forward
    int tcap;          // capacity of each expert's pair list
    int32_t* ccnt;     // [E, C] pairs of expert e among the tokens of chunk c (kRankChunk tokens)
    int32_t* cpre;     // [E, C] exclusive prefix of ccnt over the chunks
    XStat* xst;        // [T] activation statistics per token
    _Float16* H;       // [P, F] SwiGLU output, scaled by 2^-m (xscale.h): per sorted pair on the
                       // matrix-core path, per pair t k + j on the streaming path
    float* O;          // [nsplit, P, d] down-projection partials per pair t k + j (scaled by s_e)
};

struct Layout {
    uint64_t ids, g, rank, sorted, cnt, off, act, n_act, tiles, ccnt, cpre, xst, H, O, xp, list, fwd_end;
    uint64_t partial, stats_end;
    uint64_t dg, dg_bytes;   // the two counter sets of the streaming kernels' grouping (outside the
                             // bytes the statistics pass reuses; zeroed when the workspace is bound)
    uint64_t total;
};

Layout workspace_layout(int E, int d, int F, int k, int max_tokens, int nsplit);

// Optional timing of a launch: events recorded on the stream just before and
// after the kernel. Each recorded event delays the next dispatch by a few
// microseconds, part of which falls inside the pair, so the pair reads a
// little longer than the kernel itself.
struct KTimer {
    hipEvent_t start = nullptr, stop = nullptr;
};

template <typename Kern, typename... Args>
inline hipError_t launch_timed(Kern kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s,
                               hipEvent_t start, hipEvent_t stop, Args... args) {
    if (start) {
        const hipError_t e = hipEventRecord(start, s);
        if (e != hipSuccess) return e;
    }
    kernel<<<grid, block, lds, s>>>(args...);
    if (stop) {
        const hipError_t e = hipEventRecord(stop, s);
        if (e != hipSuccess) return e;
    }
    return hipGetLastError();
}

// ---- launchers (kernels_*.hip) ----
hipError_t launch_absmax(const void* w1, const void* w3, const void* w2, int f16, int E,
                         int64_t M, uint32_t* absmax, uint32_t* flags, hipStream_t s);
hipError_t launch_loss(const void* w1, const void* w3, const void* w2, int f16, int E,
                       int64_t M, const uint32_t* absmax, double* partial, double* loss, int planes,
                       hipStream_t s);
// planes: bitplane pages; first[i] (planes only) is the first plane to write
// for the i-th listed expert, up to its depth
hipError_t launch_pack(const void* w1, const void* w3, const void* w2, int f16, int d, int F,
                       DevTable tab, const int32_t* list, const int32_t* first, int nlist, int planes,
                       uint8_t* pool, hipStream_t s);

struct RouteArgs {
    const float* logits;
    const uint16_t* x;   // bf16 [T, d]: per-token statistics into FwdWork::xst (NULL: none)
    int d;
    int T, E, k, renorm;
    int tiles;   // also the large-batch kernels' token tiles (FwdWork::tiles)
    const int32_t* bits;   // [E] the table's widths, or NULL: the streaming router's active list
                           // puts the experts wider than 4 bits first (else arrival order)
    int group = 1;         // the streaming router: 0 = ids, weights and statistics only (the
                           // gate/up kernel groups the pairs)
};
hipError_t launch_route(const RouteArgs& a, const FwdWork& w, const DevTable& tab, hipStream_t s,
                        KTimer t = {});
// Router of the streaming kernels: top-k, weights, token statistics and the
// grouping of FwdWork::dg, in one launch over many workgroups.
hipError_t launch_route_decode(const RouteArgs& a, const FwdWork& w, hipStream_t s, KTimer t = {});
// n int32 zeros at p (one small kernel)
hipError_t launch_zero_i32(int32_t* p, uint64_t n, hipStream_t s);

struct FfnPlan {
    int nt_alloc;     // token rows the LDS is sized for
    int nsplit;       // workgroups along K (down product only)
    size_t lds;       // dynamic LDS bytes
    bool whole_k;     // the LDS holds every K step of nt_alloc token rows
};
FfnPlan plan_ffn(int K, int T, int nsplit);
// K-splits of the down product for a layer (partials summed by the combine)
int down_splits(int F, int d, int max_act, int max_splits);

// KV-pressure budget scheduler decision (budget.cpp); arguments checked by the caller.
pw_status budget_decide(const pw_budget_policy& pol, uint64_t kv_used, int E, const uint64_t* W,
                        uint64_t pool_now, uint64_t budget_now, int steps_since, int32_t* action,
                        uint64_t* budget_out, int32_t* pressure);

struct FfnArgs {
    const uint8_t* pool;
    DevTable tab;
    FwdWork w;
    const uint16_t* x;   // bf16 [T, d]
    int d, F, k, max_act;
    int P;               // pair stride of the split partial outputs O[split][P][d]
    int bitplane;        // 1: bitplane pages (the table's bits are depths 1..8)
    int wide;            // 1: an expert may have more than 16 tokens (wide passes)
    // own_route: 1, the gate/up kernel routes the batch itself; 2, it groups
    // the pairs of the router's ids (own_route_mode); the logits [T, E] and
    // the router's options
    int own_route;
    const float* logits;
    int T, E, renorm;
};
// 1: the gate/up kernel can route a batch of T tokens over E experts, top-k,
// itself; 2: it can group the pairs of such a batch from the router's ids
// (the router then only routes); 0: neither
int own_route_mode(int T, int E, int k);
hipError_t launch_gate_up(const FfnArgs& a, const FfnPlan& p, hipStream_t s, KTimer t = {});
hipError_t launch_down(const FfnArgs& a, const FfnPlan& p, hipStream_t s, KTimer t = {});
hipError_t launch_combine(const FwdWork& w, int T, int d, int k, int P, int nsplit, float* y,
                          hipStream_t s, KTimer t = {});

struct GemmArgs {
    const uint8_t* pool;
    DevTable tab;
    FwdWork w;
    const uint16_t* x;   // bf16 [T, d]
    const _Float16* xp;  // [3][max_tokens][d] x as fp16 in the K order of 3-, 4-, 8-bit codes
    int64_t xp_plane;    // elements per plane of xp
    int bits_mask;       // bit i: some expert uses bit-width (3, 4, 8)[i]
    int T, d, F, k, max_act;
    int64_t P_used;      // T * k of this call
};
bool gemm_supported(int d, int F);
hipError_t launch_prep_x(const GemmArgs& a, hipStream_t s);
hipError_t launch_gate_up_gemm(const GemmArgs& a, hipStream_t s, KTimer t = {});
hipError_t launch_down_gemm(const GemmArgs& a, hipStream_t s, KTimer t = {});

// Host tier: device state of the slot cache (kernels_swap.hip).
struct SwapState {
    int32_t* slot_of;     // [E] slot holding the expert's page, -1 none
    int32_t* expert_of;   // [S] expert whose page a slot holds, -1 empty
    uint32_t* last_use;   // [E] pass that last routed to the expert (0 never)
    uint32_t* step;       // [1] passes so far
    uint64_t* stats;      // [3] hits, pages copied in, pages read from the host tier
    int32_t* ncopy;       // [1] copies of the current pass
    int32_t* copy_e;      // [S] expert of each copy
    int32_t* copy_s;      // [S] slot of each copy
    uint64_t* addr;       // [E] page address for the current pass
};
// cnt: [E] pairs routed to each expert this pass (the active experts have cnt > 0)
hipError_t launch_swap_in(const SwapState& st, const int32_t* cnt, const DevTable& tab, int E, int S,
                          int max_copies, uint64_t We, uint8_t* pool, const uint8_t* host, uint64_t slot_bytes,
                          hipStream_t s);
hipError_t launch_swap_invalidate(const SwapState& st, const int32_t* list, int n, hipStream_t s);

// ---- static scratch of the allocation-free forward (noalloc.hip) ----
uint64_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(int device, void** out);   // the device's copy; device must be current

// ---- host allocator (alloc.cpp) ----
pw_status solve_allocation(int E, const uint64_t* W, const double* p, const double* L,
                           uint64_t B, uint8_t* bits_out, std::string* err);

}  // namespace pw
