// Host tier (PagedWeight page, section "Dynamic Paging": pages are fetched
// for the experts the router selects, and inactive experts' pages can be
// swapped out to CPU memory). Every page lives in pinned host memory; the
// device pool is a cache of S page slots. Per forward pass, on the GPU and
// without a round trip to the host:
//
//   plan  (one workgroup): the active experts that hold a slot are hits; the
//         others (misses, ascending expert id) take empty slots (ascending
//         index), then the slots of inactive experts, least recently used
//         first (ties: lower expert id); misses left over are read from the
//         host tier directly in this pass. Writes the copy list and each
//         expert's page address for this pass.
//   copy  the listed pages host -> slot (reads over the host link).
//
// The expert kernels then read every page through the address list, with
// a null pool base (their page address is base + offset).
#include <hip/hip_runtime.h>

#include "pw_internal.h"

namespace pw {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPlanThreads = 1024;
constexpr int kCopyThreads = 256;
constexpr int64_t kCopyChunk = 256 * 1024;   // bytes per copy workgroup

__global__ __launch_bounds__(kPlanThreads) void swap_plan_kernel(SwapState st, const int32_t* cnt, DevTable tab, int E,
                                                                   int S, const uint8_t* pool,
                                                                   const uint8_t* host, uint64_t slot_bytes) {
    __shared__ int32_t s_slot[kMaxExperts];     // slot of each expert (-1: none)
    __shared__ int32_t s_exp[kMaxExperts];      // expert of each slot (-1: empty)
    __shared__ uint8_t s_act[kMaxExperts];
    __shared__ int32_t s_miss[kMaxExperts];     // misses in ascending id
    __shared__ int32_t s_cand[kMaxExperts];     // candidate slots in hand-out order
    __shared__ uint64_t s_key[kMaxExperts];
    __shared__ int32_t s_scan[kPlanThreads];
    __shared__ int s_nact;
    const int tid = threadIdx.x;
    const uint32_t step = st.step[0] + 1;
    if (tid == 0) s_nact = 0;
    __syncthreads();
    // the active experts: those the router gave at least one pair
    for (int e = tid; e < E; e += kPlanThreads) {
        s_slot[e] = st.slot_of[e];
        s_act[e] = cnt[e] > 0;
        if (s_act[e]) atomicAdd(&s_nact, 1);
    }
    for (int s = tid; s < S; s += kPlanThreads) s_exp[s] = st.expert_of[s];
    __syncthreads();
    const int n_act = s_nact;

    // misses ranked by expert id: a block scan over the E flags, each thread
    // owning a contiguous run of ceil(E / threads) experts
    const int per = (E + kPlanThreads - 1) / kPlanThreads;
    int mine = 0;
    for (int e = tid * per; e < min(E, tid * per + per); ++e) mine += (s_act[e] && s_slot[e] < 0);
    s_scan[tid] = mine;
    __syncthreads();
    for (int o = 1; o < kPlanThreads; o <<= 1) {
        const int v = tid >= o ? s_scan[tid - o] : 0;
        __syncthreads();
        s_scan[tid] += v;
        __syncthreads();
    }
    const int n_miss = s_scan[kPlanThreads - 1];
    int r = s_scan[tid] - mine;
    for (int e = tid * per; e < min(E, tid * per + per); ++e)
        if (s_act[e] && s_slot[e] < 0) s_miss[r++] = e;

    // candidate slots: empty ones keyed by index, then those of inactive
    // experts keyed by (last use, expert); slots of active experts are not
    // candidates. All keys differ, so a slot's rank is the number of
    // smaller keys.
    constexpr uint64_t kNone = ~0ull;
    for (int s = tid; s < S; s += kPlanThreads) {
        const int e = s_exp[s];
        uint64_t key;
        if (e < 0) key = (uint64_t)s;
        else if (s_act[e]) key = kNone;
        else key = (1ull << 62) | ((uint64_t)st.last_use[e] << 10) | (uint64_t)e;
        s_key[s] = key;
    }
    __syncthreads();
    int n_cand_part = 0;
    for (int s = tid; s < S; s += kPlanThreads) {
        const uint64_t k = s_key[s];
        if (k == kNone) continue;
        ++n_cand_part;
        int rank = 0;
        for (int q = 0; q < S; ++q) rank += s_key[q] < k;
        s_cand[rank] = s;
    }
    s_scan[tid] = n_cand_part;
    __syncthreads();
    for (int o = 1; o < kPlanThreads; o <<= 1) {
        const int v = tid >= o ? s_scan[tid - o] : 0;
        __syncthreads();
        s_scan[tid] += v;
        __syncthreads();
    }
    const int n_cand = s_scan[kPlanThreads - 1];
    const int ncopy = min(n_miss, n_cand);

    // hand out the slots: miss i takes candidate i; the expert that held it
    // (inactive, so no other miss and no hit) loses it
    for (int i = tid; i < ncopy; i += kPlanThreads) {
        const int e = s_miss[i], s = s_cand[i];
        const int old = s_exp[s];
        if (old >= 0) s_slot[old] = -1;
        st.copy_e[i] = e;
        st.copy_s[i] = s;
    }
    __syncthreads();
    for (int i = tid; i < ncopy; i += kPlanThreads) {
        const int e = s_miss[i], s = s_cand[i];
        s_exp[s] = e;
        s_slot[e] = s;
    }
    __syncthreads();

    for (int e = tid; e < E; e += kPlanThreads) {
        const int s = s_slot[e];
        st.slot_of[e] = s;
        st.addr[e] = s >= 0 ? (uint64_t)(pool + (uint64_t)s * slot_bytes) : (uint64_t)(host + tab.off[e]);
        if (s_act[e]) st.last_use[e] = step;
    }
    for (int s = tid; s < S; s += kPlanThreads) st.expert_of[s] = s_exp[s];
    if (tid == 0) {
        st.step[0] = step;
        st.ncopy[0] = ncopy;
        st.stats[0] += (uint64_t)(n_act - n_miss);
        st.stats[1] += (uint64_t)ncopy;
        st.stats[2] += (uint64_t)(n_miss - ncopy);
    }
}

// grid (chunks of a slot, listed copies): workgroup (x, j) copies bytes
// [x kCopyChunk, (x + 1) kCopyChunk) of copy j's page, 16 bytes per thread
// and iteration; pages are multiples of 256 bytes.
__global__ __launch_bounds__(kCopyThreads) void swap_copy_kernel(SwapState st, DevTable tab, uint64_t We,
                                                                   uint8_t* pool, const uint8_t* host,
                                                                   uint64_t slot_bytes) {
    const int j = blockIdx.y;
    if (j >= st.ncopy[0]) return;
    const int e = st.copy_e[j], s = st.copy_s[j];
    const uint64_t nbytes = (We * (uint64_t)tab.bits[e] / 8 + kPageAlign - 1) / kPageAlign * kPageAlign;
    const uint64_t lo = (uint64_t)blockIdx.x * kCopyChunk;
    if (lo >= nbytes) return;
    const uint64_t hi = min(nbytes, lo + (uint64_t)kCopyChunk);
    const u32x4* src = reinterpret_cast<const u32x4*>(host + tab.off[e]);
    u32x4* dst = reinterpret_cast<u32x4*>(pool + (uint64_t)s * slot_bytes);
    for (uint64_t i = lo / 16 + threadIdx.x; i < hi / 16; i += kCopyThreads)
        dst[i] = __builtin_nontemporal_load(src + i);
}

// Experts whose pages were rewritten lose their slots (the list holds
// distinct experts).
__global__ __launch_bounds__(256) void swap_invalidate_kernel(SwapState st, const int32_t* list, int n) {
    for (int i = threadIdx.x; i < n; i += 256) {
        const int e = list[i];
        const int s = st.slot_of[e];
        if (s >= 0) {
            st.expert_of[s] = -1;
            st.slot_of[e] = -1;
        }
    }
}

}  // namespace

hipError_t launch_swap_in(const SwapState& st, const int32_t* cnt, const DevTable& tab, int E, int S,
                          int max_copies, uint64_t We, uint8_t* pool, const uint8_t* host, uint64_t slot_bytes,
                          hipStream_t s) {
    swap_plan_kernel<<<1, kPlanThreads, 0, s>>>(st, cnt, tab, E, S, pool, host, slot_bytes);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || max_copies <= 0) return err;
    const dim3 grid((unsigned)((slot_bytes + kCopyChunk - 1) / kCopyChunk), (unsigned)max_copies);
    swap_copy_kernel<<<grid, kCopyThreads, 0, s>>>(st, tab, We, pool, host, slot_bytes);
    return hipGetLastError();
}

hipError_t launch_swap_invalidate(const SwapState& st, const int32_t* list, int n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    swap_invalidate_kernel<<<1, 256, 0, s>>>(st, list, n);
    return hipGetLastError();
}

}  // namespace pw
