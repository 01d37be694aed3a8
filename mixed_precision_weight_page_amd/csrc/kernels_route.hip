// Router and grouping (PagedWeight page, section "Dynamic Paging": the
// router determines which experts each token needs, and those experts'
// pages are fetched through the page table).
//
//   route_kernel     one wave per token: top-k of the logits (equal values ->
//                    lower expert index), softmax weights g.
//   rank_kernel      one block per expert: stable rank of its (token, slot)
//                    pairs in token order (block-wide scan), and its count.
//   finalize_kernel  one block: expert offsets (exclusive scan), the list of
//                    active experts, and the expert-sorted pair order.
// No host synchronisation: every later kernel reads the counts from device
// memory and its grid is sized for the worst case.
#include <hip/hip_runtime.h>

#include <math.h>

#include "pw_internal.h"

namespace pw {
namespace {

constexpr int kMaxPerLane = kMaxExperts / 64;  // 16 logits per lane

__device__ __forceinline__ bool better(float v, int e, float v2, int e2) {
    return v > v2 || (v == v2 && e < e2);
}

// grid ceil(T / 4), 256 threads: wave w of block b handles token 4b + w.
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a, FwdWork w) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (t >= a.T) return;
    const float* row = a.logits + (int64_t)t * a.E;
    float v[kMaxPerLane];
    const int per = (a.E + 63) / 64;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
        const int e = lane + 64 * i;
        v[i] = (i < per && e < a.E) ? row[e] : -INFINITY;
    }
    // full softmax denominator needs the max and the values before masking
    float my_id = 0.0f;   // this lane keeps slot j == lane
    float my_val = -INFINITY;
    float top = -INFINITY;
    uint32_t taken = 0;   // bit i: v[i] already chosen
    for (int j = 0; j < a.k; ++j) {
        float bv = -INFINITY;
        int be = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i) {
            const int e = lane + 64 * i;
            if (i < per && e < a.E && !((taken >> i) & 1u) && better(v[i], e, bv, be)) {
                bv = v[i];
                be = e;
            }
        }
        for (int o = 32; o > 0; o >>= 1) {
            const float ov = __shfl_xor(bv, o);
            const int oe = __shfl_xor(be, o);
            if (better(ov, oe, bv, be)) { bv = ov; be = oe; }
        }
        if ((be & 63) == lane) taken |= 1u << (be >> 6);
        if (j == 0) top = bv;
        if (lane == j) { my_id = (float)be; my_val = bv; }
    }
    // softmax over all experts (or over the chosen k when renormalising)
    float sum_all = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
        const int e = lane + 64 * i;
        if (i < per && e < a.E) sum_all += expf(v[i] - top);
    }
    const float mine = lane < a.k ? expf(my_val - top) : 0.0f;
    float den = a.renorm ? mine : sum_all;
    for (int o = 32; o > 0; o >>= 1) den += __shfl_xor(den, o);
    if (lane < a.k) {
        w.ids[(int64_t)t * a.k + lane] = (int)my_id;
        w.g[(int64_t)t * a.k + lane] = mine / den;
    }
}

// grid E, 256 threads: rank of expert e's pairs in token order.
__global__ __launch_bounds__(256) void rank_kernel(int T, int k, FwdWork w) {
    const int e = blockIdx.x;
    __shared__ int wave_tot[4];
    int running = 0;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int t0 = 0; t0 < T; t0 += 256) {
        const int t = t0 + threadIdx.x;
        int slot = -1;
        if (t < T)
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
    if (threadIdx.x == 0) w.cnt[e] = running;
}

// one block of 1024 threads
__global__ __launch_bounds__(1024) void finalize_kernel(int T, int E, int k, FwdWork w) {
    __shared__ int sc[kMaxExperts];
    __shared__ int sa[kMaxExperts];
    const int tid = threadIdx.x;
    const int c = tid < E ? w.cnt[tid] : 0;
    sc[tid] = c;
    sa[tid] = (tid < E && c > 0) ? 1 : 0;
    __syncthreads();
    // Hillis-Steele inclusive scans of counts and of the active flags
    for (int o = 1; o < kMaxExperts; o <<= 1) {
        const int x = tid >= o ? sc[tid - o] : 0;
        const int y = tid >= o ? sa[tid - o] : 0;
        __syncthreads();
        sc[tid] += x;
        sa[tid] += y;
        __syncthreads();
    }
    if (tid < E) {
        w.off[tid] = sc[tid] - c;
        if (c > 0) w.act[sa[tid] - 1] = tid;
    }
    if (tid == 0) {
        w.off[E] = sc[E - 1];
        w.n_act[0] = sa[E - 1];
    }
    __syncthreads();
    const int P = T * k;
    for (int p = tid; p < P; p += 1024) {
        const int e = w.ids[p];
        const int pos = (sc[e] - w.cnt[e]) + w.rank[p];
        w.pos[p] = pos;
        w.sorted[pos] = p;
    }
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, const FwdWork& w, hipStream_t s) {
    route_kernel<<<(a.T + 3) / 4, 256, 0, s>>>(a, w);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    rank_kernel<<<a.E, 256, 0, s>>>(a.T, a.k, w);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    finalize_kernel<<<1, 1024, 0, s>>>(a.T, a.E, a.k, w);
    return hipGetLastError();
}

}  // namespace pw
