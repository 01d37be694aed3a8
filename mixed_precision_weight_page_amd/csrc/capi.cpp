// C ABI of the per-expert mixed-precision MoE expert layer: context, page
// pool placement, page-table upload, and the order of kernel launches.
// The operations follow the PagedWeight page: Eq. 2 (section
// "Implementation Details") for the quantizer, Eq. 1 (section
// "Quality-Aware Quantization") for the allocation, the page table of
// "Memory Management" and the on-the-fly dequantization of section
// "Dynamic Paging".
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "pw_internal.h"

using namespace pw;

struct pw_ctx {
    pw_layer_desc desc{};
    int E = 0, d = 0, F = 0, k = 0;
    int64_t M = 0;        // F * d weights per matrix
    int nsplit = 1;       // most K-splits of the down product the workspace holds (per pair)
    uint64_t We = 0;      // 3 * M weights per expert
    Layout lay{};

    const void* w1 = nullptr;
    const void* w3 = nullptr;
    const void* w2 = nullptr;
    uint64_t masters_gen = 0;   // bumped by every pw_bind_masters
    uint8_t* pool = nullptr;
    uint64_t pool_cap = 0;
    uint8_t* ws = nullptr;
    uint64_t ws_bytes = 0;
    int dg_parity = 0;    // counter set of the streaming kernels' grouping used by the next forward
    bool dg_clean = false;   // both counter sets cleared since the workspace was bound

    // host tier: with pinned host memory bound, the pages live there and the
    // pool is a cache of page slots (residency state on the device)
    uint8_t* host = nullptr;
    uint64_t host_cap = 0;
    uint8_t* swap_dev = nullptr;

    // host mirror of the page table
    std::vector<pw_page_entry> table;
    bool pages_valid = false;
    uint64_t pages_gen = 0;     // masters generation the pages were packed from

    // per-expert statistics of the bound masters
    bool absmax_valid = false, loss_valid = false;
    std::vector<float> absmax;
    std::vector<double> loss;

    // device state (allocated on first device use)
    int device = -1;
    uint8_t* dev = nullptr;     // two tables (each off/scale/bits/list), absmax, flags, loss
    uint8_t* host_stage = nullptr;   // pinned: table upload + statistics readback
    hipEvent_t upload_done = nullptr;
    int cur = 0;                // active device table

    // budget of the current pages (set by pw_set_budget; the bits' total
    // after pw_quantize_experts) and pw_budget_step calls since they changed
    uint64_t budget_now = 0;
    int32_t steps_since_change = 0;

    // profiling
    int profile_mask = 0;      // bit 0 route, 1 gate/up, 2 down, 3 combine
    std::vector<hipEvent_t> ev_pool;
    std::vector<int> ev_kind;   // kernel class of each (start, stop) pair in use
    size_t ev_used = 0;
    int64_t forwards_timed = 0;

    std::string err;
};

namespace {

constexpr size_t kAlign = 256;
inline uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

pw_status fail(pw_ctx* c, pw_status s, const char* fmt, ...) {
    if (c) {
        char buf[512];
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(buf, sizeof buf, fmt, ap);
        va_end(ap);
        c->err = buf;
        if (getenv("PW_LOG")) fprintf(stderr, "[pagedweight] %s\n", buf);
    }
    return s;
}

#define HIP_TRY(ctx, expr)                                                                    \
    do {                                                                                      \
        hipError_t e_ = (expr);                                                               \
        if (e_ != hipSuccess)                                                                 \
            return fail(ctx, PW_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(e_));     \
    } while (0)

// device block: per table [off u64 E][scale f32 E][bits i32 E][list i32 E]
// [first plane i32 E]
size_t table_bytes(int E) { return align_up((size_t)E * 24, kAlign); }
size_t dev_bytes(int E) { return 2 * table_bytes(E) + align_up((size_t)E * 4 + 16, kAlign) + (size_t)E * 24; }

DevTable dev_table(pw_ctx* c, int which) {
    uint8_t* b = c->dev + which * table_bytes(c->E);
    DevTable t;
    t.off = reinterpret_cast<uint64_t*>(b);
    t.scale = reinterpret_cast<float*>(b + (size_t)c->E * 8);
    t.bits = reinterpret_cast<int32_t*>(b + (size_t)c->E * 12);
    return t;
}
int32_t* dev_list(pw_ctx* c, int which) {
    return reinterpret_cast<int32_t*>(c->dev + which * table_bytes(c->E) + (size_t)c->E * 16);
}
int32_t* dev_first(pw_ctx* c, int which) {
    return reinterpret_cast<int32_t*>(c->dev + which * table_bytes(c->E) + (size_t)c->E * 20);
}
uint32_t* dev_absmax(pw_ctx* c) { return reinterpret_cast<uint32_t*>(c->dev + 2 * table_bytes(c->E)); }
uint32_t* dev_flags(pw_ctx* c) { return dev_absmax(c) + c->E; }
double* dev_loss(pw_ctx* c) {
    return reinterpret_cast<double*>(c->dev + 2 * table_bytes(c->E) + align_up((size_t)c->E * 4 + 16, kAlign));
}

// Host tier helpers. A slot holds any page (the 8-bit page size); at most
// one slot per expert is useful.
bool swap_mode(const pw_ctx* c) { return c->host != nullptr; }
uint64_t slot_bytes(const pw_ctx* c) { return align_up(c->We, kPageAlign); }
int n_slots(const pw_ctx* c) {
    if (!c->pool) return 0;
    return (int)std::min<uint64_t>((uint64_t)c->E, c->pool_cap / slot_bytes(c));
}
uint8_t* page_base(const pw_ctx* c) { return swap_mode(c) ? c->host : c->pool; }
uint64_t page_cap(const pw_ctx* c) { return swap_mode(c) ? c->host_cap : c->pool_cap; }

// residency arrays: addr u64[E], stats u64[3], then i32/u32 slot_of[E],
// expert_of[E], last_use[E], copy_e[E], copy_s[E], step, ncopy
size_t swap_bytes(int E) { return (size_t)E * 8 + 24 + (size_t)E * 20 + 8; }
SwapState swap_state(pw_ctx* c) {
    SwapState st;
    uint8_t* b = c->swap_dev;
    const size_t E = (size_t)c->E;
    st.addr = reinterpret_cast<uint64_t*>(b);
    st.stats = reinterpret_cast<uint64_t*>(b + E * 8);
    int32_t* i = reinterpret_cast<int32_t*>(b + E * 8 + 24);
    st.slot_of = i;
    st.expert_of = i + E;
    st.last_use = reinterpret_cast<uint32_t*>(i + 2 * E);
    st.copy_e = i + 3 * E;
    st.copy_s = i + 4 * E;
    st.step = reinterpret_cast<uint32_t*>(i + 5 * E);
    st.ncopy = i + 5 * E + 1;
    return st;
}

pw_status ensure_device(pw_ctx* c) {
    if (c->dev) {
        int cur = -1;
        HIP_TRY(c, hipGetDevice(&cur));
        if (cur != c->device)
            return fail(c, PW_ERR_STATE, "context belongs to device %d, current device is %d",
                        c->device, cur);
        return PW_OK;
    }
    HIP_TRY(c, hipGetDevice(&c->device));
    void* p = nullptr;
    HIP_TRY(c, hipMalloc(&p, dev_bytes(c->E)));
    c->dev = static_cast<uint8_t*>(p);
    HIP_TRY(c, hipMemset(c->dev, 0, dev_bytes(c->E)));
    void* h = nullptr;
    HIP_TRY(c, hipHostMalloc(&h, dev_bytes(c->E), hipHostMallocDefault));
    c->host_stage = static_cast<uint8_t*>(h);
    HIP_TRY(c, hipEventCreateWithFlags(&c->upload_done, hipEventDisableTiming));
    HIP_TRY(c, hipEventRecord(c->upload_done, nullptr));
    return PW_OK;
}

// Device memory a forward works in: the bound workspace, or the library's
// static scratch (pw_moe_forward_noalloc), with the layout it is carved by.
struct WsView {
    uint8_t* base;
    Layout lay;
    int max_tokens;   // tokens the layout is sized for
    int nsplit;       // K-splits per pair its partial-output buffer holds
};

WsView bound_ws(const pw_ctx* c) { return WsView{c->ws, c->lay, c->desc.max_tokens, c->nsplit}; }

// The forward scratch of a view; `parity` picks the grouping counter set.
FwdWork fwd_work(const pw_ctx* c, const WsView& v, int parity) {
    FwdWork w;
    uint8_t* b = v.base;
    const Layout& L = v.lay;
    w.ids = reinterpret_cast<int32_t*>(b + L.ids);
    w.g = reinterpret_cast<float*>(b + L.g);
    w.rank = reinterpret_cast<int32_t*>(b + L.rank);
    w.sorted = reinterpret_cast<int32_t*>(b + L.sorted);
    w.cnt = reinterpret_cast<int32_t*>(b + L.cnt);
    w.off = reinterpret_cast<int32_t*>(b + L.off);
    w.act = reinterpret_cast<int32_t*>(b + L.act);
    w.n_act = reinterpret_cast<int32_t*>(b + L.n_act);
    w.tiles = reinterpret_cast<TileDesc*>(b + L.tiles);
    // the two counter sets: cnt [E], act [E], n_act [2], each set 256-byte aligned
    auto set = [&](int i) {
        uint8_t* q = b + L.dg + (uint64_t)i * (L.dg_bytes / 2);
        DecodeGroup g;
        g.cnt = reinterpret_cast<int32_t*>(q);
        g.act = g.cnt + c->E;
        g.n_act = g.act + c->E;
        g.list = reinterpret_cast<int32_t*>(b + L.list);
        g.E = c->E;
        return g;
    };
    w.dg = set(parity);
    w.dg_next = set(1 - parity);
    w.tcap = std::max(v.max_tokens, 16);
    w.ccnt = reinterpret_cast<int32_t*>(b + L.ccnt);
    w.cpre = reinterpret_cast<int32_t*>(b + L.cpre);
    w.xst = reinterpret_cast<XStat*>(b + L.xst);
    w.H = reinterpret_cast<_Float16*>(b + L.H);
    w.O = reinterpret_cast<float*>(b + L.O);
    return w;
}

// Empty slots, nothing used yet, counters zero (ordered before later work
// on any stream: hipMemset is synchronous with respect to the host).
pw_status reset_swap(pw_ctx* c) {
    const SwapState st = swap_state(c);
    HIP_TRY(c, hipMemset(c->swap_dev, 0, swap_bytes(c->E)));
    HIP_TRY(c, hipMemset(st.slot_of, 0xff, (size_t)c->E * 8));   // slot_of and expert_of
    return PW_OK;
}

// s = the fp32 value nearest m / qmax; bitplane pages use Eq. 2's 8-bit
// scale s8 at every depth
float scale_for(const pw_ctx* c, float m, int b) {
    if (c->desc.layout == PW_LAYOUT_BITPLANE) b = 8;
    return m == 0.0f ? 0.0f : (float)((double)m / (double)qmax_of(b));
}

// bit-widths a page may have: {3, 4, 8} (Eq. 2), depths 1..8 (bitplane)
bool bits_ok(const pw_ctx* c, int b) {
    return c->desc.layout == PW_LAYOUT_BITPLANE ? (b >= 1 && b <= 8) : bits_index(b) >= 0;
}

uint64_t page_bytes(const pw_ctx* c, int b) { return align_up(c->We * (uint64_t)b / 8, kPageAlign); }

// max|w| per expert (one stream synchronisation per binding of the masters)
pw_status ensure_absmax(pw_ctx* c, hipStream_t s) {
    if (c->absmax_valid) return PW_OK;
    const int f16 = c->desc.master_dtype == PW_MASTER_F16;
    HIP_TRY(c, hipMemsetAsync(dev_absmax(c), 0, (size_t)c->E * 4 + 16, s));
    HIP_TRY(c, launch_absmax(c->w1, c->w3, c->w2, f16, c->E, c->M, dev_absmax(c), dev_flags(c), s));
    HIP_TRY(c, hipEventSynchronize(c->upload_done));
    HIP_TRY(c, hipMemcpyAsync(c->host_stage, dev_absmax(c), (size_t)c->E * 4 + 16,
                              hipMemcpyDeviceToHost, s));
    HIP_TRY(c, hipStreamSynchronize(s));
    const uint32_t* h = reinterpret_cast<const uint32_t*>(c->host_stage);
    if (h[c->E] != 0) return fail(c, PW_ERR_NONFINITE_WEIGHTS, "masters contain NaN or Inf");
    c->absmax.resize(c->E);
    for (int e = 0; e < c->E; ++e) {
        uint32_t u = h[e];
        float f;
        std::memcpy(&f, &u, 4);
        c->absmax[e] = f;
    }
    c->absmax_valid = true;
    return PW_OK;
}

pw_status ensure_loss(pw_ctx* c, hipStream_t s) {
    if (c->loss_valid) return PW_OK;
    pw_status st = ensure_absmax(c, s);
    if (st != PW_OK) return st;
    if (!c->ws || c->ws_bytes < c->lay.total)
        return fail(c, PW_ERR_WORKSPACE, "measuring losses needs a workspace of %llu bytes",
                    (unsigned long long)c->lay.total);
    const int f16 = c->desc.master_dtype == PW_MASTER_F16;
    HIP_TRY(c, launch_loss(c->w1, c->w3, c->w2, f16, c->E, c->M, dev_absmax(c),
                           reinterpret_cast<double*>(c->ws + c->lay.partial), dev_loss(c),
                           c->desc.layout == PW_LAYOUT_BITPLANE ? 1 : 0, s));
    HIP_TRY(c, hipEventSynchronize(c->upload_done));
    HIP_TRY(c, hipMemcpyAsync(c->host_stage, dev_loss(c), (size_t)c->E * 24, hipMemcpyDeviceToHost, s));
    HIP_TRY(c, hipStreamSynchronize(s));
    c->loss.assign(reinterpret_cast<const double*>(c->host_stage),
                   reinterpret_cast<const double*>(c->host_stage) + 3 * c->E);
    c->loss_valid = true;
    return PW_OK;
}

// Bytes the pages span: the end of the highest page (0 without pages).
uint64_t extent_of(const pw_ctx* c, const std::vector<pw_page_entry>& t) {
    uint64_t end = 0;
    for (int e = 0; e < c->E; ++e)
        if (t[e].bits) end = std::max(end, t[e].offset + page_bytes(c, t[e].bits));
    return end;
}

bool bitplane(const pw_ctx* c) { return c->desc.layout == PW_LAYOUT_BITPLANE; }

// Place the pages of the new allocation; `pack` receives (expert, first
// plane to write) for every page that needs writing (Eq. 2 pages: always
// from plane 0, i.e. the whole page). Unchanged experts keep their pages.
// Eq. 2 pages whose width changes go first-fit (largest first) into the
// space the kept pages leave, lowest addresses first. Bitplane pages whose
// depth drops keep their place and lose their last planes (nothing is
// written: a shallower page is a prefix of the deeper one); those whose
// depth grows get their missing planes written after the ones they have
// when the bytes there are free, else go first-fit like Eq. 2 pages and
// are written whole. If placement fails, or leaves the pages spanning more
// than max_extent bytes, every page is rewritten densely in expert order
// (compaction: the pages then occupy the head of the pool, exactly their
// total size).
pw_status place(pw_ctx* c, const uint8_t* bits, std::vector<pw_page_entry>& nt,
                std::vector<std::pair<int32_t, int32_t>>& pack, uint64_t max_extent) {
    const int E = c->E;
    const bool fresh = !c->pages_valid || c->pages_gen != c->masters_gen;
    const bool bp = bitplane(c);
    nt.assign(E, pw_page_entry{});
    // 0: keep, 1: place anew (whole page), 2: bitplane page grown (in place
    // if possible)
    std::vector<char> kind(E, 1);
    for (int e = 0; e < E; ++e) {
        nt[e].bits = bits[e];
        nt[e].nbytes = c->We * bits[e] / 8;
        nt[e].scale = scale_for(c, c->absmax[e], bits[e]);
        if (fresh) continue;
        const int old = c->table[e].bits;
        if (old == bits[e] || (bp && bits[e] < old)) {
            kind[e] = 0;
            nt[e].offset = c->table[e].offset;
        } else if (bp) {
            kind[e] = 2;
        }
    }
    pack.clear();
    bool ok = !fresh;
    if (ok) {
        std::vector<std::pair<uint64_t, uint64_t>> used;
        for (int e = 0; e < E; ++e)
            if (kind[e] == 0) used.push_back({nt[e].offset, nt[e].offset + page_bytes(c, bits[e])});
        // grown bitplane pages first try to extend where they are
        auto overlaps = [&](uint64_t lo, uint64_t hi) {
            for (auto& u : used)
                if (lo < u.second && u.first < hi) return true;
            return false;
        };
        for (int e = 0; e < E; ++e) {
            if (kind[e] != 2) continue;
            const uint64_t lo = c->table[e].offset, hi = lo + page_bytes(c, bits[e]);
            if (hi <= page_cap(c) && !overlaps(lo, hi)) {
                nt[e].offset = lo;
                used.push_back({lo, hi});
                pack.push_back({e, (int32_t)c->table[e].bits});
                kind[e] = 0;
            } else {
                kind[e] = 1;
            }
        }
        std::sort(used.begin(), used.end());
        std::vector<std::pair<uint64_t, uint64_t>> holes;
        uint64_t at = 0;
        for (auto& u : used) {
            if (u.first > at) holes.push_back({at, u.first});
            at = std::max(at, u.second);
        }
        if (page_cap(c) > at) holes.push_back({at, page_cap(c)});
        std::vector<int> order;
        for (int e = 0; e < E; ++e)
            if (kind[e] == 1) order.push_back(e);
        std::stable_sort(order.begin(), order.end(),
                         [&](int a, int b) { return bits[a] > bits[b]; });
        for (int e : order) {
            const uint64_t need = page_bytes(c, bits[e]);
            bool placed = false;
            for (auto& h : holes) {
                if (h.second - h.first >= need) {
                    nt[e].offset = h.first;
                    h.first += need;
                    placed = true;
                    pack.push_back({e, 0});
                    break;
                }
            }
            if (!placed) { ok = false; break; }
        }
        if (ok && extent_of(c, nt) > max_extent) ok = false;
    }
    if (!ok) {
        pack.clear();
        uint64_t at = 0;
        for (int e = 0; e < E; ++e) {
            nt[e].offset = at;
            at += page_bytes(c, bits[e]);
            pack.push_back({e, 0});
        }
        if (at > page_cap(c))
            return fail(c, PW_ERR_POOL_CAPACITY, "pages need %llu bytes, %s holds %llu",
                        (unsigned long long)at, swap_mode(c) ? "host tier" : "pool",
                        (unsigned long long)page_cap(c));
    }
    std::sort(pack.begin(), pack.end());
    return PW_OK;
}

// Quantize at the given bits: place, upload the new table (into the idle
// device copy), pack the changed experts, then make the new table current.
pw_status apply_bits(pw_ctx* c, const uint8_t* bits, hipStream_t s, uint64_t max_extent = UINT64_MAX) {
    std::vector<pw_page_entry> nt;
    std::vector<std::pair<int32_t, int32_t>> pack;
    pw_status st = place(c, bits, nt, pack, max_extent);
    if (st != PW_OK) return st;
    const int E = c->E;
    bool same = c->pages_valid && c->pages_gen == c->masters_gen;
    for (int e = 0; same && e < E; ++e)
        same = nt[e].bits == c->table[e].bits && nt[e].offset == c->table[e].offset;
    if (same) return PW_OK;
    const int n = (int)pack.size();
    const int next = 1 - c->cur;
    HIP_TRY(c, hipEventSynchronize(c->upload_done));   // staging buffer free again
    uint8_t* h = c->host_stage;
    for (int e = 0; e < E; ++e) {
        std::memcpy(h + (size_t)e * 8, &nt[e].offset, 8);
        std::memcpy(h + (size_t)E * 8 + (size_t)e * 4, &nt[e].scale, 4);
        const int32_t b = nt[e].bits;
        std::memcpy(h + (size_t)E * 12 + (size_t)e * 4, &b, 4);
    }
    for (int i = 0; i < n; ++i) {
        std::memcpy(h + (size_t)E * 16 + (size_t)i * 4, &pack[i].first, 4);
        std::memcpy(h + (size_t)E * 20 + (size_t)i * 4, &pack[i].second, 4);
    }
    c->pages_valid = false;   // until the pack is enqueued
    HIP_TRY(c, hipMemcpyAsync(dev_table(c, next).off, h, (size_t)E * 24, hipMemcpyHostToDevice, s));
    HIP_TRY(c, hipEventRecord(c->upload_done, s));
    const int f16 = c->desc.master_dtype == PW_MASTER_F16;
    HIP_TRY(c, launch_pack(c->w1, c->w3, c->w2, f16, c->d, c->F, dev_table(c, next), dev_list(c, next),
                           dev_first(c, next), n, bitplane(c) ? 1 : 0, page_base(c), s));
    // rewritten pages: their slot copies are stale (a bitplane page that only
    // lost planes keeps a valid slot: its planes are a prefix of the slot's)
    if (swap_mode(c)) HIP_TRY(c, launch_swap_invalidate(swap_state(c), dev_list(c, next), n, s));
    c->table = nt;
    c->cur = next;
    c->pages_valid = true;
    c->pages_gen = c->masters_gen;
    return PW_OK;
}

pw_status check_bits(pw_ctx* c, const uint8_t* bits) {
    if (!bits) return fail(c, PW_ERR_INVALID_ARG, "bits is NULL");
    for (int e = 0; e < c->E; ++e)
        if (!bits_ok(c, bits[e]))
            return fail(c, PW_ERR_UNSUPPORTED_BITS, "expert %d: %d bits (supported: %s)", e, (int)bits[e],
                        c->desc.layout == PW_LAYOUT_BITPLANE ? "depths 1 to 8" : "3, 4, 8");
    return PW_OK;
}

pw_status need_masters_pool(pw_ctx* c) {
    if (!c->w1 || !c->w3 || !c->w2) return fail(c, PW_ERR_STATE, "no masters bound");
    if (!swap_mode(c) && !c->pool) return fail(c, PW_ERR_STATE, "no pool bound");
    return PW_OK;
}

// Profiling events only carry timestamps, so they are created without the
// system-scope fence (a cache writeback and invalidate at each record).
hipEvent_t next_event(pw_ctx* c) {
    if (c->ev_used == c->ev_pool.size()) {
        hipEvent_t e;
        if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
        c->ev_pool.push_back(e);
    }
    return c->ev_pool[c->ev_used++];
}

}  // namespace

namespace pw {
Layout workspace_layout(int E, int d, int F, int k, int max_tokens, int nsplit) {
    Layout L{};
    const uint64_t P = (uint64_t)max_tokens * k;
    uint64_t at = 0;
    auto take = [&](uint64_t bytes) {
        const uint64_t o = at;
        at = align_up(at + bytes, kAlign);
        return o;
    };
    const uint64_t scratch = at;
    // forward scratch
    L.ids = take(4 * P);
    L.g = take(4 * P);
    L.rank = take(4 * P);
    L.sorted = take(4 * P);
    L.cnt = take(4 * (uint64_t)E);
    L.off = take(4 * (uint64_t)(E + 1));
    L.act = take(4 * (uint64_t)E);
    L.n_act = take(8);
    L.tiles = take(sizeof(TileDesc) * ((P + kGemmTokens - 1) / kGemmTokens + (uint64_t)E));
    const uint64_t chunks = ((uint64_t)max_tokens + kRankChunk - 1) / kRankChunk;
    L.ccnt = take(4 * (uint64_t)E * chunks);
    L.cpre = take(4 * (uint64_t)E * chunks);
    L.xst = take(sizeof(XStat) * (uint64_t)max_tokens);
    L.H = take(2 * P * (uint64_t)F);
    L.O = take(4 * (uint64_t)nsplit * P * (uint64_t)d);
    L.xp = take(2 * 3 * (uint64_t)max_tokens * (uint64_t)d);
    // pair lists of the streaming kernels: at least 16 entries per expert
    L.list = take(4 * (uint64_t)E * (uint64_t)std::max(max_tokens, 16));
    L.fwd_end = at;
    // the loss pass reuses the forward scratch (calls on one stream are ordered)
    const uint64_t nblk = 3 * (uint64_t)F * d / kStatChunk;
    L.partial = scratch;
    L.stats_end = scratch + align_up(8 * 3 * nblk * (uint64_t)E, kAlign);
    // the grouping counters keep their values between forwards: after
    // everything the statistics pass may overwrite
    L.dg_bytes = 2 * align_up(4 * (2 * (uint64_t)E + 2), kAlign);
    L.dg = std::max(L.fwd_end, L.stats_end);
    L.total = L.dg + L.dg_bytes;
    return L;
}
}  // namespace pw

extern "C" {

const char* pw_status_str(int32_t s) {
    switch (s) {
        case PW_OK: return "ok";
        case PW_ERR_INVALID_ARG: return "invalid argument";
        case PW_ERR_UNSUPPORTED_BITS: return "unsupported bit-width";
        case PW_ERR_INFEASIBLE_BUDGET: return "infeasible budget";
        case PW_ERR_NONFINITE_WEIGHTS: return "non-finite weights";
        case PW_ERR_POOL_CAPACITY: return "pool capacity exceeded";
        case PW_ERR_WORKSPACE: return "workspace missing or too small";
        case PW_ERR_STATE: return "call out of order";
        case PW_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

pw_status pw_create(const pw_layer_desc* desc, pw_ctx** out) {
    if (!desc || !out) return PW_ERR_INVALID_ARG;
    *out = nullptr;
    const pw_layer_desc& d = *desc;
    if (d.num_experts < 1 || d.num_experts > kMaxExperts || d.d_model < kRowAlign ||
        d.d_ff < kRowAlign || d.d_model % kRowAlign || d.d_ff % kRowAlign || d.top_k < 1 ||
        d.top_k > kMaxTopK || d.top_k > d.num_experts || d.max_tokens < 0 ||
        (d.renorm != 0 && d.renorm != 1) ||
        (d.master_dtype != PW_MASTER_F32 && d.master_dtype != PW_MASTER_F16) ||
        (d.layout != PW_LAYOUT_EQ2 && d.layout != PW_LAYOUT_BITPLANE))
        return PW_ERR_INVALID_ARG;
    if ((int64_t)d.max_tokens * d.top_k > (int64_t)1 << 30) return PW_ERR_INVALID_ARG;
    pw_ctx* c = new (std::nothrow) pw_ctx;
    if (!c) return PW_ERR_INVALID_ARG;
    c->desc = d;
    c->E = d.num_experts;
    c->d = d.d_model;
    c->F = d.d_ff;
    c->k = d.top_k;
    c->M = (int64_t)d.d_model * d.d_ff;
    c->We = 3 * (uint64_t)c->M;
    // partial-output buffers for the down product's K splits: room for the
    // splits a single routed expert would want (the most any forward takes),
    // unless the batch is large (then the buffer of max_tokens k d floats is
    // big enough on its own: a forward's split stride is its own pair count,
    // so small batches split within it)
    const int64_t max_pairs = (int64_t)d.max_tokens * d.top_k;
    c->nsplit = max_pairs > 2048 ? 1 : down_splits(c->F, c->d, 1, 1 << 30);
    c->lay = workspace_layout(c->E, c->d, c->F, c->k, d.max_tokens, c->nsplit);
    c->table.assign(c->E, pw_page_entry{});
    *out = c;
    return PW_OK;
}

void pw_destroy(pw_ctx* c) {
    if (!c) return;
    for (hipEvent_t e : c->ev_pool) (void)hipEventDestroy(e);
    if (c->upload_done) {
        (void)hipEventSynchronize(c->upload_done);
        (void)hipEventDestroy(c->upload_done);
    }
    if (c->host_stage) (void)hipHostFree(c->host_stage);
    if (c->swap_dev) (void)hipFree(c->swap_dev);
    if (c->dev) (void)hipFree(c->dev);
    delete c;
}

pw_status pw_bind_masters(pw_ctx* c, const void* w1, const void* w3, const void* w2) {
    if (!c) return PW_ERR_INVALID_ARG;
    if (!w1 || !w3 || !w2) return fail(c, PW_ERR_INVALID_ARG, "null master pointer");
    const uintptr_t a = 16;
    if ((uintptr_t)w1 % a || (uintptr_t)w3 % a || (uintptr_t)w2 % a)
        return fail(c, PW_ERR_INVALID_ARG, "masters must be 16-byte aligned");
    c->w1 = w1;
    c->w3 = w3;
    c->w2 = w2;
    c->masters_gen++;
    c->absmax_valid = c->loss_valid = false;
    return PW_OK;
}

uint64_t pw_pool_bytes_for_bits(const pw_ctx* c, const uint8_t* bits) {
    if (!c || !bits) return 0;
    uint64_t t = 0;
    for (int e = 0; e < c->E; ++e) {
        if (!bits_ok(c, bits[e])) return 0;
        t += page_bytes(c, bits[e]);
    }
    return t;
}

pw_status pw_bind_pool(pw_ctx* c, void* pool, uint64_t cap) {
    if (!c) return PW_ERR_INVALID_ARG;
    if (!pool || (uintptr_t)pool % kPageAlign)
        return fail(c, PW_ERR_INVALID_ARG, "pool must be non-NULL and 256-byte aligned");
    c->pool = static_cast<uint8_t*>(pool);
    c->pool_cap = cap;
    if (swap_mode(c)) return reset_swap(c);   // pages stay in the host tier; slots start empty
    c->pages_valid = false;
    c->table.assign(c->E, pw_page_entry{});
    return PW_OK;
}

pw_status pw_bind_host_tier(pw_ctx* c, void* host, uint64_t bytes) {
    if (!c) return PW_ERR_INVALID_ARG;
    if (host && (uintptr_t)host % kPageAlign)
        return fail(c, PW_ERR_INVALID_ARG, "host tier must be 256-byte aligned");
    pw_status st = ensure_device(c);
    if (st != PW_OK) return st;
    c->pages_valid = false;
    c->table.assign(c->E, pw_page_entry{});
    if (!host) {
        c->host = nullptr;
        c->host_cap = 0;
        return PW_OK;
    }
    // the kernels read and write the tier directly: it must be pinned host
    // memory mapped into the device's address space at the same address
    // (first and last byte)
    for (const uint8_t* q : {static_cast<const uint8_t*>(host), static_cast<const uint8_t*>(host) + (bytes ? bytes - 1 : 0)}) {
        hipPointerAttribute_t at{};
        if (hipPointerGetAttributes(&at, q) != hipSuccess || at.type != hipMemoryTypeHost ||
            at.devicePointer != (const void*)q) {
            (void)hipGetLastError();
            return fail(c, PW_ERR_INVALID_ARG, "host tier must be pinned, device-mapped host memory (hipHostMalloc)");
        }
    }
    if (!c->swap_dev) {
        void* p = nullptr;
        HIP_TRY(c, hipMalloc(&p, swap_bytes(c->E)));
        c->swap_dev = static_cast<uint8_t*>(p);
    }
    c->host = static_cast<uint8_t*>(host);
    c->host_cap = bytes;
    return reset_swap(c);
}

pw_status pw_get_residency(pw_ctx* c, int32_t* slot_of, uint64_t* stats, void* stream) {
    if (!c) return PW_ERR_INVALID_ARG;
    if (!swap_mode(c)) return fail(c, PW_ERR_STATE, "no host tier bound");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const SwapState st = swap_state(c);
    HIP_TRY(c, hipEventSynchronize(c->upload_done));   // staging buffer free
    HIP_TRY(c, hipMemcpyAsync(c->host_stage, st.slot_of, (size_t)c->E * 4, hipMemcpyDeviceToHost, s));
    HIP_TRY(c, hipMemcpyAsync(c->host_stage + (size_t)c->E * 4, st.stats, 24, hipMemcpyDeviceToHost, s));
    HIP_TRY(c, hipStreamSynchronize(s));
    if (slot_of) std::memcpy(slot_of, c->host_stage, (size_t)c->E * 4);
    if (stats) std::memcpy(stats, c->host_stage + (size_t)c->E * 4, 24);
    return PW_OK;
}

uint64_t pw_workspace_bytes(const pw_ctx* c) { return c ? c->lay.total : 0; }

pw_status pw_bind_workspace(pw_ctx* c, void* ws, uint64_t bytes) {
    if (!c) return PW_ERR_INVALID_ARG;
    if (!ws || (uintptr_t)ws % kAlign) return fail(c, PW_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    if (bytes < c->lay.total)
        return fail(c, PW_ERR_WORKSPACE, "workspace of %llu bytes, need %llu",
                    (unsigned long long)bytes, (unsigned long long)c->lay.total);
    c->ws = static_cast<uint8_t*>(ws);
    c->ws_bytes = bytes;
    c->dg_parity = 0;
    c->dg_clean = false;   // cleared by the first streaming forward's stream
    return PW_OK;
}

pw_status pw_quantize_experts(pw_ctx* c, const uint8_t* bits, void* stream) {
    if (!c) return PW_ERR_INVALID_ARG;
    pw_status st = check_bits(c, bits);
    if (st != PW_OK) return st;
    if ((st = need_masters_pool(c)) != PW_OK) return st;
    uint64_t need = 0;
    for (int e = 0; e < c->E; ++e) need += page_bytes(c, bits[e]);
    if (need > page_cap(c))
        return fail(c, PW_ERR_POOL_CAPACITY, "pages need %llu bytes, %s holds %llu",
                    (unsigned long long)need, swap_mode(c) ? "host tier" : "pool",
                    (unsigned long long)page_cap(c));
    if ((st = ensure_device(c)) != PW_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = ensure_absmax(c, s)) != PW_OK) return st;
    if ((st = apply_bits(c, bits, s)) != PW_OK) return st;
    c->budget_now = 0;
    for (int e = 0; e < c->E; ++e) c->budget_now += (uint64_t)bits[e] * c->We;
    c->steps_since_change = 0;
    return PW_OK;
}

// pw_set_budget with an extent the placement keeps the pages within when it
// can (the KV-pressure scheduler passes the bytes the KV cache leaves).
static pw_status set_budget(pw_ctx* c, uint64_t budget_bits, const double* importance, const double* loss,
                            uint8_t* bits_out, void* stream, uint64_t max_extent) {
    if (!c) return PW_ERR_INVALID_ARG;
    if (!importance) return fail(c, PW_ERR_INVALID_ARG, "importance is NULL");
    pw_status st = need_masters_pool(c);
    if (st != PW_OK) return st;
    if (budget_bits < 3 * c->We * (uint64_t)c->E)
        return fail(c, PW_ERR_INFEASIBLE_BUDGET, "budget %llu bits < 3 bits per weight",
                    (unsigned long long)budget_bits);
    if ((st = ensure_device(c)) != PW_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = ensure_absmax(c, s)) != PW_OK) return st;
    const double* L = loss;
    if (!L) {
        if ((st = ensure_loss(c, s)) != PW_OK) return st;
        L = c->loss.data();
    }
    std::vector<uint64_t> W(c->E, c->We);
    std::vector<uint8_t> bits(c->E);
    st = solve_allocation(c->E, W.data(), importance, L, budget_bits, bits.data(), &c->err);
    if (st != PW_OK) return st;
    if ((st = apply_bits(c, bits.data(), s, max_extent)) != PW_OK) return st;
    c->budget_now = budget_bits;
    c->steps_since_change = 0;
    if (bits_out) std::memcpy(bits_out, bits.data(), c->E);
    return PW_OK;
}

pw_status pw_set_budget(pw_ctx* c, uint64_t budget_bits, const double* importance,
                        const double* loss, uint8_t* bits_out, void* stream) {
    return set_budget(c, budget_bits, importance, loss, bits_out, stream, UINT64_MAX);
}

uint64_t pw_pool_used_bytes(const pw_ctx* c) { return c && c->pages_valid ? extent_of(c, c->table) : 0; }

pw_status pw_budget_step(pw_ctx* c, const pw_budget_policy* policy, uint64_t kv_used_bytes,
                         const double* importance, const double* loss, int32_t* action,
                         uint64_t* budget_out, int32_t* pressure, void* stream) {
    if (!c) return PW_ERR_INVALID_ARG;
    if (!policy || !importance || !action || !budget_out || !pressure)
        return fail(c, PW_ERR_INVALID_ARG, "null policy, importance or output pointer");
    // the pool's size for the decision is the span of its pages (a page
    // above the memory the KV cache leaves overlaps it, holes or not)
    const uint64_t pool_now = c->pages_valid ? extent_of(c, c->table) : UINT64_MAX;
    std::vector<uint64_t> W(c->E, c->We);
    int32_t act = PW_BUDGET_KEEP, press = 0;
    uint64_t target = 0;
    pw_status st = pw_budget_decide(policy, kv_used_bytes, c->E, W.data(), pool_now, c->budget_now,
                                    c->steps_since_change, &act, &target, &press);
    if (st != PW_OK) return fail(c, st, "invalid budget policy");
    if (act != PW_BUDGET_KEEP) {
        // the new pages stay within the memory the KV cache leaves (compacted
        // if first-fit placement would reach above it)
        uint64_t avail = 0;
        if (policy->memory_bytes > kv_used_bytes && policy->memory_bytes - kv_used_bytes > policy->reserve_bytes)
            avail = policy->memory_bytes - kv_used_bytes - policy->reserve_bytes;
        if ((st = set_budget(c, target, importance, loss, nullptr, stream, avail)) != PW_OK) return st;
    } else {
        c->steps_since_change++;
    }
    *action = act;
    *budget_out = target;
    *pressure = press;
    return PW_OK;
}

// Whether a batch of T tokens takes the matrix-core kernels: many tokens per
// routed expert (weights read once per 64 tokens); else the streaming kernels
// (weights read once).
static bool dense_path(const pw_ctx* c, int32_t T) {
    if (c->desc.layout == PW_LAYOUT_BITPLANE) return false;   // the streaming kernels decode bitplanes
    const int64_t pairs = (int64_t)T * c->k;
    const int64_t max_act = std::min<int64_t>(c->E, pairs);
    return gemm_supported(c->d, c->F) && pairs >= (int64_t)kGemmMinTokens * max_act;
}

// Router and grouping for the path of the batch. The streaming kernels'
// router also takes the token statistics (x may be NULL: none). With the
// bound workspace it uses the current counter set and the next forward the
// other one (both cleared once after binding); the static scratch, shared by
// every context on the device, has both sets cleared at each call. Returns
// the per-expert counts.
static pw_status route_batch(pw_ctx* c, const WsView& v, const FwdWork& w, const float* logits, const void* x,
                             int32_t T, bool dense, bool scratch, hipStream_t s, KTimer t,
                             const int32_t** counts, int own_route = 0) {
    // bitplane pages: the streaming router lists the experts deeper than 4
    // planes first (their workgroups decode the most planes per row and run
    // longest: dispatched first, measured 7% faster on the 128-expert decode
    // layer); Eq. 2 pages keep arrival order (heavy-first measured 2% slower)
    RouteArgs ra{logits, static_cast<const uint16_t*>(x), c->d, T, c->E, c->k, c->desc.renorm, 1,
                 bitplane(c) ? dev_table(c, c->cur).bits : nullptr};
    if (dense) {
        ra.x = nullptr;   // prep_x takes the statistics on this path
        HIP_TRY(c, launch_route(ra, w, dev_table(c, c->cur), s, t));
        *counts = w.cnt;
        return PW_OK;
    }
    if (scratch || !c->dg_clean) {
        // a kernel, not a memset: the stream may be under graph capture
        HIP_TRY(c, launch_zero_i32(reinterpret_cast<int32_t*>(v.base + v.lay.dg), v.lay.dg_bytes / 4, s));
        if (!scratch) c->dg_clean = true;
    }
    if (own_route == 1) {
        // the gate/up kernel routes this batch and fills the counter set
        // (the timing events, if any, enclose no work)
        if (t.start) HIP_TRY(c, hipEventRecord(t.start, s));
        if (t.stop) HIP_TRY(c, hipEventRecord(t.stop, s));
    } else {
        // own_route 2: the gate/up kernel groups the pairs of these ids
        ra.group = own_route == 2 ? 0 : 1;
        HIP_TRY(c, launch_route_decode(ra, w, s, t));
    }
    if (!scratch) c->dg_parity ^= 1;
    *counts = w.dg.cnt;
    return PW_OK;
}

static pw_status forward_checks(pw_ctx* c, const void* logits, int32_t T) {
    if (T < 0 || T > c->desc.max_tokens)
        return fail(c, PW_ERR_INVALID_ARG, "T = %d outside [0, %d]", T, c->desc.max_tokens);
    if (T > 0 && !logits) return fail(c, PW_ERR_INVALID_ARG, "null logits");
    if (!c->ws) return fail(c, PW_ERR_WORKSPACE, "no workspace bound");
    return PW_OK;
}

pw_status pw_route(pw_ctx* c, const float* logits, int32_t T, int32_t* ids, float* g,
                   int32_t* counts, void* stream) {
    if (!c) return PW_ERR_INVALID_ARG;
    pw_status st = forward_checks(c, logits, T);
    if (st != PW_OK) return st;
    if (T == 0) return PW_OK;
    if (!ids || !g || !counts) return fail(c, PW_ERR_INVALID_ARG, "null output pointer");
    if ((st = ensure_device(c)) != PW_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const WsView v = bound_ws(c);
    const FwdWork w = fwd_work(c, v, c->dg_parity);
    const int32_t* cnt = nullptr;
    if ((st = route_batch(c, v, w, logits, nullptr, T, dense_path(c, T), false, s, KTimer{}, &cnt)) != PW_OK)
        return st;
    const size_t P = (size_t)T * c->k;
    HIP_TRY(c, hipMemcpyAsync(ids, w.ids, P * 4, hipMemcpyDeviceToDevice, s));
    HIP_TRY(c, hipMemcpyAsync(g, w.g, P * 4, hipMemcpyDeviceToDevice, s));
    HIP_TRY(c, hipMemcpyAsync(counts, cnt, (size_t)c->E * 4, hipMemcpyDeviceToDevice, s));
    return PW_OK;
}

// The forward over a workspace view (a1-a5: route and group, gate/up +
// SwiGLU, down, combine). `scratch`: the view is the static scratch (no
// timing events, counters cleared at each call).
static pw_status forward_core(pw_ctx* c, const WsView& v, const void* x, const float* logits, int32_t T,
                              float* y, hipStream_t s, bool scratch) {
    const FwdWork w = fwd_work(c, v, scratch ? 0 : c->dg_parity);
    KTimer tm[4];
    if (c->profile_mask && !scratch) {
        for (int j = 0; j < 4; ++j) {
            if (!((c->profile_mask >> j) & 1)) continue;
            tm[j].start = next_event(c);
            tm[j].stop = next_event(c);
            if (!tm[j].start || !tm[j].stop) return fail(c, PW_ERR_HIP, "hipEventCreate failed");
            c->ev_kind.push_back(j);
        }
    }
    const int64_t pairs = (int64_t)T * c->k;
    const int max_act = (int)std::min<int64_t>(c->E, pairs);
    const bool dense = dense_path(c, T);
    // small decode batches are routed by the gate/up kernel itself (not with
    // a host tier: its plan needs the counts before the expert kernels)
    const int own_route = (!dense && !swap_mode(c)) ? own_route_mode(T, c->E, c->k) : 0;
    const int32_t* cnt = nullptr;
    pw_status st = route_batch(c, v, w, logits, x, T, dense, scratch, s, tm[0], &cnt, own_route);
    if (st != PW_OK) return st;
    // pages: pool + offset, or with a host tier the addresses of this pass
    // (slot or host tier) after the missing pages are copied in
    const uint8_t* base = c->pool;
    DevTable tab = dev_table(c, c->cur);
    if (swap_mode(c)) {
        const SwapState ss = swap_state(c);
        const int S = n_slots(c);
        HIP_TRY(c, launch_swap_in(ss, cnt, tab, c->E, S, std::min(S, max_act), c->We, c->pool, c->host,
                                  slot_bytes(c), s));
        tab.off = ss.addr;
        base = nullptr;
    }
    // partial outputs of the down product: O[split][pair][d] with this
    // batch's pair count as the split stride, so a view sized for large
    // batches splits small ones as far as its buffer allows
    const int P = (int)pairs;
    if (dense) {
        GemmArgs ga;
        ga.pool = base;
        ga.tab = tab;
        ga.w = w;
        ga.x = static_cast<const uint16_t*>(x);
        ga.d = c->d;
        ga.F = c->F;
        ga.k = c->k;
        ga.max_act = max_act;
        ga.P_used = pairs;
        ga.T = T;
        ga.xp = reinterpret_cast<const _Float16*>(v.base + v.lay.xp);
        ga.xp_plane = (int64_t)v.max_tokens * c->d;
        ga.bits_mask = 0;
        for (int e = 0; e < c->E; ++e) ga.bits_mask |= 1 << bits_index(c->table[e].bits);
        HIP_TRY(c, launch_prep_x(ga, s));
        HIP_TRY(c, launch_gate_up_gemm(ga, s, tm[1]));
        HIP_TRY(c, launch_down_gemm(ga, s, tm[2]));
        HIP_TRY(c, launch_combine(w, T, c->d, c->k, P, 1, y, s, tm[3]));
    } else {
        FfnArgs fa;
        fa.pool = base;
        fa.tab = tab;
        fa.w = w;
        fa.x = static_cast<const uint16_t*>(x);
        fa.d = c->d;
        fa.F = c->F;
        fa.k = c->k;
        fa.max_act = max_act;
        fa.P = P;
        fa.bitplane = c->desc.layout == PW_LAYOUT_BITPLANE ? 1 : 0;
        // an expert may receive more than 16 tokens
        fa.wide = T > 16 ? 1 : 0;
        fa.own_route = own_route;
        fa.logits = logits;
        fa.T = T;
        fa.E = c->E;
        fa.renorm = c->desc.renorm;
        // K splits of the down product for this batch, within the buffer
        const int64_t cap_pairs = (int64_t)v.nsplit * v.max_tokens * c->k;
        const int nsplit = down_splits(c->F, c->d, max_act, (int)std::min<int64_t>(cap_pairs / pairs, 1 << 30));
        HIP_TRY(c, launch_gate_up(fa, plan_ffn(c->d, T, 1), s, tm[1]));
        HIP_TRY(c, launch_down(fa, plan_ffn(c->F, T, nsplit), s, tm[2]));
        HIP_TRY(c, launch_combine(w, T, c->d, c->k, P, nsplit, y, s, tm[3]));
    }
    if (c->profile_mask && !scratch) c->forwards_timed++;
    return PW_OK;
}

static pw_status forward_args(pw_ctx* c, const void* x, const float* logits, int32_t T, const float* y) {
    if (!c->pages_valid) return fail(c, PW_ERR_STATE, "no quantized pages: call pw_quantize_experts or pw_set_budget first");
    if (T == 0) return PW_OK;
    if (!x || !y) return fail(c, PW_ERR_INVALID_ARG, "null x or y");
    if ((uintptr_t)x % 16 || (uintptr_t)y % 16)
        return fail(c, PW_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
    return PW_OK;
}

pw_status pw_moe_forward(pw_ctx* c, const void* x, const float* logits, int32_t T, float* y,
                         void* stream) {
    if (!c) return PW_ERR_INVALID_ARG;
    pw_status st = forward_checks(c, logits, T);
    if (st != PW_OK) return st;
    if ((st = forward_args(c, x, logits, T, y)) != PW_OK || T == 0) return st;
    if ((st = ensure_device(c)) != PW_OK) return st;
    return forward_core(c, bound_ws(c), x, logits, T, y, static_cast<hipStream_t>(stream), false);
}

pw_status pw_moe_forward_noalloc(pw_ctx* c, const void* x, const float* logits, int32_t T, float* y,
                                 void* stream) {
    if (!c) return PW_ERR_INVALID_ARG;
    if (T < 0 || T > c->desc.max_tokens)
        return fail(c, PW_ERR_INVALID_ARG, "T = %d outside [0, %d]", T, c->desc.max_tokens);
    if (T > 0 && !logits) return fail(c, PW_ERR_INVALID_ARG, "null logits");
    pw_status st = forward_args(c, x, logits, T, y);
    if (st != PW_OK || T == 0) return st;
    // the device state exists once pages do; ensure_device then only checks
    // that the context's device is current
    if (!c->dev) return fail(c, PW_ERR_STATE, "no device state: quantize first");
    if ((st = ensure_device(c)) != PW_OK) return st;
    // the scratch laid out for exactly this batch; the fewest K-splits the
    // down product's partial outputs may need (one per pair) if the usual
    // capacity does not fit
    WsView v;
    v.max_tokens = T;
    v.nsplit = (int64_t)T * c->k > 2048 ? 1 : down_splits(c->F, c->d, 1, 1 << 30);
    v.lay = workspace_layout(c->E, c->d, c->F, c->k, T, v.nsplit);
    if (v.lay.total > noalloc_scratch_bytes()) {
        v.nsplit = 1;
        v.lay = workspace_layout(c->E, c->d, c->F, c->k, T, 1);
    }
    if (v.lay.total > noalloc_scratch_bytes())
        return fail(c, PW_ERR_WORKSPACE, "a forward of %d tokens needs %llu bytes of scratch, the static scratch "
                    "holds %llu", T, (unsigned long long)v.lay.total,
                    (unsigned long long)noalloc_scratch_bytes());
    void* p = nullptr;
    if (noalloc_scratch(c->device, &p) != hipSuccess || !p)
        return fail(c, PW_ERR_HIP, "hipGetSymbolAddress of the static scratch failed on device %d", c->device);
    v.base = static_cast<uint8_t*>(p);
    return forward_core(c, v, x, logits, T, y, static_cast<hipStream_t>(stream), true);
}

pw_status pw_get_page_table(const pw_ctx* c, pw_page_entry* out) {
    if (!c || !out) return PW_ERR_INVALID_ARG;
    std::memcpy(out, c->table.data(), sizeof(pw_page_entry) * c->E);
    return PW_OK;
}

pw_status pw_get_loss_table(pw_ctx* c, double* out, void* stream) {
    if (!c || !out) return PW_ERR_INVALID_ARG;
    if (!c->w1) return fail(c, PW_ERR_STATE, "no masters bound");
    pw_status st = ensure_device(c);
    if (st != PW_OK) return st;
    if ((st = ensure_loss(c, static_cast<hipStream_t>(stream))) != PW_OK) return st;
    std::memcpy(out, c->loss.data(), sizeof(double) * 3 * c->E);
    return PW_OK;
}

pw_status pw_solve_allocation(int32_t E, const uint64_t* W, const double* p, const double* L,
                              uint64_t budget_bits, uint8_t* bits_out) {
    return solve_allocation(E, W, p, L, budget_bits, bits_out, nullptr);
}

pw_status pw_profile(pw_ctx* c, int32_t mask) {
    if (!c) return PW_ERR_INVALID_ARG;
    if (mask < 0 || mask > 15) return fail(c, PW_ERR_INVALID_ARG, "profile mask must be in [0, 15]");
    c->profile_mask = mask;
    if (mask) {
        c->ev_used = 0;
        c->ev_kind.clear();
        c->forwards_timed = 0;
    }
    return PW_OK;
}

pw_status pw_profile_read(pw_ctx* c, pw_profile_data* out) {
    if (!c || !out) return PW_ERR_INVALID_ARG;
    std::memset(out, 0, sizeof *out);
    if (c->ev_used) HIP_TRY(c, hipEventSynchronize(c->ev_pool[c->ev_used - 1]));
    double* slot[4] = {&out->route_ms, &out->gate_up_ms, &out->down_ms, &out->combine_ms};
    for (size_t i = 0; i < c->ev_kind.size(); ++i) {
        float ms = 0.f;
        HIP_TRY(c, hipEventElapsedTime(&ms, c->ev_pool[2 * i], c->ev_pool[2 * i + 1]));
        *slot[c->ev_kind[i]] += ms;
    }
    out->forwards = c->forwards_timed;
    return PW_OK;
}

const char* pw_last_error(const pw_ctx* c) { return c ? c->err.c_str() : "null context"; }

}  // extern "C"
