/*
 * pagedweight.h -- C ABI of the per-expert mixed-precision MoE expert layer
 * (PagedWeight) for AMD Instinct MI355X (gfx950).
 *
 * What the library computes (PagedWeight page):
 *   - section "Implementation Details", Eq. 2: each expert's SwiGLU weights
 *     are quantized uniformly and symmetrically with one scale per expert,
 *     s_e = max|w| / (2^(b_e-1) - 1), q = round(w / s_e), b_e in {3, 4, 8};
 *   - section "Quality-Aware Quantization", Eq. 1: the bit-widths solve
 *     min sum_e p_e L_e(b_e)  s.t.  sum_e b_e W_e <= B;
 *   - section "Dynamic Paging": codes live in pages of a GPU page pool, a
 *     page table maps expert id -> page (section "Implementation Details",
 *     "Memory Management"), the router picks the experts a token needs and
 *     their pages are dequantized on the fly inside the expert FFN.
 *
 * Conventions (every entry point):
 *   - Returns pw_status: 0 on success, a negative code on error. Nothing
 *     aborts or throws. pw_last_error(ctx) gives a message for the last
 *     failed call on that context.
 *   - Device pointers are BORROWED: the caller (for example PyTorch) owns
 *     the memory and keeps it alive while the context uses it. Host
 *     pointers are read or written only during the call.
 *   - Tensor arguments are row-major and contiguous (the page layout is
 *     described at pw_quantize_experts).
 *   - `stream` is a hipStream_t (NULL = the default stream). All device
 *     work is enqueued on it in call order; a later call on the same stream
 *     sees the results of an earlier one. Calls on different streams must be
 *     ordered by the caller.
 *   - A context is not thread-safe: serialise calls on one context.
 *   - On error the page table and the pool contents stay as they were.
 *   - Shapes: d_model and d_ff must be multiples of 128, 1 <= top_k <= 32,
 *     top_k <= num_experts <= 1024.
 */
#ifndef PAGEDWEIGHT_H
#define PAGEDWEIGHT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PW_OK = 0,
    PW_ERR_INVALID_ARG = -1,       /* null pointer, bad shape, bad value      */
    PW_ERR_UNSUPPORTED_BITS = -2,  /* a bit-width outside {3, 4, 8}           */
    PW_ERR_INFEASIBLE_BUDGET = -3, /* B < 3 * sum_e W_e                       */
    PW_ERR_NONFINITE_WEIGHTS = -4, /* NaN or Inf in the bound masters         */
    PW_ERR_POOL_CAPACITY = -5,     /* the pages do not fit the bound pool     */
    PW_ERR_WORKSPACE = -6,         /* no workspace bound, or too small        */
    PW_ERR_STATE = -7,             /* call out of order (e.g. forward before
                                      any quantization, or no masters bound)  */
    PW_ERR_HIP = -8                /* a HIP runtime call failed               */
} pw_status;

typedef enum { PW_MASTER_F32 = 0, PW_MASTER_F16 = 1 } pw_master_dtype;

/* Page layout of a layer.
 * PW_LAYOUT_EQ2: pages of Eq. 2 codes at 3, 4 or 8 bits (the PagedWeight
 *   page), the layout described at pw_quantize_experts.
 * PW_LAYOUT_BITPLANE: the PagedMoE page's prefix-compatible layout (its
 *   Abstract: one stored state per expert, a lower precision a prefix of a
 *   higher one), read as a tree codebook over Eq. 2's 8-bit codes: with
 *   s8 = max|w| / 127 (nearest fp32) and u8 = q8 + 128 Eq. 2's 8-bit code, a
 *   weight at depth b in 1..8 is s8 ((2p + 1) 2^(7-b) - 128.5) for the prefix
 *   p = u8 >> (8 - b) (the centre of the node it names; Eq. 2's 8-bit weight
 *   at depth 8). Bitplane j holds bit 7 - j of every u8; a depth-b page is
 *   planes 0 .. b-1 in order, each plane the W1, W3 and W2 bits (W_e / 8
 *   bytes, every matrix in the tiles of pw_quantize_experts at 1 bit per
 *   code: 256 bytes per 16 x 128 tile, lane l = 16 g + r holding the bits
 *   of codes 32 g .. 32 g + 31 of row r as one little-endian word). The
 *   "bits" of every call are depths; lowering a depth drops the page's last
 *   planes in place without reading the masters, raising it writes only
 *   the missing planes when the bytes after the page are free. The table's
 *   scale is s8; the loss table holds depths 3, 4, 8 (the allocation of
 *   pw_set_budget chooses among them); forwards use the streaming kernels
 *   for every batch. */
typedef enum { PW_LAYOUT_EQ2 = 0, PW_LAYOUT_BITPLANE = 1 } pw_layout;

/* One MoE layer. W_e = 3 * d_model * d_ff weights per expert. */
typedef struct {
    int32_t num_experts;   /* E                                                 */
    int32_t d_model;       /* d                                                 */
    int32_t d_ff;          /* F                                                 */
    int32_t top_k;         /* k experts per token                               */
    int32_t renorm;        /* 0: g = softmax over all E experts;
                              1: softmax renormalised over the k chosen         */
    int32_t max_tokens;    /* largest T passed to pw_moe_forward                */
    int32_t master_dtype;  /* pw_master_dtype of the bound masters              */
    int32_t layout;        /* pw_layout of the pages                            */
} pw_layer_desc;

/* Host copy of one page-table entry. */
typedef struct {
    uint64_t offset;   /* byte offset of the page in the pool (256-B aligned)  */
    uint64_t nbytes;   /* page bytes = 3 * d * F * bits / 8                    */
    float scale;       /* s_e, the fp32 value nearest max|w| / (2^(b-1) - 1)   */
    uint8_t bits;      /* 3, 4 or 8; 0 = no page yet                           */
    uint8_t pad_[3];
} pw_page_entry;

/* Per-kernel timing gathered by pw_profile (milliseconds, summed). */
typedef struct {
    double route_ms;     /* router + grouping kernels          */
    double gate_up_ms;   /* gate/up + SwiGLU kernels           */
    double down_ms;      /* down-projection kernels            */
    double combine_ms;   /* weighted combine kernel            */
    int64_t forwards;    /* pw_moe_forward calls timed         */
} pw_profile_data;

typedef struct pw_ctx pw_ctx;   /* opaque, owned by the library */

/* Validate `desc` and create a context. No device memory is touched until
 * the first call that needs the GPU (that call uses the current device). */
pw_status pw_create(const pw_layer_desc* desc, pw_ctx** out);
void pw_destroy(pw_ctx* ctx);

/* Bind the fp32 or fp16 masters (device): w1 and w3 are [E, F, d] (gate,
 * up), w2 is [E, d, F] (down). Invalidates cached max|w| and losses;
 * existing pages stay valid until the next quantization. */
pw_status pw_bind_masters(pw_ctx* ctx, const void* w1, const void* w3, const void* w2);

/* Pool bytes needed for the given host bits[E] (each page 256-B aligned);
 * 0 if a bit-width is unsupported. */
uint64_t pw_pool_bytes_for_bits(const pw_ctx* ctx, const uint8_t* bits);

/* Bind the device page pool: `pool` 256-B aligned, `capacity_bytes` usable.
 * Rebinding drops all pages (the next quantization rewrites them). */
pw_status pw_bind_pool(pw_ctx* ctx, void* pool, uint64_t capacity_bytes);

/* Device workspace bytes needed by every call for max_tokens. */
uint64_t pw_workspace_bytes(const pw_ctx* ctx);
pw_status pw_bind_workspace(pw_ctx* ctx, void* ws, uint64_t bytes);

/* Quantize every expert at the host bits[E] (each in {3, 4, 8}) from the
 * masters into the pool and upload the page table. The first call after
 * pw_bind_masters measures max|w| per expert on the device and waits for
 * it (one stream synchronisation). Eq. 2; layout of a page: the W1 codes,
 * then W3, then W2, each matrix [out, in] with every row a little-endian
 * LSB-first bitstream of b-bit codes u = q + 2^(b-1), arranged in tiles of
 * 16 rows x 128 codes in (row block, K step) order; inside a tile, lane
 * l = 16 g + r of a 64-lane wave holds codes 32 g .. 32 g + 31 of row r
 * (4 b bytes), cut into pieces of at most 16 bytes, and piece p of all 64
 * lanes is stored together. Pages are 256-byte aligned. */
pw_status pw_quantize_experts(pw_ctx* ctx, const uint8_t* bits, void* stream);

/* Move the weight budget: solve Eq. 1 on the host for budget_bits B with
 * host importance[E] (>= 0) and host loss[E][3] (L for b = 3, 4, 8) or
 * NULL to use the measured per-expert MSE of Eq. 2 (computed on the
 * device once per binding of the masters; the first such call waits for
 * it). Only experts whose bit-width changes are re-quantized from the
 * masters and re-placed; the new page table is uploaded after their pages
 * are written. bits_out (host [E]) receives the allocation if non-NULL. */
pw_status pw_set_budget(pw_ctx* ctx, uint64_t budget_bits, const double* importance,
                        const double* loss, uint8_t* bits_out, void* stream);

/* Forward pass of the expert layer (section "Dynamic Paging"):
 * x bf16 [T, d] and logits fp32 [T, E] in, y fp32 [T, d] out (overwritten).
 * Per token: the top_k largest logits (equal values -> lower expert index),
 * g = softmax weight (see desc.renorm), y = sum_j g_j * W2 (silu(W1 x) *
 * (W3 x)) with W = s_e * q read from the pages. 0 <= T <= max_tokens; T = 0
 * does nothing. Asynchronous: no host synchronisation. Not replayable from
 * a captured graph (the grouping counters it uses alternate between calls
 * on the host side); pw_moe_forward_noalloc is. */
pw_status pw_moe_forward(pw_ctx* ctx, const void* x, const float* logits, int32_t T,
                         float* y, void* stream);

/* pw_moe_forward without device allocation, for callers that cannot
 * allocate (code under stream capture, tight serving loops, harnesses that
 * forbid hipMalloc). Same arguments, checks and results as pw_moe_forward
 * (up to the fp32 summation order of the down product's K-splits), but its
 * scratch lives in a static 64 MiB device array of the library (one per
 * device, held until the process ends) instead of the bound workspace,
 * which it neither needs nor touches; no timing events are recorded. The
 * array is laid out for exactly T tokens; a batch whose scratch does not fit
 * returns PW_ERR_WORKSPACE (decode batches fit: for example 64 tokens of
 * 128 experts, d_model 2048, d_ff 768, top-8 need about 27 MiB). Every call
 * on a device shares that device's array: calls that may overlap on one
 * device (several streams, several contexts) race and must be serialized by
 * the caller. The context's pages must exist (PW_ERR_STATE otherwise). It
 * only launches kernels on the stream (its counters are cleared by a kernel
 * on every call), so a call captured in a graph may be replayed, with the
 * inputs it was captured with updated in place between replays. */
pw_status pw_moe_forward_noalloc(pw_ctx* ctx, const void* x, const float* logits, int32_t T, float* y,
                                 void* stream);

/* Router and grouping only (the first steps of pw_moe_forward), for
 * inspection: ids int32 [T, k] (descending logit order), g fp32 [T, k] and
 * counts int32 [E] (tokens routed to each expert), all device pointers. */
pw_status pw_route(pw_ctx* ctx, const float* logits, int32_t T, int32_t* ids, float* g,
                   int32_t* counts, void* stream);

/* Host copy of the page table (entries [E]). */
pw_status pw_get_page_table(const pw_ctx* ctx, pw_page_entry* out);

/* Measured loss table L[E][3] (b = 3, 4, 8; float64) into host memory,
 * computing it first if needed. Synchronises `stream`. */
pw_status pw_get_loss_table(pw_ctx* ctx, double* out, void* stream);

/* Eq. 1 solved exactly on the host (no context, no GPU): W[E] weights per
 * expert, p[E] importance, L[E][3] losses, budget B in bits. Writes
 * bits_out[E]. Among allocations with the same objective it returns the
 * one with the fewest total bits. */
pw_status pw_solve_allocation(int32_t E, const uint64_t* W, const double* p, const double* L,
                              uint64_t budget_bits, uint8_t* bits_out);

/* One budget shared by several layers (host, no GPU): Eq. 1 over the union
 * of the layers' experts, minimising sum_l w_l sum_e p_{l,e} L_{l,e}(b)
 * subject to sum over all experts of b W <= B. E[n_layers] experts per
 * layer; W, p, bits_out have sum(E) entries and L has 3 sum(E), all in
 * layer order; layer_weight[n_layers] may be NULL (all 1). Writes the
 * objective to objective_out if not NULL. At most 65536 experts in all;
 * PW_ERR_INFEASIBLE_BUDGET when B < 3 sum W, PW_ERR_INVALID_ARG for bad
 * sizes, negative or non-finite inputs, or a budget too finely divided for
 * the exact solver. Each layer then applies its share with
 * pw_quantize_experts. */
pw_status pw_solve_allocation_layers(int32_t n_layers, const int32_t* E, const uint64_t* W, const double* p,
                                     const double* L, const double* layer_weight, uint64_t budget_bits,
                                     uint8_t* bits_out, double* objective_out);

/* Comparison mode, not a solver of Eq. 1: the simplified sketch printed on
 * the PagedWeight page (after "Implementation Details"): expert e's share
 * B p_e / sum(p) divided by W_e, bucketized up to {3, 4, 8} (a share equal
 * to an option takes it; above 8 gives 8). The budget is read in bits. The
 * bits may exceed the budget: used_bits_out (may be NULL) receives
 * sum_e b_e W_e. PW_ERR_INVALID_ARG for E outside [1, 65536], W_e = 0,
 * negative or non-finite p, or all p zero. */
pw_status pw_proportional_bits(int32_t E, const uint64_t* W, const double* p, uint64_t budget_bits,
                               uint8_t* bits_out, uint64_t* used_bits_out);

/* ---- KV-pressure budget scheduler ----
 * The pool's budget follows the KV-cache occupancy (PagedWeight page,
 * section "Implementation Details": the scheduler adjusts page sizes from
 * the current KV-cache occupancy; the news digest's paging comparison:
 * precision drops as the cache grows and comes back when pressure eases).
 * Reading of the policy (the pages give none):
 *   A = memory - kv_used - reserve bytes (at least 0) may hold the pool;
 *   target = 8 * (floor(A * (1 - headroom)) - 256 * E) code bits (at least
 *     0; a page is its codes rounded up to 256 bytes, so any allocation
 *     within target fits in A), clamped to [3 W, 8 W], W = sum_e W_e;
 *   INIT: no allocation yet -> target;
 *   SHRINK: the current pool does not fit in A and target is lower than the
 *     current budget -> target (never held back);
 *   GROW: at least min_interval steps since the last change, target above
 *     the current budget and >= ceil(budget * (1 + headroom)) -> target;
 *   KEEP otherwise. pressure = 1 when even the all-3-bit pool does not fit
 *   in A (the caller has to free KV cache). Fractions in double, floored. */
typedef struct {
    uint64_t memory_bytes;   /* bytes the weight pool and the KV cache share */
    uint64_t reserve_bytes;  /* bytes kept free */
    double headroom;         /* in [0, 0.5] */
    int32_t min_interval;    /* >= 0: steps from a change to the next grow */
} pw_budget_policy;

enum { PW_BUDGET_KEEP = 0, PW_BUDGET_SHRINK = 1, PW_BUDGET_GROW = 2, PW_BUDGET_INIT = 3 };

/* The decision alone (host only, no device work): W[E] weights per expert,
 * pool_bytes_now = bytes of the current pages (sum of their 256-byte
 * aligned sizes) and budget_now its budget, or UINT64_MAX and 0 before the
 * first allocation; steps_since_change >= 0. Writes action, the budget to
 * move to (budget_now on KEEP) and pressure. Errors: INVALID_ARG for null
 * pointers, E <= 0, a W_e of 0, headroom outside [0, 0.5], min_interval < 0. */
pw_status pw_budget_decide(const pw_budget_policy* policy, uint64_t kv_used_bytes, int32_t E,
                           const uint64_t* W, uint64_t pool_bytes_now, uint64_t budget_now,
                           int32_t steps_since_change, int32_t* action, uint64_t* budget_out,
                           int32_t* pressure);

/* One scheduler step on a layer: the decision from the layer's pages (the
 * bytes they span, pw_pool_used_bytes; the budget of the last scheduler
 * move, or the bits of pages set by pw_quantize_experts) and the steps
 * since the last move; on INIT, SHRINK or GROW it re-allocates as
 * pw_set_budget does with importance and loss (host, as there) on stream,
 * and places the new pages so that they span at most A bytes from the
 * start of the pool: first fit when that stays within A, else every page is
 * rewritten densely (compaction). Without pressure the pages then fit in A,
 * so after a SHRINK the caller may hand the pool's bytes from
 * pw_pool_used_bytes on to the KV cache. The step counter advances only on
 * KEEP. A failed re-allocation leaves pages, table and scheduler state
 * unchanged and returns its status. */
pw_status pw_budget_step(pw_ctx* ctx, const pw_budget_policy* policy, uint64_t kv_used_bytes,
                         const double* importance, const double* loss, int32_t* action,
                         uint64_t* budget_out, int32_t* pressure, void* stream);

/* Bytes of the pool the current pages span: the end of the highest page
 * (0 without pages). The pool's bytes beyond it are unused. */
uint64_t pw_pool_used_bytes(const pw_ctx* ctx);

/* ---- Host tier: expert pages swapped out to CPU memory ----
 * PagedWeight page, section "Dynamic Paging": the router decides which
 * experts a pass needs and their pages are fetched; inactive experts' pages
 * can be swapped out to CPU memory.
 *
 * pw_bind_host_tier binds `bytes` of pinned host memory (hipHostMalloc, or
 * a pinned PyTorch tensor; 256-byte aligned, caller-owned, device
 * accessible). From then on the pages are packed into it (placement and
 * capacity as for the pool, PW_ERR_POOL_CAPACITY when they do not fit) and
 * the pool bound with pw_bind_pool becomes a cache of min(E, pool bytes /
 * slot) page slots of one 8-bit page each (align_up(3 d F, 256) bytes; no
 * pool, or one smaller than a slot: no slots). Binding it, or NULL (back
 * to pages in the pool), invalidates the pages: quantize again. Rebinding
 * the pool empties the slots and keeps the pages. In each pw_moe_forward,
 * on the device and without host synchronisation, the routed experts
 * holding a slot are hits; the others, in ascending expert id, take empty
 * slots (ascending index), then the slots of experts not routed in this
 * pass, least recently used first (ties: lower expert id), and have their
 * page copied in; those left without a slot are read from the host tier
 * directly in this pass. Requantizing an expert empties its slot. The
 * library allocates (40 E + 32) bytes of device memory for this state.
 * Results equal those without a host tier bit for bit. */
pw_status pw_bind_host_tier(pw_ctx* ctx, void* host, uint64_t bytes);

/* Residency after the forwards enqueued so far (waits for the stream):
 * slot_of[E] (slot holding each expert's page, -1 none; may be NULL) and
 * stats[3] (cumulative routed experts that hit, pages copied in, pages read
 * from the host tier; may be NULL). PW_ERR_STATE without a host tier. */
pw_status pw_get_residency(pw_ctx* ctx, int32_t* slot_of, uint64_t* stats, void* stream);

/* Timing of the forward kernels on the forward's stream: HIP events
 * (created without the system-scope fence) are recorded just before and
 * after each timed kernel; an event delays the next dispatch by a few
 * microseconds, so the sums read slightly above the kernels' own durations
 * and untimed forwards run slightly faster. mask selects the kernels: bit 0 router/grouping,
 * bit 1 gate/up, bit 2 down, bit 3 combine; a nonzero mask starts (and
 * clears) collection, 0 stops it. pw_profile_read waits for the recorded
 * events and returns the per-class sums over the timed forwards. */
pw_status pw_profile(pw_ctx* ctx, int32_t mask);
pw_status pw_profile_read(pw_ctx* ctx, pw_profile_data* out);

const char* pw_last_error(const pw_ctx* ctx);
const char* pw_status_str(int32_t status);

#ifdef __cplusplus
}
#endif
#endif /* PAGEDWEIGHT_H */
