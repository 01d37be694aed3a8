// KV-pressure budget scheduler: the decision (host only). The PagedWeight
// page (section "Implementation Details") has the scheduler size the pages
// from the current KV-cache occupancy; the news digest's restatement
// compares it to operating-system paging (precision drops as the cache
// grows, comes back when the pressure eases). The pages give no formula;
// the policy implemented here is the one stated in include/pagedweight.h.
#include <cmath>
#include <cstdint>

#include "pw_internal.h"

namespace pw {

namespace {
constexpr uint64_t kAlignBytes = 256;

// Bytes of one page of W_e codes at b bits: whole bytes, then 256-byte aligned.
uint64_t page_nbytes(uint64_t We, int b) {
    const uint64_t code_bytes = (We * (uint64_t)b + 7) / 8;
    return (code_bytes + kAlignBytes - 1) / kAlignBytes * kAlignBytes;
}
}  // namespace

pw_status budget_decide(const pw_budget_policy& pol, uint64_t kv_used, int E, const uint64_t* W,
                        uint64_t pool_now, uint64_t budget_now, int steps_since, int32_t* action,
                        uint64_t* budget_out, int32_t* pressure) {
    uint64_t total = 0, pool3 = 0;
    for (int e = 0; e < E; ++e) {
        total += W[e];
        pool3 += page_nbytes(W[e], 3);
    }
    const uint64_t bmin = 3 * total, bmax = 8 * total;
    // bytes the pool may use: memory - kv_used - reserve, at least 0
    uint64_t avail = 0;
    if (pol.memory_bytes > kv_used && pol.memory_bytes - kv_used > pol.reserve_bytes)
        avail = pol.memory_bytes - kv_used - pol.reserve_bytes;
    const uint64_t room = (uint64_t)std::floor((double)avail * (1.0 - pol.headroom));
    const uint64_t slack = kAlignBytes * (uint64_t)E;   // page rounding, 256 bytes per expert at most
    uint64_t target = room > slack ? 8 * (room - slack) : 0;
    if (target < bmin) target = bmin;
    if (target > bmax) target = bmax;
    *pressure = pool3 > avail ? 1 : 0;
    if (pool_now == UINT64_MAX) {
        *action = PW_BUDGET_INIT;
        *budget_out = target;
    } else if (pool_now > avail) {
        const bool lower = target < budget_now;
        *action = lower ? PW_BUDGET_SHRINK : PW_BUDGET_KEEP;
        *budget_out = lower ? target : budget_now;
    } else if (steps_since >= pol.min_interval && target > budget_now &&
               (double)target >= std::ceil((double)budget_now * (1.0 + pol.headroom))) {
        *action = PW_BUDGET_GROW;
        *budget_out = target;
    } else {
        *action = PW_BUDGET_KEEP;
        *budget_out = budget_now;
    }
    return PW_OK;
}

}  // namespace pw

extern "C" pw_status pw_budget_decide(const pw_budget_policy* policy, uint64_t kv_used_bytes, int32_t E,
                                      const uint64_t* W, uint64_t pool_bytes_now, uint64_t budget_now,
                                      int32_t steps_since_change, int32_t* action, uint64_t* budget_out,
                                      int32_t* pressure) {
    if (!policy || !W || !action || !budget_out || !pressure || E <= 0 || steps_since_change < 0)
        return PW_ERR_INVALID_ARG;
    if (!(policy->headroom >= 0.0 && policy->headroom <= 0.5) || policy->min_interval < 0)
        return PW_ERR_INVALID_ARG;
    for (int e = 0; e < E; ++e)
        if (W[e] == 0) return PW_ERR_INVALID_ARG;
    return pw::budget_decide(*policy, kv_used_bytes, E, W, pool_bytes_now, budget_now, steps_since_change,
                             action, budget_out, pressure);
}
