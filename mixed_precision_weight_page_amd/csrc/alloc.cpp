// Exact solver of the budgeted precision allocation (PagedWeight page,
// section "Quality-Aware Quantization", Eq. 1):
//   minimise sum_e p_e * L_e(b_e)  subject to  sum_e b_e * W_e <= B,
//   b_e in {3, 4, 8}.
// A multiple-choice knapsack solved by dynamic programming over the budget
// left after giving every expert 3 bits, in units of g = gcd_e W_e: moving
// expert e from 3 to 4 bits costs W_e / g units, from 3 to 8 bits 5 W_e / g.
#include <cmath>
#include <cstring>
#include <limits>
#include <numeric>
#include <vector>

#include "pw_internal.h"

namespace pw {

namespace {

pw_status solve_core(int E, int max_experts, const uint64_t* W, const double* p, const double* L,
                     uint64_t B, uint8_t* bits_out, double* objective, std::string* err) {
    auto fail = [&](pw_status s, const char* m) {
        if (err) *err = m;
        return s;
    };
    if (E <= 0 || E > max_experts || !W || !p || !L || !bits_out)
        return fail(PW_ERR_INVALID_ARG, "solve_allocation: bad E or null pointer");
    unsigned __int128 sumW = 0;
    uint64_t g = 0;
    for (int e = 0; e < E; ++e) {
        if (W[e] == 0) return fail(PW_ERR_INVALID_ARG, "solve_allocation: W_e must be > 0");
        if (!(p[e] >= 0.0) || !std::isfinite(p[e]))
            return fail(PW_ERR_INVALID_ARG, "solve_allocation: importance must be finite and >= 0");
        for (int i = 0; i < 3; ++i)
            if (!(L[3 * e + i] >= 0.0) || !std::isfinite(L[3 * e + i]))
                return fail(PW_ERR_INVALID_ARG, "solve_allocation: losses must be finite and >= 0");
        sumW += W[e];
        g = std::gcd(g, W[e]);
    }
    const unsigned __int128 base = 3 * sumW;
    if ((unsigned __int128)B < base)
        return fail(PW_ERR_INFEASIBLE_BUDGET, "budget below 3 bits for every weight");
    // Budget units left after 3 bits everywhere; more than 5 * sumW / g units
    // cannot be used.
    unsigned __int128 spare = ((unsigned __int128)B - base) / g;
    const unsigned __int128 most = 5 * (sumW / g);
    if (spare > most) spare = most;
    const uint64_t C = (uint64_t)spare;
    if ((unsigned __int128)E * (C + 1) > ((unsigned __int128)1 << 28))
        return fail(PW_ERR_INVALID_ARG,
                    "solve_allocation: budget granularity too fine for the exact solver");

    const double INF = std::numeric_limits<double>::infinity();
    std::vector<double> best(C + 1, INF), next(C + 1);
    std::vector<uint8_t> choice((size_t)E * (C + 1), 0);
    best[0] = 0.0;
    static const int kExtra[3] = {0, 1, 5};  // units per W_e/g for b = 3, 4, 8
    for (int e = 0; e < E; ++e) {
        std::fill(next.begin(), next.end(), INF);
        uint8_t* ch = &choice[(size_t)e * (C + 1)];
        const uint64_t u = W[e] / g;
        for (uint64_t c = 0; c <= C; ++c) {
            if (best[c] == INF) continue;
            for (int i = 0; i < 3; ++i) {
                const unsigned __int128 c2 = (unsigned __int128)c + (unsigned __int128)kExtra[i] * u;
                if (c2 > C) continue;
                const double v = best[c] + p[e] * L[3 * e + i];
                const int b = bits_of_index(i);
                // strict improvement; an exact tie keeps the larger bit-width
                if (v < next[(size_t)c2] || (v == next[(size_t)c2] && b > ch[(size_t)c2])) {
                    next[(size_t)c2] = v;
                    ch[(size_t)c2] = (uint8_t)b;
                }
            }
        }
        best.swap(next);
    }
    // Least objective, and among equal objectives the fewest bits.
    uint64_t cb = 0;
    for (uint64_t c = 1; c <= C; ++c)
        if (best[c] < best[cb]) cb = c;
    if (objective) *objective = best[cb];
    for (int e = E - 1; e >= 0; --e) {
        const int b = choice[(size_t)e * (C + 1) + cb];
        bits_out[e] = (uint8_t)b;
        cb -= (uint64_t)kExtra[bits_index(b)] * (W[e] / g);
    }
    return PW_OK;
}

}  // namespace

pw_status solve_allocation(int E, const uint64_t* W, const double* p, const double* L,
                           uint64_t B, uint8_t* bits_out, std::string* err) {
    return solve_core(E, kMaxExperts, W, p, L, B, bits_out, nullptr, err);
}

}  // namespace pw

namespace {
// Experts over all layers of one shared budget (the exact solver's table is
// E x (budget units + 1) bytes and is capped separately).
constexpr int kMaxSolveExperts = 1 << 16;
}  // namespace

extern "C" {

// One budget over several layers: Eq. 1 over the union of their experts with
// importances w_l p_{l,e} (the constraint and the objective are sums over
// that union).
pw_status pw_solve_allocation_layers(int32_t n_layers, const int32_t* E, const uint64_t* W, const double* p,
                                     const double* L, const double* layer_weight, uint64_t budget_bits,
                                     uint8_t* bits_out, double* objective_out) {
    if (n_layers <= 0 || !E || !W || !p || !L || !bits_out) return PW_ERR_INVALID_ARG;
    int64_t total = 0;
    for (int l = 0; l < n_layers; ++l) {
        if (E[l] <= 0) return PW_ERR_INVALID_ARG;
        total += E[l];
        if (total > kMaxSolveExperts) return PW_ERR_INVALID_ARG;
        if (layer_weight && !(layer_weight[l] >= 0.0 && std::isfinite(layer_weight[l])))
            return PW_ERR_INVALID_ARG;
    }
    std::vector<double> pw_(total);
    for (int l = 0, i = 0; l < n_layers; ++l)
        for (int e = 0; e < E[l]; ++e, ++i) pw_[i] = (layer_weight ? layer_weight[l] : 1.0) * p[i];
    return pw::solve_core((int)total, kMaxSolveExperts, W, pw_.data(), L, budget_bits, bits_out, objective_out,
                          nullptr);
}

// The page's simplified sketch, for comparison (not a solver of Eq. 1): the
// budget shared in proportion to importance, divided by each expert's
// weight count, bucketized up to {3, 4, 8}. The result may exceed the
// budget; used_bits_out receives sum_e b_e W_e.
pw_status pw_proportional_bits(int32_t E, const uint64_t* W, const double* p, uint64_t budget_bits,
                               uint8_t* bits_out, uint64_t* used_bits_out) {
    if (E <= 0 || E > kMaxSolveExperts || !W || !p || !bits_out) return PW_ERR_INVALID_ARG;
    double total = 0.0;
    for (int e = 0; e < E; ++e) {
        if (W[e] == 0 || !(p[e] >= 0.0) || !std::isfinite(p[e])) return PW_ERR_INVALID_ARG;
        total += p[e];
    }
    if (!(total > 0.0) || !std::isfinite(total)) return PW_ERR_INVALID_ARG;
    unsigned __int128 used = 0;
    for (int e = 0; e < E; ++e) {
        const double x = (double)budget_bits * p[e] / total / (double)W[e];
        const int b = x <= 3.0 ? 3 : (x <= 4.0 ? 4 : 8);
        bits_out[e] = (uint8_t)b;
        used += (unsigned __int128)b * W[e];
    }
    if (used_bits_out) *used_bits_out = used > UINT64_MAX ? UINT64_MAX : (uint64_t)used;
    return PW_OK;
}

}  // extern "C"
