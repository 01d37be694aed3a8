// CPU oracle in plain C++ of the per-expert mixed-precision MoE expert layer
// of the PagedWeight page: the quantizer and page bytes of Eq. 2 (section
// "Implementation Details"), the loss table and the budgeted allocation of
// Eq. 1 (section "Quality-Aware Quantization"), and the forward pass of
// section "Dynamic Paging" (top-k router, SwiGLU experts on the dequantized
// weights s_e q, routing-weighted combine).
//
// TEST INFRASTRUCTURE: loaded (through oracle/c_oracle.py) only by the
// tests, the smoke check and the benchmark's CPU baseline. The GPU library
// never links, loads or calls it, and this file includes nothing of the
// library.
//
// Plain loops, in the order the definitions state them; double precision
// everywhere except where a rounding is part of the definition (the fp32
// scale). Built with -ffp-contract=off, so no multiply and add are fused.
// Readings where the pages are silent:
//  * the scale's max is over all of an expert's weights (W1, W3, W2);
//  * s = the fp32 value nearest max / qmax; max = 0 gives s = 0 and codes 0;
//  * round() is round half to even of the exact quotient w / s, then the
//    code is clamped to +-qmax; for fp32 w and s the double quotient is a
//    half-integer only when the exact one is, so rounding the double gives
//    the exact quotient's rounding;
//  * a code q is stored as u = q + 2^(b-1); a page is W1 [F rows of d], W3
//    [F rows of d], W2 [d rows of F], each row an LSB-first bitstream of its
//    codes (code j in stream bits b j .. b j + b - 1, stream bit n in bit
//    n % 8 of byte n / 8) padded with zero codes to a multiple of 128 codes,
//    the page padded with zero bytes to a multiple of 256;
//  * L(b) is the mean squared error of Eq. 2 over the expert's weights;
//  * B counts code bits; several optimal allocations: at each expert the DP
//    keeps the larger bit-width on an exact tie, and among equal objectives
//    the fewest bits;
//  * router: equal logits go to the lower expert index; g is the softmax
//    over all E logits, or over the k chosen (renorm);
//  * SwiGLU: h = silu(W1 x) * (W3 x), silu(z) = z / (1 + exp(-z)), o = W2 h.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <vector>

namespace {

const int kBits[3] = {3, 4, 8};

int qmax_of(int b) { return (1 << (b - 1)) - 1; }

bool bits_ok(int b) { return b == 3 || b == 4 || b == 8; }

int64_t padded_codes(int K) { return ((int64_t)K + 127) / 128 * 128; }

double bf16_value(uint16_t h) {
    const uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

int code_of(float w, float s, int b) {
    if (s == 0.0f) return 0;
    const int qm = qmax_of(b);
    double r = nearbyint((double)w / (double)s);   // default rounding: half to even
    if (r > qm) r = qm;
    if (r < -qm) r = -qm;
    return (int)r;
}

}  // namespace

extern "C" {

int orc_qmax(int b) { return qmax_of(b); }

// max |w| over n weights (exact in any order)
double orc_absmax(const float* w, int64_t n) {
    double m = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        const double a = fabs((double)w[i]);
        if (a > m) m = a;
    }
    return m;
}

// Eq. 2's scale: the fp32 value nearest m / (2^(b-1) - 1)
float orc_scale(double m, int b) {
    if (m == 0.0) return 0.0f;
    return (float)(m / (double)qmax_of(b));
}

// signed codes of n weights at scale s
void orc_codes(const float* w, int64_t n, float s, int b, int8_t* q) {
    for (int64_t i = 0; i < n; ++i) q[i] = (int8_t)code_of(w[i], s, b);
}

// bytes of one packed row of K codes
int64_t orc_row_bytes(int K, int b) { return padded_codes(K) * b / 8; }

// bytes of one expert's page
int64_t orc_page_bytes(int d, int F, int b) {
    const int64_t raw = 2 * (int64_t)F * orc_row_bytes(d, b) + (int64_t)d * orc_row_bytes(F, b);
    return (raw + 255) / 256 * 256;
}

// rows x K signed codes -> rows x orc_row_bytes(K, b) bytes of stored codes
void orc_pack_rows(const int8_t* q, int rows, int K, int b, uint8_t* out) {
    const int64_t rb = orc_row_bytes(K, b);
    memset(out, 0, (size_t)(rows * rb));
    for (int r = 0; r < rows; ++r) {
        uint8_t* row = out + r * rb;
        for (int j = 0; j < K; ++j) {
            const unsigned u = (unsigned)(q[(int64_t)r * K + j] + (1 << (b - 1)));
            for (int i = 0; i < b; ++i) {
                if ((u >> i) & 1u) {
                    const int64_t bit = (int64_t)b * j + i;
                    row[bit / 8] = (uint8_t)(row[bit / 8] | (1u << (bit % 8)));
                }
            }
        }
    }
}

// One expert at b bits: its scale, its 3 d F codes (W1, W3, W2, row after
// row) and, if page is not NULL, its orc_page_bytes(d, F, b) page bytes.
// Returns 0, or -1 for an unsupported width.
int orc_quantize_expert(const float* w1, const float* w3, const float* w2, int d, int F, int b,
                        float* s_out, int8_t* q, uint8_t* page) {
    if (!bits_ok(b)) return -1;
    const int64_t n = (int64_t)d * F;
    double m = orc_absmax(w1, n);
    const double m3 = orc_absmax(w3, n), m2 = orc_absmax(w2, n);
    if (m3 > m) m = m3;
    if (m2 > m) m = m2;
    const float s = orc_scale(m, b);
    *s_out = s;
    orc_codes(w1, n, s, b, q);
    orc_codes(w3, n, s, b, q + n);
    orc_codes(w2, n, s, b, q + 2 * n);
    if (page) {
        memset(page, 0, (size_t)orc_page_bytes(d, F, b));
        const int64_t m1 = (int64_t)F * orc_row_bytes(d, b);
        orc_pack_rows(q, F, d, b, page);
        orc_pack_rows(q + n, F, d, b, page + m1);
        orc_pack_rows(q + 2 * n, d, F, b, page + 2 * m1);
    }
    return 0;
}

// L(b): mean over the expert's 3 d F weights of (w - s q)^2. The squared
// errors are summed row by row (W1, W3: F rows of d; W2: d rows of F), then
// the row sums: the sum's relative rounding error stays below
// (row length + rows) 2^-53 instead of 3 d F 2^-53.
double orc_loss(const float* w1, const float* w3, const float* w2, int d, int F, int b) {
    const int64_t n = (int64_t)d * F;
    double m = orc_absmax(w1, n);
    const double m3 = orc_absmax(w3, n), m2 = orc_absmax(w2, n);
    if (m3 > m) m = m3;
    if (m2 > m) m = m2;
    const float s = orc_scale(m, b);
    const float* mats[3] = {w1, w3, w2};
    double total = 0.0;
    for (int t = 0; t < 3; ++t) {
        const int rows = t < 2 ? F : d, K = t < 2 ? d : F;
        for (int r = 0; r < rows; ++r) {
            double row = 0.0;
            for (int j = 0; j < K; ++j) {
                const float w = mats[t][(int64_t)r * K + j];
                const double e = (double)w - (double)s * code_of(w, s, b);
                row += e * e;
            }
            total += row;
        }
    }
    return total / (double)(3 * n);
}

// Eq. 1 over E experts: least sum_e p_e L_e(b_e) subject to
// sum_e b_e W_e <= B, b_e in {3, 4, 8}; L is [E][3] for 3, 4 and 8 bits.
// Dynamic programme over the budget in units of g = gcd of the W_e: after
// expert e, best[c] is the least objective of experts 0..e that use exactly
// c units. Returns 0 (bits and objective written), 1 if even all-3-bit
// does not fit, 2 for bad input (or a table too large to hold).
int orc_allocate(int E, const double* p, const double* L, const uint64_t* W, uint64_t B, uint8_t* bits,
                 double* objective) {
    if (E <= 0) return 2;
    uint64_t g = 0, w3 = 0;
    for (int e = 0; e < E; ++e) {
        if (W[e] == 0) return 2;
        uint64_t a = W[e], c = g;
        while (c) {   // gcd(a, c)
            const uint64_t t = a % c;
            a = c;
            c = t;
        }
        g = a;
        w3 += 3 * W[e];
    }
    if (w3 > B) return 1;
    const uint64_t cap = B / g;
    if (cap > (1u << 26) || (uint64_t)E * (cap + 1) > (1ull << 31)) return 2;
    const int C = (int)cap;
    const double inf = INFINITY;
    std::vector<double> best(C + 1, inf), next(C + 1);
    std::vector<uint8_t> choice((size_t)E * (C + 1), 0);
    best[0] = 0.0;
    for (int e = 0; e < E; ++e) {
        for (int c = 0; c <= C; ++c) next[c] = inf;
        uint8_t* ch = &choice[(size_t)e * (C + 1)];
        for (int c = 0; c <= C; ++c) {
            if (best[c] == inf) continue;
            for (int i = 0; i < 3; ++i) {
                const uint64_t units = (uint64_t)kBits[i] * W[e] / g;
                if (c + units > cap) continue;
                const int c2 = c + (int)units;
                const double v = best[c] + p[e] * L[3 * e + i];
                if (v < next[c2] || (v == next[c2] && kBits[i] > ch[c2])) {
                    next[c2] = v;
                    ch[c2] = (uint8_t)kBits[i];
                }
            }
        }
        best.swap(next);
    }
    int cb = -1;
    for (int c = 0; c <= C; ++c)
        if (best[c] < inf && (cb < 0 || best[c] < best[cb])) cb = c;   // first (fewest units) of the least
    if (cb < 0) return 1;
    *objective = best[cb];
    int c = cb;
    for (int e = E - 1; e >= 0; --e) {
        const uint8_t b = choice[(size_t)e * (C + 1) + c];
        bits[e] = b;
        c -= (int)((uint64_t)b * W[e] / g);
    }
    return c == 0 ? 0 : 2;
}

// Eq. 1 by enumerating all 3^E assignments (E <= 12); ties: fewer bits, then
// the larger width at the lowest expert index where two assignments differ.
int orc_allocate_brute(int E, const double* p, const double* L, const uint64_t* W, uint64_t B, uint8_t* bits,
                       double* objective) {
    if (E <= 0 || E > 12) return 2;
    int n = 1;
    for (int e = 0; e < E; ++e) n *= 3;
    bool found = false;
    double best_obj = 0.0;
    uint64_t best_used = 0;
    std::vector<int> cur(E), best(E);
    for (int a = 0; a < n; ++a) {
        int r = a;
        uint64_t used = 0;
        double obj = 0.0;
        for (int e = 0; e < E; ++e) {
            cur[e] = r % 3;
            r /= 3;
        }
        for (int e = 0; e < E; ++e) used += (uint64_t)kBits[cur[e]] * W[e];
        if (used > B) continue;
        for (int e = 0; e < E; ++e) obj += p[e] * L[3 * e + cur[e]];
        bool take = !found || obj < best_obj || (obj == best_obj && used < best_used);
        if (found && obj == best_obj && used == best_used) {
            for (int e = 0; e < E; ++e) {
                if (cur[e] != best[e]) {
                    take = cur[e] > best[e];
                    break;
                }
            }
        }
        if (take) {
            found = true;
            best_obj = obj;
            best_used = used;
            best = cur;
        }
    }
    if (!found) return 1;
    for (int e = 0; e < E; ++e) bits[e] = (uint8_t)kBits[best[e]];
    *objective = best_obj;
    return 0;
}

// Router: for each of T tokens the k largest of its E logits (equal logits:
// lower expert first), in descending order, and their weights.
int orc_route(const float* logits, int T, int E, int k, int renorm, int32_t* ids, double* g) {
    if (k < 1 || k > E) return 2;
    std::vector<char> taken(E);
    for (int t = 0; t < T; ++t) {
        const float* l = logits + (int64_t)t * E;
        for (int e = 0; e < E; ++e) taken[e] = 0;
        for (int j = 0; j < k; ++j) {
            int b = -1;
            for (int e = 0; e < E; ++e)
                if (!taken[e] && (b < 0 || l[e] > l[b])) b = e;
            taken[b] = 1;
            ids[(int64_t)t * k + j] = b;
        }
        double mx = (double)l[0];
        for (int e = 1; e < E; ++e)
            if ((double)l[e] > mx) mx = (double)l[e];
        double den = 0.0;
        if (renorm) {
            for (int j = 0; j < k; ++j) den += exp((double)l[ids[(int64_t)t * k + j]] - mx);
        } else {
            for (int e = 0; e < E; ++e) den += exp((double)l[e] - mx);
        }
        for (int j = 0; j < k; ++j) g[(int64_t)t * k + j] = exp((double)l[ids[(int64_t)t * k + j]] - mx) / den;
    }
    return 0;
}

// The layer's forward pass, y [T][d] in double. x: T x d bf16 bit patterns
// (each the exact value of its bf16 number); codes[e]: expert e's 3 d F
// codes as orc_quantize_expert writes them, or NULL when no token routes to
// e; scales[e] its scale. For each token and each chosen expert:
// a = (s W1) x, c = (s W3) x, h = silu(a) c, o = (s W2) h, y += g o, the
// chosen experts in descending logit order. With nthreads > 1 the tokens
// are spread over OpenMP threads; every token is computed the same way
// whatever the count. Returns 0, or 2 (bad k, or a routed expert without
// codes).
int orc_moe_forward(const uint16_t* x, const float* logits, int T, int d, int F, int E, int k, int renorm,
                    const int8_t* const* codes, const float* scales, double* y, int nthreads) {
    std::vector<int32_t> ids((size_t)T * k);
    std::vector<double> g((size_t)T * k);
    if (orc_route(logits, T, E, k, renorm, ids.data(), g.data()) != 0) return 2;
    for (size_t i = 0; i < ids.size(); ++i)
        if (!codes[ids[i]]) return 2;
    const int64_t n = (int64_t)d * F;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (int t = 0; t < T; ++t) {
        std::vector<double> xt(d), h(F);
        double* yt = y + (int64_t)t * d;
        for (int i = 0; i < d; ++i) {
            xt[i] = bf16_value(x[(int64_t)t * d + i]);
            yt[i] = 0.0;
        }
        for (int j = 0; j < k; ++j) {
            const int e = ids[(int64_t)t * k + j];
            const double s = (double)scales[e];
            const int8_t* q1 = codes[e];
            const int8_t* q3 = codes[e] + n;
            const int8_t* q2 = codes[e] + 2 * n;
            for (int f = 0; f < F; ++f) {
                double a = 0.0, c = 0.0;
                for (int i = 0; i < d; ++i) {
                    a += (s * q1[(int64_t)f * d + i]) * xt[i];
                    c += (s * q3[(int64_t)f * d + i]) * xt[i];
                }
                h[f] = a / (1.0 + exp(-a)) * c;
            }
            const double gw = g[(int64_t)t * k + j];
            for (int i = 0; i < d; ++i) {
                double o = 0.0;
                for (int f = 0; f < F; ++f) o += (s * q2[(int64_t)i * F + f]) * h[f];
                yt[i] += gw * o;
            }
        }
    }
    return 0;
}

}  // extern "C"
