// NF4 codebook and quantizer thresholds, built on the host once.
//
// chkda.github.io "Why do we need LoRA and QLoRA?", section "Building the NF4
// codebook": equally spaced cumulative probabilities become standard-normal
// quantiles, then the set is normalised to [-1, 1]; the section notes that the
// sketch needs a finite tail cutoff and an exact zero, and the section "NF4:
// Choose the codebook to fit the distribution" prints the result (exact 0,
// 7 negative and 8 positive levels, -1 and +1 at the ends).  The construction
// used here: with p = 0.967705, positive levels Q(p - i (p - 1/2) / 8) for
// i = 0..7, negative levels -Q(p - i (p - 1/2) / 7) for i = 0..6, plus 0,
// divided by the largest magnitude and rounded to fp32.  This reproduces every
// printed 4-decimal level and the 5-decimal 0.16093 of the worked example.
//
// Q is computed here by bisection on the standard-normal CDF
// Phi(z) = erfc(-z / sqrt(2)) / 2 with the C library's erfc.
#include <algorithm>
#include <cmath>

#include "launch.hpp"

namespace qnf4 {
namespace {

constexpr double kPMax = 0.967705;

double normal_cdf(double z) { return 0.5 * std::erfc(-z / std::sqrt(2.0)); }

// Smallest-bracket bisection: stops when the midpoint no longer moves.
double normal_quantile(double p) {
    double lo = -40.0, hi = 40.0;
    for (int it = 0; it < 2000; ++it) {
        const double mid = 0.5 * (lo + hi);
        if (mid <= lo || mid >= hi) break;
        if (normal_cdf(mid) < p) lo = mid; else hi = mid;
    }
    return 0.5 * (lo + hi);
}

Nf4Consts build() {
    double v[16];
    int n = 0;
    for (int i = 0; i < 8; ++i) v[n++] = normal_quantile(kPMax - i * (kPMax - 0.5) / 8.0);
    for (int i = 0; i < 7; ++i) v[n++] = -normal_quantile(kPMax - i * (kPMax - 0.5) / 7.0);
    v[n++] = 0.0;
    std::sort(v, v + 16);
    double top = 0.0;
    for (double x : v) top = std::max(top, std::fabs(x));
    Nf4Consts t{};
    for (int j = 0; j < 16; ++j) t.level[j] = static_cast<float>(v[j] / top);
    // T_j: the smallest fp32 strictly above the exact midpoint of C[j], C[j+1]
    // (the sum of two fp32 values of magnitude <= 1 is exact in double).
    for (int j = 0; j < 15; ++j) {
        const double mid = (static_cast<double>(t.level[j]) + static_cast<double>(t.level[j + 1])) * 0.5;
        float f = static_cast<float>(mid);
        if (static_cast<double>(f) <= mid) f = std::nextafter(f, INFINITY);
        t.thresh[j] = f;
    }
    t.bucket_ok = 1;
    for (int j = 0; j < 15; ++j) {
        const float ty = t.thresh[j] * 64.0f + 64.0f;  // the kernel's fp32 arithmetic
        if (std::fabs(ty - std::nearbyint(ty)) <= 0x1p-11f) t.bucket_ok = 0;
    }
    return t;
}

}  // namespace

const Nf4Consts &nf4_consts() {
    static const Nf4Consts table = build();  // thread-safe one-time initialisation
    return table;
}

}  // namespace qnf4
