// Host generator of the projection P (predictor.rs page: P is written once, in
// the constructor, from projection_seed; the generator itself is not on the
// pages).  P[d, j] = bf16(z / sqrt(r)) with z standard normal number d*r + j of
// stream 0, from this counter-based rule:
//   mix64            SplitMix64 output function (Steele, Lea & Flood 2014)
//   stream state     s = mix64(seed + (stream + 1) * GAMMA)
//   64-bit draw i    x_i = mix64(s + (i + 1) * GAMMA)
//   uniform (0, 1]   ((x >> 11) + 1) * 2^-53
//   normal i         sqrt(-2 ln u(x_2i)) * cos(2 pi u(x_2i+1))   (Box-Muller, cosine branch)
// all in float64 with the C library's log/cos/sqrt, rounded once to bf16 (RNE).
// Built without fast-math or FMA contraction so every step is one IEEE operation.
#include <cmath>
#include <cstdint>

#include "common.h"

namespace pred {

namespace {
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

double unit_interval(uint64_t x) { return (double)((x >> 11) + 1) * 0x1.0p-53; }
}  // namespace

void build_projection(int head_dim, int r, uint64_t seed, uint16_t* out) {
    const uint64_t s = mix64(seed + 1ull * kGamma);  // stream 0
    const double scale = std::sqrt((double)r);
    const int64_t count = (int64_t)head_dim * r;
    for (int64_t i = 0; i < count; ++i) {
        const double u0 = unit_interval(mix64(s + (uint64_t)(2 * i + 1) * kGamma));
        const double u1 = unit_interval(mix64(s + (uint64_t)(2 * i + 2) * kGamma));
        const double z = std::sqrt(-2.0 * std::log(u0)) * std::cos(6.283185307179586 * u1);
        out[i] = f64_to_bf16_rne(z / scale);
    }
}

}  // namespace pred
