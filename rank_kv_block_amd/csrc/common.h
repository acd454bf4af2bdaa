// Shared device/host helpers of the predictor library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

namespace pred {

// Bits of the device error word.
enum : uint32_t { DEVERR_TABLE = 1u, DEVERR_FILL = 2u };

__host__ __device__ inline uint64_t f64_bits(double x) {
#if defined(__HIP_DEVICE_COMPILE__)
    return (uint64_t)__double_as_longlong(x);
#else
    uint64_t b;
    memcpy(&b, &x, 8);
    return b;
#endif
}

// float64 -> bf16 bit pattern, round to nearest, ties to even, in one step from
// the float64 value (no float32 intermediate, so no double rounding).  Keeps
// bf16 subnormals, overflows to +/-inf, maps NaN to 0x7FC0.
//
// Works on the integer significand: the bf16 quantum is 2^qe with
// qe = max(e, -126) - 7 for a value with leading-bit exponent e; the
// significand is shifted right to units of 2^qe and rounded half-even on the
// bits shifted out.  The biased bf16 pattern is then ((qe + 133) << 7) + n,
// which also carries a rounding overflow of n = 256 into the exponent and gives
// the subnormal encoding when qe = -133.
//
// Values in bf16's normal range (2^-126 <= |x| < 2^128) take a shorter route
// with the same result: there the quantum is the float64 significand's bit 45,
// so adding 2^44 - 1 plus bit 45 (half-even) and dropping 45 bits rounds the
// 7-bit fraction in place, a carry moving into the exponent; subtracting
// (1023 - 127) << 7 rebiases the exponent (a carry up to 2^128 lands exactly on
// the infinity pattern).
__host__ __device__ inline uint16_t f64_to_bf16_rne(double x) {
    const uint64_t b = f64_bits(x);
    const uint32_t sign = (uint32_t)(b >> 48) & 0x8000u;
    const uint64_t a = b & 0x7FFFFFFFFFFFFFFFull;
    if (a - 0x3810000000000000ull < 0x47F0000000000000ull - 0x3810000000000000ull) {
        const uint64_t r = (a + 0x00000FFFFFFFFFFFull + ((a >> 45) & 1ull)) >> 45;
        return (uint16_t)(sign | ((uint32_t)r - (896u << 7)));
    }
    if (a > 0x7FF0000000000000ull) return 0x7FC0;     // NaN
    const int biased = (int)(a >> 52);
    if (biased == 0) return (uint16_t)sign;            // zero / float64 subnormal -> +/-0
    const int e = biased - 1023;
    if (e >= 128) return (uint16_t)(sign | 0x7F80u);   // >= 2^128, inf
    const uint64_t sig = (a & 0x000FFFFFFFFFFFFFull) | 0x0010000000000000ull;
    const int qe = (e > -126 ? e : -126) - 7;
    const int s = 52 + qe - e;                         // >= 45
    uint64_t n = 0;
    if (s < 64) {
        n = sig >> s;
        const uint64_t rem = sig & ((1ull << s) - 1ull);
        const uint64_t half = 1ull << (s - 1);
        if (rem > half || (rem == half && (n & 1ull))) ++n;
    }
    uint32_t mag = ((uint32_t)(qe + 133) << 7) + (uint32_t)n;
    if (mag >= 0x7F80u) mag = 0x7F80u;
    return (uint16_t)(sign | mag);
}

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Totally ordered uint32 key of a float32 score: ascending key = ascending
// score; -0 and +0 share a key; every NaN gets key 0 (ranks first).
__device__ inline uint32_t order_key(float x) {
    uint32_t u = __float_as_uint(x);
    if (u == 0x80000000u) u = 0u;
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0u;
    return (u & 0x80000000u) ? ~u : (u ^ 0x80000000u);
}

// Float max of v into the float at p, on its bit pattern: non-negative floats
// order as signed integers, negative ones in reverse as unsigned integers, so
// an integer max (v >= 0) or min (v < 0) is the float max.  A score starts at
// -inf (0xFF800000), the identity of both.  The quiet NaN 0x7FC00000, stored
// with the integer max, stays once stored: as a signed integer it is above
// every finite or infinite non-negative pattern, and as an unsigned integer
// above every negative one.
__device__ inline void atomic_max_bits(uint32_t* p, float v) {
    const uint32_t u = __float_as_uint(v);
    if ((int32_t)u >= 0) atomicMax(reinterpret_cast<int*>(p), (int)u);
    else atomicMin(p, u);
}

// MFMA operand and accumulator types (v_mfma_f32_32x32x16_bf16).
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// 16 bytes as a plain vector (uint4 is a union-based struct, which keeps arrays
// of it from being split into registers)
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Eight bf16 from 16 aligned bytes.
__device__ inline bf16x8_t load8(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
}

// A float from another lane: M = 1, 2 swap neighbours and pairs (DPP quad
// permutes); M = 7 and 15 mirror within 8 and 16 lanes (DPP row half-mirror and
// mirror: after the quads agree, one step combines the two quads or the two
// halves); other M through ds_swizzle / ds_bpermute.
template <int M>
__device__ inline float lane_xor(float v) {
    if constexpr (M == 1) return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));
    if constexpr (M == 2) return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true));
    if constexpr (M == 7) return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, true));
    if constexpr (M == 15) return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, true));
    return __shfl_xor(v, M);
}


}  // namespace pred
