// Device helpers shared by the gfx950 kernel files: vector types, wave
// synchronisation, binary16 conversions, the double-binary16 codebook grid and
// the fp32 codewords a_p * q_s (so that every kernel that decodes forms
// bit-identical values).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hqmq {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// Dword 3 of raw buffer resources (gfx9: 32-bit data format, no swizzle):
// loads at or past num_records bytes return 0, stores there are dropped.
constexpr int kBufWord3 = 0x00020000;

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// (e_m * q)[k] = sign(m, k) q[m ^ k] for e = (1, i, j, k) under the Hamilton
// product: i q = (-q1, q0, -q3, q2), j q = (-q2, q3, q0, -q1),
// k q = (-q3, -q2, q1, q0).  Bit (4 m + k) of kNegMask marks a minus sign.
constexpr uint32_t kNegMask = 0x3950u;

__device__ __forceinline__ float unit_row(const float *q, int m, int k) {
    const float v = q[m ^ k];
    return ((kNegMask >> (4 * m + k)) & 1u) ? -v : v;
}

// binary16 helpers (round to nearest even: the hardware default mode).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Codebook values are used on the double-binary16 grid: hi + lo with
// hi = fp16(q), lo = fp16(q - hi) (q - hi and the sum are exact in fp32).
// Generated codebooks are already on it; any other codebook is rounded the
// same way wherever the kernels read it.
__device__ __forceinline__ float double_f16(float q) {
    const _Float16 hi = static_cast<_Float16>(q);
    const _Float16 lo = static_cast<_Float16>(q - static_cast<float>(hi));
    return static_cast<float>(hi) + static_cast<float>(lo);
}

// Codeword a_p * q_s in fp32 from the four rows e_m * q_s.
__device__ __forceinline__ f32x4 codeword_f32(const float *q, int p) {
    f32x4 c;
    if (p < 8) {
        const int m = p >> 1;
        const bool ng = p & 1;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float v = unit_row(q, m, k);
            c[k] = ng ? -v : v;
        }
    } else {
        const int bits = p - 8;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float r[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float v = unit_row(q, m, k);
                r[m] = ((bits >> m) & 1) ? -v : v;
            }
            c[k] = ((r[0] + r[1]) + (r[2] + r[3])) * 0.5f;
        }
    }
    return c;
}

// Compact norm code of a binary16 half-norm record h (b bits, 5 <= b <= 15):
// the flag bit maps to the all-ones code; otherwise h is rounded to a float
// with 5 exponent bits and b - 5 mantissa bits, i.e. to the nearest binary16
// pattern whose low 15 - b bits are zero (positive binary16 patterns are
// ordered like their values and evenly spaced within a binade, so rounding
// the pattern rounds the value; on a tie the even code wins), capped at the
// largest finite value of the narrower format.  The code is the top b bits
// of that pattern.
__device__ __forceinline__ uint32_t compact_norm_code(uint32_t h, int bits) {
    if (h & 0x8000u) return (1u << bits) - 1u;
    const int sh = 15 - bits;
    const uint32_t c = sh > 0 ? (h + (1u << (sh - 1)) - 1u + ((h >> sh) & 1u)) >> sh : h;
    const uint32_t cap = (31u << (bits - 5)) - 1u;
    return c < cap ? c : cap;
}

// The binary16 half-norm record a compact code stands for (the flag for the
// all-ones code).
__device__ __forceinline__ uint32_t compact_norm_h16(uint32_t c, int bits) {
    return c == (1u << bits) - 1u ? 0x8000u : c << (15 - bits);
}

// Exact-rate records (HQMQ_NORM_EXACT, S a power of two): the index and the
// norm code both have R = 24 S = 3 2^m values; a code is 2^m d + l with l
// its m low bits and d a ternary digit.  Digits are stored eight to a
// 13-bit field as sum_i d_i 3^i.
constexpr int kExactRows = 4;          // token rows per group
constexpr int kDigitsPerField = 8;
constexpr int kFieldBits = 13;

// binary16 pattern of norm level n < R - 1: the integer nearest
// n 2^15 / R = n 2^(15 - m) / 3 (never a tie).  n 2^(15 - m) / 3 is at most
// 2^15 and its fraction is 0, 1/3 or 2/3, so the fp32 product with the
// rounded constant (error below 0.01) plus 1/2 truncates to the nearest
// integer.
__device__ __forceinline__ uint32_t exact_level_pattern(uint32_t n, float level_step) {
    return static_cast<uint32_t>(__builtin_fmaf(static_cast<float>(n), level_step, 0.5f));
}

// The binary16 half-norm record an exact-rate norm code stands for: the
// flag for R - 1, else the level's pattern.
__device__ __forceinline__ uint32_t exact_norm_h16(uint32_t n, uint32_t flag_code, float level_step) {
    return n == flag_code ? 0x8000u : exact_level_pattern(n, level_step);
}

// Exact-rate norm code of a binary16 half-norm record h: R - 1 for a flagged
// record; otherwise the level with the nearest value (a tie to the even
// level), at most nmax (the top finite level).  h lies between the patterns
// of levels floor(3 h / 2^(15 - m)) and the next, so those two are compared
// (differences of nearby binary16 values are exact in fp32).  The flag and
// the cap are applied last by selects (the comparison then runs on a
// clamped level, whose result they discard).
__device__ __forceinline__ uint32_t exact_norm_code(uint32_t h, int m, uint32_t nmax, float level_step) {
    const uint32_t hv = h & 0x7FFFu;
    const uint32_t nr = (3u * hv) >> (15 - m);
    const uint32_t n0 = nr < nmax ? nr : nmax;
    const float v = f16_bits_to_f32(static_cast<uint16_t>(hv));
    const float d0 = v - f16_bits_to_f32(static_cast<uint16_t>(exact_level_pattern(n0, level_step)));
    const float d1 = f16_bits_to_f32(static_cast<uint16_t>(exact_level_pattern(n0 + 1u, level_step))) - v;
    uint32_t n = d0 < d1 ? n0 : (d1 < d0 ? n0 + 1u : n0 + (n0 & 1u));
    n = nr >= nmax ? nmax : n;
    return (h & 0x8000u) ? (3u << m) - 1u : n;
}

// floor(q / 3) for q < 2^13 with a full-rate 24-bit multiply:
// ceil(2^16 / 3) = 21846 overestimates 1/3 by 2/3 2^-16, which moves q / 3
// by less than 1/12, and the fraction of q / 3 is at most 2/3.
__device__ __forceinline__ uint32_t div3_small(uint32_t q) { return __umul24(q, 21846u) >> 16; }

}  // namespace
}  // namespace hqmq
