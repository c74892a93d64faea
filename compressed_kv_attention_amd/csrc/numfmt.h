// Device number-format helpers shared by the encode and pack kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ada {

// double -> IEEE binary16, round to nearest with ties to even, magnitudes
// that would round past 65504 saturate to 65504, NaN -> quiet NaN.  Works on
// the bits so the double is rounded once (going through float would round
// twice).
__device__ __forceinline__ uint16_t f64_to_f16_sat(double x)
{
    const uint64_t b = (uint64_t)__double_as_longlong(x);
    const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
    const uint64_t a = b & 0x7fffffffffffffffull;
    if (a > 0x7ff0000000000000ull)
        return 0x7e00;
    if (a >= 0x40effe0000000000ull) // 65520.0: rounds past the largest finite
        return sign | 0x7bff;
    const int e = (int)(a >> 52) - 1023;
    if (e < -25) // below half the smallest subnormal (2^-25 itself ties to 0)
        return sign;
    const uint64_t m = (a & 0x000fffffffffffffull) | 0x0010000000000000ull;
    const int qe = e < -14 ? -14 : e;          // exponent of the target binade
    const int shift = 42 + (qe - e);           // 52 - 10 fraction bits, more when subnormal
    uint64_t n = m >> shift;
    const uint64_t rem = m & ((1ull << shift) - 1);
    const uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (n & 1)))
        n++;
    if (e < -14)
        return sign | (uint16_t)n; // subnormal (n == 1024 is the smallest normal)
    return sign | (uint16_t)((((uint32_t)(e + 15)) << 10) + (uint32_t)(n - 1024));
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h)
{
    return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b)
{
    return __uint_as_float((uint32_t)b << 16);
}

// float -> bfloat16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Byte offset of element (t, d) in a wide (2-byte) / narrow (1-byte)
// section: lane (t % 8) * 8 + d / B holds slots t % 8 and t % 8 + 8 over
// dims [d / B * B, +B), B = D / 8; chunk c of every lane is the c-th KiB.
__device__ __forceinline__ int wide_off(int D, int t, int d)
{
    const int B = D / 8;
    const int lane = (t % 8) * 8 + d / B, w = (t / 8) * B + d % B;
    return (w / 8) * 1024 + lane * 16 + (w % 8) * 2;
}
__device__ __forceinline__ int narrow_off(int D, int t, int d)
{
    const int B = D / 8;
    const int lane = (t % 8) * 8 + d / B, w = (t / 8) * B + d % B;
    return (w / 16) * 1024 + lane * 16 + (w % 16);
}

} // namespace ada
