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

// Byte offsets of element (slot t, dim d) in a page section: 64 lanes of
// 16-byte chunks, chunk c of every lane forming the c-th KiB, dims in blocks
// b = d / 16.  Row sections (keys) give lane t + 16 q dims 4q..4q+3 of each
// block; column sections (values) give lane n + 16 r slots 4r..4r+3 of dim n
// of each block -- the B-operand layouts of a 16x16x16 MFMA.
__device__ __forceinline__ int row_off(int t, int d)
{
    const int b = d / 16;
    return (b / 2) * 1024 + (t + 16 * ((d % 16) / 4)) * 16 + (b % 2) * 8 + (d % 4) * 2;
}
__device__ __forceinline__ int col_off(int t, int d)
{
    const int b = d / 16;
    return (b / 2) * 1024 + (d % 16 + 16 * (t / 4)) * 16 + (b % 2) * 8 + (t % 4) * 2;
}
__device__ __forceinline__ int col8_off(int t, int d)
{
    const int b = d / 16;
    return (b / 4) * 1024 + (d % 16 + 16 * (t / 4)) * 16 + (b % 4) * 4 + t % 4;
}

} // namespace ada
