// Fast form of the code error with a rounding test, for the code error
// kernel.
//
// The error of a state's codes is e = sum_g sum_j (u_j - w_j)^2 in double,
// u = x / ||x|| (x the binary16 key), rounded once to binary32.  Computed
// as defined, each coordinate costs a correctly rounded division, a
// subtraction, a square and an addition.  The fast form takes
// t_j = RN(x_j y - w_j) with one fused multiply-add from y = RN(1 / r), and
// adds t_j^2 with another, the groups' sums added as in the definition.
//
// Error bound (u = 2^-53, T = sum_j t_j^2 exactly, r the same norm on both
// sides).  The defined computation rounds x_j / r, the difference and the
// square once each and adds every term at most 22 times, so it lies within
// (25 u) T + 2 u sqrt(T) + 3 u^2 of T; the fast form rounds y, the fused
// difference and at most 22 sums, so it lies within (24 u) T + 2 u sqrt(T) +
// 3 u^2 of T (each coordinate's error is at most u |x_j| / r + u |t_j|, and
// sum_j |x_j| |t_j| / r <= sqrt(T) since sum_j x_j^2 / r^2 is 1 up to
// rounding).  The two values thus differ by less than
//     B = 2^-45 e + 2^-48 sqrt(e) + 2^-100,
// which covers 49 u T + 4 u sqrt(T) + 6 u^2 about four times over.  When the
// binary32 roundings of e - B and e + B agree, every value within B of e,
// the defined one included, rounds to that same binary32 (rounding is
// monotone), and the fast value is returned; otherwise the caller computes
// the state as defined.  Codes at a typical distance from the key
// practically never fail the test; a zero error (a code equal to the key's
// direction) always does.
//
// The header compiles as device code by default; a host test build defines
// ADA_CODE_ERR_QUAL (e.g. as "static inline").
#pragma once

#ifndef ADA_CODE_ERR_QUAL
#define ADA_CODE_ERR_QUAL __device__ __forceinline__
#endif

// acc + (x y - w)^2 with the difference and the sum rounded once each
ADA_CODE_ERR_QUAL double ce_term(double acc, double x, double y, double w)
{
    const double t = __builtin_fma(x, y, -w);
    return __builtin_fma(t, t, acc);
}

// Nonzero when every double within the fast form's error bound of e rounds to
// the same binary32 as e does.
ADA_CODE_ERR_QUAL int ce_rounds_alike(double e)
{
    const float ef = (float)e;
    const float b = 0x1p-45f * ef + 0x1p-48f * __builtin_sqrtf(ef) + 0x1p-100f;
    return (float)(e - (double)b) == (float)(e + (double)b);
}
