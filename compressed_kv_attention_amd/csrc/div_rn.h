// Double-precision x / r rounded to nearest from a reciprocal, for the code
// error kernel (keys divided by their norm).
//
// x / r rounded to nearest, for finite r > 0, from y = RN(1 / r) with fused
// multiply-adds (Markstein, "Computation of elementary functions on the IBM
// RISC System/6000 processor", IBM J. Res. Dev. 34(1), 1990).  q0 = x y lies
// within 1.5 ulp of x / r; the correction q1 = q0 + (x - r q0) y lies within
// an ulp, so the residual x - r q1 is exact, and by Markstein's theorem (y
// within half an ulp of 1 / r, q1 within an ulp of x / r) q1 + (x - r q1) y
// rounded once is x / r rounded to nearest.  Valid while no residual
// underflows: here x is a binary16 value (zero or |x| >= 2^-24) and
// 2^-24 <= r < 2^20.  A zero x gives a zero of either sign.
//
// The header compiles as device code by default; a host test build defines
// ADA_DIV_RN_QUAL (e.g. as "static inline") to check it against IEEE
// division on the CPU.
#pragma once

#ifndef ADA_DIV_RN_QUAL
#define ADA_DIV_RN_QUAL __device__ __forceinline__
#endif

ADA_DIV_RN_QUAL double div_rn(double x, double r, double y)
{
    const double q0 = x * y;
    const double q1 = __builtin_fma(__builtin_fma(-q0, r, x), y, q0);
    return __builtin_fma(__builtin_fma(-q1, r, x), y, q1);
}
