// Cross-lane helpers for gfx950 waves (64 lanes): the permlane row swaps
// and a (distance, index) argmin over the wave built from DPP permutes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace ada {

// x of lane (l & ~16) and of lane (l | 16), in that order (rows 2r and
// 2r + 1 of 16 lanes).
__device__ __forceinline__ void pair16(uint32_t x, uint32_t &lo, uint32_t &hi)
{
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    lo = r[0];
    hi = r[1];
}

// x of lane (l & ~32) and of lane (l | 32).
__device__ __forceinline__ void pair32(uint32_t x, uint32_t &lo, uint32_t &hi)
{
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    lo = r[0];
    hi = r[1];
}

// (distance, index) of lane l ^ x, for the DPP permutes within a row
template <int CTRL>
__device__ __forceinline__ void dpp_pair(double d, int i, double &od, int &oi)
{
    const uint64_t v = (uint64_t)__double_as_longlong(d);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xf, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xf, 0xf, false);
    od = __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
    oi = __builtin_amdgcn_mov_dpp(i, CTRL, 0xf, 0xf, false);
}

__device__ __forceinline__ void lexmin(double &d, int &i, double od, int oi)
{
    if (od < d || (od == d && oi < i)) {
        d = od;
        i = oi;
    }
}

// The two lanes' (distance, index) of a permlane pair, merged.
template <bool ROW32>
__device__ __forceinline__ void perm_merge(double &d, int &i)
{
    const uint64_t v = (uint64_t)__double_as_longlong(d);
    uint32_t al, bl, ah, bh, ai, bi;
    if (ROW32) {
        pair32((uint32_t)v, al, bl);
        pair32((uint32_t)(v >> 32), ah, bh);
        pair32((uint32_t)i, ai, bi);
    } else {
        pair16((uint32_t)v, al, bl);
        pair16((uint32_t)(v >> 32), ah, bh);
        pair16((uint32_t)i, ai, bi);
    }
    d = __longlong_as_double((long long)(((uint64_t)ah << 32) | al));
    i = (int)ai;
    lexmin(d, i, __longlong_as_double((long long)(((uint64_t)bh << 32) | bl)), (int)bi);
}

// Lexicographic (distance, index) minimum over the wave, in every lane:
// lane pairs xor 1 and xor 2 (quad permutes), the 8-lane and 16-lane
// mirrors, then rows 2r / 2r + 1 and the two halves.
__device__ __forceinline__ void wave_argmin(double &d, int &i)
{
    double od;
    int oi;
    dpp_pair<0xB1>(d, i, od, oi); // quad_perm 1,0,3,2
    lexmin(d, i, od, oi);
    dpp_pair<0x4E>(d, i, od, oi); // quad_perm 2,3,0,1
    lexmin(d, i, od, oi);
    dpp_pair<0x141>(d, i, od, oi); // row_half_mirror
    lexmin(d, i, od, oi);
    dpp_pair<0x140>(d, i, od, oi); // row_mirror
    lexmin(d, i, od, oi);
    perm_merge<false>(d, i);
    perm_merge<true>(d, i);
}

// Minimum of an unsigned value over the wave, in every lane (the same
// permutes as wave_argmin).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v)
{
    v = min(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xf, 0xf, false));
    v = min(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xf, 0xf, false));
    v = min(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xf, 0xf, false));
    v = min(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xf, 0xf, false));
    uint32_t lo, hi;
    pair16(v, lo, hi);
    v = min(lo, hi);
    pair32(v, lo, hi);
    return min(lo, hi);
}

// Sum of a double over each row of 16 lanes (or each half row of 8 when
// HALF), in every lane of it: quad, half-row and row butterflies.  The
// additions' order differs between lanes, so the lanes agree only when the
// sums are exact.
template <bool HALF>
__device__ __forceinline__ double row_sum_f64(double x)
{
    auto step = [](double y, auto ctrl) {
        const uint64_t v = (uint64_t)__double_as_longlong(y);
        constexpr int C = decltype(ctrl)::value;
        const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, C, 0xf, 0xf, false);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), C, 0xf, 0xf, false);
        return y + __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
    };
    x = step(x, std::integral_constant<int, 0xB1>{});
    x = step(x, std::integral_constant<int, 0x4E>{});
    x = step(x, std::integral_constant<int, 0x141>{});
    if (!HALF)
        x = step(x, std::integral_constant<int, 0x140>{});
    return x;
}

// Minimum of an int over each row of 16 lanes (or half row of 8).
template <bool HALF>
__device__ __forceinline__ int row_min_i32(int x)
{
    x = min(x, __builtin_amdgcn_mov_dpp(x, 0xB1, 0xf, 0xf, false));
    x = min(x, __builtin_amdgcn_mov_dpp(x, 0x4E, 0xf, 0xf, false));
    x = min(x, __builtin_amdgcn_mov_dpp(x, 0x141, 0xf, 0xf, false));
    if (!HALF)
        x = min(x, __builtin_amdgcn_mov_dpp(x, 0x140, 0xf, 0xf, false));
    return x;
}

} // namespace ada
