// RDR for gfx950: angular error of the stored codes and the byte-budget solver.
//
// SPHERICAL KV (arXiv 2605.18856), gist.science technical summary, section
// 2.2: "Joint Optimization" (a residency bit and a precision tier per
// token/head state, chosen by a discrete rate-distortion allocation under a
// fixed memory budget), "Distortion Surrogate" (the logit error is taken to be
// the angular approximation error scaled by the query and key magnitudes) and
// "Protection Constraints" (protected states stay at the top tier).
//
// The solver is the Lagrangian (lower-convex-hull) solution of that
// multiple-choice knapsack, per sequence over all of its (token, kv-head)
// states:
//   rate of a state in tier b      R_b = page bytes of tier b / 16, R_3 = 0
//   distortion                     D_b = w r~ e_b, e = 0, sqrt(err8),
//                                  sqrt(err4), 1 (dropped)
//   w the utility score, r~ the stored radius.  Each state's hull gives a
//   chain of demotions whose slopes (distortion added per byte saved) do not
//   decrease.  With need = (bytes at tier 0) - cap, where the cap keeps 15
//   slots of each tier per row in reserve for partial pages, s* is the least
//   slope whose demotions of slope <= s* save `need` bytes, and every state
//   takes the prefix of its chain with slopes <= s*.
// s* is found exactly by a radix select over the 32-bit order-preserving key
// of the slope: four passes of 8 bits, each a histogram of the bytes saved
// per digit among the demotions that match the digits found so far.  The
// arithmetic that decides the chains is binary32 in a fixed order (IEEE
// division and square root), so every decision is reproducible.
//
// Kernels: code_error (64 states per block), solve_zero (clears the digit
// histograms), solve_pass<P> (P = 0..3; one block per 1024 states of one
// sequence), solve_assign (writes the tiers), tier_counts (one block per
// row).
#include "ada_internal.h"
#include "numfmt.h"

namespace ada {
namespace {

#pragma clang fp contract(off)

// ---- angular error of the codes ---------------------------------------------
// err = sum_g || u_g - C_g[code_g] ||^2 with u = k / ||k|| in double: the norm
// summed sequentially over the D coordinates, each group's distance summed
// over its 8 coordinates, groups added in order, the total rounded to f32.
// A block takes 64 consecutive states: their keys are staged in LDS with
// coalesced 16-byte loads; one wave sums the 64 norms; every thread then
// scores a quarter of one state's groups; 64 threads add each state's group
// distances in order.
constexpr int kErrItems = 64;

template <int D>
__global__ __launch_bounds__(256) void code_error_kernel(int Hkv, int64_t n_items, const uint16_t *keys,
                                                         const float *cb8, const float *cb4,
                                                         const uint8_t *codes8, const uint8_t *codes4,
                                                         float *err8, float *err4)
{
    constexpr int G = D / 8;
    constexpr int RW = D / 2 + 1;  // LDS row stride in words (odd: the norm loop is conflict-free)
    constexpr int GPT = G / 4;     // groups per thread
    __shared__ uint32_t xk[kErrItems * RW];
    __shared__ double rn[kErrItems];
    __shared__ double d8s[kErrItems][G], d4s[kErrItems][G];
    const int tid = threadIdx.x;
    const int64_t e0 = (int64_t)blockIdx.x * kErrItems;
    const int n_here = (int)(n_items - e0 < kErrItems ? n_items - e0 : kErrItems);
    for (int i = tid; i < kErrItems * (D / 8); i += 256) {
        const int it = i / (D / 8), c = i % (D / 8);
        uint4 w = make_uint4(0, 0, 0, 0);
        if (it < n_here)
            w = *reinterpret_cast<const uint4 *>(keys + (e0 + it) * D + 8 * c);
        uint32_t *dst = xk + it * RW + 4 * c;
        dst[0] = w.x;
        dst[1] = w.y;
        dst[2] = w.z;
        dst[3] = w.w;
    }
    __syncthreads();
    if (tid < kErrItems) {
        double ss = 0.0;
        for (int c = 0; c < D / 2; c++) {
            const uint32_t w = xk[tid * RW + c];
            const double lo = (double)f16_bits_to_f32((uint16_t)(w & 0xffff));
            const double hi = (double)f16_bits_to_f32((uint16_t)(w >> 16));
            ss = ss + lo * lo;
            ss = ss + hi * hi;
        }
        rn[tid] = sqrt(ss);
    }
    __syncthreads();
    {
        const int it = tid / 4, g0 = (tid % 4) * GPT;
        if (it < n_here) {
            const int64_t e = e0 + it;
            const int h = (int)(e % Hkv);
            const double r = rn[it];
#pragma unroll
            for (int gi = 0; gi < GPT; gi++) {
                const int g = g0 + gi;
                const int c8 = codes8[e * G + g];
                const int c4 = (codes4[e * (G / 2) + g / 2] >> (4 * (g & 1))) & 15;
                const float4 *p8 = reinterpret_cast<const float4 *>(cb8 + (((size_t)h * G + g) * kCodes8 + c8) * 8);
                const float4 *p4 = reinterpret_cast<const float4 *>(cb4 + (((size_t)h * G + g) * kCodes4 + c4) * 8);
                const float4 a0 = p8[0], a1 = p8[1], b0 = p4[0], b1 = p4[1];
                const float w8[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                const float w4[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
                double d8 = 0.0, d4 = 0.0;
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const uint32_t w = xk[it * RW + 4 * g + q];
                    const double lo = (double)f16_bits_to_f32((uint16_t)(w & 0xffff));
                    const double hi = (double)f16_bits_to_f32((uint16_t)(w >> 16));
                    const double u0 = r > 0.0 ? lo / r : 0.0;
                    const double u1 = r > 0.0 ? hi / r : 0.0;
                    const double x0 = u0 - (double)w8[2 * q], y0 = u0 - (double)w4[2 * q];
                    d8 = d8 + x0 * x0;
                    d4 = d4 + y0 * y0;
                    const double x1 = u1 - (double)w8[2 * q + 1], y1 = u1 - (double)w4[2 * q + 1];
                    d8 = d8 + x1 * x1;
                    d4 = d4 + y1 * y1;
                }
                d8s[it][g] = d8;
                d4s[it][g] = d4;
            }
        }
    }
    __syncthreads();
    if (tid < n_here) {
        double e8 = 0.0, e4 = 0.0;
        for (int g = 0; g < G; g++) {
            e8 = e8 + d8s[tid][g];
            e4 = e4 + d4s[tid][g];
        }
        err8[e0 + tid] = (float)e8;
        err4[e0 + tid] = (float)e4;
    }
}

// ---- budget solver ------------------------------------------------------------
// Order-preserving map of a finite float to uint32 (-0 becomes +0 first).
__device__ __forceinline__ uint32_t ord_key(float f)
{
    const uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Demotion chain of one state: n <= 3 steps, each with its slope key, the
// bytes it saves and the tier it ends at.
struct Chain {
    uint32_t key[3];
    int dr[3], to[3], n;
};

__device__ __forceinline__ Chain make_chain(int D, float w, uint16_t rbits, float e8, float e4)
{
    const int R1 = page_bytes(D, 1) / kSlots, R2 = page_bytes(D, 2) / kSlots, R0 = page_bytes(D, 0) / kSlots;
    const float wr = w * f16_bits_to_f32(rbits);
    const float D1 = wr * sqrtf(e8), D2 = wr * sqrtf(e4), D3 = wr;
    auto dist = [&](int i) { return i == 0 ? 0.0f : i == 1 ? D1 : i == 2 ? D2 : D3; };
    auto rate = [&](int i) { return i == 0 ? R0 : i == 1 ? R1 : i == 2 ? R2 : 0; };
    // (every loop is unrolled and every array index constant, so the chain
    // lives in registers)
    Chain ch;
    ch.n = 0;
    int c = 0;
    float prev = -INFINITY;
#pragma unroll
    for (int it = 0; it < 3; it++) {
        const bool active = c < 3;
        int best = -1;
        float bs = 0.0f;
#pragma unroll
        for (int j = 1; j < 4; j++) {
            if (j > c) {
                const float sl = (dist(j) - dist(c)) / (float)(rate(c) - rate(j)) + 0.0f;
                if (best < 0 || sl <= bs) {
                    best = j;
                    bs = sl;
                }
            }
        }
        bs = bs < prev ? prev : bs;
        ch.key[it] = active ? ord_key(bs) : 0u;
        ch.dr[it] = active ? rate(c) - rate(best) : 0;
        ch.to[it] = active ? best : 3;
        ch.n += active ? 1 : 0;
        if (active) {
            prev = bs;
            c = best;
        }
    }
    return ch;
}

// Selection state of one sequence after `passes` histogram scans.
struct Sel {
    uint32_t prefix;    // digits found so far
    long long need;     // bytes still to save inside that prefix
    int state;          // 0 searching / exact, 1 no demotion at all, 2 every demotion
};

// One wave: walks the digit histograms of passes 0 .. passes-1.  Digit d of a
// pass is the least with (bytes of digits <= d) >= need.  Every lane returns
// the same result.
__device__ Sel select_prefix(const SolveArgs &a, int s, int passes)
{
    const int lane = threadIdx.x & 63;
    Sel r;
    r.prefix = 0;
    r.need = a.seqs[s].need;
    r.state = r.need <= 0 ? 1 : 0;
    for (int p = 0; p < passes && r.state == 0; p++) {
        const unsigned long long *h = a.hist + ((size_t)p * a.S + s) * 256 + 4 * lane;
        const unsigned long long b0 = h[0], b1 = h[1], b2 = h[2], b3 = h[3];
        const unsigned long long mine = b0 + b1 + b2 + b3;
        unsigned long long incl = mine;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const unsigned long long t = __shfl_up(incl, o, 64);
            if (lane >= o)
                incl += t;
        }
        const unsigned long long need = (unsigned long long)r.need;
        const unsigned long long hit = __ballot(incl >= need);
        if (hit == 0) { // the demotions cannot save enough: take them all
            r.state = 2;
            break;
        }
        const int f = __ffsll((long long)hit) - 1;
        // in lane f: the first of its four digits that reaches the need
        unsigned long long cum = incl - mine;
        int d = 3;
        long long rem = 0;
        const unsigned long long bb[4] = {b0, b1, b2, b3};
        for (int k = 0; k < 4; k++) {
            if (cum + bb[k] >= need) {
                d = k;
                break;
            }
            cum += bb[k];
        }
        rem = (long long)(need - cum);
        d = __shfl(4 * lane + d, f, 64);
        rem = __shfl(rem, f, 64);
        r.prefix = (r.prefix << 8) | (uint32_t)d;
        r.need = rem;
    }
    return r;
}

// Clears the digit histograms; gives every sequence's threshold its value
// for the cases with no search (no demotion needed: -inf; every demotion:
// +inf, the result for a sequence with no states and a negative cap).
__global__ __launch_bounds__(256) void solve_zero(SolveArgs a, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n)
        a.hist[i] = 0ull;
    if (a.threshold != nullptr && i < a.S)
        a.threshold[i] = a.seqs[i].need <= 0 ? -INFINITY : INFINITY;
}

template <int P>
__global__ __launch_bounds__(kSolveThreads) void solve_pass(SolveArgs a)
{
    __shared__ unsigned long long h[256];
    __shared__ Sel sel;
    const SolveBlock blk = a.blocks[blockIdx.x];
    const SolveSeq sq = a.seqs[blk.seq];
    const int tid = threadIdx.x;
    if (sq.need <= 0)
        return;
    h[tid] = 0ull;
    if (tid < 64) {
        const Sel r = select_prefix(a, blk.seq, P);
        if (tid == 0)
            sel = r;
    }
    __syncthreads();
    if (sel.state != 0)
        return;
    const uint32_t prefix = sel.prefix;
    const int64_t end = sq.begin + sq.n_items;
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const int64_t i = blk.first + tid + k * kSolveThreads;
        if (i >= end || (a.protect != nullptr && a.protect[i] != 0))
            continue;
        const Chain ch = make_chain(a.D, a.scores[i], a.radius[i], a.err8[i], a.err4[i]);
#pragma unroll
        for (int n = 0; n < 3; n++) {
            const uint32_t key = ch.key[n];
            if (n < ch.n && (P == 0 || (key >> (32 - 8 * P)) == prefix))
                atomicAdd(&h[(key >> (24 - 8 * P)) & 255u], (unsigned long long)ch.dr[n]);
        }
    }
    __syncthreads();
    if (h[tid] != 0ull)
        atomicAdd(&a.hist[((size_t)P * a.S + blk.seq) * 256 + tid], h[tid]);
}

__global__ __launch_bounds__(kSolveThreads) void solve_assign(SolveArgs a)
{
    __shared__ Sel sel;
    const SolveBlock blk = a.blocks[blockIdx.x];
    const SolveSeq sq = a.seqs[blk.seq];
    const int tid = threadIdx.x;
    if (tid < 64) {
        const Sel r = select_prefix(a, blk.seq, kSolvePasses);
        if (tid == 0)
            sel = r;
    }
    __syncthreads();
    const int state = sel.state;
    const uint32_t kstar = sel.prefix;
    if (a.threshold != nullptr && tid == 0 && blk.first == sq.begin) {
        // s* back from its order-preserving key
        const uint32_t bits = (kstar & 0x80000000u) ? (kstar & 0x7fffffffu) : ~kstar;
        a.threshold[blk.seq] = state == 1 ? -INFINITY : state == 2 ? INFINITY : __uint_as_float(bits);
    }
    const int64_t end = sq.begin + sq.n_items;
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const int64_t i = blk.first + tid + k * kSolveThreads;
        if (i >= end)
            continue;
        int t = 0;
        if (state != 1 && (a.protect == nullptr || a.protect[i] == 0)) {
            const Chain ch = make_chain(a.D, a.scores[i], a.radius[i], a.err8[i], a.err4[i]);
            bool go = true;
#pragma unroll
            for (int n = 0; n < 3; n++) {
                go = go && n < ch.n && (state == 2 || ch.key[n] <= kstar);
                t = go ? ch.to[n] : t;
            }
        }
        a.tiers[i] = (uint8_t)t;
    }
}

// ---- per-row tier counts --------------------------------------------------------
__global__ __launch_bounds__(256) void tier_counts_kernel(int Hkv, const int32_t *cu, const uint8_t *tiers,
                                                          int32_t *counts)
{
    __shared__ int part[4][3];
    const int row = blockIdx.x, s = row / Hkv, h = row % Hkv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int c[3] = {0, 0, 0};
    // eight tokens per thread per round, their loads issued together
    const int64_t t0 = cu[s], t1 = cu[s + 1];
    int64_t t = t0 + tid;
    for (; t + 7 * 256 < t1; t += 8 * 256) {
        int v[8];
#pragma unroll
        for (int j = 0; j < 8; j++)
            v[j] = tiers[(t + j * 256) * Hkv + h];
#pragma unroll
        for (int j = 0; j < 8; j++) {
            c[0] += v[j] == 0;
            c[1] += v[j] == 1;
            c[2] += v[j] == 2;
        }
    }
    for (; t < t1; t += 256) {
        const int v = tiers[t * Hkv + h];
        c[0] += v == 0;
        c[1] += v == 1;
        c[2] += v == 2;
    }
#pragma unroll
    for (int k = 0; k < 3; k++) {
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1)
            c[k] += __shfl_xor(c[k], o, 64);
        if (lane == 0)
            part[wave][k] = c[k];
    }
    __syncthreads();
    if (tid < 3)
        counts[row * 3 + tid] = part[0][tid] + part[1][tid] + part[2][tid] + part[3][tid];
}

} // namespace

hipError_t launch_code_error(int D, int Hkv, int64_t n_tokens, const uint16_t *keys, const float *cb8,
                             const float *cb4, const uint8_t *codes8, const uint8_t *codes4,
                             float *err8, float *err4, hipStream_t st)
{
    const int64_t n = n_tokens * Hkv;
    if (n == 0)
        return hipSuccess;
    const dim3 grid((unsigned)((n + kErrItems - 1) / kErrItems));
    if (D == 128)
        hipLaunchKernelGGL(code_error_kernel<128>, grid, dim3(256), 0, st, Hkv, n, keys, cb8, cb4, codes8,
                           codes4, err8, err4);
    else if (D == 64)
        hipLaunchKernelGGL(code_error_kernel<64>, grid, dim3(256), 0, st, Hkv, n, keys, cb8, cb4, codes8,
                           codes4, err8, err4);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_solve(const SolveArgs &a, hipStream_t st)
{
    if (a.S == 0)
        return hipSuccess;
    const int64_t nh = (int64_t)kSolvePasses * a.S * 256;
    hipLaunchKernelGGL(solve_zero, dim3((unsigned)((nh + 255) / 256)), dim3(256), 0, st, a, nh);
    if (hipError_t e = hipGetLastError(); e != hipSuccess)
        return e;
    const dim3 grid((unsigned)a.n_blocks), blk(kSolveThreads);
    hipLaunchKernelGGL(solve_pass<0>, grid, blk, 0, st, a);
    hipLaunchKernelGGL(solve_pass<1>, grid, blk, 0, st, a);
    hipLaunchKernelGGL(solve_pass<2>, grid, blk, 0, st, a);
    hipLaunchKernelGGL(solve_pass<3>, grid, blk, 0, st, a);
    hipLaunchKernelGGL(solve_assign, grid, blk, 0, st, a);
    return hipGetLastError();
}

hipError_t launch_tier_counts(int Hkv, int S, const int32_t *cu_dev, const uint8_t *tiers, int32_t *counts,
                              hipStream_t st)
{
    if (S * Hkv == 0)
        return hipSuccess;
    hipLaunchKernelGGL(tier_counts_kernel, dim3((unsigned)(S * Hkv)), dim3(256), 0, st, Hkv, cu_dev, tiers,
                       counts);
    return hipGetLastError();
}

} // namespace ada
