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
// Kernels: code_error (256 tokens of one kv-head per block), solve_zero (clears the digit
// histograms), solve_pass<P> (P = 0..3; one block per 1024 states of one
// sequence), solve_assign (writes the tiers), tier_counts (one block per
// row).
#include "ada_internal.h"
#include "code_err.h"
#include "div_rn.h"
#include "numfmt.h"

namespace ada {
namespace {

#pragma clang fp contract(off)

// ---- angular error of the codes ---------------------------------------------
// err = sum_g || u_g - C_g[code_g] ||^2 with u = k / ||k|| in double: the norm
// summed sequentially over the D coordinates, each group's distance summed
// over its 8 coordinates, groups added in order, the total rounded to f32.
// A block takes 256 consecutive tokens of one kv-head, one state per
// thread.  The keys are loaded with 16-byte loads (64 contiguous bytes per
// key and load) and passed through LDS, 32 dimensions a round, so each
// thread ends with its own key in registers.  The head's codebooks are
// staged in LDS one group at a time (8-bit and 4-bit codewords, 8.5 KiB,
// double-buffered; each group's loads are issued two groups ahead), so each
// state's codewords are LDS reads rather than scattered global loads.  The
// distances use the fast form of code_err.h; a state whose rounding test
// fails is recomputed as defined, its codewords then read from global
// memory.  (Gathering every state's codewords from global memory, 256
// consecutive states of all heads per block, kept the kernel waiting on
// its loads about two thirds of the time: 2.5 ms at 19.5 M states.)
typedef float cbvec __attribute__((ext_vector_type(4))); // (a plain vector type stays in registers)
constexpr int kErrItems = 256;                         // tokens per block, one per thread
constexpr int kCbVec = (kCodes8 + kCodes4) * 8 / 4;    // float4 per group's codebooks (544)
constexpr int kCbPer = (kCbVec + kErrItems - 1) / kErrItems;

// The 8-bit and 4-bit codewords of group g of one state (two float4 each).
__device__ __forceinline__ void gather_codewords(const float *cb8, const float *cb4, int h, int G, int g,
                                                 const uint32_t *c8w, const uint32_t *c4w, float4 (&w)[4])
{
    const int c8 = (c8w[g / 4] >> (8 * (g % 4))) & 255;
    const int c4 = (c4w[g / 8] >> (4 * (g % 8))) & 15;
    const float4 *p8 = reinterpret_cast<const float4 *>(cb8 + (((size_t)h * G + g) * kCodes8 + c8) * 8);
    const float4 *p4 = reinterpret_cast<const float4 *>(cb4 + (((size_t)h * G + g) * kCodes4 + c4) * 8);
    w[0] = p8[0];
    w[1] = p8[1];
    w[2] = p4[0];
    w[3] = p4[1];
}

// Group g's codebooks of head h as kCbVec float4 (8-bit codewords, then
// 4-bit): thread tid loads entries tid + kErrItems i (the last entry again
// past the end).
__device__ __forceinline__ void load_codebook(const float *cb8, const float *cb4, int h, int G, int g, int tid,
                                              cbvec (&v)[kCbPer])
{
    const cbvec *p8 = reinterpret_cast<const cbvec *>(cb8 + ((size_t)h * G + g) * kCodes8 * 8);
    const cbvec *p4 = reinterpret_cast<const cbvec *>(cb4 + ((size_t)h * G + g) * kCodes4 * 8);
#pragma unroll
    for (int i = 0; i < kCbPer; i++) {
        const int k = min(tid + kErrItems * i, kCbVec - 1);
        v[i] = k < kCodes8 * 2 ? p8[k] : p4[k - kCodes8 * 2];
    }
}
__device__ __forceinline__ void store_codebook(cbvec *dst, int tid, const cbvec (&v)[kCbPer])
{
#pragma unroll
    for (int i = 0; i < kCbPer; i++)
        dst[min(tid + kErrItems * i, kCbVec - 1)] = v[i];
}

// (four waves per SIMD: 128 registers; with three, a third group in flight
// ran slower)
template <int D>
__global__ __launch_bounds__(kErrItems) __attribute__((amdgpu_waves_per_eu(4))) void
code_error_kernel(int Hkv, int64_t n_tokens, const uint16_t *keys, const float *cb8, const float *cb4,
                  const uint8_t *codes8, const uint8_t *codes4, float *err8, float *err4)
{
    constexpr int G = D / 8;
    constexpr int RND = D / 32;  // staging rounds of 32 dimensions
    constexpr int SW = 17;       // LDS row stride in words (odd: conflict-free reads)
    __shared__ uint32_t xs[kErrItems * SW];
    __shared__ cbvec cbs[2][kCbVec];
    const int tid = threadIdx.x;
    const int h = (int)(blockIdx.x % (unsigned)Hkv);
    const int64_t t0 = (int64_t)(blockIdx.x / (unsigned)Hkv) * kErrItems;
    const int n_here = (int)(n_tokens - t0 < kErrItems ? n_tokens - t0 : kErrItems);
    // Load order: this thread's codes, the block's keys, the first group's
    // codebooks.  Threads past the block's end take the last token's codes
    // and key, and write nothing.
    const int64_t e = (t0 + (tid < n_here ? tid : n_here - 1)) * Hkv + h;
    uint32_t c8w[G / 4], c4w[G / 8];
#pragma unroll
    for (int k = 0; k < G / 4; k++)
        c8w[k] = *reinterpret_cast<const uint32_t *>(codes8 + e * G + 4 * k);
#pragma unroll
    for (int k = 0; k < G / 8; k++)
        c4w[k] = *reinterpret_cast<const uint32_t *>(codes4 + e * (G / 2) + 4 * k);
    // round k, load j: chunk c = tid % 4 (8 dims) of token tid / 4 + 64 j
    uint4 kv[RND][4];
#pragma unroll
    for (int k = 0; k < RND; k++) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int it = tid / 4 + 64 * j, c = tid % 4;
            const int64_t ek = (t0 + (it < n_here ? it : n_here - 1)) * Hkv + h;
            kv[k][j] = *reinterpret_cast<const uint4 *>(keys + ek * D + 32 * k + 8 * c);
        }
    }
    // Group k's codebooks are loaded into registers two groups ahead and
    // stored to LDS buffer k % 2 one group ahead: f1 and f2 hold groups
    // g + 1 and g + 2 while group g is computed (named arrays, shifted each
    // group, so they stay in registers).
    cbvec f1[kCbPer], f2[kCbPer];
    load_codebook(cb8, cb4, h, G, 0, tid, f2);
    load_codebook(cb8, cb4, h, G, 1, tid, f1);
    uint32_t kw[D / 2]; // this thread's key, two binary16 values a word
#pragma unroll
    for (int k = 0; k < RND; k++) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int it = tid / 4 + 64 * j, c = tid % 4;
            uint32_t *dst = xs + it * SW + 4 * c;
            dst[0] = kv[k][j].x;
            dst[1] = kv[k][j].y;
            dst[2] = kv[k][j].z;
            dst[3] = kv[k][j].w;
        }
        if (k == 0)
            store_codebook(cbs[0], tid, f2);
        __syncthreads();
#pragma unroll
        for (int c = 0; c < 16; c++)
            kw[16 * k + c] = xs[tid * SW + c];
        __syncthreads();
    }
    // (a binary16 value's square is exact in double, so the fused
    // multiply-add rounds as the ordered sum of squares does)
    double ss = 0.0;
#pragma unroll
    for (int c = 0; c < D / 2; c++) {
        const double lo = (double)f16_bits_to_f32((uint16_t)(kw[c] & 0xffff));
        const double hi = (double)f16_bits_to_f32((uint16_t)(kw[c] >> 16));
        ss = __builtin_fma(lo, lo, ss);
        ss = __builtin_fma(hi, hi, ss);
    }
    const double r = sqrt(ss);
    const bool fin = r > 0.0 && r < INFINITY;
    // (an empty asm that takes the key's registers: the conversions below
    // are redone per group instead of being kept from the norm's, which
    // would hold D doubles)
#pragma unroll
    for (int c = 0; c < D / 2; c++)
        asm volatile("" : "+v"(kw[c]));
    // The fast form (code_err.h): t = RN(x y - w) from y = RN(1 / r),
    // squares added with fused multiply-adds, groups added in order; kept
    // when its binary32 rounding cannot differ from the defined
    // computation's.  Every thread runs the loop (it holds the block's
    // barriers); a non-finite or zero norm takes the defined path below.
    const double y = fin ? 1.0 / r : 0.0;
    double e8 = 0.0, e4 = 0.0;
#pragma unroll
    for (int g = 0; g < G; g++) {
        if (g + 2 < G)
            load_codebook(cb8, cb4, h, G, g + 2, tid, f2);
        const cbvec *cb = cbs[g & 1];
        const int c8 = (c8w[g / 4] >> (8 * (g % 4))) & 255;
        const int c4 = (c4w[g / 8] >> (4 * (g % 8))) & 15;
        const cbvec a0 = cb[2 * c8], a1 = cb[2 * c8 + 1];
        const cbvec b0 = cb[2 * kCodes8 + 2 * c4], b1 = cb[2 * kCodes8 + 2 * c4 + 1];
        const float w8[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        const float w4[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        double d8 = 0.0, d4 = 0.0;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const uint32_t wd = kw[4 * g + j / 2];
            const double x = (double)f16_bits_to_f32((uint16_t)(j & 1 ? wd >> 16 : wd & 0xffff));
            d8 = ce_term(d8, x, y, (double)w8[j]);
            d4 = ce_term(d4, x, y, (double)w4[j]);
        }
        e8 = e8 + d8;
        e4 = e4 + d4;
        // (an empty asm that takes the sums: the group's arithmetic stays
        // ahead of the barrier instead of being deferred past the later
        // groups' LDS reads, which would hold all their codewords)
        asm volatile("" : "+v"(e8), "+v"(e4));
        if (g + 1 < G) {
            store_codebook(cbs[(g + 1) & 1], tid, f1);
            __syncthreads();
        }
#pragma unroll
        for (int i = 0; i < kCbPer; i++) {
            f1[i] = f2[i];
        }
    }
    if (tid >= n_here)
        return;
    if (!(fin && ce_rounds_alike(e8) && ce_rounds_alike(e4))) {
        // As defined: u = x / r rounded (div_rn for a finite positive
        // norm; a zero key gives u = 0, a non-finite norm divides), each
        // difference squared and added with its own rounding.  (The key is
        // read again from global memory: a rolled loop cannot index the
        // key's registers.)
        const uint32_t *kg = reinterpret_cast<const uint32_t *>(keys + e * D);
        e8 = 0.0;
        e4 = 0.0;
        for (int g = 0; g < G; g++) {
            float4 c[4];
            gather_codewords(cb8, cb4, h, G, g, c8w, c4w, c);
            const float w8[8] = {c[0].x, c[0].y, c[0].z, c[0].w, c[1].x, c[1].y, c[1].z, c[1].w};
            const float w4[8] = {c[2].x, c[2].y, c[2].z, c[2].w, c[3].x, c[3].y, c[3].z, c[3].w};
            double d8 = 0.0, d4 = 0.0;
            for (int j = 0; j < 8; j++) {
                const uint32_t wd = kg[4 * g + j / 2];
                const double x = (double)f16_bits_to_f32((uint16_t)(j & 1 ? wd >> 16 : wd & 0xffff));
                const double u = fin ? div_rn(x, r, y) : r > 0.0 ? x / r : 0.0;
                const double xa = u - (double)w8[j], xb = u - (double)w4[j];
                d8 = d8 + xa * xa;
                d4 = d4 + xb * xb;
            }
            e8 = e8 + d8;
            e4 = e4 + d4;
        }
    }
    err8[e] = (float)e8;
    err4[e] = (float)e4;
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

// A thread's four states' inputs, all loaded at kernel start (before the
// digit search, which does not need them): one memory latency.
struct SolveIn {
    float w[4], e8[4], e4[4];
    uint16_t r[4];
    bool live[4];
};

__device__ __forceinline__ SolveIn solve_inputs(const SolveArgs &a, int64_t first, int64_t end, int tid)
{
    SolveIn in;
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const int64_t i = first + tid + k * kSolveThreads;
        const bool ok = i < end;
        const int64_t j = ok ? i : first; // (a valid index; its values are unused)
        in.w[k] = a.scores[j];
        in.r[k] = a.radius[j];
        in.e8[k] = a.err8[j];
        in.e4[k] = a.err4[j];
        in.live[k] = ok && (a.protect == nullptr || a.protect[j] == 0);
    }
    return in;
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
    const int64_t end = sq.begin + sq.n_items;
    const SolveIn in = solve_inputs(a, blk.first, end, tid);
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
#pragma unroll
    for (int k = 0; k < 4; k++) {
        if (!in.live[k])
            continue;
        const Chain ch = make_chain(a.D, in.w[k], in.r[k], in.e8[k], in.e4[k]);
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
    const int64_t end = sq.begin + sq.n_items;
    const SolveIn in = solve_inputs(a, blk.first, end, tid);
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
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const int64_t i = blk.first + tid + k * kSolveThreads;
        if (i >= end)
            continue;
        int t = 0;
        if (state != 1 && in.live[k]) {
            const Chain ch = make_chain(a.D, in.w[k], in.r[k], in.e8[k], in.e4[k]);
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
    if (n_tokens == 0 || Hkv == 0)
        return hipSuccess;
    const int64_t blocks = (n_tokens + kErrItems - 1) / kErrItems * Hkv;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks);
    if (D == 128)
        hipLaunchKernelGGL(code_error_kernel<128>, grid, dim3(kErrItems), 0, st, Hkv, n_tokens, keys, cb8, cb4,
                           codes8, codes4, err8, err4);
    else if (D == 64)
        hipLaunchKernelGGL(code_error_kernel<64>, grid, dim3(kErrItems), 0, st, Hkv, n_tokens, keys, cb8, cb4,
                           codes8, codes4, err8, err4);
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
    if (a.n_blocks == 0) // no states: the thresholds are all the call computes
        return hipSuccess;
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
