// ADA encode for gfx950: scalar radius + per-group nearest-codeword codes.
//
// SPHERICAL KV (arXiv 2605.18856), gist.science technical summary, section
// 2.1 "Spherical Parameterization" (radius and direction of each key) and
// "Compressed-Domain Similarity" (quantized radius, packed angular codes),
// section 2.3 (dense keys are mapped to codes before tiering).  The angle
// code is one codebook index per group of 8 direction coordinates.
//
// Definition kept exactly: the norm is summed in double, sequentially over
// the D coordinates, with no fused multiply-add; the direction is u = k / r
// in double (u = 0 for a zero key); the code is the argmin, lowest index on
// ties, of the double distance sum_j (u_j - c_j)^2 summed in order.
//
// The search is a dense contraction: for a tile of 16 tokens and 16
// codewords the matrix cores form |c|^2 - 2 u.c in binary32 (two chained
// 16x16x4 MFMAs over the 8 coordinates, from an accumulator holding |c|^2),
// so the codebook stays in registers as MFMA operands and the vector ALU
// only keeps each token's best and second-best score.  A binary32 score is
// a filter: where its best two are too close to be ordered for certain (see
// kFilterRel), the token-group is rescanned in double, so the codes are
// still the exact double argmin.
//
// Grid: blocks of (64-token chunk range (grid-stride), kv-head, quarter of
// the groups), XCD-aware (below).  A block has one wave per group of its
// quarter (4 waves).
// Per chunk it stages the 64 keys in LDS and sums a fast-order norm per
// token (four lanes a token); the last wave also sums the defining norms
// (one lane a token) for the radius and the rescans; every wave scores its
// group for the 4 tiles of 16 tokens, queues its near ties, and leaves the
// codes in LDS; the queued rescans are dealt to the waves; byte stores.
#include "ada_internal.h"
#include "numfmt.h"
#include "wave_ops.h"

namespace ada {
namespace {

#pragma clang fp contract(off)

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 64;          // tokens per chunk
constexpr float kCodeMax = 0x1p20f; // larger (or non-finite) codebooks skip the filter

// Filter bound.  Let n = |u|^2 over the group, d the distance of codeword c
// and s = fl(|c|^2 - 2 u.c) the matrix-core score (the accumulator starts
// at the binary32 |c|^2); s estimates d - n and may be negative.  With
// T = |c|^2 + 2 sum_j |u_j c_j| (at most 7 (n + d), since |c| <= |u| +
// sqrt(d)): rounding u to binary32 (through a double reciprocal of a norm
// within 2^-45 of r) moves s by at most 3 2^-24 T; the binary32 |c|^2 by at
// most 2^-21 T; the two MFMAs -- eight products and eight additions, each
// assumed within one ulp (2^-23 relative) whatever the matrix core's order
// and rounding -- by at most 9 2^-23 T.  So |s - (d - n)| <= 2^-16 (n + d).
// The tracked scores also carry a codeword index in their low 6 mantissa
// bits, which moves them by at most 2^-17 |s| <= 2^-17 (n + d).  Together
// eps = 1.5 2^-16, and codeword c is strictly farther in double than the
// best-scored one whenever s_c - s_1 > eps ((n + d_c) + (n + d_1)), i.e.
// eps (4 n + s_c + s_1) up to those same errors; that holds for every c once
// the gap to the second-best score s_2 exceeds eps (4 n + s_1 + s_2).  The
// test below asks for 2^-14 (4 n + s_1 + s_2) with n in binary32, over 2.6
// times that, plus a tiny absolute term for flushed subnormals (codewords
// are at most 2^20 in magnitude on this path).
constexpr float kFilterRel = 0x1p-14f;
constexpr float kFilterAbs = 0x1p-90f;

// Lowest codeword index of the smallest double distance (a NaN distance never
// wins; all NaN or infinite -> 0): the defining scan, shared by the wave.
// u is the group's direction slice in double (the same in every lane).
template <int K>
__device__ __forceinline__ int exact_nearest(const double (&u)[8], const float *cbg, int lane)
{
    constexpr int PER = (K + 63) / 64;
    float4 cw[PER][2];
#pragma unroll
    for (int i = 0; i < PER; i++) { // (all loads first: one memory latency)
        const int c = lane + 64 * i < K ? lane + 64 * i : K - 1;
        cw[i][0] = *reinterpret_cast<const float4 *>(cbg + c * 8);
        cw[i][1] = *reinterpret_cast<const float4 *>(cbg + c * 8 + 4);
    }
    double bd = INFINITY;
    int bi = 0;
#pragma unroll
    for (int i = 0; i < PER; i++) {
        const float cf[8] = {cw[i][0].x, cw[i][0].y, cw[i][0].z, cw[i][0].w,
                             cw[i][1].x, cw[i][1].y, cw[i][1].z, cw[i][1].w};
        double d = 0.0;
#pragma unroll
        for (int q = 0; q < 8; q++) {
            const double df = u[q] - (double)cf[q];
            d = d + df * df;
        }
        if (lane + 64 * i < K && d < bd) {
            bd = d;
            bi = lane + 64 * i;
        }
    }
    wave_argmin(bd, bi);
    return bi;
}

// Sum over the four lanes of a token column (every lane gets the same value:
// each pairwise sum has the same operands in the same order).
__device__ __forceinline__ float column_sum(float x)
{
    uint32_t a, b;
    pair16(__float_as_uint(x), a, b);
    x = __uint_as_float(a) + __uint_as_float(b);
    pair32(__float_as_uint(x), a, b);
    return __uint_as_float(a) + __uint_as_float(b);
}

__device__ __forceinline__ double column_sum(double x)
{
#pragma unroll
    for (int step = 0; step < 2; step++) {
        const uint64_t v = (uint64_t)__double_as_longlong(x);
        uint32_t al, bl, ah, bh;
        if (step == 0) {
            pair16((uint32_t)v, al, bl);
            pair16((uint32_t)(v >> 32), ah, bh);
        } else {
            pair32((uint32_t)v, al, bl);
            pair32((uint32_t)(v >> 32), ah, bh);
        }
        x = __longlong_as_double((long long)(((uint64_t)ah << 32) | al)) +
            __longlong_as_double((long long)(((uint64_t)bh << 32) | bl));
    }
    return x;
}

// The defining norm of a staged key: squares summed in order, in double.
// (The words are read 16 ahead of the adds, so that only the adds form the
// chain.)
template <int D>
__device__ __forceinline__ double exact_norm(const uint32_t *row)
{
    double ss = 0.0;
#pragma unroll
    for (int c0 = 0; c0 < D / 2; c0 += 16) {
        uint32_t kw[16];
#pragma unroll
        for (int c = 0; c < 16; c++)
            kw[c] = row[c0 + c];
#pragma unroll
        for (int c = 0; c < 16; c++) {
            // (a binary16 value's square is exact in double: the fused
            // multiply-add rounds as the sum of the square does)
            const double lo = (double)f16_bits_to_f32((uint16_t)(kw[c] & 0xffff));
            const double hi = (double)f16_bits_to_f32((uint16_t)(kw[c] >> 16));
            ss = __builtin_fma(lo, lo, ss);
            ss = __builtin_fma(hi, hi, ss);
        }
    }
    return sqrt(ss);
}

// A lane's running best two packed scores (value bits | 6-bit slot),
// compared as floats (the minimum is the median of a, b and -inf: no NaN
// reaches this path, and the median needs no canonicalising moves).
struct Best {
    float k1, k2;
};

__device__ __forceinline__ void best_init(Best &s)
{
    s.k1 = __uint_as_float(0x7f7fffffu);
    s.k2 = __uint_as_float(0x7f7fffffu);
}

// ninf: -inf held in a register (the minimum is the median of a, b and -inf)
__device__ __forceinline__ void best_add(Best &s, float score, int slot, float ninf)
{
    const float k = __uint_as_float((__float_as_uint(score) & ~63u) | (uint32_t)slot);
    s.k2 = __builtin_amdgcn_fmed3f(s.k1, s.k2, k);
    s.k1 = __builtin_amdgcn_fmed3f(s.k1, k, ninf);
}

// Best value, its codeword and the second-best value over a token column.
// Equal best values leave v2 == v1, which the filter rejects.
struct Column {
    float v1, v2;
    int i1;
};

__device__ __forceinline__ Column best_column(const Best &s, int cw)
{
    Column c{__uint_as_float(__float_as_uint(s.k1) & ~63u), __uint_as_float(__float_as_uint(s.k2) & ~63u), cw};
#pragma unroll
    for (int step = 0; step < 2; step++) {
        uint32_t a1, b1, a2, b2, ai, bi;
        if (step == 0) {
            pair16(__float_as_uint(c.v1), a1, b1);
            pair16(__float_as_uint(c.v2), a2, b2);
            pair16((uint32_t)c.i1, ai, bi);
        } else {
            pair32(__float_as_uint(c.v1), a1, b1);
            pair32(__float_as_uint(c.v2), a2, b2);
            pair32((uint32_t)c.i1, ai, bi);
        }
        const float x1 = __uint_as_float(a1), y1 = __uint_as_float(b1);
        c.v2 = __builtin_amdgcn_fmed3f(x1, y1, fminf(__uint_as_float(a2), __uint_as_float(b2)));
        const bool lt = y1 < x1;
        c.i1 = lt ? (int)bi : (int)ai;
        c.v1 = lt ? y1 : x1;
    }
    return c;
}

// The defining codes of one group of a key (its 8 fp16 coordinates in kw)
// of norm r (the defining one): direction, then the double scans; which:
// 1 = the 8-bit code, 2 = the 4-bit code.  Returns code8 | code4 << 8.
// Called by the whole wave.
__device__ __attribute__((noinline)) uint32_t rescan(uint4 kw, double r, const float *c8g,
                                                     const float *c4g, int lane, int which)
{
    const uint32_t ws[4] = {kw.x, kw.y, kw.z, kw.w};
    double u[8];
#pragma unroll
    for (int p = 0; p < 8; p++) {
        const uint16_t hb = (uint16_t)(p & 1 ? ws[p / 2] >> 16 : ws[p / 2] & 0xffff);
        u[p] = r > 0.0 ? (double)f16_bits_to_f32(hb) / r : 0.0;
    }
    uint32_t e = 0;
    if (which & 1)
        e |= (uint32_t)exact_nearest<kCodes8>(u, c8g, lane);
    if (which & 2)
        e |= (uint32_t)exact_nearest<kCodes4>(u, c4g, lane) << 8;
    return e;
}

template <int D>
__global__ __launch_bounds__(256, 4) void encode_kernel(int Hkv, int gx, int64_t n_tokens, int64_t n_chunks,
                                                        const uint16_t *__restrict__ keys,
                                                        const float *__restrict__ cb8,
                                                        const float *__restrict__ cb4,
                                                        uint16_t *__restrict__ radius,
                                                        uint8_t *__restrict__ codes8,
                                                        uint8_t *__restrict__ codes4)
{
    constexpr int G = D / 8;
    constexpr int RW = D / 2 + 1; // LDS row stride in 32-bit words (odd: conflict-free norms)
    // the block's four codebooks while the operands are loaded, then a
    // chunk's keys
    constexpr int kCbWords = 4 * (kCodes8 + kCodes4) * 8;
    constexpr int kKeyNormWords = kChunk * RW + 4 * 17 * 16;
    constexpr int kLdsWords = kCbWords > kKeyNormWords ? kCbWords : kKeyNormWords;
    __shared__ __align__(16) uint32_t lds[kLdsWords];
    uint32_t *xk = lds;
    __shared__ double xri[kChunk]; // 1 / (norm in a fast order)
    __shared__ double xr[kChunk];  // the defining norm
    __shared__ uint8_t s8[kChunk][4];
    __shared__ uint8_t s4[kChunk][4];
    __shared__ uint32_t rq[kChunk * 4]; // rescans: token | wave << 8 | which << 12
    __shared__ int rqn;
    // Blocks are dealt round-robin over the 8 XCDs, each with its own L2:
    // XCD x takes the blocks whose index is x mod 8.  With a multiple of 8
    // kv-heads, XCD x serves heads x, x + 8, ... only, so each head's
    // codebooks are fetched into one L2, not all eight.  The quarter blocks
    // of one (chunk range, kv-head) are adjacent in their XCD's order, so
    // they run at about the same time and the chunk's keys come from HBM
    // once, then from that L2.  (Otherwise heads take the XCDs in turn.)
    constexpr int NQ = G / 4;
    const int bid = blockIdx.x, x = bid & 7, j = bid >> 3;
    int h, bx, gq;
    if (Hkv % 8 == 0) {
        const int hpx = Hkv / 8; // heads per XCD
        const int per_head = gx * NQ;
        if (j >= hpx * per_head)
            return;
        h = x + 8 * (j / per_head);
        bx = (j % per_head) / NQ;
        gq = j % NQ;
    } else {
        gq = j % NQ;
        const int item = (j / NQ) * 8 + x;
        if (item >= gx * Hkv)
            return;
        h = item / gx;
        bx = item % gx;
    }
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = 4 * gq + w;
    const int col = lane & 15, q = lane >> 4;
    const float *c8g = cb8 + ((size_t)h * G + g) * kCodes8 * 8;
    const float *c4g = cb4 + ((size_t)h * G + g) * kCodes4 * 8;
    const uint16_t *xk16 = reinterpret_cast<const uint16_t *>(xk);

    // The four groups' codebooks are contiguous: stage them with 16-byte loads.
    {
        const uint4 *src8 = reinterpret_cast<const uint4 *>(cb8 + ((size_t)h * G + 4 * gq) * kCodes8 * 8);
        const uint4 *src4 = reinterpret_cast<const uint4 *>(cb4 + ((size_t)h * G + 4 * gq) * kCodes4 * 8);
        uint4 *dst = reinterpret_cast<uint4 *>(lds);
        constexpr int N8 = 4 * kCodes8 * 2, N4 = 4 * kCodes4 * 2;
        constexpr int PER = (N8 + N4 + 255) / 256; // loads per thread, all issued first
        uint4 v[PER];
#pragma unroll
        for (int k = 0; k < PER; k++) {
            const int i = tid + 256 * k;
            v[k] = i < N8 ? src8[i] : i < N8 + N4 ? src4[i - N8] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < PER; k++)
            if (tid + 256 * k < N8 + N4)
                dst[tid + 256 * k] = v[k];
    }
    __syncthreads();
    // A operands (rows = codewords): lane holds coordinates q and 4 + q of
    // codeword 16 t + col of tile t (tile 16 = the 4-bit codebook).  The
    // norms |c|^2 go to LDS (after the codebooks, past the keys' rows), where
    // lane (col, q) reads those of codewords 16 t + 4 q .. + 3.
    float a0[17], a1[17], nrm[17];
    {
        const float *s8w = reinterpret_cast<const float *>(lds) + w * kCodes8 * 8;
        const float *s4w = reinterpret_cast<const float *>(lds) + 4 * kCodes8 * 8 + w * kCodes4 * 8;
#pragma unroll
        for (int t = 0; t < 17; t++) {
            const float *cw = t < 16 ? s8w + (16 * t + col) * 8 : s4w + col * 8;
            a0[t] = cw[q];
            a1[t] = cw[4 + q];
        }
    }
    bool fin = true;
#pragma unroll
    for (int t = 0; t < 17; t++) {
        fin &= fabsf(a0[t]) <= kCodeMax;
        fin &= fabsf(a1[t]) <= kCodeMax;
        const float p = column_sum(fmaf(a1[t], a1[t], a0[t] * a0[t]));
        nrm[t] = p;
    }
    const bool filter = __ballot(!fin) == 0; // (wave-uniform)
    __syncthreads(); // (the codebooks have been read)
    float *norms = reinterpret_cast<float *>(lds + kChunk * RW) + w * 17 * 16;
    if (q == 0) {
#pragma unroll
        for (int t = 0; t < 17; t++)
            norms[16 * t + col] = nrm[t];
    }
    __syncthreads(); // (the keys reuse the rest of the codebooks' LDS)

    for (int64_t chunk = bx; chunk < n_chunks; chunk += gx) {
        const int64_t n0 = chunk * kChunk;
        if (tid == 0)
            rqn = 0;
        // stage the chunk's keys (zeros past the end)
        for (int i = tid; i < kChunk * (D / 8); i += 256) {
            const int tk = i / (D / 8), c = i % (D / 8);
            uint4 kw = make_uint4(0, 0, 0, 0);
            if (n0 + tk < n_tokens)
                kw = *reinterpret_cast<const uint4 *>(keys + ((size_t)(n0 + tk) * Hkv + h) * D + 8 * c);
            uint32_t *dst = xk + tk * RW + 4 * c;
            dst[0] = kw.x;
            dst[1] = kw.y;
            dst[2] = kw.z;
            dst[3] = kw.w;
        }
        __syncthreads();
        // Norms for the filter, wave w taking tokens 16 w + col: the four
        // lanes of a column each sum a quarter of the squares (exact in
        // double), then the quarters are added.  This order differs from the
        // defining one by at most 2^-45 r, which the filter's bound absorbs.
        {
            const int tk = 16 * w + col;
            const uint32_t *row = xk + tk * RW + (D / 8) * q;
            double part = 0.0;
#pragma unroll
            for (int c = 0; c < D / 8; c++) {
                const uint32_t kw = row[c];
                const double lo = (double)f16_bits_to_f32((uint16_t)(kw & 0xffff));
                const double hi = (double)f16_bits_to_f32((uint16_t)(kw >> 16));
                part = __builtin_fma(lo, lo, part); // (exact squares)
                part = __builtin_fma(hi, hi, part);
            }
            const double r = sqrt(column_sum(part));
            if (q == 0)
                xri[tk] = r > 0.0 ? 1.0 / r : 0.0;
        }
        __syncthreads();
        // The defining norms (a serial sum per token) for the radius and the
        // rescans: the last wave, before its tiles; the others go on.
        if (w == 3) {
            const double r = exact_norm<D>(xk + lane * RW);
            xr[lane] = r;
            if (gq == 0 && n0 + lane < n_tokens)
                radius[(size_t)(n0 + lane) * Hkv + h] = f64_to_f16_sat(r);
        }

        for (int tt = 0; tt < kChunk / 16; tt++) {
            const int tk = 16 * tt + col; // this lane's token (B column)
            const uint16_t *kg = xk16 + tk * (2 * RW) + 8 * g;
            int code8 = 0, code4 = 0;
            uint32_t redo = 0xffffffffu; // tokens to rescan: 8-bit | 4-bit << 16 (all
                                         // for a codebook outside the filter's range)
            if (filter) {
                const double ri = xri[tk];
                const float ua = (float)((double)f16_bits_to_f32(kg[q]) * ri);
                const float ub = (float)((double)f16_bits_to_f32(kg[4 + q]) * ri);
                const float b0 = -2.f * ua, b1 = -2.f * ub;
                const float n32 = column_sum(fmaf(ub, ub, ua * ua));
                float ninf;
                asm("; -inf" : "=v"(ninf) : "0"(-INFINITY));
                Best s8b, s4b;
                best_init(s8b);
                best_init(s4b);
#pragma unroll
                for (int t = 0; t < 17; t++) {
                    const float4 cn = *reinterpret_cast<const float4 *>(norms + 16 * t + 4 * q);
                    f32x4 acc = {cn.x, cn.y, cn.z, cn.w};
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[t], b0, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[t], b1, acc, 0, 0, 0);
                    // element v: codeword (16 t +) 4 q + v of token tk; its
                    // slot in the packed score is 4 t + v
#pragma unroll
                    for (int v = 0; v < 4; v++) {
                        if (t < 16)
                            best_add(s8b, acc[v], 4 * t + v, ninf);
                        else
                            best_add(s4b, acc[v], v, ninf);
                    }
                    if (t % 4 == 3)
                        __builtin_amdgcn_sched_barrier(0);
                }
                const int j8 = (int)(__float_as_uint(s8b.k1) & 63u), j4 = (int)(__float_as_uint(s4b.k1) & 63u);
                const Column c8 = best_column(s8b, 16 * (j8 >> 2) + 4 * q + (j8 & 3));
                const Column c4 = best_column(s4b, 4 * q + j4);
                const bool ok8 = c8.v2 - c8.v1 > fmaf(kFilterRel, 4.f * n32 + c8.v1 + c8.v2, kFilterAbs);
                const bool ok4 = c4.v2 - c4.v1 > fmaf(kFilterRel, 4.f * n32 + c4.v1 + c4.v2, kFilterAbs);
                code8 = c8.i1;
                code4 = c4.i1;
                // near ties: rescanned in double after the chunk's tiles
                redo = (uint32_t)(__ballot(!ok8) & 0xffffull) | ((uint32_t)(__ballot(!ok4) & 0xffffull) << 16);
            }
            if (q == 0) {
                s8[tk][w] = (uint8_t)code8;
                s4[tk][w] = (uint8_t)code4;
            }
            // queue the near ties for the whole block
            uint32_t m = (redo | (redo >> 16)) & 0xffffu;
            while (m) {
                const int j = __builtin_ctz(m);
                m &= m - 1;
                const uint32_t which = ((redo >> j) & 1u) | (((redo >> (16 + j)) & 1u) << 1);
                if (lane == 0)
                    rq[atomicAdd(&rqn, 1)] = (uint32_t)(16 * tt + j) | ((uint32_t)w << 8) | (which << 12);
            }
        }
        __syncthreads(); // (the queue and the defining norms are in)
        // the rescans, dealt round-robin to the waves, one token-group at a
        // time by a whole wave (out of line: the filter loop keeps its
        // registers)
        for (int i = w; i < rqn; i += 4) {
            const uint32_t ent = rq[i];
            const int tk = (int)(ent & 0xff), ew = (int)((ent >> 8) & 3), which = (int)(ent >> 12);
            const int gg = 4 * gq + ew;
            const uint32_t *kw = xk + tk * RW + 4 * gg;
            const uint32_t e = rescan(make_uint4(kw[0], kw[1], kw[2], kw[3]), xr[tk],
                                      cb8 + ((size_t)h * G + gg) * kCodes8 * 8,
                                      cb4 + ((size_t)h * G + gg) * kCodes4 * 8, lane, which);
            if (lane == 0) {
                if (which & 1)
                    s8[tk][ew] = (uint8_t)(e & 0xff);
                if (which & 2)
                    s4[tk][ew] = (uint8_t)(e >> 8);
            }
        }
        __syncthreads();
        {
            const int tk = tid >> 2, k = tid & 3;
            if (n0 + tk < n_tokens) {
                const size_t e = (size_t)(n0 + tk) * Hkv + h;
                codes8[e * G + 4 * gq + k] = s8[tk][k];
                if (k < 2)
                    codes4[e * (G / 2) + 2 * gq + k] = (uint8_t)(s4[tk][2 * k] | (s4[tk][2 * k + 1] << 4));
            }
        }
        __syncthreads();
    }
}

} // namespace

hipError_t launch_encode(int D, int Hkv, int64_t n_tokens, const uint16_t *keys, const float *cb8,
                         const float *cb4, uint16_t *radius, uint8_t *codes8, uint8_t *codes4,
                         hipStream_t st)
{
    if (n_tokens == 0)
        return hipSuccess;
    const int64_t n_chunks = (n_tokens + kChunk - 1) / kChunk;
    // about four blocks per compute unit; each block walks its chunks
    const int64_t by = (int64_t)Hkv * (D / 32);
    const int64_t want = (1024 + by - 1) / by;
    const int gx = (int)(n_chunks < want ? n_chunks : want);
    // (chunk range, kv-head) items times quarters, in groups of 8 items
    const int64_t nq = D / 32;
    const int64_t items = (int64_t)gx * Hkv;
    const dim3 grid((unsigned)(Hkv % 8 == 0 ? items * nq : (items + 7) / 8 * 8 * nq));
    if (D == 128)
        hipLaunchKernelGGL(encode_kernel<128>, grid, dim3(256), 0, st, Hkv, gx, n_tokens, n_chunks, keys,
                           cb8, cb4, radius, codes8, codes4);
    else if (D == 64)
        hipLaunchKernelGGL(encode_kernel<64>, grid, dim3(256), 0, st, Hkv, gx, n_tokens, n_chunks, keys,
                           cb8, cb4, radius, codes8, codes4);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

} // namespace ada
