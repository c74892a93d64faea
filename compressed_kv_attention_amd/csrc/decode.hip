// ADA decode step for gfx950: code-table logits, online softmax, split-K.
//
// Method: SPHERICAL KV (arXiv 2605.18856), gist.science technical summary,
// section 2.1 "Compressed-Domain Similarity" -- logits come straight from the
// stored radius and angle codes, no dense key is rebuilt in device memory --
// and section 2.2 "Tier-Homogeneous Pages" -- pages of one tier are streamed
// in a single pass guided by their metadata.  With per-group codebooks the
// logit |q| r~ f_b(codes) is r~ * sum_g (q_g . C_g[code_g]) (times the softmax
// scale); the per-group dot products are tabulated once per query head
// (the "LUT") and each coded key costs G table reads.
//
// Work decomposition.  A step is two kernels: the page stream and, with
// more than one split per row, the split merge.  In the page stream one
// workgroup (12 wave64s, or 8 for groups of more than 4 heads at D = 128;
// one workgroup per CU at D = 128) serves one (sequence,
// kv-head) row and one of `nsplit` interleaved page subsets of it, for all
// NH query heads of the GQA group, so every page is read from HBM once.  It
// tabulates the row's LUT into LDS while its first pages are in flight.
// Wave w of split s takes pages s + (w + W i) * nsplit (W waves), one page (16 slots)
// at a time, with the next page's loads in flight while the current one is
// computed.
//
// Per page the wave forms a 16 x 16 tile of logits, rows = query heads
// (NH used, the rest zero), columns = slots, held the way a 16x16x16 MFMA
// takes its A operand: lane h + 16 r holds slots 4r .. 4r+3 of head h.
//   - fp16 / bf16 key pages: one MFMA chain, keys (stored in the B^T order,
//     so each lane's 8-byte half chunk is its operand) times the query
//     block held in registers; the result lands in the tile layout.
//   - coded pages: lane j + 16 r sums the LUT entries of slot 4r + j/4 over
//     a quarter of the groups, a quad reduction completes each slot, and
//     DPP row rotations (three per quad of heads) move head h's values of
//     the row's four slots into lane h + 16 r; the radii scale them there.
// The softmax runs on that tile (running maxima per head, rescaled only
// when a page's maximum exceeds the running one by 2^8, so every weight is
// at most 2^8), and the weights are split into bf16 hi + lo parts (about
// 16 significant bits) for two MFMAs per 16-dim value block.  Value
// sections are stored as the B operand (lane n + 16 r: slots 4r .. 4r+3 of
// dim n); int8 values become bf16 exactly, and their per-slot scales are
// folded into the weights.  The output accumulators are the MFMA C tiles
// (rows = heads: element h % 4 of lane 16 (h / 4) + n holds dim n of head h).
//
// At the end the waves are merged through LDS and the split's partial
// (m, l, acc) is written; the merge kernel combines a row's splits into the
// outputs (with one split the stream writes them directly).
#include "ada_internal.h"
#include "wave_ops.h"

#include <atomic>

#include <mutex>
#include <type_traits>

// Split partials of ada_decode_noalloc: a library-owned device array, one
// copy per GPU the library runs on, kept until the process ends.  Host code
// never passes this name to a kernel (on the host it is only a stand-in):
// noalloc_scratch() gives each device's address.
static __device__ __align__(256) unsigned char scratch[ada::kNoAllocScratchBytes];

namespace ada {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescale = 8.0f; // log2 of the largest weight kept between rescales
// Waves per page-stream workgroup: 12 (three per SIMD, up to 168 VGPRs
// each).  Groups of more than four heads at D = 128 need more registers
// than that in the page loop and run 8 waves of up to 256.
template <int D, int NH>
struct Waves {
    static constexpr int W = (D == 128 && NH > 4) ? 8 : 12;
    static constexpr int THREADS = 64 * W;
};
constexpr int kMaxSplitsDev = 1024; // the ABI's split limit

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef const u32x4 __attribute__((address_space(1))) *gchunk;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float f16_to_f32(uint32_t h)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Two floats -> packed bf16 pair (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b)
{
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// A lane permutation within rows (quad_perm, row_ror, row mirrors: every
// source lane exists, so bound_ctrl changes nothing; with it set the
// compiler folds the move into the consuming add).
template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}

// Max / sum over the four lanes h, h+16, h+32, h+48 (every lane receives it).
__device__ __forceinline__ float rows_max(float x)
{
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// max(a, b) for non-NaN operands in one instruction (the median of a, b
// and +inf), with no canonicalising moves
// (+inf is passed through an empty asm so that the median is not folded
// back into a maxnum, which would canonicalise both operands first)
__device__ __forceinline__ float max_nn(float a, float b)
{
    float inf;
    asm("; +inf" : "=v"(inf) : "0"(INFINITY));
    return __builtin_amdgcn_fmed3f(a, b, inf);
}
// rows_max for non-NaN values
__device__ __forceinline__ float rows_max_nn(float x)
{
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = max_nn(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return max_nn(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float x)
{
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// s_waitcnt immediate that waits until at most n vector-memory operations
// are outstanding (expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Heads of a GQA group: NH = 4 NQF + REM.  The LUT holds NQF regions of
// [G][kLutCodes] float4 entries (heads 4 j .. 4 j + 3), then one region of
// [G][kLutCodes][REM] floats for the remaining heads, so every lookup is
// one aligned LDS read per region.
template <int NH>
struct Heads {
    static_assert(NH >= 1 && NH <= 8 && NH % 4 != 3, "GQA group of 1, 2, 4, 5, 6 or 8 query heads");
    static constexpr int NQF = NH / 4, REM = NH % 4;
    static constexpr int NQ = (NH + 3) / 4; // head quads of the output tile
};

// sum[h] += LUT entry (idx, h), or sum[h] = the entry when FIRST
template <int NH, int G, bool FIRST>
__device__ __forceinline__ void lut_add(const float *lut, int idx, float (&sum)[NH])
{
    constexpr int NQF = Heads<NH>::NQF, REM = Heads<NH>::REM;
    constexpr int REGION = G * kLutCodes * 4; // floats of one head-quad region
    auto put = [&](int h, float v) { sum[h] = FIRST ? v : sum[h] + v; };
#pragma unroll
    for (int j = 0; j < NQF; j++) {
        const float4 v = *reinterpret_cast<const float4 *>(lut + j * REGION + idx * 4);
        put(4 * j, v.x); put(4 * j + 1, v.y); put(4 * j + 2, v.z); put(4 * j + 3, v.w);
    }
    if constexpr (REM == 2) {
        const float2 v = *reinterpret_cast<const float2 *>(lut + NQF * REGION + idx * 2);
        put(4 * NQF, v.x); put(4 * NQF + 1, v.y);
    } else if constexpr (REM == 1) {
        put(4 * NQF, lut[NQF * REGION + idx]);
    }
}

template <int NH, int G>
__device__ __forceinline__ void lut_store(float *lut, int idx, const float (&o)[NH])
{
    constexpr int NQF = Heads<NH>::NQF, REM = Heads<NH>::REM;
    constexpr int REGION = G * kLutCodes * 4;
#pragma unroll
    for (int j = 0; j < NQF; j++)
        *reinterpret_cast<float4 *>(lut + j * REGION + idx * 4) =
            make_float4(o[4 * j], o[4 * j + 1], o[4 * j + 2], o[4 * j + 3]);
    if constexpr (REM == 2)
        *reinterpret_cast<float2 *>(lut + NQF * REGION + idx * 2) = make_float2(o[4 * NQF], o[4 * NQF + 1]);
    else if constexpr (REM == 1)
        lut[NQF * REGION + idx] = o[4 * NQF];
}

// The bytes from offset o (0..15) of a 16-byte chunk up to the end of its
// 8-byte half, picked with masks and a 64-bit shift so the chunk stays in
// registers.  A lane's code bytes never straddle an 8-byte boundary.
__device__ __forceinline__ uint32_t bits_at(const u32x4 &v, int o)
{
    // (32-bit masks, so each half is one bitfield insert)
    const uint32_t m = 0u - (((uint32_t)o >> 3) & 1u);
    const uint32_t lo = (v.z & m) | (v.x & ~m), hi = (v.w & m) | (v.y & ~m);
    return (uint32_t)((((uint64_t)hi << 32) | lo) >> (8 * (o & 7)));
}

// Per-lane constants of the page walk.
struct Lane {
    int lane, hl, r;      // lane = hl + 16 r
    int gq, g0;           // coded logits: group quarter, first group
    uint32_t cblk1, cblk2; // code block of the lane's slot, tiers 1 and 2
    int co1, co2;         // byte of the lane's codes inside that block
    uint32_t rblk1, rblk2, sblk2; // radius blocks (tiers 1, 2), scale block (tier 2)
    int nv_off;           // 4 r, or a large value for lanes of unused heads
};

template <int D, int NH>
__device__ __forceinline__ Lane make_lane(int lane)
{
    constexpr int G = D / 8, GPL = G / 4;
    Lane L;
    L.lane = lane;
    L.hl = lane & 15;
    L.r = lane >> 4;
    const int t = 4 * L.r + (L.hl >> 2); // slot whose codes this lane reads
    L.gq = L.hl & 3;
    L.g0 = L.gq * GPL;
    const int b1 = t * G + L.g0, b2 = t * (G / 2) + L.g0 / 2;
    L.cblk1 = codes_off(D, 1) + (b1 & ~15);
    L.co1 = b1 & 15;
    L.cblk2 = codes_off(D, 2) + (b2 & ~15);
    L.co2 = b2 & 15;
    L.rblk1 = radius_off(D, 1) + 16 * (L.r >> 1);
    L.rblk2 = radius_off(D, 2) + 16 * (L.r >> 1);
    L.sblk2 = vscale_off(D) + 16 * (L.r >> 1);
    L.nv_off = L.hl < NH ? 4 * L.r : 64;
    return L;
}

// Raw bytes of one page as this lane sees them: NL 16-byte loads.  With
// NV = D / 32 (the chunks of a bf16 value section):
//   tiers 0/3: c[0 .. NV) value chunks, c[NV .. 2 NV) key chunks
//   tier 1:    c[0 .. NV) value chunks; c[NV] the lane's code block;
//              c[NV+1] the 16-byte block of radii holding slots 4r .. 4r+3
//   tier 2:    c[0 .. NV/2) int8 value chunks; c[NV/2] the value-scale
//              block (as the radii); c[NV], c[NV+1] as in tier 1
// Unused loads repeat chunk 0 (same cache lines, no extra HBM traffic).
// Every tier issues the same loads with no branch, so the next page's loads
// stay in flight while the current page is computed.  The value chunks sit
// in the same registers for every tier, so one MFMA sequence serves all.
template <int D>
struct PageRegs {
    static constexpr int NV = D / 32;
    static constexpr int NL = 2 * NV > NV + 2 ? 2 * NV : NV + 2;
    u32x4 c[NL];
    int tier, nvalid;
};

template <int D, bool DENSE>
__device__ __forceinline__ void fetch_page(PageRegs<D> &pr, const uint8_t *page, int tier, int nvalid,
                                           const Lane &L)
{
    constexpr int NL = PageRegs<D>::NL, NV = PageRegs<D>::NV;
    pr.tier = tier;
    pr.nvalid = nvalid;
    const uint32_t lo = L.lane * 16;
    uint32_t o[NL];
#pragma unroll
    for (int c = 0; c < NL; c++) {
        // tiers 0/3: the value section starts at 32 D, the key section at 0
        const uint32_t dense = c < NV ? 32 * D + lo + c * 1024 : c < 2 * NV ? lo + (c - NV) * 1024 : lo;
        uint32_t t1 = c < NV ? lo + c * 1024 : lo;
        uint32_t t2 = c < NV / 2 ? lo + c * 1024 : lo;
        if (c == NV) {
            t1 = L.cblk1;
            t2 = L.cblk2;
        }
        if (c == NV + 1) {
            t1 = L.rblk1;
            t2 = L.rblk2;
        }
        if (c == NV / 2)
            t2 = L.sblk2;
        o[c] = (DENSE || tier == 0) ? dense : tier == 1 ? t1 : t2;
    }
    // (non-temporal: every page byte is read once per step, so its lines
    // are not worth keeping in the caches)
#pragma unroll
    for (int c = 0; c < NL; c++)
        pr.c[c] = __builtin_nontemporal_load((gchunk)(page + o[c]));
}

// The four fp16 values of slots 4r .. 4r+3 from a 16-byte block holding
// slots 8 (r/2) .. 8 (r/2) + 7.
__device__ __forceinline__ void quad_f16(const u32x4 &blk, int r, float (&v)[4])
{
    const uint32_t a = (r & 1) ? blk.z : blk.x;
    const uint32_t b = (r & 1) ? blk.w : blk.y;
    v[0] = f16_to_f32(a & 0xffffu);
    v[1] = f16_to_f32(a >> 16);
    v[2] = f16_to_f32(b & 0xffffu);
    v[3] = f16_to_f32(b >> 16);
}

template <int D, int NH>
struct WaveState {
    f32x4 acc[D / 16]; // C tiles: lane n (< 16) element h = output dim 16 b + n of head h
    float m[NH];       // running max per head, log2 units (wave-uniform)
    float mlane;       // running max of this lane's head (0 for unused heads)
    float l;           // softmax denominator: this lane's head, its slots
};

// Query operand of the key MFMA: lane h + 16 q holds dims 16 b + 4 q .. +3
// of head h for each 16-dim block b (zero for h >= NH).
template <int D, bool DENSE>
struct QOperand {
    typedef typename std::conditional<DENSE, s16x4, f16x4>::type T;
    T blk[D / 16];
};

// Logits of a key page (fp16 keys, or bf16 keys in the dense cache) in the
// tile layout, in log2 units.
template <int D, bool DENSE>
__device__ __forceinline__ void key_logits(const PageRegs<D> &cur, const QOperand<D, DENSE> &qo,
                                           float lsc, float (&x)[4])
{
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
    for (int b = 0; b < D / 16; b++) {
        const u32x4 &ch = cur.c[PageRegs<D>::NV + b / 2];
        const u32x2 k2 = (b & 1) ? u32x2{ch.z, ch.w} : u32x2{ch.x, ch.y};
        f32x4 &s = (b & 1) ? s1 : s0;
        if constexpr (DENSE)
            s = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, k2), qo.blk[b], s, 0, 0, 0);
        else
            s = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, k2), qo.blk[b], s, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < 4; e++)
        x[e] = (s0[e] + s1[e]) * lsc;
}

// Logits of a coded page in the tile layout, in log2 units.
template <int D, int NH>
__device__ __forceinline__ void coded_logits(const PageRegs<D> &cur, const float *lut, const Lane &L,
                                             float sig2, float (&x)[4])
{
    constexpr int GPL = D / 32; // groups per lane
    constexpr int NV = PageRegs<D>::NV;
    const bool t8 = cur.tier == 1;
    const uint32_t bits = bits_at(cur.c[NV], t8 ? L.co1 : L.co2);
    // code field k: 8 bits (tier 1) or 4 bits (tier 2, LUT entries from 256)
    const uint32_t width = t8 ? 8u : 4u;
    const int base = t8 ? 0 : kCodes8;
    float s[NH];
#pragma unroll
    for (int k = 0; k < GPL; k++) {
        const int code = base + (int)__builtin_amdgcn_ubfe(bits, k * width, width);
        if (k == 0)
            lut_add<NH, D / 8, true>(lut, (L.g0 + k) * kLutCodes + code, s);
        else
            lut_add<NH, D / 8, false>(lut, (L.g0 + k) * kLutCodes + code, s);
    }
    // complete each slot's sum over its four lanes (a quad)
#pragma unroll
    for (int h = 0; h < NH; h++) {
        s[h] += dpp<0xb1>(s[h]); // quad_perm [1,0,3,2]
        s[h] += dpp<0x4e>(s[h]); // quad_perm [2,3,0,1]
    }
    // For head quad q, lane j of a row offers head 4 q + j % 4 of its slot;
    // lane 4 q + i of the row then collects head 4 q + i of slots 4 r + e
    // from lane 4 e + i, a rotation of the row by 4 (q - e) lanes.
    constexpr int NQ = Heads<NH>::NQ;
    float v[4];
#pragma unroll
    for (int q = 0; q < NQ; q++) {
        // (the loop is unrolled, so the head bounds fold away)
        float sel = s[4 * q];
        if (4 * q + 1 < NH)
            sel = (L.gq & 1) ? s[min(4 * q + 1, NH - 1)] : sel;
        if (4 * q + 2 < NH)
            sel = L.gq == 2 ? s[min(4 * q + 2, NH - 1)] : sel;
        if (4 * q + 3 < NH)
            sel = L.gq == 3 ? s[min(4 * q + 3, NH - 1)] : sel;
        // row_ror:n moves lane i - n to lane i
        const float r0 = sel, r4 = dpp<0x124>(sel), r8 = dpp<0x128>(sel), r12 = dpp<0x12c>(sel);
        const float vq[4] = {q == 0 ? r0 : r4, q == 0 ? r12 : r0, q == 0 ? r8 : r12, q == 0 ? r4 : r8};
#pragma unroll
        for (int e = 0; e < 4; e++)
            v[e] = (q == 0 || (L.hl >> 2) == q) ? vq[e] : v[e];
    }
    float rad[4];
    quad_f16(cur.c[NV + 1], L.r, rad);
#pragma unroll
    for (int e = 0; e < 4; e++)
        x[e] = v[e] * (rad[e] * sig2);
}

// Logits, online-softmax update and PV product of one page (page index p in
// its row) for the wave's NH query heads.
template <int D, int NH, bool DENSE>
__device__ __forceinline__ void process_page(PageRegs<D> &cur, int p, WaveState<D, NH> &st,
                                             const float *lut, const QOperand<D, DENSE> &qo, float lsc,
                                             float sig2, float *lgout, int maxp, const Lane &L)
{
    // This page's loads were issued before the next page's NL loads: wait
    // until at most those NL are outstanding.  Every register of this page
    // is then complete on every path, including chunks a tier never reads,
    // so the wait-count pass needs no full drain where they are reused.
    constexpr int NL = PageRegs<D>::NL;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(NL));
    const int tier = cur.tier;
    float x[4];
    if (DENSE || tier == 0)
        key_logits<D, DENSE>(cur, qo, lsc, x);
    else
        coded_logits<D, NH>(cur, lut, L, sig2, x);

    // mask slots past the page's valid count, and unused heads
    const int nv = cur.nvalid - L.nv_off;
#pragma unroll
    for (int e = 0; e < 4; e++)
        x[e] = e < nv ? x[e] : -INFINITY;

    if (lgout != nullptr && L.hl < NH) {
        float *lo = lgout + (size_t)L.hl * maxp * kSlots + (size_t)p * kSlots + 4 * L.r;
#pragma unroll
        for (int e = 0; e < 4; e++)
            if (e < nv)
                lo[e] = x[e] * kLn2;
    }

    // online softmax: per-head page maxima; one wave-wide test whether any
    // of them runs ahead of its running maximum (lanes of unused heads have
    // pm = -inf and never do), the per-head rescale only then
    // (logits are finite or -inf)
    const float pm = rows_max_nn(max_nn(max_nn(x[0], x[1]), max_nn(x[2], x[3])));
    if (__builtin_amdgcn_ballot_w64(pm > st.mlane + kRescale) != 0) {
        // head h's outputs are element h % 4 of the C tiles in lanes
        // 16 (h / 4) .. 16 (h / 4) + 15
        constexpr int NQ = Heads<NH>::NQ;
        float fe[4] = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
        for (int h = 0; h < NH; h++) {
            const float pmh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pm), h));
            if (pmh > st.m[h] + kRescale) {
                const float f = __builtin_amdgcn_exp2f(st.m[h] - pmh);
                st.m[h] = pmh;
                if constexpr (NQ == 1) {
#pragma unroll
                    for (int b = 0; b < D / 16; b++)
                        st.acc[b][h] *= f;
                } else {
                    fe[h % 4] = L.r == h / 4 ? f : fe[h % 4];
                }
                const bool mine = L.hl == h;
                st.l = mine ? st.l * f : st.l;
                st.mlane = mine ? pmh : st.mlane;
            }
        }
        if constexpr (NQ > 1) {
#pragma unroll
            for (int b = 0; b < D / 16; b++)
#pragma unroll
                for (int e = 0; e < 4; e++)
                    st.acc[b][e] *= fe[e];
        }
    }
    float w[4];
#pragma unroll
    for (int e = 0; e < 4; e++)
        w[e] = __builtin_amdgcn_exp2f(x[e] - st.mlane);
    st.l += (w[0] + w[1]) + (w[2] + w[3]);

    constexpr int NV = PageRegs<D>::NV;
    const bool int8v = !DENSE && tier == 2;
    if (int8v) {
        float sc[4];
        quad_f16(cur.c[NV / 2], L.r, sc);
#pragma unroll
        for (int e = 0; e < 4; e++)
            w[e] *= sc[e];
        // int8 values -> bf16 (exact), into the registers the bf16 tiers
        // use: block b is dword b % 4 of int8 chunk b / 4, and becomes
        // half b % 2 of chunk b / 2
        u32x4 cv[NV];
#pragma unroll
        for (int b = 0; b < D / 16; b++) {
            const u32x4 &ch = cur.c[b / 4];
            const uint32_t q = (b % 4 == 0) ? ch.x : (b % 4 == 1) ? ch.y : (b % 4 == 2) ? ch.z : ch.w;
            const uint32_t v01 = pack_bf16((float)(signed char)(q & 255u), (float)(signed char)((q >> 8) & 255u));
            const uint32_t v23 = pack_bf16((float)(signed char)((q >> 16) & 255u), (float)(signed char)(q >> 24));
            if (b & 1) {
                cv[b / 2].z = v01;
                cv[b / 2].w = v23;
            } else {
                cv[b / 2].x = v01;
                cv[b / 2].y = v23;
            }
        }
#pragma unroll
        for (int c = 0; c < NV; c++)
            cur.c[c] = cv[c];
    }
    // weights as bf16 hi + lo (A operands)
    const uint32_t h01 = pack_bf16(w[0], w[1]), h23 = pack_bf16(w[2], w[3]);
    const uint32_t l01 = pack_bf16(w[0] - bf16_lo(h01), w[1] - bf16_hi(h01));
    const uint32_t l23 = pack_bf16(w[2] - bf16_lo(h23), w[3] - bf16_hi(h23));
    const s16x4 ahi = __builtin_bit_cast(s16x4, u32x2{h01, h23});
    const s16x4 alo = __builtin_bit_cast(s16x4, u32x2{l01, l23});
#pragma unroll
    for (int b = 0; b < D / 16; b++) {
        const u32x4 &ch = cur.c[b / 2];
        const s16x4 bv = __builtin_bit_cast(s16x4, (b & 1) ? u32x2{ch.z, ch.w} : u32x2{ch.x, ch.y});
        st.acc[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ahi, bv, st.acc[b], 0, 0, 0);
    }
#pragma unroll
    for (int b = 0; b < D / 16; b++) {
        const u32x4 &ch = cur.c[b / 2];
        const s16x4 bv = __builtin_bit_cast(s16x4, (b & 1) ? u32x2{ch.z, ch.w} : u32x2{ch.x, ch.y});
        st.acc[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(alo, bv, st.acc[b], 0, 0, 0);
    }
}

// Issues the loads of the page whose table entry is e = (offset in 128-byte
// units, metadata byte); e is the same in every lane.
template <int D, bool DENSE>
__device__ __forceinline__ void fetch_entry(PageRegs<D> &pr, uint2 e, const uint8_t *arena, const Lane &L)
{
    const uint32_t off = __builtin_amdgcn_readfirstlane(e.x);
    const uint32_t meta = __builtin_amdgcn_readfirstlane(e.y);
    fetch_page<D, DENSE>(pr, arena + (size_t)off * kUnit, meta & 3, ((meta >> 2) & 15) + 1, L);
}

// ---- phase timestamps (tracing builds only) ------------------------------------
// With ADA_PHASE_TRACE defined, lane 0 of each wave writes the 100 MHz
// real-time counter at the phase boundaries of the page stream to
// a.trace[(block * waves + wave) * 8 + k]: k = 0 entry, 1 prologue loads in,
// 2 table built, 3 past the table barrier, 4 page loop done, 5 end (every
// load and store complete), then 6 HW_ID and 7 XCC_ID.  Other builds compile
// none of it.
#ifdef ADA_PHASE_TRACE
#define ADA_PHASE(k)                                                                                   \
    do {                                                                                               \
        if (a.trace != nullptr && lane == 0)                                                           \
            a.trace[((size_t)blockIdx.x * kWaves + wave) * 8 + (k)] = __builtin_amdgcn_s_memrealtime(); \
    } while (0)
#else
#define ADA_PHASE(k) ((void)0)
#endif

// ---- page stream ------------------------------------------------------------
// SYM: the symmetric variant; the row's LUT was tabulated by sym_lut_kernel
// and is copied into LDS instead of being built from the query.
template <int D, int NH, bool DENSE, bool SYM>
__global__ __launch_bounds__((Waves<D, NH>::THREADS)) void decode_main(DecodeArgs a)
{
    constexpr int kWaves = Waves<D, NH>::W, kThreads = Waves<D, NH>::THREADS;
    constexpr int G = D / 8; // code groups
    constexpr int LUT_FLOATS = DENSE ? 0 : G * kLutCodes * NH;

    extern __shared__ float smem[];
    float *lut = smem;
    uint2 *tbl = reinterpret_cast<uint2 *>(smem + LUT_FLOATS); // [n_wg] page-table entries

    // Blocks are dealt round-robin over the 8 XCDs, each with its own L2.
    // All splits of a row run on one XCD (one L2 holds the row's codebooks
    // and table).  With a multiple of 8 rows, XCD x takes rows x, x + 8,
    // x + 16, ...: with 8 kv-heads that is one head of every sequence, so
    // ragged sequence lengths load the XCDs evenly.  Otherwise each XCD
    // takes a contiguous range of rows.
    const int nblk = gridDim.x, rows = a.S * a.Hkv;
    int row, split;
    if (rows % 8 == 0) {
        const int i = blockIdx.x / 8;
        row = 8 * (i / a.nsplit) + blockIdx.x % 8;
        split = i % a.nsplit;
    } else {
        int logical = blockIdx.x;
        if (nblk % 8 == 0)
            logical = (blockIdx.x % 8) * (nblk / 8) + blockIdx.x / 8;
        row = logical / a.nsplit;
        split = logical % a.nsplit;
    }
    const int s = row / a.Hkv, hkv = row % a.Hkv;
    // the wave index is wave-uniform; say so, so the page loop is scalar
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const Lane L = make_lane<D, NH>(lane);
    ADA_PHASE(0);

    // Prologue loads, all issued before any is waited for.  First those
    // that need only the row: the codewords and query slices of the LUT and
    // the query operand (ahead of the row's page count, a scalar load whose
    // wait would otherwise hold them back by one memory latency).
    // Code tables: thread t serves group g = t / TPG and codes t % TPG +
    // TPG k; its codewords and the group's query slices load with the rest.
    constexpr int TPG = kThreads / G;
    constexpr int NC = (kLutCodes + TPG - 1) / TPG;
    const int g = tid / TPG, c0 = tid % TPG;
    const uint16_t *qrow = a.q + ((size_t)s * a.Hq + (size_t)hkv * NH) * D;
    float4 w0[DENSE ? 1 : NC], w1[DENSE ? 1 : NC];
    uint4 qv[NH];
    if constexpr (!DENSE && !SYM) {
        const float *cb8 = a.cb8 + ((size_t)hkv * G + g) * kCodes8 * 8;
        const float *cb4 = a.cb4 + ((size_t)hkv * G + g) * kCodes4 * 8;
#pragma unroll
        for (int k = 0; k < NC; k++) {
            const int c = min(c0 + k * TPG, kLutCodes - 1);
            const float *w = c < kCodes8 ? cb8 + c * 8 : cb4 + (c - kCodes8) * 8;
            w0[k] = *reinterpret_cast<const float4 *>(w);
            w1[k] = *reinterpret_cast<const float4 *>(w + 4);
        }
#pragma unroll
        for (int h = 0; h < NH; h++)
            qv[h] = *reinterpret_cast<const uint4 *>(qrow + h * D + 8 * g);
    }
    // SYM: the row's tabulated LUT (already in the LDS layout), loaded with
    // the rest and written to LDS after the one wait
    constexpr int LPT = SYM ? (LUT_FLOATS / 4 + kThreads - 1) / kThreads : 1;
    f32x4 lv[LPT];
    if constexpr (SYM) {
        const f32x4 *src = reinterpret_cast<const f32x4 *>(a.glut + (size_t)row * LUT_FLOATS);
#pragma unroll
        for (int k = 0; k < LPT; k++) {
            const int i = tid + k * kThreads;
            lv[k] = src[i < LUT_FLOATS / 4 ? i : LUT_FLOATS / 4 - 1];
        }
    }
    // Query operand of the key MFMA: lane h + 16 r takes dims 16 b + 4 r ..
    // +3 of head h (zero for h >= NH), as bf16 (bf16 keys) or as fp16
    // scaled by 2^-e_h with the head's largest |q| in [2^14, 2^15).
    // (branch-free: lanes of unused heads read head NH - 1 and drop it)
    u32x2 qraw[D / 16];
    const int hq_ld = L.hl < NH ? L.hl : NH - 1;
#pragma unroll
    for (int b = 0; b < D / 16; b++)
        qraw[b] = *reinterpret_cast<const u32x2 *>(qrow + (size_t)hq_ld * D + 16 * b + 4 * L.r);
    // This workgroup's pages are p_k = split + k * nsplit, k < n_wg; wave w
    // takes k = w + kWaves * i, i < n_mine.  Their table entries are staged
    // in LDS.
    const int np = a.num_pages[row];
    const int n_wg = split < np ? (np - split + a.nsplit - 1) / a.nsplit : 0;
    const int n_mine = wave < n_wg ? (n_wg - wave + kWaves - 1) / kWaves : 0;
    const int last = n_mine - 1;
    const uint32_t *pt = a.page_table + (size_t)row * a.maxp;
    const uint8_t *pm = a.page_meta + (size_t)row * a.maxp;
    // Then, once the page count is in, the wave's first table entry and the
    // workgroup's table entries.  The first page's loads go out only after
    // the prologue's one wait: vector-memory
    // waits drain in issue order, so a page issued earlier would hold up
    // the tabulation behind its own latency.  The tabulation then overlaps
    // the page's loads.
    PageRegs<D> bufA, bufB;
    uint2 first = make_uint2(0u, 0u);
    if (n_mine > 0) {
        const int p0 = split + wave * a.nsplit;
        first = make_uint2(pt[p0], pm[p0]);
    }
    constexpr int TE = 2; // table entries per thread held in registers
    uint32_t te_off[TE], te_meta[TE];
#pragma unroll
    for (int j = 0; j < TE; j++) {
        const int k = tid + j * kThreads;
        te_off[j] = 0u;
        te_meta[j] = 0u;
        if (k < n_wg) {
            const int p = split + k * a.nsplit;
            te_off[j] = pt[p];
            te_meta[j] = pm[p];
        }
    }
    // (lanes of unused heads zero their query slices only now: the select
    // waits for the loads)
#pragma unroll
    for (int b = 0; b < D / 16; b++)
        qraw[b] = L.hl < NH ? qraw[b] : u32x2{0u, 0u};
    // per-head max |q| (each wave on its own: in pass p lane j holds 8 dims
    // of head p HPP + j / (D/8))
    int eh = 0;
    if constexpr (!DENSE) {
        constexpr int LPH = D / 8;   // lanes per head
        constexpr int HPP = 64 / LPH; // heads per pass
#pragma unroll
        for (int h0 = 0; h0 < NH; h0 += HPP) {
            float mx = 0.f;
            {
                // (branch-free: lanes past the group's heads read its last
                // slice and drop it)
                const int nl = (NH - h0 < HPP ? NH - h0 : HPP) * LPH;
                const uint4 v = *reinterpret_cast<const uint4 *>(qrow + (size_t)h0 * D + 8 * (lane < nl ? lane : nl - 1));
                const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; e++)
                    mx = fmaxf(mx, fmaxf(fabsf(bf16_lo(u[e])), fabsf(bf16_hi(u[e]))));
                mx = lane < nl ? mx : 0.f;
            }
#pragma unroll
            for (int o = 1; o < LPH; o <<= 1)
                mx = fmaxf(mx, __shfl_xor(mx, o, 64));
#pragma unroll
            for (int h = h0; h < NH && h < h0 + HPP; h++) {
                const float m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx), (h - h0) * LPH));
                int ex = 0;
                if (m > 0.f) {
                    frexpf(m, &ex);
                    ex -= 15;
                }
                eh = L.hl == h ? ex : eh;
            }
        }
    }
    if constexpr (SYM) {
        // (an empty asm that takes the table's registers: the compiler may
        // not defer its loads to their LDS stores, which would wait for
        // each in turn)
#pragma unroll
        for (int k = 0; k < LPT; k++)
            asm volatile("" : "+v"(lv[k]));
    }
    QOperand<D, DENSE> qo;
#pragma unroll
    for (int b = 0; b < D / 16; b++) {
        if constexpr (DENSE) {
            qo.blk[b] = __builtin_bit_cast(s16x4, qraw[b]);
        } else {
            f16x4 o;
            o[0] = (_Float16)ldexpf(bf16_lo(qraw[b].x), -eh);
            o[1] = (_Float16)ldexpf(bf16_hi(qraw[b].x), -eh);
            o[2] = (_Float16)ldexpf(bf16_lo(qraw[b].y), -eh);
            o[3] = (_Float16)ldexpf(bf16_hi(qraw[b].y), -eh);
            qo.blk[b] = o;
        }
    }
    const float lsc = ldexpf(a.sigma, eh) * kLog2e;
    if constexpr (SYM) {
        // (threads past the end rewrite the last entry with its own value,
        // so no write is conditional and no load is deferred)
#pragma unroll
        for (int k = 0; k < LPT; k++) {
            const int i = tid + k * kThreads;
            reinterpret_cast<f32x4 *>(lut)[i < LUT_FLOATS / 4 ? i : LUT_FLOATS / 4 - 1] = lv[k];
        }
    }
    ADA_PHASE(1);
    // The wave's first page: its loads go out only now, after every other
    // prologue load has been waited for, so the tabulation below overlaps
    // them instead of waiting behind them.
    if (n_mine > 0)
        fetch_entry<D, DENSE>(bufA, first, a.arena, L);
#pragma unroll
    for (int j = 0; j < TE; j++)
        if (tid + j * kThreads < n_wg)
            tbl[tid + j * kThreads] = make_uint2(te_off[j], te_meta[j]);
    for (int k = tid + TE * kThreads; k < n_wg; k += kThreads) {
        const int p = split + k * a.nsplit;
        tbl[k] = make_uint2(pt[p], pm[p]);
    }
    if constexpr (SYM) {
        // (written to LDS before the first page was issued)
    } else if constexpr (!DENSE) {
        // LUT[g][c][h] = q_h[8g .. 8g+8) . C[g][c] (c < 256 from cb8, else cb4)
        float qq[NH][8];
#pragma unroll
        for (int h = 0; h < NH; h++) {
            const uint32_t u[4] = {qv[h].x, qv[h].y, qv[h].z, qv[h].w};
#pragma unroll
            for (int e = 0; e < 4; e++) {
                qq[h][2 * e] = bf16_lo(u[e]);
                qq[h][2 * e + 1] = bf16_hi(u[e]);
            }
        }
#pragma unroll
        for (int k = 0; k < NC; k++) {
            const int c = c0 + k * TPG;
            if (c < kLutCodes) {
                float o[NH];
#pragma unroll
                for (int h = 0; h < NH; h++) {
                    float acc = qq[h][0] * w0[k].x;
                    acc = fmaf(qq[h][1], w0[k].y, acc);
                    acc = fmaf(qq[h][2], w0[k].z, acc);
                    acc = fmaf(qq[h][3], w0[k].w, acc);
                    acc = fmaf(qq[h][4], w1[k].x, acc);
                    acc = fmaf(qq[h][5], w1[k].y, acc);
                    acc = fmaf(qq[h][6], w1[k].z, acc);
                    acc = fmaf(qq[h][7], w1[k].w, acc);
                    o[h] = acc;
                }
                lut_store<NH, G>(lut, g * kLutCodes + c, o);
            }
        }
    }
    const float sig2 = a.sigma * kLog2e;
    ADA_PHASE(2);

    __syncthreads();
    ADA_PHASE(3);

    WaveState<D, NH> st;
#pragma unroll
    for (int b = 0; b < D / 16; b++)
        st.acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < NH; h++)
        st.m[h] = -INFINITY;
    st.mlane = L.hl < NH ? -INFINITY : 0.f;
    st.l = 0.f;
    float *lgout = a.logits ? a.logits + ((size_t)s * a.Hq + (size_t)hkv * NH) * a.maxp * kSlots
                            : nullptr;

    // Two register buffers in turn: page i+1's loads are in flight while
    // page i is computed.  Pages go in pairs through a loop with one exit;
    // every half-step issues one page's loads (past the end it reloads the
    // last page), so the wait counts are fixed.  The table entry of the
    // page after next is read from LDS a half-step ahead.  An odd last page
    // is in bufA.
    uint2 next = n_mine > 0 ? tbl[wave + kWaves * min(1, last)] : make_uint2(0u, 0u);
    int i = 0;
    for (; i + 1 < n_mine; i += 2) {
        fetch_entry<D, DENSE>(bufB, next, a.arena, L);
        next = tbl[wave + kWaves * min(i + 2, last)];
        process_page<D, NH, DENSE>(bufA, split + (wave + kWaves * i) * a.nsplit, st, lut, qo, lsc, sig2,
                                   lgout, a.maxp, L);
        fetch_entry<D, DENSE>(bufA, next, a.arena, L);
        next = tbl[wave + kWaves * min(i + 3, last)];
        process_page<D, NH, DENSE>(bufB, split + (wave + kWaves * (i + 1)) * a.nsplit, st, lut, qo, lsc,
                                   sig2, lgout, a.maxp, L);
    }
    if (i < n_mine) {
        fetch_entry<D, DENSE>(bufB, next, a.arena, L); // keeps the wait count
        process_page<D, NH, DENSE>(bufA, split + (wave + kWaves * i) * a.nsplit, st, lut, qo, lsc, sig2,
                                   lgout, a.maxp, L);
    }
    ADA_PHASE(4);

    // Waves -> LDS (the LUT space is free now): [wave][D][NHP] accumulators
    // (element h = head h) and [wave][h] (m, l).
    constexpr int NHP = 4 * Heads<NH>::NQ;
    float *red = smem;
    float *redml = smem + kWaves * D * NHP;
    const float lsum = rows_sum(st.l);
    __syncthreads();
    if (lane < 16 * Heads<NH>::NQ) {
#pragma unroll
        for (int b = 0; b < D / 16; b++)
            *reinterpret_cast<f32x4 *>(red + ((size_t)wave * D + 16 * b + L.hl) * NHP + 4 * L.r) = st.acc[b];
    }
    if (lane < NH) {
        redml[(wave * NH + lane) * 2] = st.mlane;
        redml[(wave * NH + lane) * 2 + 1] = lsum;
    }
    __syncthreads();

    // Merge the waves into this split's (m, l, acc), or into the outputs
    // when the row has one split.
    const size_t part = (size_t)row * a.nsplit + split;
    for (int i2 = tid; i2 < NH * D; i2 += kThreads) {
        const int h = i2 / D, d = i2 - h * D;
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; w++)
            mx = fmaxf(mx, redml[(w * NH + h) * 2]);
        float o = 0.f, l = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; w++) {
            const float mw = redml[(w * NH + h) * 2];
            const float f = mw > -INFINITY ? __builtin_amdgcn_exp2f(mw - mx) : 0.f;
            o = fmaf(red[((size_t)w * D + d) * NHP + h], f, o);
            l = fmaf(redml[(w * NH + h) * 2 + 1], f, l);
        }
        if (a.nsplit == 1) {
            const size_t sh = (size_t)s * a.Hq + (size_t)hkv * NH + h;
            a.out[sh * D + d] = mx > -INFINITY ? o / l : 0.f;
            if (a.lse != nullptr && d == 0)
                a.lse[sh] = mx > -INFINITY ? (mx + __log2f(l)) * kLn2 : -INFINITY;
            continue;
        }
        a.part_acc[(part * NH + h) * D + d] = o;
        if (d == 0) {
            a.part_ml[(part * NH + h) * 2] = mx;
            a.part_ml[(part * NH + h) * 2 + 1] = l;
        }
    }
#ifdef ADA_PHASE_TRACE
    __builtin_amdgcn_s_waitcnt(0);
    ADA_PHASE(5);
    if (a.trace != nullptr && lane == 0) {
        unsigned long long *t = a.trace + ((size_t)blockIdx.x * kWaves + wave) * 8;
        t[6] = __builtin_amdgcn_s_getreg((4 << 0) | (0 << 6) | (31 << 11));  // HW_ID
        t[7] = __builtin_amdgcn_s_getreg((20 << 0) | (0 << 6) | (15 << 11)); // XCC_ID
    }
#endif
}

// ---- split merge --------------------------------------------------------------
// One workgroup per (row, query head): out = sum_i acc_i 2^(m_i - m) /
// sum_i l_i 2^(m_i - m) over the row's splits (m = max m_i, empty splits
// with m_i = -inf skipped), lse = (m + log2 of the denominator) in nats.
// The partials come from the page-stream kernel before it in the stream.
// The first batch of partial columns is loaded together with the (m, l)
// pairs, so the merge costs about one memory latency.
constexpr int kMergeThreads = 256;
constexpr int kMergeBatch = 8;

template <int D, int NH>
__global__ __launch_bounds__(kMergeThreads) void decode_merge(DecodeArgs a)
{
    constexpr int ITEMS = D / 4;                 // 4-float columns of one head
    constexpr int KS = kMergeThreads / ITEMS;    // threads per column
    __shared__ float sm[kMaxSplitsDev], sl[kMaxSplitsDev];
    __shared__ float swave[kMergeThreads / 64][2];
    __shared__ float4 scol[KS][ITEMS];
    const int row = blockIdx.x, h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int s = row / a.Hkv, hkv = row % a.Hkv;
    const int ns = a.nsplit;
    const int item = tid % ITEMS, part_i = tid / ITEMS;
    const size_t base = (size_t)row * ns * NH + h;  // split k of this head: base + k * NH
    const float *acc = a.part_acc + base * D + 4 * item;

    float4 v[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; j++)
        v[j] = *reinterpret_cast<const float4 *>(acc + (size_t)min(part_i + j * KS, ns - 1) * NH * D);
    float mx = -INFINITY;
    for (int k = tid; k < ns; k += kMergeThreads) {
        const float2 ml = *reinterpret_cast<const float2 *>(a.part_ml + (base + (size_t)k * NH) * 2);
        sm[k] = ml.x;
        sl[k] = ml.y;
        mx = fmaxf(mx, ml.x);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    if (lane == 0)
        swave[wave][0] = mx;
    __syncthreads();
    mx = swave[0][0];
#pragma unroll
    for (int w = 1; w < kMergeThreads / 64; w++)
        mx = fmaxf(mx, swave[w][0]);
    // weights 2^(m_i - m) in place of m_i, and the denominator
    float l = 0.f;
    for (int k = tid; k < ns; k += kMergeThreads) {
        const float m = sm[k];
        const float f = m > -INFINITY ? __builtin_amdgcn_exp2f(m - mx) : 0.f;
        sm[k] = f;
        l = fmaf(sl[k], f, l);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        l += __shfl_xor(l, o, 64);
    if (lane == 0)
        swave[wave][1] = l;
    __syncthreads();
    l = 0.f;
#pragma unroll
    for (int w = 0; w < kMergeThreads / 64; w++)
        l += swave[w][1];

    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k0 = part_i;; ) {
#pragma unroll
        for (int j = 0; j < kMergeBatch; j++) {
            const int k = k0 + j * KS;
            const float f = k < ns ? sm[k] : 0.f;
            o.x = fmaf(v[j].x, f, o.x);
            o.y = fmaf(v[j].y, f, o.y);
            o.z = fmaf(v[j].z, f, o.z);
            o.w = fmaf(v[j].w, f, o.w);
        }
        k0 += kMergeBatch * KS;
        if (k0 >= ns)
            break;
#pragma unroll
        for (int j = 0; j < kMergeBatch; j++)
            v[j] = *reinterpret_cast<const float4 *>(acc + (size_t)min(k0 + j * KS, ns - 1) * NH * D);
    }
    scol[part_i][item] = o;
    __syncthreads();
    if (tid < ITEMS) {
        float4 t = scol[0][tid];
#pragma unroll
        for (int k = 1; k < KS; k++) {
            t.x += scol[k][tid].x;
            t.y += scol[k][tid].y;
            t.z += scol[k][tid].z;
            t.w += scol[k][tid].w;
        }
        const bool any = mx > -INFINITY;
        const float inv = any ? 1.f / l : 0.f;
        const size_t sh = (size_t)s * a.Hq + (size_t)hkv * NH + h;
        *reinterpret_cast<float4 *>(a.out + sh * D + 4 * tid) =
            make_float4(t.x * inv, t.y * inv, t.z * inv, t.w * inv);
        if (a.lse != nullptr && tid == 0)
            a.lse[sh] = any ? (mx + __log2f(l)) * kLn2 : -INFINITY;
    }
}

// ---- symmetric variant: the LUT from the query's codes -------------------------
// One wave per (row, group g, query head h), with no barrier and no LDS.
// The query direction u_q = q / |q| (|q| summed sequentially over D, in
// double) takes in each codebook the index of its nearest codeword (squared
// distance in double, lowest index on ties), as a key does in encode; then
// LUT_g[c][h] = |q_h| C_g[cq_h] . C_g[c] (fp32 dot product), written in the
// page stream's LDS layout.
template <int NH, int G>
__device__ __forceinline__ float *lut_slot(float *lut, int idx, int h)
{
    constexpr int NQF = Heads<NH>::NQF, REM = Heads<NH>::REM;
    constexpr int REGION = G * kLutCodes * 4;
    return h < 4 * NQF ? lut + (h / 4) * REGION + idx * 4 + (h % 4)
                       : lut + NQF * REGION + idx * REM + (h - 4 * NQF);
}

__device__ __forceinline__ double readlane_f64(double x, int l)
{
    const uint64_t v = (uint64_t)__double_as_longlong(x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ float readlane_f32(float x, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

template <int D, int NH>
__global__ __launch_bounds__(64 * NH) void sym_lut_kernel(DecodeArgs a)
{
    // the query code is decided in double with every product rounded
    // before it is added, as the definition does: no fused multiply-adds
#pragma clang fp contract(off)
    constexpr int G = D / 8, LUT_FLOATS = G * kLutCodes * NH;
    const int row = blockIdx.x, g = blockIdx.y, lane = threadIdx.x & 63;
    const int h = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int s = row / a.Hkv, hkv = row % a.Hkv;
    const uint16_t *qh = a.q + ((size_t)s * a.Hq + (size_t)hkv * NH + h) * D;
    const float *c8 = a.cb8 + ((size_t)hkv * G + g) * kCodes8 * 8;
    const float *c4 = a.cb4 + ((size_t)hkv * G + g) * kCodes4 * 8;
    // Every global load is issued before any is used (one memory latency):
    // lane l's 8-bit codewords l + 64 k, its 4-bit codeword l % 16, and
    // (lanes below G) query coordinates 8 l .. 8 l + 7.
    float4 w0[4], w1[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        w0[k] = *reinterpret_cast<const float4 *>(c8 + (lane + 64 * k) * 8);
        w1[k] = *reinterpret_cast<const float4 *>(c8 + (lane + 64 * k) * 8 + 4);
    }
    const int c4i = lane & 15; // (lanes 16 .. 63 repeat lanes 0 .. 15)
    const float4 v0 = *reinterpret_cast<const float4 *>(c4 + c4i * 8);
    const float4 v1 = *reinterpret_cast<const float4 *>(c4 + c4i * 8 + 4);
    const uint4 qv = *reinterpret_cast<const uint4 *>(qh + 8 * (lane < G ? lane : 0));
    const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};

    // |q_h| is the squares summed in order in double, as the keys' norms.
    // That sum is the exact sum whenever no partial sum needs rounding:
    // every square is a multiple of 2^e (e the smallest exponent of a
    // square's last bit), so when the exact total is below 2^(52 + e) every
    // partial sum, in any order, is exact.  The G lanes (8 coordinates
    // each) sum in a tree and test that; otherwise the wave sums in order.
    double part = 0.0;
    int emin = 1 << 20;
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const float x = __uint_as_float((j & 1 ? qw[j / 2] >> 16 : qw[j / 2] & 0xffffu) << 16);
        part = part + (double)x * (double)x;
        const uint32_t bits = __float_as_uint(x);
        const int ex = (int)((bits >> 23) & 0xff);
        // last bit of a bf16 value: 2^(E - 134); subnormals 2^-133
        const int last = ex == 0 ? -133 : ex - 134;
        emin = (bits & 0x7fffffffu) != 0 ? min(emin, 2 * last) : emin;
    }
    const double tot = readlane_f64(row_sum_f64<D == 64>(part), 0);
    const int emin0 = __builtin_amdgcn_readlane(row_min_i32<D == 64>(emin), 0);
    double ss = tot;
    if (!(tot < ldexp(1.0, 52 + max(emin0, -1000)))) {
        ss = 0.0;
        for (int j8 = 0; j8 < G; j8++) {
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const uint32_t wv = (uint32_t)__builtin_amdgcn_readlane((int)qw[e], j8);
                const double lo = (double)__uint_as_float(wv << 16);
                const double hi = (double)__uint_as_float(wv & 0xffff0000u);
                ss = ss + lo * lo;
                ss = ss + hi * hi;
            }
        }
    }
    const double qn = sqrt(ss);
    // this group's direction slice, from lane g's coordinates
    double u[8];
#pragma unroll
    for (int e = 0; e < 4; e++) {
        const uint32_t wv = (uint32_t)__builtin_amdgcn_readlane((int)qw[e], g);
        const double lo = (double)__uint_as_float(wv << 16);
        const double hi = (double)__uint_as_float(wv & 0xffff0000u);
        u[2 * e] = qn > 0.0 ? lo / qn : 0.0;
        u[2 * e + 1] = qn > 0.0 ? hi / qn : 0.0;
    }
    // nearest 8-bit codeword: lane l scores l, l + 64, l + 128, l + 192
    double bd = INFINITY;
    int bc = 0;
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const float w[8] = {w0[k].x, w0[k].y, w0[k].z, w0[k].w, w1[k].x, w1[k].y, w1[k].z, w1[k].w};
        double d = 0.0;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const double df = u[j] - (double)w[j];
            d = d + df * df;
        }
        if (k == 0 || d < bd) {
            bd = d;
            bc = lane + 64 * k;
        }
    }
    wave_argmin(bd, bc);
    const int cq8 = __builtin_amdgcn_readfirstlane(bc);
    // nearest 4-bit codeword
    {
        const float w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        double d = 0.0;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const double df = u[j] - (double)w[j];
            d = d + df * df;
        }
        bd = d;
        bc = c4i;
    }
    wave_argmin(bd, bc);
    const int cq4 = __builtin_amdgcn_readfirstlane(bc);
    // the two query codewords, read from the lanes that hold them (every
    // candidate register is read and the uniform index picks one, so no
    // register array is indexed at run time)
    float wq8[8], wq4[8];
    {
        const int kq = cq8 >> 6, lq = cq8 & 63;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            float r[4];
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const float4 &c = j < 4 ? w0[k] : w1[k];
                const float x = (j & 3) == 0 ? c.x : (j & 3) == 1 ? c.y : (j & 3) == 2 ? c.z : c.w;
                r[k] = readlane_f32(x, lq);
            }
            wq8[j] = kq == 0 ? r[0] : kq == 1 ? r[1] : kq == 2 ? r[2] : r[3];
        }
        const float t4[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int j = 0; j < 8; j++)
            wq4[j] = readlane_f32(t4[j], cq4);
    }
    float *lut = a.glut + (size_t)row * LUT_FLOATS;
    const float qf = (float)qn;
    auto entry = [&](const float4 &c0, const float4 &c1, const float (&wq)[8], int c) {
        const float wc[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        float acc = wq[0] * wc[0];
#pragma unroll
        for (int j = 1; j < 8; j++)
            acc = fmaf(wq[j], wc[j], acc);
        *lut_slot<NH, G>(lut, g * kLutCodes + c, h) = acc * qf;
    };
#pragma unroll
    for (int k = 0; k < 4; k++)
        entry(w0[k], w1[k], wq8, lane + 64 * k);
    if (lane < kCodes4)
        entry(v0, v1, wq4, kCodes8 + lane);
}

template <int D, int NH, bool DENSE>
size_t shmem_bytes(int max_wg_pages)
{
    const size_t lut = DENSE ? 0 : (size_t)(D / 8) * kLutCodes * NH * sizeof(float);
    const size_t b = lut + (size_t)max_wg_pages * sizeof(uint2);
    constexpr size_t W = Waves<D, NH>::W;
    const size_t red = (W * D * 4 * Heads<NH>::NQ + W * NH * 2) * sizeof(float);
    return b > red ? b : red;
}

template <int D, int NH, bool DENSE, bool SYM>
hipError_t launch_t(const DecodeArgs &a, hipStream_t st, unsigned stages)
{
    const int rows = a.S * a.Hkv;
    if (rows <= 0 || a.nsplit <= 0)
        return hipSuccess;
    const size_t shmem = shmem_bytes<D, NH, DENSE>((a.maxp + a.nsplit - 1) / a.nsplit);
    // the kernel's dynamic-LDS limit, raised once per device as needed
    constexpr int kMaxDevices = 64;
    static std::atomic<size_t> attr_set[kMaxDevices];
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    if (shmem > attr_set[dev].load()) {
        hipError_t e = hipFuncSetAttribute((const void *)decode_main<D, NH, DENSE, SYM>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
        if (e != hipSuccess)
            return e;
        size_t cur = attr_set[dev].load();
        while (shmem > cur && !attr_set[dev].compare_exchange_weak(cur, shmem)) {
        }
    }
    hipError_t e = hipSuccess;
    if constexpr (SYM) {
        if (stages & kStageStream) {
            hipLaunchKernelGGL((sym_lut_kernel<D, NH>), dim3(rows, D / 8), dim3(64 * NH), 0, st, a);
            e = hipGetLastError();
            if (e != hipSuccess)
                return e;
        }
    }
    if (stages & kStageStream) {
        hipLaunchKernelGGL((decode_main<D, NH, DENSE, SYM>), dim3(rows * a.nsplit), dim3(Waves<D, NH>::THREADS),
                           shmem, st, a);
        e = hipGetLastError();
    }
    if (e != hipSuccess || a.nsplit == 1 || !(stages & kStageMerge))
        return e;
    hipLaunchKernelGGL((decode_merge<D, NH>), dim3(rows, NH), dim3(kMergeThreads), 0, st, a);
    return hipGetLastError();
}

} // namespace

size_t decode_lut_floats(int D, int NH) { return (size_t)(D / 8) * kLutCodes * NH; }

int decode_waves(int D, int NH) { return (D == 128 && NH > 4) ? Waves<128, 8>::W : Waves<64, 1>::W; }

hipError_t noalloc_scratch(void **ptr)
{
    // looked up once per device, with that device current (the caller's)
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void *p = nullptr;
        if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)); e != hipSuccess)
            return e;
        if (p == nullptr)
            return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

size_t decode_shmem_bytes(int D, int NH, bool dense, int nsplit, int maxp)
{
    const int wg = (maxp + nsplit - 1) / nsplit;
#define ADA_CASE(DD, NN)                                                                          \
    if (D == DD && NH == NN)                                                                      \
        return dense ? shmem_bytes<DD, NN, true>(wg) : shmem_bytes<DD, NN, false>(wg);
    ADA_CASE(64, 1)
    ADA_CASE(64, 2)
    ADA_CASE(64, 4)
    ADA_CASE(64, 5)
    ADA_CASE(64, 8)
    ADA_CASE(128, 1)
    ADA_CASE(128, 2)
    ADA_CASE(128, 4)
    ADA_CASE(128, 5)
    ADA_CASE(128, 8)
#undef ADA_CASE
    return 0;
}

hipError_t launch_decode(int D, int NH, bool dense, const DecodeArgs &a, hipStream_t st, unsigned stages,
                         bool sym)
{
#define ADA_CASE(DD, NN)                                                                          \
    if (D == DD && NH == NN)                                                                      \
        return dense ? launch_t<DD, NN, true, false>(a, st, stages)                               \
                     : sym ? launch_t<DD, NN, false, true>(a, st, stages)                          \
                           : launch_t<DD, NN, false, false>(a, st, stages);
    ADA_CASE(64, 1)
    ADA_CASE(64, 2)
    ADA_CASE(64, 4)
    ADA_CASE(64, 5)
    ADA_CASE(64, 8)
    ADA_CASE(128, 1)
    ADA_CASE(128, 2)
    ADA_CASE(128, 4)
    ADA_CASE(128, 5)
    ADA_CASE(128, 8)
#undef ADA_CASE
    return hipErrorInvalidValue;
}

} // namespace ada
