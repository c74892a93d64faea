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
// Work decomposition.  One workgroup (8 wave64s, one per CU at D = 128)
// serves one (sequence, kv-head) row and one of `nsplit` interleaved page
// subsets of it, for all NH query heads of the GQA group, so every page is
// read from HBM once.  Wave w of split s takes pages s + (w + 8i) * nsplit.
// A wave holds a page in 64 lanes: lane (tl, db) = tl * 8 + db keeps slots tl
// and tl + 8 for the dims of block db ([db * D/8, (db + 1) * D/8)), and the
// codes of the groups inside that block.  The page format stores exactly
// these values as the lane's own 16-byte chunks, so every load is one
// coalesced dwordx4 per lane.  Each wave keeps the next page's loads in
// flight while it computes the current one (a register double buffer), and
// its page-table entries sit in lane registers, 64 pages at a time.
// Logits are summed over the 8 dim blocks of a slot with three DPP steps
// inside a row; each lane then weights its own value chunks, so the PV
// product needs no lane exchange.  Running maxima are wave-wide (DPP row
// max + two row broadcasts per head and page); accumulators are rescaled
// only when the maximum grows by more than 2^8, which keeps every weight
// <= 2^8.  At the end the 8 slot pairs are summed with lane exchanges, the
// 8 waves are merged through LDS, and the split's partial (m, l, acc) is
// written; the last split of each row to finish (an atomic counter per row)
// merges the row's partials into the outputs, so one decode step is one
// kernel launch.
#include "ada_internal.h"

namespace ada {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescale = 8.0f; // log2 of the largest weight kept between rescales
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ float f16_to_f32(uint32_t h)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Sum over the 8 dim-block lanes of a slot pair (lanes 8k..8k+7); every lane
// of the group receives the total.
__device__ __forceinline__ float block_sum8(float x)
{
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xb1, 0xf, 0xf, false)); // xor 1
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4e, 0xf, 0xf, false)); // xor 2
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xf, 0xf, false)); // half-row mirror
    return x;
}

// Max over the whole wave, returned as a wave-uniform value.  Lanes of one
// slot pair hold equal values, so the row step only needs the 8-lane rotate.
__device__ __forceinline__ float wave_max(float x)
{
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xf, 0xf, false))); // row_ror 8
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), 0x142, 0xa, 0xf, false))); // row_bcast 15
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), 0x143, 0xc, 0xf, false))); // row_bcast 31
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// Device-coherent (agent-scope) accesses to the split partials.
__device__ __forceinline__ void coherent_store(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sum over the 8 slot pairs (lanes db, db+8, ..., db+56).
__device__ __forceinline__ float pair_sum8(float x)
{
    x += __shfl_xor(x, 8, 64);
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    return x;
}

template <int NH>
__device__ __forceinline__ void lut_add(const float *lut, int idx, float (&sum)[NH])
{
    if constexpr (NH == 4) {
        float4 v = *reinterpret_cast<const float4 *>(lut + idx * 4);
        sum[0] += v.x; sum[1] += v.y; sum[2] += v.z; sum[3] += v.w;
    } else if constexpr (NH == 2) {
        float2 v = *reinterpret_cast<const float2 *>(lut + idx * 2);
        sum[0] += v.x; sum[1] += v.y;
    } else {
        sum[0] += lut[idx];
    }
}

// Raw bytes of one page as this lane sees them: eight 16-byte loads.
//   tiers 0/3: c[0..D/32) K chunks, then D/32 V chunks
//   tier 1:    c[0..D/32) V chunks; c[4], c[5] the 16-byte blocks holding
//              slot t0's / t1's codes; c[6], c[7] radius[0..8) / [8..16)
//   tier 2:    c[0..D/64) V chunks; c[2], c[3] value scale[0..8) / [8..16);
//              c[4..7] as in tier 1
// Unused slots repeat the page's first chunk (same cache lines, no extra
// HBM traffic).  Every tier issues the same eight loads with no branch, so
// the next page's loads stay in flight while the current page is computed.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef const u32x4 __attribute__((address_space(1))) *gchunk;

struct PageRegs {
    u32x4 c[8];
    int tier, nvalid;
};

template <int D, bool DENSE>
__device__ __forceinline__ void fetch_page(PageRegs &pr, const uint8_t *page, int tier, int nvalid,
                                           int lane, int t0)
{
    constexpr int G = D / 8;
    const int t1 = t0 + 8;
    pr.tier = tier;
    pr.nvalid = nvalid;
    // byte offsets inside the page (the page address is wave-uniform)
    uint32_t o[8];
    const uint32_t lo = lane * 16;
    if (DENSE || tier == 0) {
#pragma unroll
        for (int c = 0; c < 8; c++)
            o[c] = c < D / 16 ? lo + c * 1024 : lo;
    } else {
        const int rb = tier == 1 ? G : G / 2; // code bytes per slot
        const uint32_t codes = codes_off(D, tier), rad = radius_off(D, tier);
        const int nv = tier == 1 ? D / 32 : D / 64;
#pragma unroll
        for (int c = 0; c < 4; c++)
            o[c] = c < nv ? lo + c * 1024 : lo;
        if (tier == 2) {
            o[2] = vscale_off(D);
            o[3] = vscale_off(D) + 16;
        }
        o[4] = codes + ((t0 * rb) & ~15);
        o[5] = codes + ((t1 * rb) & ~15);
        o[6] = rad;
        o[7] = rad + 16;
    }
#pragma unroll
    for (int c = 0; c < 8; c++)
        pr.c[c] = *(gchunk)(page + o[c]);
}

// Bytes at a per-lane offset o (0..15) of a 16-byte chunk, picked with
// masks and a 64-bit shift so the chunk stays in registers.
__device__ __forceinline__ uint32_t bits_at(const u32x4 &v, int o)
{
    const uint64_t lo = ((uint64_t)v.y << 32) | v.x;
    const uint64_t hi = ((uint64_t)v.w << 32) | v.z;
    const uint64_t m = 0ull - (uint64_t)((o >> 3) & 1);
    return (uint32_t)(((lo & ~m) | (hi & m)) >> (8 * (o & 7)));
}
__device__ __forceinline__ uint32_t u8_at(const u32x4 &v, int o) { return bits_at(v, o) & 255u; }
__device__ __forceinline__ uint32_t u16_at(const u32x4 &v, int o) { return bits_at(v, o) & 0xffffu; }

template <int D, int NH>
struct WaveState {
    float m_run[NH], l_run[NH], corr[NH], acc[NH][D / 8];
};

// Logits, online-softmax update and PV product of one page (page index p in
// its row) for the wave's NH query heads.
template <int D, int NH, bool DENSE>
__device__ __forceinline__ void process_page(const PageRegs &cur, int p, WaveState<D, NH> &st,
                                             const float *lut, const uint32_t *qh,
                                             const float (&lscale)[NH], float sigma, float *lgout,
                                             int maxp, int t0, int db)
{
    constexpr int G = D / 8, B = D / 8, GPL = B / 8, NWC = D / 32, NNC = D / 64;
    const int t1 = t0 + 8;
    const int tier = cur.tier;
    const bool v0 = t0 < cur.nvalid, v1 = t1 < cur.nvalid;

    float lg0[NH], lg1[NH];
    if (DENSE || tier == 0) {
        // dot-product tier: the lane's K chunks (slot t0 first), then the
        // sum over the 8 dim blocks
        float p0[NH], p1[NH];
#pragma unroll
        for (int h = 0; h < NH; h++)
            p0[h] = p1[h] = 0.f;
#pragma unroll
        for (int c = 0; c < NWC; c++) {
            const uint32_t kw[4] = {cur.c[c].x, cur.c[c].y, cur.c[c].z, cur.c[c].w};
            const int qo = db * (B / 2) + ((8 * c) % B) / 2; // first q pair of this chunk
            const bool second = (8 * c) >= B;
#pragma unroll
            for (int h = 0; h < NH; h++) {
                const u32x4 qv = *reinterpret_cast<const u32x4 *>(qh + h * (D / 2) + qo);
                const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
                for (int w = 0; w < 4; w++) {
                    float &pp = second ? p1[h] : p0[h];
                    if constexpr (DENSE)
                        pp = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, qw[w]),
                                                             __builtin_bit_cast(bf162_t, kw[w]), pp, false);
                    else
                        pp = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, qw[w]),
                                                    __builtin_bit_cast(half2_t, kw[w]), pp, false);
                }
            }
        }
#pragma unroll
        for (int h = 0; h < NH; h++) {
            lg0[h] = block_sum8(p0[h]) * lscale[h];
            lg1[h] = block_sum8(p1[h]) * lscale[h];
        }
    } else {
        float s0[NH], s1[NH];
#pragma unroll
        for (int h = 0; h < NH; h++)
            s0[h] = s1[h] = 0.f;
        // the lane's code byte(s) inside its two 16-byte code blocks
        const int rb = tier == 1 ? G : G / 2;
        const int ob = tier == 1 ? GPL * db : (GPL * db) / 2;
        const int o0 = ((t0 * rb) & 15) + ob, o1 = ((t1 * rb) & 15) + ob;
        if (tier == 1) {
            const uint32_t code0 = GPL == 2 ? u16_at(cur.c[4], o0) : u8_at(cur.c[4], o0);
            const uint32_t code1 = GPL == 2 ? u16_at(cur.c[5], o1) : u8_at(cur.c[5], o1);
#pragma unroll
            for (int k = 0; k < GPL; k++) {
                lut_add<NH>(lut, (GPL * db + k) * kLutCodes + ((code0 >> (8 * k)) & 255), s0);
                lut_add<NH>(lut, (GPL * db + k) * kLutCodes + ((code1 >> (8 * k)) & 255), s1);
            }
        } else {
            const int sh = GPL == 2 ? 0 : 4 * (db & 1);
            const uint32_t code0 = u8_at(cur.c[4], o0), code1 = u8_at(cur.c[5], o1);
#pragma unroll
            for (int k = 0; k < GPL; k++) {
                lut_add<NH>(lut, (GPL * db + k) * kLutCodes + kCodes8 + ((code0 >> (sh + 4 * k)) & 15), s0);
                lut_add<NH>(lut, (GPL * db + k) * kLutCodes + kCodes8 + ((code1 >> (sh + 4 * k)) & 15), s1);
            }
        }
        const float r0 = sigma * f16_to_f32(u16_at(cur.c[6], 2 * t0));
        const float r1 = sigma * f16_to_f32(u16_at(cur.c[7], 2 * t0));
#pragma unroll
        for (int h = 0; h < NH; h++) {
            lg0[h] = block_sum8(s0[h]) * r0;
            lg1[h] = block_sum8(s1[h]) * r1;
        }
    }

    if (lgout != nullptr && db == 0) {
#pragma unroll
        for (int h = 0; h < NH; h++) {
            float *lo = lgout + (size_t)h * maxp * kSlots + (size_t)p * kSlots;
            if (v0)
                lo[t0] = lg0[h];
            if (v1)
                lo[t1] = lg1[h];
        }
    }

    // online softmax, log2 domain
    float w0[NH], w1[NH];
#pragma unroll
    for (int h = 0; h < NH; h++) {
        const float x0 = v0 ? lg0[h] * kLog2e : -INFINITY;
        const float x1 = v1 ? lg1[h] * kLog2e : -INFINITY;
        const float pmax = wave_max(fmaxf(x0, x1));
        if (pmax > st.m_run[h] + kRescale) {
            const float f = __builtin_amdgcn_exp2f(st.m_run[h] - pmax);
            st.l_run[h] *= f;
            st.corr[h] *= f;
#pragma unroll
            for (int e = 0; e < B; e++)
                st.acc[h][e] *= f;
            st.m_run[h] = pmax;
        }
        w0[h] = __builtin_amdgcn_exp2f(x0 - st.m_run[h]);
        w1[h] = __builtin_amdgcn_exp2f(x1 - st.m_run[h]);
        st.l_run[h] += w0[h] + w1[h];
    }

    if (DENSE || tier != 2) {
        const bool kfirst = DENSE || tier == 0; // V chunks follow K in tiers 0 and 3
#pragma unroll
        for (int c = 0; c < NWC; c++) {
            const u32x4 v = kfirst ? cur.c[NWC + c] : cur.c[c];
            const float vf[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                                 bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
            const int eo = (8 * c) % B;
            const bool second = (8 * c) >= B;
#pragma unroll
            for (int h = 0; h < NH; h++) {
                const float wt = second ? w1[h] : w0[h];
#pragma unroll
                for (int e = 0; e < 8; e++)
                    st.acc[h][eo + e] = fmaf(wt, vf[e], st.acc[h][eo + e]);
            }
        }
    } else {
        // int8 values: weight * scale applied to the biased bytes
        // (byte ^ 0x80 = v + 128); the bias is removed once at the end.
        const float sc0 = f16_to_f32(u16_at(cur.c[2], 2 * t0));
        const float sc1 = f16_to_f32(u16_at(cur.c[3], 2 * t0));
        float pv0[NH], pv1[NH];
#pragma unroll
        for (int h = 0; h < NH; h++) {
            pv0[h] = w0[h] * sc0;
            pv1[h] = w1[h] * sc1;
            st.corr[h] += pv0[h] + pv1[h];
        }
#pragma unroll
        for (int c = 0; c < NNC; c++) {
            const u32x4 v = cur.c[c];
            const uint32_t vw[4] = {v.x ^ 0x80808080u, v.y ^ 0x80808080u, v.z ^ 0x80808080u,
                                    v.w ^ 0x80808080u};
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const int w = 16 * c + e; // lane element
                const float b = (float)((vw[e / 4] >> (8 * (e % 4))) & 255u);
#pragma unroll
                for (int h = 0; h < NH; h++) {
                    const float wt = w >= B ? pv1[h] : pv0[h];
                    st.acc[h][w % B] = fmaf(wt, b, st.acc[h][w % B]);
                }
            }
        }
    }
}

// Issues the loads of the page whose table entry is e = (offset in 128-byte
// units, metadata byte); e is the same in every lane.
template <int D, bool DENSE>
__device__ __forceinline__ void fetch_entry(PageRegs &pr, uint2 e, const uint8_t *arena, int lane, int t0)
{
    const uint32_t off = __builtin_amdgcn_readfirstlane(e.x);
    const uint32_t meta = __builtin_amdgcn_readfirstlane(e.y);
    fetch_page<D, DENSE>(pr, arena + (size_t)off * kUnit, meta & 3, ((meta >> 2) & 15) + 1, lane, t0);
}

template <int D, int NH, bool DENSE>
__global__ __launch_bounds__(kThreads) void decode_main(DecodeArgs a)
{
    constexpr int G = D / 8;      // code groups
    constexpr int B = D / 8;      // dims per lane block
    constexpr int LUT_FLOATS = DENSE ? 0 : G * kLutCodes * NH;

    extern __shared__ float smem[];
    float *lut = smem;
    float *qs = smem + LUT_FLOATS;                                  // [NH][D] fp32 queries
    uint32_t *qh = reinterpret_cast<uint32_t *>(qs + NH * D);        // [NH][D/2] query pairs
    uint2 *tbl = reinterpret_cast<uint2 *>(qh + NH * D / 2);        // [n_wg] page-table entries

    // Consecutive logical blocks share an XCD (blocks are dealt round-robin
    // over the 8 XCDs), so one row's splits hit one L2.
    const int nblk = gridDim.x;
    int logical = blockIdx.x;
    if (nblk % 8 == 0)
        logical = (blockIdx.x % 8) * (nblk / 8) + blockIdx.x / 8;
    const int row = logical / a.nsplit, split = logical % a.nsplit;
    const int s = row / a.Hkv, hkv = row % a.Hkv;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int tl = lane >> 3, db = lane & 7;
    const int t0 = tl; // the lane's slots are t0 and t0 + 8

    // This workgroup's pages are p_k = split + k * nsplit, k < n_wg; wave w
    // takes k = w + kWaves * i, i < n_mine.  Their table entries are staged
    // in LDS.
    const int np = a.num_pages[row];
    const int n_wg = split < np ? (np - split + a.nsplit - 1) / a.nsplit : 0;
    const int n_mine = wave < n_wg ? (n_wg - wave + kWaves - 1) / kWaves : 0;
    {
        const uint32_t *pt = a.page_table + (size_t)row * a.maxp;
        const uint8_t *pm = a.page_meta + (size_t)row * a.maxp;
        for (int k = tid; k < n_wg; k += kThreads) {
            const int p = split + k * a.nsplit;
            tbl[k] = make_uint2(pt[p], pm[p]);
        }
    }
    const uint16_t *qg = a.q + ((size_t)s * a.Hq + (size_t)hkv * NH) * D;
    for (int i = tid; i < NH * D; i += kThreads)
        qs[i] = __uint_as_float((uint32_t)qg[i] << 16);
    __syncthreads();

    // the first page's loads overlap the code-table build
    PageRegs bufA, bufB;
    if (n_mine > 0)
        fetch_entry<D, DENSE>(bufA, tbl[wave], a.arena, lane, t0);

    if constexpr (!DENSE) {
        // LUT[g][c][h] = q_h[8g..8g+8) . C[g][c]; c < 256 from cb8, else cb4.
        // All of a thread's codeword loads are issued before any is used.
        constexpr int CW = G * kLutCodes;
        constexpr int PER = (CW + kThreads - 1) / kThreads;
        const float *cb8 = a.cb8 + (size_t)hkv * G * kCodes8 * 8;
        const float *cb4 = a.cb4 + (size_t)hkv * G * kCodes4 * 8;
        float4 w0[PER], w1[PER];
#pragma unroll
        for (int k = 0; k < PER; k++) {
            const int i = min(tid + k * kThreads, CW - 1);
            const int g = i / kLutCodes, c = i - g * kLutCodes;
            const float *w = c < kCodes8 ? cb8 + ((size_t)g * kCodes8 + c) * 8
                                         : cb4 + ((size_t)g * kCodes4 + (c - kCodes8)) * 8;
            w0[k] = *reinterpret_cast<const float4 *>(w);
            w1[k] = *reinterpret_cast<const float4 *>(w + 4);
        }
#pragma unroll
        for (int k = 0; k < PER; k++) {
            const int i = tid + k * kThreads;
            if (i < CW) {
                const int g = i / kLutCodes;
#pragma unroll
                for (int h = 0; h < NH; h++) {
                    const float *qq = qs + h * D + 8 * g;
                    float acc = qq[0] * w0[k].x;
                    acc = fmaf(qq[1], w0[k].y, acc);
                    acc = fmaf(qq[2], w0[k].z, acc);
                    acc = fmaf(qq[3], w0[k].w, acc);
                    acc = fmaf(qq[4], w1[k].x, acc);
                    acc = fmaf(qq[5], w1[k].y, acc);
                    acc = fmaf(qq[6], w1[k].z, acc);
                    acc = fmaf(qq[7], w1[k].w, acc);
                    lut[i * NH + h] = acc;
                }
            }
        }
    }

    // Query pairs for the dot-product tiers, in LDS.  Tier 0 (fp16 keys): q
    // as fp16 pairs, each head scaled by 2^-e_h so its largest |q| lies in
    // [2^14, 2^15) (exact for bf16 values within 2^-28 of that maximum);
    // tier 3 (bf16 keys): q as bf16 pairs, exact.
    float lscale[NH]; // softmax scale (times 2^e_h for tier 0)
#pragma unroll
    for (int h = 0; h < NH; h++) {
        float mx = 0.f;
        for (int d = lane; d < D; d += 64)
            mx = fmaxf(mx, fabsf(qs[h * D + d]));
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1)
            mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        int e = 0;
        if (!DENSE && mx > 0.f) {
            int ex;
            frexpf(mx, &ex);
            e = ex - 15;
        }
        lscale[h] = ldexpf(a.sigma, e);
        if (wave == 0) {
            for (int k = lane; k < D / 2; k += 64) {
                const float x0 = qs[h * D + 2 * k], x1 = qs[h * D + 2 * k + 1];
                if constexpr (DENSE) {
                    qh[h * (D / 2) + k] = (__float_as_uint(x0) >> 16) | (__float_as_uint(x1) & 0xffff0000u);
                } else {
                    half2_t v;
                    v.x = (_Float16)ldexpf(x0, -e);
                    v.y = (_Float16)ldexpf(x1, -e);
                    qh[h * (D / 2) + k] = __builtin_bit_cast(uint32_t, v);
                }
            }
        }
    }
    __syncthreads();

    WaveState<D, NH> st;
#pragma unroll
    for (int h = 0; h < NH; h++) {
        st.m_run[h] = -INFINITY;
        st.l_run[h] = 0.f;
        st.corr[h] = 0.f;
#pragma unroll
        for (int e = 0; e < B; e++)
            st.acc[h][e] = 0.f;
    }
    float *lgout = a.logits ? a.logits + ((size_t)s * a.Hq + (size_t)hkv * NH) * a.maxp * kSlots
                            : nullptr;

    // Two register buffers in turn: page i+1's loads are in flight while
    // page i is computed.  Every half-step issues its eight loads (past the
    // end it reloads the last page), so the wait counts are fixed.
    const int last = n_mine - 1;
    for (int i = 0; i < n_mine; i += 2) {
        fetch_entry<D, DENSE>(bufB, tbl[wave + kWaves * min(i + 1, last)], a.arena, lane, t0);
        process_page<D, NH, DENSE>(bufA, split + (wave + kWaves * i) * a.nsplit, st, lut, qh, lscale,
                                   a.sigma, lgout, a.maxp, t0, db);
        if (i + 1 >= n_mine)
            break;
        fetch_entry<D, DENSE>(bufA, tbl[wave + kWaves * min(i + 2, last)], a.arena, lane, t0);
        process_page<D, NH, DENSE>(bufB, split + (wave + kWaves * (i + 1)) * a.nsplit, st, lut, qh,
                                   lscale, a.sigma, lgout, a.maxp, t0, db);
    }

    // Sum the 8 slot pairs of each dim block in registers, then the waves
    // through LDS (the LUT space is free now): [wave][h][D] accumulators and
    // [wave][h] (m, l).
    float *red = smem;
    float *redml = smem + kWaves * NH * D;
    __syncthreads();
#pragma unroll
    for (int h = 0; h < NH; h++) {
        float *dst = red + ((size_t)wave * NH + h) * D + db * B;
#pragma unroll
        for (int e = 0; e < B; e++) {
            const float v = pair_sum8(st.acc[h][e] - 128.f * st.corr[h]);
            if (tl == 0)
                dst[e] = v;
        }
        const float lsum = pair_sum8(st.l_run[h]);
        if (lane == 0) {
            redml[(wave * NH + h) * 2] = st.m_run[h];
            redml[(wave * NH + h) * 2 + 1] = lsum;
        }
    }
    __syncthreads();

    // Merge the waves into this split's (m, l, acc).
    const size_t part = (size_t)row * a.nsplit + split;
    for (int i = tid; i < NH * D; i += kThreads) {
        const int h = i / D, d = i - h * D;
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; w++)
            mx = fmaxf(mx, redml[(w * NH + h) * 2]);
        float o = 0.f, l = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; w++) {
            const float mw = redml[(w * NH + h) * 2];
            const float f = mw > -INFINITY ? __builtin_amdgcn_exp2f(mw - mx) : 0.f;
            o = fmaf(red[((size_t)w * NH + h) * D + d], f, o);
            l = fmaf(redml[(w * NH + h) * 2 + 1], f, l);
        }
        const size_t sh = (size_t)s * a.Hq + (size_t)hkv * NH + h;
        if (a.nsplit == 1) {
            a.out[sh * D + d] = mx > -INFINITY ? o / l : 0.f;
            if (a.lse != nullptr && d == 0)
                a.lse[sh] = mx > -INFINITY ? (mx + __log2f(l)) * kLn2 : -INFINITY;
            continue;
        }
        coherent_store(a.part_acc + (part * NH + h) * D + d, o);
        if (d == 0) {
            coherent_store(a.part_ml + (part * NH + h) * 2, mx);
            coherent_store(a.part_ml + (part * NH + h) * 2 + 1, l);
        }
    }
    if (a.nsplit == 1)
        return;

    // The last split of a row to finish merges all of them:
    // out = sum_i acc_i 2^(m_i - m) / sum_i l_i 2^(m_i - m), lse in nats.
    // Partials move through device-coherent accesses (agent-scope atomic
    // stores and loads, which bypass the per-XCD L2), so the hand-off needs
    // only the stores to have completed before the counter moves -- no L2
    // write-back or invalidate.  The counter is reset for the next call.
    __shared__ int is_last;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const unsigned prev = __hip_atomic_fetch_add(a.counters + row, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        is_last = prev == (unsigned)a.nsplit - 1;
    }
    __syncthreads();
    if (!is_last)
        return;

    // LDS: per (split, head) m, l and the weight f = 2^(m - m*); per head
    // m*, l*; then [KS][NH][D] partial column sums.
    const int ns = a.nsplit;
    float *sm = smem;           // [ns][NH]
    float *sf = sm + ns * NH;   // [ns][NH]
    float *sl = sf + ns * NH;   // [ns][NH]
    float *smax = sl + ns * NH; // [NH]
    float *ssum = smax + NH;    // [NH]
    float *scol = ssum + NH;    // [KS][NH][D]
    const size_t base = (size_t)row * ns * NH;
    for (int i = tid; i < ns * NH; i += kThreads) {
        sm[i] = coherent_load(a.part_ml + (base + i) * 2);
        sl[i] = coherent_load(a.part_ml + (base + i) * 2 + 1);
    }
    __syncthreads();
    // wave h < NH: m* and l* of head h
    if (wave < NH) {
        const int h = wave;
        float mx = -INFINITY;
        for (int k = lane; k < ns; k += 64)
            mx = fmaxf(mx, sm[k * NH + h]);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1)
            mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        float l = 0.f;
        for (int k = lane; k < ns; k += 64) {
            const float m = sm[k * NH + h];
            const float f = m > -INFINITY ? __builtin_amdgcn_exp2f(m - mx) : 0.f;
            sf[k * NH + h] = f;
            l = fmaf(sl[k * NH + h], f, l);
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1)
            l += __shfl_xor(l, o, 64);
        if (lane == 0) {
            smax[h] = mx;
            ssum[h] = l;
        }
    }
    __syncthreads();
    // columns: item = (h, 4 dims); KS threads share an item, each summing
    // every KS-th split, with many loads in flight
    constexpr int ITEMS = NH * D / 4;
    constexpr int KS = kThreads / ITEMS;
    {
        const int item = tid % ITEMS, part_i = tid / ITEMS;
        const int h = item / (D / 4), d4 = item % (D / 4);
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
        if (part_i < KS) {
            const float *src = a.part_acc + (base + h) * D + 4 * d4;
            // batches of 16 splits: all loads of a batch are in flight at once
            for (int k0 = part_i; k0 < ns; k0 += 16 * KS) {
                float v[16][4];
#pragma unroll
                for (int j = 0; j < 16; j++) {
                    const int k = min(k0 + j * KS, ns - 1);
                    const float *pv = src + (size_t)k * NH * D;
#pragma unroll
                    for (int e = 0; e < 4; e++)
                        v[j][e] = coherent_load(pv + e);
                }
#pragma unroll
                for (int j = 0; j < 16; j++) {
                    const int k = k0 + j * KS;
                    const float f = k < ns ? sf[k * NH + h] : 0.f;
                    o.x = fmaf(v[j][0], f, o.x);
                    o.y = fmaf(v[j][1], f, o.y);
                    o.z = fmaf(v[j][2], f, o.z);
                    o.w = fmaf(v[j][3], f, o.w);
                }
            }
            *reinterpret_cast<float4 *>(scol + ((size_t)part_i * NH + h) * D + 4 * d4) = o;
        }
    }
    __syncthreads();
    for (int i = tid; i < NH * D; i += kThreads) {
        const int h = i / D, d = i - h * D;
        float o = 0.f;
#pragma unroll
        for (int k = 0; k < KS; k++)
            o += scol[((size_t)k * NH + h) * D + d];
        const float mx = smax[h], l = ssum[h];
        const size_t sh = (size_t)s * a.Hq + (size_t)hkv * NH + h;
        a.out[sh * D + d] = mx > -INFINITY ? o / l : 0.f;
        if (a.lse != nullptr && d == 0)
            a.lse[sh] = mx > -INFINITY ? (mx + __log2f(l)) * kLn2 : -INFINITY;
    }
    if (tid == 0)
        __hip_atomic_store(a.counters + row, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, int NH, bool DENSE>
size_t shmem_bytes(int nsplit, int max_wg_pages)
{
    const size_t lut = DENSE ? 0 : (size_t)(D / 8) * kLutCodes * NH * sizeof(float);
    size_t b = lut + (size_t)NH * D * sizeof(float) + (size_t)NH * D / 2 * sizeof(uint32_t) +
               (size_t)max_wg_pages * sizeof(uint2);
    const size_t red = ((size_t)kWaves * NH * D + (size_t)kWaves * NH * 2) * sizeof(float);
    constexpr int KS = kThreads / (NH * D / 4);
    const size_t merge = ((size_t)3 * nsplit * NH + 2 * NH + (size_t)KS * NH * D) * sizeof(float);
    b = b > red ? b : red;
    return b > merge ? b : merge;
}

template <int D, int NH, bool DENSE>
hipError_t launch_t(const DecodeArgs &a, hipStream_t st)
{
    const int rows = a.S * a.Hkv;
    const size_t shmem = shmem_bytes<D, NH, DENSE>(a.nsplit, (a.maxp + a.nsplit - 1) / a.nsplit);
    static size_t attr_set = 0;
    if (shmem > attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)decode_main<D, NH, DENSE>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
        if (e != hipSuccess)
            return e;
        attr_set = shmem;
    }
    if (rows > 0 && a.nsplit > 0) {
        hipLaunchKernelGGL((decode_main<D, NH, DENSE>), dim3(rows * a.nsplit), dim3(kThreads), shmem, st, a);
        return hipGetLastError();
    }
    return hipSuccess;
}

} // namespace

size_t decode_shmem_bytes(int D, int NH, bool dense, int nsplit, int maxp)
{
    const int wg = (maxp + nsplit - 1) / nsplit;
#define ADA_CASE(DD, NN)                                                                          \
    if (D == DD && NH == NN)                                                                      \
        return dense ? shmem_bytes<DD, NN, true>(nsplit, wg) : shmem_bytes<DD, NN, false>(nsplit, wg);
    ADA_CASE(64, 1)
    ADA_CASE(64, 2)
    ADA_CASE(64, 4)
    ADA_CASE(128, 1)
    ADA_CASE(128, 2)
    ADA_CASE(128, 4)
#undef ADA_CASE
    return 0;
}

hipError_t launch_decode(int D, int NH, bool dense, const DecodeArgs &a, hipStream_t st)
{
#define ADA_CASE(DD, NN)                                                                          \
    if (D == DD && NH == NN)                                                                      \
        return dense ? launch_t<DD, NN, true>(a, st) : launch_t<DD, NN, false>(a, st);
    ADA_CASE(64, 1)
    ADA_CASE(64, 2)
    ADA_CASE(64, 4)
    ADA_CASE(128, 1)
    ADA_CASE(128, 2)
    ADA_CASE(128, 4)
#undef ADA_CASE
    return hipErrorInvalidValue;
}

} // namespace ada
