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
// Work decomposition.  One workgroup (4 wave64s) serves one (sequence,
// kv-head) row and one of `nsplit` interleaved page subsets of it, for all
// NH query heads of the GQA group, so every page is read from HBM once.
// Wave w of split s takes pages s + (w + 4i) * nsplit.  A wave holds a page
// in 64 lanes: lane (tl, db) = tl * 8 + db keeps slots tl and tl + 8 for the
// dims of block db ([db * D/8, (db + 1) * D/8)), and the codes of the groups
// inside that block.  The page format stores exactly these values as the
// lane's own 16-byte chunks, so every load is one coalesced dwordx4 per lane.
// Logits are summed over the 8 dim blocks of a slot with three DPP steps
// inside a row; each lane then weights its own value chunks, so the PV
// product needs no lane exchange.  Running maxima are wave-wide (DPP row
// max + two row broadcasts per head and page); accumulators are rescaled
// only when the maximum grows by more than 2^8, which keeps every weight
// <= 2^8.  At the end the lanes' partial sums go through LDS, the 4 waves
// and 8 slot pairs are merged, and the split's partial (m, l, acc) is
// written; the last split of each row to finish (an atomic counter per row)
// merges the row's partials into the outputs, so one decode step is one
// kernel launch.
#include "ada_internal.h"

namespace ada {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescale = 8.0f; // log2 of the largest weight kept between rescales

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ float f16_to_f32(uint16_t h)
{
    return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ float uniform(float x)
{
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
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

template <int D, int NH, bool DENSE>
__global__ __launch_bounds__(256) void decode_main(DecodeArgs a)
{
    constexpr int G = D / 8;      // code groups
    constexpr int B = D / 8;      // dims per lane block
    constexpr int GPL = B / 8;    // code groups per lane block
    constexpr int NWC = D / 32;   // 16-byte chunks per lane, 2-byte elements
    constexpr int NNC = D / 64;   // 16-byte chunks per lane, 1-byte elements
    constexpr int LUT_FLOATS = DENSE ? 0 : G * kLutCodes * NH;

    extern __shared__ float smem[];
    float *lut = smem;
    float *qs = smem + LUT_FLOATS; // [NH][D] fp32 queries

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

    const uint16_t *qg = a.q + ((size_t)s * a.Hq + (size_t)hkv * NH) * D;
    for (int i = tid; i < NH * D; i += 256)
        qs[i] = __uint_as_float((uint32_t)qg[i] << 16);
    __syncthreads();

    if constexpr (!DENSE) {
        // LUT[g][c][h] = q_h[8g..8g+8) . C[g][c]; c < 256 from cb8, else cb4.
        const float *cb8 = a.cb8 + (size_t)hkv * G * kCodes8 * 8;
        const float *cb4 = a.cb4 + (size_t)hkv * G * kCodes4 * 8;
        for (int i = tid; i < G * kLutCodes; i += 256) {
            const int g = i / kLutCodes, c = i - g * kLutCodes;
            const float *w = c < kCodes8 ? cb8 + ((size_t)g * kCodes8 + c) * 8
                                         : cb4 + ((size_t)g * kCodes4 + (c - kCodes8)) * 8;
            const float4 w0 = *reinterpret_cast<const float4 *>(w);
            const float4 w1 = *reinterpret_cast<const float4 *>(w + 4);
#pragma unroll
            for (int h = 0; h < NH; h++) {
                const float *qq = qs + h * D + 8 * g;
                float acc = qq[0] * w0.x;
                acc = fmaf(qq[1], w0.y, acc);
                acc = fmaf(qq[2], w0.z, acc);
                acc = fmaf(qq[3], w0.w, acc);
                acc = fmaf(qq[4], w1.x, acc);
                acc = fmaf(qq[5], w1.y, acc);
                acc = fmaf(qq[6], w1.z, acc);
                acc = fmaf(qq[7], w1.w, acc);
                lut[i * NH + h] = acc;
            }
        }
    }

    // Query registers for the dot-product tiers, the lane block's B dims per
    // head.  Tier 0 (fp16 keys): q as fp16 pairs, each head scaled by 2^-e_h
    // so its largest |q| lies in [2^14, 2^15) (exact for bf16 values within
    // 2^-28 of that maximum); tier 3 (bf16 keys): q as bf16 pairs, exact.
    uint32_t qreg[NH][B / 2];
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
#pragma unroll
        for (int k = 0; k < B / 2; k++) {
            const float x0 = qs[h * D + db * B + 2 * k], x1 = qs[h * D + db * B + 2 * k + 1];
            if constexpr (DENSE) {
                qreg[h][k] = (__float_as_uint(x0) >> 16) | (__float_as_uint(x1) & 0xffff0000u);
            } else {
                half2_t v;
                v.x = (_Float16)ldexpf(x0, -e);
                v.y = (_Float16)ldexpf(x1, -e);
                qreg[h][k] = __builtin_bit_cast(uint32_t, v);
            }
        }
    }
    __syncthreads();

    float m_run[NH], l_run[NH], corr[NH], acc[NH][B];
#pragma unroll
    for (int h = 0; h < NH; h++) {
        m_run[h] = -INFINITY;
        l_run[h] = 0.f;
        corr[h] = 0.f;
#pragma unroll
        for (int e = 0; e < B; e++)
            acc[h][e] = 0.f;
    }

    const int np = a.num_pages[row];
    const uint32_t *pt = a.page_table + (size_t)row * a.maxp;
    const uint8_t *pm = a.page_meta + (size_t)row * a.maxp;
    const int step = 4 * a.nsplit;
    float *lgout = a.logits ? a.logits + ((size_t)s * a.Hq + (size_t)hkv * NH) * a.maxp * kSlots
                            : nullptr;
    const int t0 = tl, t1 = tl + 8; // the lane's two slots

    for (int p = split + wave * a.nsplit; p < np; p += step) {
        const uint32_t off = pt[p];
        const uint32_t meta = pm[p];
        const int tier = meta & 3;
        const int nvalid = ((meta >> 2) & 15) + 1;
        const uint8_t *page = a.arena + (size_t)off * kUnit;
        const bool v0 = t0 < nvalid, v1 = t1 < nvalid;

        float lg0[NH], lg1[NH];
        float sc0 = 1.f, sc1 = 1.f;
        if (DENSE || tier == 0) {
            // dot-product tier: the lane's K chunks (slot t0 first), then the
            // sum over the 8 dim blocks
            float p0[NH], p1[NH];
#pragma unroll
            for (int h = 0; h < NH; h++)
                p0[h] = p1[h] = 0.f;
#pragma unroll
            for (int c = 0; c < NWC; c++) {
                const uint4 k = *reinterpret_cast<const uint4 *>(page + c * 1024 + lane * 16);
                const uint32_t kw[4] = {k.x, k.y, k.z, k.w};
                const int qo = ((8 * c) % B) / 2; // first q pair of this chunk
                const bool second = (8 * c) >= B;
#pragma unroll
                for (int h = 0; h < NH; h++)
#pragma unroll
                    for (int w = 0; w < 4; w++) {
                        float &pp = second ? p1[h] : p0[h];
                        if constexpr (DENSE)
                            pp = __builtin_amdgcn_fdot2_f32_bf16(
                                __builtin_bit_cast(bf162_t, qreg[h][qo + w]),
                                __builtin_bit_cast(bf162_t, kw[w]), pp, false);
                        else
                            pp = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, qreg[h][qo + w]),
                                                        __builtin_bit_cast(half2_t, kw[w]), pp, false);
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
            const uint8_t *codes = page + codes_off(D, tier);
            if (tier == 1) {
                if constexpr (GPL == 2) {
                    const uint32_t c0 = *reinterpret_cast<const uint16_t *>(codes + t0 * G + 2 * db);
                    const uint32_t c1 = *reinterpret_cast<const uint16_t *>(codes + t1 * G + 2 * db);
#pragma unroll
                    for (int k = 0; k < 2; k++) {
                        lut_add<NH>(lut, (2 * db + k) * kLutCodes + ((c0 >> (8 * k)) & 255), s0);
                        lut_add<NH>(lut, (2 * db + k) * kLutCodes + ((c1 >> (8 * k)) & 255), s1);
                    }
                } else {
                    lut_add<NH>(lut, db * kLutCodes + codes[t0 * G + db], s0);
                    lut_add<NH>(lut, db * kLutCodes + codes[t1 * G + db], s1);
                }
            } else {
                if constexpr (GPL == 2) {
                    const uint32_t c0 = codes[t0 * (G / 2) + db];
                    const uint32_t c1 = codes[t1 * (G / 2) + db];
#pragma unroll
                    for (int k = 0; k < 2; k++) {
                        lut_add<NH>(lut, (2 * db + k) * kLutCodes + kCodes8 + ((c0 >> (4 * k)) & 15), s0);
                        lut_add<NH>(lut, (2 * db + k) * kLutCodes + kCodes8 + ((c1 >> (4 * k)) & 15), s1);
                    }
                } else {
                    const int sh = 4 * (db & 1);
                    const uint32_t c0 = codes[t0 * (G / 2) + db / 2];
                    const uint32_t c1 = codes[t1 * (G / 2) + db / 2];
                    lut_add<NH>(lut, db * kLutCodes + kCodes8 + ((c0 >> sh) & 15), s0);
                    lut_add<NH>(lut, db * kLutCodes + kCodes8 + ((c1 >> sh) & 15), s1);
                }
                const uint16_t *vs = reinterpret_cast<const uint16_t *>(page + vscale_off(D));
                sc0 = f16_to_f32(vs[t0]);
                sc1 = f16_to_f32(vs[t1]);
            }
            const uint16_t *rr = reinterpret_cast<const uint16_t *>(page + radius_off(D, tier));
            const float r0 = a.sigma * f16_to_f32(rr[t0]);
            const float r1 = a.sigma * f16_to_f32(rr[t1]);
#pragma unroll
            for (int h = 0; h < NH; h++) {
                lg0[h] = block_sum8(s0[h]) * r0;
                lg1[h] = block_sum8(s1[h]) * r1;
            }
        }

        if (lgout != nullptr && db == 0) {
#pragma unroll
            for (int h = 0; h < NH; h++) {
                float *lo = lgout + (size_t)h * a.maxp * kSlots + (size_t)p * kSlots;
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
            if (pmax > m_run[h] + kRescale) {
                const float f = __builtin_amdgcn_exp2f(m_run[h] - pmax);
                l_run[h] *= f;
                corr[h] *= f;
#pragma unroll
                for (int e = 0; e < B; e++)
                    acc[h][e] *= f;
                m_run[h] = pmax;
            }
            w0[h] = __builtin_amdgcn_exp2f(x0 - m_run[h]);
            w1[h] = __builtin_amdgcn_exp2f(x1 - m_run[h]);
            l_run[h] += w0[h] + w1[h];
        }

        if (DENSE || tier != 2) {
            const uint8_t *vp = page + v_off(D, DENSE ? 3 : tier);
#pragma unroll
            for (int c = 0; c < NWC; c++) {
                const uint4 v = *reinterpret_cast<const uint4 *>(vp + c * 1024 + lane * 16);
                const float vf[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                                     bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
                const int eo = (8 * c) % B;
                const bool second = (8 * c) >= B;
#pragma unroll
                for (int h = 0; h < NH; h++) {
                    const float wt = second ? w1[h] : w0[h];
#pragma unroll
                    for (int e = 0; e < 8; e++)
                        acc[h][eo + e] = fmaf(wt, vf[e], acc[h][eo + e]);
                }
            }
        } else {
            // int8 values: weight * scale applied to the biased bytes
            // (byte ^ 0x80 = v + 128); the bias is removed once at the end.
            float pv0[NH], pv1[NH];
#pragma unroll
            for (int h = 0; h < NH; h++) {
                pv0[h] = w0[h] * sc0;
                pv1[h] = w1[h] * sc1;
                corr[h] += pv0[h] + pv1[h];
            }
#pragma unroll
            for (int c = 0; c < NNC; c++) {
                const uint4 v = *reinterpret_cast<const uint4 *>(page + c * 1024 + lane * 16);
                const uint32_t vw[4] = {v.x ^ 0x80808080u, v.y ^ 0x80808080u, v.z ^ 0x80808080u,
                                        v.w ^ 0x80808080u};
#pragma unroll
                for (int e = 0; e < 16; e++) {
                    const int w = 16 * c + e; // lane element
                    const float b = (float)((vw[e / 4] >> (8 * (e % 4))) & 255u);
#pragma unroll
                    for (int h = 0; h < NH; h++) {
                        const float wt = w >= B ? pv1[h] : pv0[h];
                        acc[h][w % B] = fmaf(wt, b, acc[h][w % B]);
                    }
                }
            }
        }
    }

    // Partials through LDS (the LUT space is free now): [wave][tl][h][D]
    // accumulators, then [wave][h] (m, l).
    float *red = smem;
    float *redml = smem + 4 * 8 * NH * D;
    __syncthreads();
#pragma unroll
    for (int h = 0; h < NH; h++) {
        float *dst = red + (((size_t)wave * 8 + tl) * NH + h) * D + db * B;
#pragma unroll
        for (int e = 0; e < B; e += 4) {
            float4 v;
            v.x = acc[h][e] - 128.f * corr[h];
            v.y = acc[h][e + 1] - 128.f * corr[h];
            v.z = acc[h][e + 2] - 128.f * corr[h];
            v.w = acc[h][e + 3] - 128.f * corr[h];
            *reinterpret_cast<float4 *>(dst + e) = v;
        }
        const float lsum = pair_sum8(l_run[h]);
        if (lane == 0) {
            redml[(wave * NH + h) * 2] = m_run[h];
            redml[(wave * NH + h) * 2 + 1] = lsum;
        }
    }
    __syncthreads();

    // Merge the 4 waves and 8 slot pairs into this split's (m, l, acc).
    const size_t part = (size_t)row * a.nsplit + split;
    for (int i = tid; i < NH * D; i += 256) {
        const int h = i / D, d = i - h * D;
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; w++)
            mx = fmaxf(mx, redml[(w * NH + h) * 2]);
        float o = 0.f, l = 0.f;
        if (mx > -INFINITY) {
#pragma unroll
            for (int w = 0; w < 4; w++) {
                const float mw = redml[(w * NH + h) * 2];
                if (mw > -INFINITY) {
                    const float f = __builtin_amdgcn_exp2f(mw - mx);
                    float sum = 0.f;
#pragma unroll
                    for (int k = 0; k < 8; k++)
                        sum += red[(((size_t)w * 8 + k) * NH + h) * D + d];
                    o = fmaf(sum, f, o);
                    l = fmaf(redml[(w * NH + h) * 2 + 1], f, l);
                }
            }
        }
        const size_t sh = (size_t)s * a.Hq + (size_t)hkv * NH + h;
        if (a.nsplit == 1) {
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
    if (a.nsplit == 1)
        return;

    // The last split of a row to finish merges all of them:
    // out = sum_i acc_i 2^(m_i - m) / sum_i l_i 2^(m_i - m), lse in nats.
    // The counter is reset so the next call finds it at zero.
    __shared__ int is_last;
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const unsigned prev = __hip_atomic_fetch_add(a.counters + row, 1u, __ATOMIC_ACQ_REL,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        is_last = prev == (unsigned)a.nsplit - 1;
    }
    __syncthreads();
    if (!is_last)
        return;
    __threadfence();
    for (int i = tid; i < NH * D; i += 256) {
        const int h = i / D, d = i - h * D;
        const size_t base = (size_t)row * a.nsplit * NH + h;
        float mx = -INFINITY;
        for (int k = 0; k < a.nsplit; k++)
            mx = fmaxf(mx, a.part_ml[(base + (size_t)k * NH) * 2]);
        float o = 0.f, l = 0.f;
        if (mx > -INFINITY) {
            for (int k = 0; k < a.nsplit; k++) {
                const size_t pi = base + (size_t)k * NH;
                const float m = a.part_ml[pi * 2];
                if (m > -INFINITY) {
                    const float f = __builtin_amdgcn_exp2f(m - mx);
                    l = fmaf(a.part_ml[pi * 2 + 1], f, l);
                    o = fmaf(a.part_acc[pi * D + d], f, o);
                }
            }
        }
        const size_t sh = (size_t)s * a.Hq + (size_t)hkv * NH + h;
        a.out[sh * D + d] = mx > -INFINITY ? o / l : 0.f;
        if (a.lse != nullptr && d == 0)
            a.lse[sh] = mx > -INFINITY ? (mx + __log2f(l)) * kLn2 : -INFINITY;
    }
    if (tid == 0)
        a.counters[row] = 0;
}

template <int D, int NH, bool DENSE>
hipError_t launch_t(const DecodeArgs &a, hipStream_t st)
{
    const int rows = a.S * a.Hkv;
    const size_t lut = DENSE ? 0 : (size_t)(D / 8) * kLutCodes * NH * sizeof(float);
    size_t shmem = lut + (size_t)NH * D * sizeof(float);
    const size_t red = ((size_t)4 * 8 * NH * D + (size_t)4 * NH * 2) * sizeof(float);
    if (shmem < red)
        shmem = red;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)decode_main<D, NH, DENSE>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
        if (e != hipSuccess)
            return e;
        attr_set = true;
    }
    if (rows > 0 && a.nsplit > 0) {
        hipLaunchKernelGGL((decode_main<D, NH, DENSE>), dim3(rows * a.nsplit), dim3(256), shmem, st, a);
        return hipGetLastError();
    }
    return hipSuccess;
}

} // namespace

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
