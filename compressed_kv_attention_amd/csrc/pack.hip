// RDR pack for gfx950: per-row tiering and tier-homogeneous pages.
//
// SPHERICAL KV (arXiv 2605.18856), gist.science technical summary, section
// 2.2: each (token, head) state gets a residency bit and a precision tier;
// protected states are kept at the top tier; retained states are grouped into
// pages of a single tier.  The abstract adds that the choice is made per token
// and head under a fixed budget.  Either a row's tokens are ranked by
// (protected, utility score, -index) and cut at the tier counts the host
// computed from the sequence's cumulative basis points, or every token's tier
// is given (by the budget solver in rdr.hip).
//
// Kernels, in stream order:
//   pack_rows    one thread per row: advance num_pages and tier_tokens;
//   pack_rank    one 1024-thread block per row: radix-select the keys at the
//                three tier boundaries (8 passes of 8 bits over 64-bit keys,
//                exact because keys are unique; skipped when the tiers are
//                given), then walk the row in index
//                order with a block-wide scan to give every token its tier
//                page and slot (src[page][slot] = the token-head it holds);
//   pack_fill    one block per new page: assemble the page image in LDS in its
//                final byte layout (fields copied, values of the 4-bit tier
//                quantized, every other byte zero), write it with 16-byte
//                stores, then its page-table entry, metadata byte and
//                slot_token entries.
#include "ada_internal.h"
#include "numfmt.h"

namespace ada {
namespace {

#pragma clang fp contract(off)

__global__ __launch_bounds__(256) void pack_rows(PackPlan plan, PackCache cache)
{
    const int row = blockIdx.x * 256 + threadIdx.x;
    if (row >= plan.S * plan.Hkv)
        return;
    const PackRow rw = plan.rows[row];
    int pages = 0;
    for (int k = 0; k < 3; k++)
        pages += (rw.count[k] + kSlots - 1) / kSlots;
    cache.num_pages[row] += pages;
    if (!plan.dense && cache.tier_tokens != nullptr)
        for (int k = 0; k < 3; k++)
            cache.tier_tokens[row * 3 + k] += rw.count[k];
}

// Order-preserving map of a finite float (with -0 == +0) to uint32.
__device__ __forceinline__ uint32_t ord_score(float f)
{
    const uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t rank_key(const PackPlan &plan, const PackData &data,
                                             size_t e, int i)
{
    const uint64_t prot = plan.protect != nullptr && plan.protect[e] != 0 ? 1ull : 0ull;
    return (prot << 63) | ((uint64_t)ord_score(data.scores[e]) << 31) |
           (uint64_t)(0x7fffffffu - (uint32_t)i);
}

__global__ __launch_bounds__(1024) void pack_rank(PackPlan plan, PackData data)
{
    __shared__ uint32_t hist[3][256];
    __shared__ uint64_t prefix[3], mask[3], thr[3];
    __shared__ int64_t krem[3];
    __shared__ int has[3];
    __shared__ int wave_tot[16][3];
    __shared__ int running[3];

    const int row = blockIdx.x;
    const int s = row / plan.Hkv, h = row % plan.Hkv;
    const PackSeq sq = plan.seqs[s];
    const PackRow rw = plan.rows[row];
    const int T = sq.len;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    if (!plan.dense && plan.tiers == nullptr) {
        if (tid < 3) {
            has[tid] = sq.n_cum[tid] > 0;
            krem[tid] = (int64_t)sq.n_cum[tid] - 1;
            prefix[tid] = 0;
            mask[tid] = 0;
        }
        // the first kKeyRegs keys of each thread stay in registers across
        // the passes (all of them for rows of up to 4096 tokens)
        constexpr int kKeyRegs = 4;
        uint64_t kc[kKeyRegs];
#pragma unroll
        for (int v = 0; v < kKeyRegs; v++) {
            const int i = tid + 1024 * v;
            kc[v] = i < T ? rank_key(plan, data, ((size_t)sq.begin + i) * plan.Hkv + h, i) : 0ull;
        }
        __syncthreads();
        for (int pass = 0; pass < 8; pass++) {
            const int shift = 56 - 8 * pass;
            for (int i = tid; i < 3 * 256; i += 1024)
                (&hist[0][0])[i] = 0;
            __syncthreads();
            const uint64_t p0 = prefix[0], p1 = prefix[1], p2 = prefix[2];
            const uint64_t m0 = mask[0], m1 = mask[1], m2 = mask[2];
            auto count = [&](uint64_t K) {
                const uint32_t dg = (uint32_t)(K >> shift) & 255u;
                if (has[0] && (K & m0) == p0)
                    atomicAdd(&hist[0][dg], 1u);
                if (has[1] && (K & m1) == p1)
                    atomicAdd(&hist[1][dg], 1u);
                if (has[2] && (K & m2) == p2)
                    atomicAdd(&hist[2][dg], 1u);
            };
#pragma unroll
            for (int v = 0; v < kKeyRegs; v++)
                if (tid + 1024 * v < T)
                    count(kc[v]);
            for (int i = tid + 1024 * kKeyRegs; i < T; i += 1024)
                count(rank_key(plan, data, ((size_t)sq.begin + i) * plan.Hkv + h, i));
            __syncthreads();
            // wave k finds select k's digit: lane j holds digits 255 - 4j ..
            // 252 - 4j (descending), a wave scan gives the counts above each
            // lane's digits, and the first lane whose running count passes
            // krem holds the digit
            if (wave < 3 && has[wave]) {
                const int k = wave;
                uint32_t c[4];
                int sum = 0;
#pragma unroll
                for (int v = 0; v < 4; v++) {
                    c[v] = hist[k][255 - 4 * lane - v];
                    sum += (int)c[v];
                }
                int incl = sum;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const int t = __shfl_up(incl, off, 64);
                    if (lane >= off)
                        incl += t;
                }
                const int64_t kr = krem[k];
                const uint64_t hit = __ballot((int64_t)incl > kr);
                if (hit != 0 && lane == __builtin_ctzll(hit)) {
                    int64_t cum = incl - sum;
#pragma unroll
                    for (int v = 0; v < 4; v++) {
                        if (cum + (int64_t)c[v] > kr) {
                            prefix[k] |= (uint64_t)(255 - 4 * lane - v) << shift;
                            mask[k] |= 255ull << shift;
                            krem[k] = kr - cum;
                            break;
                        }
                        cum += c[v];
                    }
                }
            }
            __syncthreads();
        }
        if (tid < 3)
            thr[tid] = prefix[tid];
    }
    if (tid < 3)
        running[tid] = 0;
    // every slot of the row's new pages starts empty (the walk fills the
    // first `count` of each tier)
    for (int k = 0; k < 3; k++) {
        const int n16 = (rw.count[k] + kSlots - 1) / kSlots * kSlots;
        for (int i = tid; i < n16; i += 1024)
            plan.src[(size_t)rw.lp_first[k] * kSlots + i] = -1;
    }
    __syncthreads();

    for (int base = 0; base < T; base += 1024) {
        const int i = base + tid;
        const size_t e = ((size_t)sq.begin + i) * plan.Hkv + h;
        int tier = 3;
        if (i < T) {
            if (plan.dense) {
                tier = 0;
            } else if (plan.tiers != nullptr) {
                const int t = plan.tiers[e];
                tier = t < 3 ? t : 3;
            } else {
                const uint64_t K = rank_key(plan, data, e, i);
                tier = has[0] && K >= thr[0] ? 0 : has[1] && K >= thr[1] ? 1 : has[2] && K >= thr[2] ? 2 : 3;
            }
        }
        const uint64_t below = (1ull << lane) - 1ull;
        int lane_pre = 0;
#pragma unroll
        for (int k = 0; k < 3; k++) {
            const uint64_t b = __ballot(tier == k);
            if (lane == 0)
                wave_tot[wave][k] = __popcll(b);
            if (tier == k)
                lane_pre = __popcll(b & below);
        }
        __syncthreads();
        if (i < T) {
            if (tier < 3) {
                int pos = running[tier] + lane_pre;
                for (int w = 0; w < wave; w++)
                    pos += wave_tot[w][tier];
                // a position past the tier's count cannot happen with exact
                // thresholds; it is dropped rather than written out of range
                if (pos < rw.count[tier])
                    plan.src[(size_t)(rw.lp_first[tier] + pos / kSlots) * kSlots + pos % kSlots] = (int32_t)e;
            }
        }
        __syncthreads();
        if (tid < 3) {
            int tot = 0;
            for (int w = 0; w < 16; w++)
                tot += wave_tot[w][tid];
            running[tid] += tot;
        }
        __syncthreads();
    }
}

constexpr int kFillThreads = 256;
constexpr int kMaxPageBytes = 8192; // the largest page (D = 128, tiers 0 and 3)

__global__ __launch_bounds__(kFillThreads) void pack_fill(PackPlan plan, PackData data, PackCache cache)
{
    __shared__ uint4 img4[kMaxPageBytes / 16];
    __shared__ int64_t src_s[kSlots];
    const PackPage pg = plan.pages[blockIdx.x];
    const int tier = pg.meta & 3, nv = ((pg.meta >> 2) & 15) + 1;
    const int D = plan.D, G = D / 8, H = plan.Hkv;
    const int n16 = page_bytes(D, tier) / 16;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint8_t *img = reinterpret_cast<uint8_t *>(img4);
    for (int i = tid; i < n16; i += kFillThreads)
        img4[i] = make_uint4(0, 0, 0, 0);
    if (tid < kSlots)
        src_s[tid] = tid < nv ? (int64_t)plan.src[(size_t)blockIdx.x * kSlots + tid] : -1;
    __syncthreads();

    if (tier == 0 || tier == 3) {
        // keys: dims d, d+1 of a slot are adjacent in the row section
        for (int i = tid; i < kSlots * D / 2; i += kFillThreads) {
            const int t = i / (D / 2), d = 2 * (i % (D / 2));
            const int64_t e = src_s[t];
            if (e < 0)
                continue;
            uint32_t kk = *reinterpret_cast<const uint32_t *>(data.keys + e * D + d);
            if (tier == 3)
                kk = (uint32_t)f32_to_bf16(f16_bits_to_f32((uint16_t)(kk & 0xffff))) |
                     ((uint32_t)f32_to_bf16(f16_bits_to_f32((uint16_t)(kk >> 16))) << 16);
            *reinterpret_cast<uint32_t *>(img + row_off(t, d)) = kk;
            const uint32_t vv = *reinterpret_cast<const uint32_t *>(data.values + e * D + d);
            *reinterpret_cast<uint16_t *>(img + 32 * D + col_off(t, d)) = (uint16_t)(vv & 0xffff);
            *reinterpret_cast<uint16_t *>(img + 32 * D + col_off(t, d + 1)) = (uint16_t)(vv >> 16);
        }
    } else if (tier == 1) {
        for (int i = tid; i < kSlots * D / 2; i += kFillThreads) {
            const int t = i / (D / 2), d = 2 * (i % (D / 2));
            const int64_t e = src_s[t];
            if (e < 0)
                continue;
            const uint32_t vv = *reinterpret_cast<const uint32_t *>(data.values + e * D + d);
            *reinterpret_cast<uint16_t *>(img + col_off(t, d)) = (uint16_t)(vv & 0xffff);
            *reinterpret_cast<uint16_t *>(img + col_off(t, d + 1)) = (uint16_t)(vv >> 16);
        }
        for (int i = tid; i < kSlots * G; i += kFillThreads) {
            const int t = i / G, g = i % G;
            if (src_s[t] >= 0)
                img[codes_off(D, 1) + i] = data.codes8[src_s[t] * G + g];
        }
        if (tid < kSlots && src_s[tid] >= 0)
            *reinterpret_cast<uint16_t *>(img + radius_off(D, 1) + 2 * tid) = data.radius[src_s[tid]];
    } else {
        // int8 values with one fp16 scale: scale = fp16(fp32(max|v| / 127)),
        // q = clamp(rint(fp32(v / scale)), -127, 127), zero scale -> q = 0;
        // wave w quantizes slots w, w + 4, w + 8, w + 12
        for (int t = wave; t < kSlots; t += kFillThreads / 64) {
            const int64_t e = src_s[t];
            if (e < 0)
                continue;
            const uint16_t *vv = data.values + e * D;
            float amax = 0.f;
            for (int d = lane; d < D; d += 64)
                amax = fmaxf(amax, fabsf(bf16_bits_to_f32(vv[d])));
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1)
                amax = fmaxf(amax, __shfl_xor(amax, o, 64));
            const float s32 = amax / 127.0f;
            const uint16_t sh = f64_to_f16_sat((double)s32);
            const float sc = f16_bits_to_f32(sh);
            for (int d = lane; d < D; d += 64) {
                int q = 0;
                if (sc != 0.f) {
                    float y = rintf(bf16_bits_to_f32(vv[d]) / sc);
                    y = fminf(fmaxf(y, -127.f), 127.f);
                    q = (int)y;
                }
                img[col8_off(t, d)] = (uint8_t)(int8_t)q;
            }
            if (lane < G / 2)
                img[codes_off(D, 2) + t * (G / 2) + lane] = data.codes4[e * (G / 2) + lane];
            if (lane == 0) {
                *reinterpret_cast<uint16_t *>(img + radius_off(D, 2) + 2 * t) = data.radius[e];
                *reinterpret_cast<uint16_t *>(img + vscale_off(D) + 2 * t) = sh;
            }
        }
    }
    __syncthreads();
    uint4 *dst = reinterpret_cast<uint4 *>(cache.arena + (size_t)pg.off * kUnit);
    for (int i = tid; i < n16; i += kFillThreads)
        dst[i] = img4[i];
    const size_t slot = (size_t)pg.row * plan.maxp + pg.pi;
    if (tid == 0) {
        cache.page_table[slot] = pg.off;
        cache.page_meta[slot] = (uint8_t)pg.meta;
    }
    if (cache.slot_token != nullptr && tid < kSlots) {
        const int64_t e = src_s[tid];
        int32_t pos = -1;
        if (e >= 0) {
            const PackSeq sq = plan.seqs[pg.row / H];
            pos = (int32_t)(sq.pos_base + (e / H - sq.begin));
        }
        cache.slot_token[slot * kSlots + tid] = pos;
    }
}

} // namespace

hipError_t launch_pack(const PackPlan &plan, const PackData &data, const PackCache &cache,
                       hipStream_t st)
{
    const int rows = plan.S * plan.Hkv;
    if (rows > 0) {
        hipLaunchKernelGGL(pack_rows, dim3((rows + 255) / 256), dim3(256), 0, st, plan, cache);
        if (hipError_t e = hipGetLastError(); e != hipSuccess)
            return e;
    }
    if (plan.n_tokens > 0 && rows > 0) {
        hipLaunchKernelGGL(pack_rank, dim3(rows), dim3(1024), 0, st, plan, data);
        if (hipError_t e = hipGetLastError(); e != hipSuccess)
            return e;
    }
    if (plan.n_pages > 0) {
        hipLaunchKernelGGL(pack_fill, dim3(plan.n_pages), dim3(kFillThreads), 0, st, plan, data, cache);
        if (hipError_t e = hipGetLastError(); e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

} // namespace ada
