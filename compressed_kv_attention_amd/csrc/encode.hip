// ADA encode for gfx950: scalar radius + per-group nearest-codeword codes.
//
// SPHERICAL KV (arXiv 2605.18856), gist.science technical summary, section
// 2.1 "Spherical Parameterization" (radius and direction of each key) and
// "Compressed-Domain Similarity" (quantized radius, packed angular codes),
// section 2.3 (dense keys are mapped to codes before tiering).  The angle
// code is one codebook index per group of 8 direction coordinates.
//
// Precision: the norm, the direction and every candidate distance are
// evaluated in double, in a fixed order with no fused multiply-add, so the
// result is the exact argmin of the defined distances (ties -> lowest index).
// The norm is summed sequentially over the D coordinates.
//
// Grid: x = blocks of 256 tokens, y = (kv-head, pair of groups).  The block
// stages the two groups' codebooks (2 x 272 codewords) in LDS; every thread
// takes one token, so all lanes read the same codeword at a time (LDS
// broadcast).  The thread writes both groups' 8-bit codes and the byte that
// packs their two 4-bit codes; pair 0 also writes the radius.
#include "ada_internal.h"
#include "numfmt.h"

namespace ada {
namespace {

#pragma clang fp contract(off)

template <int D>
__global__ __launch_bounds__(256) void encode_kernel(int Hkv, int64_t n_tokens, const uint16_t *keys,
                                                     const float *cb8, const float *cb4,
                                                     uint16_t *radius, uint8_t *codes8,
                                                     uint8_t *codes4)
{
    constexpr int G = D / 8;
    __shared__ float c8[2][kCodes8][8];
    __shared__ float c4[2][kCodes4][8];
    const int h = blockIdx.y / (G / 2), gp = blockIdx.y % (G / 2);
    for (int i = threadIdx.x; i < 2 * kCodes8 * 8; i += 256) {
        const int g = i / (kCodes8 * 8), rest = i % (kCodes8 * 8);
        (&c8[g][0][0])[rest] = cb8[(((size_t)h * G + 2 * gp + g) * kCodes8) * 8 + rest];
    }
    for (int i = threadIdx.x; i < 2 * kCodes4 * 8; i += 256) {
        const int g = i / (kCodes4 * 8), rest = i % (kCodes4 * 8);
        (&c4[g][0][0])[rest] = cb4[(((size_t)h * G + 2 * gp + g) * kCodes4) * 8 + rest];
    }
    __syncthreads();
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (n >= n_tokens)
        return;
    const size_t e = (size_t)n * Hkv + h;
    const uint16_t *k = keys + e * D;

    double ss = 0.0;
    for (int c = 0; c < D / 8; c++) {
        const uint4 w = *reinterpret_cast<const uint4 *>(k + 8 * c);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const double lo = (double)f16_bits_to_f32((uint16_t)(ws[q] & 0xffff));
            const double hi = (double)f16_bits_to_f32((uint16_t)(ws[q] >> 16));
            ss = ss + lo * lo;
            ss = ss + hi * hi;
        }
    }
    const double r = sqrt(ss);
    if (gp == 0)
        radius[e] = f64_to_f16_sat(r);

    int best8[2], best4[2];
#pragma unroll
    for (int g = 0; g < 2; g++) {
        double u[8];
        const uint4 w = *reinterpret_cast<const uint4 *>(k + 8 * (2 * gp + g));
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const double lo = (double)f16_bits_to_f32((uint16_t)(ws[q] & 0xffff));
            const double hi = (double)f16_bits_to_f32((uint16_t)(ws[q] >> 16));
            u[2 * q] = r > 0.0 ? lo / r : 0.0;
            u[2 * q + 1] = r > 0.0 ? hi / r : 0.0;
        }
        int b = 0;
        double bd = INFINITY;
        for (int c = 0; c < kCodes8; c++) {
            double d = 0.0;
#pragma unroll
            for (int q = 0; q < 8; q++) {
                const double df = u[q] - (double)c8[g][c][q];
                d = d + df * df;
            }
            if (d < bd) {
                bd = d;
                b = c;
            }
        }
        best8[g] = b;
        b = 0;
        bd = INFINITY;
        for (int c = 0; c < kCodes4; c++) {
            double d = 0.0;
#pragma unroll
            for (int q = 0; q < 8; q++) {
                const double df = u[q] - (double)c4[g][c][q];
                d = d + df * df;
            }
            if (d < bd) {
                bd = d;
                b = c;
            }
        }
        best4[g] = b;
    }
    *reinterpret_cast<uint16_t *>(codes8 + e * G + 2 * gp) = (uint16_t)(best8[0] | (best8[1] << 8));
    codes4[e * (G / 2) + gp] = (uint8_t)(best4[0] | (best4[1] << 4));
}

} // namespace

hipError_t launch_encode(int D, int Hkv, int64_t n_tokens, const uint16_t *keys, const float *cb8,
                         const float *cb4, uint16_t *radius, uint8_t *codes8, uint8_t *codes4,
                         hipStream_t st)
{
    if (n_tokens == 0)
        return hipSuccess;
    const dim3 grid((unsigned)((n_tokens + 255) / 256), (unsigned)(Hkv * (D / 16)));
    if (D == 128)
        hipLaunchKernelGGL(encode_kernel<128>, grid, dim3(256), 0, st, Hkv, n_tokens, keys, cb8,
                           cb4, radius, codes8, codes4);
    else if (D == 64)
        hipLaunchKernelGGL(encode_kernel<64>, grid, dim3(256), 0, st, Hkv, n_tokens, keys, cb8, cb4,
                           radius, codes8, codes4);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

} // namespace ada
