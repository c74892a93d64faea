/*
 * CPU oracle for the Angle-Domain Attention (ADA) decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark load this file's library.  The product path
 * (the HIP library under compressed_kv_attention_amd/) never calls it, and
 * the two share no code: no header, helper, table or constant.
 *
 * Plain, slow and single-threaded inside every unit of work.  Floating point
 * is carried in double except where an operation is defined at a stated
 * storage precision (fp16 radius, fp16 scale, fp32 division of the int8 value
 * quantiser); those spots say so.
 *
 * Sources (two web pages on one paper, arXiv 2605.18856):
 *   [TS]  gist.science, "SPHERICAL KV: Angle-Domain Attention and
 *         Rate-Distortion Retention ...", section "Technical Summary".
 *   [ABS] fugumt.com, the same paper's arXiv abstract.
 * The pages fix the shape of the method (a key becomes a scalar radius and
 * compact angle codes; logits come straight from the codes; tokens get a
 * keep/drop decision and a precision tier per token and head; retained tokens
 * sit in pages that hold one tier each).  They fix no encoding, bit width,
 * page layout or tie rule.  Each such choice below is stated where it is
 * made, as "Reading:".
 *
 * Parity pins: every exported function is pinned by a CPU test against a
 * closed form, an invariant or brute force (tests/test_oracle_*.py).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Number formats.                                                           */
/* ------------------------------------------------------------------------ */

/* IEEE binary16 -> double (exact). */
static double f16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int exp = (h >> 10) & 0x1f;
    int man = h & 0x3ff;
    double v;
    if (exp == 0)
        v = ldexp((double)man, -24); /* zero or subnormal */
    else if (exp == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(man + 1024), exp - 25);
    return sign ? -v : v;
}

/* bfloat16 -> double (exact): the upper half of an IEEE binary32. */
static double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* double -> binary16, round to nearest, ties to even.  Magnitudes that would
 * round to infinity saturate to the largest finite value 65504 (Reading: a
 * stored radius or scale is always finite).  NaN maps to the quiet NaN. */
static uint16_t double_to_f16_sat(double x)
{
    uint16_t sign = 0;
    if (isnan(x))
        return 0x7e00;
    if (x < 0 || (x == 0 && signbit(x))) {
        sign = 0x8000;
        x = -x;
    }
    if (x == 0)
        return sign;
    if (x >= 65520.0) /* rounds past 65504 */
        return sign | 0x7bff;
    if (x < ldexp(1.0, -14)) {
        /* subnormal range: units of 2^-24; 1024 units is the smallest normal */
        double m = nearbyint(ldexp(x, 24)); /* default rounding: ties to even */
        return sign | (uint16_t)m;
    }
    int e;
    frexp(x, &e); /* x = f * 2^e, f in [0.5, 1) */
    e -= 1;       /* x in [2^e, 2^(e+1)) */
    double m = nearbyint(ldexp(x, 10 - e)); /* in [1024, 2048] */
    if (m == 2048.0) {
        m = 1024.0;
        e += 1;
    }
    if (e > 15)
        return sign | 0x7bff;
    return sign | (uint16_t)(((e + 15) << 10) | ((int)m - 1024));
}

/* double -> bfloat16, round to nearest, ties to even (finite inputs). */
static uint16_t double_to_bf16(double x)
{
    float f = (float)x; /* exact for the values used (fp16 inputs) */
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lsb = (u >> 16) & 1;
    u += 0x7fff + lsb;
    return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------------ */
/* Page format.                                                              */
/*                                                                           */
/* Reading: [TS] 2.2 asks for pages whose items share one precision tier so */
/* that the decoder can stream them guided by a small header; [ABS] adds    */
/* that the metadata is small and the reads coalesced.  Nothing more is     */
/* given.  The format used here (the HIP library implements the same format */
/* from this description, in code of its own):                              */
/*                                                                           */
/* A page holds P = 16 slots of one (sequence, kv-head) row.  D is the head  */
/* dimension (64 or 128), G = D/8 code groups.  Sizes are padded to 128     */
/* bytes, the page-table unit.                                               */
/*   tier 0 (fp16 keys):   K fp16 "row" section | V bf16 "column" section    */
/*   tier 1 (8-bit codes): V bf16 column | codes u8 [16][G] | radius fp16 [16]*/
/*   tier 2 (4-bit codes): V int8 "column" | codes u8 [16][G/2] |            */
/*                         radius fp16 [16] | value scale fp16 [16]          */
/*   tier 3 (dense bf16, comparison path): K bf16 row | V bf16 column        */
/* Each section stores a 16 x D matrix (slot t, dim d) as 64 "lanes" of     */
/* 16-byte chunks, chunk c of all lanes forming the c-th KiB; the D dims   */
/* split into blocks b = d / 16 of 16 dims.                                 */
/*   row section (2-byte elements): slot t, dims 4q..4q+3 of a block are    */
/*     lane t + 16 q, 8 bytes per block: byte                                */
/*     (b/2)*1024 + (t + 16*((d%16)/4))*16 + (b%2)*8 + (d%4)*2               */
/*   column section (2-byte elements): dim n of a block, slots 4r..4r+3 are */
/*     lane n + 16 r, 8 bytes per block: byte                                */
/*     (b/2)*1024 + (d%16 + 16*(t/4))*16 + (b%2)*8 + (t%4)*2                 */
/*   int8 column section: the same lanes, 4 bytes per block: byte           */
/*     (b/4)*1024 + (d%16 + 16*(t/4))*16 + (b%4)*4 + t%4                     */
/* 4-bit codes: byte b of a slot holds group 2b in its low nibble and group  */
/* 2b+1 in its high nibble.  Slots past the page's valid count, and all      */
/* padding, are zero.  The page's metadata byte is tier | (n_valid-1) << 2.  */
/* ------------------------------------------------------------------------ */

enum { SLOTS = 16, UNIT = 128 };

static size_t row_off(int t, int d)
{
    int b = d / 16;
    return (size_t)(b / 2) * 1024 + (size_t)(t + 16 * ((d % 16) / 4)) * 16 + (size_t)(b % 2) * 8 +
           (size_t)(d % 4) * 2;
}

static size_t col_off(int t, int d)
{
    int b = d / 16;
    return (size_t)(b / 2) * 1024 + (size_t)(d % 16 + 16 * (t / 4)) * 16 + (size_t)(b % 2) * 8 +
           (size_t)(t % 4) * 2;
}

static size_t col8_off(int t, int d)
{
    int b = d / 16;
    return (size_t)(b / 4) * 1024 + (size_t)(d % 16 + 16 * (t / 4)) * 16 + (size_t)(b % 4) * 4 +
           (size_t)(t % 4);
}

static size_t pad_unit(size_t b) { return (b + UNIT - 1) / UNIT * UNIT; }

/* Byte size of one page of a tier. */
size_t oracle_page_bytes(int D, int tier)
{
    int G = D / 8;
    switch (tier) {
    case 0: return pad_unit((size_t)64 * D);
    case 1: return pad_unit((size_t)32 * D + (size_t)16 * G + 32);
    case 2: return pad_unit((size_t)16 * D + (size_t)8 * G + 64);
    case 3: return pad_unit((size_t)64 * D);
    default: return 0;
    }
}

/* Section offsets inside a page. */
static size_t off_codes(int D, int tier) { return tier == 1 ? (size_t)32 * D : (size_t)16 * D; }
static size_t off_radius(int D, int tier)
{
    int G = D / 8;
    return tier == 1 ? (size_t)32 * D + 16 * G : (size_t)16 * D + 8 * G;
}
static size_t off_vscale(int D) { return off_radius(D, 2) + 32; }
static size_t off_v(int D, int tier) { return (tier == 0 || tier == 3) ? (size_t)32 * D : 0; }

/* ------------------------------------------------------------------------ */
/* Encode.                                                                   */
/*                                                                           */
/* [TS] 2.1 "Spherical Parameterization": a key k becomes a scalar radius    */
/* r = ||k|| and a direction; "Compressed-Domain Similarity": the cache keeps */
/* a quantized radius and packed angular codes.  Reading of the codes: the   */
/* unit direction u = k / r is cut into G groups of 8 coordinates and each   */
/* group is replaced by the index of its nearest codeword (squared Euclidean */
/* distance, lowest index on ties) in a per-head codebook of 256 entries     */
/* (8-bit tier) and of 16 entries (4-bit tier).  Reading of the radius: the  */
/* norm of the fp16 key rounded once to fp16; u uses the unrounded norm;     */
/* a zero key has u = 0.                                                     */
/* ------------------------------------------------------------------------ */

typedef struct {
    int D, Hkv;
    const uint16_t *keys; /* [N][Hkv][D] fp16 */
    const float *cb8;     /* [Hkv][G][256][8] */
    const float *cb4;     /* [Hkv][G][16][8] */
    uint16_t *radius;     /* [N][Hkv] fp16 */
    uint8_t *codes8;      /* [N][Hkv][G] */
    uint8_t *codes4;      /* [N][Hkv][G/2] */
    double *dist8;        /* optional [N][Hkv][G][256] */
    double *dist4;        /* optional [N][Hkv][G][16] */
} encode_args;

static int nearest(const double *u8, const float *cb, int K, double *dist_out)
{
    int best = 0;
    double bestd = INFINITY;
    for (int c = 0; c < K; c++) {
        double d = 0;
        for (int j = 0; j < 8; j++) {
            double diff = u8[j] - (double)cb[c * 8 + j];
            d += diff * diff;
        }
        if (dist_out)
            dist_out[c] = d;
        if (d < bestd) {
            bestd = d;
            best = c;
        }
    }
    return best;
}

static void encode_one(const encode_args *a, int64_t i /* token*Hkv + head */)
{
    int D = a->D, G = D / 8, h = (int)(i % a->Hkv);
    const uint16_t *k = a->keys + i * D;
    double x[128], u[128];
    double ss = 0;
    for (int j = 0; j < D; j++) {
        x[j] = f16_to_double(k[j]);
        ss += x[j] * x[j];
    }
    double r = sqrt(ss);
    a->radius[i] = double_to_f16_sat(r);
    for (int j = 0; j < D; j++)
        u[j] = r > 0 ? x[j] / r : 0.0;
    for (int g = 0; g < G; g++) {
        const float *c8 = a->cb8 + ((size_t)h * G + g) * 256 * 8;
        const float *c4 = a->cb4 + ((size_t)h * G + g) * 16 * 8;
        double *d8 = a->dist8 ? a->dist8 + ((size_t)i * G + g) * 256 : NULL;
        double *d4 = a->dist4 ? a->dist4 + ((size_t)i * G + g) * 16 : NULL;
        a->codes8[i * G + g] = (uint8_t)nearest(u + 8 * g, c8, 256, d8);
        int c = nearest(u + 8 * g, c4, 16, d4);
        uint8_t *b = a->codes4 + i * (G / 2) + g / 2;
        if (g % 2 == 0)
            *b = (uint8_t)c;
        else
            *b = (uint8_t)(*b | (c << 4));
    }
}

typedef struct {
    const encode_args *a;
    int64_t begin, end;
} encode_job;

static void *encode_worker(void *p)
{
    encode_job *j = (encode_job *)p;
    for (int64_t i = j->begin; i < j->end; i++)
        encode_one(j->a, i);
    return NULL;
}

/* Encode n_tokens x Hkv keys.  dist8/dist4, when non-NULL, receive every
 * candidate's squared distance (for tests of the argmin).  nthreads > 1
 * splits independent (token, head) items across threads. */
int oracle_encode(int D, int Hkv, int64_t n_tokens, const uint16_t *keys, const float *cb8,
                  const float *cb4, uint16_t *radius, uint8_t *codes8, uint8_t *codes4,
                  double *dist8, double *dist4, int nthreads)
{
    if ((D != 64 && D != 128) || Hkv <= 0 || n_tokens < 0)
        return 1;
    encode_args a = {D, Hkv, keys, cb8, cb4, radius, codes8, codes4, dist8, dist4};
    int64_t n = n_tokens * Hkv;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    pthread_t th[256];
    encode_job jobs[256];
    for (int t = 0; t < nthreads; t++) {
        jobs[t].a = &a;
        jobs[t].begin = n * t / nthreads;
        jobs[t].end = n * (t + 1) / nthreads;
        if (nthreads == 1)
            encode_worker(&jobs[t]);
        else
            pthread_create(&th[t], NULL, encode_worker, &jobs[t]);
    }
    if (nthreads > 1)
        for (int t = 0; t < nthreads; t++)
            pthread_join(th[t], NULL);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Angular error of the stored codes (input of the RDR distortion surrogate). */
/*                                                                           */
/* [TS] 2.2 "Distortion Surrogate": the controller's proxy says the logit    */
/* error is dominated by the angular approximation error, scaled by the      */
/* query and key magnitudes.  Reading of the angular error of a tier: the   */
/* squared Euclidean distance between the unit direction u and its code      */
/* reconstruction (the chosen codeword of every group, concatenated),        */
/*     err = sum_g || u_g - C_g[code_g] ||^2,                                */
/* whose square root bounds |q . (u - u~)| / |q|.  u is formed exactly as in */
/* encode (double, sequential norm); each group's distance is summed over    */
/* its 8 coordinates in order and added to the total in group order, in      */
/* double; the total is rounded once to binary32.                            */
/* ------------------------------------------------------------------------ */

int oracle_code_error(int D, int Hkv, int64_t n_tokens, const uint16_t *keys, const float *cb8,
                      const float *cb4, const uint8_t *codes8, const uint8_t *codes4, float *err8,
                      float *err4)
{
    if ((D != 64 && D != 128) || Hkv <= 0 || n_tokens < 0)
        return 1;
    int G = D / 8;
    for (int64_t i = 0; i < n_tokens * Hkv; i++) {
        int h = (int)(i % Hkv);
        const uint16_t *k = keys + i * D;
        double x[128], u[128], ss = 0;
        for (int j = 0; j < D; j++) {
            x[j] = f16_to_double(k[j]);
            ss += x[j] * x[j];
        }
        double r = sqrt(ss);
        for (int j = 0; j < D; j++)
            u[j] = r > 0 ? x[j] / r : 0.0;
        double e8 = 0, e4 = 0;
        for (int g = 0; g < G; g++) {
            int c8 = codes8[i * G + g];
            int c4 = (codes4[i * (G / 2) + g / 2] >> (4 * (g % 2))) & 15;
            const float *w8 = cb8 + (((size_t)h * G + g) * 256 + c8) * 8;
            const float *w4 = cb4 + (((size_t)h * G + g) * 16 + c4) * 8;
            double d8 = 0, d4 = 0;
            for (int j = 0; j < 8; j++) {
                double a = u[8 * g + j] - (double)w8[j];
                double b = u[8 * g + j] - (double)w4[j];
                d8 += a * a;
                d4 += b * b;
            }
            e8 += d8;
            e4 += d4;
        }
        err8[i] = (float)e8;
        err4[i] = (float)e4;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* RDR budget solver.                                                        */
/*                                                                           */
/* [TS] 2.2 "Joint Optimization": for every token/head state i the          */
/* controller picks a residency bit z_i and a tier b_i by solving a discrete */
/* rate-distortion allocation under a fixed memory budget; "Distortion       */
/* Surrogate": the error proxy is the angular error scaled by the query and  */
/* key magnitudes; "Protection Constraints": protected states are kept at    */
/* the top tier.  [ABS]: retention and precision follow estimated future     */
/* utility, per token and head, under a fixed budget.  The pages give no     */
/* solver.  Readings used here:                                              */
/*   options of a state: tier 0 (fp16 key), 1 (8-bit codes), 2 (4-bit       */
/*     codes), 3 (dropped);                                                  */
/*   rate R_b: bytes one state takes in a full page of its tier (page bytes  */
/*     / 16), R_3 = 0;                                                       */
/*   distortion D_b = w * r~ * e_b with w the state's utility score, r~ its  */
/*     stored radius, e_0 = 0, e_1 = sqrt(err8), e_2 = sqrt(err4) (the chord */
/*     error of the code reconstruction, see above) and e_3 = 1 (a dropped   */
/*     key keeps none of its direction, as if u~ = 0).  The query magnitude */
/*     is the same unknown factor for every state and is left out;          */
/*   the budget is a cap per sequence on the bytes of all its rows' pages,   */
/*     so the solver keeps 15 slots of every tier per row in reserve for the */
/*     partial last pages: cap = budget - Hkv * 15 * (R_0 + R_1 + R_2);      */
/*   the allocation is the Lagrangian (convex-hull) solution of the          */
/*     multiple-choice knapsack: every state starts at tier 0, its lower     */
/*     convex hull in the (rate, distortion) plane gives a chain of          */
/*     demotions with increasing slopes (distortion added per byte saved),   */
/*     and demotions are taken in order of slope, all of the sequence's      */
/*     states together, until the rows fit under the cap.  Exactly: with     */
/*     need = (bytes at tier 0) - cap, s* is the smallest slope such that    */
/*     the demotions of slope <= s* save at least `need` bytes (+inf if none */
/*     does); every state takes the longest prefix of its chain whose        */
/*     slopes are <= s*.  need <= 0 keeps everything at tier 0.  Protected   */
/*     states have no demotions.                                             */
/* Arithmetic is binary32, in the order written (it decides integers, so     */
/* the HIP solver uses the same): wr = w * r~; D_1 = wr * sqrtf(err8);       */
/* D_2 = wr * sqrtf(err4); D_3 = wr; slope = (D_j - D_c) / (R_c - R_j) + 0;  */
/* the hull walk from the current point c takes the candidate j > c of least */
/* slope (the largest j on ties); a slope below its predecessor in the chain */
/* is raised to it, so chains are non-decreasing.                            */
/* ------------------------------------------------------------------------ */

enum { OR_EINVAL_SOLVE = 1 };

typedef struct {
    float slope;
    int32_t dr;
} rdr_step;

static int step_cmp(const void *pa, const void *pb)
{
    float a = ((const rdr_step *)pa)->slope, b = ((const rdr_step *)pb)->slope;
    return a < b ? -1 : (a > b ? 1 : 0);
}

/* Demotion chain of one state: up to 3 steps; returns their number and the
 * tier each one ends at. */
static int rdr_chain(const int32_t R[4], float w, uint16_t r_f16, float e8, float e4,
                     float slope[3], int32_t dr[3], int to[3])
{
    float wr = w * (float)f16_to_double(r_f16);
    float Dv[4] = {0.0f, wr * sqrtf(e8), wr * sqrtf(e4), wr};
    int c = 0, n = 0;
    float prev = -INFINITY;
    while (c < 3) {
        int best = -1;
        float bs = 0.0f;
        for (int j = c + 1; j < 4; j++) {
            float sl = (Dv[j] - Dv[c]) / (float)(R[c] - R[j]) + 0.0f;
            if (best < 0 || sl <= bs) {
                best = j;
                bs = sl;
            }
        }
        if (bs < prev)
            bs = prev;
        slope[n] = bs;
        dr[n] = R[c] - R[best];
        to[n] = best;
        prev = bs;
        n++;
        c = best;
    }
    return n;
}

int oracle_rdr_solve(int D, int Hkv, int S, const int32_t *cu_tokens, const int64_t *budget_bytes,
                     const uint16_t *radius, const float *err8, const float *err4,
                     const float *scores, const uint8_t *protect, uint8_t *tiers, float *threshold)
{
    if ((D != 64 && D != 128) || Hkv <= 0 || S < 0)
        return OR_EINVAL_SOLVE;
    int32_t R[4] = {(int32_t)(oracle_page_bytes(D, 0) / SLOTS), (int32_t)(oracle_page_bytes(D, 1) / SLOTS),
                    (int32_t)(oracle_page_bytes(D, 2) / SLOTS), 0};
    for (int s = 0; s < S; s++)
        if (cu_tokens[s + 1] < cu_tokens[s] || budget_bytes[s] < 0)
            return OR_EINVAL_SOLVE;
    for (int s = 0; s < S; s++) {
        int64_t b = cu_tokens[s], T = cu_tokens[s + 1] - cu_tokens[s];
        int64_t items = T * Hkv;
        int64_t cap = budget_bytes[s] - (int64_t)Hkv * 15 * (R[0] + R[1] + R[2]);
        int64_t need = items * R[0] - cap;
        for (int64_t i = 0; i < items; i++)
            tiers[b * Hkv + i] = 0;
        if (threshold)
            threshold[s] = need <= 0 ? -INFINITY : INFINITY;
        if (need <= 0)
            continue;
        /* every demotion of the sequence, sorted by slope */
        rdr_step *all = malloc((size_t)(3 * items + 1) * sizeof(rdr_step));
        int64_t n_all = 0;
        for (int64_t i = 0; i < items; i++) {
            int64_t e = b * Hkv + i;
            if (protect && protect[e])
                continue;
            float sl[3];
            int32_t dr[3];
            int to[3];
            int n = rdr_chain(R, scores[e], radius[e], err8[e], err4[e], sl, dr, to);
            for (int k = 0; k < n; k++) {
                all[n_all].slope = sl[k];
                all[n_all].dr = dr[k];
                n_all++;
            }
        }
        qsort(all, (size_t)n_all, sizeof(rdr_step), step_cmp);
        float sstar = INFINITY;
        int64_t cum = 0;
        for (int64_t k = 0; k < n_all; k++) {
            cum += all[k].dr;
            if (cum >= need) {
                sstar = all[k].slope;
                break;
            }
        }
        free(all);
        if (threshold)
            threshold[s] = sstar;
        for (int64_t i = 0; i < items; i++) {
            int64_t e = b * Hkv + i;
            if (protect && protect[e])
                continue;
            float sl[3];
            int32_t dr[3];
            int to[3];
            int n = rdr_chain(R, scores[e], radius[e], err8[e], err4[e], sl, dr, to);
            int t = 0;
            for (int k = 0; k < n && sl[k] <= sstar; k++)
                t = to[k];
            tiers[e] = (uint8_t)t;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Pack (RDR tiering into tier-homogeneous pages).                           */
/*                                                                           */
/* [TS] 2.2 "Joint Optimization": every token/head state gets a residency    */
/* bit z and a tier b; "Protection Constraints": a protected state is kept   */
/* at the top tier; "Tier-Homogeneous Pages": retained states are grouped    */
/* into pages that hold one tier each.  [ABS]: decisions are per token and   */
/* head.  The pages give no solver.  Reading used here: each sequence comes   */
/* with cumulative tier shares in basis points (fp16, +8-bit, +4-bit); the    */
/* token counts are n_cum = floor((bp * T + 5000) / 10000); in every         */
/* (sequence, kv-head) row the tokens are ranked by (protected first, higher  */
/* utility score first, lower index first); the first n_cum[0] go to fp16,   */
/* the next to 8-bit, then 4-bit, the rest are dropped.  Inside a tier the   */
/* tokens keep index order and fill 16-slot pages; each row gains its fp16   */
/* pages, then 8-bit, then 4-bit, after any pages it already had.  Pages of  */
/* one call are numbered (sequence, head, tier, page) and take arena space   */
/* by bump allocation in the order given by place_perm (identity if NULL).   */
/* ------------------------------------------------------------------------ */

typedef struct {
    const float *score;
    const uint8_t *prot;
    int64_t stride; /* Hkv */
} rank_ctx;

static rank_ctx g_rank; /* qsort has no context argument; pack is serial */

static int rank_cmp(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    int pa_ = g_rank.prot ? g_rank.prot[a * g_rank.stride] : 0;
    int pb_ = g_rank.prot ? g_rank.prot[b * g_rank.stride] : 0;
    if (pa_ != pb_)
        return pa_ > pb_ ? -1 : 1;
    float sa = g_rank.score[a * g_rank.stride], sb = g_rank.score[b * g_rank.stride];
    if (sa != sb)
        return sa > sb ? -1 : 1;
    return a < b ? -1 : (a > b ? 1 : 0);
}

static int idx_cmp(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return a < b ? -1 : (a > b ? 1 : 0);
}

/* int8 value quantiser for the 4-bit tier.  Reading: one scale per (token,
 * head): amax = max |v|; scale = fp16(fp32(amax / 127)), saturating;
 * q = clamp(rint_even(fp32(v / scale)), -127, 127); a zero scale gives q = 0.
 * Carried out in binary32 as written (fp32 division, correctly rounded). */
static void quant_v(int D, const uint16_t *v, int8_t *q, uint16_t *scale_out)
{
    float amax = 0.0f;
    for (int d = 0; d < D; d++) {
        float x = (float)bf16_to_double(v[d]);
        float ax = fabsf(x);
        if (ax > amax)
            amax = ax;
    }
    float s32 = amax / 127.0f;
    uint16_t sh = double_to_f16_sat((double)s32);
    float s = (float)f16_to_double(sh);
    *scale_out = sh;
    for (int d = 0; d < D; d++) {
        if (s == 0.0f) {
            q[d] = 0;
            continue;
        }
        float x = (float)bf16_to_double(v[d]);
        float y = rintf(x / s);
        if (y > 127.0f)
            y = 127.0f;
        if (y < -127.0f)
            y = -127.0f;
        q[d] = (int8_t)y;
    }
}

/* Tier token counts for one sequence of T tokens: n_cum[0..2] cumulative. */
void oracle_tier_counts(int64_t T, const int32_t *bp, int64_t *n_cum)
{
    for (int i = 0; i < 3; i++)
        n_cum[i] = (bp[i] * T + 5000) / 10000;
}

/* Write one token's fields into slot t of a page. */
static void put_slot(int D, int tier, uint8_t *page, int t, const uint16_t *k, const uint16_t *v,
                     uint16_t r, const uint8_t *c8, const uint8_t *c4)
{
    int G = D / 8;
    if (tier == 0 || tier == 3) {
        for (int d = 0; d < D; d++) {
            uint16_t kv = k[d];
            if (tier == 3)
                kv = double_to_bf16(f16_to_double(k[d]));
            memcpy(page + row_off(t, d), &kv, 2);
        }
    }
    if (tier == 0 || tier == 1 || tier == 3) {
        size_t base = off_v(D, tier);
        for (int d = 0; d < D; d++)
            memcpy(page + base + col_off(t, d), &v[d], 2);
    }
    if (tier == 1) {
        memcpy(page + off_codes(D, 1) + (size_t)t * G, c8, (size_t)G);
        memcpy(page + off_radius(D, 1) + (size_t)t * 2, &r, 2);
    }
    if (tier == 2) {
        int8_t q[128];
        uint16_t sc;
        quant_v(D, v, q, &sc);
        for (int d = 0; d < D; d++)
            page[col8_off(t, d)] = (uint8_t)q[d];
        memcpy(page + off_codes(D, 2) + (size_t)t * (G / 2), c4, (size_t)(G / 2));
        memcpy(page + off_radius(D, 2) + (size_t)t * 2, &r, 2);
        memcpy(page + off_vscale(D) + (size_t)t * 2, &sc, 2);
    }
}

/* Return codes shared by pack and dense_pack. */
enum { OR_OK = 0, OR_EINVAL = 1, OR_ENOSPACE = 3 };

/*
 * Pack one call's tokens into the cache.
 *   cu_tokens[S+1]    token ranges of each sequence in the flat arrays
 *   tier_cum_bp[S][3] cumulative basis points (fp16, +8-bit, +4-bit)
 *   keys/values [N][Hkv][D] (fp16 / bf16), radius [N][Hkv], codes8 [N][Hkv][G],
 *   codes4 [N][Hkv][G/2], scores [N][Hkv] (f32), protect [N][Hkv] or NULL,
 *   place_perm [pages of this call] or NULL, pos_base [S] or NULL.
 *   arena / arena_units / cursor (in/out, 128-byte units); page_table and
 *   page_meta [S*Hkv][maxp]; num_pages [S*Hkv]; tier_tokens [S*Hkv][3];
 *   slot_token [S*Hkv][maxp][16] or NULL.
 * tiers [N][Hkv] (0-2 kept tier, any other value dropped), when non-NULL, replaces the
 * ranking: each row's tokens of a tier keep index order (tier_cum_bp, scores
 * and protect are then unused).
 * dense != 0 packs every token of the call into tier-3 pages instead.
 */
static int pack_impl(int D, int Hkv, int S, const int32_t *cu_tokens, const int32_t *tier_cum_bp,
                     const uint8_t *tiers, const uint16_t *keys, const uint16_t *values, const uint16_t *radius,
                     const uint8_t *codes8, const uint8_t *codes4, const float *scores,
                     const uint8_t *protect, const uint32_t *place_perm, const int64_t *pos_base,
                     uint8_t *arena, uint64_t arena_units, uint64_t *cursor, uint32_t *page_table,
                     uint8_t *page_meta, int32_t *num_pages, int32_t *tier_tokens,
                     int32_t *slot_token, int maxp, int dense)
{
    int G = D / 8;
    if ((D != 64 && D != 128) || Hkv <= 0 || S < 0 || maxp < 0)
        return OR_EINVAL;
    /* Per (sequence, head, tier): the token list of the tier in index order. */
    int64_t rows = (int64_t)S * Hkv;
    int64_t n_logical = 0;
    int32_t **lists = calloc((size_t)rows * 3 + 1, sizeof(int32_t *));
    int64_t *counts = calloc((size_t)rows * 3 + 1, sizeof(int64_t));
    int rc = OR_OK;
    for (int s = 0; s < S && rc == OR_OK; s++) {
        int64_t b = cu_tokens[s], T = cu_tokens[s + 1] - cu_tokens[s];
        if (T < 0) {
            rc = OR_EINVAL;
            break;
        }
        int64_t n_cum[3];
        if (dense) { /* every token, index order, one list */
            n_cum[0] = n_cum[1] = n_cum[2] = T;
        } else if (tiers) { /* given tiers: sort tokens by (tier, index) */
            n_cum[0] = n_cum[1] = n_cum[2] = 0;
        } else {
            const int32_t *bp = tier_cum_bp + 3 * s;
            if (bp[0] < 0 || bp[0] > bp[1] || bp[1] > bp[2] || bp[2] > 10000) {
                rc = OR_EINVAL;
                break;
            }
            oracle_tier_counts(T, bp, n_cum);
        }
        for (int h = 0; h < Hkv; h++) {
            int32_t *order = malloc((size_t)(T > 0 ? T : 1) * sizeof(int32_t));
            for (int64_t i = 0; i < T; i++)
                order[i] = (int32_t)i;
            if (!dense && tiers) {
                int64_t at = 0, cnt[4] = {0, 0, 0, 0};
                /* Reading: a state carries a residency bit and, when it is
                 * resident, a tier (technical summary, section 2.2); a value
                 * other than the kept tiers 0-2 means not resident, like 3 */
                for (int64_t i = 0; i < T; i++) {
                    int t = tiers[(b + i) * Hkv + h];
                    cnt[t < 3 ? t : 3]++;
                }
                for (int tier = 0; tier < 4; tier++)
                    for (int64_t i = 0; i < T; i++) {
                        int t = tiers[(b + i) * Hkv + h];
                        if ((t < 3 ? t : 3) == tier)
                            order[at++] = (int32_t)i;
                    }
                n_cum[0] = cnt[0];
                n_cum[1] = cnt[0] + cnt[1];
                n_cum[2] = cnt[0] + cnt[1] + cnt[2];
            } else if (!dense) {
                g_rank.score = scores + b * Hkv + h;
                g_rank.prot = protect ? protect + b * Hkv + h : NULL;
                g_rank.stride = Hkv;
                qsort(order, (size_t)T, sizeof(int32_t), rank_cmp);
                if (protect) {
                    int64_t np = 0;
                    for (int64_t i = 0; i < T; i++)
                        np += protect[(b + i) * Hkv + h] != 0;
                    if (np > n_cum[0])
                        rc = OR_EINVAL;
                }
            }
            int64_t lo = 0;
            for (int tier = 0; tier < 3; tier++) {
                int64_t hi = n_cum[tier];
                int64_t n = hi - lo;
                int32_t *lst = malloc((size_t)(n > 0 ? n : 1) * sizeof(int32_t));
                memcpy(lst, order + lo, (size_t)n * sizeof(int32_t));
                qsort(lst, (size_t)n, sizeof(int32_t), idx_cmp);
                int64_t r = (int64_t)s * Hkv + h;
                lists[r * 3 + tier] = lst;
                counts[r * 3 + tier] = n;
                n_logical += (n + SLOTS - 1) / SLOTS;
                lo = hi;
            }
            free(order);
        }
    }
    /* Logical page descriptors in (s, h, tier, page) order. */
    int64_t *lp_row = malloc((size_t)(n_logical + 1) * sizeof(int64_t));
    int *lp_tier = malloc((size_t)(n_logical + 1) * sizeof(int));
    int64_t *lp_first = malloc((size_t)(n_logical + 1) * sizeof(int64_t)); /* first slot in tier list */
    int64_t *lp_index = malloc((size_t)(n_logical + 1) * sizeof(int64_t)); /* page index in row */
    int *lp_list = malloc((size_t)(n_logical + 1) * sizeof(int)); /* which tier list feeds it */
    uint64_t *lp_off = malloc((size_t)(n_logical + 1) * sizeof(uint64_t));
    if (rc == OR_OK) {
        int64_t k = 0;
        for (int64_t r = 0; r < rows && rc == OR_OK; r++) {
            int64_t pi = num_pages[r];
            for (int tier = 0; tier < 3; tier++) {
                int64_t n = counts[r * 3 + tier];
                for (int64_t f = 0; f < n; f += SLOTS) {
                    lp_row[k] = r;
                    lp_tier[k] = dense ? 3 : tier;
                    lp_list[k] = tier;
                    lp_first[k] = f;
                    lp_index[k] = pi++;
                    k++;
                }
            }
            if (pi > maxp)
                rc = OR_EINVAL;
        }
    }
    /* Bump allocation in placement order. */
    if (rc == OR_OK) {
        uint64_t cur = *cursor;
        char *seen = calloc((size_t)(n_logical + 1), 1);
        for (int64_t k = 0; k < n_logical; k++) {
            int64_t p = place_perm ? (int64_t)place_perm[k] : k;
            if (p < 0 || p >= n_logical || seen[p]) {
                rc = OR_EINVAL;
                break;
            }
            seen[p] = 1;
            lp_off[p] = cur;
            cur += oracle_page_bytes(D, lp_tier[p]) / UNIT;
        }
        free(seen);
        if (rc == OR_OK && cur > arena_units)
            rc = OR_ENOSPACE;
        if (rc == OR_OK && cur > 0xffffffffull)
            rc = OR_ENOSPACE;
        if (rc == OR_OK)
            *cursor = cur;
    }
    /* Fill pages and tables. */
    if (rc == OR_OK) {
        for (int64_t k = 0; k < n_logical; k++) {
            int64_t r = lp_row[k];
            int s = (int)(r / Hkv), h = (int)(r % Hkv), tier = lp_tier[k];
            int64_t b = cu_tokens[s];
            const int32_t *lst = lists[r * 3 + lp_list[k]];
            int64_t n = counts[r * 3 + lp_list[k]];
            size_t bytes = oracle_page_bytes(D, tier);
            uint8_t *page = arena + lp_off[k] * UNIT;
            memset(page, 0, bytes);
            int nv = (int)((n - lp_first[k]) < SLOTS ? (n - lp_first[k]) : SLOTS);
            for (int t = 0; t < nv; t++) {
                int64_t idx = lst[lp_first[k] + t];
                int64_t e = (b + idx) * Hkv + h;
                put_slot(D, tier, page, t, keys + e * D, values + e * D, radius ? radius[e] : 0,
                         codes8 ? codes8 + e * G : NULL, codes4 ? codes4 + e * (G / 2) : NULL);
            }
            int64_t pi = lp_index[k];
            page_table[r * maxp + pi] = (uint32_t)lp_off[k];
            page_meta[r * maxp + pi] = (uint8_t)(tier | ((nv - 1) << 2));
            if (slot_token) {
                int64_t pb = pos_base ? pos_base[s] : 0;
                for (int t = 0; t < SLOTS; t++)
                    slot_token[(r * maxp + pi) * SLOTS + t] =
                        t < nv ? (int32_t)(pb + lst[lp_first[k] + t]) : -1;
            }
        }
        for (int64_t r = 0; r < rows; r++) {
            for (int tier = 0; tier < 3; tier++) {
                int64_t n = counts[r * 3 + tier];
                num_pages[r] += (int32_t)((n + SLOTS - 1) / SLOTS);
                if (!dense && tier_tokens)
                    tier_tokens[r * 3 + tier] += (int32_t)n;
            }
        }
    }
    for (int64_t r = 0; r < rows * 3; r++)
        free(lists[r]);
    free(lists);
    free(counts);
    free(lp_row);
    free(lp_tier);
    free(lp_first);
    free(lp_index);
    free(lp_list);
    free(lp_off);
    return rc;
}

int oracle_pack(int D, int Hkv, int S, const int32_t *cu_tokens, const int32_t *tier_cum_bp,
                const uint16_t *keys, const uint16_t *values, const uint16_t *radius,
                const uint8_t *codes8, const uint8_t *codes4, const float *scores,
                const uint8_t *protect, const uint32_t *place_perm, const int64_t *pos_base,
                uint8_t *arena, uint64_t arena_units, uint64_t *cursor, uint32_t *page_table,
                uint8_t *page_meta, int32_t *num_pages, int32_t *tier_tokens, int32_t *slot_token,
                int maxp)
{
    return pack_impl(D, Hkv, S, cu_tokens, tier_cum_bp, NULL, keys, values, radius, codes8, codes4,
                     scores, protect, place_perm, pos_base, arena, arena_units, cursor, page_table,
                     page_meta, num_pages, tier_tokens, slot_token, maxp, 0);
}

/* Pack with the tier of every (token, head) given (e.g. by the solver). */
int oracle_pack_tiers(int D, int Hkv, int S, const int32_t *cu_tokens, const uint8_t *tiers,
                      const uint16_t *keys, const uint16_t *values, const uint16_t *radius,
                      const uint8_t *codes8, const uint8_t *codes4, const uint32_t *place_perm,
                      const int64_t *pos_base, uint8_t *arena, uint64_t arena_units,
                      uint64_t *cursor, uint32_t *page_table, uint8_t *page_meta,
                      int32_t *num_pages, int32_t *tier_tokens, int32_t *slot_token, int maxp)
{
    if (tiers == NULL)
        return OR_EINVAL;
    return pack_impl(D, Hkv, S, cu_tokens, NULL, tiers, keys, values, radius, codes8, codes4, NULL,
                     NULL, place_perm, pos_base, arena, arena_units, cursor, page_table, page_meta,
                     num_pages, tier_tokens, slot_token, maxp, 0);
}

/* ------------------------------------------------------------------------ */
/* Decode-step append.                                                       */
/*                                                                           */
/* [TS] 2.3: the pipeline maps dense keys to spherical codes, applies RDR to */
/* filter and tier them, and stores the result; [TS] 2.2: retained states    */
/* sit in tier-homogeneous pages.  Reading for the decode loop, where each   */
/* step brings one new token per sequence: its key is encoded as in encode  */
/* (the code errors are the chosen codewords' distances, summed as in        */
/* code_error), its tier follows from the solver's chain rule with the       */
/* sequence's slope threshold s* of the last solve (the online continuation */
/* of the same Lagrangian allocation; protected states take tier 0), and a  */
/* kept state goes into the next free slot of its row's open page of that    */
/* tier.  A row without an open page of the tier, or whose open page is      */
/* full, takes a new page: the row's next page-table index, arena space by   */
/* bump allocation, all bytes zero before the slot is written.  open_page    */
/* [rows][3] holds each row's open page index + 1 (0: none).  Rows are       */
/* visited in (sequence, head) order.  A row whose page table is full sets   */
/* status bit 1 and one that finds no arena space sets bit 2; its token is   */
/* not stored.                                                              */
/* ------------------------------------------------------------------------ */

static int nearest_dist(const double *u8, const float *cb, int K, double *bestd)
{
    int best = 0;
    double bd = INFINITY;
    for (int c = 0; c < K; c++) {
        double d = 0;
        for (int j = 0; j < 8; j++) {
            double diff = u8[j] - (double)cb[c * 8 + j];
            d += diff * diff;
        }
        if (d < bd) {
            bd = d;
            best = c;
        }
    }
    *bestd = bd;
    return best;
}

int oracle_append(int D, int Hkv, int S, const uint16_t *keys, const uint16_t *values, const float *scores,
                  const uint8_t *protect, const float *cb8, const float *cb4, const float *threshold,
                  const int64_t *pos, uint8_t *arena, uint64_t arena_units, uint64_t *cursor,
                  uint32_t *page_table, uint8_t *page_meta, int32_t *num_pages, int32_t *tier_tokens,
                  int32_t *slot_token, int maxp, int32_t *open_page, uint8_t *tiers_out, int32_t *status)
{
    if ((D != 64 && D != 128) || Hkv <= 0 || S < 0)
        return OR_EINVAL;
    int G = D / 8;
    int32_t R[4] = {(int32_t)(oracle_page_bytes(D, 0) / SLOTS), (int32_t)(oracle_page_bytes(D, 1) / SLOTS),
                    (int32_t)(oracle_page_bytes(D, 2) / SLOTS), 0};
    for (int64_t row = 0; row < (int64_t)S * Hkv; row++) {
        int s = (int)(row / Hkv), h = (int)(row % Hkv);
        const uint16_t *k = keys + row * D;
        const uint16_t *v = values + row * D;
        /* encode */
        double x[128], u[128], ss = 0;
        for (int j = 0; j < D; j++) {
            x[j] = f16_to_double(k[j]);
            ss += x[j] * x[j];
        }
        double r = sqrt(ss);
        uint16_t rb = double_to_f16_sat(r);
        for (int j = 0; j < D; j++)
            u[j] = r > 0 ? x[j] / r : 0.0;
        uint8_t c8[16], c4[8];
        double e8 = 0, e4 = 0;
        for (int g = 0; g < G; g++) {
            double d8, d4;
            c8[g] = (uint8_t)nearest_dist(u + 8 * g, cb8 + ((size_t)h * G + g) * 256 * 8, 256, &d8);
            int q4 = nearest_dist(u + 8 * g, cb4 + ((size_t)h * G + g) * 16 * 8, 16, &d4);
            if (g % 2 == 0)
                c4[g / 2] = (uint8_t)q4;
            else
                c4[g / 2] = (uint8_t)(c4[g / 2] | (q4 << 4));
            e8 += d8;
            e4 += d4;
        }
        /* tier */
        int tier = 0;
        if (!(protect && protect[row])) {
            float sl[3];
            int32_t dr[3];
            int to[3];
            int n = rdr_chain(R, scores[row], rb, (float)e8, (float)e4, sl, dr, to);
            for (int q = 0; q < n && sl[q] <= threshold[s]; q++)
                tier = to[q];
        }
        tiers_out[row] = (uint8_t)tier;
        if (tier == 3)
            continue;
        /* place */
        int32_t pi = open_page[row * 3 + tier] - 1, slot = SLOTS;
        if (pi >= 0)
            slot = ((page_meta[row * maxp + pi] >> 2) & 15) + 1;
        if (slot == SLOTS) {
            pi = num_pages[row];
            uint64_t units = oracle_page_bytes(D, tier) / UNIT;
            if (pi >= maxp) {
                *status |= 1;
                continue;
            }
            if (*cursor + units > arena_units) {
                *status |= 2;
                continue;
            }
            page_table[row * maxp + pi] = (uint32_t)*cursor;
            memset(arena + *cursor * UNIT, 0, oracle_page_bytes(D, tier));
            *cursor += units;
            num_pages[row] = pi + 1;
            open_page[row * 3 + tier] = pi + 1;
            slot = 0;
            if (slot_token)
                for (int t = 0; t < SLOTS; t++)
                    slot_token[((int64_t)row * maxp + pi) * SLOTS + t] = -1;
        }
        uint8_t *page = arena + (size_t)page_table[row * maxp + pi] * UNIT;
        put_slot(D, tier, page, slot, k, v, rb, c8, c4);
        page_meta[row * maxp + pi] = (uint8_t)(tier | (slot << 2));
        tier_tokens[row * 3 + tier] += 1;
        if (slot_token)
            slot_token[((int64_t)row * maxp + pi) * SLOTS + slot] = (int32_t)pos[s];
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Re-tiering as T grows.                                                    */
/*                                                                           */
/* [TS] 2.2: states are kept and tiered under a strict memory budget, in     */
/* tier-homogeneous pages.  As decode steps append states, a sequence's      */
/* pages outgrow its budget; re-tiering brings it back.  Readings:           */
/*   mechanics -- a full or partial fp16 page can be demoted in place to an  */
/*   8-bit or 4-bit page: its keys are encoded from the page's own fp16 keys  */
/*   exactly as encode does, its values kept (8-bit) or quantised (4-bit),    */
/*   the result written to new arena space and the page-table entry pointed  */
/*   at it (same index, same slots, same slot positions); any page can be    */
/*   evicted: per row, in descending page index, the row's last page moves   */
/*   into the evicted page's place.  Demotions run before evictions.  An     */
/*   entry that cannot apply -- a row outside the cache, a page not in use, a */
/*   demotion of a page that is not fp16, an eviction of a tier-3 page (the   */
/*   dense comparison format, which has no per-tier count), or a target      */
/*   other than 1-3 -- sets status bit 4 and is skipped; no arena space sets */
/*   bit 2.                                                                   */
/*   policy -- stored pages keep no utility scores, so age stands in for     */
/*   utility: while a sequence's page bytes exceed its budget, its oldest    */
/*   full fp16 page (lowest page index, then lowest head) is demoted to the  */
/*   given tier; when none is left, its oldest coded page is evicted; then   */
/*   its oldest remaining fp16 page.                                         */
/* ------------------------------------------------------------------------ */

static void read_key_value(int D, const uint8_t *page, int t, uint16_t *k, uint16_t *v)
{
    for (int d = 0; d < D; d++) {
        memcpy(&k[d], page + row_off(t, d), 2);
        memcpy(&v[d], page + off_v(D, 0) + col_off(t, d), 2);
    }
}

int oracle_retier(int D, int Hkv, int S, int n, const int32_t *rows, const int32_t *pages,
                  const uint8_t *target, const float *cb8, const float *cb4, uint8_t *arena,
                  uint64_t arena_units, uint64_t *cursor, uint32_t *page_table, uint8_t *page_meta,
                  int32_t *num_pages, int32_t *tier_tokens, int32_t *slot_token, int maxp,
                  int32_t *open_page, int32_t *status)
{
    if ((D != 64 && D != 128) || Hkv <= 0 || S < 0 || n < 0)
        return OR_EINVAL;
    int G = D / 8;
    int64_t nrows = (int64_t)S * Hkv;
    /* entries that can never apply */
    for (int i = 0; i < n; i++)
        if (target[i] < 1 || target[i] > 3 || rows[i] < 0 || rows[i] >= nrows)
            *status |= 4;
    /* demotions, in list order */
    for (int i = 0; i < n; i++) {
        if (target[i] != 1 && target[i] != 2)
            continue;
        int32_t row = rows[i], p = pages[i];
        int tier = target[i], h = row % Hkv;
        if (row < 0 || row >= nrows)
            continue;
        if (p < 0 || p >= num_pages[row] || (page_meta[(int64_t)row * maxp + p] & 3) != 0) {
            *status |= 4;
            continue;
        }
        uint64_t units = oracle_page_bytes(D, tier) / UNIT;
        if (*cursor + units > arena_units) {
            *status |= 2;
            continue;
        }
        int nv = ((page_meta[(int64_t)row * maxp + p] >> 2) & 15) + 1;
        const uint8_t *old = arena + (size_t)page_table[(int64_t)row * maxp + p] * UNIT;
        uint8_t *pg = arena + *cursor * UNIT;
        memset(pg, 0, oracle_page_bytes(D, tier));
        for (int t = 0; t < nv; t++) {
            uint16_t k[128], v[128], r;
            uint8_t c8[16], c4[8];
            read_key_value(D, old, t, k, v);
            encode_args a = {D, 1, k, cb8 + (size_t)h * G * 256 * 8, cb4 + (size_t)h * G * 16 * 8,
                             &r, c8, c4, NULL, NULL};
            encode_one(&a, 0);
            put_slot(D, tier, pg, t, k, v, r, c8, c4);
        }
        page_table[(int64_t)row * maxp + p] = (uint32_t)*cursor;
        *cursor += units;
        page_meta[(int64_t)row * maxp + p] = (uint8_t)(tier | ((nv - 1) << 2));
        tier_tokens[row * 3 + 0] -= nv;
        tier_tokens[row * 3 + tier] += nv;
        if (open_page[row * 3 + 0] == p + 1)
            open_page[row * 3 + 0] = 0;
    }
    /* evictions: each row's, in descending page index */
    int32_t *ev = malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    for (int i = 0; i < n; i++) {
        if (target[i] != 3)
            continue;
        int32_t row = rows[i];
        if (row < 0 || row >= nrows)
            continue;
        int seen = 0;
        for (int j = 0; j < i; j++)
            seen |= target[j] == 3 && rows[j] == row;
        if (seen)
            continue; /* the row's evictions were done with its first entry */
        int m = 0;
        for (int j = i; j < n; j++)
            if (target[j] == 3 && rows[j] == row)
                ev[m++] = pages[j];
        for (int a = 1; a < m; a++) /* descending */
            for (int b = a; b > 0 && ev[b] > ev[b - 1]; b--) {
                int32_t t = ev[b];
                ev[b] = ev[b - 1];
                ev[b - 1] = t;
            }
        for (int a = 0; a < m; a++) {
            int32_t p = ev[a], last = num_pages[row] - 1;
            if (p < 0 || p > last) {
                *status |= 4;
                continue;
            }
            uint8_t meta = page_meta[(int64_t)row * maxp + p];
            if ((meta & 3) == 3) { /* a dense comparison page: no tier count */
                *status |= 4;
                continue;
            }
            tier_tokens[row * 3 + (meta & 3)] -= ((meta >> 2) & 15) + 1;
            for (int t = 0; t < 3; t++)
                if (open_page[row * 3 + t] == p + 1)
                    open_page[row * 3 + t] = 0;
            if (p != last) {
                page_table[(int64_t)row * maxp + p] = page_table[(int64_t)row * maxp + last];
                page_meta[(int64_t)row * maxp + p] = page_meta[(int64_t)row * maxp + last];
                if (slot_token)
                    for (int t = 0; t < SLOTS; t++)
                        slot_token[((int64_t)row * maxp + p) * SLOTS + t] =
                            slot_token[((int64_t)row * maxp + last) * SLOTS + t];
                for (int t = 0; t < 3; t++)
                    if (open_page[row * 3 + t] == last + 1)
                        open_page[row * 3 + t] = p + 1;
            }
            num_pages[row] = last;
        }
    }
    free(ev);
    return OR_OK;
}

/* The re-tiering policy: the (row, page, target) list, at most cap entries;
 * returns the number of entries. */
int oracle_retier_plan(int D, int Hkv, int S, const int64_t *budget_bytes, const int32_t *num_pages,
                       const uint8_t *page_meta, int maxp, int demote_to, int cap, int32_t *rows,
                       int32_t *pages, uint8_t *target)
{
    int n = 0;
    for (int s = 0; s < S; s++) {
        int64_t bytes = 0;
        int maxn = 0;
        for (int h = 0; h < Hkv; h++) {
            int row = s * Hkv + h;
            for (int p = 0; p < num_pages[row]; p++)
                bytes += (int64_t)oracle_page_bytes(D, page_meta[(int64_t)row * maxp + p] & 3);
            if (num_pages[row] > maxn)
                maxn = num_pages[row];
        }
        /* three sweeps over (page index, head): full fp16 pages demoted,
         * coded pages evicted, remaining fp16 pages evicted */
        for (int sweep = 0; sweep < 3; sweep++)
            for (int p = 0; p < maxn && bytes > budget_bytes[s]; p++)
                for (int h = 0; h < Hkv && bytes > budget_bytes[s]; h++) {
                    int row = s * Hkv + h;
                    if (p >= num_pages[row])
                        continue;
                    uint8_t meta = page_meta[(int64_t)row * maxp + p];
                    int tier = meta & 3, full = ((meta >> 2) & 15) == 15;
                    int32_t tgt = -1;
                    if (sweep == 0 && tier == 0 && full)
                        tgt = demote_to;
                    if (sweep == 1 && (tier == 1 || tier == 2))
                        tgt = 3;
                    /* (pages demoted by this plan are not evicted by it; a
                     * later call sees them as coded) */
                    if (sweep == 2 && tier == 0 && !full)
                        tgt = 3;
                    if (tgt < 0)
                        continue;
                    if (n >= cap)
                        return n;
                    rows[n] = row;
                    pages[n] = p;
                    target[n] = (uint8_t)tgt;
                    n++;
                    if (tgt == 3)
                        bytes -= (int64_t)oracle_page_bytes(D, tier);
                    else
                        bytes -= (int64_t)oracle_page_bytes(D, 0) - (int64_t)oracle_page_bytes(D, tgt);
                }
    }
    return n;
}

/* Dense comparison cache: every token of the call, in index order, in tier-3
 * pages (K converted fp16 -> bf16 with round-to-nearest-even, V bf16). */
int oracle_dense_pack(int D, int Hkv, int S, const int32_t *cu_tokens, const uint16_t *keys,
                      const uint16_t *values, const uint32_t *place_perm, uint8_t *arena,
                      uint64_t arena_units, uint64_t *cursor, uint32_t *page_table,
                      uint8_t *page_meta, int32_t *num_pages, int maxp)
{
    return pack_impl(D, Hkv, S, cu_tokens, NULL, NULL, keys, values, NULL, NULL, NULL, NULL, NULL,
                     place_perm, NULL, arena, arena_units, cursor, page_table, page_meta,
                     num_pages, NULL, NULL, maxp, 1);
}

/* ------------------------------------------------------------------------ */
/* Decode.                                                                   */
/*                                                                           */
/* [TS] 2.1 "Compressed-Domain Similarity": the logit is computed from the   */
/* codes as |q| * r~ * f_b(codes), f_b a cosine computed from the codes.     */
/* With the encoding above that is                                          */
/*     l(t) = sigma * r~_t * sum_g  q_g . C_g[code_{t,g}]                     */
/*          = sigma * |q| * r~_t * (q/|q|) . u^(t),                           */
/* u^ the concatenation of the chosen codewords, sigma the softmax scale.    */
/* It is evaluated here through a per-(head, group) table                   */
/* LUT_g[c] = q_g . C_g[c] as the formula groups it, and, separately, with   */
/* the key direction rebuilt in full (logits_explicit) so tests can hold the */
/* two against each other.  fp16-tier (and dense bf16) slots use the plain   */
/* dot product sigma * q . k.  Attention over the retained slots is the      */
/* ordinary softmax: out = sum_t e^(l_t - m) v^_t / sum_t e^(l_t - m),       */
/* lse = m + ln sum_t e^(l_t - m), m = max_t l_t.  Dropped tokens are absent */
/* from both sums.  A row with no retained slot gives out = 0, lse = -inf.   */
/* v^ is the stored bf16 value, or int8 * scale in the 4-bit tier.           */
/* Reading: no causal mask (decode attends to every cached token);          */
/* q-head hq reads kv-head hq / (Hq / Hkv).                                 */
/*                                                                           */
/* Symmetric variant.  [TS] 2.1 writes f_b(c_q, c_k): a cosine computed from */
/* the angular codes of both the query and the key.  Reading: the query's    */
/* unit direction u_q = q / |q| (|q| summed sequentially over D, in double)  */
/* takes, per group and per codebook, the index of its nearest codeword      */
/* exactly as a key does in encode, and                                     */
/*     l(t) = sigma * |q| * r~_t * sum_g C_g[cq_g] . C_g[code_{t,g}],         */
/* with the 8-bit codebook for 8-bit keys and the 4-bit codebook for 4-bit   */
/* keys.  As a table, LUT_g[c] = |q| C_g[cq_g] . C_g[c]: the asymmetric      */
/* table with q_g replaced by |q| C_g[cq_g].  fp16-tier keys keep sigma q.k. */
/* ------------------------------------------------------------------------ */

typedef struct {
    int D, Hq, Hkv, S, maxp;
    const uint8_t *arena;
    const uint32_t *page_table;
    const uint8_t *page_meta;
    const int32_t *num_pages;
    const float *cb8, *cb4;
    const uint16_t *q; /* [S][Hq][D] bf16 */
    double sigma;
    double *out;             /* [S][Hq][D] */
    double *lse;             /* [S][Hq] */
    double *logits;          /* [S][Hq][maxp*16] or NULL */
    double *logits_explicit; /* same, or NULL */
    int sym;                 /* symmetric (query codes) variant for coded keys */
} decode_args;

/* Query codes of the symmetric variant: per group, the nearest codeword of
 * u_q = q / |q| in the 8-bit and the 4-bit codebook; returns |q|. */
static double query_codes(int D, const double *q, const float *cb8, const float *cb4, int *cq8, int *cq4)
{
    int G = D / 8;
    double ss = 0, u[128];
    for (int j = 0; j < D; j++)
        ss += q[j] * q[j];
    double qn = sqrt(ss);
    for (int j = 0; j < D; j++)
        u[j] = qn > 0 ? q[j] / qn : 0.0;
    for (int g = 0; g < G; g++) {
        cq8[g] = nearest(u + 8 * g, cb8 + (size_t)g * 256 * 8, 256, NULL);
        cq4[g] = nearest(u + 8 * g, cb4 + (size_t)g * 16 * 8, 16, NULL);
    }
    return qn;
}

static void decode_unit(const decode_args *a, int64_t unit)
{
    int D = a->D, G = D / 8, s = (int)(unit / a->Hq), hq = (int)(unit % a->Hq);
    int hkv = hq / (a->Hq / a->Hkv);
    int64_t row = (int64_t)s * a->Hkv + hkv;
    double q[128];
    for (int j = 0; j < D; j++)
        q[j] = bf16_to_double(a->q[((int64_t)s * a->Hq + hq) * D + j]);
    /* The query the coded tiers see: q itself, or in the symmetric variant
     * |q| times the codeword reconstruction of its direction (one per
     * codebook). */
    double q8[128], q4[128];
    for (int j = 0; j < D; j++)
        q8[j] = q4[j] = q[j];
    if (a->sym) {
        int cq8[16], cq4[16];
        const float *c8h = a->cb8 + (size_t)hkv * G * 256 * 8, *c4h = a->cb4 + (size_t)hkv * G * 16 * 8;
        double qn = query_codes(D, q, c8h, c4h, cq8, cq4);
        for (int g = 0; g < G; g++)
            for (int j = 0; j < 8; j++) {
                q8[8 * g + j] = qn * (double)c8h[((size_t)g * 256 + cq8[g]) * 8 + j];
                q4[8 * g + j] = qn * (double)c4h[((size_t)g * 16 + cq4[g]) * 8 + j];
            }
    }
    /* Per-group tables LUT_g[c] = q_g . C_g[c]: 256 entries (8-bit), 16 (4-bit). */
    double *lut8 = malloc(sizeof(double) * (size_t)G * 256);
    double *lut4 = malloc(sizeof(double) * (size_t)G * 16);
    for (int g = 0; g < G; g++) {
        for (int c = 0; c < 256; c++) {
            const float *w = a->cb8 + (((size_t)hkv * G + g) * 256 + c) * 8;
            double acc = 0;
            for (int j = 0; j < 8; j++)
                acc += q8[8 * g + j] * (double)w[j];
            lut8[g * 256 + c] = acc;
        }
        for (int c = 0; c < 16; c++) {
            const float *w = a->cb4 + (((size_t)hkv * G + g) * 16 + c) * 8;
            double acc = 0;
            for (int j = 0; j < 8; j++)
                acc += q4[8 * g + j] * (double)w[j];
            lut4[g * 16 + c] = acc;
        }
    }
    int np = a->num_pages[row];
    int64_t nslots = (int64_t)np * SLOTS;
    double *lg = malloc(sizeof(double) * (size_t)(nslots > 0 ? nslots : 1));
    double *vv = malloc(sizeof(double) * (size_t)(nslots > 0 ? nslots : 1) * D);
    char *valid = calloc((size_t)(nslots > 0 ? nslots : 1), 1);
    for (int p = 0; p < np; p++) {
        const uint8_t *page = a->arena + (size_t)a->page_table[row * a->maxp + p] * UNIT;
        uint8_t meta = a->page_meta[row * a->maxp + p];
        int tier = meta & 3, nv = ((meta >> 2) & 15) + 1;
        for (int t = 0; t < nv; t++) {
            int64_t slot = (int64_t)p * SLOTS + t;
            double l = 0, lx = 0;
            if (tier == 0 || tier == 3) {
                for (int d = 0; d < D; d++) {
                    uint16_t kb;
                    memcpy(&kb, page + row_off(t, d), 2);
                    l += q[d] * (tier == 0 ? f16_to_double(kb) : bf16_to_double(kb));
                }
                l *= a->sigma;
                lx = l;
            } else {
                uint16_t rb;
                memcpy(&rb, page + off_radius(D, tier) + (size_t)t * 2, 2);
                double r = f16_to_double(rb);
                const uint8_t *cd = page + off_codes(D, tier);
                double sum = 0, dot = 0;
                for (int g = 0; g < G; g++) {
                    int c;
                    const float *w;
                    if (tier == 1) {
                        c = cd[t * G + g];
                        sum += lut8[g * 256 + c];
                        w = a->cb8 + (((size_t)hkv * G + g) * 256 + c) * 8;
                    } else {
                        uint8_t byte = cd[t * (G / 2) + g / 2];
                        c = g % 2 == 0 ? (byte & 15) : (byte >> 4);
                        sum += lut4[g * 16 + c];
                        w = a->cb4 + (((size_t)hkv * G + g) * 16 + c) * 8;
                    }
                    /* explicit form: rebuild the coded direction, then dot */
                    const double *qq = tier == 1 ? q8 : q4;
                    for (int j = 0; j < 8; j++)
                        dot += qq[8 * g + j] * (double)w[j];
                }
                l = a->sigma * r * sum;
                lx = a->sigma * r * dot;
            }
            lg[slot] = l;
            valid[slot] = 1;
            if (a->logits)
                a->logits[((int64_t)s * a->Hq + hq) * a->maxp * SLOTS + slot] = l;
            if (a->logits_explicit)
                a->logits_explicit[((int64_t)s * a->Hq + hq) * a->maxp * SLOTS + slot] = lx;
            double *v = vv + slot * D;
            if (tier == 2) {
                uint16_t sb;
                memcpy(&sb, page + off_vscale(D) + (size_t)t * 2, 2);
                double sc = f16_to_double(sb);
                for (int d = 0; d < D; d++)
                    v[d] = (double)(int8_t)page[col8_off(t, d)] * sc;
            } else {
                for (int d = 0; d < D; d++) {
                    uint16_t vb;
                    memcpy(&vb, page + off_v(D, tier) + col_off(t, d), 2);
                    v[d] = bf16_to_double(vb);
                }
            }
        }
    }
    double m = -INFINITY;
    for (int64_t i = 0; i < nslots; i++)
        if (valid[i] && lg[i] > m)
            m = lg[i];
    double *o = a->out + ((int64_t)s * a->Hq + hq) * D;
    for (int d = 0; d < D; d++)
        o[d] = 0;
    if (m == -INFINITY) {
        a->lse[(int64_t)s * a->Hq + hq] = -INFINITY;
    } else {
        double l = 0;
        for (int64_t i = 0; i < nslots; i++) {
            if (!valid[i])
                continue;
            double w = exp(lg[i] - m);
            l += w;
            for (int d = 0; d < D; d++)
                o[d] += w * vv[i * D + d];
        }
        for (int d = 0; d < D; d++)
            o[d] /= l;
        a->lse[(int64_t)s * a->Hq + hq] = m + log(l);
    }
    free(lg);
    free(vv);
    free(valid);
    free(lut8);
    free(lut4);
}

typedef struct {
    const decode_args *a;
    int64_t begin, end;
} decode_job;

static void *decode_worker(void *p)
{
    decode_job *j = (decode_job *)p;
    for (int64_t u = j->begin; u < j->end; u++)
        decode_unit(j->a, u);
    return NULL;
}

/* One decode step over a cache view.  units_begin/units_end select a range
 * of (sequence, q-head) units, s * Hq + hq (for bounded samples); the rest
 * of out/lse is left untouched.  nthreads > 1 runs independent units on
 * separate threads.  Returns 0, or 1 on bad geometry. */
static int decode_impl(int D, int Hq, int Hkv, int S, int maxp, const uint8_t *arena,
                       const uint32_t *page_table, const uint8_t *page_meta, const int32_t *num_pages,
                       const float *cb8, const float *cb4, const uint16_t *q, double sigma, double *out,
                       double *lse, double *logits, double *logits_explicit, int64_t units_begin,
                       int64_t units_end, int nthreads, int sym)
{
    if ((D != 64 && D != 128) || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || S < 0)
        return 1;
    decode_args a = {D, Hq, Hkv, S, maxp, arena, page_table, page_meta, num_pages, cb8, cb4,
                     q, sigma, out, lse, logits, logits_explicit, sym};
    int64_t n = units_end - units_begin;
    if (n <= 0)
        return 0;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if (nthreads > n)
        nthreads = (int)n;
    pthread_t th[256];
    decode_job jobs[256];
    for (int t = 0; t < nthreads; t++) {
        jobs[t].a = &a;
        jobs[t].begin = units_begin + n * t / nthreads;
        jobs[t].end = units_begin + n * (t + 1) / nthreads;
        if (nthreads == 1)
            decode_worker(&jobs[t]);
        else
            pthread_create(&th[t], NULL, decode_worker, &jobs[t]);
    }
    if (nthreads > 1)
        for (int t = 0; t < nthreads; t++)
            pthread_join(th[t], NULL);
    return 0;
}

int oracle_decode(int D, int Hq, int Hkv, int S, int maxp, const uint8_t *arena,
                  const uint32_t *page_table, const uint8_t *page_meta, const int32_t *num_pages,
                  const float *cb8, const float *cb4, const uint16_t *q, double sigma, double *out,
                  double *lse, double *logits, double *logits_explicit, int64_t units_begin,
                  int64_t units_end, int nthreads)
{
    return decode_impl(D, Hq, Hkv, S, maxp, arena, page_table, page_meta, num_pages, cb8, cb4, q, sigma,
                       out, lse, logits, logits_explicit, units_begin, units_end, nthreads, 0);
}

/* The symmetric variant (query codes); arguments as oracle_decode. */
int oracle_decode_sym(int D, int Hq, int Hkv, int S, int maxp, const uint8_t *arena,
                      const uint32_t *page_table, const uint8_t *page_meta, const int32_t *num_pages,
                      const float *cb8, const float *cb4, const uint16_t *q, double sigma, double *out,
                      double *lse, double *logits, double *logits_explicit, int64_t units_begin,
                      int64_t units_end, int nthreads)
{
    return decode_impl(D, Hq, Hkv, S, maxp, arena, page_table, page_meta, num_pages, cb8, cb4, q, sigma,
                       out, lse, logits, logits_explicit, units_begin, units_end, nthreads, 1);
}

/* Query codes of the symmetric variant for every (sequence, q-head):
 * qc8, qc4 [S][Hq][G]; qnorm [S][Hq]. */
int oracle_query_codes(int D, int Hq, int Hkv, int S, const uint16_t *qbits, const float *cb8,
                       const float *cb4, int32_t *qc8, int32_t *qc4, double *qnorm)
{
    if ((D != 64 && D != 128) || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || S < 0)
        return 1;
    int G = D / 8;
    for (int64_t u = 0; u < (int64_t)S * Hq; u++) {
        int hkv = (int)(u % Hq) / (Hq / Hkv);
        double q[128];
        int c8[16], c4[16];
        for (int j = 0; j < D; j++)
            q[j] = bf16_to_double(qbits[u * D + j]);
        qnorm[u] = query_codes(D, q, cb8 + (size_t)hkv * G * 256 * 8, cb4 + (size_t)hkv * G * 16 * 8, c8, c4);
        for (int g = 0; g < G; g++) {
            qc8[u * G + g] = c8[g];
            qc4[u * G + g] = c4[g];
        }
    }
    return 0;
}

/* Textbook attention of one query over an explicit token set:
 * out = softmax(sigma * q K^T) V, lse = log-sum-exp of the logits.
 * q[D], K[n][D], V[n][D] in double.  n = 0 gives out = 0, lse = -inf. */
void oracle_dense_attention(int D, int64_t n, const double *q, const double *K, const double *V,
                            double sigma, double *out, double *lse)
{
    double m = -INFINITY;
    double *l = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; i++) {
        double acc = 0;
        for (int d = 0; d < D; d++)
            acc += q[d] * K[i * D + d];
        l[i] = sigma * acc;
        if (l[i] > m)
            m = l[i];
    }
    for (int d = 0; d < D; d++)
        out[d] = 0;
    if (n == 0) {
        *lse = -INFINITY;
        free(l);
        return;
    }
    double z = 0;
    for (int64_t i = 0; i < n; i++) {
        double w = exp(l[i] - m);
        z += w;
        for (int d = 0; d < D; d++)
            out[d] += w * V[i * D + d];
    }
    for (int d = 0; d < D; d++)
        out[d] /= z;
    *lse = m + log(z);
    free(l);
}

/* Exposed number-format helpers, for the tests that pin them. */
double oracle_f16_to_double(uint16_t h) { return f16_to_double(h); }
uint16_t oracle_double_to_f16(double x) { return double_to_f16_sat(x); }
double oracle_bf16_to_double(uint16_t b) { return bf16_to_double(b); }
uint16_t oracle_double_to_bf16(double x) { return double_to_bf16(x); }
void oracle_quant_v(int D, const uint16_t *v, int8_t *q, uint16_t *scale)
{
    quant_v(D, v, q, scale);
}
size_t oracle_row_off(int t, int d) { return row_off(t, d); }
size_t oracle_col_off(int t, int d) { return col_off(t, d); }
size_t oracle_col8_off(int t, int d) { return col8_off(t, d); }
