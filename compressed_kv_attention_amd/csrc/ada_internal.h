// Internal interface between the host entry points (ada_abi.cpp) and the
// gfx950 kernels (decode.hip, encode.hip, pack.hip, rdr.hip, append.hip).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ada {

constexpr int kSlots = 16;      // slots per page
constexpr int kUnit = 128;      // page-table unit, bytes
constexpr int kCodes8 = 256;    // codewords per group, 8-bit tier
constexpr int kCodes4 = 16;     // codewords per group, 4-bit tier
constexpr int kLutCodes = kCodes8 + kCodes4;

// Byte layout of one page (see include/ada.h for the format).
struct PageLayout {
    int bytes[4];
    int codes_off[3];   // per tier; -1 where absent
    int radius_off[3];
    int vscale_off;     // tier 2
    int v_off[4];       // V section per tier
};

__host__ __device__ constexpr int pad_unit(int b) { return (b + kUnit - 1) / kUnit * kUnit; }
__host__ __device__ constexpr int page_bytes(int D, int tier)
{
    return tier == 0 || tier == 3 ? pad_unit(64 * D)
         : tier == 1              ? pad_unit(32 * D + 2 * D + 32)
         : tier == 2              ? pad_unit(16 * D + D + 64)
                                  : 0;
}
__host__ __device__ constexpr int codes_off(int D, int tier) { return tier == 1 ? 32 * D : 16 * D; }
__host__ __device__ constexpr int radius_off(int D, int tier)
{
    return tier == 1 ? 32 * D + 2 * D : 16 * D + D;
}
__host__ __device__ constexpr int vscale_off(int D) { return 16 * D + D + 32; }
__host__ __device__ constexpr int v_off(int D, int tier) { return tier == 0 || tier == 3 ? 32 * D : 0; }

struct DecodeArgs {
    const uint8_t *arena;
    const uint32_t *page_table;
    const uint8_t *page_meta;
    const int32_t *num_pages;
    const float *cb8;
    const float *cb4;
    const uint16_t *q;
    float *out;
    float *lse;
    float *logits;
    float *part_ml;    // [rows][nsplit][NH][2]  (running max in log2 units, sum)
    float *part_acc;   // [rows][nsplit][NH][D]  (unnormalised output)
    float *glut;       // [rows][LUT floats]: symmetric variant's tabulated LUT, else null
    unsigned long long *trace; // [blocks][waves][8] phase timestamps (tracing builds), else null
    float sigma;
    int S, Hq, Hkv, maxp, nsplit;
};

// Decode stages: the page stream, and the split merge (only with more than
// one split).
enum : unsigned { kStageStream = 2, kStageMerge = 4, kStageAll = 6 };
hipError_t launch_decode(int D, int NH, bool dense, const DecodeArgs &a, hipStream_t st,
                         unsigned stages = kStageAll, bool sym = false);
// Floats of one row's LUT (the symmetric variant keeps every row's in the
// workspace).
size_t decode_lut_floats(int D, int NH);
// Waves per workgroup of the page-stream kernel.
int decode_waves(int D, int NH);

// Device address, on the current device, of the library-owned array that
// holds ada_decode_noalloc's split partials (kNoAllocScratchBytes).
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
hipError_t noalloc_scratch(void **ptr);

// LDS bytes the page-stream workgroup needs; the device offers 160 KiB.
size_t decode_shmem_bytes(int D, int NH, bool dense, int nsplit, int maxp);
constexpr size_t kMaxLds = 160 * 1024;

hipError_t launch_encode(int D, int Hkv, int64_t n_tokens, const uint16_t *keys, const float *cb8,
                         const float *cb4, uint16_t *radius, uint8_t *codes8, uint8_t *codes4,
                         hipStream_t st);

// ---- RDR: code error and budget solver ------------------------------------
hipError_t launch_code_error(int D, int Hkv, int64_t n_tokens, const uint16_t *keys, const float *cb8,
                             const float *cb4, const uint8_t *codes8, const uint8_t *codes4,
                             float *err8, float *err4, hipStream_t st);

struct SolveSeq {
    int64_t begin;   // first flat item (token * Hkv + head) of the sequence
    int64_t n_items; // tokens * Hkv
    int64_t need;    // bytes the demotions must save; <= 0: every state stays at tier 0
};
struct SolveBlock {
    int32_t seq;
    int32_t pad;
    int64_t first;   // first flat item of the block (kSolveItems items, cut at the sequence's end)
};
constexpr int kSolveThreads = 256;
constexpr int kSolveItems = 4 * kSolveThreads;
constexpr int kSolvePasses = 4; // 8-bit digits of the 32-bit slope key
struct SolveArgs {
    const SolveSeq *seqs;
    const SolveBlock *blocks;
    unsigned long long *hist; // [kSolvePasses][S][256]: bytes saved per key digit
    const uint16_t *radius;
    const float *err8, *err4, *scores;
    const uint8_t *protect;   // or null
    uint8_t *tiers;
    float *threshold;         // [S] slope threshold s* out, or null
    int S, D, n_blocks;
};
hipError_t launch_solve(const SolveArgs &a, hipStream_t st);
hipError_t launch_tier_counts(int Hkv, int S, const int32_t *cu_dev, const uint8_t *tiers,
                              int32_t *counts, hipStream_t st);

// ---- decode-step append ----------------------------------------------------
struct AppendArgs {
    uint8_t *arena;
    uint32_t *page_table;
    uint8_t *page_meta;
    int32_t *num_pages;
    int32_t *tier_tokens;
    int32_t *slot_token;        // or null
    const float *cb8, *cb4;
    const uint16_t *keys, *values; // [S][Hkv][D]
    const float *scores;        // [S][Hkv]
    const uint8_t *protect;     // [S][Hkv] or null
    const float *threshold;     // [S]
    const int64_t *pos;         // [S]
    uint8_t *tiers_out;         // [S][Hkv] or null
    unsigned long long *cursor; // arena cursor, 128-byte units
    unsigned int *status;       // sticky bits: 1 page table full, 2 arena full
    int32_t *open;              // [rows][3] open page index + 1
    unsigned long long capacity;
    int maxp, Hkv;
};
hipError_t launch_append(int D, const AppendArgs &a, int rows, hipStream_t st);

struct RetierArgs {
    uint8_t *arena;
    uint32_t *page_table;
    uint8_t *page_meta;
    int32_t *num_pages;
    int32_t *tier_tokens;
    int32_t *slot_token;        // or null
    const float *cb8, *cb4;
    const int32_t *rows, *pages; // [n]
    const uint8_t *target;       // [n]: 1, 2 demote to that tier; 3 evict
    unsigned long long *cursor;
    unsigned int *status;        // adds bit 4: a listed page could not be re-tiered
    int32_t *open;
    unsigned long long capacity;
    int n, maxp, Hkv, nrows;
};
hipError_t launch_retier(int D, const RetierArgs &a, int rows, hipStream_t st);

// ---- pack ----------------------------------------------------------------
// Host-built plan of one pack call, copied into the workspace.  The page
// list is built on the host only for a given placement order; in arena
// order (the default) the row kernel writes it from the rows' entries.
struct PackSeq {
    int32_t begin;     // first flat token of the sequence in this call
    int32_t len;       // T_s
    int32_t n_cum[3];  // cumulative tier counts
    int32_t pad;
    int64_t pos_base;  // position recorded in slot_token for index 0
};
struct PackRow {
    int32_t lp_first[3]; // logical index of the row's first page of each tier
    int32_t count[3];    // tokens per tier
    int32_t pi0;         // the row's page count before this call
    uint32_t off[3];     // arena offset of the row's first page of each tier (arena order)
};
struct PackPage {
    uint32_t off;        // arena offset, 128-byte units
    int32_t row;
    int32_t pi;          // page index inside the row
    int32_t meta;        // tier | (valid - 1) << 2
};
struct PackPlan {
    const PackSeq *seqs;
    const PackRow *rows;
    PackPage *pages;        // written by pack_rank when gen_pages is set
    const uint8_t *protect; // [N][Hkv] or null
    const uint8_t *tiers;   // [N][Hkv] given tiers (0-2 kept, other values dropped) or null
    int32_t *src;           // [n_pages][16]: flat (token, head) index a slot holds, or -1
    int S, Hkv, D, maxp, n_pages, dense, gen_pages;
    int64_t n_tokens;
    // Device-side page planning (dev_plan): each row counts its given tiers,
    // takes its pages' arena space from the bump cursor and its page
    // indices from num_pages itself.  Row r's pages then sit at plan.pages
    // [rows[r].lp_first[0] ...), a range the host sized for the row's
    // tokens; unused entries there get meta = -1.
    int dev_plan;
    unsigned long long *cursor; // arena cursor, 128-byte units
    unsigned int *status;       // sticky bits: 1 a row's page table full, 2 arena full
    unsigned long long capacity;
};
struct PackData {
    const uint16_t *keys, *values, *radius;
    const uint8_t *codes8, *codes4;
    const float *scores;
};
struct PackCache {
    uint8_t *arena;
    uint32_t *page_table;
    uint8_t *page_meta;
    int32_t *num_pages;
    int32_t *tier_tokens;
    int32_t *slot_token;
};

hipError_t launch_pack(const PackPlan &plan, const PackData &data, const PackCache &cache,
                       hipStream_t st);

} // namespace ada
