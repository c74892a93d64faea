/*
 * libada -- C ABI of the Angle-Domain Attention (ADA) decode path for
 * MI355X (gfx950).
 *
 * Method sources (arXiv 2605.18856, "SPHERICAL KV: Angle-Domain Attention and
 * Rate-Distortion Retention for Efficient Long-Context Inference"):
 *   [TS]  the gist.science technical summary of the paper, sections 2.1-2.3;
 *   [ABS] the paper's abstract as shown on fugumt.com.
 *
 * Conventions for every entry point:
 *   - Pointers named *_host are host memory.  All other data pointers are
 *     device memory (HIP device allocations or views into them).
 *   - The caller owns every buffer.  The library allocates nothing, frees
 *     nothing and keeps no pointer after a call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Device work is enqueued on it and the call returns; results are ready
 *     once the caller synchronises that stream.  The library never
 *     synchronises the device.
 *   - Argument, shape and capacity errors are found on the host before any
 *     device work is enqueued and leave every buffer and every *_host
 *     in/out value unchanged.  A failed launch returns ADA_EHIP.  A device
 *     fault surfaces at the caller's next synchronisation.
 *   - Nothing throws across the ABI.  Calls keep no hidden state and may be
 *     made from several host threads (on different data).
 *   - fp16 is IEEE binary16, bf16 is bfloat16; both are passed as uint16_t.
 *
 * Page format (a reading: [TS] 2.2 asks for tier-homogeneous pages read in
 * one pass guided by a small header, [ABS] for small metadata and coalesced
 * reads; nothing else is given).  A page holds 16 slots of one
 * (sequence, kv-head) row, all of one tier.  D = head_dim, G = D / 8 code
 * groups.  Page sizes are multiples of 128 bytes, the unit of the page table.
 *   tier 0  fp16 keys:    K fp16 row | V bf16 column              64*D bytes
 *   tier 1  8-bit codes:  V bf16 column | codes u8 [16][G] | radius fp16 [16]
 *   tier 2  4-bit codes:  V int8 column | codes u8 [16][G/2] | radius fp16 [16]
 *                         | value scale fp16 [16]
 *   tier 3  dense bf16 (comparison cache): K bf16 row | V bf16 column
 * A section holds a 16 x D matrix (slot t, dim d) as 64 lanes of 16-byte
 * chunks, chunk c of all 64 lanes forming the c-th KiB of the section; the
 * dims split into blocks b = d / 16 of 16.  These are the operand layouts of
 * a 16x16x16 matrix-core product:
 *   row (2-byte):     byte (b/2)*1024 + (t + 16*((d%16)/4))*16 + (b%2)*8 + (d%4)*2
 *   column (2-byte):  byte (b/2)*1024 + (d%16 + 16*(t/4))*16 + (b%2)*8 + (t%4)*2
 *   column (int8):    byte (b/4)*1024 + (d%16 + 16*(t/4))*16 + (b%4)*4 + t%4
 * A 4-bit code byte holds group 2b in its low nibble, group 2b+1 in its
 * high nibble.  Unused slots and padding are zero.  page_meta byte:
 * tier | (valid_slots - 1) << 2.  For D = 128 the sizes are 8192 / 4480 /
 * 2304 / 8192 bytes; for D = 64, 4096 / 2304 / 1152 / 4096.
 */
#ifndef ADA_H
#define ADA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ADA_OK = 0,
    ADA_EINVAL = 1,       /* bad argument, shape or value */
    ADA_EUNSUPPORTED = 2, /* valid but not built (head_dim, GQA ratio) */
    ADA_ENOSPACE = 3,     /* arena too small for the pages of a pack call */
    ADA_EWORKSPACE = 4,   /* workspace missing or smaller than required */
    ADA_EHIP = 5          /* a HIP launch or copy failed */
} ada_status;

/* Static text for a status code (never NULL). */
const char *ada_status_str(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int ada_version(void);

/* Identity of the sources the library was built from: the hex SHA-256 that
 * the build computes over them ("unknown" for a build that gave none).  A
 * binding compares it with its own sources to refuse a stale library. */
const char *ada_build_id(void);

/* Phase timestamps of the page-stream kernel, for profiling the decode
 * step's fixed costs.  Only a library built with ADA_PHASE_TRACE
 * (`python -m compressed_kv_attention_amd.build --phase-trace`, which makes
 * libada_trace.so) records them; any other build returns ADA_EUNSUPPORTED
 * and changes nothing.
 *   buf    device memory the caller owns and keeps alive while it is set,
 *          8-byte aligned; NULL stops tracing.
 *   bytes  its size.
 * While set, every decode call whose trace fits (64 bytes per wave: blocks
 * = num_seqs x num_kv_heads x splits, each of 12 waves, or 8 at head_dim
 * 128 with more than 4 query heads per kv-head) overwrites it: for block b
 * and wave w, 8 u64 at (b x waves + w) x 8: the 100 MHz real-time counter at
 * kernel entry, prologue loads in, table built, past the table barrier,
 * page loop done, end (every load and store complete), then the wave's
 * HW_ID and XCC_ID registers.  A call whose trace does not fit records
 * nothing.  Not synchronised with calls in flight: set it between steps.
 * Errors: ADA_EINVAL for a misaligned buffer or fewer than 64 bytes. */
ada_status ada_phase_trace(void *buf, size_t bytes);

typedef struct {
    int32_t head_dim;     /* D: 64 or 128 */
    int32_t num_q_heads;  /* Hq */
    int32_t num_kv_heads; /* Hkv; Hq % Hkv == 0 and Hq / Hkv in {1, 2, 4, 5, 8} */
    int32_t page_size;    /* must be 16 */
} ada_geom;

/* One layer's cache view.  Rows are (sequence, kv-head) pairs,
 * row = s * Hkv + h.  All pointers are device memory owned by the caller. */
typedef struct {
    uint8_t *arena;          /* page bytes; 256-byte aligned */
    uint64_t arena_units;    /* arena size in 128-byte units (<= 2^32) */
    uint32_t *page_table;    /* [rows][max_pages_per_head]: page offset, 128-byte units */
    uint8_t *page_meta;      /* [rows][max_pages_per_head]: tier | (valid-1) << 2 */
    int32_t *num_pages;      /* [rows] pages in use per row */
    int32_t *tier_tokens;    /* [rows][3] retained tokens per tier (may be NULL for dense caches) */
    int32_t *slot_token;     /* [rows][max_pages_per_head][16] token position or -1; may be NULL */
    int32_t num_seqs;        /* S */
    int32_t max_pages_per_head;
} ada_cache;

/* Bytes of one page of `tier` (0..3) for head_dim D; 0 if unsupported. */
size_t ada_page_bytes(int32_t head_dim, int32_t tier);

/*
 * ada_encode -- keys to radius + angle codes.
 * [TS] 2.1 (spherical parameterization; quantized radius and packed angular
 * codes).  Reading: r = ||k|| of the fp16 key (double precision), stored
 * as fp16 (round to nearest even, saturating at 65504); the direction
 * u = k / r (u = 0 for a zero key) is split into G groups of 8 and each
 * group takes the index of its nearest codeword (squared Euclidean
 * distance, evaluated in double; lowest index on ties) among the 256
 * codewords of cb8 and, separately, the 16 codewords of cb4.
 *   keys    [n_tokens][Hkv][D] fp16 (16-byte aligned)
 *   cb8     [Hkv][G][256][8] f32,  cb4 [Hkv][G][16][8] f32 (one layer;
 *           both 16-byte aligned)
 *   radius  [n_tokens][Hkv] fp16 out (2-byte aligned)
 *   codes8  [n_tokens][Hkv][G] u8 out
 *   codes4  [n_tokens][Hkv][G/2] u8 out (two 4-bit codes per byte)
 * n_tokens may be 0 (no work).  Misaligned or null pointers -> ADA_EINVAL.
 * The codes are the exact double-precision argmin (the kernel scores in
 * binary32 and rescans near ties in double).
 */
ada_status ada_encode(const ada_geom *geom, int64_t n_tokens, const uint16_t *keys,
                      const float *cb8, const float *cb4, uint16_t *radius, uint8_t *codes8,
                      uint8_t *codes4, void *stream);

/*
 * rdr_pack_num_pages -- number of pages one rdr_pack call with these
 * sequences and mixes creates (the length of its place_perm_host).
 */
ada_status rdr_pack_num_pages(const ada_geom *geom, int32_t num_seqs,
                              const int32_t *cu_tokens_host, const int32_t *tier_cum_bp_host,
                              int64_t *n_pages_out);

/* Workspace bytes rdr_pack and dense_pack need for a call of n_tokens tokens
 * over num_seqs sequences. */
size_t rdr_pack_workspace_size(const ada_geom *geom, int64_t n_tokens, int32_t num_seqs);

/*
 * rdr_pack -- keep/drop + tier per (token, head), then tier-homogeneous pages.
 * [TS] 2.2 (joint residency/tier choice per state; protection forces the top
 * tier; pages hold one tier) and [ABS] (per token and head, under a fixed
 * budget).  The pages give no solver.  Reading: sequence s of this call owns
 * tokens cu_tokens_host[s] .. cu_tokens_host[s+1]-1 of the flat arrays
 * (T_s of them); tier_cum_bp_host[s][0..2] are cumulative basis points
 * (fp16, +8-bit, +4-bit; 0 <= b0 <= b1 <= b2 <= 10000) and give token
 * counts n_cum = floor((b * T_s + 5000) / 10000).  In each row the tokens
 * are ranked by (protected first, higher score first, lower index first):
 * the first n_cum[0] take tier 0, the next take tier 1 up to n_cum[1],
 * then tier 2 up to n_cum[2]; the rest are dropped (stored nowhere).  Inside
 * a tier, tokens keep index order and fill 16-slot pages.  Each row gains
 * its tier-0 pages, then tier-1, then tier-2, after the pages it had.  The
 * call's pages, numbered (s, h, tier, page), are placed in the arena by bump
 * allocation from *arena_cursor_host in the order place_perm_host[0..n)
 * (identity when NULL).  The 4-bit tier stores values as int8 with one fp16
 * scale per (token, head): scale = fp16(fp32(max|v| / 127)),
 * q = clamp(rint(fp32(v / scale)), -127, 127), q = 0 when scale = 0.
 *   num_seqs must equal cache->num_seqs (a sequence may bring 0 tokens).
 *   keys fp16 / values bf16 [N][Hkv][D] (both 16-byte aligned); radius
 *   [N][Hkv] (2-byte aligned); codes8 [N][Hkv][G], codes4 [N][Hkv][G/2]
 *   (from ada_encode; both 4-byte aligned); scores f32 [N][Hkv] (finite).
 *   A misaligned pointer is ADA_EINVAL.
 *   protect_host [N][Hkv] u8 (nonzero = protected) or NULL; more protected
 *     tokens in a row than its tier-0 count is ADA_EINVAL.
 *   place_perm_host: permutation of [0, n_pages) or NULL.
 *   pos_base_host [S]: position of each sequence's first token of this call,
 *     recorded in slot_token (NULL = 0).
 *   arena_cursor_host (in/out): next free 128-byte unit of the arena.
 *   num_pages_host [S*Hkv] (in/out): host copy of cache->num_pages; the call
 *     checks row capacity against it and advances it.
 *   ws: device workspace of rdr_pack_workspace_size bytes.
 * Errors: ADA_ENOSPACE when the pages do not fit in the arena, ADA_EINVAL
 * when a row would exceed max_pages_per_head -- both before any device work.
 */
ada_status rdr_pack(const ada_geom *geom, const ada_cache *cache, int32_t num_seqs,
                    const int32_t *cu_tokens_host, const int32_t *tier_cum_bp_host,
                    const uint16_t *keys, const uint16_t *values, const uint16_t *radius,
                    const uint8_t *codes8, const uint8_t *codes4, const float *scores,
                    const uint8_t *protect_host, const uint32_t *place_perm_host,
                    const int64_t *pos_base_host, uint64_t *arena_cursor_host,
                    int32_t *num_pages_host, void *ws, size_t ws_bytes, void *stream);

/*
 * dense_pack -- the comparison cache: every token of the call, in index
 * order, in tier-3 pages (keys rounded fp16 -> bf16, values bf16).  Not part
 * of the method; it feeds dense_decode, the dense bf16 paged-attention
 * baseline the pages compare against ([TS] section 4).  Arguments as in
 * rdr_pack; place_perm_host has one entry per page of the call
 * (rows * ceil(T_s / 16) summed over sequences).
 */
ada_status dense_pack(const ada_geom *geom, const ada_cache *cache, int32_t num_seqs,
                      const int32_t *cu_tokens_host, const uint16_t *keys,
                      const uint16_t *values, const uint32_t *place_perm_host,
                      uint64_t *arena_cursor_host, int32_t *num_pages_host, void *ws,
                      size_t ws_bytes, void *stream);

/*
 * ada_code_error -- angular error of the stored codes of each (token, head),
 * the input of the RDR distortion surrogate.  [TS] 2.2 (the logit error is
 * dominated by the angular approximation error, scaled by the query and key
 * magnitudes).  Reading: the chord error of the code reconstruction,
 *   err = sum_g || u_g - C_g[code_g] ||^2,  u = k / ||k|| (u = 0 for k = 0),
 * for the 8-bit codes (err8) and the 4-bit codes (err4); sqrt(err) bounds
 * |q . (u - u~)| / |q|.  u is formed as in ada_encode; every sum runs in
 * double (each group over its 8 coordinates, then the groups in order) and
 * the total is rounded once to f32.
 *   keys [n_tokens][Hkv][D] fp16 (16-byte aligned); cb8 / cb4 as in
 *   ada_encode (16-byte aligned); codes8 / codes4 as ada_encode writes them
 *   (any codes are accepted; both 4-byte aligned); err8, err4
 *   [n_tokens][Hkv] f32 out.
 */
ada_status ada_code_error(const ada_geom *geom, int64_t n_tokens, const uint16_t *keys,
                          const float *cb8, const float *cb4, const uint8_t *codes8,
                          const uint8_t *codes4, float *err8, float *err4, void *stream);

/* Workspace bytes of rdr_solve for num_seqs sequences of n_tokens tokens in
 * total. */
size_t rdr_solve_workspace_size(const ada_geom *geom, int32_t num_seqs, int64_t n_tokens);

/*
 * rdr_solve -- the tier of every (token, head) under a byte budget per
 * sequence.  [TS] 2.2 (a residency bit and a tier per state from a discrete
 * rate-distortion allocation under a strict memory budget; the distortion
 * surrogate; protection keeps a state at the top tier) and [ABS] (retention
 * and precision follow estimated utility, per token and head).  The pages
 * give no solver.  Reading:
 *   rate of a state in tier b: R_b = ada_page_bytes(D, b) / 16, R_3 = 0
 *     (tier 3 = dropped);
 *   distortion: D_b = w * r~ * e_b, w = scores (utility), r~ = radius,
 *     e_0 = 0, e_1 = sqrt(err8), e_2 = sqrt(err4), e_3 = 1 (a dropped key
 *     keeps none of its direction); the common query magnitude is left out;
 *   cap = budget_bytes_host[s] - Hkv * 15 * (R_0 + R_1 + R_2): room for the
 *     partial last page of each tier in every row, so the pages rdr_pack_tiers
 *     writes for this call stay within the budget;
 *   every state starts at tier 0; the lower convex hull of its four
 *     (rate, distortion) points is a chain of demotions of non-decreasing
 *     slope (distortion added per byte saved); with need = (bytes at tier 0)
 *     - cap, s* is the least slope such that the demotions of slope <= s*
 *     over all the sequence's states save at least `need` bytes (+inf when
 *     none does: every unprotected state is dropped), and each state takes
 *     the longest prefix of its chain with slopes <= s*.  need <= 0 leaves
 *     every state at tier 0.  Protected states stay at tier 0.
 *   The result is optimal, for its own byte count, among all assignments
 *   (the Lagrangian property).  The chain arithmetic is binary32 in a fixed
 *   order: wr = w * r~, D_1 = wr * sqrtf(err8), D_2 = wr * sqrtf(err4),
 *   D_3 = wr, slope = (D_j - D_c) / (R_c - R_j) + 0 (IEEE division and
 *   square root); the hull walk takes the least slope, the lower rate on
 *   ties, and a slope below its predecessor is raised to it.
 *   budget_bytes_host [S] (>= 0).  radius [N][Hkv] fp16, err8 / err4 [N][Hkv]
 *   f32 (ada_code_error), scores [N][Hkv] f32: finite and >= 0 (device).
 *   protect [N][Hkv] u8 on the DEVICE (nonzero = protected) or NULL.
 *   tiers [N][Hkv] u8 out: 0, 1, 2 kept tier, 3 dropped.
 *   threshold [S] f32 out (device) or NULL: each sequence's s*; -inf when
 *     need <= 0, +inf when every demotion is taken (ada_append's input).
 *   ws: rdr_solve_workspace_size bytes, 256-byte aligned, any content.
 * Seven kernels on `stream`; the small per-sequence table is copied from
 * host memory first.
 */
ada_status rdr_solve(const ada_geom *geom, int32_t num_seqs, const int32_t *cu_tokens_host,
                     const int64_t *budget_bytes_host, const uint16_t *radius, const float *err8,
                     const float *err4, const float *scores, const uint8_t *protect,
                     uint8_t *tiers, float *threshold, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes of rdr_tier_counts. */
size_t rdr_tier_counts_workspace_size(const ada_geom *geom, int32_t num_seqs);

/*
 * rdr_tier_counts -- tokens of tier 0, 1 and 2 in every row (s, h) of a
 * tiers array (values other than 0-2 count as dropped), copied to
 * row_counts_host [S*Hkv][3].  Synchronizes `stream`: the counts are on the
 * host when the call returns.  They size the pages of rdr_pack_tiers.
 */
ada_status rdr_tier_counts(const ada_geom *geom, int32_t num_seqs, const int32_t *cu_tokens_host,
                           const uint8_t *tiers, int32_t *row_counts_host, void *ws,
                           size_t ws_bytes, void *stream);

/* Number of pages rdr_pack_tiers creates for these row counts (the length of
 * its place_perm_host). */
ada_status rdr_pack_tiers_num_pages(const ada_geom *geom, int32_t num_seqs,
                                    const int32_t *row_counts_host, int64_t *n_pages_out);

/*
 * rdr_pack_tiers -- rdr_pack with the tier of every (token, head) given
 * (rdr_solve's output) instead of ranked from basis points.  [TS] 2.2
 * (tier-homogeneous pages).  Each row's tokens of one tier keep index order
 * and fill 16-slot pages; tier values other than 0-2 are dropped.
 * row_counts_host [S*Hkv][3] must be rdr_tier_counts of the same tiers
 * (the page plan is built from them on the host; a row's counts may not
 * exceed its tokens).  Everything else -- page order, placement, value
 * quantisation, workspace (rdr_pack_workspace_size), errors -- is as in
 * rdr_pack.
 */
ada_status rdr_pack_tiers(const ada_geom *geom, const ada_cache *cache, int32_t num_seqs,
                          const int32_t *cu_tokens_host, const int32_t *row_counts_host,
                          const uint8_t *tiers, const uint16_t *keys, const uint16_t *values,
                          const uint16_t *radius, const uint8_t *codes8, const uint8_t *codes4,
                          const uint32_t *place_perm_host, const int64_t *pos_base_host,
                          uint64_t *arena_cursor_host, int32_t *num_pages_host, void *ws,
                          size_t ws_bytes, void *stream);

/*
 * rdr_pack_tiers_device -- rdr_pack_tiers with the page plan made on the
 * device, so the solver path (ada_code_error, rdr_solve, this call) needs
 * no host round trip and no tier counts on the host.  [TS] 2.2 (retained
 * states grouped into tier-homogeneous pages).  Each row counts its own
 * tokens of tiers 0, 1 and 2 (other values are dropped, as in
 * rdr_pack_tiers); its new pages are numbered after the row's num_pages on
 * the device, and their arena space is one block per row taken from the
 * device bump cursor of `state` (ada_append's state: u64 cursor at byte 0,
 * sticky status at byte 8), tier 0's pages first.  Rows race for the
 * cursor, so where a row's block lands is not fixed; what each row holds
 * -- its pages' bytes, order, metadata, slot positions and counts -- is
 * exactly what rdr_pack_tiers writes for the same tiers.  A row whose pages
 * would pass max_pages_per_head stores nothing and sets status bit 1; a
 * row whose block would pass arena_units stores nothing and sets bit 2.
 * The host's cursor and page counts are not advanced: read them back from
 * the device (state cursor, cache->num_pages) before a host-planned pack.
 * Other arguments as rdr_pack_tiers (no row counts, no placement order);
 * ws: rdr_pack_workspace_size bytes.  keys / values 16-byte, codes 4-byte,
 * radius 2-byte aligned; state 256-byte aligned.
 */
ada_status rdr_pack_tiers_device(const ada_geom *geom, const ada_cache *cache, int32_t num_seqs,
                                 const int32_t *cu_tokens_host, const uint8_t *tiers, const uint16_t *keys,
                                 const uint16_t *values, const uint16_t *radius, const uint8_t *codes8,
                                 const uint8_t *codes4, const int64_t *pos_base_host, void *state, void *ws,
                                 size_t ws_bytes, void *stream);

/* Bytes of the device state ada_append keeps between decode steps. */
size_t ada_append_state_bytes(const ada_geom *geom, int32_t num_seqs);

/*
 * ada_append -- one decode step's new token per (sequence, kv-head) row:
 * encode, tier and place it, in one kernel, with no host round trip.
 * [TS] 2.3 (dense keys mapped to codes, filtered and tiered by RDR, stored
 * compressed) and 2.2 (tier-homogeneous pages; tiers under a budget).
 * Reading:
 *   - the key is encoded exactly as ada_encode does, and its code errors
 *     are those of ada_code_error;
 *   - its tier follows the rdr_solve chain rule with its sequence's slope
 *     threshold (threshold[s], e.g. rdr_solve's output): the online
 *     continuation of the last solve's Lagrangian allocation. Protected
 *     states take tier 0; tier 3 is a drop;
 *   - a kept state fills the next free slot of its row's open page of that
 *     tier. If the row has none, or it is full, the row takes a new page:
 *     the next page-table index and arena space from a device-side bump
 *     cursor that never passes arena_units. The page is zeroed first.
 *   keys fp16 / values bf16 [S][Hkv][D]; scores f32 [S][Hkv]; protect u8
 *   [S][Hkv] or NULL; threshold f32 [S]; pos int64 [S] (recorded in
 *   slot_token); tiers_out u8 [S][Hkv] or NULL (the tier each state was
 *   given). All device pointers.
 *   state: ada_append_state_bytes, 256-byte aligned, device memory:
 *     [0]   u64 arena cursor in 128-byte units. Set it from the host cursor
 *           before the first append, and read it back (with num_pages)
 *           before the next host-planned pack.
 *     [8]   u32 status, sticky bits: 1 = a row's page table was full,
 *           2 = the arena was full. That row's token is not stored.
 *     [256] i32 [S*Hkv][3]: each row's open page index + 1 per tier
 *           (0 = none). Zero-filled: no open page (pages from packs stay as
 *           they are).
 *   Rows race only for the cursor, so which page offset a row gets is not
 *   fixed; what each row holds is.
 */
ada_status ada_append(const ada_geom *geom, const ada_cache *cache, const float *cb8,
                      const float *cb4, const uint16_t *keys, const uint16_t *values,
                      const float *scores, const uint8_t *protect, const float *threshold,
                      const int64_t *pos, uint8_t *tiers_out, void *state, void *stream);

/*
 * ada_retier -- re-tiering as a sequence outgrows its budget: demote listed
 * fp16 pages in place, evict listed pages.  [TS] 2.2 (states kept and
 * tiered under a strict memory budget, in tier-homogeneous pages).
 * Reading:
 *   - target 1 or 2 demotes an fp16 page (full or not) to that tier. The
 *     page's keys are encoded from its own fp16 keys, exactly as ada_encode
 *     does. Its values are kept (8-bit tier) or quantised as in rdr_pack
 *     (4-bit tier). The new page goes to arena space from the state's
 *     cursor, and the page-table entry (same index, same slots) points at
 *     it. The old bytes stay behind: the arena only grows.
 *   - target 3 evicts a page: per row, in descending page index, the row's
 *     last page moves into its place.
 *   - Demotions run before evictions. Each page may be listed once.
 *   - An entry that cannot apply adds status bit 4 and is skipped: a row
 *     outside the cache, a page not in use, a target other than 1-3, a
 *     demotion of a page that is not fp16, or an eviction of a tier-3
 *     (dense comparison) page, which has no tier count. No arena space adds
 *     bit 2.
 *   - tier_tokens, num_pages and the open pages in `state` are kept
 *     current.
 *   rows, pages [n] int32 and target [n] u8 are DEVICE arrays (the call can
 *   be captured). state: as in ada_append.
 */
ada_status ada_retier(const ada_geom *geom, const ada_cache *cache, const float *cb8,
                      const float *cb4, int32_t n, const int32_t *rows, const int32_t *pages,
                      const uint8_t *target, void *state, void *stream);

/*
 * ada_retier_plan -- host-side policy for ada_retier. Stored pages keep no
 * utility scores, so age stands in for utility (reading). For each
 * sequence whose page bytes exceed budget_bytes_host[s], in three passes
 * over (page index, then head), oldest first:
 *   1. demote full fp16 pages to `demote_to` (1 or 2);
 *   2. evict coded pages;
 *   3. evict the remaining partial fp16 pages;
 * each until the sequence fits. Pages demoted by a plan are not also
 * evicted by it, so a second plan may be needed.
 *   num_pages_host [S*Hkv], page_meta_host [S*Hkv][max_pages_per_head]:
 *   host copies of the tables. Writes at most cap entries to rows_out /
 *   pages_out / target_out (host) and their number to *n_out.
 */
ada_status ada_retier_plan(const ada_geom *geom, int32_t num_seqs, const int64_t *budget_bytes_host,
                           const int32_t *num_pages_host, const uint8_t *page_meta_host,
                           int32_t max_pages_per_head, int32_t demote_to, int32_t cap,
                           int32_t *rows_out, int32_t *pages_out, uint8_t *target_out,
                           int32_t *n_out);

/* Workspace bytes of ada_decode_sym: ada_decode's plus every row's table. */
size_t ada_decode_sym_workspace_size(const ada_geom *geom, int32_t num_seqs,
                                     int32_t max_pages_per_head, int32_t num_splits);

/*
 * ada_decode_sym -- ada_decode with the symmetric angle-code logit.  [TS]
 * 2.1 writes the logit as |q| * r~ * f_b(c_q, c_k), a cosine computed from
 * the angular codes of both query and key.  Reading: the query's unit
 * direction u_q = q / |q| (|q| in double, summed sequentially over D) takes,
 * in each group and each codebook, the index of its nearest codeword as a
 * key does in ada_encode (squared distance in double, lowest index on
 * ties), and a coded slot's logit is
 *   l_t = softmax_scale * |q| * r~_t * sum_g C_g[cq_g] . C_g[code_{t,g}]
 * (the 8-bit codebook for 8-bit keys, the 4-bit one for 4-bit keys): the
 * table of ada_decode with q_g replaced by |q| C_g[cq_g], tabulated in fp32
 * as |q| * (C_g[cq_g] . C_g[c]).  fp16-tier slots keep softmax_scale * q.k.
 * Arguments and outputs as ada_decode; ws: ada_decode_sym_workspace_size
 * bytes (any content).  Up to three kernels on `stream`: the table, the
 * page stream (which copies its row's table into LDS) and the merge.
 */
ada_status ada_decode_sym(const ada_geom *geom, const ada_cache *cache, const float *cb8,
                          const float *cb4, const uint16_t *q, float softmax_scale, float *out,
                          float *lse, float *logits_dbg, int32_t num_splits, void *ws,
                          size_t ws_bytes, void *stream);

/* Split count ada_decode / dense_decode use for num_splits == 0. */
int32_t ada_decode_default_splits(const ada_geom *geom, int32_t num_seqs,
                                  int32_t max_pages_per_head);

/* Workspace bytes of ada_decode / dense_decode with this many splits
 * (0 = the default).  The workspace holds the per-split partial results. */
size_t ada_decode_workspace_size(const ada_geom *geom, int32_t num_seqs,
                                 int32_t max_pages_per_head, int32_t num_splits);

/*
 * ada_decode -- one decode step over a cache view.
 * [TS] 2.1: logits straight from the stored codes, with no dense key rebuilt
 * in device memory; the pages give l ~ |q| * r~ * f_b(codes), f_b a cosine
 * from the codes.  With the encoding above this is
 *   l_t = softmax_scale * r~_t * sum_g LUT_g[code_{t,g}],
 *   LUT_g[c] = q_g . C_g[c]      (tiers 1 and 2),
 *   l_t = softmax_scale * q . k_t (tier 0),
 * then softmax attention over the row's retained slots:
 *   out = sum_t e^(l_t - m) v_t / sum_t e^(l_t - m),  lse = m + ln sum_t e^(l_t - m),
 * v_t the stored bf16 value, or int8 * scale in tier 2.  Query head hq reads
 * kv-head hq / (Hq / Hkv).  No causal mask.  A row with no pages gives
 * out = 0, lse = -inf.
 *   cb8 / cb4 as in ada_encode (the layer's codebooks).
 *   q        [S][Hq][D] bf16
 *   out      [S][Hq][D] f32;  lse [S][Hq] f32 or NULL
 *   logits_dbg [S][Hq][max_pages_per_head * 16] f32 or NULL: for parity
 *     tests, receives l_t of every valid slot (page p, slot t at p*16+t);
 *     other entries are left untouched.
 *   num_splits: page subsets per row, 1..1024 (0 = ada_decode_default_splits).
 *     A count so small that a split's page-table entries and the row's code
 *     tables overflow the 160 KiB of LDS gives ADA_EINVAL (the default
 *     never does).
 *   ws: ada_decode_workspace_size(geom, S, max_pages_per_head, num_splits)
 *     bytes, 256-byte aligned, any content: every call writes what it
 *     reads.  Calls that overlap in time must not share a workspace.
 * The step is up to two kernels on `stream`: the page stream (which also
 * tabulates each row's code tables in LDS) and a split merge when
 * num_splits > 1.
 * Cache pages must be tiers 0-2.  Queries must be finite with |q| < 2^64.
 */
ada_status ada_decode(const ada_geom *geom, const ada_cache *cache, const float *cb8,
                      const float *cb4, const uint16_t *q, float softmax_scale, float *out,
                      float *lse, float *logits_dbg, int32_t num_splits, void *ws,
                      size_t ws_bytes, void *stream);

/*
 * ada_decode_noalloc -- ada_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  It takes no workspace: the split partials live in a
 * library-owned device array of ADA_NOALLOC_SCRATCH_BYTES, one per GPU the
 * library runs on, held until the process ends (its address is looked up
 * on the first call on each device, with that device current).  The call
 * allocates and frees nothing.  Arguments, outputs and errors are those of
 * ada_decode; a step whose partials (ada_decode_workspace_size) exceed the
 * array gives ADA_EWORKSPACE before any device work.  The partials need no
 * clearing: every call writes what it reads.  All calls on one GPU share
 * the array, so calls that overlap in time on one GPU (on different
 * streams, or from several host threads) race and must be serialised by
 * the caller.
 */
#define ADA_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
ada_status ada_decode_noalloc(const ada_geom *geom, const ada_cache *cache, const float *cb8,
                              const float *cb4, const uint16_t *q, float softmax_scale, float *out,
                              float *lse, float *logits_dbg, int32_t num_splits, void *stream);

/*
 * The two stages of ada_decode, for callers that time or schedule them
 * apart.  Each takes the arguments of ada_decode (unused ones may be NULL);
 * called in this order on one stream with the same arguments and workspace
 * they do exactly what one ada_decode call does.
 *   ada_decode_stream: the page stream; writes the split partials into ws
 *     (or out / lse / logits_dbg directly when num_splits resolves to 1).
 *   ada_decode_merge:  combines the partials into out / lse; enqueues
 *     nothing when num_splits resolves to 1.
 */
ada_status ada_decode_stream(const ada_geom *geom, const ada_cache *cache, const float *cb8,
                             const float *cb4, const uint16_t *q, float softmax_scale, float *out,
                             float *lse, float *logits_dbg, int32_t num_splits, void *ws,
                             size_t ws_bytes, void *stream);
ada_status ada_decode_merge(const ada_geom *geom, const ada_cache *cache, const float *cb8,
                            const float *cb4, const uint16_t *q, float softmax_scale, float *out,
                            float *lse, int32_t num_splits, void *ws, size_t ws_bytes, void *stream);

/*
 * dense_decode -- the dense bf16 paged-decode baseline over tier-3 pages
 * (l_t = softmax_scale * q . k_t with bf16 keys), same split/merge scheme
 * and arguments as ada_decode without codebooks.
 */
ada_status dense_decode(const ada_geom *geom, const ada_cache *cache, const uint16_t *q,
                        float softmax_scale, float *out, float *lse, float *logits_dbg,
                        int32_t num_splits, void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ADA_H */
