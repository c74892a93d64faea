// Host side of libada: argument checks, pack planning, launches.
// Declarations and the contract of every entry point are in include/ada.h.
#include "ada.h"
#include "ada_internal.h"

#include <algorithm>
#include <atomic>
#include <cstring>
#include <vector>

namespace {

// Phase-timestamp buffer of tracing builds (ada_phase_trace): a decode call
// passes it to the page stream only when its 64 bytes per wave fit.
std::atomic<void *> g_trace_buf{nullptr};
std::atomic<size_t> g_trace_bytes{0};

unsigned long long *phase_trace_for(size_t waves)
{
#ifdef ADA_PHASE_TRACE
    void *b = g_trace_buf.load();
    if (b != nullptr && waves * 64 <= g_trace_bytes.load())
        return static_cast<unsigned long long *>(b);
#else
    (void)waves;
#endif
    return nullptr;
}

using namespace ada;

constexpr int kVersion = 100; // 0.1.0
constexpr int kMaxSplits = 1024;

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

bool geom_ok(const ada_geom *g)
{
    return g != nullptr && (g->head_dim == 64 || g->head_dim == 128) && g->num_kv_heads > 0 &&
           g->num_q_heads > 0 && g->num_q_heads % g->num_kv_heads == 0 && g->page_size == kSlots;
}

bool gqa_supported(const ada_geom *g)
{
    const int r = g->num_q_heads / g->num_kv_heads;
    return r == 1 || r == 2 || r == 4 || r == 5 || r == 8;
}

bool cache_ok(const ada_cache *c)
{
    return c != nullptr && c->arena != nullptr && c->page_table != nullptr &&
           c->page_meta != nullptr && c->num_pages != nullptr && c->num_seqs >= 0 &&
           c->max_pages_per_head >= 0 && c->arena_units <= (1ull << 32);
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int64_t tier_count(int64_t T, int32_t bp) { return (bp * T + 5000) / 10000; }

// Upper bound on the pages one pack call can create.
int64_t max_pack_pages(int Hkv, int64_t n_tokens, int32_t num_seqs)
{
    return (int64_t)Hkv * (n_tokens / kSlots + 3 * (int64_t)num_seqs + 1);
}

struct PlanBuf {
    std::vector<uint8_t> blob; // [seqs][rows][pages] (each 256-byte aligned)
    size_t seq_off = 0, row_off = 0, page_off = 0;
    int n_pages = 0;
    bool gen_pages = false; // the device writes the page list
    uint64_t cursor_after = 0;
    std::vector<int32_t> new_pages_per_row;
};

size_t pack_workspace(int Hkv, int64_t n_tokens, int32_t num_seqs)
{
    const int64_t rows = (int64_t)num_seqs * Hkv;
    size_t b = align256(sizeof(PackSeq) * (size_t)std::max<int32_t>(num_seqs, 1));
    b += align256(sizeof(PackRow) * (size_t)std::max<int64_t>(rows, 1));
    b += align256(sizeof(PackPage) * (size_t)max_pack_pages(Hkv, n_tokens, num_seqs));
    b += align256((size_t)n_tokens * Hkv);                   // protect copy
    b += align256((size_t)max_pack_pages(Hkv, n_tokens, num_seqs) * kSlots * sizeof(int32_t)); // src
    return b;
}

// Plans one pack call on the host: counts, page numbering, placement.
// counts[s][3] per-tier token counts of each sequence (the ranked path), and
// row_counts[s * Hkv + h][3] those of each row; returns ADA_OK or the error.
// Pages are numbered row by row, tiers 0, 1, 2 within a row.  In arena order
// (perm null) a row's tier block is placed contiguously and the device
// writes the page list from the rows' entries; for a given order the host
// builds the list and places it.
ada_status plan_pack(const ada_geom *g, const ada_cache *c, int32_t S, const int32_t *cu,
                     const std::vector<int64_t> &counts, const std::vector<int64_t> &row_counts,
                     bool dense, const uint32_t *perm,
                     const int64_t *pos_base, uint64_t cursor, const int32_t *num_pages_host,
                     PlanBuf &pb)
{
    const int H = g->num_kv_heads, D = g->head_dim;
    const int64_t rows = (int64_t)S * H;
    std::vector<PackSeq> seqs(S);
    std::vector<PackRow> rowv(rows);
    pb.new_pages_per_row.assign(rows, 0);
    int64_t n = 0;
    for (int s = 0; s < S; s++) {
        seqs[s].begin = cu[s];
        seqs[s].len = cu[s + 1] - cu[s];
        int64_t acc = 0;
        for (int k = 0; k < 3; k++) {
            acc += counts[s * 3 + k];
            seqs[s].n_cum[k] = (int32_t)acc;
        }
        seqs[s].pad = 0;
        seqs[s].pos_base = pos_base ? pos_base[s] : 0;
        for (int h = 0; h < H; h++) {
            const int64_t r = (int64_t)s * H + h;
            int64_t row_pages = 0;
            for (int k = 0; k < 3; k++) {
                const int64_t cnt = row_counts[r * 3 + k];
                rowv[r].lp_first[k] = (int32_t)std::min<int64_t>(n + row_pages, INT32_MAX);
                rowv[r].count[k] = (int32_t)cnt;
                row_pages += (cnt + kSlots - 1) / kSlots;
            }
            rowv[r].pi0 = num_pages_host[r];
            if ((int64_t)num_pages_host[r] + row_pages > c->max_pages_per_head)
                return ADA_EINVAL;
            pb.new_pages_per_row[r] = (int32_t)row_pages;
            n += row_pages;
        }
    }
    if (n > INT32_MAX)
        return ADA_EINVAL;
    const uint64_t unit[3] = {(uint64_t)page_bytes(D, dense ? 3 : 0) / kUnit,
                              (uint64_t)page_bytes(D, dense ? 3 : 1) / kUnit,
                              (uint64_t)page_bytes(D, dense ? 3 : 2) / kUnit};
    uint64_t cur = cursor;
    std::vector<PackPage> pages;
    if (perm == nullptr) {
        // arena order: each row's tier blocks back to back
        for (int64_t r = 0; r < rows; r++)
            for (int k = 0; k < 3; k++) {
                rowv[r].off[k] = (uint32_t)std::min<uint64_t>(cur, UINT32_MAX);
                cur += unit[k] * (uint64_t)((rowv[r].count[k] + kSlots - 1) / kSlots);
                if (cur > c->arena_units)
                    return ADA_ENOSPACE;
            }
    } else {
        pages.reserve((size_t)n);
        for (int64_t r = 0; r < rows; r++)
            for (int k = 0; k < 3; k++) {
                rowv[r].off[k] = 0;
                const int64_t cnt = rowv[r].count[k];
                for (int64_t f = 0; f < cnt; f += kSlots) {
                    PackPage p;
                    p.off = 0;
                    p.row = (int32_t)r;
                    p.pi = rowv[r].pi0 + (int32_t)(pages.size() - rowv[r].lp_first[0]);
                    const int nv = (int)std::min<int64_t>(kSlots, cnt - f);
                    p.meta = (dense ? 3 : k) | ((nv - 1) << 2);
                    pages.push_back(p);
                }
            }
        std::vector<char> seen(n, 0);
        for (int64_t k = 0; k < n; k++)
            if (perm[k] >= (uint64_t)n || seen[perm[k]]++)
                return ADA_EINVAL;
        for (int64_t k = 0; k < n; k++) {
            PackPage &p = pages[perm[k]];
            p.off = (uint32_t)cur;
            cur += (uint64_t)page_bytes(D, p.meta & 3) / kUnit;
            if (cur > c->arena_units)
                return ADA_ENOSPACE;
        }
    }
    pb.n_pages = (int)n;
    pb.cursor_after = cur;
    pb.seq_off = 0;
    pb.row_off = align256(sizeof(PackSeq) * (size_t)std::max(S, 1));
    pb.page_off = pb.row_off + align256(sizeof(PackRow) * (size_t)std::max<int64_t>(rows, 1));
    pb.gen_pages = perm == nullptr;
    pb.blob.assign(pb.gen_pages ? pb.row_off + sizeof(PackRow) * (size_t)std::max<int64_t>(rows, 1)
                                : pb.page_off + sizeof(PackPage) * (size_t)std::max<int64_t>(n, 1),
                   0);
    std::memcpy(pb.blob.data() + pb.seq_off, seqs.data(), sizeof(PackSeq) * seqs.size());
    std::memcpy(pb.blob.data() + pb.row_off, rowv.data(), sizeof(PackRow) * rowv.size());
    if (!pb.gen_pages)
        std::memcpy(pb.blob.data() + pb.page_off, pages.data(), sizeof(PackPage) * pages.size());
    return ADA_OK;
}

ada_status run_pack(const ada_geom *g, const ada_cache *c, int32_t S, const int32_t *cu,
                    const std::vector<int64_t> &counts, const std::vector<int64_t> &row_counts,
                    const uint8_t *tiers, bool dense, const uint16_t *keys,
                    const uint16_t *values, const uint16_t *radius, const uint8_t *codes8,
                    const uint8_t *codes4, const float *scores, const uint8_t *protect_host,
                    const uint32_t *perm, const int64_t *pos_base, uint64_t *cursor,
                    int32_t *num_pages_host, void *ws, size_t ws_bytes, void *stream)
{
    const int H = g->num_kv_heads;
    const int64_t N = cu[S];
    // (16-byte key and value loads, 4-byte code loads)
    if ((reinterpret_cast<uintptr_t>(keys) & 15) || (reinterpret_cast<uintptr_t>(values) & 15) ||
        (reinterpret_cast<uintptr_t>(codes8) & 3) || (reinterpret_cast<uintptr_t>(codes4) & 3) ||
        (reinterpret_cast<uintptr_t>(radius) & 1))
        return ADA_EINVAL;
    if (ws == nullptr || ws_bytes < pack_workspace(H, N, S) || (reinterpret_cast<uintptr_t>(ws) & 255))
        return ADA_EWORKSPACE;
    PlanBuf pb;
    if (ada_status st = plan_pack(g, c, S, cu, counts, row_counts, dense, perm, pos_base, *cursor,
                                  num_pages_host, pb);
        st != ADA_OK)
        return st;
    if (pb.n_pages > max_pack_pages(H, N, S))
        return ADA_EWORKSPACE;
    // workspace: [plan blob][protect][src]
    uint8_t *wsb = static_cast<uint8_t *>(ws);
    const size_t blob_cap = align256(sizeof(PackSeq) * (size_t)std::max(S, 1)) +
                            align256(sizeof(PackRow) * (size_t)std::max<int64_t>((int64_t)S * H, 1)) +
                            align256(sizeof(PackPage) * (size_t)max_pack_pages(H, N, S));
    uint8_t *prot_dev = wsb + blob_cap;
    int32_t *src = reinterpret_cast<int32_t *>(prot_dev + align256((size_t)N * H));
    hipStream_t st = as_stream(stream);
    // pageable host source: the runtime copies it before returning
    if (hipMemcpyAsync(wsb, pb.blob.data(), pb.blob.size(), hipMemcpyHostToDevice, st) != hipSuccess)
        return ADA_EHIP;
    if (protect_host != nullptr && N > 0 &&
        hipMemcpyAsync(prot_dev, protect_host, (size_t)N * H, hipMemcpyHostToDevice, st) != hipSuccess)
        return ADA_EHIP;
    PackPlan plan;
    plan.seqs = reinterpret_cast<const PackSeq *>(wsb + pb.seq_off);
    plan.rows = reinterpret_cast<const PackRow *>(wsb + pb.row_off);
    plan.pages = reinterpret_cast<PackPage *>(wsb + pb.page_off);
    plan.protect = protect_host != nullptr ? prot_dev : nullptr;
    plan.tiers = tiers;
    plan.src = src;
    plan.S = S;
    plan.Hkv = H;
    plan.D = g->head_dim;
    plan.maxp = c->max_pages_per_head;
    plan.n_pages = pb.n_pages;
    plan.dense = dense ? 1 : 0;
    plan.gen_pages = pb.gen_pages ? 1 : 0;
    plan.n_tokens = N;
    plan.dev_plan = 0;
    plan.cursor = nullptr;
    plan.status = nullptr;
    plan.capacity = 0;
    PackData data{keys, values, radius, codes8, codes4, scores};
    PackCache cache{c->arena, c->page_table, c->page_meta, c->num_pages, c->tier_tokens, c->slot_token};
    if (launch_pack(plan, data, cache, st) != hipSuccess)
        return ADA_EHIP;
    *cursor = pb.cursor_after;
    for (size_t r = 0; r < pb.new_pages_per_row.size(); r++)
        num_pages_host[r] += pb.new_pages_per_row[r];
    return ADA_OK;
}

bool cu_ok(int32_t S, const int32_t *cu)
{
    if (cu == nullptr || cu[0] != 0)
        return false;
    for (int s = 0; s < S; s++)
        if (cu[s + 1] < cu[s])
            return false;
    return true;
}

// Per-row counts when every row of a sequence has the sequence's counts.
std::vector<int64_t> rows_of(int32_t S, int H, const std::vector<int64_t> &counts)
{
    std::vector<int64_t> rc((size_t)S * H * 3);
    for (int s = 0; s < S; s++)
        for (int h = 0; h < H; h++)
            for (int k = 0; k < 3; k++)
                rc[((size_t)s * H + h) * 3 + k] = counts[(size_t)s * 3 + k];
    return rc;
}

bool counts_from_bp(int32_t S, const int32_t *cu, const int32_t *bp, std::vector<int64_t> &counts)
{
    counts.assign((size_t)S * 3, 0);
    for (int s = 0; s < S; s++) {
        const int32_t *b = bp + 3 * s;
        if (b[0] < 0 || b[0] > b[1] || b[1] > b[2] || b[2] > 10000)
            return false;
        const int64_t T = cu[s + 1] - cu[s];
        int64_t prev = 0;
        for (int k = 0; k < 3; k++) {
            const int64_t n = tier_count(T, b[k]);
            counts[s * 3 + k] = n - prev;
            prev = n;
        }
    }
    return true;
}

// Byte offsets of the decode workspace parts (all 256-byte aligned): the
// split partials (m, l) and acc.
struct WsLayout {
    size_t ml_off, acc_off, lut_off, total;
};

// sym: the symmetric variant adds every row's LUT after the partials.
WsLayout ws_layout(const ada_geom *g, int32_t S, int32_t ns, bool sym = false)
{
    const size_t rows = (size_t)S * g->num_kv_heads;
    const size_t NH = (size_t)(g->num_q_heads / g->num_kv_heads);
    const size_t D = (size_t)g->head_dim;
    WsLayout l{};
    l.ml_off = 0;
    l.acc_off = align256(rows * ns * NH * 2 * sizeof(float));
    l.lut_off = l.acc_off + align256(rows * ns * NH * D * sizeof(float));
    l.total = l.lut_off;
    if (sym)
        l.total += align256(rows * decode_lut_floats(g->head_dim, (int)NH) * sizeof(float));
    return l;
}

int32_t default_splits(const ada_geom *g, int32_t S, int32_t maxp)
{
    const int64_t rows = (int64_t)S * g->num_kv_heads;
    if (rows <= 0)
        return 1;
    // about one workgroup per compute unit (four splits once the rows alone
    // fill the chip: ragged rows then still balance) and at least 16 pages
    // per split, with few enough pages per split that their table entries
    // fit in LDS beside the group's LUT
    int64_t n = rows >= 256 ? 4 : (256 + rows - 1) / rows;
    n = std::min<int64_t>(n, std::max<int64_t>(1, maxp / 16));
    n = std::max<int64_t>(n, 1);
    const int NH = g->num_q_heads / g->num_kv_heads;
    while (n < kMaxSplits && decode_shmem_bytes(g->head_dim, NH, false, (int)n, maxp) > kMaxLds)
        n++;
    return (int32_t)std::min<int64_t>(n, kMaxSplits);
}

ada_status decode_common(const ada_geom *g, const ada_cache *c, const float *cb8, const float *cb4,
                         const uint16_t *q, float scale, float *out, float *lse, float *logits,
                         int32_t num_splits, void *ws, size_t ws_bytes, void *stream, bool dense,
                         unsigned stages = kStageAll, bool sym = false)
{
    if (!geom_ok(g) || !cache_ok(c) || q == nullptr || out == nullptr || num_splits < 0)
        return ADA_EINVAL;
    if (!dense && (cb8 == nullptr || cb4 == nullptr))
        return ADA_EINVAL;
    if (!gqa_supported(g))
        return ADA_EUNSUPPORTED;
    if (num_splits > kMaxSplits)
        return ADA_EINVAL;
    const int32_t ns = num_splits > 0 ? num_splits : default_splits(g, c->num_seqs, c->max_pages_per_head);
    const size_t need = ws_layout(g, c->num_seqs, ns, sym).total;
    if (ws == nullptr || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255))
        return ADA_EWORKSPACE;
    const int NH = g->num_q_heads / g->num_kv_heads;
    const int64_t rows = (int64_t)c->num_seqs * g->num_kv_heads;
    if (rows * ns > INT32_MAX)
        return ADA_EINVAL;
    if (decode_shmem_bytes(g->head_dim, NH, dense, ns, c->max_pages_per_head) > kMaxLds)
        return ADA_EINVAL; // too many pages per split: use more splits
    DecodeArgs a;
    a.trace = phase_trace_for((size_t)rows * ns * decode_waves(g->head_dim, NH));
    a.arena = c->arena;
    a.page_table = c->page_table;
    a.page_meta = c->page_meta;
    a.num_pages = c->num_pages;
    a.cb8 = cb8;
    a.cb4 = cb4;
    a.q = q;
    a.out = out;
    a.lse = lse;
    a.logits = logits;
    // workspace: [partial (m, l)][partial acc]
    uint8_t *w = static_cast<uint8_t *>(ws);
    const WsLayout lay = ws_layout(g, c->num_seqs, ns, sym);
    a.part_ml = reinterpret_cast<float *>(w + lay.ml_off);
    a.part_acc = reinterpret_cast<float *>(w + lay.acc_off);
    a.glut = sym ? reinterpret_cast<float *>(w + lay.lut_off) : nullptr;
    a.sigma = scale;
    a.S = c->num_seqs;
    a.Hq = g->num_q_heads;
    a.Hkv = g->num_kv_heads;
    a.maxp = c->max_pages_per_head;
    a.nsplit = ns;
    if (launch_decode(g->head_dim, NH, dense, a, as_stream(stream), stages, sym) != hipSuccess)
        return ADA_EHIP;
    return ADA_OK;
}

} // namespace

extern "C" {

const char *ada_status_str(int status)
{
    switch (status) {
    case ADA_OK: return "ok";
    case ADA_EINVAL: return "invalid argument";
    case ADA_EUNSUPPORTED: return "unsupported geometry";
    case ADA_ENOSPACE: return "arena full";
    case ADA_EWORKSPACE: return "workspace missing, misaligned or too small";
    case ADA_EHIP: return "HIP launch or copy failed";
    default: return "unknown status";
    }
}

int ada_version(void) { return kVersion; }

#ifndef ADA_BUILD_ID
#define ADA_BUILD_ID "unknown"
#endif
const char *ada_build_id(void) { return ADA_BUILD_ID; }

ada_status ada_phase_trace(void *buf, size_t bytes)
{
#ifdef ADA_PHASE_TRACE
    if (buf != nullptr && ((reinterpret_cast<uintptr_t>(buf) & 7) || bytes < 64))
        return ADA_EINVAL;
    g_trace_buf.store(nullptr);
    g_trace_bytes.store(buf != nullptr ? bytes : 0);
    g_trace_buf.store(buf);
    return ADA_OK;
#else
    (void)buf;
    (void)bytes;
    return ADA_EUNSUPPORTED;
#endif
}

size_t ada_page_bytes(int32_t head_dim, int32_t tier)
{
    if ((head_dim != 64 && head_dim != 128) || tier < 0 || tier > 3)
        return 0;
    return (size_t)page_bytes(head_dim, tier);
}

ada_status ada_encode(const ada_geom *geom, int64_t n_tokens, const uint16_t *keys, const float *cb8,
                      const float *cb4, uint16_t *radius, uint8_t *codes8, uint8_t *codes4,
                      void *stream)
{
    if (!geom_ok(geom) || n_tokens < 0 || n_tokens > ((int64_t)1 << 40))
        return ADA_EINVAL;
    if (n_tokens == 0)
        return ADA_OK;
    if (!keys || !cb8 || !cb4 || !radius || !codes8 || !codes4)
        return ADA_EINVAL;
    if ((reinterpret_cast<uintptr_t>(keys) & 15) || (reinterpret_cast<uintptr_t>(cb8) & 15) ||
        (reinterpret_cast<uintptr_t>(cb4) & 15) || (reinterpret_cast<uintptr_t>(radius) & 1))
        return ADA_EINVAL;
    return launch_encode(geom->head_dim, geom->num_kv_heads, n_tokens, keys, cb8, cb4, radius, codes8,
                         codes4, as_stream(stream)) == hipSuccess
               ? ADA_OK
               : ADA_EHIP;
}

ada_status rdr_pack_num_pages(const ada_geom *geom, int32_t num_seqs, const int32_t *cu_tokens_host,
                              const int32_t *tier_cum_bp_host, int64_t *n_pages_out)
{
    if (!geom_ok(geom) || num_seqs < 0 || !cu_ok(num_seqs, cu_tokens_host) || !tier_cum_bp_host ||
        !n_pages_out)
        return ADA_EINVAL;
    std::vector<int64_t> counts;
    if (!counts_from_bp(num_seqs, cu_tokens_host, tier_cum_bp_host, counts))
        return ADA_EINVAL;
    int64_t n = 0;
    for (int s = 0; s < num_seqs; s++)
        for (int k = 0; k < 3; k++)
            n += (counts[s * 3 + k] + kSlots - 1) / kSlots;
    *n_pages_out = n * geom->num_kv_heads;
    return ADA_OK;
}

size_t rdr_pack_workspace_size(const ada_geom *geom, int64_t n_tokens, int32_t num_seqs)
{
    if (!geom_ok(geom) || n_tokens < 0 || num_seqs < 0)
        return 0;
    return pack_workspace(geom->num_kv_heads, n_tokens, num_seqs);
}

ada_status rdr_pack(const ada_geom *geom, const ada_cache *cache, int32_t num_seqs,
                    const int32_t *cu_tokens_host, const int32_t *tier_cum_bp_host,
                    const uint16_t *keys, const uint16_t *values, const uint16_t *radius,
                    const uint8_t *codes8, const uint8_t *codes4, const float *scores,
                    const uint8_t *protect_host, const uint32_t *place_perm_host,
                    const int64_t *pos_base_host, uint64_t *arena_cursor_host,
                    int32_t *num_pages_host, void *ws, size_t ws_bytes, void *stream)
{
    if (!geom_ok(geom) || !cache_ok(cache) || num_seqs != cache->num_seqs || num_seqs < 0 ||
        !cu_ok(num_seqs, cu_tokens_host) || !tier_cum_bp_host || !arena_cursor_host ||
        !num_pages_host || cache->tier_tokens == nullptr)
        return ADA_EINVAL;
    const int64_t N = cu_tokens_host[num_seqs];
    if (N > 0 && (!keys || !values || !radius || !codes8 || !codes4 || !scores))
        return ADA_EINVAL;
    if (N > 0 && (reinterpret_cast<uintptr_t>(cache->arena) & 255))
        return ADA_EINVAL;
    std::vector<int64_t> counts;
    if (!counts_from_bp(num_seqs, cu_tokens_host, tier_cum_bp_host, counts))
        return ADA_EINVAL;
    if (protect_host != nullptr) {
        const int H = geom->num_kv_heads;
        for (int s = 0; s < num_seqs; s++)
            for (int h = 0; h < H; h++) {
                int64_t np = 0;
                for (int64_t i = cu_tokens_host[s]; i < cu_tokens_host[s + 1]; i++)
                    np += protect_host[i * H + h] != 0;
                if (np > counts[s * 3])
                    return ADA_EINVAL;
            }
    }
    return run_pack(geom, cache, num_seqs, cu_tokens_host, counts,
                    rows_of(num_seqs, geom->num_kv_heads, counts), nullptr, false, keys, values,
                    radius, codes8, codes4, scores, protect_host, place_perm_host, pos_base_host, arena_cursor_host,
                    num_pages_host, ws, ws_bytes, stream);
}

ada_status dense_pack(const ada_geom *geom, const ada_cache *cache, int32_t num_seqs,
                      const int32_t *cu_tokens_host, const uint16_t *keys, const uint16_t *values,
                      const uint32_t *place_perm_host, uint64_t *arena_cursor_host,
                      int32_t *num_pages_host, void *ws, size_t ws_bytes, void *stream)
{
    if (!geom_ok(geom) || !cache_ok(cache) || num_seqs != cache->num_seqs || num_seqs < 0 ||
        !cu_ok(num_seqs, cu_tokens_host) || !arena_cursor_host || !num_pages_host)
        return ADA_EINVAL;
    const int64_t N = cu_tokens_host[num_seqs];
    if (N > 0 && (!keys || !values))
        return ADA_EINVAL;
    std::vector<int64_t> counts((size_t)num_seqs * 3, 0);
    for (int s = 0; s < num_seqs; s++)
        counts[s * 3] = cu_tokens_host[s + 1] - cu_tokens_host[s];
    return run_pack(geom, cache, num_seqs, cu_tokens_host, counts,
                    rows_of(num_seqs, geom->num_kv_heads, counts), nullptr, true, keys, values,
                    nullptr, nullptr, nullptr, nullptr, nullptr, place_perm_host, nullptr, arena_cursor_host,
                    num_pages_host, ws, ws_bytes, stream);
}

ada_status ada_code_error(const ada_geom *geom, int64_t n_tokens, const uint16_t *keys, const float *cb8,
                          const float *cb4, const uint8_t *codes8, const uint8_t *codes4, float *err8,
                          float *err4, void *stream)
{
    if (!geom_ok(geom) || n_tokens < 0 || n_tokens > ((int64_t)1 << 40))
        return ADA_EINVAL;
    if (n_tokens == 0)
        return ADA_OK;
    if (!keys || !cb8 || !cb4 || !codes8 || !codes4 || !err8 || !err4)
        return ADA_EINVAL;
    if ((reinterpret_cast<uintptr_t>(keys) & 15) || (reinterpret_cast<uintptr_t>(cb8) & 15) ||
        (reinterpret_cast<uintptr_t>(cb4) & 15) || (reinterpret_cast<uintptr_t>(codes8) & 3) ||
        (reinterpret_cast<uintptr_t>(codes4) & 3))
        return ADA_EINVAL;
    if ((n_tokens * geom->num_kv_heads + 255) / 256 > INT32_MAX)
        return ADA_EINVAL;
    return launch_code_error(geom->head_dim, geom->num_kv_heads, n_tokens, keys, cb8, cb4, codes8, codes4,
                             err8, err4, as_stream(stream)) == hipSuccess
               ? ADA_OK
               : ADA_EHIP;
}

size_t rdr_solve_workspace_size(const ada_geom *geom, int32_t num_seqs, int64_t n_tokens)
{
    if (!geom_ok(geom) || num_seqs < 0 || n_tokens < 0)
        return 0;
    const int64_t blocks = n_tokens * geom->num_kv_heads / kSolveItems + num_seqs + 1;
    return align256(sizeof(SolveSeq) * (size_t)std::max(num_seqs, 1)) +
           align256(sizeof(SolveBlock) * (size_t)blocks) +
           align256(sizeof(unsigned long long) * kSolvePasses * 256 * (size_t)std::max(num_seqs, 1));
}

ada_status rdr_solve(const ada_geom *geom, int32_t num_seqs, const int32_t *cu_tokens_host,
                     const int64_t *budget_bytes_host, const uint16_t *radius, const float *err8,
                     const float *err4, const float *scores, const uint8_t *protect, uint8_t *tiers,
                     float *threshold, void *ws, size_t ws_bytes, void *stream)
{
    if (!geom_ok(geom) || num_seqs < 0 || !cu_ok(num_seqs, cu_tokens_host) || budget_bytes_host == nullptr)
        return ADA_EINVAL;
    const int H = geom->num_kv_heads, D = geom->head_dim;
    const int64_t N = cu_tokens_host[num_seqs];
    if (N > 0 && (!radius || !err8 || !err4 || !scores || !tiers))
        return ADA_EINVAL;
    for (int s = 0; s < num_seqs; s++)
        if (budget_bytes_host[s] < 0)
            return ADA_EINVAL;
    const size_t need_ws = rdr_solve_workspace_size(geom, num_seqs, N);
    if (ws == nullptr || ws_bytes < need_ws || (reinterpret_cast<uintptr_t>(ws) & 255))
        return ADA_EWORKSPACE;
    const int64_t R0 = page_bytes(D, 0) / kSlots, R1 = page_bytes(D, 1) / kSlots,
                  R2 = page_bytes(D, 2) / kSlots;
    const int64_t reserve = (int64_t)H * 15 * (R0 + R1 + R2);
    std::vector<SolveSeq> seqs(std::max(num_seqs, 1));
    std::vector<SolveBlock> blocks;
    for (int s = 0; s < num_seqs; s++) {
        const int64_t items = (int64_t)(cu_tokens_host[s + 1] - cu_tokens_host[s]) * H;
        seqs[s].begin = (int64_t)cu_tokens_host[s] * H;
        seqs[s].n_items = items;
        seqs[s].need = items * R0 - (budget_bytes_host[s] - reserve);
        for (int64_t f = 0; f < items; f += kSolveItems)
            blocks.push_back(SolveBlock{s, 0, seqs[s].begin + f});
    }
    if (blocks.size() > (size_t)INT32_MAX)
        return ADA_EINVAL;
    // workspace: [sequences][blocks][digit histograms]
    uint8_t *w = static_cast<uint8_t *>(ws);
    const size_t seq_bytes = align256(sizeof(SolveSeq) * seqs.size());
    const size_t blk_bytes = align256(sizeof(SolveBlock) * std::max<size_t>(blocks.size(), 1));
    std::vector<uint8_t> blob(seq_bytes + sizeof(SolveBlock) * blocks.size(), 0);
    std::memcpy(blob.data(), seqs.data(), sizeof(SolveSeq) * seqs.size());
    if (!blocks.empty())
        std::memcpy(blob.data() + seq_bytes, blocks.data(), sizeof(SolveBlock) * blocks.size());
    hipStream_t st = as_stream(stream);
    // pageable host source: the runtime copies it before returning
    if (hipMemcpyAsync(w, blob.data(), blob.size(), hipMemcpyHostToDevice, st) != hipSuccess)
        return ADA_EHIP;
    SolveArgs a;
    a.seqs = reinterpret_cast<const SolveSeq *>(w);
    a.blocks = reinterpret_cast<const SolveBlock *>(w + seq_bytes);
    a.hist = reinterpret_cast<unsigned long long *>(w + seq_bytes + blk_bytes);
    a.radius = radius;
    a.err8 = err8;
    a.err4 = err4;
    a.scores = scores;
    a.protect = protect;
    a.tiers = tiers;
    a.threshold = threshold;
    a.S = num_seqs;
    a.D = D;
    a.n_blocks = (int)blocks.size();
    return launch_solve(a, st) == hipSuccess ? ADA_OK : ADA_EHIP;
}

size_t rdr_tier_counts_workspace_size(const ada_geom *geom, int32_t num_seqs)
{
    if (!geom_ok(geom) || num_seqs < 0)
        return 0;
    return align256(sizeof(int32_t) * ((size_t)num_seqs + 1)) +
           align256(sizeof(int32_t) * 3 * (size_t)std::max<int64_t>((int64_t)num_seqs * geom->num_kv_heads, 1));
}

ada_status rdr_tier_counts(const ada_geom *geom, int32_t num_seqs, const int32_t *cu_tokens_host,
                           const uint8_t *tiers, int32_t *row_counts_host, void *ws, size_t ws_bytes,
                           void *stream)
{
    if (!geom_ok(geom) || num_seqs < 0 || !cu_ok(num_seqs, cu_tokens_host) || !row_counts_host)
        return ADA_EINVAL;
    const int H = geom->num_kv_heads;
    const int64_t rows = (int64_t)num_seqs * H;
    if (rows == 0)
        return ADA_OK;
    if (cu_tokens_host[num_seqs] > 0 && tiers == nullptr)
        return ADA_EINVAL;
    if (rows > INT32_MAX)
        return ADA_EINVAL;
    if (ws == nullptr || ws_bytes < rdr_tier_counts_workspace_size(geom, num_seqs) ||
        (reinterpret_cast<uintptr_t>(ws) & 255))
        return ADA_EWORKSPACE;
    uint8_t *w = static_cast<uint8_t *>(ws);
    int32_t *cu_dev = reinterpret_cast<int32_t *>(w);
    int32_t *counts = reinterpret_cast<int32_t *>(w + align256(sizeof(int32_t) * ((size_t)num_seqs + 1)));
    hipStream_t st = as_stream(stream);
    if (hipMemcpyAsync(cu_dev, cu_tokens_host, sizeof(int32_t) * ((size_t)num_seqs + 1),
                       hipMemcpyHostToDevice, st) != hipSuccess)
        return ADA_EHIP;
    if (launch_tier_counts(H, num_seqs, cu_dev, tiers, counts, st) != hipSuccess)
        return ADA_EHIP;
    if (hipMemcpyAsync(row_counts_host, counts, sizeof(int32_t) * 3 * (size_t)rows, hipMemcpyDeviceToHost,
                       st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return ADA_EHIP;
    return ADA_OK;
}

ada_status rdr_pack_tiers_num_pages(const ada_geom *geom, int32_t num_seqs, const int32_t *row_counts_host,
                                    int64_t *n_pages_out)
{
    if (!geom_ok(geom) || num_seqs < 0 || !row_counts_host || !n_pages_out)
        return ADA_EINVAL;
    int64_t n = 0;
    for (int64_t i = 0; i < (int64_t)num_seqs * geom->num_kv_heads * 3; i++) {
        if (row_counts_host[i] < 0)
            return ADA_EINVAL;
        n += (row_counts_host[i] + kSlots - 1) / kSlots;
    }
    *n_pages_out = n;
    return ADA_OK;
}

ada_status rdr_pack_tiers(const ada_geom *geom, const ada_cache *cache, int32_t num_seqs,
                          const int32_t *cu_tokens_host, const int32_t *row_counts_host, const uint8_t *tiers,
                          const uint16_t *keys, const uint16_t *values, const uint16_t *radius,
                          const uint8_t *codes8, const uint8_t *codes4, const uint32_t *place_perm_host,
                          const int64_t *pos_base_host, uint64_t *arena_cursor_host, int32_t *num_pages_host,
                          void *ws, size_t ws_bytes, void *stream)
{
    if (!geom_ok(geom) || !cache_ok(cache) || num_seqs != cache->num_seqs || num_seqs < 0 ||
        !cu_ok(num_seqs, cu_tokens_host) || !row_counts_host || !arena_cursor_host || !num_pages_host ||
        cache->tier_tokens == nullptr)
        return ADA_EINVAL;
    const int H = geom->num_kv_heads;
    const int64_t N = cu_tokens_host[num_seqs];
    if (N > 0 && (!tiers || !keys || !values || !radius || !codes8 || !codes4))
        return ADA_EINVAL;
    std::vector<int64_t> rc((size_t)num_seqs * H * 3);
    for (int s = 0; s < num_seqs; s++) {
        const int64_t T = cu_tokens_host[s + 1] - cu_tokens_host[s];
        for (int h = 0; h < H; h++) {
            int64_t tot = 0;
            for (int k = 0; k < 3; k++) {
                const int64_t n = row_counts_host[((int64_t)s * H + h) * 3 + k];
                if (n < 0)
                    return ADA_EINVAL;
                rc[((size_t)s * H + h) * 3 + k] = n;
                tot += n;
            }
            if (tot > T)
                return ADA_EINVAL;
        }
    }
    std::vector<int64_t> counts((size_t)num_seqs * 3, 0); // (the ranked path's; unused here)
    return run_pack(geom, cache, num_seqs, cu_tokens_host, counts, rc, tiers, false, keys, values, radius,
                    codes8, codes4, nullptr, nullptr, place_perm_host, pos_base_host, arena_cursor_host,
                    num_pages_host, ws, ws_bytes, stream);
}

ada_status rdr_pack_tiers_device(const ada_geom *geom, const ada_cache *cache, int32_t num_seqs,
                                 const int32_t *cu_tokens_host, const uint8_t *tiers, const uint16_t *keys,
                                 const uint16_t *values, const uint16_t *radius, const uint8_t *codes8,
                                 const uint8_t *codes4, const int64_t *pos_base_host, void *state, void *ws,
                                 size_t ws_bytes, void *stream)
{
    if (!geom_ok(geom) || !cache_ok(cache) || num_seqs != cache->num_seqs || num_seqs < 0 ||
        !cu_ok(num_seqs, cu_tokens_host) || cache->tier_tokens == nullptr || state == nullptr ||
        (reinterpret_cast<uintptr_t>(state) & 255))
        return ADA_EINVAL;
    const int H = geom->num_kv_heads;
    const int64_t N = cu_tokens_host[num_seqs];
    if (N > 0 && (!tiers || !keys || !values || !radius || !codes8 || !codes4))
        return ADA_EINVAL;
    if (N > 0 && ((reinterpret_cast<uintptr_t>(cache->arena) & 255) || (reinterpret_cast<uintptr_t>(keys) & 15) ||
                  (reinterpret_cast<uintptr_t>(values) & 15) || (reinterpret_cast<uintptr_t>(codes8) & 3) ||
                  (reinterpret_cast<uintptr_t>(codes4) & 3) || (reinterpret_cast<uintptr_t>(radius) & 1)))
        return ADA_EINVAL;
    if (ws == nullptr || ws_bytes < pack_workspace(H, N, num_seqs) || (reinterpret_cast<uintptr_t>(ws) & 255))
        return ADA_EWORKSPACE;
    if (N == 0)
        return ADA_OK;
    // the host plans only where each row's page list goes: a range sized
    // for the row's tokens (at most one partial page per tier)
    const int64_t rows = (int64_t)num_seqs * H;
    std::vector<PackSeq> seqs(num_seqs);
    std::vector<PackRow> rowv(rows);
    int64_t n = 0;
    for (int s = 0; s < num_seqs; s++) {
        seqs[s].begin = cu_tokens_host[s];
        seqs[s].len = cu_tokens_host[s + 1] - cu_tokens_host[s];
        seqs[s].n_cum[0] = seqs[s].n_cum[1] = seqs[s].n_cum[2] = 0;
        seqs[s].pad = 0;
        seqs[s].pos_base = pos_base_host ? pos_base_host[s] : 0;
        const int64_t cap = (seqs[s].len + kSlots - 1) / kSlots + 2;
        for (int h = 0; h < H; h++) {
            PackRow &r = rowv[(int64_t)s * H + h];
            std::memset(&r, 0, sizeof(r));
            r.lp_first[0] = (int32_t)n; // first entry of the row's range
            r.lp_first[1] = (int32_t)cap; // its length
            n += cap;
        }
    }
    if (n > max_pack_pages(H, N, num_seqs) || n > INT32_MAX)
        return ADA_EWORKSPACE;
    uint8_t *wsb = static_cast<uint8_t *>(ws);
    const size_t seq_off = 0, row_off = align256(sizeof(PackSeq) * (size_t)std::max(num_seqs, 1));
    const size_t page_off = row_off + align256(sizeof(PackRow) * (size_t)std::max<int64_t>(rows, 1));
    const size_t blob_cap = page_off + align256(sizeof(PackPage) * (size_t)max_pack_pages(H, N, num_seqs));
    std::vector<uint8_t> blob(page_off, 0);
    std::memcpy(blob.data() + seq_off, seqs.data(), sizeof(PackSeq) * seqs.size());
    std::memcpy(blob.data() + row_off, rowv.data(), sizeof(PackRow) * rowv.size());
    hipStream_t st = as_stream(stream);
    // pageable host source: the runtime copies it before returning
    if (hipMemcpyAsync(wsb, blob.data(), blob.size(), hipMemcpyHostToDevice, st) != hipSuccess)
        return ADA_EHIP;
    uint8_t *st8 = static_cast<uint8_t *>(state);
    PackPlan plan;
    plan.seqs = reinterpret_cast<const PackSeq *>(wsb + seq_off);
    plan.rows = reinterpret_cast<const PackRow *>(wsb + row_off);
    plan.pages = reinterpret_cast<PackPage *>(wsb + page_off);
    plan.protect = nullptr;
    plan.tiers = tiers;
    plan.src = reinterpret_cast<int32_t *>(wsb + blob_cap + align256((size_t)N * H));
    plan.S = num_seqs;
    plan.Hkv = H;
    plan.D = geom->head_dim;
    plan.maxp = cache->max_pages_per_head;
    plan.n_pages = (int)n;
    plan.dense = 0;
    plan.gen_pages = 1;
    plan.n_tokens = N;
    plan.dev_plan = 1;
    plan.cursor = reinterpret_cast<unsigned long long *>(st8);
    plan.status = reinterpret_cast<unsigned int *>(st8 + 8);
    plan.capacity = cache->arena_units;
    PackData data{keys, values, radius, codes8, codes4, nullptr};
    PackCache pc{cache->arena, cache->page_table, cache->page_meta, cache->num_pages, cache->tier_tokens,
                 cache->slot_token};
    return launch_pack(plan, data, pc, st) == hipSuccess ? ADA_OK : ADA_EHIP;
}

int32_t ada_decode_default_splits(const ada_geom *geom, int32_t num_seqs, int32_t max_pages_per_head)
{
    if (!geom_ok(geom) || num_seqs < 0 || max_pages_per_head < 0)
        return 0;
    return default_splits(geom, num_seqs, max_pages_per_head);
}

size_t ada_decode_workspace_size(const ada_geom *geom, int32_t num_seqs, int32_t max_pages_per_head,
                                 int32_t num_splits)
{
    if (!geom_ok(geom) || num_seqs < 0 || max_pages_per_head < 0 || num_splits < 0)
        return 0;
    const int32_t ns = num_splits > 0 ? num_splits : default_splits(geom, num_seqs, max_pages_per_head);
    return ws_layout(geom, num_seqs, ns).total;
}

ada_status ada_decode(const ada_geom *geom, const ada_cache *cache, const float *cb8, const float *cb4,
                      const uint16_t *q, float softmax_scale, float *out, float *lse,
                      float *logits_dbg, int32_t num_splits, void *ws, size_t ws_bytes, void *stream)
{
    return decode_common(geom, cache, cb8, cb4, q, softmax_scale, out, lse, logits_dbg, num_splits, ws,
                         ws_bytes, stream, false);
}

ada_status ada_decode_noalloc(const ada_geom *geom, const ada_cache *cache, const float *cb8,
                              const float *cb4, const uint16_t *q, float softmax_scale, float *out,
                              float *lse, float *logits_dbg, int32_t num_splits, void *stream)
{
    static_assert(ADA_NOALLOC_SCRATCH_BYTES == kNoAllocScratchBytes, "scratch size of the header");
    if (!geom_ok(geom) || !cache_ok(cache) || num_splits < 0 || num_splits > kMaxSplits)
        return ADA_EINVAL;
    const int32_t ns = num_splits > 0 ? num_splits : default_splits(geom, cache->num_seqs, cache->max_pages_per_head);
    if (ws_layout(geom, cache->num_seqs, ns).total > kNoAllocScratchBytes)
        return ADA_EWORKSPACE; // the partials would not fit in the library's array
    void *scr = nullptr;
    if (noalloc_scratch(&scr) != hipSuccess)
        return ADA_EHIP;
    return decode_common(geom, cache, cb8, cb4, q, softmax_scale, out, lse, logits_dbg, num_splits, scr,
                         kNoAllocScratchBytes, stream, false);
}

ada_status ada_decode_stream(const ada_geom *geom, const ada_cache *cache, const float *cb8,
                             const float *cb4, const uint16_t *q, float softmax_scale, float *out,
                             float *lse, float *logits_dbg, int32_t num_splits, void *ws,
                             size_t ws_bytes, void *stream)
{
    return decode_common(geom, cache, cb8, cb4, q, softmax_scale, out, lse, logits_dbg, num_splits, ws,
                         ws_bytes, stream, false, kStageStream);
}

ada_status ada_decode_merge(const ada_geom *geom, const ada_cache *cache, const float *cb8,
                            const float *cb4, const uint16_t *q, float softmax_scale, float *out,
                            float *lse, int32_t num_splits, void *ws, size_t ws_bytes, void *stream)
{
    return decode_common(geom, cache, cb8, cb4, q, softmax_scale, out, lse, nullptr, num_splits, ws,
                         ws_bytes, stream, false, kStageMerge);
}

size_t ada_append_state_bytes(const ada_geom *geom, int32_t num_seqs)
{
    if (!geom_ok(geom) || num_seqs < 0)
        return 0;
    return 256 + align256(sizeof(int32_t) * 3 * (size_t)std::max<int64_t>((int64_t)num_seqs * geom->num_kv_heads, 1));
}

ada_status ada_append(const ada_geom *geom, const ada_cache *cache, const float *cb8, const float *cb4,
                      const uint16_t *keys, const uint16_t *values, const float *scores, const uint8_t *protect,
                      const float *threshold, const int64_t *pos, uint8_t *tiers_out, void *state, void *stream)
{
    if (!geom_ok(geom) || !cache_ok(cache) || cache->tier_tokens == nullptr || !cb8 || !cb4 || !keys ||
        !values || !scores || !threshold || !pos || !state)
        return ADA_EINVAL;
    if ((reinterpret_cast<uintptr_t>(state) & 255) || (reinterpret_cast<uintptr_t>(keys) & 3) ||
        (reinterpret_cast<uintptr_t>(values) & 3) || (reinterpret_cast<uintptr_t>(cb8) & 15) ||
        (reinterpret_cast<uintptr_t>(cb4) & 15) || (reinterpret_cast<uintptr_t>(cache->arena) & 15))
        return ADA_EINVAL;
    const int64_t rows = (int64_t)cache->num_seqs * geom->num_kv_heads;
    if (rows > INT32_MAX)
        return ADA_EINVAL;
    uint8_t *st8 = static_cast<uint8_t *>(state);
    AppendArgs a;
    a.arena = cache->arena;
    a.page_table = cache->page_table;
    a.page_meta = cache->page_meta;
    a.num_pages = cache->num_pages;
    a.tier_tokens = cache->tier_tokens;
    a.slot_token = cache->slot_token;
    a.cb8 = cb8;
    a.cb4 = cb4;
    a.keys = keys;
    a.values = values;
    a.scores = scores;
    a.protect = protect;
    a.threshold = threshold;
    a.pos = pos;
    a.tiers_out = tiers_out;
    a.cursor = reinterpret_cast<unsigned long long *>(st8);
    a.status = reinterpret_cast<unsigned int *>(st8 + 8);
    a.open = reinterpret_cast<int32_t *>(st8 + 256);
    a.capacity = cache->arena_units;
    a.maxp = cache->max_pages_per_head;
    a.Hkv = geom->num_kv_heads;
    return launch_append(geom->head_dim, a, (int)rows, as_stream(stream)) == hipSuccess ? ADA_OK : ADA_EHIP;
}

ada_status ada_retier(const ada_geom *geom, const ada_cache *cache, const float *cb8, const float *cb4,
                      int32_t n, const int32_t *rows, const int32_t *pages, const uint8_t *target, void *state,
                      void *stream)
{
    if (!geom_ok(geom) || !cache_ok(cache) || cache->tier_tokens == nullptr || !cb8 || !cb4 || !state || n < 0)
        return ADA_EINVAL;
    if (n > 0 && (!rows || !pages || !target))
        return ADA_EINVAL;
    if ((reinterpret_cast<uintptr_t>(state) & 255) || (reinterpret_cast<uintptr_t>(cb8) & 15) ||
        (reinterpret_cast<uintptr_t>(cb4) & 15) || (reinterpret_cast<uintptr_t>(cache->arena) & 15))
        return ADA_EINVAL;
    const int64_t nrows = (int64_t)cache->num_seqs * geom->num_kv_heads;
    if (nrows > INT32_MAX)
        return ADA_EINVAL;
    uint8_t *st8 = static_cast<uint8_t *>(state);
    RetierArgs a;
    a.arena = cache->arena;
    a.page_table = cache->page_table;
    a.page_meta = cache->page_meta;
    a.num_pages = cache->num_pages;
    a.tier_tokens = cache->tier_tokens;
    a.slot_token = cache->slot_token;
    a.cb8 = cb8;
    a.cb4 = cb4;
    a.rows = rows;
    a.pages = pages;
    a.target = target;
    a.cursor = reinterpret_cast<unsigned long long *>(st8);
    a.status = reinterpret_cast<unsigned int *>(st8 + 8);
    a.open = reinterpret_cast<int32_t *>(st8 + 256);
    a.capacity = cache->arena_units;
    a.n = n;
    a.maxp = cache->max_pages_per_head;
    a.Hkv = geom->num_kv_heads;
    a.nrows = (int)nrows;
    return launch_retier(geom->head_dim, a, (int)nrows, as_stream(stream)) == hipSuccess ? ADA_OK : ADA_EHIP;
}

ada_status ada_retier_plan(const ada_geom *geom, int32_t num_seqs, const int64_t *budget_bytes_host,
                           const int32_t *num_pages_host, const uint8_t *page_meta_host,
                           int32_t max_pages_per_head, int32_t demote_to, int32_t cap, int32_t *rows_out,
                           int32_t *pages_out, uint8_t *target_out, int32_t *n_out)
{
    if (!geom_ok(geom) || num_seqs < 0 || !budget_bytes_host || !num_pages_host || !page_meta_host ||
        max_pages_per_head < 0 || (demote_to != 1 && demote_to != 2) || cap < 0 || !n_out ||
        (cap > 0 && (!rows_out || !pages_out || !target_out)))
        return ADA_EINVAL;
    const int H = geom->num_kv_heads, D = geom->head_dim;
    int32_t n = 0;
    for (int s = 0; s < num_seqs; s++) {
        int64_t bytes = 0;
        int32_t deepest = 0;
        for (int h = 0; h < H; h++) {
            const int64_t r = (int64_t)s * H + h;
            const int32_t np = num_pages_host[r];
            if (np < 0 || np > max_pages_per_head)
                return ADA_EINVAL;
            for (int32_t q = 0; q < np; q++)
                bytes += page_bytes(D, page_meta_host[r * max_pages_per_head + q] & 3);
            deepest = std::max(deepest, np);
        }
        // passes over (page index, head): demote full fp16 pages; evict coded
        // pages; evict the remaining (partial) fp16 pages
        for (int pass = 0; pass < 3 && bytes > budget_bytes_host[s]; pass++) {
            for (int32_t q = 0; q < deepest && bytes > budget_bytes_host[s]; q++) {
                for (int h = 0; h < H && bytes > budget_bytes_host[s]; h++) {
                    const int64_t r = (int64_t)s * H + h;
                    if (q >= num_pages_host[r])
                        continue;
                    const uint8_t m = page_meta_host[r * max_pages_per_head + q];
                    const int tier = m & 3;
                    const bool full = ((m >> 2) & 15) == 15;
                    int tgt = 0;
                    if (pass == 0 && tier == 0 && full)
                        tgt = demote_to;
                    else if (pass == 1 && (tier == 1 || tier == 2))
                        tgt = 3;
                    else if (pass == 2 && tier == 0 && !full)
                        tgt = 3;
                    if (tgt == 0)
                        continue;
                    if (n == cap) {
                        *n_out = n;
                        return ADA_OK;
                    }
                    rows_out[n] = (int32_t)r;
                    pages_out[n] = q;
                    target_out[n] = (uint8_t)tgt;
                    n++;
                    bytes -= tgt == 3 ? page_bytes(D, tier) : page_bytes(D, 0) - page_bytes(D, tgt);
                }
            }
        }
    }
    *n_out = n;
    return ADA_OK;
}

size_t ada_decode_sym_workspace_size(const ada_geom *geom, int32_t num_seqs, int32_t max_pages_per_head,
                                     int32_t num_splits)
{
    if (!geom_ok(geom) || num_seqs < 0 || max_pages_per_head < 0 || num_splits < 0)
        return 0;
    const int32_t ns = num_splits > 0 ? num_splits : default_splits(geom, num_seqs, max_pages_per_head);
    return ws_layout(geom, num_seqs, ns, true).total;
}

ada_status ada_decode_sym(const ada_geom *geom, const ada_cache *cache, const float *cb8, const float *cb4,
                          const uint16_t *q, float softmax_scale, float *out, float *lse, float *logits_dbg,
                          int32_t num_splits, void *ws, size_t ws_bytes, void *stream)
{
    return decode_common(geom, cache, cb8, cb4, q, softmax_scale, out, lse, logits_dbg, num_splits, ws,
                         ws_bytes, stream, false, kStageAll, true);
}

ada_status dense_decode(const ada_geom *geom, const ada_cache *cache, const uint16_t *q,
                        float softmax_scale, float *out, float *lse, float *logits_dbg,
                        int32_t num_splits, void *ws, size_t ws_bytes, void *stream)
{
    return decode_common(geom, cache, nullptr, nullptr, q, softmax_scale, out, lse, logits_dbg,
                         num_splits, ws, ws_bytes, stream, true);
}

} // extern "C"
