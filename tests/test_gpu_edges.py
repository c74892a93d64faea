"""GPU edge cases of the C ABI: entries and inputs that must do nothing, run
to run determinism, guard bytes around outputs, and calls on a stream other
than torch's current one."""
import numpy as np
import pytest
import torch

import compressed_kv_attention_amd as ada
import oracle
import synth
from gpu_util import flush, geom_of, gpu_encode, to_dev, upload_cache
from helpers import make_case, oracle_cache, small_workload

pytestmark = pytest.mark.gpu


def _gpu_layer(number, layer=0):
    """Workload `number` encoded and packed on the GPU (its benchmark cache)."""
    cfg = synth.WORKLOADS[number]
    H, D = cfg.num_kv_heads, cfg.head_dim
    geom = ada.Geom(D, cfg.num_q_heads, H)
    lens = synth.seq_lens(cfg)
    cu = synth.cu_tokens(lens)
    N = int(cu[-1])
    bp = synth.tier_mix(cfg)
    keys = synth.keys(cfg, layer, N, "cuda")
    vals = synth.values(cfg, layer, N, "cuda")
    cb8, cb4 = (t.cuda() for t in synth.codebooks(cfg, layer))
    r, c8, c4 = gpu_encode(geom, keys, cb8, cb4)
    maxp = int(max(lens)) // 16 + 4
    dc = ada.Cache(geom, cfg.num_seqs, maxp, N * H * 512 + (1 << 20))
    ada.rdr_pack(geom, dc, cu, bp, keys, vals, r, c8, c4, synth.scores(cfg, layer, N).cuda(),
                 place_perm=synth.place_perm(cfg, layer, ada.pack_num_pages(geom, cu, bp)))
    torch.cuda.synchronize()
    return cfg, geom, dc, cb8, cb4, synth.queries(cfg, layer, "cuda")


def test_retier_entries_that_cannot_apply_on_the_gpu():
    """As the oracle: tier-3 pages are not evicted, rows outside the cache and
    unknown targets are skipped; each sets status bit 4 and nothing moves."""
    cfg = small_workload(D=64, Hq=2, Hkv=2, S=1, T=50, seed=47)
    geom = geom_of(cfg)
    case = make_case(cfg, lens=[50])
    dc = ada.Cache(geom, 1, 8, 1 << 20)
    ada.dense_pack(geom, dc, case["cu"], to_dev(case["keys"]), to_dev(case["values"]))
    dc.tier_tokens[:2] = torch.tensor([[50, 0, 0], [50, 0, 0]], dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    snap = [t.clone() for t in (dc.page_table, dc.page_meta, dc.num_pages, dc.arena, dc.tier_tokens)]
    cb8, cb4 = to_dev(case["cb8"]), to_dev(case["cb4"])
    for rows, pages, tgt in (([0], [1], [3]), ([1], [0], [1]), ([2], [0], [3]), ([-1], [0], [2]),
                             ([0], [0], [0]), ([0], [0], [4])):
        st = ada.AppendState(geom, dc)
        ada.retier(geom, dc, st, cb8, cb4, torch.tensor(rows, dtype=torch.int32, device="cuda"),
                   torch.tensor(pages, dtype=torch.int32, device="cuda"),
                   torch.tensor(tgt, dtype=torch.uint8, device="cuda"))
        assert st.pull() == 4, (rows, pages, tgt)
        for a, b in zip(snap, (dc.page_table, dc.page_meta, dc.num_pages, dc.arena, dc.tier_tokens)):
            assert torch.equal(a, b)
    flush("[retier] unusable entries: bit 4, nothing moved")


def test_rdr_solve_with_no_tokens():
    """Sequences with no tokens: nothing to tier; each threshold is -inf when
    the budget covers the reserve, else +inf (as the oracle gives them)."""
    geom = ada.Geom(128, 32, 8)
    cu = np.array([0, 0, 0], np.int32)
    budgets = np.array([0, 1 << 30], np.int64)
    th = torch.full((2,), float("nan"), device="cuda")
    z16 = torch.empty((0, 8), dtype=torch.float16, device="cuda")
    z32 = torch.empty((0, 8), device="cuda")
    tiers = torch.empty((0, 8), dtype=torch.uint8, device="cuda")
    ada.rdr_solve(geom, cu, budgets, z16, z32, z32, z32, tiers, threshold=th)
    torch.cuda.synchronize()
    _, ref = oracle.rdr_solve(128, cu, budgets, np.zeros((0, 8), np.uint16), np.zeros((0, 8), np.float32),
                              np.zeros((0, 8), np.float32), np.zeros((0, 8), np.float32), with_threshold=True)
    assert np.array_equal(th.cpu().numpy(), ref) and np.isinf(ref).all()


@pytest.mark.parametrize("splits", [0, 1, 5])
def test_decode_run_twice_bitwise_identical(splits):
    """The split merge adds partials in a fixed order: two runs of the same
    step give the same bits (ADA, symmetric variant and dense baseline)."""
    cfg, geom, dc, cb8, cb4, q = _gpu_layer(2)
    S, Hq, D = cfg.num_seqs, cfg.num_q_heads, cfg.head_dim
    res = []
    for _ in range(2):
        o = torch.empty((S, Hq, D), device="cuda")
        l = torch.empty((S, Hq), device="cuda")
        ada.decode(geom, dc, cb8, cb4, q, cfg.sigma, o, l, num_splits=splits)
        oy = torch.empty_like(o)
        ly = torch.empty_like(l)
        ada.decode_sym(geom, dc, cb8, cb4, q, cfg.sigma, oy, ly, num_splits=splits)
        torch.cuda.synchronize()
        res.append((o, l, oy, ly))
    for a, b in zip(*res):
        assert torch.equal(a, b)
    flush(f"[determinism] splits={splits}: two runs bitwise identical")


def test_decode_writes_nothing_outside_its_outputs():
    """Outputs placed inside larger buffers filled with a guard pattern: after
    decode (and the symmetric and dense variants) every guard byte is intact."""
    cfg = small_workload(D=128, Hq=8, Hkv=2, S=3, T=300, seed=71)
    case = make_case(cfg, lens=[300, 17, 150])
    hc, _ = oracle_cache(case)
    geom = geom_of(cfg)
    dc = upload_cache(hc, geom)
    S, Hq, D = 3, 8, 128
    G = 4096  # guard floats on each side
    pat = float.fromhex("0x1.5a5a5ap+3")

    def guarded(n):
        buf = torch.full((n + 2 * G,), pat, device="cuda")
        return buf, buf[G:G + n]

    for kind in ("ada", "sym"):
        for splits in (0, 1, 4):
            ob, o = guarded(S * Hq * D)
            lb, l = guarded(S * Hq)
            gb, g = guarded(S * Hq * hc.maxp * 16)
            args = (geom, dc, to_dev(case["cb8"]), to_dev(case["cb4"]), to_dev(case["q"]), cfg.sigma,
                    o.view(S, Hq, D), l.view(S, Hq), g.view(S, Hq, hc.maxp * 16))
            (ada.decode if kind == "ada" else ada.decode_sym)(*args, num_splits=splits)
            torch.cuda.synchronize()
            for b in (ob, lb, gb):
                assert (b[:G] == pat).all() and (b[-G:] == pat).all(), (kind, splits)
            assert not torch.isnan(o).any() and not (o == pat).all()
    flush("[guards] outputs stay inside their buffers")


def test_calls_on_a_side_stream_match_the_current_stream():
    """Every call takes its stream argument: decode on a side stream, with the
    workspace allocated by the binding, gives the current stream's bits."""
    cfg, geom, dc, cb8, cb4, q = _gpu_layer(2)
    S, Hq, D = cfg.num_seqs, cfg.num_q_heads, cfg.head_dim
    o0 = torch.empty((S, Hq, D), device="cuda")
    ada.decode(geom, dc, cb8, cb4, q, cfg.sigma, o0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(4):
        with torch.cuda.stream(side):
            o = torch.empty((S, Hq, D), device="cuda")
        ada.decode(geom, dc, cb8, cb4, q, cfg.sigma, o, stream=side)  # ws allocated on `side`
        outs.append(o)
    side.synchronize()
    for o in outs:
        assert torch.equal(o, o0)
