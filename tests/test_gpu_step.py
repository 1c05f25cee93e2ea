"""GPU parity of the whole decode step (decode_step through the C ABI) against
the oracle's decode_step_ref: page bytes after the step's row store exact,
top-k within the near-tie rule, output within the attention tolerance.

Small workloads are checked on every sequence; the full-size ones (256K
context, B = 32) in the launch configuration the bench times, on sampled
sequences the oracle recomputes one by one.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as OF
from oracle import indexer as OI
from oracle import step as OS
from tests import parity as PT

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_decode_mxfp4_amd as m
    m.lib()
    return m


def run_step(mx, inp, num_partitions=0):
    import workloads.gpu as WG
    wl = inp.wl
    pools = WG.fill_prefix(inp, WG.empty_pools(inp))
    cache = WG.make_cache(inp, pools)
    t = WG.step_tensors(inp)
    table = torch.empty((wl.B, wl.q, wl.topk), dtype=torch.int32, device="cuda")
    scores = torch.empty((wl.B, wl.q, inp.max_pages), dtype=torch.float32, device="cuda")
    step = mx.DecodeStep(cache, t["query"], t["q_idx"], t["w"], wl.topk, wl.sm_scale,
                         k_new=t.get("k_new"), v_new=t.get("v_new"), idx_new=t.get("idx_new"),
                         num_partitions=num_partitions, block_table_out=table, scores_out=scores)
    step.run()
    torch.cuda.synchronize()
    return {"pools": {s: p.cpu().numpy() for s, p in pools.items()}, "table": table.cpu().numpy(),
            "scores": scores.cpu().numpy().astype(np.float64), "O": step.out.float().cpu().numpy(),
            "lse": step.lse.cpu().numpy()}


def check_step(inp, g, seqs):
    wl = inp.wl
    r = OS.decode_step_ref(inp, seqs=seqs)
    fmts = {"k": wl.kv_format, "v": wl.kv_format, "idx": wl.idx_format}
    qa, _ = OS.attention_query(inp)
    qI = OF.bf16_to_f64(inp.q_idx)
    n_equal = n_rows = 0
    for b in seqs:
        L = int(inp.contexts[b])
        pages = PT.seq_pages(inp.page_table[b], L)
        for s, f in fmts.items():
            PT.compare_pool_pages(g["pools"][s], r["pools"][s], pages, OF.PAGE_BYTES[f], f"{wl.name} {s} b={b}")
        kI = OF.READ[wl.idx_format](r["pools"]["idx"], inp.page_table[b], L)
        Sa = PT.score_bound(kI, qI[b], inp.w[b].astype(np.float64), L)
        nc = OI.n_candidates(L, wl.q)
        PT.check_scores(g["scores"][b], r["scores"][b][:, :Sa.shape[1]], Sa, nc)
        same = []
        for j in range(wl.q):
            same.append(PT.check_topk(g["table"][b, j], r["block_table"][b, j], r["scores"][b, j], int(nc[j]),
                                      wl.topk))
        # attention over the GPU's own selection, every row
        Oref, lref, _, _ = PT.oracle_attention_with_table(inp, r["pools"], qa, g["table"][b], b)
        PT.check_attention(g["O"][b], Oref, f"{wl.name} b={b}")
        np.testing.assert_allclose(g["lse"][b], lref, rtol=1e-4, atol=1e-4)
        # end to end, on the rows whose selection equals the oracle's
        for j in range(wl.q):
            n_rows += 1
            if same[j]:
                n_equal += 1
                PT.check_attention(g["O"][b, j], r["O"][b, j], f"{wl.name} b={b} j={j} end-to-end")
    assert n_equal >= 0.9 * n_rows, f"only {n_equal}/{n_rows} rows select the oracle's exact set"


@pytest.mark.parametrize("name", ["tiny", "fp8", "mxfp4_65k", "nvfp4"])
def test_decode_step_small(mx, name):
    inp = W.make_inputs(W.WORKLOADS[name])
    g = run_step(mx, inp)
    check_step(inp, g, range(inp.wl.B))


def test_decode_step_saturating_query(mx):
    """The 65K workload with +-500 and +-inf injected into the query: the e4m3
    store saturates them to +-448 and the step stays finite and in parity."""
    inp = W.make_inputs(W.WORKLOADS["mxfp4_65k"], inject_q=True)
    g = run_step(mx, inp)
    check_step(inp, g, [0, 3])


@pytest.mark.parametrize("P", [1, 64])
def test_decode_step_partition_counts(mx, P):
    inp = W.make_inputs(W.WORKLOADS["mxfp4_65k"].with_(B=2))
    g = run_step(mx, inp, num_partitions=P)
    check_step(inp, g, [0, 1])


@pytest.mark.parametrize("kw,P", [
    (dict(B=1, q=6, topk=16), 4),     # 24 workgroups dealt to the XCDs in runs of 3: each row's 4 partitions split
    (dict(B=1, q=3, topk=16), 3),     # 9 workgroups (not a multiple of 8): every row spread over several XCDs
    (dict(B=2, q=8, topk=32), 8),     # runs of 16: every row on one XCD (its merge reads through that L2)
])
def test_decode_step_rows_on_one_or_several_xcds(mx, kw, P):
    """The row merge reads its partials through the L2 only when every
    partition of the row ran on the merging workgroup's XCD, and with
    device-coherent loads otherwise: both paths, and rows that straddle two
    XCDs' runs of work items."""
    wl = W.WORKLOADS["mxfp4_65k"].with_(name="xcd", **kw)
    inp = W.make_inputs(wl)
    g = run_step(mx, inp, num_partitions=P)
    check_step(inp, g, range(wl.B))


@pytest.mark.parametrize("kw", [
    dict(ctx_rule=("list", (9, 130, 1000, 4096)), B=4, q=8, H=16, topk=16),      # contexts near q, ragged
    dict(ctx_rule=("list", (8, 300)), B=2, q=8, H=1, H_I=1, topk=64),            # L == q; H = 1; H_I = 1
    dict(ctx_rule=("list", (5000, 3000)), B=2, q=16, H=7, H_I=3, topk=5),        # q = 16, odd head counts
    dict(ctx_rule=("list", (2048,)), B=1, q=1, H=4, H_I=2, topk=16),             # top-k covers every block
])
def test_decode_step_edge_shapes(mx, kw):
    wl = W.WORKLOADS["mxfp4_65k"].with_(name="edge", **kw)
    inp = W.make_inputs(wl)
    g = run_step(mx, inp)
    check_step(inp, g, range(wl.B))


def test_decode_step_empty_batch(mx):
    import workloads.gpu as WG
    inp = W.make_inputs(W.WORKLOADS["tiny"])
    pools = WG.fill_prefix(inp, WG.empty_pools(inp))
    cache = WG.make_cache(inp, pools)
    t = WG.step_tensors(inp)
    q0 = t["query"][:0]
    step = mx.DecodeStep(cache, q0, t["q_idx"][:0], t["w"][:0], 4, 0.1)
    step.run()
    torch.cuda.synchronize()
    assert step.out.numel() == 0


# One GPU run per full-size workload (and partition count), kept while its
# sequences are checked one test at a time; the oracle recomputes each
# sequence on its own.
_RUNS = {}


def cached_run(mx, name, P=0, **kw):
    key = (name, P, tuple(sorted(kw.items())))
    if key not in _RUNS:
        _RUNS.clear()
        wl = W.WORKLOADS[name].with_(**kw) if kw else W.WORKLOADS[name]
        inp = W.make_inputs(wl)
        _RUNS[key] = (inp, run_step(mx, inp, num_partitions=P))
    return _RUNS[key]


B32_SEQS = (0, 4, 9, 13, 17, 22, 26, 31)


@pytest.mark.parametrize("name,b", [("headline", b) for b in range(4)] + [("long", b) for b in range(4)]
                         + [("b32", b) for b in B32_SEQS] + [("headline_nvfp4", b) for b in (0, 3)])
def test_decode_step_full_size(mx, name, b):
    """The bench's workloads in the launch configuration it times: every
    sequence of the 256K and ragged 128K-256K steps, 8 of the 32 sequences of
    the B = 32 step, 2 of the 4 sequences of the 256K step over NVFP4 caches,
    each against the oracle's step for that sequence."""
    inp, g = cached_run(mx, name)
    check_step(inp, g, [b])
    if b == 0:
        # every row of every sequence: finite output and a valid selection
        # (min(k, candidates) ascending ids below the row's candidate count)
        assert np.isfinite(g["O"]).all()
        for bb in range(inp.wl.B):
            nc = OI.n_candidates(int(inp.contexts[bb]), inp.wl.q)
            for j in range(inp.wl.q):
                sel = g["table"][bb, j]
                k = min(inp.wl.topk, int(nc[j]))
                assert (sel[:k] >= 0).all() and (np.diff(sel[:k]) > 0).all() and sel[k - 1] < nc[j]
                assert (sel[k:] == -1).all()


@pytest.mark.parametrize("b", [0, 3])
def test_decode_step_long_with_empty_partitions(mx, b):
    """The ragged 128K-256K workload with 24 partitions for top-k 32: each
    partition holds ceil(32 / 24) = 2 slots, so partitions 16..23 of every
    row are empty and merge in as (-inf, 0, 0)."""
    inp, g = cached_run(mx, "long", P=24)
    check_step(inp, g, [b])


@pytest.mark.parametrize("kw", [
    # 4-wave x 1-page scorer workgroups (4 pages each): the 8 new rows at 508..515 and
    # 1020..1027 fall on both sides of a workgroup boundary (pages 3 | 4 and 7 | 8)
    dict(B=2, ctx_rule=("list", (516, 1028)), topk=16),
    # 4 x 4 pages (16-page workgroups; 4096 pages in all): boundaries at 2048-token multiples
    dict(B=4, ctx_rule=("list", (131072, 2052, 4100, 8196)), topk=16),
    # the same shape at the headline's 8192 pages (the single-launch step's 32-page
    # scoring workgroups have boundaries at 4096-token multiples: the same positions)
    dict(B=4, ctx_rule=("list", (262144, 4100, 8196, 65540)), topk=32),
    # 16-page workgroups again, the new rows split between two pages of one wave:
    # 4220..4227 over pages 32 | 33 and 4476..4483 over pages 34 | 35 (the wave's
    # pages 32..35 taken from its last valid page down, so the earlier page's second
    # half is the wave's fourth chunk), and 8252..8259 over the two halves of page 64
    dict(B=4, ctx_rule=("list", (131072, 4228, 4484, 8260)), topk=16),
    # the same rows in 4 x 8-page waves (a 4096-entry table: 16384 pages in all, the shape
    # of 32-page workgroups), 4092..4099 across a workgroup boundary (pages 31 | 32)
    dict(B=4, ctx_rule=("list", (4100, 4228, 4484, 8260)), topk=16, table_stride=4096),
])
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_decode_step_new_rows_straddle_scorer_workgroups(mx, kw, fmt):
    """The step's new index rows split between two scorer workgroups, or
    between two pages or chunks of one wave, in each of the scorer's launch
    shapes for MXFP4 pages (NVFP4 pages take the same shapes)."""
    wl = W.WORKLOADS["mxfp4_65k"].with_(name="straddle", kv_format=fmt, idx_format=fmt,
                                        q_dtype="f32" if fmt == "mxfp4" else "bf16", **kw)
    inp = W.make_inputs(wl)
    g = run_step(mx, inp)
    check_step(inp, g, range(wl.B))


@pytest.mark.parametrize("stride", [4096, 8192])
def test_decode_step_wide_page_table(mx, stride):
    """The 65K workload with its page table padded to 4096 entries per
    sequence, and to the largest table the library takes (8192 pages, 1M
    tokens), with -1 past each sequence: the scorer's 16-page workgroups past
    the context and the selection's 32-candidates-per-thread variant."""
    inp, g = cached_run(mx, "mxfp4_65k", table_stride=stride)
    assert inp.max_pages == stride
    check_step(inp, g, range(inp.wl.B))


def test_decode_step_fp8_65k(mx):
    """The FP8 workload at 65536 tokens (2048 pages in all): the scorer's
    2-pages-per-wave shape for FP8 pages."""
    inp, g = cached_run(mx, "fp8", ctx_rule=("fixed", 65536))
    check_step(inp, g, range(inp.wl.B))


def test_decode_step_nvfp4_65k(mx):
    """The NVFP4 workload at 65536 - u tokens (2048 pages in all, the last
    page of each sequence partly filled and NaN-poisoned past it)."""
    inp, g = cached_run(mx, "nvfp4", ctx_rule=("fixed_minus_u", 65536, 127))
    check_step(inp, g, range(inp.wl.B))


@pytest.mark.parametrize("kv,idx", [("nvfp4", "mxfp4"), ("mxfp4", "nvfp4"), ("fp8", "nvfp4"), ("nvfp4", "fp8")])
def test_decode_step_mixed_formats(mx, kv, idx):
    """K / V pages in one format and index pages in another (each cache slot
    takes its own format id)."""
    wl = W.WORKLOADS["mxfp4_65k"].with_(name=f"mixed_{kv}_{idx}", B=2, kv_format=kv, idx_format=idx,
                                        q_dtype="f32" if kv == "mxfp4" else "bf16")
    inp = W.make_inputs(wl)
    g = run_step(mx, inp)
    check_step(inp, g, range(wl.B))


# "one_launch": the 65K workload with 2048-entry page tables (B x stride =
# 8192 pages, which decode_step_one_launch takes) run through that entry point
def _wl(name):
    if name == "one_launch":
        return W.WORKLOADS["mxfp4_65k"].with_(name="one_launch", table_stride=2048)
    return W.WORKLOADS[name].with_(B=4)


@pytest.mark.parametrize("name", ["mxfp4_65k", "fp8", "nvfp4", "one_launch"])
def test_decode_step_repeats_bit_exact(mx, name):
    """The same step run many times gives bit-identical output and lse: each
    row is merged by whichever of its partition workgroups finishes last, from
    partials the others wrote in the same launch, and the merge order is fixed,
    so any partial not yet visible to the merging workgroup would show as a
    difference. Also checked against the oracle once."""
    import workloads.gpu as WG
    inp = W.make_inputs(_wl(name))
    wl = inp.wl
    pools = WG.fill_prefix(inp, WG.empty_pools(inp))
    cache = WG.make_cache(inp, pools)
    t = WG.step_tensors(inp)
    step = mx.DecodeStep(cache, t["query"], t["q_idx"], t["w"], wl.topk, wl.sm_scale,
                         k_new=t.get("k_new"), v_new=t.get("v_new"), idx_new=t.get("idx_new"),
                         one_launch=name == "one_launch")
    step.run()
    torch.cuda.synchronize()
    out0, lse0 = step.out.clone(), step.lse.clone()
    for i in range(200):
        step.run()
        assert torch.equal(step.out, out0) and torch.equal(step.lse, lse0), f"run {i + 1} differs"
    r = OS.decode_step_ref(inp, seqs=range(wl.B))
    O = out0.float().cpu().numpy()
    for b in range(wl.B):
        PT.check_attention(O[b], r["O"][b], f"{name} b={b}")


@pytest.mark.parametrize("name", ["mxfp4_65k", "fp8", "one_launch"])
def test_decode_step_alternating_inputs_share_a_workspace(mx, name):
    """Two steps with different queries run alternately on one workspace: each
    run's output and lse equal its own first run bit for bit, so no merge ever
    reads a partial left in the workspace (or in a cache) by the other step's
    previous run."""
    import workloads.gpu as WG
    inp = W.make_inputs(_wl(name))
    wl = inp.wl
    pools = WG.fill_prefix(inp, WG.empty_pools(inp))
    cache = WG.make_cache(inp, pools)
    t = WG.step_tensors(inp)
    qb = (t["query"].float() * -0.75 + 0.5).to(t["query"].dtype).contiguous()
    nb = mx.workspace_bytes(wl.B, wl.q, wl.H, wl.H_I, wl.topk, cache.stride)
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    kw = dict(k_new=t.get("k_new"), v_new=t.get("v_new"), idx_new=t.get("idx_new"), ws=ws,
              one_launch=name == "one_launch")
    steps = [mx.DecodeStep(cache, q, t["q_idx"], t["w"], wl.topk, wl.sm_scale, **kw) for q in (t["query"], qb)]
    first = []
    for s_ in steps:
        s_.run()
        torch.cuda.synchronize()
        first.append((s_.out.clone(), s_.lse.clone()))
    assert not torch.equal(first[0][0], first[1][0])
    for i in range(100):
        for k, s_ in enumerate(steps):
            s_.run()
            assert torch.equal(s_.out, first[k][0]) and torch.equal(s_.lse, first[k][1]), f"run {i}, step {k}"
    r = OS.decode_step_ref(inp, seqs=[0, 1])
    O = first[0][0].float().cpu().numpy()
    for b in (0, 1):
        PT.check_attention(O[b], r["O"][b], f"{name} b={b}")


@pytest.mark.parametrize("name", ["mxfp4_65k", "fp8"])
def test_decode_step_workspace_needs_no_initialization(mx, name):
    """The workspace's contents before a call do not matter (the step clears
    its merge counters itself): a workspace filled with 0xFF or 0x01 bytes
    gives the output and lse of a zero-filled one, bit for bit."""
    import workloads.gpu as WG
    inp = W.make_inputs(_wl(name))
    wl = inp.wl
    pools = WG.fill_prefix(inp, WG.empty_pools(inp))
    cache = WG.make_cache(inp, pools)
    t = WG.step_tensors(inp)
    nb = mx.workspace_bytes(wl.B, wl.q, wl.H, wl.H_I, wl.topk, cache.stride)
    assert mx.lib().mxs_default_partitions(wl.B, wl.q, wl.topk) > 1      # the merge counters are in use
    res = []
    for fill in (0x00, 0xFF, 0x01):
        ws = torch.full((nb,), fill, dtype=torch.uint8, device="cuda")
        s_ = mx.DecodeStep(cache, t["query"], t["q_idx"], t["w"], wl.topk, wl.sm_scale, k_new=t.get("k_new"),
                           v_new=t.get("v_new"), idx_new=t.get("idx_new"), ws=ws)
        s_.run()
        torch.cuda.synchronize()
        res.append((s_.out.clone(), s_.lse.clone()))
    for k in (1, 2):
        assert torch.equal(res[k][0], res[0][0]) and torch.equal(res[k][1], res[0][1]), f"fill {k}"


def test_one_launch_workspace_init(mx):
    """decode_step_one_launch over a workspace filled with 0xFF or 0x01 bytes
    and then zeroed by mxs_workspace_init gives the output and lse of a freshly
    zeroed one, bit for bit; each call leaves the workspace ready for the next
    (a second call without re-zeroing gives the same again)."""
    import workloads.gpu as WG
    inp = W.make_inputs(_wl("one_launch"))
    wl = inp.wl
    pools = WG.fill_prefix(inp, WG.empty_pools(inp))
    cache = WG.make_cache(inp, pools)
    t = WG.step_tensors(inp)
    nb = mx.workspace_bytes(wl.B, wl.q, wl.H, wl.H_I, wl.topk, cache.stride)
    res = []
    for fill in (0x00, 0xFF, 0x01):
        ws = torch.full((nb,), fill, dtype=torch.uint8, device="cuda")
        mx.workspace_init(ws)
        s_ = mx.DecodeStep(cache, t["query"], t["q_idx"], t["w"], wl.topk, wl.sm_scale, k_new=t.get("k_new"),
                           v_new=t.get("v_new"), idx_new=t.get("idx_new"), ws=ws, one_launch=True)
        for _ in range(2):
            s_.run()
            torch.cuda.synchronize()
            res.append((s_.out.clone(), s_.lse.clone()))
    for k in range(1, len(res)):
        assert torch.equal(res[k][0], res[0][0]) and torch.equal(res[k][1], res[0][1]), f"run {k}"


@pytest.mark.parametrize("name,kw", [
    ("headline", {}), ("long", dict(table_stride=2048)), ("b32", {}),               # ragged contexts
    ("mxfp4_65k", dict(name="wide", table_stride=4096)),                              # 32 candidates per thread
    ("mxfp4_65k", dict(name="straddle", B=4, ctx_rule=("list", (262144, 4100, 8196, 65540)), topk=32)),
])
def test_one_launch_equals_two_launches(mx, name, kw):
    """decode_step_one_launch gives decode_step's output, lse, block table and
    K / V / index pages bit for bit (the same device code for every stage;
    decode_step itself is checked against the oracle above)."""
    import workloads.gpu as WG
    inp = W.make_inputs(W.WORKLOADS[name].with_(**kw) if kw else W.WORKLOADS[name])
    wl = inp.wl
    res = []
    for one in (False, True):
        pools = WG.fill_prefix(inp, WG.empty_pools(inp))
        cache = WG.make_cache(inp, pools)
        t = WG.step_tensors(inp)
        table = torch.empty((wl.B, wl.q, wl.topk), dtype=torch.int32, device="cuda")
        s_ = mx.DecodeStep(cache, t["query"], t["q_idx"], t["w"], wl.topk, wl.sm_scale, k_new=t.get("k_new"),
                           v_new=t.get("v_new"), idx_new=t.get("idx_new"), block_table_out=table, one_launch=one)
        s_.run()
        torch.cuda.synchronize()
        res.append((s_.out.clone(), s_.lse.clone(), table.clone(), {k: p.clone() for k, p in pools.items()}))
        del pools, cache
    (o0, l0, t0, p0), (o1, l1, t1, p1) = res
    assert torch.equal(t0, t1), "block tables differ"
    assert torch.equal(o0, o1) and torch.equal(l0, l1), "output or lse differs"
    for k in p0:
        assert torch.equal(p0[k], p1[k]), f"{k} pages differ"


def test_one_launch_refuses_unsupported(mx):
    """FP8 caches (or fewer than 8192 pages) are refused before any launch."""
    import workloads.gpu as WG
    inp = W.make_inputs(W.WORKLOADS["fp8"])
    wl = inp.wl
    pools = WG.fill_prefix(inp, WG.empty_pools(inp))
    cache = WG.make_cache(inp, pools)
    t = WG.step_tensors(inp)
    s_ = mx.DecodeStep(cache, t["query"], t["q_idx"], t["w"], wl.topk, wl.sm_scale, one_launch=True)
    with pytest.raises(mx.MxsError) as e:
        s_.run()
    assert e.value.status == mx.MXS_EUNSUPPORTED and "one_launch" in str(e.value)
