"""GPU parity of the step that reuses an earlier layer's block selection
(decode_step_reuse through the C ABI) against the oracle's
decode_step_reuse_ref: K / V page bytes after the row store exact, the index
pool untouched, output within the attention tolerance; and against the full
decode step on the same selection, bit for bit.
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


def random_table(inp, seed):
    """A reused selection: per row, min(k, candidates) distinct candidate blocks
    (always the row's last one, which holds the step's new rows), ascending,
    -1 padded."""
    wl = inp.wl
    rng = np.random.default_rng(seed)
    t = np.full((wl.B, wl.q, wl.topk), -1, dtype=np.int64)
    for b in range(wl.B):
        nc = OI.n_candidates(int(inp.contexts[b]), wl.q)
        for j in range(wl.q):
            n = int(nc[j])
            k = min(wl.topk, n)
            if k == 0:
                continue
            ids = np.concatenate([rng.choice(n - 1, k - 1, replace=False), [n - 1]]) if n > 1 else np.array([0])
            t[b, j, :k] = np.sort(ids)
    return t


def run_reuse(mx, inp, table, num_partitions=0, store=True, one_launch=False):
    import workloads.gpu as WG
    wl = inp.wl
    pools = WG.fill_prefix(inp, WG.empty_pools(inp))
    idx_before = pools["idx"].clone()
    cache = WG.make_cache(inp, pools)
    t = WG.step_tensors(inp)
    tab = torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32)).cuda()
    step = mx.DecodeStepReuse(cache, t["query"], tab, wl.sm_scale, k_new=t.get("k_new") if store else None,
                              v_new=t.get("v_new") if store else None, num_partitions=num_partitions,
                              one_launch=one_launch)
    step.run()
    torch.cuda.synchronize()
    assert torch.equal(pools["idx"], idx_before), "the index pool changed"
    return {"pools": {s: pools[s].cpu().numpy() for s in ("k", "v")}, "O": step.out.float().cpu().numpy(),
            "lse": step.lse.cpu().numpy()}


def check_reuse(inp, g, table, seqs):
    wl = inp.wl
    r = OS.decode_step_reuse_ref(inp, table, seqs=seqs)
    for b in seqs:
        L = int(inp.contexts[b])
        pages = PT.seq_pages(inp.page_table[b], L)
        for s in ("k", "v"):
            PT.compare_pool_pages(g["pools"][s], r["pools"][s], pages, OF.PAGE_BYTES[wl.kv_format],
                                  f"{wl.name} reuse {s} b={b}")
        PT.check_attention(g["O"][b], r["O"][b], f"{wl.name} reuse b={b}")
        fin = np.isfinite(r["lse"][b])
        np.testing.assert_allclose(g["lse"][b][fin], r["lse"][b][fin], rtol=1e-4, atol=1e-4)
        assert (np.isneginf(g["lse"][b]) == np.isneginf(r["lse"][b])).all()


@pytest.mark.parametrize("one_launch", [False, True])
@pytest.mark.parametrize("name", ["tiny", "fp8", "mxfp4_65k", "nvfp4"])
def test_reuse_step_small(mx, name, one_launch):
    inp = W.make_inputs(W.WORKLOADS[name])
    table = random_table(inp, 11)
    g = run_reuse(mx, inp, table, one_launch=one_launch)
    check_reuse(inp, g, table, range(inp.wl.B))


# decode_step_reuse_one_launch against decode_step_reuse on every path the
# two-launch tests cover: (workload overrides, table kind, partitions, row store)
ONE_LAUNCH_CASES = [
    ("mxfp4_65k", {}, "random", 0, True),
    ("mxfp4_65k", dict(B=2), "random", 1, True),                  # P = 1: the row written without an exchange
    ("mxfp4_65k", dict(B=2), "random", 64, True),                 # empty partitions
    ("mxfp4_65k", dict(B=2), "noisy", 0, True),                   # entries < 0, past the table, past the position
    ("mxfp4_65k", dict(B=2, full_step=False), "random", 0, False),   # no row store
    ("tiny", dict(q=2), "empty", 0, True),                        # every slot -1
    ("mxfp4_65k", dict(name="edge", ctx_rule=("list", (9, 130, 1000, 4096)), B=4, q=8, H=16, topk=16), "random", 0,
     True),
    ("mxfp4_65k", dict(name="edge", ctx_rule=("list", (5000, 3000)), B=2, q=16, H=7, H_I=3, topk=5), "random", 0,
     True),
    ("mxfp4_65k", dict(q_dtype="bf16"), "random", 0, True),       # bf16 source of the e4m3 query
    ("fp8", {}, "random", 0, True),
    ("nvfp4", {}, "random", 0, True),
    ("long", dict(B=2), "random", 0, True),                       # 128K-256K contexts
]


@pytest.mark.parametrize("case", range(len(ONE_LAUNCH_CASES)))
def test_reuse_one_launch_equals_two_launches(mx, case):
    """decode_step_reuse_one_launch gives the output, lse and K / V pages of
    decode_step_reuse bit for bit, and is checked against the oracle too."""
    name, kw, kind, P, store = ONE_LAUNCH_CASES[case]
    inp = W.make_inputs(W.WORKLOADS[name].with_(**kw) if kw else W.WORKLOADS[name])
    wl = inp.wl
    table = random_table(inp, 7)
    if kind == "noisy":
        table[:, :, 1] = -3
        table[0, :, 2] = inp.max_pages + 7
        table[1, :, 2] = 2 ** 30
    elif kind == "empty":
        table[:] = -1
    two = run_reuse(mx, inp, table, num_partitions=P, store=store)
    one = run_reuse(mx, inp, table, num_partitions=P, store=store, one_launch=True)
    assert np.array_equal(one["O"], two["O"]) and np.array_equal(one["lse"], two["lse"])
    for s in ("k", "v"):
        assert np.array_equal(one["pools"][s], two["pools"][s]), s
    if kind == "empty":                           # nothing attended: O = 0, lse = -inf (the oracle's row is 0 / 0)
        assert (one["O"] == 0).all() and np.isneginf(one["lse"]).all()
    else:
        check_reuse(inp, one, table, range(wl.B) if name != "long" else [0])


@pytest.mark.parametrize("name", ["tiny", "fp8", "mxfp4_65k", "nvfp4", "one_launch"])
def test_reuse_step_on_the_full_steps_selection_is_bitwise_the_full_step(mx, name):
    """decode_step, then decode_step_reuse over the block table it wrote, from
    the same pre-step caches: identical output, lse and K / V pages (also after
    decode_step_one_launch over 2048-entry page tables)."""
    import workloads.gpu as WG
    if name == "one_launch":
        inp = W.make_inputs(W.WORKLOADS["mxfp4_65k"].with_(name="one_launch", table_stride=2048))
    else:
        inp = W.make_inputs(W.WORKLOADS[name])
    wl = inp.wl
    pools = WG.fill_prefix(inp, WG.empty_pools(inp))
    cache = WG.make_cache(inp, pools)
    t = WG.step_tensors(inp)
    table = torch.empty((wl.B, wl.q, wl.topk), dtype=torch.int32, device="cuda")
    full = mx.DecodeStep(cache, t["query"], t["q_idx"], t["w"], wl.topk, wl.sm_scale, k_new=t.get("k_new"),
                         v_new=t.get("v_new"), idx_new=t.get("idx_new"), block_table_out=table,
                         one_launch=name == "one_launch")
    full.run()
    torch.cuda.synchronize()
    g = run_reuse(mx, inp, table.cpu().numpy())
    assert np.array_equal(g["O"], full.out.float().cpu().numpy())
    assert np.array_equal(g["lse"], full.lse.cpu().numpy())
    for s in ("k", "v"):
        assert np.array_equal(g["pools"][s], pools[s].cpu().numpy()), s


def test_reuse_step_skips_bad_entries(mx):
    """Entries < 0, past the page table or past the row's position add nothing."""
    inp = W.make_inputs(W.WORKLOADS["mxfp4_65k"].with_(B=2))
    wl = inp.wl
    table = random_table(inp, 5)
    noisy = table.copy()
    stride = inp.max_pages
    noisy[:, :, 1] = -3
    noisy[0, :, 2] = stride + 7
    noisy[1, :, 2] = 2 ** 30
    g = run_reuse(mx, inp, noisy)
    check_reuse(inp, g, noisy, [0, 1])
    assert wl.topk >= 3


@pytest.mark.parametrize("P", [1, 5, 64])
def test_reuse_step_partition_counts(mx, P):
    inp = W.make_inputs(W.WORKLOADS["mxfp4_65k"].with_(B=2))
    table = random_table(inp, 3)
    g = run_reuse(mx, inp, table, num_partitions=P)
    check_reuse(inp, g, table, [0, 1])


@pytest.mark.parametrize("kw", [
    dict(ctx_rule=("list", (9, 130, 1000, 4096)), B=4, q=8, H=16, topk=16),      # contexts near q, ragged
    dict(ctx_rule=("list", (8, 300)), B=2, q=8, H=1, H_I=1, topk=64),            # L == q; H = 1
    dict(ctx_rule=("list", (5000, 3000)), B=2, q=16, H=7, H_I=3, topk=5),        # q = 16, odd head count
])
def test_reuse_step_edge_shapes(mx, kw):
    wl = W.WORKLOADS["mxfp4_65k"].with_(name="edge", **kw)
    inp = W.make_inputs(wl)
    table = random_table(inp, 8)
    g = run_reuse(mx, inp, table)
    check_reuse(inp, g, table, range(wl.B))


def test_reuse_step_without_row_store(mx):
    """k_new / v_new not given: the cache already holds every position."""
    inp = W.make_inputs(W.WORKLOADS["mxfp4_65k"].with_(B=2, full_step=False))
    table = random_table(inp, 4)
    g = run_reuse(mx, inp, table, store=False)
    check_reuse(inp, g, table, [0, 1])


def test_reuse_step_empty_table(mx):
    """Every slot -1: each row attends to nothing (O = 0, lse = -inf)."""
    inp = W.make_inputs(W.WORKLOADS["tiny"].with_(q=2))
    wl = inp.wl
    table = np.full((wl.B, wl.q, wl.topk), -1)
    g = run_reuse(mx, inp, table)
    assert (g["O"] == 0).all() and np.isneginf(g["lse"]).all()


@pytest.mark.parametrize("one_launch", [False, True])
def test_reuse_step_alternating_tables_share_a_workspace(mx, one_launch):
    """Two reuse steps over different tables alternate on one workspace: every
    run equals its own first run bit for bit (the single launch's counters
    reset themselves between runs)."""
    import workloads.gpu as WG
    inp = W.make_inputs(W.WORKLOADS["mxfp4_65k"])
    wl = inp.wl
    pools = WG.fill_prefix(inp, WG.empty_pools(inp))
    cache = WG.make_cache(inp, pools)
    t = WG.step_tensors(inp)
    nb = mx.workspace_bytes(wl.B, wl.q, wl.H, 1, wl.topk, cache.stride)
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    tabs = [torch.from_numpy(random_table(inp, s).astype(np.int32)).cuda() for s in (1, 2)]
    steps = [mx.DecodeStepReuse(cache, t["query"], tb, wl.sm_scale, k_new=t.get("k_new"), v_new=t.get("v_new"),
                                ws=ws, one_launch=one_launch) for tb in tabs]
    first = []
    for s_ in steps:
        s_.run()
        torch.cuda.synchronize()
        first.append((s_.out.clone(), s_.lse.clone()))
    for i in range(100):
        for k, s_ in enumerate(steps):
            s_.run()
            assert torch.equal(s_.out, first[k][0]) and torch.equal(s_.lse, first[k][1]), f"run {i}, step {k}"
    r = OS.decode_step_reuse_ref(inp, random_table(inp, 1), seqs=[0])
    PT.check_attention(first[0][0].float().cpu().numpy()[0], r["O"][0], "alternating reuse b=0")


def test_reuse_step_workspace_needs_no_initialization(mx):
    """As for the full step: a workspace filled with 0xFF or 0x01 bytes gives
    the output and lse of a zero-filled one, bit for bit."""
    import workloads.gpu as WG
    inp = W.make_inputs(W.WORKLOADS["mxfp4_65k"])
    wl = inp.wl
    pools = WG.fill_prefix(inp, WG.empty_pools(inp))
    cache = WG.make_cache(inp, pools)
    t = WG.step_tensors(inp)
    nb = mx.workspace_bytes(wl.B, wl.q, wl.H, 1, wl.topk, cache.stride)
    assert mx.lib().mxs_default_partitions(wl.B, wl.q, wl.topk) > 1
    tb = torch.from_numpy(random_table(inp, 1).astype(np.int32)).cuda()
    res = []
    for fill in (0x00, 0xFF, 0x01):
        ws = torch.full((nb,), fill, dtype=torch.uint8, device="cuda")
        s_ = mx.DecodeStepReuse(cache, t["query"], tb, wl.sm_scale, k_new=t.get("k_new"), v_new=t.get("v_new"), ws=ws)
        s_.run()
        torch.cuda.synchronize()
        res.append((s_.out.clone(), s_.lse.clone()))
    for k in (1, 2):
        assert torch.equal(res[k][0], res[0][0]) and torch.equal(res[k][1], res[0][1]), f"fill {k}"
