"""GPU parity of each stage against the oracle, through the C ABI
(sparse_attention_decode_mxfp4_amd -> libmxsparse.so), on seeded inputs.

Bars: page bytes, q codes and block ids exact; scores, top-k and attention
within the tolerances of tests/parity.py.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from oracle import formats as OF
from oracle import indexer as OI
from oracle import step as OS
from tests import parity as PT

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_decode_mxfp4_amd as m
    m.lib()
    return m


# ------------------------------------------------------------------ row store
def _tricky_rows(n, seed):
    """fp32 rows that hit every e2m1 rounding case: exact ties after scaling,
    saturation between 6 and 8, zero and subnormal groups, -0, wide exponents."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 128)).astype(np.float32)
    x *= np.ldexp(1.0, rng.integers(-60, 60, size=(n, 1))).astype(np.float32)
    g = x.reshape(n, 4, 32)
    k = rng.integers(-100, 100, size=(n, 4, 1))
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 7.75, 0.0, 6.0, 4.0], dtype=np.float64)
    sel = rng.random((n, 4)) < 0.5                        # half of the groups: values on tie points
    tie = (rng.choice(mids, size=(n, 4, 32)) * rng.choice([-1.0, 1.0], size=(n, 4, 32)) *
           np.ldexp(1.0, k)).astype(np.float32)
    tie[:, :, 0] = (6.0 * np.ldexp(1.0, k[:, :, 0])).astype(np.float32)      # fixes the group scale at 2^k
    g[sel] = tie[sel]
    x[0] = 0.0
    x[1, :32] = -0.0
    x[2, 32:64] = np.float32(1e-40)                       # subnormal group
    x[3, 64:96] = -np.float32(3e-39)
    x[4] = np.float32(3.0e38)
    return x


def _tricky_nv_rows(n, seed):
    """fp32 rows for the NVFP4 row store: wide exponents; half the rows on the
    format's grid with elements on e2m1 tie points (token scale a power of two,
    block 0 holding 6 * 448 of it, every block's scale an exact e4m3 value), so
    every division lands exactly on a tie; a zero row, an all -0 row, zero and
    sub-range blocks, a row of fp32 subnormals (token scale clamped at 2^-149)
    and values near the fp32 maximum."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 128)).astype(np.float32)
    x *= np.ldexp(1.0, rng.integers(-60, 60, size=(n, 1))).astype(np.float32)
    x[rng.random((n, 128)) < 0.01] *= np.float32(20.0)
    sel = np.flatnonzero(rng.random(n) < 0.5)
    m = sel.size
    S = np.ldexp(1.0, rng.integers(-40, 40, size=(m, 1, 1)))
    cb = OF.E4M3_TABLE[rng.integers(1, 127, size=(m, 8, 1))]
    cb[:, 0] = 448.0
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.0, 6.0, 4.0, 0.5])
    v = rng.choice(mids, size=(m, 8, 16)) * rng.choice([-1.0, 1.0], size=(m, 8, 16))
    v[:, :, 0] = 6.0
    x[sel] = (v * cb * S).reshape(m, 128).astype(np.float32)
    x[0] = 0.0
    x[1] = -0.0
    x[2, 16:32] = 0.0
    x[2, 48:64] *= np.float32(1e-7)
    with np.errstate(under="ignore"):
        x[3] = (rng.standard_normal(128) * 1e-41).astype(np.float32)
    x[4] = rng.uniform(-3e38, 3e38, 128).astype(np.float32)
    return x


@pytest.mark.parametrize("fmt", ["mxfp4", "fp8", "nvfp4"])
def test_row_store_bit_exact(mx, fmt):
    n = {"mxfp4": 1 << 20, "fp8": 1 << 17, "nvfp4": 1 << 18}[fmt]
    if fmt == "mxfp4":
        x = _tricky_rows(n, 7)
    elif fmt == "nvfp4":
        x = _tricky_nv_rows(n, 12)
    else:
        x = np.random.default_rng(8).standard_normal((n, 128)).astype(np.float32) * 3
        x[0] = 0.0
        x[1, 5] = 1e4
    pages = (n + 127) // 128
    num_pages = pages + 7
    table = np.random.default_rng(9).permutation(num_pages)[:pages].astype(np.int32)
    ref = W.new_pool(num_pages, OF.PAGE_BYTES[fmt])
    OF.STORE[fmt](ref, table, 0, x)
    t = np.arange(n)
    slots = table[t // 128].astype(np.int64) * 128 + t % 128
    pool = torch.full((num_pages * OF.PAGE_BYTES[fmt],), 0xFF, dtype=torch.uint8, device=DEV)
    store = {"mxfp4": mx.mxfp4_row_store, "fp8": mx.fp8_row_store, "nvfp4": mx.nvfp4_row_store}[fmt]
    store(torch.from_numpy(x).to(DEV), torch.from_numpy(slots).to(DEV), pool)
    got = pool.cpu().numpy()
    PT.compare_pool_pages(got, ref, np.arange(num_pages), OF.PAGE_BYTES[fmt], f"{fmt} row store")


def test_row_store_skips_bad_slots(mx):
    x = np.random.default_rng(1).standard_normal((6, 128)).astype(np.float32)
    slots = np.array([-1, 3, 2 * 128 + 5, 3 * 128, 10 ** 9, -7], dtype=np.int64)     # 3 * 128 is past 3 pages
    pool = torch.full((3 * 8704,), 0xFF, dtype=torch.uint8, device=DEV)
    mx.mxfp4_row_store(torch.from_numpy(x).to(DEV), torch.from_numpy(slots).to(DEV), pool)
    ref = W.new_pool(3, 8704)
    OF.mxfp4_store(ref, np.array([0], dtype=np.int32), 3, x[1:2])
    OF.mxfp4_store(ref, np.array([2], dtype=np.int32), 5, x[2:3])
    PT.compare_pool_pages(pool.cpu().numpy(), ref, np.arange(3), 8704, "skipped slots")


def test_row_store_empty(mx):
    pool = torch.full((8704,), 0xFF, dtype=torch.uint8, device=DEV)
    mx.mxfp4_row_store(torch.empty((0, 128), device=DEV), torch.empty((0,), dtype=torch.int64, device=DEV), pool)
    torch.cuda.synchronize()
    assert (pool == 0xFF).all()


# ------------------------------------------------------------------ q store
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_pack_q_bit_exact(mx, dtype):
    rng = np.random.default_rng(3)
    vals = OF.E4M3_TABLE[:127]
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([rng.standard_normal(200000) * 30, rng.standard_normal(20000) * 1e-3,
                        mids, -mids, vals, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                        [448, 449, 464, 465, 500, -500, 1e30, -1e30, np.inf, -np.inf, np.nan, -np.nan, 0.0, -0.0,
                         1e-40, 2 ** -10, 3 * 2 ** -11]]).astype(np.float32)
    x = x[: (x.size // 4) * 4 + 3]                        # a ragged length
    if dtype == "bf16":
        bits = W.bf16_bits(x)
        src = OF.bf16_to_f64(bits)
        qt = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    else:
        src = x.astype(np.float64)
        qt = torch.from_numpy(x).to(DEV)
    want = OF.e4m3_encode(src)
    got = mx.pack_q_e4m3(qt).cpu().numpy()
    nan = np.isnan(src)
    np.testing.assert_array_equal(got[~nan], want[~nan])
    assert ((got[nan] & 0x7F) == 0x7F).all()
    assert (got[src == 500] == 0x7E).all() and (got[src == -np.inf] == 0xFE).all()


# ------------------------------------------------------------------ scores and top-k
def _setup(mx, name, **kw):
    inp = W.make_inputs(W.WORKLOADS[name].with_(full_step=False, **kw))
    import workloads.gpu as WG
    pools = WG.fill_prefix(inp, WG.empty_pools(inp))
    cache = WG.make_cache(inp, pools)
    return inp, pools, cache, WG.step_tensors(inp)


SMALL = ["tiny", "fp8", "mxfp4_65k", "nvfp4"]


@pytest.mark.parametrize("name", SMALL)
def test_index_scores(mx, name):
    inp, pools, cache, t = _setup(mx, name)
    S = mx.index_score(cache, t["q_idx"], t["w"]).cpu().numpy().astype(np.float64)
    wl = inp.wl
    ref_pool = OS.build_cache(inp, "idx", wl.idx_format)
    qI = OF.bf16_to_f64(inp.q_idx)
    for b in range(wl.B):
        L = int(inp.contexts[b])
        kI = OF.READ[wl.idx_format](ref_pool, inp.page_table[b], L)
        Sr = OI.index_scores(kI, qI[b], inp.w[b].astype(np.float64), L)
        Sa = PT.score_bound(kI, qI[b], inp.w[b].astype(np.float64), L)
        PT.check_scores(S[b], Sr, Sa, OI.n_candidates(L, wl.q))


def test_index_scores_nvfp4_query_magnitudes(mx):
    """NVFP4 index keys run on the f16 MFMA with each query row scaled by a
    power of two into f16's range: rows scaled by 2^-60 .. 2^60, and a row
    whose elements span 2^-40 .. 1 of its largest, score within the usual
    bound of the oracle's bf16 arithmetic."""
    inp, pools, cache, t = _setup(mx, "nvfp4")
    wl = inp.wl
    rng = np.random.default_rng(21)
    q = OF.bf16_to_f64(inp.q_idx)                                  # [B][q][H_I][128]
    q *= np.ldexp(1.0, rng.integers(-60, 61, size=q.shape[:3]))[..., None]
    q[0, 0, 0] *= np.ldexp(1.0, -rng.integers(0, 41, size=128))    # one row spanning 2^-40 .. 1
    inp.q_idx = W.bf16_bits(q.astype(np.float32))
    assert np.array_equal(OF.bf16_to_f64(inp.q_idx), q)            # the scaling is exact in bf16
    import workloads.gpu as WG
    t = WG.step_tensors(inp)
    S = mx.index_score(cache, t["q_idx"], t["w"]).cpu().numpy().astype(np.float64)
    ref_pool = OS.build_cache(inp, "idx", wl.idx_format)
    for b in range(wl.B):
        L = int(inp.contexts[b])
        kI = OF.READ[wl.idx_format](ref_pool, inp.page_table[b], L)
        Sr = OI.index_scores(kI, q[b], inp.w[b].astype(np.float64), L)
        Sa = PT.score_bound(kI, q[b], inp.w[b].astype(np.float64), L)
        PT.check_scores(S[b], Sr, Sa, OI.n_candidates(L, wl.q))


def test_index_score_one_hot_structure(mx):
    """A single non-zero key element and a one-hot query pin the element,
    token and head mapping of the scorer."""
    wl = W.WORKLOADS["tiny"].with_(full_step=False, q=3, H_I=4, ctx_rule=("fixed", 700))
    inp = W.make_inputs(wl)
    import workloads.gpu as WG
    pools = WG.empty_pools(inp)
    rng = np.random.default_rng(0)
    rows = {s: np.zeros((700, 128), dtype=np.float32) for s in WG.STREAMS}
    hot = [(5, 0), (200, 37), (333, 127), (650, 64), (698, 95)]
    for t, d in hot:
        rows["idx"][t, d] = rng.uniform(1, 5)
    inp._row_cache.update({(s, 0): r for s, r in rows.items()})
    pools = WG.fill_prefix(inp, pools)
    cache = WG.make_cache(inp, pools)
    qI = np.zeros((1, 3, 4, 128), dtype=np.float32)
    for j in range(3):
        for h in range(4):
            qI[0, j, h, hot[(j + h) % 5][1]] = 1.0 + h
    inp.q_idx = W.bf16_bits(qI)
    t = WG.step_tensors(inp)
    S = mx.index_score(cache, t["q_idx"], t["w"]).cpu().numpy().astype(np.float64)
    ref = OS.build_cache(inp, "idx", "mxfp4")
    kI = OF.mxfp4_read(ref, inp.page_table[0], 700)
    Sr = OI.index_scores(kI, OF.bf16_to_f64(inp.q_idx[0]), inp.w[0].astype(np.float64), 700)
    PT.check_scores(S[0], Sr, PT.score_bound(kI, OF.bf16_to_f64(inp.q_idx[0]), inp.w[0].astype(np.float64), 700),
                    OI.n_candidates(700, 3))


@pytest.mark.parametrize("stride", [300, 2000, 2100])
@pytest.mark.parametrize("k", [1, 4, 16, 32, 64])
def test_topk_exact_on_given_scores(mx, k, stride):
    """Top-k of the same fp32 scores: the GPU selection equals the oracle's
    exactly, including heavy ties (ties go to the lower block id), a few ties
    at the k-th score, and rows with fewer candidates than k."""
    rng = np.random.default_rng(k + stride)
    B, q = 5, 8
    ctx = np.array([stride * 128, 1000, 128 * 64 + 3, 77, 128 * 2000], dtype=np.int64)
    S = rng.integers(-20, 20, size=(B, q, stride)).astype(np.float32)          # many ties
    S[1] = rng.standard_normal((q, stride)).astype(np.float32)
    S[3] = (np.round(rng.standard_normal((q, stride)) * 6) / 6).astype(np.float32)   # some ties near the top
    S[4, :, :] = 1.0                                                            # all equal
    S[0, 3, ::7] = -np.inf
    table = np.zeros((B, stride), dtype=np.int32)
    cache = mx.Cache(None, None, torch.zeros(8704, dtype=torch.uint8, device=DEV),
                     torch.from_numpy(table).to(DEV), torch.from_numpy(ctx.astype(np.int32)).to(DEV))
    got = mx.topk_blocks(cache, torch.from_numpy(S).to(DEV), k).cpu().numpy()
    for b in range(B):
        for j in range(q):
            nc = min(int((ctx[b] - q + j) // 128 + 1), stride)
            want = OI.topk_blocks(S[b, j].astype(np.float64), nc, k)
            np.testing.assert_array_equal(got[b, j], want, err_msg=f"row {b},{j}")


@pytest.mark.parametrize("name", SMALL)
def test_index_score_topk(mx, name):
    inp, pools, cache, t = _setup(mx, name)
    wl = inp.wl
    table = mx.index_score_topk(cache, t["q_idx"], t["w"], wl.topk).cpu().numpy()
    ref_pool = OS.build_cache(inp, "idx", wl.idx_format)
    qI = OF.bf16_to_f64(inp.q_idx)
    for b in range(wl.B):
        L = int(inp.contexts[b])
        kI = OF.READ[wl.idx_format](ref_pool, inp.page_table[b], L)
        Sr = OI.index_scores(kI, qI[b], inp.w[b].astype(np.float64), L)
        nc = OI.n_candidates(L, wl.q)
        for j in range(wl.q):
            PT.check_topk(table[b, j], OI.topk_blocks(Sr[j], int(nc[j]), wl.topk), Sr[j], int(nc[j]), wl.topk)


# ------------------------------------------------------------------ attention
def _q_att(mx, inp, t):
    qa, codes = OS.attention_query(inp)
    if inp.wl.kv_format == "mxfp4":
        q8 = mx.pack_q_e4m3(t["query"])
        assert np.array_equal(q8.cpu().numpy(), codes)
        return qa, q8
    return qa, t["query"]


@pytest.mark.parametrize("name", SMALL)
@pytest.mark.parametrize("P", [0, 1, 3, 70])
def test_split_attention_and_merge(mx, name, P):
    inp, pools, cache, t = _setup(mx, name)
    wl = inp.wl
    if P > 64:
        P = 64                                              # more partitions than blocks: empty ones
    table = mx.index_score_topk(cache, t["q_idx"], t["w"], wl.topk)
    qa, qdev = _q_att(mx, inp, t)
    sp_m, sp_l, sp_o = mx.sparse_split_attn(cache, qdev, table, wl.sm_scale, num_partitions=P)
    O, lse = mx.lse_merge(sp_m, sp_l, sp_o)
    Pn = sp_m.shape[-1]
    tbl = table.cpu().numpy()
    ref_pools = {s: OS.build_cache(inp, s, f) for s, f in (("k", wl.kv_format), ("v", wl.kv_format))}
    O_g = O.float().cpu().numpy()
    lse_g = lse.cpu().numpy()
    m_g, l_g, o_g = sp_m.cpu().numpy(), sp_l.cpu().numpy(), sp_o.cpu().numpy()
    for b in range(wl.B):
        Oref, lref, K_all, V_all = PT.oracle_attention_with_table(inp, ref_pools, qa, tbl[b], b)
        PT.check_attention(O_g[b], Oref, f"{name} b={b} P={Pn}")
        np.testing.assert_allclose(lse_g[b], lref, rtol=1e-4, atol=1e-4)
        pos = OI.row_positions(int(inp.contexts[b]), wl.q)
        for j in range(wl.q):
            m, l, o = OA.split_partials(qa[b, j], K_all, V_all, tbl[b, j], int(pos[j]), wl.sm_scale, Pn)
            empty = np.isneginf(m)
            assert (np.isneginf(m_g[b, j]) == empty).all()
            assert (l_g[b, j][empty] == 0).all() and (o_g[b, j][empty] == 0).all()
            fin = ~empty
            np.testing.assert_allclose(m_g[b, j][fin], m[fin], rtol=1e-4, atol=1e-4)
            # partial sums relative to the partition's own mass
            np.testing.assert_allclose(l_g[b, j][fin], l[fin], rtol=1e-2)
            scale = np.abs(o).max(axis=-1, keepdims=True) + 1e-30
            assert (np.abs(o_g[b, j] - o) <= 1e-2 * scale + 1e-3 * l[..., None]).all()


def test_wrong_table_negative_control(mx):
    """Attention over a perturbed block table must fail the parity tolerance."""
    inp, pools, cache, t = _setup(mx, "mxfp4_65k")
    wl = inp.wl
    table = mx.index_score_topk(cache, t["q_idx"], t["w"], wl.topk)
    qa, qdev = _q_att(mx, inp, t)
    bad = table.clone()
    bad[..., 0] = torch.where(bad[..., 0] > 0, bad[..., 0] - 1, bad[..., 0] + 1)   # shift the first block
    bad[..., 1] = torch.where(bad[..., 1] > 1, bad[..., 1] - 1, bad[..., 1])
    O, _ = mx.lse_merge(*mx.sparse_split_attn(cache, qdev, bad, wl.sm_scale))
    ref_pools = {s: OS.build_cache(inp, s, wl.kv_format) for s in ("k", "v")}
    Oref, *_ = PT.oracle_attention_with_table(inp, ref_pools, qa, table.cpu().numpy()[0], 0)
    with pytest.raises(AssertionError):
        PT.check_attention(O.float().cpu().numpy()[0], Oref, "wrong table")


def test_lse_merge_partials(mx):
    rng = np.random.default_rng(5)
    n, P = 300, 13
    m = (rng.standard_normal((n, P)) * 5).astype(np.float32)
    l = (rng.random((n, P)) * 10 + 0.1).astype(np.float32)
    o = rng.standard_normal((n, P, 128)).astype(np.float32)
    empty = rng.random((n, P)) < 0.3
    m[empty] = -np.inf
    l[empty] = 0
    o[empty] = 0
    m[7] = -np.inf
    l[7] = 0
    o[7] = 0                                                # a row with only empty partitions
    O, lse = mx.lse_merge(torch.from_numpy(m).to(DEV), torch.from_numpy(l).to(DEV), torch.from_numpy(o).to(DEV))
    Oref, lref = OA.lse_merge(m.astype(np.float64), l.astype(np.float64), o.astype(np.float64))
    Og = O.float().cpu().numpy()
    assert (Og[7] == 0).all() and np.isneginf(lse.cpu().numpy()[7])
    # bf16 output: relative 2^-8 of each element, plus fp32 accumulation
    assert (np.abs(Og - Oref) <= 2 ** -8 * np.abs(Oref) + 1e-5 * np.abs(Oref).max()).all()
    ok = np.isfinite(lref)
    np.testing.assert_allclose(lse.cpu().numpy()[ok], lref[ok], rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("name", SMALL)
def test_read_index_pages_reads_and_writes_nothing_else(mx, name):
    """The scan's read-ceiling launch (a measurement aid): it completes over
    real tables and over tables holding entries outside the pool (skipped),
    leaves the pages untouched and writes nothing but its one-word sink."""
    inp, pools, cache, t = _setup(mx, name)
    before = pools["idx"].clone()
    guard = torch.zeros(64, dtype=torch.int32, device=DEV)      # sink = guard[0]; the rest must stay zero
    mx.read_index_pages(cache, inp.wl.B, guard[:1])
    table = cache.page_table.clone()
    bad = cache.page_table.clone()
    bad.view(-1)[::3] = -1
    bad.view(-1)[1::3] = cache.num_pages + 7
    cache.page_table.copy_(bad)
    mx.read_index_pages(cache, inp.wl.B, guard[:1])
    cache.page_table.copy_(table)
    torch.cuda.synchronize()
    assert torch.equal(pools["idx"], before)
    assert int(guard[1:].abs().sum()) == 0
    assert int(guard[0]) in (0, 0x9E3779B9 - (1 << 32))
