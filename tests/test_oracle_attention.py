"""Pins of the oracle's sparse attention, split partials and merge: the dense
special case against torch's scaled-dot-product attention (float64, CPU),
closed forms, scipy's logsumexp, and invariants of the whole oracle step."""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import workloads as W
from oracle import attention as A
from oracle import formats as F
from oracle import step as S


def _row_setup(seed=0, L=1000, H=16):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((H, 128)), rng.standard_normal((L, 128)),
            rng.standard_normal((L, 128)))


def test_all_blocks_equals_torch_sdpa_causal():
    """With every block selected, sparse attention is dense causal attention."""
    L, q, H = 777, 8, 4
    rng = np.random.default_rng(1)
    Q = rng.standard_normal((q, H, 128))
    K = rng.standard_normal((L, 128))
    V = rng.standard_normal((L, 128))
    blocks = np.arange((L + 127) // 128)
    scale = 1 / np.sqrt(128)
    mask = torch.arange(L)[None, :] <= torch.arange(L - q, L)[:, None]            # [q][L]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q).permute(1, 0, 2)[None], torch.from_numpy(K)[None, None].expand(1, H, L, 128),
        torch.from_numpy(V)[None, None].expand(1, H, L, 128), attn_mask=mask[None, None], scale=scale)[0]
    for j in range(q):
        O, lse = A.sparse_attention_row(Q[j], K, V, blocks, L - q + j, scale)
        np.testing.assert_allclose(O, ref[:, j].numpy(), rtol=1e-12, atol=1e-13)
        s = scale * Q[j] @ K[:L - q + j + 1].T
        np.testing.assert_allclose(lse, logsumexp(s, axis=1), rtol=1e-13)


def test_identical_keys_give_mean_of_values():
    q, K, V = _row_setup(2)
    K[:] = K[0]
    blocks = np.array([1, 4, 6])
    O, _ = A.sparse_attention_row(q, K, V, blocks, 999, 0.1)
    toks = np.concatenate([np.arange(128 * i, 128 * i + 128) for i in blocks])
    np.testing.assert_allclose(O, np.broadcast_to(V[toks].mean(0), O.shape), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("P", [1, 2, 3, 5, 8, 13, 16, 40])
def test_split_then_merge_equals_unsplit(P):
    """Any partition count, including partitions that are empty (P > k, or the
    -1 padding of a short row), merges back to the unsplit result."""
    q, K, V = _row_setup(3, L=2000)
    blocks = np.array([0, 3, 4, 7, 8, 11, 12, 15, -1, -1, -1, -1, -1, -1, -1, -1])
    pos = 1950
    O, lse = A.sparse_attention_row(q, K, V, blocks, pos, 0.09)
    m, l, o = A.split_partials(q, K, V, blocks, pos, 0.09, P)
    assert m.shape == (16, P)
    if P > 8:
        assert np.isneginf(m).any() and (l[np.isneginf(m)] == 0).all()
    O2, lse2 = A.lse_merge(m, l, o)
    np.testing.assert_allclose(O2, O, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13)


def test_merge_all_empty_row():
    m = np.full((2, 4), -np.inf)
    O, lse = A.lse_merge(m, np.zeros((2, 4)), np.zeros((2, 4, 128)))
    assert (O == 0).all() and np.isneginf(lse).all()


def test_merge_against_logsumexp():
    rng = np.random.default_rng(4)
    m = rng.standard_normal((5, 6)) * 10
    l = rng.random((5, 6)) + 0.5
    o = rng.standard_normal((5, 6, 128))
    O, lse = A.lse_merge(m, l, o)
    np.testing.assert_allclose(lse, logsumexp(m + np.log(l), axis=1), rtol=1e-13)
    wts = np.exp(m + np.log(l) - lse[:, None])                 # each partition's share of the mass
    np.testing.assert_allclose(O, (o / l[..., None] * wts[..., None]).sum(1), rtol=1e-11, atol=1e-13)


def test_causality_tokens_after_pos_ignored():
    q, K, V = _row_setup(5)
    blocks = np.array([2, 5, 7])
    O, lse = A.sparse_attention_row(q, K, V, blocks, 960, 0.1)
    K2, V2 = K.copy(), V.copy()
    K2[961:] = 1e6
    V2[961:] = np.nan
    O2, lse2 = A.sparse_attention_row(q, K2, V2, blocks, 960, 0.1)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(lse, lse2)


def test_wrong_block_table_fails_tolerance():
    """Negative control: attending over other blocks is far outside the parity
    tolerance (1e-2 max|O| + 1e-3)."""
    q, K, V = _row_setup(6, L=4096)
    O, _ = A.sparse_attention_row(q, K, V, np.array([1, 5, 9, 20]), 4095, 1 / np.sqrt(128))
    O2, _ = A.sparse_attention_row(q, K, V, np.array([1, 5, 9, 21]), 4095, 1 / np.sqrt(128))
    assert np.abs(O2 - O).max() > 1e-2 * np.abs(O).max() + 1e-3


# ---------------------------------------------------------------- whole step
def _tiny(**kw):
    return W.make_inputs(W.WORKLOADS["tiny"].with_(**kw))


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_step_dense_topk_equals_sdpa_over_dequantized_cache(fmt):
    inp = _tiny(topk=16, kv_format=fmt, idx_format=fmt)    # 16 pages: top-k covers every block
    r = S.decode_step_ref(inp)
    assert list(r["block_table"][0, 0]) == list(range(16))
    L = int(inp.contexts[0])
    K = F.READ[fmt](r["pools"]["k"], inp.page_table[0], L)
    V = F.READ[fmt](r["pools"]["v"], inp.page_table[0], L)
    # the cache holds the quantized rows: within the format's error of the fp32 rows
    assert np.abs(K - inp.rows("k", 0)).max() <= 0.25 * np.abs(inp.rows("k", 0)).max()
    qa, codes = S.attention_query(inp)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qa[0, 0])[None, :, None], torch.from_numpy(K)[None, None].expand(1, 4, L, 128),
        torch.from_numpy(V)[None, None].expand(1, 4, L, 128), scale=1 / np.sqrt(128))[0, :, 0]
    np.testing.assert_allclose(r["O"][0, 0], ref.numpy(), rtol=1e-12, atol=1e-13)


def test_step_store_writes_new_rows_where_prefix_ends():
    inp = _tiny()
    pre = {s: S.build_cache(inp, s, "mxfp4") for s in ("k", "v", "idx")}
    r = S.decode_step_ref(inp, pools=pre)
    L = int(inp.contexts[0])
    for s in ("k", "v", "idx"):
        got = F.mxfp4_read(r["pools"][s], inp.page_table[0], L)
        want = F.mxfp4_dequantize(*F.mxfp4_quantize_rows(inp.rows(s, 0)))
        np.testing.assert_array_equal(got, want)
        # before the step the last slot is still poisoned
        assert np.isnan(F.mxfp4_read(pre[s], inp.page_table[0], L, [L - 1])).all()


def test_step_page_table_permutation_invariance():
    inp = _tiny()
    r = S.decode_step_ref(inp)
    perm = np.random.default_rng(9).permutation(inp.num_pages)
    inp2 = _tiny()
    inp2.page_table = np.where(inp.page_table >= 0, perm[inp.page_table], -1).astype(np.int32)
    r2 = S.decode_step_ref(inp2)
    np.testing.assert_array_equal(r["block_table"], r2["block_table"])
    np.testing.assert_array_equal(r["O"], r2["O"])


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_step_poison_vs_zero_tails_identical(fmt):
    wl = W.WORKLOADS["tiny"].with_(ctx_rule=("fixed", 2000), kv_format=fmt, idx_format=fmt)   # last page partly filled
    inp = W.make_inputs(wl)
    pre = {s: S.build_cache(inp, s, fmt) for s in ("k", "v", "idx")}
    r = S.decode_step_ref(inp, pools=pre)
    zero = {s: S.build_cache(inp, s, fmt, fill=0) for s in ("k", "v", "idx")}
    r2 = S.decode_step_ref(inp, pools=zero)
    np.testing.assert_array_equal(r["O"], r2["O"])
    np.testing.assert_array_equal(r["block_table"], r2["block_table"])


# ---------------------------------------------------------------- a step that reuses a selection
def test_reuse_step_with_its_own_selection_is_the_full_step():
    """A layer that reuses the block selection the full step would make gets the
    full step's attention output and K / V pages, bit for bit."""
    inp = _tiny(q=3)
    r = S.decode_step_ref(inp)
    r2 = S.decode_step_reuse_ref(inp, r["block_table"])
    np.testing.assert_array_equal(r2["O"], r["O"])
    np.testing.assert_array_equal(r2["lse"], r["lse"])
    np.testing.assert_array_equal(r2["q8"], r["q8"])
    for s in ("k", "v"):
        np.testing.assert_array_equal(r2["pools"][s], r["pools"][s])
    assert "idx" not in r2["pools"]


def test_reuse_step_over_every_block_is_causal_dense_attention():
    """Every block listed: each row is plain causal attention over the whole
    dequantized cache (torch SDPA over positions <= the row's position)."""
    inp = _tiny(q=3, topk=16)
    L = int(inp.contexts[0])
    table = np.tile(np.arange(16), (1, 3, 1))
    r = S.decode_step_reuse_ref(inp, table)
    K = F.mxfp4_read(r["pools"]["k"], inp.page_table[0], L)
    V = F.mxfp4_read(r["pools"]["v"], inp.page_table[0], L)
    qa, _ = S.attention_query(inp)
    for j in range(3):
        pos = L - 3 + j
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qa[0, j])[None, :, None],
            torch.from_numpy(K[:pos + 1])[None, None].expand(1, 4, pos + 1, 128),
            torch.from_numpy(V[:pos + 1])[None, None].expand(1, 4, pos + 1, 128), scale=1 / np.sqrt(128))[0, :, 0]
        np.testing.assert_allclose(r["O"][0, j], ref.numpy(), rtol=1e-12, atol=1e-13)


def test_reuse_step_skips_empty_and_out_of_range_entries():
    inp = _tiny(q=2, topk=6)
    clean = np.array([[[3, 7, 9, 15, -1, -1], [3, 7, 9, 15, -1, -1]]])
    noisy = np.array([[[-1, 3, 400, 7, -7, 9], [15, 3, 7, 9, 16, 10**6]]])
    noisy[0, 0, 2] = 400                                  # 400 * 128 is past every position
    noisy[0, 0, 4] = 15
    a = S.decode_step_reuse_ref(inp, clean)
    b = S.decode_step_reuse_ref(inp, noisy)
    np.testing.assert_allclose(b["O"], a["O"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(b["lse"], a["lse"], rtol=1e-12)
