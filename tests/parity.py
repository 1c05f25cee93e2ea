"""Parity helpers shared by the GPU tests: tolerances and comparisons against
the oracle. Tolerances, each with its derivation:

- page bytes, q codes, block ids: exact;
- block scores: |S_gpu - S_ref| <= 1e-5 * S_abs + 1e-30, where S_abs is the
  block score computed over |q| and |k| (no cancellation): the bf16 products
  are exact on the GPU, and fp32 accumulation of 128 products plus the 4-head
  weighted sum is within (128 + 8) * 2^-24 < 1e-5 of that magnitude;
- top-k: the GPU set may differ from the oracle's only in blocks whose oracle
  score is within 1e-4 * |S_(k)| of the oracle's k-th score S_(k);
- attention output: max |O_gpu - O_ref| <= 1e-2 * max |O_ref| + 1e-3 over a
  workload's output tensor.
"""
from __future__ import annotations

import numpy as np

from oracle import attention as OA
from oracle import formats as OF
from oracle import indexer as OI

SCORE_REL = 1e-5
TIE_REL = 1e-4
ATT_REL, ATT_ABS = 1e-2, 1e-3


def bf16_tensor_to_f64(t) -> np.ndarray:
    import torch
    return t.float().cpu().numpy().astype(np.float64) if t.dtype == torch.bfloat16 else t.cpu().numpy()


def score_bound(kI, qI, w, L):
    """Per-block error scale: the block score over |q| and |k|."""
    return OI.index_scores(np.abs(kI), np.abs(qI), w, L)


def check_scores(S_gpu, S_ref, S_abs, ncand):
    """S_* [q][n_blocks]; candidate entries within the bound, others -inf."""
    for j in range(S_ref.shape[0]):
        nc = int(ncand[j])
        g, r, a = S_gpu[j, :nc], S_ref[j, :nc], S_abs[j, :nc]
        err = np.abs(g - r)
        bad = ~(err <= SCORE_REL * a + 1e-30)
        assert not bad.any(), (f"row {j}: {bad.sum()} scores out of bound; worst block {np.argmax(err - SCORE_REL * a)}"
                               f" gpu {g[bad][:3]} ref {r[bad][:3]}")
        assert np.isneginf(S_gpu[j, nc:S_ref.shape[1]]).all(), f"row {j}: non-candidate blocks not -inf"


def check_topk(table_gpu, table_ref, S_ref_row, ncand, k):
    """One row: equal sets, or differences only among near-ties of the k-th score."""
    g = set(int(x) for x in table_gpu if x >= 0)
    r = set(int(x) for x in table_ref if x >= 0)
    assert len(g) == min(k, ncand) == len(r), (sorted(g), sorted(r))
    assert list(table_gpu[:len(g)]) == sorted(g) and all(x == -1 for x in table_gpu[len(g):])
    if g == r:
        return True
    kth = OI.kth_score(S_ref_row, ncand, k)
    for i in g ^ r:
        assert abs(S_ref_row[i] - kth) <= TIE_REL * abs(kth), \
            f"block {i} differs and is not a near tie: {S_ref_row[i]} vs k-th {kth}"
    return False


def check_attention(O_gpu, O_ref, what=""):
    err = np.abs(O_gpu - O_ref)
    bound = ATT_REL * np.abs(O_ref).max() + ATT_ABS
    assert np.isfinite(O_gpu).all(), f"{what}: non-finite output"
    assert err.max() <= bound, f"{what}: max err {err.max():.3e} > {bound:.3e}"
    return err.max(), bound


def seq_pages(page_table_row, L):
    n = (int(L) + 127) // 128
    return page_table_row[:n].astype(np.int64)


def compare_pool_pages(pool_gpu: np.ndarray, pool_ref: np.ndarray, pages, page_bytes: int, what=""):
    a = pool_gpu.reshape(-1, page_bytes)[pages]
    b = pool_ref.reshape(-1, page_bytes)[pages]
    if not np.array_equal(a, b):
        diff = np.argwhere(a != b)
        p, off = diff[0]
        raise AssertionError(f"{what}: {len(diff)} bytes differ; first at page {pages[p]} byte {off}: "
                             f"gpu {a[p, off]:#04x} ref {b[p, off]:#04x}")


def oracle_attention_with_table(inp, pools, q_att, table, b, seq_read=None):
    """Oracle attention of sequence b's rows over a given block table [q][k]."""
    wl = inp.wl
    L = int(inp.contexts[b])
    sel = np.unique(table[table >= 0])
    toks = np.concatenate([np.arange(i * 128, min((i + 1) * 128, L)) for i in sel])
    K_all = np.zeros((L, 128))
    V_all = np.zeros((L, 128))
    K_all[toks] = OF.READ[wl.kv_format](pools["k"], inp.page_table[b], L, toks)
    V_all[toks] = OF.READ[wl.kv_format](pools["v"], inp.page_table[b], L, toks)
    pos = OI.row_positions(L, wl.q)
    O = np.empty((wl.q, wl.H, 128))
    lse = np.empty((wl.q, wl.H))
    for j in range(wl.q):
        O[j], lse[j] = OA.sparse_attention_row(q_att[b, j], K_all, V_all, table[j], int(pos[j]), wl.sm_scale)
    return O, lse, K_all, V_all
