"""Sparse softmax attention over selected blocks, split partials and their
log-sum-exp merge (oracle; test infrastructure only).

ATOM PR #2812, "Mono decode over the MXFP4 KV and index caches", commit
message of the MXFP4 main-KV commit: the split stage attends over the pages
of the sparse (block) table, a selected block being one 128-token page, and
writes per-partition partial outputs, maxima and sums (sp_o / sp_m / sp_l)
that a merge combines. The main KV has one head shared by every query head
(GQA), head_dim 128.

For query row j at pos_j, head h, over the token set T of its selected blocks
(tokens t <= pos_j only):

    s_t = sm_scale * q[h] . K[t];  m = max s;  l = sum exp(s - m)
    O[h] = sum exp(s_t - m) V[t] / l;  lse = m + ln l

Partition p of a row (a reading: the library's contract for its partials)
covers block-table slots [p * c, min((p + 1) * c, k)) with c = ceil(k / P);
slots holding -1 are empty. A partition with no token gives (m, l, o) =
(-inf, 0, 0); the merge skips it.
"""
from __future__ import annotations

import math

import numpy as np

TOKENS = 128


def gather_tokens(block_ids: np.ndarray, pos: int) -> np.ndarray:
    """Token positions of the selected blocks that a row at ``pos`` sees."""
    toks = []
    for i in block_ids:
        if i < 0:
            continue
        t = np.arange(i * TOKENS, (i + 1) * TOKENS)
        toks.append(t[t <= pos])
    return np.concatenate(toks) if toks else np.zeros(0, dtype=np.int64)


def softmax_partial(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float):
    """Unnormalized partial (m, l, o) of heads q [H][128] over rows K, V [T][128]."""
    H = q.shape[0]
    if K.shape[0] == 0:
        return np.full(H, -np.inf), np.zeros(H), np.zeros((H, V.shape[1]))
    s = sm_scale * (q @ K.T)                                  # [H][T]
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    return m, p.sum(axis=1), p @ V


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float):
    """Normalized attention (O [H][128], lse [H]) of heads q over K, V."""
    m, l, o = softmax_partial(q, K, V, sm_scale)
    return o / l[:, None], m + np.log(l)


def sparse_attention_row(q: np.ndarray, K_all: np.ndarray, V_all: np.ndarray,
                         block_ids: np.ndarray, pos: int, sm_scale: float):
    """One query row: q [H][128], K_all / V_all [L][128] (dequantized sequence)."""
    t = gather_tokens(block_ids, pos)
    return attend(q, K_all[t], V_all[t], sm_scale)


def split_partials(q: np.ndarray, K_all: np.ndarray, V_all: np.ndarray, block_ids: np.ndarray,
                   pos: int, sm_scale: float, P: int):
    """Per-partition (m [H][P], l [H][P], o [H][P][128]) of one query row."""
    k = len(block_ids)
    c = math.ceil(k / P)
    H = q.shape[0]
    m = np.empty((H, P))
    l = np.empty((H, P))
    o = np.empty((H, P, V_all.shape[1]))
    for p in range(P):
        t = gather_tokens(block_ids[p * c:min((p + 1) * c, k)], pos)
        m[:, p], l[:, p], o[:, p, :] = softmax_partial(q, K_all[t], V_all[t], sm_scale)
    return m, l, o


def lse_merge(m: np.ndarray, l: np.ndarray, o: np.ndarray):
    """Merge partials over the last partition axis: m, l [..][P], o [..][P][D].

    M = max_p m_p;  L = sum_p l_p exp(m_p - M);  O = sum_p o_p exp(m_p - M) / L;
    lse = M + ln L. Empty partitions (m_p = -inf) weigh 0. A row whose partitions
    are all empty gives O = 0, lse = -inf."""
    M = m.max(axis=-1)
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    wgt = np.where(np.isfinite(m), np.exp(m - Ms[..., None]), 0.0)
    L = (l * wgt).sum(axis=-1)
    num = (o * wgt[..., None]).sum(axis=-2)
    with np.errstate(invalid="ignore", divide="ignore"):
        O = np.where(finite[..., None], num / np.where(L > 0, L, 1.0)[..., None], 0.0)
        lse = np.where(finite, M + np.log(np.where(L > 0, L, 1.0)), -np.inf)
    return O, lse
