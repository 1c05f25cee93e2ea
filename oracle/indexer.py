"""Indexer block scores and exact top-k block selection (oracle; test infrastructure only).

Score of block i for query row j (the tiny decode configuration's definition:
"block score = max over tokens in the block of sum_h w_h * ReLU(q_h . k)",
served by the index scorer of ATOM PR #2812, "Mono decode over the MXFP4 KV
and index caches", commit message of the MXFP4 index-cache commit):

    S[j, i] = max over t in block i, t <= pos_j, of  sum_h w[j, h] * max(0, q_I[j, h] . k_I[t])

Readings where the pages are silent:
- causal speculative rows: row j of a sequence with context L (which already
  holds the step's q new rows) sits at pos_j = L - q + j and sees tokens
  t <= pos_j only (fixed-draft verify, ATOM PR #2686 Summary);
- a block is a candidate for row j when it holds at least one token t <= pos_j,
  i.e. blocks 0 .. pos_j // 128; there is no forced sink or local block;
- top-k is per query row; the k highest scores win, ties go to the lower block
  id, a row with fewer than k candidates takes all of them; the selected ids are
  listed in ascending order and the list is padded with -1.
"""
from __future__ import annotations

import numpy as np

TOKENS = 128


def row_positions(L: int, q: int) -> np.ndarray:
    """Positions of a sequence's q query rows (the last q tokens of its context)."""
    return np.arange(L - q, L, dtype=np.int64)


def index_scores(k_idx: np.ndarray, q_idx: np.ndarray, w: np.ndarray, L: int) -> np.ndarray:
    """Block scores of one sequence.

    k_idx: float64 [L][128] dequantized index keys (positions 0 .. L-1)
    q_idx: float64 [q][H_I][128]; w: float64 [q][H_I]
    Returns float64 [q][ceil(L/128)]; -inf where a block is not a candidate.
    """
    q = q_idx.shape[0]
    pos = row_positions(L, q)
    logits = np.einsum("jhd,td->jht", q_idx, k_idx[:L], optimize=True)        # q_h . k_t
    tok = np.einsum("jh,jht->jt", w, np.maximum(logits, 0.0))                 # sum_h w_h ReLU(.)
    t = np.arange(L)
    tok = np.where(t[None, :] <= pos[:, None], tok, -np.inf)                  # causal rows
    nb = (L + TOKENS - 1) // TOKENS
    padded = np.full((q, nb * TOKENS), -np.inf)
    padded[:, :L] = tok
    return padded.reshape(q, nb, TOKENS).max(axis=2)


def n_candidates(L: int, q: int) -> np.ndarray:
    """Candidate block count of each row: blocks 0 .. pos_j // 128."""
    return row_positions(L, q) // TOKENS + 1


def topk_blocks(scores_row: np.ndarray, n_cand: int, k: int) -> np.ndarray:
    """Exact top-k over the first n_cand blocks: order by (score descending,
    block id ascending), keep min(k, n_cand), list ascending, pad with -1."""
    s = np.asarray(scores_row[:n_cand], dtype=np.float64)
    ids = np.arange(n_cand)
    order = np.lexsort((ids, -s))            # primary key -s, secondary key id
    keep = np.sort(order[:min(k, n_cand)])
    out = np.full(k, -1, dtype=np.int64)
    out[:keep.size] = keep
    return out


def kth_score(scores_row: np.ndarray, n_cand: int, k: int) -> float:
    """The k-th largest candidate score (the boundary the tie tolerance is measured at)."""
    s = np.sort(np.asarray(scores_row[:n_cand], dtype=np.float64))[::-1]
    return float(s[min(k, n_cand) - 1])
