"""Seeded synthetic inputs for the sparse-attention decode step.

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic (no quantization, no scoring, no selection, no softmax), so
that the CPU oracle and the GPU path can both consume it without sharing any
of the computation they are compared on.

Every array comes from ``numpy.random.default_rng`` keyed by
``(seed, stream, sequence)``, so any single sequence of a large workload can be
regenerated alone (the oracle checks sampled sequences of the big workloads).

Workloads (the shapes of the pages' decode configurations, one TP rank's share):

- ``tiny``   B=1, q=1, 4:1 GQA, 2048-token context (16 pages), top-k 4, MXFP4.
- ``fp8``    B=4, q=4 (1 + 3 speculative), 16:1, FP8 e4m3 cache with a
             per-token fp32 scale, context 16384, top-k 16, 1 % outliers x20.
- ``mxfp4_65k`` B=4, q=8 (1 + 7 draft), 16:1, MXFP4 K/V/index, context
             65536 - u (u in 1..127, so the last page is partly filled and its
             tail stays poisoned), random non-contiguous page tables, top-k 16.
- ``long``   B=4, q=8, MXFP4, ragged contexts U[131072, 262144], top-k 32.
- ``headline`` B=4, q=8, MXFP4, every context 262144, top-k 32, full step.
- ``b32``    B=32, q=8, MXFP4, ragged U[8192, 262144], top-k 32, full step.
- ``nvfp4``  B=4, q=8, 16:1, NVFP4 K/V and index (e2m1 in 16-element blocks,
             e4m3 block scales, per-token fp32 scale), context 16384 - u,
             top-k 16, 1 % outliers x20.
- ``headline_nvfp4`` the headline shape (B=4, q=8, every context 262144,
             top-k 32) over NVFP4 K/V and index caches, bf16 query.

Values: K, V, index-K and q are N(0, 1) fp32; with ``outliers`` about 1 % of
the elements (Binomial(N, 0.01) uniformly drawn positions) are multiplied by 20. Index queries are bf16 (fp32 N(0,1)
rounded to nearest even); index-head weights are U(0, 1) fp32.

Pools: every cache pool starts filled with the byte 0xFF. In every cache format
that byte pattern decodes to NaN (an all-ones e8m0 scale, an e4m3 0xFF code or
block scale, an all-ones fp32 scale), so unused pages and the unwritten tail of
a partly filled page are NaN-poisoned without this module knowing the page
layout.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

PAGE_TOKENS = 128          # tokens per page (= one selectable block)
HEAD_DIM = 128             # head_dim of main K/V/q and of the index keys
POISON_BYTE = 0xFF

# random-stream ids, so that every array has its own independent generator
_S_K, _S_V, _S_IDX, _S_Q, _S_QI, _S_W, _S_TABLE, _S_CTX, _S_INJ = range(9)
_STREAM_OF = {"k": _S_K, "v": _S_V, "idx": _S_IDX}


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    q: int                 # query rows per sequence (1 + drafts)
    H: int                 # query heads sharing the one KV head
    H_I: int               # index heads
    topk: int
    kv_format: str         # "mxfp4" | "fp8" | "nvfp4"
    idx_format: str        # "mxfp4" | "fp8" | "nvfp4"
    q_dtype: str           # dtype of the attention q handed to the step: "f32" | "bf16"
    outliers: bool
    ctx_rule: tuple        # ("fixed", L) | ("fixed_minus_u", L, umax) | ("uniform", lo, hi) | ("list", (...))
    full_step: bool = True # the step's q new rows are stored by the step itself
    pool_slack: float = 1.25
    table_stride: int = 0  # page-table row length; 0 = the longest sequence's page count

    # ---- context lengths -------------------------------------------------
    def contexts(self) -> np.ndarray:
        """Context length of each sequence, including the step's q new rows."""
        kind = self.ctx_rule[0]
        if kind == "fixed":
            return np.full(self.B, self.ctx_rule[1], dtype=np.int64)
        rng = np.random.default_rng([self.seed, _S_CTX])
        if kind == "fixed_minus_u":
            L, umax = self.ctx_rule[1], self.ctx_rule[2]
            return (L - rng.integers(1, umax + 1, size=self.B)).astype(np.int64)
        if kind == "uniform":
            lo, hi = self.ctx_rule[1], self.ctx_rule[2]
            return rng.integers(lo, hi + 1, size=self.B).astype(np.int64)
        if kind == "list":
            return np.asarray(self.ctx_rule[1], dtype=np.int64)
        raise ValueError(kind)

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(HEAD_DIM)

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    "tiny": Workload("tiny", 0, 1, 1, 4, 4, 4, "mxfp4", "mxfp4", "bf16", False, ("fixed", 2048)),
    "fp8": Workload("fp8", 1, 4, 4, 16, 4, 16, "fp8", "fp8", "bf16", True, ("fixed", 16384)),
    "mxfp4_65k": Workload("mxfp4_65k", 2, 4, 8, 16, 4, 16, "mxfp4", "mxfp4", "f32", True,
                          ("fixed_minus_u", 65536, 127)),
    "long": Workload("long", 3, 4, 8, 16, 4, 32, "mxfp4", "mxfp4", "f32", True,
                     ("uniform", 131072, 262144)),
    "headline": Workload("headline", 5, 4, 8, 16, 4, 32, "mxfp4", "mxfp4", "f32", True,
                         ("fixed", 262144)),
    "b32": Workload("b32", 4, 32, 8, 16, 4, 32, "mxfp4", "mxfp4", "f32", True,
                    ("uniform", 8192, 262144)),
    "nvfp4": Workload("nvfp4", 6, 4, 8, 16, 4, 16, "nvfp4", "nvfp4", "bf16", True,
                      ("fixed_minus_u", 16384, 127)),
    "headline_nvfp4": Workload("headline_nvfp4", 7, 4, 8, 16, 4, 32, "nvfp4", "nvfp4", "bf16", True,
                               ("fixed", 262144)),
}


def pages_for(L: int) -> int:
    return (int(L) + PAGE_TOKENS - 1) // PAGE_TOKENS


@dataclass
class StepInputs:
    """Everything one decode step consumes, as host numpy arrays.

    Row tensors are produced lazily per (stream, sequence) by ``rows``.
    """
    wl: Workload
    contexts: np.ndarray          # int64 [B]
    num_pages: int                # pool size in pages (same numbering for K, V and index pools)
    page_table: np.ndarray        # int32 [B][max_pages], -1 past a sequence's pages
    q: np.ndarray                 # fp32 [B][q][H][128]   attention query (post norm/rope)
    q_bf16: np.ndarray            # uint16 [B][q][H][128] bf16 bits of q (used when q_dtype == "bf16")
    q_idx: np.ndarray             # uint16 [B][q][H_I][128] bf16 bits of the index query
    w: np.ndarray                 # fp32 [B][q][H_I]      index-head weights
    _row_cache: dict = field(default_factory=dict, repr=False)

    @property
    def max_pages(self) -> int:
        return self.page_table.shape[1]

    def rows(self, stream: str, b: int) -> np.ndarray:
        """fp32 [L_b][128] rows of one cache stream ("k", "v", "idx") for sequence b.

        Token t's row is the value the step's producer wrote (or writes) at
        position t; the last q rows are the step's new rows."""
        key = (stream, b)
        if key in self._row_cache:
            return self._row_cache[key]
        L = int(self.contexts[b])
        rng = np.random.default_rng([self.wl.seed, _STREAM_OF[stream], b])
        x = rng.standard_normal((L, HEAD_DIM), dtype=np.float32)
        if self.wl.outliers:
            # Binomial(N, 1 %) element positions, drawn uniformly (a repeat is scaled once)
            cnt = rng.binomial(L * HEAD_DIM, 0.01)
            x.reshape(-1)[rng.integers(0, L * HEAD_DIM, size=cnt)] *= np.float32(20.0)
        return x

    def cache_rows(self, stream: str, b: int, keep: bool = False) -> np.ndarray:
        x = self.rows(stream, b)
        if keep:
            self._row_cache[(stream, b)] = x
        return x

    def new_rows(self, stream: str) -> np.ndarray:
        """fp32 [B][q][128]: the step's new rows (positions L_b - q .. L_b - 1)."""
        out = np.empty((self.wl.B, self.wl.q, HEAD_DIM), dtype=np.float32)
        for b in range(self.wl.B):
            out[b] = self.rows(stream, b)[-self.wl.q:]
        return out

    def prefix_len(self, b: int) -> int:
        """Tokens already in the cache before the step (the step stores the rest)."""
        L = int(self.contexts[b])
        return L - self.wl.q if self.wl.full_step else L

    def slot_mapping(self, b: int, t0: int, t1: int) -> np.ndarray:
        """Caller-side slot ids (page * 128 + offset) of positions [t0, t1) of sequence b,
        the way a serving framework hands a cache writer its slot mapping."""
        t = np.arange(t0, t1, dtype=np.int64)
        return self.page_table[b, t // PAGE_TOKENS].astype(np.int64) * PAGE_TOKENS + t % PAGE_TOKENS


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (torch's dtype conversion)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def make_inputs(wl: Workload, inject_q: bool = False) -> StepInputs:
    """Draw the step's inputs for workload ``wl``.

    ``inject_q`` replaces 1 % of the attention-q elements by +-500 and +-inf
    (values outside the e4m3 range, to exercise the saturating q store)."""
    ctx = wl.contexts()
    n_pages = np.array([pages_for(L) for L in ctx], dtype=np.int64)
    need = int(n_pages.sum())
    num_pages = int(math.ceil(need * wl.pool_slack)) + 1
    max_pages = max(int(n_pages.max()), int(wl.table_stride))      # rows padded with -1 past a sequence
    rng = np.random.default_rng([wl.seed, _S_TABLE])
    perm = rng.permutation(num_pages)[:need].astype(np.int32)
    table = np.full((wl.B, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(wl.B):
        table[b, :n_pages[b]] = perm[off:off + n_pages[b]]
        off += n_pages[b]

    q = np.empty((wl.B, wl.q, wl.H, HEAD_DIM), dtype=np.float32)
    q_idx_f = np.empty((wl.B, wl.q, wl.H_I, HEAD_DIM), dtype=np.float32)
    w = np.empty((wl.B, wl.q, wl.H_I), dtype=np.float32)
    for b in range(wl.B):
        q[b] = np.random.default_rng([wl.seed, _S_Q, b]).standard_normal(q.shape[1:], dtype=np.float32)
        q_idx_f[b] = np.random.default_rng([wl.seed, _S_QI, b]).standard_normal(q_idx_f.shape[1:],
                                                                                dtype=np.float32)
        w[b] = np.random.default_rng([wl.seed, _S_W, b]).random(w.shape[1:], dtype=np.float32)
    if inject_q:
        r = np.random.default_rng([wl.seed, _S_INJ])
        sel = r.random(q.shape) < 0.01
        choice = r.integers(0, 4, size=q.shape)
        vals = np.array([500.0, -500.0, np.inf, -np.inf], dtype=np.float32)
        q[sel] = vals[choice[sel]]
    return StepInputs(wl=wl, contexts=ctx, num_pages=num_pages, page_table=table,
                      q=q, q_bf16=bf16_bits(q), q_idx=bf16_bits(q_idx_f), w=w)


def new_pool(num_pages: int, page_bytes: int) -> np.ndarray:
    """A host cache pool filled with the poison byte."""
    return np.full(num_pages * page_bytes, POISON_BYTE, dtype=np.uint8)
