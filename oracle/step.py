"""The whole decode step, stage by stage, in the pages' order (oracle; test
infrastructure only).

ATOM PR #2812, "Mono decode over the MXFP4 KV and index caches" (What, and
the commit messages): the step's first kernel stores the new index-key, K and
V rows into the cache pages and the query as e4m3 (MXFP4 main KV; an FP8 main
KV keeps a bf16 query, commit message of the e4m3 q store); the index scorer
scores every page of the index cache and the select stage picks the top-k
blocks; the split stage attends over the selected pages and the merge
combines its partials. This module runs those stages unsplit (the merge of
partials is exercised separately in ``attention``).

Cache contents before the step: positions 0 .. L - q - 1 of each sequence
(all L positions when the workload does not include the store); the step
stores positions L - q .. L - 1.
"""
from __future__ import annotations

import numpy as np

from . import attention, formats, indexer

TOKENS = 128


def build_cache(inp, stream: str, fmt: str, seqs=None, fill=None) -> np.ndarray:
    """A pool holding the pre-step rows of every (or the listed) sequence,
    quantized by the oracle; every other byte is the input's poison (or ``fill``)."""
    from workloads import new_pool
    pool = new_pool(inp.num_pages, formats.PAGE_BYTES[fmt])
    if fill is not None:
        pool[:] = fill
    for b in (range(inp.wl.B) if seqs is None else seqs):
        n = inp.prefix_len(b)
        if n:
            formats.STORE[fmt](pool, inp.page_table[b], 0, inp.rows(stream, b)[:n])
    return pool


def attention_query(inp) -> tuple:
    """(query as float64 [B][q][H][128], e4m3 codes or None).

    MXFP4 main KV: the query is stored as saturating e4m3 with unit scale and the
    split stage consumes those codes. FP8 and NVFP4 main KV: the bf16 query is
    used as is (the e4m3 query store is the MXFP4 path's; a reading for NVFP4,
    which the pages do not describe)."""
    wl = inp.wl
    if wl.kv_format == "mxfp4":
        src = formats.bf16_to_f64(inp.q_bf16) if wl.q_dtype == "bf16" else inp.q.astype(np.float64)
        codes = formats.e4m3_encode(src)
        return formats.E4M3_TABLE[codes.astype(np.int64)], codes
    return formats.bf16_to_f64(inp.q_bf16), None


def decode_step_ref(inp, pools=None, seqs=None) -> dict:
    """Run the step on sequences ``seqs`` (default: all).

    pools: {"k", "v", "idx"} pre-step pools (copied, not modified); built with
    ``build_cache`` when None. Returns the post-step pools, the query codes,
    block scores [B][q][max_pages] (-inf outside the candidates), the block
    table [B][q][topk] and the output O [B][q][H][128] with lse [B][q][H]
    (rows of sequences not in ``seqs`` are NaN / -2)."""
    wl = inp.wl
    seqs = list(range(wl.B)) if seqs is None else list(seqs)
    fmts = {"k": wl.kv_format, "v": wl.kv_format, "idx": wl.idx_format}
    if pools is None:
        pools = {s: build_cache(inp, s, fmts[s], seqs) for s in fmts}
    pools = {s: p.copy() for s, p in pools.items()}

    # 1. row store of the step's new rows (positions L - q .. L - 1)
    if wl.full_step:
        for s, f in fmts.items():
            for b in seqs:
                L = int(inp.contexts[b])
                formats.STORE[f](pools[s], inp.page_table[b], L - wl.q, inp.rows(s, b)[L - wl.q:])

    # 2. query store
    q_att, q8 = attention_query(inp)

    B, q, H = wl.B, wl.q, wl.H
    maxp = inp.max_pages
    scores = np.full((B, q, maxp), -np.inf)
    table = np.full((B, q, wl.topk), -2, dtype=np.int64)
    O = np.full((B, q, H, 128), np.nan)
    lse = np.full((B, q, H), np.nan)
    qI = formats.bf16_to_f64(inp.q_idx)
    w = inp.w.astype(np.float64)
    for b in seqs:
        L = int(inp.contexts[b])
        # 3. index scores over every page of the sequence, 4. top-k per row
        kI = formats.READ[wl.idx_format](pools["idx"], inp.page_table[b], L)
        S = indexer.index_scores(kI, qI[b], w[b], L)
        scores[b, :, :S.shape[1]] = S
        ncand = indexer.n_candidates(L, q)
        pos = indexer.row_positions(L, q)
        for j in range(q):
            table[b, j] = indexer.topk_blocks(S[j], int(ncand[j]), wl.topk)
        # 5. attention over the selected blocks (the union of the rows' blocks is read once)
        sel = np.unique(table[b][table[b] >= 0])
        toks = np.concatenate([np.arange(i * TOKENS, min((i + 1) * TOKENS, L)) for i in sel])
        Kd = formats.READ[wl.kv_format](pools["k"], inp.page_table[b], L, toks)
        Vd = formats.READ[wl.kv_format](pools["v"], inp.page_table[b], L, toks)
        K_all = np.zeros((L, 128))
        V_all = np.zeros((L, 128))
        K_all[toks] = Kd
        V_all[toks] = Vd
        for j in range(q):
            O[b, j], lse[b, j] = attention.sparse_attention_row(
                q_att[b, j], K_all, V_all, table[b, j], int(pos[j]), wl.sm_scale)
    return {"pools": pools, "q8": q8, "scores": scores, "block_table": table, "O": O, "lse": lse}


def decode_step_reuse_ref(inp, block_table: np.ndarray, pools=None, seqs=None) -> dict:
    """The step of a layer that reuses an earlier layer's sparse block selection
    (ATOM PR #2686, "Enable Mono decode with fixed DSpark verify", the review
    thread's commit message: under an index_topk_freq schedule a layer can
    reuse a selection instead of making its own).

    Reading: such a layer scores nothing, so the step is the row store of its
    new K and V rows, the query store and attention of each row over the given
    blocks [B][q][k] (entries < 0 or past the row's position contribute no
    tokens), then the merge. The index pool is neither read nor written.
    Returns the post-step pools ("k", "v"), the query codes and O, lse as
    ``decode_step_ref`` does."""
    wl = inp.wl
    seqs = list(range(wl.B)) if seqs is None else list(seqs)
    fmts = {"k": wl.kv_format, "v": wl.kv_format}
    if pools is None:
        pools = {s: build_cache(inp, s, fmts[s], seqs) for s in fmts}
    pools = {s: pools[s].copy() for s in fmts}
    if wl.full_step:
        for s, f in fmts.items():
            for b in seqs:
                L = int(inp.contexts[b])
                formats.STORE[f](pools[s], inp.page_table[b], L - wl.q, inp.rows(s, b)[L - wl.q:])
    q_att, q8 = attention_query(inp)
    B, q, H = wl.B, wl.q, wl.H
    O = np.full((B, q, H, 128), np.nan)
    lse = np.full((B, q, H), np.nan)
    for b in seqs:
        L = int(inp.contexts[b])
        pos = indexer.row_positions(L, q)
        ids = np.asarray(block_table[b])
        sel = np.unique(ids[(ids >= 0) & (ids * TOKENS < L)])
        toks = (np.concatenate([np.arange(i * TOKENS, min((i + 1) * TOKENS, L)) for i in sel])
                if len(sel) else np.zeros(0, dtype=np.int64))
        K_all = np.zeros((L, 128))
        V_all = np.zeros((L, 128))
        if len(toks):
            K_all[toks] = formats.READ[wl.kv_format](pools["k"], inp.page_table[b], L, toks)
            V_all[toks] = formats.READ[wl.kv_format](pools["v"], inp.page_table[b], L, toks)
        for j in range(q):
            O[b, j], lse[b, j] = attention.sparse_attention_row(
                q_att[b, j], K_all, V_all, ids[j], int(pos[j]), wl.sm_scale)
    return {"pools": pools, "q8": q8, "O": O, "lse": lse}
