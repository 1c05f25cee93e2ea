"""Device-side copies of a workload's inputs, for the GPU tests and the bench.

The caches are filled by the library's own row store from the seeded fp32 rows
(the oracle fills its copy with its own quantizer), so the two sides share
only the random inputs. Importing this module loads the HIP library; the
oracle never imports it.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import sparse_attention_decode_mxfp4_amd as mx

from . import POISON_BYTE, StepInputs

STREAMS = ("k", "v", "idx")


def empty_pools(inp: StepInputs, device="cuda"):
    wl = inp.wl
    fmts = {"k": wl.kv_format, "v": wl.kv_format, "idx": wl.idx_format}
    return {s: torch.full((inp.num_pages * mx.PAGE_BYTES[fmts[s]],), POISON_BYTE, dtype=torch.uint8, device=device)
            for s in STREAMS}


def fill_prefix(inp: StepInputs, pools, seqs=None, chunk_rows=1 << 20, device="cuda"):
    """Store the pre-step rows of every (or the listed) sequence with the
    library's row store."""
    wl = inp.wl
    fmts = {"k": wl.kv_format, "v": wl.kv_format, "idx": wl.idx_format}
    store = {"mxfp4": mx.mxfp4_row_store, "fp8": mx.fp8_row_store, "nvfp4": mx.nvfp4_row_store}
    jobs = [(s, b) for s in STREAMS for b in (range(wl.B) if seqs is None else seqs)]
    with ThreadPoolExecutor(max_workers=8) as ex:          # numpy draws release the GIL
        for (s, b), rows in zip(jobs, ex.map(lambda sb: inp.rows(*sb), jobs)):
            n = inp.prefix_len(b)
            for c0 in range(0, n, chunk_rows):
                c1 = min(n, c0 + chunk_rows)
                r = torch.from_numpy(np.ascontiguousarray(rows[c0:c1])).to(device)
                sl = torch.from_numpy(inp.slot_mapping(b, c0, c1)).to(device)
                store[fmts[s]](r, sl, pools[s])
    return pools


def make_cache(inp: StepInputs, pools, device="cuda", table=None, ctx=None) -> mx.Cache:
    """A cache view over `pools`; `table` / `ctx` (device tensors) let several
    caches share one page table and one context-length vector, as the layers of
    a decode step share the sequences' block table."""
    wl = inp.wl
    if table is None:
        table = torch.from_numpy(inp.page_table).to(device)
    if ctx is None:
        ctx = torch.from_numpy(inp.contexts.astype(np.int32)).to(device)
    return mx.Cache(pools["k"], pools["v"], pools["idx"], table, ctx, wl.kv_format, wl.idx_format)


def step_tensors(inp: StepInputs, device="cuda") -> dict:
    """The step's per-call inputs on the device."""
    wl = inp.wl
    if wl.q_dtype == "f32" and wl.kv_format == "mxfp4":
        query = torch.from_numpy(inp.q).to(device)
    else:
        query = torch.from_numpy(inp.q_bf16.view(np.int16)).to(device).view(torch.bfloat16)
    d = {
        "query": query,
        "q_idx": torch.from_numpy(inp.q_idx.view(np.int16)).to(device).view(torch.bfloat16),
        "w": torch.from_numpy(inp.w).to(device),
    }
    if wl.full_step:
        for s in STREAMS:
            d[s + "_new"] = torch.from_numpy(inp.new_rows(s)).to(device)
    return d
