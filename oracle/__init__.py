"""CPU oracle for the sparse-attention decode step over MXFP4 / FP8 caches.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code, tables or
constants with the HIP library, and it never consumes a value the HIP library
produced.

It is plain NumPy, float64 for every floating-point quantity and exact
integers for codes, written to be checked against the pages by eye:

- ``formats``   e2m1 / e8m0 / e4m3 codecs, the MXFP4 row quantizer, the FP8
                per-token quantizer and the two page layouts.
- ``indexer``   block scores of the index cache and the exact top-k.
- ``attention`` sparse softmax attention, split partials and their LSE merge.
- ``step``      the whole decode step: row store, q store, scoring, top-k,
                attention.

Sources (the pages): ATOM PR #2812 "[MiniMax-M3.1] Mono decode over the MXFP4
KV and index caches" (its commit messages, What, Tested, Limits), ATOM PR
#2686 "[MiniMax-M3.1] Enable Mono decode with fixed DSpark verify" (Summary),
and vLLM PR #60528 (MiniMax-M3 sparse decode through ATOM's tensor library;
Overview, Details). Where the pages leave a step open, the plain reading taken
is stated at the function; the OCP Microscaling Formats (MX) v1.0
specification is the public definition used for e2m1 and e8m0.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, library routines (torch's e4m3 and e8m0 dtypes, torch's
scaled-dot-product attention), invariants or brute force, except the two items
marked "parity unpinned" in ``formats``: byte identity of the MXFP4 page with
the pages' own writer (not available), and the FP8 per-token scale rule (the
pages name a per-token fp32 scale but not its rule).
"""
from . import formats, indexer, attention, step  # noqa: F401
