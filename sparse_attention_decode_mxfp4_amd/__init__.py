"""Python binding of libmxsparse (include/mxsparse.h): argument marshalling only.

Every function checks tensor device, dtype, shape and contiguity, then passes
raw device pointers and torch's current HIP stream to the C ABI of the same
name. All computation happens in the library's HIP kernels; there is no other
implementation behind these functions. If the library is not built, every
call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxsparse.so")

MXS_OK, MXS_EINVAL, MXS_EUNSUPPORTED, MXS_EWORKSPACE, MXS_ELAUNCH = range(5)
FMT = {"mxfp4": 0, "fp8": 1, "nvfp4": 2}
MXS_F32, MXS_BF16, MXS_E4M3 = 0, 1, 2
PAGE_BYTES = {"mxfp4": 8704, "fp8": 16896, "nvfp4": 9728}

EXPORTS = [
    "mxfp4_row_store", "fp8_row_store", "nvfp4_row_store", "pack_q_e4m3", "index_score", "topk_blocks",
    "index_score_topk", "mxs_score_workspace_bytes", "sparse_split_attn", "mxs_default_partitions",
    "mxs_default_partitions_for",
    "lse_merge", "decode_step", "decode_step_reuse", "mxs_workspace_bytes", "mxs_status_str", "mxs_last_error",
    "mxs_abi_version", "mxs_read_index_pages", "decode_step_noalloc", "mxs_workspace_init",
    "decode_step_one_launch", "decode_step_reuse_one_launch",
]
NOALLOC_SCRATCH_BYTES = 8 << 20        # MXS_NOALLOC_SCRATCH_BYTES


class MxsError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"mxsparse status {status}: {msg}")
        self.status = status


class CacheStruct(ctypes.Structure):
    _fields_ = [
        ("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p), ("idx_pages", ctypes.c_void_p),
        ("num_pages", ctypes.c_int32), ("kv_format", ctypes.c_int32), ("idx_format", ctypes.c_int32),
        ("page_table", ctypes.c_void_p), ("page_table_stride", ctypes.c_int32),
        ("context_lens", ctypes.c_void_p),
    ]


class StepStruct(ctypes.Structure):
    _fields_ = [
        ("cache", CacheStruct),
        ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p), ("idx_new", ctypes.c_void_p),
        ("query", ctypes.c_void_p), ("q_dtype", ctypes.c_int32),
        ("q_idx", ctypes.c_void_p), ("w", ctypes.c_void_p),
        ("B", ctypes.c_int32), ("q", ctypes.c_int32), ("H", ctypes.c_int32), ("H_I", ctypes.c_int32),
        ("topk", ctypes.c_int32), ("num_partitions", ctypes.c_int32), ("sm_scale", ctypes.c_float),
        ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("block_table_out", ctypes.c_void_p),
        ("scores_out", ctypes.c_void_p),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_attention_decode_mxfp4_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
        sig = {
            "mxfp4_row_store": [P, I64, P, P, I32, P],
            "fp8_row_store": [P, I64, P, P, I32, P],
            "nvfp4_row_store": [P, I64, P, P, I32, P],
            "pack_q_e4m3": [P, I32, I64, P, P],
            "index_score": [P, P, P, I32, I32, I32, P, P],
            "topk_blocks": [P, P, I32, I32, I32, P, P],
            "index_score_topk": [P, P, P, I32, I32, I32, I32, P, P, P, SZ, P],
            "sparse_split_attn": [P, P, I32, P, I32, I32, I32, I32, I32, F32, P, P, P, P],
            "lse_merge": [P, P, P, I32, I32, P, P, P],
            "decode_step": [P, P, SZ, P],
            "decode_step_reuse": [P, P, P, SZ, P],
            "decode_step_reuse_one_launch": [P, P, P, SZ, P],
            "decode_step_noalloc": [P, P],
            "mxs_workspace_init": [P, SZ, P],
            "decode_step_one_launch": [P, P, SZ, P],
            "mxs_read_index_pages": [P, I32, P, P],
            "mxs_default_partitions": [I32, I32, I32],
            "mxs_default_partitions_for": [I32, I32, I32, I32],
            "mxs_score_workspace_bytes": [I32, I32, I32],
            "mxs_workspace_bytes": [I32, I32, I32, I32, I32, I32, I32],
            "mxs_status_str": [ctypes.c_int],
            "mxs_last_error": [],
            "mxs_abi_version": [],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.mxs_status_str.restype = ctypes.c_char_p
        L.mxs_last_error.restype = ctypes.c_char_p
        L.mxs_score_workspace_bytes.restype = SZ
        L.mxs_workspace_bytes.restype = SZ
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != MXS_OK:
        raise MxsError(status, lib().mxs_last_error().decode())


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, dtype, name: str, shape=None) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name}: expected a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _opt(t, dtype, name, shape=None) -> int:
    return 0 if t is None else _dev(t, dtype, name, shape)


class Cache:
    """A layer's paged caches (caller-owned GPU tensors) and the ctypes struct over them."""

    def __init__(self, k_pages, v_pages, idx_pages, page_table, context_lens, kv_format="mxfp4",
                 idx_format="mxfp4"):
        self.k_pages, self.v_pages, self.idx_pages = k_pages, v_pages, idx_pages
        self.page_table, self.context_lens = page_table, context_lens
        self.kv_format, self.idx_format = kv_format, idx_format
        if page_table.dim() != 2:
            raise ValueError("page_table: expected [B][stride]")
        self.B, self.stride = page_table.shape
        nps = []
        for name, t, fmt in (("k_pages", k_pages, kv_format), ("v_pages", v_pages, kv_format),
                             ("idx_pages", idx_pages, idx_format)):
            if t is None:
                continue
            _dev(t, torch.uint8, name)
            if t.numel() % PAGE_BYTES[fmt]:
                raise ValueError(f"{name}: size is not a multiple of the {fmt} page")
            nps.append(t.numel() // PAGE_BYTES[fmt])
        self.num_pages = min(nps) if nps else 1
        self.struct = CacheStruct(
            _opt(k_pages, torch.uint8, "k_pages"), _opt(v_pages, torch.uint8, "v_pages"),
            _opt(idx_pages, torch.uint8, "idx_pages"), self.num_pages, FMT[kv_format], FMT[idx_format],
            _dev(page_table, torch.int32, "page_table"), self.stride,
            _dev(context_lens, torch.int32, "context_lens", (self.B,)))

    def ref(self):
        return ctypes.byref(self.struct)

    def check_batch(self, B: int) -> None:
        """The kernels index page_table and context_lens by sequence: B must
        not exceed the rows given here (device memory the C ABI cannot size)."""
        if B > self.B:
            raise ValueError(f"batch of {B} sequences, but the cache has page-table rows for {self.B}")


# ----------------------------------------------------------------- stages
def mxfp4_row_store(rows, slots, pages):
    n = rows.shape[0]
    _check(lib().mxfp4_row_store(_dev(rows, torch.float32, "rows", (n, 128)), n,
                                 _dev(slots, torch.int64, "slots", (n,)), _dev(pages, torch.uint8, "pages"),
                                 pages.numel() // PAGE_BYTES["mxfp4"], _stream()))


def fp8_row_store(rows, slots, pages):
    n = rows.shape[0]
    _check(lib().fp8_row_store(_dev(rows, torch.float32, "rows", (n, 128)), n,
                               _dev(slots, torch.int64, "slots", (n,)), _dev(pages, torch.uint8, "pages"),
                               pages.numel() // PAGE_BYTES["fp8"], _stream()))


def nvfp4_row_store(rows, slots, pages):
    n = rows.shape[0]
    _check(lib().nvfp4_row_store(_dev(rows, torch.float32, "rows", (n, 128)), n,
                                 _dev(slots, torch.int64, "slots", (n,)), _dev(pages, torch.uint8, "pages"),
                                 pages.numel() // PAGE_BYTES["nvfp4"], _stream()))


def pack_q_e4m3(q, q8=None):
    if q.dtype == torch.float32:
        dt = MXS_F32
    elif q.dtype == torch.bfloat16:
        dt = MXS_BF16
    else:
        raise TypeError("q: fp32 or bf16")
    if q8 is None:
        q8 = torch.empty(q.shape, dtype=torch.uint8, device=q.device)
    _check(lib().pack_q_e4m3(_dev(q, q.dtype, "q"), dt, q.numel(), _dev(q8, torch.uint8, "q8", q.shape),
                             _stream()))
    return q8


def index_score(cache: Cache, q_idx, w, scores=None):
    B, q, H_I, _ = q_idx.shape
    cache.check_batch(B)
    if scores is None:
        scores = torch.empty((B, q, cache.stride), dtype=torch.float32, device=q_idx.device)
    _check(lib().index_score(cache.ref(), _dev(q_idx, torch.bfloat16, "q_idx", (B, q, H_I, 128)),
                             _dev(w, torch.float32, "w", (B, q, H_I)), B, q, H_I,
                             _dev(scores, torch.float32, "scores", (B, q, cache.stride)), _stream()))
    return scores


def read_index_pages(cache: Cache, B, sink=None):
    """Streaming read of every index page of sequences 0..B-1 (a measurement
    aid: the scan's bandwidth ceiling; computes nothing of the method)."""
    cache.check_batch(B)
    if sink is None:
        sink = torch.empty(1, dtype=torch.int32, device="cuda")
    _check(lib().mxs_read_index_pages(cache.ref(), B, _dev(sink, torch.int32, "sink"), _stream()))
    return sink


def topk_blocks(cache: Cache, scores, topk, block_table=None):
    B, q, _ = scores.shape
    cache.check_batch(B)
    if block_table is None:
        block_table = torch.empty((B, q, topk), dtype=torch.int32, device=scores.device)
    _check(lib().topk_blocks(cache.ref(), _dev(scores, torch.float32, "scores", (B, q, cache.stride)), B, q,
                             topk, _dev(block_table, torch.int32, "block_table", (B, q, topk)), _stream()))
    return block_table


def index_score_topk(cache: Cache, q_idx, w, topk, block_table=None, scores=None, ws=None):
    B, q, H_I, _ = q_idx.shape
    cache.check_batch(B)
    if block_table is None:
        block_table = torch.empty((B, q, topk), dtype=torch.int32, device=q_idx.device)
    if scores is None and ws is None:
        ws = torch.empty(lib().mxs_score_workspace_bytes(B, q, cache.stride), dtype=torch.uint8,
                         device=q_idx.device)
    _check(lib().index_score_topk(
        cache.ref(), _dev(q_idx, torch.bfloat16, "q_idx", (B, q, H_I, 128)),
        _dev(w, torch.float32, "w", (B, q, H_I)), B, q, H_I, topk,
        _dev(block_table, torch.int32, "block_table", (B, q, topk)),
        _opt(scores, torch.float32, "scores", (B, q, cache.stride)),
        _opt(ws, torch.uint8, "ws"), 0 if ws is None else ws.numel(), _stream()))
    return block_table


def default_partitions(B, q, topk, kv_format="mxfp4") -> int:
    return lib().mxs_default_partitions_for(B, q, topk, FMT[kv_format])


def sparse_split_attn(cache: Cache, q, block_table, sm_scale, num_partitions=0, out=None):
    """q: uint8 e4m3 codes (MXFP4 KV) or bf16 (FP8 KV), [B][q][H][128].
    Returns (sp_m [B][q][H][P], sp_l, sp_o [B][q][H][P][128])."""
    B, qr, H, _ = q.shape
    cache.check_batch(B)
    topk = block_table.shape[2]
    P = num_partitions or default_partitions(B, qr, topk, cache.kv_format)
    if out is None:
        dev = q.device
        out = (torch.empty((B, qr, H, P), dtype=torch.float32, device=dev),
               torch.empty((B, qr, H, P), dtype=torch.float32, device=dev),
               torch.empty((B, qr, H, P, 128), dtype=torch.float32, device=dev))
    sp_m, sp_l, sp_o = out
    if q.dtype == torch.uint8:
        qd = MXS_E4M3
    elif q.dtype == torch.bfloat16:
        qd = MXS_BF16
    else:
        raise TypeError("q: uint8 (e4m3 codes) or bfloat16")
    _check(lib().sparse_split_attn(
        cache.ref(), _dev(q, q.dtype, "q"), qd, _dev(block_table, torch.int32, "block_table", (B, qr, topk)),
        B, qr, H, topk, P, float(sm_scale), _dev(sp_m, torch.float32, "sp_m", (B, qr, H, P)),
        _dev(sp_l, torch.float32, "sp_l", (B, qr, H, P)), _dev(sp_o, torch.float32, "sp_o", (B, qr, H, P, 128)),
        _stream()))
    return sp_m, sp_l, sp_o


def lse_merge(sp_m, sp_l, sp_o, out=None, lse=None):
    """Partials [..][P], [..][P][128] -> (O bf16 [..][128], lse fp32 [..])."""
    lead = sp_m.shape[:-1]
    P = sp_m.shape[-1]
    n = 1
    for d in lead:
        n *= d
    if out is None:
        out = torch.empty((*lead, 128), dtype=torch.bfloat16, device=sp_m.device)
    if lse is None:
        lse = torch.empty(lead, dtype=torch.float32, device=sp_m.device)
    _check(lib().lse_merge(_dev(sp_m, torch.float32, "sp_m"), _dev(sp_l, torch.float32, "sp_l", sp_m.shape),
                           _dev(sp_o, torch.float32, "sp_o", (*sp_m.shape, 128)), n, P,
                           _dev(out, torch.bfloat16, "out", (*lead, 128)),
                           _opt(lse, torch.float32, "lse", lead), _stream()))
    return out, lse


def workspace_bytes(B, q, H, H_I, topk, stride, num_partitions=0) -> int:
    return lib().mxs_workspace_bytes(B, q, H, H_I, topk, stride, num_partitions)


def workspace_init(ws):
    """Zero-fill a step workspace (uint8 GPU tensor, 256-byte aligned) on the current stream."""
    _check(lib().mxs_workspace_init(_dev(ws, torch.uint8, "ws"), ws.numel(), _stream()))
    return ws


class DecodeStep:
    """decode_step over fixed tensors: builds the argument struct once, so that
    ``run()`` is a single C call (the launch chain), fit for timing and capture.

    With ``noalloc=True`` no workspace is taken or allocated and ``run()``
    calls decode_step_noalloc, whose workspace is the library's own device
    array (out and lse are still allocated here unless given). With
    ``one_launch=True`` ``run()`` calls decode_step_one_launch (the workspace
    allocated here starts zero-filled, as that entry point requires)."""

    def __init__(self, cache: Cache, query, q_idx, w, topk, sm_scale, k_new=None, v_new=None, idx_new=None,
                 num_partitions=0, out=None, lse=None, block_table_out=None, scores_out=None, ws=None,
                 noalloc=False, one_launch=False):
        B, q, H, _ = query.shape
        cache.check_batch(B)
        H_I = q_idx.shape[2]
        dev = query.device
        if query.dtype == torch.float32:
            qd = MXS_F32
        elif query.dtype == torch.bfloat16:
            qd = MXS_BF16
        else:
            raise TypeError("query: fp32 or bf16")
        self.out = out if out is not None else torch.empty((B, q, H, 128), dtype=torch.bfloat16, device=dev)
        self.lse = lse if lse is not None else torch.empty((B, q, H), dtype=torch.float32, device=dev)
        nb = workspace_bytes(B, q, H, H_I, topk, cache.stride, num_partitions)
        self.noalloc, self.one_launch = noalloc, one_launch
        if noalloc:
            self.ws = None
        else:
            self.ws = ws if ws is not None else torch.zeros(nb, dtype=torch.uint8, device=dev)
        self.cache = cache
        self._keep = (query, q_idx, w, k_new, v_new, idx_new, block_table_out, scores_out)
        self.block_table_out, self.scores_out = block_table_out, scores_out
        self.struct = StepStruct(
            cache.struct,
            _opt(k_new, torch.float32, "k_new", (B, q, 128)), _opt(v_new, torch.float32, "v_new", (B, q, 128)),
            _opt(idx_new, torch.float32, "idx_new", (B, q, 128)),
            _dev(query, query.dtype, "query"), qd,
            _dev(q_idx, torch.bfloat16, "q_idx", (B, q, H_I, 128)), _dev(w, torch.float32, "w", (B, q, H_I)),
            B, q, H, H_I, topk, num_partitions, float(sm_scale),
            _dev(self.out, torch.bfloat16, "out", (B, q, H, 128)), _opt(self.lse, torch.float32, "lse", (B, q, H)),
            _opt(block_table_out, torch.int32, "block_table_out", (B, q, topk)),
            _opt(scores_out, torch.float32, "scores_out", (B, q, cache.stride)))
        if not noalloc:
            if self.ws.numel() < nb:
                raise ValueError(f"ws: {self.ws.numel()} bytes, needs {nb}")
            self._ws_ptr = _dev(self.ws, torch.uint8, "ws")

    def run(self, stream=None):
        s = _stream() if stream is None else stream
        if self.noalloc:
            _check(lib().decode_step_noalloc(ctypes.byref(self.struct), s))
        elif self.one_launch:
            _check(lib().decode_step_one_launch(ctypes.byref(self.struct), self._ws_ptr, self.ws.numel(), s))
        else:
            _check(lib().decode_step(ctypes.byref(self.struct), self._ws_ptr, self.ws.numel(), s))
        return self.out


class DecodeStepReuse:
    """decode_step_reuse over fixed tensors: the step of a layer that reuses an
    earlier layer's block selection (``block_table`` [B][q][topk] int32). Stores
    the new K / V rows (both or neither), packs the query and attends over the
    given blocks; the index side is not touched. ``run()`` is a single C call.
    ``one_launch``: decode_step_reuse_one_launch (one grid; the workspace must
    be zero before its first use, which a workspace made here is)."""

    def __init__(self, cache: Cache, query, block_table, sm_scale, k_new=None, v_new=None, num_partitions=0,
                 out=None, lse=None, ws=None, one_launch=False):
        B, q, H, _ = query.shape
        cache.check_batch(B)
        topk = block_table.shape[-1]
        dev = query.device
        if query.dtype == torch.float32:
            qd = MXS_F32
        elif query.dtype == torch.bfloat16:
            qd = MXS_BF16
        else:
            raise TypeError("query: fp32 or bf16")
        self.out = out if out is not None else torch.empty((B, q, H, 128), dtype=torch.bfloat16, device=dev)
        self.lse = lse if lse is not None else torch.empty((B, q, H), dtype=torch.float32, device=dev)
        nb = workspace_bytes(B, q, H, 1, topk, cache.stride, num_partitions)
        self.ws = ws if ws is not None else torch.zeros(nb, dtype=torch.uint8, device=dev)
        if self.ws.numel() < nb:
            raise ValueError(f"ws: {self.ws.numel()} bytes, needs {nb}")
        self.cache = cache
        self._keep = (query, block_table, k_new, v_new)
        self._table = _dev(block_table, torch.int32, "block_table", (B, q, topk))
        self.struct = StepStruct(
            cache.struct,
            _opt(k_new, torch.float32, "k_new", (B, q, 128)), _opt(v_new, torch.float32, "v_new", (B, q, 128)),
            None, _dev(query, query.dtype, "query"), qd, None, None,
            B, q, H, 0, topk, num_partitions, float(sm_scale),
            _dev(self.out, torch.bfloat16, "out", (B, q, H, 128)), _opt(self.lse, torch.float32, "lse", (B, q, H)),
            None, None)
        self._ws_ptr = _dev(self.ws, torch.uint8, "ws")
        self._fn = "decode_step_reuse_one_launch" if one_launch else "decode_step_reuse"

    def run(self, stream=None):
        s = _stream() if stream is None else stream
        _check(getattr(lib(), self._fn)(ctypes.byref(self.struct), self._table, self._ws_ptr, self.ws.numel(), s))
        return self.out
