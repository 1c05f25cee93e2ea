"""The C ABI without a GPU: the library loads, exports every function that
include/mxsparse.h declares, and rejects bad arguments on the host before
anything is launched (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import sparse_attention_decode_mxfp4_amd as mx

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mxsparse.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mx.LIB_PATH):
        pytest.skip("library not built (python -m sparse_attention_decode_mxfp4_amd.build)")
    return mx.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_stages():
    names = declared_functions()
    for f in ["mxfp4_row_store", "fp8_row_store", "nvfp4_row_store", "pack_q_e4m3", "index_score", "topk_blocks",
              "index_score_topk", "sparse_split_attn", "lse_merge", "decode_step", "decode_step_reuse",
              "mxs_workspace_bytes",
              "mxs_default_partitions", "mxs_default_partitions_for", "mxs_status_str", "mxs_last_error",
              "mxs_abi_version",
              "mxs_score_workspace_bytes", "decode_step_noalloc", "decode_step_reuse_one_launch"]:
        assert f in names, f
    assert set(names) == set(mx.EXPORTS)


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_version_and_status_strings(L):
    assert L.mxs_abi_version() == 1
    assert L.mxs_status_str(0) == b"ok"
    assert L.mxs_status_str(2) == b"unsupported configuration"
    assert L.mxs_status_str(99) == b"unknown status"


def test_workspace_sizes(L):
    assert L.mxs_default_partitions(4, 8, 32) == 8          # ceil(32 / 4) x 32 rows = 256 workgroups
    assert L.mxs_default_partitions(1, 1, 1000) == 64
    # once the rows alone fill the GPU's 256 CUs, fewer (longer) partitions
    assert L.mxs_default_partitions(16, 8, 32) == 2
    assert L.mxs_default_partitions(32, 8, 32) == 1
    assert L.mxs_default_partitions(64, 16, 64) == 1
    # ceil(topk / 4) leaves CUs without a workgroup: two blocks per workgroup, ceil(topk / 2), same cap
    assert L.mxs_default_partitions(1, 1, 4) == 2
    assert L.mxs_default_partitions(4, 4, 16) == 8           # 16 rows: 4 -> 8 (cap 16)
    assert L.mxs_default_partitions(4, 8, 16) == 8           # 32 rows: 4 -> 8 (cap 8)
    assert L.mxs_default_partitions(4, 8, 20) == 8           # ceil(20 / 2) = 10, capped at 8
    assert L.mxs_default_partitions(8, 8, 16) == 4           # 64 rows: 4 x 64 = 256 already
    # the same rule for every format
    assert [L.mxs_default_partitions_for(4, 4, 16, f) for f in (0, 1, 2, 7)] == [8, 8, 8, 8]
    assert [L.mxs_default_partitions_for(32, 8, 32, f) for f in (0, 1, 2)] == [1, 1, 1]
    # with num_partitions = 0 the workspace fits the default (the FP8 workload: P = 8)
    rows = 16
    need8 = rows * 128 * 4 + rows * 16 * 4 + rows * 16 * 128 + 2 * rows * 128 * 4 + rows * 16 * 8 * 128 * 4
    assert L.mxs_workspace_bytes(4, 4, 16, 4, 16, 128, 0) >= need8
    ws = L.mxs_workspace_bytes(4, 8, 16, 4, 32, 2048, 0)
    rows, P = 32, 8
    need = rows * 2048 * 4 + rows * 32 * 4 + rows * 16 * 128 + 2 * rows * 16 * P * 4 + rows * 16 * P * 128 * 4
    assert need <= ws <= need + 6 * 256
    assert L.mxs_score_workspace_bytes(4, 8, 2048) == 4 * 8 * 2048 * 4


def _err(L):
    return L.mxs_last_error().decode()


def test_row_store_rejects_before_launch(L):
    assert L.mxfp4_row_store(None, -1, None, None, 1, None) == mx.MXS_EINVAL
    assert "n = -1" in _err(L)
    assert L.mxfp4_row_store(None, 4, None, ctypes.c_void_p(256), 1, None) == mx.MXS_EINVAL
    assert "rows" in _err(L)
    assert L.fp8_row_store(ctypes.c_void_p(256), 4, ctypes.c_void_p(256), ctypes.c_void_p(3), 1, None) == mx.MXS_EINVAL
    assert "16-byte" in _err(L)
    assert L.nvfp4_row_store(ctypes.c_void_p(256), 4, ctypes.c_void_p(260), ctypes.c_void_p(256), 1, None) == \
        mx.MXS_EINVAL
    assert "nvfp4_row_store" in _err(L) and "slots" in _err(L)


def test_pack_q_rejects_dtype(L):
    assert L.pack_q_e4m3(ctypes.c_void_p(256), 2, 16, ctypes.c_void_p(256), None) == mx.MXS_EUNSUPPORTED


def _cache(**kw):
    c = dict(k_pages=256, v_pages=512, idx_pages=768, num_pages=4, kv_format=0, idx_format=0, page_table=1024,
             page_table_stride=16, context_lens=2048)
    c.update(kw)
    return mx.CacheStruct(**c)


def test_refusal_matrix(L):
    P = ctypes.byref
    good_q, good_w = ctypes.c_void_p(4096), ctypes.c_void_p(8192)
    # format ids other than MXFP4 = 0, FP8 = 1 and NVFP4 = 2 are refused, naming the accepted ones
    for bad in (3, -1):
        c = _cache(idx_format=bad)
        assert L.index_score(P(c), good_q, good_w, 1, 1, 4, ctypes.c_void_p(256), None) == mx.MXS_EUNSUPPORTED
        assert "NVFP4 = 2" in _err(L)
    c = _cache()
    assert L.index_score(P(c), good_q, good_w, 1, 1, 5, ctypes.c_void_p(256), None) == mx.MXS_EUNSUPPORTED
    assert L.index_score(P(c), good_q, good_w, 1, 17, 4, ctypes.c_void_p(256), None) == mx.MXS_EUNSUPPORTED
    assert L.index_score(P(_cache(page_table_stride=9000)), good_q, good_w, 1, 1, 4, ctypes.c_void_p(256),
                         None) == mx.MXS_EUNSUPPORTED
    assert L.topk_blocks(P(c), ctypes.c_void_p(256), 1, 1, 65, ctypes.c_void_p(256), None) == mx.MXS_EUNSUPPORTED
    assert L.topk_blocks(P(c), ctypes.c_void_p(256), 1, 1, 0, ctypes.c_void_p(256), None) == mx.MXS_EINVAL
    # attention: head count, partition count, query dtype against the KV format
    args = lambda c, qd, H, P_: (P(c), good_q, qd, ctypes.c_void_p(256), 1, 1, H, 4, P_, ctypes.c_float(0.1),
                                 ctypes.c_void_p(256), ctypes.c_void_p(512), ctypes.c_void_p(1024), None)
    assert L.sparse_split_attn(*args(c, mx.MXS_E4M3, 17, 1)) == mx.MXS_EUNSUPPORTED
    assert L.sparse_split_attn(*args(c, mx.MXS_E4M3, 16, 65)) == mx.MXS_EUNSUPPORTED
    assert L.sparse_split_attn(*args(c, mx.MXS_BF16, 16, 1)) == mx.MXS_EUNSUPPORTED
    assert L.sparse_split_attn(*args(_cache(kv_format=3), mx.MXS_BF16, 16, 1)) == mx.MXS_EUNSUPPORTED
    assert "kv_format" in _err(L)
    # FP8 and NVFP4 K/V take a bf16 query, not e4m3 codes
    for f in (1, 2):
        assert L.sparse_split_attn(*args(_cache(kv_format=f), mx.MXS_E4M3, 16, 1)) == mx.MXS_EUNSUPPORTED
        assert "bf16 query" in _err(L)
    assert L.sparse_split_attn(*args(_cache(k_pages=0), mx.MXS_E4M3, 16, 1)) == mx.MXS_EINVAL
    assert L.lse_merge(ctypes.c_void_p(256), ctypes.c_void_p(256), ctypes.c_void_p(256), 1, 65,
                       ctypes.c_void_p(256), None, None) == mx.MXS_EUNSUPPORTED


def test_decode_step_workspace_check(L):
    s = mx.StepStruct(_cache(), 0, 0, 0, 4096, mx.MXS_F32, 8192, 12288, 2, 8, 16, 4, 32, 0, 0.1, 16384, 0, 0, 0)
    # the exact need of this MXFP4 step (P = 0 sizes for the larger, FP8, default)
    need = L.mxs_workspace_bytes(2, 8, 16, 4, 32, 16, L.mxs_default_partitions(2, 8, 32))
    assert L.mxs_workspace_bytes(2, 8, 16, 4, 32, 16, 0) >= need
    assert L.decode_step(ctypes.byref(s), ctypes.c_void_p(1 << 20), need - 1, None) == mx.MXS_EWORKSPACE
    assert L.decode_step(ctypes.byref(s), None, 0, None) == mx.MXS_EWORKSPACE
    assert L.decode_step(ctypes.byref(s), ctypes.c_void_p((1 << 20) + 16), need, None) == mx.MXS_EINVAL
    s.k_new = 4096                    # only one of the three new-row arrays
    assert L.decode_step(ctypes.byref(s), ctypes.c_void_p(1 << 20), need, None) == mx.MXS_EINVAL
    s.k_new = 0
    s.q_dtype = mx.MXS_E4M3           # an MXFP4 step takes fp32 / bf16 and stores e4m3 itself
    assert L.decode_step(ctypes.byref(s), ctypes.c_void_p(1 << 20), need, None) == mx.MXS_EUNSUPPORTED
    s.q_dtype = mx.MXS_F32
    s.B = 0                           # an empty batch does nothing and succeeds
    assert L.decode_step(ctypes.byref(s), None, 0, None) == mx.MXS_OK


def test_decode_step_reuse_rejects_before_launch(L):
    P = ctypes.byref
    s = mx.StepStruct(_cache(idx_pages=0), 0, 0, 0, 4096, mx.MXS_F32, 0, 0, 2, 8, 16, 0, 32, 0, 0.1, 16384, 0, 0, 0)
    need = L.mxs_workspace_bytes(2, 8, 16, 1, 32, 16, L.mxs_default_partitions(2, 8, 32))
    ws, table = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 16)
    assert L.decode_step_reuse(P(s), None, ws, need, None) == mx.MXS_EINVAL
    assert "block_table" in _err(L)
    assert L.decode_step_reuse(P(s), table, ws, need - 1, None) == mx.MXS_EWORKSPACE
    assert L.decode_step_reuse(P(s), ctypes.c_void_p((1 << 16) + 2), ws, need, None) == mx.MXS_EINVAL
    s.k_new = 4096                    # K rows without V rows
    assert L.decode_step_reuse(P(s), table, ws, need, None) == mx.MXS_EINVAL
    assert "both or neither" in _err(L)
    s.k_new = 0
    s.topk = 65
    assert L.decode_step_reuse(P(s), table, ws, need, None) == mx.MXS_EUNSUPPORTED
    s.topk = 32
    s.q_dtype = mx.MXS_E4M3
    assert L.decode_step_reuse(P(s), table, ws, need, None) == mx.MXS_EUNSUPPORTED
    s.q_dtype = mx.MXS_F32
    s.B = 0                           # an empty batch does nothing and succeeds
    assert L.decode_step_reuse(P(s), table, None, 0, None) == mx.MXS_OK


def test_decode_step_reuse_one_launch_rejects_like_the_two_launch_step(L):
    """The one-launch reuse step shares the two-launch step's argument checks
    (and names itself in the messages)."""
    P = ctypes.byref
    s = mx.StepStruct(_cache(idx_pages=0), 0, 0, 0, 4096, mx.MXS_F32, 0, 0, 2, 8, 16, 0, 32, 0, 0.1, 16384, 0, 0, 0)
    need = L.mxs_workspace_bytes(2, 8, 16, 1, 32, 16, L.mxs_default_partitions(2, 8, 32))
    ws, table = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 16)
    assert L.decode_step_reuse_one_launch(P(s), None, ws, need, None) == mx.MXS_EINVAL
    assert L.decode_step_reuse_one_launch(P(s), table, ws, need - 1, None) == mx.MXS_EWORKSPACE
    assert "decode_step_reuse_one_launch" in _err(L)
    s.k_new = 4096
    assert L.decode_step_reuse_one_launch(P(s), table, ws, need, None) == mx.MXS_EINVAL
    s.k_new = 0
    s.q_dtype = mx.MXS_E4M3
    assert L.decode_step_reuse_one_launch(P(s), table, ws, need, None) == mx.MXS_EUNSUPPORTED
    s.q_dtype = mx.MXS_F32
    s.B = 0
    assert L.decode_step_reuse_one_launch(P(s), table, None, 0, None) == mx.MXS_OK


def test_read_index_pages_rejects_before_launch(L):
    P = ctypes.byref
    sink = ctypes.c_void_p(256)
    assert L.mxs_read_index_pages(P(_cache()), 1, None, None) == mx.MXS_EINVAL
    assert L.mxs_read_index_pages(P(_cache()), 1, ctypes.c_void_p(258), None) == mx.MXS_EINVAL
    assert L.mxs_read_index_pages(P(_cache()), -1, sink, None) == mx.MXS_EINVAL
    assert L.mxs_read_index_pages(P(_cache(idx_pages=0)), 1, sink, None) == mx.MXS_EINVAL
    assert L.mxs_read_index_pages(P(_cache(idx_format=3)), 1, sink, None) == mx.MXS_EUNSUPPORTED
    assert L.mxs_read_index_pages(P(_cache()), 0, sink, None) == mx.MXS_OK    # nothing to read


def test_noalloc_refuses_steps_beyond_its_scratch(L):
    """decode_step_noalloc refuses, before touching any device, a step whose
    workspace would exceed the library's array (MXS_NOALLOC_SCRATCH_BYTES)."""
    text = open(HEADER).read()
    assert "#define MXS_NOALLOC_SCRATCH_BYTES (8u << 20)" in text
    assert mx.NOALLOC_SCRATCH_BYTES == 8 << 20
    assert L.decode_step_noalloc(None, None) == mx.MXS_EINVAL
    # 64 sequences x 8 rows over 8192-page tables: 16 MiB of scores alone
    st = mx.StepStruct()
    st.cache.page_table_stride = 8192
    st.B, st.q, st.H, st.H_I, st.topk = 64, 8, 16, 4, 32
    need = L.mxs_workspace_bytes(64, 8, 16, 4, 32, 8192, 0)
    assert need > mx.NOALLOC_SCRATCH_BYTES
    assert L.decode_step_noalloc(ctypes.byref(st), None) == mx.MXS_EWORKSPACE
    assert "scratch" in _err(L) and str(need) in _err(L)
