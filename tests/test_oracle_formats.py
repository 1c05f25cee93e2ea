"""Pins of the oracle's number formats and page layouts against closed forms,
library routines (torch's e8m0 and e4m3 dtypes) and brute force.

Sources: OCP Microscaling Formats (MX) v1.0 for e2m1 / e8m0 and the scale
rule; ATOM PR #2812 ("Mono decode over the MXFP4 KV and index caches") for the
8704-byte page and the saturating e4m3 q store.
"""
import math

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import formats as F
import workloads as W


# ---------------------------------------------------------------- page sizes
def test_page_sizes_closed_form():
    # 128 tokens x 128 elements x 4 bits + one e8m0 byte per 32 elements
    assert F.MXFP4_PAGE_BYTES == 128 * 128 // 2 + 128 * 128 // 32 == 8704
    # 128 x 128 e4m3 bytes + one fp32 scale per token
    assert F.FP8_PAGE_BYTES == 128 * 128 + 128 * 4 == 16896
    # 128 x 128 x 4 bits + one e4m3 byte per 16 elements + one fp32 scale per token
    assert F.NVFP4_PAGE_BYTES == 128 * 128 // 2 + 128 * 128 // 16 + 128 * 4 == 9728


# ---------------------------------------------------------------- e2m1
def test_e2m1_table_is_ocp_fp4():
    # OCP MX v1.0, FP4 E2M1: the 8 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(F.E2M1_TABLE[:8]) == mags
    assert list(F.E2M1_TABLE[8:]) == [-m for m in mags]
    assert math.copysign(1.0, F.E2M1_TABLE[8]) == -1.0


def test_e2m1_roundtrip_all_codes():
    vals = F.E2M1_TABLE.copy()
    vals[8] = -0.0
    assert list(F.e2m1_encode(vals)) == list(range(16))


def test_e2m1_midpoints_round_half_even():
    # every midpoint between neighbouring magnitudes goes to the code with mantissa bit 0
    mid = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    want = [0, 2, 2, 4, 4, 6, 6]            # 0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0
    assert list(F.e2m1_encode(np.array(mid))) == want
    assert list(F.e2m1_encode(-np.array(mid))) == [c | 8 for c in want]


def test_e2m1_saturation_and_sign():
    assert list(F.e2m1_encode(np.array([6.0, 6.5, 7.99, 1e30]))) == [7, 7, 7, 7]
    assert list(F.e2m1_encode(np.array([-7.0, -1e-30, -0.0]))) == [15, 8, 8]


def test_e2m1_nearest_brute_force():
    rng = np.random.default_rng(11)
    v = np.concatenate([rng.uniform(-7, 7, 4000), rng.standard_normal(1000) * 0.3])
    codes = F.e2m1_encode(v)
    for x, c in zip(v, codes):
        a = min(abs(x), 6.0)
        best = min(range(8), key=lambda k: (abs(a - F.E2M1_TABLE[k]), k & 1))
        assert (c & 7) == best and (c >> 3) == (1 if x < 0 or (x == 0 and math.copysign(1, x) < 0) else 0)


# ---------------------------------------------------------------- e8m0
def test_e8m0_matches_torch_all_bytes():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    got = F.e8m0_value(np.arange(256))
    assert np.isnan(ref[255]) and np.isnan(got[255])
    np.testing.assert_array_equal(got[:255], ref[:255])


def test_scale_byte_brackets_amax():
    rng = np.random.default_rng(3)
    amax = np.ldexp(rng.uniform(1, 2, 5000), rng.integers(-120, 120, 5000))
    b = F.mx_scale_byte(amax)
    # OCP: 2^(b - 127) is the largest power of two with amax / 2^(b-127) < 8,
    # i.e. 2^(b-127+2) <= amax < 2^(b-127+3)
    assert np.all(np.ldexp(1.0, b - 127 + 2) <= amax)
    assert np.all(amax < np.ldexp(1.0, b - 127 + 3))


def test_scale_byte_worked_values():
    assert F.mx_scale_byte(1.0) == 125           # 1 = 4 * 2^-2
    assert F.mx_scale_byte(6.0) == 127
    assert F.mx_scale_byte(7.9) == 127
    assert F.mx_scale_byte(8.0) == 128
    assert F.mx_scale_byte(0.0) == 0
    assert F.mx_scale_byte(1e-45) == 0           # fp32 subnormal: clamps to 2^-127
    assert F.mx_scale_byte(2.0 ** -125) == 0     # floor(log2) - 2 = -127 -> byte 0
    assert F.mx_scale_byte(2.0 ** -124) == 1
    for k in range(-100, 101, 7):
        assert F.mx_scale_byte(6.0 * 2.0 ** k) == 127 + k


# ---------------------------------------------------------------- MXFP4 rows
def test_quantize_worked_rows():
    x = np.zeros((1, 128), dtype=np.float32)
    x[0, :32] = 1.0                      # amax 1 -> byte 125 -> 1.0 / 0.25 = 4.0 -> code 6
    x[0, 32] = 6.0                       # amax 6 -> byte 127, 6 -> code 7, rest 0
    x[0, 64] = 7.9                       # amax 7.9 -> byte 127, 7.9 clips to 6 -> code 7
    x[0, 65] = -2.5                      # -2.5 at scale 1 -> tie -> -2.0 -> code 0xC
    codes, sb = F.mxfp4_quantize_rows(x)
    assert list(sb[0]) == [125, 127, 127, 0]
    assert list(codes[0, :32]) == [6] * 32
    assert codes[0, 32] == 7 and (codes[0, 33:64] == 0).all()
    assert codes[0, 64] == 7 and codes[0, 65] == 0xC
    assert (codes[0, 96:] == 0).all()    # all-zero group: byte 0, codes 0


def test_quantize_roundtrip_on_grid():
    """Rows already on an MX grid (each group holds a magnitude 4 or 6) survive
    quantize(dequantize(.)) exactly, codes and scale bytes alike."""
    rng = np.random.default_rng(5)
    N = 512
    codes = rng.integers(0, 16, size=(N, 128)).astype(np.uint8)
    for g in range(4):                               # force the group's amax code
        codes[:, 32 * g + rng.integers(0, 32)] = rng.choice([6, 7, 14, 15], size=N)
    sb = rng.integers(2, 250, size=(N, 4)).astype(np.uint8)
    x = F.mxfp4_dequantize(codes, sb).astype(np.float32)
    c2, s2 = F.mxfp4_quantize_rows(x)
    np.testing.assert_array_equal(s2, sb)
    np.testing.assert_array_equal(c2, codes)


@settings(max_examples=60, deadline=None)
@given(st.integers(0, 2**31 - 1))
def test_quantize_error_bound(seed):
    x = np.random.default_rng(seed).standard_normal((4, 128)).astype(np.float32) * 3
    codes, sb = F.mxfp4_quantize_rows(x)
    dq = F.mxfp4_dequantize(codes, sb).reshape(4, 4, 32)
    scale = np.ldexp(1.0, sb.astype(np.int64) - 127)[..., None]
    err = np.abs(dq - x.reshape(4, 4, 32)) / scale
    # gap between e2m1 neighbours is at most 2 (4 -> 6), values in (6, 8) clip: error < 2
    assert err.max() < 2.0
    # below 2 the grid step is 0.5: error at most 0.25 there
    small = np.abs(x.reshape(4, 4, 32)) / scale < 2.0
    assert (err[small] <= 0.25).all()


# ---------------------------------------------------------------- e4m3
def _torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_in_range_matches_torch():
    rng = np.random.default_rng(7)
    vals = F.E4M3_TABLE[:127]
    mids = (vals[:-1] + vals[1:]) / 2                      # every tie between neighbours
    x = np.concatenate([
        rng.standard_normal(20000) * 50, rng.standard_normal(5000) * 1e-2,
        rng.uniform(-448, 448, 20000), mids, -mids, vals, -vals,
        np.nextafter(mids.astype(np.float32), np.float32(0)),
        np.nextafter(mids.astype(np.float32), np.float32(1e9)),
    ]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    np.testing.assert_array_equal(F.e4m3_encode(x), _torch_e4m3(x))


def test_e4m3_saturates_and_keeps_nan():
    x = np.array([448.0, 449.0, 464.0, 500.0, 1e30, np.inf, -500.0, -np.inf, np.nan, -np.nan, -0.0],
                 dtype=np.float32)
    got = F.e4m3_encode(x)
    assert list(got[:6]) == [0x7E] * 6
    assert list(got[6:8]) == [0xFE] * 2
    assert got[8] in (0x7F, 0xFF) and got[9] in (0x7F, 0xFF)
    assert got[10] == 0x80
    assert np.isnan(F.E4M3_TABLE[0x7F]) and F.E4M3_TABLE[0x7E] == 448.0


def test_e4m3_clamp_negative_control():
    """Without the clamp the cast turns large values into NaN (torch does so
    above 464), and the saturation check above catches it."""
    x = np.array([500.0, np.inf], dtype=np.float32)
    assert list(_torch_e4m3(x)) != list(F.e4m3_encode(x))


# ---------------------------------------------------------------- FP8 rows (reading)
def test_fp8_rows_roundtrip_bound():
    x = np.random.default_rng(9).standard_normal((300, 128)).astype(np.float32)
    x[0] = 0.0
    codes, scale = F.fp8_quantize_rows(x)
    assert scale[0] == 1.0 and (codes[0] == 0).all()
    dq = F.E4M3_TABLE[codes.astype(np.int64)] * scale[:, None].astype(np.float64)
    # e4m3 keeps 3 mantissa bits: relative error <= 2^-4 for normals, absolute
    # <= 2^-10 * scale in the subnormal range
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * scale[:, None])
    assert (np.abs(dq - x) <= bound + 1e-30).all()
    # the largest element lands on +-448
    i = np.abs(x[1:]).argmax(axis=1)
    assert set(np.unique(codes[1:][np.arange(299), i] & 0x7F)) == {0x7E}


# ---------------------------------------------------------------- pages
@pytest.mark.parametrize("fmt", ["mxfp4", "fp8", "nvfp4"])
def test_store_read_and_poison(fmt):
    rng = np.random.default_rng(2)
    L = 300                                            # 3 pages, last one partly filled
    table = np.array([5, 1, 3], dtype=np.int32)
    pool = W.new_pool(7, F.PAGE_BYTES[fmt])
    x = rng.standard_normal((L, 128)).astype(np.float32)
    F.STORE[fmt](pool, table, 0, x[:200])
    F.STORE[fmt](pool, table, 200, x[200:])            # second write continues the sequence
    got = F.READ[fmt](pool, table, L)
    if fmt == "mxfp4":
        want = F.mxfp4_dequantize(*F.mxfp4_quantize_rows(x))
    elif fmt == "nvfp4":
        want = F.nvfp4_dequantize(*F.nvfp4_quantize_rows(x))
    else:
        c, s = F.fp8_quantize_rows(x)
        want = F.E4M3_TABLE[c.astype(np.int64)] * s[:, None].astype(np.float64)
    np.testing.assert_array_equal(got, want)
    pages = pool.reshape(7, -1)
    for p in (0, 2, 4, 6):                             # pages never written stay poisoned
        assert (pages[p] == 0xFF).all()
    # the unwritten tail of page 3 (tokens 44..127) still reads as NaN
    tail = F.READ[fmt](pool, np.array([5, 1, 3], dtype=np.int32), 384, np.arange(300, 384))
    assert np.isnan(tail).all()


def test_mxfp4_byte_layout():
    """Token t of a page: 64 data bytes at 64 t (element 2i low nibble), 4 scale
    bytes at 8192 + 4 t."""
    x = np.zeros((2, 128), dtype=np.float32)
    x[1, 0] = 0.5                 # group 0: amax 0.5 -> byte 124 (2^-3), 0.5 -> 4.0 -> code 6
    x[1, 1] = -0.5                # code 0xE
    x[1, 127] = 6.0               # group 3: byte 127, code 7 in the high nibble of byte 63
    pool = W.new_pool(1, F.MXFP4_PAGE_BYTES)
    F.mxfp4_store(pool, np.array([0], dtype=np.int32), 0, x)
    row1 = pool[64:128]
    assert row1[0] == 0xE6 and row1[63] == 0x70 and (row1[1:63] == 0).all()
    assert list(pool[8192 + 4:8192 + 8]) == [124, 0, 0, 127]
    assert list(pool[8192:8196]) == [0, 0, 0, 0]
    assert (pool[128:8192] == 0xFF).all() and (pool[8200:] == 0xFF).all()


def test_fp8_byte_layout():
    """Token t of an FP8 page: 128 e4m3 codes at 128 t, its fp32 scale (little
    endian) at 16384 + 4 t; worked bytes from a row with a known amax."""
    x = np.zeros((3, 128), dtype=np.float32)
    x[2, 0] = 448.0 * 4.0         # amax 1792 -> scale 4.0 (0x40800000); 1792 / 4 = 448 -> code 0x7E
    x[2, 5] = -1.0                # -1 / 4 = -0.25 = 2^-2 -> exponent field 5, mantissa 0 -> 0xA8
    x[2, 127] = 2.0               # 0.5 = 2^-1 -> exponent field 6 -> 0x30
    pool = W.new_pool(1, F.FP8_PAGE_BYTES)
    F.fp8_store(pool, np.array([0], dtype=np.int32), 1, x[1:])     # positions 1 and 2
    row2 = pool[256:384]
    assert row2[0] == 0x7E and row2[5] == 0xA8 and row2[127] == 0x30
    assert (np.delete(row2, [0, 5, 127]) == 0).all()
    assert (pool[128:256] == 0).all()                               # the all-zero row: codes 0
    assert list(pool[16384 + 8:16384 + 12]) == [0x00, 0x00, 0x80, 0x40]    # 4.0f, little endian
    assert list(pool[16384 + 4:16384 + 8]) == [0x00, 0x00, 0x80, 0x3F]     # 1.0f for the zero row
    assert (pool[:128] == 0xFF).all() and (pool[384:16384] == 0xFF).all()  # other slots untouched
    assert (pool[16384:16388] == 0xFF).all() and (pool[16396:] == 0xFF).all()
    # and the read path takes the same bytes back: code * scale
    got = F.fp8_read(pool, np.array([0], dtype=np.int32), 3, np.array([2]))
    assert got[0, 0] == 1792.0 and got[0, 5] == -1.0 and got[0, 127] == 2.0


def test_bf16_to_f64_matches_torch_all_patterns():
    """Every one of the 65536 bf16 bit patterns decodes as torch's
    bfloat16 -> float32 conversion does (NaNs compared as NaN)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    with np.errstate(invalid="ignore"):          # NaN payloads widen with a warning, not an error
        got = F.bf16_to_f64(bits)
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    np.testing.assert_array_equal(got[~nan], ref[~nan].astype(np.float64))
    assert (np.signbit(got[~nan]) == np.signbit(ref[~nan])).all()       # -0 keeps its sign


def test_page_table_permutation_invariance():
    """Relabelling physical pages (and moving their bytes) leaves every read bit-identical."""
    rng = np.random.default_rng(4)
    L = 1000
    table = rng.permutation(12)[:8].astype(np.int32)
    pool = W.new_pool(12, F.MXFP4_PAGE_BYTES)
    F.mxfp4_store(pool, table, 0, rng.standard_normal((L, 128)).astype(np.float32))
    perm = rng.permutation(12)
    pool2 = np.empty_like(pool).reshape(12, -1)
    pool2[perm] = pool.reshape(12, -1)
    a = F.mxfp4_read(pool, table, L)
    b = F.mxfp4_read(pool2.reshape(-1), perm[table].astype(np.int32), L)
    np.testing.assert_array_equal(a, b)


# ---------------------------------------------------------------- NVFP4 (reading)
# e2m1 elements in 16-element blocks with e4m3 block scales and a per-token fp32
# scale S = amax / 2688; c_b = e4m3(a_b / 6 S); code = e2m1(x / (e4m3(c_b) S)).
# Every expected byte below is worked out by hand from those rules.
def _nv_worked_row():
    x = np.zeros(128, dtype=np.float32)
    x[0], x[1], x[2] = 2688.0, -1344.0, 224.0     # block 0: a = 2688 -> 448 = 0x7E; 6, -3, 0.5 -> 7, 0xD, 1
    x[16], x[17], x[18] = 1.0, 1.5, -0.75         # block 1: a = 1.5 -> 0.25 = 0x28; 4, 6, -3 -> 6, 7, 0xD
    x[32], x[33], x[34], x[35] = 3.0, 0.125, 0.375, -1.25   # block 2: 0.5 = 0x30; 6, .25, .75, -2.5 -> 7, 0, 2, 0xC
    # block 3 (elements 48..63) all zero: scale code 0, codes 0
    x[64], x[65] = 6.375, -6.375                  # block 4: 6.375 / 6 = 1.0625, a tie -> 1.0 = 0x38; 6.375 saturates to 6
    x[80] = 1e-6                                  # block 5: 1e-6 / 6 below half of 2^-9 -> scale code 0, codes 0
    x[96], x[97] = 6 * 2.0 ** -8, 2.0 ** -9       # block 6: 2^-8 = subnormal 2 * 2^-9 -> 0x02; 6, 0.5 -> 7, 1
    x[112], x[113] = -96.0, 40.0                  # block 7: 16 = 2^4 -> 0x58; -6, 2.5 -> 0xF, 4
    codes = np.zeros(64, dtype=np.uint8)
    codes[0], codes[1] = 0xD7, 0x01
    codes[8], codes[9] = 0x76, 0x0D
    codes[16], codes[17] = 0x07, 0xC2
    codes[32] = 0xF7
    codes[48] = 0x17
    codes[56] = 0x4F
    return x, codes, [0x7E, 0x28, 0x30, 0x00, 0x38, 0x00, 0x02, 0x58]


def test_nvfp4_worked_bytes():
    """One page, three tokens: a zero row, the worked row (S = 1) and the worked
    row times 2^-20 (S = 2^-20 exactly, every quotient unchanged): codes at
    64 t, block scales at 8192 + 8 t, token scale at 9216 + 4 t."""
    x, codes, cb = _nv_worked_row()
    rows = np.stack([np.zeros(128, dtype=np.float32), x, x * np.float32(2.0 ** -20)])
    pool = W.new_pool(1, F.NVFP4_PAGE_BYTES)
    F.nvfp4_store(pool, np.array([0], dtype=np.int32), 1, rows)       # positions 1, 2, 3
    assert (pool[64:128] == 0).all() and (pool[8192 + 8:8192 + 16] == 0).all()
    assert list(pool[9216 + 4:9216 + 8]) == [0x00, 0x00, 0x80, 0x3F]            # 1.0f for the zero row
    for t, s_bytes in ((2, [0x00, 0x00, 0x80, 0x3F]), (3, [0x00, 0x00, 0x80, 0x35])):   # 1.0f, 2^-20
        np.testing.assert_array_equal(pool[64 * t:64 * t + 64], codes)
        assert list(pool[8192 + 8 * t:8192 + 8 * t + 8]) == cb
        assert list(pool[9216 + 4 * t:9216 + 4 * t + 4]) == s_bytes
    # untouched bytes stay poisoned
    assert (pool[:64] == 0xFF).all() and (pool[256:8192] == 0xFF).all()
    assert (pool[8192:8200] == 0xFF).all() and (pool[8224:9216] == 0xFF).all()
    assert (pool[9216:9220] == 0xFF).all() and (pool[9232:] == 0xFF).all()
    # the read path: e2m1 * e4m3 * S
    got = F.nvfp4_read(pool, np.array([0], dtype=np.int32), 4, np.array([2, 3]))
    want = np.zeros(128)
    want[[0, 1, 2]] = [2688.0, -1344.0, 224.0]
    want[[16, 17, 18]] = [1.0, 1.5, -0.75]
    want[[32, 33, 34, 35]] = [3.0, 0.0, 0.5, -1.0]           # 0.125 -> 0, 0.375 -> 1 * 0.5, -1.25 -> -2 * 0.5
    want[[64, 65]] = [6.0, -6.0]
    want[[96, 97]] = [6 * 2.0 ** -8, 2.0 ** -9]
    want[[112, 113]] = [-96.0, 32.0]
    np.testing.assert_array_equal(got[0], want)
    np.testing.assert_array_equal(got[1], want * 2.0 ** -20)


def _nv_brute(x):
    """The NVFP4 reading by exhaustive nearest-value search over every e4m3 and
    e2m1 code (ties to the even code, saturation at the largest value)."""
    x = np.asarray(x, dtype=np.float32)
    e4 = F.E4M3_TABLE[:127]
    e2 = F.E2M1_TABLE[:8]

    def nearest(table, v):
        v = min(v, table[-1])
        d = np.abs(table - v)
        best = np.flatnonzero(d == d.min())
        return int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])

    amax = np.float32(np.abs(x).max())
    S = np.float32(1.0) if amax == 0 else max(np.float32(amax / np.float32(2688.0)), np.float32(2.0 ** -149))
    codes = np.zeros(128, dtype=np.uint8)
    cb = np.zeros(8, dtype=np.uint8)
    for b in range(8):
        blk = x[16 * b:16 * b + 16]
        t = np.float32(np.float32(np.abs(blk).max()) / np.float32(np.float32(6.0) * S))
        cb[b] = nearest(e4, float(t))
        d = np.float32(np.float32(e4[cb[b]]) * S)
        for i, v in enumerate(blk):
            if d > 0:
                q = np.float32(v / d)
                codes[16 * b + i] = nearest(e2, abs(float(q))) | (8 if np.signbit(q) else 0)
    return codes, cb, S


def test_nvfp4_brute_force():
    rng = np.random.default_rng(13)
    rows = [rng.standard_normal(128) * 10.0 ** rng.uniform(-30, 30) for _ in range(40)]
    r = rng.standard_normal(128)
    r[rng.integers(0, 128, 4)] *= 20.0                      # outliers
    rows.append(r)
    r = rng.standard_normal(128)
    r[16:32] = 0.0                                           # a zero block
    r[48:64] *= 1e-7                                         # a block far below the row's scale
    rows.append(r)
    rows.append(np.full(128, -3.0))                          # a constant row
    with np.errstate(under="ignore"):
        rows.append(rng.standard_normal(128) * 1e-41)            # subnormal fp32: S clamps at 2^-149
    x = np.stack(rows).astype(np.float32)
    codes, cb, S = F.nvfp4_quantize_rows(x)
    for n in range(x.shape[0]):
        bc, bcb, bS = _nv_brute(x[n])
        assert S[n] == bS, n
        np.testing.assert_array_equal(cb[n], bcb, err_msg=f"row {n}")
        np.testing.assert_array_equal(codes[n], bc, err_msg=f"row {n}")


def test_nvfp4_roundtrip_on_grid():
    """Rows built from representable values (each block holding +-6 times its
    scale, token scale a power of two) come back exactly."""
    rng = np.random.default_rng(17)
    N = 200
    c = rng.integers(0, 16, (N, 8, 16))
    c[:, :, 0] = 7 | (rng.integers(0, 2, (N, 8)) << 3)      # +-6 in every block
    cb = rng.integers(1, 127, (N, 8))                        # any finite non-zero e4m3
    cb[:, 0] = 0x7E                                          # block 0 holds the row's amax (6 * 448)
    S = 2.0 ** rng.integers(-40, 40, N)
    x = (F.E2M1_TABLE[c] * F.E4M3_TABLE[cb][:, :, None] * S[:, None, None]).reshape(N, 128).astype(np.float32)
    with np.errstate(under="ignore"):
        codes, gcb, gS = F.nvfp4_quantize_rows(x)
    np.testing.assert_array_equal(gS, S.astype(np.float32))
    np.testing.assert_array_equal(gcb, cb)
    np.testing.assert_array_equal(F.nvfp4_dequantize(codes, gcb, gS), x.astype(np.float64))


@settings(max_examples=40, deadline=None)
@given(st.integers(0, 2**31 - 1))
def test_nvfp4_error_bound(seed):
    """|x - x^| <= (9/8) a_b / 6 + 2^-10 * 6 S per block: the e2m1 step is at
    most 2 (half-step 1) in units of d_b ~ a_b / 6, the e4m3 rounding of the
    block scale (3 mantissa bits) moves d_b by at most 1/16 relative, and a
    block whose scale rounds below e4m3's range is stored as zeros."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((64, 128)) * 10.0 ** rng.uniform(-6, 6, (64, 1))).astype(np.float32)
    x[rng.random((64, 128)) < 0.01] *= 20.0
    codes, cb, S = F.nvfp4_quantize_rows(x)
    dq = F.nvfp4_dequantize(codes, cb, S).reshape(64, 8, 16)
    ab = np.abs(x).reshape(64, 8, 16).max(axis=2).astype(np.float64)
    bound = 1.125 * ab / 6.0 + 2.0 ** -10 * 6.0 * S[:, None].astype(np.float64)
    err = np.abs(dq - x.reshape(64, 8, 16)).max(axis=2)
    assert (err <= bound * (1 + 1e-6)).all()
    # the element holding the row's amax decodes to +-6 * 448 * S
    i = np.abs(x).argmax(axis=1)
    np.testing.assert_array_equal(np.abs(dq.reshape(64, 128)[np.arange(64), i]), 2688.0 * S.astype(np.float64))
