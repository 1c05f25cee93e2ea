"""Number formats and cache page layouts (oracle; test infrastructure only).

MXFP4 (ATOM PR #2812, "Mono decode over the MXFP4 KV and index caches", the
commit messages of the MXFP4 index-cache commit and of the MXFP4 main-KV commit):
a page holds 128 tokens of head_dim 128 as 4-bit e2m1 elements in 32-element
groups, each group with one e8m0 (power-of-two) scale, 8704 bytes in all, and
one layout serves the index keys, K and V. The pages name the quantizer
(``mxfp4ScaleE8m0``) without defining it; the reading taken here is the OCP
MX v1.0 quantizer, whose scale is 2^(floor(log2 amax) - 2), where 2 is e2m1's
largest exponent.

FP8 (ATOM PR #2686, "Enable Mono decode with fixed DSpark verify", Summary:
an FP8 K/V and index cache in 128-token blocks; vLLM PR #60528, Details): e4m3 elements with
a per-token fp32 scale. Reading (parity unpinned, the pages give no rule):
scale = fp32(amax / 448), 1.0 for an all-zero row, code = e4m3(fp32(x / scale)).

NVFP4 (ATOM PR #2686, timeline entry #2744, "FP4 index cache and NVFP4 sparse
KV cache"; ATOM PR #2812, commit messages of the MXFP4 index-cache and main-KV
commits, where NVFP4 K/V and index caches are named and refused). The pages
name the format without defining it. Reading (parity unpinned against the
pages' own writer, which is not available): the public NVFP4 description of
e2m1 elements in 16-element blocks, each block scaled by an e4m3 factor, under
a second-level fp32 scale. Here that second level is one per token, kept in the page
(as the FP8 cache keeps its per-token scale), so that a row can be written
alone. Quantizer, every step an IEEE fp32 operation:
  amax = max |x|;  S = 1 if amax == 0, else max(amax / 2688, 2^-149)
  (2688 = 6 * 448: the largest e2m1 value times the largest e4m3 value);
  block b: c_b = e4m3(a_b / (6 S)), a_b its largest magnitude;
  d_b = e4m3_value(c_b) * S;  element code = e2m1(x / d_b), 0 when d_b == 0.
Decoded value: e2m1_value(code) * e4m3_value(c_b) * S (exact in float64).

e4m3 q store (ATOM PR #2812, commit message of the e4m3 q store, and the one
that factors out ``pack_q_e4m3``): unit scale, round to nearest even, values
beyond +-448 and +-inf saturate to +-448, NaN stays NaN.

Page layouts (a reading; the pages only say that the scorer reads a tile with
one 16-byte load of key codes plus one dword holding its e8m0 scales, which
this layout allows). Parity unpinned against the
pages' own writer, which is not available; oracle and library agree on it.

  MXFP4 page (8704 B): token t's 128 codes at [64 t, 64 t + 64), element 2i in
  the low nibble and 2i+1 in the high nibble of byte i; token t's four group
  scales (groups of elements 0-31, 32-63, 64-95, 96-127) at 8192 + 4 t + g.

  FP8 page (16896 B): token t's 128 e4m3 codes at [128 t, 128 t + 128); token
  t's fp32 scale (little endian) at 16384 + 4 t.

  NVFP4 page (9728 B): token t's codes at [64 t, 64 t + 64) as in the MXFP4
  page; token t's eight e4m3 block scales (elements 16 b .. 16 b + 15) at
  8192 + 8 t + b; token t's fp32 scale (little endian) at 9216 + 4 t.
"""
from __future__ import annotations

import math

import numpy as np

TOKENS = 128
DIM = 128
GROUP = 32

MXFP4_PAGE_BYTES = TOKENS * DIM // 2 + TOKENS * (DIM // GROUP)   # 8192 + 512
MXFP4_SCALE_OFFSET = TOKENS * DIM // 2
FP8_PAGE_BYTES = TOKENS * DIM + TOKENS * 4                        # 16384 + 512
FP8_SCALE_OFFSET = TOKENS * DIM
NV_BLOCK = 16
NVFP4_PAGE_BYTES = TOKENS * DIM // 2 + TOKENS * (DIM // NV_BLOCK) + TOKENS * 4   # 8192 + 1024 + 512
NVFP4_BSCALE_OFFSET = TOKENS * DIM // 2
NVFP4_TSCALE_OFFSET = NVFP4_BSCALE_OFFSET + TOKENS * (DIM // NV_BLOCK)


# --------------------------------------------------------------------------
# e2m1 (OCP MX v1.0, FP4 E2M1): 1 sign, 2 exponent (bias 1), 1 mantissa bit.
# --------------------------------------------------------------------------
def e2m1_value(code: int) -> float:
    """Value of one 4-bit e2m1 code, from its bit fields."""
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return -mag if s else mag


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
_E2M1_MAGS = E2M1_TABLE[:8]                      # codes 0..7, ascending magnitudes


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """Round already-scaled values to e2m1 codes.

    Nearest representable magnitude; on an exact tie the code with mantissa bit
    0 (round half to even); magnitudes above 6 saturate to 6 (OCP MX clamps to
    the largest normal); the sign bit is kept, so a negative value that rounds
    to zero gives code 8 (-0). Inputs are finite (finite rows are the
    contract)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), 6.0)
    hi = np.clip(np.searchsorted(_E2M1_MAGS, a, side="left"), 0, 7)     # first magnitude >= a
    lo = np.clip(hi - 1, 0, 7)
    d_lo = a - _E2M1_MAGS[lo]
    d_hi = _E2M1_MAGS[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))          # tie: even code
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    return code | (np.signbit(v).astype(np.uint8) << 3)


# --------------------------------------------------------------------------
# e8m0 (OCP MX v1.0 shared scale): 2^(byte - 127), byte 255 is NaN.
# --------------------------------------------------------------------------
def e8m0_value(byte) -> np.ndarray:
    b = np.asarray(byte, dtype=np.int64)
    out = np.ldexp(1.0, b - 127).astype(np.float64)
    return np.where(b == 255, np.nan, out)


def mx_scale_byte(amax) -> np.ndarray:
    """e8m0 bytes of groups whose largest magnitudes are ``amax`` (OCP MX v1.0):
    shared exponent floor(log2 amax) - 2, clamped to the e8m0 range; an
    all-zero group takes the smallest scale (byte 0)."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)              # amax = f * 2^e, f in [0.5, 1)
    floor_log2 = e.astype(np.int64) - 1
    byte = np.clip(floor_log2 - 2 + 127, 0, 254)
    return np.where(amax == 0.0, 0, byte).astype(np.int64)


def mxfp4_quantize_rows(x: np.ndarray):
    """Quantize fp32 rows [N][128] to (codes uint8 [N][128], scale bytes uint8 [N][4]).

    Per 32-element group: the e8m0 byte from the group's amax, then every
    element divided by that power of two and rounded to e2m1."""
    x = np.asarray(x, dtype=np.float32)
    N = x.shape[0]
    codes = np.empty((N, DIM), dtype=np.uint8)
    sbytes = np.empty((N, DIM // GROUP), dtype=np.uint8)
    for c0 in range(0, N, 8192):                   # chunks only bound the temporaries
        g = x[c0:c0 + 8192].astype(np.float64).reshape(-1, DIM // GROUP, GROUP)
        sb = mx_scale_byte(np.abs(g).max(axis=-1))
        scale = np.ldexp(1.0, sb - 127)
        codes[c0:c0 + 8192] = e2m1_encode(g / scale[..., None]).reshape(-1, DIM)
        sbytes[c0:c0 + 8192] = sb
    return codes, sbytes


def mxfp4_dequantize(codes: np.ndarray, sbytes: np.ndarray) -> np.ndarray:
    """Table dequantization: e2m1 value times its group's 2^(byte - 127)."""
    vals = E2M1_TABLE[codes.astype(np.int64)]
    N = codes.shape[0]
    sc = e8m0_value(sbytes).reshape(N, DIM // GROUP, 1)
    return (vals.reshape(N, DIM // GROUP, GROUP) * sc).reshape(N, DIM)


# --------------------------------------------------------------------------
# e4m3 (OCP FP8 E4M3FN): bias 7, no infinities, 0x7F / 0xFF are NaN, max 448.
# --------------------------------------------------------------------------
def e4m3_value(code: int) -> float:
    s = (code >> 7) & 1
    e = (code >> 3) & 15
    m = code & 7
    if e == 15 and m == 7:
        return math.nan
    mag = m * 2.0 ** -9 if e == 0 else 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return -mag if s else mag


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
_E4M3_MAGS = E4M3_TABLE[:127]          # codes 0..126: every finite non-negative value, ascending


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Saturating e4m3 codes of fp32/float64 values: nearest finite value, ties to
    the even code, |x| > 448 and +-inf to +-448, NaN to 0x7F with the sign kept."""
    x = np.asarray(x, dtype=np.float64)
    nan = np.isnan(x)
    a = np.minimum(np.abs(np.where(nan, 0.0, x)), 448.0)
    hi = np.clip(np.searchsorted(_E4M3_MAGS, a, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo = a - _E4M3_MAGS[lo]
    d_hi = _E4M3_MAGS[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F), code)
    return code | (np.signbit(x).astype(np.uint8) << 7)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns to float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def fp8_quantize_rows(x: np.ndarray):
    """FP8 per-token quantization (reading; parity unpinned): returns
    (codes uint8 [N][128], scales fp32 [N])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=1)
    scale = np.where(amax == 0, np.float32(1.0), amax / np.float32(448.0)).astype(np.float32)
    v = (x / scale[:, None]).astype(np.float32)                  # IEEE fp32 division
    return e4m3_encode(v), scale


# --------------------------------------------------------------------------
# NVFP4 (reading, see the module docstring): e2m1 in 16-element blocks, e4m3
# block scales, a per-token fp32 scale.
# --------------------------------------------------------------------------
_F32_TINY = np.float32(2.0 ** -149)        # the smallest positive fp32 (a subnormal)


def nvfp4_quantize_rows(x: np.ndarray):
    """Quantize fp32 rows [N][128] to (codes uint8 [N][128], block scale codes
    uint8 [N][8], token scales fp32 [N]); each step in fp32 as the reading
    states (numpy's float32 operations round as IEEE fp32 does)."""
    x = np.asarray(x, dtype=np.float32)
    N = x.shape[0]
    a = np.abs(x)
    amax = a.max(axis=1)
    with np.errstate(divide="ignore", invalid="ignore", under="ignore"):
        S = np.where(amax == 0, np.float32(1.0),
                     np.maximum(amax / np.float32(2688.0), _F32_TINY)).astype(np.float32)
        ab = a.reshape(N, DIM // NV_BLOCK, NV_BLOCK).max(axis=2)                    # [N][8]
        six_s = (np.float32(6.0) * S).astype(np.float32)
        cb = e4m3_encode((ab / six_s[:, None]).astype(np.float32))                  # block scale codes
        d = (E4M3_TABLE[cb.astype(np.int64)].astype(np.float32) * S[:, None]).astype(np.float32)
        xb = x.reshape(N, DIM // NV_BLOCK, NV_BLOCK)
        v = (xb / d[:, :, None]).astype(np.float32)
    codes = np.where(d[:, :, None] > 0, e2m1_encode(np.where(d[:, :, None] > 0, v, 0.0)), 0).astype(np.uint8)
    return codes.reshape(N, DIM), cb.astype(np.uint8), S


def nvfp4_dequantize(codes: np.ndarray, cb: np.ndarray, S: np.ndarray) -> np.ndarray:
    """e2m1 value times its block's e4m3 value times the token scale, in float64."""
    N = codes.shape[0]
    vals = E2M1_TABLE[codes.astype(np.int64)].reshape(N, DIM // NV_BLOCK, NV_BLOCK)
    sc = E4M3_TABLE[cb.astype(np.int64)] * np.asarray(S, dtype=np.float64)[:, None]
    return (vals * sc[:, :, None]).reshape(N, DIM)


# --------------------------------------------------------------------------
# Page stores and reads. ``pool`` is a flat uint8 array of num_pages pages.
# --------------------------------------------------------------------------
def _page_runs(page_table_row: np.ndarray, t: np.ndarray):
    """Split sorted positions t into runs that share a page: yields
    (index range into t, page id, slot offsets)."""
    pages = t // TOKENS
    cuts = np.flatnonzero(np.diff(pages)) + 1
    for r in np.split(np.arange(t.size), cuts):
        if r.size == 0:
            continue
        page = int(page_table_row[pages[r[0]]])
        assert page >= 0, "position outside the sequence's pages"
        yield r, page, t[r] % TOKENS


def mxfp4_store(pool: np.ndarray, page_table_row: np.ndarray, t0: int, rows: np.ndarray) -> None:
    """Quantize rows for positions t0.. of one sequence and write them into their
    slots (page_table_row[t // 128], t % 128)."""
    codes, sbytes = mxfp4_quantize_rows(rows)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)       # [N][64]
    pages = pool.reshape(-1, MXFP4_PAGE_BYTES)
    for r, page, off in _page_runs(page_table_row, np.arange(t0, t0 + rows.shape[0])):
        data = pages[page, :MXFP4_SCALE_OFFSET].reshape(TOKENS, 64)
        scl = pages[page, MXFP4_SCALE_OFFSET:].reshape(TOKENS, 4)
        data[off] = packed[r]
        scl[off] = sbytes[r]


def mxfp4_read(pool: np.ndarray, page_table_row: np.ndarray, L: int, positions=None) -> np.ndarray:
    """Dequantized float64 rows of one sequence: positions 0 .. L-1, or the
    given ascending ``positions`` (each < L)."""
    t = np.arange(L) if positions is None else np.asarray(positions, dtype=np.int64)
    packed = np.empty((t.size, 64), dtype=np.uint8)
    sbytes = np.empty((t.size, 4), dtype=np.uint8)
    pages = pool.reshape(-1, MXFP4_PAGE_BYTES)
    for r, page, off in _page_runs(page_table_row, t):
        packed[r] = pages[page, :MXFP4_SCALE_OFFSET].reshape(TOKENS, 64)[off]
        sbytes[r] = pages[page, MXFP4_SCALE_OFFSET:].reshape(TOKENS, 4)[off]
    codes = np.empty((t.size, DIM), dtype=np.uint8)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    return mxfp4_dequantize(codes, sbytes)


def fp8_store(pool: np.ndarray, page_table_row: np.ndarray, t0: int, rows: np.ndarray) -> None:
    codes, scale = fp8_quantize_rows(rows)
    sb = scale.astype("<f4").view(np.uint8).reshape(-1, 4)
    pages = pool.reshape(-1, FP8_PAGE_BYTES)
    for r, page, off in _page_runs(page_table_row, np.arange(t0, t0 + rows.shape[0])):
        pages[page, :FP8_SCALE_OFFSET].reshape(TOKENS, DIM)[off] = codes[r]
        pages[page, FP8_SCALE_OFFSET:].reshape(TOKENS, 4)[off] = sb[r]


def fp8_read(pool: np.ndarray, page_table_row: np.ndarray, L: int, positions=None) -> np.ndarray:
    t = np.arange(L) if positions is None else np.asarray(positions, dtype=np.int64)
    codes = np.empty((t.size, DIM), dtype=np.uint8)
    sb = np.empty((t.size, 4), dtype=np.uint8)
    pages = pool.reshape(-1, FP8_PAGE_BYTES)
    for r, page, off in _page_runs(page_table_row, t):
        codes[r] = pages[page, :FP8_SCALE_OFFSET].reshape(TOKENS, DIM)[off]
        sb[r] = pages[page, FP8_SCALE_OFFSET:].reshape(TOKENS, 4)[off]
    scale = sb.view("<f4").reshape(t.size).astype(np.float64)
    return E4M3_TABLE[codes.astype(np.int64)] * scale[:, None]


def nvfp4_store(pool: np.ndarray, page_table_row: np.ndarray, t0: int, rows: np.ndarray) -> None:
    codes, cb, S = nvfp4_quantize_rows(rows)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)       # [N][64]
    sb = S.astype("<f4").view(np.uint8).reshape(-1, 4)
    pages = pool.reshape(-1, NVFP4_PAGE_BYTES)
    for r, page, off in _page_runs(page_table_row, np.arange(t0, t0 + rows.shape[0])):
        pages[page, :NVFP4_BSCALE_OFFSET].reshape(TOKENS, 64)[off] = packed[r]
        pages[page, NVFP4_BSCALE_OFFSET:NVFP4_TSCALE_OFFSET].reshape(TOKENS, DIM // NV_BLOCK)[off] = cb[r]
        pages[page, NVFP4_TSCALE_OFFSET:].reshape(TOKENS, 4)[off] = sb[r]


def nvfp4_read(pool: np.ndarray, page_table_row: np.ndarray, L: int, positions=None) -> np.ndarray:
    t = np.arange(L) if positions is None else np.asarray(positions, dtype=np.int64)
    packed = np.empty((t.size, 64), dtype=np.uint8)
    cb = np.empty((t.size, DIM // NV_BLOCK), dtype=np.uint8)
    sb = np.empty((t.size, 4), dtype=np.uint8)
    pages = pool.reshape(-1, NVFP4_PAGE_BYTES)
    for r, page, off in _page_runs(page_table_row, t):
        packed[r] = pages[page, :NVFP4_BSCALE_OFFSET].reshape(TOKENS, 64)[off]
        cb[r] = pages[page, NVFP4_BSCALE_OFFSET:NVFP4_TSCALE_OFFSET].reshape(TOKENS, DIM // NV_BLOCK)[off]
        sb[r] = pages[page, NVFP4_TSCALE_OFFSET:].reshape(TOKENS, 4)[off]
    codes = np.empty((t.size, DIM), dtype=np.uint8)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    return nvfp4_dequantize(codes, cb, sb.view("<f4").reshape(t.size))


PAGE_BYTES = {"mxfp4": MXFP4_PAGE_BYTES, "fp8": FP8_PAGE_BYTES, "nvfp4": NVFP4_PAGE_BYTES}
STORE = {"mxfp4": mxfp4_store, "fp8": fp8_store, "nvfp4": nvfp4_store}
READ = {"mxfp4": mxfp4_read, "fp8": fp8_read, "nvfp4": nvfp4_read}
