"""NVFP4 weight format of the oracle: decoders, encoders, two-level quantizer.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources: the "metrale_model_arch/nemotron_moe.rs" source page
(``ExpertPtrTable``: per expert a packed 4-bit table, a block-scale table and
one per-tensor ``scale2`` value) and the "Struct MoeLayer" page (weights packed
as ``[N, K/2]`` bytes, scales per 16 along K). The pages name the format but
print neither the code points nor the quantizer, so the following readings are
taken (also listed in the design notes):

  * E2M1 element: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0;
    magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
  * E4M3 block scale (OCP "fn" variant): sign bit 7, exponent bits 6..3
    (bias 7), mantissa bits 2..0; exponent 0 is subnormal; 0x7F/0xFF are NaN;
    largest finite 448. One scale per 16 consecutive K elements of a row.
  * Packing: element ``k`` of a row sits in byte ``k // 2``, low nibble when
    ``k`` is even.
  * Quantizer, per matrix ``W`` (one expert's projection), every step in
    fp32 arithmetic (the precision the device quantizer decides in):
      scale2 = amax|W| / 2688                  (2688 = 6 * 448)
      s_b    = E4M3_rne(amax_b / (6 * scale2)) per 16-element block b
      q      = E2M1_rne(w / (dec(s_b) * scale2)), saturating at 6
    with round-to-nearest, ties to the even code. A zero magnitude is stored
    with the sign bit clear. If ``scale2`` or ``dec(s_b)`` is 0 the block's
    codes are 0.
  * Dequant: ``w = dec(q) * dec(s_b) * scale2``.

Pins: exhaustive 16-code and 256-code tables written out from the format
definitions in the tests; encode(decode(c)) == c for every finite code;
hand-worked rounding cases (ties, saturation, subnormals); quantize is
idempotent on its own dequantized output.
"""

from __future__ import annotations

import numpy as np

F32 = np.float32


def e2m1_decode(codes):
    """Value of 4-bit E2M1 codes (array of ints 0..15) as float64."""
    c = np.asarray(codes, dtype=np.int64)
    mag = c & 7
    e = mag >> 1
    m = mag & 1
    val = np.where(e == 0, m * 0.5, np.ldexp(1.0 + m * 0.5, (e - 1).astype(np.int64)))
    return np.where(c & 8, -val, val).astype(np.float64)


def e4m3_decode(codes):
    """Value of 8-bit E4M3 (fn) codes as float64 (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.int64)
    e = (c >> 3) & 15
    m = c & 7
    val = np.where(e == 0, np.ldexp(m / 8.0, -6),
                   np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64)))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return np.where(c & 128, -val, val).astype(np.float64)


_E2M1_POS = e2m1_decode(np.arange(8))          # codes 0..7, increasing
_E4M3_POS = e4m3_decode(np.arange(127))        # codes 0..126 (0x7E = 448)


def _nearest_code(x, table):
    """Nearest entry of an increasing table for x >= 0; ties to the even code;
    values past the end saturate to the last code."""
    x = np.asarray(x, dtype=np.float64)
    hi = np.searchsorted(table, x, side="left")
    hi = np.clip(hi, 0, len(table) - 1)
    lo = np.clip(hi - 1, 0, len(table) - 1)
    d_lo = np.abs(x - table[lo])
    d_hi = np.abs(table[hi] - x)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(x >= table[-1], len(table) - 1, code)
    return code.astype(np.int64)


def e4m3_encode_pos(x):
    """Round non-negative finite values to the nearest E4M3 code (ties even, saturating)."""
    return _nearest_code(x, _E4M3_POS)


def e2m1_encode(x):
    """Round values to the nearest E2M1 code (ties even, saturating at 6).
    Negative values get the sign bit unless they round to zero."""
    x = np.asarray(x, dtype=np.float64)
    mag = _nearest_code(np.abs(x), _E2M1_POS)
    return np.where((x < 0) & (mag != 0), mag | 8, mag).astype(np.int64)


def quantize(w):
    """Two-level NVFP4 quantization of one matrix ``w [rows, K]`` (K % 16 == 0).

    Returns ``(packed u8 [rows, K/2], scales u8 [rows, K/16], scale2 float32)``.
    """
    w32 = np.asarray(w, dtype=F32)
    rows, K = w32.shape
    assert K % 16 == 0, "K must be a multiple of 16"
    amax = F32(np.max(np.abs(w32))) if w32.size else F32(0)
    scale2 = F32(amax / F32(2688.0))
    blocks = w32.reshape(rows, K // 16, 16)
    if scale2 == 0:
        codes = np.zeros((rows, K), dtype=np.int64)
        sb = np.zeros((rows, K // 16), dtype=np.int64)
    else:
        amax_b = np.max(np.abs(blocks), axis=-1).astype(F32)
        t = F32(F32(6.0) * scale2)
        sb = e4m3_encode_pos((amax_b / t).astype(F32))
        sdec = e4m3_decode(sb).astype(F32)
        denom = (sdec * scale2).astype(F32)                  # [rows, K/16]
        safe = np.where(denom > 0, denom, F32(1.0)).astype(F32)
        ratio = (blocks / safe[..., None]).astype(F32)
        codes = e2m1_encode(ratio)
        codes = np.where((denom > 0)[..., None], codes, 0).reshape(rows, K)
    lo = codes[:, 0::2]
    hi = codes[:, 1::2]
    packed = (lo | (hi << 4)).astype(np.uint8)
    return packed, sb.astype(np.uint8), scale2


def unpack_codes(packed):
    """``[rows, K/2]`` bytes -> ``[rows, K]`` 4-bit codes (even k = low nibble)."""
    p = np.asarray(packed, dtype=np.int64)
    rows, half = p.shape
    out = np.empty((rows, half * 2), dtype=np.int64)
    out[:, 0::2] = p & 15
    out[:, 1::2] = p >> 4
    return out


def dequantize(packed, scales, scale2):
    """``dec(q) * dec(s_b) * scale2`` as float64 ``[rows, K]``."""
    codes = unpack_codes(packed)
    rows, K = codes.shape
    vals = e2m1_decode(codes).reshape(rows, K // 16, 16)
    sdec = e4m3_decode(np.asarray(scales))[..., None]
    return (vals * sdec * float(scale2)).reshape(rows, K)


def quantize_stack(w):
    """Quantize ``w [G, rows, K]`` one matrix at a time (one scale2 per matrix)."""
    w = np.asarray(w)
    res = [quantize(w[g]) for g in range(w.shape[0])]
    packed = np.stack([r[0] for r in res])
    scales = np.stack([r[1] for r in res])
    scale2 = np.array([r[2] for r in res], dtype=F32)
    return packed, scales, scale2


def dequantize_stack(packed, scales, scale2):
    return np.stack([dequantize(packed[g], scales[g], scale2[g])
                     for g in range(packed.shape[0])])
