"""Pins of the oracle's NVFP4 decoders, encoders and block quantizer."""

import os

import numpy as np
import pytest
import torch

from oracle import nvfp4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            rows.append((int(c, 0), float(v)))
    return rows


def test_e2m1_decode_matches_spec_table():
    table = _read_table("e2m1_values.txt")
    assert len(table) == 16
    codes = np.array([c for c, _ in table])
    got = nvfp4.e2m1_decode(codes)
    want = np.array([v for _, v in table])
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(np.signbit(got), np.signbit(want))


def test_e4m3_decode_spot_values():
    for code, val in _read_table("e4m3_spot_values.txt"):
        got = float(nvfp4.e4m3_decode(np.array([code]))[0])
        if np.isnan(val):
            assert np.isnan(got), hex(code)
        else:
            assert got == val and np.signbit(got) == np.signbit(val), hex(code)


def test_e4m3_decode_all_256_codes_match_torch():
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = nvfp4.e4m3_decode(np.arange(256))
    np.testing.assert_array_equal(np.isnan(got), np.isnan(lib))
    ok = ~np.isnan(lib)
    np.testing.assert_array_equal(got[ok], lib[ok])


def test_e4m3_encode_matches_torch_rne():
    rng = np.random.default_rng(0)
    # Random values across all binades plus exact midpoints between codes.
    x = np.exp(rng.uniform(np.log(1e-4), np.log(460.0), size=20000)).astype(np.float32)
    vals = nvfp4.e4m3_decode(np.arange(127))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, vals.astype(np.float32), np.float32([0.0, 1e-30])])
    x = x[x < 448.0 + 8.0]            # torch maps >= 464 to NaN; the oracle saturates
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int64)
    got = nvfp4.e4m3_encode_pos(x)
    np.testing.assert_array_equal(got, lib)
    assert nvfp4.e4m3_encode_pos(np.float32([500.0, 1e9]))[0] == 0x7E


def test_encoders_invert_decoders():
    c = np.arange(16)
    back = nvfp4.e2m1_encode(nvfp4.e2m1_decode(c))
    # -0 (code 8) is stored with the sign bit clear.
    np.testing.assert_array_equal(back, np.where(c == 8, 0, c))
    c = np.arange(127)
    np.testing.assert_array_equal(nvfp4.e4m3_encode_pos(nvfp4.e4m3_decode(c)), c)


@pytest.mark.parametrize("x,code", [
    (0.25, 0), (0.2499, 0), (0.2501, 1), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4),
    (3.5, 6), (5.0, 6), (5.01, 7), (7.0, 7), (1e6, 7),
    (-0.25, 0), (-0.3, 9), (-1.25, 10), (-5.0, 14), (-9.0, 15), (0.0, 0), (-0.0, 0),
])
def test_e2m1_rounding_hand_cases(x, code):
    assert int(nvfp4.e2m1_encode(np.array([x]))[0]) == code


def test_pack_order_low_nibble_first():
    # Largest magnitude 6, so the block scale decodes to 448 and scale2 * 448 ~ 1.
    codes = np.array([[1, 2, 3, 7] + [0] * 12])
    vals = nvfp4.e2m1_decode(codes)
    packed, scales, s2 = nvfp4.quantize(vals * 1.0)
    assert packed[0, 0] == (0x2 << 4) | 0x1
    assert packed[0, 1] == (0x7 << 4) | 0x3
    np.testing.assert_array_equal(nvfp4.unpack_codes(packed)[:, :4], codes[:, :4])


def test_quantize_scale_chain_and_error_bound():
    rng = np.random.default_rng(1)
    w = (rng.normal(size=(64, 256)) / 16).astype(np.float32)
    packed, scales, scale2 = nvfp4.quantize(w)
    assert packed.shape == (64, 128) and scales.shape == (64, 16)
    assert scale2 == np.float32(np.float32(np.abs(w).max()) / np.float32(2688))
    deq = nvfp4.dequantize(packed, scales, scale2)
    sdec = nvfp4.e4m3_decode(scales)
    # The block holding the global maximum gets the largest scale code (448).
    assert sdec.max() == 448.0
    # Per element: at most one E2M1 step of the block's scale (half a step from
    # rounding plus the scale's own rounding, which can push the ratio to 6.4).
    step = np.repeat(sdec, 16, axis=1) * float(scale2)
    assert np.all(np.abs(deq - w) <= step * 1.0 + 1e-12)
    rel = np.linalg.norm(deq - w) / np.linalg.norm(w)
    assert rel < 0.15


def test_quantize_is_idempotent_on_its_output():
    rng = np.random.default_rng(2)
    w = (rng.normal(size=(32, 128)) * 0.03).astype(np.float32)
    p1, s1, a1 = nvfp4.quantize(w)
    d1 = nvfp4.dequantize(p1, s1, a1).astype(np.float32)
    p2, s2, a2 = nvfp4.quantize(d1)
    np.testing.assert_array_equal(p2, p1)
    np.testing.assert_array_equal(s2, s1)
    assert a2 == a1


def test_quantize_zero_blocks_and_zero_matrix():
    w = np.zeros((2, 32), np.float32)
    w[1, 16:] = 3.0
    p, s, a = nvfp4.quantize(w)
    assert (nvfp4.unpack_codes(p)[0] == 0).all() and (s[0] == 0).all()
    np.testing.assert_allclose(nvfp4.dequantize(p, s, a), w, rtol=2e-7, atol=0)
    p, s, a = nvfp4.quantize(np.zeros((3, 16), np.float32))
    assert a == 0 and (p == 0).all() and (s == 0).all()
