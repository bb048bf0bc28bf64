"""Precision of 8-bit and 4-bit activation arms, measured on the CPU.

The pages pre-dequantize dense projections to FP8 for prefill and run 4-bit x
4-bit grouped GEMMs (page "metrale_model_arch/nemotron_moe.rs":
`NemotronMoeLayer` fields for FP8 shared-up / fc1 copies, the FP8 and W4A4
GEMM handles resolved in `new`). Either arm needs the activations in that
format too, since an MFMA takes both operands in one type. This study fixes
whether such an arm can meet the 3e-2 relative Frobenius bar of 4-bit-weight
layers: one routed expert FFN at the direct layer's shapes (H = 2688,
I = 1856, N(0, 1/fan_in) weights, 64 unit-RMS token rows), its up input z and
down input h = relu(up z)^2 quantized with the oracle's own E4M3 / E2M1
codecs, everything else in float64. Reference: the same FFN unquantized.

Findings pinned here (relative Frobenius error of the FFN output): bf16
activations, the built path, about 0.3%; E4M3 activations 4.0% with one fp32
scale per row, 5.0% with one power-of-two scale per 32 (the OCP MX format
that gfx950's scaled fp8 MFMA applies), about 3.2% with one fp32 scale per
32, and about 3.0% -- at the bar, with no margin for the layer's other
roundings -- with one fp32 scale per 16: a 3-bit mantissa rounds each element
by up to 1/16 and a dot product keeps that relative error, finer scales only
avoid the subnormal range. E4M3 weights add to it; 4-bit activations (E2M1,
per-16 E4M3 block scales) reach about 13%. No fp8 or 4-bit activation scheme
stays under the bar with a margin, so neither arm is built.
"""

import numpy as np
import pytest
import torch

from mixture_experts_ffn_gate_amd import workloads as wlm
from oracle import moe_oracle as mo
from oracle import nvfp4

BAR = 3e-2
E4M3_MAX = 448.0


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy() \
        .astype(np.float64)


def _e4m3(x):
    """Round to the nearest E4M3 value (ties even, saturating at 448), signed."""
    x = np.asarray(x, np.float64)
    mag = nvfp4.e4m3_decode(nvfp4.e4m3_encode_pos(np.abs(x)))
    return np.where(x < 0, -mag, mag)


def _blocks(x, size):
    rows, cols = x.shape
    assert cols % size == 0
    return x.reshape(rows, cols // size, size)


def fp8_per_row(x):
    s = np.max(np.abs(x), axis=1, keepdims=True) / E4M3_MAX
    s = np.where(s > 0, s, 1.0)
    return _e4m3(x / s) * s


def fp8_per_block_fp32(x, size=16):
    b = _blocks(x, size)
    s = np.max(np.abs(b), axis=2, keepdims=True) / E4M3_MAX
    s = np.where(s > 0, s, 1.0)
    return (_e4m3(b / s) * s).reshape(x.shape)


def fp8_mx(x, size=32):
    """OCP MX: one power-of-two scale per 32, 2^(floor(log2 amax) - 8) for E4M3."""
    b = _blocks(x, size)
    amax = np.max(np.abs(b), axis=2, keepdims=True)
    e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8
    s = np.exp2(e)
    return (_e4m3(b / s) * s).reshape(x.shape)


def fp4_nvfp4(x):
    """E2M1 values with one E4M3 scale per 16 and an fp32 scale per matrix,
    through the oracle's two-level quantizer."""
    p, sc, s2 = nvfp4.quantize(np.asarray(x, np.float32))
    return nvfp4.dequantize(p, sc, s2)


SCHEMES = {"bf16": _bf16, "fp8_row": fp8_per_row, "fp8_mx32": fp8_mx,
           "fp8_block32": lambda x: fp8_per_block_fp32(x, 32),
           "fp8_block16": fp8_per_block_fp32, "fp4_nvfp4": fp4_nvfp4}


@pytest.fixture(scope="module")
def expert():
    wl = wlm.Workload("study", H=2688, E=1, k=1, I=1856, S=0, L=0, N=64)
    W = wlm.make_weights(wl, seed=3, device="cpu")
    up = wlm.to_numpy_f32(W["up"][0]).astype(np.float64)
    down = wlm.to_numpy_f32(W["down"][0]).astype(np.float64)
    hidden, _ = wlm.make_hidden(wl, wl.N, seed=3, device="cpu")
    z = mo.rms_norm(wlm.to_numpy_f32(hidden), np.ones(wl.H), wl.eps)
    return z, up, down


def _ffn_error(z, up, down, quant, wquant=None):
    ref = mo.expert_ffn(z, up, down)
    if wquant is not None:
        up, down = wquant(up), wquant(down)
    h = quant(mo.relu2(quant(z) @ up.T))
    got = h @ down.T
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def test_quantizers_are_faithful():
    # Each quantizer returns representable values on the given grid:
    # E4M3 values times the scale, and exact values pass through.
    x = np.array([[0.0, 1.0, -2.0, 448.0, 1.125, 3.0, -0.5, 6.0] * 4])
    np.testing.assert_array_equal(_e4m3(x), x)                 # all exact in E4M3
    assert _e4m3(np.array([1.0625]))[0] == 1.0                 # tie to even mantissa
    assert _e4m3(np.array([1000.0]))[0] == 448.0               # saturates
    y = fp8_per_row(x)
    np.testing.assert_allclose(y, x, rtol=0, atol=0)           # amax 448: scale 1
    m = fp8_mx(x)                                              # amax 448: scale 2^0
    np.testing.assert_array_equal(m, x)


@pytest.mark.parametrize("scheme", list(SCHEMES))
def test_activation_precision_against_bar(expert, scheme):
    z, up, down = expert
    err = _ffn_error(z, up, down, SCHEMES[scheme])
    print(f"{scheme}: relative error {err:.4f}")
    if scheme == "bf16":
        assert err < 1e-2                   # the built path: well inside every bar
    elif scheme == "fp8_block16":
        # one fp32 scale per 16 sits at the bar (2.96-3.03% over four seeds),
        # with no margin left for the layer's other roundings (bf16 normed,
        # shared expert, output), which add to the same delta
        assert 0.9 * BAR < err < 1.1 * BAR
    elif scheme.startswith("fp8"):
        assert BAR < err < 0.06             # over the bar: per row, per 32 (MX or fp32)
    else:
        assert err > 0.1                    # 4-bit activations: far over it


def test_fp8_weights_add_error(expert):
    # The pages' pre-dequantized FP8 copies: E4M3 weights with one scale per
    # output row, on top of the best fp8 activation scheme an fp8 MFMA can
    # apply (fp32 scales per 32) -- further over the bar.
    z, up, down = expert
    err = _ffn_error(z, up, down, SCHEMES["fp8_block32"], wquant=fp8_per_row)
    act_only = _ffn_error(z, up, down, SCHEMES["fp8_block32"])
    print(f"fp8 weights + fp8_block32 activations: relative error {err:.4f}")
    assert err > act_only > BAR
