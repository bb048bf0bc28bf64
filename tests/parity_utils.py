"""Helpers of the GPU parity tests: run the oracle on host copies of the exact
inputs the GPU saw and compare with the tolerances of the parity bar."""

from __future__ import annotations

import numpy as np
import torch

from mixture_experts_ffn_gate_amd import workloads as wl_mod
from oracle import moe_oracle as mo
from oracle import nvfp4 as onv

ID_MARGIN = 1e-3          # ids compared exactly where the oracle rank margin >= this
TOL = {"f32": 1e-4, "bf16": 1e-2, "nvfp4": 3e-2}


def rel_fro(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


class LazyExperts:
    """Per-expert host fp32 copies of a device [E, out, in] tensor, fetched on use."""

    def __init__(self, t: torch.Tensor):
        self.t = t
        self.cache = {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            self.cache[e] = wl_mod.to_numpy_f32(self.t[e])
        return self.cache[e]


class LazyNvfp4Experts:
    """Per-expert oracle NVFP4 quantize + dequantize of a device fp32 master
    stack, computed on first use (the oracle's own encoder, never the GPU's)."""

    def __init__(self, t: torch.Tensor):
        self.t = t
        self.cache = {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            p, s, s2 = onv.quantize(wl_mod.to_numpy_f32(self.t[e]))
            self.cache[e] = onv.dequantize(p, s, s2)
        return self.cache[e]


def oracle_weights(W: dict, nvfp4: bool = False, lazy_experts: bool = False) -> dict:
    """Host weights for the oracle. For NVFP4 layers the expert and shared
    projections are the oracle's own quantization of the fp32 masters,
    dequantized (per expert on first use when ``lazy_experts``)."""
    out = {}
    for k, v in W.items():
        if nvfp4 and k in ("up", "down"):
            if lazy_experts:
                out[k] = LazyNvfp4Experts(v)
            else:
                p, s, s2 = onv.quantize_stack(wl_mod.to_numpy_f32(v))
                out[k] = onv.dequantize_stack(p, s, s2)
        elif nvfp4 and k in ("shared_up", "shared_down"):
            p, s, s2 = onv.quantize(wl_mod.to_numpy_f32(v))
            out[k] = onv.dequantize(p, s, s2)
        elif k in ("up", "down") and lazy_experts:
            out[k] = LazyExperts(v)
        else:
            out[k] = wl_mod.to_numpy_f32(v)
    return out


def oracle_routing(x_np, Wn, wl):
    n = mo.rms_norm(x_np, Wn["gamma"], wl.eps)
    scores = mo.sigmoid_scores(mo.gate_logits(n, Wn["gate"]))
    ids, _ = mo.topk_select(scores, wl.k)
    return ids, mo.rank_margin(scores, wl.k), scores


def check_ids(gpu_ids, ref_ids, margin, max_loose_frac=0.05):
    """Ids must match exactly wherever the oracle's rank margin >= ID_MARGIN.
    Returns the rows whose ids differ (all of them near-ties)."""
    diff = np.any(gpu_ids != ref_ids, axis=1)
    bad = diff & (margin >= ID_MARGIN)
    assert not bad.any(), (
        f"{bad.sum()} tokens differ with margin >= {ID_MARGIN}: rows {np.nonzero(bad)[0][:10]}")
    assert diff.mean() <= max_loose_frac, f"too many near-tie flips: {diff.mean():.3f}"
    return np.nonzero(diff)[0]


def compare_layer(wl, Wn, x_np, out_gpu, res_gpu, gpu_ids, rows=None, tol=None):
    """Oracle on ``rows`` (all if None) with the GPU's ids forced on near-tie
    rows; returns (err_out, err_delta). Asserts the residual is the input."""
    rows = np.arange(x_np.shape[0]) if rows is None else np.asarray(rows)
    xs = x_np[rows]
    ref_ids, margin, _ = oracle_routing(xs, Wn, wl)
    flips = check_ids(gpu_ids[rows], ref_ids, margin)
    override = (flips, gpu_ids[rows][flips]) if len(flips) else None
    ref_out, ref_res = mo.layer_forward(xs, Wn, wl.oracle_cfg(), ids_override=override)
    np.testing.assert_array_equal(res_gpu[rows], xs)
    e_out = rel_fro(out_gpu[rows], ref_out)
    e_delta = rel_fro(out_gpu[rows] - xs, ref_out - ref_res)
    tol = TOL[wl.expert_dtype if wl.expert_dtype == "nvfp4" else wl.act_dtype] if tol is None else tol
    assert e_out <= tol and e_delta <= tol, (e_out, e_delta, tol)
    return e_out, e_delta
