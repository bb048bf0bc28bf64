"""Helpers of the GPU parity tests: run the oracle on host copies of the exact
inputs the GPU saw and compare with the tolerances of the parity bar."""

from __future__ import annotations

import json
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from mixture_experts_ffn_gate_amd import workloads as wl_mod
from oracle import moe_oracle as mo
from oracle import nvfp4 as onv

ID_MARGIN = 1e-3          # ids compared exactly where the oracle's margins >= this
TOL = {"f32": 1e-4, "bf16": 1e-2, "nvfp4": 3e-2}
# Set to a file path to append one JSON line per compared case (errors and
# exemption counts), e.g. to record how far each configuration sits from its bar.
LOG_ENV = "MOE_PARITY_LOG"


def rel_fro(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def log_case(record: dict):
    path = os.environ.get(LOG_ENV)
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(record) + "\n")


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


class Nvfp4Experts:
    """The oracle's NVFP4 quantize + dequantize of a device fp32 master stack,
    one expert at a time (the oracle's own encoder, never the GPU's).

    The product e2m1(q) * e4m3(s) has at most 6 significant bits, so it is
    cached exactly in fp32; scale2 multiplies in float64 on use. ``prepare``
    quantizes a set of experts up front on a thread pool (numpy releases the
    GIL in the encoder's vector steps)."""

    def __init__(self, t: torch.Tensor):
        self.t = t
        self.cache = {}

    @staticmethod
    def _quant(w):
        p, s, s2 = onv.quantize(w)
        unit = onv.dequantize(p, s, 1.0).astype(np.float32)  # exact: <= 6 significant bits
        return unit, float(s2)

    def prepare(self, experts, threads: int = 16):
        todo = sorted({int(e) for e in experts} - set(self.cache))
        if not todo:
            return
        masters = [wl_mod.to_numpy_f32(self.t[e]) for e in todo]
        with ThreadPoolExecutor(threads) as ex:
            for e, res in zip(todo, ex.map(self._quant, masters)):
                self.cache[e] = res

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            self.prepare([e], threads=1)
        unit, s2 = self.cache[e]
        return unit.astype(np.float64) * s2


def oracle_weights(W: dict, nvfp4: bool = False, lazy_experts: bool = False) -> dict:
    """Host weights for the oracle. For NVFP4 layers the expert and shared
    projections are the oracle's own quantization of the fp32 masters,
    dequantized (per expert on first use when ``lazy_experts``)."""
    out = {}
    for k, v in W.items():
        if nvfp4 and k in ("up", "down"):
            if lazy_experts:
                out[k] = Nvfp4Experts(v)
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
    """Oracle ids, rank margin, scores and top-k score margin s_(k) - s_(k+1)."""
    n = mo.rms_norm(x_np, Wn["gamma"], wl.eps)
    scores = mo.sigmoid_scores(mo.gate_logits(n, Wn["gate"]))
    ids, topk_margin = mo.topk_select(scores, wl.k)
    return ids, mo.rank_margin(scores, wl.k), scores, topk_margin


def check_ids(gpu_ids, ref_ids, rank_margin, topk_margin, max_loose_frac=0.05):
    """The id bar. Where the oracle's top-k score margin s_(k) - s_(k+1) is at
    least ID_MARGIN, the GPU must select exactly the oracle's set of experts.
    Where moreover the rank margin (smallest adjacent gap among the top k+1)
    is at least ID_MARGIN, the slot order must match too. Returns the rows
    whose ids differ in any way (set or order) and the two exemption counts."""
    gpu_ids = np.asarray(gpu_ids)
    ref_ids = np.asarray(ref_ids)
    diff = np.any(gpu_ids != ref_ids, axis=1)
    set_diff = np.any(np.sort(gpu_ids, axis=1) != np.sort(ref_ids, axis=1), axis=1)
    bad_set = set_diff & (topk_margin >= ID_MARGIN)
    assert not bad_set.any(), (
        f"{bad_set.sum()} tokens select another expert set with top-k margin >= {ID_MARGIN}: "
        f"rows {np.nonzero(bad_set)[0][:10]}")
    bad_order = diff & (rank_margin >= ID_MARGIN)
    assert not bad_order.any(), (
        f"{bad_order.sum()} tokens differ with rank margin >= {ID_MARGIN}: "
        f"rows {np.nonzero(bad_order)[0][:10]}")
    assert diff.mean() <= max_loose_frac, f"too many near-tie flips: {diff.mean():.3f}"
    stats = dict(rows=int(len(diff)), set_flips=int(set_diff.sum()),
                 order_flips=int((diff & ~set_diff).sum()),
                 exempt_topk=int((topk_margin < ID_MARGIN).sum()),
                 exempt_rank=int((rank_margin < ID_MARGIN).sum()))
    return np.nonzero(diff)[0], stats


def compare_layer(wl, Wn, x_np, out_gpu, res_gpu, gpu_ids, rows=None, tol=None, case=None):
    """Oracle on ``rows`` (all if None) with the GPU's ids forced on the rows
    whose ids differ (all of them near-ties, checked by check_ids); asserts
    the residual is the input and the relative Frobenius errors of hidden_out
    and of the MoE delta hidden_out - residual, both over all compared rows
    and over the rows that needed no forcing. Returns (err_out, err_delta)."""
    rows = np.arange(x_np.shape[0]) if rows is None else np.asarray(rows)
    xs = x_np[rows]
    ref_ids, rmargin, _, tmargin = oracle_routing(xs, Wn, wl)
    flips, stats = check_ids(gpu_ids[rows], ref_ids, rmargin, tmargin)
    override = (flips, gpu_ids[rows][flips]) if len(flips) else None
    ref_out, ref_res = mo.layer_forward(xs, Wn, wl.oracle_cfg(), ids_override=override)
    np.testing.assert_array_equal(res_gpu[rows], xs)
    got = out_gpu[rows]
    e_out = rel_fro(got, ref_out)
    e_delta = rel_fro(got - xs, ref_out - ref_res)
    # Cross-check: the same metrics with the forced rows left out.
    keep = np.ones(len(rows), bool)
    keep[flips] = False
    if keep.any():
        m_out = rel_fro(got[keep], ref_out[keep])
        m_delta = rel_fro(got[keep] - xs[keep], ref_out[keep] - ref_res[keep])
    else:
        m_out = m_delta = 0.0
    tol = TOL[wl.expert_dtype if wl.expert_dtype == "nvfp4" else wl.act_dtype] if tol is None else tol
    log_case(dict(case=case or wl.name, H=wl.H, E=wl.E, k=wl.k, I=wl.I, S=wl.S, L=wl.L,
                  compared_rows=int(len(rows)), e_out=e_out, e_delta=e_delta,
                  masked_e_out=m_out, masked_e_delta=m_delta, tol=tol, **stats))
    assert e_out <= tol and e_delta <= tol, (e_out, e_delta, tol)
    assert m_out <= tol and m_delta <= tol, ("forced rows masked out", m_out, m_delta, tol)
    return e_out, e_delta


def rows_covering_experts(ids, E, extra, seed):
    """Token rows whose routes touch every expert that any token touches:
    greedily the row adding the most uncovered experts (lowest index on ties),
    then ``extra`` more rows at random, plus the first and last rows."""
    ids = np.asarray(ids)
    n = ids.shape[0]
    touched = set(np.unique(ids).tolist())
    covered, chosen = set(), []
    sets = [set(r.tolist()) for r in ids]
    while covered != touched:
        gains = np.array([len(s - covered) for s in sets])
        best = int(np.argmax(gains))
        chosen.append(best)
        covered |= sets[best]
    rng = np.random.default_rng(seed)
    rest = np.setdiff1d(np.arange(n), chosen)
    more = rng.choice(rest, size=min(extra, len(rest)), replace=False).tolist()
    return np.array(sorted(set(chosen) | set(more) | {0, n - 1}))
