"""Seeded generator checks and the oracle on the tiny fp32 workload (CPU only)."""

import numpy as np
import torch

from mixture_experts_ffn_gate_amd import workloads as wl
from oracle import moe_oracle as mo

from test_oracle_pins import _brute_layer


def test_generator_is_deterministic_and_shaped():
    w = wl.WORKLOADS["tiny_direct_f32"]
    a = wl.make_weights(w, seed=3)
    b = wl.make_weights(w, seed=3)
    c = wl.make_weights(w, seed=4)
    assert a["up"].shape == (w.E, w.I, w.H) and a["down"].shape == (w.E, w.H, w.I)
    assert a["shared_up"].shape == (w.S, w.H) and a["shared_down"].shape == (w.H, w.S)
    for key in a:
        assert torch.equal(a[key], b[key])
    assert not torch.equal(a["up"], c["up"])
    # N(0, 1/fan_in): the sample std is close to 1/sqrt(fan_in).
    std = a["up"].float().std().item()
    assert abs(std * np.sqrt(w.H) - 1) < 0.02
    h, r = wl.make_hidden(w, seed=3)
    assert h.shape == (w.N, w.H) and r.shape == (w.N, w.H)
    assert not torch.equal(h, r)


def test_bf16_storage_rounds_to_nearest_even():
    w = wl.WORKLOADS["nemotron_direct_bf16"].with_(E=4, I=64, S=64, H=128, N=8)
    a = wl.make_weights(w, seed=1)
    assert a["up"].dtype == torch.bfloat16 and a["gate"].dtype == torch.bfloat16
    assert a["gamma"].dtype == torch.bfloat16


def test_oracle_on_tiny_workload_matches_brute_force_rows():
    w = wl.WORKLOADS["tiny_direct_f32"]
    W = {k: wl.to_numpy_f32(v) for k, v in wl.make_weights(w, seed=0).items()}
    h, _ = wl.make_hidden(w, seed=0)
    x = wl.to_numpy_f32(h)
    out, res = mo.layer_forward(x, W, w.oracle_cfg())
    assert out.shape == (w.N, w.H)
    rows = [0, 37, 63]
    ref = _brute_layer(x[rows].astype(np.float64), W, w.E, w.k, 0, w.S, w.eps, w.scale)
    np.testing.assert_allclose(out[rows], ref, rtol=1e-10, atol=1e-11)


def test_zipf_workload_routes_follow_popularity():
    w = wl.WORKLOADS["decode_zipf_bf16"].with_(H=512, I=64, S=64, N=2000)
    W = wl.make_weights(w, seed=0)
    h, _ = wl.make_hidden(w, seed=0, gate=W["gate"])
    Wn = {"gamma": wl.to_numpy_f32(W["gamma"]), "gate": wl.to_numpy_f32(W["gate"])}
    n = mo.rms_norm(wl.to_numpy_f32(h), Wn["gamma"], w.eps)
    ids, _ = mo.topk_select(mo.sigmoid_scores(mo.gate_logits(n, Wn["gate"])), w.k)
    p = wl.zipf_expert_probs(w, seed=0).numpy()
    first = np.bincount(ids[:, 0], minlength=w.E) / ids.shape[0]
    top = np.argsort(-p)[:5]
    # The first choice follows Zipf: the most popular experts dominate it.
    assert np.all(np.abs(first[top] - p[top]) < 0.04)
    assert first[top].sum() > 0.4
