"""Seeded synthetic workloads for the MoE FFN layer.

This module only draws inputs. It holds none of the layer's arithmetic and
imports nothing from the HIP binding or from the oracle; both sides take the
tensors it returns.

Recipe (every tensor has its own generator, seeded from the workload seed and
a fixed tensor id, so any tensor can be redrawn on its own):
  * weights ~ N(0, 1/fan_in) with fan_in the ``in`` dimension, drawn in fp32
    and rounded (RNE) to the workload's storage dtype;
  * RMSNorm gamma = 1 (``gamma_noise`` > 0 gives 1 + noise * N(0, 1));
  * hidden ~ N(0, 1), residual ~ N(0, 1) (the layer overwrites residual);
  * NVFP4 workloads return the fp32 master weights of the routed and shared
    experts; each side quantizes them with its own encoder;
  * the Zipf decode workload biases routing: with ``p_e`` ∝ rank^-s over a
    seeded permutation of experts and Gumbel noise ``G``, it sets
    ``b_t = log p + G_t`` and builds ``hidden_t = P z_t + V b_t`` where
    ``V = W_g^T (W_g W_g^T)^-1`` and ``P = I - V W_g``, so the gate sees
    ``b_t`` scaled by the row's RMS and top-k is a Plackett-Luce draw whose
    first choice follows Zipf(s).

Shapes follow the layer: H hidden, E experts, k top_k, I expert inter,
S shared inter (0 = none), L latent (0 = direct), N tokens.
"""

from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    H: int
    E: int
    k: int
    I: int
    S: int
    L: int
    N: int
    act_dtype: str = "bf16"      # "f32" | "bf16": hidden, residual, gamma, gate, fc1, fc2
    expert_dtype: str = "bf16"   # "f32" | "bf16" | "nvfp4": routed + shared experts
    zipf_s: float = 0.0          # > 0: Zipf-biased routing (decode sweep)
    eps: float = 1e-5
    scale: float = 1.0

    @property
    def D(self) -> int:
        return self.L if self.L > 0 else self.H

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def oracle_cfg(self) -> dict:
        return dict(E=self.E, k=self.k, L=self.L, S=self.S, eps=self.eps, scale=self.scale)

    # Algorithmic work of one forward over n tokens (weights read once).
    def flops(self, n: int | None = None) -> float:
        n = self.N if n is None else n
        R = n * self.k
        f = 2.0 * n * self.H * self.E                     # gate
        f += 2.0 * R * self.D * self.I * 2                # routed up + down
        f += 2.0 * n * self.H * self.S * 2                # shared up + down
        if self.L:
            f += 2.0 * n * self.H * self.L * 2            # fc1 + fc2
        return f


WORKLOADS = {
    # Tiny direct layer in fp32 (the oracle finishes in well under a second).
    "tiny_direct_f32": Workload("tiny_direct_f32", H=256, E=8, k=2, I=128, S=256, L=0,
                                N=64, act_dtype="f32", expert_dtype="f32"),
    # Nemotron-H-style direct layer, bf16 storage, fp32 accumulation.
    "nemotron_direct_bf16": Workload("nemotron_direct_bf16", H=2688, E=128, k=6, I=1856,
                                     S=3712, L=0, N=1024),
    # LatentMoE layer: experts act on a 1024-wide latent.
    "latent_bf16": Workload("latent_bf16", H=4096, E=128, k=8, I=2688, S=5376, L=1024,
                            N=2048),
    # Decode-sized sweep on the direct shapes with Zipf(1.1) expert popularity.
    "decode_zipf_bf16": Workload("decode_zipf_bf16", H=2688, E=128, k=6, I=1856, S=3712,
                                 L=0, N=16, zipf_s=1.1),
    # NVFP4 routed + shared experts, bf16 activations.
    "nvfp4_direct": Workload("nvfp4_direct", H=2688, E=128, k=6, I=1856, S=3712, L=0,
                             N=4096, expert_dtype="nvfp4"),
}
DECODE_NS = (1, 2, 4, 8, 16)

_TENSOR_IDS = dict(gamma=1, gate=2, fc1=3, fc2=4, up=5, down=6, shared_up=7,
                   shared_down=8, hidden=9, residual=10, zipf_perm=11, zipf_gumbel=12,
                   zipf_z=13)

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _gen(seed: int, tensor: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + _TENSOR_IDS[tensor] * 7919) & 0x7FFF_FFFF_FFFF)
    return g


def _normal(shape, std, seed, tensor, device):
    g = _gen(seed, tensor, device)
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def make_weights(w: Workload, seed: int = 0, device="cpu", gamma_noise: float = 0.0) -> dict:
    """Layer weights as torch tensors on ``device``.

    Activation-side tensors use ``w.act_dtype``. Expert tensors use
    ``w.expert_dtype``; for "nvfp4" they stay fp32 masters.
    """
    adt = _TORCH_DT[w.act_dtype]
    edt = torch.float32 if w.expert_dtype == "nvfp4" else _TORCH_DT[w.expert_dtype]
    D = w.D
    out = {}
    if gamma_noise > 0:
        out["gamma"] = (1.0 + _normal((w.H,), gamma_noise, seed, "gamma", device)).to(adt)
    else:
        out["gamma"] = torch.ones(w.H, device=device, dtype=adt)
    out["gate"] = _normal((w.E, w.H), 1 / math.sqrt(w.H), seed, "gate", device).to(adt)
    if w.L:
        out["fc1"] = _normal((w.L, w.H), 1 / math.sqrt(w.H), seed, "fc1", device).to(adt)
        out["fc2"] = _normal((w.H, w.L), 1 / math.sqrt(w.L), seed, "fc2", device).to(adt)
    out["up"] = _normal((w.E, w.I, D), 1 / math.sqrt(D), seed, "up", device).to(edt)
    out["down"] = _normal((w.E, D, w.I), 1 / math.sqrt(w.I), seed, "down", device).to(edt)
    if w.S:
        out["shared_up"] = _normal((w.S, w.H), 1 / math.sqrt(w.H), seed, "shared_up",
                                   device).to(edt)
        out["shared_down"] = _normal((w.H, w.S), 1 / math.sqrt(w.S), seed, "shared_down",
                                     device).to(edt)
    return out


def make_hidden(w: Workload, n: int | None = None, seed: int = 0, device="cpu",
                gate: torch.Tensor | None = None):
    """``(hidden, residual)`` for ``n`` tokens in the activation dtype.

    For Zipf workloads ``gate`` (the layer's gate weight) is required.
    """
    n = w.N if n is None else n
    adt = _TORCH_DT[w.act_dtype]
    residual = _normal((n, w.H), 1.0, seed, "residual", device).to(adt)
    if w.zipf_s <= 0:
        hidden = _normal((n, w.H), 1.0, seed, "hidden", device).to(adt)
        return hidden, residual
    if gate is None:
        raise ValueError("Zipf workloads need the gate weight")
    return _zipf_hidden(w, n, seed, gate).to(device=device, dtype=adt), residual


def _zipf_hidden(w: Workload, n: int, seed: int, gate: torch.Tensor) -> torch.Tensor:
    """Hidden rows whose gate projection is a Gumbel-perturbed log-Zipf vector."""
    cpu = "cpu"
    g_perm = _gen(seed, "zipf_perm", cpu)
    perm = torch.randperm(w.E, generator=g_perm)
    rank = torch.empty(w.E, dtype=torch.float64)
    rank[perm] = torch.arange(1, w.E + 1, dtype=torch.float64)
    p = rank.pow(-w.zipf_s)
    p = p / p.sum()
    g_gum = _gen(seed, "zipf_gumbel", cpu)
    u = torch.rand(n, w.E, generator=g_gum, dtype=torch.float64).clamp_(1e-12, 1 - 1e-12)
    b = p.log()[None, :] - torch.log(-torch.log(u))                  # [n, E]
    Wg = gate.detach().to(cpu, torch.float64)                           # [E, H]
    V = Wg.T @ torch.linalg.inv(Wg @ Wg.T)                              # [H, E]
    z = torch.randn(n, w.H, generator=_gen(seed, "zipf_z", cpu), dtype=torch.float64)
    hid = z - (z @ Wg.T) @ V.T + b @ V.T
    return hid.to(torch.float32)


def zipf_expert_probs(w: Workload, seed: int = 0) -> torch.Tensor:
    """The Zipf popularity vector p_e of a Zipf workload (for reports)."""
    g_perm = _gen(seed, "zipf_perm", "cpu")
    perm = torch.randperm(w.E, generator=g_perm)
    rank = torch.empty(w.E, dtype=torch.float64)
    rank[perm] = torch.arange(1, w.E + 1, dtype=torch.float64)
    p = rank.pow(-w.zipf_s)
    return p / p.sum()


def to_numpy_f32(t: torch.Tensor):
    """Host fp32 copy of a tensor (bf16 widens exactly)."""
    return t.detach().to("cpu", torch.float32).numpy()
