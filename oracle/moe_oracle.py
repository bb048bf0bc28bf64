"""Plain float64 CPU oracle of the Nemotron-H MoE FFN layer forward.

TEST INFRASTRUCTURE ONLY: imported by the tests, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.

Sources (web pages; cited by page and section):
  [src]  "metrale_model_arch/nemotron_moe.rs" source page: the module doc
         (what the forward computes), ``NemotronMoeLayer::new`` (config
         checks, per-layer defaults) and ``NemotronMoeLayer::prefill``
         (order of the prologue steps, scratch carve-out, sorted path).
  [moe]  "Struct MoeLayer" page: ``forward_prefill`` (the sorted grouped-GEMM
         pipeline: gate, top-k, sort, grouped up, activation, grouped down,
         unpermute + weighted reduce, shared expert) and
         ``fp32_routing_active`` (router fed at full precision).
  [lay]  "Struct NemotronMoeLayer" page: ``decode`` (hidden modified in
         place), ``prefill`` (batched projections).

Precision: every step runs in float64 on inputs widened exactly from their
storage dtype (bf16 and fp32 widen exactly). The one exception is the routing
decision, a floating-point comparison that picks integers: it is taken on
fp32 sigmoid scores of fp32-rounded logits, the precision the pages' router
works in (fp32 gate-logit buffer; the full-precision router lever on [moe]).

Readings where the pages are silent (each also listed in the design notes):
  * ``residual`` is written with the pre-norm ``hidden`` and the output is
    ``hidden <- residual + routed + shared`` (the module doc of [src] says
    the result is added to ``hidden``; ``rms_norm_residual`` writes it).
  * RMSNorm is ``x / sqrt(mean(x^2) + eps) * gamma`` (no 1+gamma offset).
  * Top-k orders experts by (score descending, index ascending); slot j of a
    token holds its j-th choice. Weights are the selected scores divided by
    their sum, times ``routed_scaling_factor``; if that sum is 0 each weight
    is 1/k.
  * The sort is stable: expert e's routes sit at ``offsets[e]..offsets[e+1]``
    in ascending route id ``r = t*k + j``.
  * relu^2 is ``max(x, 0)^2``; experts are not gated (up and down only).
  * LatentMoE: ``fc1`` maps normed hidden to latent before the experts, and
    ``fc2`` maps the weighted routed sum back to hidden; the gate and the
    shared expert read the hidden-space normed vector.
  * The shared expert is added unweighted; ``routed_scaling_factor`` scales
    only the routed sum.

Weight layout: every matrix is ``[out][in]`` row-major: gate ``[E,H]``,
fc1 ``[L,H]``, fc2 ``[H,L]``, up ``[E,I,D]``, down ``[E,D,I]``, shared_up
``[S,H]``, shared_down ``[H,S]`` with ``D = L`` if latent else ``H``.

Pins (tests that tie each function to something other than itself):
  rms_norm          closed form on constant rows; exact rational brute force
  gate_logits       one-hot gate rows select normed entries; brute force loop
  sigmoid_scores    closed values (0 -> 0.5, symmetric pairs sum to 1)
  rank_margin       brute force over sorted score lists
  topk_select       brute force over all k-subsets / Python ``sorted`` with an
                    explicit key, forced ties
  routing_weights   sum to scale; all-equal scores give 1/k
  sort_routes       Python ``sorted`` brute force; counts/offset/permutation
                    invariants; permute-then-unpermute identity
  expert_ffn        [I;-I] / [I|-I] experts give z*|z|; scalar loop
  layer_forward     pure-Python per-token loop (no sort, no matmul); top_k=E
                    with a zero gate gives the mean of all experts; identity-
                    like experts reproduce the normed input; E=k=1 is a dense
                    relu^2 FFN; latent with identity fc1/fc2 equals direct;
                    row-split invariance and token-permutation equivariance
"""

from __future__ import annotations

import numpy as np

F64 = np.float64


class ConfigError(ValueError):
    """Raised for a layer configuration the pages' constructor refuses."""


def check_config(num_experts: int, top_k: int, max_experts: int = 512,
                 max_top_k: int = 16) -> None:
    """Config checks of ``NemotronMoeLayer::new`` [src].

    The constructor refuses a ``top_k`` outside ``1..=num_experts`` and values
    over the routing kernels' bounds. The pages do not print those bounds; the
    ones used here are this library's (512 experts, top_k 16).
    """
    if not (1 <= top_k <= num_experts):
        raise ConfigError(f"top_k={top_k} must be in 1..={num_experts}")
    if top_k > max_top_k:
        raise ConfigError(f"top_k={top_k} exceeds the routing bound {max_top_k}")
    if num_experts > max_experts:
        raise ConfigError(f"num_experts={num_experts} exceeds the routing bound {max_experts}")


def rms_norm(x, gamma, eps: float):
    """RMS norm of each row [src module doc; prefill step ``rms_norm_residual``].

    ``n_t = x_t / sqrt(mean_i x_ti^2 + eps) * gamma``.
    """
    x = np.asarray(x, dtype=F64)
    g = np.asarray(gamma, dtype=F64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def gate_logits(normed, w_gate):
    """Router projection ``logits = normed @ W_g^T`` [src prefill, gate GEMM]."""
    return np.asarray(normed, dtype=F64) @ np.asarray(w_gate, dtype=F64).T


def sigmoid_scores(logits):
    """Sigmoid scores in fp32, the routing decision precision [src module doc].

    The logits are rounded to fp32 and ``1 / (1 + exp(-l))`` is evaluated in
    fp32 arithmetic, so that the integer decision that follows (top-k) is taken
    in the precision the router works in.
    """
    l32 = np.asarray(logits, dtype=F64).astype(np.float32)
    one = np.float32(1.0)
    with np.errstate(over="ignore"):
        return (one / (one + np.exp(-l32))).astype(np.float32)


def topk_select(scores, k: int):
    """Top-k experts per token [src module doc: sigmoid top-k routing].

    Experts are ordered by (score descending, index ascending) and the first
    ``k`` are taken in that order. Returns ``ids`` int32 ``[N,k]`` and the
    score margin ``s_(k) - s_(k+1)`` per token (``inf`` when ``k == E``).
    """
    s = np.asarray(scores)
    n, e = s.shape
    # A stable sort of the negated scores keeps equal scores in index order.
    order = np.argsort(-s.astype(F64), axis=-1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    if k < e:
        ranked = np.take_along_axis(s.astype(F64), order, axis=-1)
        margin = ranked[:, k - 1] - ranked[:, k]
    else:
        margin = np.full(n, np.inf)
    return ids, margin


def rank_margin(scores, k: int):
    """Smallest gap between adjacent ranks among a token's top ``k+1`` scores.

    A token whose rank margin is small can legally change its selected set or
    its slot order under a different rounding of the logits; the parity tests
    compare ids exactly only where this margin is at least their threshold.
    (With k == E the top k are all experts and only their order matters.)
    """
    s = np.asarray(scores).astype(F64)
    n, e = s.shape
    ranked = -np.sort(-s, axis=-1)[:, :min(k + 1, e)]
    if ranked.shape[1] < 2:
        return np.full(n, np.inf)
    return np.min(ranked[:, :-1] - ranked[:, 1:], axis=-1)


def routing_weights(scores, ids, scale: float = 1.0):
    """Renormalized routing weights times the routed scaling factor [src prefill, ``scale``].

    ``w_tj = s_t[ids_tj] / sum_j s_t[ids_tj] * scale``; ``1/k`` each if the sum is 0.
    """
    sel = np.take_along_axis(np.asarray(scores, dtype=F64), np.asarray(ids), axis=-1)
    k = sel.shape[-1]
    tot = sel.sum(axis=-1, keepdims=True)
    safe = np.where(tot > 0, tot, 1.0)
    w = np.where(tot > 0, sel / safe, 1.0 / k)
    return w * float(scale)


def sort_routes(ids, num_experts: int):
    """Sort (token, slot) routes by expert [moe forward_prefill: sort step].

    Route ``r = t*k + j`` goes to expert ``ids[t, j]``. Returns
    ``counts[E]``, ``offsets[E+1]`` (exclusive prefix sum),
    ``perm[R]`` (route id at each sorted position, ascending r within an
    expert) and ``inv[R]`` (sorted position of each route). All int32.
    """
    flat = np.asarray(ids).reshape(-1).astype(np.int64)
    r = flat.size
    counts = np.bincount(flat, minlength=num_experts)[:num_experts]
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    perm = np.argsort(flat, kind="stable")
    inv = np.empty(r, dtype=np.int64)
    inv[perm] = np.arange(r)
    return (counts.astype(np.int32), offsets.astype(np.int32),
            perm.astype(np.int32), inv.astype(np.int32))


def relu2(x):
    """``max(x, 0)^2`` [src module doc: relu^2]."""
    x = np.asarray(x, dtype=F64)
    return np.maximum(x, 0.0) ** 2


def expert_ffn(z, up_e, down_e):
    """One non-gated expert: ``down_e @ relu2(up_e @ z)`` on rows of ``z``."""
    h = relu2(np.asarray(z, dtype=F64) @ np.asarray(up_e, dtype=F64).T)
    return h @ np.asarray(down_e, dtype=F64).T


def layer_forward(hidden, weights: dict, cfg: dict, ids_override=None,
                  return_aux: bool = False):
    """Whole-layer forward [src module doc; NemotronMoeLayer::prefill; moe forward_prefill].

    ``hidden`` is ``[N, H]``. ``weights`` holds ``gamma, gate, up, down`` and
    optionally ``fc1, fc2`` (latent) and ``shared_up, shared_down`` (S > 0);
    each indexable array-like in any float dtype (``up[e]`` is read per
    expert, so a lazy per-expert accessor also works). ``cfg`` holds
    ``E, k, L, S, eps, scale``.

    ``ids_override`` is an optional ``(rows, ids_rows)`` pair: the listed
    tokens take the given expert ids (their weights are recomputed from this
    oracle's own scores). Parity tests use it only on tokens whose oracle
    score margin is under the id-comparison threshold.

    Returns ``(hidden_out, residual_out)`` float64, plus a dict of
    intermediates when ``return_aux``.
    """
    x = np.asarray(hidden, dtype=F64)
    n_tok = x.shape[0]
    E, k = int(cfg["E"]), int(cfg["k"])
    L = int(cfg.get("L", 0))
    S = int(cfg.get("S", 0))
    eps = float(cfg.get("eps", 1e-5))
    scale = float(cfg.get("scale", 1.0))
    check_config(E, k)

    residual_out = x.copy()                       # residual <- pre-norm hidden
    if n_tok == 0:
        out = (x.copy(), residual_out)
        return out + ({},) if return_aux else out

    normed = rms_norm(x, weights["gamma"], eps)   # 1. norm
    logits = gate_logits(normed, weights["gate"])  # 2. gate
    scores = sigmoid_scores(logits)               # 3. sigmoid (fp32)
    ids, margin = topk_select(scores, k)          # 4. top-k
    if ids_override is not None:
        rows, ids_rows = ids_override
        ids = ids.copy()
        ids[np.asarray(rows)] = np.asarray(ids_rows, dtype=np.int32)
    w = routing_weights(scores, ids, scale)       # 5. weights

    if L > 0:                                     # 6. latent input
        z = normed @ np.asarray(weights["fc1"], dtype=F64).T
    else:
        z = normed

    counts, offsets, perm, inv = sort_routes(ids, E)   # 7. sort
    D = z.shape[1]
    y = np.zeros((n_tok * k, D), dtype=F64)
    for e in range(E):                            # 8. experts, in sorted order
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        toks = perm[lo:hi] // k
        y[lo:hi] = expert_ffn(z[toks], weights["up"][e], weights["down"][e])

    o = np.zeros((n_tok, D), dtype=F64)           # 9. unpermute + weighted reduce
    for j in range(k):
        o += w[:, j:j + 1] * y[inv[np.arange(n_tok) * k + j]]
    if L > 0:
        o = o @ np.asarray(weights["fc2"], dtype=F64).T

    if S > 0:                                     # 10. shared expert
        sh = expert_ffn(normed, weights["shared_up"], weights["shared_down"])
    else:
        sh = np.zeros_like(x)

    hidden_out = residual_out + o + sh            # 11. residual add
    if not return_aux:
        return hidden_out, residual_out
    aux = dict(normed=normed, logits=logits, scores=scores, ids=ids,
               margin=margin, w=w, z=z, counts=counts, offsets=offsets,
               perm=perm, inv=inv, y=y, routed=o, shared=sh)
    return hidden_out, residual_out, aux
