"""Pins of the float64 oracle against closed forms, invariants and brute force.

Each test ties one oracle function to something other than the oracle itself,
so that a dropped term, a wrong sign or index, or a transposed operand fails.
"""

import itertools
import math

import numpy as np
import pytest

from oracle import moe_oracle as mo


def _rng(seed=0):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------- RMSNorm --

@pytest.mark.parametrize("c", [0.25, 1.0, -3.0, 17.5])
@pytest.mark.parametrize("H", [1, 8, 256])
def test_rms_norm_constant_rows_closed_form(c, H):
    eps = 1e-5
    x = np.full((1, H), c)
    n = mo.rms_norm(x, np.ones(H), eps)
    # mean(x^2) = c^2, so n = c / sqrt(c^2 + eps) for every entry.
    np.testing.assert_allclose(n, c / math.sqrt(c * c + eps), rtol=1e-14)


def test_rms_norm_worked_example():
    # x = (3, 4, 0, 0): mean of squares 25/4, rms 5/2; eps = 0.
    n = mo.rms_norm(np.array([[3.0, 4.0, 0.0, 0.0]]), np.ones(4), 0.0)
    np.testing.assert_allclose(n, [[1.2, 1.6, 0.0, 0.0]], rtol=1e-15, atol=0)
    # gamma scales each column independently.
    n = mo.rms_norm(np.array([[3.0, 4.0, 0.0, 0.0]]), np.array([2.0, -1.0, 5.0, 1.0]), 0.0)
    np.testing.assert_allclose(n, [[2.4, -1.6, 0.0, 0.0]], rtol=1e-15, atol=0)


def test_rms_norm_rows_independent_and_scale_invariant():
    x = _rng(1).normal(size=(5, 32))
    n1 = mo.rms_norm(x, np.ones(32), 0.0)
    n2 = mo.rms_norm(7.0 * x, np.ones(32), 0.0)
    np.testing.assert_allclose(n1, n2, rtol=1e-13)
    np.testing.assert_allclose(np.mean(n1 * n1, axis=1), 1.0, rtol=1e-13)


# -------------------------------------------------------------------- gate --

def test_gate_one_hot_rows_select_columns():
    rng = _rng(2)
    normed = rng.normal(size=(3, 10))
    cols = [7, 0, 3, 9]                       # E = 4 rows of a [E, H=10] gate
    wg = np.zeros((4, 10))
    wg[np.arange(4), cols] = 1.0
    logits = mo.gate_logits(normed, wg)
    assert logits.shape == (3, 4)
    np.testing.assert_array_equal(logits, normed[:, cols])


def test_gate_brute_force_loop():
    rng = _rng(3)
    normed = rng.normal(size=(2, 5))
    wg = rng.normal(size=(3, 5))
    logits = mo.gate_logits(normed, wg)
    for t in range(2):
        for e in range(3):
            ref = math.fsum(normed[t, i] * wg[e, i] for i in range(5))
            assert abs(logits[t, e] - ref) < 1e-13


# ----------------------------------------------------------------- sigmoid --

def test_sigmoid_closed_values():
    s = mo.sigmoid_scores(np.array([[0.0, 1e-30, -200.0, 200.0]]))
    assert s.dtype == np.float32
    assert s[0, 0] == np.float32(0.5)
    assert s[0, 1] == np.float32(0.5)
    assert s[0, 2] == 0.0
    assert s[0, 3] == 1.0


def test_sigmoid_matches_double_within_fp32_ulps():
    x = _rng(4).normal(size=(1, 4000)) * 6
    s = mo.sigmoid_scores(x).astype(np.float64)
    ref = 1.0 / (1.0 + np.exp(-x.astype(np.float32).astype(np.float64)))
    # Three fp32 roundings (exp, add, divide): relative error under 4 * 2^-24.
    assert np.all(np.abs(s - ref) <= 4 * 2.0 ** -24 * ref)
    # Symmetry: s(x) + s(-x) = 1 up to fp32 rounding.
    s_neg = mo.sigmoid_scores(-x).astype(np.float64)
    assert np.max(np.abs(s + s_neg - 1.0)) < 2e-7


# ------------------------------------------------------------------- top-k --

def _brute_topk(row, k):
    order = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))
    return order[:k]


@pytest.mark.parametrize("E,k", [(8, 2), (16, 5), (128, 6), (128, 8), (7, 7)])
def test_topk_brute_force_with_forced_ties(E, k):
    rng = _rng(E * 31 + k)
    # Scores on a coarse grid force many exact ties.
    s = (rng.integers(0, 5, size=(400, E)) / 8.0 + 0.25).astype(np.float32)
    ids, margin = mo.topk_select(s, k)
    for t in range(s.shape[0]):
        ref = _brute_topk(s[t], k)
        assert list(ids[t]) == ref
        if k < E:
            srt = sorted((float(v) for v in s[t]), reverse=True)
            assert margin[t] == srt[k - 1] - srt[k]
        else:
            assert margin[t] == np.inf


def test_topk_brute_force_subsets_small():
    # Exhaustive over all k-subsets: the chosen set maximizes the score sum and
    # among equal sums the lexicographically smallest index set is taken when
    # scores are distinct per set.
    rng = _rng(5)
    for _ in range(50):
        s = rng.permutation(6).astype(np.float32) / 10 + 0.05
        ids, _ = mo.topk_select(s[None, :], 3)
        best = max(itertools.combinations(range(6), 3), key=lambda c: sum(s[list(c)]))
        assert sorted(ids[0]) == sorted(best)
        assert list(s[ids[0]]) == sorted(s[ids[0]], reverse=True)


def test_topk_all_equal_and_k_equals_E():
    s = np.full((3, 8), 0.5, dtype=np.float32)
    ids, margin = mo.topk_select(s, 3)
    assert (ids == np.arange(3)).all()
    assert (margin == 0).all()
    ids, margin = mo.topk_select(s, 8)
    assert (ids == np.arange(8)).all()
    assert np.isinf(margin).all()


def test_rank_margin_brute_force():
    rng = _rng(21)
    s = (rng.integers(0, 40, size=(300, 10)) / 64.0).astype(np.float32)
    for k in (1, 3, 9, 10):
        m = mo.rank_margin(s, k)
        for t in range(s.shape[0]):
            top = sorted((float(v) for v in s[t]), reverse=True)[:k + 1]
            gaps = [top[i] - top[i + 1] for i in range(len(top) - 1)]
            assert m[t] == (min(gaps) if gaps else np.inf)


# ---------------------------------------------------------------- weights --

def test_routing_weights_invariants():
    rng = _rng(6)
    s = rng.uniform(0.01, 1, size=(50, 16)).astype(np.float32)
    ids, _ = mo.topk_select(s, 4)
    w = mo.routing_weights(s, ids, 1.0)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-14)
    w25 = mo.routing_weights(s, ids, 2.5)
    np.testing.assert_allclose(w25, 2.5 * w, rtol=1e-14)
    # Proportional to the selected scores.
    sel = np.take_along_axis(s.astype(np.float64), ids, 1)
    np.testing.assert_allclose(w / w[:, :1], sel / sel[:, :1], rtol=1e-13)
    eq = mo.routing_weights(np.full((2, 8), 0.5, np.float32), np.array([[0, 1, 2], [5, 6, 7]]))
    np.testing.assert_allclose(eq, 1 / 3, rtol=1e-15)
    zero = mo.routing_weights(np.zeros((1, 8), np.float32), np.array([[1, 2]]))
    np.testing.assert_allclose(zero, 0.5)


# ------------------------------------------------------------------- sort --

@pytest.mark.parametrize("N,E,k", [(1, 4, 1), (13, 8, 2), (64, 8, 2), (97, 128, 6), (5, 16, 16)])
def test_sort_routes_brute_force_and_invariants(N, E, k):
    rng = _rng(N * 7 + E)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(N)]).astype(np.int32)
    counts, offsets, perm, inv = mo.sort_routes(ids, E)
    flat = ids.reshape(-1)
    R = N * k
    ref = sorted(range(R), key=lambda r: (int(flat[r]), r))
    assert list(perm) == ref
    assert counts.sum() == R
    assert offsets[0] == 0 and offsets[-1] == R
    assert (np.diff(offsets) == counts).all()
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert (flat[seg] == e).all()
        assert (np.diff(seg) > 0).all()
    assert (perm[inv] == np.arange(R)).all()
    assert (inv[perm] == np.arange(R)).all()
    # Permute then unpermute gives each token's row back k times.
    X = rng.normal(size=(N, 3))
    Xp = X[perm // k]
    for j in range(k):
        back = Xp[inv[np.arange(N) * k + j]]
        np.testing.assert_array_equal(back, X)


def test_sort_routes_empty_experts_and_skew():
    ids = np.zeros((10, 1), dtype=np.int32)
    counts, offsets, perm, inv = mo.sort_routes(ids, 4)
    assert list(counts) == [10, 0, 0, 0]
    assert list(offsets) == [0, 10, 10, 10, 10]
    assert list(perm) == list(range(10))


# ---------------------------------------------------------------- experts --

def test_expert_identity_like_closed_form():
    rng = _rng(7)
    D = 12
    z = rng.normal(size=(9, D))
    U = np.concatenate([np.eye(D), -np.eye(D)])          # [2D, D]
    Dn = np.concatenate([np.eye(D), -np.eye(D)], axis=1)  # [D, 2D]
    y = mo.expert_ffn(z, U, Dn)
    # relu(z)^2 - relu(-z)^2 = z * |z|
    np.testing.assert_allclose(y, z * np.abs(z), rtol=1e-15)


def test_expert_ffn_scalar_loop():
    rng = _rng(8)
    z = rng.normal(size=(2, 4))
    U = rng.normal(size=(3, 4))
    Dn = rng.normal(size=(5, 3))
    y = mo.expert_ffn(z, U, Dn)
    for t in range(2):
        h = [max(math.fsum(U[i, d] * z[t, d] for d in range(4)), 0.0) ** 2 for i in range(3)]
        for o in range(5):
            ref = math.fsum(Dn[o, i] * h[i] for i in range(3))
            assert abs(y[t, o] - ref) < 1e-12 * max(1.0, abs(ref))


# ------------------------------------------------------------ whole layer --

def _tiny_weights(rng, H, E, I, S, L):
    D = L if L else H
    w = dict(gamma=1 + 0.1 * rng.normal(size=H), gate=rng.normal(size=(E, H)) / math.sqrt(H),
             up=rng.normal(size=(E, I, D)) / math.sqrt(D), down=rng.normal(size=(E, D, I)) / math.sqrt(I))
    if S:
        w["shared_up"] = rng.normal(size=(S, H)) / math.sqrt(H)
        w["shared_down"] = rng.normal(size=(H, S)) / math.sqrt(S)
    if L:
        w["fc1"] = rng.normal(size=(L, H)) / math.sqrt(H)
        w["fc2"] = rng.normal(size=(H, L)) / math.sqrt(L)
    return w


def _brute_layer(x, w, E, k, L, S, eps, scale):
    """Per-token pure-Python loops: no sort, no permutation, no matmul."""
    N, H = x.shape
    out = np.zeros_like(x)
    for t in range(N):
        row = [float(v) for v in x[t]]
        rms = math.sqrt(math.fsum(v * v for v in row) / H + eps)
        n = [row[i] / rms * float(w["gamma"][i]) for i in range(H)]
        logits = [math.fsum(float(w["gate"][e, i]) * n[i] for i in range(H)) for e in range(E)]
        s = [np.float32(1) / (np.float32(1) + np.exp(np.float32(-np.float32(l)))) for l in logits]
        chosen = sorted(range(E), key=lambda e: (-float(s[e]), e))[:k]
        tot = math.fsum(float(s[e]) for e in chosen)
        if L:
            z = [math.fsum(float(w["fc1"][a, i]) * n[i] for i in range(H)) for a in range(L)]
        else:
            z = n
        Dd = len(z)
        routed = [0.0] * Dd
        for e in chosen:
            we = float(s[e]) / tot * scale
            h = [max(math.fsum(float(w["up"][e, i, d]) * z[d] for d in range(Dd)), 0.0) ** 2
                 for i in range(w["up"].shape[1])]
            for d in range(Dd):
                routed[d] += we * math.fsum(float(w["down"][e, d, i]) * h[i] for i in range(len(h)))
        if L:
            routed = [math.fsum(float(w["fc2"][o, a]) * routed[a] for a in range(L)) for o in range(H)]
        sh = [0.0] * H
        if S:
            g = [max(math.fsum(float(w["shared_up"][j, i]) * n[i] for i in range(H)), 0.0) ** 2
                 for j in range(S)]
            sh = [math.fsum(float(w["shared_down"][o, j]) * g[j] for j in range(S)) for o in range(H)]
        out[t] = [row[i] + routed[i] + sh[i] for i in range(H)]
    return out


@pytest.mark.parametrize("H,E,k,I,S,L,scale", [
    (8, 4, 2, 6, 4, 0, 1.0),
    (8, 5, 3, 4, 0, 0, 2.5),
    (6, 4, 1, 5, 3, 3, 1.0),
    (8, 6, 6, 3, 2, 4, 1.0),
])
def test_layer_matches_per_token_brute_force(H, E, k, I, S, L, scale):
    rng = _rng(H * 100 + E * 10 + k)
    N = 9
    w = _tiny_weights(rng, H, E, I, S, L)
    x = rng.normal(size=(N, H))
    cfg = dict(E=E, k=k, L=L, S=S, eps=1e-5, scale=scale)
    out, res = mo.layer_forward(x, w, cfg)
    ref = _brute_layer(x, w, E, k, L, S, 1e-5, scale)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_array_equal(res, x)


def test_topk_equals_E_with_zero_gate_is_expert_mean():
    rng = _rng(9)
    H, E, I = 16, 5, 7
    w = _tiny_weights(rng, H, E, I, 0, 0)
    w["gate"] = np.zeros((E, H))
    x = rng.normal(size=(6, H))
    cfg = dict(E=E, k=E, L=0, S=0, eps=1e-5, scale=1.0)
    out, _ = mo.layer_forward(x, w, cfg)
    n = mo.rms_norm(x, w["gamma"], 1e-5)
    mean = sum(mo.expert_ffn(n, w["up"][e], w["down"][e]) for e in range(E)) / E
    np.testing.assert_allclose(out - x, mean, rtol=1e-12, atol=1e-14)


def test_identity_like_experts_reproduce_input():
    rng = _rng(10)
    H, E, k = 64, 8, 2
    U = np.concatenate([np.eye(H), -np.eye(H)])
    Dn = np.concatenate([np.eye(H), -np.eye(H)], axis=1)
    w = dict(gamma=np.ones(H), gate=rng.normal(size=(E, H)) / 8,
             up=np.stack([U] * E), down=np.stack([Dn] * E))
    x = rng.choice([-1.0, 1.0], size=(20, H))
    eps = 1e-5
    out, _ = mo.layer_forward(x, w, dict(E=E, k=k, L=0, S=0, eps=eps, scale=1.0))
    # normed = x / sqrt(1 + eps); each expert returns normed*|normed| = x / (1 + eps);
    # the weights sum to 1, so hidden_out = x + x / (1 + eps).
    np.testing.assert_allclose(out, x + x / (1 + eps), rtol=1e-14)


def test_single_expert_is_dense_relu2_ffn():
    rng = _rng(11)
    H, I = 12, 9
    w = _tiny_weights(rng, H, 1, I, 0, 0)
    x = rng.normal(size=(7, H))
    out, _ = mo.layer_forward(x, w, dict(E=1, k=1, L=0, S=0, eps=1e-5, scale=1.0))
    # Same FFN placed as the (dense, unrouted) shared expert instead.
    w2 = dict(gamma=w["gamma"], gate=np.zeros((1, H)), up=np.zeros((1, I, H)),
              down=np.zeros((1, H, I)), shared_up=w["up"][0], shared_down=w["down"][0])
    out2, _ = mo.layer_forward(x, w2, dict(E=1, k=1, L=0, S=I, eps=1e-5, scale=1.0))
    np.testing.assert_allclose(out, out2, rtol=1e-13)


def test_latent_with_identity_projections_equals_direct():
    rng = _rng(12)
    H, E, k, I, S = 16, 6, 2, 10, 8
    w = _tiny_weights(rng, H, E, I, S, 0)
    x = rng.normal(size=(11, H))
    out_d, _ = mo.layer_forward(x, w, dict(E=E, k=k, L=0, S=S))
    wl = dict(w, fc1=np.eye(H), fc2=np.eye(H))
    out_l, _ = mo.layer_forward(x, wl, dict(E=E, k=k, L=H, S=S))
    np.testing.assert_allclose(out_l, out_d, rtol=1e-13)


def test_row_split_invariance_and_permutation_equivariance():
    rng = _rng(13)
    H, E, k, I, S = 16, 8, 3, 12, 10
    w = _tiny_weights(rng, H, E, I, S, 0)
    cfg = dict(E=E, k=k, L=0, S=S)
    x = rng.normal(size=(17, H))
    full, _ = mo.layer_forward(x, w, cfg)
    a, _ = mo.layer_forward(x[:5], w, cfg)
    b, _ = mo.layer_forward(x[5:], w, cfg)
    np.testing.assert_allclose(np.concatenate([a, b]), full, rtol=1e-13)
    p = rng.permutation(17)
    xp, _ = mo.layer_forward(x[p], w, cfg)
    np.testing.assert_allclose(xp, full[p], rtol=1e-13)


def test_zero_tokens_and_config_errors():
    w = _tiny_weights(_rng(14), 8, 4, 4, 0, 0)
    out, res = mo.layer_forward(np.zeros((0, 8)), w, dict(E=4, k=2))
    assert out.shape == (0, 8) and res.shape == (0, 8)
    for E, k in [(4, 0), (4, 5), (600, 2), (32, 17)]:
        with pytest.raises(mo.ConfigError):
            mo.check_config(E, k)


def test_ids_override_forces_routes():
    rng = _rng(15)
    H, E, k, I = 8, 6, 2, 5
    w = _tiny_weights(rng, H, E, I, 0, 0)
    x = rng.normal(size=(4, H))
    cfg = dict(E=E, k=k)
    _, _, aux = mo.layer_forward(x, w, cfg, return_aux=True)
    forced = np.array([[5, 4]], dtype=np.int32)
    out, _, aux2 = mo.layer_forward(x, w, cfg, ids_override=([2], forced), return_aux=True)
    assert list(aux2["ids"][2]) == [5, 4]
    np.testing.assert_array_equal(aux2["ids"][[0, 1, 3]], aux["ids"][[0, 1, 3]])
    n = mo.rms_norm(x[2:3], w["gamma"], 1e-5)
    s = aux["scores"][2].astype(np.float64)
    w5, w4 = s[5] / (s[5] + s[4]), s[4] / (s[5] + s[4])
    ref = x[2] + w5 * mo.expert_ffn(n, w["up"][5], w["down"][5])[0] \
        + w4 * mo.expert_ffn(n, w["up"][4], w["down"][4])[0]
    np.testing.assert_allclose(out[2], ref, rtol=1e-13)
