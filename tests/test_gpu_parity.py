"""GPU parity of the HIP path against the float64 oracle (through the C ABI).

Bars: sort stage and quantizer bit-exact; top-k ids exact wherever the
oracle's rank margin is >= 1e-3; layer outputs within relative Frobenius
1e-4 (fp32), 1e-2 (bf16), 3e-2 (NVFP4) on both hidden_out and the MoE delta
hidden_out - residual.
"""

import numpy as np
import pytest
import torch

from mixture_experts_ffn_gate_amd import workloads as wlm
from oracle import moe_oracle as mo
from oracle import nvfp4 as onv

import parity_utils as pu

pytestmark = pytest.mark.gpu
f32np = wlm.to_numpy_f32


@pytest.fixture(scope="module")
def ml():
    from mixture_experts_ffn_gate_amd import moe_layer
    torch.cuda.init()
    return moe_layer


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def run_layer(ml, wl, n, seed=0, W=None, hidden=None, max_tokens=None):
    _announce(f"{wl.name} H={wl.H} E={wl.E} k={wl.k} I={wl.I} S={wl.S} L={wl.L} N={n} seed={seed}")
    if W is None:
        W = wlm.make_weights(wl, seed, "cuda")
    if hidden is None:
        hidden, residual = wlm.make_hidden(wl, n, seed, "cuda", gate=W["gate"])
    else:
        residual = torch.randn_like(hidden)
    x = f32np(hidden)
    layer = ml.layer_from_workload(wl, W, max_tokens=max_tokens or n)
    layer.forward(hidden, residual)
    ids = torch.empty(n, wl.k, dtype=torch.int32, device="cuda")
    layer.debug_read("ids", ids)
    torch.cuda.synchronize()
    return dict(layer=layer, W=W, x=x, out=f32np(hidden), res=f32np(residual),
                ids=ids.cpu().numpy(), hidden=hidden, residual=residual)


# ------------------------------------------------------------------ stages --

@pytest.mark.parametrize("n,E,k,ties", [(1000, 128, 6, False), (257, 8, 2, False),
                                        (300, 512, 16, False), (123, 200, 7, False),
                                        (500, 64, 4, True), (64, 16, 16, True)])
def test_topk_stage(ml, n, E, k, ties):
    _announce(f"topk n={n} E={E} k={k} ties={ties}")
    g = torch.Generator().manual_seed(n * 7 + E)
    logits = torch.randn(n, E, generator=g)
    if ties:
        logits = torch.round(logits * 2) / 2
    ids, w = ml.topk_sigmoid(logits.cuda(), k, scale=1.0)
    ids, w = ids.cpu().numpy(), w.cpu().numpy()
    scores = mo.sigmoid_scores(logits.numpy())
    ref_ids, tmargin = mo.topk_select(scores, k)
    margin = mo.rank_margin(scores, k)
    pu.check_ids(ids, ref_ids, margin, tmargin, max_loose_frac=1.0 if ties else 0.05)
    same = np.all(ids == ref_ids, axis=1)
    ref_w = mo.routing_weights(scores, ref_ids, 1.0)
    np.testing.assert_allclose(w[same], ref_w[same], rtol=2e-6, atol=1e-7)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-5)
    if ties:
        # Exact ties in fp32 scores: both sides break them by the lower index.
        exact = np.all(ids == ref_ids, axis=1).mean()
        assert exact > 0.99


def test_topk_scale_and_ties_lowest_index(ml):
    logits = torch.zeros(5, 32)
    ids, w = ml.topk_sigmoid(logits.cuda(), 4, scale=2.5)
    assert (ids.cpu().numpy() == np.arange(4)).all()
    np.testing.assert_allclose(w.cpu().numpy(), 2.5 / 4, rtol=1e-6)


@pytest.mark.parametrize("n,k,E,mode", [(1024, 6, 128, "uniform"), (4096, 6, 128, "uniform"),
                                        (77, 4, 16, "uniform"), (3000, 8, 128, "one"),
                                        (513, 2, 512, "sparse"), (1, 1, 8, "uniform"),
                                        (2048, 16, 64, "uniform")])
def test_route_sort_stage_bit_exact(ml, n, k, E, mode):
    _announce(f"route_sort n={n} k={k} E={E} mode={mode}")
    rng = np.random.default_rng(n + k + E)
    if mode == "one":
        # Every token routes to expert 0 plus k-1 experts drawn from a few.
        ids = np.stack([np.concatenate([[0], rng.choice(np.arange(1, k + 3), k - 1,
                                                        replace=False)]) for _ in range(n)])
    elif mode == "sparse":
        ids = np.stack([rng.choice(np.arange(0, E, 37), k, replace=False) for _ in range(n)])
    else:
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(n)])
    ids = ids.astype(np.int32)
    c, o, p, i = ml.route_sort(torch.from_numpy(ids).cuda(), E)
    rc, ro, rp, ri = mo.sort_routes(ids, E)
    np.testing.assert_array_equal(c.cpu().numpy(), rc)
    np.testing.assert_array_equal(o.cpu().numpy(), ro)
    np.testing.assert_array_equal(p.cpu().numpy(), rp)
    np.testing.assert_array_equal(i.cpu().numpy(), ri)


@pytest.mark.parametrize("G,rows,cols", [(3, 64, 256), (2, 48, 2688), (1, 16, 16)])
def test_nvfp4_quantize_stage_bit_exact(ml, G, rows, cols):
    _announce(f"nvfp4_quantize G={G} rows={rows} cols={cols}")
    g = torch.Generator().manual_seed(G * rows + cols)
    w = torch.randn(G, rows, cols, generator=g) / np.sqrt(cols)
    # Exact E2M1 / E4M3 rounding ties: a block whose entries land on midpoints.
    w[0, 0, :16] = torch.tensor([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0,
                                 -0.25, -0.75, -2.5, -5.0, 0.0, -0.0, 4.0, -6.0]) * 0.01
    if G > 1:
        w[1, 1] = 0.0
    packed, scales, scale2 = ml.nvfp4_quantize(w.cuda())
    rp, rs, r2 = onv.quantize_stack(w.numpy())
    np.testing.assert_array_equal(scale2.cpu().numpy(), r2)
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)
    np.testing.assert_array_equal(packed.cpu().numpy(), rp)


# ------------------------------------------------------------- whole layer --

SMALL = {
    "direct_ragged": wlm.Workload("direct_ragged", H=512, E=16, k=4, I=192, S=320, L=0, N=77),
    "latent_ragged": wlm.Workload("latent_ragged", H=512, E=16, k=4, I=256, S=320, L=192, N=130),
    "no_shared": wlm.Workload("no_shared", H=256, E=8, k=2, I=128, S=0, L=0, N=200),
    "topk_all": wlm.Workload("topk_all", H=256, E=8, k=8, I=64, S=64, L=0, N=40),
    "many_rows": wlm.Workload("many_rows", H=256, E=4, k=2, I=128, S=128, L=0, N=700),
    # E not a multiple of 16 (gate padded with zero rows), H not of 128
    "odd_experts": wlm.Workload("odd_experts", H=320, E=20, k=3, I=128, S=64, L=0, N=90),
    # 97-168 rows per expert: 192-row tiles (12 row blocks, operand reads in
    # two batches, 2-stage ring), one per expert or a second partial one
    "rows_192": wlm.Workload("rows_192", H=512, E=8, k=3, I=512, S=128, L=0, N=400),
    "latent_192": wlm.Workload("latent_192", H=512, E=8, k=4, I=256, S=256, L=192, N=300),
}


def _cmp(wl, Wn, r, case, rows=None, tol=None):
    e = pu.compare_layer(wl, Wn, r["x"], r["out"], r["res"], r["ids"], rows=rows, tol=tol,
                         case=case)
    print(f"errors {case}: out {e[0]:.3e} delta {e[1]:.3e}", flush=True)
    return e


def test_tiny_f32_full(ml):
    wl = wlm.WORKLOADS["tiny_direct_f32"]
    r = run_layer(ml, wl, wl.N)
    Wn = pu.oracle_weights(r["W"])
    _cmp(wl, Wn, r, "tiny_direct_f32 N=64")


@pytest.mark.parametrize("name", list(SMALL))
def test_small_bf16(ml, name):
    wl = SMALL[name]
    r = run_layer(ml, wl, wl.N, seed=5)
    Wn = pu.oracle_weights(r["W"])
    _cmp(wl, Wn, r, f"{name} N={wl.N}")


def test_decode_routing_max_routes(ml):
    # The decode routing kernel at its largest shape: 16 tokens x top-16 = 256
    # routes over 512 experts (32 expert tiles x 2 hidden slices), every id and
    # the whole sort stage checked.
    wl = wlm.Workload("decode_max", H=512, E=512, k=16, I=64, S=64, L=0, N=16)
    r = run_layer(ml, wl, 16, seed=16)
    R = 16 * 16
    bufs = {nm: torch.empty(sz, dtype=torch.int32, device="cuda")
            for nm, sz in (("counts", wl.E), ("offsets", wl.E + 1), ("perm", R), ("inv", R))}
    for nm, t in bufs.items():
        r["layer"].debug_read(nm, t)
    torch.cuda.synchronize()
    rc, ro, rp, ri = mo.sort_routes(r["ids"], wl.E)
    for nm, ref in zip(("counts", "offsets", "perm", "inv"), (rc, ro, rp, ri)):
        np.testing.assert_array_equal(bufs[nm].cpu().numpy(), ref, err_msg=nm)
    _cmp(wl, pu.oracle_weights(r["W"]), r, "decode_max N=16")


@pytest.mark.parametrize("n", [1, 7])
def test_odd_experts_decode_sizes(ml, n):
    # decode-size routing kernel with a partial last expert tile
    wl = SMALL["odd_experts"]
    r = run_layer(ml, wl, n, seed=12, max_tokens=32)
    Wn = pu.oracle_weights(r["W"])
    _cmp(wl, Wn, r, f"odd_experts N={n}")


@pytest.mark.parametrize("n", [1, 2, 3, 16, 17, 64])
def test_small_bf16_token_counts(ml, n):
    wl = SMALL["direct_ragged"]
    r = run_layer(ml, wl, n, seed=11, max_tokens=128)
    Wn = pu.oracle_weights(r["W"])
    _cmp(wl, Wn, r, f"direct_ragged N={n}")


@pytest.mark.parametrize("n", [1, 5, 16])
def test_latent_decode_arm(ml, n):
    # LatentMoE at decode sizes: fc1 GEMV, routed GEMVs in latent space, the
    # latent reduce into o, and the fc2 GEMV with residual + shared added.
    wl = SMALL["latent_ragged"]
    r = run_layer(ml, wl, n, seed=13, max_tokens=32)
    Wn = pu.oracle_weights(r["W"])
    _cmp(wl, Wn, r, f"latent_ragged N={n}")


def test_latent_decode_arm_nvfp4(ml):
    wl = NVFP4_SMALL["nvfp4_latent"]
    r = run_layer(ml, wl, 3, seed=14, max_tokens=16)
    Wn = pu.oracle_weights(r["W"], nvfp4=True)
    _cmp(wl, Wn, r, "nvfp4_latent N=3")


def test_skewed_routing_many_row_blocks(ml):
    # Nearly identical rows route to the same experts: one expert gets every
    # token, so its rows span several row blocks of the grouped GEMMs.
    wl = wlm.Workload("skewed", H=256, E=8, k=2, I=128, S=64, L=0, N=600)
    W = wlm.make_weights(wl, 3, "cuda")
    base = torch.randn(1, wl.H, device="cuda")
    hidden = (base + 0.05 * torch.randn(wl.N, wl.H, device="cuda")).to(torch.bfloat16)
    r = run_layer(ml, wl, wl.N, W=W, hidden=hidden)
    assert np.bincount(r["ids"].ravel(), minlength=wl.E).max() > 300
    Wn = pu.oracle_weights(W)
    _cmp(wl, Wn, r, "skewed N=600")


@pytest.mark.parametrize("name", ["direct_ragged", "multiblock_sort", "multiblock_512"])
def test_sort_stage_bit_exact_inside_forward(ml, name):
    # Large route counts take the multi-block sort (2048 routes per block).
    wl = {"direct_ragged": SMALL["direct_ragged"],
          "multiblock_sort": wlm.Workload("mb", H=256, E=32, k=8, I=64, S=0, L=0, N=1000),
          "multiblock_512": wlm.Workload("mb512", H=256, E=512, k=16, I=64, S=0, L=0, N=301),
          }[name]
    r = run_layer(ml, wl, wl.N, seed=2)
    L = r["layer"]
    R = wl.N * wl.k
    bufs = {nm: torch.empty(sz, dtype=torch.int32, device="cuda")
            for nm, sz in (("counts", wl.E), ("offsets", wl.E + 1), ("perm", R), ("inv", R))}
    for nm, t in bufs.items():
        L.debug_read(nm, t)
    torch.cuda.synchronize()
    rc, ro, rp, ri = mo.sort_routes(r["ids"], wl.E)
    for nm, ref in zip(("counts", "offsets", "perm", "inv"), (rc, ro, rp, ri)):
        np.testing.assert_array_equal(bufs[nm].cpu().numpy(), ref, err_msg=nm)


WIDE_H = {
    # 16 rows of H = 5120 or 8192 exceed the LDS staging of the batched
    # norm+gate kernel: these take norm_gate_mfma_kernel (and, at N <= 16, the
    # decode routing kernel with more than one load round per wave).
    "hidden5120": wlm.Workload("hidden5120", H=5120, E=16, k=2, I=128, S=128, L=0, N=40),
    "hidden8192": wlm.Workload("hidden8192", H=8192, E=24, k=3, I=128, S=64, L=0, N=20),
    "hidden5120_latent": wlm.Workload("hidden5120_latent", H=5120, E=16, k=2, I=128, S=128,
                                      L=256, N=70),
}


def _check_logits_normed(r, wl, n):
    logits = torch.empty(n, wl.E, dtype=torch.float32, device="cuda")
    normed = torch.empty(n, wl.H, dtype=torch.bfloat16, device="cuda")
    r["layer"].debug_read("logits", logits)
    r["layer"].debug_read("normed", normed)
    torch.cuda.synchronize()
    Wn = pu.oracle_weights(r["W"])
    n64 = mo.rms_norm(r["x"], Wn["gamma"], wl.eps)
    ref = mo.gate_logits(n64, Wn["gate"])
    assert np.max(np.abs(logits.cpu().numpy() - ref)) < 2e-4
    # normed is the bf16 rounding of the fp32 value: within one bf16 ulp.
    nb = f32np(normed)
    assert np.all(np.abs(nb - n64) <= 2.0 ** -8 * np.abs(n64) * (1 + 1e-5) + 1e-30)
    return Wn


@pytest.mark.parametrize("name", ["direct_ragged", "latent_ragged"])
def test_gate_logits_and_normed_inside_forward(ml, name):
    # The gate is fed the fp32 normed vector (split into bf16 hi + lo parts):
    # logits agree with the float64 oracle far below the top-k margin bar.
    wl = SMALL[name]
    r = run_layer(ml, wl, wl.N, seed=9)
    _check_logits_normed(r, wl, wl.N)


@pytest.mark.parametrize("name,n", [("hidden5120", 40), ("hidden5120", 5), ("hidden8192", 20),
                                    ("hidden8192", 16), ("hidden5120_latent", 70)])
def test_wide_hidden(ml, name, n):
    wl = WIDE_H[name]
    r = run_layer(ml, wl, n, seed=15, max_tokens=max(n, 16))
    Wn = _check_logits_normed(r, wl, n)
    _cmp(wl, Wn, r, f"{name} N={n}")


def test_residual_input_ignored_and_deterministic(ml):
    wl = SMALL["direct_ragged"]
    W = wlm.make_weights(wl, 4, "cuda")
    h0, _ = wlm.make_hidden(wl, wl.N, 4, "cuda")
    layer = ml.layer_from_workload(wl, W)
    outs = []
    for garbage in (0.0, 1e30):
        h = h0.clone()
        res = torch.full_like(h, garbage)
        layer.forward(h, res)
        outs.append((h.clone(), res.clone()))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], h0) and torch.equal(outs[1][1], h0)


@pytest.mark.parametrize("name", ["no_shared", "direct_ragged", "topk_all"])
def test_one_token_fused_down_reduce(ml, name):
    # One token runs the down projection, weighted reduce, shared expert and
    # residual add as one launch (per-wave LDS partials summed in wave order):
    # without a shared expert, with one, and with more items (8 routes + 1
    # shared split) than waves. Run twice on the same inputs: bit-identical.
    wl = SMALL[name]
    r = run_layer(ml, wl, 1, seed=21, max_tokens=8)
    _cmp(wl, pu.oracle_weights(r["W"]), r, f"{name} N=1 (fused down + reduce)")
    h = r["hidden"].clone()
    h.copy_(torch.from_numpy(r["x"]).to(h.dtype))
    r["layer"].forward(h, torch.empty_like(h))
    torch.cuda.synchronize()
    assert np.array_equal(f32np(h), r["out"])


def test_errors_and_zero_tokens(ml):
    wl = SMALL["no_shared"]
    W = wlm.make_weights(wl, 0, "cuda")
    layer = ml.layer_from_workload(wl, W, max_tokens=8)
    h = torch.randn(9, wl.H, device="cuda").to(torch.bfloat16)
    r = torch.empty_like(h)
    with pytest.raises(ml.MoeError) as ei:
        layer.forward(h, r)
    assert ei.value.code == ml.MOE_ERR_TOO_MANY_TOKENS
    h2 = h[:4].clone()
    layer.forward(h2, r[:4].contiguous(), num_tokens=0)
    torch.cuda.synchronize()
    assert torch.equal(h2, h[:4])


def test_create_out_of_memory(ml):
    # A workspace far beyond HBM: create must fail with MOE_ERR_OOM, free what
    # it allocated, and leave the device usable.
    wl = wlm.Workload("oom", H=8192, E=8, k=2, I=64, S=64, L=0, N=1)
    W = wlm.make_weights(wl, 0, "cuda")
    with pytest.raises(ml.MoeError) as ei:
        ml.layer_from_workload(wl, W, max_tokens=50_000_000)
    assert ei.value.code == ml.MOE_ERR_OOM
    small = wl.with_(N=4)
    r = run_layer(ml, small, 4, W=W)
    _cmp(small, pu.oracle_weights(W), r, "after OOM N=4")


def _capture_and_replay(ml, wl, n, seed):
    # A forward enqueues no host synchronization, allocation or readback, so
    # it can be captured; replays (with eager work between them) must match
    # the eager run bit for bit, and the oracle within the bar.
    W = wlm.make_weights(wl, seed, "cuda")
    h0, _ = wlm.make_hidden(wl, n, seed, "cuda")
    layer = ml.layer_from_workload(wl, W, max_tokens=n)
    eager = h0.clone()
    res = torch.empty_like(eager)
    layer.forward(eager, res)
    torch.cuda.synchronize()
    hbuf = h0.clone()
    rbuf = torch.empty_like(hbuf)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            layer.forward(hbuf, rbuf, stream=s)
    torch.cuda.synchronize()
    Wn = pu.oracle_weights(W)
    x = f32np(h0)
    for rep in range(3):
        hbuf.copy_(h0)
        rbuf.fill_(7.0)
        junk = torch.randn(1000, device="cuda").sum()  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(hbuf, eager), f"replay {rep}"
        assert torch.equal(rbuf, h0)
        ids = torch.empty(n, wl.k, dtype=torch.int32, device="cuda")
        layer.debug_read("ids", ids)
        torch.cuda.synchronize()
        r = dict(x=x, out=f32np(hbuf), res=f32np(rbuf), ids=ids.cpu().numpy())
        _cmp(wl, Wn, r, f"{wl.name} N={n} graph replay {rep}")
        del junk


def test_graph_capture_replays_match_eager(ml):
    wl = SMALL["latent_ragged"]
    _capture_and_replay(ml, wl, wl.N, 6)


def test_graph_capture_dynamic_item_order(ml):
    # Experts of several row tiles: the grouped launches take their items
    # from per-XCD counters that each launch re-arms; every replay must
    # still match the eager run bit for bit.
    wl = SMALL["many_rows"]
    _capture_and_replay(ml, wl, wl.N, 9)


@pytest.mark.parametrize("name,n", [("direct_ragged", 5), ("latent_ragged", 3), ("direct_ragged", 1)])
def test_graph_capture_decode_arm(ml, name, n):
    # The decode-sized arm (one routing kernel whose last block re-arms a
    # device counter, GEMV launches; at one token the fused down projection
    # and reduce) captured whole.
    _capture_and_replay(ml, SMALL[name], n, 9)


# ------------------------------------------------ full sizes (bench shapes) --

def _sample_rows(n, count, seed):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(n, size=min(n, count), replace=False).tolist()) | {0, n - 1}
    return np.array(sorted(rows))


@pytest.mark.slow
@pytest.mark.parametrize("name", ["nemotron_direct_bf16", "latent_bf16"])
def test_full_size_sampled(ml, name):
    wl = wlm.WORKLOADS[name]
    r = run_layer(ml, wl, wl.N, seed=0)
    Wn = pu.oracle_weights(r["W"], lazy_experts=True)
    # Every token's ids (gate on all rows is cheap), then the outputs of rows
    # whose routes touch every expert, plus random rows.
    ref_ids, rmargin, _, tmargin = pu.oracle_routing(r["x"], Wn, wl)
    pu.check_ids(r["ids"], ref_ids, rmargin, tmargin)
    rows = pu.rows_covering_experts(r["ids"], wl.E, extra=160, seed=1)
    assert len(np.unique(r["ids"][rows])) == len(np.unique(r["ids"]))
    _cmp(wl, Wn, r, f"{name} N={wl.N} ({len(rows)} rows)", rows=rows)


@pytest.mark.slow
def test_full_size_direct_4096_sampled(ml):
    # The direct shapes at 4096 tokens: experts of about 192 rows (two row
    # tiles, dynamic item order) on 128 x 384 grouped tiles, and the shared
    # down projection on 128 x 384 dense tiles. Every id, the rows covering
    # every expert plus random rows.
    wl = wlm.WORKLOADS["nemotron_direct_bf16"]
    n = 4096
    r = run_layer(ml, wl, n, seed=4, max_tokens=n)
    Wn = pu.oracle_weights(r["W"], lazy_experts=True)
    ref_ids, rmargin, _, tmargin = pu.oracle_routing(r["x"], Wn, wl)
    pu.check_ids(r["ids"], ref_ids, rmargin, tmargin)
    rows = pu.rows_covering_experts(r["ids"], wl.E, extra=64, seed=4)
    assert len(np.unique(r["ids"][rows])) == len(np.unique(r["ids"]))
    _cmp(wl, Wn, r, f"nemotron_direct_bf16 N={n} ({len(rows)} rows)", rows=rows)


def test_wide_tiles_sampled(ml):
    # 128-row tiles with 8 waves per workgroup (grouped up: 1024 rows per
    # expert; shared up: 32 row tiles x 16 feature tiles) next to 4-wave
    # ones (the 256-wide down projections). All ids, sampled output rows.
    wl = wlm.Workload("wide_tiles", H=256, E=8, k=2, I=2048, S=4096, L=0, N=4096)
    r = run_layer(ml, wl, wl.N, seed=5)
    Wn = pu.oracle_weights(r["W"])
    ref_ids, rmargin, _, tmargin = pu.oracle_routing(r["x"], Wn, wl)
    pu.check_ids(r["ids"], ref_ids, rmargin, tmargin)
    rows = _sample_rows(wl.N, 48, 2)
    _cmp(wl, Wn, r, "wide_tiles N=4096 (sampled)", rows=rows)


def test_grouped_wide48_sampled(ml):
    # Grouped bf16 launches over experts of several row tiles (about 1024 rows
    # each, ragged last tiles, dynamic item order) on 48-feature waves:
    # 1152 = 3 x 384 for both projections, 640 items each.
    wl = wlm.Workload("grouped_wide48", H=1152, E=16, k=4, I=1152, S=256, L=0, N=4096)
    r = run_layer(ml, wl, wl.N, seed=12)
    Wn = pu.oracle_weights(r["W"])
    ref_ids, rmargin, _, tmargin = pu.oracle_routing(r["x"], Wn, wl)
    pu.check_ids(r["ids"], ref_ids, rmargin, tmargin)
    rows = pu.rows_covering_experts(r["ids"], wl.E, extra=48, seed=3)
    _cmp(wl, Wn, r, "grouped_wide48 N=4096 (sampled)", rows=rows)


def test_dense_wide48_sampled(ml):
    # Dense bf16 launches on 48-feature waves (128 x 384 tiles) where that
    # needs fewer item rounds: 48 row tiles x 1344 features (3.5 tiles of 384,
    # the last one half dead) for the shared up (relu^2), the shared down
    # (store) and fc2 (residual + shared epilogue); ragged last row tile.
    wl = wlm.Workload("dense_wide48", H=1344, E=8, k=2, I=128, S=1344, L=256, N=6100)
    r = run_layer(ml, wl, wl.N, seed=11)
    Wn = pu.oracle_weights(r["W"])
    ref_ids, rmargin, _, tmargin = pu.oracle_routing(r["x"], Wn, wl)
    pu.check_ids(r["ids"], ref_ids, rmargin, tmargin)
    rows = np.union1d(_sample_rows(wl.N, 48, 4), np.arange(wl.N - 84, wl.N))
    _cmp(wl, Wn, r, "dense_wide48 N=6100 (sampled)", rows=rows)


def test_seven_wave_tiles(ml):
    # Grouped down projection 1344 = 4 x 336 wide with one 128-row tile per
    # expert (64 rows each, 128 experts): 7-wave workgroups of 48-feature
    # waves (128 x 336 tiles), 2-stage ring. Every token's ids; the outputs of
    # rows covering every expert plus random rows.
    wl = wlm.Workload("seven_wave", H=1344, E=128, k=4, I=256, S=128, L=0, N=2048)
    r = run_layer(ml, wl, wl.N, seed=13)
    Wn = pu.oracle_weights(r["W"])
    ref_ids, rmargin, _, tmargin = pu.oracle_routing(r["x"], Wn, wl)
    pu.check_ids(r["ids"], ref_ids, rmargin, tmargin)
    rows = pu.rows_covering_experts(r["ids"], wl.E, extra=96, seed=5)
    _cmp(wl, Wn, r, "seven_wave N=2048 (sampled)", rows=rows)


def test_six_wave_tiles(ml):
    # Grouped down projection 1152 = 6 x 192 wide (4.5 tiles of 256; 336 does
    # not divide it) with one 128-row tile per expert (64 rows each, 128
    # experts): 6-wave workgroups, 4 k-steps (the 3-stage ring's tail only).
    # Every token compared.
    wl = wlm.Workload("six_wave", H=1152, E=128, k=4, I=256, S=128, L=0, N=2048)
    r = run_layer(ml, wl, wl.N, seed=10)
    Wn = pu.oracle_weights(r["W"])
    _cmp(wl, Wn, r, "six_wave N=2048")


NVFP4_SMALL = {
    "nvfp4_direct": wlm.Workload("nvfp4_direct_s", H=512, E=16, k=4, I=192, S=320, L=0, N=150,
                                 expert_dtype="nvfp4"),
    "nvfp4_latent": wlm.Workload("nvfp4_latent_s", H=512, E=8, k=2, I=256, S=256, L=128, N=70,
                                 expert_dtype="nvfp4"),
    "nvfp4_many_rows": wlm.Workload("nvfp4_many_rows", H=256, E=4, k=2, I=128, S=0, L=0, N=600,
                                    expert_dtype="nvfp4"),
    # 129-168 rows per expert: 192-row tiles (12 row blocks, operand reads in
    # two batches, 2-stage ring), one per expert or a second partial one
    "nvfp4_192rows": wlm.Workload("nvfp4_192rows", H=512, E=8, k=3, I=512, S=128, L=0, N=400,
                                  expert_dtype="nvfp4"),
    # 512 items of 128 x 256: the up projection takes 48-feature waves (128 x
    # 384 tiles; 2048 = 5.33 tiles, the last one partly dead), batched operand
    # reads, two row tiles per expert in dynamic item order
    "nvfp4_wide48": wlm.Workload("nvfp4_wide48", H=256, E=32, k=4, I=2048, S=256, L=0, N=2048,
                                 expert_dtype="nvfp4"),
}


@pytest.mark.parametrize("name", list(NVFP4_SMALL))
def test_small_nvfp4(ml, name):
    wl = NVFP4_SMALL[name]
    r = run_layer(ml, wl, wl.N, seed=7)
    Wn = pu.oracle_weights(r["W"], nvfp4=True)
    _cmp(wl, Wn, r, f"{name} N={wl.N}")


@pytest.mark.parametrize("n", [1, 5, 16])
def test_small_nvfp4_decode_sizes(ml, n):
    wl = NVFP4_SMALL["nvfp4_direct"]
    r = run_layer(ml, wl, n, seed=8, max_tokens=64)
    Wn = pu.oracle_weights(r["W"], nvfp4=True)
    _cmp(wl, Wn, r, f"nvfp4_direct N={n}")


def test_wide_tiles_nvfp4_sampled(ml):
    # NVFP4 weights on 128-row tiles with 8 waves per workgroup and the
    # 3-stage ring (grouped up: 512 rows per expert, 16 feature tiles of 256)
    # next to 4-wave ones (grouped down, shared). All ids, sampled output rows.
    wl = wlm.Workload("wide_tiles_nvfp4", H=512, E=8, k=2, I=4096, S=512, L=0, N=2048,
                      expert_dtype="nvfp4")
    r = run_layer(ml, wl, wl.N, seed=9)
    Wn = pu.oracle_weights(r["W"], nvfp4=True)
    ref_ids, rmargin, _, tmargin = pu.oracle_routing(r["x"], Wn, wl)
    pu.check_ids(r["ids"], ref_ids, rmargin, tmargin)
    rows = _sample_rows(wl.N, 48, 3)
    _cmp(wl, Wn, r, "wide_tiles_nvfp4 N=2048 (sampled)", rows=rows)


@pytest.mark.slow
def test_full_size_nvfp4_sampled(ml):
    wl = wlm.WORKLOADS["nvfp4_direct"]
    r = run_layer(ml, wl, wl.N, seed=0)
    Wn = pu.oracle_weights(r["W"], nvfp4=True, lazy_experts=True)
    ref_ids, rmargin, _, tmargin = pu.oracle_routing(r["x"], Wn, wl)
    pu.check_ids(r["ids"], ref_ids, rmargin, tmargin)
    rows = pu.rows_covering_experts(r["ids"], wl.E, extra=60, seed=2)
    touched = np.unique(r["ids"][rows])
    assert len(touched) == len(np.unique(r["ids"]))
    # The oracle's own quantization of every touched expert, once, on a pool.
    Wn["up"].prepare(touched)
    Wn["down"].prepare(touched)
    _cmp(wl, Wn, r, f"nvfp4_direct N={wl.N} ({len(rows)} rows)", rows=rows)


@pytest.mark.parametrize("n", wlm.DECODE_NS)
def test_decode_zipf_full(ml, n):
    wl = wlm.WORKLOADS["decode_zipf_bf16"]
    r = run_layer(ml, wl, n, seed=0)
    Wn = pu.oracle_weights(r["W"], lazy_experts=True)
    _cmp(wl, Wn, r, f"decode_zipf_bf16 N={n}")
