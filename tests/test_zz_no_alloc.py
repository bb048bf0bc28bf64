"""The allocation-free route sort (moe_route_sort_static, static device
scratch) against moe_route_sort and the oracle, through the C ABI."""

import numpy as np
import pytest
import torch

from oracle import moe_oracle as mo

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ml():
    from mixture_experts_ffn_gate_amd import moe_layer
    torch.cuda.init()
    return moe_layer


def _ids(n, k, E, seed):
    rng = np.random.default_rng(seed)
    return np.stack([rng.choice(E, k, replace=False) for _ in range(n)]).astype(np.int32)


def _same(a, b):
    for x, y, nm in zip(a, b, ("counts", "offsets", "perm", "inv")):
        np.testing.assert_array_equal(x.cpu().numpy(), y.cpu().numpy(), err_msg=nm)


def test_static_sort_two_calls_then_smaller(ml):
    # Two calls in a row on one GPU, the second smaller: the static scratch
    # keeps the first call's counts, which the second must not see.
    for n, k, E, seed in ((4096, 8, 128, 1), (700, 6, 128, 2), (300, 3, 512, 3)):
        print(f"\n[case] static sort n={n} k={k} E={E}", flush=True)
        ids = _ids(n, k, E, seed)
        t = torch.from_numpy(ids).cuda()
        ref = ml.route_sort(t, E)
        got = ml.route_sort_static(t, E)
        torch.cuda.synchronize()
        _same(got, ref)
        rc, ro, rp, ri = mo.sort_routes(ids, E)
        np.testing.assert_array_equal(got[2].cpu().numpy(), rp)
        np.testing.assert_array_equal(got[3].cpu().numpy(), ri)
        np.testing.assert_array_equal(got[0].cpu().numpy(), rc)
        np.testing.assert_array_equal(got[1].cpu().numpy(), ro)


def test_static_sort_skewed_and_largest(ml):
    # All routes on a few experts; then the largest size the scratch holds at
    # E = 512 (ceil(n*k/2048) * 512 = 262144 ints).
    rng = np.random.default_rng(5)
    ids = np.stack([np.concatenate([[0], rng.choice(np.arange(1, 9), 3, replace=False)])
                    for _ in range(9000)]).astype(np.int32)
    t = torch.from_numpy(ids).cuda()
    _same(ml.route_sort_static(t, 16), ml.route_sort(t, 16))
    n, k, E = 65536, 16, 512        # 1M routes = 512 blocks of 2048
    ids = np.random.default_rng(6).integers(0, E, size=(n, k), dtype=np.int32)
    t = torch.from_numpy(ids).cuda()
    got = ml.route_sort_static(t, E)
    torch.cuda.synchronize()
    rc, ro, rp, ri = mo.sort_routes(ids, E)
    np.testing.assert_array_equal(got[0].cpu().numpy(), rc)
    np.testing.assert_array_equal(got[1].cpu().numpy(), ro)
    np.testing.assert_array_equal(got[2].cpu().numpy(), rp)
    np.testing.assert_array_equal(got[3].cpu().numpy(), ri)


def test_static_sort_rejects_oversize_and_captures(ml):
    t = torch.zeros(65536 + 1, 16, dtype=torch.int32, device="cuda")
    with pytest.raises(ml.MoeError) as ei:
        ml.route_sort_static(t, 512)
    assert ei.value.code == ml.MOE_ERR_INVALID_ARG and "scratch" in str(ei.value)
    # Under graph capture (the callers it is for): replays match an eager run.
    ids = torch.from_numpy(_ids(3000, 6, 128, 7)).cuda()
    ref = ml.route_sort(ids, 128)
    n, k = ids.shape
    outs = [torch.full((sz,), -1, dtype=torch.int32, device="cuda")
            for sz in (128, 129, n * k, n * k)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    lib = ml.lib()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            rc = lib.moe_route_sort_static(ml._ptr(ids), n, k, 128, *(ml._ptr(o) for o in outs),
                                           ml._stream(s))
    assert rc == ml.MOE_OK
    torch.cuda.synchronize()
    for rep in range(2):
        for o in outs:
            o.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _same(outs, ref)
