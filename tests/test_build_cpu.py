"""Build-level checks that need no GPU: every kernel compiles for gfx950
without register spills (scratch), which cost the grouped GEMMs up to 4% when
one slipped in."""

import pytest

from mixture_experts_ffn_gate_amd import build as b


@pytest.mark.parametrize("src", ["gemm.hip", "routing.hip", "reduce.hip", "nvfp4.hip"])
def test_kernels_do_not_spill(src):
    rows = b.resource_usage(src)
    assert rows, f"no kernels reported for {src}"
    spills = [(r["kernel"], r.get("scratch")) for r in rows if r.get("scratch", 0) > 0]
    assert not spills, f"kernels with scratch in {src}: {spills}"
