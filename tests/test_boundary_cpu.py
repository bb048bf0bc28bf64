"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before touching the GPU (no compute calls here)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_layer.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(moe_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def mod():
    from mixture_experts_ffn_gate_amd import moe_layer
    return moe_layer


def test_header_declares_the_binding_exports(mod):
    assert _declared_functions() == sorted(mod.EXPORTS)


def test_library_exports_every_declared_symbol(mod):
    lib = ctypes.CDLL(mod.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_struct_layouts_match_header(mod):
    # 7 int32 + 2 float + 2 int32, no padding.
    assert ctypes.sizeof(mod.Config) == 11 * 4
    # 8 pointers + 4 NVFP4 triplets of pointers.
    assert ctypes.sizeof(mod.Weights) == (8 + 12) * ctypes.sizeof(ctypes.c_void_p)


def _cfg(mod, **kw):
    base = dict(hidden_size=256, num_experts=8, top_k=2, moe_inter=128, shared_inter=256,
                latent_size=0, max_tokens=64, rms_eps=1e-5, routed_scaling_factor=1.0,
                act_dtype=mod.MOE_DT_BF16, expert_dtype=mod.MOE_DT_BF16)
    base.update(kw)
    return mod.Config(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(top_k=0), -2), (dict(top_k=9), -2), (dict(num_experts=600, top_k=2), -2),
    (dict(num_experts=32, top_k=17), -2), (dict(hidden_size=100), -2),
    (dict(moe_inter=96), -2), (dict(max_tokens=0), -2),
    (dict(act_dtype=0, expert_dtype=1), -2), (dict(act_dtype=7), -2),
    (dict(shared_inter=-64), -2), (dict(hidden_size=16384), -2),
    # routes are indexed by 32-bit ints: max_tokens * top_k is bounded
    (dict(max_tokens=600_000_000, top_k=2), -2),
])
def test_create_rejects_bad_config_on_host(mod, kw, code):
    lib = mod.lib()
    cfg = _cfg(mod, **kw)
    w = mod.Weights()
    out = ctypes.c_void_p(123)
    rc = lib.moe_layer_create(ctypes.byref(cfg), ctypes.byref(w), None, ctypes.byref(out))
    assert rc == code
    assert out.value is None
    assert lib.moe_last_error().decode()


def test_null_arguments_rejected(mod):
    lib = mod.lib()
    out = ctypes.c_void_p()
    assert lib.moe_layer_create(None, None, None, ctypes.byref(out)) == -1
    assert lib.moe_layer_forward(None, None, None, 4, None) == -1
    assert lib.moe_topk_sigmoid(None, 4, 8, 2, 1.0, None, None, None) == -1
    assert lib.moe_topk_sigmoid(None, 0, 8, 9, 1.0, None, None, None) == -2
    assert lib.moe_route_sort(None, 4, 2, 8, None, None, None, None, None) == -1
    assert lib.moe_nvfp4_quantize(None, 1, 4, 20, None, None, None, None) == -1
    assert lib.moe_layer_debug_read(None, 0, None, 0, None) == -1
    lib.moe_layer_destroy(None)   # no-op


def test_fp32_layers_accept_multiples_of_16(mod):
    lib = mod.lib()
    cfg = _cfg(mod, act_dtype=0, expert_dtype=0, hidden_size=48, moe_inter=96)
    w = mod.Weights()   # all NULL: fails on the missing weights, after the config passed
    out = ctypes.c_void_p()
    rc = lib.moe_layer_create(ctypes.byref(cfg), ctypes.byref(w), None, ctypes.byref(out))
    assert rc in (-1, -5)  # -5 only where no HIP device can be queried


def test_profile_kernel_labels():
    # Labels of the rocprofv3 summaries: mangled and demangled symbol forms.
    from mixture_experts_ffn_gate_amd.profiling import short_name
    assert short_name("_Z16gemm_mfma_kernelILi32ELi64ELi4ELi1EDF16bLi0ELb1ELb1EEv8GemmArgsiiii") \
        == "gemm[grouped,store,bf16,128x64,nt]"
    assert short_name("_Z16gemm_mfma_kernelILi32ELi128ELi8ELi0EDF16bLi0ELb0ELb0EEv8GemmArgsiiii") \
        == "gemm[dense,relu2,bf16,256x128]"
    assert short_name("void gemm_mfma_kernel<32, 128, 4, 0, bool _Accum, int, E, true, false>"
                      "(GemmArgs, int, int, int, int)") == "gemm[grouped,relu2,nvfp4,128x128]"
    # current symbols carry a third flag (the deep-pipeline dense variant)
    assert short_name("_Z16gemm_mfma_kernelILi32ELi64ELi4ELi1EDF16bLi0ELb1ELb1ELb0EEv8GemmArgsiiii") \
        == "gemm[grouped,store,bf16,128x64,nt]"
    assert short_name("_Z16gemm_mfma_kernelILi32ELi128ELi4ELi0EDF16bLi0ELb0ELb0ELb1EEv8GemmArgsiiii") \
        == "gemm[dense,relu2,bf16,128x128,deep]"
    assert short_name("void gemm_mfma_kernel<32, 128, 4, 0, bool _Accum, int, E, true, false, false>"
                      "(GemmArgs, int, int, int, int)") == "gemm[grouped,relu2,nvfp4,128x128]"
    assert short_name("void gemm_mfma_kernel<32, 128, 4, 1, bool _Accum, int, E, false, false, false>"
                      "(GemmArgs, int, int, int, int)") == "gemm[dense,store,nvfp4,128x128]"
    # 48-feature waves: 8 x 48 = 384 and 7 x 48 = 336 features per workgroup
    assert short_name("_Z16gemm_mfma_kernelILi48ELi128ELi7ELi1EDF16bLi0ELb1ELb1ELb0EEv8GemmArgsiiii") \
        == "gemm[grouped,store,bf16,336x128,nt]"
    assert short_name("_Z16gemm_mfma_kernelILi48ELi128ELi8ELi2EDF16bLi0ELb0ELb0ELb0EEv8GemmArgsiiii") \
        == "gemm[dense,add_res,bf16,384x128]"
    assert short_name("_Z11gemv_kernelILi1EDF16bLi0EEv8GemvArgs") == "gemv[store,bf16]"
    assert short_name("_Z11gemv_kernelILi1EDF16bLi1EEv8GemvArgs") == "gemv[store,nvfp4]"
    assert short_name("void route_small_kernel<2>(bool _Accum const*)") == "route_small"


def _bare_layer(mod, act_dtype, hidden_size):
    # A MoeLayer object without a device handle: only its host-side checks run.
    import torch
    L = object.__new__(mod.MoeLayer)
    L._h = None
    L.act_dtype = act_dtype
    L.hidden_size = hidden_size
    return L


def test_forward_argument_checks_on_host(mod):
    import torch
    L = _bare_layer(mod, torch.bfloat16, 64)
    h = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        L.forward(h.float(), h)                      # wrong dtype
    with pytest.raises(TypeError):
        L.forward(h, h.float())
    with pytest.raises(ValueError):
        L.forward(torch.zeros(4, 32, dtype=torch.bfloat16), h)   # wrong width
    with pytest.raises(ValueError):
        L.forward(h, torch.zeros(3, 64, dtype=torch.bfloat16))   # residual shape
    with pytest.raises(ValueError):
        L.forward(h, h.clone(), num_tokens=5)        # more tokens than rows
    with pytest.raises(ValueError):
        L.forward(h, h.clone(), num_tokens=-1)
    with pytest.raises(ValueError):
        L.forward(h, h.clone())                      # host memory, not a GPU
    with pytest.raises(ValueError):
        L.debug_read("ids", torch.zeros(8, dtype=torch.int32))


def test_stage_argument_checks_on_host(mod):
    import torch
    with pytest.raises(TypeError):
        mod.topk_sigmoid(torch.zeros(4, 8, dtype=torch.bfloat16), 2)
    with pytest.raises(ValueError):
        mod.topk_sigmoid(torch.zeros(4, 8), 2)        # host memory
    with pytest.raises(TypeError):
        mod.route_sort(torch.zeros(4, 2, dtype=torch.int64), 8)
    with pytest.raises(ValueError):
        mod.route_sort(torch.zeros(8, dtype=torch.int32), 8)
    with pytest.raises(TypeError):
        mod.nvfp4_quantize(torch.zeros(1, 4, 16, dtype=torch.float64))


def test_static_sort_rejects_oversize_on_host(mod):
    # The size check of the allocation-free sort runs before anything else
    # (NULL pointers here: nothing could be launched even if it did not).
    lib = mod.lib()
    assert lib.moe_route_sort_static(None, 65537, 16, 512, None, None, None, None, None) == -1
    assert "scratch" in lib.moe_last_error().decode()
    assert lib.moe_route_sort_static(None, 4, 2, 600, None, None, None, None, None) == -2
    assert lib.moe_route_sort_static(None, 4, 0, 8, None, None, None, None, None) == -1
