"""ctypes binding of libmoe_layer.so (include/moe_layer.h): argument marshalling only.

Tensors are torch tensors on the current HIP device; their ``data_ptr()`` is
passed through, and the stream defaults to torch's current stream. Every step
of the layer runs in the library's HIP kernels. If the library is missing the
import of this module raises; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_layer.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_INVALID_CONFIG = -2
MOE_ERR_TOO_MANY_TOKENS = -3
MOE_ERR_OOM = -4
MOE_ERR_HIP = -5
MOE_DT_F32, MOE_DT_BF16, MOE_DT_NVFP4 = 0, 1, 2
MOE_MAX_EXPERTS = 512
MOE_MAX_TOP_K = 16
DBG = dict(normed=0, logits=1, ids=2, weights=3, counts=4, offsets=5, perm=6, inv=7)

# Every function the header declares (checked by the CPU test suite).
EXPORTS = ("moe_layer_create", "moe_layer_forward", "moe_layer_destroy", "moe_last_error",
           "moe_topk_sigmoid", "moe_route_sort", "moe_nvfp4_quantize", "moe_layer_debug_read",
           "moe_layer_timing_begin", "moe_layer_timing_end", "moe_route_sort_static")
STAGES = ("norm_gate", "shared_up", "shared_down", "fc1", "topk", "sort", "grouped_up",
          "grouped_down", "reduce", "fc2")


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class Config(ctypes.Structure):
    _fields_ = [("hidden_size", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("moe_inter", ctypes.c_int32),
                ("shared_inter", ctypes.c_int32), ("latent_size", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("routed_scaling_factor", ctypes.c_float), ("act_dtype", ctypes.c_int32),
                ("expert_dtype", ctypes.c_int32)]


class Nvfp4(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("scale2", ctypes.c_void_p)]


class Weights(ctypes.Structure):
    _fields_ = [("norm_gamma", ctypes.c_void_p), ("gate", ctypes.c_void_p),
                ("fc1", ctypes.c_void_p), ("fc2", ctypes.c_void_p), ("up", ctypes.c_void_p),
                ("down", ctypes.c_void_p), ("shared_up", ctypes.c_void_p),
                ("shared_down", ctypes.c_void_p), ("up_q", Nvfp4), ("down_q", Nvfp4),
                ("shared_up_q", Nvfp4), ("shared_down_q", Nvfp4)]


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m mixture_experts_ffn_gate_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, f32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_int64
    sig = {
        "moe_layer_create": (i32, [ctypes.POINTER(Config), ctypes.POINTER(Weights), vp,
                                   ctypes.POINTER(vp)]),
        "moe_layer_forward": (i32, [vp, vp, vp, i32, vp]),
        "moe_layer_destroy": (None, [vp]),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_topk_sigmoid": (i32, [vp, i32, i32, i32, f32, vp, vp, vp]),
        "moe_route_sort": (i32, [vp, i32, i32, i32, vp, vp, vp, vp, vp]),
        "moe_route_sort_static": (i32, [vp, i32, i32, i32, vp, vp, vp, vp, vp]),
        "moe_nvfp4_quantize": (i32, [vp, i32, i32, i32, vp, vp, vp, vp]),
        "moe_layer_debug_read": (i32, [vp, i32, vp, i64, vp]),
        "moe_layer_timing_begin": (i32, [vp, ctypes.c_uint32, i32]),
        "moe_layer_timing_end": (i32, [vp, ctypes.POINTER(f32), ctypes.POINTER(i32)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = load_library()


def lib() -> ctypes.CDLL:
    return _lib


def _check(rc: int):
    if rc != MOE_OK:
        raise MoeError(rc, _lib.moe_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


_DT = {torch.float32: MOE_DT_F32, torch.bfloat16: MOE_DT_BF16}


class MoeLayer:
    """A layer built by moe_layer_create; ``forward`` runs moe_layer_forward."""

    def __init__(self, *, hidden_size, num_experts, top_k, moe_inter, shared_inter=0,
                 latent_size=0, max_tokens, weights: dict, rms_eps=1e-5,
                 routed_scaling_factor=1.0, act_dtype=torch.bfloat16, expert_dtype=None,
                 nvfp4: dict | None = None, stream=None):
        if expert_dtype is None:
            expert_dtype = "nvfp4" if nvfp4 is not None else act_dtype
        self.cfg = Config(hidden_size, num_experts, top_k, moe_inter, shared_inter, latent_size,
                          max_tokens, rms_eps, routed_scaling_factor, _DT[act_dtype],
                          MOE_DT_NVFP4 if expert_dtype == "nvfp4" else _DT[expert_dtype])
        self.act_dtype = act_dtype
        w = Weights()
        keep = []
        dense_names = ("norm_gamma", "gate", "fc1", "fc2")
        expert_names = ("up", "down", "shared_up", "shared_down")
        for name in dense_names + (() if nvfp4 is not None else expert_names):
            key = "gamma" if name == "norm_gamma" else name
            t = weights.get(key)
            if t is not None:
                t = t.contiguous()
                keep.append(t)
                setattr(w, name, t.data_ptr())
        if nvfp4 is not None:
            for name in ("up_q", "down_q", "shared_up_q", "shared_down_q"):
                q = nvfp4.get(name.replace("_q", ""))
                if q is not None:
                    packed, scales, scale2 = (x.contiguous() for x in q)
                    keep += [packed, scales, scale2]
                    setattr(w, name, Nvfp4(packed.data_ptr(), scales.data_ptr(),
                                           scale2.data_ptr()))
        handle = ctypes.c_void_p()
        _check(_lib.moe_layer_create(ctypes.byref(self.cfg), ctypes.byref(w), _stream(stream),
                                     ctypes.byref(handle)))
        self._h = handle
        self.hidden_size = hidden_size
        self.num_experts = num_experts
        self.top_k = top_k

    def _check_rows(self, hidden: torch.Tensor, residual: torch.Tensor, num_tokens):
        """Host-side shape, dtype and device checks of a forward's arguments:
        the library trusts these pointers, so a mismatch would otherwise be
        an out-of-bounds device access."""
        for name, t in (("hidden", hidden), ("residual", residual)):
            if not isinstance(t, torch.Tensor):
                raise TypeError(f"{name} must be a torch tensor")
            if t.dtype != self.act_dtype:
                raise TypeError(f"{name} is {t.dtype}, the layer's activations are "
                                f"{self.act_dtype}")
            if t.dim() != 2 or t.shape[1] != self.hidden_size:
                raise ValueError(f"{name} must be [N, {self.hidden_size}], got "
                                 f"{tuple(t.shape)}")
        if residual.shape != hidden.shape:
            raise ValueError(f"residual {tuple(residual.shape)} and hidden "
                             f"{tuple(hidden.shape)} differ")
        n = hidden.shape[0] if num_tokens is None else int(num_tokens)
        if n < 0 or n > hidden.shape[0]:
            raise ValueError(f"num_tokens={n} outside 0..{hidden.shape[0]} (rows of hidden)")
        for name, t in (("hidden", hidden), ("residual", residual)):
            if t.device.type != "cuda":
                raise ValueError(f"{name} must be on a GPU, got {t.device}")
        return n

    def forward(self, hidden: torch.Tensor, residual: torch.Tensor, num_tokens=None,
                stream=None):
        n = self._check_rows(hidden, residual, num_tokens)
        _check(_lib.moe_layer_forward(self._h, _ptr(hidden), _ptr(residual), n, _stream(stream)))
        return hidden

    def debug_read(self, which: str, out: torch.Tensor, stream=None):
        if out.device.type != "cuda":
            raise ValueError(f"debug_read copies into GPU memory, got {out.device}")
        _check(_lib.moe_layer_debug_read(self._h, DBG[which], _ptr(out),
                                         out.numel() * out.element_size(), _stream(stream)))
        return out

    def timing_begin(self, stages=STAGES, max_forwards=4096):
        mask = 0
        for st in stages:
            mask |= 1 << STAGES.index(st)
        _check(_lib.moe_layer_timing_begin(self._h, mask, max_forwards))

    def timing_end(self) -> dict:
        """{stage: (total_ms, launches)} for the stages recorded since timing_begin."""
        tot = (ctypes.c_float * len(STAGES))()
        cnt = (ctypes.c_int32 * len(STAGES))()
        _check(_lib.moe_layer_timing_end(self._h, tot, cnt))
        return {st: (tot[i], cnt[i]) for i, st in enumerate(STAGES) if cnt[i]}

    def close(self):
        if getattr(self, "_h", None):
            _lib.moe_layer_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _check_tensor(name, t, dtype, dims):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dimensions, got {tuple(t.shape)}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {t.device}")


def topk_sigmoid(logits: torch.Tensor, k: int, scale: float = 1.0, stream=None):
    _check_tensor("logits", logits, torch.float32, 2)
    n, E = logits.shape
    ids = torch.empty(n, k, dtype=torch.int32, device=logits.device)
    w = torch.empty(n, k, dtype=torch.float32, device=logits.device)
    _check(_lib.moe_topk_sigmoid(_ptr(logits), n, E, k, scale, _ptr(ids), _ptr(w),
                                 _stream(stream)))
    return ids, w


def route_sort(ids: torch.Tensor, num_experts: int, stream=None):
    _check_tensor("ids", ids, torch.int32, 2)
    n, k = ids.shape
    dev = ids.device
    counts = torch.empty(num_experts, dtype=torch.int32, device=dev)
    offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(n * k, dtype=torch.int32, device=dev)
    inv = torch.empty(n * k, dtype=torch.int32, device=dev)
    _check(_lib.moe_route_sort(_ptr(ids), n, k, num_experts, _ptr(counts), _ptr(offsets),
                               _ptr(perm), _ptr(inv), _stream(stream)))
    return counts, offsets, perm, inv


def route_sort_static(ids: torch.Tensor, num_experts: int, stream=None):
    """moe_route_sort_static: the same sort with its per-block counts in the
    library's static device scratch (no allocation inside the library)."""
    _check_tensor("ids", ids, torch.int32, 2)
    n, k = ids.shape
    dev = ids.device
    counts = torch.empty(num_experts, dtype=torch.int32, device=dev)
    offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(n * k, dtype=torch.int32, device=dev)
    inv = torch.empty(n * k, dtype=torch.int32, device=dev)
    _check(_lib.moe_route_sort_static(_ptr(ids), n, k, num_experts, _ptr(counts), _ptr(offsets),
                                      _ptr(perm), _ptr(inv), _stream(stream)))
    return counts, offsets, perm, inv


def nvfp4_quantize(w: torch.Tensor, stream=None):
    """fp32 [G, rows, cols] -> (packed u8 [G, rows, cols/2], scales u8 [G, rows, cols/16],
    scale2 fp32 [G])."""
    _check_tensor("w", w, torch.float32, 3)
    G, rows, cols = w.shape
    dev = w.device
    packed = torch.empty(G, rows, cols // 2, dtype=torch.uint8, device=dev)
    scales = torch.empty(G, rows, cols // 16, dtype=torch.uint8, device=dev)
    scale2 = torch.empty(G, dtype=torch.float32, device=dev)
    _check(_lib.moe_nvfp4_quantize(_ptr(w), G, rows, cols, _ptr(packed), _ptr(scales),
                                   _ptr(scale2), _stream(stream)))
    return packed, scales, scale2


def quantize_experts(weights: dict, stream=None) -> dict:
    """NVFP4 triplets of the routed and shared expert stacks of ``weights``
    (fp32 masters), quantized on the device by moe_nvfp4_quantize."""
    out = {}
    for key in ("up", "down", "shared_up", "shared_down"):
        t = weights.get(key)
        if t is None:
            continue
        t3 = t.float().contiguous()
        if t3.dim() == 2:
            t3 = t3.unsqueeze(0)
        out[key] = nvfp4_quantize(t3, stream=stream)
    return out


def layer_from_workload(wl, weights: dict, max_tokens=None, nvfp4=None, stream=None) -> MoeLayer:
    """Build a layer for a ``workloads.Workload`` from its weight dict (NVFP4
    workloads quantize their fp32 expert masters with the library unless
    ``nvfp4`` triplets are given)."""
    act = torch.float32 if wl.act_dtype == "f32" else torch.bfloat16
    if wl.expert_dtype == "nvfp4" and nvfp4 is None:
        nvfp4 = quantize_experts(weights, stream=stream)
    return MoeLayer(hidden_size=wl.H, num_experts=wl.E, top_k=wl.k, moe_inter=wl.I,
                    shared_inter=wl.S, latent_size=wl.L,
                    max_tokens=wl.N if max_tokens is None else max_tokens, weights=weights,
                    rms_eps=wl.eps, routed_scaling_factor=wl.scale, act_dtype=act,
                    expert_dtype="nvfp4" if wl.expert_dtype == "nvfp4" else act,
                    nvfp4=nvfp4, stream=stream)
