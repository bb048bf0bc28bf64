"""Build libmoe_layer.so for gfx950 with hipcc (in-tree, next to this file).

Usage: ``python -m mixture_experts_ffn_gate_amd.build`` or ``build()``.
Every HIP source is compiled with packed-fp32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``).
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe_layer.so")
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")

SOURCES = ["routing.hip", "gemm.hip", "reduce.hip", "nvfp4.hip", "scratch.hip", "layer.cpp"]

# -amdgpu-mfma-vgpr-form: MFMA accumulators in ordinary VGPRs. With the
# default heuristic the compiler kept some in AGPRs and rotated them through
# the VGPRs on every unrolled k-step group (92 moves per 96 MFMAs in the dense
# 128x128 kernel); in VGPR form the k-loops hold no copies, the 64-row tiles
# fit three waves per SIMD, and the layer measured 1-3% faster.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-mfma-vgpr-form",
             "-Wno-unused-result", f"-I{INCLUDE}", f"-I{CSRC}"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, verbose: bool, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *HIP_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in res.stderr.splitlines()
                     if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    return obj


def build(verbose: bool = False, extra_flags=(), out: str = LIB, build_dir: str = BUILD) -> str:
    """Compile every source and link the shared library; returns its path.

    ``extra_flags`` (e.g. ``-D`` tuning macros) and ``out``/``build_dir`` let a
    caller build a variant next to the default library."""
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, tuple(extra_flags)),
                           SOURCES))
    tmp = out + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, out)
    return out


def resource_usage(src: str, build_dir: str = BUILD) -> list:
    """Per-kernel register, scratch and LDS use of one source, from hipcc's
    kernel-resource-usage remarks: [{"kernel", "vgprs", "agprs", "scratch",
    "occupancy", "lds"}]. A kernel with scratch > 0 spills registers."""
    import re
    import tempfile

    os.makedirs(build_dir, exist_ok=True)
    with tempfile.TemporaryDirectory(dir=build_dir) as tmp:
        obj = os.path.join(tmp, "ru.o")
        cmd = [_hipcc(), *HIP_FLAGS, "--cuda-device-only", "-c", os.path.join(CSRC, src),
               "-o", obj, "-Rpass-analysis=kernel-resource-usage"]
        res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr[-4000:]}")
    rows = []
    fields = {"VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch",
              "Occupancy [waves/SIMD]": "occupancy", "LDS Size [bytes/block]": "lds"}
    for line in res.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            rows.append({"kernel": m.group(1)})
            continue
        for key, name in fields.items():
            m = re.search(r"remark:\s+" + re.escape(key) + r": (\d+)", line)
            if m and rows:
                rows[-1][name] = int(m.group(1))
    return rows


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
