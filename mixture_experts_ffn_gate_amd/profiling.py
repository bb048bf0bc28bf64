"""rocprofv3 output -> short text summaries and the measured HBM traffic record.

    python -m mixture_experts_ffn_gate_amd.profiling stats  STATS_CSV  OUT_MD  --cmd "..."
    python -m mixture_experts_ffn_gate_amd.profiling traffic FETCH_CSV WRITE_CSV OUT_JSON \
        --calib-mib 512 --workload NAME --tokens N --cmd "..."
    python -m mixture_experts_ffn_gate_amd.profiling mfma COUNTER_CSV STATS_CSV OUT_MD --cmd "..."

``traffic`` reads two ``--pmc`` runs (FETCH_SIZE, then WRITE_SIZE; KiB per
dispatch) of a ``bench.py --calibrate-copy-mib M`` command. The M MiB
device-to-device copy in the same run gives each counter's scale factor:
true KiB / counted KiB. The record stores, per layer kernel, the mean scaled
bytes per dispatch, plus a hash of the kernel and launch sources. ``bench.py``
reports the traffic only while that hash matches the current source.
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
# The kernel and launch sources, and the build script (its compiler flags
# change the generated kernels too).
KERNEL_SOURCES = ("csrc/gemm.hip", "csrc/routing.hip", "csrc/reduce.hip", "csrc/layer.cpp",
                  "csrc/common.h", "csrc/kernels.h", "csrc/wsrc.h", "build.py")


def source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


_MANGLED = re.compile(
    r"gemm_mfma_kernelILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)E\w+?Li(\d+)ELb(\d)E(?:Lb(\d)E)?(?:Lb(\d)E)?")
# The profiler's demangler renders the bf16 argument as "bool _Accum" and an
# NVFP4 weight flag as "int, E"; it leaves the bf16-weight kernels mangled.
_DEMANGLED = re.compile(
    r"gemm_mfma_kernel<(\d+), (\d+), (\d+), (\d+), (.*?), (true|false)(?:, (true|false))?"
    r"(?:, (true|false))?>")
_GEMV_MANGLED = re.compile(r"gemv_kernelILi(\d+)E\w+?Li(\d+)EE()")
_GEMV_DEMANGLED = re.compile(r"gemv_kernel<(\d+), (.*)>()")
_EPI = {"0": "relu2", "1": "store", "2": "add_res"}


def _wq(mid: str) -> str:
    return "bf16" if mid.strip().endswith("0") else "nvfp4"


def short_name(name: str) -> str:
    """Readable kernel label; GEMMs by role (grouped/dense, epilogue, weights, tile)."""
    m = _MANGLED.search(name)
    if m:
        wf, bmt, nw, epi, wq, g, nt, deep = m.groups()
        return (f"gemm[{'grouped' if g == '1' else 'dense'},{_EPI.get(epi, epi)},"
                f"{'nvfp4' if wq == '1' else 'bf16'},{int(wf) * int(nw)}x{bmt}"
                f"{',nt' if nt == '1' else ''}{',deep' if deep == '1' else ''}]")
    m = _DEMANGLED.search(name)
    if m:
        wf, bmt, nw, epi, mid, g, nt, deep = m.groups()
        return (f"gemm[{'grouped' if g == 'true' else 'dense'},{_EPI.get(epi, epi)},"
                f"{_wq(mid)},{int(wf) * int(nw)}x{bmt}{',nt' if nt == 'true' else ''}"
                f"{',deep' if deep == 'true' else ''}]")
    m = _GEMV_MANGLED.search(name)
    if m:
        epi, wq, norm = m.groups()
        return f"gemv[{_EPI.get(epi, epi)},{'nvfp4' if wq == '1' else 'bf16'}]"
    m = _GEMV_DEMANGLED.search(name)
    if m:
        epi, mid, norm = m.groups()
        return f"gemv[{_EPI.get(epi, epi)},{_wq(mid)}]"
    for key in ("gemv_down_reduce", "route_small", "norm_gate", "topk_sigmoid", "route_sort",
                "route_hist",
                "route_scatter", "unpermute_reduce", "retile", "nvfp4_pack", "nvfp4_scale2",
                "copyBuffer"):
        if key in name:
            return key
    if "at::native" in name:
        return "torch:" + name.split("at::native::")[1].split("<")[0][:40]
    return name[:60]


_SETUP = ("torch:", "retile", "nvfp4_pack", "nvfp4_scale2", "copyBuffer", "__amd_rocclr")


def stats(csv_path: str, out_md: str, cmd: str) -> None:
    """Kernel-duration table of the layer's kernels (set-up kernels that build
    the weights and inputs are left out), slowest total first."""
    rows = list(csv.DictReader(open(csv_path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    layer = [r for r in rows if not short_name(r["Name"]).startswith(_SETUP)]
    # Every layer kernel runs at least once per forward (some twice, e.g. the
    # dense GEMM shared by fc1 and the shared down projection).
    forwards = min((int(r["Calls"]) for r in layer), default=0)
    per_fwd = sum(float(r["TotalDurationNs"]) for r in layer) / max(1, forwards) / 1e3
    lines = [f"# Kernel durations: `{os.path.basename(out_md)}`", "",
             "Commands (`$REPO` = repository root):", "", "```", cmd, "```", "",
             "Layer kernels only (weight/input set-up kernels omitted); the",
             "graph-replayed and the eagerly timed forwards are both counted.", "",
             "| kernel | symbol (truncated) | calls | avg µs | min µs | max µs |",
             "|---|---|---|---|---|---|"]
    for r in layer:
        lines.append(f"| {short_name(r['Name'])} | `{r['Name'][:70]}` | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                     f"{float(r['MaxNs']) / 1e3:.1f} |")
    lines += ["", f"Layer kernel time per forward ({forwards} forwards): {per_fwd:.1f} µs."]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def _per_dispatch(csv_path: str, counter: str):
    out = []
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] == counter:
            out.append((r["Kernel_Name"], int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    return out


def traffic(fetch_csv: str, write_csv: str, out_json: str, calib_mib: int, workload: str,
            tokens: int, cmd: str) -> None:
    calib_kib = calib_mib * 1024
    rec = {"workload": workload, "tokens": tokens, "source_hash": source_hash(), "command": cmd,
           "calibration_copy_kib": calib_kib, "kernels": {}}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _per_dispatch(path, counter)
        # The calibration copy: the runtime's device-to-device copy kernel with
        # the largest count (the known-size copy; the layer's own copies are
        # a few KiB).
        copies = [v for n, _, v in rows if "copyBuffer" in n]
        counted = max(copies) if copies else 0.0
        factor = calib_kib / counted if counted > 0 else None
        rec[f"{counter.lower()}_factor"] = factor
        acc = defaultdict(list)
        for name, _, v in rows:
            acc[short_name(name)].append(v)
        for k, vals in acc.items():
            if factor is None:
                continue
            d = rec["kernels"].setdefault(k, {})
            d[f"{counter.lower()}_bytes"] = sum(vals) / len(vals) * factor * 1024
            d["dispatches"] = len(vals)
    with open(out_json, "w") as f:
        json.dump(rec, f, indent=1)


def mfma(counter_csv: str, stats_csv: str, out_md: str, cmd: str) -> None:
    """MFMA utilisation of the layer's GEMM kernels from one --pmc run with
    SQ_VALU_MFMA_BUSY_CYCLES, SQ_BUSY_CU_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_BF16
    and GRBM_GUI_ACTIVE, plus the kernel-trace durations of the same command.

    On gfx950 one MOPS unit is 512 flops and SQ_VALU_MFMA_BUSY_CYCLES counts the
    issued MFMA work in SIMD-cycles (16 per 16x16x32 bf16 MFMA, 1024 flops per
    SIMD-cycle), so busy / (4 x SQ_BUSY_CU_CYCLES) is the matrix cores' share
    of the cycles in which the CUs were busy, and busy / (1024 SIMDs x duration
    x 2.4 GHz) the share of the chip's nominal MFMA issue rate over the launch.
    Both count executed MFMAs, padding rows and dead features included."""
    acc = defaultdict(lambda: defaultdict(list))
    for r in csv.DictReader(open(counter_csv)):
        k = short_name(r["Kernel_Name"])
        if k.startswith(("gemm", "gemv")):
            acc[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
    dur = {short_name(r["Name"]): float(r["AverageNs"]) for r in csv.DictReader(open(stats_csv))}
    lines = [f"# MFMA utilisation: `{os.path.basename(out_md)}`", "",
             "Commands (`$REPO` = repository root):", "", "```", cmd, "```", "",
             "Per launch, averaged over the dispatches of the run (eager forwards under the",
             "profiler). Executed TFLOP = MOPS x 512; busy/CU = SQ_VALU_MFMA_BUSY_CYCLES /",
             "(4 x SQ_BUSY_CU_CYCLES); busy/nominal = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x",
             "duration x 2.4 GHz); both count executed MFMAs (padding rows and dead features",
             "included).", "",
             "| kernel | executed GFLOP | MFMA busy (SIMD-cycles) | CU-busy cycles | avg µs | busy/CU | busy/nominal |",
             "|---|---|---|---|---|---|---|"]
    for k in sorted(acc, key=lambda x: -dur.get(x, 0.0)):
        m = {c: sum(v) / len(v) for c, v in acc[k].items()}
        busy, cu = m.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0), m.get("SQ_BUSY_CU_CYCLES", 0.0)
        mops = m.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)
        us = dur.get(k, 0.0) / 1e3
        per_cu = busy / (4 * cu) if cu else float("nan")
        nominal = busy / (1024 * us * 1e-6 * 2.4e9) if us else float("nan")
        lines.append(f"| {k} | {mops * 512 / 1e9:.1f} | {busy:.3g} | {cu:.3g} | {us:.1f} | "
                     f"{per_cu:.2f} | {nominal:.2f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("out")
    s.add_argument("--cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("out")
    t.add_argument("--calib-mib", type=int, required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--tokens", type=int, required=True)
    t.add_argument("--cmd", required=True)
    mf = sub.add_parser("mfma")
    mf.add_argument("counter_csv")
    mf.add_argument("stats_csv")
    mf.add_argument("out")
    mf.add_argument("--cmd", required=True)
    a = ap.parse_args()
    if a.cmd_name == "mfma":
        mfma(a.counter_csv, a.stats_csv, a.out, a.cmd)
    elif a.cmd_name == "stats":
        stats(a.csv, a.out, a.cmd)
    else:
        traffic(a.fetch_csv, a.write_csv, a.out, a.calib_mib, a.workload, a.tokens, a.cmd)


if __name__ == "__main__":
    main()
