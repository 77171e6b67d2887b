"""Profiling helpers: the copy kernel that calibrates rocprofv3's HBM byte
counters, and the summary of rocprofv3 outputs into the text kept in profiles/.

  python -m sparse_mixture_experts_permute_amd.profiling copy [--mib 1024]
      runs a plain device-to-device copy of a known size (the calibration
      kernel for FETCH_SIZE / WRITE_SIZE)
  python -m sparse_mixture_experts_permute_amd.profiling summarize --stats S.csv
      [--fetch F.csv --write W.csv --cal-fetch CF.csv --cal-write CW.csv]
      [--trace T.csv] [--kernel SUBSTR] [--bench bench.json] [--cmd "..."]
      prints a markdown summary (kernel table, per-dispatch traffic of the
      selected kernel scaled by the copy calibration)
  python -m sparse_mixture_experts_permute_amd.profiling fp8-decode --T 8 [--steps 20]
      runs back-to-back decode steps of the Mixtral-shaped layer with FP8
      experts (weights quantised once, before the steps) for a kernel trace
      or counter pass, and prints the mean step time
"""
from __future__ import annotations

import argparse
import csv
import json
import statistics
import sys
from collections import defaultdict

COPY_MIB_DEFAULT = 1024


def run_copy(mib: int) -> None:
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {mib} MiB x 3", flush=True)


def run_fp8_decode(T: int, steps: int) -> None:
    import os

    import torch
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:  # run as a script path
        sys.path.insert(0, root)

    from sparse_mixture_experts_permute_amd import moe
    from sparse_mixture_experts_permute_amd.inputs import CONFIGS, make_inputs
    cfg = CONFIGS["mixtral_decode_T128"]
    host = make_inputs(cfg, T=max(T, cfg.T))
    dev = {n: moe.tensor_from_numpy(a) for n, a in host.items() if a is not None}
    layer = moe.MoELayerFP8(dev["Wg"], dev["W1"], dev["W3"], dev["W2"], cfg.k)
    x = dev["x"][:T].contiguous()
    y = torch.empty_like(x)
    for _ in range(3):
        layer(x, y)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        layer(x, y)
    b.record()
    torch.cuda.synchronize()
    print(f"fp8 decode T={T}: {a.elapsed_time(b) / steps * 1e3:.1f} us/step "
          f"(back-to-back, {steps} steps)", flush=True)


def _short(name: str) -> str:
    name = name.replace("moe::(anonymous namespace)::", "")
    name = name.split("(")[0] if "(" in name else name
    return name.replace("void ", "")


def _read_stats(path):
    rows = list(csv.DictReader(open(path)))
    out = []
    for r in rows:
        out.append(dict(name=r["Name"], calls=int(r["Calls"]),
                        avg_us=float(r["AverageNs"]) / 1e3,
                        total_ms=float(r["TotalDurationNs"]) / 1e6,
                        pct=float(r["Percentage"])))
    out.sort(key=lambda r: -r["total_ms"])
    return out


def _durations(path, substr):
    """Per-dispatch durations (us) of the kernels whose name holds substr."""
    out = []
    for r in csv.DictReader(open(path)):
        if substr in r["Kernel_Name"]:
            out.append((float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) / 1e3)
    return out


def _per_dispatch(path, counter):
    """{kernel name: [value per dispatch]} for one counter (summed over agents)."""
    per = defaultdict(lambda: defaultdict(float))
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        per[r["Kernel_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: list(v.values()) for k, v in per.items()}


def _calibration(path, counter, mib):
    """expected KiB / measured KiB for the copy kernel's largest dispatch."""
    vals = []
    for k, v in _per_dispatch(path, counter).items():
        vals.extend(v)
    measured = max(vals)
    return (mib * 1024.0) / measured, measured


def summarize(a) -> str:
    lines = []
    if a.cmd:
        lines += ["Commands:", "", "```", a.cmd.strip(), "```", ""]
    stats = _read_stats(a.stats)
    lines += ["Kernel trace (`rocprofv3 --kernel-trace --stats`):", "",
              "| kernel | calls | avg (us) | total (ms) | % |", "|---|---|---|---|---|"]
    for r in stats[:12]:
        lines.append(f"| `{_short(r['name'])}` | {r['calls']} | {r['avg_us']:.1f} | "
                     f"{r['total_ms']:.3f} | {r['pct']:.1f} |")
    lines.append("")
    sel = [r for r in stats if a.kernel in r["name"]]
    if sel:
        k = sel[0]
        lines.append(f"Selected kernel `{_short(k['name'])}`: {k['calls']} dispatches, "
                     f"average {k['avg_us']:.1f} us.")
        if a.trace:
            d = sorted(_durations(a.trace, a.kernel))
            if d:
                lines.append(f"Per-dispatch durations from the kernel trace: median "
                             f"{statistics.median(d):.1f} us, fastest {d[0]:.1f} us, slowest "
                             f"{d[-1]:.1f} us over {len(d)} dispatches (the warm-up dispatches, "
                             f"before the clocks settle, are the slow ones).")
        lines.append("")
    if a.fetch and a.write and a.cal_fetch and a.cal_write and sel:
        cf, mf = _calibration(a.cal_fetch, "FETCH_SIZE", a.cal_mib)
        cw, mw = _calibration(a.cal_write, "WRITE_SIZE", a.cal_mib)
        fetch = [v for kk, vs in _per_dispatch(a.fetch, "FETCH_SIZE").items()
                 if a.kernel in kk for v in vs]
        write = [v for kk, vs in _per_dispatch(a.write, "WRITE_SIZE").items()
                 if a.kernel in kk for v in vs]
        f_kib, w_kib = statistics.median(fetch), statistics.median(write)
        traffic = (f_kib * cf + w_kib * cw) * 1024.0
        lines += [
            "HBM traffic (`rocprofv3 --pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`, KiB per "
            "dispatch):", "",
            f"- copy calibration ({a.cal_mib} MiB read + {a.cal_mib} MiB written): FETCH_SIZE "
            f"read {mf:.0f} KiB -> factor {cf:.4f}; WRITE_SIZE read {mw:.0f} KiB -> factor "
            f"{cw:.4f}",
            f"- selected kernel, median over {len(fetch)} dispatches: FETCH_SIZE {f_kib:.0f} KiB, "
            f"WRITE_SIZE {w_kib:.0f} KiB",
            f"- calibrated traffic per dispatch: {traffic / 1e9:.4f} GB "
            f"({f_kib * cf * 1024 / 1e9:.4f} read + {w_kib * cw * 1024 / 1e9:.4f} written)",
            ""]
    if a.bench:
        b = json.loads(open(a.bench).read().strip().splitlines()[-1])
        rl = b.get("roofline", {})
        lines += ["bench.py line for the same command:", "",
                  f"- workload {b['config']['workload']}: {b['value']} {b['unit']}, "
                  f"{b['ms_per_step']} ms/step",
                  f"- roofline ({rl.get('kernel')}): {rl.get('achieved')} {rl.get('unit')} of "
                  f"{rl.get('peak')} (frac {rl.get('frac')}), kernel {rl.get('kernel_ms')} ms "
                  f"by in-run HIP events", ""]
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=COPY_MIB_DEFAULT)
    f = sub.add_parser("fp8-decode")
    f.add_argument("--T", type=int, default=8)
    f.add_argument("--steps", type=int, default=20)
    s = sub.add_parser("summarize")
    s.add_argument("--stats", required=True)
    s.add_argument("--trace", help="kernel_trace.csv of the same run (per-dispatch durations)")
    s.add_argument("--fetch")
    s.add_argument("--write")
    s.add_argument("--cal-fetch")
    s.add_argument("--cal-write")
    s.add_argument("--cal-mib", type=int, default=COPY_MIB_DEFAULT)
    s.add_argument("--kernel", default="grouped_gemm_dl_kernel<256, 256, true>")
    s.add_argument("--bench")
    s.add_argument("--cmd", default="")
    a = ap.parse_args(argv)
    if a.cmd_name == "copy":
        run_copy(a.mib)
    elif a.cmd_name == "fp8-decode":
        run_fp8_decode(a.T, a.steps)
    else:
        print(summarize(a))


if __name__ == "__main__":
    sys.exit(main())
