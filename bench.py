"""Benchmark of the MoE layer on one MI355X.

One step = one full layer forward (router, top-k and gate, permutation,
grouped SwiGLU GEMM, grouped down GEMM, combine) over one batch of seeded
synthetic tokens already resident in HBM.  Default workload: the
Mixtral-8x7B-shaped prefill layer (T=8192, d=4096, E=8, d_ff=14336, top-2,
bf16).  Prints one JSON line.

Per-stage kernel times come from HIP events that the library records on the
stream it launches on (moe_forward_timed).  The CPU baseline times the CPU
oracle on a bounded prefix of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

# Context, not targets: the numpy timings of the 7-config granularity table on
# "Trillion-parameter MoE activates only 4.9%: 7 expert configs measured"
# (results table; 2-core i5-1340P under WSL, T=512, d=512, float32; median and
# fastest of 20 runs, ms).  The page times its own function: sigmoid route
# weights and a sigmoid-gated expert.
PAGE_NUMPY_MS = {(1, 32768, 1): (1195.30, 1014.21), (8, 4096, 1): (117.49, 109.76),
                 (8, 4096, 2): (235.78, 208.57), (32, 1024, 1): (65.45, 61.45),
                 (32, 1024, 2): (150.10, 111.87), (64, 512, 4): (160.41, 128.77),
                 (128, 256, 8): (219.62, 203.44)}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="mixtral_prefill_T8192")
    ap.add_argument("--layout", choices=("outin", "inout"), default="outin",
                    help="expert weights as Linear weights [out][in] or as [in][out] (x @ W)")
    ap.add_argument("--no-extra", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens in the CPU-oracle sample (0: size it to ~15 s)")
    return ap.parse_args()


def algorithmic(cfg, counts):
    """Algorithmic work of the SwiGLU GEMM (the dominant kernel) and of the layer.

    SwiGLU GEMM per routed pair: 4*d*d_ff FLOP (W1 and W3 rows); bytes: the W1 and
    W3 matrices of every expert hit once + the pair's x row in + its H row out.
    Layer: 6*d*d_ff FLOP per pair (+6*d*d_ffs per token for a shared expert);
    bytes: the weights of the experts hit + x + y + router weights.
    """
    es = 2 if cfg.dtype == "bf16" else 4
    P = cfg.T * cfg.k
    hit = int((counts > 0).sum())
    g1_flop = 4.0 * cfg.d * cfg.d_ff * P
    g1_bytes = (hit * 2.0 * cfg.d * cfg.d_ff * es + P * cfg.d * es + P * cfg.d_ff * es)
    layer_flop = 6.0 * cfg.d * cfg.d_ff * P + 6.0 * cfg.d * cfg.d_ff_shared * cfg.T
    layer_bytes = (hit * 3.0 * cfg.d * cfg.d_ff * es + 3.0 * cfg.d * cfg.d_ff_shared * es
                   + 2.0 * cfg.T * cfg.d * es + cfg.E * cfg.d * es)
    return dict(g1_flop=g1_flop, g1_bytes=g1_bytes, layer_flop=layer_flop,
                layer_bytes=layer_bytes, experts_hit=hit)


def transposed(dev):
    """The expert weights of `dev` in the [in][out] layout (copies)."""
    out = dict(dev)
    for n in ("W1", "W3", "W2", "Ws1", "Ws3", "Ws2"):
        if out.get(n) is not None:
            out[n] = out[n].transpose(-1, -2).contiguous()
    return out


def run_workload(cfg, host, dev, steps, warmup, flush_mb=0, graph=False, min_warm_s=0.0,
                 inout=False, **variants):
    """Time `steps` layer forwards.

    Pass 1 (the timed region for ms_per_step): back-to-back moe_forward calls
    with HIP events on their stream only around the region; ms_per_step is its
    elapsed time / steps.  With flush_mb, a buffer of that size is read before
    every step (to evict the 256 MB MALL, which would otherwise hold the hit
    experts' weights between steps) and the step time is measured per step
    around the forward only.
    Pass 2 (the stage breakdown): the same forwards through moe_forward_timed,
    which records a HIP event at every stage boundary on the stream the kernels
    run on; each kernel's duration comes from there.  The extra event records
    cost a few microseconds each, which is why they stay out of pass 1.
    With graph=True, one forward is also captured in a HIP graph and replayed
    (reported separately).  min_warm_s: warm-up continues past `warmup` steps
    until that much time has passed (the clocks settle after the host-side
    set-up of a workload).
    """
    import numpy as np
    import torch

    from sparse_mixture_experts_permute_amd import moe

    T = cfg.T
    x = dev["x"][:T].contiguous()
    bias = None
    if cfg.skew:
        b = np.zeros(cfg.E, np.float32)
        b[0] = cfg.skew
        bias = torch.from_numpy(b).cuda()
    shared = (dev["Ws1"], dev["Ws3"], dev["Ws2"]) if cfg.d_ff_shared else None
    layer = moe.MoELayer(dev["Wg"], dev["W1"], dev["W3"], dev["W2"], cfg.k, bias, shared,
                         weight_layout=moe.LAYOUT_IN_OUT if inout else moe.LAYOUT_OUT_IN,
                         **variants)
    y = torch.empty_like(x)
    layer.workspace(T)
    flush = (torch.ones(flush_mb << 18, dtype=torch.float32, device="cuda") if flush_mb
             else None)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    events = [[ev() for _ in range(moe.NSTAGE_EVENTS)] for _ in range(steps)]
    for row in events:
        for e in row:
            e.record()
    n_warm, w_start = 0, time.perf_counter()
    while n_warm < warmup or time.perf_counter() - w_start < min_warm_s:
        if flush is not None:
            flush.sum()
        layer(x, y)
        n_warm += 1
        if n_warm % 8 == 0:
            torch.cuda.synchronize()  # keep the host clock in step with the device
    torch.cuda.synchronize()
    # pass 1: step time
    t_start, t_end = ev(), ev()
    step_ev = [(ev(), ev()) for _ in range(steps)]
    w0 = time.perf_counter()
    t_start.record()
    for i in range(steps):
        if flush is not None:
            flush.sum()  # read flush_mb MB: evicts the 256 MB MALL without dirty lines
            step_ev[i][0].record()
        layer(x, y)
        if flush is not None:
            step_ev[i][1].record()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    if flush is None:
        ms = t_start.elapsed_time(t_end) / steps
        # the same steps again, each between events of its own (median and
        # fastest step; ms_per_step above keeps the events out of its region)
        for a, b_ in step_ev:
            a.record()
            layer(x, y)
            b_.record()
        torch.cuda.synchronize()
    per_step = [a.elapsed_time(b_) for a, b_ in step_ev]
    if flush is not None:
        ms = float(np.mean(per_step))
    # pass 2: stage breakdown
    for i in range(steps):
        if flush is not None:
            flush.sum()
        layer.timed(x, y, events[i])
    torch.cuda.synchronize()
    stage = np.zeros(len(moe.STAGES))
    for row in events:
        for s in range(len(moe.STAGES)):
            stage[s] += row[s].elapsed_time(row[s + 1])
    stage /= steps
    out = dict(ms=ms, wall_s=wall, stage_ms=stage, counts=layer.intermediates(T)["counts"].cpu().numpy(),
               step_ms={"median": round(float(np.median(per_step)), 4),
                        "min": round(float(np.min(per_step)), 4)})
    if graph:
        # one forward captured in a HIP graph, replayed; per-replay time between events
        g = torch.cuda.CUDAGraph()
        s_cap = torch.cuda.Stream()
        s_cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s_cap):
            layer(x, y)  # warm the capture stream
        torch.cuda.current_stream().wait_stream(s_cap)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            layer(x, y)
        torch.cuda.synchronize()
        times = []
        for _ in range(steps):
            if flush is not None:
                flush.sum()
            a, b_ = ev(), ev()
            a.record()
            g.replay()
            b_.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b_))
        out["graph_ms"] = float(np.median(times))
        del g
    return out


def run_fp8(cfg, dev, steps, warmup, flush_mb, layer=None):
    """Decode step with FP8 experts (moe_forward_fp8; weights quantised once,
    outside the timed region): mean per-step time around the forward with the
    MALL flushed before each step, and the expert counts."""
    import numpy as np
    import torch

    from sparse_mixture_experts_permute_amd import moe
    T = cfg.T
    x = dev["x"][:T].contiguous()
    if layer is None:
        layer = moe.MoELayerFP8(dev["Wg"], dev["W1"], dev["W3"], dev["W2"], cfg.k)
    y = torch.empty_like(x)
    flush = torch.ones(flush_mb << 18, dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        layer(x, y)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b_ in ev:
        flush.sum()
        a.record()
        layer(x, y)
        b_.record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b_) for a, b_ in ev]))
    counts = layer.intermediates(T)["counts"].cpu().numpy()
    return dict(ms=ms, counts=counts)


def run_variant(cfg, dev, steps, warmup, **variants):
    """Whole-layer time of moe_forward_ex with the given variants (HIP events
    around `steps` back-to-back forwards) and the pairs the experts kept."""
    import numpy as np
    import torch

    from sparse_mixture_experts_permute_amd import moe
    T = cfg.T
    x = dev["x"][:T].contiguous()
    bias = None
    if cfg.skew:
        b = np.zeros(cfg.E, np.float32)
        b[0] = cfg.skew
        bias = torch.from_numpy(b).cuda()
    layer = moe.MoELayer(dev["Wg"], dev["W1"], dev["W3"], dev["W2"], cfg.k, bias, None,
                         **variants)
    y = torch.empty_like(x)
    for _ in range(warmup):
        layer(x, y)
    torch.cuda.synchronize()
    a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        layer(x, y)
    b_.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b_) / steps
    it = layer.intermediates(T)
    counts = it["counts"].cpu().numpy()
    return dict(ms=ms, counts=counts, kept=int(counts.sum()))


def measured_traffic(cfg):
    """HBM traffic per dispatch of the SwiGLU GEMM from the committed rocprofv3
    counter runs (profiles/traffic.json), or None when those counters were
    taken on another workload or on a different GEMM source."""
    import hashlib
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
        src = open(os.path.join(ROOT, "sparse_mixture_experts_permute_amd", "csrc", "gemm.hip"),
                   "rb").read()
    except (OSError, ValueError):
        return None
    sha = hashlib.sha256(src).hexdigest()[:16]
    if rec.get("gemm_source_sha256_prefix") != sha or rec.get("workload") != cfg.name:
        return None
    return rec.get("traffic_bytes")


def count_summary(counts):
    """Rows per expert of one step: min / max / mean, every expert's count
    when there are at most 64, else an 8-bin histogram of the counts."""
    import numpy as np
    c = np.asarray(counts)
    out = {"min": int(c.min()), "max": int(c.max()), "mean": float(c.mean())}
    if c.size <= 64:
        out["per_expert"] = [int(v) for v in c]
    else:
        h, edges = np.histogram(c, bins=8)
        out["histogram"] = {"bin_edges": [round(float(e), 1) for e in edges],
                            "experts": [int(v) for v in h]}
    return out


def roofline_for(cfg, res):
    from sparse_mixture_experts_permute_amd import moe
    a = algorithmic(cfg, res["counts"])
    g1_ms = float(res["stage_ms"][moe.STAGES.index("gemm_swiglu")])
    ai = a["g1_flop"] / a["g1_bytes"]
    peak_f = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    ridge = peak_f * 1e12 / (PEAK_HBM_GBS * 1e9)
    if ai >= ridge:
        ach = a["g1_flop"] / (g1_ms * 1e-3) / 1e12
        rl = dict(bound="mfma", achieved=round(ach, 2), peak=peak_f, unit="TFLOP/s",
                  frac=round(ach / peak_f, 4))
    else:
        ach = a["g1_bytes"] / (g1_ms * 1e-3) / 1e9
        rl = dict(bound="hbm", achieved=round(ach, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                  frac=round(ach / PEAK_HBM_GBS, 4))
    rl.update(traffic=measured_traffic(cfg), kernel="grouped_gemm_swiglu",
              kernel_ms=round(g1_ms, 4),
              algorithmic_flop=a["g1_flop"], algorithmic_bytes=a["g1_bytes"])
    # whole-layer fractions
    lt = res["ms"] * 1e-3
    layer = dict(mfma_frac=round(a["layer_flop"] / lt / (peak_f * 1e12), 4),
                 hbm_frac=round(a["layer_bytes"] / lt / (PEAK_HBM_GBS * 1e9), 4),
                 experts_hit=a["experts_hit"])
    return rl, layer


def cpu_baseline(cfg, host, n_tokens):
    import numpy as np

    from oracle import oracle as O
    if n_tokens <= 0:
        # size the sample from a short probe run to about 15 s of CPU work
        probe = 8
        t0 = time.perf_counter()
        O.forward(host["x"][:probe], host["Wg"], host["W1"], host["W3"], host["W2"], cfg.k)
        rate = probe / max(time.perf_counter() - t0, 1e-6)
        n_tokens = int(min(cfg.T, max(16, rate * 15.0)))
    x = np.ascontiguousarray(host["x"][:n_tokens])
    bias = None
    if cfg.skew:
        bias = np.zeros(cfg.E, np.float32)
        bias[0] = cfg.skew
    shared = (host["Ws1"], host["Ws3"], host["Ws2"]) if cfg.d_ff_shared else None
    t0 = time.perf_counter()
    O.forward(x, host["Wg"], host["W1"], host["W3"], host["W2"], cfg.k, bias=bias, shared=shared)
    el = time.perf_counter() - t0
    return dict(value=round(n_tokens / el, 3), unit="tokens/s", cores=O.num_threads(),
                kind="oracle", affinity_cores=len(os.sched_getaffinity(0)),
                cpu_model=cpu_model(),
                sample=f"first {n_tokens} of {cfg.T} tokens of {cfg.name}, whole layer "
                       f"(fp64 router, top-k, permutation, experts, combine) in {el:.1f} s")


def cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_small(cfg):
    """The oracle on the 512-token fp32 layer (E=8, top-2, d_ff=4096): its
    first 64 tokens on one core, then all 512 on every core of the affinity
    mask (tokens/s each)."""
    from oracle import oracle as O
    from sparse_mixture_experts_permute_amd.inputs import make_inputs
    h = make_inputs(cfg)
    out = {}
    n_all = len(os.sched_getaffinity(0))
    for label, n_tok, threads in (("one_core", 64, 1), ("all_cores", cfg.T, n_all)):
        O.set_threads(threads)
        t0 = time.perf_counter()
        O.forward(h["x"][:n_tok], h["Wg"], h["W1"], h["W3"], h["W2"], cfg.k)
        el = time.perf_counter() - t0
        out[label] = dict(value=round(n_tok / el, 2), unit="tokens/s", cores=O.num_threads(),
                          sample=f"first {n_tok} of {cfg.T} tokens, {el:.2f} s")
    O.set_threads(n_all)
    return out


def small_runs(CONFIGS):
    """The small layers, each step preceded by a 512 MB read (MALL flush)."""
    import numpy as np
    import torch

    from sparse_mixture_experts_permute_amd import moe
    from sparse_mixture_experts_permute_amd.inputs import make_inputs
    out = []
    names = ["small_fp32"] + [n for n in CONFIGS if n.startswith("granularity_")]
    for name in names:
        c2 = CONFIGS[name]
        h = make_inputs(c2)
        d2 = {n: moe.tensor_from_numpy(a) for n, a in h.items() if a is not None}
        runs = [("method", {})]
        if c2.dtype == "f32" and name != "small_fp32":
            # the timed function of the granularity page, at its own shape
            runs.append(("page_function_sigmoid_gates_sigmoid_glu",
                         dict(gate_mode=moe.GATE_SIGMOID, activation=moe.ACT_GLU_SIGMOID)))
        for label, kw in runs:
            r2 = run_workload(c2, None, d2, 10, 3, flush_mb=512, min_warm_s=0.1, **kw)
            a = algorithmic(c2, r2["counts"])
            lt = r2["ms"] * 1e-3
            peak = PEAK_BF16_TFLOPS if c2.dtype == "bf16" else PEAK_F32_TFLOPS
            e = dict(workload=name, function=label, dtype=c2.dtype, T=c2.T, E=c2.E,
                     d_ff=c2.d_ff, k=c2.k, ms_per_step=round(r2["ms"], 4),
                     step_ms=r2["step_ms"], tokens_per_s=round(c2.T / lt, 1),
                     mfma_frac=round(a["layer_flop"] / lt / (peak * 1e12), 4),
                     mfma_peak_tflops=peak,
                     hbm_frac=round(a["layer_bytes"] / lt / (PEAK_HBM_GBS * 1e9), 4),
                     mall_flushed=True)
            page = PAGE_NUMPY_MS.get((c2.E, c2.d_ff, c2.k))
            if page and label != "method":
                e["page_numpy_2core_ms"] = {"median": page[0], "fastest": page[1]}
            log(f"{name} {label}: {r2['ms']:.4f} ms/step, mfma {e['mfma_frac']}, "
                f"hbm {e['hbm_frac']}")
            out.append(e)
        del d2
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the layer is "
              "measured on a single GPU", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from sparse_mixture_experts_permute_amd import moe
    from sparse_mixture_experts_permute_amd.inputs import CONFIGS, make_inputs

    moe.lib()
    cfg = CONFIGS[args.workload]
    fam_T = max(cfg.T, 8192 if cfg.d == 4096 and cfg.E == 8 else cfg.T)
    log(f"generating inputs for {cfg.name} (x for {fam_T} tokens)")
    t0 = time.perf_counter()
    host = make_inputs(cfg.with_(skew=0.0), T=fam_T)
    dev = {n: moe.tensor_from_numpy(a) for n, a in host.items() if a is not None}
    torch.cuda.synchronize()
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s")
    inout = args.layout == "inout"
    head_dev = transposed(dev) if inout else dev

    res = run_workload(cfg, host, head_dev, args.steps, args.warmup, inout=inout)
    if inout:
        del head_dev
        torch.cuda.empty_cache()
    rl, layer_fr = roofline_for(cfg, res)
    ms = res["ms"]
    value = cfg.T / (ms * 1e-3)
    stage = {s: round(float(v), 4) for s, v in zip(moe.STAGES, res["stage_ms"])}
    log(f"{cfg.name}: {ms:.3f} ms/step, {value:.0f} tokens/s, stages {stage}")
    counts = res["counts"]

    extra = []
    if not args.no_extra and cfg.d == 4096 and cfg.E == 8:
        for name, steps, flush in [("mixtral_prefill_T2048", 10, 0),
                                   ("mixtral_prefill_T8192_skew", 5, 0),
                                   ("mixtral_decode_T1", 20, 512),
                                   ("mixtral_decode_T8", 20, 512),
                                   ("mixtral_decode_T32", 20, 512),
                                   ("mixtral_decode_T128", 20, 512)]:
            if name == cfg.name:
                continue
            c2 = CONFIGS[name]
            r2 = run_workload(c2, host, dev, steps, 2, flush_mb=flush, graph=bool(flush), min_warm_s=0.25)
            rl2, lf2 = roofline_for(c2, r2)
            ms2 = r2["ms"]
            e = dict(workload=name, T=c2.T, ms_per_step=round(ms2, 4),
                     tokens_per_s=round(c2.T / (ms2 * 1e-3), 1),
                     stage_ms={s: round(float(v), 4) for s, v in zip(moe.STAGES,
                                                                      r2["stage_ms"])},
                     step_ms=r2["step_ms"], roofline=rl2, layer=lf2, mall_flushed=bool(flush),
                     expert_counts=count_summary(r2["counts"]))
            if "graph_ms" in r2:
                gms = r2["graph_ms"]
                e["graph_replay"] = dict(
                    ms_per_step=round(gms, 4), tokens_per_s=round(c2.T / (gms * 1e-3), 1),
                    hbm_frac=round(algorithmic(c2, r2["counts"])["layer_bytes"] / (gms * 1e-3)
                                   / (PEAK_HBM_GBS * 1e9), 4))
            if c2.skew:
                e["hot_expert_share"] = round(float(r2["counts"][0] / r2["counts"].sum()), 4)
            log(f"{name}: {ms2:.4f} ms/step, {e['tokens_per_s']} tokens/s")
            extra.append(e)
        # the headline shape and two decode steps with the other weight layout
        other = not inout
        odev = transposed(dev) if other else dev
        for name, steps, flush in [(cfg.name, 10, 0), ("mixtral_decode_T1", 20, 512),
                                   ("mixtral_decode_T128", 20, 512)]:
            c2 = CONFIGS[name]
            r2 = run_workload(c2, host, odev, steps, 2, flush_mb=flush, min_warm_s=0.25,
                              inout=other)
            rl2, lf2 = roofline_for(c2, r2)
            e = dict(workload=name, weight_layout="in_out" if other else "out_in", T=c2.T,
                     ms_per_step=round(r2["ms"], 4),
                     tokens_per_s=round(c2.T / (r2["ms"] * 1e-3), 1), step_ms=r2["step_ms"],
                     stage_ms={s_: round(float(v), 4) for s_, v in zip(moe.STAGES,
                                                                        r2["stage_ms"])},
                     roofline=rl2, layer=lf2, mall_flushed=bool(flush))
            log(f"{name} ({e['weight_layout']} weights): {r2['ms']:.4f} ms/step")
            extra.append(e)
        if other:
            del odev
            torch.cuda.empty_cache()
        # weight-only FP8 experts for decode steps (weights quantised once)
        l8 = moe.MoELayerFP8(dev["Wg"], dev["W1"], dev["W3"], dev["W2"], cfg.k)
        for name in ("mixtral_decode_T1", "mixtral_decode_T8", "mixtral_decode_T32",
                     "mixtral_decode_T128"):
            c2 = CONFIGS[name]
            r8 = run_fp8(c2, dev, 20, 3, 512, layer=l8)
            hit = int(np.count_nonzero(r8["counts"]))
            b8 = (hit * 3.0 * c2.d * c2.d_ff + 2.0 * c2.T * c2.d * 2 + c2.E * c2.d * 2
                  + 3 * c2.E * 4)
            e = dict(workload=name, weights="fp8_e4m3_per_expert_scale",
                     T=c2.T, ms_per_step=round(r8["ms"], 4),
                     tokens_per_s=round(c2.T / (r8["ms"] * 1e-3), 1),
                     layer=dict(hbm_frac=round(b8 / (r8["ms"] * 1e-3) / (PEAK_HBM_GBS * 1e9), 4),
                                algorithmic_bytes=b8, experts_hit=hit),
                     mall_flushed=True)
            log(f"{name} fp8 experts: {r8['ms']:.4f} ms/step, hbm {e['layer']['hbm_frac']}")
            extra.append(e)
        del l8
        torch.cuda.empty_cache()

    # the fine-grained layer with a shared expert (256 experts, top-8)
    if not args.no_extra and cfg.d == 4096 and cfg.E == 8:
        del dev
        torch.cuda.empty_cache()
        fcfg = CONFIGS["fine_shared_T8192"]
        log("generating inputs for the 256-expert layer")
        fhost = make_inputs(fcfg)
        fdev = {n: moe.tensor_from_numpy(a) for n, a in fhost.items() if a is not None}
        del fhost
        for name in ("fine_shared_T512", "fine_shared_T8192"):
            c2 = CONFIGS[name]
            r2 = run_workload(c2, None, fdev, 5, 2, min_warm_s=0.25)
            rl2, lf2 = roofline_for(c2, r2)
            ms2 = r2["ms"]
            e = dict(workload=name, T=c2.T, ms_per_step=round(ms2, 4),
                     tokens_per_s=round(c2.T / (ms2 * 1e-3), 1),
                     stage_ms={s_: round(float(v), 4) for s_, v in zip(moe.STAGES,
                                                                        r2["stage_ms"])},
                     step_ms=r2["step_ms"], roofline=rl2, layer=lf2, mall_flushed=False,
                     expert_counts=count_summary(r2["counts"]))
            log(f"{name}: {ms2:.4f} ms/step, {e['tokens_per_s']} tokens/s, "
                f"layer mfma {lf2['mfma_frac']} hbm {lf2['hbm_frac']}")
            extra.append(e)
        del fdev
        torch.cuda.empty_cache()
        dev = {n: moe.tensor_from_numpy(a) for n, a in host.items() if a is not None}

    # the variants beside the method, at the headline shape (whole-layer time)
    variants = []
    if not args.no_extra and cfg.d == 4096 and cfg.E == 8 and cfg.T == 8192:
        skew = CONFIGS["mixtral_prefill_T8192_skew"]
        cap = moe.capacity_mean(skew.T, skew.k, skew.E, 1.2)  # 1.2 x the mean load
        for label, c2, kw in [
                ("capacity_1.2x_mean_load_skew", skew, dict(capacity=cap)),
                ("gate_softmax_all", cfg, dict(gate_mode=moe.GATE_SOFTMAX_ALL)),
                ("sigmoid_gate_sigmoid_glu", cfg,
                 dict(gate_mode=moe.GATE_SIGMOID, activation=moe.ACT_GLU_SIGMOID)),
                # entropy-aware k: 3 slots, a token takes 3 or 2 experts
                ("entropy_k3_or_2", cfg.with_(k=3), dict(gate_mode=moe.GATE_ENTROPY))]:
            r3 = run_variant(c2, dev, 5, 2, **kw)
            flop = 6.0 * c2.d * c2.d_ff * r3["kept"]
            v = dict(variant=label, workload=c2.name, options=kw, ms_per_step=round(r3["ms"], 4),
                     tokens_per_s=round(c2.T / (r3["ms"] * 1e-3), 1),
                     pairs_kept=r3["kept"], pairs=c2.T * c2.k,
                     layer_mfma_frac=round(flop / (r3["ms"] * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
                                           4))
            log(f"variant {label}: {r3['ms']:.3f} ms/step, kept {r3['kept']} of {c2.T * c2.k}")
            variants.append(v)

    # the 512-wide layers the pages time: the small fp32 layer and the 7-config
    # granularity sweep in fp32 and bf16 (weights fit the 256 MB MALL, so a
    # 512 MB read evicts them before every step), and the pages' own function
    # (sigmoid route weights, sigmoid-gated experts) at the sweep's shapes
    small = []
    if not args.no_extra:
        del dev
        torch.cuda.empty_cache()
        small = small_runs(CONFIGS)
        dev = None

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(cfg, host, args.cpu_tokens)
        if not args.no_extra:
            cpu["granularity_E8_k2_f32"] = cpu_small(CONFIGS["granularity_E8_k2_f32"])
        log(f"cpu baseline: {cpu}")

    out = {
        "metric": "MoE-layer tokens/s; % bf16 MFMA peak (prefill) and % HBM BW (decode)",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) tokens, N(0,1/fan_in) expert weights, "
                "router N(0,0.02^2), bf16-rounded)",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "E": cfg.E, "d_ff": cfg.d_ff,
                   "k": cfg.k, "d_ff_shared": cfg.d_ff_shared, "skew": cfg.skew,
                   "global_batch": cfg.T, "parallelism": "single GPU"},
        "roofline": rl,
        "layer_roofline": layer_fr,
        "step_ms": res["step_ms"],
        "stage_ms": stage,
        "expert_counts": count_summary(counts),
        "cpu_baseline": cpu,
        "weight_layout": "in_out" if inout else "out_in",
        "extra": extra,
        "variants": variants,
        "small_layers": small,
        "wall_s_timed": round(res["wall_s"], 3),
        "timing": "HIP events on the stream the kernels run on: ms_per_step over back-to-back "
                  "moe_forward calls; step_ms (median, fastest) from the same steps again, "
                  "each between events of its own; stage and kernel times from a pass through "
                  "moe_forward_timed (events at every stage boundary)",
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
