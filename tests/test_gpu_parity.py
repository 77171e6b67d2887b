"""Parity of the HIP path (through the C ABI) with the CPU oracle, on an MI355X.

Bars: routing indices, counts, offsets and the permutation bit-exact against the
oracle run on the GPU's own router scores; gates within 1e-6; y within 1e-4
relative L2 (fp32 path) or 1e-2 (bf16 path) against the oracle on the same
bf16-rounded inputs.  Small workloads are compared element by element; the
full-size workloads are compared on sampled rows the oracle evaluates one by
one, plus the whole routing and permutation.
"""
import math

import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_mixture_experts_permute_amd import moe
from sparse_mixture_experts_permute_amd.inputs import (CONFIGS, LayerConfig, bf16_bits_to_f32,
                                                       make_inputs, shared_tuple)

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 1e-2}


def say(msg):
    print(f"\n[gpu-parity] {msg}", flush=True)


def f64(a):
    return (bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)


def rel_l2(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


# ---------------------------------------------------------------- inputs ---

_SLOT = {"key": None, "host": None, "dev": None}


def family(cfg: LayerConfig, T_max: int):
    """Host and device inputs for a weight family, generated once for the
    largest token count (smaller T are prefixes of x)."""
    key = (cfg.d, cfg.E, cfg.d_ff, cfg.k, cfg.dtype, cfg.d_ff_shared, cfg.seed, T_max)
    if _SLOT["key"] != key:
        _SLOT.update(key=None, host=None, dev=None)
        torch.cuda.empty_cache()
        host = make_inputs(cfg.with_(skew=0.0), T=T_max)
        dev = {n: moe.tensor_from_numpy(a) for n, a in host.items() if a is not None}
        _SLOT.update(key=key, host=host, dev=dev)
    return _SLOT["host"], _SLOT["dev"]


def case(cfg: LayerConfig, T_max=None):
    host, dev = family(cfg, T_max or cfg.T)
    T = cfg.T
    h = dict(host)
    d = dict(dev)
    h["x"], d["x"] = host["x"][:T], dev["x"][:T].contiguous()
    if cfg.skew:
        b = np.zeros(cfg.E, np.float32)
        b[0] = cfg.skew
        h["bias"], d["bias"] = b, torch.from_numpy(b).cuda()
    else:
        h["bias"], d["bias"] = None, None
    return h, d


def layer(d, cfg):
    sh = (d["Ws1"], d["Ws3"], d["Ws2"]) if cfg.d_ff_shared else None
    return moe.MoELayer(d["Wg"], d["W1"], d["W3"], d["W2"], cfg.k, d["bias"], sh)


def gamma(n):
    u = 2.0 ** -24
    return n * u / (1 - n * u)


def check_routing(h, cfg, idx, gate, logits):
    """idx bit-exact and gates within 1e-6 vs the oracle on the GPU's scores;
    GPU scores within the fp32 dot-product error bound of the oracle's own."""
    lg = logits.double().cpu().numpy()
    idx = idx.cpu().numpy()
    gate = gate.cpu().numpy()
    idx_ref = O.topk(lg, cfg.k)
    np.testing.assert_array_equal(idx, idx_ref)
    gate_ref = O.gate(lg, idx_ref)
    assert np.max(np.abs(gate - gate_ref)) <= 1e-6
    own = O.logits(h["x"], h["Wg"], h["bias"])
    S = np.abs(f64(h["x"])) @ np.abs(f64(h["Wg"])).T
    bound = 1.01 * gamma(cfg.d + 2) * S + 1e-7
    assert np.all(np.abs(lg - own) <= bound)
    # tokens whose own-score routing differs must be near-ties
    idx_own = O.topk(own, cfg.k)
    diff = np.nonzero(np.any(idx_own != idx, axis=1))[0]
    for t in diff:
        s = np.sort(own[t])[::-1][:cfg.k + 1]
        gap = float(np.min(s[:-1] - s[1:])) if len(s) > 1 else 0.0
        assert gap < 1e-4 * np.max(np.abs(own[t])), f"token {t} flipped with gap {gap}"
    return idx_ref, gate_ref, len(diff)


def check_permutation(idx, E, counts, offsets, perm, inv):
    c, o, p, i = O.permute(idx, E)
    np.testing.assert_array_equal(counts.cpu().numpy(), c)
    np.testing.assert_array_equal(offsets.cpu().numpy(), o)
    np.testing.assert_array_equal(perm.cpu().numpy(), p)
    np.testing.assert_array_equal(inv.cpu().numpy(), i)


# ---------------------------------------------------------- small, full ---

SMALL = ["small_fp32"] + [n for n in CONFIGS if n.startswith("granularity_")]


@pytest.mark.parametrize("name", SMALL)
def test_forward_full_output(name):
    cfg = CONFIGS[name]
    say(f"forward full output {name} T={cfg.T} E={cfg.E} d_ff={cfg.d_ff} k={cfg.k} {cfg.dtype}")
    h, d = case(cfg)
    L = layer(d, cfg)
    y = L(d["x"])
    torch.cuda.synchronize()
    inter = {kk: v.cpu() for kk, v in L.intermediates(cfg.T).items()}
    idx_ref, _, _ = check_routing(h, cfg, inter["idx"], inter["gate"], inter["logits"])
    check_permutation(idx_ref, cfg.E, inter["counts"], inter["offsets"], inter["perm"],
                      inter["inv"])
    ref = O.forward(h["x"], h["Wg"], h["W1"], h["W3"], h["W2"], cfg.k, bias=h["bias"],
                    logits_in=inter["logits"].double().numpy())
    got = f64(moe.tensor_to_numpy(y))
    err = rel_l2(got, ref["y"])
    say(f"{name}: rel-L2 {err:.3e} (bar {TOL[cfg.dtype]})")
    assert err <= TOL[cfg.dtype]


@pytest.mark.parametrize("name", ["small_fp32", "granularity_E128_k8_bf16",
                                  "granularity_E1_k1_f32"])
def test_route_entry_point(name):
    cfg = CONFIGS[name]
    say(f"moe_route {name}")
    h, d = case(cfg)
    idx, gate, logits = moe.route(d["x"], d["Wg"], cfg.k, d["bias"])
    torch.cuda.synchronize()
    idx_ref, _, nflip = check_routing(h, cfg, idx, gate, logits)
    assert np.allclose(gate.sum(1).cpu().numpy(), 1.0, atol=cfg.k * 2.0 ** -23)
    counts, offsets, perm, inv = moe.permute(idx, cfg.E)
    torch.cuda.synchronize()
    check_permutation(idx_ref, cfg.E, counts, offsets, perm, inv)
    assert int(counts.sum()) == cfg.T * cfg.k


# ----------------------------------------------------- full size, sampled ---

BIG = ["mixtral_prefill_T2048", "mixtral_prefill_T8192", "mixtral_prefill_T2048_skew",
       "mixtral_prefill_T8192_skew", "mixtral_decode_T1", "mixtral_decode_T8",
       "mixtral_decode_T32", "mixtral_decode_T128", "fine_shared_T512", "fine_shared_T8192"]


def sample_rows(T, rng, n=24):
    rows = {0, T - 1}
    rows |= set(rng.choice(T, size=min(T, n), replace=False).tolist())
    return sorted(rows)


@pytest.mark.parametrize("name", BIG)
def test_forward_sampled_full_size(name):
    cfg = CONFIGS[name]
    say(f"forward sampled {name} T={cfg.T} d={cfg.d} E={cfg.E} d_ff={cfg.d_ff} k={cfg.k} "
        f"shared={cfg.d_ff_shared} skew={cfg.skew}")
    h, d = case(cfg, T_max=8192)
    L = layer(d, cfg)
    y = L(d["x"])
    torch.cuda.synchronize()
    inter = {kk: v.cpu() for kk, v in L.intermediates(cfg.T).items()}
    idx_ref, gate_ref, nflip = check_routing(h, cfg, inter["idx"], inter["gate"],
                                             inter["logits"])
    check_permutation(idx_ref, cfg.E, inter["counts"], inter["offsets"], inter["perm"],
                      inter["inv"])
    counts = inter["counts"].numpy()
    if cfg.skew:
        say(f"{name}: hot-expert share {counts[0] / counts.sum():.3f}")
    rng = np.random.default_rng(7)
    rows = set(sample_rows(cfg.T, rng))
    # Whole tiles: every token of the last non-empty expert (its tiles end the
    # tile order, so they are the ones a last-round K split cuts into parts,
    # over every column block), every token in the last two 256-row tiles of
    # the most-loaded expert (its ragged last tile) and a few tokens of the
    # least-loaded one
    perm = inter["perm"].numpy()
    offsets = inter["offsets"].numpy()
    nz = np.nonzero(counts)[0]
    elast, emax, emin = nz[-1], int(np.argmax(counts)), nz[np.argmin(counts[nz])]
    tiles = {}  # (expert, 256-row tile of its slots) -> tokens
    for e, first in ((elast, 0), (emax, max(0, (counts[emax] - 1) // 256 - 1) * 256)):
        for s_ in range(offsets[e] + first, offsets[e + 1]):
            t = int(perm[s_]) // cfg.k
            tiles.setdefault((int(e), (s_ - offsets[e]) // 256), []).append(t)
            rows.add(t)
    rows |= set(np.nonzero(np.any(idx_ref == emin, axis=1))[0][:4].tolist())
    rows = sorted(rows)
    ref = O.forward_rows(h["x"], h["W1"], h["W3"], h["W2"], rows, idx_ref[rows], gate_ref[rows],
                         shared=shared_tuple(h))
    got = f64(moe.tensor_to_numpy(y[rows]))
    err = rel_l2(got, ref)
    pos = {t: i for i, t in enumerate(rows)}
    worst, worst_tile = 0.0, None
    for key, toks in tiles.items():
        sel = [pos[t] for t in toks]
        e_t = rel_l2(got[sel], ref[sel])
        if e_t > worst:
            worst, worst_tile = e_t, key
    say(f"{name}: {len(rows)} rows ({len(tiles)} whole m-tiles of experts {elast} and {emax}) "
        f"rel-L2 {err:.3e}; worst m-tile {worst_tile} {worst:.3e}; own-score route flips {nflip}")
    assert err <= TOL[cfg.dtype]
    assert worst <= TOL[cfg.dtype]


@pytest.mark.parametrize("name", ["mixtral_prefill_T2048", "fine_shared_T512",
                                  "mixtral_decode_T1"])
def test_deterministic(name):
    cfg = CONFIGS[name]
    say(f"determinism {name}")
    h, d = case(cfg, T_max=8192)
    L = layer(d, cfg)
    y1 = L(d["x"]).clone()
    # the second call starts from a workspace full of garbage (stale arrival
    # counters and partial tiles of the down GEMM's last-round split)
    L._ws.fill_(0x5A)
    y2 = L(d["x"]).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


# ------------------------------------------------------------ edge cases ---

EDGE = [
    # (label, T, d, E, d_ff, k, dtype, d_ff_shared, bias)
    ("T1", 1, 128, 8, 128, 2, "bf16", 0, None),
    ("T7_ragged", 7, 128, 8, 192, 2, "f32", 0, None),
    ("T129_ragged_tile", 129, 192, 6, 128, 3, "bf16", 0, None),
    ("T513", 513, 64, 4, 64, 2, "f32", 0, None),
    ("E1_k1_dense", 65, 128, 1, 256, 1, "bf16", 0, None),
    ("k_equals_E", 40, 128, 4, 128, 4, "f32", 0, None),
    ("all_to_one_expert", 300, 128, 8, 128, 1, "bf16", 0, ("hot", 3, 100.0)),
    ("all_to_one_k2", 300, 128, 8, 128, 2, "f32", 0, ("hot", 5, 100.0)),
    ("E256_mostly_empty", 5, 64, 256, 64, 1, "bf16", 0, None),
    ("E256_k8_shared", 33, 128, 256, 64, 8, "bf16", 192, None),
    ("shared_f32", 45, 128, 16, 64, 4, "f32", 128, None),
    ("N_tail", 70, 192, 5, 192, 2, "bf16", 0, None),
    # weight-streaming path (few rows per expert)
    ("skinny_T5", 5, 256, 4, 256, 2, "bf16", 0, None),
    ("skinny_hot_expert_two_passes", 70, 256, 4, 512, 2, "bf16", 0, ("hot", 2, 100.0)),
    ("skinny_shared", 40, 256, 8, 256, 2, "bf16", 256, None),
    ("skinny_E256_k8", 64, 512, 256, 256, 8, "bf16", 0, None),
    # long K: d = 5120 with 64-row and 256-row tiles, a 14336-wide shared expert
    ("K5120_bm64", 64, 5120, 4, 256, 2, "bf16", 0, None),
    ("K5120_bm256", 256, 5120, 2, 256, 1, "bf16", 0, None),
    ("shared_K14336", 96, 256, 4, 256, 2, "bf16", 14336, None),
    # every tile of a small down projection split into 16 K planes
    ("kplanes_down", 64, 256, 4, 14336, 2, "bf16", 0, None),
    # vector-ALU weight streaming (at most four tokens, K a multiple of 2048)
    ("gemv_T1", 1, 2048, 8, 2048, 2, "bf16", 0, None),
    ("gemv_T2_K6144_shared", 2, 2048, 4, 6144, 2, "bf16", 2048, None),
    ("gemv_T4_hot_expert", 4, 2048, 8, 4096, 2, "bf16", 0, ("hot", 1, 100.0)),
    # 256-row tiles with under 512 rows per expert: 64-row tiles for short remainders
    # (one or two remainder tiles, remainders over 128 rows kept whole, experts below
    # 256 rows and at exactly 256, K planes)
    ("split_remainders_E4_k1", 1300, 256, 4, 256, 1, "bf16", 0, None),
    ("split_ceil_E4_k1", 1800, 256, 4, 256, 1, "bf16", 0, None),
    ("split_below_256_E12", 3000, 256, 12, 256, 1, "bf16", 0, None),
    ("split_kplanes", 1100, 256, 4, 2048, 1, "bf16", 0, None),
    ("split_shared", 1500, 256, 4, 256, 1, "bf16", 256, None),
    # the one-launch router (a wavefront per token, up to 2048 tokens): its largest expert count and k,
    # an expert count that leaves part of its 32-wide register block unused, and the first batch past
    # it (feature-split scores plus a top-k launch)
    ("router_wave_T2048_E32_k16", 2048, 512, 32, 256, 16, "bf16", 0, None),
    ("router_wave_E17_f32", 300, 512, 17, 256, 3, "f32", 0, None),
    ("router_split_T2049_E17_f32", 2049, 512, 17, 256, 3, "f32", 0, None),
    # one token routed inside the SwiGLU weight-streaming kernel (E * d <= 65536)
    ("routed_T1_E32_k4_hot", 1, 2048, 32, 2048, 4, "bf16", 0, ("hot", 31, 100.0)),
    ("routed_T1_E16_shared_limit", 1, 4096, 16, 2048, 2, "bf16", 4096, None),
    # d = 6144: the routed kernel whose four waves split K (the per-wavefront one takes d of
    # 2048 or 4096)
    ("routed_T1_d6144", 1, 6144, 8, 2048, 2, "bf16", 0, None),
    # one token on a dense layer (E = k = 1) and on every expert (k = E)
    ("routed_T1_dense_E1", 1, 2048, 1, 2048, 1, "bf16", 0, None),
    ("routed_T1_k_equals_E", 1, 2048, 8, 4096, 8, "bf16", 0, None),
]


@pytest.mark.parametrize("case_", EDGE, ids=[c[0] for c in EDGE])
def test_edge_cases(case_):
    label, T, d, E, dff, k, dt, dffs, bias = case_
    say(f"edge {label}: T={T} d={d} E={E} d_ff={dff} k={k} {dt} shared={dffs}")
    cfg = LayerConfig(label, T, d, E, dff, k, dt, d_ff_shared=dffs, seed=1234)
    h = make_inputs(cfg)
    if bias is not None:
        b = np.zeros(E, np.float32)
        b[bias[1]] = bias[2]
        h["bias"] = b
    d_ = {n: moe.tensor_from_numpy(a) for n, a in h.items() if a is not None}
    d_.setdefault("bias", None)
    L = layer(d_, cfg)
    y = L(d_["x"])
    torch.cuda.synchronize()
    inter = {kk: v.cpu() for kk, v in L.intermediates(T).items()}
    idx_ref, _, _ = check_routing(h, cfg, inter["idx"], inter["gate"], inter["logits"])
    check_permutation(idx_ref, E, inter["counts"], inter["offsets"], inter["perm"], inter["inv"])
    ref = O.forward(h["x"], h["Wg"], h["W1"], h["W3"], h["W2"], k, bias=h["bias"],
                    shared=shared_tuple(h), logits_in=inter["logits"].double().numpy())
    got = f64(moe.tensor_to_numpy(y))
    err = rel_l2(got, ref["y"])
    # every row on its own as well: a wrong tile of a few rows (a light
    # remainder tile, say) hardly moves the whole output's error
    row_err = max((rel_l2(got[t], ref["y"][t]) for t in range(T)), default=0.0)
    say(f"edge {label}: rel-L2 {err:.3e}, worst row {row_err:.3e}")
    assert err <= TOL[dt]
    assert row_err <= 3 * TOL[dt]
    if label.startswith(("kplanes", "gemv_T1", "routed", "split")):
        # a workspace full of garbage gives the same bits
        y1 = y.clone()
        L._ws.fill_(0x5A)
        y2 = L(d_["x"])
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


# Exact ties in the router scores: duplicated router rows (experts 3 and 5, 1
# and 6) score bit-identically, and biases put them on top, so top-k must
# break each tie to the lower index (3 before 5, then 1 before 6), on every
# router path: one token routed inside the SwiGLU kernel, the tiny decode
# path, the one-launch router, the feature-split router with its top-k launch,
# the router with its weights in LDS, and the many-expert score kernel.
TIES = [
    # (label, T, d, E, k)
    ("T1_fused", 1, 2048, 8, 3),
    ("T3_tiny", 3, 512, 8, 3),
    ("T64_wave", 64, 512, 8, 3),
    ("T64_wave_k1", 64, 512, 8, 1),
    ("T3000_split", 3000, 512, 16, 3),
    ("T4096_lds", 4096, 2048, 16, 3),
    ("T64_E64_scores", 64, 512, 64, 3),
]


@pytest.mark.parametrize("case_", TIES, ids=[c[0] for c in TIES])
def test_router_exact_ties(case_):
    label, T, dm, E, k = case_
    say(f"router ties {label}: T={T} d={dm} E={E} k={k}")
    cfg = LayerConfig(f"ties_{label}", T, dm, E, 256, k, "bf16", seed=7)
    h = make_inputs(cfg)
    h["Wg"] = h["Wg"].copy()
    h["Wg"][5] = h["Wg"][3]
    h["Wg"][6] = h["Wg"][1]
    b = np.zeros(E, np.float32)
    b[3] = b[5] = 40.0  # far above any score of these inputs
    b[1] = b[6] = 20.0
    h["bias"] = b
    d_ = {n: moe.tensor_from_numpy(a) for n, a in h.items() if a is not None}
    L = layer(d_, cfg)
    L(d_["x"])
    torch.cuda.synchronize()
    it = {kk: v.cpu() for kk, v in L.intermediates(T).items()}
    lg = it["logits"]
    assert torch.equal(lg[:, 3], lg[:, 5]) and torch.equal(lg[:, 1], lg[:, 6])
    idx = it["idx"].numpy()
    want = [3, 5, 1][:k]
    assert (idx == np.array(want, np.int32)).all(), idx[:4]
    idx_ref, _, _ = check_routing(h, cfg, it["idx"], it["gate"], it["logits"])
    check_permutation(idx_ref, E, it["counts"], it["offsets"], it["perm"], it["inv"])


def test_zero_tokens():
    say("edge T=0")
    cfg = LayerConfig("empty", 4, 64, 4, 64, 2, "bf16")
    h = make_inputs(cfg)
    d_ = {n: moe.tensor_from_numpy(a) for n, a in h.items() if a is not None}
    L = moe.MoELayer(d_["Wg"], d_["W1"], d_["W3"], d_["W2"], 2)
    x0 = d_["x"][:0]
    y = L(x0)
    torch.cuda.synchronize()
    assert y.shape == (0, 64)


def test_permute_extremes():
    say("permute extremes")
    rng = np.random.default_rng(3)
    for (T, E, k, mode) in [(4096, 256, 8, "random"), (5000, 8, 2, "one"), (1, 256, 1, "random"),
                            (257, 64, 4, "random"), (8192, 16, 2, "two")]:
        if mode == "random":
            idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(
                np.int32)
        elif mode == "one":
            idx = np.tile(np.array([3, 0][:k], np.int32), (T, 1))
        else:
            idx = np.tile(np.array([E - 1, 0], np.int32), (T, 1))
        di = torch.from_numpy(idx).cuda()
        counts, offsets, perm, inv = moe.permute(di, E)
        torch.cuda.synchronize()
        check_permutation(idx, E, counts, offsets, perm, inv)
