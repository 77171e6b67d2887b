"""Parity of the variants beside the method (gate modes, the sigmoid-gated
expert, the expert capacity limit) with the CPU oracle, on an MI355X.

Same bars as the method's own parity tests: routing indices, counts, offsets,
the permutation and the dropped pairs bit-exact against the oracle run on the
GPU's router scores; gates within 1e-6; y within 1e-4 (fp32) or 1e-2 (bf16)
relative L2.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_mixture_experts_permute_amd import moe
from sparse_mixture_experts_permute_amd.inputs import LayerConfig, bf16_bits_to_f32, make_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 1e-2}


def say(msg):
    print(f"\n[gpu-variants] {msg}", flush=True)


def f64(a):
    return (bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)


def rel_l2(got, ref):
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def inputs(T, d, E, dff, k, dtype, dffs=0, seed=7, skew=0.0):
    cfg = LayerConfig("variant", T, d, E, dff, k, dtype, d_ff_shared=dffs, skew=skew, seed=seed)
    h = make_inputs(cfg)
    dev = {n: moe.tensor_from_numpy(a) for n, a in h.items() if a is not None}
    dev["bias"] = torch.from_numpy(h["bias"]).cuda() if h["bias"] is not None else None
    return cfg, h, dev


# (label, T, d, E, d_ff, k, dtype, d_ff_shared, skew, gate_mode, activation, capacity[,
#  seed])
CASES = [
    ("softmax_all_bf16", 300, 256, 8, 512, 2, "bf16", 0, 0.0, 1, 0, None),
    ("sigmoid_gate_glu_f32", 200, 128, 6, 256, 2, "f32", 0, 0.0, 2, 1, None),
    ("numpy_function_E32_bf16", 512, 512, 32, 1024, 2, "bf16", 0, 0.0, 2, 1, None),
    ("glu_shared_bf16", 96, 256, 8, 256, 2, "bf16", 256, 0.0, 0, 1, None),
    ("capacity_20_bf16", 300, 256, 8, 512, 2, "bf16", 0, 1.5, 0, 0, 20),
    ("capacity_1_f32", 64, 128, 4, 128, 3, "f32", 0, 0.0, 0, 0, 1),
    ("capacity_0_shared_bf16", 40, 256, 8, 256, 2, "bf16", 256, 0.0, 0, 0, 0),
    ("capacity_multiblock_bf16", 5000, 128, 16, 128, 2, "bf16", 0, 2.0, 0, 0, 300),
    ("capacity_decode_T3_bf16", 3, 2048, 8, 2048, 2, "bf16", 0, 0.0, 1, 1, 1),
    ("capacity_page_cf_bf16", 512, 256, 8, 256, 2, "bf16", 0, 3.0, 0, 0, "page"),
    ("capacity_cf_0.3_bf16", 512, 256, 8, 256, 2, "bf16", 0, 3.0, 2, 0, 0.3),
    # combine over more than eight pairs per token (rows loaded eight at a time):
    # k = 16 with dropped pairs, and k = 12 (a partly filled second group) with
    # a shared expert
    ("combine_k16_cap_bf16", 64, 256, 64, 256, 16, "bf16", 0, 0.0, 0, 0, 10),
    ("combine_k12_shared_f32", 40, 128, 32, 128, 12, "f32", 64, 0.0, 0, 0, None),
    # decode steps (T <= 4, E <= 64): top-k and grouping in one launch
    ("tiny_sigmoid_skew_f32", 3, 128, 8, 256, 2, "f32", 0, 1.5, 2, 0, None),
    ("tiny_E64_k16_cap3_bf16", 4, 256, 64, 256, 16, "bf16", 0, 0.0, 0, 0, 3),
    ("tiny_E20_k3_shared_f32", 4, 192, 20, 128, 3, "f32", 64, 0.0, 1, 1, None),
    # weight-streaming down projection with the combine inside, every pair dropped
    ("capacity_0_gemv_T2_bf16", 2, 2048, 8, 2048, 2, "bf16", 0, 0.0, 0, 0, 0),
    # entropy-aware k ("Mixtral 8x7B model architecture" 4.1): 3 or 2 experts per token
    ("entropy_k3_bf16", 300, 256, 8, 512, 3, "bf16", 0, 0.0, 3, 0, None),
    ("entropy_k3_shared_cap_f32", 150, 128, 6, 128, 3, "f32", 64, 0.0, 3, 0, 40),
    ("entropy_decode_T4_bf16", 4, 2048, 8, 2048, 3, "bf16", 0, 0.0, 3, 0, None),
    # one token, routed by the SwiGLU weight-streaming kernel itself (E * d <= 65536)
    ("routed_T1_skew_softmax_all_glu_bf16", 1, 2048, 8, 2048, 2, "bf16", 0, 1.5, 1, 1, None),
    ("routed_T1_E32_k4_cap1_bf16", 1, 2048, 32, 2048, 4, "bf16", 0, 0.0, 0, 0, 1),
    ("routed_T1_sigmoid_shared_bf16", 1, 2048, 16, 2048, 2, "bf16", 2048, 0.0, 2, 0, None),
    ("routed_T1_cap0_bf16", 1, 4096, 8, 2048, 2, "bf16", 0, 0.0, 0, 0, 0),
    ("routed_T1_entropy_k2_bf16", 1, 4096, 8, 2048, 3, "bf16", 0, 0.0, 3, 0, None),
    ("routed_T1_entropy_k3_bf16", 1, 4096, 8, 2048, 3, "bf16", 0, 0.0, 3, 0, None, 41),
    # the same section's listing as printed: one k for the batch, its largest per-token k
    ("entropy_batch_k3_bf16", 300, 256, 8, 512, 3, "bf16", 0, 0.0, 4, 0, None),
    ("entropy_batch_low_f32", 200, 128, 8, 256, 3, "f32", 0, 4.0, 4, 0, None),
    ("entropy_batch_cap_shared_bf16", 150, 256, 6, 256, 3, "bf16", 128, 0.0, 4, 1, 40),
    ("entropy_batch_decode_T3_bf16", 3, 2048, 8, 2048, 3, "bf16", 0, 0.0, 4, 0, None),
    ("routed_T1_entropy_batch_bf16", 1, 4096, 8, 2048, 3, "bf16", 0, 0.0, 4, 0, None, 41),
]


@pytest.mark.parametrize("c", CASES, ids=[c[0] for c in CASES])
def test_variant_forward(c):
    label, T, d, E, dff, k, dtype, dffs, skew, gm, act, cap = c[:12]
    seed = c[12] if len(c) > 12 else 7
    cfg, h, dev = inputs(T, d, E, dff, k, dtype, dffs, skew=skew, seed=seed)
    if cap == "page":
        cap = moe.capacity(T, k, 1.2)        # min(k*T, floor(1.2*T))
    elif isinstance(cap, float):
        cap = moe.capacity(T, k, cap)
    capacity = -1 if cap is None else cap
    say(f"{label}: T={T} d={d} E={E} d_ff={dff} k={k} {dtype} shared={dffs} gate={gm} "
        f"act={act} capacity={capacity}")
    sh = (dev["Ws1"], dev["Ws3"], dev["Ws2"]) if dffs else None
    L = moe.MoELayer(dev["Wg"], dev["W1"], dev["W3"], dev["W2"], k, dev["bias"], sh,
                     gate_mode=gm, activation=act, capacity=capacity)
    y = L(dev["x"])
    torch.cuda.synchronize()
    it = {n: v.cpu().numpy() for n, v in L.intermediates(T).items()}
    lg = it["logits"].astype(np.float64)
    if gm in (O.GATE_ENTROPY, O.GATE_ENTROPY_BATCH):
        # the per-token k is a decision on the entropy (fp32 on the GPU, fp64
        # here, from the same scores): these inputs keep every token clear of
        # the threshold, so both sides decide alike
        H = O.entropy(lg)
        assert np.min(np.abs(H - O.ENTROPY_THRESHOLD)) > 1e-4
        say(f"{label}: {int(np.sum(H > O.ENTROPY_THRESHOLD))} of {T} tokens take k={k}")
    ref = O.forward(h["x"], h["Wg"], h["W1"], h["W3"], h["W2"], k, bias=h["bias"],
                    shared=(h["Ws1"], h["Ws3"], h["Ws2"]) if dffs else None, logits_in=lg,
                    gate_mode=gm, act=act, capacity=cap)
    np.testing.assert_array_equal(it["idx"], ref["idx"])
    assert np.max(np.abs(it["gate"] - ref["gate"])) <= 1e-6
    np.testing.assert_array_equal(it["counts"], ref["counts"])
    np.testing.assert_array_equal(it["offsets"], ref["offsets"])
    kept = int(ref["offsets"][E])
    np.testing.assert_array_equal(it["perm"][:kept], ref["perm"])
    np.testing.assert_array_equal(it["inv"], ref["inv"])
    got = f64(moe.tensor_to_numpy(y))
    dropped = int(np.sum(ref["inv"] < 0))
    if not np.any(ref["y"]):
        say(f"{label}: every pair dropped, y must be zero")
        assert not np.any(got)
        return
    err = rel_l2(got, ref["y"])
    say(f"{label}: dropped {dropped} of {T * k} pairs, rel-L2 {err:.3e} (bar {TOL[dtype]})")
    assert err <= TOL[dtype]


def test_route_entropy():
    # entropy-aware k through moe_route_ex against the oracle on the GPU's
    # scores.  A token whose fp64 entropy lies within 1e-4 of the threshold may
    # take either k (the GPU decides in fp32); its experts and gates must then
    # match the oracle's routing with that k.
    cfg, h, dev = inputs(777, 512, 16, 64, 3, "bf16", seed=12)
    idx, gate, logits = moe.route(dev["x"], dev["Wg"], 3, None, gate_mode=moe.GATE_ENTROPY)
    torch.cuda.synchronize()
    lg = logits.double().cpu().numpy()
    gi, gg = idx.cpu().numpy(), gate.cpu().numpy()
    H = O.entropy(lg)
    ri, rg = O.route_entropy(lg, 3)
    hi_i, hi_g = O.route_entropy(lg, 3, threshold=-1.0)    # k experts for every token
    lo_i, lo_g = O.route_entropy(lg, 3, threshold=1e30)    # k - 1 for every token
    near = np.abs(H - O.ENTROPY_THRESHOLD) < 1e-4
    for t in range(lg.shape[0]):
        if near[t]:
            ok_i = hi_i[t] if gi[t, 2] >= 0 else lo_i[t]
            ok_g = hi_g[t] if gi[t, 2] >= 0 else lo_g[t]
        else:
            ok_i, ok_g = ri[t], rg[t]
        np.testing.assert_array_equal(gi[t], ok_i)
        assert np.max(np.abs(gg[t] - ok_g)) <= 1e-6
    n3 = int(np.sum(gi[:, 2] >= 0))
    say(f"moe_route_ex entropy: {n3} of {lg.shape[0]} tokens take 3 experts, {int(near.sum())} "
        f"near the threshold")
    assert 0 < n3 < lg.shape[0]


def check_route(lg, gi, gg, k, gm):
    """GPU top-k and gates against the oracle on the GPU's scores; with the
    entropy rule a token within 1e-4 of the threshold may take either k."""
    if gm != O.GATE_ENTROPY:
        idx_ref = O.topk(lg, k)
        np.testing.assert_array_equal(gi, idx_ref)
        return float(np.max(np.abs(gg - O.gate_mode(lg, idx_ref, gm))))
    H = O.entropy(lg)
    ri, rg = O.route_entropy(lg, k)
    hi_i, hi_g = O.route_entropy(lg, k, threshold=-1.0)
    lo_i, lo_g = O.route_entropy(lg, k, threshold=1e30)
    near = np.abs(H - O.ENTROPY_THRESHOLD) < 1e-4
    ri, rg = ri.copy(), rg.copy()
    full = gi[:, k - 1] >= 0
    ri[near & full], rg[near & full] = hi_i[near & full], hi_g[near & full]
    ri[near & ~full], rg[near & ~full] = lo_i[near & ~full], lo_g[near & ~full]
    np.testing.assert_array_equal(gi, ri)
    return float(np.max(np.abs(gg - rg)))


# many tokens with a small router: the score kernel also runs top-k and the
# gate (router weights in LDS up to E * d * size = 64 KB and E <= 16, else the
# register-tiled score kernel with one feature slice)
ROUTE_FUSED = [
    # (label, T, d, E, k, dtype, gate_mode, skew)
    ("lds_E8_k2_skew_bf16", 4100, 4096, 8, 2, "bf16", 0, 1.5),
    ("lds_E8_k8_softmax_all_bf16", 4096, 2048, 8, 8, "bf16", 1, 0.0),
    ("lds_E16_k4_sigmoid_f32", 4096, 1024, 16, 4, "f32", 2, 0.0),
    ("lds_E16_k3_entropy_bf16", 4111, 2048, 16, 3, "bf16", 3, 0.0),
    ("narrow_E32_k16_bf16", 8192, 512, 32, 16, "bf16", 0, 0.0),
    ("narrow_E24_k3_entropy_f32", 8200, 256, 24, 3, "f32", 3, 0.0),
    ("narrow_E12_k2_sigmoid_skew_bf16", 9000, 384, 12, 2, "bf16", 2, 2.0),
]


@pytest.mark.parametrize("c", ROUTE_FUSED, ids=[c[0] for c in ROUTE_FUSED])
def test_route_fused_topk(c):
    label, T, d, E, k, dtype, gm, skew = c
    cfg = LayerConfig("route", T, d, E, 64, k, dtype, skew=skew, seed=21)
    h = make_inputs(cfg, with_weights=False)
    x = moe.tensor_from_numpy(h["x"])
    Wg = moe.tensor_from_numpy(h["Wg"])
    bias = torch.from_numpy(h["bias"]).cuda() if h["bias"] is not None else None
    idx, gate, logits = moe.route(x, Wg, k, bias, gate_mode=gm)
    torch.cuda.synchronize()
    lg = logits.double().cpu().numpy()
    # the scores themselves: fp32 sums of the bf16-rounded inputs
    ref_lg = O.logits(h["x"], h["Wg"], h["bias"])
    lerr = float(np.max(np.abs(lg - ref_lg)) / np.max(np.abs(ref_lg)))
    err = check_route(lg, idx.cpu().numpy(), gate.cpu().numpy(), k, gm)
    say(f"moe_route_ex {label}: max |gate - oracle| {err:.2e}, scores rel {lerr:.1e}")
    assert err <= 1e-6
    assert lerr <= 1e-5


@pytest.mark.parametrize("gm", [0, 1, 2])
def test_route_gate_modes(gm):
    cfg, h, dev = inputs(777, 512, 64, 64, 4, "bf16", seed=11)
    idx, gate, logits = moe.route(dev["x"], dev["Wg"], 4, None, gate_mode=gm)
    torch.cuda.synchronize()
    lg = logits.double().cpu().numpy()
    idx_ref = O.topk(lg, 4)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_ref)
    gref = O.gate_mode(lg, idx_ref, gm)
    err = float(np.max(np.abs(gate.cpu().numpy() - gref)))
    say(f"moe_route_ex gate_mode {gm}: max |gate - oracle| {err:.2e}")
    assert err <= 1e-6


@pytest.mark.parametrize("T,E,k,cap", [(1000, 8, 2, 100), (9000, 12, 3, 1500), (50, 4, 1, 0),
                                       (4097, 256, 8, 7)])
def test_permute_capacity(T, E, k, cap):
    rng = np.random.default_rng(T + E)
    # skewed expert choices, k distinct experts per token
    w = np.exp(-np.arange(E) / 3.0)
    idx = np.stack([rng.choice(E, size=k, replace=False, p=w / w.sum()) for _ in range(T)])
    idx = idx.astype(np.int32)
    counts, offsets, perm, inv = moe.permute(torch.from_numpy(idx).cuda(), E, capacity=cap)
    torch.cuda.synchronize()
    keep = O.keep(idx, E, cap).astype(bool)
    kc = np.bincount(idx.reshape(-1)[keep], minlength=E)
    np.testing.assert_array_equal(counts.cpu().numpy(), kc)
    np.testing.assert_array_equal(offsets.cpu().numpy(), np.concatenate([[0], np.cumsum(kc)]))
    order = np.flatnonzero(keep)[np.argsort(idx.reshape(-1)[keep], kind="stable")]
    np.testing.assert_array_equal(perm.cpu().numpy()[:len(order)], order)
    inv_ref = np.full(T * k, -1, np.int32)
    inv_ref[order] = np.arange(len(order), dtype=np.int32)
    np.testing.assert_array_equal(inv.cpu().numpy(), inv_ref)
    say(f"moe_permute_ex T={T} E={E} k={k} capacity={cap}: kept {len(order)} of {T * k}")


@pytest.mark.parametrize("skew,expect_k", [(0.0, 3), (4.0, 2)])
def test_route_entropy_batch_branches(skew, expect_k):
    """One k for the batch: the full k when any token's entropy exceeds the
    threshold, else every token's last slot empty (moe_route_ex)."""
    cfg, h, dev = inputs(256, 256, 8, 256, 3, "bf16", skew=skew, seed=19)
    say(f"entropy batch routing, skew {skew}")
    idx, gate, logits = moe.route(dev["x"], dev["Wg"], 3, dev["bias"],
                                  gate_mode=moe.GATE_ENTROPY_BATCH)
    torch.cuda.synchronize()
    lg = logits.double().cpu().numpy()
    H = O.entropy(lg)
    assert np.min(np.abs(H - O.ENTROPY_THRESHOLD)) > 1e-4
    idx_ref, gate_ref, kb = O.route_entropy_batch(lg, 3)
    assert kb == expect_k
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_ref)
    assert np.max(np.abs(gate.cpu().numpy() - gate_ref)) <= 1e-6
