"""Weight-only FP8 experts on an MI355X against the CPU oracle.

"Mistral 8x7B SMoE architecture deep dive", section 5.3: the expert weights are
quantised with one scale per expert and the router stays in high precision.
Bars: the quantiser's codes and scales bit-exact against the oracle's; the
layer's routing bit-exact, y within the bf16 bar (1e-2 relative L2) of the
oracle's fp64 layer on the dequantised weights (scale * E4M3 code), with the
router run on the GPU's scores.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_mixture_experts_permute_amd import moe
from sparse_mixture_experts_permute_amd.inputs import (CONFIGS, LayerConfig, bf16_bits_to_f32,
                                                      make_inputs)

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"\n[gpu-fp8] {msg}", flush=True)


def f64(a):
    return (bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)


def rel_l2(got, ref):
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


@pytest.mark.parametrize("dtype,shape", [("bf16", (4, 256, 2048)), ("f32", (3, 64, 96)),
                                         ("bf16", (2, 7, 5))])
def test_quantize_bit_exact(dtype, shape):
    rng = np.random.default_rng(sum(shape))
    W = (rng.standard_normal(shape) * np.array([0.03, 1.0, 250.0, 1e-3][:shape[0]])
         [:, None, None]).astype(np.float32)
    W[-1, 0, :] = 0.0
    if shape[0] > 2:
        W[1] = 0.0  # an all-zero expert: scale 1, every code 0
    if dtype == "bf16":
        bits = (W.view(np.uint32) >> 16).astype(np.uint16)  # truncation: any bf16 values
        host = bits
        dev = moe.tensor_from_numpy(bits)
    else:
        host = W
        dev = torch.from_numpy(W).cuda()
    q, sc = moe.quantize_fp8(dev)
    torch.cuda.synchronize()
    q_ref, sc_ref = O.quantize_fp8(host)
    np.testing.assert_array_equal(sc.cpu().numpy(), sc_ref)
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)
    say(f"quantize {dtype} {shape}: {q_ref.size} codes bit-exact")


def fp8_case(T, d, E, dff, k, seed=3, skew=0.0):
    cfg = LayerConfig("fp8", T, d, E, dff, k, "bf16", skew=skew, seed=seed)
    h = make_inputs(cfg)
    dev = {n: moe.tensor_from_numpy(a) for n, a in h.items() if a is not None}
    dev["bias"] = torch.from_numpy(h["bias"]).cuda() if h["bias"] is not None else None
    return cfg, h, dev


@pytest.mark.parametrize("T,E,k,dff,gm,cap", [(1, 8, 2, 2048, 0, None), (2, 8, 2, 4096, 0, None),
                                             (3, 8, 2, 2048, 1, None), (4, 4, 2, 2048, 0, None),
                                             (4, 8, 3, 2048, 3, None), (3, 8, 2, 2048, 0, 1),
                                             (1, 8, 3, 4096, 3, None), (1, 16, 4, 2048, 2, None)])
def test_forward_fp8(T, E, k, dff, gm, cap):
    d = 2048
    cfg, h, dev = fp8_case(T, d, E, dff, k, seed=T * 10 + E, skew=1.5 if cap else 0.0)
    say(f"forward_fp8 T={T} E={E} k={k} d={d} d_ff={dff} gate={gm} capacity={cap}")
    L = moe.MoELayerFP8(dev["Wg"], dev["W1"], dev["W3"], dev["W2"], k, dev["bias"],
                        gate_mode=gm, capacity=-1 if cap is None else cap)
    y = L(dev["x"])
    torch.cuda.synchronize()
    it = {n: v.cpu().numpy() for n, v in L.intermediates(T).items()}
    lg = it["logits"].astype(np.float64)
    deq = {}
    for n, qn, sn in (("W1", "W1q", "s1"), ("W3", "W3q", "s3"), ("W2", "W2q", "s2")):
        q_ref, s_ref = O.quantize_fp8(h[n])
        np.testing.assert_array_equal(getattr(L, sn).cpu().numpy(), s_ref)
        np.testing.assert_array_equal(getattr(L, qn).cpu().numpy(), q_ref)
        deq[n] = O.dequant_fp8(q_ref, s_ref)
    ref = O.forward(f64(h["x"]), f64(h["Wg"]), deq["W1"], deq["W3"], deq["W2"], k,
                    bias=h["bias"], logits_in=lg, gate_mode=gm, capacity=cap)
    if gm == O.GATE_ENTROPY:
        assert np.min(np.abs(O.entropy(lg) - O.ENTROPY_THRESHOLD)) > 1e-4
    np.testing.assert_array_equal(it["idx"], ref["idx"])
    np.testing.assert_array_equal(it["inv"], ref["inv"])
    got = f64(moe.tensor_to_numpy(y))
    err = rel_l2(got, ref["y"])
    # the dequantised layer is another layer: how far it is from the bf16 one
    ref16 = O.forward(h["x"], h["Wg"], h["W1"], h["W3"], h["W2"], k, bias=h["bias"],
                      logits_in=lg, gate_mode=gm, capacity=cap)
    qerr = rel_l2(ref["y"], ref16["y"])
    say(f"forward_fp8: rel-L2 {err:.3e} against the dequantised oracle (bar 1e-2); the FP8 "
        f"weights move y by {qerr:.3e} from the bf16 layer")
    assert err <= 1e-2


def test_forward_fp8_mixtral_T1_sampled():
    # the Mixtral-shaped decode step: the two hit experts quantised and
    # dequantised on the CPU, the token's output checked against them
    cfg = CONFIGS["mixtral_decode_T1"]
    h = make_inputs(cfg)
    dev = {n: moe.tensor_from_numpy(a) for n, a in h.items() if a is not None}
    L = moe.MoELayerFP8(dev["Wg"], dev["W1"], dev["W3"], dev["W2"], cfg.k)
    y = L(dev["x"])
    torch.cuda.synchronize()
    it = {n: v.cpu().numpy() for n, v in L.intermediates(1).items()}
    idx, gate = it["idx"][0], it["gate"][0].astype(np.float64)
    ref = np.zeros(cfg.d)
    for j, e in enumerate(idx):
        parts = {}
        for n, qn, sn in (("W1", "W1q", "s1"), ("W3", "W3q", "s3"), ("W2", "W2q", "s2")):
            q_ref, s_ref = O.quantize_fp8(h[n][e:e + 1])
            np.testing.assert_array_equal(getattr(L, qn)[e].cpu().numpy(), q_ref[0])
            assert getattr(L, sn)[e].item() == s_ref[0]
            parts[n] = O.dequant_fp8(q_ref, s_ref)
        ref += gate[j] * O.expert_row(f64(h["x"]), 0, parts["W1"], parts["W3"], parts["W2"], 0)
    err = rel_l2(f64(moe.tensor_to_numpy(y))[0], ref)
    say(f"mixtral decode T=1 fp8: experts {idx.tolist()}, rel-L2 {err:.3e}")
    assert err <= 1e-2


# more than four tokens: 64-row matrix-core tiles that widen the codes to bf16
@pytest.mark.parametrize("T,E,k,d,dff,gm,cap", [
    (8, 8, 2, 2048, 2048, 0, None), (32, 8, 2, 1024, 1536, 0, None),
    (128, 8, 2, 512, 1024, 1, None), (40, 16, 4, 256, 512, 3, None),
    (64, 8, 2, 256, 14336, 0, None),  # every down-projection tile split into K planes
    (100, 4, 1, 384, 640, 2, 20), (5, 8, 2, 256, 384, 0, None), (300, 32, 2, 128, 256, 0, None),
    (384, 8, 2, 256, 512, 0, None)])  # 96 rows per expert: two or more 64-row tiles each
def test_forward_fp8_tiled(T, E, k, d, dff, gm, cap):
    cfg, h, dev = fp8_case(T, d, E, dff, k, seed=T + E + d, skew=1.5 if cap else 0.0)
    say(f"forward_fp8 tiled T={T} E={E} k={k} d={d} d_ff={dff} gate={gm} capacity={cap}")
    L = moe.MoELayerFP8(dev["Wg"], dev["W1"], dev["W3"], dev["W2"], k, dev["bias"],
                        gate_mode=gm, capacity=-1 if cap is None else cap)
    y = L(dev["x"])
    torch.cuda.synchronize()
    it = {n: v.cpu().numpy() for n, v in L.intermediates(T).items()}
    lg = it["logits"].astype(np.float64)
    deq = {}
    for n, qn, sn in (("W1", "W1q", "s1"), ("W3", "W3q", "s3"), ("W2", "W2q", "s2")):
        q_ref, s_ref = O.quantize_fp8(h[n])
        np.testing.assert_array_equal(getattr(L, sn).cpu().numpy(), s_ref)
        np.testing.assert_array_equal(getattr(L, qn).cpu().numpy(), q_ref)
        deq[n] = O.dequant_fp8(q_ref, s_ref)
    ref = O.forward(f64(h["x"]), f64(h["Wg"]), deq["W1"], deq["W3"], deq["W2"], k,
                    bias=h["bias"], logits_in=lg, gate_mode=gm, capacity=cap)
    if gm == O.GATE_ENTROPY:
        assert np.min(np.abs(O.entropy(lg) - O.ENTROPY_THRESHOLD)) > 1e-4
    np.testing.assert_array_equal(it["idx"], ref["idx"])
    np.testing.assert_array_equal(it["inv"], ref["inv"])
    err = rel_l2(f64(moe.tensor_to_numpy(y)), ref["y"])
    say(f"forward_fp8 tiled: rel-L2 {err:.3e} against the dequantised oracle (bar 1e-2)")
    assert err <= 1e-2


@pytest.mark.parametrize("name", ["mixtral_decode_T8", "mixtral_decode_T128"])
def test_forward_fp8_mixtral_sampled(name):
    """Mixtral-shaped decode batches with FP8 experts: every token against the
    oracle on the dequantised weights of each expert it reaches (one expert's
    matrices at a time, so that the fp64 copies stay small), so every 64-row
    tile and every column block of both GEMMs is compared."""
    cfg = CONFIGS[name]
    h = make_inputs(cfg)
    dev = {n: moe.tensor_from_numpy(a) for n, a in h.items() if a is not None}
    L = moe.MoELayerFP8(dev["Wg"], dev["W1"], dev["W3"], dev["W2"], cfg.k)
    y = L(dev["x"])
    torch.cuda.synchronize()
    it = {n: v.cpu().numpy() for n, v in L.intermediates(cfg.T).items()}
    idx, gate = it["idx"], it["gate"].astype(np.float64)
    ref = np.zeros((cfg.T, cfg.d))
    x64 = f64(h["x"])
    for e in sorted(set(idx.ravel().tolist())):
        parts = {}
        for n, qn, sn in (("W1", "W1q", "s1"), ("W3", "W3q", "s3"), ("W2", "W2q", "s2")):
            q_ref, s_ref = O.quantize_fp8(h[n][e:e + 1])
            np.testing.assert_array_equal(getattr(L, qn)[e].cpu().numpy(), q_ref[0])
            assert getattr(L, sn)[e].item() == s_ref[0]
            parts[n] = O.dequant_fp8(q_ref, s_ref)
        # the tokens that reach expert e, each with the gate of that pair
        tok, slot = np.nonzero(idx == e)
        ref[tok] += O.forward_rows(x64, parts["W1"], parts["W3"], parts["W2"], tok,
                                   np.zeros((len(tok), 1), np.int32),
                                   gate[tok, slot][:, None])
    got = f64(moe.tensor_to_numpy(y))
    err = rel_l2(got, ref)
    worst = max(rel_l2(got[t], ref[t]) for t in range(cfg.T))
    say(f"{name} fp8: all {cfg.T} tokens, rel-L2 {err:.3e}, worst token {worst:.3e}")
    assert err <= 1e-2
    # each token on its own as well (three times the bar, as for the edge
    # cases): one wrong 64-row tile hardly moves the whole output's error
    assert worst <= 3e-2
