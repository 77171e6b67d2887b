"""The [in][out] expert-weight layout (MOE_LAYOUT_IN_OUT: W1, W3 [E][d][d_ff],
W2 [E][d_ff][d], the layout of the numpy forward on "Trillion-parameter MoE
... 7 expert configs measured") through the C ABI, on an MI355X.

Bars: y against the CPU oracle as in the parity tests (rel-L2 1e-4 fp32, 1e-2
bf16); and, where the tiled kernels serve (more than four tokens), bit for bit
equal to the [out][in] layer on the same weights, since the transposing LDS
reads hand the matrix cores the same fragments.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_mixture_experts_permute_amd import moe
from sparse_mixture_experts_permute_amd.inputs import CONFIGS, LayerConfig, make_inputs, shared_tuple
from test_gpu_parity import SMALL, TOL, case, f64, rel_l2, sample_rows

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"\n[gpu-layout] {msg}", flush=True)


def t12(w):
    return w.transpose(-1, -2).contiguous()


def layers(d, cfg, **kw):
    """(the [out][in] layer, the [in][out] layer) on the same weights."""
    sh = (d["Ws1"], d["Ws3"], d["Ws2"]) if cfg.d_ff_shared else None
    a = moe.MoELayer(d["Wg"], d["W1"], d["W3"], d["W2"], cfg.k, d.get("bias"), sh, **kw)
    sh_t = tuple(t12(w) for w in sh) if sh else None
    b = moe.MoELayer(d["Wg"], t12(d["W1"]), t12(d["W3"]), t12(d["W2"]), cfg.k, d.get("bias"),
                     sh_t, weight_layout=moe.LAYOUT_IN_OUT, **kw)
    return a, b


def run_both(d, cfg, **kw):
    a, b = layers(d, cfg, **kw)
    ya = a(d["x"])
    yb = b(d["x"])
    torch.cuda.synchronize()
    return a, b, ya, yb


def same_bits(ya, yb):
    u, v = moe.tensor_to_numpy(ya), moe.tensor_to_numpy(yb)
    return int(np.count_nonzero(u != v))


@pytest.mark.parametrize("name", SMALL)
def test_inout_small_full_output(name):
    cfg = CONFIGS[name]
    say(f"{name}: T={cfg.T} E={cfg.E} d_ff={cfg.d_ff} k={cfg.k} {cfg.dtype}")
    h, d = case(cfg)
    a, b, ya, yb = run_both(d, cfg)
    lg = b.intermediates(cfg.T)["logits"].double().cpu().numpy()
    ref = O.forward(h["x"], h["Wg"], h["W1"], h["W3"], h["W2"], cfg.k, bias=h["bias"],
                    logits_in=lg)
    err = rel_l2(f64(moe.tensor_to_numpy(yb)), ref["y"])
    nd = same_bits(ya, yb)
    say(f"{name}: [in][out] rel-L2 {err:.3e}; elements differing from [out][in]: {nd}")
    assert err <= TOL[cfg.dtype]
    assert nd == 0


MIXTRAL = ["mixtral_prefill_T2048", "mixtral_decode_T1", "mixtral_decode_T8",
           "mixtral_decode_T32", "mixtral_decode_T128", "fine_shared_T512"]


@pytest.mark.parametrize("name", MIXTRAL)
def test_inout_full_size(name):
    cfg = CONFIGS[name]
    say(f"{name}: T={cfg.T} d={cfg.d} E={cfg.E} d_ff={cfg.d_ff} k={cfg.k} shared={cfg.d_ff_shared}")
    h, d = case(cfg, T_max=8192)
    a, b, ya, yb = run_both(d, cfg)
    inter = {kk: v.cpu() for kk, v in b.intermediates(cfg.T).items()}
    lg = inter["logits"].double().numpy()
    idx_ref = O.topk(lg, cfg.k)
    np.testing.assert_array_equal(inter["idx"].numpy(), idx_ref)
    gate_ref = O.gate(lg, idx_ref)
    rows = sample_rows(cfg.T, np.random.default_rng(11))
    ref = O.forward_rows(h["x"], h["W1"], h["W3"], h["W2"], rows, idx_ref[rows], gate_ref[rows],
                         shared=shared_tuple(h))
    err = rel_l2(f64(moe.tensor_to_numpy(yb[rows])), ref)
    nd = same_bits(ya, yb)
    say(f"{name}: [in][out] sampled {len(rows)} rows rel-L2 {err:.3e}; "
        f"elements differing from [out][in]: {nd}")
    assert err <= TOL[cfg.dtype]
    if cfg.T > 4:
        assert nd == 0


EDGE = [
    # (label, T, d, E, d_ff, k, dtype, d_ff_shared)
    ("T7_ragged_f32", 7, 128, 8, 192, 2, "f32", 0),
    ("N_tail_192", 70, 192, 5, 192, 2, "bf16", 0),
    ("E256_k8_shared", 33, 128, 256, 64, 8, "bf16", 192),
    ("shared_f32", 45, 128, 16, 64, 4, "f32", 128),
    ("K5120_bm256", 256, 5120, 2, 256, 1, "bf16", 0),
    ("kplanes_down", 64, 256, 4, 14336, 2, "bf16", 0),
    ("split_shared", 1500, 256, 4, 256, 1, "bf16", 256),
    ("split_remainders_E4_k1", 1300, 256, 4, 256, 1, "bf16", 0),
    # few tokens: the [K][N] weight-streaming kernel (64- and 32-column blocks)
    ("stream_T1", 1, 2048, 8, 2048, 2, "bf16", 0),
    # one token routed inside the [K][N] SwiGLU kernel: with a shared expert, and with k = 4
    # of 32 experts and one expert's bias dominant
    ("stream_T1_routed_shared", 1, 4096, 8, 2048, 2, "bf16", 2048),
    ("stream_T1_routed_k4_hot", 1, 2048, 32, 1024, 4, "bf16", 0),
    ("stream_T2_shared", 2, 2048, 4, 6144, 2, "bf16", 2048),
    ("stream_T3_k4", 3, 1024, 8, 1536, 4, "bf16", 0),
    ("stream_T4_hot", 4, 2048, 8, 4096, 2, "bf16", 0),
    ("stream_T4_E256_shared", 4, 1024, 256, 512, 8, "bf16", 1024),
    # K not a multiple of 512: tiled kernels even for one token
    ("tiles_T1_d256", 1, 256, 8, 256, 2, "bf16", 0),
]


@pytest.mark.parametrize("case_", EDGE, ids=[c[0] for c in EDGE])
def test_inout_edge_cases(case_):
    label, T, dm, E, dff, k, dt, dffs = case_
    say(f"edge {label}: T={T} d={dm} E={E} d_ff={dff} k={k} {dt} shared={dffs}")
    cfg = LayerConfig(label, T, dm, E, dff, k, dt, d_ff_shared=dffs, seed=99)
    h = make_inputs(cfg)
    if label.endswith("_hot"):
        h["bias"] = np.zeros(E, np.float32)
        h["bias"][1] = 100.0
    d = {n: moe.tensor_from_numpy(a) for n, a in h.items() if a is not None}
    d.setdefault("bias", None)
    a, b, ya, yb = run_both(d, cfg)
    # the same routing in both layouts (the same router arithmetic, whichever kernel runs it)
    ia, ib = a.intermediates(T), b.intermediates(T)
    for n in ("idx", "gate", "counts", "offsets", "perm", "inv"):
        assert torch.equal(ia[n], ib[n]), n
    lg = ib["logits"].double().cpu().numpy()
    ref = O.forward(h["x"], h["Wg"], h["W1"], h["W3"], h["W2"], k, bias=h.get("bias"),
                    shared=shared_tuple(h), logits_in=lg)
    err = rel_l2(f64(moe.tensor_to_numpy(yb)), ref["y"])
    nd = same_bits(ya, yb)
    say(f"edge {label}: rel-L2 {err:.3e}; elements differing from [out][in]: {nd}")
    assert err <= TOL[dt]
    if not label.startswith("stream"):
        assert nd == 0


def test_inout_variants_match_outin():
    """The gate, activation and capacity variants read [in][out] weights the
    same way (moe_forward_ex)."""
    cfg = LayerConfig("variants", 300, 256, 8, 512, 2, "bf16", seed=5)
    h = make_inputs(cfg)
    d = {n: moe.tensor_from_numpy(a) for n, a in h.items() if a is not None}
    for kw in (dict(gate_mode=moe.GATE_SIGMOID, activation=moe.ACT_GLU_SIGMOID),
               dict(capacity=40), dict(gate_mode=moe.GATE_SOFTMAX_ALL)):
        a, b, ya, yb = run_both(d, cfg, **kw)
        assert same_bits(ya, yb) == 0, kw
