"""The layer captured in a HIP graph and replayed: every replay must give the
bits of the eager forward.  The forward keeps arrival counters and per-XCD
tile queues in its workspace (or in the allocation-free entry point's static
scratch) that its own launches clear or put back, so a replay that found
them in another state would differ.  Each case replays several times with
eager work and synchronisations between the replays."""
import numpy as np
import pytest
import torch

from sparse_mixture_experts_permute_amd import moe
from sparse_mixture_experts_permute_amd.inputs import LayerConfig, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    LayerConfig("graph_T1_routed", 1, 2048, 8, 2048, 2, "bf16", seed=7),          # one token: 2 launches
    LayerConfig("graph_T4_gemv", 4, 2048, 8, 2048, 2, "bf16", seed=8),            # down + combine counters
    LayerConfig("graph_T24_tiles64", 24, 512, 8, 1024, 2, "bf16", seed=9),        # 64-row tiles, K planes
    LayerConfig("graph_T1024_light", 1024, 512, 8, 1024, 2, "bf16", seed=10),     # 256-row + light tiles, tile queues
    LayerConfig("graph_T2048_split", 2048, 4096, 8, 5120, 2, "bf16", seed=11),    # last-round K split (down GEMM)
    LayerConfig("graph_shared", 160, 256, 8, 512, 2, "bf16", d_ff_shared=128, seed=12),
    LayerConfig("graph_f32", 256, 256, 8, 512, 2, "f32", seed=13),
]


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).clone()


def _replays_match(fwd, y, ref, n=4):
    g = torch.cuda.CUDAGraph()
    s_cap = torch.cuda.Stream()
    s_cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s_cap):
        fwd()  # the capture stream's first use outside the capture
    torch.cuda.current_stream().wait_stream(s_cap)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fwd()
    torch.cuda.synchronize()
    other = torch.randn(256, 256, device="cuda")
    for i in range(n):
        y.zero_()
        (other @ other).sum().item()  # eager work and a synchronisation between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(y), ref), f"replay {i} differs from the eager forward"
    del g


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_graph_replay_matches_eager(cfg):
    print(f"\n[gpu-graph] {cfg.name}: T={cfg.T} d={cfg.d} E={cfg.E} d_ff={cfg.d_ff} "
          f"k={cfg.k} {cfg.dtype}", flush=True)
    h = make_inputs(cfg)
    d = {n: moe.tensor_from_numpy(a) for n, a in h.items() if a is not None}
    sh = (d["Ws1"], d["Ws3"], d["Ws2"]) if cfg.d_ff_shared else None
    layer = moe.MoELayer(d["Wg"], d["W1"], d["W3"], d["W2"], cfg.k, None, sh)
    x = d["x"]
    y = torch.empty_like(x)
    layer(x, y)
    torch.cuda.synchronize()
    ref = _bits(y)
    _replays_match(lambda: layer(x, y), y, ref)


def test_graph_replay_noalloc():
    """moe_forward_noalloc is meant for callers that capture: replays of a
    captured call give the eager call's bits (its scratch is the library's
    static array, shared by every call on the GPU)."""
    cfg = LayerConfig("graph_noalloc", 200, 512, 8, 1024, 2, "bf16", seed=14)
    h = make_inputs(cfg)
    d = {n: moe.tensor_from_numpy(a) for n, a in h.items() if a is not None}
    L = moe.lib()
    p = moe._p
    x = d["x"]
    y = torch.empty_like(x)

    def fwd():
        rc = L.moe_forward_noalloc(p(x), p(d["Wg"]), None, p(d["W1"]), p(d["W3"]), p(d["W2"]),
                                   None, None, None, 0, cfg.T, cfg.E, cfg.k, cfg.d, cfg.d_ff,
                                   moe._dt(x), p(y), moe._stream())
        assert rc == 0, L.moe_strerror(rc)

    fwd()
    torch.cuda.synchronize()
    ref = _bits(y)
    layer = moe.MoELayer(d["Wg"], d["W1"], d["W3"], d["W2"], cfg.k)
    y2 = layer(x)
    torch.cuda.synchronize()
    assert torch.equal(_bits(y2), ref), "noalloc and workspace forwards differ"
    _replays_match(fwd, y, ref)
