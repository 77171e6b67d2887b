"""Two layers on two HIP streams at once, each with its own workspace: the
library keeps no state outside the caller's workspace (the arrival counters
and per-XCD tile queues of a forward live there), so concurrent forwards give
the bits of the same forwards run one after the other."""
import pytest
import torch

from sparse_mixture_experts_permute_amd import moe
from sparse_mixture_experts_permute_amd.inputs import LayerConfig, make_inputs

pytestmark = pytest.mark.gpu


def _layer(cfg):
    h = make_inputs(cfg)
    d = {n: moe.tensor_from_numpy(a) for n, a in h.items() if a is not None}
    sh = (d["Ws1"], d["Ws3"], d["Ws2"]) if cfg.d_ff_shared else None
    return moe.MoELayer(d["Wg"], d["W1"], d["W3"], d["W2"], cfg.k, None, sh), d["x"]


@pytest.mark.parametrize("ca,cb", [
    (LayerConfig("streams_light", 1024, 512, 8, 1024, 2, "bf16", seed=21),
     LayerConfig("streams_tiles64", 40, 512, 8, 1024, 2, "bf16", seed=22)),
    (LayerConfig("streams_T1", 1, 2048, 8, 2048, 2, "bf16", seed=23),
     LayerConfig("streams_shared", 160, 256, 8, 512, 2, "bf16", d_ff_shared=128, seed=24)),
])
def test_concurrent_streams_match_serial(ca, cb):
    print(f"\n[gpu-streams] {ca.name} beside {cb.name}", flush=True)
    la, xa = _layer(ca)
    lb, xb = _layer(cb)
    ya, yb = torch.empty_like(xa), torch.empty_like(xb)
    la(xa, ya)
    lb(xb, yb)
    torch.cuda.synchronize()
    ra, rb = ya.view(torch.int16).clone(), yb.view(torch.int16).clone()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    for i in range(6):
        with torch.cuda.stream(sa):
            ya.zero_()
            la(xa, ya)
        with torch.cuda.stream(sb):
            yb.zero_()
            lb(xb, yb)
        torch.cuda.synchronize()
        assert torch.equal(ya.view(torch.int16), ra), f"{ca.name}: round {i} differs"
        assert torch.equal(yb.view(torch.int16), rb), f"{cb.name}: round {i} differs"
