"""moe_forward_noalloc (scratch in the library's static device array) against
moe_forward (caller's workspace), through the C ABI: the same kernels on the
same inputs, so y must agree bit for bit.  Two calls in a row, the second on
a smaller input, so that the second call runs on the scratch the first one
left behind."""
import ctypes

import numpy as np
import pytest
import torch

from sparse_mixture_experts_permute_amd import moe
from sparse_mixture_experts_permute_amd.inputs import LayerConfig, make_inputs

pytestmark = pytest.mark.gpu


def _run_noalloc(L, d, cfg, T, y):
    sh = (d["Ws1"], d["Ws3"], d["Ws2"]) if cfg.d_ff_shared else (None, None, None)
    p = moe._p
    x = d["x"][:T].contiguous()
    rc = L.moe_forward_noalloc(p(x), p(d["Wg"]), None, p(d["W1"]), p(d["W3"]), p(d["W2"]),
                               p(sh[0]), p(sh[1]), p(sh[2]), cfg.d_ff_shared, T, cfg.E, cfg.k,
                               cfg.d, cfg.d_ff, moe._dt(x), p(y), moe._stream())
    assert rc == 0, L.moe_strerror(rc)


@pytest.mark.parametrize("cfg,T_first,T_second", [
    (LayerConfig("noalloc_shared", 160, 256, 8, 512, 2, "bf16", d_ff_shared=128, seed=42), 160, 37),
    (LayerConfig("noalloc_fp32", 512, 512, 8, 4096, 2, "f32", seed=42), 512, 200),
    (LayerConfig("noalloc_mixtral", 32, 4096, 8, 14336, 2, "bf16", seed=42), 32, 1),
])
def test_noalloc_matches_forward(cfg, T_first, T_second):
    L = moe.lib()
    print(f"\n[no-alloc] {cfg.name}: T={T_first} then T={T_second}", flush=True)
    host = make_inputs(cfg, T=T_first)
    d = {n: moe.tensor_from_numpy(a) for n, a in host.items() if a is not None}
    sh = (d["Ws1"], d["Ws3"], d["Ws2"]) if cfg.d_ff_shared else None
    layer = moe.MoELayer(d["Wg"], d["W1"], d["W3"], d["W2"], cfg.k, None, sh)
    for T in (T_first, T_second):
        x = d["x"][:T].contiguous()
        ref = layer(x)
        y = torch.full_like(ref, float("nan"))
        _run_noalloc(L, d, cfg, T, y)
        torch.cuda.synchronize()
        a, b = moe.tensor_to_numpy(y), moe.tensor_to_numpy(ref)
        assert np.array_equal(a, b), f"T={T}: {np.count_nonzero(a != b)} elements differ"


def test_noalloc_rejects_oversized_shape():
    L = moe.lib()
    fake = ctypes.c_void_p(0x1000)
    # the Mixtral-shaped layer at 8192 tokens needs about 1.1 GB of scratch
    rc = L.moe_forward_noalloc(fake, fake, None, fake, fake, fake, None, None, None, 0, 8192, 8,
                               2, 4096, 14336, moe.MOE_BF16, fake, None)
    assert rc == -6
