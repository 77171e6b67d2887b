"""The library called from plain C: tests/c_abi/moe_c_caller.c allocates its
buffers with hipMalloc, creates a HIP stream and calls moe_forward, in a
process with no Python and no torch.  Its y must carry the same bits as the
Python binding's (same library, same kernels) and match the CPU oracle within
the bf16 bar, with the router run on the GPU's scores ("Chapter 10 MoE"
sections 10.3-10.4; the gate is the softmax over the selected scores)."""
import os
import subprocess

import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_mixture_experts_permute_amd import moe
from sparse_mixture_experts_permute_amd.build import C_CALLER
from sparse_mixture_experts_permute_amd.inputs import LayerConfig, bf16_bits_to_f32, make_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,d,E,dff,k", [(96, 256, 8, 512, 2), (300, 512, 16, 1024, 4),
                                         (1, 2048, 8, 2048, 2)])
def test_c_caller_matches_binding_and_oracle(tmp_path, T, d, E, dff, k):
    assert os.path.exists(C_CALLER), f"{C_CALLER} not built (the package build compiles it)"
    cfg = LayerConfig("c_abi", T, d, E, dff, k, "bf16", seed=T + d + E)
    h = make_inputs(cfg)
    for n in ("x", "Wg", "W1", "W3", "W2"):
        assert h[n].dtype == np.uint16
        h[n].tofile(tmp_path / f"{n}.bin")
    print(f"\n[gpu-c-abi] C caller T={T} d={d} E={E} d_ff={dff} k={k}", flush=True)
    r = subprocess.run([C_CALLER, str(tmp_path), str(T), str(d), str(E), str(dff), str(k)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    y_c = np.fromfile(tmp_path / "y.bin", dtype=np.uint16).reshape(T, d)

    dev = {n: moe.tensor_from_numpy(a) for n, a in h.items() if a is not None}
    layer = moe.MoELayer(dev["Wg"], dev["W1"], dev["W3"], dev["W2"], k)
    y = layer(dev["x"])
    torch.cuda.synchronize()
    assert np.array_equal(moe.tensor_to_numpy(y), y_c), "C caller and binding differ"

    lg = layer.intermediates(T)["logits"].double().cpu().numpy()
    ref = O.forward(h["x"], h["Wg"], h["W1"], h["W3"], h["W2"], k, logits_in=lg)
    got = bf16_bits_to_f32(y_c).astype(np.float64)
    err = np.linalg.norm(got - ref["y"]) / np.linalg.norm(ref["y"])
    print(f"[gpu-c-abi] rel-L2 {err:.3e} against the oracle (bar 1e-2)", flush=True)
    assert err <= 1e-2
