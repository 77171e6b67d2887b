"""The C-ABI library loads and exports what include/*.h declares; host-side
argument checks reject bad calls before touching a device (CPU only)."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = glob.glob(os.path.join(ROOT, "include", "*.h"))


def declared_functions():
    names = set()
    for h in HEADERS:
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        for m in re.finditer(r"\b(moe_[a-z0-9_]+)\s*\(", src):
            names.add(m.group(1))
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    from sparse_mixture_experts_permute_amd import moe
    if not os.path.exists(moe.LIB_PATH):
        from sparse_mixture_experts_permute_amd import build
        build.build(verbose=False)
    return moe.lib()


def test_header_declares_entry_points():
    names = declared_functions()
    for n in ("moe_route", "moe_permute", "moe_forward", "moe_workspace_bytes", "moe_strerror"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for n in declared_functions():
        assert hasattr(L, n), f"{n} declared but not exported"


def test_strerror(L):
    for code in (0, -1, -2, -3, -4, -5):
        assert L.moe_strerror(code)
    assert b"unknown" in L.moe_strerror(-99)


def test_workspace_sizes(L):
    from sparse_mixture_experts_permute_amd import moe
    n = L.moe_workspace_bytes(512, 512, 4096, 8, 2, 0, moe.MOE_F32)
    P = 1024
    # at least the permuted activations, hidden and down-projection buffers
    assert n >= P * 512 * 4 + P * 4096 * 4 + P * 512 * 4
    assert n % 256 == 0
    assert L.moe_workspace_bytes(512, 512, 4096, 8, 9, 0, moe.MOE_F32) == 0  # k > E
    assert L.moe_workspace_bytes(512, 500, 4096, 8, 2, 0, moe.MOE_F32) == 0  # d % 64
    assert L.moe_workspace_bytes(512, 512, 4096, 8, 2, 0, 7) == 0  # dtype
    assert L.moe_workspace_bytes(16, 512, 4096, 257, 2, 0, moe.MOE_BF16) == 0  # E > 256
    off = moe.workspace_offsets(100, 512, 1024, 8, 2, 0, moe.MOE_BF16)
    assert list(off) == list(moe.WS_FIELDS)
    assert all(v % 256 == 0 for v in off.values())
    assert sorted(off.values()) == list(off.values())


def test_argument_errors_before_launch(L):
    vp = ctypes.c_void_p
    fake = vp(0x1000)
    big = 1 << 30
    # bad dtype
    assert L.moe_route(fake, fake, None, 4, 64, 8, 2, 9, fake, fake, None, fake, big, None) == -2
    # k > E, k < 1, E > 256, d not a multiple of 64
    assert L.moe_route(fake, fake, None, 4, 64, 8, 9, 1, fake, fake, None, fake, big, None) == -1
    assert L.moe_route(fake, fake, None, 4, 64, 8, 0, 1, fake, fake, None, fake, big, None) == -1
    assert L.moe_route(fake, fake, None, 4, 64, 300, 2, 1, fake, fake, None, fake, big, None) == -1
    assert L.moe_route(fake, fake, None, 4, 65, 8, 2, 1, fake, fake, None, fake, big, None) == -1
    # missing required pointers
    assert L.moe_route(None, fake, None, 4, 64, 8, 2, 1, fake, fake, None, fake, big, None) == -1
    assert L.moe_route(fake, fake, None, 4, 64, 8, 2, 1, fake, fake, None, None, big, None) == -1
    # workspace too small / misaligned
    assert L.moe_route(fake, fake, None, 4, 64, 8, 2, 1, fake, fake, None, vp(0x100000), 8,
                       None) == -3
    assert L.moe_route(fake, fake, None, 4, 64, 8, 2, 1, fake, fake, None, vp(0x100008), big,
                       None) == -3
    assert L.moe_route_workspace_bytes(4, 64, 8, 1) >= 4 * 8 * 4
    assert L.moe_route_workspace_bytes(4, 64, 8, 5) == 0
    # T = 0 is a no-op
    assert L.moe_route(None, None, None, 0, 64, 8, 2, 1, None, None, None, None, 0, None) == 0
    # forward: shared-expert pointers inconsistent with d_ff_shared
    args = [fake, fake, None, fake, fake, fake, fake, None, None, 64, 4, 8, 2, 64, 64, 1,
            fake, 1 << 30, vp(0x2000), None]
    assert L.moe_forward(*args) == -1
    # forward: workspace too small
    args = [fake, fake, None, fake, fake, fake, None, None, None, 0, 4, 8, 2, 64, 64, 1,
            vp(0x100000), 16, vp(0x2000), None]
    assert L.moe_forward(*args) == -3
    # forward: misaligned workspace
    args[16] = vp(0x100010)
    args[17] = 1 << 40
    assert L.moe_forward(*args) == -3
    # forward: y aliasing x
    args = [fake, fake, None, fake, fake, fake, None, None, None, 0, 4, 8, 2, 64, 64, 1,
            vp(0x100000), 1 << 40, fake, None]
    assert L.moe_forward(*args) == -1
    # permute: too-small workspace
    assert L.moe_permute(fake, 4, 8, 2, fake, fake, fake, fake, vp(0x100000), 8, None) == -3
    # misaligned tensors (16 bytes for x, weights and y; 4 for fp32 / int32 arrays)
    for i in (0, 1, 3, 4, 5, 18):
        args = [fake, fake, None, fake, fake, fake, None, None, None, 0, 4, 8, 2, 64, 64, 1,
                vp(0x100000), 1 << 40, vp(0x2000), None]
        args[i] = vp(args[i].value + 8)
        assert L.moe_forward(*args) == -1, i
    args = [fake, fake, vp(0x3002), fake, fake, fake, None, None, None, 0, 4, 8, 2, 64, 64, 1,
            vp(0x100000), 1 << 40, vp(0x2000), None]
    assert L.moe_forward(*args) == -1  # bias
    assert L.moe_route(vp(0x1008), fake, None, 4, 64, 8, 2, 1, fake, fake, None, fake, big,
                       None) == -1
    assert L.moe_route(fake, fake, None, 4, 64, 8, 2, 1, vp(0x1002), fake, None, fake, big,
                       None) == -1
    assert L.moe_permute(vp(0x1002), 4, 8, 2, fake, fake, fake, fake, vp(0x100000), 1 << 30,
                         None) == -1


def test_variant_entry_points_check_arguments(L):
    from sparse_mixture_experts_permute_amd import moe
    vp = ctypes.c_void_p
    fake = vp(0x1000)
    big = 1 << 30
    # capacity of "Mistral 8x7B SMoE architecture deep dive", section 2.4:
    # min(k*T, floor(1.2*T)) -> 38 for a batch of 32 (k=2), 19 for 16
    assert moe.capacity(32, 2, 1.2) == 38
    assert moe.capacity(16, 2, 1.2) == 19
    assert moe.capacity(10, 1, 5.0) == 10   # never above k*T
    assert moe.capacity(0, 2, 1.2) == 0
    assert L.moe_capacity(-1, 2, 1.2) == -1
    assert L.moe_capacity(4, 0, 1.2) == -1
    assert L.moe_capacity(4, 2, -0.5) == -1
    # unknown gate mode; the entropy-aware mode needs k >= 2
    for mode, k in ((-1, 2), (5, 2), (3, 1), (4, 1)):
        assert L.moe_route_ex(fake, fake, None, 4, 64, 8, k, 1, mode, fake, fake, None, fake, big,
                              None) == -1
    # unknown gate mode / activation in the forward options
    for gm, act, k in ((5, 0, 2), (0, 2, 2), (-1, 0, 2), (3, 0, 1), (4, 0, 1)):
        opt = moe._Options(gm, act, -1, 0)
        args = [fake, fake, None, fake, fake, fake, None, None, None, 0, 4, 8, k, 64, 64, 1,
                ctypes.byref(opt), vp(0x100000), 1 << 40, vp(0x2000), None]
        assert L.moe_forward_ex(*args) == -1
    # an unknown weight layout
    for lay in (-1, 2):
        opt = moe._Options(0, 0, -1, lay)
        args = [fake, fake, None, fake, fake, fake, None, None, None, 0, 4, 8, 2, 64, 64, 1,
                ctypes.byref(opt), vp(0x100000), 1 << 40, vp(0x2000), None]
        assert L.moe_forward_ex(*args) == -1
    # FP8 experts: quantiser dtype / sizes; the forward serves decode-sized
    # batches (weight streaming up to four tokens, 64-row tiles up to 96 rows
    # per expert), expert weights [out][in] only
    assert L.moe_quantize_fp8(fake, 4, 16, 7, fake, fake, None) == -2
    assert L.moe_quantize_fp8(fake, -1, 16, 1, fake, fake, None) == -1
    assert L.moe_quantize_fp8(None, 0, 16, 1, None, None, None) == 0
    for T, d, dff in ((4096, 2048, 2048), (5, 192, 256), (2, 2048, 192)):
        assert L.moe_forward_fp8(fake, fake, None, fake, fake, fake, fake, fake, fake, T, 8, 2,
                                 d, dff, None, vp(0x100000), 1 << 40, vp(0x2000), None) == -1
    opt = moe._Options(0, 0, -1, 1)
    assert L.moe_forward_fp8(fake, fake, None, fake, fake, fake, fake, fake, fake, 8, 8, 2,
                             2048, 2048, ctypes.byref(opt), vp(0x100000), 1 << 40, vp(0x2000),
                             None) == -1
    # permute_ex: too-small workspace is still caught
    assert L.moe_permute_ex(fake, 4, 8, 2, 3, fake, fake, fake, fake, vp(0x100000), 8,
                            None) == -3


def _layer_tensors(dtype=None, E=4, d=64, d_ff=128):
    import torch
    dtype = dtype or torch.bfloat16
    return dict(Wg=torch.zeros(E, d, dtype=dtype), W1=torch.zeros(E, d_ff, d, dtype=dtype),
                W3=torch.zeros(E, d_ff, d, dtype=dtype), W2=torch.zeros(E, d, d_ff, dtype=dtype))


def test_binding_rejects_mismatched_layers():
    """The binding checks shapes, dtypes and devices before calling the
    library, whose one dtype covers every tensor of a call."""
    import torch

    from sparse_mixture_experts_permute_amd import moe
    t = _layer_tensors()
    moe.MoELayer(t["Wg"], t["W1"], t["W3"], t["W2"], 2)  # consistent: accepted
    bad = [
        dict(W3=torch.zeros(4, 128, 64, dtype=torch.float32)),  # dtype differs
        dict(W3=torch.zeros(4, 64, 128, dtype=torch.bfloat16)),  # W3 not like W1
        dict(W2=torch.zeros(4, 128, 64, dtype=torch.bfloat16)),  # W2 transposed
        dict(Wg=torch.zeros(3, 64, dtype=torch.bfloat16)),  # fewer router rows than E
        dict(Wg=torch.zeros(4, 64, dtype=torch.float32)),  # router dtype
    ]
    for change in bad:
        u = dict(t, **change)
        with pytest.raises(moe.MoEError):
            moe.MoELayer(u["Wg"], u["W1"], u["W3"], u["W2"], 2)
    with pytest.raises(moe.MoEError):  # bias must be fp32 [E]
        moe.MoELayer(t["Wg"], t["W1"], t["W3"], t["W2"], 2, bias=torch.zeros(4, dtype=torch.bfloat16))
    with pytest.raises(moe.MoEError):
        moe.MoELayer(t["Wg"], t["W1"], t["W3"], t["W2"], 2, bias=torch.zeros(5))
    sh = (torch.zeros(32, 64, dtype=torch.bfloat16), torch.zeros(32, 64, dtype=torch.bfloat16),
          torch.zeros(64, 32, dtype=torch.bfloat16))
    moe.MoELayer(t["Wg"], t["W1"], t["W3"], t["W2"], 2, shared=sh)
    with pytest.raises(moe.MoEError):  # Ws2 must be [d][d_ff_shared]
        moe.MoELayer(t["Wg"], t["W1"], t["W3"], t["W2"], 2, shared=(sh[0], sh[1], sh[0]))


def test_binding_rejects_mismatched_tokens():
    import torch

    from sparse_mixture_experts_permute_amd import moe
    t = _layer_tensors()
    layer = moe.MoELayer(t["Wg"], t["W1"], t["W3"], t["W2"], 2)
    for x, y in [(torch.zeros(8, 64, dtype=torch.float32), None),  # x dtype differs
                 (torch.zeros(8, 32, dtype=torch.bfloat16), None),  # x width is not d
                 (torch.zeros(8, 64, dtype=torch.bfloat16),
                  torch.zeros(8, 64, dtype=torch.float32)),  # y dtype differs
                 (torch.zeros(8, 64, dtype=torch.bfloat16),
                  torch.zeros(4, 64, dtype=torch.bfloat16)),  # y too short
                 (torch.zeros(8, 64, dtype=torch.bfloat16), None)]:  # host tensors
        with pytest.raises(moe.MoEError):
            layer(x, y)
    with pytest.raises(moe.MoEError):  # router dtype differs from x
        moe.route(torch.zeros(8, 64, dtype=torch.bfloat16), torch.zeros(4, 64), 2)
    with pytest.raises(moe.MoEError):
        moe.route(torch.zeros(8, 64), torch.zeros(4, 32), 2)


def test_noalloc_rejects_before_launch(L):
    """moe_forward_noalloc checks its arguments, and that the shape fits its
    static scratch, before it touches a device."""
    fake = ctypes.c_void_p(0x1000)
    args = [fake, fake, None, fake, fake, fake, None, None, None, 0]
    # 1.1 GB of scratch for the Mixtral-shaped layer at 8192 tokens: too large
    assert L.moe_forward_noalloc(*args, 8192, 8, 2, 4096, 14336, 1, fake, None) == -6
    assert L.moe_forward_noalloc(*args, 8, 8, 9, 4096, 14336, 1, fake, None) == -1  # k > E
    assert L.moe_forward_noalloc(*args, 8, 8, 2, 4096, 14336, 5, fake, None) == -2  # dtype
    assert b"static" in L.moe_strerror(-6)


def test_capacity_mean(L):
    """ceil(cf * T * k / E): 1.2 x the mean load of the Mixtral-shaped prefill
    (8192 tokens, top-2, 8 experts: mean 2048) is 2457.6 -> 2458."""
    assert L.moe_capacity_mean(8192, 2, 8, 1.2) == 2458
    assert L.moe_capacity_mean(512, 8, 128, 1.0) == 32
    assert L.moe_capacity_mean(512, 8, 128, 1.25) == 40
    assert L.moe_capacity_mean(1, 1, 256, 1.0) == 1
    assert L.moe_capacity_mean(0, 2, 8, 1.2) == 0
    assert L.moe_capacity_mean(-1, 2, 8, 1.2) == -1
    assert L.moe_capacity_mean(4, 2, 0, 1.2) == -1


def test_c_caller_built_and_linked():
    """The plain C caller of the ABI (run on the GPU by test_gpu_c_abi.py) is
    built and resolves the library and the HIP runtime: without arguments it
    prints its usage before touching a device."""
    import subprocess

    from sparse_mixture_experts_permute_amd.build import C_CALLER
    assert os.path.exists(C_CALLER), f"{C_CALLER} not built (the package build compiles it)"
    r = subprocess.run([C_CALLER], capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "usage" in r.stderr
