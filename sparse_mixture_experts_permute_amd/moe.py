"""Thin torch-facing binding of the C ABI in ``include/moe_mi355x.h``.

Argument marshalling only: every step of the layer runs in the HIP library
``libmoe_mi355x.so``.  Tensors must be contiguous and on the current HIP
device; work is enqueued on torch's current stream.  There is no fallback: if
the library is missing or the device is not a gfx950 GPU the calls raise.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")

MOE_F32, MOE_BF16 = 0, 1
GATE_SOFTMAX_TOPK, GATE_SOFTMAX_ALL, GATE_SIGMOID, GATE_ENTROPY = 0, 1, 2, 3
GATE_ENTROPY_BATCH = 4
ACT_SWIGLU, ACT_GLU_SIGMOID = 0, 1
LAYOUT_OUT_IN, LAYOUT_IN_OUT = 0, 1
NSTAGE_EVENTS = 8
STAGES = ("router", "permute", "gather", "gemm_swiglu", "gemm_down", "shared_expert", "combine")
WS_FIELDS = ("logits", "idx", "gate", "counts", "offsets", "perm", "inv")

_lib = None


class _Options(ctypes.Structure):
    _fields_ = [("gate_mode", ctypes.c_int), ("activation", ctypes.c_int),
                ("capacity", ctypes.c_int), ("weight_layout", ctypes.c_int)]


class MoEError(RuntimeError):
    pass


def lib():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MoEError(f"HIP library not built: {LIB_PATH} "
                           "(run python -m sparse_mixture_experts_permute_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.moe_route_workspace_bytes.argtypes = [i, i, i, i]
        L.moe_route_workspace_bytes.restype = sz
        L.moe_route.argtypes = [vp, vp, vp, i, i, i, i, i, vp, vp, vp, vp, sz, vp]
        L.moe_route.restype = i
        L.moe_permute_workspace_bytes.argtypes = [i, i, i]
        L.moe_permute_workspace_bytes.restype = sz
        L.moe_permute.argtypes = [vp, i, i, i, vp, vp, vp, vp, vp, sz, vp]
        L.moe_permute.restype = i
        L.moe_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
        L.moe_workspace_bytes.restype = sz
        L.moe_workspace_offsets.argtypes = [i, i, i, i, i, i, i, ctypes.POINTER(sz)]
        L.moe_workspace_offsets.restype = i
        L.moe_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp,
                                  sz, vp, vp]
        L.moe_forward.restype = i
        L.moe_forward_timed.argtypes = (L.moe_forward.argtypes[:16] + [ctypes.POINTER(_Options)]
                                        + L.moe_forward.argtypes[16:] + [vp])
        L.moe_forward_timed.restype = i
        L.moe_strerror.argtypes = [i]
        L.moe_strerror.restype = ctypes.c_char_p
        L.moe_capacity.argtypes = [i, i, ctypes.c_double]
        L.moe_capacity.restype = i
        L.moe_capacity_mean.argtypes = [i, i, i, ctypes.c_double]
        L.moe_capacity_mean.restype = i
        L.moe_route_ex.argtypes = [vp, vp, vp, i, i, i, i, i, i, vp, vp, vp, vp, sz, vp]
        L.moe_route_ex.restype = i
        L.moe_permute_ex.argtypes = [vp, i, i, i, i, vp, vp, vp, vp, vp, sz, vp]
        L.moe_permute_ex.restype = i
        L.moe_forward_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i,
                                     ctypes.POINTER(_Options), vp, sz, vp, vp]
        L.moe_forward_ex.restype = i
        L.moe_quantize_fp8.argtypes = [vp, i, ctypes.c_longlong, i, vp, vp, vp]
        L.moe_quantize_fp8.restype = i
        L.moe_forward_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i,
                                      ctypes.POINTER(_Options), vp, sz, vp, vp]
        L.moe_forward_fp8.restype = i
        L.moe_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i,
                                          i, vp, vp]
        L.moe_forward_noalloc.restype = i
        L.moe_forward_inout.argtypes = L.moe_forward.argtypes
        L.moe_forward_inout.restype = i
        _lib = L
    return _lib


def _check(rc: int, what: str):
    if rc != 0:
        raise MoEError(f"{what}: {lib().moe_strerror(rc).decode()} (status {rc})")


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise MoEError(f"unsupported dtype {t.dtype}")


def _p(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise MoEError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _same(t, ref, shape, name):
    """t must have `shape`, ref's dtype and ref's device (MoEError otherwise)."""
    if tuple(t.shape) != tuple(shape):
        raise MoEError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != ref.dtype:
        raise MoEError(f"{name}: dtype {t.dtype}, expected {ref.dtype}")
    if t.device != ref.device:
        raise MoEError(f"{name}: on {t.device}, expected {ref.device}")


def _check_bias(bias, E, ref):
    if bias is None:
        return
    if tuple(bias.shape) != (E,) or bias.dtype != torch.float32:
        raise MoEError(f"bias: expected fp32 [{E}], got {bias.dtype} {tuple(bias.shape)}")
    if bias.device != ref.device:
        raise MoEError(f"bias: on {bias.device}, expected {ref.device}")


def _check_tokens(x, y, d, ref):
    """x [..., d] (and y of x's shape) with ref's dtype and device."""
    if x.dim() < 1 or x.shape[-1] != d:
        raise MoEError(f"x: last dimension {tuple(x.shape)[-1:]} , expected {d}")
    _same(x, ref, x.shape, "x")
    if x.device.type != "cuda":
        raise MoEError(f"x: on {x.device}; the layer runs on a HIP device")
    if y is not None:
        _same(y, ref, x.shape, "y")
        if y.data_ptr() == x.data_ptr():
            raise MoEError("y may not alias x")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def tensor_from_numpy(a: np.ndarray, device="cuda") -> torch.Tensor:
    """numpy -> device tensor; uint16 arrays are taken as bf16 bit patterns."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def tensor_to_numpy(t: torch.Tensor) -> np.ndarray:
    """device tensor -> numpy; bf16 comes back as uint16 bit patterns."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def capacity(T: int, k: int, capacity_factor: float = 1.2) -> int:
    """Per-expert capacity min(k*T, floor(cf*T)) for a batch of T tokens."""
    c = lib().moe_capacity(T, k, float(capacity_factor))
    if c < 0:
        raise MoEError("invalid capacity arguments")
    return c


def capacity_mean(T: int, k: int, E: int, capacity_factor: float = 1.2) -> int:
    """Per-expert capacity ceil(cf * T * k / E): cf times an expert's mean load."""
    c = lib().moe_capacity_mean(T, k, E, float(capacity_factor))
    if c < 0:
        raise MoEError("invalid capacity arguments")
    return c


def route(x: torch.Tensor, Wg: torch.Tensor, k: int, bias: torch.Tensor | None = None,
          gate_mode: int = GATE_SOFTMAX_TOPK):
    """(idx [T][k] int32, gate [T][k] fp32, logits [T][E] fp32)."""
    if x.dim() != 2 or Wg.dim() != 2:
        raise MoEError("route: x [T][d] and Wg [E][d]")
    T, d = x.shape
    E = Wg.shape[0]
    _same(Wg, x, (E, d), "Wg")
    _check_bias(bias, E, x)
    if x.device.type != "cuda":
        raise MoEError(f"x: on {x.device}; the router runs on a HIP device")
    idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    gate = torch.empty((T, k), dtype=torch.float32, device=x.device)
    logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    nbytes = lib().moe_route_workspace_bytes(T, d, E, _dt(x))
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=x.device)
    _check(lib().moe_route_ex(_p(x), _p(Wg), _p(bias), T, d, E, k, _dt(x), int(gate_mode),
                              _p(idx), _p(gate), _p(logits), _p(ws), nbytes, _stream()),
           "moe_route_ex")
    return idx, gate, logits


def permute(idx: torch.Tensor, E: int, capacity: int = -1):
    """(counts [E], offsets [E+1], perm [T*k], inv [T*k]), all int32.  Under a
    capacity only kept pairs are placed (perm has offsets[E] valid entries)
    and inv is -1 for a dropped pair."""
    T, k = idx.shape
    dev = idx.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    inv = torch.empty(T * k, dtype=torch.int32, device=dev)
    nbytes = lib().moe_permute_workspace_bytes(T, E, k)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    _check(lib().moe_permute_ex(_p(idx), T, E, k, int(capacity), _p(counts), _p(offsets),
                                _p(perm), _p(inv), _p(ws), nbytes, _stream()), "moe_permute_ex")
    return counts, offsets, perm, inv


def workspace_bytes(T, d, d_ff, E, k, d_ff_shared=0, dtype=MOE_BF16) -> int:
    n = lib().moe_workspace_bytes(T, d, d_ff, E, k, d_ff_shared, dtype)
    if n == 0:
        raise MoEError("invalid layer shape")
    return n


def workspace_offsets(T, d, d_ff, E, k, d_ff_shared=0, dtype=MOE_BF16) -> dict:
    arr = (ctypes.c_size_t * len(WS_FIELDS))()
    _check(lib().moe_workspace_offsets(T, d, d_ff, E, k, d_ff_shared, dtype, arr),
           "moe_workspace_offsets")
    return dict(zip(WS_FIELDS, list(arr)))


class MoELayer:
    """One layer's weights plus a reusable workspace.

    Expert weights in the layout `weight_layout` names: LAYOUT_OUT_IN (Linear
    weights) W1, W3 [E][d_ff][d], W2 [E][d][d_ff], shared (Ws1 [dffs][d], Ws3
    [dffs][d], Ws2 [d][dffs]); LAYOUT_IN_OUT (x @ W) W1, W3 [E][d][d_ff], W2
    [E][d_ff][d], shared (Ws1 [d][dffs], Ws3 [d][dffs], Ws2 [dffs][d]).
    Wg [E][d]; optional bias [E] fp32.  The variants (gate_mode, activation,
    capacity) follow moe_options in the C header; the defaults are the method
    itself.
    """

    def __init__(self, Wg, W1, W3, W2, k, bias=None, shared=None,
                 gate_mode=GATE_SOFTMAX_TOPK, activation=ACT_SWIGLU, capacity=-1,
                 weight_layout=LAYOUT_OUT_IN):
        self.Wg, self.W1, self.W3, self.W2, self.k, self.bias = Wg, W1, W3, W2, k, bias
        if weight_layout not in (LAYOUT_OUT_IN, LAYOUT_IN_OUT):
            raise MoEError(f"unknown weight layout {weight_layout}")
        self.inout = weight_layout == LAYOUT_IN_OUT
        self.options = _Options(int(gate_mode), int(activation), int(capacity),
                                int(weight_layout))
        self._default = (gate_mode == GATE_SOFTMAX_TOPK and activation == ACT_SWIGLU
                         and capacity < 0)
        if W1.dim() != 3:
            raise MoEError("W1: expected a 3-d expert tensor")
        if self.inout:
            self.E, self.d, self.d_ff = W1.shape
        else:
            self.E, self.d_ff, self.d = W1.shape
        self.dtype = _dt(W1)
        E, d, d_ff = self.E, self.d, self.d_ff
        io = (lambda a, b: (b, a)) if self.inout else (lambda a, b: (a, b))  # [out][in]
        _same(W3, W1, (E,) + io(d_ff, d), "W3")
        _same(W2, W1, (E,) + io(d, d_ff), "W2")
        _same(Wg, W1, (E, d), "Wg")
        _check_bias(bias, E, W1)
        self.shared = shared
        self.d_ff_shared = 0
        if shared is not None:
            Ws1, Ws3, Ws2 = shared
            if Ws1.dim() != 2:
                raise MoEError("Ws1: expected a 2-d matrix")
            dffs = Ws1.shape[1] if self.inout else Ws1.shape[0]
            _same(Ws1, W1, io(dffs, d), "Ws1")
            _same(Ws3, W1, io(dffs, d), "Ws3")
            _same(Ws2, W1, io(d, dffs), "Ws2")
            self.d_ff_shared = dffs
        self._ws = None
        self._ws_T = -1

    def workspace(self, T):
        n = workspace_bytes(T, self.d, self.d_ff, self.E, self.k, self.d_ff_shared, self.dtype)
        if self._ws is None or self._ws.numel() < n:
            self._ws = torch.empty(n, dtype=torch.uint8, device=self.W1.device)
        return self._ws, n

    def __call__(self, x: torch.Tensor, y: torch.Tensor | None = None) -> torch.Tensor:
        _check_tokens(x, y, self.d, self.W1)
        shape = x.shape
        x2 = x.reshape(-1, self.d)  # batch dims flattened into tokens
        T = x2.shape[0]
        if y is None:
            y = torch.empty_like(x2)
        ws, n = self.workspace(T)
        Ws1, Ws3, Ws2 = self.shared if self.shared is not None else (None, None, None)
        if self._default and self.inout:
            _check(lib().moe_forward_inout(_p(x2), _p(self.Wg), _p(self.bias), _p(self.W1),
                                           _p(self.W3), _p(self.W2), _p(Ws1), _p(Ws3), _p(Ws2),
                                           self.d_ff_shared, T, self.E, self.k, self.d,
                                           self.d_ff, self.dtype, _p(ws), n, _p(y), _stream()),
                   "moe_forward_inout")
        elif self._default:
            _check(lib().moe_forward(_p(x2), _p(self.Wg), _p(self.bias), _p(self.W1),
                                     _p(self.W3), _p(self.W2), _p(Ws1), _p(Ws3), _p(Ws2),
                                     self.d_ff_shared, T, self.E, self.k, self.d, self.d_ff,
                                     self.dtype, _p(ws), n, _p(y), _stream()), "moe_forward")
        else:
            _check(lib().moe_forward_ex(_p(x2), _p(self.Wg), _p(self.bias), _p(self.W1),
                                        _p(self.W3), _p(self.W2), _p(Ws1), _p(Ws3), _p(Ws2),
                                        self.d_ff_shared, T, self.E, self.k, self.d, self.d_ff,
                                        self.dtype, ctypes.byref(self.options), _p(ws), n, _p(y),
                                        _stream()), "moe_forward_ex")
        return y.reshape(shape)

    def timed(self, x: torch.Tensor, y: torch.Tensor, events) -> torch.Tensor:
        """Same as a call, recording `events` (NSTAGE_EVENTS torch.cuda.Event,
        already created by a record) at the stage boundaries on the stream."""
        _check_tokens(x, y, self.d, self.W1)
        T = x.shape[0]
        ws, n = self.workspace(T)
        Ws1, Ws3, Ws2 = self.shared if self.shared is not None else (None, None, None)
        handles = (ctypes.c_void_p * NSTAGE_EVENTS)(*[ctypes.c_void_p(e.cuda_event)
                                                      for e in events])
        _check(lib().moe_forward_timed(_p(x), _p(self.Wg), _p(self.bias), _p(self.W1),
                                       _p(self.W3), _p(self.W2), _p(Ws1), _p(Ws3), _p(Ws2),
                                       self.d_ff_shared, T, self.E, self.k, self.d, self.d_ff,
                                       self.dtype, ctypes.byref(self.options), _p(ws), n, _p(y),
                                       _stream(), handles),
               "moe_forward_timed")
        return y

    def intermediates(self, T) -> dict:
        """Views of the routing intermediates of the last call with T tokens."""
        off = workspace_offsets(T, self.d, self.d_ff, self.E, self.k, self.d_ff_shared,
                                self.dtype)
        ws = self._ws
        P = T * self.k

        def view(name, n, dtype):
            o = off[name]
            return ws[o:o + n * 4].view(dtype)

        return dict(logits=view("logits", T * self.E, torch.float32).view(T, self.E),
                    idx=view("idx", P, torch.int32).view(T, self.k),
                    gate=view("gate", P, torch.float32).view(T, self.k),
                    counts=view("counts", self.E, torch.int32),
                    offsets=view("offsets", self.E + 1, torch.int32),
                    perm=view("perm", P, torch.int32), inv=view("inv", P, torch.int32))


def forward(x, Wg, W1, W3, W2, k, bias=None, shared=None, **variants):
    """y = MoE(x) for x [..., d] (allocates its workspace); `variants` are
    MoELayer's gate_mode / activation / capacity."""
    return MoELayer(Wg, W1, W3, W2, k, bias, shared, **variants)(x)


def quantize_fp8(W: torch.Tensor):
    """Per-expert FP8 (E4M3) quantisation of expert weights W [E, ...] (bf16 or
    fp32) on the GPU: (codes uint8 of W's shape, scale fp32 [E])."""
    E = W.shape[0]
    q = torch.empty(W.shape, dtype=torch.uint8, device=W.device)
    scale = torch.empty(E, dtype=torch.float32, device=W.device)
    _check(lib().moe_quantize_fp8(_p(W), E, W.numel() // max(E, 1), _dt(W), _p(q), _p(scale),
                                  _stream()), "moe_quantize_fp8")
    return q, scale


class MoELayerFP8:
    """A layer whose experts hold FP8 weights (decode: at most four tokens per
    call).  Built from bf16 weights, quantised once on the GPU; the router
    stays bf16."""

    def __init__(self, Wg, W1, W3, W2, k, bias=None, gate_mode=GATE_SOFTMAX_TOPK,
                 activation=ACT_SWIGLU, capacity=-1):
        self.Wg, self.k, self.bias = Wg, k, bias
        if W1.dim() != 3 or W1.dtype != torch.bfloat16:
            raise MoEError("W1: expected bf16 [E][d_ff][d]")
        self.E, self.d_ff, self.d = W1.shape
        E, d, d_ff = self.E, self.d, self.d_ff
        _same(W3, W1, (E, d_ff, d), "W3")
        _same(W2, W1, (E, d, d_ff), "W2")
        _same(Wg, W1, (E, d), "Wg")
        _check_bias(bias, E, W1)
        self.W1q, self.s1 = quantize_fp8(W1)
        self.W3q, self.s3 = quantize_fp8(W3)
        self.W2q, self.s2 = quantize_fp8(W2)
        self.options = _Options(int(gate_mode), int(activation), int(capacity), LAYOUT_OUT_IN)
        self._ws = None

    def workspace(self, T):
        n = workspace_bytes(T, self.d, self.d_ff, self.E, self.k, 0, MOE_BF16)
        if self._ws is None or self._ws.numel() < n:
            self._ws = torch.empty(n, dtype=torch.uint8, device=self.W1q.device)
        return self._ws, n

    def __call__(self, x: torch.Tensor, y: torch.Tensor | None = None) -> torch.Tensor:
        if x.dim() != 2:
            raise MoEError("x: expected [T][d]")
        _check_tokens(x, y, self.d, self.Wg)
        T = x.shape[0]
        if y is None:
            y = torch.empty_like(x)
        ws, n = self.workspace(T)
        _check(lib().moe_forward_fp8(_p(x), _p(self.Wg), _p(self.bias), _p(self.W1q),
                                     _p(self.W3q), _p(self.W2q), _p(self.s1), _p(self.s3),
                                     _p(self.s2), T, self.E, self.k, self.d, self.d_ff,
                                     ctypes.byref(self.options), _p(ws), n, _p(y), _stream()),
               "moe_forward_fp8")
        return y

    def intermediates(self, T) -> dict:
        """Routing intermediates of the last call (as MoELayer.intermediates)."""
        proxy = MoELayer.__new__(MoELayer)
        proxy.d, proxy.d_ff, proxy.E, proxy.k = self.d, self.d_ff, self.E, self.k
        proxy.d_ff_shared, proxy.dtype, proxy._ws = 0, MOE_BF16, self._ws
        return MoELayer.intermediates(proxy, T)
