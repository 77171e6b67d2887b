"""Python access to the CPU oracle (``moe_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the test suite, by the smoke entry point
and by the benchmark's CPU-baseline leg.  The product path (the HIP library and
its binding) never imports this module.

Every function takes numpy arrays in the layouts documented in
``moe_oracle.c`` and returns fp64 results (int32 for indices).  bf16 inputs are
passed as uint16 bit patterns, fp32 inputs as float32.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16, F64 = 0, 1, 2
# gate variants (orc_gate_mode) and expert activations (swiglu in moe_oracle.c)
GATE_SOFTMAX_TOPK, GATE_SOFTMAX_ALL, GATE_SIGMOID, GATE_ENTROPY = 0, 1, 2, 3
GATE_ENTROPY_BATCH = 4  # the entropy-aware routing with the batch's largest k
# the entropy-aware routing's temperature and entropy threshold as printed
ENTROPY_TAU, ENTROPY_THRESHOLD = 0.1, 0.8
ACT_SWIGLU, ACT_GLU_SIGMOID = 0, 1


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
             "-ffp-contract=off", "-fno-fast-math", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None
_current = None


def _bind(path: str):
    """Load an oracle shared library and declare its signatures."""
    L = ctypes.CDLL(path)
    vp, i32p, f64p, f32p = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    L.orc_logits.argtypes = [vp, vp, f32p, ctypes.c_int, ctypes.c_long, ctypes.c_int,
                             ctypes.c_int, f64p]
    L.orc_topk.argtypes = [f64p, ctypes.c_long, ctypes.c_int, ctypes.c_int, i32p]
    L.orc_topk.restype = ctypes.c_int
    L.orc_gate.argtypes = [f64p, i32p, ctypes.c_long, ctypes.c_int, ctypes.c_int, f64p]
    L.orc_count.argtypes = [i32p, ctypes.c_long, ctypes.c_int, ctypes.c_int, i32p, i32p]
    L.orc_permute.argtypes = [i32p, ctypes.c_long, ctypes.c_int, ctypes.c_int, i32p, i32p,
                              i32p]
    L.orc_swiglu_row.argtypes = [vp, ctypes.c_int, ctypes.c_long, ctypes.c_int, vp, vp, vp,
                                 ctypes.c_int, ctypes.c_int, ctypes.c_int, f64p]
    L.orc_gate_mode.argtypes = [f64p, i32p, ctypes.c_long, ctypes.c_int, ctypes.c_int,
                                ctypes.c_int, f64p]
    L.orc_capacity.argtypes = [ctypes.c_long, ctypes.c_int, ctypes.c_double]
    L.orc_capacity.restype = ctypes.c_long
    L.orc_keep.argtypes = [i32p, ctypes.c_long, ctypes.c_int, ctypes.c_int, ctypes.c_long, i32p]
    L.orc_entropy.argtypes = [f64p, ctypes.c_long, ctypes.c_int, ctypes.c_double, f64p]
    L.orc_fp8_decode.argtypes = [ctypes.c_uint8]
    L.orc_fp8_decode.restype = ctypes.c_double
    L.orc_fp8_encode.argtypes = [ctypes.c_double]
    L.orc_fp8_encode.restype = ctypes.c_uint8
    L.orc_quantize_fp8.argtypes = [vp, ctypes.c_int, ctypes.c_long, ctypes.c_long, vp, f32p]
    L.orc_dequant_fp8.argtypes = [vp, ctypes.c_long, ctypes.c_long, f32p, f64p]
    L.orc_route_entropy.argtypes = [f64p, ctypes.c_long, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_double, ctypes.c_double, i32p, f64p]
    L.orc_route_entropy.restype = ctypes.c_int
    L.orc_route_entropy_batch.argtypes = L.orc_route_entropy.argtypes
    L.orc_route_entropy_batch.restype = ctypes.c_int
    L.orc_forward_ex.argtypes = ([vp, vp, f32p, vp, vp, vp, vp, vp, vp, ctypes.c_int,
                                  ctypes.c_long, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_long]
                                 + [f64p, f64p, i32p, f64p, i32p, i32p, i32p, i32p, f64p])
    L.orc_forward_ex.restype = ctypes.c_int
    L.orc_forward.argtypes = ([vp, vp, f32p, vp, vp, vp, vp, vp, vp, ctypes.c_int,
                               ctypes.c_long, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                               ctypes.c_int, ctypes.c_int]
                              + [f64p, f64p, i32p, f64p, i32p, i32p, i32p, i32p, f64p])
    L.orc_forward.restype = ctypes.c_int
    L.orc_forward_rows.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_long, vp, i32p, f64p, f64p]
    L.orc_param_count.argtypes = [ctypes.c_longlong] * 3
    L.orc_param_count.restype = ctypes.c_longlong
    L.orc_active_fraction.argtypes = [ctypes.c_int, ctypes.c_int]
    L.orc_active_fraction.restype = ctypes.c_double
    L.orc_num_threads.restype = ctypes.c_int
    L.orc_set_threads.argtypes = [ctypes.c_int]
    L.orc_set_threads.restype = None
    return L


def lib():
    """The oracle library in use (the built one unless ``use_library`` swapped it)."""
    global _lib
    if _current is not None:
        return _current
    if _lib is None:
        build()
        _lib = _bind(_LIB)
    return _lib


def use_library(path: str | None):
    """Route this module's functions to another build of the oracle source
    (used by the tests that plant a mistake in a copy of it); None restores."""
    global _current
    _current = None if path is None else _bind(path)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"oracle inputs are float32, float64 or bf16 bits (uint16), got {a.dtype}")


def _c(a, dtype=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))
    return a


def logits(x, Wg, bias=None):
    x, Wg = _c(x), _c(Wg)
    bias = _c(bias, np.float32)
    T, d = x.shape
    E = Wg.shape[0]
    assert Wg.shape == (E, d) and Wg.dtype == x.dtype
    out = np.empty((T, E), np.float64)
    lib().orc_logits(_ptr(x), _ptr(Wg), _ptr(bias), _dtype_code(x), T, d, E, _ptr(out))
    return out


def topk(lg, k):
    lg = _c(lg, np.float64)
    T, E = lg.shape
    idx = np.empty((T, k), np.int32)
    if lib().orc_topk(_ptr(lg), T, E, k, _ptr(idx)) != 0:
        raise ValueError("k must satisfy 1 <= k <= E")
    return idx


def gate(lg, idx):
    lg, idx = _c(lg, np.float64), _c(idx, np.int32)
    T, E = lg.shape
    k = idx.shape[1]
    g = np.empty((T, k), np.float64)
    lib().orc_gate(_ptr(lg), _ptr(idx), T, E, k, _ptr(g))
    return g


def gate_mode(lg, idx, mode):
    """Gates of one of the variants (GATE_SOFTMAX_TOPK, GATE_SOFTMAX_ALL, GATE_SIGMOID)."""
    lg, idx = _c(lg, np.float64), _c(idx, np.int32)
    T, E = lg.shape
    k = idx.shape[1]
    g = np.empty((T, k), np.float64)
    lib().orc_gate_mode(_ptr(lg), _ptr(idx), T, E, k, int(mode), _ptr(g))
    return g


def entropy(lg, tau=ENTROPY_TAU):
    """Entropy (natural log) of each token's softmax(logits / tau) over all experts."""
    lg = _c(lg, np.float64)
    T, E = lg.shape
    H = np.empty(T, np.float64)
    lib().orc_entropy(_ptr(lg), T, E, float(tau), _ptr(H))
    return H


def route_entropy(lg, k, tau=ENTROPY_TAU, threshold=ENTROPY_THRESHOLD):
    """(idx, gate) of the entropy-aware routing: k experts where the entropy is
    above the threshold, else k - 1 (the last slot then holds idx -1, gate 0)."""
    lg = _c(lg, np.float64)
    T, E = lg.shape
    idx = np.empty((T, k), np.int32)
    g = np.empty((T, k), np.float64)
    if lib().orc_route_entropy(_ptr(lg), T, E, k, float(tau), float(threshold), _ptr(idx),
                               _ptr(g)) != 0:
        raise ValueError("entropy-aware routing needs 2 <= k <= E")
    return idx, g


def route_entropy_batch(lg, k, tau=ENTROPY_TAU, threshold=ENTROPY_THRESHOLD):
    """(idx, gate, kb) of the entropy-aware routing with one k for the batch:
    kb = the largest per-token k (k where the entropy is above the threshold,
    else k - 1); every token keeps its top kb experts, and the slot past kb
    holds idx -1, gate 0."""
    lg = _c(lg, np.float64)
    T, E = lg.shape
    idx = np.empty((T, k), np.int32)
    g = np.empty((T, k), np.float64)
    kb = lib().orc_route_entropy_batch(_ptr(lg), T, E, k, float(tau), float(threshold),
                                       _ptr(idx), _ptr(g))
    if kb < 0:
        raise ValueError("entropy-aware routing needs 2 <= k <= E")
    return idx, g, kb


def fp8_decode(codes):
    """E4M3 (OCP, 'FN') value of each uint8 code (fp64)."""
    return np.array([lib().orc_fp8_decode(int(c)) for c in np.asarray(codes).reshape(-1)],
                    np.float64).reshape(np.shape(codes))


def fp8_encode(values):
    """Nearest E4M3 code of each value (ties to even; above 448 gives 448)."""
    return np.array([lib().orc_fp8_encode(float(v)) for v in np.asarray(values).reshape(-1)],
                    np.uint8).reshape(np.shape(values))


def quantize_fp8(W):
    """Per-expert FP8 quantisation of W [E, ...] (bf16 bits or float32):
    (codes uint8 of W's shape, scale float32 [E])."""
    W = _c(W)
    E = W.shape[0]
    n = W.size // E
    q = np.empty(W.shape, np.uint8)
    scale = np.empty(E, np.float32)
    lib().orc_quantize_fp8(_ptr(W), _dtype_code(W), E, n, _ptr(q), _ptr(scale))
    return q, scale


def dequant_fp8(q, scale):
    """scale[e] * decode(q[e]) in fp64, q [E, ...]."""
    q, scale = _c(q, np.uint8), _c(scale, np.float32)
    E = q.shape[0]
    out = np.empty(q.shape, np.float64)
    lib().orc_dequant_fp8(_ptr(q), E, q.size // E, _ptr(scale), _ptr(out))
    return out


def capacity(T, k, cf) -> int:
    """Per-expert capacity min(k*T, floor(cf*T))."""
    return int(lib().orc_capacity(T, k, float(cf)))


def keep(idx, E, cap):
    """1 for the pairs an expert keeps under capacity `cap` (first by pair id)."""
    idx = _c(idx, np.int32)
    T, k = idx.shape
    out = np.empty(T * k, np.int32)
    lib().orc_keep(_ptr(idx), T, E, k, int(cap), _ptr(out))
    return out


def route(x, Wg, k, bias=None, logits_in=None, gate_mode_=GATE_SOFTMAX_TOPK):
    """(logits, idx, gate) with the oracle's own fp64 logits or given ones."""
    lg = logits(x, Wg, bias) if logits_in is None else _c(logits_in, np.float64)
    if gate_mode_ == GATE_ENTROPY:
        return (lg,) + route_entropy(lg, k)
    if gate_mode_ == GATE_ENTROPY_BATCH:
        return (lg,) + route_entropy_batch(lg, k)[:2]
    idx = topk(lg, k)
    return lg, idx, gate_mode(lg, idx, gate_mode_)


def count(idx, E):
    idx = _c(idx, np.int32)
    T, k = idx.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    lib().orc_count(_ptr(idx), T, E, k, _ptr(counts), _ptr(offsets))
    return counts, offsets


def permute(idx, E):
    idx = _c(idx, np.int32)
    T, k = idx.shape
    counts, offsets = count(idx, E)
    perm = np.empty(T * k, np.int32)
    inv = np.empty(T * k, np.int32)
    lib().orc_permute(_ptr(idx), T, E, k, _ptr(offsets), _ptr(perm), _ptr(inv))
    return counts, offsets, perm, inv


def expert_row(x, t, W1, W3, W2, e, act=ACT_SWIGLU):
    """W2_e(act(W1_e x_t, W3_e x_t)) for one token (fp64, length d)."""
    x, W1, W3, W2 = _c(x), _c(W1), _c(W3), _c(W2)
    d = x.shape[1]
    dff = W1.shape[1]
    out = np.empty(d, np.float64)
    lib().orc_swiglu_row(_ptr(x), _dtype_code(x), t, d, _ptr(W1), _ptr(W3), _ptr(W2), e, dff,
                         int(act), _ptr(out))
    return out


def forward(x, Wg, W1, W3, W2, k, bias=None, shared=None, logits_in=None,
            gate_mode=GATE_SOFTMAX_TOPK, act=ACT_SWIGLU, capacity=None):
    """Whole layer through the permutation.  Returns a dict with y and every
    intermediate (logits, idx, gate, counts, offsets, perm, inv).  With a
    capacity, counts/offsets/perm cover the kept pairs (perm has offsets[E]
    entries) and inv is -1 for a dropped pair."""
    x, Wg, W1, W3, W2 = _c(x), _c(Wg), _c(W1), _c(W3), _c(W2)
    bias = _c(bias, np.float32)
    T, d = x.shape
    E, dff = W1.shape[0], W1.shape[1]
    assert W1.shape == (E, dff, d) and W3.shape == (E, dff, d) and W2.shape == (E, d, dff)
    dt = _dtype_code(x)
    Ws1 = Ws3 = Ws2 = None
    dffs = 0
    if shared is not None:
        Ws1, Ws3, Ws2 = (_c(a) for a in shared)
        dffs = Ws1.shape[0]
        assert Ws1.shape == (dffs, d) and Ws3.shape == (dffs, d) and Ws2.shape == (d, dffs)
    lg_in = None if logits_in is None else _c(logits_in, np.float64)
    P = T * k
    out = dict(logits=np.empty((T, E)), idx=np.empty((T, k), np.int32),
               gate=np.empty((T, k)), counts=np.empty(E, np.int32),
               offsets=np.empty(E + 1, np.int32), perm=np.empty(P, np.int32),
               inv=np.empty(P, np.int32), y=np.empty((T, d)))
    cap = P if capacity is None else int(capacity)
    if gate_mode == GATE_SOFTMAX_TOPK and act == ACT_SWIGLU and capacity is None:
        rc = lib().orc_forward(_ptr(x), _ptr(Wg), _ptr(bias), _ptr(W1), _ptr(W3), _ptr(W2),
                               _ptr(Ws1), _ptr(Ws3), _ptr(Ws2), dffs, T, E, k, d, dff, dt,
                               _ptr(lg_in), _ptr(out["logits"]), _ptr(out["idx"]),
                               _ptr(out["gate"]), _ptr(out["counts"]), _ptr(out["offsets"]),
                               _ptr(out["perm"]), _ptr(out["inv"]), _ptr(out["y"]))
    else:
        rc = lib().orc_forward_ex(_ptr(x), _ptr(Wg), _ptr(bias), _ptr(W1), _ptr(W3), _ptr(W2),
                                  _ptr(Ws1), _ptr(Ws3), _ptr(Ws2), dffs, T, E, k, d, dff, dt,
                                  int(gate_mode), int(act), cap, _ptr(lg_in),
                                  _ptr(out["logits"]), _ptr(out["idx"]), _ptr(out["gate"]),
                                  _ptr(out["counts"]), _ptr(out["offsets"]), _ptr(out["perm"]),
                                  _ptr(out["inv"]), _ptr(out["y"]))
    if rc != 0:
        raise ValueError("invalid layer shape, k or capacity")
    out["perm"] = out["perm"][: int(out["offsets"][E])]
    return out


def forward_rows(x, W1, W3, W2, tokens, idx_rows, gate_rows, shared=None, act=ACT_SWIGLU):
    """y rows for the listed tokens given those tokens' routing rows (a zero
    gate marks a dropped pair)."""
    x, W1, W3, W2 = _c(x), _c(W1), _c(W3), _c(W2)
    tokens = _c(np.asarray(tokens), np.int64)
    idx_rows, gate_rows = _c(idx_rows, np.int32), _c(gate_rows, np.float64)
    d = x.shape[1]
    dff = W1.shape[1]
    k = idx_rows.shape[1]
    Ws1 = Ws3 = Ws2 = None
    dffs = 0
    if shared is not None:
        Ws1, Ws3, Ws2 = (_c(a) for a in shared)
        dffs = Ws1.shape[0]
    n = tokens.shape[0]
    y = np.empty((n, d), np.float64)
    lib().orc_forward_rows(_ptr(x), _ptr(W1), _ptr(W3), _ptr(W2), _ptr(Ws1), _ptr(Ws3),
                           _ptr(Ws2), dffs, k, d, dff, _dtype_code(x), int(act), n, _ptr(tokens),
                           _ptr(idx_rows), _ptr(gate_rows), _ptr(y))
    return y


def param_count(d, E, dff) -> int:
    return int(lib().orc_param_count(d, E, dff))


def active_fraction(E, k) -> float:
    return float(lib().orc_active_fraction(E, k))


def num_threads() -> int:
    """Threads the oracle's OpenMP regions use."""
    return int(lib().orc_num_threads())


def set_threads(n: int) -> None:
    """Threads for the oracle's later OpenMP regions."""
    lib().orc_set_threads(int(n))
