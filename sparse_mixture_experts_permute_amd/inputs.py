"""Seeded synthetic inputs for the MoE layer (shared by the tests, the benchmark
and the smoke check; holds none of the layer's arithmetic).

Every tensor is drawn in fp32 from numpy's PCG64 normal generator, scaled, and
rounded to bf16 with round-to-nearest-even.  The bf16 bit patterns feed the
bf16 path; the same values widened to fp32 feed the fp32 path.  So both paths,
and the CPU oracle, see identical input values.

Streams are independent and addressed by (seed, tensor, block):
  x    rows in blocks of 1024 tokens   (a shorter T is a prefix of a longer one)
  Wg   one stream                      N(0,1) * 0.02
  W1   one stream per expert           N(0,1) / sqrt(d)     layout [E][d_ff][d]
  W3   one stream per expert           N(0,1) / sqrt(d)     layout [E][d_ff][d]
  W2   one stream per expert           N(0,1) / sqrt(d_ff)  layout [E][d][d_ff]
  Ws1, Ws3, Ws2 (shared expert)        same scales, one stream each
Weights are held as Linear weights [out][in].  The skewed router adds a
per-expert logit bias (+1.5 on expert 0) instead of changing Wg.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

X_BLOCK = 1024
_TID = dict(x=0, Wg=1, W1=2, W3=3, W2=4, Ws1=5, Ws3=6, Ws2=7)


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    d: int
    E: int
    d_ff: int
    k: int
    dtype: str = "bf16"          # "bf16" or "f32"
    d_ff_shared: int = 0         # 0: no shared expert
    skew: float = 0.0            # logit bias added to expert 0 (0: balanced)
    seed: int = 42
    tags: tuple = field(default=())

    @property
    def P(self) -> int:
        return self.T * self.k

    def with_(self, **kw) -> "LayerConfig":
        d = dict(self.__dict__)
        d.update(kw)
        return LayerConfig(**d)


def _granularity():
    out = []
    for dt in ("f32", "bf16"):
        for (E, dff, k) in [(1, 32768, 1), (8, 4096, 1), (8, 4096, 2), (32, 1024, 1),
                            (32, 1024, 2), (64, 512, 4), (128, 256, 8)]:
            out.append(LayerConfig(f"granularity_E{E}_k{k}_{dt}", 512, 512, E, dff, k, dt,
                                   tags=("granularity",)))
    return out


# Workloads: shapes and distributions of the layers the pages measure.
CONFIGS = {c.name: c for c in (
    [LayerConfig("small_fp32", 512, 512, 8, 4096, 2, "f32", tags=("small",))]
    + _granularity()
    + [LayerConfig(f"mixtral_prefill_T{T}", T, 4096, 8, 14336, 2, "bf16", tags=("prefill",))
       for T in (2048, 8192)]
    + [LayerConfig(f"mixtral_prefill_T{T}_skew", T, 4096, 8, 14336, 2, "bf16", skew=1.5,
                   tags=("prefill", "skew")) for T in (2048, 8192)]
    + [LayerConfig(f"mixtral_decode_T{T}", T, 4096, 8, 14336, 2, "bf16", tags=("decode",))
       for T in (1, 8, 32, 128)]
    + [LayerConfig(f"fine_shared_T{T}", T, 7168, 256, 2048, 8, "bf16", d_ff_shared=2048,
                   tags=("shared",)) for T in (512, 8192)]
)}


def bf16_round_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 values."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def _rng(seed: int, tensor: str, block: int) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(_TID[tensor], block))
    return np.random.Generator(np.random.PCG64(ss))


def _fill(out_bits: np.ndarray, seed: int, tensor: str, block: int, scale: float) -> None:
    g = _rng(seed, tensor, block)
    tmp = g.standard_normal(out_bits.shape, dtype=np.float32)
    if scale != 1.0:
        tmp *= np.float32(scale)
    out_bits[...] = bf16_round_bits(tmp)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def make_inputs(cfg: LayerConfig, T: int | None = None, with_weights: bool = True) -> dict:
    """All inputs of one layer as numpy arrays.

    bf16 configs return uint16 bit patterns; f32 configs return float32 holding
    the same bf16-rounded values.  ``T`` overrides the token count (x is a
    prefix of the longer stream).  Keys: x, Wg, bias (or None), W1, W3, W2 and,
    with a shared expert, Ws1, Ws3, Ws2.
    """
    T = cfg.T if T is None else T
    d, E, dff, dffs, seed = cfg.d, cfg.E, cfg.d_ff, cfg.d_ff_shared, cfg.seed
    jobs = []
    arrs = {}
    nxb = (T + X_BLOCK - 1) // X_BLOCK
    xb = np.empty((nxb * X_BLOCK, d), np.uint16)
    for b in range(nxb):
        jobs.append((xb[b * X_BLOCK:(b + 1) * X_BLOCK], "x", b, 1.0))
    arrs["Wg"] = np.empty((E, d), np.uint16)
    jobs.append((arrs["Wg"], "Wg", 0, 0.02))
    if with_weights:
        arrs["W1"] = np.empty((E, dff, d), np.uint16)
        arrs["W3"] = np.empty((E, dff, d), np.uint16)
        arrs["W2"] = np.empty((E, d, dff), np.uint16)
        for e in range(E):
            jobs.append((arrs["W1"][e], "W1", e, 1.0 / math.sqrt(d)))
            jobs.append((arrs["W3"][e], "W3", e, 1.0 / math.sqrt(d)))
            jobs.append((arrs["W2"][e], "W2", e, 1.0 / math.sqrt(dff)))
        if dffs:
            arrs["Ws1"] = np.empty((dffs, d), np.uint16)
            arrs["Ws3"] = np.empty((dffs, d), np.uint16)
            arrs["Ws2"] = np.empty((d, dffs), np.uint16)
            jobs.append((arrs["Ws1"], "Ws1", 0, 1.0 / math.sqrt(d)))
            jobs.append((arrs["Ws3"], "Ws3", 0, 1.0 / math.sqrt(d)))
            jobs.append((arrs["Ws2"], "Ws2", 0, 1.0 / math.sqrt(dffs)))
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(lambda j: _fill(j[0], seed, j[1], j[2], j[3]), jobs))
    arrs["x"] = xb[:T]
    out = {}
    for key, a in arrs.items():
        out[key] = a if cfg.dtype == "bf16" else bf16_bits_to_f32(a)
    out["x"] = np.ascontiguousarray(out["x"])
    bias = None
    if cfg.skew:
        bias = np.zeros(E, np.float32)
        bias[0] = np.float32(cfg.skew)
    out["bias"] = bias
    return out


def shared_tuple(inp: dict):
    return (inp["Ws1"], inp["Ws3"], inp["Ws2"]) if "Ws1" in inp else None
