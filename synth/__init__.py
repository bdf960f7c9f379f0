"""Seeded synthetic inputs for the MoE FFN layer (shared by the oracle's tests,
the GPU parity tests and the benchmark).

This module draws numbers and nothing else: it holds none of the layer's
arithmetic. Values come from a counter-based SplitMix64 + Box-Muller generator
written in C (``synth.c``), so the same bytes feed the CPU oracle and the GPU
library.

Workloads (the layer shapes the Colibri pages keep returning to, at the sizes
this project measures):

============== ====== ====== ===== === ====== ===== ==========================
name           T      d      E     k   d_ff   dtype router bias
============== ====== ====== ===== === ====== ===== ==========================
tiny-f32       64     128    8     2   256    f32   0
mixtral        4096   4096   8     2   14336  bf16  0
fine-grained   8192   2048   128   4   768    bf16  0
decode         32     4096   8     2   14336  bf16  0
skewed         16384  4096   64    2   1408   bf16  +4.0 on experts 0 and 3
skewed-masked  16384  4096   64    2   1408   bf16  as skewed, -1e4 on 44..63
============== ====== ====== ===== === ====== ===== ==========================

Distributions: x ~ N(0, 1); W_r, W_gate, W_up ~ N(0, std = d^-1/2);
W_down ~ N(0, std = d_ff^-1/2); bf16 tensors are the fp32 draw rounded
to nearest even. The router bias is fp32 and never drawn.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")

# Stream ids of the tensors (the second key of the generator).
TID_X, TID_WR, TID_WG, TID_WU, TID_WD = 0, 1, 2, 3, 4


def build(verbose: bool = False) -> str:
    """Compile ``synth.c`` into ``libsynth.so`` (gcc, OpenMP)."""
    import subprocess

    src = os.path.join(_HERE, "synth.c")
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-ffp-contract=off", src, "-o", LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        u64, sz = ctypes.c_uint64, ctypes.c_size_t
        L.synth_raw.restype = u64
        L.synth_raw.argtypes = [u64, u64, u64, ctypes.c_int]
        L.synth_mix64.restype = u64
        L.synth_mix64.argtypes = [u64]
        L.synth_f32_to_bf16.restype = ctypes.c_uint16
        L.synth_f32_to_bf16.argtypes = [ctypes.c_float]
        for name in ("synth_normal_f32", "synth_normal_bf16"):
            fn = getattr(L, name)
            fn.restype = None
            fn.argtypes = [u64, u64, u64, sz, ctypes.c_double, ctypes.c_double, ctypes.c_void_p]
        _lib = L
    return _lib


def normal(seed: int, tensor_id: int, n: int, std: float = 1.0, mean: float = 0.0,
           dtype: str = "f32", offset: int = 0) -> np.ndarray:
    """n draws of N(mean, std^2) from stream (seed, tensor_id).

    dtype "f32" returns float32; "bf16" returns the bf16 bit patterns as uint16.
    """
    L = lib()
    if dtype == "f32":
        out = np.empty(n, dtype=np.float32)
        L.synth_normal_f32(seed, tensor_id, offset, n, mean, std, out.ctypes.data)
    elif dtype == "bf16":
        out = np.empty(n, dtype=np.uint16)
        L.synth_normal_bf16(seed, tensor_id, offset, n, mean, std, out.ctypes.data)
    else:
        raise ValueError(dtype)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    d: int
    E: int
    k: int
    f: int
    dtype: str  # "f32" or "bf16"
    bias: dict = field(default_factory=dict)  # expert -> fp32 bias value
    seed: int = 0

    @property
    def A(self) -> int:
        return self.T * self.k

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)

    def flops(self) -> float:
        """Algorithmic flops: router GEMM + 3 expert GEMMs per assignment."""
        return 2.0 * self.T * self.d * self.E + 6.0 * self.d * self.f * self.T * self.k

    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


_SKEW = {0: 4.0, 3: 4.0}
_SKEW_MASKED = {**_SKEW, **{e: -1.0e4 for e in range(44, 64)}}

CONFIGS = {
    "tiny-f32": LayerConfig("tiny-f32", 64, 128, 8, 2, 256, "f32"),
    "mixtral": LayerConfig("mixtral", 4096, 4096, 8, 2, 14336, "bf16"),
    "fine-grained": LayerConfig("fine-grained", 8192, 2048, 128, 4, 768, "bf16"),
    "decode": LayerConfig("decode", 32, 4096, 8, 2, 14336, "bf16"),
    "skewed": LayerConfig("skewed", 16384, 4096, 64, 2, 1408, "bf16", _SKEW),
    "skewed-masked": LayerConfig("skewed-masked", 16384, 4096, 64, 2, 1408, "bf16", _SKEW_MASKED),
    # one expert takes every token: the expert GEMMs are plain dense GEMMs
    # (gate/up 8192 x 28672 x 4096), a reference point for the grouped kernel
    "dense": LayerConfig("dense", 8192, 4096, 1, 1, 14336, "bf16"),
    # square GEMM for the attainable-MFMA record: gate/up is 8192 x 8192 x 8192
    "square": LayerConfig("square", 8192, 8192, 1, 1, 4096, "bf16"),
}


def router_bias(cfg: LayerConfig) -> np.ndarray:
    b = np.zeros(cfg.E, dtype=np.float32)
    for e, v in cfg.bias.items():
        if e < cfg.E:
            b[e] = v
    return b


def make_inputs(cfg: LayerConfig, weights: bool = True, tokens: bool = True) -> dict:
    """All layer inputs of ``cfg`` as host arrays (uint16 bf16 bits or float32).

    Shapes: x [T][d]; w_router [d][E]; b_router [E] fp32;
    w_gate, w_up [E][d_ff][d]; w_down [E][d][d_ff].
    """
    s, dt = cfg.seed, cfg.dtype
    out = {}
    if tokens:
        out["x"] = normal(s, TID_X, cfg.T * cfg.d, 1.0, dtype=dt).reshape(cfg.T, cfg.d)
    if weights:
        sd_in = cfg.d ** -0.5
        sd_ff = cfg.f ** -0.5
        out["w_router"] = normal(s, TID_WR, cfg.d * cfg.E, sd_in, dtype=dt).reshape(cfg.d, cfg.E)
        out["b_router"] = router_bias(cfg)
        out["w_gate"] = normal(s, TID_WG, cfg.E * cfg.f * cfg.d, sd_in, dtype=dt).reshape(cfg.E, cfg.f, cfg.d)
        out["w_up"] = normal(s, TID_WU, cfg.E * cfg.f * cfg.d, sd_in, dtype=dt).reshape(cfg.E, cfg.f, cfg.d)
        out["w_down"] = normal(s, TID_WD, cfg.E * cfg.d * cfg.f, sd_ff, dtype=dt).reshape(cfg.E, cfg.d, cfg.f)
    return out


def make_tokens(cfg: LayerConfig, T: int, stream_offset_tokens: int = 0) -> np.ndarray:
    """T token rows drawn from the x stream starting at token ``stream_offset_tokens``."""
    return normal(cfg.seed, TID_X, T * cfg.d, 1.0, dtype=cfg.dtype,
                  offset=stream_offset_tokens * cfg.d).reshape(T, cfg.d)
