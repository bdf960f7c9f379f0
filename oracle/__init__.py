"""CPU oracle of the MoE FFN layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package. The GPU library
(``sparse_moe_gemm_amd``) never imports, links or calls it, and the two share
no code. The arithmetic lives in plain C11 (``moe_oracle.c``, built with
``-O2 -ffp-contract=off``); this file only marshals numpy arrays through
ctypes. Definitions and page citations are in ``moe_oracle.h``.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(hand examples, closed forms, brute force, invariants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")

F32, BF16 = 0, 1


def build(verbose: bool = False) -> str:
    src = os.path.join(_HERE, "moe_oracle.c")
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           "-Wall", "-Wextra", src, "-o", LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


class _Layer(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("f", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("w_router", ctypes.c_void_p), ("b_router", ctypes.c_void_p),
                ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        LP = ctypes.POINTER(_Layer)
        sigs = {
            "moe_oracle_widen": [P, ctypes.c_int, i64, P],
            "moe_oracle_router": [LP, P, i32, P],
            "moe_oracle_topk": [P, i32, i32, i32, P, P, P],
            "moe_oracle_route_weights": [P, i32, i32, i32, P, P, P],
            "moe_oracle_dispatch": [P, i32, i32, i32, P, P, P, P, P],
            "moe_oracle_expert_ffn": [LP, i32, P, P, P],
            "moe_oracle_expert_ffn_ex": [LP, i32, P, P, P, i32],
            "moe_oracle_forward": [LP, P, i32, P, P, i32, P, P],
            "moe_oracle_forward_ex": [LP, P, i32, P, P, i32, P, P, i32],
            "moe_oracle_quantize_fp8": [P, ctypes.c_int, i64, i64, P, P],
            "moe_oracle_dequantize_fp8": [P, P, i64, i64, P],
        }
        for name, args in sigs.items():
            fn = getattr(L, name)
            fn.restype = ctypes.c_int
            fn.argtypes = args
        L.moe_oracle_fp8_value.restype = ctypes.c_double
        L.moe_oracle_fp8_value.argtypes = [ctypes.c_uint8]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _dtype_code(arr) -> int:
    if arr.dtype == np.uint16:
        return BF16
    if arr.dtype == np.float32:
        return F32
    raise TypeError(f"tensor dtype {arr.dtype}: expected uint16 (bf16 bits) or float32")


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"{what} failed with {rc}")


ACT_FP8 = 1  # MOE_ORACLE_ACT_FP8


class Layer:
    """Holds contiguous host copies of one layer's weights for the oracle.

    w_router [d][E], b_router [E] fp32 or None, w_gate/w_up [E][f][d],
    w_down [E][d][f]; all uint16 (bf16 bits) or all float32.
    """

    def __init__(self, w_router, b_router, w_gate, w_up, w_down, k: int):
        self.w_router = np.ascontiguousarray(w_router)
        self.b_router = None if b_router is None else np.ascontiguousarray(b_router, dtype=np.float32)
        self.w_gate = np.ascontiguousarray(w_gate)
        self.w_up = np.ascontiguousarray(w_up)
        self.w_down = np.ascontiguousarray(w_down)
        self.dtype = _dtype_code(self.w_router)
        for a in (self.w_gate, self.w_up, self.w_down):
            if _dtype_code(a) != self.dtype:
                raise TypeError("all weight tensors must share one dtype")
        self.d, self.E = self.w_router.shape
        self.f = self.w_gate.shape[1]
        self.k = int(k)
        assert self.w_gate.shape == (self.E, self.f, self.d)
        assert self.w_up.shape == (self.E, self.f, self.d)
        assert self.w_down.shape == (self.E, self.d, self.f)
        self._s = _Layer(self.d, self.f, self.E, self.k, self.dtype, _ptr(self.w_router),
                         _ptr(self.b_router), _ptr(self.w_gate), _ptr(self.w_up), _ptr(self.w_down))

    @classmethod
    def from_inputs(cls, inp: dict, k: int) -> "Layer":
        return cls(inp["w_router"], inp.get("b_router"), inp["w_gate"], inp["w_up"], inp["w_down"], k)

    def _x(self, x):
        x = np.ascontiguousarray(x)
        if _dtype_code(x) != self.dtype or x.ndim != 2 or x.shape[1] != self.d:
            raise TypeError("x must be [T][d] of the layer's dtype")
        return x

    def router(self, x) -> np.ndarray:
        x = self._x(x)
        T = x.shape[0]
        out = np.empty((T, self.E), dtype=np.float32)
        _check(lib().moe_oracle_router(ctypes.byref(self._s), _ptr(x), T, _ptr(out)), "router")
        return out

    def expert_ffn(self, e: int, v, want_h: bool = False, act_fp8: bool = False):
        """FFN of expert e on one row v; with act_fp8 the 8-bit activation
        mode (h returned as the quantized values the down GEMM uses)."""
        v = np.ascontiguousarray(v)
        assert _dtype_code(v) == self.dtype and v.shape == (self.d,)
        out = np.empty(self.d, dtype=np.float64)
        h = np.empty(self.f, dtype=np.float64) if want_h else None
        _check(lib().moe_oracle_expert_ffn_ex(ctypes.byref(self._s), int(e), _ptr(v), _ptr(out), _ptr(h),
                                              ACT_FP8 if act_fp8 else 0), "expert_ffn")
        return (out, h) if want_h else out

    def forward(self, x, tokens=None, forced_ids=None, want_slots: bool = False, act_fp8: bool = False):
        """y [n][d] double for the listed tokens (all tokens if None); act_fp8
        selects the 8-bit activation mode of the expert FFN."""
        x = self._x(x)
        T = x.shape[0]
        tl = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
        n = T if tl is None else tl.shape[0]
        fi = None if forced_ids is None else np.ascontiguousarray(forced_ids, dtype=np.int32)
        if fi is not None:
            assert fi.shape == (T, self.k)
        y = np.empty((n, self.d), dtype=np.float64)
        ys = np.empty((n, self.k, self.d), dtype=np.float64) if want_slots else None
        _check(lib().moe_oracle_forward_ex(ctypes.byref(self._s), _ptr(x), T, _ptr(fi), _ptr(tl), n,
                                           _ptr(y), _ptr(ys), ACT_FP8 if act_fp8 else 0), "forward")
        return (y, ys) if want_slots else y


def widen(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    out = np.empty(a.shape, dtype=np.float32)
    _check(lib().moe_oracle_widen(_ptr(a), _dtype_code(a), a.size, _ptr(out)), "widen")
    return out


def topk(logits, k: int):
    """(ids [T][k] int32, w [T][k] fp32, w [T][k] double) from fp32 logits [T][E]."""
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = lg.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    wd = np.empty((T, k), dtype=np.float64)
    _check(lib().moe_oracle_topk(_ptr(lg), T, E, k, _ptr(ids), _ptr(w), _ptr(wd)), "topk")
    return ids, w, wd


def route_weights(logits, ids):
    """(w [T][k] fp32, w [T][k] double): the softmax over the logits of the given
    experts ids [T][k], renormalised, exponent shifted by slot 0's logit."""
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, E = lg.shape
    k = ids.shape[1]
    assert ids.shape[0] == T
    w = np.empty((T, k), dtype=np.float32)
    wd = np.empty((T, k), dtype=np.float64)
    _check(lib().moe_oracle_route_weights(_ptr(lg), T, E, k, _ptr(ids), _ptr(w), _ptr(wd)), "route_weights")
    return w, wd


def dispatch(ids, E: int):
    """Stable counting sort of assignments by expert.

    Returns dict(counts [E], offsets [E+1], perm [A], perm_slot [A], inv [A]).
    """
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    A = T * k
    out = dict(counts=np.empty(E, np.int32), offsets=np.empty(E + 1, np.int32),
               perm=np.empty(A, np.int32), perm_slot=np.empty(A, np.int32), inv=np.empty(A, np.int32))
    _check(lib().moe_oracle_dispatch(_ptr(ids), T, k, E, _ptr(out["counts"]), _ptr(out["offsets"]),
                                     _ptr(out["perm"]), _ptr(out["perm_slot"]), _ptr(out["inv"])),
           "dispatch")
    return out


def near_tie_tokens(logits, k: int, rel: float = 1e-5) -> np.ndarray:
    """Boolean [T]: tokens whose sorted fp32 logits have an adjacent pair among
    the first k+1 closer than ``rel`` relative (GPU and oracle may then order
    or select them differently, so ids are not compared bit for bit)."""
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    s = -np.sort(-lg, axis=1)[:, : min(k + 1, E)].astype(np.float64)
    if s.shape[1] < 2:
        return np.zeros(T, dtype=bool)
    a, b = s[:, :-1], s[:, 1:]
    close = (a - b) < rel * np.maximum(np.abs(a), np.abs(b))
    return close.any(axis=1)


def boundary_tie_tokens(logits, k: int, rel: float = 1e-5) -> np.ndarray:
    """Boolean [T]: tokens whose k-th and (k+1)-th largest logits are near-tied
    (then even the selected set may differ)."""
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    if k >= E:
        return np.zeros(T, dtype=bool)
    s = -np.sort(-lg, axis=1).astype(np.float64)
    a, b = s[:, k - 1], s[:, k]
    return (a - b) < rel * np.maximum(np.abs(a), np.abs(b))


def quantize_fp8(w) -> tuple:
    """8-bit expert weights (reading in moe_oracle.h): w [rows][cols] (bf16 bits
    as uint16, or float32) -> (codes uint8 [rows][cols], scales float32 [rows])."""
    w = np.ascontiguousarray(w)
    rows, cols = w.shape[0], int(np.prod(w.shape[1:]))
    codes = np.empty((rows, cols), dtype=np.uint8)
    scales = np.empty(rows, dtype=np.float32)
    _check(lib().moe_oracle_quantize_fp8(_ptr(w), _dtype_code(w), rows, cols, _ptr(codes), _ptr(scales)),
           "quantize_fp8")
    return codes.reshape(w.shape), scales


def dequantize_fp8(codes, scales) -> np.ndarray:
    """codes [rows][...] uint8, scales [rows] -> bf16 bit patterns (uint16), exact."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    rows, cols = codes.shape[0], int(np.prod(codes.shape[1:]))
    out = np.empty(codes.shape, dtype=np.uint16)
    _check(lib().moe_oracle_dequantize_fp8(_ptr(codes), _ptr(scales), rows, cols, _ptr(out)), "dequantize_fp8")
    return out


def fp8_value(code: int) -> float:
    return float(lib().moe_oracle_fp8_value(code))


def quantized_expert_weights(inp: dict) -> dict:
    """The layer's inputs with every expert weight matrix replaced by its 8-bit
    quantized-and-dequantized value (per expert, per output row); router and x
    unchanged. Running the ordinary layer on these is the 8-bit layer."""
    out = dict(inp)
    for name in ("w_gate", "w_up", "w_down"):
        w = inp[name]
        E, rows, cols = w.shape
        codes, scales = quantize_fp8(w.reshape(E * rows, cols))
        out[name] = dequantize_fp8(codes, scales).reshape(E, rows, cols)
    return out
