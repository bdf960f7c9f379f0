"""Python binding of the MI355X MoE FFN layer library (libcolibri_moe.so).

Argument marshalling only: the functions below carry the C ABI's names
(``include/colibri_moe.h``) and pass plain pointers and sizes through ctypes;
every step of the layer runs in the library's HIP kernels. PyTorch is used for
device memory and streams only (``MoELayer``). There is no CPU fallback: if the
library is missing or fails to load, importing the layer raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcolibri_moe.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_ALIGNMENT, ERR_OUT_OF_MEMORY, ERR_HIP, ERR_TOO_LARGE = range(7)
STATIC_SCRATCH_BYTES = 64 << 20  # COLIBRI_MOE_STATIC_SCRATCH_BYTES
F32, BF16 = 0, 1
FLAG_ASYNC = 1 << 0
FLAG_STAGE_TIMING = 1 << 1
FLAG_FP8_WEIGHTS = 1 << 2
FLAG_FP8_ACTIVATIONS = 1 << 3
STAGES = ("router", "dispatch", "gate_up_gemm", "gate_up_reduce", "down_gemm", "combine")


class Config(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("max_tokens", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]


class Weights(ctypes.Structure):
    _fields_ = [("w_router", ctypes.c_void_p), ("b_router", ctypes.c_void_p), ("w_gate", ctypes.c_void_p),
                ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p)]


class Routing(ctypes.Structure):
    _fields_ = [("logits", ctypes.c_void_p), ("topk_ids", ctypes.c_void_p), ("topk_w", ctypes.c_void_p),
                ("expert_counts", ctypes.c_void_p), ("expert_offsets", ctypes.c_void_p),
                ("perm", ctypes.c_void_p), ("perm_slot", ctypes.c_void_p), ("inv", ctypes.c_void_p)]


EXPORTS = ("colibri_moe_init", "colibri_moe_forward", "colibri_moe_forward_static", "colibri_moe_free",
           "colibri_moe_status_string", "colibri_moe_stage_times", "colibri_moe_stage_name",
           "colibri_moe_quantize_fp8", "colibri_moe_stream_copy")

_lib = None


def lib() -> ctypes.CDLL:
    """Load libcolibri_moe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        P, i32 = ctypes.c_void_p, ctypes.c_int32
        L.colibri_moe_init.restype = ctypes.c_int
        L.colibri_moe_init.argtypes = [ctypes.POINTER(P), ctypes.POINTER(Config), ctypes.POINTER(Weights), P]
        L.colibri_moe_forward.restype = ctypes.c_int
        L.colibri_moe_forward.argtypes = [P, P, i32, P, ctypes.POINTER(Routing)]
        L.colibri_moe_forward_static.restype = ctypes.c_int
        L.colibri_moe_forward_static.argtypes = [P, P, i32, P, ctypes.POINTER(Routing)]
        L.colibri_moe_free.restype = ctypes.c_int
        L.colibri_moe_free.argtypes = [P]
        L.colibri_moe_status_string.restype = ctypes.c_char_p
        L.colibri_moe_status_string.argtypes = [ctypes.c_int]
        L.colibri_moe_stage_times.restype = i32
        L.colibri_moe_stage_times.argtypes = [P, ctypes.POINTER(ctypes.c_float), i32]
        L.colibri_moe_stage_name.restype = ctypes.c_char_p
        L.colibri_moe_stage_name.argtypes = [i32]
        L.colibri_moe_quantize_fp8.restype = ctypes.c_int
        L.colibri_moe_quantize_fp8.argtypes = [P, ctypes.c_int64, ctypes.c_int64, P, P, P]
        L.colibri_moe_stream_copy.restype = ctypes.c_int
        L.colibri_moe_stream_copy.argtypes = [P, P, ctypes.c_int64, P]
        _lib = L
    return _lib


# --- the C ABI, one Python function per entry point -------------------------

def colibri_moe_init(cfg: Config, weights: Weights, hip_stream: int = 0):
    """Returns (status, handle)."""
    h = ctypes.c_void_p()
    st = lib().colibri_moe_init(ctypes.byref(h), ctypes.byref(cfg), ctypes.byref(weights),
                                ctypes.c_void_p(hip_stream))
    return st, h.value


def colibri_moe_forward(handle, x_ptr: int, T: int, y_ptr: int, routing: Routing | None = None) -> int:
    return lib().colibri_moe_forward(ctypes.c_void_p(handle), ctypes.c_void_p(x_ptr), T, ctypes.c_void_p(y_ptr),
                                     None if routing is None else ctypes.byref(routing))


def colibri_moe_forward_static(handle, x_ptr: int, T: int, y_ptr: int, routing: Routing | None = None) -> int:
    return lib().colibri_moe_forward_static(ctypes.c_void_p(handle), ctypes.c_void_p(x_ptr), T,
                                            ctypes.c_void_p(y_ptr),
                                            None if routing is None else ctypes.byref(routing))


def colibri_moe_free(handle) -> int:
    return lib().colibri_moe_free(ctypes.c_void_p(handle))


def colibri_moe_status_string(status: int) -> str:
    return lib().colibri_moe_status_string(status).decode()


def colibri_moe_stage_times(handle) -> list:
    buf = (ctypes.c_float * len(STAGES))()
    n = lib().colibri_moe_stage_times(ctypes.c_void_p(handle), buf, len(STAGES))
    if n < 0:
        raise RuntimeError("stage timing not available (handle created without FLAG_STAGE_TIMING?)")
    return [float(buf[i]) for i in range(n)]


def colibri_moe_stage_name(stage: int):
    s = lib().colibri_moe_stage_name(stage)
    return None if s is None else s.decode()


def colibri_moe_quantize_fp8(w_ptr: int, rows: int, cols: int, codes_ptr: int, scales_ptr: int,
                             hip_stream: int = 0) -> int:
    return lib().colibri_moe_quantize_fp8(ctypes.c_void_p(w_ptr), rows, cols, ctypes.c_void_p(codes_ptr),
                                          ctypes.c_void_p(scales_ptr), ctypes.c_void_p(hip_stream))


def quantize_fp8(w, stream=None):
    """(codes uint8 [rows][cols], scales fp32 [rows]) of a contiguous bf16
    device tensor [rows][cols]: the 8-bit codes a layer built with
    FLAG_FP8_WEIGHTS keeps."""
    import torch

    if w.dtype != torch.bfloat16 or w.dim() != 2 or not w.is_cuda or not w.is_contiguous():
        raise TypeError("w must be a contiguous 2-D bfloat16 device tensor")
    rows, cols = w.shape
    codes = torch.empty(rows, cols, dtype=torch.uint8, device=w.device)
    scales = torch.empty(rows, dtype=torch.float32, device=w.device)
    s = stream if stream is not None else torch.cuda.current_stream()
    st = colibri_moe_quantize_fp8(w.data_ptr(), rows, cols, codes.data_ptr(), scales.data_ptr(), s.cuda_stream)
    if st != OK:
        raise ColibriError("colibri_moe_quantize_fp8", st)
    return codes, scales


def colibri_moe_stream_copy(src_ptr: int, dst_ptr: int, nbytes: int, hip_stream: int = 0) -> int:
    return lib().colibri_moe_stream_copy(ctypes.c_void_p(src_ptr), ctypes.c_void_p(dst_ptr), nbytes,
                                         ctypes.c_void_p(hip_stream))


def stream_copy(src, dst, stream=None):
    """dst <- src with the library's streaming copy kernel (measurement only):
    contiguous device tensors of the same byte size, a multiple of 16."""
    import torch

    if not (src.is_cuda and dst.is_cuda and src.is_contiguous() and dst.is_contiguous()):
        raise TypeError("src and dst must be contiguous device tensors")
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("src and dst differ in size")
    s = stream if stream is not None else torch.cuda.current_stream()
    st = colibri_moe_stream_copy(src.data_ptr(), dst.data_ptr(), n, s.cuda_stream)
    if st != OK:
        raise ColibriError("colibri_moe_stream_copy", st)


class ColibriError(RuntimeError):
    def __init__(self, where: str, status: int):
        super().__init__(f"{where}: {colibri_moe_status_string(status)} ({status})")
        self.status = status


# --- torch convenience wrapper (device memory and streams only) -------------

class MoELayer:
    """One layer handle with weights copied into the library at construction.

    Weight tensors are CUDA (HIP) tensors: w_router [d][E], b_router [E] fp32 or
    None, w_gate/w_up [E][f][d], w_down [E][d][f], all torch.bfloat16 or all
    torch.float32.
    """

    def __init__(self, w_router, b_router, w_gate, w_up, w_down, top_k: int, max_tokens: int,
                 flags: int = 0, stream=None):
        import torch

        self._torch = torch
        dt = w_router.dtype
        if dt not in (torch.bfloat16, torch.float32):
            raise TypeError("weights must be bfloat16 or float32")
        d, E = w_router.shape
        f = w_gate.shape[1]
        self.d, self.E, self.f, self.k, self.max_tokens = d, E, f, int(top_k), int(max_tokens)
        self.dtype = dt
        self.cfg = Config(d, f, E, self.k, self.max_tokens, BF16 if dt == torch.bfloat16 else F32, flags)
        for t in (w_router, w_gate, w_up, w_down):
            if not t.is_cuda or not t.is_contiguous() or t.dtype != dt:
                raise TypeError("weights must be contiguous device tensors of one dtype")
        if b_router is not None and (b_router.dtype != torch.float32 or not b_router.is_cuda):
            raise TypeError("b_router must be a float32 device tensor")
        wts = Weights(w_router.data_ptr(), None if b_router is None else b_router.data_ptr(),
                      w_gate.data_ptr(), w_up.data_ptr(), w_down.data_ptr())
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        st, h = colibri_moe_init(self.cfg, wts, self.stream.cuda_stream)
        if st != OK:
            raise ColibriError("colibri_moe_init", st)
        self.handle = h

    def routing_buffers(self, T: int) -> dict:
        torch = self._torch
        dev = "cuda"
        A = T * self.k
        return dict(logits=torch.empty(T, self.E, dtype=torch.float32, device=dev),
                    topk_ids=torch.empty(T, self.k, dtype=torch.int32, device=dev),
                    topk_w=torch.empty(T, self.k, dtype=torch.float32, device=dev),
                    expert_counts=torch.empty(self.E, dtype=torch.int32, device=dev),
                    expert_offsets=torch.empty(self.E + 1, dtype=torch.int32, device=dev),
                    perm=torch.empty(A, dtype=torch.int32, device=dev),
                    perm_slot=torch.empty(A, dtype=torch.int32, device=dev),
                    inv=torch.empty(A, dtype=torch.int32, device=dev))

    def forward(self, x, y=None, routing: dict | None = None, static_scratch: bool = False):
        """y [T][d] = layer(x). ``routing`` (from routing_buffers) receives the
        routing outputs; missing keys are not written. static_scratch: call
        colibri_moe_forward_static (working memory in the library's fixed
        per-GPU array instead of the handle's)."""
        torch = self._torch
        if x.dtype != self.dtype or x.dim() != 2 or x.shape[1] != self.d or not x.is_contiguous():
            raise TypeError("x must be a contiguous [T][d] tensor of the layer dtype")
        T = x.shape[0]
        if y is None:
            y = torch.empty_like(x)
        r = None
        if routing is not None:
            r = Routing(*[routing[n].data_ptr() if routing.get(n) is not None else None
                          for n, _ in Routing._fields_])
        fn = colibri_moe_forward_static if static_scratch else colibri_moe_forward
        st = fn(self.handle, x.data_ptr(), T, y.data_ptr(), r)
        if st != OK:
            raise ColibriError(fn.__name__, st)
        return y

    def stage_times(self) -> dict:
        return dict(zip(STAGES, colibri_moe_stage_times(self.handle)))

    def close(self):
        if getattr(self, "handle", None):
            st = colibri_moe_free(self.handle)
            self.handle = None
            if st != OK:
                raise ColibriError("colibri_moe_free", st)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
