"""Python binding of libsage.so: argument marshalling only.

Every step of the attention path runs in the library's HIP kernels; this
module turns PyTorch device tensors and the current stream into the C ABI's
pointers (see include/sage.h) and allocates the buffers a caller needs.
There is no fallback: if the library or a GPU is missing, the calls raise.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Dict, Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsage.so")

SAGE_OK, SAGE_EINVAL, SAGE_EUNSUPPORTED, SAGE_EHIP, SAGE_ESCRATCH = 0, -1, -2, -3, -4
NOALLOC_SCRATCH_BYTES = 8 << 20   # SAGE_NOALLOC_SCRATCH_BYTES of include/sage.h
SAGE_FP16, SAGE_BF16 = 0, 1


class SageError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class c_shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32), ("D", ctypes.c_int32),
                ("bq", ctypes.c_int32), ("bkv", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("k_smooth", ctypes.c_int32), ("q_smooth", ctypes.c_int32),
                ("sm_scale", ctypes.c_float), ("dp_int8", ctypes.c_int32), ("p_static", ctypes.c_int32),
                ("qk_norm", ctypes.c_int32), ("fp8", ctypes.c_int32)]


_P = ctypes.c_void_p
QT_FIELDS = ("q", "sq", "k", "sk", "vt", "sv", "vr", "mu_k", "mu_q", "qk_bias", "rq", "rk")
DO_FIELDS = ("delta", "dot", "sdo", "dor")


class c_qtensors(ctypes.Structure):
    _fields_ = [(f, _P) for f in QT_FIELDS]


class c_dotensors(ctypes.Structure):
    _fields_ = [(f, _P) for f in DO_FIELDS]


# C symbol -> (restype, argtypes)
SIGNATURES = {
    "sage_quantize_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(c_shape)]),
    "sage_quantize": (ctypes.c_int, [ctypes.POINTER(c_shape), _P, _P, _P, ctypes.POINTER(c_qtensors), _P, _P]),
    "sage_quantize_noalloc": (ctypes.c_int, [ctypes.POINTER(c_shape), _P, _P, _P, ctypes.POINTER(c_qtensors), _P]),
    "sage_fwd": (ctypes.c_int, [ctypes.POINTER(c_shape), ctypes.POINTER(c_qtensors), _P, _P, _P]),
    "sage_bwd_pre": (ctypes.c_int, [ctypes.POINTER(c_shape), _P, _P, ctypes.POINTER(c_dotensors), _P]),
    "sage_bwd_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(c_shape)]),
    "sage_bwd": (ctypes.c_int, [ctypes.POINTER(c_shape), ctypes.POINTER(c_qtensors), ctypes.POINTER(c_dotensors),
                                _P, _P, _P, _P, _P, _P, _P, _P]),
    "sage_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "sage_last_hip_error": (ctypes.c_int, []),
    "sage_version": (ctypes.c_char_p, []),
    "sage_qk_norm_bwd": (ctypes.c_int, [ctypes.POINTER(c_shape), _P, _P, ctypes.POINTER(c_qtensors), _P, _P, _P]),
    "sage_cast_grads": (ctypes.c_int, [ctypes.POINTER(c_shape), _P, _P, _P, _P, _P, _P, _P]),
    # include/sage_probe.h (measurement aid)
    "sage_probe_mfma_i8": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _P, _P]),
    "sage_probe_mfma_bf16": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _P, _P]),
    "sage_probe_fp8_products": (ctypes.c_int, [_P, _P, _P, _P, _P]),
}

_lib = None


def load(path: str = LIB_PATH):
    """Load libsage.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing; build it with "
                               "`python -m bit_trainable_attention_block_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib
    return _lib


def _check(status: int, what: str):
    if status != SAGE_OK:
        lib = load()
        msg = lib.sage_status_str(status).decode()
        if status == SAGE_EHIP:
            msg += f" (hip error {lib.sage_last_hip_error()})"
        raise SageError(status, f"{what}: {msg}")


@dataclasses.dataclass(frozen=True)
class Shape:
    B: int
    H: int
    N: int
    D: int
    bq: int = 128
    bkv: int = 64
    dtype: int = SAGE_BF16
    causal: bool = False
    k_smooth: bool = True
    q_smooth: bool = False
    sm_scale: float = 0.0
    dp_int8: bool = False   # ablation: dP from INT8 codes (see include/sage.h)
    p_static: bool = False  # ablation: static forward P scale 1/127 (see include/sage.h)
    qk_norm: bool = False   # QK-norm fused into sage_quantize (see include/sage.h)
    fp8: bool = False       # variant: E4M3 codes in place of INT8 (see include/sage.h)

    @staticmethod
    def of(cfg) -> "Shape":
        return Shape(B=cfg.B, H=cfg.H, N=cfg.N, D=cfg.D, bq=cfg.bq, bkv=cfg.bkv, dtype=cfg.dtype,
                     causal=bool(cfg.causal), k_smooth=bool(cfg.k_smooth), q_smooth=bool(cfg.q_smooth),
                     dp_int8=bool(getattr(cfg, "dp_int8", False)), p_static=bool(getattr(cfg, "p_static", False)),
                     qk_norm=bool(getattr(cfg, "qk_norm_fused", False)), fp8=bool(getattr(cfg, "fp8", False)))

    def c(self) -> c_shape:
        return c_shape(self.B, self.H, self.N, self.D, self.bq, self.bkv, self.dtype, int(self.causal),
                       int(self.k_smooth), int(self.q_smooth), float(self.sm_scale), int(self.dp_int8),
                       int(self.p_static), int(self.qk_norm), int(self.fp8))

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == SAGE_BF16 else torch.float16

    @property
    def Tm(self):
        return self.N // self.bq

    @property
    def Tn(self):
        return self.N // self.bkv


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def alloc_qtensors(sh: Shape, device="cuda") -> Dict[str, torch.Tensor]:
    """Buffers for sage_quantize's outputs (layouts in include/sage.h)."""
    B, H, N, D = sh.B, sh.H, sh.N, sh.D
    i8 = dict(dtype=torch.int8, device=device)
    f32 = dict(dtype=torch.float32, device=device)
    t = {
        "q": torch.empty((B, H, N * D), **i8),
        "sq": torch.empty((B, H, sh.Tm), **f32),
        "k": torch.empty((B, H, N * D), **i8),
        "sk": torch.empty((B, H, sh.Tn), **f32),
        "vt": torch.empty((B, H, N * D), **i8), "sv": torch.empty((B, H, sh.Tn), **f32),
        "vr": torch.empty((B, H, N * D), **i8) if sh.dp_int8 else None,
        "mu_k": torch.zeros((B, H, D), **f32),
        "mu_q": torch.empty((B, H, sh.Tm, D), **f32) if sh.q_smooth else None,
        "qk_bias": torch.empty((B, H, sh.Tm, N), **f32) if sh.q_smooth else None,
        "rq": torch.empty((B, H, N), **f32) if sh.qk_norm else None,
        "rk": torch.empty((B, H, N), **f32) if sh.qk_norm else None,
        "ws": torch.empty((max(1, load().sage_quantize_workspace_bytes(ctypes.byref(sh.c())) // 8),),
                          dtype=torch.float64, device=device),
    }
    return t


def alloc_dotensors(sh: Shape, device="cuda") -> Dict[str, torch.Tensor]:
    B, H, N, D = sh.B, sh.H, sh.N, sh.D
    return {
        "delta": torch.empty((B, H, N), dtype=torch.float32, device=device),
        "dot": torch.empty((B, H, N * D), dtype=torch.int8, device=device),
        "sdo": torch.empty((B, H, sh.Tm), dtype=torch.float32, device=device),
        "dor": torch.empty((B, H, N * D), dtype=torch.int8, device=device) if sh.dp_int8 else None,
    }


def _qstruct(t: Dict[str, torch.Tensor]) -> c_qtensors:
    return c_qtensors(*[_ptr(t.get(f)) for f in QT_FIELDS])


def _dostruct(t: Dict[str, torch.Tensor]) -> c_dotensors:
    return c_dotensors(*[_ptr(t.get(f)) for f in DO_FIELDS])


def quantize(sh: Shape, Q, K, V, out: Optional[Dict[str, torch.Tensor]] = None, stream=None):
    lib = load()
    out = alloc_qtensors(sh, Q.device) if out is None else out
    cs = sh.c()
    _check(lib.sage_quantize(ctypes.byref(cs), _ptr(Q), _ptr(K), _ptr(V), ctypes.byref(_qstruct(out)),
                             _ptr(out["ws"]), _stream(stream)), "sage_quantize")
    return out


def quantize_noalloc(sh: Shape, Q, K, V, out: Dict[str, torch.Tensor], stream=None):
    """sage_quantize_noalloc: sage_quantize with the library's own fixed device
    scratch in place of the workspace (out["ws"] is not used)."""
    cs = sh.c()
    _check(load().sage_quantize_noalloc(ctypes.byref(cs), _ptr(Q), _ptr(K), _ptr(V), ctypes.byref(_qstruct(out)),
                                        _stream(stream)), "sage_quantize_noalloc")
    return out


def fwd(sh: Shape, qt: Dict[str, torch.Tensor], O=None, L=None, stream=None):
    lib = load()
    dev = qt["q"].device
    O = torch.empty((sh.B, sh.H, sh.N, sh.D), dtype=sh.torch_dtype, device=dev) if O is None else O
    L = torch.empty((sh.B, sh.H, sh.N), dtype=torch.float32, device=dev) if L is None else L
    cs = sh.c()
    _check(lib.sage_fwd(ctypes.byref(cs), ctypes.byref(_qstruct(qt)), _ptr(O), _ptr(L), _stream(stream)),
           "sage_fwd")
    return O, L


def bwd_pre(sh: Shape, O, dO, out=None, stream=None):
    lib = load()
    out = alloc_dotensors(sh, O.device) if out is None else out
    cs = sh.c()
    _check(lib.sage_bwd_pre(ctypes.byref(cs), _ptr(O), _ptr(dO), ctypes.byref(_dostruct(out)), _stream(stream)),
           "sage_bwd_pre")
    return out


def bwd_workspace(sh: Shape, device="cuda") -> torch.Tensor:
    n = load().sage_bwd_workspace_bytes(ctypes.byref(sh.c()))
    return torch.empty((max(n, 16),), dtype=torch.uint8, device=device)


def bwd(sh: Shape, qt, dot, V, dO, L, dQ=None, dK=None, dV=None, ws=None, stream=None):
    """sage_bwd: V and dO are the 16-bit tensors given to quantize and bwd_pre."""
    lib = load()
    dev = L.device
    ws = bwd_workspace(sh, dev) if ws is None else ws
    shape = (sh.B, sh.H, sh.N, sh.D)
    dQ = torch.empty(shape, dtype=torch.float32, device=dev) if dQ is None else dQ
    dK = torch.empty(shape, dtype=torch.float32, device=dev) if dK is None else dK
    dV = torch.empty(shape, dtype=torch.float32, device=dev) if dV is None else dV
    cs = sh.c()
    _check(lib.sage_bwd(ctypes.byref(cs), ctypes.byref(_qstruct(qt)), ctypes.byref(_dostruct(dot)), _ptr(V),
                        _ptr(dO), _ptr(L), _ptr(ws), _ptr(dQ), _ptr(dK), _ptr(dV), _stream(stream)), "sage_bwd")
    return dQ, dK, dV


def qk_norm_bwd(sh: Shape, Q, K, qt, dQ, dK, stream=None):
    """In place: dQ, dK w.r.t. the QK-normed rows -> w.r.t. the inputs Q, K."""
    cs = sh.c()
    _check(load().sage_qk_norm_bwd(ctypes.byref(cs), _ptr(Q), _ptr(K), ctypes.byref(_qstruct(qt)), _ptr(dQ),
                                   _ptr(dK), _stream(stream)), "sage_qk_norm_bwd")
    return dQ, dK


def cast_grads(sh: Shape, dQ=None, dK=None, dV=None, stream=None):
    """The float32 gradients (any subset) rounded to the shape's 16-bit I/O
    dtype by the library (nearest, ties to even); returns the 16-bit tensors
    (None where the input was None)."""
    out = [None if t is None else torch.empty(t.shape, dtype=sh.torch_dtype, device=t.device)
           for t in (dQ, dK, dV)]
    cs = sh.c()
    _check(load().sage_cast_grads(ctypes.byref(cs), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(out[0]), _ptr(out[1]),
                                  _ptr(out[2]), _stream(stream)), "sage_cast_grads")
    return tuple(out)


def probe_mfma_i8(blocks: int, iters: int, clk: torch.Tensor, stream=None):
    """Measurement aid (include/sage_probe.h): `blocks` workgroups of 8 waves,
    each wave issuing iters x 8 INT8 16x16x64 products; clk (3 int64 on the
    device) receives the shader cycles and 100 MHz ticks of workgroup 0."""
    _check(load().sage_probe_mfma_i8(blocks, iters, _ptr(clk), _stream(stream)), "sage_probe_mfma_i8")


def probe_mfma_bf16(blocks: int, iters: int, clk: torch.Tensor, stream=None):
    """Measurement aid (include/sage_probe.h): as probe_mfma_i8, on the BF16
    16x16x32 product."""
    _check(load().sage_probe_mfma_bf16(blocks, iters, _ptr(clk), _stream(stream)), "sage_probe_mfma_bf16")


def probe_fp8_products(a, b, c32, c128, stream=None):
    """Measurement aid (include/sage_probe.h): one wave of the two E4M3 matrix
    products on a, b (64 x 32 bytes each, device) into c32, c128 (64 x 4
    floats each, device)."""
    _check(load().sage_probe_fp8_products(_ptr(a), _ptr(b), _ptr(c32), _ptr(c128), _stream(stream)),
           "sage_probe_fp8_products")


def run(sh: Shape, Q, K, V, dO, stream=None):
    """quantize -> fwd -> bwd_pre -> bwd; returns every intermediate."""
    qt = quantize(sh, Q, K, V, stream=stream)
    O, L = fwd(sh, qt, stream=stream)
    dot = bwd_pre(sh, O, dO, stream=stream)
    dQ, dK, dV = bwd(sh, qt, dot, V, dO, L, stream=stream)
    out = {"qt": qt, "O": O, "L": L, "dot": dot, "dQ": dQ, "dK": dK, "dV": dV}
    if sh.qk_norm:
        # dQ, dK above are w.r.t. the normalised rows; these w.r.t. Q and K
        out["dQ_in"], out["dK_in"] = qk_norm_bwd(sh, Q, K, qt, dQ.clone(), dK.clone(), stream=stream)
    return out


# ----------------------------------------------------------------- layouts
# Host-side inverses of the code layouts in include/sage.h, for tests.

def _rows_cols(N, D):
    import numpy as np
    return np.arange(N)[:, None], np.arange(D)[None, :]


def layout_offsets(kind: str, N: int, D: int):
    """[N, D] array of byte offsets of element (row, col)."""
    import numpy as np
    r, c = _rows_cols(N, D)
    r = np.broadcast_to(r, (N, D)); c = np.broadcast_to(c, (N, D))
    if kind == "R32":
        return (r // 32) * (32 * D) + (((c // 16) * 32 + r % 32) * 16) + c % 16
    if kind == "C64P":
        rr = r % 64
        g = (rr // 4) % 4
        e = (rr // 16) * 4 + rr % 4
        return (r // 64) * (64 * D) + (g * D + c) * 16 + e
    raise ValueError(kind)


def unpack_codes(flat, kind: str, N: int, D: int):
    """flat [..., N*D] (numpy) in layout ``kind`` -> [..., N, D] row-major."""
    off = layout_offsets(kind, N, D)
    return flat[..., off]
