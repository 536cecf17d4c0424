"""Python binding of libpi, the gfx950 neuron-aware sparse FFN.

Argument marshalling only: every step runs in the HIP kernels of
``libpi.so`` (declared in ``include/pi.h``).  Tensors are torch device
tensors; torch supplies memory and streams and nothing else.  The binding
raises :class:`PiError` if the library is missing or a call fails; there is
no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

PI_F32, PI_F16, PI_I4G128 = 0, 1, 2
PI_RELU, PI_GATED_RELU = 0, 1
PI_OK, PI_EINVAL, PI_EWORKSPACE, PI_EUNSUPPORTED, PI_EHIP = 0, 1, 2, 3, 4
PI_OP_PREDICT, PI_OP_COMPACT, PI_OP_SPARSE_FFN, PI_OP_MERGE, PI_OP_FFN_LAYER, PI_OP_PREDICT_OUTPUT = 0, 1, 2, 3, 4, 5
PI_OP_FFN_LAYER_NORMED = 6
PI_READ_PROBE_DEPTH, PI_READ_PROBE_BLOCKS_PER_CU = 16, 8
PI_STAGE_HIDDEN, PI_STAGE_OUTPUT, PI_STAGE_FC1, PI_STAGE_FC2, PI_STAGE_SUM, PI_STAGE_ALL = 1, 2, 4, 8, 16, 31
PI_MAX_BATCH = 32
PI_MAX_NEURONS = 65536
PI_ABI_VERSION = 3

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpi.so")

EXPORTS = ("pi_predict", "pi_predict_output", "pi_compact", "pi_sparse_ffn", "pi_merge", "pi_table_bytes",
           "pi_table_prepare", "pi_ffn_layer", "pi_ffn_layer_stages", "pi_workspace_bytes", "pi_status_string",
           "pi_last_hip_error", "pi_abi_version", "pi_read_probe", "pi_ffn_layer_ahead",
           "pi_layer_norm", "pi_ffn_layer_static", "pi_ffn_layer_normed", "pi_attn_decode",
           "pi_attn_workspace_bytes")
PI_STATIC_WORKSPACE_BYTES = 16 << 20


class PiError(RuntimeError):
    pass


class _Mat(C.Structure):
    _fields_ = [("data", C.c_void_p), ("scales", C.c_void_p), ("dtype", C.c_int32)]


class _Vec(C.Structure):
    _fields_ = [("data", C.c_void_p), ("dtype", C.c_int32)]


class _Layer(C.Structure):
    _fields_ = [("d", C.c_int32), ("N", C.c_int32), ("H", C.c_int32), ("n_g", C.c_int32), ("kind", C.c_int32),
                ("cold", C.c_int32), ("P1", _Mat), ("c1", _Vec), ("P2", _Mat), ("c2", _Vec), ("table", C.c_void_p),
                ("W1", _Mat), ("b1", _Vec), ("Wup", _Mat), ("W2", _Mat), ("b2", _Vec)]


class _Attn(C.Structure):
    _fields_ = [("d", C.c_int32), ("n_heads", C.c_int32), ("dh", C.c_int32), ("Ha", C.c_int32), ("L_max", C.c_int32),
                ("Pa1", _Mat), ("ca1", _Vec), ("Pa2", _Mat), ("ca2", _Vec), ("Wq", _Mat), ("bq", _Vec), ("Wk", _Mat),
                ("bk", _Vec), ("Wv", _Mat), ("bv", _Vec), ("WoT", _Mat), ("bo", _Vec), ("Kc", C.c_void_p),
                ("Vc", C.c_void_p)]


_lib = None


def load():
    """Load libpi.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise PiError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = C.CDLL(LIB_PATH)
        P, I = C.c_void_p, C.c_int32
        L.pi_predict.argtypes = [P, I, I, I, I, P, _Mat, _Vec, _Mat, _Vec, P, P, C.c_size_t]
        L.pi_predict_output.argtypes = [P, I, I, I, P, _Mat, _Vec, C.c_float, P, P, P, C.c_size_t]
        L.pi_predict_output.restype = C.c_int
        L.pi_compact.argtypes = [P, I, I, P, C.c_float, P, I, P, P, P, I, P, P, P, C.c_size_t]
        L.pi_sparse_ffn.argtypes = [P, I, I, I, I, P, _Mat, _Vec, _Mat, _Mat, P, P, P, P, C.c_size_t]
        L.pi_merge.argtypes = [P, I, I, P, P, P, _Vec]
        L.pi_layer_norm.argtypes = [P, I, I, P, C.c_float, P]
        L.pi_layer_norm.restype = C.c_int
        L.pi_read_probe.argtypes = [P, P, C.c_size_t, I, I, P]
        L.pi_read_probe.restype = C.c_int
        L.pi_table_bytes.argtypes = [I]
        L.pi_table_bytes.restype = C.c_size_t
        L.pi_table_prepare.argtypes = [I, P, I, P, C.c_size_t]
        L.pi_table_prepare.restype = C.c_int
        L.pi_ffn_layer.argtypes = [P, C.POINTER(_Layer), I, P, C.c_float, P, P, P, P, P, P, P, P, C.c_size_t, P]
        L.pi_ffn_layer.restype = C.c_int
        L.pi_ffn_layer_static.argtypes = [P, C.POINTER(_Layer), I, P, C.c_float, P, P, P, P, P, P, P]
        L.pi_ffn_layer_static.restype = C.c_int
        L.pi_ffn_layer_stages.argtypes = [P, C.POINTER(_Layer), I, P, C.c_float, P, P, P, P, P, P, P, P, C.c_size_t, P,
                                          C.c_uint32, P]
        L.pi_ffn_layer_stages.restype = C.c_int
        L.pi_ffn_layer_ahead.argtypes = [P, C.POINTER(_Layer), I, P, C.c_float, P, P, P, P, P, P, P, P, C.c_size_t,
                                         C.c_uint32, C.POINTER(_Layer), P, C.c_size_t]
        L.pi_ffn_layer_ahead.restype = C.c_int
        L.pi_ffn_layer_normed.argtypes = [P, C.POINTER(_Layer), I, P, C.c_float, C.c_float, P, P, P, P, P, P, P, P,
                                          P, C.c_size_t]
        L.pi_ffn_layer_normed.restype = C.c_int
        L.pi_attn_decode.argtypes = [P, C.POINTER(_Attn), I, P, C.c_float, P, P, P, P, P, C.c_size_t]
        L.pi_attn_decode.restype = C.c_int
        L.pi_attn_workspace_bytes.argtypes = [C.POINTER(_Attn)]
        L.pi_attn_workspace_bytes.restype = C.c_size_t
        L.pi_workspace_bytes.argtypes = [I, I, I, I, I, I]
        L.pi_workspace_bytes.restype = C.c_size_t
        L.pi_status_string.argtypes = [I]
        L.pi_status_string.restype = C.c_char_p
        L.pi_last_hip_error.restype = I
        L.pi_abi_version.restype = I
        for name in ("pi_predict", "pi_compact", "pi_sparse_ffn", "pi_merge"):
            getattr(L, name).restype = C.c_int
        _lib = L
    return _lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


@dataclass
class Matrix:
    """Device weights: float32 / float16 tensor [rows, cols], or uint8 packed
    int4 [rows, cols/2] with int16 fp16-bit scales [rows, cols/128].  The
    predictor's output layer P2 is stored hidden-major, [H, N]."""
    data: object
    dtype: int
    scales: object = None

    def _c(self) -> _Mat:
        return _Mat(_ptr(self.data), _ptr(self.scales), self.dtype)


@dataclass
class Vector:
    """Device bias, float32 or float16 (fp16 bits); ``data=None`` = zero."""
    data: object = None
    dtype: int = PI_F32

    def _c(self) -> _Vec:
        return _Vec(_ptr(self.data), self.dtype)


_NO_MAT = Matrix(None, PI_F16)
_NO_VEC = Vector(None, PI_F32)


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, what: str) -> None:
    if status != PI_OK:
        L = load()
        msg = L.pi_status_string(status).decode()
        if status == PI_EHIP:
            msg += f" (hipError {L.pi_last_hip_error()})"
        raise PiError(f"{what}: {msg}")


def pi_workspace_bytes(op: int, B: int, d: int, H: int = 0, N: int = 0, n_g: int = 0) -> int:
    return int(load().pi_workspace_bytes(op, B, d, H, N, n_g))


def pi_predict(B, d, H, N, x, P1: Matrix, c1: Vector, P2: Matrix, c2: Vector, logits, ws, ws_bytes=None,
               stream=None) -> None:
    nbytes = ws_bytes if ws_bytes is not None else ws.numel() * ws.element_size()
    _check(load().pi_predict(_stream(stream), B, d, H, N, _ptr(x), P1._c(), (c1 or _NO_VEC)._c(), P2._c(),
                             (c2 or _NO_VEC)._c(), _ptr(logits), _ptr(ws), nbytes), "pi_predict")


def pi_predict_output(B, H, N, h, P2: Matrix, c2: Vector, tau, logits, mask=None, ws=None, ws_bytes=None,
                      stream=None) -> None:
    nbytes = ws_bytes if ws_bytes is not None else (ws.numel() * ws.element_size() if ws is not None else 0)
    _check(load().pi_predict_output(_stream(stream), B, H, N, _ptr(h), P2._c(), (c2 or _NO_VEC)._c(), float(tau),
                                    _ptr(logits), _ptr(mask), _ptr(ws), nbytes), "pi_predict_output")


def pi_compact(B, N, logits, tau, T_g, n_g, A_g, K, T_c=None, n_c=0, A_c=None, K_c=None, stream=None) -> None:
    _check(load().pi_compact(_stream(stream), B, N, _ptr(logits), float(tau), _ptr(T_g), n_g, _ptr(A_g), _ptr(K),
                             _ptr(T_c), n_c, _ptr(A_c), _ptr(K_c), None, 0), "pi_compact")


def pi_sparse_ffn(B, d, n_g, kind, x, W1: Matrix, b1: Vector, Wup: Optional[Matrix], W2: Matrix, A_g, K, y_g, ws,
                  ws_bytes=None, stream=None) -> None:
    nbytes = ws_bytes if ws_bytes is not None else ws.numel() * ws.element_size()
    _check(load().pi_sparse_ffn(_stream(stream), B, d, n_g, kind, _ptr(x), W1._c(), (b1 or _NO_VEC)._c(),
                                (Wup or _NO_MAT)._c(), W2._c(), _ptr(A_g), _ptr(K), _ptr(y_g), _ptr(ws), nbytes),
           "pi_sparse_ffn")


def pi_read_probe(buf, nbytes: int, out, blocks: int = 0, stream=None, depth: int = 0) -> None:
    """The streaming-read reference: read nbytes of buf once (blocks / depth 0: the library's defaults)."""
    _check(load().pi_read_probe(_stream(stream), _ptr(buf), int(nbytes), int(blocks), int(depth), _ptr(out)),
           "pi_read_probe")


def pi_layer_norm(B, d, y, x, eps: float = 1e-5, stream=None) -> None:
    """Chained layers: x[b] = (y[b] - mean) / sqrt(var + eps) per row (x may be y)."""
    _check(load().pi_layer_norm(_stream(stream), int(B), int(d), _ptr(y), float(eps), _ptr(x)), "pi_layer_norm")


def pi_merge(B, d, y, y_c=None, K_c=None, b2: Optional[Vector] = None, stream=None) -> None:
    _check(load().pi_merge(_stream(stream), B, d, _ptr(y), _ptr(y_c), _ptr(K_c), (b2 or _NO_VEC)._c()), "pi_merge")


def pi_table_bytes(N: int) -> int:
    return int(load().pi_table_bytes(N))


def pi_table_prepare(N: int, T_g):
    """Prepared neuron table (host numpy uint8 buffer) of an ascending host int32 T_g."""
    import numpy as np
    T = np.ascontiguousarray(T_g, dtype=np.int32)
    nb = pi_table_bytes(N)
    buf = np.zeros(max(nb, 1), np.uint8)
    _check(load().pi_table_prepare(N, T.ctypes.data if len(T) else None, len(T), buf.ctypes.data, nb),
           "pi_table_prepare")
    return buf


@dataclass
class Layer:
    """Arguments of pi_ffn_layer that describe one layer (device tensors)."""
    d: int
    N: int
    H: int
    n_g: int
    kind: int
    cold: bool
    P1: Matrix
    c1: Optional[Vector]
    P2: Matrix
    c2: Optional[Vector]
    table: object
    W1: Matrix
    b1: Optional[Vector]
    Wup: Optional[Matrix]
    W2: Matrix
    b2: Optional[Vector] = None

    def _c(self) -> _Layer:
        return _Layer(self.d, self.N, self.H, self.n_g, self.kind, int(bool(self.cold)), self.P1._c(),
                      (self.c1 or _NO_VEC)._c(), self.P2._c(), (self.c2 or _NO_VEC)._c(), _ptr(self.table),
                      self.W1._c(), (self.b1 or _NO_VEC)._c(), (self.Wup or _NO_MAT)._c(), self.W2._c(),
                      (self.b2 or _NO_VEC)._c())


def event_handles(events):
    """Raw hipEvent_t handles of torch events (each recorded once so that it exists)."""
    import torch
    hs = []
    for e in events:
        if not e.cuda_event:
            e.record()
        hs.append(e.cuda_event)
    torch.cuda.current_stream().synchronize()
    return (C.c_void_p * len(hs))(*hs)


def pi_ffn_layer(layer: Layer, B: int, x, tau: float, y_c, y, logits, A_g, K, A_c, K_c, ws, ws_bytes=None,
                 events=None, stream=None, _cstruct=None) -> None:
    """One layer: predictor, compaction, FFN over the GPU-resident neurons, merge."""
    nbytes = ws_bytes if ws_bytes is not None else ws.numel() * ws.element_size()
    cl = _cstruct if _cstruct is not None else layer._c()
    _check(load().pi_ffn_layer(_stream(stream), C.byref(cl), B, _ptr(x), float(tau), _ptr(y_c), _ptr(y),
                               _ptr(logits), _ptr(A_g), _ptr(K), _ptr(A_c), _ptr(K_c), _ptr(ws), nbytes, events),
           "pi_ffn_layer")


def pi_ffn_layer_static(layer: Layer, B: int, x, tau: float, y_c, y, logits, A_g, K, A_c, K_c, stream=None,
                        _cstruct=None) -> None:
    """pi_ffn_layer with the library's static workspace (no caller workspace; allocates nothing)."""
    cl = _cstruct if _cstruct is not None else layer._c()
    _check(load().pi_ffn_layer_static(_stream(stream), C.byref(cl), B, _ptr(x), float(tau), _ptr(y_c), _ptr(y),
                                      _ptr(logits), _ptr(A_g), _ptr(K), _ptr(A_c), _ptr(K_c)), "pi_ffn_layer_static")


def pi_ffn_layer_ahead(layer: Layer, B: int, x, tau: float, y_c, y, logits, A_g, K, A_c, K_c, ws, stages: int,
                       next_layer: Layer, ws_next, ws_bytes=None, ws_next_bytes=None, stream=None, _cstruct=None,
                       _next_cstruct=None) -> None:
    """pi_ffn_layer_stages on `layer`, plus `next_layer`'s predictor hidden layer from this x into ws_next."""
    nbytes = ws_bytes if ws_bytes is not None else ws.numel() * ws.element_size()
    nnext = ws_next_bytes if ws_next_bytes is not None else ws_next.numel() * ws_next.element_size()
    cl = _cstruct if _cstruct is not None else layer._c()
    cn = _next_cstruct if _next_cstruct is not None else next_layer._c()
    _check(load().pi_ffn_layer_ahead(_stream(stream), C.byref(cl), B, _ptr(x), float(tau), _ptr(y_c), _ptr(y),
                                     _ptr(logits), _ptr(A_g), _ptr(K), _ptr(A_c), _ptr(K_c), _ptr(ws), nbytes,
                                     int(stages), C.byref(cn), _ptr(ws_next), nnext), "pi_ffn_layer_ahead")


def pi_ffn_layer_normed(layer: Layer, B: int, y_prev, eps: float, tau: float, y_c, y, logits, A_g, K, A_c, K_c, ws,
                        x_out=None, ws_bytes=None, stream=None, _cstruct=None) -> None:
    """pi_ffn_layer on the layer normalisation of y_prev (the chained-layer input), in the layer's own kernels."""
    nbytes = ws_bytes if ws_bytes is not None else ws.numel() * ws.element_size()
    cl = _cstruct if _cstruct is not None else layer._c()
    _check(load().pi_ffn_layer_normed(_stream(stream), C.byref(cl), B, _ptr(y_prev), float(eps), float(tau),
                                      _ptr(y_c), _ptr(y), _ptr(logits), _ptr(A_g), _ptr(K), _ptr(A_c), _ptr(K_c),
                                      _ptr(x_out), _ptr(ws), nbytes), "pi_ffn_layer_normed")


def pi_ffn_layer_stages(layer: Layer, B: int, x, tau: float, y_c, y, logits, A_g, K, A_c, K_c, ws, stages: int,
                        rows_read=None, ws_bytes=None, events=None, stream=None, _cstruct=None) -> None:
    """pi_ffn_layer restricted to some stages (PI_STAGE_* bits), with the optional rows-read report."""
    nbytes = ws_bytes if ws_bytes is not None else ws.numel() * ws.element_size()
    cl = _cstruct if _cstruct is not None else layer._c()
    _check(load().pi_ffn_layer_stages(_stream(stream), C.byref(cl), B, _ptr(x), float(tau), _ptr(y_c), _ptr(y),
                                      _ptr(logits), _ptr(A_g), _ptr(K), _ptr(A_c), _ptr(K_c), _ptr(ws), nbytes,
                                      events, int(stages), _ptr(rows_read)), "pi_ffn_layer_stages")


@dataclass
class Attn:
    """The self-attention block of pi_attn_decode: fp16 matrices (Pa1 [Ha, d], Pa2 [n_heads, Ha],
    Wq / Wk / Wv [d, d] with row = output element, WoT [d, d] with row = head element), fp16 or
    absent biases, and the fp16 caches Kc / Vc [n_heads, L_max, dh]."""
    d: int
    n_heads: int
    dh: int
    Ha: int
    L_max: int
    Pa1: Matrix
    Pa2: Matrix
    Wq: Matrix
    Wk: Matrix
    Wv: Matrix
    WoT: Matrix
    Kc: object
    Vc: object
    ca1: Optional[Vector] = None
    ca2: Optional[Vector] = None
    bq: Optional[Vector] = None
    bk: Optional[Vector] = None
    bv: Optional[Vector] = None
    bo: Optional[Vector] = None

    def _c(self) -> _Attn:
        v = lambda b: (b or Vector(None, PI_F16))._c()
        return _Attn(self.d, self.n_heads, self.dh, self.Ha, self.L_max, self.Pa1._c(), v(self.ca1), self.Pa2._c(),
                     v(self.ca2), self.Wq._c(), v(self.bq), self.Wk._c(), v(self.bk), self.Wv._c(), v(self.bv),
                     self.WoT._c(), v(self.bo), _ptr(self.Kc), _ptr(self.Vc))


def pi_attn_workspace_bytes(attn: Attn) -> int:
    c = attn._c()
    return int(load().pi_attn_workspace_bytes(C.byref(c)))


def pi_attn_decode(attn: Attn, t: int, x, tau: float, y, head_logits, heads, n_active, ws, ws_bytes=None,
                   stream=None, _cstruct=None) -> None:
    """One decode step of the attention block with head sparsity (position t)."""
    nbytes = ws_bytes if ws_bytes is not None else ws.numel() * ws.element_size()
    c = _cstruct if _cstruct is not None else attn._c()
    _check(load().pi_attn_decode(_stream(stream), C.byref(c), int(t), _ptr(x), float(tau), _ptr(y),
                                 _ptr(head_logits), _ptr(heads), _ptr(n_active), _ptr(ws), nbytes), "pi_attn_decode")
