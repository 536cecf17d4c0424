"""Python front end of the CPU oracle (``oracle/oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this module.  It shares no
code with the HIP library and never touches a GPU.

Arrays are numpy; every weight argument is a :class:`Mat` holding the stored
bits (float32, float16 bits as uint16, or packed int4 + fp16 scale bits).
The sources each function follows are listed in ``oracle/oracle.h``.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

F32, F16, I4G128 = 0, 1, 2
RELU, GATED_RELU = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")


def build() -> str:
    """Compile the oracle with gcc (plain C, OpenMP, no contraction)."""
    import subprocess
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-Wall",
           "-o", _LIB_PATH, os.path.join(_HERE, "oracle.c"), "-lm"]
    subprocess.run(cmd, check=True)
    return _LIB_PATH


class _OrMat(C.Structure):
    _fields_ = [("data", C.c_void_p), ("scales", C.c_void_p), ("dtype", C.c_int32), ("cols", C.c_int64)]


class _OrVec(C.Structure):
    _fields_ = [("data", C.c_void_p), ("dtype", C.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = C.CDLL(_LIB_PATH)
        P = C.c_void_p
        L.or_f16_to_double.restype = C.c_double
        L.or_f16_to_double.argtypes = [C.c_uint16]
        L.or_predict.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, P, _OrMat, _OrVec, _OrMat, _OrVec, P, P]
        L.or_compact.argtypes = [C.c_int, C.c_int, P, C.c_float, P, C.c_int, P, P, P, C.c_int, P, P]
        L.or_sparse_ffn.argtypes = [C.c_int, C.c_int, C.c_int, P, _OrMat, _OrVec, _OrMat, _OrMat, P, C.c_int, P, P]
        L.or_dense_ffn.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, P, _OrMat, _OrVec, _OrMat, _OrMat, _OrVec, P]
        L.or_merge.argtypes = [C.c_int, C.c_int, P, P, C.c_int, _OrVec, P]
        L.or_layer_norm.argtypes = [C.c_int, C.c_int, P, C.c_double, P]
        L.or_double_to_f16.argtypes = [C.c_double]
        L.or_double_to_f16.restype = C.c_uint16
        L.or_attn_decode.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, P, _OrMat, _OrVec, _OrMat, _OrVec,
                                     C.c_float, _OrMat, _OrVec, _OrMat, _OrVec, _OrMat, _OrVec, _OrMat, _OrVec, P, P,
                                     C.c_int, P, P, P, P, P, P]
        L.or_set_threads.argtypes = [C.c_int]
        L.or_get_threads.restype = C.c_int
        _lib = L
    return _lib


@dataclass
class Mat:
    """Stored weights: ``data`` is float32 [rows, cols], uint16 fp16 bits
    [rows, cols], or uint8 packed int4 [rows, cols/2] with ``scales`` uint16
    fp16 bits [rows, cols/128]."""
    data: np.ndarray
    dtype: int
    cols: int
    scales: Optional[np.ndarray] = None

    @property
    def rows(self) -> int:
        return self.data.shape[0]

    def _c(self) -> _OrMat:
        d = np.ascontiguousarray(self.data)
        self.data = d
        s = None
        if self.scales is not None:
            self.scales = np.ascontiguousarray(self.scales)
            s = self.scales.ctypes.data
        return _OrMat(d.ctypes.data, s, self.dtype, self.cols)


@dataclass
class Vec:
    """Stored bias: float32 or uint16 fp16 bits; ``data=None`` means zeros."""
    data: Optional[np.ndarray]
    dtype: int = F32

    def _c(self) -> _OrVec:
        if self.data is None:
            return _OrVec(None, self.dtype)
        self.data = np.ascontiguousarray(self.data)
        return _OrVec(self.data.ctypes.data, self.dtype)


def _none_mat() -> Mat:
    return Mat(np.zeros((1, 1), np.float32), F32, 1)


def set_threads(n: int) -> None:
    lib().or_set_threads(int(n))


def get_threads() -> int:
    return int(lib().or_get_threads())


def f16_to_double(bits: int) -> float:
    return float(lib().or_f16_to_double(int(bits)))


def predict(x: np.ndarray, P1: Mat, c1: Vec, P2: Mat, c2: Vec, return_hidden: bool = False):
    """Two-layer predictor MLP in fp64 -> logits [B, N] (and h [B, H])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    B, d = x.shape
    H, N = P1.rows, P2.rows
    assert P1.cols == d and P2.cols == H
    logits = np.empty((B, N), np.float64)
    h = np.empty((B, H), np.float64)
    lib().or_predict(B, d, H, N, x.ctypes.data, P1._c(), c1._c(), P2._c(), c2._c(), h.ctypes.data, logits.ctypes.data)
    return (logits, h) if return_hidden else logits


def compact(logits: np.ndarray, tau: float, T_g: np.ndarray, T_c: Optional[np.ndarray] = None):
    """Union mask over the batch (fp32 compare), then ascending slot lists.
    Returns (A_g, A_c) with A_c None when T_c is None."""
    logits = np.ascontiguousarray(logits, dtype=np.float64)
    B, N = logits.shape
    T_g = np.ascontiguousarray(T_g, dtype=np.int32)
    A_g = np.empty(max(len(T_g), 1), np.int32)
    K = np.zeros(1, np.int32)
    if T_c is not None:
        T_c = np.ascontiguousarray(T_c, dtype=np.int32)
        A_c = np.empty(max(len(T_c), 1), np.int32)
        K_c = np.zeros(1, np.int32)
        lib().or_compact(B, N, logits.ctypes.data, float(tau), T_g.ctypes.data, len(T_g), A_g.ctypes.data,
                         K.ctypes.data, T_c.ctypes.data, len(T_c), A_c.ctypes.data, K_c.ctypes.data)
        return A_g[:K[0]].copy(), A_c[:K_c[0]].copy()
    lib().or_compact(B, N, logits.ctypes.data, float(tau), T_g.ctypes.data, len(T_g), A_g.ctypes.data,
                     K.ctypes.data, None, 0, None, None)
    return A_g[:K[0]].copy(), None


def sparse_ffn(x: np.ndarray, W1: Mat, b1: Vec, W2: Mat, rows: np.ndarray, kind: int = RELU,
               Wup: Optional[Mat] = None, return_act: bool = False):
    """y[b] = sum_j a[b,j] W2[rows_j]; a = ReLU(W1[rows_j].x_b + b1) (x Wup.x if gated)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    B, d = x.shape
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    K = len(rows)
    y = np.empty((B, d), np.float64)
    a = np.empty((B, max(K, 1)), np.float64)
    up = Wup if Wup is not None else _none_mat()
    lib().or_sparse_ffn(B, d, kind, x.ctypes.data, W1._c(), b1._c(), up._c(), W2._c(),
                        rows.ctypes.data if K else None, K, a.ctypes.data, y.ctypes.data)
    return (y, a[:, :K]) if return_act else y


def dense_ffn(x: np.ndarray, W1: Mat, b1: Vec, W2: Mat, kind: int = RELU, Wup: Optional[Mat] = None,
              b2: Optional[Vec] = None):
    x = np.ascontiguousarray(x, dtype=np.float32)
    B, d = x.shape
    y = np.empty((B, d), np.float64)
    up = Wup if Wup is not None else _none_mat()
    lib().or_dense_ffn(B, d, W1.rows, kind, x.ctypes.data, W1._c(), b1._c(), up._c(), W2._c(),
                       (b2 or Vec(None))._c(), y.ctypes.data)
    return y


def merge(y_g: np.ndarray, y_c: Optional[np.ndarray], K_c: int, b2: Optional[Vec] = None):
    y_g = np.ascontiguousarray(y_g, dtype=np.float64)
    B, d = y_g.shape
    y = np.empty_like(y_g)
    yc = None
    if y_c is not None:
        yc = np.ascontiguousarray(y_c, dtype=np.float64)
    lib().or_merge(B, d, y_g.ctypes.data, yc.ctypes.data if yc is not None else None, int(K_c),
                   (b2 or Vec(None))._c(), y.ctypes.data)
    return y


def layer_norm(y: np.ndarray, eps: float) -> np.ndarray:
    """Chained-layer input from a layer's output: per row, subtract the mean and divide by
    sqrt(population variance + eps), in fp64 from the fp32 y -> [B, d] float64."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    if y.ndim == 1:
        y = y[None, :]
    B, d = y.shape
    x = np.empty((B, d), np.float64)
    lib().or_layer_norm(B, d, y.ctypes.data, float(eps), x.ctypes.data)
    return x


def double_to_f16(v: float) -> int:
    """fp16 bits of v, round to nearest even (the oracle's own conversion)."""
    return int(lib().or_double_to_f16(float(v)))


def attn_decode(x: np.ndarray, Pa1: Mat, ca1: Vec, Pa2: Mat, ca2: Vec, tau: float, Wq: Mat, bq: Vec, Wk: Mat,
                bk: Vec, Wv: Mat, bv: Vec, WoT: Mat, bo: Vec, Kc: np.ndarray, Vc: np.ndarray, n_heads: int,
                d_h: int, t: int) -> dict:
    """Self-attention block with head sparsity at decode (see or_attn_decode in oracle.h).
    x: [d] float32; Kc, Vc: uint16 fp16 bits [n_heads, L_max, d_h] (positions < t are read).
    Returns head_logits [n_heads] float64, heads (ascending active heads) int32, k_new and v_new
    [d] uint16 fp16 bits (this token's cache entry), y [d] float64."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    d = x.shape[0]
    Kc = np.ascontiguousarray(Kc, dtype=np.uint16)
    Vc = np.ascontiguousarray(Vc, dtype=np.uint16)
    L_max = Kc.shape[1]
    assert Kc.shape == (n_heads, L_max, d_h) and Vc.shape == Kc.shape and n_heads * d_h == d and 0 <= t < L_max
    Ha = Pa1.rows
    logits = np.empty(n_heads, np.float64)
    heads = np.empty(n_heads, np.int32)
    na = np.zeros(1, np.int32)
    k_new = np.empty(d, np.uint16)
    v_new = np.empty(d, np.uint16)
    y = np.empty(d, np.float64)
    lib().or_attn_decode(d, n_heads, d_h, Ha, int(t), x.ctypes.data, Pa1._c(), ca1._c(), Pa2._c(), ca2._c(),
                         float(tau), Wq._c(), bq._c(), Wk._c(), bk._c(), Wv._c(), bv._c(), WoT._c(), bo._c(),
                         Kc.ctypes.data, Vc.ctypes.data, L_max, logits.ctypes.data, heads.ctypes.data, na.ctypes.data,
                         k_new.ctypes.data, v_new.ctypes.data, y.ctypes.data)
    return {"head_logits": logits, "heads": heads[:int(na[0])].copy(), "k_new": k_new, "v_new": v_new, "y": y}
