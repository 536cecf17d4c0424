"""Python binding of libpi_host, the CPU side of the hybrid layer (``include/pi_host.h``).

Argument marshalling only: the work runs in ``libpi_host.so``.  Arrays are
host arrays (numpy arrays or CPU torch tensors).  Raises
:class:`activation_sparse_amd.PiError` if the library is missing or a call
fails.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

from . import PiError, Matrix, Vector, _Mat, _Vec, PI_OK, PI_RELU

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpi_host.so")
EXPORTS = ("pi_cold_ffn", "pi_cold_ffn_ex", "pi_host_vector_path")

_lib = None


def load():
    """Load libpi_host.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise PiError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = C.CDLL(LIB_PATH)
        P, I = C.c_void_p, C.c_int32
        L.pi_cold_ffn.argtypes = [I, I, I, I, P, _Mat, _Vec, _Mat, _Mat, P, I, P, I]
        L.pi_cold_ffn.restype = C.c_int
        L.pi_cold_ffn_ex.argtypes = [I, I, I, I, P, _Mat, _Vec, _Mat, _Mat, P, I, P, I, I]
        L.pi_cold_ffn_ex.restype = C.c_int
        L.pi_host_vector_path.restype = C.c_int
        _lib = L
    return _lib


def _hptr(a) -> Optional[int]:
    if a is None:
        return None
    if isinstance(a, int):
        return a
    if hasattr(a, "ctypes"):
        return a.ctypes.data
    return a.data_ptr()


def _hmat(m: Optional[Matrix]) -> _Mat:
    if m is None:
        return _Mat(None, None, 0)
    return _Mat(_hptr(m.data), _hptr(m.scales), m.dtype)


def _hvec(v: Optional[Vector]) -> _Vec:
    if v is None:
        return _Vec(None, 0)
    return _Vec(_hptr(v.data), v.dtype)


_STATUS = {0: "PI_OK", 1: "PI_EINVAL", 2: "PI_EWORKSPACE", 3: "PI_EUNSUPPORTED", 4: "PI_EHIP"}


def pi_cold_ffn(B: int, d: int, n_c: int, x, W1: Matrix, b1: Optional[Vector], W2: Matrix, A_c, K_c: int, y_c,
                kind: int = PI_RELU, Wup: Optional[Matrix] = None, threads: int = 0, path: int = -1) -> None:
    """y_c[b,:] = sum over the K_c listed CPU-table slots of a[b,j] W2[slot] (see pi_host.h);
    path: -1 the best this CPU has, 1 AVX2, 0 scalar."""
    st = load().pi_cold_ffn_ex(B, d, n_c, kind, _hptr(x), _hmat(W1), _hvec(b1), _hmat(Wup), _hmat(W2), _hptr(A_c),
                               int(K_c), _hptr(y_c), threads, path)
    if st != PI_OK:
        raise PiError(f"pi_cold_ffn: {_STATUS.get(st, st)}")


def vector_path() -> int:
    """1 when pi_cold_ffn runs its AVX2 + FMA + F16C loops on this CPU, 0 for the scalar ones."""
    return load().pi_host_vector_path()
