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

from . import PiError, Matrix, Vector, _Mat, _Vec, _Layer, PI_OK, PI_RELU

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpi_host.so")
EXPORTS = ("pi_cold_ffn", "pi_cold_ffn_ex", "pi_host_vector_path", "pi_host_read_probe", "pi_hybrid_layer",
           "pi_hybrid_prime", "pi_hybrid_layer_ahead", "pi_hybrid_stack_ahead")

class _HostCold(C.Structure):
    _fields_ = [("n_c", C.c_int32), ("W1", _Mat), ("b1", _Vec), ("Wup", _Mat), ("W2", _Mat)]


class _HybridScratch(C.Structure):
    _fields_ = [("logits", C.c_void_p), ("A_g", C.c_void_p), ("K", C.c_void_p), ("cold_list", C.c_void_p),
                ("y_c", C.c_void_p), ("ws_pred", C.c_void_p), ("ws_pred_bytes", C.c_size_t),
                ("ws_ffn", C.c_void_p), ("ws_ffn_bytes", C.c_size_t), ("x_host", C.c_void_p),
                ("cold_list_host", C.c_void_p), ("y_c_host", C.c_void_p), ("event", C.c_void_p)]


class _HybridAheadScratch(C.Structure):
    _fields_ = [("logits", C.c_void_p), ("ws_pred", C.c_void_p), ("ws_pred_bytes", C.c_size_t),
                ("ws_ffn", C.c_void_p), ("ws_ffn_bytes", C.c_size_t), ("A_g", C.c_void_p * 2), ("K", C.c_void_p * 2),
                ("cold_list", C.c_void_p * 2), ("cold_list_host", C.c_void_p * 2), ("list_event", C.c_void_p * 2),
                ("y_c", C.c_void_p), ("x_host", C.c_void_p), ("y_c_host", C.c_void_p), ("x_event", C.c_void_p),
                ("cur", C.c_int32)]


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
        L.pi_host_read_probe.argtypes = [P, C.c_size_t, I, C.POINTER(C.c_uint64)]
        L.pi_host_read_probe.restype = C.c_int
        L.pi_hybrid_layer.argtypes = [P, C.POINTER(_Layer), P, P, C.POINTER(_HostCold), I, P, C.c_float, P,
                                      C.POINTER(_HybridScratch), I, C.POINTER(C.c_int32)]
        L.pi_hybrid_layer.restype = C.c_int
        L.pi_hybrid_prime.argtypes = [P, C.POINTER(_Layer), P, P, I, I, P, C.c_float, C.POINTER(_HybridAheadScratch)]
        L.pi_hybrid_prime.restype = C.c_int
        L.pi_hybrid_layer_ahead.argtypes = [P, C.POINTER(_Layer), C.POINTER(_HostCold), C.POINTER(_Layer), P, P, I, I,
                                            P, C.c_float, P, C.POINTER(_HybridAheadScratch), I, C.POINTER(C.c_int32)]
        L.pi_hybrid_layer_ahead.restype = C.c_int
        L.pi_hybrid_stack_ahead.argtypes = [P, I, P, P, P, P, P, I, P, C.c_float, P, C.POINTER(_HybridAheadScratch), I,
                                            P]
        L.pi_hybrid_stack_ahead.restype = C.c_int
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


def pi_host_read_probe(buf, nbytes: int, threads: int = 0) -> int:
    """Streaming read of nbytes of host memory at buf (address or numpy array) by `threads`
    threads; returns the XOR of every 8-byte word read."""
    out = C.c_uint64(0)
    ptr = buf.ctypes.data if hasattr(buf, "ctypes") else buf
    st = load().pi_host_read_probe(ptr, int(nbytes), int(threads), C.byref(out))
    if st != PI_OK:
        raise PiError(f"pi_host_read_probe: {_STATUS.get(st, st)}")
    return int(out.value)


def pi_hybrid_layer(stream: int, layer_c, T_g: int, T_c: Optional[int], cold_c, B: int, x: int, tau: float, y: int,
                    scratch_c, threads: int = 0) -> int:
    """One hybrid layer (see pi_host.h); pointers are ints, the structs prebuilt; returns K_c."""
    kc = C.c_int32(0)
    st = load().pi_hybrid_layer(stream, C.byref(layer_c), T_g, T_c, C.byref(cold_c) if cold_c is not None else None,
                                B, x, float(tau), y, C.byref(scratch_c), threads, C.byref(kc))
    if st != PI_OK:
        raise PiError(f"pi_hybrid_layer: {_STATUS.get(st, st)}")
    return kc.value


def pi_hybrid_prime(stream: int, layer_c, T_g: int, T_c: Optional[int], n_c: int, B: int, x: int, tau: float,
                    scratch_c) -> None:
    """Predict `layer` from x into the scratch's current list set (see pi_host.h)."""
    st = load().pi_hybrid_prime(stream, C.byref(layer_c), T_g, T_c, n_c, B, x, float(tau), C.byref(scratch_c))
    if st != PI_OK:
        raise PiError(f"pi_hybrid_prime: {_STATUS.get(st, st)}")


def pi_hybrid_layer_ahead(stream: int, layer_c, cold_c, next_c, T_g_next: Optional[int], T_c_next: Optional[int],
                          n_c_next: int, B: int, x: int, tau: float, y: int, scratch_c, threads: int = 0) -> int:
    """One look-ahead hybrid layer (see pi_host.h); returns K_c."""
    kc = C.c_int32(0)
    st = load().pi_hybrid_layer_ahead(stream, C.byref(layer_c), C.byref(cold_c) if cold_c is not None else None,
                                      C.byref(next_c) if next_c is not None else None, T_g_next, T_c_next, n_c_next,
                                      B, x, float(tau), y, C.byref(scratch_c), threads, C.byref(kc))
    if st != PI_OK:
        raise PiError(f"pi_hybrid_layer_ahead: {_STATUS.get(st, st)}")
    return kc.value


def pi_hybrid_stack_ahead(stream: int, layers_arr, colds_arr, T_g_arr, T_c_arr, n_c_arr, n_layers: int, B: int,
                          xs_arr, tau: float, ys_arr, scratch_c, threads: int = 0, K_c_out=None) -> None:
    """A stack of look-ahead hybrid layers in one native call (see pi_host.h); the arrays are
    prebuilt ctypes arrays (pi_layer structs, pointers), K_c_out an int32 array or None."""
    st = load().pi_hybrid_stack_ahead(stream, n_layers, C.cast(layers_arr, C.c_void_p), C.cast(colds_arr, C.c_void_p),
                                      C.cast(T_g_arr, C.c_void_p), C.cast(T_c_arr, C.c_void_p),
                                      C.cast(n_c_arr, C.c_void_p), B, C.cast(xs_arr, C.c_void_p), float(tau),
                                      C.cast(ys_arr, C.c_void_p), C.byref(scratch_c), threads,
                                      _hptr(K_c_out) if K_c_out is not None else None)
    if st != PI_OK:
        raise PiError(f"pi_hybrid_stack_ahead: {_STATUS.get(st, st)}")
