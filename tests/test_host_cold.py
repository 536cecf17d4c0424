"""The CPU side of the hybrid layer (libpi_host, include/pi_host.h), on the CPU:
parity with the oracle's sparse FFN over the cold rows, bitwise repeatability
over thread counts and between the AVX2 and scalar paths, the exported
symbols and the argument checks."""
import os
import re

import numpy as np
import pytest

import synth
import oracle as orc
import activation_sparse_amd as pi
from activation_sparse_amd import host
from tests import parity_harness as ph

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_host_symbols():
    text = open(os.path.join(ROOT, "include", "pi_host.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|int32_t|size_t)\s+(pi_\w+)\s*\(", text, re.M)))


def test_host_header_and_library_agree():
    assert declared_host_symbols() == sorted(host.EXPORTS)
    L = host.load()
    for name in declared_host_symbols():
        assert hasattr(L, name), name


def _case(dt, n_c, d, seed, gated=False, bias=True):
    """Cold rows of one layer: W1 (+ Wup), b1 placing each neuron's activation
    probability near 1/2, W2; stored as the formats of pi.h."""
    W1 = ph.host_mat(dt, seed, synth.TAG_W1, 0, d, 1 / np.sqrt(d), nrows=n_c)
    W2 = ph.host_mat(dt, seed, synth.TAG_W2, 0, d, 1 / np.sqrt(4 * d), nrows=n_c)
    Wup = ph.host_mat(dt, seed, synth.TAG_WUP, 0, d, 1 / np.sqrt(d), nrows=n_c) if gated else None
    b1 = None
    if bias:
        g = np.random.default_rng(seed)
        b1 = orc.Vec((g.standard_normal(n_c) * 0.3).astype(np.float16).view(np.uint16), orc.F16)
    return W1, b1, Wup, W2


def _pm(m):
    return None if m is None else pi.Matrix(m.data, m.dtype, m.scales)


def _pv(v):
    return pi.Vector(None, pi.PI_F32) if v is None else pi.Vector(v.data, v.dtype)


def _run_host(x, W1, b1, Wup, W2, A_c, n_c, threads=0, path=-1):
    B, d = x.shape
    y = np.full((B, d), np.nan, np.float32)
    host.pi_cold_ffn(B, d, n_c, x, _pm(W1), _pv(b1), _pm(W2), A_c, len(A_c), y,
                     kind=pi.PI_GATED_RELU if Wup is not None else pi.PI_RELU, Wup=_pm(Wup), threads=threads, path=path)
    return y


CASES = [("f16", synth.F16, False), ("f32", synth.F32, False), ("i4", synth.I4G128, False),
         ("f16-gated", synth.F16, True)]


@pytest.mark.parametrize("B", [1, 3, 32])
@pytest.mark.parametrize("key,dt,gated", CASES, ids=[c[0] for c in CASES])
def test_cold_ffn_matches_the_oracle(key, dt, gated, B):
    """y_c against the oracle's fp64 sparse FFN on the same stored weights and list
    (the cold side computes exactly what the GPU side computes, over the CPU table)."""
    n_c, d = 700, 512
    W1, b1, Wup, W2 = _case(dt, n_c, d, 31 + B, gated)
    g = np.random.default_rng(7 + B)
    A_c = np.sort(g.choice(n_c, size=230, replace=False)).astype(np.int32)
    x = g.standard_normal((B, d)).astype(np.float32)
    y = _run_host(x, W1, b1, Wup, W2, A_c, n_c)
    ref = orc.sparse_ffn(x, W1, b1 if b1 is not None else orc.Vec(None), W2, A_c,
                         kind=orc.GATED_RELU if gated else orc.RELU, Wup=Wup)
    assert ph.rel_err(y.astype(np.float64), ref) <= ph.RTOL
    # fp32 sums of unit-scale terms over d = 512: far inside the bound
    assert ph.rel_err(y.astype(np.float64), ref) <= 1e-5


# batch counts that take each register block of the vector dot (1-4 rows, and 4 + 1, 4 + 2) and
# row lengths that end in a partial 32-column block (8, 16 and 24 columns) or none
@pytest.mark.parametrize("B,d", [(4, 1024), (1, 1048), (2, 1032), (3, 1040), (5, 1024), (6, 1048)])
def test_bits_do_not_depend_on_threads_or_vector_unit(B, d):
    n_c = 900
    W1, b1, _, W2 = _case(synth.F16, n_c, d, 5)
    g = np.random.default_rng(11)
    A_c = np.sort(g.choice(n_c, size=400, replace=False)).astype(np.int32)
    x = g.standard_normal((B, d)).astype(np.float32)
    outs = [_run_host(x, W1, b1, None, W2, A_c, n_c, threads=t) for t in (1, 3, 8)]
    outs.append(_run_host(x, W1, b1, None, W2, A_c, n_c, threads=4, path=0))
    if host.vector_path() == 1:
        outs.append(_run_host(x, W1, b1, None, W2, A_c, n_c, threads=2, path=1))
    for o in outs[1:]:
        assert o.tobytes() == outs[0].tobytes()


def test_empty_list_and_inactive_neurons():
    """K_c = 0 gives y_c = 0; neurons whose FC1 output is 0 add nothing (ReLU gate)."""
    n_c, d = 64, 256
    W1, _, _, W2 = _case(synth.F16, n_c, d, 3, bias=False)
    x = np.random.default_rng(2).standard_normal((2, d)).astype(np.float32)
    y = _run_host(x, W1, None, None, W2, np.zeros(0, np.int32), n_c)
    assert not np.any(y)
    # a bias of -1e4 turns every listed neuron off
    off = orc.Vec(np.full(n_c, -1e4, np.float32), orc.F32)
    y = _run_host(x, W1, off, None, W2, np.arange(n_c, dtype=np.int32), n_c)
    assert not np.any(y)


def test_argument_checks():
    n_c, d = 16, 64
    W1, b1, _, W2 = _case(synth.F16, n_c, d, 9)
    x = np.zeros((1, d), np.float32)
    y = np.zeros((1, d), np.float32)
    bad_slot = np.array([0, n_c], np.int32)
    with pytest.raises(pi.PiError, match="EINVAL"):
        host.pi_cold_ffn(1, d, n_c, x, _pm(W1), _pv(b1), _pm(W2), bad_slot, 2, y)
    with pytest.raises(pi.PiError, match="EINVAL"):
        host.pi_cold_ffn(33, d, n_c, x, _pm(W1), _pv(b1), _pm(W2), bad_slot[:1], 1, y)
    with pytest.raises(pi.PiError, match="EINVAL"):
        host.pi_cold_ffn(1, 60, n_c, x, _pm(W1), _pv(b1), _pm(W2), bad_slot[:1], 1, y)
    W2_32 = pi.Matrix(np.zeros((n_c, d), np.float32), pi.PI_F32)
    with pytest.raises(pi.PiError, match="EUNSUPPORTED"):
        host.pi_cold_ffn(1, d, n_c, x, _pm(W1), _pv(b1), W2_32, bad_slot[:1], 1, y)
    with pytest.raises(pi.PiError, match="EINVAL"):
        host.pi_cold_ffn(1, d, n_c, x, _pm(W1), _pv(b1), _pm(W2), bad_slot[:1], 1, y, kind=pi.PI_GATED_RELU)


def test_hybrid_layer_rejects_bad_arguments():
    """pi_hybrid_layer checks its arguments before any HIP call: a missing layer, scratch, input,
    output or GPU table, a batch outside 1..PI_MAX_BATCH, and a CPU table without the host
    buffers and the event it needs."""
    import ctypes as C
    FAKE = 1 << 20
    lay = pi.Layer(256, 1024, 64, 512, pi.PI_RELU, True, pi.Matrix(FAKE, pi.PI_F16), None,
                   pi.Matrix(FAKE, pi.PI_F16), None, FAKE, pi.Matrix(FAKE, pi.PI_F16), None, None,
                   pi.Matrix(FAKE, pi.PI_F16), None)._c()
    full = host._HybridScratch(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, FAKE, 1 << 20, FAKE, FAKE, FAKE, FAKE)
    cold = host._HostCold(512, host._Mat(FAKE, None, pi.PI_F16), host._Vec(None, 0), host._Mat(None, None, 0),
                          host._Mat(FAKE, None, pi.PI_F16))
    L = host.load()

    def call(layer=lay, T_g=FAKE, T_c=FAKE, cold_c=cold, B=1, x=FAKE, y=FAKE, scratch=full):
        return L.pi_hybrid_layer(0, C.byref(layer) if layer is not None else None, T_g, T_c,
                                 C.byref(cold_c) if cold_c is not None else None, B, x, 0.0, y,
                                 C.byref(scratch) if scratch is not None else None, 0, None)

    assert call(layer=None) == pi.PI_EINVAL
    assert call(scratch=None) == pi.PI_EINVAL
    assert call(x=None) == pi.PI_EINVAL and call(y=None) == pi.PI_EINVAL and call(T_g=None) == pi.PI_EINVAL
    assert call(B=0) == pi.PI_EINVAL and call(B=pi.PI_MAX_BATCH + 1) == pi.PI_EINVAL
    for field in ("cold_list", "y_c", "x_host", "cold_list_host", "y_c_host", "event"):
        s = host._HybridScratch.from_buffer_copy(full)
        setattr(s, field, None)
        assert call(scratch=s) == pi.PI_EINVAL, field


@pytest.mark.parametrize("K", [40, 127, 128, 600, 1500])
def test_both_fc2_orders_match_the_oracle(K):
    """FC2 takes column ranges over few contributing rows and chunks of whole rows over many
    (which, by the row count alone): both against the oracle, and bitwise across thread counts.
    A bias of +4 makes every listed neuron contribute, so K is the row count."""
    n_c, d, B = 1600, 256, 2
    W1, _, _, W2 = _case(synth.F16, n_c, d, 21 + K, bias=False)
    on = orc.Vec(np.full(n_c, 4.0, np.float32), orc.F32)
    g = np.random.default_rng(K)
    A_c = np.sort(g.choice(n_c, size=K, replace=False)).astype(np.int32)
    x = g.standard_normal((B, d)).astype(np.float32)
    ys = [_run_host(x, W1, on, None, W2, A_c, n_c, threads=t) for t in (1, 5, 16)]
    for y in ys[1:]:
        assert y.tobytes() == ys[0].tobytes()
    ref = orc.sparse_ffn(x, W1, on, W2, A_c, kind=orc.RELU)
    assert ph.rel_err(ys[0].astype(np.float64), ref) <= 1e-5


def test_lookahead_hybrid_rejects_bad_arguments():
    """pi_hybrid_prime and pi_hybrid_layer_ahead check their arguments before any HIP call."""
    import ctypes as C
    FAKE = 1 << 20
    lay = pi.Layer(256, 1024, 64, 512, pi.PI_RELU, True, pi.Matrix(FAKE, pi.PI_F16), None,
                   pi.Matrix(FAKE, pi.PI_F16), None, FAKE, pi.Matrix(FAKE, pi.PI_F16), None, None,
                   pi.Matrix(FAKE, pi.PI_F16), None)._c()
    P2 = C.c_void_p * 2
    full = host._HybridAheadScratch(FAKE, FAKE, 1 << 20, FAKE, 1 << 20, P2(FAKE, FAKE), P2(FAKE, FAKE),
                                    P2(FAKE, FAKE), P2(FAKE, FAKE), P2(FAKE, FAKE), FAKE, FAKE, FAKE, FAKE, 0)
    L = host.load()

    def prime(s=full, n_c=10, T_c=FAKE, B=1):
        return L.pi_hybrid_prime(0, C.byref(lay), FAKE, T_c, n_c, B, FAKE, 0.0, C.byref(s))

    def ahead(s=full, nxt=lay, T_g_next=FAKE, B=1, y=FAKE + (1 << 24)):
        return L.pi_hybrid_layer_ahead(0, C.byref(lay), None, C.byref(nxt) if nxt is not None else None, T_g_next,
                                       FAKE, 10, B, FAKE, 0.0, y, C.byref(s), 0, None)

    assert prime(n_c=-1) == pi.PI_EINVAL and prime(T_c=None) == pi.PI_EINVAL and prime(B=0) == pi.PI_EINVAL
    assert ahead(T_g_next=None) == pi.PI_EINVAL and ahead(y=None) == pi.PI_EINVAL
    assert ahead(B=pi.PI_MAX_BATCH + 1) == pi.PI_EINVAL
    assert ahead(y=FAKE) == pi.PI_EINVAL and ahead(y=FAKE + 512) == pi.PI_EINVAL   # y overlapping x (1 KB)
    bad = host._HybridAheadScratch.from_buffer_copy(full)
    bad.cur = 2
    assert prime(s=bad) == pi.PI_EINVAL and ahead(s=bad) == pi.PI_EINVAL
    for field in ("logits", "y_c", "x_host", "y_c_host", "x_event"):
        s = host._HybridAheadScratch.from_buffer_copy(full)
        setattr(s, field, None)
        assert prime(s=s) == pi.PI_EINVAL and ahead(s=s) == pi.PI_EINVAL, field
    s = host._HybridAheadScratch.from_buffer_copy(full)
    s.list_event[1] = None
    assert ahead(s=s) == pi.PI_EINVAL


def test_hybrid_stack_rejects_bad_arguments():
    import ctypes as C
    L = host.load()
    FAKE = 1 << 20
    arr = (C.c_void_p * 1)(FAKE)
    s = host._HybridAheadScratch()

    def call(n=1, layers=FAKE, xs=arr):
        return L.pi_hybrid_stack_ahead(0, n, layers, arr, arr, arr, arr, 1, xs, 0.0, arr, C.byref(s), 0, None)

    assert call(n=0) == pi.PI_EINVAL
    assert call(layers=None) == pi.PI_EINVAL
    assert call(xs=None) == pi.PI_EINVAL


def _aligned_words(n_words, seed):
    """uint64 words in a numpy buffer whose start is 64-byte aligned."""
    raw = np.empty(n_words + 8, np.uint64)
    off = (-raw.ctypes.data % 64) // 8
    w = raw[off:off + n_words]
    w[:] = np.random.default_rng(seed).integers(0, 2**63, n_words, dtype=np.uint64)
    return raw, w


@pytest.mark.parametrize("n_words,threads", [(8, 1), (8 * 1000, 3), (8 * 99991, 0), (8 * 4096, 16)])
def test_host_read_probe_reads_every_word(n_words, threads):
    raw, w = _aligned_words(n_words, n_words + threads)
    want = int(np.bitwise_xor.reduce(w))
    assert host.pi_host_read_probe(w.ctypes.data, w.nbytes, threads) == want
    w[n_words // 2] ^= np.uint64(1 << 17)                 # one flipped bit changes the result
    assert host.pi_host_read_probe(w.ctypes.data, w.nbytes, threads) == want ^ (1 << 17)


def test_host_read_probe_argument_checks():
    raw, w = _aligned_words(64, 5)
    p = w.ctypes.data
    for args in [(0, 64, 1), (p, 0, 1), (p, 96, 1), (p + 8, 64, 1)]:
        with pytest.raises(pi.PiError):
            host.pi_host_read_probe(*args)
