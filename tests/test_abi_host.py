"""C-ABI checks that need no GPU: the library loads, exports every symbol
include/pi.h declares, and rejects bad arguments before any HIP call."""
import ctypes as C
import os
import re

import pytest

import activation_sparse_amd as pi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "pi.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|int32_t|size_t|const char\*)\s+(pi_\w+)\s*\(", text, re.M)))


def test_header_declares_the_expected_entry_points():
    assert declared_symbols() == sorted(pi.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = pi.load()
    for name in declared_symbols():
        assert hasattr(L, name), name
    assert L.pi_abi_version() == pi.PI_ABI_VERSION == 3


def test_status_strings():
    L = pi.load()
    for s in range(5):
        assert L.pi_status_string(s).decode().startswith("PI_")
    assert b"unknown" in L.pi_status_string(99)


def test_workspace_sizes():
    assert pi.pi_workspace_bytes(pi.PI_OP_PREDICT, 1, 7168, 1024, 28672, 0) >= 1024 * 4
    assert pi.pi_workspace_bytes(pi.PI_OP_COMPACT, 1, 7168, 1024, 28672, 11468) == 0
    w1 = pi.pi_workspace_bytes(pi.PI_OP_SPARSE_FFN, 1, 7168, 0, 0, 11468)
    w32 = pi.pi_workspace_bytes(pi.PI_OP_SPARSE_FFN, 32, 7168, 0, 0, 11468)
    assert w1 >= 11468 * 4 + 7168 * 4 and w32 > w1


FAKE = 1 << 20       # a 16-byte aligned fake device address; never dereferenced on these paths


def mat(dt=pi.PI_F16, ptr=FAKE, scales=None):
    return pi.Matrix(ptr, dt, scales)


def status(fn, *args):
    try:
        fn(*args)
        return pi.PI_OK
    except pi.PiError as e:
        msg = str(e)
        for code, name in [(pi.PI_EINVAL, "PI_EINVAL"), (pi.PI_EWORKSPACE, "PI_EWORKSPACE"),
                           (pi.PI_EUNSUPPORTED, "PI_EUNSUPPORTED"), (pi.PI_EHIP, "PI_EHIP")]:
            if name in msg:
                return code
        raise


@pytest.mark.parametrize("B,d,H,N,dt,note", [
    (0, 256, 64, 512, pi.PI_F16, "batch 0"),
    (33, 256, 64, 512, pi.PI_F16, "batch above the maximum"),
    (1, 0, 64, 512, pi.PI_F16, "d = 0"),
    (1, 260, 64, 512, pi.PI_F16, "d not a multiple of 8"),
    (1, 192, 64, 512, pi.PI_I4G128, "int4 with d not a multiple of 128"),
    (1, 256, 64, 512, 7, "unknown dtype"),
])
def test_predict_rejects_bad_arguments(B, d, H, N, dt, note):
    st = status(pi.pi_predict, B, d, H, N, FAKE, mat(dt, scales=FAKE), None, mat(dt, scales=FAKE), None, FAKE,
                FAKE, 1 << 30, 0)
    assert st == pi.PI_EINVAL, note


def test_predict_rejects_short_workspace_and_misaligned_pointers():
    assert status(pi.pi_predict, 1, 256, 64, 512, FAKE, mat(), None, mat(), None, FAKE, FAKE, 16, 0) == pi.PI_EWORKSPACE
    assert status(pi.pi_predict, 1, 256, 64, 512, FAKE + 4, mat(), None, mat(), None, FAKE, FAKE, 1 << 30, 0) == pi.PI_EINVAL
    assert status(pi.pi_predict, 1, 256, 64, 512, FAKE, mat(ptr=FAKE + 8), None, mat(), None, FAKE, FAKE, 1 << 30,
                  0) == pi.PI_EINVAL
    assert status(pi.pi_predict, 1, 256, 64, 512, FAKE, mat(pi.PI_I4G128), None, mat(), None, FAKE, FAKE, 1 << 30,
                  0) == pi.PI_EINVAL    # int4 without scales


def test_sparse_ffn_rejects_bad_arguments():
    args = dict(B=1, d=256, n_g=100, kind=pi.PI_RELU)
    ws = 1 << 30

    def call(B=1, d=256, n_g=100, kind=pi.PI_RELU, W1=None, W2=None, Wup=None, A=FAKE, K=FAKE, wsb=ws):
        return status(pi.pi_sparse_ffn, B, d, n_g, kind, FAKE, W1 or mat(), None, Wup, W2 or mat(), A, K, FAKE, FAKE,
                      wsb, 0)

    assert call(kind=5) == pi.PI_EINVAL
    assert call(kind=pi.PI_GATED_RELU) == pi.PI_EINVAL              # gated without Wup
    assert call(W2=mat(pi.PI_F32)) == pi.PI_EUNSUPPORTED             # mixed dtypes
    assert call(K=None) == pi.PI_EINVAL
    assert call(A=None) == pi.PI_EINVAL
    assert call(n_g=-1) == pi.PI_EINVAL
    assert call(wsb=64) == pi.PI_EWORKSPACE


def test_predict_output_rejects_bad_arguments():
    f = pi.pi_predict_output
    # (B, H, N, h, P2 [H x N], c2, tau, logits, mask, ws, ws_bytes, stream)
    assert status(f, 0, 64, 104, FAKE, mat(), None, 0.0, FAKE, FAKE, None, 0, 0) == pi.PI_EINVAL
    assert status(f, 1, 64, 100, FAKE, mat(), None, 0.0, FAKE, FAKE, None, 0, 0) == pi.PI_EINVAL  # N not /8 (P2 rows)
    assert status(f, 2, 64, 104, FAKE, mat(), None, 0.0, None, FAKE, FAKE, 1 << 30, 0) == pi.PI_EINVAL  # logits, B > 1
    assert status(f, 1, 64, 104, FAKE, mat(), None, 0.0, None, None, None, 0, 0) == pi.PI_EINVAL  # nothing to write
    # batch > 1 sums partials in the workspace
    need = pi.pi_workspace_bytes(pi.PI_OP_PREDICT_OUTPUT, 2, 0, 64, 104)
    assert need >= 2 * 104 * 4
    assert pi.pi_workspace_bytes(pi.PI_OP_PREDICT_OUTPUT, 1, 0, 64, 104) == 0
    assert status(f, 2, 64, 104, FAKE, mat(), None, 0.0, FAKE, None, None, 0, 0) == pi.PI_EWORKSPACE
    assert status(f, 2, 64, 104, FAKE, mat(), None, 0.0, FAKE, None, FAKE, need - 1, 0) == pi.PI_EWORKSPACE


def _layer(d=256, N=1024, H=64, n_g=1024):
    return pi.Layer(d, N, H, n_g, pi.PI_RELU, False, mat(), None, mat(), None, FAKE, mat(), None, None, mat(), None)


def test_ffn_layer_stages_rejects_bad_stage_sets_and_shapes():
    L = _layer()
    ws = 1 << 30

    def call(stages, layer=L, B=1):
        return status(pi.pi_ffn_layer_stages, layer, B, FAKE, 0.0, None, FAKE, None, FAKE, FAKE, None, None, FAKE,
                      stages, None, ws, None, 0)

    assert call(0) == pi.PI_EINVAL
    assert call(pi.PI_STAGE_ALL + 1) == pi.PI_EINVAL
    assert call(64) == pi.PI_EINVAL
    assert call(pi.PI_STAGE_ALL, layer=_layer(N=1020)) == pi.PI_EINVAL     # P2 [H x N] rows need N % 8 == 0
    assert call(pi.PI_STAGE_ALL, layer=_layer(n_g=2048)) == pi.PI_EINVAL   # more GPU neurons than N
    assert call(pi.PI_STAGE_ALL, B=33) == pi.PI_EINVAL
    big = pi.PI_MAX_NEURONS + 8                                          # the lists' LDS bound
    assert call(pi.PI_STAGE_ALL, layer=_layer(N=big, n_g=big)) == pi.PI_EUNSUPPORTED
    assert status(pi.pi_ffn_layer_stages, L, 1, FAKE, 0.0, None, FAKE, None, FAKE, FAKE, None, None, FAKE,
                  pi.PI_STAGE_ALL, None, 64, None, 0) == pi.PI_EWORKSPACE


def test_ffn_layer_ahead_rejects_bad_arguments():
    L = _layer()
    ws = 1 << 30

    X, Y, WS = FAKE, FAKE + (1 << 20), FAKE + (1 << 24)

    def call(next_layer=L, ws_next=WS + 2 * ws, nbytes=ws, layer=L, y=Y):
        return status(pi.pi_ffn_layer_ahead, layer, 1, X, 0.0, None, y, None, FAKE, FAKE, None, None, WS,
                      pi.PI_STAGE_ALL, next_layer, ws_next, ws, nbytes, 0)

    assert call(next_layer=_layer(d=512)) == pi.PI_EINVAL          # another d
    assert call(next_layer=_layer(n_g=2048)) == pi.PI_EINVAL       # more GPU neurons than N
    assert call(ws_next=WS) == pi.PI_EINVAL                        # the same workspace
    assert call(ws_next=WS + 4096) == pi.PI_EINVAL                 # a workspace overlapping the other
    assert call(y=X) == pi.PI_EINVAL and call(y=X + 512) == pi.PI_EINVAL   # y overlapping x (1 KB)
    assert call(ws_next=None) == pi.PI_EWORKSPACE
    assert call(nbytes=64) == pi.PI_EWORKSPACE
    assert call(layer=_layer(N=1020)) == pi.PI_EINVAL              # this layer's own checks still apply


def test_ffn_layer_normed_rejects_bad_arguments():
    L = _layer()
    need = pi.pi_workspace_bytes(pi.PI_OP_FFN_LAYER_NORMED, 1, 256, 64, 1024, 1024)
    assert need >= pi.pi_workspace_bytes(pi.PI_OP_FFN_LAYER, 1, 256, 64, 1024, 1024) + 256 + 256 * 4
    YP, Y, XO, WS = FAKE, FAKE + (1 << 20), FAKE + (2 << 20), FAKE + (1 << 24)

    def call(y_prev=YP, eps=1e-5, y=Y, x_out=XO, nbytes=need, layer=L, B=1, ws=WS):
        return status(pi.pi_ffn_layer_normed, layer, B, y_prev, eps, 0.0, None, y, None, FAKE, FAKE, None, None, ws,
                      x_out, nbytes, 0)

    assert call(y_prev=None) == pi.PI_EINVAL
    assert call(y_prev=YP + 4) == pi.PI_EINVAL                     # unaligned input
    assert call(x_out=XO + 8) == pi.PI_EINVAL                      # unaligned normalised row
    for eps in (-1e-5, float("nan"), float("inf")):
        assert call(eps=eps) == pi.PI_EINVAL
    assert call(B=0) == pi.PI_EINVAL and call(B=pi.PI_MAX_BATCH + 1) == pi.PI_EINVAL
    assert call(x_out=YP + 512) == pi.PI_EINVAL                    # x_out overlapping y_prev (1 KB row)
    assert call(x_out=Y) == pi.PI_EINVAL                           # x_out overlapping y
    assert call(ws=None) == pi.PI_EWORKSPACE
    assert call(ws=WS + 8) == pi.PI_EWORKSPACE                     # unaligned workspace
    assert call(nbytes=need - 16) == pi.PI_EWORKSPACE
    assert call(layer=_layer(N=1020)) == pi.PI_EINVAL              # the layer's own checks still apply


def test_table_prepare_validates_and_builds_bitmap_and_prefix():
    import numpy as np
    N = 200
    T = np.array([1, 5, 64, 65, 130, 199], np.int32)
    buf = pi.pi_table_prepare(N, T)
    W = 2 * ((N + 63) // 64)
    bits = buf[:W * 4].view(np.uint32)
    pre = buf[W * 4:].view(np.int32)
    got = [i for i in range(N) if bits[i // 32] >> (i % 32) & 1]
    assert got == T.tolist()
    assert pre.tolist() == [0, 2, 4, 5]          # GPU-resident ids below each 64-id block
    for bad in ([3, 3], [5, 4], [-1], [200]):
        with pytest.raises(pi.PiError):
            pi.pi_table_prepare(N, np.array(bad, np.int32))
    assert len(pi.pi_table_prepare(N, np.zeros(0, np.int32))) == pi.pi_table_bytes(N)


def test_read_probe_rejects_bad_arguments():
    # (buf, bytes, out, blocks, stream)
    assert status(pi.pi_read_probe, None, 1024, FAKE, 0, 0) == pi.PI_EINVAL
    assert status(pi.pi_read_probe, FAKE, 0, FAKE, 0, 0) == pi.PI_EINVAL
    assert status(pi.pi_read_probe, FAKE, 1000, FAKE, 0, 0) == pi.PI_EINVAL          # not whole 16-byte vectors
    assert status(pi.pi_read_probe, FAKE, 1024, FAKE, 65537, 0) == pi.PI_EINVAL
    assert status(pi.pi_read_probe, FAKE, 1024, None, 0, 0) == pi.PI_EINVAL
    assert status(pi.pi_read_probe, FAKE + 8, 1024, FAKE, 0, 0) == pi.PI_EINVAL      # unaligned
    for depth in (1, 3, 12, 64, -8):
        assert status(pi.pi_read_probe, FAKE, 1024, FAKE, 0, 0, depth) == pi.PI_EINVAL   # unknown depth


def test_layer_norm_rejects_bad_arguments():
    # (B, d, y, x, eps, stream)
    n = 4 * 16
    assert status(pi.pi_layer_norm, 0, 16, FAKE, FAKE, 1e-5, 0) == pi.PI_EINVAL
    assert status(pi.pi_layer_norm, 4, 0, FAKE, FAKE, 1e-5, 0) == pi.PI_EINVAL
    assert status(pi.pi_layer_norm, 1, (1 << 30) + 1, FAKE, FAKE + (1 << 33), 1e-5, 0) == pi.PI_EINVAL
    assert status(pi.pi_layer_norm, 4, 16, None, FAKE, 1e-5, 0) == pi.PI_EINVAL
    assert status(pi.pi_layer_norm, 4, 16, FAKE, None, 1e-5, 0) == pi.PI_EINVAL
    assert status(pi.pi_layer_norm, 4, 16, FAKE, FAKE + 4 * n, -1e-5, 0) == pi.PI_EINVAL
    assert status(pi.pi_layer_norm, 4, 16, FAKE, FAKE + 4 * n, float("nan"), 0) == pi.PI_EINVAL
    assert status(pi.pi_layer_norm, 4, 16, FAKE, FAKE + 4 * n, float("inf"), 0) == pi.PI_EINVAL
    # x overlapping y without being y
    assert status(pi.pi_layer_norm, 4, 16, FAKE, FAKE + 4, 1e-5, 0) == pi.PI_EINVAL
    assert status(pi.pi_layer_norm, 4, 16, FAKE + 4 * (n - 1), FAKE, 1e-5, 0) == pi.PI_EINVAL


def test_compact_and_merge_reject_bad_arguments():
    assert status(pi.pi_compact, 1, 0, FAKE, 0.0, FAKE, 10, FAKE, FAKE, None, 0, None, None, 0) == pi.PI_EINVAL
    assert status(pi.pi_compact, 1, 100, FAKE, 0.0, None, 10, FAKE, FAKE, None, 0, None, None, 0) == pi.PI_EINVAL
    assert status(pi.pi_compact, 1, 100, FAKE, 0.0, FAKE, 10, FAKE, FAKE, FAKE, 5, None, FAKE, 0) == pi.PI_EINVAL
    big = pi.PI_MAX_NEURONS + 1
    assert status(pi.pi_compact, 1, big, FAKE, 0.0, FAKE, 10, FAKE, FAKE, None, 0, None, None, 0) == pi.PI_EUNSUPPORTED
    assert status(pi.pi_merge, 0, 16, FAKE, FAKE, None, None, 0) == pi.PI_EINVAL
    assert status(pi.pi_merge, 1, 16, None, FAKE, None, None, 0) == pi.PI_EINVAL
    # nothing to add: accepted without any launch
    assert status(pi.pi_merge, 1, 16, FAKE, None, None, None, 0) == pi.PI_OK


def test_attn_decode_rejects_bad_arguments():
    def attn(**kw):
        base = dict(d=512, n_heads=8, dh=64, Ha=64, L_max=256)
        base.update(kw)
        m = lambda: pi.Matrix(FAKE, pi.PI_F16)
        return pi.Attn(base["d"], base["n_heads"], base["dh"], base["Ha"], base["L_max"], m(), m(), m(), m(), m(),
                       m(), FAKE, FAKE)
    X, Y, WS = FAKE, FAKE + (1 << 20), FAKE + (1 << 24)
    need = pi.pi_attn_workspace_bytes(attn())
    assert need > 0

    def call(A=None, t=10, x=X, y=Y, nbytes=need, ws=WS):
        return status(pi.pi_attn_decode, A or attn(), t, x, 0.0, y, None, FAKE, FAKE, ws, nbytes, 0)

    assert call(t=-1) == pi.PI_EINVAL and call(t=256) == pi.PI_EINVAL          # outside the cache
    assert call(A=attn(d=500)) == pi.PI_EINVAL                                  # d != n_heads * dh
    assert call(A=attn(dh=32, d=256)) == pi.PI_EUNSUPPORTED
    assert call(A=attn(Ha=2000)) == pi.PI_EUNSUPPORTED and call(A=attn(Ha=6)) == pi.PI_EUNSUPPORTED
    assert call(A=attn(n_heads=80, d=80 * 128, dh=128)) == pi.PI_EUNSUPPORTED  # d above 8192
    assert call(x=X + 4) == pi.PI_EINVAL and call(y=None) == pi.PI_EINVAL
    assert call(y=X + 1024) == pi.PI_EINVAL                                     # y overlapping x
    A = attn()
    A.Wq = pi.Matrix(FAKE, pi.PI_F32)
    assert call(A=A) == pi.PI_EINVAL                                            # fp16 weights only
    A = attn()
    A.bo = pi.Vector(FAKE, pi.PI_F32)
    assert call(A=A) == pi.PI_EINVAL
    A = attn()
    A.Kc = None
    assert call(A=A) == pi.PI_EINVAL
    assert call(nbytes=need - 16) == pi.PI_EWORKSPACE and call(ws=None) == pi.PI_EWORKSPACE
