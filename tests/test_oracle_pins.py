"""Pins of the CPU oracle against facts the pages and plain mathematics fix.

Each test below checks the oracle against something other than its own
formula: hand-derived values (tests/golden), numpy float64 computations done
a different way, invariants that follow from the ReLU gate and from the
two-table split, and brute force over every mask of a tiny layer.
"""
import ctypes as C
import json
import os

import numpy as np
import pytest

import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def f32mat(a):
    a = np.asarray(a, np.float32)
    return orc.Mat(a, orc.F32, a.shape[1])


def f32vec(v):
    return orc.Vec(np.asarray(v, np.float32), orc.F32)


def rand_layer(d, N, scale=1.0, seed=0):
    g = np.random.default_rng(seed)
    W1 = (g.standard_normal((N, d)) * scale / np.sqrt(d)).astype(np.float32)
    b1 = (g.standard_normal(N) * 0.5).astype(np.float32)
    W2 = (g.standard_normal((N, d)) / np.sqrt(N)).astype(np.float32)
    x = g.standard_normal((3, d)).astype(np.float32)
    return x, W1, b1, W2


def numpy_ffn(x, W1, b1, W2, rows=None):
    """FFN computed with numpy float64 matrix products (independent of the oracle's loops)."""
    x64, W1_64, W2_64 = x.astype(np.float64), W1.astype(np.float64), W2.astype(np.float64)
    z = x64 @ W1_64.T + b1.astype(np.float64)
    a = np.maximum(z, 0.0)
    if rows is not None:
        m = np.zeros(W1.shape[0])
        m[rows] = 1.0
        a = a * m
    return a @ W2_64


# --------------------------------------------------------------------------- closed forms

def test_f16_widening_matches_numpy_for_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    L = orc.lib()
    got = np.array([L.or_f16_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_int4_nibble_order_sign_and_scale_by_hand():
    # one row of 128 int4 elements; byte 0 = 0x8F: element 0 (low nibble) = 0xF -> -1,
    # element 1 (high nibble) = 0x8 -> -8; byte 1 = 0x71: element 2 = 1, element 3 = 7.
    packed = np.zeros((1, 64), np.uint8)
    packed[0, 0] = 0x8F
    packed[0, 1] = 0x71
    scale = np.array([[0x3800]], np.uint16)  # fp16 0.5
    m = orc.Mat(packed, orc.I4G128, 128, scale)
    L = orc.lib()
    L.or_mat_at.restype = C.c_double
    L.or_mat_at.argtypes = [orc._OrMat, C.c_int64, C.c_int64]
    cm = m._c()
    vals = [L.or_mat_at(cm, 0, k) for k in range(5)]
    assert vals == [-0.5, -4.0, 0.5, 3.5, 0.0]


def test_dense_ffn_hand_example():
    g = load("hand_ffn.json")
    x = np.array([g["x"]], np.float32)
    y = orc.dense_ffn(x, f32mat(g["W1"]), f32vec(g["b1"]), f32mat(g["W2"]))
    assert y[0].tolist() == g["y"]
    y2, a = orc.sparse_ffn(x, f32mat(g["W1"]), f32vec(g["b1"]), f32mat(g["W2"]), np.arange(3), return_act=True)
    assert a[0].tolist() == g["a"] and y2[0].tolist() == g["y"]


def test_predictor_hand_example():
    g = load("hand_predictor.json")
    x = np.array([g["x"]], np.float32)
    logits, h = orc.predict(x, f32mat(g["P1"]), f32vec(g["c1"]), f32mat(g["P2"]), f32vec(g["c2"]), return_hidden=True)
    assert h[0].tolist() == g["h"]
    assert logits[0].tolist() == g["logits"]


def test_predictor_matches_numpy_mlp():
    g = np.random.default_rng(7)
    d, H, N = 24, 16, 40
    P1 = g.standard_normal((H, d)).astype(np.float32)
    c1 = g.standard_normal(H).astype(np.float32)
    P2 = g.standard_normal((N, H)).astype(np.float32)
    c2 = g.standard_normal(N).astype(np.float32)
    x = g.standard_normal((4, d)).astype(np.float32)
    logits = orc.predict(x, f32mat(P1), f32vec(c1), f32mat(P2), f32vec(c2))
    h = np.maximum(x.astype(np.float64) @ P1.astype(np.float64).T + c1, 0)
    ref = h @ P2.astype(np.float64).T + c2
    assert np.allclose(logits, ref, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------- worked example

def test_worked_example_gpu_cpu_partition():
    g = load("worked_example.json")
    N = g["N"]
    T_g = np.array(g["gpu_table"], np.int32)
    T_c = np.array(g["cpu_table"], np.int32)
    logits = -np.ones((1, N))
    logits[0, g["predicted_active"]] = 1.0
    A_g, A_c = orc.compact(logits, 0.0, T_g, T_c)
    assert A_g.tolist() == g["expected_gpu_slots"]
    assert T_g[A_g].tolist() == g["expected_gpu_ids"]
    assert A_c.tolist() == g["expected_cpu_slots"]
    assert T_c[A_c].tolist() == g["expected_cpu_ids"]
    assert not set(g["skipped_hot"]) & set(T_g[A_g].tolist())
    # the merged result equals the FFN restricted to the predicted neurons
    x, W1, b1, W2 = rand_layer(6, N, seed=3)
    b1[:] = 1.0  # every neuron would fire, so only the prediction decides
    yg = orc.sparse_ffn(x, f32mat(W1), f32vec(b1), f32mat(W2), T_g[A_g])
    yc = orc.sparse_ffn(x, f32mat(W1), f32vec(b1), f32mat(W2), T_c[A_c])
    y = orc.merge(yg, yc, len(A_c))
    ref = numpy_ffn(x, W1, b1, W2, rows=g["predicted_active"])
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------- invariants

def test_all_active_mask_equals_dense_and_numpy():
    x, W1, b1, W2 = rand_layer(32, 96, seed=1)
    dense = orc.dense_ffn(x, f32mat(W1), f32vec(b1), f32mat(W2))
    logits = np.zeros((3, 96))
    A, _ = orc.compact(logits, -np.inf, np.arange(96, dtype=np.int32))
    assert len(A) == 96
    sparse = orc.sparse_ffn(x, f32mat(W1), f32vec(b1), f32mat(W2), A)
    assert np.array_equal(sparse, dense)
    assert np.allclose(dense, numpy_ffn(x, W1, b1, W2), rtol=1e-12, atol=1e-12)


def test_relu_gate_superset_masks_give_the_dense_result():
    x, W1, b1, W2 = rand_layer(32, 128, seed=2)
    z = x[:1].astype(np.float64) @ W1.astype(np.float64).T + b1
    true_active = np.flatnonzero(z[0] > 0)
    assert 0 < len(true_active) < 128
    dense = orc.dense_ffn(x[:1], f32mat(W1), f32vec(b1), f32mat(W2))
    g = np.random.default_rng(5)
    extra = np.flatnonzero(g.random(128) < 0.3)
    superset = np.union1d(true_active, extra).astype(np.int32)
    y_sup = orc.sparse_ffn(x[:1], f32mat(W1), f32vec(b1), f32mat(W2), superset)
    y_true = orc.sparse_ffn(x[:1], f32mat(W1), f32vec(b1), f32mat(W2), true_active.astype(np.int32))
    assert np.array_equal(y_sup, y_true)        # the ReLU-zero neurons add exactly nothing
    assert np.allclose(y_sup, dense, rtol=1e-12, atol=1e-13)
    # dropping one truly active neuron changes the result
    y_drop = orc.sparse_ffn(x[:1], f32mat(W1), f32vec(b1), f32mat(W2), true_active[1:].astype(np.int32))
    assert not np.allclose(y_drop, dense, rtol=1e-9, atol=0)


def test_two_table_split_is_additive_and_tables_are_a_permutation():
    N, d = 200, 16
    x, W1, b1, W2 = rand_layer(d, N, seed=4)
    g = np.random.default_rng(9)
    T_g = np.sort(g.choice(N, 80, replace=False)).astype(np.int32)
    T_c = np.setdiff1d(np.arange(N), T_g).astype(np.int32)
    assert np.array_equal(np.sort(np.concatenate([T_g, T_c])), np.arange(N))
    logits = g.standard_normal((2, N))
    A_g, A_c = orc.compact(logits, 0.3, T_g, T_c)
    M = np.flatnonzero((logits.astype(np.float32) > np.float32(0.3)).any(axis=0))
    assert np.array_equal(np.sort(np.concatenate([T_g[A_g], T_c[A_c]])), M)
    # GPU-resident storage: rows in slot order; the tables map slots back to ids
    W1g, b1g, W2g = W1[T_g], b1[T_g], W2[T_g]
    W1c, b1c, W2c = W1[T_c], b1[T_c], W2[T_c]
    yg = orc.sparse_ffn(x, f32mat(W1g), f32vec(b1g), f32mat(W2g), A_g)
    yc = orc.sparse_ffn(x, f32mat(W1c), f32vec(b1c), f32mat(W2c), A_c)
    y = orc.merge(yg, yc, len(A_c))
    ref = numpy_ffn(x, W1, b1, W2, rows=M)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-13)
    # permuting the stored neuron order leaves the result unchanged
    perm = g.permutation(N).astype(np.int32)
    inv = np.argsort(perm).astype(np.int32)
    y_perm = orc.sparse_ffn(x, f32mat(W1[perm]), f32vec(b1[perm]), f32mat(W2[perm]), inv[M])
    assert np.allclose(y_perm, ref, rtol=1e-12, atol=1e-13)


def test_compaction_is_flatnonzero_of_the_union_mask():
    g = np.random.default_rng(11)
    N = 300
    logits = g.standard_normal((3, N))
    T_g = np.sort(g.choice(N, 170, replace=False)).astype(np.int32)
    A, _ = orc.compact(logits, 0.5, T_g)
    M = (logits.astype(np.float32) > np.float32(0.5)).any(axis=0)
    assert np.array_equal(A, np.flatnonzero(M[T_g]))
    assert np.all(np.diff(A) > 0)
    # batch union: a neuron active in only one row is in the list
    only_row2 = np.flatnonzero((logits[2] > 0.5) & ~(logits[:2] > 0.5).any(axis=0))
    assert len(only_row2) and set(only_row2) & set(T_g[A]) == set(only_row2) & set(T_g)


def test_threshold_is_strict_and_decided_in_fp32():
    T = np.arange(4, dtype=np.int32)
    logits = np.array([[0.0, 1e-9, -1e-9, 1.0 + 1e-12]])
    A, _ = orc.compact(logits, 0.0, T)
    assert A.tolist() == [1, 3]          # 0.0 > 0 is false; 1e-9 is positive in fp32
    A1, _ = orc.compact(logits, 1.0, T)
    assert A1.tolist() == []             # 1 + 1e-12 rounds to 1.0 in fp32: not above 1.0


def test_brute_force_every_mask_of_a_tiny_layer():
    d, N = 4, 6
    x, W1, b1, W2 = rand_layer(d, N, seed=6)
    x = x[:2]
    z = x.astype(np.float64) @ W1.astype(np.float64).T + b1
    for mask in range(1 << N):
        rows = np.array([i for i in range(N) if mask >> i & 1], np.int32)
        y = orc.sparse_ffn(x, f32mat(W1), f32vec(b1), f32mat(W2), rows)
        ref = np.zeros((2, d))
        for b in range(2):
            for i in rows:
                if z[b, i] > 0:
                    ref[b] += z[b, i] * W2[i].astype(np.float64)
        assert np.allclose(y, ref, rtol=1e-12, atol=1e-14), mask
        W2z = W2.copy()
        W2z[[i for i in range(N) if not mask >> i & 1]] = 0
        yd = orc.dense_ffn(x, f32mat(W1), f32vec(b1), f32mat(W2z))
        assert np.allclose(y, yd, rtol=1e-12, atol=1e-14), mask


def test_empty_mask_gives_zero_and_merge_skips_cold_partial():
    x, W1, b1, W2 = rand_layer(8, 10, seed=8)
    y = orc.sparse_ffn(x, f32mat(W1), f32vec(b1), f32mat(W2), np.zeros(0, np.int32))
    assert np.array_equal(y, np.zeros_like(y))
    yc = np.ones_like(y)
    assert np.array_equal(orc.merge(y, yc, 0), y)            # no active cold neuron: skipped
    assert np.array_equal(orc.merge(y, yc, 3), yc)
    b2 = np.arange(8, dtype=np.float32)
    assert np.array_equal(orc.merge(y, yc, 0, orc.Vec(b2, orc.F32)), np.tile(b2.astype(np.float64), (3, 1)))


def test_gated_ffn_matches_numpy():
    g = np.random.default_rng(12)
    d, N = 16, 48
    Wg = g.standard_normal((N, d)).astype(np.float32)
    Wu = g.standard_normal((N, d)).astype(np.float32)
    W2 = g.standard_normal((N, d)).astype(np.float32)
    bg = g.standard_normal(N).astype(np.float32)
    x = g.standard_normal((2, d)).astype(np.float32)
    rows = np.flatnonzero(g.random(N) < 0.5).astype(np.int32)
    y = orc.sparse_ffn(x, f32mat(Wg), f32vec(bg), f32mat(W2), rows, kind=orc.GATED_RELU, Wup=f32mat(Wu))
    x64 = x.astype(np.float64)
    a = np.maximum(x64 @ Wg.astype(np.float64).T + bg, 0) * (x64 @ Wu.astype(np.float64).T)
    ref = a[:, rows] @ W2.astype(np.float64)[rows]
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)
    # a negative gate kills the neuron even when the up projection is large
    assert np.all(a[x64 @ Wg.astype(np.float64).T + bg <= 0] == 0)


def test_fp16_and_int4_weights_are_widened_exactly():
    g = np.random.default_rng(13)
    d, N = 256, 20
    W1 = (g.standard_normal((N, d)) / 16).astype(np.float16)
    W2 = (g.standard_normal((N, d)) / 4).astype(np.float16)
    b1 = (g.standard_normal(N) * 0.1).astype(np.float16)
    x = g.standard_normal((2, d)).astype(np.float32)
    m1 = orc.Mat(W1.view(np.uint16), orc.F16, d)
    m2 = orc.Mat(W2.view(np.uint16), orc.F16, d)
    y = orc.dense_ffn(x, m1, orc.Vec(b1.view(np.uint16), orc.F16), m2)
    ref = numpy_ffn(x, W1.astype(np.float32), b1.astype(np.float32), W2.astype(np.float32))
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-13)
    # int4, group 128: numpy dequantisation from the packed nibbles
    q = g.integers(-8, 8, size=(N, d))
    nib = (q & 0xF).astype(np.uint8)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    sc = (g.random((N, d // 128)) * 0.02 + 0.001).astype(np.float16)
    Wdq = q * np.repeat(sc.astype(np.float64), 128, axis=1)
    mq = orc.Mat(packed, orc.I4G128, d, sc.view(np.uint16))
    y4 = orc.dense_ffn(x, mq, orc.Vec(b1.view(np.uint16), orc.F16), mq)
    z = x.astype(np.float64) @ Wdq.T + b1.astype(np.float64)
    ref4 = np.maximum(z, 0) @ Wdq
    assert np.allclose(y4, ref4, rtol=1e-12, atol=1e-13)


# ---- chained layers: the normalisation between one layer's output and the next layer's input ----
# (not on the pages; reading: layer normalisation with unit gain and zero bias)

def test_layer_norm_hand_example():
    # mean 2.5, population variance (2.25 + 0.25 + 0.25 + 2.25) / 4 = 1.25
    y = np.array([[1.0, 2.0, 3.0, 4.0]], np.float32)
    x = orc.layer_norm(y, 0.0)
    assert np.allclose(x, np.array([[-1.5, -0.5, 0.5, 1.5]]) / np.sqrt(1.25), rtol=0, atol=1e-15)
    # eps enters under the root: y = (-1, 1) has variance 1
    x = orc.layer_norm(np.array([[-1.0, 1.0]], np.float32), 0.25)
    assert np.allclose(x, [[-1.0 / np.sqrt(1.25), 1.0 / np.sqrt(1.25)]], rtol=0, atol=1e-15)


def test_layer_norm_invariants():
    rng = np.random.default_rng(41)
    y = rng.standard_normal((5, 96)).astype(np.float32) * 3.0 + 0.7
    x = orc.layer_norm(y, 0.0)
    # zero mean and unit population variance per row (a sample variance would give (d-1)/d)
    assert np.allclose(x.mean(axis=1), 0.0, atol=1e-13)
    assert np.allclose((x * x).mean(axis=1), 1.0, rtol=0, atol=1e-12)
    # invariant under a positive scale and a shift of each row (exact in fp32: powers of two)
    y2 = (y * np.float32(4.0) + np.float32(-8.0)).astype(np.float32)
    assert np.allclose(orc.layer_norm(y2, 0.0), x, rtol=0, atol=1e-5)
    # rows are independent
    assert np.array_equal(orc.layer_norm(y[2:3], 0.0), x[2:3])
    # a constant row gives zeros (eps > 0)
    c = np.full((1, 33), 3.25, np.float32)
    assert np.array_equal(orc.layer_norm(c, 1e-5), np.zeros((1, 33)))


def test_layer_norm_matches_torch_functional():
    import torch
    rng = np.random.default_rng(42)
    y = (rng.standard_normal((3, 7168)) * 0.05).astype(np.float32)
    want = torch.nn.functional.layer_norm(torch.from_numpy(y).double(), (7168,), eps=1e-5).numpy()
    assert np.allclose(orc.layer_norm(y, 1e-5), want, rtol=0, atol=1e-12)
