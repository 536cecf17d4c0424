"""Pins of the self-attention oracle (or_attn_decode) to things other than itself: the fp16
rounding against numpy's conversion; with every head active, the projections against numpy's
float64 matmul and the attention against torch's scaled_dot_product_attention in float64; the
closed forms of one cached position (the output is the value) and of a zero query (the values'
mean) and of very large scores (the value of the highest score); the additivity of heads (skipped
heads add exactly nothing, no head leaves an empty set but the output bias); the invariance under
a permutation of the cached positions; the head predictor as the FFN predictor's MLP."""
import numpy as np
import pytest

import oracle as orc

F16 = orc.F16


def _f16(a):
    return np.asarray(a, np.float64).astype(np.float16).view(np.uint16)


def _vals(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def _case(seed=0, n_heads=4, d_h=8, Ha=16, t=5, L_max=9, bias=True, q_scale=1.0):
    rng = np.random.default_rng(seed)
    d = n_heads * d_h
    m = lambda r, c, s: _f16(rng.standard_normal((r, c)) * s)
    c = {
        "x": rng.standard_normal(d).astype(np.float32),
        "Pa1": m(Ha, d, d ** -0.5), "ca1": _f16(rng.standard_normal(Ha) * 0.1),
        "Pa2": m(n_heads, Ha, Ha ** -0.5), "ca2": _f16(rng.standard_normal(n_heads) * 0.3),
        "Wq": m(d, d, q_scale * d ** -0.5), "Wk": m(d, d, d ** -0.5), "Wv": m(d, d, d ** -0.5),
        "WoT": m(d, d, d ** -0.5),
        "Kc": _f16(rng.standard_normal((n_heads, L_max, d_h))), "Vc": _f16(rng.standard_normal((n_heads, L_max, d_h))),
        "n_heads": n_heads, "d_h": d_h, "t": t, "d": d,
    }
    for b in ("bq", "bk", "bv", "bo"):
        c[b] = _f16(rng.standard_normal(d) * 0.1) if bias else None
    return c


def _run(c, tau=0.0, **over):
    c = {**c, **over}
    d = c["d"]
    M = lambda k, cols: orc.Mat(c[k], F16, cols)
    V = lambda k: orc.Vec(c[k], F16) if c[k] is not None else orc.Vec(None, F16)
    return orc.attn_decode(c["x"], M("Pa1", d), V("ca1"), M("Pa2", c["Pa1"].shape[0]), V("ca2"), tau,
                           M("Wq", d), V("bq"), M("Wk", d), V("bk"), M("Wv", d), V("bv"), M("WoT", d), V("bo"),
                           c["Kc"], c["Vc"], c["n_heads"], c["d_h"], c["t"])


def _proj(c, W, b):
    v = _vals(c[W]) @ c["x"].astype(np.float64)
    return v + (_vals(c[b]) if c[b] is not None else 0.0)


def test_f16_rounding_matches_numpy():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 5, 20000),
                        [0.0, -0.0, 65504.0, 65519.99, 65520.0, 70000.0, -65520.0, 2 ** -24, 2 ** -25,
                         3 * 2 ** -26, 2 ** -14, 2 ** -14 - 2 ** -25, 1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11,
                         np.inf, -np.inf]])
    # the halfway points between consecutive fp16 values (ties go to the even neighbour)
    h = np.arange(0, 0x7bff, 37, dtype=np.uint16)
    v = np.concatenate([v, (_vals(h) + _vals(h + 1)) / 2])
    got = np.array([orc.double_to_f16(float(a)) for a in v], np.uint16)
    assert np.array_equal(got, v.astype(np.float16).view(np.uint16))


def test_all_heads_active_match_numpy_and_torch_sdpa():
    torch = pytest.importorskip("torch")
    c = _case(seed=3)
    r = _run(c, tau=-3.0e38)
    nh, dh, t, d = c["n_heads"], c["d_h"], c["t"], c["d"]
    assert np.array_equal(r["heads"], np.arange(nh))
    k = _proj(c, "Wk", "bk")
    v = _proj(c, "Wv", "bv")
    assert np.array_equal(r["k_new"], _f16(k)) and np.array_equal(r["v_new"], _f16(v))
    q = _proj(c, "Wq", "bq").reshape(nh, dh)
    K = _vals(c["Kc"])[:, :t + 1].copy()
    Vv = _vals(c["Vc"])[:, :t + 1].copy()
    K[:, t] = _vals(_f16(k)).reshape(nh, dh)
    Vv[:, t] = _vals(_f16(v)).reshape(nh, dh)
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, None, :], torch.from_numpy(K), torch.from_numpy(Vv))[:, 0, :].numpy()
    y = _vals(c["WoT"]).T @ o.reshape(d) + _vals(c["bo"])
    assert np.max(np.abs(r["y"] - y)) <= 1e-12 * max(1.0, np.max(np.abs(y)))


def test_one_cached_position_gives_the_value():
    c = _case(seed=4, t=0)
    r = _run(c, tau=-3.0e38)
    o = _vals(r["v_new"])                      # softmax over one position is 1
    y = _vals(c["WoT"]).T @ o + _vals(c["bo"])
    assert np.max(np.abs(r["y"] - y)) <= 1e-12 * np.max(np.abs(y))


def test_zero_query_averages_the_values():
    c = _case(seed=5, t=6)
    c["Wq"] = np.zeros_like(c["Wq"])
    c["bq"] = None
    r = _run(c, tau=-3.0e38)
    nh, dh, t = c["n_heads"], c["d_h"], c["t"]
    Vv = _vals(c["Vc"])[:, :t + 1].copy()
    Vv[:, t] = _vals(r["v_new"]).reshape(nh, dh)
    o = Vv.mean(axis=1).reshape(-1)
    y = _vals(c["WoT"]).T @ o + _vals(c["bo"])
    assert np.max(np.abs(r["y"] - y)) <= 1e-12 * np.max(np.abs(y))


def test_large_scores_pick_the_highest_position():
    c = _case(seed=6, t=7, q_scale=2000.0)
    r = _run(c, tau=-3.0e38)
    assert np.all(np.isfinite(r["y"]))
    nh, dh, t = c["n_heads"], c["d_h"], c["t"]
    q = _proj(c, "Wq", "bq").reshape(nh, dh)
    K = _vals(c["Kc"])[:, :t + 1].copy()
    Vv = _vals(c["Vc"])[:, :t + 1].copy()
    K[:, t] = _vals(r["k_new"]).reshape(nh, dh)
    Vv[:, t] = _vals(r["v_new"]).reshape(nh, dh)
    e = np.einsum("hd,hjd->hj", q, K) / np.sqrt(dh)
    srt = np.sort(e, axis=1)
    assert np.all(srt[:, -1] - srt[:, -2] > 50.0)      # the weight of every other position is below e^-50
    o = Vv[np.arange(nh), np.argmax(e, axis=1)].reshape(-1)
    y = _vals(c["WoT"]).T @ o + _vals(c["bo"])
    assert np.max(np.abs(r["y"] - y)) <= 1e-9 * np.max(np.abs(y))


def test_heads_add_independently_and_skipped_heads_add_nothing():
    c = _case(seed=7, n_heads=6)
    nh = c["n_heads"]

    def with_heads(S):
        ca2 = np.where(np.isin(np.arange(nh), S), 30000.0, -30000.0)    # fp16 sentinels: the set S is active
        r = _run(c, tau=0.0, ca2=_f16(ca2))
        assert np.array_equal(r["heads"], np.sort(np.asarray(S, np.int32)))
        return r["y"] - _vals(c["bo"])
    none = with_heads([])
    assert np.array_equal(none, np.zeros_like(none))                     # only the output bias is left
    S1, S2 = [0, 3], [1, 4, 5]
    both = with_heads(S1 + S2)
    assert np.max(np.abs(both - (with_heads(S1) + with_heads(S2)))) <= 1e-12 * np.max(np.abs(both))
    # the cache entry does not depend on the prediction
    r0 = _run(c, tau=3.0e38)
    r1 = _run(c, tau=-3.0e38)
    assert np.array_equal(r0["k_new"], r1["k_new"]) and np.array_equal(r0["v_new"], r1["v_new"])


def test_permuting_the_cached_positions_changes_nothing():
    c = _case(seed=8, t=8, L_max=12)
    r = _run(c, tau=-3.0e38)
    perm = np.random.default_rng(9).permutation(c["t"])
    Kp, Vp = c["Kc"].copy(), c["Vc"].copy()
    Kp[:, :c["t"]] = c["Kc"][:, perm]
    Vp[:, :c["t"]] = c["Vc"][:, perm]
    rp = _run(c, tau=-3.0e38, Kc=Kp, Vc=Vp)
    assert np.max(np.abs(rp["y"] - r["y"])) <= 1e-12 * np.max(np.abs(r["y"]))
    # positions past t are never read
    Kz = c["Kc"].copy()
    Kz[:, c["t"]:] = 0x7e00                                              # NaN
    assert np.array_equal(_run(c, tau=-3.0e38, Kc=Kz)["y"], r["y"])


def test_head_logits_are_the_predictor_mlp_and_decide_in_fp32():
    c = _case(seed=10, n_heads=8)
    r = _run(c, tau=0.05)
    logits_ffn, _ = orc.predict(c["x"][None, :], orc.Mat(c["Pa1"], F16, c["d"]), orc.Vec(c["ca1"], F16),
                                orc.Mat(c["Pa2"], F16, c["Pa1"].shape[0]), orc.Vec(c["ca2"], F16), return_hidden=True)
    assert np.array_equal(r["head_logits"], logits_ffn[0])
    assert np.array_equal(r["heads"], np.flatnonzero(r["head_logits"].astype(np.float32) > np.float32(0.05)))
