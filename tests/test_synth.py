"""Checks of the seeded input generator (host side; the device side is
compared bit for bit in the GPU tests)."""
import math

import numpy as np
import pytest

import synth


def test_f16_rounding_matches_numpy():
    g = np.random.default_rng(0)
    vals = np.concatenate([
        g.standard_normal(20000) * 0.01, g.standard_normal(2000) * 1e-6, g.standard_normal(2000) * 1e4,
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, -1e6, 2.0 ** -25, 2.0 ** -24, 3 * 2.0 ** -26,
                  1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 2.0 ** -14 - 2.0 ** -25]),
    ])
    L = synth.host_lib()
    got = np.array([L.sx_f16_bits(float(v)) for v in vals], np.uint16)
    ref = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)
    back = np.array([L.sx_f16_value(int(b)) for b in ref[:500]])
    assert np.array_equal(back, ref[:500].view(np.float16).astype(np.float64))


def test_irwin_hall_values_have_unit_variance_and_bounded_range():
    x = synth.host_x(3, 0, 0, 64, 4096).astype(np.float64)
    assert abs(x.mean()) < 0.01
    assert abs(x.var() - 1.0) < 0.01
    assert np.abs(x).max() <= 2 * math.sqrt(3) + 1e-6
    # excess kurtosis of Irwin-Hall(4) is -6/(5*4) = -0.3
    k = ((x - x.mean()) ** 4).mean() / x.var() ** 2 - 3
    assert abs(k + 0.3) < 0.03


def test_generation_is_deterministic_and_row_addressed():
    a, _ = synth.host_rows(synth.F16, 5, synth.TAG_W1, 2, 256, 0.1, nrows=10)
    b, _ = synth.host_rows(synth.F16, 5, synth.TAG_W1, 2, 256, 0.1, row_ids=np.array([7, 3], np.int32))
    assert np.array_equal(a[7], b[0]) and np.array_equal(a[3], b[1])
    c, _ = synth.host_rows(synth.F16, 5, synth.TAG_W2, 2, 256, 0.1, nrows=10)
    assert not np.array_equal(a, c)


def test_int4_rows_use_the_full_range_and_valid_scales():
    data, sc = synth.host_rows(synth.I4G128, 5, synth.TAG_W1, 0, 512, 1 / math.sqrt(512), nrows=16)
    lo = (data & 0xF).astype(np.int16)
    hi = (data >> 4).astype(np.int16)
    q = np.where(np.concatenate([lo, hi]) >= 8, np.concatenate([lo, hi]) - 16, np.concatenate([lo, hi]))
    assert q.min() >= -8 and q.max() == 7
    s = sc.view(np.float16).astype(np.float64)
    assert np.all(s > 0) and np.all(np.isfinite(s))


def test_density_scale_and_cap():
    c = synth.solve_scale(3072, 0.10, 1.1)
    p = np.minimum(0.95, c * np.arange(1, 3073) ** -1.1)
    assert abs(p.mean() - 0.10) < 1e-9
    assert abs(c - 117.47) < 0.01
    assert int((p >= 0.95).sum()) == 79
    spec = synth.layer_spec(synth.CONFIGS["opt-768"], 0)
    assert abs(spec.p.mean() - 0.1) < 1e-9
    assert sorted(spec.p) == sorted(p)      # permutation of the same ranks


def test_fc1_bias_construction_gives_the_target_activation_frequency():
    cfg = synth.small_config("gen", d=512, N=256, H=64, wdtype=synth.F32, pdtype=synth.F32, bdtype=synth.F32,
                             rho=0.2, seed=21)
    spec = synth.layer_spec(cfg, 0)
    W1, _ = synth.host_rows(synth.F32, cfg.seed, synth.TAG_W1, 0, cfg.d, 1 / math.sqrt(cfg.d), nrows=cfg.N)
    T = 6000
    X, _ = synth.host_rows(synth.F32, 99, synth.TAG_X, 0, cfg.d, 1.0, nrows=T)
    z = X.astype(np.float64) @ W1.astype(np.float64).T + spec.b1.astype(np.float64)
    freq = (z > 0).mean(axis=0)
    sd = np.sqrt(spec.p * (1 - spec.p) / T)
    assert np.all(np.abs(freq - spec.p) <= 4.5 * sd + 0.01)
    assert abs(freq.mean() - 0.2) < 0.01


def test_predictor_calibration_gives_the_target_predicted_frequency():
    cfg = synth.small_config("genp", d=512, N=256, H=128, wdtype=synth.F32, pdtype=synth.F32, bdtype=synth.F32,
                             rho=0.2, seed=22)
    spec = synth.layer_spec(cfg, 0)
    P1, _ = synth.host_rows(synth.F32, cfg.seed, synth.TAG_P1, 0, cfg.d, 1 / math.sqrt(cfg.d), nrows=spec.H)
    P2, _ = synth.host_rows(synth.F32, cfg.seed, synth.TAG_P2, 0, spec.H, 1 / math.sqrt(spec.H), nrows=cfg.N)
    X, _ = synth.host_rows(synth.F32, 98, synth.TAG_X, 0, cfg.d, 1.0, nrows=4000)
    h = np.maximum(X.astype(np.float64) @ P1.astype(np.float64).T, 0)
    logits = h @ P2.astype(np.float64).T + spec.c2.astype(np.float64)
    freq = (logits > 0).mean(axis=0)
    assert abs(freq.mean() - 0.2) < 0.02
    # hotness is preserved: the hottest decile fires far more often than the coldest
    order = np.argsort(-spec.p)
    assert freq[order[:25]].mean() > 0.6 and freq[order[-25:]].mean() < 0.1
    assert np.corrcoef(freq, spec.p)[0, 1] > 0.9


def test_top40_table_from_simulated_profiling():
    spec = synth.layer_spec(synth.CONFIGS["opt-30b"], 0)
    N = spec.N
    assert spec.n_g == int(0.4 * N) == 11468
    assert np.all(np.diff(spec.T_g) > 0) and np.all(np.diff(spec.T_c) > 0)
    assert np.array_equal(np.sort(np.concatenate([spec.T_g, spec.T_c])), np.arange(N))
    # every GPU neuron was profiled at least as often as every CPU neuron
    assert spec.counts[spec.T_g].min() >= spec.counts[spec.T_c].max()
    share = spec.p[spec.T_g].sum() / spec.p.sum()
    assert 0.80 < share < 0.86            # hot neurons carry most activations


def test_int4_quantiser_rule_and_packing():
    """synth.i4_quantize_rows: the scale is fp16(max|w| / 7) per 128 values, each value is
    within half a step of q * s with q in [-8, 7], the even element sits in the low nibble, and
    an all-zero group stores zeros."""
    g = np.random.default_rng(3)
    w = (g.standard_normal((5, 384)) * 0.05).astype(np.float16)
    w[2, 128:256] = 0
    w[4, 7] = np.float16(-0.5)                        # the group's largest magnitude, negative
    packed, scales = synth.i4_quantize_rows(w.view(np.uint16))
    assert packed.shape == (5, 192) and scales.shape == (5, 3)
    s = scales.view(np.float16).astype(np.float64)
    grp = np.abs(w.astype(np.float64)).reshape(5, 3, 128).max(axis=2)
    assert np.array_equal(s, (grp / 7).astype(np.float16).astype(np.float64))
    v = synth.i4_dequant(packed, scales)
    err = np.abs(v - w.astype(np.float64))
    assert np.all(err <= np.repeat(s, 128, axis=1) / 2 * (1 + 1e-6) + 1e-12)
    assert not np.any(v[2, 128:256])
    q0 = int(packed[4, 3] & 0xF)                       # element 6 (even): low nibble
    q1 = int(packed[4, 3] >> 4)                        # element 7 (odd): high nibble, the -0.5
    assert (q1 - 16 if q1 >= 8 else q1) == -7 and v[4, 6] == ((q0 - 16 if q0 >= 8 else q0) * s[4, 0])


def test_extreme_layers_of_the_parity_cases():
    """The full-size parity cases name the layers of smallest and largest density (and predictor
    hidden size) of the stacks whose layers vary; they must still be those layers."""
    from tests.test_parity_gpu import EXTREME_LAYERS
    for key, (lo, hi) in EXTREME_LAYERS.items():
        cfg = synth.CONFIGS[key]
        rho = np.array([cfg.rho(L) for L in range(cfg.n_layers)])
        H = np.array([cfg.hidden(L) for L in range(cfg.n_layers)])
        assert int(rho.argmin()) == lo and int(rho.argmax()) == hi
        assert H[lo] == H.min() and H[hi] == H.max()


def test_attention_head_predictor_is_calibrated():
    """With the calibrated output bias, head h is predicted active for a fraction p_h of seeded
    inputs (the oracle's head logits over 3,000 inputs, within 4.5 binomial deviations)."""
    import oracle as orc
    cfg = synth.ATTN_CONFIGS["attn-small"]
    spec = synth.attn_spec(cfg, 0)
    h = synth.attn_host(spec)
    n = 3000
    X, _ = synth.host_rows(synth.F32, cfg.seed, synth.TAG_XA, 0, cfg.d, 1.0, row0=10_000, nrows=n)
    logits = orc.predict(X, orc.Mat(h["Pa1"], orc.F16, cfg.d), orc.Vec(None, orc.F16),
                         orc.Mat(h["Pa2"], orc.F16, cfg.Ha), orc.Vec(h["ca2"], orc.F16))
    freq = (logits.astype(np.float32) > 0).mean(axis=0)
    sd = np.sqrt(spec.p * (1 - spec.p) / n)
    assert np.all(np.abs(freq - spec.p) <= 4.5 * sd + 0.01), (freq, spec.p)
    assert abs(spec.p.mean() - 0.5) < 1e-12          # half the heads active on average
