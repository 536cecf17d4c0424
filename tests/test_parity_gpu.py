"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Sizes: reduced shapes that the oracle finishes in seconds yet span several
tiles and ragged tails, then one layer of each full-size workload (the oracle
handles one layer, with rows generated only for the neurons it needs).
"""
import sys

import numpy as np
import pytest

import synth
from tests import parity_harness as ph

pytestmark = pytest.mark.gpu


def _dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _run(cfg, **kw):
    print(f"[parity] cfg={cfg.key} d={cfg.d} N={cfg.N} kw={kw}", flush=True)
    r = ph.run_layer_parity(cfg, **kw)
    print(f"[parity]   -> {r}", flush=True)
    ph.assert_report(r)
    return r


# --------------------------------------------------------------------------- generator identity

@pytest.mark.parametrize("dtype,cols", [(synth.F32, 264), (synth.F16, 520), (synth.I4G128, 384)])
def test_device_generator_matches_host_bits(dtype, cols):
    torch = _dev()
    rows = np.array([5, 0, 77, 1023, 4], np.int32)
    host, hs = synth.host_rows(dtype, 9, synth.TAG_W1, 3, cols, 0.05, row_ids=rows)
    m = ph.dev_matrix(len(rows), cols, dtype, "cuda:0")
    ph.fill_matrix(m, dtype, 9, synth.TAG_W1, 3, cols, 0.05, torch.from_numpy(rows).cuda())
    torch.cuda.synchronize()
    dev = m.data.cpu().numpy()
    if dtype == synth.F16:
        dev = dev.view(np.uint16)
    assert np.array_equal(dev.view(np.uint8), host.view(np.uint8))
    if hs is not None:
        assert np.array_equal(m.scales.cpu().numpy().view(np.uint16), hs)


def test_device_int4_quantiser_matches_host_bits():
    """The hidden-major int4 predictor weights: the device quantiser gives the host's bits."""
    torch = _dev()
    from synth.device import i4_quantize_rows_dev
    v16, _ = synth.host_rows(synth.F16, 4, synth.TAG_P2, 2, 640, 1 / np.sqrt(640), nrows=96)
    v16[3, :128] = 0                                     # an all-zero group
    m = i4_quantize_rows_dev(torch.from_numpy(v16.view(np.float16)).cuda())
    packed, scales = synth.i4_quantize_rows(v16)
    assert np.array_equal(m.data.cpu().numpy(), packed)
    assert np.array_equal(m.scales.cpu().numpy().view(np.uint16), scales)


# --------------------------------------------------------------------------- reduced shapes

SMALL = [
    ph.small_case("f16-ragged", d=264, N=1000, H=72, wdtype=synth.F16),        # ragged tiles, N not /64
    ph.small_case("f32", d=768, N=3072, H=128, wdtype=synth.F32, seed=12),
    ph.small_case("f16", d=1024, N=4096, H=256, wdtype=synth.F16, seed=13),
    ph.small_case("i4", d=1024, N=2048, H=128, wdtype=synth.I4G128, seed=14),
    ph.small_case("gated", d=512, N=1536, H=128, wdtype=synth.F16, gated=True, rho=0.15, seed=15),
    ph.small_case("gated-i4", d=640, N=1280, H=64, wdtype=synth.I4G128, gated=True, seed=16),
    ph.small_case("cold40", d=512, N=2048, H=128, wdtype=synth.F16, gpu_frac=0.4, seed=17),
    ph.small_case("i4pred", d=768, N=2560, H=192, wdtype=synth.F16, pdtype=synth.I4G128, gpu_frac=0.4, seed=18),
]


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
@pytest.mark.parametrize("cfg", SMALL, ids=[c.key for c in SMALL])
@pytest.mark.parametrize("B", [1, 3, 8])
def test_small_layer_parity(cfg, B, fused):
    _dev()
    _run(cfg, layer=0, step=1, B=B, fused=fused)


# rows past the register-held x of the batch-1 hidden-layer kernel: the LDS-x kernel at each of its
# vector counts (24, 32, 24 and 8 vectors per lane), with row counts that leave its last workgroup
# part empty
WIDE = [
    ph.small_case("wide-f16", d=8264, N=1024, H=37, wdtype=synth.F16, seed=21),
    ph.small_case("wide-f16-32", d=16384, N=640, H=20, wdtype=synth.F16, seed=22),
    ph.small_case("wide-f32", d=4104, N=768, H=24, wdtype=synth.F32, seed=23),
    ph.small_case("wide-i4pred", d=8320, N=1024, H=40, wdtype=synth.F16, pdtype=synth.I4G128, seed=24),
]


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
@pytest.mark.parametrize("cfg", WIDE, ids=[c.key for c in WIDE])
def test_wide_row_hidden_layer_parity(cfg, fused):
    _dev()
    _run(cfg, layer=0, step=1, B=1, fused=fused)


# rows of the fused kernel's FC1 and of the hidden-layer kernel at 10, 12 and 14 vectors per lane
# (fp16 rows of 640, 704 / 768 and 832 vectors, fp32 rows of 640, 768 and 896), gated and not
FC1_WIDTHS = [
    ph.small_case("nv10-f16-gated", d=5120, N=1024, H=40, wdtype=synth.F16, gated=True, rho=0.15, seed=31),
    ph.small_case("nv12-f16", d=5632, N=1088, H=48, wdtype=synth.F16, seed=32),
    ph.small_case("nv12-f16-gated", d=6144, N=960, H=36, wdtype=synth.F16, gated=True, seed=33),
    ph.small_case("nv14-f16", d=6656, N=1024, H=44, wdtype=synth.F16, seed=35),
    ph.small_case("nv10-f32", d=2560, N=1024, H=40, wdtype=synth.F32, seed=34),
    ph.small_case("nv12-f32", d=3072, N=1024, H=40, wdtype=synth.F32, seed=36),
    ph.small_case("nv14-f32", d=3584, N=1024, H=40, wdtype=synth.F32, seed=37),
]


@pytest.mark.parametrize("cfg", FC1_WIDTHS, ids=[c.key for c in FC1_WIDTHS])
def test_fused_fc1_row_widths(cfg):
    _dev()
    _run(cfg, layer=0, step=1, B=1, fused=True)


# int4 P2 tiles are placed die by die for the first (tiles / 8) * 8 of them and in order after: 42
# tiles leave 2 in that tail, 6 tiles (fewer than the dies) keep their order
I4_TILE_ORDER = [
    ph.small_case("i4p-42-tiles", d=512, N=2688, H=96, wdtype=synth.F16, pdtype=synth.I4G128, seed=38),
    ph.small_case("i4p-6-tiles", d=512, N=384, H=64, wdtype=synth.F16, pdtype=synth.I4G128, seed=39),
]


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
@pytest.mark.parametrize("cfg", I4_TILE_ORDER, ids=[c.key for c in I4_TILE_ORDER])
def test_int4_predictor_tile_order(cfg, fused):
    _dev()
    _run(cfg, layer=0, step=1, B=1, fused=fused)


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
@pytest.mark.parametrize("B", [16, 32])
def test_large_batch_union(B, fused):
    _dev()
    r = _run(SMALL[6], layer=0, step=2, B=B, fused=fused)
    assert r["K"] > 0


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
@pytest.mark.parametrize("B", [1, 2])
def test_all_active_list_is_the_whole_table(B, fused):
    _dev()
    cfg = SMALL[2]
    r = _run(cfg, layer=0, step=0, B=B, tau_all_active=True, fused=fused)
    assert r["K"] == cfg.N


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
def test_empty_list_gives_zero_output(fused):
    _dev()
    r = _run(SMALL[6], layer=0, step=0, B=1, tau=1e30, fused=fused)
    assert r["K"] == 0 and r["K_c"] == 0 and r["y_norm"] == 0.0


@pytest.mark.parametrize("B", [1, 4])
def test_fused_and_separate_paths_agree(B):
    """Same logits bits and lists; outputs agree to the parity tolerance (the FC2 chunking differs)."""
    torch = _dev()
    for cfg in (SMALL[2], SMALL[6], SMALL[4]):
        spec = synth.layer_spec(cfg, 0)
        dl = ph.DeviceLayer(spec)
        outs = []
        for fused in (False, True):
            buf = ph.DeviceBuffers(cfg, spec.H, spec.n_g, len(spec.T_c), B)
            buf.x.copy_(torch.from_numpy(synth.host_x(cfg.seed, 0, 9, B, cfg.d)))
            ph._gpu_stages(dl, buf, B, 0.0, True, fused)
            torch.cuda.synchronize()
            K = int(buf.K.cpu()[0])
            Kc = int(buf.K_c.cpu()[0]) if len(spec.T_c) else 0
            outs.append((K, buf.A_g.cpu().numpy()[:K].tobytes(), Kc, buf.A_c.cpu().numpy()[:Kc].tobytes(),
                         buf.logits.cpu().numpy().tobytes(), buf.y.cpu().numpy().astype(np.float64)))
        assert outs[0][:5] == outs[1][:5], cfg.key
        assert ph.rel_err(outs[1][5], outs[0][5]) <= 1e-5, cfg.key


def test_outputs_are_bitwise_repeatable():
    torch = _dev()
    cfg = SMALL[3]
    spec = synth.layer_spec(cfg, 0)
    dl = ph.DeviceLayer(spec)
    outs = []
    for _ in range(3):
        buf = ph.DeviceBuffers(cfg, spec.H, spec.n_g, 0, 4)
        buf.x.copy_(torch.from_numpy(synth.host_x(cfg.seed, 0, 5, 4, cfg.d)))
        ph.run_gpu_layer(dl, buf, 4)
        torch.cuda.synchronize()
        outs.append((buf.logits.cpu().numpy().tobytes(), buf.A_g.cpu().numpy()[:int(buf.K.cpu()[0])].tobytes(),
                     buf.y.cpu().numpy().tobytes()))
    assert outs[0] == outs[1] == outs[2]


# --------------------------------------------------------------------------- full-size workloads, one layer each

# The layers whose density and predictor hidden size are the smallest and largest of their stack
# (LLaMA-13B-gated: layer 3, rho 0.113 / H 640, and layer 14, rho 0.206 / H 960; OPT-175B-int4:
# layer 15, rho 0.056 / H 1408, and layer 14, rho 0.090 / H 3520) are among them; tests/test_synth.py
# checks that they still are.
EXTREME_LAYERS = {"llama-13b-gated": (3, 14), "opt-175b-int4": (15, 14)}
FULL = [("opt-768", 0, 1), ("opt-6.7b", 5, 1), ("llama-13b-gated", 7, 1), ("opt-30b", 3, 1), ("opt-30b", 3, 4),
        ("opt-30b", 11, 16), ("opt-30b", 11, 32), ("opt-175b-int4", 42, 1), ("opt-30b-i4pred", 3, 1),
        ("opt-30b", 20, 2), ("llama-13b-gated", 9, 2)]
FULL += [(k, l, 1) for k, ls in EXTREME_LAYERS.items() for l in ls]


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
@pytest.mark.parametrize("key,layer,B", FULL, ids=[f"{k}-L{l}-B{b}" for k, l, b in FULL])
def test_full_size_layer_parity(key, layer, B, fused):
    _dev()
    _run(synth.CONFIGS[key], layer=layer, step=3, B=B, fused=fused)


# A seeded sample of the OPT-30B stack's (step, layer) pairs of the benchmark (64 steps, 48 layers):
# numpy.random.default_rng(2026), four pairs at batch 1, then two at batch 32.
SAMPLED = [(54, 17, 1), (11, 22, 1), (1, 3, 1), (40, 17, 1), (41, 39, 32), (22, 37, 32)]


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
@pytest.mark.parametrize("step,layer,B", SAMPLED, ids=[f"S{s}-L{l}-B{b}" for s, l, b in SAMPLED])
def test_opt30b_sampled_step_layer_parity(step, layer, B, fused):
    _dev()
    _run(synth.CONFIGS["opt-30b"], layer=layer, step=step, B=B, fused=fused)


@pytest.mark.parametrize("B", [1, 3])
@pytest.mark.parametrize("cfg", [SMALL[0], SMALL[1], SMALL[2]], ids=["f16-ragged", "f32", "f16"])
def test_predict_output_logits_and_mask(cfg, B):
    """pi_predict_output on a given hidden activation: logits vs the oracle (the
    output layer alone is the oracle's predictor with an identity first layer)."""
    import oracle as orc
    import activation_sparse_amd as pi
    torch = _dev()
    spec = synth.layer_spec(cfg, 0)
    H, N = spec.H, cfg.N
    dl = ph.DeviceLayer(spec)
    g = np.random.default_rng(3)
    h = np.abs(g.standard_normal((B, H))).astype(np.float32)
    h[:, ::5] = 0.0
    h_dev = torch.from_numpy(h).cuda()
    logits = torch.empty((B, N), dtype=torch.float32, device="cuda")
    mask = torch.empty(2 * ((N + 63) // 64), dtype=torch.int32, device="cuda")
    ws = torch.empty(max(pi.pi_workspace_bytes(pi.PI_OP_PREDICT_OUTPUT, B, 0, H, N), 256), dtype=torch.uint8,
                     device="cuda")
    pi.pi_predict_output(B, H, N, h_dev, dl.P2, dl.c2, 0.0, logits, mask, ws)
    torch.cuda.synchronize()
    P2 = ph.host_mat(cfg.pdtype, cfg.seed, synth.TAG_P2, 0, H, spec.sigmas()[synth.TAG_P2], nrows=N)
    eye = orc.Mat(np.eye(H, dtype=np.float32), orc.F32, H)
    ref = orc.predict(h, eye, orc.Vec(None), P2, ph.host_vec(spec.c2, cfg.bdtype))
    lg = logits.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(lg - ref)) <= ph.LOGIT_ATOL
    words = mask.cpu().numpy().view(np.uint32)
    bits = ((words[np.arange(N) // 32] >> (np.arange(N) % 32)) & 1).astype(bool)
    want = (lg.astype(np.float32) > np.float32(0.0)).any(axis=0)
    assert np.array_equal(bits, want)        # the kernel's own logits decide its bits
    tail = ((words[np.arange(N, 32 * len(words)) // 32] >> (np.arange(N, 32 * len(words)) % 32)) & 1)
    assert not tail.any()
    near = np.min(np.abs(ref), axis=0) <= ph.BAND
    assert np.array_equal(bits[~near], (ref > 0).any(axis=0)[~near])


# --------------------------------------------------------------------------- fp16 range of the matrix-core path

def test_matrix_core_activations_near_the_fp16_range():
    """At batch >= 3 with fp16 weights, FC2 on the matrix cores takes the FC1 outputs a rounded to fp16
    (and the predictor's output layer takes h as two fp16 parts), so pi.h bounds |a| and |h| by fp16's
    largest value, 65504.  A gated layer at batch 4 with its inputs scaled by 40 drives a into the tens
    of thousands (checked on the oracle's own FC1 outputs), and the result stays within the parity
    bounds, the logits' absolute bound scaled with the inputs."""
    torch = _dev()
    import oracle as orc
    cfg = SMALL[4]                       # gated fp16, d=512, N=1536
    assert cfg.gated and cfg.wdtype == synth.F16
    B, scale = 4, 40.0
    x = synth.host_x(cfg.seed, 0, 0, B, cfg.d) * np.float32(scale)
    r = ph.run_layer_parity(cfg, layer=0, step=0, B=B, x_override=x, fused=True)
    print(f"[parity] large inputs -> {r}", flush=True)
    assert r["ascending"] and r["list_outside_band"] == 0, r
    assert r["logit_max_abs_err"] <= ph.LOGIT_ATOL * scale, r
    assert r["rel_err_ffn"] <= ph.RTOL and r["rel_err"] <= ph.RTOL, r
    # the oracle's FC1 outputs over the predicted GPU-resident neurons
    spec = synth.layer_spec(cfg, 0)
    logits, _ = ph.oracle_predict(spec, x)
    A_g, _ = orc.compact(logits, 0.0, spec.T_g, None)
    ids = spec.T_g[A_g]
    sig = spec.sigmas()
    w1 = synth.host_rows(synth.F16, cfg.seed, synth.TAG_W1, 0, cfg.d, sig[synth.TAG_W1], row_ids=ids)[0]
    wu = synth.host_rows(synth.F16, cfg.seed, synth.TAG_WUP, 0, cfg.d, sig[synth.TAG_WUP], row_ids=ids)[0]
    w1 = w1.view(np.float16).astype(np.float64)
    wu = wu.view(np.float16).astype(np.float64)
    b1 = synth.stored_to_f64(spec.b1[ids], cfg.bdtype)
    z = x.astype(np.float64) @ w1.T + b1
    a = np.maximum(z, 0.0) * (x.astype(np.float64) @ wu.T)
    a_max = float(np.max(np.abs(a)))
    print(f"[parity] largest |a| = {a_max:.1f}", flush=True)
    assert 1e4 <= a_max < 65504.0, a_max
