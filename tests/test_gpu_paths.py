"""GPU tests of the paths beside the four-step parity: the stage-restricted
layer call and its rows-read report, the hidden-major output layer with int4
weights and with more hidden units than one pass covers, and batches whose
size is not a multiple of the matrix-core tile.  Every check is against the
CPU oracle (or a property the oracle's outputs fix)."""
import numpy as np
import pytest

import synth
import oracle as orc
from tests import parity_harness as ph

pytestmark = pytest.mark.gpu


def _dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _layer_call(pi, dl, buf, B, stages, rows=None, cold=False):
    pi.pi_ffn_layer_stages(dl.layer, B, buf.x, 0.0, None, buf.y, buf.logits, buf.A_g, buf.K,
                           buf.A_c if cold else None, buf.K_c if cold else None, buf.ws_layer, stages, rows_read=rows)


def _state(buf, cold):
    K = int(buf.K.cpu()[0])
    Kc = int(buf.K_c.cpu()[0]) if cold else 0
    return (K, buf.A_g.cpu().numpy()[:K].tobytes(), Kc, buf.A_c.cpu().numpy()[:Kc].tobytes(),
            buf.logits.cpu().numpy().tobytes(), buf.y.cpu().numpy().tobytes())


@pytest.mark.parametrize("B", [1, 4, 16])
def test_stages_one_by_one_reproduce_the_full_call(B):
    """Enqueueing the stages separately, in order, gives the full call's bits."""
    import activation_sparse_amd as pi
    torch = _dev()
    cfg = ph.small_case("cold40", d=512, N=2048, H=128, wdtype=synth.F16, gpu_frac=0.4, seed=17)
    spec = synth.layer_spec(cfg, 0)
    dl = ph.DeviceLayer(spec)
    cold = len(spec.T_c) > 0
    assert cold and dl.layer.cold
    outs = []
    for split in (False, True):
        buf = ph.DeviceBuffers(cfg, spec.H, spec.n_g, len(spec.T_c), B)
        buf.x.copy_(torch.from_numpy(synth.host_x(cfg.seed, 0, 4, B, cfg.d)))
        if split:
            for st in (pi.PI_STAGE_HIDDEN, pi.PI_STAGE_OUTPUT, pi.PI_STAGE_FC1, pi.PI_STAGE_FC2, pi.PI_STAGE_SUM):
                _layer_call(pi, dl, buf, B, st, cold=cold)
        else:
            _layer_call(pi, dl, buf, B, pi.PI_STAGE_ALL, cold=cold)
        torch.cuda.synchronize()
        outs.append(_state(buf, cold))
    assert outs[0] == outs[1]


def _count_with_band(z, band=1e-4):
    """(certain, possible) number of pre-activations > 0, given the fp32-vs-fp64 difference
    of the GPU's sums (far below the band at these sizes)."""
    return int(np.sum(z > band)), int(np.sum(z > -band))


def _f64(m):
    """Exact float64 values of stored fp32 / fp16 rows."""
    return m.data.astype(np.float64) if m.dtype == synth.F32 else m.data.view(np.float16).astype(np.float64)


@pytest.mark.parametrize("key,layer,B", [("opt-30b", 2, 1), ("opt-6.7b", 1, 1), ("opt-30b", 2, 4)])
def test_rows_read_report(key, layer, B):
    """rows_read[0] = P2 rows read: at batch 1 the hidden units with h > 0, else H;
    rows_read[1] = W2 rows read: at batch 1 the listed neurons whose FC1 output is
    non-zero, else K.  The pre-activations are recomputed in float64 from the stored bits
    (a plain matrix product, c1 = 0)."""
    import activation_sparse_amd as pi
    torch = _dev()
    cfg = synth.CONFIGS[key]
    spec = synth.layer_spec(cfg, layer)
    dl = ph.DeviceLayer(spec)
    cold = len(spec.T_c) > 0
    buf = ph.DeviceBuffers(cfg, spec.H, spec.n_g, len(spec.T_c), B)
    x = synth.host_x(cfg.seed, layer, 6, B, cfg.d)
    buf.x.copy_(torch.from_numpy(x))
    rows = torch.full((2,), -1, dtype=torch.int32, device="cuda")
    _layer_call(pi, dl, buf, B, pi.PI_STAGE_ALL, rows=rows, cold=cold)
    torch.cuda.synchronize()
    r = rows.cpu().numpy()
    K = int(buf.K.cpu()[0])
    A_g = buf.A_g.cpu().numpy()[:K]
    if B > 1:
        assert r[0] == spec.H and r[1] == K
        return
    sig = spec.sigmas()
    x64 = x[0].astype(np.float64)
    P1 = ph.host_mat(cfg.pdtype, cfg.seed, synth.TAG_P1, layer, cfg.d, sig[synth.TAG_P1], nrows=spec.H)
    lo, hi = _count_with_band(_f64(P1) @ x64)
    assert lo <= r[0] <= hi and hi - lo <= 2, (r, lo, hi)
    ids = spec.T_g[A_g]
    W1 = ph.host_mat(cfg.wdtype, cfg.seed, synth.TAG_W1, layer, cfg.d, sig[synth.TAG_W1], row_ids=ids)
    b1 = synth.stored_to_f64(spec.b1[ids], cfg.bdtype)
    lo, hi = _count_with_band(_f64(W1) @ x64 + b1)
    assert lo <= r[1] <= hi and hi - lo <= 4, (r, lo, hi)


def test_output_layer_int4_hidden_major():
    """pi_predict_output with int4-g128 P2 stored hidden-major (groups run along N): logits
    against the oracle on the exactly dequantised weights, and the activation bits."""
    import activation_sparse_amd as pi
    torch = _dev()
    H, N, B = 96, 1280, 1
    data, scales = synth.host_rows(synth.I4G128, 21, synth.TAG_P2, 0, N, 1 / np.sqrt(H), nrows=H)
    # exact values q * s of the stored bits, [H x N]
    q = np.empty((H, N), np.float64)
    q[:, 0::2] = (data & 0xF).astype(np.int64)
    q[:, 1::2] = (data >> 4).astype(np.int64)
    q = np.where(q >= 8, q - 16, q)
    s = scales.view(np.float16).astype(np.float64)
    w = q * np.repeat(s, 128, axis=1)
    P2t_dev = pi.Matrix(torch.from_numpy(data).cuda(), pi.PI_I4G128, torch.from_numpy(scales.view(np.int16)).cuda())
    g = np.random.default_rng(5)
    c2 = (g.standard_normal(N) * 0.3).astype(np.float32)
    h = np.abs(g.standard_normal((B, H))).astype(np.float32)
    h[:, ::3] = 0.0
    logits = torch.empty((B, N), dtype=torch.float32, device="cuda")
    mask = torch.empty(2 * ((N + 63) // 64), dtype=torch.int32, device="cuda")
    pi.pi_predict_output(B, H, N, torch.from_numpy(h).cuda(), P2t_dev, pi.Vector(torch.from_numpy(c2).cuda(), pi.PI_F32),
                         0.0, logits, mask, None)
    torch.cuda.synchronize()
    eye = orc.Mat(np.eye(H, dtype=np.float32), orc.F32, H)
    ref = orc.predict(h, eye, orc.Vec(None), orc.Mat(np.ascontiguousarray(w.T.astype(np.float32)), orc.F32, H),
                      orc.Vec(c2, orc.F32))
    lg = logits.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(lg - ref)) <= ph.LOGIT_ATOL
    words = mask.cpu().numpy().view(np.uint32)
    bits = ((words[np.arange(N) // 32] >> (np.arange(N) % 32)) & 1).astype(bool)
    assert np.array_equal(bits, lg[0].astype(np.float32) > 0)


# more hidden units than one pass of the batch-1 output-layer kernel reads (1024 rows a pass)
BIG_H = ph.small_case("h1536", d=512, N=2048, H=1536, wdtype=synth.F16, seed=23)
# batch sizes that leave the matrix-core batch tiles partly empty
RAGGED_B = ph.small_case("mm-ragged", d=1024, N=2048, H=256, wdtype=synth.F16, gpu_frac=0.4, seed=24)


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
def test_output_layer_two_passes(fused):
    _dev()
    r = ph.run_layer_parity(BIG_H, layer=0, step=1, B=1, fused=fused)
    print("[parity]", r)
    ph.assert_report(r)


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
@pytest.mark.parametrize("B", [2, 3, 8, 9, 17, 31])
def test_matrix_core_batches(B, fused):
    _dev()
    r = ph.run_layer_parity(RAGGED_B, layer=0, step=2, B=B, fused=fused)
    print("[parity]", r)
    ph.assert_report(r)
    assert r["K"] > 0 and r["K_c"] > 0


@pytest.mark.parametrize("B", [1, 3])
def test_hybrid_layer(B):
    """The hybrid executor: the GPU predicts, compacts and computes its hot neurons while the
    CPU (libpi_host) computes the cold ones, merged on the GPU; lists and the merged output
    against the oracle, over three calls in a row with different inputs (each call's copies
    and lists are its own)."""
    torch = _dev()
    from activation_sparse_amd.hybrid import HybridLayer
    from synth.device import HostColdLayer
    cfg = ph.small_case("cold40", d=512, N=2048, H=128, wdtype=synth.F16, gpu_frac=0.4, seed=17)
    spec = synth.layer_spec(cfg, 0)
    hy = HybridLayer(ph.DeviceLayer(spec), HostColdLayer(spec), B)
    y = torch.empty((B, cfg.d), dtype=torch.float32, device="cuda")
    for step in (5, 6, 7):
        x = synth.host_x(cfg.seed, 0, step, B, cfg.d)
        kc = hy(torch.from_numpy(x).cuda(), y)
        torch.cuda.synchronize()
        K = int(hy.K.cpu()[0])
        A_g = hy.A_g.cpu().numpy()[:K]
        A_c = hy.A_c_h.numpy()[:kc].copy()
        assert int(hy.K_c_h[0]) == kc and np.array_equal(hy.cold_list.cpu().numpy()[4:4 + kc], A_c)
        assert np.array_equal(hy.x_h.numpy(), x)
        logits_or, _ = ph.oracle_predict(spec, x)
        A_g_or, A_c_or = orc.compact(logits_or, 0.0, spec.T_g, spec.T_c)
        _, out_g, asc_g = ph.list_check(A_g, A_g_or, spec.T_g, logits_or, 0.0)
        _, out_c, asc_c = ph.list_check(A_c, A_c_or, spec.T_c, logits_or, 0.0)
        assert kc > 0 and K > 0 and out_g == 0 and out_c == 0 and asc_g and asc_c
        y_or = ph.oracle_ffn_on_ids(spec, x, spec.T_g[A_g]) + ph.oracle_ffn_on_ids(spec, x, spec.T_c[A_c])
        assert ph.rel_err(y.cpu().numpy(), y_or) <= ph.RTOL, step


def test_hybrid_layer_skips_the_merge_without_cold_neurons():
    """Selective synchronisation: no active neuron on either side gives y = 0 and no merge."""
    torch = _dev()
    from activation_sparse_amd.hybrid import HybridLayer
    from synth.device import HostColdLayer
    cfg = ph.small_case("cold40", d=512, N=2048, H=128, wdtype=synth.F16, gpu_frac=0.4, seed=17)
    spec = synth.layer_spec(cfg, 0)
    hy = HybridLayer(ph.DeviceLayer(spec), HostColdLayer(spec), 1)
    x = synth.host_x(cfg.seed, 0, 5, 1, cfg.d)
    y = torch.full((1, cfg.d), 7.0, dtype=torch.float32, device="cuda")
    kc = hy(torch.from_numpy(x).cuda(), y, tau=1e30)
    torch.cuda.synchronize()
    assert kc == 0 and int(hy.K.cpu()[0]) == 0 and not torch.any(y).item()


COMPACT_CASES = [  # (N, n_g, B, density): ragged table sizes, both tables split over many blocks
    (28672, 20071, 1, 0.1), (28672, 20071, 3, 0.05), (28672, 9000, 32, 0.01), (4097, 4097, 2, 0.5),
    (65536, 40000, 4, 0.2), (1000, 0, 1, 0.3), (2048, 1, 5, 0.9)]


@pytest.mark.parametrize("N,n_g,B,density", COMPACT_CASES)
def test_compact_lists_are_exact_over_any_table_order(N, n_g, B, density):
    """pi_compact against the oracle's compaction, bit for bit: tables in a random order
    (slot order need not follow the ids), logits that tie with tau (not active: the
    compare is strict), neurons active for one batch row only (the union)."""
    import activation_sparse_amd as pi
    torch = _dev()
    g = np.random.default_rng(N + 7 * n_g + B)
    perm = g.permutation(N).astype(np.int32)
    T_g, T_c = perm[:n_g].copy(), perm[n_g:].copy()
    tau = 0.25
    z = g.standard_normal((B, N)).astype(np.float32) - 2.0
    on = g.random((B, N)) < density / B
    z[on] = tau + np.abs(z[on]) + 1e-3
    z[g.random((B, N)) < 0.02] = tau                      # ties: inactive
    A_g_or, A_c_or = orc.compact(z.astype(np.float64), tau, T_g, T_c)
    dev = "cuda:0"
    i32 = torch.int32
    logits = torch.from_numpy(z).to(dev)
    Tg = torch.from_numpy(T_g if n_g else np.zeros(1, np.int32)).to(dev)
    Tc = torch.from_numpy(T_c if len(T_c) else np.zeros(1, np.int32)).to(dev)   # n_c = 0: a table, empty
    A_g = torch.full((max(n_g, 1),), -7, dtype=i32, device=dev)
    A_c = torch.full((max(N - n_g, 1),), -7, dtype=i32, device=dev)
    K = torch.full((1,), -1, dtype=i32, device=dev)
    K_c = torch.full((1,), -1, dtype=i32, device=dev)
    print(f"pi_compact N={N} n_g={n_g} B={B}", flush=True)
    for _ in range(2):                                    # the second call overwrites the first
        pi.pi_compact(B, N, logits, tau, Tg, n_g, A_g, K, Tc, N - n_g, A_c, K_c)
    torch.cuda.synchronize()
    k, kc = int(K.cpu()[0]), int(K_c.cpu()[0])
    assert k == len(A_g_or) and kc == len(A_c_or)
    assert np.array_equal(A_g.cpu().numpy()[:k], A_g_or)
    assert np.array_equal(A_c.cpu().numpy()[:kc], A_c_or)
    # entries past the counts are untouched
    assert np.all(A_g.cpu().numpy()[k:] == -7) and np.all(A_c.cpu().numpy()[kc:] == -7)
    # without the cold table only the GPU list is written
    K.fill_(-1)
    pi.pi_compact(B, N, logits, tau, Tg, n_g, A_g, K)
    torch.cuda.synchronize()
    assert int(K.cpu()[0]) == k and np.array_equal(A_g.cpu().numpy()[:k], A_g_or)


@pytest.mark.parametrize("B", [1, 4])
def test_lookahead_prediction_on_two_streams(B):
    """Look-ahead prediction: layer l+1's predictor hidden layer runs on layer l's input, on a
    second stream beside layer l's FFN; its remaining stages take layer l+1's own input.  Each
    layer's logits and lists against the oracle's prediction from that earlier input (and not
    from its own), its output against the oracle's FFN on its own input over the GPU's list."""
    import activation_sparse_amd as pi
    torch = _dev()
    cfg = ph.small_case("cold40", d=512, N=2048, H=128, wdtype=synth.F16, gpu_frac=0.4, seed=17)
    nl = 3
    specs = [synth.layer_spec(cfg, l) for l in range(nl)]
    dls = [ph.DeviceLayer(s) for s in specs]
    bufs = [ph.DeviceBuffers(cfg, s.H, s.n_g, len(s.T_c), B) for s in specs]
    xs = [synth.host_x(cfg.seed, l, 3, B, cfg.d) for l in range(nl)]
    for b, x in zip(bufs, xs):
        b.x.copy_(torch.from_numpy(x))
    torch.cuda.synchronize()
    main, ahead = torch.cuda.current_stream(), torch.cuda.Stream()
    rest = pi.PI_STAGE_ALL & ~pi.PI_STAGE_HIDDEN

    def stage(l, x, stages, st):
        b = bufs[l]
        pi.pi_ffn_layer_stages(dls[l].layer, B, x, 0.0, None, b.y, b.logits, b.A_g, b.K, b.A_c, b.K_c, b.ws_layer,
                               stages, stream=st)

    print(f"look-ahead B={B}", flush=True)
    stage(0, bufs[0].x, pi.PI_STAGE_HIDDEN, main)
    for l in range(nl):
        if l + 1 < nl:
            ahead.wait_stream(main)
            stage(l + 1, bufs[l].x, pi.PI_STAGE_HIDDEN, ahead)
        stage(l, bufs[l].x, rest, main)
        if l + 1 < nl:
            main.wait_stream(ahead)
    torch.cuda.synchronize()
    for l in range(nl):
        spec, b = specs[l], bufs[l]
        logits_or, _ = ph.oracle_predict(spec, xs[max(l - 1, 0)])
        assert np.max(np.abs(b.logits.cpu().numpy().astype(np.float64) - logits_or)) <= ph.LOGIT_ATOL, l
        K, K_c = int(b.K.cpu()[0]), int(b.K_c.cpu()[0])
        A_g, A_c = b.A_g.cpu().numpy()[:K], b.A_c.cpu().numpy()[:K_c]
        A_g_or, A_c_or = orc.compact(logits_or, 0.0, spec.T_g, spec.T_c)
        _, out_g, asc_g = ph.list_check(A_g, A_g_or, spec.T_g, logits_or, 0.0)
        _, out_c, asc_c = ph.list_check(A_c, A_c_or, spec.T_c, logits_or, 0.0)
        assert K > 0 and out_g == 0 and out_c == 0 and asc_g and asc_c, l
        if l > 0:      # the list is the earlier input's, not the layer's own
            own, _ = orc.compact(ph.oracle_predict(spec, xs[l])[0], 0.0, spec.T_g)
            assert not np.array_equal(own, A_g_or)
        y_or = ph.oracle_ffn_on_ids(spec, xs[l], spec.T_g[A_g])
        assert ph.rel_err(b.y.cpu().numpy(), y_or) <= ph.RTOL, l


@pytest.mark.parametrize("nbytes,blocks,depth", [(16, 1, 0), (4096 + 48, 3, 4), (63 * 2**20 + 16, 0, 0),
                                                  (2**26, 4096, 8), (2**26 + 16 * 37, 512, 16),
                                                  (2**20 + 16 * 5, 2048, 32), (16 * 31, 1, 32)])
def test_read_probe_reads_every_word(nbytes, blocks, depth):
    """The streaming-read reference reads each 16-byte vector once: the XOR of what every wave
    reports equals the XOR of all the buffer's words (a skipped or repeated vector changes it)."""
    import activation_sparse_amd as pi
    torch = _dev()
    g = np.random.default_rng(nbytes)
    host = g.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    nb = blocks if blocks > 0 else pi.PI_READ_PROBE_BLOCKS_PER_CU * 256
    out = torch.zeros(4 * nb, dtype=torch.int32, device="cuda")
    print(f"read probe {nbytes} B, {nb} blocks, depth {depth}", flush=True)
    pi.pi_read_probe(buf, nbytes, out, blocks, depth=depth)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


@pytest.mark.parametrize("B", [1, 4])
def test_graph_replays_match_the_eager_call(B):
    """A three-layer stack captured in a HIP graph (as the benchmark times it) and replayed four
    times, with eager layer calls on other buffers and host synchronisations between the replays:
    every replay's outputs (y, logits, lists and counts) equal the eager call's bits."""
    import activation_sparse_amd as pi
    torch = _dev()
    cfg = ph.small_case("cold40", d=512, N=2048, H=128, wdtype=synth.F16, gpu_frac=0.4, seed=17)
    specs = [synth.layer_spec(cfg, l) for l in range(3)]
    dls = [ph.DeviceLayer(s) for s in specs]
    bufs = [ph.DeviceBuffers(cfg, s.H, s.n_g, len(s.T_c), B) for s in specs]
    other = ph.DeviceBuffers(cfg, specs[0].H, specs[0].n_g, len(specs[0].T_c), B)
    g = np.random.default_rng(B)
    for l, b in enumerate(bufs):
        b.x.copy_(torch.from_numpy(synth.host_x(cfg.seed, l, 9, B, cfg.d)))
        b.y_c.copy_(torch.from_numpy((g.standard_normal((B, cfg.d)) * 0.05).astype(np.float32)))
    other.x.copy_(torch.from_numpy(synth.host_x(cfg.seed, 0, 10, B, cfg.d)))

    def call(l, b):
        pi.pi_ffn_layer(dls[l].layer, B, b.x, 0.0, b.y_c, b.y, b.logits, b.A_g, b.K, b.A_c, b.K_c, b.ws_layer)

    def state():
        out = []
        for b in bufs:
            K, Kc = int(b.K.cpu()[0]), int(b.K_c.cpu()[0])
            out.append((b.y.cpu().numpy().tobytes(), b.logits.cpu().numpy().tobytes(), K, Kc,
                        b.A_g.cpu().numpy()[:K].tobytes(), b.A_c.cpu().numpy()[:Kc].tobytes()))
        return out

    def clear():
        for b in bufs:
            b.y.fill_(float("nan")); b.logits.fill_(float("nan")); b.K.fill_(-1); b.K_c.fill_(-1)
            b.A_g.fill_(-1); b.A_c.fill_(-1)

    print(f"graph replays B={B}", flush=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for l, b in enumerate(bufs):
            call(l, b)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = state()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for l, b in enumerate(bufs):
            call(l, b)
    torch.cuda.synchronize()
    for r in range(4):
        clear()
        call(0, other)                       # eager work of its own between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert state() == eager, r


@pytest.mark.parametrize("B", [1, 4])
def test_lookahead_entry_point(B):
    """pi_ffn_layer_ahead: layer l's stages and, in the same call, layer l+1's predictor hidden
    layer from layer l's input (at batch 1 inside the launch that runs layer l's output layer
    and FC1; at batch 4 by the separate kernels).  Each layer's logits and lists against the
    oracle's prediction from the earlier input, its output against the oracle's FFN on its own
    input over the GPU's list."""
    import activation_sparse_amd as pi
    torch = _dev()
    cfg = ph.small_case("cold40", d=512, N=2048, H=128, wdtype=synth.F16, gpu_frac=0.4, seed=17)
    nl = 3
    specs = [synth.layer_spec(cfg, l) for l in range(nl)]
    dls = [ph.DeviceLayer(s) for s in specs]
    bufs = [ph.DeviceBuffers(cfg, s.H, s.n_g, len(s.T_c), B) for s in specs]
    xs = [synth.host_x(cfg.seed, l, 4, B, cfg.d) for l in range(nl)]
    for b, x in zip(bufs, xs):
        b.x.copy_(torch.from_numpy(x))
    torch.cuda.synchronize()
    rest = pi.PI_STAGE_ALL & ~pi.PI_STAGE_HIDDEN
    print(f"look-ahead entry point B={B}", flush=True)
    b0 = bufs[0]
    pi.pi_ffn_layer_stages(dls[0].layer, B, b0.x, 0.0, None, b0.y, b0.logits, b0.A_g, b0.K, b0.A_c, b0.K_c,
                           b0.ws_layer, pi.PI_STAGE_HIDDEN)
    for l in range(nl):
        b = bufs[l]
        if l + 1 < nl:
            pi.pi_ffn_layer_ahead(dls[l].layer, B, b.x, 0.0, None, b.y, b.logits, b.A_g, b.K, b.A_c, b.K_c,
                                  b.ws_layer, rest, dls[l + 1].layer, bufs[l + 1].ws_layer)
        else:
            pi.pi_ffn_layer_stages(dls[l].layer, B, b.x, 0.0, None, b.y, b.logits, b.A_g, b.K, b.A_c, b.K_c,
                                   b.ws_layer, rest)
    torch.cuda.synchronize()
    for l in range(nl):
        spec, b = specs[l], bufs[l]
        logits_or, _ = ph.oracle_predict(spec, xs[max(l - 1, 0)])
        assert np.max(np.abs(b.logits.cpu().numpy().astype(np.float64) - logits_or)) <= ph.LOGIT_ATOL, l
        K, K_c = int(b.K.cpu()[0]), int(b.K_c.cpu()[0])
        A_g, A_c = b.A_g.cpu().numpy()[:K], b.A_c.cpu().numpy()[:K_c]
        A_g_or, A_c_or = orc.compact(logits_or, 0.0, spec.T_g, spec.T_c)
        _, out_g, asc_g = ph.list_check(A_g, A_g_or, spec.T_g, logits_or, 0.0)
        _, out_c, asc_c = ph.list_check(A_c, A_c_or, spec.T_c, logits_or, 0.0)
        assert K > 0 and out_g == 0 and out_c == 0 and asc_g and asc_c, l
        y_or = ph.oracle_ffn_on_ids(spec, xs[l], spec.T_g[A_g])
        assert ph.rel_err(b.y.cpu().numpy(), y_or) <= ph.RTOL, l


@pytest.mark.parametrize("B", [1, 3])
def test_hybrid_lookahead_stack(B):
    """The look-ahead hybrid over two layers: layer 0 predicted from its own input (prime), layer 1
    from layer 0's input while the CPU computes layer 0's cold neurons.  Each layer's lists (both
    list sets survive a two-layer call) against the oracle's prediction from that input, and each
    output against the oracle's FFN on the layer's own input over the GPU's and the CPU's lists."""
    torch = _dev()
    from activation_sparse_amd.hybrid import HybridStack
    from synth.device import HostColdLayer
    cfg = ph.small_case("cold40", d=512, N=2048, H=128, wdtype=synth.F16, gpu_frac=0.4, seed=17)
    specs = [synth.layer_spec(cfg, l) for l in range(2)]
    dls = [ph.DeviceLayer(s) for s in specs]
    hy = HybridStack(dls, [HostColdLayer(s) for s in specs], B)
    xs_h = [synth.host_x(cfg.seed, l, 8, B, cfg.d) for l in range(2)]
    xs = [torch.from_numpy(x).cuda() for x in xs_h]
    ys = [torch.empty((B, cfg.d), dtype=torch.float32, device="cuda") for _ in range(2)]
    print(f"hybrid look-ahead B={B}", flush=True)
    for rep in range(2):                           # a second call reuses the scratch
        kcs = hy(xs, ys)
        torch.cuda.synchronize()
    for l in range(2):
        spec = specs[l]
        K = int(hy.K[l].cpu()[0])
        A_g = hy.A_g[l].cpu().numpy()[:K]
        kc = int(hy.cold_list_h[l][0])
        A_c = hy.cold_list_h[l].numpy()[4:4 + kc].copy()
        assert kc == kcs[l]
        logits_or, _ = ph.oracle_predict(spec, xs_h[max(l - 1, 0)])
        A_g_or, A_c_or = orc.compact(logits_or, 0.0, spec.T_g, spec.T_c)
        _, out_g, asc_g = ph.list_check(A_g, A_g_or, spec.T_g, logits_or, 0.0)
        _, out_c, asc_c = ph.list_check(A_c, A_c_or, spec.T_c, logits_or, 0.0)
        assert K > 0 and kc > 0 and out_g == 0 and out_c == 0 and asc_g and asc_c, l
        y_or = ph.oracle_ffn_on_ids(spec, xs_h[l], spec.T_g[A_g]) + ph.oracle_ffn_on_ids(spec, xs_h[l], spec.T_c[A_c])
        assert ph.rel_err(ys[l].cpu().numpy(), y_or) <= ph.RTOL, l
    # the same stack in one native call (pi_hybrid_stack_ahead): the same bits and counts
    ys2 = [torch.full((B, cfg.d), float("nan"), dtype=torch.float32, device="cuda") for _ in range(2)]
    kcs2 = hy.native(xs, ys2)
    torch.cuda.synchronize()
    assert kcs2 == kcs
    for l in range(2):
        assert ys2[l].cpu().numpy().tobytes() == ys[l].cpu().numpy().tobytes(), l


@pytest.mark.parametrize("B", [1, 2])
def test_lookahead_gated_layers_of_different_hidden_sizes(B):
    """pi_ffn_layer_ahead across gated layers whose predictors differ in size (H = 128, then
    192): the next layer's hidden rows, computed in this layer's launch at batch 1 (separately at
    batch 2), give lists and outputs that match the oracle's prediction from this layer's input."""
    import activation_sparse_amd as pi
    torch = _dev()
    cfg = synth.Config("gated-h", "reduced 512/1536 gated", 2, 512, 1536, synth.F16, synth.F16, synth.F16, True,
                       (0.08, 0.25), 1.1, (128, 256), 0.4, (1,), 4, 39)
    specs = [synth.layer_spec(cfg, l) for l in range(2)]
    assert [s.H for s in specs] == [128, 192]
    dls = [ph.DeviceLayer(s) for s in specs]
    bufs = [ph.DeviceBuffers(cfg, s.H, s.n_g, len(s.T_c), B) for s in specs]
    xs = [synth.host_x(cfg.seed, l, 2, B, cfg.d) for l in range(2)]
    for b, x in zip(bufs, xs):
        b.x.copy_(torch.from_numpy(x))
    torch.cuda.synchronize()
    rest = pi.PI_STAGE_ALL & ~pi.PI_STAGE_HIDDEN
    print(f"look-ahead gated B={B}", flush=True)
    b0, b1 = bufs
    pi.pi_ffn_layer_stages(dls[0].layer, B, b0.x, 0.0, None, b0.y, b0.logits, b0.A_g, b0.K, b0.A_c, b0.K_c,
                           b0.ws_layer, pi.PI_STAGE_HIDDEN)
    pi.pi_ffn_layer_ahead(dls[0].layer, B, b0.x, 0.0, None, b0.y, b0.logits, b0.A_g, b0.K, b0.A_c, b0.K_c,
                          b0.ws_layer, rest, dls[1].layer, b1.ws_layer)
    pi.pi_ffn_layer_stages(dls[1].layer, B, b1.x, 0.0, None, b1.y, b1.logits, b1.A_g, b1.K, b1.A_c, b1.K_c,
                           b1.ws_layer, rest)
    torch.cuda.synchronize()
    for l in range(2):
        spec, b = specs[l], bufs[l]
        logits_or, _ = ph.oracle_predict(spec, xs[0])
        assert np.max(np.abs(b.logits.cpu().numpy().astype(np.float64) - logits_or)) <= ph.LOGIT_ATOL, l
        K, K_c = int(b.K.cpu()[0]), int(b.K_c.cpu()[0])
        A_g, A_c = b.A_g.cpu().numpy()[:K], b.A_c.cpu().numpy()[:K_c]
        A_g_or, A_c_or = orc.compact(logits_or, 0.0, spec.T_g, spec.T_c)
        _, out_g, asc_g = ph.list_check(A_g, A_g_or, spec.T_g, logits_or, 0.0)
        _, out_c, asc_c = ph.list_check(A_c, A_c_or, spec.T_c, logits_or, 0.0)
        assert K > 0 and out_g == 0 and out_c == 0 and asc_g and asc_c, l
        y_or = ph.oracle_ffn_on_ids(spec, xs[l], spec.T_g[A_g])
        assert ph.rel_err(b.y.cpu().numpy(), y_or) <= ph.RTOL, l


def test_lookahead_ragged_shapes():
    """pi_ffn_layer_ahead at batch 1 on ragged shapes: N not a multiple of the 64-id tile, d not a
    multiple of the lane width, and a next-layer H that leaves the last look-ahead workgroup part
    empty (76 rows, 8 per workgroup)."""
    import activation_sparse_amd as pi
    torch = _dev()
    cfg = ph.small_case("ragged-ahead", d=264, N=1000, H=76, wdtype=synth.F16, gpu_frac=0.4, seed=23)
    cfg = synth.Config(cfg.key, cfg.desc, 2, cfg.d, cfg.N, cfg.wdtype, cfg.pdtype, cfg.bdtype, cfg.gated,
                       cfg.density, cfg.alpha, cfg.H, cfg.gpu_frac, cfg.batches, cfg.steps, cfg.seed)
    specs = [synth.layer_spec(cfg, l) for l in range(2)]
    dls = [ph.DeviceLayer(s) for s in specs]
    bufs = [ph.DeviceBuffers(cfg, s.H, s.n_g, len(s.T_c), 1) for s in specs]
    xs = [synth.host_x(cfg.seed, l, 6, 1, cfg.d) for l in range(2)]
    for b, x in zip(bufs, xs):
        b.x.copy_(torch.from_numpy(x))
    torch.cuda.synchronize()
    rest = pi.PI_STAGE_ALL & ~pi.PI_STAGE_HIDDEN
    b0, b1 = bufs
    print("look-ahead ragged", flush=True)
    pi.pi_ffn_layer_stages(dls[0].layer, 1, b0.x, 0.0, None, b0.y, b0.logits, b0.A_g, b0.K, b0.A_c, b0.K_c,
                           b0.ws_layer, pi.PI_STAGE_HIDDEN)
    pi.pi_ffn_layer_ahead(dls[0].layer, 1, b0.x, 0.0, None, b0.y, b0.logits, b0.A_g, b0.K, b0.A_c, b0.K_c,
                          b0.ws_layer, rest, dls[1].layer, b1.ws_layer)
    pi.pi_ffn_layer_stages(dls[1].layer, 1, b1.x, 0.0, None, b1.y, b1.logits, b1.A_g, b1.K, b1.A_c, b1.K_c,
                           b1.ws_layer, rest)
    torch.cuda.synchronize()
    spec, b = specs[1], b1
    logits_or, _ = ph.oracle_predict(spec, xs[0])
    assert np.max(np.abs(b.logits.cpu().numpy().astype(np.float64) - logits_or)) <= ph.LOGIT_ATOL
    K = int(b.K.cpu()[0])
    A_g = b.A_g.cpu().numpy()[:K]
    A_g_or, _ = orc.compact(logits_or, 0.0, spec.T_g, spec.T_c)
    _, out_g, asc_g = ph.list_check(A_g, A_g_or, spec.T_g, logits_or, 0.0)
    assert K > 0 and out_g == 0 and asc_g
    y_or = ph.oracle_ffn_on_ids(spec, xs[1], spec.T_g[A_g])
    assert ph.rel_err(b.y.cpu().numpy(), y_or) <= ph.RTOL


# Layer normalisation between chained layers, fp32 on the GPU against the oracle's fp64 on the
# same fp32 rows.  Each fp32 sum runs at most 16 terms per thread, 6 butterfly levels and 16 wave
# sums in sequence, so its error is below 38 u sum|y| (u = 2^-24); for rows whose mean is within
# 3 standard deviations the mean and the deviation are then off by < 38 u (|m| + sigma) / sigma
# <= 1e-5 of sigma, and the unit-scale output by about that plus a few ulps of |x|.
LN_ATOL = 2e-5


@pytest.mark.parametrize("B,d,scale,offset", [
    (1, 7168, 0.05, 0.0),       # an OPT-30B layer output at batch 1
    (4, 7168, 3.0, 1.0),
    (32, 7168, 0.02, -0.01),    # the largest batch
    (3, 768, 1.0, 0.5),
    (2, 13, 1.0, 0.0),          # ragged: fewer elements than one wave
    (2, 1000, 1e15, 0.0),       # large magnitudes (squares still within fp32)
    (2, 1000, 1e-15, 0.0),      # small magnitudes (eps dominates the variance)
    (1, 16384, 1.0, 0.0),       # the most elements the registers hold
    (2, 16385, 1.0, 0.0),       # one more: the rows are read again in each pass
    (1, 50000, 2.0, -1.0),
    (1, 50002, 1.0, 0.0),       # long and not a multiple of 4
    (300, 64, 1.0, 0.0),        # many short rows
])
def test_layer_norm_parity(B, d, scale, offset):
    import activation_sparse_amd as pi
    torch = _dev()
    rng = np.random.default_rng(B * 7919 + d)
    y = (rng.standard_normal((B, d)) * scale + offset * scale).astype(np.float32)
    print(f"layer norm B={B} d={d} scale={scale}", flush=True)
    yd = torch.from_numpy(y).cuda()
    x = torch.empty_like(yd)
    pi.pi_layer_norm(B, d, yd, x, 1e-5)
    x2 = torch.empty_like(yd)
    pi.pi_layer_norm(B, d, yd, x2, 1e-5)
    yi = yd.clone()
    pi.pi_layer_norm(B, d, yi, yi, 1e-5)              # in place
    torch.cuda.synchronize()
    got = x.cpu().numpy()
    assert np.max(np.abs(got.astype(np.float64) - orc.layer_norm(y, 1e-5))) <= LN_ATOL
    assert np.array_equal(got.view(np.uint32), x2.cpu().numpy().view(np.uint32))     # repeatable
    assert np.array_equal(got.view(np.uint32), yi.cpu().numpy().view(np.uint32))     # in place: same bits
    assert np.array_equal(yd.cpu().numpy(), y)                                        # input untouched


def test_layer_norm_unaligned_rows():
    """Rows that do not start on a 16-byte boundary take the single-float loads; same values."""
    import activation_sparse_amd as pi
    torch = _dev()
    B, d = 3, 7168
    rng = np.random.default_rng(77)
    y = rng.standard_normal((B, d)).astype(np.float32)
    big = torch.zeros(B * d + 8, dtype=torch.float32, device="cuda")
    yv = big[1:1 + B * d]                              # 4 bytes past an aligned start
    yv.copy_(torch.from_numpy(y.reshape(-1)))
    out = torch.zeros(B * d + 8, dtype=torch.float32, device="cuda")
    xv = out[3:3 + B * d]
    xa = torch.empty((B, d), dtype=torch.float32, device="cuda")
    print("layer norm unaligned", flush=True)
    pi.pi_layer_norm(B, d, yv, xv, 1e-5)
    pi.pi_layer_norm(B, d, torch.from_numpy(y).cuda(), xa, 1e-5)
    torch.cuda.synchronize()
    got = xv.cpu().numpy().reshape(B, d)
    assert np.max(np.abs(got.astype(np.float64) - orc.layer_norm(y, 1e-5))) <= LN_ATOL
    assert np.max(np.abs(xa.cpu().numpy().astype(np.float64) - orc.layer_norm(y, 1e-5))) <= LN_ATOL
    assert not np.any(out[:3].cpu().numpy()) and not np.any(out[3 + B * d:].cpu().numpy())   # nothing outside


def test_layer_norm_constant_rows_give_zeros():
    import activation_sparse_amd as pi
    torch = _dev()
    y = np.stack([np.full(7168, 3.25, np.float32), np.zeros(7168, np.float32)])
    yd = torch.from_numpy(y).cuda()
    x = torch.full_like(yd, 7.0)
    print("layer norm constant rows", flush=True)
    pi.pi_layer_norm(2, 7168, yd, x, 1e-5)
    torch.cuda.synchronize()
    assert np.array_equal(x.cpu().numpy(), orc.layer_norm(y, 1e-5).astype(np.float32))
    assert not np.any(x.cpu().numpy())


@pytest.mark.parametrize("B,ahead", [(1, False), (1, True), (4, False), (4, True), (1, "normed"), (4, "normed")])
def test_chained_layers(B, ahead):
    """Three chained layers: layer l+1's input is the layer normalisation of layer l's output, made
    on the GPU (pi_layer_norm, or inside the layer call with pi_ffn_layer_normed).  Exact prediction
    (pi_ffn_layer) or look-ahead (pi_ffn_layer_ahead: layer l+1's hidden layer from layer l's
    input).  Each layer against the oracle on the input the GPU gave it: logits and lists from the
    predictor's input, the output over the GPU's list, and the next input against the oracle's
    normalisation of the GPU's output."""
    import activation_sparse_amd as pi
    torch = _dev()
    cfg = ph.small_case("cold40", d=512, N=2048, H=128, wdtype=synth.F16, gpu_frac=0.4, seed=29)
    nl = 3
    specs = [synth.layer_spec(cfg, l) for l in range(nl)]
    dls = [ph.DeviceLayer(s) for s in specs]
    bufs = [ph.DeviceBuffers(cfg, s.H, s.n_g, len(s.T_c), B) for s in specs]
    bufs[0].x.copy_(torch.from_numpy(synth.host_x(cfg.seed, 0, 5, B, cfg.d)))
    torch.cuda.synchronize()
    rest = pi.PI_STAGE_ALL & ~pi.PI_STAGE_HIDDEN
    print(f"chained layers B={B} ahead={ahead}", flush=True)
    if ahead == "normed":
        # layer l >= 1 normalises layer l-1's output itself and reports the row it used in x
        ahead = False
        for l in range(nl):
            b = bufs[l]
            if l == 0:
                pi.pi_ffn_layer(dls[0].layer, B, b.x, 0.0, None, b.y, b.logits, b.A_g, b.K, b.A_c, b.K_c, b.ws_layer)
                continue
            need = pi.pi_workspace_bytes(pi.PI_OP_FFN_LAYER_NORMED, B, cfg.d, specs[l].H, cfg.N, specs[l].n_g)
            ws = torch.empty(need, dtype=torch.uint8, device="cuda")
            pi.pi_ffn_layer_normed(dls[l].layer, B, bufs[l - 1].y, 1e-5, 0.0, None, b.y, b.logits, b.A_g, b.K,
                                   b.A_c, b.K_c, ws, x_out=b.x)
    else:
        if ahead:
            b0 = bufs[0]
            pi.pi_ffn_layer_stages(dls[0].layer, B, b0.x, 0.0, None, b0.y, b0.logits, b0.A_g, b0.K, b0.A_c, b0.K_c,
                                   b0.ws_layer, pi.PI_STAGE_HIDDEN)
        for l in range(nl):
            b = bufs[l]
            if ahead and l + 1 < nl:
                pi.pi_ffn_layer_ahead(dls[l].layer, B, b.x, 0.0, None, b.y, b.logits, b.A_g, b.K, b.A_c, b.K_c,
                                      b.ws_layer, rest, dls[l + 1].layer, bufs[l + 1].ws_layer)
            else:
                pi.pi_ffn_layer_stages(dls[l].layer, B, b.x, 0.0, None, b.y, b.logits, b.A_g, b.K, b.A_c, b.K_c,
                                       b.ws_layer, rest if ahead else pi.PI_STAGE_ALL)
            if l + 1 < nl:
                pi.pi_layer_norm(B, cfg.d, b.y, bufs[l + 1].x, 1e-5)
    torch.cuda.synchronize()
    xs = [b.x.cpu().numpy() for b in bufs]
    for l in range(nl):
        spec, b = specs[l], bufs[l]
        x_pred = xs[max(l - 1, 0)] if ahead else xs[l]
        logits_or, _ = ph.oracle_predict(spec, x_pred)
        assert np.max(np.abs(b.logits.cpu().numpy().astype(np.float64) - logits_or)) <= ph.LOGIT_ATOL, l
        K, K_c = int(b.K.cpu()[0]), int(b.K_c.cpu()[0])
        A_g, A_c = b.A_g.cpu().numpy()[:K], b.A_c.cpu().numpy()[:K_c]
        A_g_or, A_c_or = orc.compact(logits_or, 0.0, spec.T_g, spec.T_c)
        _, out_g, asc_g = ph.list_check(A_g, A_g_or, spec.T_g, logits_or, 0.0)
        _, out_c, asc_c = ph.list_check(A_c, A_c_or, spec.T_c, logits_or, 0.0)
        assert K > 0 and out_g == 0 and out_c == 0 and asc_g and asc_c, l
        y = b.y.cpu().numpy()
        assert ph.rel_err(y, ph.oracle_ffn_on_ids(spec, xs[l], spec.T_g[A_g])) <= ph.RTOL, l
        if l + 1 < nl:
            assert np.max(np.abs(xs[l + 1].astype(np.float64) - orc.layer_norm(y, 1e-5))) <= LN_ATOL, l


@pytest.mark.parametrize("case,B", [("opt-30b", 1), ("gated", 1), ("i4ffn", 1), ("wide-i4ffn", 1), ("i4pred", 1),
                                    ("opt-30b", 4), ("gated", 3)])
def test_normed_layer_is_the_layer_on_its_normalised_input(case, B):
    """pi_ffn_layer_normed(y_prev) gives bit for bit what pi_ffn_layer gives on the normalised row it
    reports in x_out (at batch 1 the predictor's kernel and the FC1 kernel normalise with the same
    two statistics, so both see x_out's values); x_out is the oracle's layer normalisation within
    the normalisation bound; the result against the oracle on that x; y_prev == y (in place) gives
    the same bits.  Batch 1 runs the fused kernels, other batches normalise first (x_out then equals
    pi_layer_norm's output bit for bit)."""
    import activation_sparse_amd as pi
    torch = _dev()
    if case == "opt-30b":
        cfg, layer = synth.CONFIGS["opt-30b"], 7
    elif case == "gated":
        cfg, layer = ph.small_case("ln-gated", d=1024, N=4096, H=256, wdtype=synth.F16, gated=True, seed=41), 0
    elif case == "wide-i4ffn":     # 24 KB predictor rows: the hidden-layer kernel at 24 vectors per lane
        cfg, layer = ph.small_case("ln-wide-i4", d=12288, N=1024, H=40, wdtype=synth.I4G128, pdtype=synth.F16,
                                   bdtype=synth.F16, seed=44), 0
    elif case == "i4pred":         # int4 predictor rows in the normalising hidden-layer kernel
        cfg, layer = ph.small_case("ln-i4pred", d=2048, N=2048, H=128, wdtype=synth.F16, pdtype=synth.I4G128,
                                   gpu_frac=0.4, seed=45), 0
    else:
        cfg, layer = ph.small_case("ln-i4", d=1024, N=4096, H=256, wdtype=synth.I4G128, pdtype=synth.F16,
                                   bdtype=synth.F16, gpu_frac=0.4, seed=43), 0
    spec = synth.layer_spec(cfg, layer)
    d, N = cfg.d, cfg.N
    rng = np.random.default_rng(B * 131 + d)
    y_prev = (rng.standard_normal((B, d)) * 0.07 + 0.02).astype(np.float32)
    dl = ph.DeviceLayer(spec)
    n_c = len(spec.T_c)
    b1, b2, b3 = (ph.DeviceBuffers(cfg, spec.H, spec.n_g, n_c, B) for _ in range(3))
    ws = torch.empty(pi.pi_workspace_bytes(pi.PI_OP_FFN_LAYER_NORMED, B, d, spec.H, N, spec.n_g), dtype=torch.uint8,
                     device="cuda")
    yp = torch.from_numpy(y_prev).cuda()
    x_out = torch.empty((B, d), dtype=torch.float32, device="cuda")
    print(f"normed layer {case} B={B} d={d} N={N}", flush=True)
    pi.pi_ffn_layer_normed(dl.layer, B, yp, 1e-5, 0.0, None, b1.y, b1.logits, b1.A_g, b1.K, b1.A_c, b1.K_c, ws,
                           x_out=x_out)
    b2.x.copy_(x_out)
    pi.pi_ffn_layer(dl.layer, B, b2.x, 0.0, None, b2.y, b2.logits, b2.A_g, b2.K, b2.A_c, b2.K_c, b2.ws_layer)
    yi = yp.clone()                                   # in place: y_prev is y
    pi.pi_ffn_layer_normed(dl.layer, B, yi, 1e-5, 0.0, None, yi, None, b3.A_g, b3.K, b3.A_c, b3.K_c, ws)
    ln_ref = torch.empty_like(yp)
    pi.pi_layer_norm(B, d, yp, ln_ref, 1e-5)
    torch.cuda.synchronize()
    x = x_out.cpu().numpy()
    assert np.max(np.abs(x.astype(np.float64) - orc.layer_norm(y_prev, 1e-5))) <= LN_ATOL
    if B > 1:
        assert np.array_equal(x.view(np.uint32), ln_ref.cpu().numpy().view(np.uint32))
    K = int(b1.K.cpu()[0])
    assert K == int(b2.K.cpu()[0]) and np.array_equal(b1.A_g.cpu().numpy()[:K], b2.A_g.cpu().numpy()[:K])
    if n_c:
        K_c = int(b1.K_c.cpu()[0])
        assert K_c == int(b2.K_c.cpu()[0])
        assert np.array_equal(b1.A_c.cpu().numpy()[:K_c], b2.A_c.cpu().numpy()[:K_c])
    y1 = b1.y.cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), b2.y.cpu().numpy().view(np.uint32))
    assert np.array_equal(b1.logits.cpu().numpy().view(np.uint32), b2.logits.cpu().numpy().view(np.uint32))
    assert np.array_equal(y1.view(np.uint32), yi.cpu().numpy().view(np.uint32))
    # against the oracle on the reported x
    logits_or, _ = ph.oracle_predict(spec, x)
    assert np.max(np.abs(b1.logits.cpu().numpy().astype(np.float64) - logits_or)) <= ph.LOGIT_ATOL
    A_g = b1.A_g.cpu().numpy()[:K]
    A_g_or, _ = orc.compact(logits_or, 0.0, spec.T_g, None)
    _, out_g, asc_g = ph.list_check(A_g, A_g_or, spec.T_g, logits_or, 0.0)
    assert K > 0 and out_g == 0 and asc_g
    assert ph.rel_err(y1, ph.oracle_ffn_on_ids(spec, x, spec.T_g[A_g])) <= ph.RTOL
