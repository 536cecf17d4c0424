"""pi_ffn_layer_static, the layer call that allocates nothing (its workspace is a static device
array inside libpi), against pi_ffn_layer with a caller workspace: the same bits, on two calls in a
row, the second with a smaller layer; and a layer too large for the static array is refused."""
import numpy as np
import pytest

import synth
from tests import parity_harness as ph

pytestmark = pytest.mark.gpu


def _run(cfg, layer, step, B, static):
    import torch
    import activation_sparse_amd as pi
    from synth.device import DeviceLayer
    spec = synth.layer_spec(cfg, layer)
    dl = DeviceLayer(spec, "cuda:0")
    buf = ph.DeviceBuffers(cfg, spec.H, spec.n_g, len(spec.T_c), B, "cuda:0")
    buf.x.copy_(torch.from_numpy(synth.host_x(cfg.seed, layer, step, B, cfg.d)))
    cold = len(spec.T_c) > 0
    if cold:
        buf.y_c.copy_(torch.from_numpy(synth.host_yc(cfg.seed, layer, step, B, cfg.d, 0.05)))
    args = (dl.layer, B, buf.x, 0.0, buf.y_c if cold else None, buf.y, buf.logits, buf.A_g, buf.K,
            buf.A_c if cold else None, buf.K_c if cold else None)
    print(f"[no-alloc] {cfg.key} layer {layer} step {step} B {B} static={static}", flush=True)
    if static:
        pi.pi_ffn_layer_static(*args)
    else:
        pi.pi_ffn_layer(*args, buf.ws_layer)
    torch.cuda.synchronize()
    K = int(buf.K.cpu()[0])
    K_c = int(buf.K_c.cpu()[0]) if cold else 0
    return dict(y=buf.y.cpu().numpy().copy(), logits=buf.logits.cpu().numpy().copy(), K=K, K_c=K_c,
                A_g=buf.A_g.cpu().numpy()[:K].copy(), A_c=buf.A_c.cpu().numpy()[:K_c].copy() if cold else None)


def _same(a, b):
    assert a["K"] == b["K"] and a["K_c"] == b["K_c"]
    assert np.array_equal(a["A_g"], b["A_g"])
    assert (a["A_c"] is None) == (b["A_c"] is None) and (a["A_c"] is None or np.array_equal(a["A_c"], b["A_c"]))
    assert a["y"].tobytes() == b["y"].tobytes()
    assert a["logits"].tobytes() == b["logits"].tobytes()


def test_static_workspace_call_matches_the_workspace_call():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import activation_sparse_amd as pi
    # a full OPT-30B layer at batch 4 (12.8 MB of workspace), then a smaller layer at batch 1: the
    # second call finds the first one's contents in the array
    cases = [(synth.CONFIGS["opt-30b"], 3, 5, 4), (ph.small_case("no-alloc-small", d=512, N=2048, H=128), 0, 1, 1)]
    for cfg, layer, step, B in cases:
        need = pi.pi_workspace_bytes(pi.PI_OP_FFN_LAYER, B, cfg.d, synth.layer_spec(cfg, layer).H, cfg.N,
                                     synth.layer_spec(cfg, layer).n_g)
        assert need <= pi.PI_STATIC_WORKSPACE_BYTES
        ref = _run(cfg, layer, step, B, static=False)
        got = _run(cfg, layer, step, B, static=True)
        _same(ref, got)
    # a layer whose workspace exceeds the array is refused before anything is enqueued
    cfg = synth.CONFIGS["opt-30b"]
    spec = synth.layer_spec(cfg, 0)
    assert pi.pi_workspace_bytes(pi.PI_OP_FFN_LAYER, 32, cfg.d, spec.H, cfg.N, spec.n_g) > pi.PI_STATIC_WORKSPACE_BYTES
    from synth.device import DeviceLayer
    dl = DeviceLayer(spec, "cuda:0")
    buf = ph.DeviceBuffers(cfg, spec.H, spec.n_g, len(spec.T_c), 32, "cuda:0")
    with pytest.raises(pi.PiError, match="PI_EWORKSPACE"):
        pi.pi_ffn_layer_static(dl.layer, 32, buf.x, 0.0, buf.y_c, buf.y, buf.logits, buf.A_g, buf.K, buf.A_c, buf.K_c)
