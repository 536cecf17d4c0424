"""The offline placement solver's per-layer GPU tables run through the layer call on the GPU,
against the oracle: tables of different sizes per layer (the solver splits one GPU budget over
the layers by their profiled activation counts), at reduced size for every layer of a small gated
stack, and at full size on the LLaMA-13B gated stack's layers with the smallest and the largest
solver table.  Also the stack form: the layers in sequence through one set of buffers sized for
the largest table, as a serving loop holds them."""
import numpy as np
import pytest

import synth
from tests import parity_harness as ph
from tests.placement_cases import SMALL, solver_specs

pytestmark = pytest.mark.gpu


def _dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.mark.parametrize("B", [1, 4])
def test_small_stack_with_solver_tables(B):
    _dev()
    specs = solver_specs(SMALL)
    for l, spec in specs.items():
        print(f"[placement] {SMALL.key} layer={l} n_g={spec.n_g} n_c={len(spec.T_c)} B={B}", flush=True)
        r = ph.run_layer_parity(SMALL, layer=l, step=3, B=B, fused=True, spec=spec)
        print(f"[placement]   -> {r}", flush=True)
        ph.assert_report(r)


def test_full_size_layers_with_the_smallest_and_largest_solver_tables():
    _dev()
    cfg = synth.CONFIGS["llama-13b-gated-40"]
    specs = solver_specs(cfg)
    n_g = {l: s.n_g for l, s in specs.items()}
    for l in (min(n_g, key=n_g.get), max(n_g, key=n_g.get)):
        print(f"[placement] {cfg.key} layer={l} n_g={n_g[l]} B=1", flush=True)
        r = ph.run_layer_parity(cfg, layer=l, step=1, B=1, fused=True, spec=specs[l])
        print(f"[placement]   -> {r}", flush=True)
        ph.assert_report(r)


def test_stack_through_shared_buffers():
    """The small stack's layers one after another through pi_ffn_layer with one buffer set (the
    largest table's), each layer's GPU-side output and lists against the oracle."""
    torch = _dev()
    import activation_sparse_amd as pi
    import oracle as orc
    B = 4
    specs = solver_specs(SMALL)
    maxH = max(s.H for s in specs.values())
    n_g = max(s.n_g for s in specs.values())
    n_c = max(len(s.T_c) for s in specs.values())
    buf = ph.DeviceBuffers(SMALL, maxH, n_g, n_c, B)
    dls = {l: ph.DeviceLayer(s) for l, s in specs.items()}
    for l, spec in specs.items():
        x = synth.host_x(SMALL.seed, l, 5, B, SMALL.d)
        buf.x.copy_(torch.from_numpy(x))
        print(f"[placement] stack layer={l} n_g={spec.n_g}", flush=True)
        pi.pi_ffn_layer(dls[l].layer, B, buf.x, 0.0, None, buf.y, buf.logits, buf.A_g, buf.K, buf.A_c, buf.K_c,
                        buf.ws_layer)
        torch.cuda.synchronize()
        K, K_c = int(buf.K.cpu()[0]), int(buf.K_c.cpu()[0])
        A_g, A_c = buf.A_g.cpu().numpy()[:K], buf.A_c.cpu().numpy()[:K_c]
        logits_or, _ = ph.oracle_predict(spec, x)
        A_g_or, A_c_or = orc.compact(logits_or, 0.0, spec.T_g, spec.T_c)
        mis, out, asc = ph.list_check(A_g, A_g_or, spec.T_g, logits_or, 0.0)
        mis_c, out_c, asc_c = ph.list_check(A_c, A_c_or, spec.T_c, logits_or, 0.0)
        assert asc and asc_c and out == 0 and out_c == 0
        assert np.all(A_g < spec.n_g) and np.all(A_c < len(spec.T_c))
        y_or = ph.oracle_ffn_on_ids(spec, x, spec.T_g[A_g])
        err = ph.rel_err(buf.y.cpu().numpy(), y_or)
        print(f"[placement]   -> K={K} K_c={K_c} rel_err={err:.3g}", flush=True)
        assert err <= ph.RTOL
