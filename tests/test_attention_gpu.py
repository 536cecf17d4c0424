"""GPU parity of the self-attention block with head sparsity (pi_attn_decode) against the oracle:
reduced shapes at head sizes 64 and 128 over positions that leave the 64-position chunks full,
ragged or single, the last cache position, every head active and none, consecutive decode steps
that read the entries the earlier steps wrote, repeatability, and the OPT-30B shape at full size
(56 heads x 128, 1,024 cached positions)."""
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
    print(f"[attn] cfg={cfg.key} d={cfg.d} heads={cfg.n_heads}x{cfg.dh} kw={ {k: v for k, v in kw.items() if k not in ('dl', 'host')} }",
          flush=True)
    r = ph.run_attn_parity(cfg, **kw)
    print(f"[attn]   -> {r}", flush=True)
    ph.assert_attn_report(r)
    return r


def test_device_generator_matches_host_bits():
    torch = _dev()
    cfg = synth.ATTN_CONFIGS["attn-small"]
    spec = synth.attn_spec(cfg, 1)
    h = synth.attn_host(spec)
    dl = synth.device.DeviceAttn(spec)
    torch.cuda.synchronize()
    for name in ("Pa1", "Pa2", "Wq", "Wk", "Wv", "WoT"):
        assert np.array_equal(dl.mats[name].data.cpu().numpy().view(np.uint16), h[name]), name
    assert np.array_equal(dl.caches[0].cpu().numpy().view(np.uint16), h["Kc"])
    assert np.array_equal(dl.caches[1].cpu().numpy().view(np.uint16), h["Vc"])
    assert np.array_equal(dl.bias.data.cpu().numpy().view(np.uint16)[3], h["bo"])


@pytest.mark.parametrize("key,layer,t", [("attn-small", 0, 0), ("attn-small", 0, 1), ("attn-small", 1, 63),
                                         ("attn-small", 1, 64), ("attn-small", 0, 65), ("attn-small", 1, 200),
                                         ("attn-small", 0, 255), ("attn-mid", 0, 0), ("attn-mid", 1, 127),
                                         ("attn-mid", 0, 199)])
def test_attention_parity(key, layer, t):
    _dev()
    _run(synth.ATTN_CONFIGS[key], layer=layer, t=t, step=t % 7)


@pytest.mark.parametrize("tau,expect", [(-3.0e38, "all"), (3.0e38, "none")])
def test_every_head_and_no_head(tau, expect):
    _dev()
    cfg = synth.ATTN_CONFIGS["attn-mid"]
    r = _run(cfg, layer=1, t=150, tau=tau)
    assert r["n_active"] == (cfg.n_heads if expect == "all" else 0)


def test_consecutive_steps_read_what_the_earlier_steps_wrote():
    torch = _dev()
    cfg = synth.ATTN_CONFIGS["attn-small"]
    spec = synth.attn_spec(cfg, 0)
    h = synth.attn_host(spec)
    dl = synth.device.DeviceAttn(spec)
    torch.cuda.synchronize()
    for s, t in enumerate((100, 101, 102, 103)):
        _run(cfg, layer=0, t=t, step=s, dl=dl, host=h)


def test_repeatable_bits():
    torch = _dev()
    import activation_sparse_amd as pi
    cfg = synth.ATTN_CONFIGS["attn-mid"]
    dl = synth.device.DeviceAttn(synth.attn_spec(cfg, 0))
    x = torch.from_numpy(synth.attn_x(cfg, 0, 3)).cuda()
    ws = torch.empty(pi.pi_attn_workspace_bytes(dl.attn), dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(3):
        y = torch.empty(cfg.d, dtype=torch.float32, device="cuda")
        heads = torch.empty(cfg.n_heads, dtype=torch.int32, device="cuda")
        na = torch.empty(1, dtype=torch.int32, device="cuda")
        pi.pi_attn_decode(dl.attn, 190, x, 0.0, y, None, heads, na, ws, _cstruct=dl.attn_c)
        torch.cuda.synchronize()
        n = int(na.cpu()[0])
        outs.append((y.cpu().numpy().view(np.uint32).copy(), heads.cpu().numpy()[:n].copy()))
    for o in outs[1:]:
        assert np.array_equal(o[0], outs[0][0]) and np.array_equal(o[1], outs[0][1])


@pytest.mark.parametrize("layer,t", [(0, 1023), (7, 1000)])
def test_opt30b_attention_full_size(layer, t):
    _dev()
    r = _run(synth.ATTN_CONFIGS["attn-opt-30b"], layer=layer, t=t, step=1)
    assert 0 < r["n_active"] < 56
