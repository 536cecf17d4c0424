"""GPU-vs-oracle parity harness for one FFN layer.

Test infrastructure: runs the four C-ABI stages (pi_predict, pi_compact,
pi_sparse_ffn, pi_merge) on seeded synthetic inputs and checks them against
the CPU oracle, which sees the same stored bits.

Parity rule:
  * logits: max |gpu - oracle| reported and bounded (fp32 vs fp64 sums);
  * active lists: ascending, and identical to the oracle's except for neurons
    whose oracle logit lies within BAND of the threshold for some batch row;
  * outputs: the oracle re-runs the FFN on the GPU's own list ("given the same
    mask") and max_b ||y_gpu[b] - y_or[b]||_inf / ||y_or[b]||_inf <= RTOL.
"""
from __future__ import annotations

import math
from dataclasses import replace
from typing import Optional

import numpy as np

import synth
import oracle as orc

BAND = 1e-3
RTOL = 2e-3
LOGIT_ATOL = 1e-4


def small_case(key="small", d=256, N=1024, H=64, wdtype=synth.F16, pdtype=None, bdtype=None, gated=False,
               rho=0.1, alpha=1.1, gpu_frac=1.0, seed=11):
    if pdtype is None:     # int4 FFN weights come with an fp16 predictor unless asked otherwise
        pdtype = synth.F16 if wdtype == synth.I4G128 else wdtype
    if bdtype is None:
        bdtype = synth.F32 if wdtype == synth.F32 else synth.F16
    return synth.small_config(key, d=d, N=N, H=H, wdtype=wdtype, pdtype=pdtype, bdtype=bdtype, gated=gated,
                              rho=rho, alpha=alpha, gpu_frac=gpu_frac, seed=seed)


# ----------------------------------------------------------------------------- device buffers

from synth.device import DeviceLayer, dev_matrix, fill_matrix, dev_vector  # noqa: E402,F401


def _torch():
    import torch
    return torch


class DeviceBuffers:
    """Per-call outputs and workspaces for batch B."""

    def __init__(self, cfg, H, n_g, n_c, B, device="cuda:0"):
        import activation_sparse_amd as pi
        torch = _torch()
        d, N = cfg.d, cfg.N
        self.x = torch.empty((B, d), dtype=torch.float32, device=device)
        self.logits = torch.empty((B, N), dtype=torch.float32, device=device)
        self.A_g = torch.empty(max(n_g, 1), dtype=torch.int32, device=device)
        self.K = torch.empty(1, dtype=torch.int32, device=device)
        self.A_c = torch.empty(max(n_c, 1), dtype=torch.int32, device=device)
        self.K_c = torch.empty(1, dtype=torch.int32, device=device)
        self.y = torch.empty((B, d), dtype=torch.float32, device=device)
        self.y_c = torch.zeros((B, d), dtype=torch.float32, device=device)
        wp = pi.pi_workspace_bytes(pi.PI_OP_PREDICT, B, d, H, N, n_g)
        wf = pi.pi_workspace_bytes(pi.PI_OP_SPARSE_FFN, B, d, H, N, n_g)
        self.ws_pred = torch.empty(max(wp, 256), dtype=torch.uint8, device=device)
        self.ws_ffn = torch.empty(max(wf, 256), dtype=torch.uint8, device=device)
        wl = pi.pi_workspace_bytes(pi.PI_OP_FFN_LAYER, B, d, H, N, n_g)
        self.ws_layer = torch.empty(max(wl, 256), dtype=torch.uint8, device=device)


def run_gpu_layer(dl: DeviceLayer, buf: DeviceBuffers, B: int, tau: float = 0.0, y_c=None, with_cold=True,
                  stream=None):
    """Enqueue the four stages for one layer (no host synchronisation)."""
    import activation_sparse_amd as pi
    spec = dl.spec
    cfg = spec.cfg
    d, N, H, n_g = cfg.d, cfg.N, spec.H, spec.n_g
    n_c = len(spec.T_c)
    pi.pi_predict(B, d, H, N, buf.x, dl.P1, dl.c1, dl.P2, dl.c2, buf.logits, buf.ws_pred, stream=stream)
    cold = with_cold and n_c > 0
    pi.pi_compact(B, N, buf.logits, tau, dl.T_g, n_g, buf.A_g, buf.K, dl.T_c if cold else None, n_c if cold else 0,
                  buf.A_c if cold else None, buf.K_c if cold else None, stream=stream)
    kind = pi.PI_GATED_RELU if cfg.gated else pi.PI_RELU
    pi.pi_sparse_ffn(B, d, n_g, kind, buf.x, dl.W1, dl.b1, dl.Wup, dl.W2, buf.A_g, buf.K, buf.y, buf.ws_ffn,
                     stream=stream)
    if y_c is not None:
        pi.pi_merge(B, d, buf.y, y_c, buf.K_c if cold else None, None, stream=stream)


# ----------------------------------------------------------------------------- oracle side

def host_mat(dtype, seed, tag, layer, cols, sigma, row_ids=None, nrows=None):
    data, scales = synth.host_rows(dtype, seed, tag, layer, cols, sigma, row_ids=row_ids, nrows=nrows)
    return orc.Mat(data, dtype, cols, scales)


def host_vec(stored, dtype):
    return orc.Vec(np.ascontiguousarray(stored), dtype)


def oracle_p2(spec):
    """The output layer's stored weights as the oracle takes them, [N x H].  An int4 predictor
    stores them hidden-major with groups along N: the exact values q * s, transposed back, in
    fp32 (exact: an fp16 scale times a 4-bit integer)."""
    cfg, L, sig = spec.cfg, spec.layer, spec.sigmas()
    if cfg.pdtype != synth.I4G128:
        return host_mat(cfg.pdtype, cfg.seed, synth.TAG_P2, L, spec.H, sig[synth.TAG_P2], nrows=cfg.N)
    v16, _ = synth.host_rows(synth.F16, cfg.seed, synth.TAG_P2, L, spec.H, sig[synth.TAG_P2], nrows=cfg.N)
    packed, scales = synth.i4_quantize_rows(np.ascontiguousarray(v16.T))
    w = synth.i4_dequant(packed, scales)                   # [H x N]
    return orc.Mat(np.ascontiguousarray(w.T.astype(np.float32)), orc.F32, spec.H)


def oracle_predict(spec, x):
    cfg, L, sig = spec.cfg, spec.layer, spec.sigmas()
    P1 = host_mat(cfg.pdtype, cfg.seed, synth.TAG_P1, L, cfg.d, sig[synth.TAG_P1], nrows=spec.H)
    return orc.predict(x, P1, orc.Vec(None, cfg.bdtype), oracle_p2(spec), host_vec(spec.c2, cfg.bdtype),
                       return_hidden=True)


def oracle_ffn_on_ids(spec, x, ids: np.ndarray):
    """FFN over the neurons with original ids `ids` (rows generated for just those)."""
    cfg, L, sig = spec.cfg, spec.layer, spec.sigmas()
    ids = np.ascontiguousarray(ids, np.int32)
    W1 = host_mat(cfg.wdtype, cfg.seed, synth.TAG_W1, L, cfg.d, sig[synth.TAG_W1], row_ids=ids)
    W2 = host_mat(cfg.wdtype, cfg.seed, synth.TAG_W2, L, cfg.d, sig[synth.TAG_W2], row_ids=ids)
    Wup = host_mat(cfg.wdtype, cfg.seed, synth.TAG_WUP, L, cfg.d, sig[synth.TAG_WUP], row_ids=ids) if cfg.gated else None
    b1 = host_vec(spec.b1[ids] if len(ids) else spec.b1[:1], cfg.bdtype)
    kind = orc.GATED_RELU if cfg.gated else orc.RELU
    return orc.sparse_ffn(x, W1, b1, W2, np.arange(len(ids), dtype=np.int32), kind=kind, Wup=Wup)


def list_check(A_gpu: np.ndarray, A_or: np.ndarray, table: np.ndarray, logits_or: np.ndarray, tau: float):
    """Returns (n_mismatch, n_outside_band, ascending)."""
    asc = bool(np.all(np.diff(A_gpu) > 0)) if len(A_gpu) > 1 else True
    sd = np.setxor1d(A_gpu, A_or)
    if len(sd) == 0:
        return 0, 0, asc
    ids = table[sd]
    dist = np.min(np.abs(logits_or[:, ids] - tau), axis=0)
    return int(len(sd)), int(np.sum(dist > BAND)), asc


def rel_err(y_gpu: np.ndarray, y_or: np.ndarray) -> float:
    worst = 0.0
    for b in range(y_or.shape[0]):
        den = float(np.max(np.abs(y_or[b])))
        num = float(np.max(np.abs(y_gpu[b].astype(np.float64) - y_or[b])))
        if den == 0.0:
            if num != 0.0:
                return math.inf
            continue
        worst = max(worst, num / den)
    return worst


def _gpu_stages(dl, buf, B, tau, with_cold, fused, y_c=None):
    """Run the layer on the GPU; fused = one pi_ffn_layer call, else the four calls."""
    import activation_sparse_amd as pi
    spec = dl.spec
    cold = with_cold and len(spec.T_c) > 0
    if fused:
        layer = dl.layer
        if layer.cold != cold:
            from dataclasses import replace as _r
            layer = _r(layer, cold=cold)
        ws = buf.ws_layer
        pi.pi_ffn_layer(layer, B, buf.x, tau, y_c, buf.y, buf.logits, buf.A_g, buf.K, buf.A_c if cold else None,
                        buf.K_c if cold else None, ws)
    else:
        run_gpu_layer(dl, buf, B, tau, y_c=None, with_cold=with_cold)
        if y_c is not None:
            pi.pi_merge(B, spec.cfg.d, buf.y, y_c, buf.K_c if cold else None, None)


def run_layer_parity(cfg: synth.Config, layer: int = 0, step: int = 0, B: int = 1, tau: float = 0.0,
                     device="cuda:0", with_cold=True, x_override: Optional[np.ndarray] = None,
                     tau_all_active: bool = False, fused: bool = False, spec: Optional[synth.LayerSpec] = None):
    """Full parity of one layer at batch B; returns a report dict.  spec, when given, replaces
    the config's own spec of the layer (another GPU table, e.g. the placement solver's)."""
    torch = _torch()
    if spec is None:
        spec = synth.layer_spec(cfg, layer)
    d, N = cfg.d, cfg.N
    n_c = len(spec.T_c)
    x = synth.host_x(cfg.seed, layer, step, B, d) if x_override is None else np.ascontiguousarray(x_override, np.float32)
    if tau_all_active:
        tau = -3.0e38
    dl = DeviceLayer(spec, device)
    buf = DeviceBuffers(cfg, spec.H, spec.n_g, n_c, B, device)
    buf.x.copy_(torch.from_numpy(x))
    _gpu_stages(dl, buf, B, tau, with_cold, fused)
    torch.cuda.synchronize()
    logits_gpu = buf.logits.cpu().numpy()
    K = int(buf.K.cpu()[0])
    A_g = buf.A_g.cpu().numpy()[:K].copy()
    y_g_gpu = buf.y.cpu().numpy().copy()
    cold = with_cold and n_c > 0
    K_c = int(buf.K_c.cpu()[0]) if cold else 0
    A_c = buf.A_c.cpu().numpy()[:K_c].copy() if cold else np.zeros(0, np.int32)

    logits_or, h_or = oracle_predict(spec, x)
    A_g_or, A_c_or = orc.compact(logits_or, tau, spec.T_g, spec.T_c if cold else None)
    mis_g, out_g, asc_g = list_check(A_g, A_g_or, spec.T_g, logits_or, tau)
    mis_c, out_c, asc_c = (0, 0, True)
    if cold:
        mis_c, out_c, asc_c = list_check(A_c, A_c_or, spec.T_c, logits_or, tau)

    y_g_or = oracle_ffn_on_ids(spec, x, spec.T_g[A_g])
    report = dict(cfg=cfg.key, layer=layer, step=step, B=B, fused=fused, K=K, K_c=K_c, n_g=spec.n_g,
                  logit_max_abs_err=float(np.max(np.abs(logits_gpu.astype(np.float64) - logits_or))),
                  list_mismatch=mis_g + mis_c, list_outside_band=out_g + out_c, ascending=asc_g and asc_c,
                  rel_err_ffn=rel_err(y_g_gpu, y_g_or))
    y_final_or = y_g_or
    if cold:
        y_c_or = oracle_ffn_on_ids(spec, x, spec.T_c[A_c])
        y_c32 = y_c_or.astype(np.float32)
        buf.y_c.copy_(torch.from_numpy(y_c32))
        if fused:
            _gpu_stages(dl, buf, B, tau, with_cold, fused, y_c=buf.y_c)
        else:
            import activation_sparse_amd as pi
            pi.pi_merge(B, d, buf.y, buf.y_c, buf.K_c, None)
        torch.cuda.synchronize()
        if fused:   # the second call recomputes everything: its lists must be the same
            assert int(buf.K.cpu()[0]) == K and np.array_equal(buf.A_g.cpu().numpy()[:K], A_g)
            assert int(buf.K_c.cpu()[0]) == K_c
        y_final_or = orc.merge(y_g_or, y_c32.astype(np.float64), K_c)
    report["rel_err"] = rel_err(buf.y.cpu().numpy(), y_final_or)
    report["y_norm"] = float(np.max(np.abs(y_final_or))) if y_final_or.size else 0.0
    return report


def assert_report(r: dict) -> None:
    assert r["ascending"], r
    assert r["list_outside_band"] == 0, r
    assert r["logit_max_abs_err"] <= LOGIT_ATOL, r
    assert r["rel_err_ffn"] <= RTOL, r
    assert r["rel_err"] <= RTOL, r


# ----------------------------------------------------------------------------- attention blocks

def attn_oracle_inputs(h: dict, d: int):
    """Oracle matrices and vectors of an attention block from synth.attn_host's fp16 bits."""
    M = lambda k, cols: orc.Mat(h[k], orc.F16, cols)
    V = lambda k: orc.Vec(h[k], orc.F16)
    return dict(Pa1=M("Pa1", d), ca1=orc.Vec(None, orc.F16), Pa2=M("Pa2", h["Pa1"].shape[0]), ca2=V("ca2"),
                Wq=M("Wq", d), bq=V("bq"), Wk=M("Wk", d), bk=V("bk"), Wv=M("Wv", d), bv=V("bv"), WoT=M("WoT", d),
                bo=V("bo"))


def f16_ulps(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in fp16 units in the last place between two arrays of finite fp16 bits."""
    def key(u):
        u = u.astype(np.int32)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(key(np.asarray(a, np.uint16)) - key(np.asarray(b, np.uint16)))


def run_attn_parity(cfg, layer: int = 0, t: int = 0, step: int = 0, tau: float = 0.0, device="cuda:0",
                    dl=None, host=None):
    """One decode step of an attention block on the GPU (pi_attn_decode) against the oracle: head
    logits, the head list (exact outside the 1e-3 band around tau), y given the GPU's head set,
    this position's cache entry (normwise within 1e-3 of the oracle's, about two fp16 units at its
    largest element) and every other cache position untouched.  Returns a report dict."""
    torch = _torch()
    import activation_sparse_amd as pi
    spec = synth.attn_spec(cfg, layer)
    h = host if host is not None else synth.attn_host(spec)
    if dl is None:
        dl = synth.device.DeviceAttn(spec, device)
    d, nh = cfg.d, cfg.n_heads
    x = synth.attn_x(cfg, layer, step)
    Kc0 = dl.caches[0].cpu().numpy().view(np.uint16).copy()
    Vc0 = dl.caches[1].cpu().numpy().view(np.uint16).copy()
    xd = torch.from_numpy(x).to(device)
    y = torch.empty(d, dtype=torch.float32, device=device)
    lg = torch.empty(nh, dtype=torch.float32, device=device)
    heads = torch.full((nh,), -1, dtype=torch.int32, device=device)
    na = torch.zeros(1, dtype=torch.int32, device=device)
    ws = torch.empty(max(pi.pi_attn_workspace_bytes(dl.attn), 256), dtype=torch.uint8, device=device)
    pi.pi_attn_decode(dl.attn, t, xd, tau, y, lg, heads, na, ws, _cstruct=dl.attn_c)
    torch.cuda.synchronize()
    n_act = int(na.cpu()[0])
    heads_gpu = heads.cpu().numpy()[:n_act].copy()
    Kc = dl.caches[0].cpu().numpy().view(np.uint16)
    Vc = dl.caches[1].cpu().numpy().view(np.uint16)
    o = attn_oracle_inputs(h, d)
    ref = orc.attn_decode(x, o["Pa1"], o["ca1"], o["Pa2"], o["ca2"], tau, o["Wq"], o["bq"], o["Wk"], o["bk"], o["Wv"],
                          o["bv"], o["WoT"], o["bo"], Kc0, Vc0, nh, cfg.dh, t)
    logits_gpu = lg.cpu().numpy()
    band = np.abs(ref["head_logits"] - tau) < 1e-3
    on_gpu = np.zeros(nh, bool)
    on_gpu[heads_gpu] = True
    on_or = np.zeros(nh, bool)
    on_or[ref["heads"]] = True
    report = dict(cfg=cfg.key, layer=layer, t=t, n_active=n_act, n_active_oracle=len(ref["heads"]),
                  logit_max_abs_err=float(np.max(np.abs(logits_gpu.astype(np.float64) - ref["head_logits"]))),
                  list_outside_band=int(np.sum((on_gpu != on_or) & ~band)),
                  ascending=bool(np.all(np.diff(heads_gpu) > 0)))
    if not np.array_equal(on_gpu, on_or):
        # the oracle again with the GPU's head set (output-bias sentinels select it)
        ca2 = orc.Vec(np.where(on_gpu, 30000.0, -30000.0).astype(np.float16).view(np.uint16), orc.F16)
        ref = orc.attn_decode(x, o["Pa1"], o["ca1"], o["Pa2"], ca2, 0.0, o["Wq"], o["bq"], o["Wk"], o["bk"], o["Wv"],
                              o["bv"], o["WoT"], o["bo"], Kc0, Vc0, nh, cfg.dh, t)
    report["rel_err"] = rel_err(y.cpu().numpy()[None, :], ref["y"][None, :])
    report["cache_ulps"] = int(max(f16_ulps(Kc[:, t].reshape(-1), ref["k_new"]).max(),
                                   f16_ulps(Vc[:, t].reshape(-1), ref["v_new"]).max()))
    # normwise: entries near zero may sit several fp16 units from the oracle's rounding, since an
    # fp32 dot product over d terms errs by far more than one fp16 unit of a small value
    f = lambda b: np.asarray(b, np.uint16).view(np.float16).astype(np.float64)
    report["cache_rel_err"] = float(max(
        np.max(np.abs(f(Kc[:, t].reshape(-1)) - f(ref["k_new"]))) / np.max(np.abs(f(ref["k_new"]))),
        np.max(np.abs(f(Vc[:, t].reshape(-1)) - f(ref["v_new"]))) / np.max(np.abs(f(ref["v_new"])))))
    others = np.ones(cfg.L_max, bool)
    others[t] = False
    report["cache_others_untouched"] = bool(np.array_equal(Kc[:, others], Kc0[:, others]) and
                                            np.array_equal(Vc[:, others], Vc0[:, others]))
    return report


def assert_attn_report(r: dict) -> None:
    assert r["ascending"], r
    assert r["list_outside_band"] == 0, r
    assert r["logit_max_abs_err"] <= LOGIT_ATOL, r
    assert r["rel_err"] <= RTOL, r
    assert r["cache_rel_err"] <= 1e-3, r
    assert r["cache_others_untouched"], r
