"""Device-resident synthetic layers (weights generated on the GPU).

Input generation only: allocates torch device tensors and fills them with the
same bits the host generator produces.  Used by the GPU tests and the
benchmark.
"""
from __future__ import annotations

import numpy as np

import synth
from activation_sparse_amd import Matrix, Vector, PI_F32, PI_F16, PI_I4G128


def _torch():
    import torch
    return torch


def dev_matrix(rows, cols, dtype, device):
    torch = _torch()
    if dtype == synth.F32:
        return Matrix(torch.empty((rows, cols), dtype=torch.float32, device=device), PI_F32)
    if dtype == synth.F16:
        return Matrix(torch.empty((rows, cols), dtype=torch.float16, device=device), PI_F16)
    return Matrix(torch.empty((rows, cols // 2), dtype=torch.uint8, device=device), PI_I4G128,
                  torch.empty((rows, cols // 128), dtype=torch.int16, device=device))


def fill_matrix(m, dtype, seed, tag, layer, cols, sigma, row_ids_dev=None, nrows=None):
    torch = _torch()
    n = m.data.shape[0] if nrows is None else nrows
    synth.dev_fill(m.data.data_ptr(), m.scales.data_ptr() if m.scales is not None else None, dtype, seed, tag,
                   layer, cols, sigma, row_ids_ptr=row_ids_dev.data_ptr() if row_ids_dev is not None else None,
                   nrows=n, stream=torch.cuda.current_stream().cuda_stream)


def i4_quantize_rows_dev(t16):
    """Device twin of synth.i4_quantize_rows (same rule, fp32 arithmetic): fp16 tensor
    [rows, cols] -> Matrix int4-g128 (uint8 [rows, cols/2], int16 scales [rows, cols/128])."""
    torch = _torch()
    rows, cols = t16.shape
    g = t16.float().view(rows, cols // 128, 128)
    s = (g.abs().amax(dim=2) / 7.0).half()
    sf = s.float().unsqueeze(2)
    safe = torch.where(sf > 0, sf, torch.ones_like(sf))
    q = torch.where(sf > 0, torch.round(g / safe).clamp(-8, 7), torch.zeros_like(g)).to(torch.int16).view(rows, cols)
    packed = ((q[:, 0::2] & 0xF) | ((q[:, 1::2] & 0xF) << 4)).to(torch.uint8)
    return Matrix(packed.contiguous(), PI_I4G128, s.view(torch.int16).contiguous())


def dev_matrix_hidden_major(N, H, dtype, seed, tag, layer, sigma, device):
    """The [N x H] generated matrix stored transposed, [H x N] (fp32 / fp16 bits unchanged).
    int4: the fp16 values, transposed, then quantised in groups of 128 along N."""
    torch = _torch()
    gen = synth.F16 if dtype == synth.I4G128 else dtype
    tmp = dev_matrix(N, H, gen, device)
    fill_matrix(tmp, gen, seed, tag, layer, H, sigma)
    out = Matrix(tmp.data.t().contiguous(), tmp.dtype)
    del tmp
    if dtype == synth.I4G128:
        out = i4_quantize_rows_dev(out.data)
    torch.cuda.current_stream().synchronize()
    return out


def dev_vector(stored: np.ndarray, dtype: int, device):
    torch = _torch()
    if dtype == synth.F32:
        return Vector(torch.from_numpy(np.ascontiguousarray(stored, np.float32)).to(device), PI_F32)
    t = torch.from_numpy(np.ascontiguousarray(stored).view(np.int16)).to(device).view(torch.float16)
    return Vector(t, PI_F16)


class DeviceLayer:
    """One layer's GPU-resident tensors, generated on the device."""

    def __init__(self, spec: synth.LayerSpec, device="cuda:0"):
        torch = _torch()
        cfg, L = spec.cfg, spec.layer
        sig = spec.sigmas()
        self.spec = spec
        d, N, H, n_g = cfg.d, cfg.N, spec.H, spec.n_g
        self.T_g = torch.from_numpy(spec.T_g).to(device)
        self.T_c = torch.from_numpy(spec.T_c).to(device) if len(spec.T_c) else None
        self.P1 = dev_matrix(H, d, cfg.pdtype, device)
        fill_matrix(self.P1, cfg.pdtype, cfg.seed, synth.TAG_P1, L, d, sig[synth.TAG_P1])
        # the output layer's weights P2[i, m] (neuron i, hidden unit m) are generated
        # row by row per neuron and stored hidden-major, [H, N]
        self.P2 = dev_matrix_hidden_major(N, H, cfg.pdtype, cfg.seed, synth.TAG_P2, L, sig[synth.TAG_P2], device)
        self.c1 = None
        self.c2 = dev_vector(spec.c2, cfg.bdtype, device)
        self.W1 = dev_matrix(max(n_g, 1), d, cfg.wdtype, device)
        self.W2 = dev_matrix(max(n_g, 1), d, cfg.wdtype, device)
        self.Wup = dev_matrix(max(n_g, 1), d, cfg.wdtype, device) if cfg.gated else None
        if n_g:
            fill_matrix(self.W1, cfg.wdtype, cfg.seed, synth.TAG_W1, L, d, sig[synth.TAG_W1], self.T_g, n_g)
            fill_matrix(self.W2, cfg.wdtype, cfg.seed, synth.TAG_W2, L, d, sig[synth.TAG_W2], self.T_g, n_g)
            if cfg.gated:
                fill_matrix(self.Wup, cfg.wdtype, cfg.seed, synth.TAG_WUP, L, d, sig[synth.TAG_WUP], self.T_g, n_g)
        self.b1 = dev_vector(spec.b1[spec.T_g] if n_g else spec.b1[:1], cfg.bdtype, device)
        from activation_sparse_amd import pi_table_prepare, Layer, PI_RELU, PI_GATED_RELU
        self.table = torch.from_numpy(pi_table_prepare(N, spec.T_g)).to(device)
        self.layer = Layer(d, N, H, n_g, PI_GATED_RELU if cfg.gated else PI_RELU, len(spec.T_c) > 0, self.P1,
                           self.c1, self.P2, self.c2, self.table, self.W1, self.b1, self.Wup, self.W2, None)
        self.layer_c = self.layer._c()




class HostColdLayer:
    """One layer's CPU-resident (cold) neurons in host memory, generated on the device
    (the same bits as the host generator) and copied out: W1, W2 (and Wup) rows of the
    CPU table's neurons in CPU-table slot order, and their b1."""

    def __init__(self, spec: synth.LayerSpec, device="cuda:0"):
        torch = _torch()
        cfg, L = spec.cfg, spec.layer
        sig = spec.sigmas()
        d, n_c = cfg.d, len(spec.T_c)
        self.n_c = n_c
        T_c = torch.from_numpy(spec.T_c).to(device)

        def host_rows(tag):
            m = dev_matrix(max(n_c, 1), d, cfg.wdtype, device)
            if n_c:
                fill_matrix(m, cfg.wdtype, cfg.seed, tag, L, d, sig[tag], T_c, n_c)
            out = Matrix(m.data.cpu(), m.dtype, m.scales.cpu() if m.scales is not None else None)
            del m
            return out
        self.W1 = host_rows(synth.TAG_W1)
        self.W2 = host_rows(synth.TAG_W2)
        self.Wup = host_rows(synth.TAG_WUP) if cfg.gated else None
        b = np.ascontiguousarray(spec.b1[spec.T_c] if n_c else spec.b1[:1])
        self.b1 = Vector(b if cfg.bdtype == synth.F32 else b.view(np.uint16), PI_F32 if cfg.bdtype == synth.F32 else PI_F16)


class DeviceAttn:
    """One attention block's weights and caches, generated on the device (the host's bits)."""

    def __init__(self, spec: synth.AttnSpec, device="cuda:0"):
        torch = _torch()
        from activation_sparse_amd import Attn, Matrix as M, Vector as V, PI_F16
        c, L, sg = spec.cfg, spec.layer, spec.sigmas()
        self.spec = spec
        mats = {}
        for name, tag, rows, cols in (("Pa1", synth.TAG_PA1, c.Ha, c.d), ("Pa2", synth.TAG_PA2, c.n_heads, c.Ha),
                                      ("Wq", synth.TAG_WQ, c.d, c.d), ("Wk", synth.TAG_WK, c.d, c.d),
                                      ("Wv", synth.TAG_WV, c.d, c.d), ("WoT", synth.TAG_WO, c.d, c.d)):
            m = dev_matrix(rows, cols, synth.F16, device)
            fill_matrix(m, synth.F16, c.seed, tag, L, cols, sg[tag])
            mats[name] = m
        bias = dev_matrix(4, c.d, synth.F16, device)
        fill_matrix(bias, synth.F16, c.seed, synth.TAG_ABIAS, L, c.d, sg[synth.TAG_ABIAS])
        self.bias = bias
        self.caches = []
        for tag in (synth.TAG_KC, synth.TAG_VC):
            m = dev_matrix(c.n_heads * c.L_max, c.dh, synth.F16, device)
            fill_matrix(m, synth.F16, c.seed, tag, L, c.dh, 1.0)
            self.caches.append(m.data.view(c.n_heads, c.L_max, c.dh))
        self.ca2 = dev_vector(spec.ca2, synth.F16, device)
        self.mats = mats
        self.attn = Attn(c.d, c.n_heads, c.dh, c.Ha, c.L_max, mats["Pa1"], mats["Pa2"], mats["Wq"], mats["Wk"],
                         mats["Wv"], mats["WoT"], self.caches[0], self.caches[1], ca1=None, ca2=self.ca2,
                         bq=V(bias.data[0], PI_F16), bk=V(bias.data[1], PI_F16), bv=V(bias.data[2], PI_F16),
                         bo=V(bias.data[3], PI_F16))
        self.attn_c = self.attn._c()
