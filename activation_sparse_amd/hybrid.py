"""The pages' GPU-CPU hybrid layer: buffers for the native executor.

Per layer and step (CSDN summary of "PowerInfer: Fast Large Language Model
Serving with a Consumer-grade GPU", section GPU-CPU混合执行) the executor in
libpi_host (pi_hybrid_layer, include/pi_host.h) runs the GPU's predictor and
compaction, copies x and the CPU-table list to the host, enqueues the GPU's own
neurons, computes the cold neurons on the host while those run, and merges the
CPU's partial on the GPU, skipping the copy and the merge when no cold neuron
is active (the pages' selective synchronisation).

This class only allocates the executor's buffers (torch device memory, pinned
host memory and an event) and marshals the call.
"""
from __future__ import annotations

import activation_sparse_amd as pi
from activation_sparse_amd import host


class HybridLayer:
    """One layer split between a DeviceLayer-like object (dl: the predictor and the
    GPU-resident neurons, with T_g / T_c device tables and its pi_layer struct) and a
    host object (hl: the CPU-resident neurons' W1, b1, W2, Wup in host memory), for
    batch B."""

    def __init__(self, dl, hl, B: int, threads: int = 0, device="cuda:0"):
        import torch
        spec = dl.spec
        cfg = spec.cfg
        self.dl, self.hl, self.B, self.threads = dl, hl, B, threads
        self.d, self.N, self.H, self.n_g, self.n_c = cfg.d, cfg.N, spec.H, spec.n_g, len(spec.T_c)
        i32, f32 = torch.int32, torch.float32
        self.logits = torch.empty((B, self.N), dtype=f32, device=device)
        self.A_g = torch.empty(max(self.n_g, 1), dtype=i32, device=device)
        self.K = torch.zeros(1, dtype=i32, device=device)
        self.cold_list = torch.zeros(4 + max(self.n_c, 1), dtype=i32, device=device)
        self.y_c = torch.empty((B, self.d), dtype=f32, device=device)
        wsp = max(pi.pi_workspace_bytes(pi.PI_OP_PREDICT, B, self.d, self.H, self.N, 0), 256)
        wsf = max(pi.pi_workspace_bytes(pi.PI_OP_SPARSE_FFN, B, self.d, 0, 0, self.n_g), 256)
        self.ws_pred = torch.empty(wsp, dtype=torch.uint8, device=device)
        self.ws_ffn = torch.empty(wsf, dtype=torch.uint8, device=device)
        self.x_h = torch.empty((B, self.d), dtype=f32, pin_memory=True)
        self.cold_list_h = torch.zeros(4 + max(self.n_c, 1), dtype=i32, pin_memory=True)
        self.y_c_h = torch.empty((B, self.d), dtype=f32, pin_memory=True)
        self.event = torch.cuda.Event()
        self.event.record()            # creates the underlying hipEvent_t
        self.scratch = host._HybridScratch(
            self.logits.data_ptr(), self.A_g.data_ptr(), self.K.data_ptr(), self.cold_list.data_ptr(),
            self.y_c.data_ptr(), self.ws_pred.data_ptr(), wsp, self.ws_ffn.data_ptr(), wsf, self.x_h.data_ptr(),
            self.cold_list_h.data_ptr(), self.y_c_h.data_ptr(), self.event.cuda_event)
        self.cold = None
        if self.n_c:
            self.cold = host._HostCold(self.n_c, host._hmat(hl.W1), host._hvec(hl.b1), host._hmat(hl.Wup),
                                       host._hmat(hl.W2))
        self.T_g = dl.T_g.data_ptr()
        self.T_c = dl.T_c.data_ptr() if self.n_c else None

    @property
    def K_c_h(self):
        """The last call's K_c (pinned host)."""
        return self.cold_list_h[:1]

    @property
    def A_c_h(self):
        """The last call's CPU list (pinned host; the first K_c entries are valid)."""
        return self.cold_list_h[4:]

    def __call__(self, x, y, tau: float = 0.0, stream=None) -> int:
        """y [B x d] (device) = the layer's output for x [B x d] (device); returns the number
        of active cold neurons (0: no cold partial was merged)."""
        return host.pi_hybrid_layer(pi._stream(stream), self.dl.layer_c, self.T_g, self.T_c, self.cold, self.B,
                                    x.data_ptr(), tau, y.data_ptr(), self.scratch, self.threads)


class HybridStack:
    """The look-ahead hybrid over a stack of layers (pi_hybrid_prime / pi_hybrid_layer_ahead): each
    layer's neurons are predicted from the previous layer's input while the CPU computes that
    layer's cold neurons.  dls / hls: DeviceLayer-like and host objects per layer, as for
    HybridLayer.  One scratch serves every layer (sized for the largest)."""

    def __init__(self, dls, hls, B: int, threads: int = 0, device="cuda:0"):
        import torch
        self.dls, self.hls, self.B, self.threads = dls, hls, B, threads
        specs = [dl.spec for dl in dls]
        cfg = specs[0].cfg
        self.d = cfg.d
        N = max(s.cfg.N for s in specs)
        H = max(s.H for s in specs)
        n_g = max(s.n_g for s in specs)
        self.n_cs = [len(s.T_c) for s in specs]
        n_c = max(self.n_cs)
        i32, f32 = torch.int32, torch.float32
        self.logits = torch.empty((B, N), dtype=f32, device=device)
        wsp = max(pi.pi_workspace_bytes(pi.PI_OP_PREDICT, B, self.d, H, N, 0), 256)
        wsf = max(pi.pi_workspace_bytes(pi.PI_OP_SPARSE_FFN, B, self.d, 0, 0, n_g), 256)
        self.ws_pred = torch.empty(wsp, dtype=torch.uint8, device=device)
        self.ws_ffn = torch.empty(wsf, dtype=torch.uint8, device=device)
        self.A_g = [torch.empty(max(n_g, 1), dtype=i32, device=device) for _ in range(2)]
        self.K = [torch.zeros(1, dtype=i32, device=device) for _ in range(2)]
        self.cold_list = [torch.zeros(4 + max(n_c, 1), dtype=i32, device=device) for _ in range(2)]
        self.cold_list_h = [torch.zeros(4 + max(n_c, 1), dtype=i32, pin_memory=True) for _ in range(2)]
        self.y_c = torch.empty((B, self.d), dtype=f32, device=device)
        self.x_h = torch.empty((B, self.d), dtype=f32, pin_memory=True)
        self.y_c_h = torch.empty((B, self.d), dtype=f32, pin_memory=True)
        self.events = [torch.cuda.Event() for _ in range(3)]
        for e in self.events:
            e.record()                 # creates the underlying hipEvent_t
        P2 = host.C.c_void_p * 2
        self.scratch = host._HybridAheadScratch(
            self.logits.data_ptr(), self.ws_pred.data_ptr(), wsp, self.ws_ffn.data_ptr(), wsf,
            P2(*(t.data_ptr() for t in self.A_g)), P2(*(t.data_ptr() for t in self.K)),
            P2(*(t.data_ptr() for t in self.cold_list)), P2(*(t.data_ptr() for t in self.cold_list_h)),
            P2(self.events[0].cuda_event, self.events[1].cuda_event), self.y_c.data_ptr(), self.x_h.data_ptr(),
            self.y_c_h.data_ptr(), self.events[2].cuda_event, 0)
        self.colds = [host._HostCold(len(dl.spec.T_c), host._hmat(hl.W1), host._hvec(hl.b1), host._hmat(hl.Wup),
                                     host._hmat(hl.W2)) if len(dl.spec.T_c) else None for dl, hl in zip(dls, hls)]

    def native(self, xs, ys, tau: float = 0.0, stream=None):
        """The same stack in one native call (pi_hybrid_stack_ahead): no per-layer Python call.
        Returns each layer's K_c."""
        import numpy as np
        C = host.C
        n = len(self.dls)
        if getattr(self, "_arrs", None) is None or self._arrs[0] != n:
            layers = (pi._Layer * n)(*[dl.layer_c for dl in self.dls])
            colds = (C.c_void_p * n)(*[C.addressof(c) if c is not None else None for c in self.colds])
            tg = (C.c_void_p * n)(*[dl.T_g.data_ptr() for dl in self.dls])
            tc = (C.c_void_p * n)(*[dl.T_c.data_ptr() if self.n_cs[L] else None for L, dl in enumerate(self.dls)])
            nc = (C.c_int32 * n)(*self.n_cs)
            self._arrs = (n, layers, colds, tg, tc, nc)
        _, layers, colds, tg, tc, nc = self._arrs
        xa = (C.c_void_p * n)(*[x.data_ptr() for x in xs])
        ya = (C.c_void_p * n)(*[y.data_ptr() for y in ys])
        kc = np.zeros(n, np.int32)
        host.pi_hybrid_stack_ahead(pi._stream(stream), layers, colds, tg, tc, nc, n, self.B, xa, tau, ya, self.scratch,
                                   self.threads, kc)
        return kc.tolist()

    def _tables(self, L):
        dl = self.dls[L]
        return dl.T_g.data_ptr(), (dl.T_c.data_ptr() if self.n_cs[L] else None), self.n_cs[L]

    def __call__(self, xs, ys, tau: float = 0.0, stream=None):
        """ys[L] (device [B x d]) = layer L's output for xs[L]; layer L's neurons predicted from
        xs[L - 1] (layer 0 from xs[0]).  Returns each layer's K_c."""
        st = pi._stream(stream)
        T_g, T_c, n_c = self._tables(0)
        host.pi_hybrid_prime(st, self.dls[0].layer_c, T_g, T_c, n_c, self.B, xs[0].data_ptr(), tau, self.scratch)
        kcs = []
        n = len(self.dls)
        for L in range(n):
            if L + 1 < n:
                T_g, T_c, n_c = self._tables(L + 1)
                nxt = self.dls[L + 1].layer_c
            else:
                T_g, T_c, n_c, nxt = None, None, 0, None
            kcs.append(host.pi_hybrid_layer_ahead(st, self.dls[L].layer_c, self.colds[L], nxt, T_g, T_c, n_c, self.B,
                                                  xs[L].data_ptr(), tau, ys[L].data_ptr(), self.scratch, self.threads))
        return kcs
