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
