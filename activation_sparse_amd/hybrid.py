"""The pages' GPU-CPU hybrid layer, as an executor over the two C ABIs.

Per layer and step (CSDN summary of "PowerInfer: Fast Large Language Model
Serving with a Consumer-grade GPU", section GPU-CPU混合执行): the GPU runs the
predictor and the compaction, the CPU-table list is copied to the host, and
then the two units compute their own active neurons at the same time: the GPU
its hot neurons (pi_sparse_ffn, enqueued before the host waits) and the CPU
its cold ones (pi_cold_ffn).  The CPU's partial result is copied to the device
and merged there (pi_merge).  When no cold neuron is active the copy and the
merge are skipped (the pages' selective synchronisation).

Marshalling and ordering only: the computation runs in libpi (GPU) and
libpi_host (CPU).  torch supplies device memory, the stream, an event and the
pinned host buffers of the two copies.
"""
from __future__ import annotations

import time

import activation_sparse_amd as pi
from activation_sparse_amd import host


class HybridLayer:
    """One layer split between a DeviceLayer-like object (dl: GPU-resident neurons and
    the predictor, with T_g / T_c device tables) and a host object (hl: the CPU-resident
    neurons' W1, b1, W2, Wup in host memory), for batch B."""

    def __init__(self, dl, hl, B: int, threads: int = 0, device="cuda:0"):
        import torch
        spec = dl.spec
        cfg = spec.cfg
        self.dl, self.hl, self.B, self.threads = dl, hl, B, threads
        self.d, self.N, self.H, self.n_g, self.n_c = cfg.d, cfg.N, spec.H, spec.n_g, len(spec.T_c)
        self.kind = pi.PI_GATED_RELU if cfg.gated else pi.PI_RELU
        i32 = torch.int32
        self.logits = torch.empty((B, self.N), dtype=torch.float32, device=device)
        self.A_g = torch.empty(max(self.n_g, 1), dtype=i32, device=device)
        self.K = torch.zeros(1, dtype=i32, device=device)
        self.A_c = torch.empty(max(self.n_c, 1), dtype=i32, device=device)
        self.K_c = torch.zeros(1, dtype=i32, device=device)
        self.y_c = torch.empty((B, self.d), dtype=torch.float32, device=device)
        wsp = max(pi.pi_workspace_bytes(pi.PI_OP_PREDICT, B, self.d, self.H, self.N, 0), 256)
        wsf = max(pi.pi_workspace_bytes(pi.PI_OP_SPARSE_FFN, B, self.d, 0, 0, self.n_g), 256)
        self.ws_pred = torch.empty(wsp, dtype=torch.uint8, device=device)
        self.ws_ffn = torch.empty(wsf, dtype=torch.uint8, device=device)
        self.A_c_h = torch.empty(max(self.n_c, 1), dtype=i32, pin_memory=True)
        self.K_c_h = torch.zeros(1, dtype=i32, pin_memory=True)
        self.y_c_h = torch.empty((B, self.d), dtype=torch.float32, pin_memory=True)
        self.listed = torch.cuda.Event()
        self.host_s = 0.0          # time spent in pi_cold_ffn (host clock), for measurement

    def __call__(self, x, x_host, y, tau: float = 0.0) -> int:
        """y [B x d] (device) = the layer's output for x [B x d] (device) and its host copy
        x_host; returns the number of active cold neurons (0: nothing was merged)."""
        dl, hl, B, d = self.dl, self.hl, self.B, self.d
        pi.pi_predict(B, d, self.H, self.N, x, dl.P1, dl.c1, dl.P2, dl.c2, self.logits, self.ws_pred)
        pi.pi_compact(B, self.N, self.logits, tau, dl.T_g, self.n_g, self.A_g, self.K,
                      dl.T_c if self.n_c else None, self.n_c, self.A_c if self.n_c else None,
                      self.K_c if self.n_c else None)
        if self.n_c:
            self.K_c_h.copy_(self.K_c, non_blocking=True)
            self.A_c_h.copy_(self.A_c, non_blocking=True)
            self.listed.record()
        # the GPU's neurons, queued before the host waits for the cold list
        pi.pi_sparse_ffn(B, d, self.n_g, self.kind, x, dl.W1, dl.b1, dl.Wup, dl.W2, self.A_g, self.K, y, self.ws_ffn)
        if not self.n_c:
            return 0
        self.listed.synchronize()
        kc = int(self.K_c_h[0])
        if kc == 0:
            return 0
        t0 = time.perf_counter()
        host.pi_cold_ffn(B, d, self.n_c, x_host, hl.W1, hl.b1, hl.W2, self.A_c_h, kc, self.y_c_h, kind=self.kind,
                         Wup=hl.Wup, threads=self.threads)
        self.host_s += time.perf_counter() - t0
        self.y_c.copy_(self.y_c_h, non_blocking=True)
        pi.pi_merge(B, d, y, self.y_c, self.K_c)
        return kc
