"""Shared cases for the placement solver's tables run through the layer call: a small gated
multi-layer stack whose layers differ in density and predictor size (so that one GPU budget is
split unevenly), and the LLaMA-13B gated stack with 40% of its neurons on the GPU."""
from __future__ import annotations

import math

import numpy as np

import synth
from activation_sparse_amd.placement import solve_placement

# four gated layers, densities spread over [0.04, 0.35], d = 512, N = 2048
SMALL = synth.Config("place-gated-small", "small gated stack for the placement solver's tables", 4, 512, 2048,
                     synth.F16, synth.F16, synth.F16, True, (0.04, 0.35), 1.1, (64, 128), 0.4, (1, 4), 8, 21)


def solver_specs(cfg: synth.Config, layers=None):
    """Every layer's spec with the solver's GPU table: the budget is the fixed rule's (floor of
    gpu_frac N neurons per layer, summed over the layers), every neuron one unit."""
    specs = [synth.layer_spec(cfg, l) for l in range(cfg.n_layers)]
    counts = [s.counts for s in specs]
    k = int(math.floor(cfg.gpu_frac * cfg.N))
    tables = solve_placement(counts, [1] * len(counts), k * len(counts))
    keep = range(cfg.n_layers) if layers is None else layers
    return {l: synth.with_table(specs[l], tables[l]) for l in keep}
