"""Offline neuron placement: which neurons of each layer live on the GPU.

The pages' offline phase profiles each neuron's activations, gives every neuron
an impact metric, and solves an integer linear program that places neurons on
the GPU or the CPU under the units' capacities, balancing the work across
layers and maximising the impact served by the GPU (unite.ai French article
"PowerInfer : Moteur d'inférence ...", section "Phase hors ligne : résolveur
de politiques et profileur LLM"; CSDN summary of "PowerInfer: Fast Large
Language Model Serving with a Consumer-grade GPU", section 神经元放置策略).
They give neither the program's objective nor its constraints in full; the
reading taken here:

  maximise   sum over layers l and neurons i of  c[l][i] * x[l][i]
  subject to sum over l, i of  s[l] * x[l][i] <= budget            (GPU memory)
             sum over i of x[l][i] >= ceil(min_frac * N_l)  for every l   (balance)
             x[l][i] in {0, 1}

with c the profiled activation count of the neuron (its impact) and s[l] the
bytes one neuron of layer l keeps on the GPU (its FC1 row, up row, FC2 row and
bias).  Every neuron of a layer has the same size, so an optimal solution takes
each layer's neurons in descending count order (ties to the lower id), and the
problem reduces to how many each layer gets.  Taking the remaining neurons of
all layers in descending impact per byte is then exactly optimal when every
layer's neurons have the same size, and within the impact of one neuron of the
optimum otherwise (the classic greedy bound for a knapsack of small items).

Host-side and offline; it produces the GPU tables (ascending T_g) that
pi_table_prepare and the layer calls take.
"""
from __future__ import annotations

import math
from typing import List, Sequence

import numpy as np


def solve_placement(counts: Sequence[np.ndarray], neuron_bytes: Sequence[int], budget: int,
                    min_frac: float = 0.0) -> List[np.ndarray]:
    """Per-layer GPU tables (ascending int32 neuron ids) for the program above.

    counts[l]: int activation counts of layer l's N_l neurons; neuron_bytes[l]: bytes per neuron of
    layer l on the GPU; budget: GPU bytes for all layers' neurons; min_frac: the smallest share of
    each layer's neurons kept on the GPU.  Raises ValueError when the minimum shares do not fit."""
    L = len(counts)
    if len(neuron_bytes) != L or L == 0:
        raise ValueError("one neuron size per layer is needed")
    if not 0.0 <= min_frac <= 1.0:
        raise ValueError("min_frac must lie in [0, 1]")
    orders, take = [], []
    left = int(budget)
    for l in range(L):
        c = np.asarray(counts[l], dtype=np.int64)
        if neuron_bytes[l] <= 0:
            raise ValueError("neuron sizes must be positive")
        orders.append(np.lexsort((np.arange(len(c)), -c)))      # count descending, then id ascending
        k = min(len(c), math.ceil(min_frac * len(c)))
        take.append(k)
        left -= k * int(neuron_bytes[l])
    if left < 0:
        raise ValueError("the minimum GPU shares exceed the budget")
    # the remaining neurons of every layer, best impact per byte first (ties: lower layer, lower id);
    # within a layer this keeps the descending count order
    cand_l, cand_r, dens = [], [], []
    for l in range(L):
        c = np.asarray(counts[l], dtype=np.int64)
        rest = orders[l][take[l]:]
        cand_l.append(np.full(len(rest), l, np.int64))
        cand_r.append(np.arange(take[l], len(c), dtype=np.int64))
        dens.append(c[rest] / float(neuron_bytes[l]))
    cl, cr, de = np.concatenate(cand_l), np.concatenate(cand_r), np.concatenate(dens)
    ids = np.concatenate([orders[l][take[l]:] for l in range(L)])
    pick = np.lexsort((ids, cl, -de))
    nxt = list(take)                       # the next rank each layer would take
    for q in pick:
        l, r = int(cl[q]), int(cr[q])
        if r != nxt[l]:
            continue                       # a layer's neurons go in rank order (an earlier one did not fit)
        s = int(neuron_bytes[l])
        if s <= left:
            left -= s
            nxt[l] += 1
    return [np.sort(orders[l][:nxt[l]]).astype(np.int32) for l in range(L)]


def gpu_impact_share(probs: Sequence[np.ndarray], tables: Sequence[np.ndarray]) -> float:
    """Expected share of all activations that the GPU tables hold, for per-neuron activation
    probabilities probs[l]."""
    tot = sum(float(np.sum(p)) for p in probs)
    got = sum(float(np.sum(np.asarray(p)[t])) for p, t in zip(probs, tables))
    return got / tot if tot > 0 else 0.0
