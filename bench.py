"""Decode benchmark of the neuron-aware sparse FFN on one MI355X.

One step = one decoded token (batch B) through every FFN layer of the stack:
for each layer one pi_ffn_layer_stages call (predictor, activation decision
and compaction, FFN over the GPU-resident neurons, merge), all on one stream,
layers serialised.  Weights and inputs are seeded synthetic tensors
generated on the device before timing; each step has its own inputs.  Steps
are captured once into HIP graphs and replayed.

Prints one JSON line (rank 0): throughput in tokens/s, the roofline of the
dominant kernel, and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="opt-30b")
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--layers", type=int, default=0, help="0 = every layer of the config")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cpu-layers", type=int, default=4)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the measurement, run 3 plain device copies of this many MiB (the known-size "
                         "reference for rocprofv3 FETCH_SIZE / WRITE_SIZE scaling)")
    ap.add_argument("--rocprof-summary", metavar="DIR", nargs="+", default=None,
                    help="summarise the rocprofv3 CSV output under each DIR (kernel trace, counters) and "
                         "exit; no GPU use")
    ap.add_argument("--copy-mib", type=int, default=256, help="copy size the counters were taken with")
    ap.add_argument("--sweep", default="4,16,32",
                    help="after the batch-1 measurement, time the same stack at these batch sizes (union active "
                         "set, matrix-core path) and report them under detail.batch_sweep; empty = none")
    ap.add_argument("--sweep-steps", type=int, default=8)
    ap.add_argument("--hybrid-steps", type=int, default=4,
                    help="after the batch-1 measurement, time the pages' GPU-CPU hybrid layer (cold neurons on "
                         "the host CPU) over this many steps; 0 = skip")
    ap.add_argument("--no-placement", dest="placement", action="store_false",
                    help="skip the host-side placement-solver report")
    ap.add_argument("--leg", default=None, metavar="NAME",
                    help="run one leg alone and print its result instead of the benchmark line: truth, chained, "
                         "placement, attention, batch-sweep, read-probe, boundary, warm, host-cold or config:KEY[:STRIDE] (for a profiler "
                         "run over just its kernels)")
    ap.add_argument("--attn-steps", type=int, default=8,
                    help="steps of the self-attention stack with head sparsity (0 = skip)")
    ap.add_argument("--placement-steps", type=int, default=16,
                    help="steps of the fixed-rule vs solver-table timing on the LLaMA-13B gated 40%% stack, "
                         "GPU side and hybrid (0 = skip)")
    ap.add_argument("--i4pred-steps", type=int, default=16,
                    help="after the batch-1 measurement, time the stack with int4-g128 predictor weights over "
                         "this many steps; 0 = skip")
    ap.add_argument("--lookahead-steps", type=int, default=16,
                    help="after the batch-1 measurement, time look-ahead prediction (layer L+1's predictor hidden "
                         "layer from layer L's input, beside layer L's FFN) over this many steps; 0 = skip")
    ap.add_argument("--truth-steps", type=int, default=8,
                    help="steps of the sensitivity run whose mask is the true activation set (0 = skip)")
    ap.add_argument("--configs", default="opt-6.7b,llama-13b-gated,opt-175b-int4:4,opt-30b-rho20",
                    help="other configurations timed at batch 1 (key or key:layer-stride; empty = skip)")
    ap.add_argument("--config-steps", type=int, default=8)
    ap.add_argument("--chained-steps", type=int, default=16,
                    help="after the batch-1 measurement, time chained layers (layer L+1's input is the layer "
                         "normalisation of layer L's output, made on the GPU) over this many steps; 0 = skip")
    return ap.parse_args()


def wbytes(dt):
    import synth
    return {synth.F32: 4.0, synth.F16: 2.0, synth.I4G128: 0.5 + 2.0 / 128}[dt]


def bias_bytes(dt):
    import synth
    return 4.0 if dt == synth.F32 else 2.0


def layer_bytes(spec, B, K, K_c, rows_p2, rows_w2):
    """Algorithmic HBM bytes of one layer's step: the predictor weights the method
    reads (all of P1; the hidden-major P2 rows of the hidden units with h > 0,
    rows_p2 of them; c2), the active GPU-resident neurons (FC1 row + bias for
    each of the K listed neurons, + up row if gated; the FC2 row of each of the
    rows_w2 neurons whose FC1 output is non-zero), and the small vectors (x, h,
    logits, lists, y, cold partial)."""
    cfg = spec.cfg
    d, N, H = cfg.d, cfg.N, spec.H
    wp, w, wb = wbytes(cfg.pdtype), wbytes(cfg.wdtype), bias_bytes(cfg.bdtype)
    pred = H * d * wp + rows_p2 * N * wp + N * wb
    mats1 = 2 if cfg.gated else 1
    ffn = K * (mats1 * d * w + wb) + rows_w2 * d * w
    small = B * d * 4 + 2 * B * H * 4 + 2 * B * N * 4 + spec.n_g * 4 + 2 * K * 4 + B * d * 4 * 2
    if len(spec.T_c):
        small += len(spec.T_c) * 4 + 2 * K_c * 4 + (B * d * 4 if K_c else 0)
    return pred, ffn, small


STAGES = ["hidden", "output+fc1", "fc2+lists", "sum+merge"]


def kernel_bytes(spec, B, K, K_c, rows_p2, rows_w2):
    """Algorithmic bytes of each kernel of one batch-1 pi_ffn_layer call: the weights
    and biases each kernel must read and the vectors it must read or write (not the
    FC2 partial sums, which are an implementation choice)."""
    cfg = spec.cfg
    d, N, H = cfg.d, cfg.N, spec.H
    wp, w, wb = wbytes(cfg.pdtype), wbytes(cfg.wdtype), bias_bytes(cfg.bdtype)
    mats1 = 2 if cfg.gated else 1
    groups = (N + 63) // 64
    return {
        "hidden": H * d * wp + B * d * 4 + B * H * 4,
        "output+fc1": (rows_p2 * N * wp + N * wb + B * H * 4 + B * d * 4 + 3 * groups * 4
                       + K * (mats1 * d * w + wb) + 4 * K + 8 * rows_w2 + 4 * K_c + 4 * groups),
        "fc2+lists": rows_w2 * d * w + 8 * rows_w2 + 4 * groups + 2 * (4 * K + 4 * K_c) + B * d * 4 * 0,
        "sum+merge": B * d * 4 + (B * d * 4 if (len(spec.T_c) and K_c) else 0),
    }


def cpu_baseline(cfg, B, seconds, n_layers_sample):
    """The oracle's full per-step pipeline on a bounded sample of the same workload."""
    import oracle as orc
    import synth
    from tests import parity_harness as ph
    Ls = min(n_layers_sample, cfg.n_layers)
    layers = []
    for L in range(Ls):
        spec = synth.layer_spec(cfg, L)
        sig = spec.sigmas()
        P1 = ph.host_mat(cfg.pdtype, cfg.seed, synth.TAG_P1, L, cfg.d, sig[synth.TAG_P1], nrows=spec.H)
        P2 = ph.host_mat(cfg.pdtype, cfg.seed, synth.TAG_P2, L, spec.H, sig[synth.TAG_P2], nrows=cfg.N)

        def rows(tag, ids):
            return ph.host_mat(cfg.wdtype, cfg.seed, tag, L, cfg.d, sig[tag], row_ids=ids)
        g = dict(W1=rows(synth.TAG_W1, spec.T_g), W2=rows(synth.TAG_W2, spec.T_g),
                 Wup=rows(synth.TAG_WUP, spec.T_g) if cfg.gated else None,
                 b1=ph.host_vec(spec.b1[spec.T_g], cfg.bdtype))
        c = None
        if len(spec.T_c):
            c = dict(W1=rows(synth.TAG_W1, spec.T_c), W2=rows(synth.TAG_W2, spec.T_c),
                     Wup=rows(synth.TAG_WUP, spec.T_c) if cfg.gated else None,
                     b1=ph.host_vec(spec.b1[spec.T_c], cfg.bdtype))
        layers.append((spec, P1, P2, g, c))
    kind = orc.GATED_RELU if cfg.gated else orc.RELU
    t_total, n_done, step = 0.0, 0, 0
    while True:
        for (spec, P1, P2, g, c) in layers:
            x = synth.host_x(cfg.seed, spec.layer, 10_000 + step, B, cfg.d)
            t0 = time.perf_counter()
            logits = orc.predict(x, P1, orc.Vec(None, cfg.bdtype), P2, ph.host_vec(spec.c2, cfg.bdtype))
            A_g, A_c = orc.compact(logits, 0.0, spec.T_g, spec.T_c if c else None)
            y_g = orc.sparse_ffn(x, g["W1"], g["b1"], g["W2"], A_g, kind=kind, Wup=g["Wup"])
            y_c = orc.sparse_ffn(x, c["W1"], c["b1"], c["W2"], A_c, kind=kind, Wup=c["Wup"]) if c else None
            orc.merge(y_g, y_c, len(A_c) if c else 0)
            t_total += time.perf_counter() - t0
            n_done += 1
        step += 1
        if t_total >= seconds:
            break
    per_layer = t_total / n_done
    tok_s = B / (per_layer * cfg.n_layers)
    cores = orc.get_threads()
    # the same pipeline on one thread, over a few layer-steps of the same sample
    one = None
    saved = cores
    orc.set_threads(1)
    try:
        t1, n1 = 0.0, 0
        for (spec, P1, P2, g, c) in layers[:2]:
            x = synth.host_x(cfg.seed, spec.layer, 20_000, B, cfg.d)
            t0 = time.perf_counter()
            logits = orc.predict(x, P1, orc.Vec(None, cfg.bdtype), P2, ph.host_vec(spec.c2, cfg.bdtype))
            A_g, A_c = orc.compact(logits, 0.0, spec.T_g, spec.T_c if c else None)
            y_g = orc.sparse_ffn(x, g["W1"], g["b1"], g["W2"], A_g, kind=kind, Wup=g["Wup"])
            y_c = orc.sparse_ffn(x, c["W1"], c["b1"], c["W2"], A_c, kind=kind, Wup=c["Wup"]) if c else None
            orc.merge(y_g, y_c, len(A_c) if c else 0)
            t1 += time.perf_counter() - t0
            n1 += 1
        one = B / (t1 / n1 * cfg.n_layers)
    finally:
        orc.set_threads(saved)
    return {"value": tok_s, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n_done} layer-steps (layers 0..{Ls - 1}, {step} steps, batch {B}) of the same workload "
                      f"in {t_total:.1f} s, scaled to {cfg.n_layers} layers per token; includes the cold-neuron "
                      f"side; weight generation not timed",
            "value_1_thread": one, "cpu_model": cpu_model(), "nproc": os.cpu_count()}


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None where there is none)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _short_kernel(name):
    import re
    m = re.search(r"(k_\w+|__amd_rocclr_\w+)", name)
    return m.group(1) if m else name[:60]


KERNEL_SOURCES = ["activation_sparse_amd/csrc/pi_fast.hip", "activation_sparse_amd/csrc/pi_b1.h",
                  "activation_sparse_amd/csrc/pi_device.h"]
DOMINANT = "k_pred_fc1"
TRAFFIC_PROFILE = "profiles/k_pred_fc1.opt-30b.b1.hbm_traffic.txt"


def code_text(src):
    """C++ source without its comments and blank lines, trailing spaces removed: the text a change of
    code changes and a change of comments does not (none of these sources has // or /* in a string)."""
    import re
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return "\n".join(l.rstrip() for l in src.split("\n") if l.strip())


def kernel_source_digest():
    """sha256 over the code of the sources the batch-1 kernels are built from, comments left out (a
    counter reading taken on other code no longer describes the kernel)."""
    import hashlib
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()


def committed_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None when there is none
    or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, TRAFFIC_PROFILE)
    if not os.path.exists(path):
        return None
    digest, val = None, None
    for line in open(path):
        if line.startswith("kernel sources sha256: "):
            digest = line.split(": ", 1)[1].strip()
        if line.startswith(f"traffic {kernel} "):
            val = float(line.split("total_bytes=")[1].split()[0])
    return val if (digest == kernel_source_digest() and val is not None) else None


LAYER_TAILS = ("k_reduce_y", "k_reduce")   # the ordered sum with the merge closes every layer call


def _layer_call_sites(rows):
    """Per call site within a layer: the dispatches (in start order) cut into sequences after each
    ordered-sum kernel that closes a layer call; over the sequences equal to the most common one
    (whatever else ran between two layer calls makes a sequence differ), the duration of each
    position (a kernel launched twice per layer is reported at each of its sites)."""
    import collections
    import statistics as st
    seqs, cur = [], []
    for r in rows:
        k = _short_kernel(r["Kernel_Name"])
        cur.append((k, (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
        if k in LAYER_TAILS:
            seqs.append(cur)
            cur = []
    if not seqs:
        return []
    common, n = collections.Counter(tuple(k for k, _ in q) for q in seqs).most_common(1)[0]
    sel = [q for q in seqs if tuple(k for k, _ in q) == common]
    out = [f"per layer call ({n} layer sequences of {len(common)} kernels):",
           f"{'site':4s} {'kernel':28s} {'avg_us':>9s} {'median_us':>9s}"]
    tot = 0.0
    for i, k in enumerate(common):
        v = [q[i][1] for q in sel]
        tot += st.mean(v)
        out.append(f"{i:4d} {k:28s} {st.mean(v):9.2f} {st.median(v):9.2f}")
    out.append(f"     {'sum':28s} {tot:9.2f}")
    return out


def rocprof_summary(roots, copy_mib):
    """Per-kernel durations from rocprofv3 `--kernel-trace --output-format csv`, and per-dispatch HBM
    counters from `--pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs, found anywhere under the given
    directories.

    Durations: every launch of a kernel, and for the dominant kernel also the launches that follow
    another of its launches (the back-to-back isolated launches the roofline is timed on).  Counters: KiB
    per dispatch, averaged per kernel, and scaled by what the same counter reads for the plain copies of
    copy_mib MiB (the copy dispatches within 1% of the largest reading), whose true traffic is copy_mib
    MiB read and copy_mib MiB written."""
    import csv
    import glob
    import statistics as st
    out = []
    scaled = {}
    rdreq = {}
    durs = {}                  # kernel -> {dispatch: us} from the counter runs
    allc = {}                  # (counter, kernel) -> values over every counter file
    for root in roots:
        for path in sorted(glob.glob(os.path.join(root, "**", "*kernel_trace.csv"), recursive=True)):
            rows = list(csv.DictReader(open(path)))
            rows.sort(key=lambda r: int(r["Start_Timestamp"]))
            per, iso = {}, []
            prev = None
            for r in rows:
                k = _short_kernel(r["Kernel_Name"])
                dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                per.setdefault(k, []).append(dur)
                if k == DOMINANT and prev == DOMINANT:
                    iso.append(dur)
                prev = k
            tot = sum(sum(v) for v in per.values())
            out.append(f"kernel trace: {path} ({len(rows)} dispatches)")
            out.append(f"{'kernel':32s} {'calls':>7s} {'avg_us':>9s} {'median_us':>9s} {'min_us':>8s} {'share':>6s}")
            for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
                out.append(f"{k:32s} {len(v):7d} {st.mean(v):9.2f} {st.median(v):9.2f} {min(v):8.2f} "
                           f"{100 * sum(v) / tot:5.1f}%")
            if iso:
                out.append(f"{DOMINANT + ' back-to-back':32s} {len(iso):7d} {st.mean(iso):9.2f} "
                           f"{st.median(iso):9.2f} {min(iso):8.2f}")
            out.extend(_layer_call_sites(rows))
            out.append("")
        for path in sorted(glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True)):
            rows = list(csv.DictReader(open(path)))
            per = {}
            for r in rows:
                k = _short_kernel(r["Kernel_Name"])
                per.setdefault((r["Counter_Name"], k), []).append(float(r["Counter_Value"]))
                allc.setdefault((r["Counter_Name"], k), []).append(float(r["Counter_Value"]))
                if r["Counter_Name"].startswith("TCC_EA0_RDREQ"):
                    rdreq.setdefault((r["Counter_Name"], k), []).append(float(r["Counter_Value"]))
                if r.get("End_Timestamp") and r.get("Start_Timestamp") and r.get("Dispatch_Id"):
                    durs.setdefault(k, {})[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            out.append(f"counters: {path} ({len(rows)} records)")
            for c in sorted({c for c, _ in per}):
                if c.startswith("TCC_EA0_RDREQ"):   # raw request counts: summarised below
                    continue
                if c not in ("FETCH_SIZE", "WRITE_SIZE"):
                    # other counters: the raw mean per dispatch
                    out.append(f"{c}: mean per dispatch")
                    for (cc, k), v in sorted(per.items()):
                        if cc == c and k.startswith("k_"):
                            out.append(f"  {k:24s} n={len(v):5d} mean={st.mean(v):14.1f}")
                    continue
                scale = None
                copy = per.get((c, "__amd_rocclr_copyBuffer"))
                if copy:
                    big = [v for v in copy if v >= 0.99 * max(copy)]
                    scale = (copy_mib * 1024.0) / st.mean(big)
                    out.append(f"{c}: plain copy of {copy_mib} MiB reads {st.mean(big):.1f} KiB per dispatch "
                               f"({len(big)} dispatches) -> scale {scale:.4f}")
                for (cc, k), v in sorted(per.items()):
                    if cc != c or k.startswith("__amd") or not k.startswith("k_"):
                        continue
                    line = f"  {k:24s} n={len(v):5d} mean={st.mean(v):11.1f} KiB"
                    if scale is not None:
                        b = st.mean(v) * scale * 1024
                        scaled[(c, k)] = b
                        line += f"  scaled={b / 1e6:9.3f} MB per dispatch"
                    out.append(line)
            out.append("")
    # read requests by size (a second reading of the read traffic, independent of FETCH_SIZE's formula):
    # bytes = 128 * RDREQ_128B + 64 * RDREQ_64B + 32 * RDREQ_32B per dispatch
    sized = {c: w for c, w in (("TCC_EA0_RDREQ_128B_sum", 128), ("TCC_EA0_RDREQ_64B_sum", 64),
                               ("TCC_EA0_RDREQ_32B_sum", 32))}
    if all(any(c == cc for cc, _ in rdreq) for c in sized):
        out.append("read requests by size (TCC_EA0_RDREQ_{128B,64B,32B}_sum), bytes per dispatch:")
        for k in sorted({k for _, k in rdreq}):
            if not (k.startswith("k_") or k == "__amd_rocclr_copyBuffer"):
                continue
            b = sum(w * st.mean(rdreq[(c, k)]) for c, w in sized.items() if (c, k) in rdreq)
            tot = st.mean(rdreq[("TCC_EA0_RDREQ_sum", k)]) if ("TCC_EA0_RDREQ_sum", k) in rdreq else float("nan")
            n128 = st.mean(rdreq[("TCC_EA0_RDREQ_128B_sum", k)]) if ("TCC_EA0_RDREQ_128B_sum", k) in rdreq else 0.0
            line = f"  {k:26s} {b / 1e6:10.3f} MB  (requests {tot:12.0f}, of them 128-byte {n128:12.0f})"
            if k == "__amd_rocclr_copyBuffer":
                copies = [v for v in rdreq[("TCC_EA0_RDREQ_128B_sum", k)]]
                big = max(copies)
                sel = [i for i, v in enumerate(copies) if v >= 0.99 * big]
                bb = sum(w * st.mean([rdreq[(c, k)][i] for i in sel]) for c, w in sized.items() if (c, k) in rdreq)
                line = (f"  plain copy of {copy_mib} MiB ({len(sel)} dispatches): {bb / 1e6:.3f} MB read by these "
                        f"requests, {bb / (copy_mib * 2**20):.4f} of its true bytes")
            out.append(line)
        out.append("")
    # read latency at the memory side: TCC_EA0_RDREQ_LEVEL accumulates the reads in flight every cycle, so
    # LEVEL / RDREQ is the mean cycles a read waits; with the requests per microsecond, their product is
    # proportional to the mean number in flight (the clock cancels in a ratio between kernels)
    if any(c == "TCC_EA0_RDREQ_LEVEL_sum" for c, _ in rdreq):
        out.append("reads at the memory side (TCC_EA0_RDREQ_LEVEL_sum / TCC_EA0_RDREQ_sum), per dispatch:")
        ref = None
        lines = []
        for k in sorted({k for c, k in rdreq if c == "TCC_EA0_RDREQ_LEVEL_sum"}):
            if not k.startswith("k_") or ("TCC_EA0_RDREQ_sum", k) not in rdreq:
                continue
            lev, req = st.mean(rdreq[("TCC_EA0_RDREQ_LEVEL_sum", k)]), st.mean(rdreq[("TCC_EA0_RDREQ_sum", k)])
            us = st.mean(durs[k].values()) if durs.get(k) else float("nan")
            if req <= 0 or not us > 0:
                continue
            lat, rate = lev / req, req / us
            if k == "k_read_probe":
                ref = lat * rate
            lines.append((k, us, req, lat, rate))
        for k, us, req, lat, rate in lines:
            rel = f"  in flight {lat * rate / ref:5.2f} x the streaming read's" if ref else ""
            out.append(f"  {k:24s} {us:8.2f} us  {req:11.0f} reads  {lat:7.0f} cycles each  {rate:9.0f} per us{rel}")
        out.append("")
    if ("TCP_UTCL1_TRANSLATION_MISS_sum" in {c for c, _ in allc}) and ("TCP_UTCL1_REQUEST_sum" in {c for c, _ in allc}):
        out.append("address translation (TCP_UTCL1_TRANSLATION_MISS_sum / TCP_UTCL1_REQUEST_sum), per dispatch:")
        for k in sorted({k for c, k in allc if c == "TCP_UTCL1_REQUEST_sum"}):
            if not k.startswith("k_") or ("TCP_UTCL1_TRANSLATION_MISS_sum", k) not in allc:
                continue
            req, miss = st.mean(allc[("TCP_UTCL1_REQUEST_sum", k)]), st.mean(allc[("TCP_UTCL1_TRANSLATION_MISS_sum", k)])
            if req > 0:
                out.append(f"  {k:24s} {req:11.0f} requests  {miss:9.0f} misses  ({miss / req:.4%})")
        out.append("")
    ks = sorted({k for _, k in scaled})
    if any(("FETCH_SIZE", k) in scaled and ("WRITE_SIZE", k) in scaled for k in ks):
        out.append("HBM traffic per dispatch (scaled FETCH_SIZE + WRITE_SIZE):")
        for k in ks:
            if ("FETCH_SIZE", k) in scaled and ("WRITE_SIZE", k) in scaled:
                f_, w_ = scaled[("FETCH_SIZE", k)], scaled[("WRITE_SIZE", k)]
                out.append(f"traffic {k} fetch_bytes={f_:.0f} write_bytes={w_:.0f} total_bytes={f_ + w_:.0f}")
        out.append(f"kernel sources sha256: {kernel_source_digest()}")
    return "\n".join(out)


def batch_sweep(cfg, specs, dls, batches, steps, warmup):
    """The stack at other batch sizes: same layers, per-(step, layer) seeded inputs, one HIP graph per
    step, `steps` timed steps after `warmup`.  Tokens/s counts every batch row; bytes are each step's
    algorithmic bytes from its measured counts (every P2 row and every listed W2 row at batch > 1)."""
    import torch
    import synth
    import activation_sparse_amd as pi
    dev = "cuda:0"
    n_layers = len(specs)
    maxH = max(s.H for s in specs)
    n_g = max(s.n_g for s in specs)
    n_c = max(len(s.T_c) for s in specs)
    d, N = cfg.d, cfg.N
    out = {}
    for B in batches:
        S = warmup + steps
        ws_bytes = max(pi.pi_workspace_bytes(pi.PI_OP_FFN_LAYER, B, d, maxH, N, n_g), 256)
        wss = [torch.empty(ws_bytes, dtype=torch.uint8, device=dev) for _ in range(n_layers)]
        xs = torch.empty((S, n_layers, B, d), dtype=torch.float32, device=dev)
        ycs = torch.empty((S, n_layers, B, d), dtype=torch.float32, device=dev) if n_c else None
        Ks = torch.zeros((S, n_layers), dtype=torch.int32, device=dev)
        Kcs = torch.zeros((S, n_layers), dtype=torch.int32, device=dev)
        rows = torch.zeros((S, n_layers, 2), dtype=torch.int32, device=dev)
        y = torch.empty((B, d), dtype=torch.float32, device=dev)
        A_g = torch.empty(max(n_g, 1), dtype=torch.int32, device=dev)
        A_c = torch.empty(max(n_c, 1), dtype=torch.int32, device=dev)
        stream = torch.cuda.current_stream().cuda_stream
        for t in range(S):
            rid = torch.from_numpy(synth.x_row_ids(1000 + t, B)).to(dev)
            for L in range(n_layers):
                synth.dev_fill(xs[t, L].data_ptr(), None, synth.F32, cfg.seed, synth.TAG_X, L, d, 1.0,
                               row_ids_ptr=rid.data_ptr(), nrows=B, stream=stream)
                if n_c:
                    synth.dev_fill(ycs[t, L].data_ptr(), None, synth.F32, cfg.seed, synth.TAG_YC, L, d, 0.05,
                                   row_ids_ptr=rid.data_ptr(), nrows=B, stream=stream)
        torch.cuda.synchronize()

        def step_call(t):
            for L in range(n_layers):
                cold = len(specs[L].T_c) > 0
                pi.pi_ffn_layer_stages(dls[L].layer, B, xs[t, L], 0.0, ycs[t, L] if cold else None, y, None, A_g,
                                       Ks[t, L:L + 1], A_c if cold else None, Kcs[t, L:L + 1] if cold else None,
                                       wss[L], pi.PI_STAGE_ALL, rows_read=rows[t, L], _cstruct=dls[L].layer_c)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step_call(0)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for t in range(S):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step_call(t)
            graphs.append(g)
        for t in range(warmup):
            graphs[t].replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for t in range(warmup, S):
            graphs[t].replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        Kh, Kch, Rh = Ks.cpu().numpy(), Kcs.cpu().numpy(), rows.cpu().numpy()
        tot = 0.0
        for t in range(warmup, S):
            for L in range(n_layers):
                tot += sum(layer_bytes(specs[L], B, int(Kh[t, L]), int(Kch[t, L]), int(Rh[t, L, 0]), int(Rh[t, L, 1])))
        step_bytes = tot / steps
        gbs = step_bytes / (ms * 1e-3) / 1e9
        out[str(B)] = {"tokens_per_s": round(B * 1e3 / ms, 1), "ms_per_step": round(ms, 4),
                       "step_bytes": round(step_bytes), "step_gbps": round(gbs, 1),
                       "step_frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "mean_K": float(Kh[warmup:].mean()),
                       "steps": steps}
        log(f"batch {B}: {ms:.3f} ms/step, {B * 1e3 / ms:.1f} tokens/s, {gbs:.0f} GB/s")
        del graphs, wss, xs, ycs
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def pi_kind(cfg):
    import activation_sparse_amd as pi
    return pi.PI_GATED_RELU if cfg.gated else pi.PI_RELU


def lookahead_bench(cfg, specs, dls, steps, warmup, B=1):
    """Look-ahead prediction (the pages: activations can be predicted some layers ahead while the
    model runs): layer L+1's predictor hidden layer is computed from layer L's input by
    pi_ffn_layer_ahead, in the launch that runs layer L's output layer and FC1; layer L+1's
    remaining stages take layer L+1's own input.  Layer 0 predicts from its own input.  Same
    layers, seeded inputs and one HIP graph per step as the measured run; returns tokens/s."""
    import torch
    import synth
    import activation_sparse_amd as pi
    dev = "cuda:0"
    n_layers = len(specs)
    maxH = max(s.H for s in specs)
    n_g = max(s.n_g for s in specs)
    n_c = max(len(s.T_c) for s in specs)
    d, N = cfg.d, cfg.N
    S = warmup + steps
    ws_bytes = max(pi.pi_workspace_bytes(pi.PI_OP_FFN_LAYER, B, d, maxH, N, n_g), 256)
    wss = [torch.empty(ws_bytes, dtype=torch.uint8, device=dev) for _ in range(n_layers)]
    xs = torch.empty((S, n_layers, B, d), dtype=torch.float32, device=dev)
    ycs = torch.empty((S, n_layers, B, d), dtype=torch.float32, device=dev) if n_c else None
    Ks = torch.zeros((S, n_layers), dtype=torch.int32, device=dev)
    Kcs = torch.zeros((S, n_layers), dtype=torch.int32, device=dev)
    y = torch.empty((B, d), dtype=torch.float32, device=dev)
    A_g = torch.empty(max(n_g, 1), dtype=torch.int32, device=dev)
    A_c = torch.empty(max(n_c, 1), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    for t in range(S):
        rid = torch.from_numpy(synth.x_row_ids(t, B)).to(dev)
        for L in range(n_layers):
            synth.dev_fill(xs[t, L].data_ptr(), None, synth.F32, cfg.seed, synth.TAG_X, L, d, 1.0,
                           row_ids_ptr=rid.data_ptr(), nrows=B, stream=stream)
            if n_c:
                synth.dev_fill(ycs[t, L].data_ptr(), None, synth.F32, cfg.seed, synth.TAG_YC, L, d, 0.05,
                               row_ids_ptr=rid.data_ptr(), nrows=B, stream=stream)
    torch.cuda.synchronize()
    rest = pi.PI_STAGE_ALL & ~pi.PI_STAGE_HIDDEN

    def stage(t, L, stages, ahead=False):
        cold = len(specs[L].T_c) > 0
        args = (B, xs[t, L], 0.0, ycs[t, L] if cold else None, y, None, A_g, Ks[t, L:L + 1], A_c if cold else None,
                Kcs[t, L:L + 1] if cold else None, wss[L], stages)
        if ahead:
            pi.pi_ffn_layer_ahead(dls[L].layer, *args, dls[L + 1].layer, wss[L + 1], _cstruct=dls[L].layer_c,
                                  _next_cstruct=dls[L + 1].layer_c)
        else:
            pi.pi_ffn_layer_stages(dls[L].layer, *args, _cstruct=dls[L].layer_c)

    def step_call(t):
        stage(t, 0, pi.PI_STAGE_HIDDEN)
        for L in range(n_layers):
            stage(t, L, rest, ahead=L + 1 < n_layers)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step_call(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for t in range(S):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step_call(t)
        graphs.append(g)
    for t in range(warmup):
        graphs[t].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for t in range(warmup, S):
        graphs[t].replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    out = {"tokens_per_s": round(B * 1e3 / ms, 2), "ms_per_step": round(ms, 4), "steps": steps, "batch": B,
           "mean_K": float(Ks[warmup:].float().mean().item()),
           "predictor_input": "layer L+1's hidden layer from layer L's input (layer 0: its own)"}
    log(f"look-ahead prediction: {out['ms_per_step']} ms/step, {out['tokens_per_s']} tokens/s")
    del graphs
    return out


def chained_bench(cfg, specs, dls, steps, warmup, B=1, eps=1e-5):
    """Chained layers: layer L+1's input is the layer normalisation of layer L's output, so every
    layer's input is made by the step itself; layer 0's input is seeded per step.  Timed three
    ways: exact prediction with the normalisation inside the layer call (pi_ffn_layer_normed, the
    reported figure), exact prediction with pi_layer_norm between the layer calls, and look-ahead
    prediction (pi_ffn_layer_ahead: layer L+1's predictor hidden layer from layer L's input, with
    pi_layer_norm).  The cold partials stay seeded, as in the measured run.  One HIP graph per
    step; returns tokens/s of each and the normalisation kernel's own time."""
    import torch
    import synth
    import activation_sparse_amd as pi
    dev = "cuda:0"
    n_layers = len(specs)
    maxH = max(s.H for s in specs)
    n_g = max(s.n_g for s in specs)
    n_c = max(len(s.T_c) for s in specs)
    d, N = cfg.d, cfg.N
    S = warmup + steps
    # the normalising call's workspace begins with the plain layer call's
    ws_bytes = max(pi.pi_workspace_bytes(pi.PI_OP_FFN_LAYER_NORMED, B, d, maxH, N, n_g), 256)
    wss = [torch.empty(ws_bytes, dtype=torch.uint8, device=dev) for _ in range(n_layers)]
    x0 = torch.empty((S, B, d), dtype=torch.float32, device=dev)
    xl = torch.empty((n_layers, B, d), dtype=torch.float32, device=dev)
    ycs = torch.empty((S, n_layers, B, d), dtype=torch.float32, device=dev) if n_c else None
    Ks = torch.zeros((S, n_layers), dtype=torch.int32, device=dev)
    Kcs = torch.zeros((S, n_layers), dtype=torch.int32, device=dev)
    y = torch.empty((B, d), dtype=torch.float32, device=dev)
    A_g = torch.empty(max(n_g, 1), dtype=torch.int32, device=dev)
    A_c = torch.empty(max(n_c, 1), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    for t in range(S):
        rid = torch.from_numpy(synth.x_row_ids(t, B)).to(dev)
        synth.dev_fill(x0[t].data_ptr(), None, synth.F32, cfg.seed, synth.TAG_X, 0, d, 1.0,
                       row_ids_ptr=rid.data_ptr(), nrows=B, stream=stream)
        if n_c:
            for L in range(n_layers):
                synth.dev_fill(ycs[t, L].data_ptr(), None, synth.F32, cfg.seed, synth.TAG_YC, L, d, 0.05,
                               row_ids_ptr=rid.data_ptr(), nrows=B, stream=stream)
    torch.cuda.synchronize()
    rest = pi.PI_STAGE_ALL & ~pi.PI_STAGE_HIDDEN

    def step_call(t, ahead):
        for L in range(n_layers):
            x = x0[t] if L == 0 else xl[L]
            cold = len(specs[L].T_c) > 0
            if ahead == "normed":
                # the layer normalises the previous output itself (in place: y_prev is y)
                if L == 0:
                    pi.pi_ffn_layer(dls[0].layer, B, x, 0.0, ycs[t, 0] if cold else None, y, None, A_g,
                                    Ks[t, 0:1], A_c if cold else None, Kcs[t, 0:1] if cold else None, wss[0],
                                    _cstruct=dls[0].layer_c)
                else:
                    pi.pi_ffn_layer_normed(dls[L].layer, B, y, eps, 0.0, ycs[t, L] if cold else None, y, None, A_g,
                                           Ks[t, L:L + 1], A_c if cold else None, Kcs[t, L:L + 1] if cold else None,
                                           wss[L], _cstruct=dls[L].layer_c)
                continue
            args = (B, x, 0.0, ycs[t, L] if cold else None, y, None, A_g, Ks[t, L:L + 1], A_c if cold else None,
                    Kcs[t, L:L + 1] if cold else None, wss[L])
            if ahead and L == 0:
                pi.pi_ffn_layer_stages(dls[0].layer, *args, pi.PI_STAGE_HIDDEN, _cstruct=dls[0].layer_c)
            if ahead and L + 1 < n_layers:
                pi.pi_ffn_layer_ahead(dls[L].layer, *args, rest, dls[L + 1].layer, wss[L + 1],
                                      _cstruct=dls[L].layer_c, _next_cstruct=dls[L + 1].layer_c)
            else:
                pi.pi_ffn_layer_stages(dls[L].layer, *args, rest if ahead else pi.PI_STAGE_ALL,
                                       _cstruct=dls[L].layer_c)
            if L + 1 < n_layers:
                pi.pi_layer_norm(B, d, y, xl[L + 1], eps)

    def timed(ahead):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step_call(0, ahead)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for t in range(S):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step_call(t, ahead)
            graphs.append(g)
        for t in range(warmup):
            graphs[t].replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for t in range(warmup, S):
            graphs[t].replay()
        e1.record()
        torch.cuda.synchronize()
        del graphs
        return e0.elapsed_time(e1) / steps

    ms_exact = timed(False)
    K_exact = float(Ks[warmup:].float().mean().item())
    ms_normed = timed("normed")
    K_normed = float(Ks[warmup:].float().mean().item())
    ms_ahead = timed(True)
    K_ahead = float(Ks[warmup:].float().mean().item())
    # the normalisation alone: a graph of back-to-back calls on [B x d] (kernel + the gap to the next)
    n_norm = 200
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pi.pi_layer_norm(B, d, y, xl[1], eps)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n_norm):
            pi.pi_layer_norm(B, d, y, xl[1], eps)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    out = {"batch": B, "steps": steps, "eps": eps,
           "tokens_per_s": round(B * 1e3 / ms_normed, 2), "ms_per_step": round(ms_normed, 4), "mean_K": K_normed,
           "normalisation": "inside the layer call (pi_ffn_layer_normed)",
           "separate_norm_tokens_per_s": round(B * 1e3 / ms_exact, 2),
           "separate_norm_ms_per_step": round(ms_exact, 4), "separate_norm_mean_K": K_exact,
           "lookahead_tokens_per_s": round(B * 1e3 / ms_ahead, 2), "lookahead_ms_per_step": round(ms_ahead, 4),
           "lookahead_mean_K": K_ahead,
           "layer_norm_us": round(e0.elapsed_time(e1) * 1e3 / n_norm, 2),
           "input": "layer 0 seeded per step; layer L+1 = layer norm of layer L's output (unit gain, zero bias)"}
    log(f"chained layers: exact, normalised in the layer call {out['ms_per_step']} ms/step, {out['tokens_per_s']} "
        f"tokens/s; with pi_layer_norm between calls {out['separate_norm_ms_per_step']} ms/step; look-ahead "
        f"{out['lookahead_ms_per_step']} ms/step, {out['lookahead_tokens_per_s']} tokens/s; "
        f"layer norm {out['layer_norm_us']} us")
    return out


def stack_timing(cfg, specs, dls, steps, warmup, B=1, c2_of=None):
    """Times the exact batch-1 layer stack `specs` (one HIP graph per step, the headline's seeded
    inputs and cold partials) and each stage set alone (back-to-back launches over the layers on the
    state the last step left).  c2_of(t, L), when given, is the device pointer of the output bias to
    use at step t and layer L (the truth-mode leg).  Returns the step time, the algorithmic bytes
    from the kernels' own row counts, the dominant stage and the mean counts."""
    import torch
    import synth
    import activation_sparse_amd as pi
    dev = "cuda:0"
    n_layers = len(specs)
    maxH = max(s.H for s in specs)
    n_g = max(s.n_g for s in specs)
    n_c = max(len(s.T_c) for s in specs)
    d, N = cfg.d, cfg.N
    S = warmup + steps
    ws_bytes = max(pi.pi_workspace_bytes(pi.PI_OP_FFN_LAYER, B, d, maxH, N, n_g), 256)
    wss = [torch.empty(ws_bytes, dtype=torch.uint8, device=dev) for _ in range(n_layers)]
    xs = torch.empty((S, n_layers, B, d), dtype=torch.float32, device=dev)
    ycs = torch.empty((S, n_layers, B, d), dtype=torch.float32, device=dev) if n_c else None
    Ks = torch.zeros((S, n_layers), dtype=torch.int32, device=dev)
    Kcs = torch.zeros((S, n_layers), dtype=torch.int32, device=dev)
    rows = torch.zeros((S, n_layers, 2), dtype=torch.int32, device=dev)
    y = torch.empty((B, d), dtype=torch.float32, device=dev)
    A_g = torch.empty(max(n_g, 1), dtype=torch.int32, device=dev)
    A_c = torch.empty(max(n_c, 1), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    for t in range(S):
        rid = torch.from_numpy(synth.x_row_ids(t, B)).to(dev)
        for i, spec in enumerate(specs):
            synth.dev_fill(xs[t, i].data_ptr(), None, synth.F32, cfg.seed, synth.TAG_X, spec.layer, d, 1.0,
                           row_ids_ptr=rid.data_ptr(), nrows=B, stream=stream)
            if n_c:
                synth.dev_fill(ycs[t, i].data_ptr(), None, synth.F32, cfg.seed, synth.TAG_YC, spec.layer, d, 0.05,
                               row_ids_ptr=rid.data_ptr(), nrows=B, stream=stream)
    torch.cuda.synchronize()
    structs = {}

    def cstruct(t, i):
        if c2_of is None:
            return dls[i].layer_c
        key = (t, i)
        if key not in structs:
            c = pi._Layer.from_buffer_copy(dls[i].layer_c)
            c.c2 = pi._Vec(c2_of(t, i), c.c2.dtype)
            structs[key] = c
        return structs[key]

    def call(t, i, stages, with_rows=True):
        cold = len(specs[i].T_c) > 0
        pi.pi_ffn_layer_stages(dls[i].layer, B, xs[t, i], 0.0, ycs[t, i] if cold else None, y, None, A_g,
                               Ks[t, i:i + 1], A_c if cold else None, Kcs[t, i:i + 1] if cold else None, wss[i],
                               stages, rows_read=rows[t, i] if with_rows else None, _cstruct=cstruct(t, i))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(n_layers):
            call(0, i, pi.PI_STAGE_ALL)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for t in range(S):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n_layers):
                call(t, i, pi.PI_STAGE_ALL)
        graphs.append(g)
    for t in range(warmup):
        graphs[t].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for t in range(warmup, S):
        graphs[t].replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del graphs
    Kh, Kch, Rh = Ks.cpu().numpy(), Kcs.cpu().numpy(), rows.cpu().numpy()
    tot = [0.0, 0.0, 0.0]
    for t in range(warmup, S):
        for i, spec in enumerate(specs):
            for k, v in enumerate(layer_bytes(spec, B, int(Kh[t, i]), int(Kch[t, i]), int(Rh[t, i, 0]),
                                              int(Rh[t, i, 1]))):
                tot[k] += v
    step_bytes = sum(tot) / steps
    # each stage set alone, back to back over the layers, repeating the last step's work
    last = S - 1
    stage_sets = {"hidden": pi.PI_STAGE_HIDDEN, "output+fc1": pi.PI_STAGE_OUTPUT | pi.PI_STAGE_FC1,
                  "fc2+lists": pi.PI_STAGE_FC2, "sum+merge": pi.PI_STAGE_SUM}
    kb = [kernel_bytes(spec, B, int(Kh[last, i]), int(Kch[last, i]), int(Rh[last, i, 0]), int(Rh[last, i, 1]))
          for i, spec in enumerate(specs)]
    stage_us, stage_gbps = {}, {}
    reps = 4
    for name, bits in stage_sets.items():
        # one HIP graph of `reps` passes over the layers, so that launch overhead is not timed
        with torch.cuda.stream(side):
            for i in range(n_layers):
                call(last, i, bits, with_rows=False)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                for i in range(n_layers):
                    call(last, i, bits, with_rows=False)
        g.replay()
        torch.cuda.synchronize()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        del g
        us = e0.elapsed_time(e1) * 1e3 / (reps * n_layers)
        stage_us[name] = round(us, 2)
        stage_gbps[name] = round(float(np.mean([k[name] for k in kb])) / (us * 1e-6) / 1e9, 1)
    dom = max(stage_us, key=stage_us.get)
    out = {"ms_per_step_timed_layers": round(ms, 4), "layers_timed": n_layers, "step_bytes_timed_layers": round(step_bytes),
           "step_gbps": round(step_bytes / (ms * 1e-3) / 1e9, 1),
           "step_frac_of_peak": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "bytes_split": {"predictor": round(tot[0] / steps), "ffn": round(tot[1] / steps), "small": round(tot[2] / steps)},
           "mean_K": float(Kh[warmup:].mean()), "mean_K_cold": float(Kch[warmup:].mean()),
           "mean_p2_rows_read": float(Rh[warmup:, :, 0].mean()), "mean_fc2_rows_read": float(Rh[warmup:, :, 1].mean()),
           "stage_us_alone": stage_us, "stage_gbps_alone": stage_gbps,
           "dominant_stage": dom, "dominant_frac_of_peak": round(stage_gbps[dom] / HBM_PEAK_GBS, 4), "steps": steps}
    del wss, xs, ycs
    return out


# sentinel output biases of the truth-mode leg: far beyond any |P2 . h| of these workloads, inside fp16
TRUTH_BIAS = 60000.0


def truth_bench(cfg, specs, dls, steps, warmup):
    """Sensitivity run with a predictor that is always right: the activation set of each (step,
    layer) is the true one, z = W1 x + b1 > 0 over all N neurons (computed in fp32 by PyTorch from
    the same stored fp16 weights, generated on the device), fed to the unchanged layer call through
    its output bias (c2 = +TRUTH_BIAS where z > 0, -TRUTH_BIAS elsewhere) so that every predictor
    weight is still read.  Every listed neuron then has a non-zero FC1 output, so FC2 reads them all.
    Returns the stack timing, the true density and the GPU share of the true activations."""
    import torch
    import synth
    from synth.device import dev_matrix, fill_matrix
    dev = "cuda:0"
    n_layers = len(specs)
    d, N, B = cfg.d, cfg.N, 1
    S = warmup + steps
    c2s = torch.empty((S, n_layers, N), dtype=torch.float16, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    dens, share = [], []
    x = torch.empty((S, B, d), dtype=torch.float32, device=dev)
    all_ids = torch.arange(N, dtype=torch.int32, device=dev)
    for i, spec in enumerate(specs):
        for t in range(S):
            rid = torch.from_numpy(synth.x_row_ids(t, B)).to(dev)
            synth.dev_fill(x[t].data_ptr(), None, synth.F32, cfg.seed, synth.TAG_X, spec.layer, d, 1.0,
                           row_ids_ptr=rid.data_ptr(), nrows=B, stream=stream)
        W1 = dev_matrix(N, d, cfg.wdtype, dev)
        fill_matrix(W1, cfg.wdtype, cfg.seed, synth.TAG_W1, spec.layer, d, spec.sigmas()[synth.TAG_W1], all_ids, N)
        b1 = torch.from_numpy(synth.stored_to_f64(spec.b1, cfg.bdtype)).to(dev).float()
        W1f = W1.data.float()                                                   # [N, d]
        z = torch.matmul(W1f, x[:, 0, :].t().contiguous()).t() + b1             # [S, N]
        act = z > 0
        c2s[:, i, :] = torch.where(act, TRUTH_BIAS, -TRUTH_BIAS).to(torch.float16)
        g = torch.zeros(N, dtype=torch.bool, device=dev)
        g[torch.from_numpy(spec.T_g.astype(np.int64)).to(dev)] = True
        dens.append(float(act[warmup:].float().mean()))
        share.append(float((act[warmup:] & g).float().sum() / max(1.0, float(act[warmup:].float().sum()))))
        del W1, W1f, z
    torch.cuda.synchronize()
    out = stack_timing(cfg, specs, dls, steps, warmup, c2_of=lambda t, i: c2s[t, i].data_ptr())
    out.update({"tokens_per_s": round(1e3 / out["ms_per_step_timed_layers"], 2),
                "true_density": round(float(np.mean(dens)), 4),
                "gpu_share_of_true_activations": round(float(np.mean(share)), 4),
                "mask": "true activations z = W1 x + b1 > 0 (fp32, PyTorch), fed through the output bias"})
    del c2s
    return out


def config_bench(key, steps, warmup, stride=1, cpu_seconds=4.0, cpu=True):
    """One configuration at batch 1: its own layer stack (every `stride`-th layer when stride > 1,
    which keeps the spread of per-layer densities and hidden sizes; tokens/s then scales the mean
    per-layer time to every layer), the stage timings and a bounded oracle baseline."""
    import torch
    import synth
    from synth.device import DeviceLayer
    cfg = synth.CONFIGS[key]
    t0 = time.time()
    layers = list(range(0, cfg.n_layers, stride))
    specs = [synth.layer_spec(cfg, L) for L in layers]
    dls = [DeviceLayer(s, "cuda:0") for s in specs]
    torch.cuda.synchronize()
    out = stack_timing(cfg, specs, dls, steps, warmup)
    scale = cfg.n_layers / len(layers)
    ms = out["ms_per_step_timed_layers"] * scale
    out.update({"workload": cfg.desc, "layers": cfg.n_layers, "layers_timed": len(layers),
                "layer_stride": stride, "tokens_per_s": round(1e3 / ms, 2), "ms_per_step": round(ms, 4),
                "step_bytes": round(out["step_bytes_timed_layers"] * scale),
                "mean_predictor_hidden": float(np.mean([s.H for s in specs])),
                "mean_density": round(float(np.mean([s.rho for s in specs])), 4)})
    del dls
    torch.cuda.empty_cache()
    out["cpu_baseline"] = cpu_baseline(cfg, 1, cpu_seconds, 2) if cpu else None
    out["setup_and_run_s"] = round(time.time() - t0, 1)
    log(f"config {key}: {out['tokens_per_s']} tokens/s ({out['ms_per_step']} ms/step over {cfg.n_layers} layers, "
        f"{out['layers_timed']} timed), step frac {out['step_frac_of_peak']}, dominant {out['dominant_stage']} at "
        f"{out['dominant_frac_of_peak']}")
    return out


def i4pred_bench(cfg, specs, dls, steps, warmup):
    """Predictor-cost variant: the same stack, inputs and FFN weights with int4-g128 predictor
    weights (P1 as int4 rows; P2's fp16 values quantised hidden-major, groups along N), through
    the same batch-1 layer call and one HIP graph per step.  Returns tokens/s and the step's
    algorithmic bytes at the int4 widths.  None unless the stack is the OPT-30B one."""
    import torch
    import synth
    import activation_sparse_amd as pi
    from dataclasses import replace
    from synth.device import dev_matrix, fill_matrix, dev_matrix_hidden_major
    vkey = cfg.key + "-i4pred"
    if vkey not in synth.CONFIGS:
        return None
    vcfg = synth.CONFIGS[vkey]
    dev = "cuda:0"
    B, n_layers = 1, len(specs)
    d, N = cfg.d, cfg.N
    vspecs, lays, keep = [], [], []
    for spec, dl in zip(specs, dls):
        vs = synth.layer_spec(vcfg, spec.layer)
        assert np.array_equal(vs.c2, spec.c2) and np.array_equal(vs.T_g, spec.T_g)
        sig = vs.sigmas()
        P1 = dev_matrix(vs.H, d, synth.I4G128, dev)
        fill_matrix(P1, synth.I4G128, vcfg.seed, synth.TAG_P1, spec.layer, d, sig[synth.TAG_P1])
        P2 = dev_matrix_hidden_major(N, vs.H, synth.I4G128, vcfg.seed, synth.TAG_P2, spec.layer, sig[synth.TAG_P2], dev)
        lay = replace(dl.layer, P1=P1, P2=P2)
        vspecs.append(vs)
        lays.append(lay._c())
        keep.append((P1, P2))
    torch.cuda.synchronize()
    maxH = max(s.H for s in specs)
    n_g = max(s.n_g for s in specs)
    n_c = max(len(s.T_c) for s in specs)
    S = warmup + steps
    ws_bytes = max(pi.pi_workspace_bytes(pi.PI_OP_FFN_LAYER, B, d, maxH, N, n_g), 256)
    wss = [torch.empty(ws_bytes, dtype=torch.uint8, device=dev) for _ in range(n_layers)]
    xs = torch.empty((S, n_layers, B, d), dtype=torch.float32, device=dev)
    ycs = torch.empty((S, n_layers, B, d), dtype=torch.float32, device=dev) if n_c else None
    Ks = torch.zeros((S, n_layers), dtype=torch.int32, device=dev)
    Kcs = torch.zeros((S, n_layers), dtype=torch.int32, device=dev)
    rows = torch.zeros((S, n_layers, 2), dtype=torch.int32, device=dev)
    y = torch.empty((B, d), dtype=torch.float32, device=dev)
    A_g = torch.empty(max(n_g, 1), dtype=torch.int32, device=dev)
    A_c = torch.empty(max(n_c, 1), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    for t in range(S):
        rid = torch.from_numpy(synth.x_row_ids(t, B)).to(dev)
        for L in range(n_layers):
            synth.dev_fill(xs[t, L].data_ptr(), None, synth.F32, cfg.seed, synth.TAG_X, L, d, 1.0,
                           row_ids_ptr=rid.data_ptr(), nrows=B, stream=stream)
            if n_c:
                synth.dev_fill(ycs[t, L].data_ptr(), None, synth.F32, cfg.seed, synth.TAG_YC, L, d, 0.05,
                               row_ids_ptr=rid.data_ptr(), nrows=B, stream=stream)
    torch.cuda.synchronize()

    def step_call(t):
        for L in range(n_layers):
            cold = len(specs[L].T_c) > 0
            pi.pi_ffn_layer_stages(dls[L].layer, B, xs[t, L], 0.0, ycs[t, L] if cold else None, y, None, A_g,
                                   Ks[t, L:L + 1], A_c if cold else None, Kcs[t, L:L + 1] if cold else None,
                                   wss[L], pi.PI_STAGE_ALL, rows_read=rows[t, L], _cstruct=lays[L])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step_call(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for t in range(S):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step_call(t)
        graphs.append(g)
    for t in range(warmup):
        graphs[t].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for t in range(warmup, S):
        graphs[t].replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    Kh, Kch, Rh = Ks.cpu().numpy(), Kcs.cpu().numpy(), rows.cpu().numpy()
    tot = [0.0, 0.0, 0.0]
    for t in range(warmup, S):
        for L in range(n_layers):
            for i, v in enumerate(layer_bytes(vspecs[L], B, int(Kh[t, L]), int(Kch[t, L]), int(Rh[t, L, 0]),
                                              int(Rh[t, L, 1]))):
                tot[i] += v
    step_bytes = sum(tot) / steps
    out = {"tokens_per_s": round(B * 1e3 / ms, 2), "ms_per_step": round(ms, 4), "steps": steps,
           "config": vcfg.desc, "step_bytes": round(step_bytes),
           "bytes_split": {"predictor": round(tot[0] / steps), "ffn": round(tot[1] / steps),
                           "small": round(tot[2] / steps)},
           "step_gbps": round(step_bytes / (ms * 1e-3) / 1e9, 1), "mean_K": float(Kh[warmup:].mean()),
           "mean_p2_rows_read": float(Rh[warmup:, :, 0].mean())}
    log(f"int4 predictor: {out['ms_per_step']} ms/step, {out['tokens_per_s']} tokens/s, "
        f"{out['step_bytes'] / 1e9:.2f} GB per step")
    del graphs
    return out


def placement_report(keys):
    """The offline placement solver against the fixed per-layer top-40% rule, on the host: each
    config's layers profiled (seeded), the solver given the same GPU budget (40% of all neurons,
    every neuron one unit, no per-layer minimum), and the expected share of all activations the GPU
    tables hold under the true probabilities."""
    import math
    import synth
    from activation_sparse_amd.placement import solve_placement, gpu_impact_share
    out = {}
    for key in keys:
        cfg = synth.CONFIGS[key]
        specs = [synth.layer_spec(cfg, l) for l in range(cfg.n_layers)]
        counts = [synth.profile_counts(cfg, l, sp.p) for l, sp in enumerate(specs)]
        k = int(math.floor(0.4 * cfg.N))
        fixed = [np.sort(np.lexsort((np.arange(cfg.N), -c))[:k]).astype(np.int32) for c in counts]
        t0 = time.perf_counter()
        sol = solve_placement(counts, [1] * len(counts), k * len(counts))
        solve_s = time.perf_counter() - t0
        p = [sp.p for sp in specs]
        shares = [len(t) / cfg.N for t in sol]
        out[key] = {"gpu_activation_share_fixed_top40": round(gpu_impact_share(p, fixed), 4),
                    "gpu_activation_share_solver": round(gpu_impact_share(p, sol), 4),
                    "solver_layer_share_min": round(min(shares), 4), "solver_layer_share_max": round(max(shares), 4),
                    "solve_s": round(solve_s, 3), "layers": cfg.n_layers}
    log(f"placement: {out}")
    return out


def attn_bench(steps, warmup, key="attn-opt-30b", cpu=True):
    """The self-attention stack with head sparsity at decode (pi_attn_decode), batch 1, every layer at
    the last cache position (1,024 cached positions): one HIP graph per step of all layers, timed
    with the head predictor's decisions (tau = 0) and with every head active (tau = -3e38, the
    dense block).  Algorithmic bytes per layer: the head predictor, every K and V row, and per
    active head its query and output-projection rows and its cached keys and values."""
    import torch
    import synth
    import activation_sparse_amd as pi
    from synth.device import DeviceAttn
    cfg = synth.ATTN_CONFIGS[key]
    dev = "cuda:0"
    t0 = time.time()
    L, d, nh, dh = cfg.n_layers, cfg.d, cfg.n_heads, cfg.dh
    t = cfg.L_max - 1
    dls = [DeviceAttn(synth.attn_spec(cfg, l), dev) for l in range(L)]
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    S = warmup + steps
    xs = torch.empty((S, L, d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    for st in range(S):
        rid = torch.from_numpy(synth.x_row_ids(st, 1)).to(dev)
        for l in range(L):
            synth.dev_fill(xs[st, l].data_ptr(), None, synth.F32, cfg.seed, synth.TAG_XA, l, d, 1.0,
                           row_ids_ptr=rid.data_ptr(), nrows=1, stream=stream)
    ws = torch.empty(pi.pi_attn_workspace_bytes(dls[0].attn), dtype=torch.uint8, device=dev)
    y = torch.empty(d, dtype=torch.float32, device=dev)
    heads = torch.empty(nh, dtype=torch.int32, device=dev)
    nas = torch.zeros((S, L), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    def timed(tau):
        def step(st):
            for l in range(L):
                pi.pi_attn_decode(dls[l].attn, t, xs[st, l], tau, y, None, heads, nas[st, l:l + 1], ws,
                                  _cstruct=dls[l].attn_c)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(0)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        gs = []
        for st in range(S):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(st)
            gs.append(g)
        for st in range(warmup):
            gs[st].replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for st in range(warmup, S):
            gs[st].replay()
        e1.record()
        torch.cuda.synchronize()
        del gs
        ms = e0.elapsed_time(e1) / steps
        na = nas[warmup:].float().mean().item()
        per_layer = (cfg.Ha * d * 2 + nh * cfg.Ha * 2 + 2 * d * d * 2 + na * (2 * dh * d * 2 + 2 * (t + 1) * dh * 2)
                     + 5 * d * 2 + 2 * d * 4 + 2 * d * 2)
        return ms, na, per_layer * L

    ms_s, na_s, b_s = timed(0.0)
    ms_d, na_d, b_d = timed(-3.0e38)
    out = {"workload": cfg.desc, "layers": L, "cached_positions": t + 1, "batch": 1,
           "tokens_per_s": round(1e3 / ms_s, 2), "ms_per_step": round(ms_s, 4), "mean_active_heads": round(na_s, 2),
           "heads": nh, "step_bytes": round(b_s), "step_gbps": round(b_s / (ms_s * 1e-3) / 1e9, 1),
           "step_frac_of_peak": round(b_s / (ms_s * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "dense_tokens_per_s": round(1e3 / ms_d, 2), "dense_ms_per_step": round(ms_d, 4),
           "dense_step_bytes": round(b_d), "dense_step_gbps": round(b_d / (ms_d * 1e-3) / 1e9, 1),
           "dense_step_frac_of_peak": round(b_d / (ms_d * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "speedup_over_dense": round(ms_d / ms_s, 3), "weight_generation_s": round(gen_s, 1)}
    del dls, xs, ws
    torch.cuda.empty_cache()
    if cpu:
        out["cpu_baseline"] = attn_cpu_baseline(cfg, 3.0)
    log(f"attention: {out['tokens_per_s']} tokens/s with {out['mean_active_heads']} of {nh} heads, "
        f"{out['dense_tokens_per_s']} with every head; step frac {out['step_frac_of_peak']}")
    return out


def attn_cpu_baseline(cfg, seconds):
    """The attention oracle on the host threads over a bounded sample of the same workload (layers in
    turn, the last cache position), scaled to the stack's layers per token."""
    import synth
    import oracle as orc
    from tests import parity_harness as ph
    t = cfg.L_max - 1
    done, el, l = 0, 0.0, 0
    while el < seconds and done < 8:
        spec = synth.attn_spec(cfg, l % cfg.n_layers)
        h = synth.attn_host(spec)
        o = ph.attn_oracle_inputs(h, cfg.d)
        x = synth.attn_x(cfg, l % cfg.n_layers, 0)
        t1 = time.perf_counter()
        orc.attn_decode(x, o["Pa1"], o["ca1"], o["Pa2"], o["ca2"], 0.0, o["Wq"], o["bq"], o["Wk"], o["bk"], o["Wv"],
                        o["bv"], o["WoT"], o["bo"], h["Kc"], h["Vc"], cfg.n_heads, cfg.dh, t)
        el += time.perf_counter() - t1
        done += 1
        l += 1
    return {"value": round(done / el / cfg.n_layers, 4), "unit": "tokens/s", "cores": orc.get_threads(),
            "kind": "oracle", "sample": f"{done} layer-steps (layers 0..{done - 1}, the last cache position) in "
                                        f"{el:.1f} s, scaled to {cfg.n_layers} layers per token; weight generation not timed"}


def read_probe_sweep(sizes=(63137536, 2**30), depths=(4, 8, 16, 32), per_cu=(1, 2, 4, 8, 16, 32), n_rep=20):
    """The streaming-read reference over its settings: loads in flight per lane x workgroups per
    compute unit, for a kernel-sized read and 1 GiB.  Successive launches read different regions of
    a 2 GiB buffer (no launch finds its bytes in the 256 MB last-level cache from the one before),
    back to back after one warm-up launch; GB/s of each setting and the best."""
    import torch
    import activation_sparse_amd as pi
    probe = torch.empty(2**29 + 4, dtype=torch.int32, device="cuda")
    out = torch.empty(4 * 256 * max(per_cu), dtype=torch.int32, device="cuda")
    res = {}
    for nb in sizes:
        nb = nb // 16 * 16
        regions = 2**31 // nb
        views = [probe[k * (nb // 4):(k + 1) * (nb // 4)] for k in range(regions)]
        table = {}
        for depth in depths:
            for pc in per_cu:
                blocks = 256 * pc
                pi.pi_read_probe(views[0], nb, out, blocks, depth=depth)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for k in range(n_rep):
                    pi.pi_read_probe(views[(k + 1) % regions], nb, out, blocks, depth=depth)
                e1.record()
                torch.cuda.synchronize()
                table[f"depth {depth} x {pc}/CU"] = round(nb * n_rep / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
        best = max(table, key=table.get)
        res[f"{nb / 1e6:.1f} MB"] = {"gbps": table, "best": best, "best_gbps": table[best]}
        log(f"read probe {nb / 1e6:.1f} MB: best {best} at {table[best]} GB/s")
    del probe, out
    return res


def placement_bench(key, steps, warmup, hybrid_steps):
    """The offline placement solver's tables against the fixed per-layer top-share rule on the
    GPU, on the same stack (`key`, whose gpu_frac sets the budget): each variant's layers are built
    with its GPU tables and timed through the batch-1 layer stack (GPU side, cold partials given)
    and through the hybrid executor (cold neurons on the host CPU, per-layer calls and the native
    look-ahead stack), with the GPU's expected share of all activations beside them."""
    import math
    import torch
    import synth
    from synth.device import DeviceLayer
    from activation_sparse_amd.placement import solve_placement, gpu_impact_share
    cfg = synth.CONFIGS[key]
    t0 = time.time()
    fixed = [synth.layer_spec(cfg, l) for l in range(cfg.n_layers)]
    k = int(math.floor(cfg.gpu_frac * cfg.N))
    tables = solve_placement([s.counts for s in fixed], [1] * cfg.n_layers, k * cfg.n_layers)
    solved = [synth.with_table(s, t) for s, t in zip(fixed, tables)]
    p = [s.p for s in fixed]
    out = {"workload": cfg.desc, "layers": cfg.n_layers, "budget_neurons": k * cfg.n_layers}
    for name, specs in (("fixed_top_share", fixed), ("solver", solved)):
        dls = [DeviceLayer(s, "cuda:0") for s in specs]
        torch.cuda.synchronize()
        gpu = stack_timing(cfg, specs, dls, steps, warmup)
        hyb = hybrid_bench(cfg, specs, dls, hybrid_steps, 1, light=True) if hybrid_steps > 0 else None
        n_g = [s.n_g for s in specs]
        out[name] = {"gpu_activation_share": round(gpu_impact_share(p, [s.T_g for s in specs]), 4),
                     "n_g_min": min(n_g), "n_g_max": max(n_g),
                     "gpu_side_tokens_per_s": round(1e3 / gpu["ms_per_step_timed_layers"], 2),
                     "gpu_side_mean_K": gpu["mean_K"], "gpu_side_step_frac_of_peak": gpu["step_frac_of_peak"],
                     "hybrid": hyb}
        del dls
        torch.cuda.empty_cache()
        log(f"placement {name}: {out[name]}")
    out["setup_and_run_s"] = round(time.time() - t0, 1)
    return out


def hybrid_bench(cfg, specs, dls, steps, warmup, light=False):
    """The pages' hybrid layer at batch 1: the CPU-table neurons live in host memory and run on the
    host CPU (libpi_host) while the GPU runs the predictor, the compaction and its own neurons; the
    CPU's partial is copied over and merged on the GPU (skipped when it has no active neuron).
    Layers are serialised as in the GPU-only measurement.  Returns None when every neuron is on
    the GPU."""
    import torch
    import synth
    from synth.device import HostColdLayer
    from activation_sparse_amd.hybrid import HybridLayer
    from activation_sparse_amd import host
    if not any(len(s.T_c) for s in specs):
        return None
    dev = "cuda:0"
    t0 = time.time()
    hls = [HostColdLayer(s, dev) for s in specs]
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    host_bytes = sum(t.numel() * t.element_size() for hl in hls for m in (hl.W1, hl.W2, hl.Wup) if m is not None
                     for t in (m.data, m.scales) if t is not None)
    hys = [HybridLayer(dl, hl, 1) for dl, hl in zip(dls, hls)]
    S, L, d = warmup + steps, len(specs), cfg.d
    xs = torch.empty((S, L, 1, d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    for t in range(S):
        rid = torch.from_numpy(synth.x_row_ids(2000 + t, 1)).to(dev)
        for l in range(L):
            synth.dev_fill(xs[t, l].data_ptr(), None, synth.F32, cfg.seed, synth.TAG_X, l, d, 1.0,
                           row_ids_ptr=rid.data_ptr(), nrows=1, stream=stream)
    y = torch.empty((1, d), dtype=torch.float32, device=dev)
    for t in range(warmup):
        for l in range(L):
            hys[l](xs[t, l], y)
    torch.cuda.synchronize()
    kcs = []
    t1 = time.perf_counter()
    for t in range(warmup, S):
        for l in range(L):
            kcs.append(hys[l](xs[t, l], y))
    torch.cuda.synchronize()
    el = time.perf_counter() - t1
    # look-ahead: each layer's neurons predicted from the previous layer's input while the CPU works
    from activation_sparse_amd.hybrid import HybridStack
    stk = HybridStack(dls, hls, 1)
    ys = [torch.empty((1, d), dtype=torch.float32, device=dev) for _ in range(L)]
    for t in range(warmup):
        stk([xs[t, l] for l in range(L)], ys)
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    for t in range(warmup, S):
        stk([xs[t, l] for l in range(L)], ys)
    torch.cuda.synchronize()
    el_ahead = time.perf_counter() - t3
    # the same in one native call per step (no per-layer Python call)
    t4 = time.perf_counter()
    for t in range(warmup, S):
        stk.native([xs[t, l] for l in range(L)], ys)
    torch.cuda.synchronize()
    el_native = time.perf_counter() - t4
    del stk
    if light:   # the three timings only (no CPU-alone timing, no host read probe)
        out = {"tokens_per_s": round(steps / el, 2), "ms_per_step": round(el * 1e3 / steps, 3),
               "lookahead_native_tokens_per_s": round(steps / el_native, 2),
               "lookahead_tokens_per_s": round(steps / el_ahead, 2), "steps": steps,
               "mean_K_c": float(np.mean(kcs)), "host_weights_gib": round(host_bytes / 2**30, 2)}
        del hys, hls
        return out
    # the CPU side alone: each layer's last cold list and input again, through pi_cold_ffn
    y_h = np.empty((1, d), np.float32)
    t2 = time.perf_counter()
    for h in hys:
        kc = int(h.K_c_h[0])
        if kc:
            host.pi_cold_ffn(1, d, h.n_c, h.x_h, h.hl.W1, h.hl.b1, h.hl.W2, h.A_c_h, kc, y_h,
                             kind=pi_kind(cfg), Wup=h.hl.Wup)
    host_s = (time.perf_counter() - t2) * steps
    # the host's own streaming read with the same threads, over a 2 GiB buffer (successive reads
    # take different regions, as successive layers read different rows): the CPU side's reference
    w_cold = wbytes(cfg.wdtype) * d * (2 if cfg.gated else 1)
    fc1_bytes = float(np.mean(kcs)) * w_cold
    span = 2**31
    raw = np.ones(span // 8 + 8, np.uint64)
    base = raw.ctypes.data + (-raw.ctypes.data % 64)
    host_read = {}
    for nb in (int(fc1_bytes) // 64 * 64, 256 * 2**20):
        best = 0.0
        for k in range(24):
            off = (k * ((nb + 4095) // 4096 * 4096)) % (span - nb - 64)
            t5 = time.perf_counter()
            host.pi_host_read_probe(base + off, nb, 0)
            best = max(best, nb / (time.perf_counter() - t5) / 1e9)
        host_read[f"{nb / 1e6:.1f} MB"] = round(best, 1)
    del raw
    cold_gbps = fc1_bytes / (host_s / (steps * L)) / 1e9
    out = {"tokens_per_s": round(steps / el, 2), "ms_per_step": round(el * 1e3 / steps, 3), "steps": steps,
           "layers": L, "host_weights_gib": round(host_bytes / 2**30, 2),
           "cpu_threads": int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count(),
           "cpu_vector_path": "avx2+fma+f16c" if host.vector_path() else "scalar",
           "cpu_cold_ffn_us_per_layer": round(host_s * 1e6 / (steps * L), 1),
           "mean_K_c": float(np.mean(kcs)), "host_weight_setup_s": round(gen_s, 1),
           "lookahead_tokens_per_s": round(steps / el_ahead, 2), "lookahead_ms_per_step": round(el_ahead * 1e3 / steps, 3),
           "lookahead_native_tokens_per_s": round(steps / el_native, 2),
           "lookahead_native_ms_per_step": round(el_native * 1e3 / steps, 3),
           "cold_fc1_bytes_per_layer": round(fc1_bytes), "cold_ffn_gbps_fc1_only": round(cold_gbps, 1),
           "host_stream_read_gbps": host_read}
    log(f"hybrid: host streaming read {host_read} GB/s; the cold FFN moves at least {out['cold_ffn_gbps_fc1_only']} "
        f"GB/s (its FC1 rows alone)")
    log(f"hybrid: {out['ms_per_step']} ms/step, {out['tokens_per_s']} tokens/s, cold FFN on the CPU "
        f"{out['cpu_cold_ffn_us_per_layer']} us per layer (timed alone); with look-ahead prediction "
        f"{out['lookahead_ms_per_step']} ms/step, {out['lookahead_tokens_per_s']} tokens/s; in one native call per "
        f"step {out['lookahead_native_ms_per_step']} ms/step, {out['lookahead_native_tokens_per_s']} tokens/s")
    del hys, hls
    return out


def boundary_probe(reps=200):
    """What one dependent kernel boundary costs inside a HIP graph, from torch's own small kernels
    (no library code): a 256-element add alone; the same add after a fill of X bytes (a kernel that
    leaves X bytes written); and a column sum over a [32 x 7168] fp32 array (the shape of the batch-1
    layer's FC2 partials) right after a fill of that same array or of another one.  Each figure is
    the graph time per repetition (best of five replays of reps repetitions) minus that of the
    graph without the measured kernel."""
    import torch
    dev = "cuda:0"

    def graph(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
        return g

    def per_rep(g):
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        best = float("inf")
        for _ in range(5):
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e3 / reps)
        return best

    small = torch.zeros(256, device=dev)
    big = torch.zeros(64 << 20, dtype=torch.uint8, device=dev)
    out = {"tiny_kernel_alone_us": round(per_rep(graph(lambda: small.add_(1.0))), 3), "tiny_after_write_us": {}}
    for X in (4 << 10, 1 << 20, 8 << 20, 64 << 20):
        v = big[:X]
        tf = per_rep(graph(lambda: v.fill_(1)))
        tfa = per_rep(graph(lambda: (v.fill_(1), small.add_(1.0))))
        out["tiny_after_write_us"][f"{X >> 10} KiB"] = round(tfa - tf, 3)
    P = torch.randn(32, 7168, device=dev)
    Q = torch.randn(32, 7168, device=dev)
    y = torch.zeros(7168, device=dev)
    colsum = lambda: torch.sum(P, dim=0, out=y)
    out["column_sum_alone_us"] = round(per_rep(graph(colsum)), 3)
    for name, src in (("same_array", P), ("other_array", Q)):
        tw = per_rep(graph(lambda: src.fill_(0.5)))
        twr = per_rep(graph(lambda: (src.fill_(0.5), colsum())))
        out[f"column_sum_after_fill_of_{name}_us"] = round(twr - tw, 3)
    del big, P, Q
    torch.cuda.empty_cache()
    return out


def warm_probe(cfg, specs, dls, reps=10):
    """The batch-1 layer's latency floor: one HIP graph over the stack's layers, one call each (their
    bytes come from HBM), against graphs that call each layer two and three times in a row (the
    repeated calls find the layer's bytes in the caches), and against one that runs each layer's
    hidden-layer stage alone just before its call (only the predictor's hidden-layer rows warm).
    Per-layer figures are differences of whole-graph times (best of `reps` replays)."""
    import torch
    import activation_sparse_amd as pi
    dev = "cuda:0"
    nl = len(specs)
    d, N = cfg.d, cfg.N
    n_g = max(s.n_g for s in specs)
    n_c = max(len(s.T_c) for s in specs)
    H = max(s.H for s in specs)
    ws_bytes = pi.pi_workspace_bytes(pi.PI_OP_FFN_LAYER, 1, d, H, N, n_g)
    wss = [torch.zeros(ws_bytes, dtype=torch.uint8, device=dev) for _ in range(nl)]
    g0 = torch.Generator(device="cpu").manual_seed(5)
    xs = torch.randn((nl, d), generator=g0).to(dev)
    yc = (torch.randn((nl, d), generator=g0) * 0.05).to(dev)
    y = torch.empty(d, device=dev)
    A_g = torch.empty(max(n_g, 1), dtype=torch.int32, device=dev)
    A_c = torch.empty(max(n_c, 1), dtype=torch.int32, device=dev)
    K = torch.zeros(nl, dtype=torch.int32, device=dev)
    K_c = torch.zeros(nl, dtype=torch.int32, device=dev)

    def call(L, st):
        cold = len(specs[L].T_c) > 0
        pi.pi_ffn_layer_stages(dls[L].layer, 1, xs[L], 0.0, yc[L] if cold else None, y, None, A_g, K[L:L + 1],
                               A_c if cold else None, K_c[L:L + 1] if cold else None, wss[L], st,
                               _cstruct=dls[L].layer_c)

    def graph_time(seq):
        for L, st in seq:
            call(L, st)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for L, st in seq:
                call(L, st)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        best = float("inf")
        for _ in range(reps):
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e3)
        del g
        return best

    A, Hs = pi.PI_STAGE_ALL, pi.PI_STAGE_HIDDEN
    t1 = graph_time([(L, A) for L in range(nl)])
    t2 = graph_time([(L, A) for L in range(nl) for _ in range(2)])
    t3 = graph_time([(L, A) for L in range(nl) for _ in range(3)])
    th = graph_time([(L, Hs) for L in range(nl)])
    tha = graph_time([(L, s) for L in range(nl) for s in (Hs, A)])
    out = {"layers": nl, "cold_us_per_layer": round(t1 / nl, 2),
           "warm_second_call_us_per_layer": round((t2 - t1) / nl, 2),
           "warm_third_call_us_per_layer": round((t3 - t2) / nl, 2),
           "hidden_stage_alone_us_per_layer": round(th / nl, 2),
           "after_hidden_stage_us_per_layer": round((tha - th) / nl, 2)}
    out["warm_tokens_per_s_bound"] = round(1e6 / (out["warm_second_call_us_per_layer"] * nl), 1)
    del wss
    torch.cuda.empty_cache()
    return out


def host_cold_scaling(threads=(1, 2, 4, 8, 16), reps=300):
    """The host cold FFN (pi_cold_ffn, batch 1) at the OPT-30B cold table's shape, by thread count:
    FC1 alone (every FC1 output zero, so FC2 is skipped) over 497 listed rows of a 17,204 x 7,168 fp16
    table, with the rows streamed from DRAM (four tables and 64 lists in turn) or cached (one table, one
    list), and the full call (half the outputs non-zero) streamed.  Seeded normal weights (the time does
    not depend on their values).  Median microseconds per call, from Python (a call with one listed
    neuron gives the fixed cost)."""
    import time
    import numpy as np
    from activation_sparse_amd import host, Matrix, Vector, PI_F16, PI_F32
    d, n_c, K_c, NT = 7168, 17204, 497, 4
    rng = np.random.default_rng(0)

    def table():
        a = np.empty((n_c, d), np.float16)
        for i in range(0, n_c, 2048):
            a[i:i + 2048] = (rng.standard_normal((min(2048, n_c - i), d), dtype=np.float32) / np.sqrt(d)).astype(np.float16)
        return Matrix(a, PI_F16)
    W1 = [table() for _ in range(NT)]
    W2 = table()
    x = rng.standard_normal((1, d), dtype=np.float32)
    y = np.zeros((1, d), np.float32)
    b_mid = Vector(np.zeros(n_c, np.float32), PI_F32)
    b_off = Vector(np.full(n_c, -1e9, np.float32), PI_F32)
    lists = [np.sort(rng.choice(n_c, K_c, replace=False)).astype(np.int32) for _ in range(64)]

    def med(b1, rotate, T, k=K_c):
        ts = []
        for i in range(reps):
            W, lst = (W1[i % NT], lists[i % 64]) if rotate else (W1[0], lists[0])
            t0 = time.perf_counter()
            host.pi_cold_ffn(1, d, n_c, x, W, b1, W2, lst[:k], k, y, threads=T)
            ts.append(time.perf_counter() - t0)
        return round(float(np.median(ts[reps // 10:])) * 1e6, 1)
    out = {"vector_path": host.vector_path(), "fixed_us": med(b_off, False, 0, k=1), "by_threads": {}}
    for T in threads:
        out["by_threads"][str(T)] = {"fc1_streamed_us": med(b_off, True, T), "fc1_cached_us": med(b_off, False, T),
                                      "full_streamed_us": med(b_mid, True, T)}
    return out


def run_leg(args):
    """One leg alone, so that a profiler run holds just its kernels: 'truth' or 'chained' (on
    --config's stack), 'placement', 'attention', 'batch-sweep' (--sweep's batches on --config's
    stack), 'read-probe' (the streaming-read reference's sweep), 'boundary' (the cost of a dependent
    kernel boundary in a graph), 'warm' (the layer with its bytes already in the caches, on --config's
    stack), 'host-cold' (the host cold FFN by thread count), or 'config:KEY[:STRIDE]'.  Returns that leg's result (not the benchmark line)."""
    import torch
    import synth
    from synth.device import DeviceLayer
    name, _, rest = args.leg.partition(":")
    torch.cuda.set_device(0)
    if name == "config":
        key, _, stride = rest.partition(":")
        res = config_bench(key, args.config_steps, 2, int(stride or 1), cpu=not args.no_cpu_baseline)
    elif name == "truth":
        cfg = synth.CONFIGS[args.config]
        specs = [synth.layer_spec(cfg, L) for L in range(args.layers or cfg.n_layers)]
        dls = [DeviceLayer(s, "cuda:0") for s in specs]
        torch.cuda.synchronize()
        res = truth_bench(cfg, specs, dls, args.truth_steps, 2)
    elif name == "chained":
        cfg = synth.CONFIGS[args.config]
        specs = [synth.layer_spec(cfg, L) for L in range(args.layers or cfg.n_layers)]
        dls = [DeviceLayer(s, "cuda:0") for s in specs]
        torch.cuda.synchronize()
        res = chained_bench(cfg, specs, dls, args.chained_steps, 3)
    elif name == "batch-sweep":
        cfg = synth.CONFIGS[args.config]
        specs = [synth.layer_spec(cfg, L) for L in range(args.layers or cfg.n_layers)]
        dls = [DeviceLayer(s, "cuda:0") for s in specs]
        torch.cuda.synchronize()
        batches = [int(v) for v in args.sweep.split(",") if v.strip()]
        res = batch_sweep(cfg, specs, dls, batches, args.sweep_steps, 2)
        res["matrix_core_min_batch_env"] = os.environ.get("PI_MATRIX_CORE_MIN_BATCH")
    elif name == "attention":
        res = attn_bench(args.attn_steps, 2, cpu=not args.no_cpu_baseline)
    elif name == "read-probe":
        res = read_probe_sweep()
    elif name == "placement":
        res = placement_bench("llama-13b-gated-40", args.placement_steps, 2, args.placement_steps)
    elif name == "boundary":
        res = boundary_probe()
    elif name == "host-cold":
        res = host_cold_scaling()
    elif name == "warm":
        cfg = synth.CONFIGS[args.config]
        specs = [synth.layer_spec(cfg, L) for L in range(args.layers or cfg.n_layers)]
        dls = [DeviceLayer(s, "cuda:0") for s in specs]
        torch.cuda.synchronize()
        res = warm_probe(cfg, specs, dls)
    else:
        raise SystemExit(f"bench.py: unknown leg {args.leg!r} (truth, chained, placement, attention, "
                         "batch-sweep, read-probe, boundary, warm, host-cold, config:KEY[:STRIDE])")
    return {"leg": args.leg, "result": res}


def main():
    args = parse()
    if args.rocprof_summary:
        print(rocprof_summary(args.rocprof_summary, args.copy_mib))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on exactly one GPU; --gpus N with N > 1 is not supported "
              "(the multi-GPU sharding is a design note only).", file=sys.stderr)
        sys.exit(2)
    if args.leg:
        print(json.dumps(run_leg(args)), flush=True)
        return
    import torch
    import synth
    import activation_sparse_amd as pi
    from synth.device import DeviceLayer

    cfg = synth.CONFIGS[args.config]
    B = args.batch
    n_layers = args.layers or cfg.n_layers
    dev = "cuda:0"
    torch.cuda.set_device(0)
    S = args.warmup + args.steps
    t_setup = time.time()
    specs = [synth.layer_spec(cfg, L) for L in range(n_layers)]
    log(f"{cfg.key}: {n_layers} layer specs ready in {time.time() - t_setup:.1f} s")
    dls = [DeviceLayer(s, dev) for s in specs]
    torch.cuda.synchronize()
    log(f"device weights generated ({torch.cuda.memory_allocated() / 2**30:.1f} GiB) at {time.time() - t_setup:.1f} s")
    maxH = max(s.H for s in specs)
    n_g = max(s.n_g for s in specs)
    n_c = max(len(s.T_c) for s in specs)
    d, N = cfg.d, cfg.N

    class Buffers:
        logits = torch.empty((B, N), dtype=torch.float32, device=dev)
        A_g = torch.empty(max(n_g, 1), dtype=torch.int32, device=dev)
        A_c = torch.empty(max(n_c, 1), dtype=torch.int32, device=dev)
        y = torch.empty((B, d), dtype=torch.float32, device=dev)
    buf = Buffers
    # one workspace per layer, so that a stage re-run alone sees its own layer's state
    ws_bytes = max(pi.pi_workspace_bytes(pi.PI_OP_FFN_LAYER, B, d, maxH, N, n_g), 256)
    wss = [torch.empty(ws_bytes, dtype=torch.uint8, device=dev) for _ in range(n_layers)]
    # per-(step, layer) inputs, cold partials, counts and rows read
    xs = torch.empty((S, n_layers, B, d), dtype=torch.float32, device=dev)
    ycs = torch.empty((S, n_layers, B, d), dtype=torch.float32, device=dev) if n_c else None
    Ks = torch.zeros((S, n_layers), dtype=torch.int32, device=dev)
    Kcs = torch.zeros((S, n_layers), dtype=torch.int32, device=dev)
    rows = torch.zeros((S, n_layers, 2), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    for t in range(S):
        rid = torch.from_numpy(synth.x_row_ids(t, B)).to(dev)
        for L in range(n_layers):
            synth.dev_fill(xs[t, L].data_ptr(), None, synth.F32, cfg.seed, synth.TAG_X, L, d, 1.0,
                           row_ids_ptr=rid.data_ptr(), nrows=B, stream=stream)
            if n_c:
                synth.dev_fill(ycs[t, L].data_ptr(), None, synth.F32, cfg.seed, synth.TAG_YC, L, d, 0.05,
                               row_ids_ptr=rid.data_ptr(), nrows=B, stream=stream)
    torch.cuda.synchronize()

    def layer_call(t, L, events=None, stages=pi.PI_STAGE_ALL):
        spec, dl = specs[L], dls[L]
        cold = len(spec.T_c) > 0
        pi.pi_ffn_layer_stages(dl.layer, B, xs[t, L], 0.0, ycs[t, L] if cold else None, buf.y, None, buf.A_g,
                               Ks[t, L:L + 1], buf.A_c if cold else None, Kcs[t, L:L + 1] if cold else None, wss[L],
                               stages, rows_read=rows[t, L], events=events, _cstruct=dl.layer_c)

    def step_call(t):
        for L in range(n_layers):
            layer_call(t, L)

    graphs = []
    use_graph = not args.no_graph
    if use_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step_call(0)          # eager warm-up of every kernel before capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for t in range(S):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step_call(t)
            graphs.append(g)
        torch.cuda.synchronize()
    setup_s = time.time() - t_setup
    log(f"setup done in {setup_s:.1f} s (graphs: {len(graphs)}); timing {args.steps} steps")

    def run_step(t):
        if use_graph:
            graphs[t].replay()
        else:
            step_call(t)

    for t in range(args.warmup):
        run_step(t)
    torch.cuda.synchronize()
    # one event between consecutive steps: the first and last bracket the timed region, the others
    # give each step's duration (for the median)
    evs_step = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    evs_step[0].record()
    for i, t in enumerate(range(args.warmup, S)):
        run_step(t)
        evs_step[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = evs_step[0].elapsed_time(evs_step[-1])
    step_ms = [evs_step[i].elapsed_time(evs_step[i + 1]) for i in range(args.steps)]
    elapsed_s = max(wall, gpu_ms / 1e3)
    ms_per_step = elapsed_s * 1e3 / args.steps
    tokens_s = B * args.steps / elapsed_s

    # algorithmic bytes of the timed steps from the measured counts and rows read
    Kh = Ks.cpu().numpy()
    Kch = Kcs.cpu().numpy()
    Rh = rows.cpu().numpy()
    tot_pred = tot_ffn = tot_small = 0.0
    for t in range(args.warmup, S):
        for L in range(n_layers):
            p, f, sm = layer_bytes(specs[L], B, int(Kh[t, L]), int(Kch[t, L]), int(Rh[t, L, 0]), int(Rh[t, L, 1]))
            tot_pred += p; tot_ffn += f; tot_small += sm
    step_bytes = (tot_pred + tot_ffn + tot_small) / args.steps
    step_gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    step_ms_median = float(np.median(step_ms))
    # bytes a dense predictor (every P2 row) and an FC2 over every listed neuron would read
    dense_bytes = 0.0
    for t in range(args.warmup, S):
        for L in range(n_layers):
            p, f, sm = layer_bytes(specs[L], B, int(Kh[t, L]), int(Kch[t, L]), specs[L].H, int(Kh[t, L]))
            dense_bytes += p + f + sm
    dense_bytes /= args.steps

    # per-stage durations: each stage set re-run alone, back to back over the layers in one HIP graph
    # (launch overhead not timed) between two events on the launch stream, on the state the last
    # step left in each layer's workspace (so each launch repeats that step's work exactly and its
    # bytes are that step's).  At batch 1 the output layer, the activation decision and FC1 are
    # one kernel (the dominant one).
    last = S - 1
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def stage_graph_ms(bits, reps):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for L in range(n_layers):
                layer_call(last, L, stages=bits)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                for L in range(n_layers):
                    layer_call(last, L, stages=bits)
        g.replay()
        torch.cuda.synchronize()
        d0.record()
        g.replay()
        d1.record()
        torch.cuda.synchronize()
        del g
        return d0.elapsed_time(d1) / (reps * n_layers)

    stage_bits = {"hidden": pi.PI_STAGE_HIDDEN,
                  "output+fc1": pi.PI_STAGE_OUTPUT if B == 1 else (pi.PI_STAGE_OUTPUT | pi.PI_STAGE_FC1),
                  "fc2+lists": pi.PI_STAGE_FC2, "sum+merge": pi.PI_STAGE_SUM}
    kb_last = [kernel_bytes(specs[L], B, int(Kh[last, L]), int(Kch[last, L]), int(Rh[last, L, 0]), int(Rh[last, L, 1]))
               for L in range(n_layers)]
    mean_ms = {k: stage_graph_ms(b, 5) for k, b in stage_bits.items()}
    mean_bytes = {k: float(np.mean([kb[k] for kb in kb_last])) for k in STAGES}
    achieved = {k: (mean_bytes[k] / (mean_ms[k] * 1e-3) / 1e9 if mean_ms[k] > 0 else 0.0) for k in STAGES}
    # the dominant kernel, timed on its own as above
    dom = "output+fc1"
    iso = dom + " (isolated)"
    mean_ms[iso] = mean_ms[dom]
    mean_bytes[iso] = mean_bytes[dom]
    achieved[iso] = achieved[dom]
    dom_bytes = mean_bytes[dom]
    traffic = committed_traffic(DOMINANT) if (cfg.key == "opt-30b" and B == 1) else None
    roofline = {"bound": "hbm", "achieved": round(achieved[iso], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved[iso] / HBM_PEAK_GBS, 4),
                "traffic": round(traffic) if traffic is not None else None,
                "kernel": (DOMINANT + " (predictor output layer over the active hidden units + activation decision "
                           "+ FC1; pi_ffn_layer_stages PI_STAGE_OUTPUT)") if B == 1 else
                          ("output layer + lists + FC1, several kernels (pi_ffn_layer_stages PI_STAGE_OUTPUT | "
                           "PI_STAGE_FC1)"),
                "bytes_per_launch": round(mean_bytes[iso]), "avg_launch_us": round(mean_ms[iso] * 1e3, 2)}

    # the streaming-read reference: a plain read of the dominant kernel's bytes per launch, of one
    # layer-token's bytes and of 1 GiB, best over loads in flight per lane and grid sizes, back to
    # back on the launch stream.
    # Successive launches read different regions of a 2 GiB buffer, as the layers read different
    # weights, so that no launch finds its bytes in the last-level cache (256 MB) from the one before.
    stream_read = {}
    probe = torch.empty(2**29 + 4, dtype=torch.int32, device=dev)
    probe_out = torch.empty(4 * 8192, dtype=torch.int32, device=dev)
    layer_bytes_mean = step_bytes / n_layers
    for nb in (int(dom_bytes) // 16 * 16, int(layer_bytes_mean) // 16 * 16, 2**30):
        best = 0.0
        regions = 2**31 // nb
        views = [probe[k * (nb // 4):(k + 1) * (nb // 4)] for k in range(regions)]
        for depth, blocks in [(dp, 256 * pc) for dp in (8, 16) for pc in (1, 2, 4, 8, 16, 32)]:
            pi.pi_read_probe(views[0], nb, probe_out, blocks, depth=depth)
            r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n_rep = 20
            r0.record()
            for k in range(n_rep):
                pi.pi_read_probe(views[(k + 1) % regions], nb, probe_out, blocks, depth=depth)
            r1.record()
            torch.cuda.synchronize()
            best = max(best, nb * n_rep / (r0.elapsed_time(r1) * 1e-3) / 1e9)
        stream_read[f"{nb / 1e6:.1f} MB"] = round(best, 1)
    del probe, probe_out
    dom_ref = list(stream_read.values())[0]

    log(f"timed: {ms_per_step:.4f} ms/step, {tokens_s:.1f} tokens/s")
    log(f"streaming read: {stream_read} GB/s; dominant kernel at {achieved[iso] / dom_ref:.3f} of the read "
        f"of its own size")
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(cfg, B, args.cpu_seconds, args.cpu_layers)

    hybrid = None
    if args.hybrid_steps > 0 and B == 1:
        log("hybrid layer (cold neurons on the host CPU) ...")
        hybrid = hybrid_bench(cfg, specs, dls, args.hybrid_steps, 1)

    i4pred = None
    if args.i4pred_steps > 0 and B == 1:
        log("int4 predictor weights ...")
        i4pred = i4pred_bench(cfg, specs, dls, args.i4pred_steps, 3)

    lookahead = None
    if args.lookahead_steps > 0 and B == 1:
        log("look-ahead prediction ...")
        lookahead = lookahead_bench(cfg, specs, dls, args.lookahead_steps, 3)

    chained = None
    if args.chained_steps > 0 and B == 1:
        log("chained layers ...")
        chained = chained_bench(cfg, specs, dls, args.chained_steps, 3)

    truth = None
    if args.truth_steps > 0 and B == 1 and cfg.wdtype != 2:
        log("truth mode (the true activation set as the mask) ...")
        truth = truth_bench(cfg, specs, dls, args.truth_steps, 2)
        log(f"truth mode: {truth['tokens_per_s']} tokens/s, FC2 rows read {truth['mean_fc2_rows_read']:.0f} of "
            f"{truth['mean_K']:.0f} listed, true density {truth['true_density']}")

    configs = {}
    for item in [v for v in args.configs.split(",") if v.strip()] if B == 1 else []:
        key, _, stride = item.partition(":")
        configs[key] = config_bench(key, args.config_steps, 2, int(stride or 1))

    attention = None
    if args.attn_steps > 0 and B == 1:
        log("self-attention stack with head sparsity ...")
        attention = attn_bench(args.attn_steps, 2, cpu=not args.no_cpu_baseline)

    placement = None
    if args.placement and B == 1:
        log("placement solver (host) ...")
        placement = placement_report([cfg.key] + (["llama-13b-gated"] if cfg.key != "llama-13b-gated" else []))
        if args.placement_steps > 0:
            log("placement solver's tables against the fixed rule on the GPU (llama-13b-gated-40) ...")
            placement["llama-13b-gated-40"] = placement_bench("llama-13b-gated-40", args.placement_steps, 2,
                                                              args.placement_steps)

    sweep = None
    batches = [int(v) for v in args.sweep.split(",") if v.strip()] if args.sweep else []
    if batches and B == 1:
        log(f"batch sweep {batches} ...")
        sweep = batch_sweep(cfg, specs, dls, batches, args.sweep_steps, 2)

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * 2**20 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    out = {
        "metric": "sparse-FFN decode tokens/s at batch 1; achieved HBM GB/s vs peak",
        "value": round(tokens_s, 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {0: "f32", 1: "f16", 2: "int4"}[cfg.wdtype] + "-weights/f32-accumulate",
        "data": "synthetic (seeded power-law-sparse layers, random-init weights, generated on device)",
        "config": {"workload": cfg.desc, "key": cfg.key, "layers": n_layers, "batch": B, "d_model": d,
                   "d_ffn": N, "predictor_hidden": maxH, "gpu_neurons": n_g, "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "detail": {"step_bytes": round(step_bytes), "step_gbps": round(step_gbs, 1),
                   "step_frac_of_peak": round(step_gbs / HBM_PEAK_GBS, 4),
                   "step_ms_median": round(step_ms_median, 4),
                   "step_frac_of_peak_median": round(step_bytes / (step_ms_median * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                   "bytes_split": {"predictor": round(tot_pred / args.steps), "ffn": round(tot_ffn / args.steps),
                                   "small": round(tot_small / args.steps)},
                   "step_bytes_if_dense_p2_and_full_fc2": round(dense_bytes),
                   "mean_K": float(Kh[args.warmup:].mean()), "mean_K_cold": float(Kch[args.warmup:].mean()),
                   "mean_p2_rows_read": float(Rh[args.warmup:, :, 0].mean()),
                   "mean_fc2_rows_read": float(Rh[args.warmup:, :, 1].mean()),
                   "kernel_us": {k: round(v * 1e3, 2) for k, v in mean_ms.items()},
                   "kernel_gbps": {k: round(v, 1) for k, v in achieved.items()},
                   "graph": use_graph, "setup_s": round(setup_s, 1), "wall_s": round(wall, 4),
                   "event_ms": round(gpu_ms, 3),
                   "stream_read_gbps": stream_read,
                   "dominant_frac_of_stream_read": round(achieved[iso] / dom_ref, 4),
                   "batch_sweep": sweep, "hybrid": hybrid, "lookahead": lookahead, "chained": chained, "int4_predictor": i4pred,
                   "placement": placement, "attention": attention, "truth": truth, "rho20": configs.pop("opt-30b-rho20", None),
                   "configs": configs or None},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
