#!/usr/bin/env python3
"""Lighthouse Attention layer, forward + backward, on one MI355X.

One step = lh_pyramid + lh_score_topk + lh_forward + lh_backward over the
whole layer (all heads) on seeded synthetic inputs already resident in HBM;
selection is recomputed every step, as in training.  The workload is the
530M Llama-3-style attention layer at 98,304 tokens with k = 1536
(B=1, H=16, N=98304, d=64, bf16, p=4, L=4; S = 19968).

Prints ONE JSON line: tokens/s of the layer (B*N per step), the dense causal
attention baseline on the same GPU and inputs (speedup, fwd+bwd and forward
only), the roofline of the dominant kernel measured live with HIP events on
the library's stream, and the CPU oracle timed on a bounded sample.  Other
workloads of the parity suite can be timed with --workload NAME (their lines
are reported alongside, never as the headline value).

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0    # dense bf16 matrix cores
MFMA_F32_PEAK_TFS = 157.3

KERNEL_NAMES = ["pool", "score", "topk", "map", "gather", "attn_fwd", "scatter_fwd", "scatter_bwd",
                "attn_dkdv", "attn_dq", "gather_pool_bwd"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama530m_98k_k1536")
    ap.add_argument("--dense-steps", type=int, default=5)
    ap.add_argument("--probe-reps", type=int, default=5, help="probed steps per kernel (median)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extreme", action="store_true", help="skip the 512K-token sub-object")
    ap.add_argument("--extreme-steps", type=int, default=5)
    ap.add_argument("--extreme-dense", type=int, default=1, help="time one dense step at 512K (0: skip)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="also run one plain device copy of 1 GiB (scales rocprofv3 byte counters)")
    ap.add_argument("--pmc-summary", nargs="+", metavar="DIR",
                    help="print per-dispatch counter averages from rocprofv3 --pmc output directories and exit")
    return ap.parse_args()


# Files whose content determines each group of kernels: a stored HBM traffic
# figure is reported only while its group's files are unchanged.
_CSRC = "long_context_pretraining_amd/csrc/"
SOURCE_GROUPS = {
    "attn": [_CSRC + "lh_attention.hip", _CSRC + "lh_device.h", _CSRC + "lh_internal.h"],
    "select": [_CSRC + "lh_select.hip", _CSRC + "lh_device.h", _CSRC + "lh_internal.h"],
    "scatter": [_CSRC + "lh_scatter.hip", _CSRC + "lh_device.h", _CSRC + "lh_internal.h"],
    "proj": [_CSRC + "lh_proj.hip", _CSRC + "lh_device.h", _CSRC + "lh_internal.h"],
}
ATTN_SOURCES = SOURCE_GROUPS["attn"]
# bench name -> the kernel symbols (as the profiles name them) its call launches, and their source
# group; a call with several forms lists each form's symbols (the first form found in a profile counts)
KERNEL_SYMBOLS = {
    # pooling also gives the token norms, in its own pass where its lanes do not hold whole rows
    "pool": ((("pool_kernel",), ("pool_kernel", "norm_kernel")), "select"), "score": (("score_kernel",), "select"),
    "topk": (("topk_kernel",), "select"), "map": (("map_kernel",), "select"),
    "gather": (("gather_kernel",), "scatter"), "attn_fwd": (("attn_fwd_kernel",), "attn"),
    "scatter_fwd": (("scatter_fwd_kernel",), "scatter"),
    "scatter_bwd": ((("scatter_bwd_kernel",), ("scatter_bwd_tree_kernel", "slot_dot_kernel")), "scatter"),
    "attn_dkdv": (("attn_dkdv_kernel",), "attn"), "attn_dq": (("attn_dq_kernel",), "attn"),
    "gather_pool_bwd": (("gpool_bwd_kernel",), "scatter"),
}
SCATTER_EXTRA = ("transpose_kernel",)   # f32 helper of the scatter group


def kernel_forms(kernel):
    """The alternative symbol tuples of bench kernel `kernel`."""
    syms = KERNEL_SYMBOLS[kernel][0]
    return syms if isinstance(syms[0], tuple) else (syms,)
TRAFFIC_PROFILE = "profiles/lighthouse_98k_k1536_hbm_traffic.md"


def sources_sha256(paths):
    import hashlib
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for p in paths:
        with open(os.path.join(root, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def symbol_group(symbol):
    for name, (_, group) in KERNEL_SYMBOLS.items():
        if any(symbol in form for form in kernel_forms(name)):
            return group
    if symbol in SCATTER_EXTRA:
        return "scatter"
    if symbol.startswith("gemm_nt_kernel") or symbol in ("transpose_slabs_kernel", "reduce_splits_kernel"):
        return "proj"
    return None


def stored_traffic(kernel, workload="llama530m_98k_k1536"):
    """HBM bytes per launch of bench kernel `kernel` from the committed counter
    summary of the headline workload (FETCH_SIZE + WRITE_SIZE, each scaled by
    a plain copy of known size), or None when there is none, the workload is
    another one, or the kernel's sources changed since."""
    if workload != "llama530m_98k_k1536" or kernel not in KERNEL_SYMBOLS:
        return None
    group = KERNEL_SYMBOLS[kernel][1]
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, TRAFFIC_PROFILE)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.startswith("- "):
                key, val = line[2:].split(":", 1)
                fields[key.strip()] = val.strip().strip("`")
    if fields.get(f"sources_sha256.{group}") != sources_sha256(SOURCE_GROUPS[group]):
        return None
    for form in kernel_forms(kernel):
        vals = [fields.get(f"hbm_bytes_per_launch.{sym}") for sym in form]
        if all(v is not None for v in vals):
            return sum(int(v) for v in vals)
    return None


# the three instantiations of the projection GEMM, told apart by their operand / epilogue types
GEMM_ROLES = (("QkvOut", "qkv_fwd"), ("HeadMajorOp", "qkv_dx"), ("RowMajorOut<float>", "qkv_dw"),
              ("RowMajorOutIf", "qkv_dw"))


def short_kernel_name(name):
    import re
    if "gemm_nt_kernel" in name:
        role = next((r for key, r in GEMM_ROLES if key in name), "?")
        return f"gemm_nt_kernel[{role}]"
    m = re.search(r"_GLOBAL__N_1(\d+)", name)   # mangled: <length><identifier>
    if m:
        return name[m.end():m.end() + int(m.group(1))]
    m = re.search(r"(\w+)(?:<|\()", name)
    return m.group(1) if m else name[:40]


def pmc_summary(dirs):
    """Markdown tables from rocprofv3 --output-format csv directories: the
    kernel statistics of a --kernel-trace --stats run, and per-dispatch
    counter averages per kernel of --pmc runs."""
    import csv
    import glob
    trace_avg = {}
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True):
            print("| kernel | calls | total ms | avg us | min us | max us |")
            print("|---|---:|---:|---:|---:|---:|")
            with open(path) as f:
                for r in csv.DictReader(f):
                    trace_avg.setdefault(short_kernel_name(r["Name"]), round(float(r["AverageNs"]) / 1e3, 1))
                    print(f"| {short_kernel_name(r['Name'])} | {r['Calls']} | {int(r['TotalDurationNs']) / 1e6:.3f} | "
                          f"{float(r['AverageNs']) / 1e3:.1f} | {int(r['MinNs']) / 1e3:.1f} | {int(r['MaxNs']) / 1e3:.1f} |")
            print()
    agg, cnt = {}, {}
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    short = short_kernel_name(r["Kernel_Name"])
                    key = (short, r["Counter_Name"])
                    agg[key] = agg.get(key, 0.0) + float(r["Counter_Value"])
                    cnt[key] = cnt.get(key, 0) + 1
    if not agg:
        return
    counters = sorted({c for _, c in agg})
    kernels = sorted({k for k, _ in agg})
    print("| kernel | " + " | ".join(f"{c} (avg/dispatch)" for c in counters) + " | dispatches |")
    print("|---|" + "---:|" * (len(counters) + 1))
    for k in kernels:
        vals = [f"{agg[(k, c)] / cnt[(k, c)]:.1f}" if (k, c) in agg else "" for c in counters]
        n = max(cnt.get((k, c), 0) for c in counters)
        print(f"| {k} | " + " | ".join(vals) + f" | {n} |")
    # with both byte counters and the 1 GiB calibration copy: scaled HBM bytes per launch,
    # the rate over the kernel-trace average (when a trace directory was given) and the
    # machine-read lines stored_traffic() takes
    copy = "__amd_rocclr_copyBuffer"
    if not all((copy, c) in agg for c in ("FETCH_SIZE", "WRITE_SIZE")):
        return
    gib_kib = float(1 << 20)
    f_scale = gib_kib / (agg[(copy, "FETCH_SIZE")] / cnt[(copy, "FETCH_SIZE")])
    w_scale = gib_kib / (agg[(copy, "WRITE_SIZE")] / cnt[(copy, "WRITE_SIZE")])
    print()
    print(f"Calibration: the copy reads and writes {gib_kib:.0f} KiB; fetched bytes = FETCH_SIZE x "
          f"{f_scale:.5f} x 1024, written bytes = WRITE_SIZE x {w_scale:.5f} x 1024.")
    print()
    print("| kernel | HBM MB / launch | avg us | GB/s | of 8000 GB/s |")
    print("|---|---:|---:|---:|---:|")
    scaled = {}
    for k in kernels:
        if k == copy or (k, "FETCH_SIZE") not in agg or (k, "WRITE_SIZE") not in agg:
            continue
        b = (agg[(k, "FETCH_SIZE")] / cnt[(k, "FETCH_SIZE")] * f_scale +
             agg[(k, "WRITE_SIZE")] / cnt[(k, "WRITE_SIZE")] * w_scale) * 1024
        scaled[k] = b
        us = trace_avg.get(k)
        rate = f"{b / us / 1e3:.0f} | {b / us / 1e3 / HBM_PEAK_GBS * 100:.1f}%" if us else " | "
        print(f"| {k} | {b / 1e6:.1f} | {us if us else '':} | {rate} |")
    print()
    print("Machine-read by bench.py (a group's figures are dropped once its sources change):")
    print()
    for k, b in scaled.items():
        if symbol_group(k):
            print(f"- hbm_bytes_per_launch.{k}: `{int(b)}`")
    for g in sorted({symbol_group(k) for k in scaled} - {None}):
        print(f"- sources_sha256.{g}: `{sources_sha256(SOURCE_GROUPS[g])}`")


class HipEvents:
    """Raw hipEvent_t handles (the probe hook records them on the library's stream)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")

    def create(self):
        ev = ctypes.c_void_p()
        assert self.hip.hipEventCreate(ctypes.byref(ev)) == 0
        return ev

    def elapsed_ms(self, a, b):
        self.hip.hipEventSynchronize(b)
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, ev):
        self.hip.hipEventDestroy(ev)


def algorithmic_work(name, w, plan):
    """(bound, work per launch, unit) -- flops for the attention kernels
    (causal half: S(S+1)/2 score pairs per head, 2d flops per pair per
    product), bytes the method must move for the others."""
    BH, N, d, S = w.B * w.H, w.N, w.d, plan.S
    e = 2 if w.dtype == "bf16" else 4
    pairs = S * (S + 1) / 2
    Mu = plan.M_total - N
    if name == "attn_fwd":          # Q K^T and P V
        return "mfma", BH * 2 * 2 * d * pairs, "flop"
    if name == "attn_dkdv":         # recompute Q K^T, dO V^T, P^T dO, dS^T Q
        return "mfma", BH * 4 * 2 * d * pairs, "flop"
    if name == "attn_dq":           # dS K (the recomputed products are not counted)
        return "mfma", BH * 1 * 2 * d * pairs, "flop"
    table = {
        "pool": 3 * N * d * e + 3 * Mu * d * e + 2 * N * 4,   # + the token norms of q and k
        "score": 2 * N * 4 + Mu * 4,
        "gather": 2 * 3 * S * d * e + S * 4,
        "scatter_fwd": S * d * 4 + N * d * e + plan.M_total * 4,
        "scatter_bwd": N * d * e + S * d * e + S * d * 4 + S * 4,
        "gather_pool_bwd": 3 * S * d * 4 + 3 * N * d * e + plan.M_total * 4,
        "topk": Mu * 4,
        "map": plan.M_total * 4 + S * 4,
    }
    # top-K and the map are one pass over a few MB each: bound by latency, not by bytes
    return ("latency" if name in ("topk", "map") else "hbm"), BH * table[name], "byte"


def attention_block(args, w, layer, o, dod, dq, dk, dv, timed):
    """The layer with its Q, K, V projections either side (d_model = H d):
    lh_qkv_forward, the layer forward and backward, lh_qkv_backward -- on the
    same GPU, inputs x ~ N(0,1) and weights ~ N(0, 1/d_model)."""
    import torch
    from long_context_pretraining_amd import inputs
    from long_context_pretraining_amd import lighthouse as lh
    Dm = w.H * w.d
    dev = torch.device("cuda:0")
    x, wt, _ = inputs.make_proj_inputs(w.B, w.N, Dm, w.H, w.d, w.seed + 2000)
    x, wt = x.to(dev), wt.to(dev)
    pdesc = lh.make_proj_desc(w.B, w.N, Dm, w.H, w.d)
    ws = torch.empty(lh.lh_qkv_plan(pdesc), dtype=torch.uint8, device=dev)
    q, k, v = (torch.empty_like(dq) for _ in range(3))
    dx = torch.empty_like(x)
    dw = torch.empty(wt.shape, dtype=torch.float32, device=dev)

    def fwd():
        lh.lh_qkv_forward(pdesc, x, wt, q, k, v)

    def bwd():
        lh.lh_qkv_backward(pdesc, x, wt, dq, dk, dv, dx, dw, ws)

    def whole():
        fwd()
        layer.forward(q, k, v, o)
        layer.backward(dod, dq, dk, dv)
        bwd()

    n = max(args.steps, 3)
    f_ms, b_ms, t_ms = timed(fwd, n), timed(bwd, n), timed(whole, n)
    flop = 2.0 * w.B * w.N * Dm * 3 * w.H * w.d          # one of the three products
    del ws
    return {"d_model": Dm, "ms_per_step": round(t_ms, 4),
            "tokens_per_s": round(w.B * w.N / (t_ms * 1e-3), 1),
            "qkv_fwd_ms": round(f_ms, 4), "qkv_bwd_ms": round(b_ms, 4),
            "qkv_fwd_tflops": round(flop / (f_ms * 1e-3) / 1e12, 1),
            "qkv_bwd_tflops": round(2 * flop / (b_ms * 1e-3) / 1e12, 1),
            "note": "projections + layer fwd+bwd + projection gradients (dx, dw); "
                    "TFLOP/s count the GEMM flops only (the backward includes its transposes)"}


def err_over_bound(got, ref, dtype):
    """Worst error of `got` against `ref` as a fraction of the parity bound:
    f32 max|a-b| / (1e-4 max|b|) over the tensor, bf16 max of
    |a-b| / (2e-2 max(1, |b|)) element-wise (<= 1 passes)."""
    import numpy as np
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if not np.all(np.isfinite(got)):
        return float("inf")
    diff = np.abs(got - ref)
    if dtype == "f32":
        return float(diff.max() / (1e-4 * max(float(np.abs(ref).max()), 1e-30)))
    return float((diff / (2e-2 * np.maximum(1.0, np.abs(ref)))).max())


CPU_SAMPLE_HEADS = 6


def oracle_head(w, q, k, v, dout, h):
    """The oracle's forward and backward of head (0, h), and its CPU time."""
    import numpy as np
    from oracle import lighthouse_oracle as orc
    qh, kh, vh, gh = (x[0, h].float().numpy().astype(np.float64) for x in (q, k, v, dout))
    t0 = time.perf_counter()
    st = orc.head_forward(qh, kh, vh, w.p, w.L, w.k, w.dtype)
    bw = orc.head_backward(st, gh)
    return st, bw, time.perf_counter() - t0


def head_parity(w, st, bw, gpu, h):
    """Selection bit for bit and o, dq, dk, dv against their bounds, head (0, h)."""
    import numpy as np
    sel = bool(np.array_equal(gpu["gidx"][0, h].numpy(), st["gidx"]))
    errs = {name: err_over_bound(gpu[name][0, h].float().numpy(), ref, w.dtype)
            for name, ref in (("o", st["O"]), ("dq", bw["dq"]), ("dk", bw["dk"]), ("dv", bw["dv"]))}
    return sel, errs


def parity_512k(head):
    """The oracle on head 0 of the 512K-token layer against the timed run's results."""
    from long_context_pretraining_amd import inputs
    w = inputs.WORKLOADS["extreme_512k"]
    st, bw, secs = oracle_head(w, head["q"], head["k"], head["v"], head["dout"], 0)
    sel, errs = head_parity(w, st, bw, head, 0)
    return {"heads": 1, "selection_bit_exact": sel, "err_over_bound": {n: round(x, 4) for n, x in errs.items()},
            "pass": sel and all(x <= 1.0 for x in errs.values()), "oracle_s": round(secs, 1)}


def cpu_baseline(w, q, k, v, dout, nheads=CPU_SAMPLE_HEADS, gpu=None):
    """The oracle as it stands on the first `nheads` heads of the workload:
    selection, pyramid, attention, scatter and the whole backward, per head;
    scaled to the layer.  With `gpu` (the timed run's gidx, o, dq, dk, dv as
    CPU tensors [B,H,...]) the same oracle results also give a parity verdict
    for those heads: selection bit for bit, tensors against their bounds."""
    import numpy as np
    from oracle import lighthouse_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        cores = 1
    heads = w.B * w.H
    nheads = min(nheads, w.H)
    dt = 0.0
    sel_exact, worst = True, {}
    for h in range(nheads):
        st, bw, secs = oracle_head(w, q, k, v, dout, h)
        dt += secs
        if gpu is not None:
            s_ok, errs = head_parity(w, st, bw, gpu, h)
            sel_exact &= s_ok
            for name, e in errs.items():
                worst[name] = max(worst.get(name, 0.0), e)
    per_head = dt / nheads
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), cpu)
    except OSError:
        pass
    return {"value": round(w.B * w.N / (per_head * heads), 1), "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle", "cpu": cpu, "host_cpus": os.cpu_count(),
            "sample": f"{nheads} of {heads} heads (b=0, h<{nheads}), full fwd+bwd incl. selection, {dt:.1f} s "
                      f"of CPU time; value = B*N / (mean time per head x {heads} heads)",
            **({"parity": {"heads": nheads, "selection_bit_exact": sel_exact,
                           "err_over_bound": {n: round(x, 4) for n, x in worst.items()},
                           "pass": sel_exact and all(x <= 1.0 for x in worst.values()),
                           "note": "the timed run's own outputs against the oracle on the sampled heads; "
                                   "bound: bf16 |a-b| <= 2e-2 max(1,|b|), f32 max|a-b| <= 1e-4 max|b|"}}
               if gpu is not None else {})}


def median(xs):
    xs = sorted(xs)
    return xs[len(xs) // 2] if xs else None


def probe_kernels(lh, ev, step, names, reps, flush=None):
    """Median HIP-event duration of each kernel in `names` over `reps` probed
    steps (the probe records on the library's stream); with `flush` (a device
    buffer of >= 512 MB) the library reads it just before every probed
    launch, so the kernel starts with its inputs out of L2 and the Infinity
    Cache (and with no dirty lines of its own to write back)."""
    import torch
    ids = {n: i for i, n in enumerate(KERNEL_NAMES)}
    if flush is not None:
        lh.lh_set_probe_flush(flush, flush.numel())
    out = {}
    a, b = ev.create(), ev.create()
    for name in names:
        ts = []
        for _ in range(reps):
            lh.lh_set_probe(ids[name], a, b)
            step()
            torch.cuda.synchronize()
            ts.append(ev.elapsed_ms(a, b))
        out[name] = median(ts)
    lh.lh_set_probe(-1, None, None)
    lh.lh_set_probe_flush(None, 0)
    ev.destroy(a)
    ev.destroy(b)
    return out


def stage_table(w, plan, kernel_ms, kernel_ms_cold, peaks):
    """Every kernel of the step: its algorithmic rate against its roof (warm,
    inside running steps, and cold, after a cache flush), against the vendor
    peak and the measured one, and, where a counter summary of the current
    sources exists, the HBM bytes it actually moves."""
    stages = {}
    for name, ms in kernel_ms.items():
        b, wk, _ = algorithmic_work(name, w, plan)
        st = {"bound": b, "ms": round(ms, 4)}
        cold = kernel_ms_cold.get(name)
        if b == "mfma":
            pk = MFMA_BF16_PEAK_TFS if w.dtype == "bf16" else MFMA_F32_PEAK_TFS
            tf = wk / (ms * 1e-3) / 1e12
            st.update(alg_tflops=round(tf, 1), alg_frac=round(tf / pk, 3))
            if w.dtype == "bf16" and peaks.get("mfma_bf16_tflops"):
                st.update(alg_frac_of_measured=round(tf / peaks["mfma_bf16_tflops"], 3))
        else:
            gbs = wk / (ms * 1e-3) / 1e9
            st.update(alg_gbs=round(gbs, 1))
            if b == "hbm":
                st.update(alg_frac=round(gbs / HBM_PEAK_GBS, 3))
                if peaks.get("hbm_gbs"):
                    st.update(alg_frac_of_measured=round(gbs / peaks["hbm_gbs"], 3))
            if cold:
                gc = wk / (cold * 1e-3) / 1e9
                st.update(ms_cold=round(cold, 4), alg_gbs_cold=round(gc, 1))
                if b == "hbm":
                    st.update(alg_frac_cold=round(gc / HBM_PEAK_GBS, 3))
        hb = stored_traffic(name, w.name)
        if hb is not None:
            st.update(hbm_gbs=round(hb / (ms * 1e-3) / 1e9, 1), hbm_frac=round(hb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 3))
        stages[name] = st
    return stages


def measured_peaks(dev):
    """Achievable peaks measured on this GPU, the second denominators: the
    library's streams over 2 GiB (16-byte accesses: copy, counting bytes read
    + written, read only, write only; the best of the three is the measured
    HBM peak) and its loop of independent bf16 matrix products (two waves per
    SIMD, 32768 flops per product), each the median of five timed runs."""
    import torch
    from long_context_pretraining_amd import lighthouse as lh
    out = {}
    src = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def run(fn, n=6):
        ts = []
        for _ in range(n):
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return median(ts[1:])

    n = 2 << 30
    out["copy_gbs"] = round(2 * n / (run(lambda: lh.lh_peak_hbm(0, dst, src, n)) * 1e-3) / 1e9, 1)
    out["read_gbs"] = round(n / (run(lambda: lh.lh_peak_hbm(1, dst, src, n)) * 1e-3) / 1e9, 1)
    out["write_gbs"] = round(n / (run(lambda: lh.lh_peak_hbm(2, dst, None, n)) * 1e-3) / 1e9, 1)
    out["hbm_gbs"] = max(out["copy_gbs"], out["read_gbs"], out["write_gbs"])
    del src, dst
    sink = torch.empty(256 * 512, dtype=torch.float32, device=dev)
    iters = 20000
    ms = run(lambda: lh.lh_peak_mfma(sink, iters))
    out["mfma_bf16_tflops"] = round(lh.PEAK_MFMA_FLOPS_PER_ITER * iters / (ms * 1e-3) / 1e12, 1)
    out["note"] = ("2 GiB streams of 16-byte accesses (copy counts read + written bytes; hbm_gbs = best "
                   "of copy, read, write); mfma: back-to-back independent v_mfma_f32_32x32x16_bf16, "
                   "two waves per SIMD")
    del sink
    torch.cuda.empty_cache()
    return out


def timed_steps(step, n):
    """Per-step durations (ms) from events on the current stream, which is the
    library's stream here."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def extreme_512k(args, ev, peaks, dev, keep_head=False):
    """The 512K-token layer (B=1, H=16, N=524288, d=64, bf16, p=4, L=6,
    k=1536): step time, forward time, every kernel warm and cold, and one dense
    causal fwd+bwd step for the speedup.  Inputs are drawn on the device with
    torch's generator (N(0,1) times one lognormal(0, 0.5) factor per token,
    rounded to bf16): the same distribution as the parity tests' host recipe,
    generated where it is used."""
    import torch
    from long_context_pretraining_amd import inputs
    from long_context_pretraining_amd import lighthouse as lh
    w = inputs.WORKLOADS["extreme_512k"]
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed)
    shape = (w.B, w.H, w.N, w.d)
    m = torch.exp(0.5 * torch.randn((w.B, w.H, w.N, 1), device=dev, generator=g))
    q, k, v = ((torch.randn(shape, device=dev, generator=g) * m).to(torch.bfloat16) for _ in range(3))
    del m
    dout = torch.randn(shape, device=dev, generator=g).to(torch.bfloat16)
    layer = lh.LighthouseLayer(w.B, w.H, w.N, w.d, w.p, w.L, w.k, torch.bfloat16)
    plan = layer.plan
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))

    def step():
        layer.forward(q, k, v, o)
        layer.backward(dout, dq, dk, dv)

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    ts = timed_steps(step, args.extreme_steps)
    fwd = timed_steps(lambda: layer.forward(q, k, v, o), args.extreme_steps)
    # head 0's inputs and the timed run's results for it, for the oracle leg's parity verdict
    head = None
    if keep_head:
        head = {n: t[:1, :1].cpu() for n, t in (("q", q), ("k", k), ("v", v), ("dout", dout), ("o", o),
                                                ("dq", dq), ("dk", dk), ("dv", dv))}
        head["gidx"] = layer.gidx[:1, :1].cpu()
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    kms = probe_kernels(lh, ev, step, KERNEL_NAMES, 3)
    kms_cold = probe_kernels(lh, ev, step, [n for n in KERNEL_NAMES if not n.startswith("attn")], 3, flush)
    del flush
    stages = stage_table(w, plan, kms, kms_cold, peaks)
    ms = median(ts)
    out = {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "p": w.p, "L": w.L, "k": w.k,
           "S": plan.S, "S_formula": plan.S_formula, "ms_per_step_median": round(ms, 4),
           "ms_per_step_min": round(min(ts), 4), "tokens_per_s": round(w.B * w.N / (ms * 1e-3), 1),
           "fwd_ms_median": round(median(fwd), 4), "steps": args.extreme_steps, "stages": stages,
           "data": "synthetic, generated on the device (torch generator, seed 5)"}
    if args.extreme_dense:
        ddesc = lh.make_desc(w.B, w.H, w.N, w.d, w.p, 1, 1, torch.bfloat16)
        dplan = lh.lh_make_plan(ddesc)
        dws = torch.empty(dplan.dense_fwd_ws_bytes, dtype=torch.uint8, device=dev)
        dwsb = torch.empty(dplan.dense_bwd_ws_bytes, dtype=torch.uint8, device=dev)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        dense_f = lambda: lh.dense_causal_attn(ddesc, q, k, v, o, lse, dws)
        dense_fb = lambda: (dense_f(), lh.dense_causal_attn_backward(ddesc, q, k, v, lse, dws, dout, dq, dk, dv, dwsb))
        dense_f()
        torch.cuda.synchronize()
        d_fb = median(timed_steps(dense_fb, 1))
        d_f = median(timed_steps(dense_f, 1))
        out.update(dense_ms_per_step=round(d_fb, 2), dense_fwd_ms=round(d_f, 2),
                   speedup_vs_dense=round(d_fb / ms, 2), speedup_fwd_vs_dense=round(d_f / median(fwd), 2))
        del dws, dwsb, lse
    del layer, q, k, v, dout, o, dq, dk, dv
    torch.cuda.empty_cache()
    return out, head


def cpu_scaling(threads_all):
    """One head of the two small workloads through the oracle with all threads
    and with one (threadpoolctl limits the BLAS pool)."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from long_context_pretraining_amd import inputs
    from oracle import lighthouse_oracle as orc
    out = {}
    for name in ("tiny_f32", "mid_bf16"):
        w = inputs.WORKLOADS[name]
        q, k, v = inputs.make_qkv(w)
        dout = inputs.make_dout(w)
        f = lambda t: t[0, 0].float().numpy().astype(np.float64)
        r = {}
        for label, nt in (("all_threads", None), ("one_thread", 1)):
            t0 = time.perf_counter()
            with threadpool_limits(nt):
                st = orc.head_forward(f(q), f(k), f(v), w.p, w.L, w.k, w.dtype)
                orc.head_backward(st, f(dout))
            r[label + "_s"] = round(time.perf_counter() - t0, 3)
        r["threads_all"] = threads_all
        out[name + " (one head, fwd+bwd)"] = r
    return out


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: the layer is measured per GPU and the library has no "
              "multi-GPU path (heads would shard across GPUs with no communication).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from long_context_pretraining_amd import inputs
    from long_context_pretraining_amd import lighthouse as lh

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    lh.load_library()
    w = inputs.WORKLOADS[args.workload]
    dt = inputs.TORCH_DTYPE[w.dtype]
    q, k, v = inputs.make_qkv(w)
    dout = inputs.make_dout(w)
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (x.to(dev) for x in (q, k, v, dout))
    layer = lh.LighthouseLayer(w.B, w.H, w.N, w.d, w.p, w.L, w.k, dt)
    plan = layer.plan
    o, dq, dk, dv = (torch.empty_like(qd) for _ in range(4))

    def step():
        layer.forward(qd, kd, vd, o)
        layer.backward(dod, dq, dk, dv)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # every kernel's duration: median of a few probed steps, warm (inside running steps) and, for the
    # bandwidth-bound ones, cold (the library reads a 1 GiB buffer just before the probed launch)
    ev = HipEvents()
    kernel_ms = probe_kernels(lh, ev, step, KERNEL_NAMES, args.probe_reps)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    kernel_ms_cold = probe_kernels(lh, ev, step, [n for n in KERNEL_NAMES if not n.startswith("attn")],
                                   args.probe_reps, flush)
    del flush
    dominant = max(kernel_ms, key=kernel_ms.get)
    dom_id = KERNEL_NAMES.index(dominant)

    # timed region: exactly K steps, the dominant kernel probed in every step, and each step
    # bracketed by events on the library's stream
    starts = [ev.create() for _ in range(args.steps)]
    stops = [ev.create() for _ in range(args.steps)]
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        lh.lh_set_probe(dom_id, starts[i], stops[i])
        step_ev[i][0].record()
        step()
        step_ev[i][1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    lh.lh_set_probe(-1, None, None)
    elapsed = t1 - t0
    ms_step = elapsed * 1e3 / args.steps
    dom_ms = sum(ev.elapsed_ms(s, e) for s, e in zip(starts, stops)) / args.steps
    step_ms = [a.elapsed_time(b) for a, b in step_ev]
    tokens_per_s = w.B * w.N * args.steps / elapsed
    # the timed run's outputs of the heads the oracle samples, for its parity verdict (later
    # measurements overwrite o, dq, dk, dv)
    sampled = None
    if not args.no_cpu_baseline:
        nh = min(CPU_SAMPLE_HEADS, w.H)
        sampled = {"gidx": layer.gidx[:1, :nh].cpu()}
        sampled.update({n: t[:1, :nh].cpu() for n, t in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv))})

    peaks = measured_peaks(dev)
    bound, work, unit = algorithmic_work(dominant, w, plan)
    if bound == "mfma":
        peak = MFMA_BF16_PEAK_TFS if w.dtype == "bf16" else MFMA_F32_PEAK_TFS
        achieved = work / (dom_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": stored_traffic(dominant, w.name), "kernel": dominant,
                "kernel_ms": round(dom_ms, 4), "work_per_launch": work}
        if w.dtype == "bf16":
            roof.update(peak_measured=peaks["mfma_bf16_tflops"],
                        frac_of_measured=round(achieved / peaks["mfma_bf16_tflops"], 4))
    else:
        achieved = work / (dom_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": stored_traffic(dominant, w.name), "kernel": dominant,
                "kernel_ms": round(dom_ms, 4), "work_per_launch": work,
                "peak_measured": peaks["hbm_gbs"], "frac_of_measured": round(achieved / peaks["hbm_gbs"], 4)}
    stages = stage_table(w, plan, kernel_ms, kernel_ms_cold, peaks)

    # dense causal attention baseline on the same GPU and inputs
    ddesc = lh.make_desc(w.B, w.H, w.N, w.d, w.p, 1, 1, dt)
    dplan = lh.lh_make_plan(ddesc)
    dws = torch.empty(dplan.dense_fwd_ws_bytes, dtype=torch.uint8, device=dev)
    dwsb = torch.empty(dplan.dense_bwd_ws_bytes, dtype=torch.uint8, device=dev)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

    def dense_step():
        lh.dense_causal_attn(ddesc, qd, kd, vd, o, lse, dws)
        lh.dense_causal_attn_backward(ddesc, qd, kd, vd, lse, dws, dod, dq, dk, dv, dwsb)

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / n

    dense_ms = dense_fwd_ms = None
    if args.dense_steps > 0:
        dense_ms = timed(dense_step, args.dense_steps)
        dense_fwd_ms = timed(lambda: lh.dense_causal_attn(ddesc, qd, kd, vd, o, lse, dws), args.dense_steps)
    del dws, dwsb
    # forward only (selection included), after the timed region
    fwd_ms = timed(lambda: layer.forward(qd, kd, vd, o), args.steps)
    block = attention_block(args, w, layer, o, dod, dq, dk, dv, timed) if w.dtype == "bf16" else None

    if args.calibration_copy:   # a plain copy kernel of known size: reads and writes 1 GiB
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    headline = args.workload == "llama530m_98k_k1536"
    out = {
        "metric": ("Lighthouse fwd+bwd tokens/s at N=98K,k=1536; speedup vs dense causal attn" if headline
                   else f"Lighthouse fwd+bwd tokens/s, workload {w.name}; speedup vs dense causal attn"),
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_median": round(median(step_ms), 4),
        "ms_per_step_min": round(min(step_ms), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "p": w.p, "L": w.L, "k": w.k,
                   "S": plan.S, "S_formula": plan.S_formula},
        "speedup_vs_dense": round(dense_ms / ms_step, 3) if dense_ms else None,
        "dense_ms_per_step": round(dense_ms, 3) if dense_ms else None,
        "dense_steps": args.dense_steps,
        "dense_tokens_per_s": round(w.B * w.N / (dense_ms * 1e-3), 1) if dense_ms else None,
        "fwd_ms": round(fwd_ms, 4),
        "dense_fwd_ms": round(dense_fwd_ms, 3) if dense_fwd_ms else None,
        "speedup_fwd_vs_dense": round(dense_fwd_ms / fwd_ms, 3) if dense_fwd_ms else None,
        "kernel_ms": {n: round(x, 4) for n, x in kernel_ms.items()},
        "kernel_ms_note": f"median of {args.probe_reps} probed steps per kernel (HIP events on the library's stream)",
        "roofline": roof,
        "measured_peaks": peaks,
        "stages": stages,
        "attention_block": block,
    }
    head_512k = None
    if headline and not args.no_extreme:
        del layer, qd, kd, vd, dod, o, dq, dk, dv, lse
        torch.cuda.empty_cache()
        out["extreme_512k"], head_512k = extreme_512k(args, ev, peaks, dev, keep_head=not args.no_cpu_baseline)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, q, k, v, dout, CPU_SAMPLE_HEADS, gpu=sampled)
        if head_512k is not None:
            out["cpu_baseline"]["parity_512k"] = parity_512k(head_512k)
        out["cpu_baseline"]["scaling"] = cpu_scaling(out["cpu_baseline"]["cores"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
