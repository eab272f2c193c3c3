#!/usr/bin/env python3
"""Benchmark of the routed-expert layer on one MI355X.

One step is one pass of the layer over one synthetic batch that is already
resident in HBM:

* recv_share_bf16 (the default: the largest workload one GPU holds, one
  GPU's receiver share of the 8-of-384 design): three waves of receiver
  compaction -> grouped SwiGLU over the static per-expert arrays ->
  expansion to pool rows (fp32);
* layer workloads (mid_bf16, tiny_fp32, decode_bf16):
  route -> permute -> grouped SwiGLU -> un-permute/combine;
* sender_pack_bf16: route -> pooled-wave pack of all three waves.

Inputs rotate over ``--banks`` independent copies (distinct HBM addresses) so
that no step finds the previous step's operands in the 256 MB last-level
cache.  Every call is timed with HIP events on the stream it runs on; the
JSON line reports whole-step throughput (mean, and the nearest-rank median
and 95th percentile of the per-step times), the roofline of the dominant
call (algorithmic bytes or flops per launch over its measured duration, with
the HBM traffic and MFMA busy fraction that rocprofv3 counters recorded for
the same kernel sources) and the CPU oracle timed on a bounded sample of the
same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "routed tokens/s per MoE layer on 1 MI355X; HBM GB/s & MFMA % of peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
F32_PEAK_TFLOPS = 157.3        # fp32 vector
COPY_CALIB_BYTES = 256 << 20   # size of the calibration copy (read and written once)
LEAD_CYCLES = 400_000          # spin queued before each per-call timing (about 0.2 ms; touches no memory)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_busy.json")
CSRC_DIR = os.path.join(ROOT, "grouped_expert_amd", "csrc")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="recv_share_bf16", choices=sorted(W.WORKLOADS))
    ap.add_argument("--banks", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=0,
                    help="CPU oracle sample: tokens (layer, pack, router workloads) or waves (receiver workloads); "
                         "0 = the default")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no benchmark: read the counter CSVs of two rocprofv3 --pmc runs of this script "
                         "(FETCH_SIZE, then WRITE_SIZE) for --workload and record HBM bytes per call in "
                         "profiles/hbm_traffic.json")
    ap.add_argument("--record-mfma", metavar="PMC_DIR",
                    help="no benchmark: read the counter CSV of a rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES "
                         "GRBM_GUI_ACTIVE run of this script for --workload and record the MFMA busy fraction "
                         "of each GEMM call in profiles/mfma_busy.json")
    ap.add_argument("--pmc-command", default="", help="with --record-traffic / --record-mfma: the profiling "
                                                      "command, stored beside the figures")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# HBM traffic from hardware counters
# ---------------------------------------------------------------------------

# kernel sources of each call (plus the shared header and the C ABI)
_CALL_SOURCES = {"route": ["route_topk.hip"], "permute": ["permute.hip", "bucket_rank.h", "fp8.h"],
                 "swiglu": ["swiglu_gemm.hip", "gemm_core.h"], "combine": ["combine.hip"],
                 "expand": ["combine.hip"], "pool_pack": ["pool_pack.hip", "bucket_rank.h", "fp8.h"],
                 "recv_compact": ["recv_compact.hip", "bucket_rank.h", "fp8.h"], "combine_bwd": ["combine.hip"],
                 "quantize": ["fp8.hip", "fp8.h"],
                 "swiglu_bwd": ["swiglu_backward.hip", "gemm_core.h"], "dx_combine": ["combine.hip"]}


def sources_digest(call):
    """sha256 over the kernel sources of one call; recorded traffic is used
    only while the sources it was measured on are unchanged."""
    import hashlib
    h = hashlib.sha256()
    paths = [os.path.join(CSRC_DIR, n) for n in _CALL_SOURCES[call] + ["common.h"]]
    paths.append(os.path.join(ROOT, "include", "moe.h"))
    for path in paths:
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _cfg_args(kernel):
    """Template arguments of a GEMM kernel's tile configuration (Cfg<...>)."""
    m = re.search(r"Cfg<([^<>]*)>", kernel)
    return m.group(1).split(", ") if m else []


def _is_bwd_gemm(kernel):
    """Expert-backward GEMMs carry the SwiGLU-backward epilogue (tile argument
    14, EPI) or K-major B tiles (argument 15, BT)."""
    a = _cfg_args(kernel)
    return (len(a) > 13 and a[13] != "0") or (len(a) > 14 and a[14] == "true")


def _call_of(kernel, train=False):
    """The library call a dispatched kernel belongs to (None: not ours).
    Bucket-rank and tile-table kernels serve several calls and are given to
    the call of the next dispatch, by the caller of this function ("rank").
    In a training step the fp32 combine is the token-gradient pass."""
    if "grouped_gemm_" in kernel:
        return "swiglu_bwd" if _is_bwd_gemm(kernel) else "swiglu"
    table = (("route_list_kernel", "route"), ("route_topk_kernel", "route"), ("route_grouped_kernel", "route"),
             ("route_grouped16_kernel", "route"),
             ("build_tiles_kernel", "rank"),
             ("grouped_wgrad_kernel", "swiglu_bwd"), ("swiglu_bwd_rows_kernel", "swiglu_bwd"),
             ("scatter_rows_kernel", "permute"), ("permute_fused_kernel", "permute"), ("pack_kernel", "pool_pack"),
             ("compact_rows_kernel", "recv_compact"), ("compact_fp8_rows_kernel", "recv_compact"),
             ("quantize_kernel", "quantize"), ("expand_rows_kernel", "expand"),
             ("combine_backward_kernel", "combine_bwd"), ("rank_", "rank"))
    for pat, call in table:
        if pat in kernel:
            return call
    if "combine_kernel" in kernel:
        return "dx_combine" if train and "combine_kernel<float>" in kernel else "combine"
    return None


# one dispatch per call instance: counts the launches of each call
_ANCHORS = {"route": lambda n: "route_" in n,
            "swiglu": lambda n: "grouped_gemm_" in n,
            "permute": lambda n: "scatter_rows_kernel" in n or "permute_fused_kernel" in n,
            "combine": lambda n: "combine_kernel" in n,
            "expand": lambda n: "expand_rows_kernel" in n,
            "pool_pack": lambda n: "pack_kernel" in n,
            "recv_compact": lambda n: "compact_" in n,
            "quantize": lambda n: "quantize_kernel" in n,
            "combine_bwd": lambda n: "combine_backward_kernel" in n,
            # dG | dU come from the gate/up GEMM's SwiGLU-backward epilogue, or
            # from the saved activations in a row pass: one of the two per call
            "swiglu_bwd": lambda n: ("grouped_gemm_" in n and len(_cfg_args(n)) > 13 and _cfg_args(n)[13] == "1")
            or "swiglu_bwd_rows_kernel" in n,
            "dx_combine": lambda n: "combine_kernel" in n}
# calls whose anchor kernel is dispatched more than once per call
_ANCHOR_PER_CALL = {"swiglu": 2}


def record_traffic(args):
    import csv
    w = W.WORKLOADS[args.workload]
    per = {}
    for counter, d in (("FETCH_SIZE", args.record_traffic[0]), ("WRITE_SIZE", args.record_traffic[1])):
        rows = [r for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv")))
                if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        names = [r["Kernel_Name"] for r in rows]
        # the step's first call (library kernels of the untimed set-up come earlier)
        lead = "recv_compact" if workload_kind(w) == "recv" else "route"
        first_ours = next(i for i, n in enumerate(names) if _call_of(n) == lead)
        # the calibration copy is the last plain device copy before the first library kernel
        calib = max(i for i in range(first_ours) if "copyBuffer" in names[i])
        factor = COPY_CALIB_BYTES / (float(rows[calib]["Counter_Value"]) * 1024.0)
        calls = [_call_of(n, train=w.train) for n in names]
        nxt = None
        for i in range(len(calls) - 1, first_ours - 1, -1):    # rank kernels -> call of the next dispatch
            if calls[i] == "rank":
                calls[i] = nxt
            elif calls[i]:
                nxt = calls[i]
        kib, launches = {}, {}
        for i in range(first_ours, len(rows)):
            c = calls[i]
            if not c:
                continue
            kib[c] = kib.get(c, 0.0) + float(rows[i]["Counter_Value"])
            if _ANCHORS[c](names[i]):
                launches[c] = launches.get(c, 0) + 1
        launches = {c: v // _ANCHOR_PER_CALL.get(c, 1) for c, v in launches.items()}
        per[counter] = dict(factor=factor, bytes={c: kib[c] * 1024.0 * factor / launches[c] for c in kib},
                            launches=launches)
    entry = dict(command=args.pmc_command,
                 calibration=dict(copy_bytes=COPY_CALIB_BYTES, fetch_factor=round(per["FETCH_SIZE"]["factor"], 4),
                                  write_factor=round(per["WRITE_SIZE"]["factor"], 4)),
                 calls={c: dict(sources_sha256=sources_digest(c), read_bytes=int(per["FETCH_SIZE"]["bytes"][c]),
                                write_bytes=int(per["WRITE_SIZE"]["bytes"].get(c, 0.0)),
                                launches=per["FETCH_SIZE"]["launches"][c])
                        for c in sorted(per["FETCH_SIZE"]["bytes"])})
    data = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    data[w.name] = entry
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps({w.name: entry}, indent=1))


def record_mfma(args):
    """MFMA busy fraction of the GEMM calls of one workload from a rocprofv3
    --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE run of this script.

    SQ_VALU_MFMA_BUSY_CYCLES is summed over every CU and counts each of a
    CU's four SIMDs; GRBM_GUI_ACTIVE is summed over the XCDs.  Busy fraction
    of a dispatch = MFMA_BUSY / (GRBM_GUI_ACTIVE / XCDs * CUs * 4), i.e. the
    share of SIMD cycles the matrix cores were busy, at the clock the GPU ran
    (not the 2.4 GHz the published peak assumes).  Per call: cycle-weighted
    over its dispatches after the first library call (the untimed set-up is
    excluded)."""
    import csv
    w = W.WORKLOADS[args.workload]
    d = args.record_mfma
    agent = [r for r in csv.DictReader(open(os.path.join(d, "run_agent_info.csv"))) if r["Agent_Type"] == "GPU"][0]
    cus, xcds, simds = int(agent["Cu_Count"]), int(agent["Num_Xcc"]), int(agent["Simd_Per_Cu"])
    rows = list(csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))))
    by_disp = {}
    for r in rows:
        e = by_disp.setdefault(int(r["Dispatch_Id"]), dict(name=r["Kernel_Name"]))
        e[r["Counter_Name"]] = float(r["Counter_Value"])
        e["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    order = sorted(by_disp)
    lead = "recv_compact" if workload_kind(w) == "recv" else "route"
    first = next(i for i in order if _call_of(by_disp[i]["name"]) == lead)
    acc = {}
    for i in order:
        if i < first:
            continue
        e = by_disp[i]
        c = _call_of(e["name"], train=w.train)
        if c not in ("swiglu", "swiglu_bwd") or "grouped_gemm_" not in e["name"]:
            continue
        m = re.search(r"Cfg<([^<>]*)>", e["name"])
        kind = "gate_up" if m and m.group(1).split(", ")[5] == "true" else "down_or_other"
        for key in (c, f"{c}:{kind}"):
            a = acc.setdefault(key, dict(busy=0.0, avail=0.0, n=0, ns=0))
            a["busy"] += e["SQ_VALU_MFMA_BUSY_CYCLES"]
            a["avail"] += e["GRBM_GUI_ACTIVE"] / xcds * cus * simds
            a["n"] += 1
            a["ns"] += e["ns"]
    entry = dict(command=args.pmc_command, formula="SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / XCDs * CUs * 4)",
                 cus=cus, xcds=xcds,
                 calls={k: dict(sources_sha256=sources_digest(k.split(":")[0]), mfma_busy=round(a["busy"] / a["avail"], 4),
                                dispatches=a["n"], mean_dispatch_ms=round(a["ns"] / a["n"] / 1e6, 4))
                        for k, a in sorted(acc.items())})
    data = {}
    if os.path.exists(MFMA_FILE):
        with open(MFMA_FILE) as f:
            data = json.load(f)
    data[w.name] = entry
    with open(MFMA_FILE, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps({w.name: entry}, indent=1))


def recorded_mfma(w, call):
    """MFMA busy fraction recorded for ``call`` of this workload, or None when
    nothing is recorded or the kernel sources changed since."""
    try:
        with open(MFMA_FILE) as f:
            c = json.load(f)[w.name]["calls"].get(call)
    except (OSError, KeyError, ValueError):
        return None
    if not c or c.get("sources_sha256") != sources_digest(call):
        return None
    return c["mfma_busy"]


def recorded_traffic(w, call):
    """HBM bytes per launch of ``call`` recorded for this workload, or None
    when nothing is recorded or the kernel sources changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            entry = json.load(f)[w.name]
    except (OSError, KeyError, ValueError):
        return None
    c = entry.get("calls", {}).get(call)
    if not c or c.get("sources_sha256") != sources_digest(call):
        return None
    return c["read_bytes"] + c["write_bytes"]


def workload_kind(w):
    if w.train:
        return "train"
    if w.name.startswith("router"):
        return "router"
    return "recv" if w.name.startswith("recv") else "pack" if w.name.startswith("sender") else "layer"


# ---------------------------------------------------------------------------
# timing helpers
# ---------------------------------------------------------------------------

class OpTimer:
    """Per-call HIP event pairs recorded on the current stream, around every
    call or only around the calls named in ``only``.  Each timing event costs
    the stream a few microseconds, so the timed steps bracket only the call
    whose launch duration the roofline needs.  With ``lead`` (a callable that
    queues device work touching no memory) that work goes before each start
    event: the GPU is busy while the host prepares the call, so the event pair
    measures the call's device time and not host work between its kernels."""

    def __init__(self, torch, only=None, lead=None):
        self.torch = torch
        self.only = only
        self.lead = lead
        self.marks = []          # (name, start_event, end_event)

    def run(self, name, fn, *a, **kw):
        if self.only is not None and name not in self.only:
            return fn(*a, **kw)
        t = self.torch
        s, e = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        if self.lead is not None:
            self.lead()
        s.record()
        out = fn(*a, **kw)
        e.record()
        self.marks.append((name, s, e))
        return out

    def totals_ms(self):
        agg = {}
        for name, s, e in self.marks:
            agg.setdefault(name, []).append(s.elapsed_time(e))
        return agg


def to_dev(torch, a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def cpu_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
        return int(max(n)) if n else 1
    except Exception:
        return os.cpu_count() or 1


def cpu_host_info():
    """CPU model, host CPU count and the BLAS library numpy runs on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if libs:
            p = libs[0]
            blas = f"{p.get('internal_api')} {p.get('version')} ({os.path.basename(p.get('filepath', ''))}, " \
                   f"{p.get('threading_layer', 'n/a')} threading, {p.get('num_threads')} threads)"
    except Exception:
        pass
    return dict(cpu_model=model, host_cpus=os.cpu_count(), blas=blas)


def input_sha256(host):
    """SHA-256 over the host input arrays (sorted by name, lists in order):
    the bytes both the GPU (after one copy) and the oracle consume."""
    import hashlib
    h = hashlib.sha256()
    for k in sorted(host):
        for a in (host[k] if isinstance(host[k], list) else [host[k]]):
            a = np.ascontiguousarray(a)
            h.update(k.encode())
            h.update(str(a.dtype).encode() + str(a.shape).encode())
            h.update(memoryview(a.reshape(-1).view(np.uint8)))
    return h.hexdigest()


def nearest_rank(vals, q):
    """Nearest-rank percentile q (0 < q <= 100) of a list."""
    v = sorted(vals)
    i = max(1, int(np.ceil(q / 100.0 * len(v))))
    return v[i - 1]


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

def layer_setup(torch, w, banks):
    logits = W.router_logits(w)
    x = W.tokens(w)
    wg, wu, wd = W.all_expert_weights(w)
    host = dict(logits=logits, x=x, wg=wg, wu=wu, wd=wd)
    b0 = {k: to_dev(torch, v) for k, v in host.items()}
    bank_list = [b0] + [{k: v.clone() for k, v in b0.items()} for _ in range(banks - 1)]
    return host, bank_list


def layer_step(ge, timer, w, bank, flags, save_act=False):
    import torch
    T = w.T
    ids, gates = timer.run("route", ge.route_topk, bank["logits"], w.k, flags=flags)
    plan = timer.run("permute", ge.permute, bank["x"], ids, w.E, w.capacity, flags=flags)
    zdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    act = ge.new_act(T * w.k, w.d_ff, bank["x"].device) if save_act else None
    z = timer.run("swiglu", ge.grouped_swiglu, plan["x_perm"], plan["offsets"], plan["counts"], bank["wg"],
                  bank["wu"], bank["wd"], z_dtype=zdt, flags=flags, act=act)
    y = timer.run("combine", ge.unpermute_combine, z, plan["inv"], gates, T, w.k, flags=flags)
    return dict(y=y, ids=ids, gates=gates, plan=plan, z=z, act=act)


def layer_ledger(w, counts):
    """Algorithmic bytes / flops per call (unique inputs + outputs + index
    metadata; the H round trip is excluded)."""
    b = 4 if w.dtype == "f32" else 2
    bz = b
    A = int(counts.sum())
    E_act = int((counts > 0).sum())
    T, k, d, dff, E = w.T, w.k, w.d, w.d_ff, w.E
    return {
        "route": dict(bytes=4 * T * E + 8 * T * k, flops=0),
        "permute": dict(bytes=4 * T * k + T * d * b + A * d * b + 8 * T * k + 4 * (2 * E + 1), flops=0),
        "swiglu": dict(bytes=A * d * b + E_act * 3 * d * dff * b + A * d * bz, flops=6 * A * d * dff),
        "combine": dict(bytes=A * d * bz + 8 * T * k + 4 * T * d, flops=2 * A * d),
    }


def layer_cpu_baseline(w, host, sample):
    """The oracle layer (route, plan, expert-major SwiGLU, combine) on the first
    ``sample`` tokens of the batch."""
    import oracle as O
    s = min(sample, w.T)
    t0 = time.perf_counter()
    ids, gates, _ = O.route_topk(host["logits"][:s], w.k)
    bank = O.swiglu_bank(lambda e: (host["wg"][e], host["wu"][e], host["wd"][e]))
    O.moe_layer_expert_major(host["x"][:s], ids, gates, bank, w.E, w.capacity)
    dt = time.perf_counter() - t0
    return dict(value=s / dt, unit="tokens/s", cores=cpu_threads(), kind="oracle",
                sample=f"first {s} of {w.T} tokens of {w.name}, full layer (route, dispatch plan, "
                       f"fp64 SwiGLU of every routed row, combine); {dt:.2f} s")


def train_setup(torch, w, banks):
    host, bank_list = layer_setup(torch, w, banks)
    host["dy"] = W.upstream_grad(w)
    bank_list[0]["dy"] = to_dev(torch, host["dy"])
    for b in bank_list[1:]:
        b["dy"] = bank_list[0]["dy"].clone()
    return host, bank_list


def train_step(ge, timer, w, bank, flags):
    """Forward of the layer saving the experts' activations, then its
    backward: route and gate gradients, the expert backward (route-input and
    weight gradients, from the saved activations), and the token gradients
    through the inverse map."""
    out = layer_step(ge, timer, w, bank, flags, save_act=True)
    plan, T, k = out["plan"], w.T, w.k
    dz, dg = timer.run("combine_bwd", ge.combine_backward, bank["dy"], out["z"], plan["inv"], out["gates"], k,
                       flags=flags)
    bw = timer.run("swiglu_bwd", ge.grouped_swiglu_backward, plan["x_perm"], dz, plan["offsets"], plan["counts"],
                   bank["wg"], bank["wu"], bank["wd"], flags=flags, act=out["act"])
    dx = timer.run("dx_combine", ge.unpermute_combine, bw["dx"], plan["inv"], None, T, k, flags=flags)
    out.update(dx=dx, dgates=dg, grads=bw)
    return out


def train_ledger(w, counts):
    """The forward ledger plus the backward calls.  The forward also writes
    the saved activations (G | U and H, bf16: 3 A d_ff values).  The expert
    backward does 12 A d d_ff flops (dH, dX, dW_d, dW_g and dW_u; G, U and H
    are read, not recomputed) and moves x and dZ rows and the saved
    activations in, dX rows out (fp32), the active experts' weights in and
    every expert's fp32 weight gradients out."""
    led = layer_ledger(w, counts)
    A = int(counts.sum())
    E_act = int((counts > 0).sum())
    T, k, d, dff, E = w.T, w.k, w.d, w.d_ff, w.E
    led["swiglu"]["bytes"] += A * 3 * dff * 2
    led["combine_bwd"] = dict(bytes=4 * T * d + A * d * 2 + A * d * 2 + 12 * T * k, flops=2 * A * d)
    led["swiglu_bwd"] = dict(bytes=2 * A * d * 2 + A * 3 * dff * 2 + E_act * 3 * d * dff * 2 + A * d * 4 +
                                   E * 3 * d * dff * 4,
                             flops=12 * A * d * dff)
    led["dx_combine"] = dict(bytes=A * d * 4 + 4 * T * k + 4 * T * d, flops=A * d)
    return led


def train_cpu_baseline(w, host, sample):
    """The oracle layer forward and backward on the first ``sample`` tokens."""
    import oracle as O
    s = min(sample, w.T)
    t0 = time.perf_counter()
    ids, gates, _ = O.route_topk(host["logits"][:s], w.k)
    wts = lambda e: (host["wg"][e], host["wu"][e], host["wd"][e])
    O.moe_layer_backward(host["x"][:s], ids, gates.astype(np.float64), O.swiglu_bank(wts), O.swiglu_bank_backward(wts),
                         w.E, host["dy"][:s].astype(np.float64), w.capacity)
    dt = time.perf_counter() - t0
    return dict(value=s / dt, unit="tokens/s", cores=cpu_threads(), kind="oracle",
                sample=f"first {s} of {w.T} tokens of {w.name}: route, fp64 forward and backward of the layer "
                       f"(route, gate, token and weight gradients); {dt:.2f} s")


def fp8_pools(torch, ge, w, wave, pools16):
    """The wave's incoming pools as fp8 records (untimed set-up): the bf16
    data rows quantized by the library, the same local ids in the record
    pools' header rows (16-bit little-endian, 0xFFFF past the last row)."""
    S, P, d = w.n_src, w.pool_rows, w.d
    H16 = W.recv_header_rows(w)
    rows = pools16[:, H16:, :].reshape(S * P, d).contiguous()
    rec = ge.quantize_fp8(rows, w.payload)
    Wb = rec.shape[1]
    H8 = ge.header_rows(P, d, w.payload)
    out = torch.empty((S, H8 + P, Wb), dtype=torch.uint8, device=rows.device)
    hdr = out[:, :H8, :].reshape(S, H8 * Wb).view(torch.int16)
    hdr.fill_(-1)
    hdr[:, :P] = to_dev(torch, W.recv_local_ids(w, wave).view(np.int16))
    out[:, H8:, :] = rec.view(S, P, Wb)
    return out


def recv_setup(torch, w, banks):
    pools = [W.recv_pools(w, wave) for wave in range(w.n_waves)]
    wg, wu, wd = W.all_expert_weights(w, n_experts=w.n_local)
    host = dict(pools=pools, wg=wg, wu=wu, wd=wd)
    dev_pools = [to_dev(torch, p) for p in pools]
    if w.payload is not None:
        import grouped_expert_amd as ge
        dev_pools = [fp8_pools(torch, ge, w, wave, p) for wave, p in enumerate(dev_pools)]
        torch.cuda.synchronize()
    b0 = dict(pools=dev_pools, wg=to_dev(torch, wg), wu=to_dev(torch, wu), wd=to_dev(torch, wd))
    bank_list = [b0]
    for _ in range(banks - 1):
        bank_list.append(dict(pools=[p.clone() for p in b0["pools"]], wg=b0["wg"].clone(), wu=b0["wu"].clone(),
                              wd=b0["wd"].clone()))
    return host, bank_list


def recv_step(ge, timer, w, bank, flags, bufs):
    import torch
    S, P1, L, cap, d = w.n_src, ge.pool_height(w.pool_rows, w.d, w.payload), w.n_local, w.recv_cap, w.d
    starts = bufs["starts"]
    outs = []
    for wave in range(w.n_waves):
        ret = bufs["ret"][wave]
        # compaction also records each slot's pool row and zeroes the return
        # rows without a slot; the GEMM then stores straight into pool rows
        rc = timer.run("recv_compact", ge.recv_compact, bank["pools"][wave], L, cap, compact=bufs["compact"],
                       flags=flags, payload=w.payload, d=d, slot_row=bufs["slot_row"], ret=ret)
        timer.run("swiglu", ge.grouped_swiglu, bufs["compact"].view(L * cap, d), starts, rc["counts"],
                  bank["wg"], bank["wu"], bank["wd"], z=ret, z_rows=rc["slot_row"], flags=flags)
        outs.append((rc, ret))
    return outs


def recv_ledger(w, counts_per_wave):
    import grouped_expert_amd as ge
    S, P, d, dff = w.n_src, w.pool_rows, w.d, w.d_ff
    P1 = ge.pool_height(P, d, w.payload)
    rb = ge.row_bytes(d, w.payload)             # bytes of one incoming row (bf16 or fp8 record)
    zb = 2 if w.ret_dtype == "bf16" else 4      # bytes per expert-output / return element
    led = {"recv_compact": dict(bytes=0, flops=0), "swiglu": dict(bytes=0, flops=0)}
    for counts in counts_per_wave:
        A = int(counts.sum())
        E_act = int((counts > 0).sum())
        # header ids, accepted rows read and written as bf16 (receiver-dropped rows are never read), row_slot,
        # slot_row, and the zero return rows of every row without a slot
        led["recv_compact"]["bytes"] += S * P * 2 + A * rb + A * d * 2 + 4 * S * P1 + 4 * A + (S * P1 - A) * d * zb
        # accepted rows in, weights of the active experts, results stored through the row map into pool rows
        led["swiglu"]["bytes"] += A * d * 2 + E_act * 3 * d * dff * 2 + A * d * zb + 4 * A
        led["swiglu"]["flops"] += 6 * A * d * dff
    return led


def recv_cpu_baseline(w, host, sample):
    """The oracle's receiver step on the first waves of the batch, in full:
    compaction of every incoming row, the fp64 SwiGLU of every accepted row
    (fp8 records quantized and dequantized first), and the expansion back to
    pool rows.  ``sample`` is the number of waves (about 5 s of CPU each)."""
    import oracle as O
    n_w = max(1, min(sample, w.n_waves))
    t0 = time.perf_counter()
    acc = 0
    for wave in range(n_w):
        rc = O.recv_compact(host["pools"][wave], w.n_local, w.recv_cap)
        comp = rc["compact"]
        z = np.zeros((w.n_local * w.recv_cap, w.d))
        for e in range(w.n_local):
            c = int(rc["counts"][e])
            if c == 0:
                continue
            xr = comp[e, :c]
            if w.payload is not None:
                rec = O.quantize_fp8_rows(O.to_f64(xr).astype(np.float32), w.payload)
                xr = O.f32_to_bf16_rne(O.dequantize_fp8_rows(rec, w.d, w.payload))
            z[e * w.recv_cap:e * w.recv_cap + c] = O.swiglu_expert(
                O.to_f64(xr), O.to_f64(host["wg"][e]), O.to_f64(host["wu"][e]), O.to_f64(host["wd"][e]))
        O.expand_rows(z, rc["row_slot"])
        acc += int(rc["counts"].sum())
    dt = time.perf_counter() - t0
    return dict(value=n_w * w.n_src * w.pool_rows / dt, unit="incoming rows/s", cores=cpu_threads(), kind="oracle",
                extrapolated=False,
                sample=f"waves 0..{n_w - 1} of {w.name} in full: oracle compaction of {n_w}x{w.n_src}x{w.pool_rows} "
                       f"incoming rows, "
                       + ("fp8 quantize + dequantize and " if w.payload else "")
                       + f"fp64 SwiGLU of all {acc} accepted rows, expansion to pool rows; {dt:.2f} s")


def pack_setup(torch, w, banks):
    logits = W.router_logits(w)
    x = W.tokens(w)
    host = dict(logits=logits, x=x)
    b0 = {k: to_dev(torch, v) for k, v in host.items()}
    return host, [b0] + [{k: v.clone() for k, v in b0.items()} for _ in range(banks - 1)]


def pack_step(ge, timer, w, bank, flags, bufs):
    ids, gates = timer.run("route", ge.route_topk, bank["logits"], w.k, flags=flags)
    # with an fp8 payload the pack quantizes each bf16 token row itself
    out = timer.run("pool_pack", ge.pool_pack, bank["x"], ids, w.E, w.experts_per_dest, w.n_dest, w.n_waves,
                    w.pool_rows, pools=bufs["pools"], flags=flags, payload=w.payload, d=w.d)
    return dict(ids=ids, gates=gates, pack=out)


def pack_ledger(w):
    import grouped_expert_amd as ge
    T, k, d, E = w.T, w.k, w.d, w.E
    rb = ge.row_bytes(d, w.payload)
    P1 = ge.pool_height(w.pool_rows, d, w.payload)
    # token rows are read once as bf16 (quantized inside the pack for an fp8 payload)
    return {"route": dict(bytes=4 * T * E + 8 * T * k, flops=0),
            "pool_pack": dict(bytes=8 * T * k + T * d * 2 + w.n_waves * w.n_dest * P1 * rb, flops=0)}


def pack_cpu_baseline(w, host, sample):
    import oracle as O
    s = min(sample, w.T)
    t0 = time.perf_counter()
    ids, _, _ = O.route_topk(host["logits"][:s], w.k)
    rows = host["x"][:s]
    if w.payload is not None:
        rows = O.quantize_fp8_rows(O.to_f64(rows).astype(np.float32), w.payload)
    O.pool_pack(rows, ids, w.experts_per_dest, w.n_dest, w.n_waves, w.pool_rows)
    dt = time.perf_counter() - t0
    return dict(value=s / dt, unit="tokens/s", cores=cpu_threads(), kind="oracle",
                sample=f"first {s} of {w.T} tokens of {w.name}: route + "
                       + ("fp8 quantize + " if w.payload else "") + f"pack of all waves; {dt:.2f} s")


def router_setup(torch, w, banks):
    logits = W.router_logits(w)
    bias = W.router_bias(w)
    host = dict(logits=logits, bias=bias)
    b0 = {k: to_dev(torch, v) for k, v in host.items()}
    return host, [b0] + [{k: v.clone() for k, v in b0.items()} for _ in range(banks - 1)]


def router_step(ge, timer, w, bank, flags):
    if w.gating in (2, 3):
        ids, gates = timer.run("route", ge.route_topk_grouped, bank["logits"], w.k, w.gating, w.n_group,
                               w.topk_group, w.route_scale, bias=bank["bias"] if w.gating == 3 else None,
                               flags=flags)
    else:
        ids, gates = timer.run("route", ge.route_topk, bank["logits"], w.k, gating=w.gating, flags=flags)
    return dict(ids=ids, gates=gates)


def router_ledger(w):
    return {"route": dict(bytes=4 * w.T * w.E + 8 * w.T * w.k + (4 * w.E if w.gating == 3 else 0), flops=0)}


def router_cpu_baseline(w, host, sample):
    import oracle as O
    s = min(sample, w.T)
    t0 = time.perf_counter()
    if w.gating == 3:
        O.route_v3(host["logits"][:s], host["bias"], w.k, w.n_group, w.topk_group, w.route_scale)
    elif w.gating == 2:
        O.route_v2(host["logits"][:s], w.k, w.n_group, w.topk_group, w.route_scale)
    else:
        O.route_topk(host["logits"][:s], w.k)
    dt = time.perf_counter() - t0
    return dict(value=s / dt, unit="tokens/s", cores=cpu_threads(), kind="oracle",
                sample=f"first {s} of {w.T} tokens of {w.name}: the oracle router; {dt:.2f} s")


# ---------------------------------------------------------------------------

def main():
    args = parse()
    if args.record_traffic:
        record_traffic(args)
        return
    if args.record_mfma:
        record_mfma(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): this build has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import grouped_expert_amd as ge

    w = W.WORKLOADS[args.workload]
    banks = max(1, args.banks)
    torch.cuda.set_device(0)
    flags = ge.new_flags("cuda")
    kind = workload_kind(w)
    print(f"[bench] workload {w.name}: generating inputs ({banks} bank(s))", file=sys.stderr, flush=True)
    bufs = {}
    if kind == "layer":
        host, bank_list = layer_setup(torch, w, banks)
        step = lambda tm, b: layer_step(ge, tm, w, b, flags)
    elif kind == "train":
        host, bank_list = train_setup(torch, w, banks)
        step = lambda tm, b: train_step(ge, tm, w, b, flags)
    elif kind == "recv":
        host, bank_list = recv_setup(torch, w, banks)
        L, cap, d = w.n_local, w.recv_cap, w.d
        rdt = torch.bfloat16 if w.ret_dtype == "bf16" else torch.float32
        bufs = dict(compact=torch.empty((L, cap, d), dtype=torch.bfloat16, device="cuda"),
                    slot_row=torch.empty(L * cap, dtype=torch.int32, device="cuda"),
                    ret=[torch.empty((w.n_src * ge.pool_height(w.pool_rows, d, w.payload), d), dtype=rdt,
                                     device="cuda")
                         for _ in range(w.n_waves)],
                    starts=torch.arange(L, dtype=torch.int32, device="cuda") * cap)
        step = lambda tm, b: recv_step(ge, tm, w, b, flags, bufs)
    elif kind == "router":
        host, bank_list = router_setup(torch, w, banks)
        step = lambda tm, b: router_step(ge, tm, w, b, flags)
    else:
        host, bank_list = pack_setup(torch, w, banks)
        if w.payload is None:
            bufs = dict(pools=torch.empty((w.n_waves, w.n_dest, ge.pool_height(w.pool_rows, w.d), w.d),
                                          dtype=torch.bfloat16, device="cuda"))
        else:
            rb = ge.row_bytes(w.d, w.payload)
            bufs = dict(pools=torch.empty((w.n_waves, w.n_dest, ge.pool_height(w.pool_rows, w.d, w.payload), rb),
                                          dtype=torch.uint8, device="cuda"))
        step = lambda tm, b: pack_step(ge, tm, w, b, flags, bufs)
    # one plain device copy of known size (untimed): under rocprofv3 --pmc its
    # FETCH_SIZE / WRITE_SIZE readings calibrate the counters to bytes
    calib = torch.empty(COPY_CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
    calib_dst = torch.empty_like(calib)
    calib_dst.copy_(calib)
    del calib, calib_dst
    torch.cuda.synchronize()

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        last = step(OpTimer(torch), bank_list[i % banks])
    torch.cuda.synchronize()

    # per-call durations from an untimed pass with events around every call;
    # it also names the dominant call (the largest time per step)
    n_probe = max(2, min(args.steps, 5))
    print(f"[bench] per-call pass {n_probe} steps", file=sys.stderr, flush=True)
    probe = OpTimer(torch, lead=lambda: torch.cuda._sleep(LEAD_CYCLES))
    for i in range(n_probe):
        last = step(probe, bank_list[i % banks])
    torch.cuda.synchronize()
    per_op = {k: float(np.mean(v)) for k, v in probe.totals_ms().items()}
    n_calls = {k: len(v) // n_probe for k, v in probe.totals_ms().items()}
    dom = max(per_op, key=lambda k: per_op[k] * n_calls[k])

    # timed steps: events around the dominant call only (its launch duration,
    # live over the timed region, on the stream it runs on)
    # an event at every step boundary gives the per-step times (p50 / p95)
    timer = OpTimer(torch, only={dom})
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    marks[0].record()
    for i in range(args.steps):
        last = step(timer, bank_list[i % banks])
        marks[i + 1].record()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_wall
    total_ms = marks[0].elapsed_time(marks[-1])
    ms_per_step = total_ms / max(1, args.steps)
    step_ms = [marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)]
    dom_launches = timer.totals_ms()[dom]
    if int(flags.item()) != 0:
        print(f"[bench] warning: dev_flags = {int(flags.item())}", file=sys.stderr)

    # ledger and dominant call
    if kind in ("layer", "train"):
        counts = last["plan"]["counts"].cpu().numpy()
        led = layer_ledger(w, counts) if kind == "layer" else train_ledger(w, counts)
        units, unit = w.T, "tokens/s"
        per_step_calls = 1
    elif kind == "recv":
        cw = [rc["counts"].cpu().numpy() for rc, _ in last]
        led = recv_ledger(w, cw)
        units, unit = w.n_waves * w.n_src * w.pool_rows, "incoming rows/s"
        per_step_calls = w.n_waves
    elif kind == "router":
        led = router_ledger(w)
        units, unit = w.T, "tokens/s"
        per_step_calls = 1
    else:
        led = pack_ledger(w)
        units, unit = w.T, "tokens/s"
        per_step_calls = 1
    value = units / (ms_per_step / 1e3)
    dom_ms = float(np.mean(dom_launches))                 # average duration of one launch, timed region
    per_launch_bytes = led[dom]["bytes"] / per_step_calls if kind == "recv" else led[dom]["bytes"]
    per_launch_flops = led[dom]["flops"] / per_step_calls if kind == "recv" else led[dom]["flops"]
    t_s = dom_ms / 1e3
    peak_f = F32_PEAK_TFLOPS if w.dtype == "f32" else BF16_PEAK_TFLOPS
    bw = per_launch_bytes / t_s / 1e9
    tf = per_launch_flops / t_s / 1e12
    mfma_bound = per_launch_flops / (peak_f * 1e12) > per_launch_bytes / (HBM_PEAK_GBS * 1e9)
    traffic = recorded_traffic(w, dom)
    if mfma_bound:
        roof = dict(bound="mfma", achieved=round(tf, 2), peak=peak_f, unit="TFLOP/s", frac=round(tf / peak_f, 4),
                    traffic=traffic)
    else:
        roof = dict(bound="hbm", achieved=round(bw, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(bw / HBM_PEAK_GBS, 4), traffic=traffic)
    roof["traffic_unit"] = "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
    if dom in ("swiglu", "swiglu_bwd"):
        roof["mfma_busy"] = recorded_mfma(w, dom)
        roof["mfma_busy_formula"] = "SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / XCDs * CUs * 4), rocprofv3"
        roof["mfma_frac_of_peak"] = round(tf / BF16_PEAK_TFLOPS, 4) if w.dtype != "f32" else None
    if traffic:
        roof["traffic_over_alg"] = round(traffic / max(1, per_launch_bytes), 3)
    roof["kernel"] = dom
    roof["launch_ms"] = round(dom_ms, 4)
    roof["launches_timed"] = len(dom_launches)
    roof["alg_bytes_per_launch"] = int(per_launch_bytes)
    roof["alg_flops_per_launch"] = int(per_launch_flops)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        if kind == "layer":
            cpu = layer_cpu_baseline(w, host, args.cpu_sample or min(w.T, 2048))
        elif kind == "train":
            cpu = train_cpu_baseline(w, host, args.cpu_sample or min(w.T, 512))
        elif kind == "recv":
            cpu = recv_cpu_baseline(w, host, args.cpu_sample or 2)
        elif kind == "router":
            cpu = router_cpu_baseline(w, host, args.cpu_sample or 32768)
        else:
            cpu = pack_cpu_baseline(w, host, args.cpu_sample or 16384)
        cpu.setdefault("extrapolated", False)
        cpu.update(cpu_host_info())
        cpu["input_sha256"] = input_sha256(host)

    cfg = {"workload": w.name, "dtype": w.dtype}
    for key in ("T", "d", "E", "k", "d_ff", "capacity", "experts_per_dest", "n_dest", "n_waves", "pool_rows",
                "n_src", "n_local", "recv_cap", "gating", "n_group", "topk_group"):
        v = getattr(w, key)
        if v:
            cfg[key] = v
    cfg["banks"] = banks
    ops = {k: dict(ms=round(per_op[k], 4), calls_per_step=n_calls[k],
                   alg_GBps=round(led[k]["bytes"] / (per_step_calls if kind == "recv" else 1) / (per_op[k] / 1e3)
                                  / 1e9, 1) if k in led else None)
           for k in per_op}
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_p50": round(nearest_rank(step_ms, 50), 4), "ms_per_step_p95": round(nearest_rank(step_ms, 95), 4),
        "timed_ms": round(total_ms, 2), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32" if w.dtype == "f32" else "bf16",
        "data": "synthetic", "config": cfg, "roofline": roof, "cpu_baseline": cpu, "ops": ops,
        "ops_note": f"per-call device ms from {n_probe} untimed steps with events around every call, each call "
                    f"queued behind a {LEAD_CYCLES}-cycle spin kernel (no memory traffic) so that host work between "
                    f"its kernels is not counted",
        "wall_s": round(wall_s, 3),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
