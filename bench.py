#!/usr/bin/env python3
"""Benchmark of the varlen (paged) flash-attention forward on one MI355X.

One step = one ``fa_varlen_fwd`` call (every kernel of the path: planner,
attention, split combine) over one batch of seeded synthetic inputs already
resident in HBM.

Default run (no ``--workload``): the headline is the long-prefill workload
(8 sequences log-uniform in [1024, 16384] summing to 65,536 tokens, H 64 /
Hk 8, head_dim 128, causal with window_left 4096), reported as TFLOP/s against
the bf16 MFMA peak.  The same process then times the four other workloads
under the ``suite`` key: paged decode (64 x q_len 1, kv U[1,4096], page 32,
H 32 / Hk 8, D 128) and the two spec-decode workloads (32 x q_len 4, kv
U[1024,32768], page 128, D 256 MHA and D 512 MQA) as KV GB/s against HBM, and
paged chunked prefill (16 seqs, q U[1,512] over prefixes U[0,8192], page 64)
as TFLOP/s, and the 86-token causal batch (3 sequences of 17, 64 and 5 tokens,
head_dim 64), whose step time is a latency figure.  ``--workload cN`` times one
workload alone.

Timed region: W untimed warm-up steps (continued, untimed, until at least 0.2 s
of them have run, so the shader clock has settled), then exactly K steps bracketed by
``torch.cuda.synchronize()``, with no per-step events (``value``, ``ms_per_step``).
Consecutive steps read different copies of the inputs (enough copies to exceed
the 256 MB last-level cache), so K/V really come from HBM.  A second pass of K
steps records HIP events around the attention kernel of every call on its
launch stream (``fa_varlen_set_kernel_events``); an event between two
dependent kernels holds the stream for about 5 us, which is why the step time
is taken without them.  Each entry reports two roofline fractions: ``frac``
for the attention kernel alone (its mean event-timed duration) and
``frac_call`` for the whole call (the step time: planner, attention, combine).
The 86-token batch is also timed from a HIP graph of 32 captured calls replayed
10 times (``graph_replay_ms_per_step``): its latency without per-call host work.

Counters (default run; ``--no-counters`` skips them): before it touches the
GPU, the bench runs itself four times under ``rocprofv3 --pmc`` (a 1 GiB
device copy, then the usual warm-up and 3 steps of the headline workload):
  * SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE, ... -> counter-derived MFMA
    utilisation of the attention kernel (busy MFMA cycles / (GPU cycles x
    SIMDs)), the shader clock it ran at, and MFMA work issued vs algorithmic;
  * SQ_WAVE_CYCLES, SQ_ACTIVE_INST_ANY, SQ_WAIT_INST_ANY, SQ_WAIT_ANY, ... ->
    where each wave's cycles go (issuing, waiting for an issue slot, waiting
    on dependencies) and the resident waves per SIMD;
  * FETCH_SIZE, then WRITE_SIZE -> the kernel's HBM bytes per launch, each
    scaled by what the same counter reads for the 1 GiB copy (``traffic``).

Prints ONE JSON line: metric/value/unit, ms_per_step, a ``roofline`` object
for the headline's attention kernel, ``cpu_baseline`` (the fp64 oracle timed on
a bounded sample of the headline workload on this host's cores), ``suite``
and ``counters``.

``--op append`` times the paged K/V append instead (``fa_kv_append``): each
sequence of a paged workload appends as many new tokens as it has query rows
(its last keys), reported as GB/s of algorithmic HBM traffic.  ``--op padded``
times the padded (batch-major) entry ``fa_padded_fwd`` on the padded workloads
(``--workload p4``: uniform-length long prefill; ``p2``: uniform decode batch).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "varlen paged attention: prefill TFLOP/s (%MFMA peak); decode KV GB/s (%HBM)"
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
DECODE = {"c2", "c5a", "c5b"}
KERNEL_SRC = os.path.join(ROOT, "varlen_flash_attention_fa_amd", "csrc", "fa_fwd.hip")
APPEND_SRC = os.path.join(ROOT, "varlen_flash_attention_fa_amd", "csrc", "fa_append.hip")
APPEND_METRIC = "paged KV-cache append: GB/s of algorithmic HBM traffic (%HBM)"


# ------------------------------------------------------------------ HIP events

class Hip:
    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        rc = self.lib.hipEventCreate(ctypes.byref(e))
        assert rc == 0, rc
        return e.value

    def record(self, ev, stream):
        rc = self.lib.hipEventRecord(ev, stream)
        assert rc == 0, rc

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b)
        assert rc == 0, rc
        return float(ms.value)

    def destroy(self, ev):
        self.lib.hipEventDestroy(ev)


# ------------------------------------------------------------ algorithmic work

def visible_pairs(lq, lk, wl, wr):
    """Number of (query, key) pairs visible under the bottom-right aligned window."""
    total = 0
    per_seq = []
    for Lq, Lk in zip(lq, lk):
        i = np.arange(int(Lq), dtype=np.int64)
        a = i + int(Lk) - int(Lq)
        lo = np.maximum(0, a - wl) if wl >= 0 else np.zeros_like(a)
        hi = np.minimum(int(Lk), a + wr + 1) if wr >= 0 else np.full_like(a, int(Lk))
        n = np.maximum(0, hi - lo)
        per_seq.append(n)
        total += int(n.sum())
    return total, per_seq


def work_of(wl):
    H, Hk, D = wl.num_heads, wl.num_heads_k, wl.head_dim
    pairs, per_seq = visible_pairs(wl.lens_q, wl.lens_k, wl.window_left, wl.window_right)
    flops = 4.0 * D * H * pairs
    kv_bytes = 2.0 * Hk * D * 2 * float(wl.lens_k.sum())
    qo_bytes = 2.0 * float(wl.lens_q.sum()) * H * D * 2
    bt_bytes = 0.0
    if wl.paged:
        P = wl.page_block_size
        bt_bytes = 4.0 * float(((wl.lens_k + P - 1) // P).sum())
    meta = 8.0 * (wl.batch + 1)
    return dict(pairs=pairs, per_seq=per_seq, flops=flops, kv_bytes=kv_bytes,
                total_bytes=kv_bytes + qo_bytes + bt_bytes + meta)


# ------------------------------------------------------------------- profiles

def kernel_sha(src: str = KERNEL_SRC) -> str:
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


def append_work(wl):
    """Algorithmic bytes of appending each sequence's query-length worth of new tokens."""
    Hk, D = wl.num_heads_k, wl.head_dim
    total_new = float(wl.lens_q.sum())
    rows = 2.0 * total_new * Hk * D * 2          # K and V rows, bf16
    meta = 8.0 * (wl.batch + 1) + 4.0 * total_new  # cu arrays + one block id per token
    return dict(total_new=int(total_new), row_bytes=rows, total_bytes=2.0 * rows + meta)


def stored_traffic(workload: str, op: str = "fwd", dtype: str = "bf16", alibi: bool = False):
    """HBM bytes per launch from the committed counter summary, if the kernel is unchanged.

    The summaries were taken on the bf16 kernels without ALiBi slopes; other
    instantiations (fp16, ALiBi) report None."""
    if dtype != "bf16" or alibi:
        return None
    if op == "append":
        path = os.path.join(ROOT, "profiles", "kv_append_%s_hbm_traffic.md" % workload)
        src, key = APPEND_SRC, "HBM bytes per launch (scaled)"
    else:
        # the counter summary that `bench.py --workload W --counters` writes
        path = os.path.join(ROOT, "profiles", "attn_fwd_%s_counters.md" % workload)
        src, key = KERNEL_SRC, "hbm_bytes"
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel source sha256/16") != kernel_sha(src):
        return None
    try:
        return float(vals[key])
    except (KeyError, ValueError):
        return None


def counters_summary(workload, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_mib, op="fwd"):
    """Markdown summary of the main kernel's HBM traffic from rocprofv3 --pmc CSVs.

    FETCH_SIZE / WRITE_SIZE (KiB per dispatch) are scaled by what the same
    counter reads for a plain device copy of ``copy_mib`` MiB (read and write
    of exactly that many bytes)."""
    import csv

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in vals.items()}

    kname = "kv_append_kernel" if op == "append" else "attn_fwd_kernel"

    def main_kernel(d):
        k = [n for n in d if kname in n]
        assert k, kname + " not in counter file"
        return k[0], d[k[0]]

    copy_kib = copy_mib * 1024.0
    cf = per_kernel(copy_fetch_csv, "FETCH_SIZE").get("__amd_rocclr_copyBuffer")
    cw = per_kernel(copy_write_csv, "WRITE_SIZE").get("__amd_rocclr_copyBuffer")
    f_scale, w_scale = copy_kib / cf, copy_kib / cw
    name, fetch = main_kernel(per_kernel(fetch_csv, "FETCH_SIZE"))
    _, write = main_kernel(per_kernel(write_csv, "WRITE_SIZE"))
    traffic = (fetch * f_scale + write * w_scale) * 1024.0
    import workloads as W
    if op == "append":
        alg = append_work(W.append_config(workload))["total_bytes"]
    else:
        alg = work_of(W.make_config(workload))["total_bytes"]
    lines = [
        "# HBM traffic of %s, workload %s%s" % (kname, workload, " (append)" if op == "append" else ""),
        "",
        "Counters per dispatch (KiB), averaged over the profiled launches, scaled by a plain",
        "%d MiB device copy (`__amd_rocclr_copyBuffer`) read with the same counters." % copy_mib,
        "",
        "- kernel: `%s`" % name,
        "- kernel source sha256/16: `%s`" % kernel_sha(APPEND_SRC if op == "append" else KERNEL_SRC),
        "- FETCH_SIZE per launch (raw KiB): `%.1f`" % fetch,
        "- WRITE_SIZE per launch (raw KiB): `%.1f`" % write,
        "- copy calibration FETCH_SIZE / WRITE_SIZE (KiB for %d KiB moved): `%.1f` / `%.1f`" % (copy_kib, cf, cw),
        "- scale factors fetch / write: `%.4f` / `%.4f`" % (f_scale, w_scale),
        "- HBM bytes per launch (scaled): `%.0f`" % traffic,
        "- algorithmic bytes per launch: `%.0f`" % alg,
        "- traffic / algorithmic: `%.3f`" % (traffic / alg),
    ]
    return "\n".join(lines) + "\n"


# ----------------------------------------------------------------- CPU leg

def cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), or an empty string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def cpu_baseline(wl, work, decode: bool, alibi=None):
    """Time the fp64 oracle on a bounded sample of the workload on the host cores."""
    import oracle
    oracle.build()
    threads = oracle.default_threads()
    H, D = wl.num_heads, wl.head_dim
    fma_per_pair = 2.0 * D * H           # q.k and p.v, per head
    # the oracle runs ~1.5 G fp64 multiply-adds per second per thread (measured on
    # 16 host cores): this bounds the sample to roughly 10-15 s of wall time
    budget = 2.0e10 * threads
    if decode:
        # whole sequences until the budget: metric is KV bytes of the sequences served
        order = list(range(wl.batch))
        sel = np.zeros(wl.q.shape[0], np.uint8)
        kv = 0.0
        spent = 0.0
        nseq = 0
        for b in order:
            cost = float(work["per_seq"][b].sum()) * fma_per_pair
            if nseq and spent + cost > budget:
                break
            q0, q1 = int(wl.cu_seqlens_q[b]), int(wl.cu_seqlens_q[b + 1])
            sel[q0:q1] = 1
            kv += 2.0 * wl.num_heads_k * D * 2 * float(wl.lens_k[b])
            spent += cost
            nseq += 1
        reps, t0 = 0, time.perf_counter()
        while True:  # repeat a small sample until the timing is at least ~10 s long
            oracle.attention_workload(wl, token_sel=sel, nthreads=threads, alibi_slopes=alibi)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= 10.0:
                break
        return {"value": round(reps * kv / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
                "kind": "oracle", "cpu_model": cpu_model(),
                "sample": "%d of %d sequences (all their query rows), %.3g GB of K/V, run %d times "
                          "in %.2f s" % (nseq, wl.batch, kv / 1e9, reps, dt)}
    # prefill: a seeded sample of query rows; metric is FLOP of those rows
    rng = np.random.Generator(np.random.PCG64(4242))
    rows_pairs = np.concatenate(work["per_seq"]).astype(np.float64)
    T = rows_pairs.shape[0]
    perm = rng.permutation(T)
    cum = np.cumsum(rows_pairs[perm] * fma_per_pair)
    n = int(max(1, min(T, np.searchsorted(cum, budget) + 1)))
    sel = np.zeros(T, np.uint8)
    sel[perm[:n]] = 1
    flops = 4.0 * D * H * float(rows_pairs[perm[:n]].sum())
    t0 = time.perf_counter()
    oracle.attention_workload(wl, token_sel=sel, nthreads=threads, alibi_slopes=alibi)
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "%d of %d query rows (seeded), %.3g GFLOP, %.2f s" % (n, T, flops / 1e9, dt)}


# ------------------------------------------------------------- append bench

def cpu_append_baseline(wl, k_new, v_new, work):
    """Time the oracle's append of the whole workload, repeated for >= 10 s."""
    import oracle
    oracle.build()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.kv_append(k_new, v_new, wl.cu_seqlens_q, wl.cu_seqlens_k, wl.block_table, wl.k, wl.v)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0:
            break
    return {"value": round(reps * work["total_bytes"] / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "whole append (%d tokens) run %d times in %.2f s; each oracle call also copies "
                      "both pools (it returns new ones)" % (work["total_new"], reps, dt)}


def bench_append(args, fa, W, hip, dev, stream):
    import torch
    print("bench: generating %s (append)" % args.workload, file=sys.stderr, flush=True)
    wl = W.append_config(args.workload, args.seed, dtype=args.dtype)
    work = append_work(wl)
    # new rows: the pool rows of each sequence's last Lq keys (what a decode or
    # chunked-prefill step appends); rotated copies keep them out of the MALL
    P = wl.page_block_size
    rows = []
    for b in range(wl.batch):
        pos = np.arange(int(wl.lens_k[b] - wl.lens_q[b]), int(wl.lens_k[b]))
        rows.append(wl.block_table[b, pos // P].astype(np.int64) * P + pos % P)
    rows = torch.from_numpy(np.concatenate(rows))
    Hk, D = wl.num_heads_k, wl.head_dim
    k_new = wl.k.view(-1, Hk, D)[rows].contiguous()
    v_new = wl.v.view(-1, Hk, D)[rows].contiguous()
    n_new = int(min(32, max(2, math.ceil(1.0e9 / max(1.0, work["row_bytes"])))))
    with torch.cuda.stream(stream):
        news = [(k_new.to(dev), v_new.to(dev)) for _ in range(n_new)]
        pools = [(wl.k.to(dev), wl.v.to(dev)) for _ in range(2)]
        cu_n = torch.from_numpy(wl.cu_seqlens_q).to(dev)
        cu_k = torch.from_numpy(wl.cu_seqlens_k).to(dev)
        bt = torch.from_numpy(wl.block_table).to(dev)
        torch.cuda.synchronize()
    dnew = [(fa._tdesc(a), fa._tdesc(b)) for a, b in news]
    dpool = [(fa._tdesc(a), fa._tdesc(b)) for a, b in pools]
    dbt = fa._tdesc(bt)
    sh = stream.cuda_stream

    def step(i, ev_k=None):
        kn, vn = dnew[i % n_new]
        kc, vc = dpool[i % 2]
        if ev_k is not None:
            fa.fa_varlen_set_kernel_events(ev_k[0], ev_k[1])
        rc = fa.fa_kv_append(kn, vn, cu_n.data_ptr(), cu_k.data_ptr(), wl.batch, dbt, kc, vc, P, sh)
        if rc:
            raise RuntimeError(fa.fa_last_error())

    warm = warm_up(step, args.warmup)
    # A step is this one kernel: two events around the whole timed region give its
    # mean duration without the per-call event cost (a few us, comparable to the
    # kernel on the small appends).  Per-call events, in a second pass of K steps,
    # are kept as detail.
    K = args.steps
    sampled = list(range(K))
    region_k = (hip.event(), hip.event())
    print("bench: timing %d append steps" % K, file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    hip.record(region_k[0], sh)
    for i in range(K):
        step(i)
    hip.record(region_k[1], sh)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    kern_mean = hip.elapsed_ms(*region_k) / K
    ev_kern = {i: (hip.event(), hip.event()) for i in sampled}
    for i in sampled:
        step(i, ev_kern[i])
        fa.fa_varlen_set_kernel_events(0, 0)
    torch.cuda.synchronize()
    kern_ms = np.array([hip.elapsed_ms(*ev_kern[i]) for i in sampled])
    for a, b in list(ev_kern.values()) + [region_k]:
        hip.destroy(a)
        hip.destroy(b)
    # the pools must still equal the original (the new rows are the original rows)
    for kc, vc in pools:
        assert torch.equal(kc.view(torch.int16).cpu(), wl.k.view(torch.int16)), "append changed the K pool"
        assert torch.equal(vc.view(torch.int16).cpu(), wl.v.view(torch.int16)), "append changed the V pool"
    achieved = work["total_bytes"] / (kern_mean * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": stored_traffic(args.workload, "append", args.dtype)}
    cpu = None
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle append)", file=sys.stderr, flush=True)
        cpu = cpu_append_baseline(wl, k_new, v_new, work)
    props = torch.cuda.get_device_properties(dev)
    line = {
        "metric": APPEND_METRIC,
        "value": round(work["total_bytes"] / (ms_per_step * 1e-3) / 1e9, 3),
        "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": args.dtype,
        "data": "synthetic (seeded N(0,1) %s, seed %d)" % (args.dtype, wl.seed),
        "config": {
            "workload": "append into %s: %s" % (args.workload, wl.extra.get("desc", "")),
            "batch": wl.batch, "total_new": work["total_new"], "num_heads_k": Hk, "head_dim": D,
            "page_block_size": P, "parallelism": "single GPU",
        },
        "roofline": roof,
        "cpu_baseline": cpu,
        "detail": {
            "append_kernel_ms_mean": round(kern_mean, 6),
            "append_kernel_ms_per_call_events_p50": round(float(np.median(kern_ms)), 6),
            "per_call_event_samples": len(sampled), "warmup_steps_run": warm,
            "algorithmic_total_bytes": work["total_bytes"],
            "new_row_copies_rotated": n_new, "kernel_source_sha256_16": kernel_sha(APPEND_SRC),
            "device": props.name,
        },
    }
    print(json.dumps(line), flush=True)
    return 0


# ------------------------------------------------------------- padded bench

def bench_padded(args, fa, W, hip, dev, stream):
    import torch
    cfg = W.PADDED[args.workload]
    B, Sq, Sk, H, Hk, D = (cfg[x] for x in ("B", "Sq", "Sk", "num_heads", "num_heads_k", "head_dim"))
    seed = cfg["seed"] if args.seed is None else args.seed
    print("bench: generating %s (padded)" % args.workload, file=sys.stderr, flush=True)
    q, k, v = W.make_padded(B, Sq, Sk, H, Hk, D, seed=seed, dtype=args.dtype)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    # the equivalent varlen description (uniform offsets) gives the algorithmic work
    # and feeds the oracle's CPU leg
    wl = W.Workload(name=args.workload, seed=seed, q=q.reshape(B * Sq, H, D), k=k.reshape(B * Sk, Hk, D),
                    v=v.reshape(B * Sk, Hk, D), cu_seqlens_q=(np.arange(B + 1) * Sq).astype(np.int32),
                    cu_seqlens_k=(np.arange(B + 1) * Sk).astype(np.int32), block_table=None,
                    page_block_size=0, softmax_scale=scale, window_left=cfg["window_left"],
                    window_right=cfg["window_right"])
    work = work_of(wl)
    decode = Sq * (H // Hk) <= 64
    per_copy = (k.numel() + v.numel() + 2 * q.numel()) * 2
    ncopies = int(min(8, max(1, math.ceil(2.0e9 / per_copy))))
    with torch.cuda.stream(stream):
        copies = []
        for _ in range(ncopies):
            d = dict(q=q.to(dev), k=k.to(dev), v=v.to(dev))
            d["out"] = torch.empty_like(d["q"])
            copies.append(d)
        torch.cuda.synchronize()
    calls = [(fa._tdesc(d["q"]), fa._tdesc(d["k"]), fa._tdesc(d["v"]), fa._tdesc(d["out"])) for d in copies]
    ws_bytes = fa.fa_padded_workspace_bytes(*calls[0][:3])
    workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    sh = stream.cuda_stream
    alibi_t = torch.from_numpy(W.alibi_slopes(H)).to(dev) if args.alibi else None
    dal = fa._tdesc(alibi_t) if alibi_t is not None else None

    def step(i, ev_k=None):
        dq, dk, dv, do = calls[i % ncopies]
        if ev_k is not None:
            fa.fa_varlen_set_kernel_events(ev_k[0], ev_k[1])
        rc = fa.fa_padded_fwd(dq, dk, dv, do, scale, cfg["window_left"], cfg["window_right"], 0,
                              workspace.data_ptr() if ws_bytes else 0, ws_bytes, sh, dal)
        if rc:
            raise RuntimeError(fa.fa_last_error())

    warm = warm_up(step, args.warmup)
    K = args.steps
    ms_per_step, kern_ms = timed_passes(step, K, hip, True, "padded " + args.workload,
                                        lambda: fa.fa_varlen_set_kernel_events(0, 0))
    kern_mean = float(kern_ms.mean())
    if decode:
        value, unit = work["kv_bytes"] / (ms_per_step * 1e-3) / 1e9, "GB/s"
        achieved = work["total_bytes"] / (kern_mean * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    else:
        value, unit = work["flops"] / (ms_per_step * 1e-3) / 1e12, "TFLOP/s"
        achieved = work["flops"] / (kern_mean * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    roof["traffic"] = None
    cpu = None
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, work, decode, W.alibi_slopes(wl.num_heads) if args.alibi else None)
    props = torch.cuda.get_device_properties(dev)
    line = {
        "metric": "padded (batch-major) attention: prefill TFLOP/s (%MFMA peak); decode KV GB/s (%HBM)",
        "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": args.dtype,
        "data": "synthetic (seeded N(0,1) %s, seed %d)" % (args.dtype, seed),
        "config": {"workload": "%s: %s" % (args.workload, cfg["desc"]), "batch": B, "seqlen_q": Sq,
                   "seqlen_k": Sk, "num_heads": H, "num_heads_k": Hk, "head_dim": D,
                   "window_left": cfg["window_left"], "window_right": cfg["window_right"],
                   "alibi": bool(args.alibi), "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "detail": {"main_kernel_ms_mean": round(kern_mean, 5), "kernel_event_steps": int(kern_ms.size),
                   "warmup_steps_run": warm,
                   "algorithmic_flop": work["flops"], "algorithmic_total_bytes": work["total_bytes"],
                   "input_copies_rotated": ncopies, "workspace_bytes": ws_bytes,
                   "kernel_source_sha256_16": kernel_sha(), "device": props.name},
    }
    print(json.dumps(line), flush=True)
    return 0


# ------------------------------------------------------------ counter passes

# one rocprofv3 --pmc run each (SQ: at most 8 counters, GRBM 2, TCC 4 per run)
MFMA_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY",
                 "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU",
                 "GRBM_GUI_ACTIVE"]
# where each wave's cycles go: issuing (ACTIVE_INST_ANY), waiting for an issue slot
# (WAIT_INST_ANY) or waiting on dependencies, waitcnt and barriers (WAIT_ANY)
STALL_COUNTERS = ["SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU",
                  "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_SCA", "SQ_INSTS_SALU", "GRBM_GUI_ACTIVE"]
COUNTER_PASSES = [("mfma", MFMA_COUNTERS), ("stall", STALL_COUNTERS), ("fetch", ["FETCH_SIZE"]),
                  ("write", ["WRITE_SIZE"])]
COUNTER_STEPS = 3  # timed steps of a counter pass (after the same warm-up as the bench)
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_MIB = 1024
XCDS = 8          # GRBM_GUI_ACTIVE is summed over the 8 XCDs
SIMDS_PER_CU = 4


def _rocprofv3():
    import shutil
    for c in (shutil.which("rocprofv3"), "/opt/rocm/bin/rocprofv3"):
        if c and os.path.exists(c):
            return c
    return None


def parse_counter_csv(path):
    """{kernel name: {counter: [per-dispatch values]}} and per-dispatch durations (ns)."""
    import csv
    vals, durs = {}, {}
    for r in csv.DictReader(open(path)):
        k = r["Kernel_Name"]
        vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        durs.setdefault(k, {})[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    return vals, {k: list(v.values()) for k, v in durs.items()}


def _mean_tail(xs, last=None):
    """Mean over the last ``last`` dispatches (the timed steps of a counter pass,
    after its warm-up), or over all but the first when ``last`` is None."""
    xs = list(xs)
    if last:
        return float(np.mean(xs[-last:]))
    return float(np.mean(xs[1:] if len(xs) > 1 else xs))


def run_counter_passes(workload, dtype, outroot, timeout_s=170):
    """Run the counter passes as child processes; returns raw per-pass results or an error."""
    prof = _rocprofv3()
    if prof is None:
        return {"error": "rocprofv3 not found"}
    res = {"workload": workload, "passes": {}, "commands": [], "steps": COUNTER_STEPS}
    for name, counters in COUNTER_PASSES:
        d = os.path.join(outroot, name)
        os.makedirs(d, exist_ok=True)
        cmd = ["timeout", "-s", "KILL", str(timeout_s), prof, "--pmc"] + counters + [
            "--output-format", "csv", "-d", d, "-o", "run", "--", sys.executable,
            os.path.join(ROOT, "bench.py"), "--counter-child", "--workload", workload, "--dtype", dtype,
            "--steps", str(COUNTER_STEPS), "--warmup", "1"]
        res["commands"].append(" ".join(["rocprofv3", "--pmc"] + counters + [
            "--output-format", "csv", "-d", os.path.relpath(d, ROOT), "-o", "run", "--", "python3", "bench.py",
            "--counter-child", "--workload", workload, "--dtype", dtype, "--steps", str(COUNTER_STEPS),
            "--warmup", "1"]))
        print("bench: counter pass %s (%s)" % (name, " ".join(counters)), file=sys.stderr, flush=True)
        env = dict(os.environ, FA_BENCH_CHILD="1")
        import subprocess
        with open(os.path.join(d, "child.log"), "w") as log:
            rc = subprocess.call(cmd, stdout=log, stderr=subprocess.STDOUT, env=env, cwd=ROOT)
        csvp = os.path.join(d, "run_counter_collection.csv")
        if not os.path.exists(csvp):
            return dict(res, error="pass %s: no counter file (exit %d)" % (name, rc))
        # rocprofv3 may exit non-zero after the program has finished and written
        # complete results; the file is checked instead
        res["passes"][name] = parse_counter_csv(csvp)
    return res


def derive_counters(raw, kname, alg_flops, alg_bytes, cus):
    """Counter-derived figures of one kernel from the three passes (averaged over
    the pass's timed steps, one dispatch of the kernel each)."""
    if "error" in raw:
        return {"error": raw["error"]}
    out = {"kernel": None}
    mv, md = raw["passes"]["mfma"]
    names = [k for k in mv if kname in k]
    if not names:
        return {"error": "%s not in the counter file" % kname}
    k = names[0]
    out["kernel"] = k
    last = raw.get("steps")
    c = {n: _mean_tail(v, last) for n, v in mv[k].items()}
    dur_ns = _mean_tail(md[k], last)
    simds = cus * SIMDS_PER_CU
    cycles = c["GRBM_GUI_ACTIVE"] / XCDS
    out.update({
        "dispatches": len(md[k]),
        "dispatches_averaged": min(len(md[k]), last) if last else len(md[k]) - 1,
        "profiled_kernel_us": round(dur_ns / 1e3, 2),
        "gpu_cycles": cycles,
        "sclk_ghz": round(cycles / dur_ns, 3),
        "mfma_busy_cycles": c["SQ_VALU_MFMA_BUSY_CYCLES"],
        # fraction of SIMD-cycles in which the matrix core was busy
        "mfma_util": round(c["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * simds), 4),
        "mfma_flops_issued": c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0,
        "issued_over_algorithmic": round(c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0 / alg_flops, 4)
        if alg_flops else None,
        "wait_inst_over_wave_cycles": round(c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"], 4),
        "coexec_over_mfma_busy": round(c["SQ_VALU_MFMA_COEXEC_CYCLES"] / c["SQ_VALU_MFMA_BUSY_CYCLES"], 4),
        "valu_insts": c["SQ_INSTS_VALU"],
        # the bf16 MFMA peak at the clock the kernel actually ran at
        "mfma_peak_at_sclk_tflops": round(cus * 4096.0 * cycles / dur_ns / 1e3, 1),
    })
    # stall breakdown per wave (fractions of SQ_WAVE_CYCLES, same pass)
    if "stall" in raw["passes"]:
        sv, _ = raw["passes"]["stall"]
        if k in sv:
            st = {n: _mean_tail(v, last) for n, v in sv[k].items()}
            wc = st["SQ_WAVE_CYCLES"]
            out.update({
                "waves_per_simd": round(wc * 4.0 / (st["GRBM_GUI_ACTIVE"] / XCDS * simds), 3),
                "issuing_over_wave_cycles": round(st["SQ_ACTIVE_INST_ANY"] / wc, 4),
                "issue_wait_over_wave_cycles": round(st["SQ_WAIT_INST_ANY"] / wc, 4),
                "dependency_wait_over_wave_cycles": round(st["SQ_WAIT_ANY"] / wc, 4),
                "valu_active_over_wave_cycles": round(st["SQ_ACTIVE_INST_VALU"] / wc, 4),
                "lds_active_over_wave_cycles": round(st["SQ_ACTIVE_INST_LDS"] / wc, 4),
                "scalar_active_over_wave_cycles": round(st["SQ_ACTIVE_INST_SCA"] / wc, 4),
                "salu_insts": st["SQ_INSTS_SALU"],
            })
        raw_c = {"mfma:" + n: v for n, v in c.items()}
        raw_c.update({"stall:" + n: _mean_tail(x, last) for n, x in sv.get(k, {}).items()})
        out["raw_counters_per_dispatch"] = {n: round(v, 1) for n, v in sorted(raw_c.items())}
    # HBM traffic: FETCH_SIZE / WRITE_SIZE (KiB) scaled by the 1 GiB copy's reading
    try:
        fv, _ = raw["passes"]["fetch"]
        wv, _ = raw["passes"]["write"]
        copy_kib = COPY_MIB * 1024.0

        def copy_reading(v, counter):
            xs = sorted(v[COPY_KERNEL][counter])
            big = [x for x in xs if x >= 0.5 * xs[-1]]  # the calibration copies, not small transfers
            return float(np.mean(big))
        f_scale = copy_kib / copy_reading(fv, "FETCH_SIZE")
        w_scale = copy_kib / copy_reading(wv, "WRITE_SIZE")
        fk = _mean_tail(fv[k]["FETCH_SIZE"], last)
        wk = _mean_tail(wv[k]["WRITE_SIZE"], last)
        traffic = (fk * f_scale + wk * w_scale) * 1024.0
        out.update({"fetch_kib": round(fk, 1), "write_kib": round(wk, 1), "fetch_scale": round(f_scale, 4),
                    "write_scale": round(w_scale, 4), "hbm_bytes": round(traffic),
                    "hbm_over_algorithmic": round(traffic / alg_bytes, 4) if alg_bytes else None})
    except (KeyError, ValueError, ZeroDivisionError) as e:
        out["traffic_error"] = repr(e)
    return out


def counter_child(args, fa, W, hip, dev, stream):
    """Body of a counter pass: a 1 GiB device copy (the calibration) then a few steps."""
    import torch
    n = COPY_MIB << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    time_workload(fa, W, hip, dev, stream, args.workload, args.steps, args.warmup, False, args.dtype,
                  args.alibi, args.seed)
    return 0


def counters_markdown(res, raw, workload, dtype, invocation):
    """Markdown summary of the counter passes (for profiles/); ``invocation`` is
    the bench command that ran them."""
    lines = ["# Counters of the attention kernel on workload %s (%s)" % (workload, dtype), "",
             "Each pass is a separate `rocprofv3 --pmc` run of a short bench run (1 GiB device copy,",
             "then the bench's warm-up, at least 0.2 s of steps, then %d steps); values are per" % COUNTER_STEPS,
             "dispatch, averaged over the %d timed dispatches.  MFMA utilisation =" % COUNTER_STEPS,
             "SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs).  Stall pass: each wave's",
             "cycles (SQ_WAVE_CYCLES) split into issuing (SQ_ACTIVE_INST_ANY), waiting for an issue slot",
             "(SQ_WAIT_INST_ANY) and waiting on dependencies, waitcnt and barriers (SQ_WAIT_ANY).  HBM bytes = FETCH_SIZE and WRITE_SIZE, each scaled by what it reads for",
             "the 1 GiB copy.", "",
             "- kernel source sha256/16: `%s`" % kernel_sha()]
    for key, val in res.items():
        lines.append("- %s: `%s`" % (key, val))
    lines += ["", "Made from the repository root by", "", "```", invocation, "```", "",
              "which runs each counter pass as a child process:", "", "```"]
    lines += list(raw.get("commands", []))
    lines += ["```", ""]
    return "\n".join(lines)


# ------------------------------------------------------------------ timing

WARMUP_MIN_S = 0.2


def warm_up(step, W, min_s=WARMUP_MIN_S):
    """W untimed steps, continued until at least ``min_s`` seconds of them have
    run (synchronised), so the shader clock has left its idle level before the
    timed steps: after 5 steps (2 ms) of the chunked-prefill call its steps took
    0.36 ms, after 300 steps 0.30 ms.  Returns the number of steps run."""
    import torch
    n = 0
    t0 = time.perf_counter()
    while n < W or time.perf_counter() - t0 < min_s:
        for _ in range(max(1, W if n < W else 16)):
            step(n)
            n += 1
        torch.cuda.synchronize()
    return n


def timed_passes(step, K, hip, events, name, reset):
    """The two timed passes of K calls each.

    The first gives the step time: K calls back to back, no per-call events,
    bracketed by device synchronisation and read on the host clock.  The second
    repeats the K calls with the library's HIP events around the main kernel of
    every call, on its stream, for the kernel's mean duration.  An event between
    two dependent kernels holds the stream for about 5 us, so events in the
    first pass would slow the short decode steps by several percent.
    ``events`` False: the second pass is skipped (counter passes).  ``reset``
    detaches the events from the library afterwards."""
    import torch
    print("bench: timing %d steps of %s" % (K, name), file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    if not events:
        return ms_per_step, np.zeros(0)
    ev = [(hip.event(), hip.event()) for _ in range(K)]
    print("bench: %d more steps of %s with kernel events" % (K, name), file=sys.stderr, flush=True)
    try:
        for i in range(K):
            step(i, ev[i])
    finally:
        reset()
    torch.cuda.synchronize()
    kern_ms = np.array([hip.elapsed_ms(a, b) for a, b in ev])
    for a, b in ev:
        hip.destroy(a)
        hip.destroy(b)
    return ms_per_step, kern_ms


def time_workload(fa, W, hip, dev, stream, name, K, warmup, events, dtype="bf16", alibi=False, seed=None):
    """Time K calls of one workload; returns the measurements and the algorithmic work.

    ``events`` False: no HIP events (counter passes; their warm-up is the same)."""
    import torch
    print("bench: generating %s" % name, file=sys.stderr, flush=True)
    wl = W.make_config(name, seed, dtype=dtype)
    work = work_of(wl)
    decode = name in DECODE
    # enough input copies that consecutive steps do not hit in the 256 MB MALL
    per_copy = (wl.k.numel() + wl.v.numel() + 2 * wl.q.numel()) * 2
    ncopies = int(min(8, max(1, math.ceil(2.0e9 / per_copy))))
    with torch.cuda.stream(stream):
        copies = []
        for _ in range(ncopies):
            d = dict(q=wl.q.to(dev), k=wl.k.to(dev), v=wl.v.to(dev),
                     cu_q=torch.from_numpy(wl.cu_seqlens_q).to(dev),
                     cu_k=torch.from_numpy(wl.cu_seqlens_k).to(dev),
                     bt=None if wl.block_table is None else torch.from_numpy(wl.block_table).to(dev))
            d["out"] = torch.empty_like(d["q"])
            copies.append(d)
        torch.cuda.synchronize()
    calls = []
    ws_bytes = 0
    for d in copies:
        dq, dk, dv, do = fa._tdesc(d["q"]), fa._tdesc(d["k"]), fa._tdesc(d["v"]), fa._tdesc(d["out"])
        dbt = fa._tdesc(d["bt"]) if d["bt"] is not None else None
        ws_bytes = fa.fa_varlen_workspace_bytes(dq, dk, dv, wl.batch, dbt, wl.page_block_size)
        calls.append((dq, dk, dv, do, dbt, d))
    workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    sh = stream.cuda_stream
    alibi_t = torch.from_numpy(W.alibi_slopes(wl.num_heads)).to(dev) if alibi else None
    dal = fa._tdesc(alibi_t) if alibi_t is not None else None

    def step(i, ev_k=None):
        dq, dk, dv, do, dbt, d = calls[i % ncopies]
        if ev_k is not None:
            fa.fa_varlen_set_kernel_events(ev_k[0], ev_k[1])
        rc = fa.fa_varlen_fwd(dq, dk, dv, do, d["cu_q"].data_ptr(), d["cu_k"].data_ptr(), wl.batch,
                              dbt, wl.page_block_size, wl.softmax_scale, wl.window_left,
                              wl.window_right, 0, workspace.data_ptr() if ws_bytes else 0,
                              ws_bytes, sh, dal)
        if rc:
            raise RuntimeError(fa.fa_last_error())

    warm = warm_up(step, warmup)
    ms_per_step, kern_ms = timed_passes(step, K, hip, events, name, lambda: fa.fa_varlen_set_kernel_events(0, 0))
    warm_ms = None
    if events and decode and ncopies > 1:
        # for reference only: the same K steps on one input copy, whose K/V may then
        # be served partly from the 256 MB last-level cache
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            step(0)
        torch.cuda.synchronize()
        warm_ms = (time.perf_counter() - t0) * 1e3 / K
    graph_ms = None
    if events and name == "c1":
        # the latency workload once more without per-call host work: 32 calls
        # captured in one HIP graph (a call enqueues kernels only), the graph
        # replayed 10 times; one graph launch costs tens of microseconds of host
        # time, which 32 calls amortise
        G, R = 32, 10
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(G):
                step(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(R):
            g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / (R * G)
        del g
    del copies, calls, workspace, alibi_t
    torch.cuda.empty_cache()
    return dict(wl=wl, work=work, decode=decode, ms_per_step=ms_per_step, kern_ms=kern_ms,
                ncopies=ncopies, ws_bytes=ws_bytes, warmup_run=warm, warm_ms=warm_ms, graph_ms=graph_ms)


def summarize(t):
    """Throughput and both roofline fractions of one timed workload."""
    work, decode = t["work"], t["decode"]
    kern = float(t["kern_ms"].mean()) if t["kern_ms"].size else float("nan")
    call = t["ms_per_step"]
    if decode:
        per_step = work["kv_bytes"] / (t["ms_per_step"] * 1e-3) / 1e9
        ach = work["total_bytes"] / (kern * 1e-3) / 1e9
        ach_call = work["total_bytes"] / (call * 1e-3) / 1e9
        peak, unit, bound = PEAK_HBM_GBS, "GB/s", "hbm"
        value_unit = "GB/s"
    else:
        per_step = work["flops"] / (t["ms_per_step"] * 1e-3) / 1e12
        ach = work["flops"] / (kern * 1e-3) / 1e12
        ach_call = work["flops"] / (call * 1e-3) / 1e12
        peak, unit, bound = PEAK_BF16_TFLOPS, "TFLOP/s", "mfma"
        value_unit = "TFLOP/s"
    return dict(value=round(per_step, 3), unit=value_unit, ms_per_step=round(t["ms_per_step"], 5),
                kernel_ms_mean=round(kern, 5), bound=bound,
                achieved=round(ach, 2), achieved_call=round(ach_call, 2), peak=peak, roof_unit=unit,
                frac=round(ach / peak, 4), frac_call=round(ach_call / peak, 4),
                kernel_ms_p10_p50_p90=[round(float(x), 5) for x in np.percentile(t["kern_ms"], [10, 50, 90])]
                if t["kern_ms"].size else None,
                warm_cache_ms_per_step=round(t["warm_ms"], 5) if t.get("warm_ms") else None,
                graph_replay_ms_per_step=round(t["graph_ms"], 5) if t.get("graph_ms") else None,
                kernel_event_steps=int(t["kern_ms"].size), warmup_steps_run=t["warmup_run"])


def workload_config(wl, name, alibi):
    return {"workload": "%s: %s" % (name, wl.extra.get("desc", "")), "batch": wl.batch,
            "total_q": int(wl.lens_q.sum()), "total_k": int(wl.lens_k.sum()), "num_heads": wl.num_heads,
            "num_heads_k": wl.num_heads_k, "head_dim": wl.head_dim, "page_block_size": wl.page_block_size,
            "window_left": wl.window_left, "window_right": wl.window_right, "alibi": bool(alibi),
            "parallelism": "single GPU"}


# ---------------------------------------------------------------------- main

HEADLINE = "c4"
SUITE = ["c2", "c3", "c5a", "c5b", "c1"]  # c1 (86 tokens): a latency figure, its step time


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    help="c1..c5b: time one forward workload (default: the headline c4 plus the suite); "
                         "append: c2..c5b (default c2); padded: p2/p4 (default p4)")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "f16"],
                    help="element type of q/k/v/out (and the append's rows and pools)")
    ap.add_argument("--alibi", action="store_true",
                    help="forward and padded: add ALiBi (geometric slopes 2^(-8h/H), one per head)")
    ap.add_argument("--op", default="fwd", choices=["fwd", "append", "padded"],
                    help="fwd: the attention forward (default); append: the paged K/V append; "
                         "padded: the batch-major entry")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-counters", action="store_true",
                    help="skip the rocprofv3 counter passes of the default run")
    ap.add_argument("--counters", action="store_true",
                    help="run the counter passes for --workload too (the default run always does, "
                         "for the headline workload)")
    ap.add_argument("--counters-dir", default=None,
                    help="where the counter passes write their files (default: a new temporary folder)")
    ap.add_argument("--counter-child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--counters-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                            "COPY_WRITE_CSV"),
                    help="print the HBM-traffic summary of rocprofv3 --pmc runs and exit")
    args = ap.parse_args(argv)
    suite = (args.op == "fwd" and args.workload is None and not args.counter_child
             and not args.copy_calibration and not args.counters_summary)
    if args.workload is None:
        args.workload = {"padded": "p4", "append": "c2"}.get(args.op, HEADLINE)
    valid = ["p2", "p4"] if args.op == "padded" else ["c1", "c2", "c3", "c4", "c5a", "c5b"]
    if args.workload not in valid:
        ap.error("--op %s takes --workload in %s" % (args.op, valid))
    if args.counters_summary:
        print(counters_summary(args.workload, *args.counters_summary, copy_mib=1024, op=args.op), end="")
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this path runs on one GPU only; --gpus %d is not supported "
              "(no multi-GPU sharding is built)" % args.gpus, file=sys.stderr, flush=True)
        return 2

    # counter passes first, as child processes, before this process touches the GPU
    raw_counters = None
    counters_dir = None
    # never nested: a process that already runs under rocprofv3 has its GPU
    # initialised by the profiler's library, and its children must not exec
    under_profiler = any(k.startswith("ROCPROF_") for k in os.environ)
    want_counters = (suite or args.counters) and args.op == "fwd" and not args.no_counters
    if want_counters and under_profiler:
        print("bench: running under rocprofv3, counter passes skipped", file=sys.stderr, flush=True)
    if (want_counters and not under_profiler and not args.counter_child and not args.copy_calibration
            and os.environ.get("FA_BENCH_CHILD") != "1"):
        import tempfile
        # import torch here (no GPU initialisation yet) so the children find it in
        # the page cache: the first import on a fresh machine can take minutes
        print("bench: importing torch", file=sys.stderr, flush=True)
        import torch  # noqa: F401
        counters_dir = args.counters_dir
        if counters_dir is None:
            counters_dir = tempfile.mkdtemp(prefix="fa_bench_counters_")
        raw_counters = run_counter_passes(args.workload, args.dtype, counters_dir)

    import torch
    import varlen_flash_attention_fa_amd as fa
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)
        return 0

    fa.load()
    hip = Hip()
    if args.counter_child:
        return counter_child(args, fa, W, hip, dev, stream)
    if args.op == "append":
        return bench_append(args, fa, W, hip, dev, stream)
    if args.op == "padded":
        return bench_padded(args, fa, W, hip, dev, stream)

    props = torch.cuda.get_device_properties(dev)
    head = time_workload(fa, W, hip, dev, stream, args.workload, args.steps, args.warmup, True,
                         args.dtype, args.alibi, args.seed)
    hs = summarize(head)
    wl, work = head["wl"], head["work"]

    counters = None
    if raw_counters is not None:
        counters = derive_counters(raw_counters, "attn_fwd_kernel", work["flops"], work["total_bytes"],
                                   props.multi_processor_count)
        if counters_dir:
            with open(os.path.join(counters_dir, "summary.md"), "w") as f:
                f.write(counters_markdown(counters, raw_counters, args.workload, args.dtype,
                                          " ".join(["python3", "bench.py"] + list(sys.argv[1:] if argv is None
                                                                                  else argv))))
    traffic = None
    if counters and "hbm_bytes" in counters:
        traffic = counters["hbm_bytes"]
    elif not suite:
        traffic = stored_traffic(args.workload, "fwd", args.dtype, args.alibi)
    roof = {"bound": hs["bound"], "achieved": hs["achieved"], "peak": hs["peak"], "unit": hs["roof_unit"],
            "frac": hs["frac"], "traffic": traffic, "achieved_call": hs["achieved_call"],
            "frac_call": hs["frac_call"],
            "mfma_util_counters": counters.get("mfma_util") if counters else None}

    suite_out = {}
    if suite:
        for name in SUITE:
            t = time_workload(fa, W, hip, dev, stream, name, args.steps, args.warmup, True,
                              args.dtype, args.alibi, args.seed)
            s = summarize(t)
            s["config"] = workload_config(t["wl"], name, args.alibi)
            s["algorithmic_flop"] = t["work"]["flops"]
            s["algorithmic_total_bytes"] = t["work"]["total_bytes"]
            s["algorithmic_kv_bytes"] = t["work"]["kv_bytes"]
            suite_out[name] = s
            del t

    cpu = None
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, work, head["decode"], W.alibi_slopes(wl.num_heads) if args.alibi else None)

    line = {
        "metric": METRIC,
        "value": hs["value"],
        "unit": hs["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": hs["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic (seeded N(0,1) %s, seed %d)" % (args.dtype, wl.seed),
        "config": workload_config(wl, args.workload, args.alibi),
        "roofline": roof,
        "cpu_baseline": cpu,
        "suite": suite_out or None,
        "counters": counters,
        "detail": {
            "main_kernel_ms_mean": hs["kernel_ms_mean"],
            "kernel_event_steps": hs["kernel_event_steps"], "warmup_steps_run": head["warmup_run"],
            "kernel_ms_p10_p50_p90": hs["kernel_ms_p10_p50_p90"],
            "warm_cache_ms_per_step": hs["warm_cache_ms_per_step"],
            "graph_replay_ms_per_step": hs["graph_replay_ms_per_step"],
            "algorithmic_flop": work["flops"], "algorithmic_kv_bytes": work["kv_bytes"],
            "algorithmic_total_bytes": work["total_bytes"], "visible_pairs_per_head": work["pairs"],
            "tflops_per_step": round(work["flops"] / (head["ms_per_step"] * 1e-3) / 1e12, 3),
            "kv_gbs_per_step": round(work["kv_bytes"] / (head["ms_per_step"] * 1e-3) / 1e9, 2),
            "input_copies_rotated": head["ncopies"], "workspace_bytes": head["ws_bytes"],
            "kernel_source_sha256_16": kernel_sha(), "device": props.name,
            "cus": props.multi_processor_count,
        },
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
