"""Attention throughput on one MI355X: TFLOP/s (causal-adjusted) and % of MFMA peak.

One step = one fp8 forward pass over the largest single-GPU workload: block-
quantised e4m3 Q/K/V with one fp32 scale per 128-row block, B=1, H=32,
N=32768, d=128, causal, bf16 output, inputs resident in HBM.  FLOPs follow
the standard count: 4*B*H*N^2*d per forward, halved exactly when causal
(2.5x that for a backward).  W untimed warm-up steps, then exactly K steps
between two device synchronisations; `value` is the step's FLOPs over the
mean step time, and the per-launch median, p10 and p90 come from HIP events
on the launching stream.

The JSON line also carries:
  roofline      the dominant kernel's algorithmic TFLOP/s (FLOPs per launch over
                its mean launch time from those HIP events) against the dense
                MFMA peak of its dtype, and its HBM traffic per launch from the
                committed rocprofv3 counter summary when that summary was taken
                on the current kernel sources (else null);
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same
                workload's inputs (sampled heads and row blocks) on this host's
                cores, with both the causal-adjusted and the dense FLOP rate;
  kernel_check  the kernel names of the committed rocprofv3 trace summary of
                the headline workload, checked against the library's kernels;
  extra         the other workloads, each with its median (p10, p90) over 20
                repetitions after 3 warm-ups; short forwards and every backward
                start each repetition with cold caches (a 512 MiB write between
                repetitions flushes L2 and MALL), the long forwards (inputs
                larger than MALL) run back to back: the causal bf16 d=128
                forward at N >= 8192 (with the >= 50% target stated), the five
                stated problems (fp32, bf16 d=64/256, GQA prefill, training
                forward + backward), the backward at d=256 and GQA, padded /
                sliding-window / block-sparse forwards, and the KV-cache
                (decode) forward as the rate it reads the cache at, against
                the 8 TB/s HBM peak.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2516.6, "fp8": 5033.2, "f32": 157.3}   # dense MFMA, 256 CU x 2.4 GHz
HBM_GBS = 8000.0
HEADLINE = "C5"
TARGET_SHAPES = ["Ta", "Ta_gqa", "Tb", "Tc"]       # causal bf16, N >= 8192, d = 128
TARGET_FRAC = 0.5                                  # of the dense bf16 MFMA peak
EXTRA_FWD = TARGET_SHAPES + ["C1", "C2a", "C2a_nc", "C2b", "C3"]
FLUSH_BYTES = 512 << 20                            # > the 256 MB MALL + 8 x 4 MB L2
# Forward cases short enough (and with inputs small enough) for L2/MALL to
# carry data from one repetition to the next: these, and every backward, are
# timed with a 512 MiB write between repetitions.  The long forwards (the
# T-shapes, C5, W1, S1: >= 1.9 ms over >= 384 MiB of inputs, more than MALL
# holds) are timed back to back.
SHORT_FWD = {"C1", "C2a", "C2a_nc", "C2b", "C3", "P1", "D1", "D1_ragged"}
REPS, WARMUP = 20, 3                               # per extra workload and direction
EXTRA_KV = ["D1", "D1_ragged"]
EXTRA_MASKED = ["W1", "P1"]
EXTRA_BLOCKSPARSE = ["S1"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "exact_tiled_attention_amd", "csrc", f)
                  for f in ("fa_fwd.hip", "fa_bwd.hip", "fa_kvcache.hip", "fa_common.hpp")]


def source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--only", default=None, help="time one workload alone (profiling runs)")
    ap.add_argument("--with-bwd", action="store_true", help="with --only: also run the backward")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run a plain 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--check-trace", default=None, metavar="CSV",
                    help="check a rocprofv3 kernel_stats.csv of a bench run (with --only W, or the "
                         "headline) against the library's kernel names and exit")
    ap.add_argument("--summary-out", default=None, metavar="MD",
                    help="with --check-trace: also write the trace summary (markdown) here")
    ap.add_argument("--summary-cmd", default="", help="the command that produced the trace (for the summary)")
    ap.add_argument("--traffic", nargs=4, default=None,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter_collection.csv of a --only W run "
                         "and of a --copy-probe run: write W's HBM bytes per launch into profiles/traffic.json")
    ap.add_argument("--counter-summary", nargs="+", default=None, metavar="W=DIR",
                    help="summarise rocprofv3 --kernel-trace --pmc runs (one output directory per workload W, "
                         "SQ/GRBM counters) into a markdown table (--summary-out) and exit")
    return ap.parse_args()


class Case:
    """Device-resident inputs of one workload and a launcher for its kernels."""

    def __init__(self, name, dev, backward=False, keep_cpu=False):
        import torch
        import synthetic as syn
        self.w = syn.WORKLOADS[name]
        x = syn.make_inputs(self.w, with_do=backward)
        self.x = x if keep_cpu else None        # CPU copies (the oracle's inputs)
        self.scale = x["scale"]
        self.q, self.k, self.v = (x[n].to(dev) for n in ("q", "k", "v"))
        self.sc = {}
        if x["q_scale"] is not None:
            self.sc = dict(q_descale=x["q_scale"].to(dev), k_descale=x["k_scale"].to(dev),
                           v_descale=x["v_scale"].to(dev))
        B, H, N, d = self.w.B, self.w.H, self.w.N, self.w.d
        odt = torch.float32 if self.w.dtype == "f32" else torch.bfloat16
        self.o = torch.empty(B, H, N, d, device=dev, dtype=odt)
        self.lse = torch.empty(B, H, N, device=dev, dtype=torch.float32)
        self.backward = backward
        if backward:
            import exact_tiled_attention_amd as fa
            self.do = x["do"].to(dev)
            self.dq = torch.empty_like(self.q)
            self.dk = torch.empty_like(self.k)
            self.dv = torch.empty_like(self.v)
            need = fa.fa_bwd_workspace_bytes(B, H, self.w.H_kv, N, d, 1)
            self.ws = torch.empty(need, device=dev, dtype=torch.uint8)

    def fwd(self):
        import exact_tiled_attention_amd as fa
        fa.fa_fwd(self.q, self.k, self.v, causal=self.w.causal, scale=self.scale,
                  out=self.o, lse=self.lse, **self.sc)

    def bwd(self):
        import exact_tiled_attention_amd as fa
        fa.fa_bwd(self.q, self.k, self.v, self.o, self.lse, self.do, causal=self.w.causal,
                  scale=self.scale, workspace=self.ws, dq=self.dq, dk=self.dk, dv=self.dv)


class KvCase:
    """Device-resident query, caches and workspace of one decode workload."""

    def __init__(self, name, dev):
        import torch
        import synthetic as syn
        import exact_tiled_attention_amd as fa
        self.w = w = syn.KV_WORKLOADS[name]
        x = syn.make_kvcache_inputs(w)
        self.lens = x["lens"]
        self.scale = x["scale"]
        self.q, self.k, self.v = (x[n].to(dev) for n in ("q", "k", "v"))
        self.kv_len = x["kv_len"].to(dev) if x["kv_len"] is not None else None
        self.o = torch.empty(w.B, w.H, w.N_q, w.d, device=dev, dtype=torch.bfloat16)
        self.lse = torch.empty(w.B, w.H, w.N_q, device=dev, dtype=torch.float32)
        need = fa.fa_fwd_kvcache_workspace_bytes(w.B, w.H, w.H_kv, w.N_q, w.N_kv, w.d, 1)
        self.ws = torch.empty(need, device=dev, dtype=torch.uint8)

    def fwd(self):
        import exact_tiled_attention_amd as fa
        fa.fa_fwd_kvcache(self.q, self.k, self.v, self.kv_len, causal=self.w.causal, scale=self.scale,
                          out=self.o, lse=self.lse, workspace=self.ws)

    def report(self, st):
        ms = st["ms"]
        gbs = self.w.cache_bytes(self.lens) / (ms * 1e-3) / 1e9
        return {"kernel": f"kvcache_bf16_d{self.w.d}", **st,
                "cache_GBps": round(gbs, 1), "frac_hbm": round(gbs / HBM_GBS, 4),
                "cache_bytes": self.w.cache_bytes(self.lens),
                "tflops": round(self.w.flops(self.lens) / (ms * 1e-3) / 1e12, 3)}


class MaskedCase:
    """Device-resident inputs of one padded / sliding-window workload."""

    def __init__(self, name, dev):
        import torch
        import synthetic as syn
        self.w = w = syn.MASKED_WORKLOADS[name]
        x = syn.make_masked_inputs(w)
        self.lens = x["lens"]
        self.scale = x["scale"]
        self.q, self.k, self.v = (x[n].to(dev) for n in ("q", "k", "v"))
        self.seqlens = x["seqlens"].to(dev) if x["seqlens"] is not None else None
        self.o = torch.empty(w.B, w.H, w.N, w.d, device=dev, dtype=torch.bfloat16)
        self.lse = torch.empty(w.B, w.H, w.N, device=dev, dtype=torch.float32)

    def fwd(self):
        import exact_tiled_attention_amd as fa
        fa.fa_fwd_masked(self.q, self.k, self.v, self.seqlens, self.w.window, causal=self.w.causal,
                         scale=self.scale, out=self.o, lse=self.lse)

    def report(self, st):
        tf = self.w.flops_fwd(self.lens) / (st["ms"] * 1e-3) / 1e12
        return {"kernel": f"fwd_bf16_d{self.w.d}_masked", **st, "tflops": round(tf, 2),
                "frac_peak": round(tf / PEAK_TFLOPS["bf16"], 4), "window": self.w.window,
                "valid_rows": int(sum(self.lens))}

    def bwd_report(self, dev):
        """Time the backward (dQ, dK, dV) of the same masked problem."""
        import torch
        import exact_tiled_attention_amd as fa
        g = torch.Generator().manual_seed(self.w.seed + 1000)
        do = torch.randn(self.o.shape, generator=g).to(torch.bfloat16).to(dev)
        self.fwd()
        ws = torch.empty(fa.fa_bwd_workspace_bytes(self.w.B, self.w.H, self.w.H_kv, self.w.N, self.w.d, 1),
                         device=dev, dtype=torch.uint8)
        dq, dk, dv = torch.empty_like(self.q), torch.empty_like(self.k), torch.empty_like(self.v)
        fn = lambda: fa.fa_bwd_masked(self.q, self.k, self.v, self.o, self.lse, do, self.seqlens, self.w.window,
                                      causal=self.w.causal, scale=self.scale, workspace=ws, dq=dq, dk=dk, dv=dv)
        st = stats(time_launches(fn, reps=REPS, warmup=WARMUP, flush=True))
        tf = 2.5 * self.w.flops_fwd(self.lens) / (st["ms"] * 1e-3) / 1e12
        return {"kernel": f"bwd_bf16_d{self.w.d}_masked", **st, "tflops": round(tf, 2),
                "frac_peak": round(tf / PEAK_TFLOPS["bf16"], 4)}


class BlockSparseCase:
    """Device-resident inputs and block mask of one block-sparse workload."""

    def __init__(self, name, dev):
        import torch
        import synthetic as syn
        self.w = w = syn.BLOCKSPARSE_WORKLOADS[name]
        x = syn.make_blocksparse_inputs(w)
        self.bm_cpu = x["block_mask"]
        self.scale = x["scale"]
        self.q, self.k, self.v = (x[n].to(dev) for n in ("q", "k", "v"))
        self.bm = x["block_mask"].to(dev)
        self.o = torch.empty(w.B, w.H, w.N, w.d, device=dev, dtype=torch.bfloat16)
        self.lse = torch.empty(w.B, w.H, w.N, device=dev, dtype=torch.float32)

    def fwd(self):
        import exact_tiled_attention_amd as fa
        fa.fa_fwd_blocksparse(self.q, self.k, self.v, self.bm, causal=self.w.causal, scale=self.scale,
                              out=self.o, lse=self.lse)

    def report(self, st):
        tf = self.w.flops_fwd(self.bm_cpu) / (st["ms"] * 1e-3) / 1e12
        return {"kernel": f"fwd_bf16_d{self.w.d}_blocksparse", **st, "tflops": round(tf, 2),
                "frac_peak": round(tf / PEAK_TFLOPS["bf16"], 4), "block_density": self.w.density}

    def bwd_report(self, dev):
        """Time the backward (dQ, dK, dV) of the same block-sparse problem."""
        import torch
        import exact_tiled_attention_amd as fa
        g = torch.Generator().manual_seed(self.w.seed + 1000)
        do = torch.randn(self.o.shape, generator=g).to(torch.bfloat16).to(dev)
        self.fwd()
        ws = torch.empty(fa.fa_bwd_workspace_bytes(self.w.B, self.w.H, self.w.H_kv, self.w.N, self.w.d, 1),
                         device=dev, dtype=torch.uint8)
        dq, dk, dv = torch.empty_like(self.q), torch.empty_like(self.k), torch.empty_like(self.v)
        fn = lambda: fa.fa_bwd_blocksparse(self.q, self.k, self.v, self.o, self.lse, do, self.bm,
                                           causal=self.w.causal, scale=self.scale, workspace=ws,
                                           dq=dq, dk=dk, dv=dv)
        st = stats(time_launches(fn, reps=REPS, warmup=WARMUP, flush=True))
        tf = 2.5 * self.w.flops_fwd(self.bm_cpu) / (st["ms"] * 1e-3) / 1e12
        return {"kernel": f"bwd_bf16_d{self.w.d}_blocksparse", **st, "tflops": round(tf, 2),
                "frac_peak": round(tf / PEAK_TFLOPS["bf16"], 4)}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def syn_workload(name):
    import synthetic as syn
    return syn.WORKLOADS[name]


def kernel_name(w, direction="fwd"):
    if direction == "bwd":
        return f"bwd_bf16_d{w.d}_{'causal' if w.causal else 'full'}"
    return f"fwd_{w.dtype}_d{w.d}_{'causal' if w.causal else 'full'}"


# The library's kernels (the names rocprofv3 shows, without template
# arguments), and the kernel that dominates each workload's forward in the
# instance table of fa_fwd.hip / fa_bwd.hip.
LIB_KERNELS = ("fwd_bf16_kernel", "fwd_bf16_sp_kernel", "fwd_bf16_pp_kernel", "fwd_fp8_pp_kernel",
               "fwd_bf16_pairs_kernel", "fwd_f32_kernel", "bwd_prep_kernel", "bwd_dkdv_kernel",
               "bwd_dq_kernel", "bwd_dq_pair_kernel", "kv_split_kernel", "kv_combine_kernel")
DOMINANT = {"C5": "fa::fwd_fp8_pp_kernel<128, true", "Ta": "fa::fwd_bf16_pp_kernel<128, true",
            "Ta_gqa": "fa::fwd_bf16_pp_kernel<128, true", "Tb": "fa::fwd_bf16_pp_kernel<128, true",
            "Tc": "fa::fwd_bf16_pp_kernel<128, true", "C3": "fa::fwd_bf16_pp_kernel<128, true",
            "C2a": "fa::fwd_bf16_sp_kernel<64, true, true>", "C2a_nc": "fa::fwd_bf16_pp_kernel<64, false",
            "C2b": "fa::fwd_bf16_pairs_kernel<256, true", "C1": "fa::fwd_f32_kernel<64, true",
            "C4": "fa::fwd_bf16_sp_kernel<64, true, false>"}
HEADLINE_SUMMARY = os.path.join(ROOT, "profiles", "fwd_fp8_d128_causal_C5.md")


def time_launches(fn, reps, warmup, flush=False):
    """Per-launch durations (ms) from HIP events on the launching stream.  With
    flush, a 512 MiB device write runs between repetitions (outside the
    events), so every timed launch starts with L2 and MALL holding none of
    its data."""
    import torch
    for _ in range(warmup):
        fn()
    st = torch.cuda.current_stream()
    buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=torch.device("cuda", torch.cuda.current_device())) \
        if flush else None
    out = []
    for i in range(reps):
        if buf is not None:
            buf.fill_(i & 0xFF)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        fn()
        b.record(st)
        out.append((a, b))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in out]


def median(xs):
    s = sorted(xs)
    n = len(s)
    return s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])


def quantile(xs, q):
    """Linear-interpolated quantile of a sample."""
    s = sorted(xs)
    if len(s) == 1:
        return s[0]
    pos = q * (len(s) - 1)
    lo = int(math.floor(pos))
    hi = min(lo + 1, len(s) - 1)
    return s[lo] + (s[hi] - s[lo]) * (pos - lo)


def stats(xs):
    """Median (the reported time), p10 and p90 of per-launch times in ms."""
    return {"ms": round(median(xs), 4), "ms_p10": round(quantile(xs, 0.1), 4),
            "ms_p90": round(quantile(xs, 0.9), 4), "reps": len(xs)}


def load_traffic():
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return {}
    if t.get("source_hash") != source_hash():
        return {}
    return t.get("kernels", {})


def cpu_baseline(x, w, budget_s=20.0):
    """The oracle on a bounded sample of the headline workload's own inputs:
    row blocks of 256 query rows at seeded positions in seeded heads, each
    row against every key (the oracle forms whole rows of scores, masks them
    and takes the row softmax).  Reported as TFLOP/s with the metric's count
    (4 d per visible (query, key) pair), plus the dense rate (4 d per query
    and key: what the oracle actually computes)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    rng = np.random.default_rng(w.seed)
    rb = 256
    n_blocks = (w.N + rb - 1) // rb
    vis = dense = 0.0
    heads, blocks = set(), 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        b, h = int(rng.integers(w.B)), int(rng.integers(w.H))
        blk = int(rng.integers(n_blocks))
        rows = np.arange(blk * rb, min(w.N, (blk + 1) * rb))
        kv = oracle.kv_head_of(h, w.H, w.H_kv)
        oracle.forward_rows(x["q_64"][b, h], x["k_64"][b, kv], x["v_64"][b, kv], x["scale"], w.causal, rows)
        vis += float(np.sum(4.0 * w.d * ((rows + 1) if w.causal else np.full(rows.size, w.N))))
        dense += 4.0 * w.d * rows.size * w.N
        heads.add((b, h))
        blocks += 1
    dt = time.perf_counter() - t0
    return {"value": vis / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "dense_tflops": dense / dt / 1e12,
            "sample": f"fp64 numpy oracle on the {w.name} inputs (dequantised fp8 values, as the kernel "
                      f"sees them): {blocks} blocks of {rb} query rows at seeded positions in "
                      f"{len(heads)} of {w.B * w.H} heads, {dt:.1f} s; value counts 4*d per visible "
                      f"(query, key) pair as the metric does ({vis / 1e12:.2f} TFLOP), dense_tflops "
                      f"4*d per (query, key) pair the oracle computes ({dense / 1e12:.2f} TFLOP)"}


def read_summary(path):
    """(kernel, calls, average us) rows of a committed rocprofv3 trace summary."""
    rows = []
    try:
        with open(path) as f:
            for line in f:
                if line.startswith("| `"):
                    cells = [c.strip() for c in line.strip().strip("|").split("|")]
                    rows.append((cells[0].strip("`"), int(cells[1]), float(cells[2])))
    except OSError:
        return []
    return rows


def base_name(kernel):
    """'void fa::fwd_bf16_pp_kernel<...>(fa::FwdParams)' -> 'fwd_bf16_pp_kernel'."""
    k = kernel.split("(")[0].split("<")[0].split()[-1]
    return k.split("::")[-1]


def check_kernels(rows, workload):
    """The trace's kernels: every fa:: kernel must be one of the library's,
    and the forward kernel with the most time must be the one the instance
    table picks for the workload (a run with the backward also shows its
    kernels).  Returns a dict with ok and the reasons."""
    want = DOMINANT.get(workload)
    ours = [r for r in rows if "fa::" in r[0]]
    problems = []
    if not ours:
        problems.append("no fa:: kernel in the trace")
    for r in ours:
        if base_name(r[0]) not in LIB_KERNELS:
            problems.append(f"unknown kernel {r[0]}")
    fwd = [r for r in ours if base_name(r[0]).startswith(("fwd_", "kv_"))] or ours
    top = max(fwd, key=lambda r: r[1] * r[2]) if fwd else None
    if want and top and want not in top[0]:
        problems.append(f"dominant forward kernel {top[0]} is not {want}")
    return {"ok": not problems, "expected": want, "dominant": top[0] if top else None,
            "dominant_avg_us": top[2] if top else None, "problems": problems}


def parse_kernel_stats(path):
    """(kernel, calls, average us) rows of a rocprofv3 kernel_stats.csv."""
    import csv
    rows = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            rows.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e3))
    return rows


def write_summary(rows, path, workload, cmd):
    """Markdown summary of a kernel trace: per kernel, calls and durations."""
    import synthetic as syn
    tot = sum(c * a for _, c, a in rows) or 1.0
    w = syn.WORKLOADS.get(workload) or syn.KV_WORKLOADS.get(workload) or \
        syn.MASKED_WORKLOADS.get(workload) or syn.BLOCKSPARSE_WORKLOADS.get(workload)
    what = (f"B={w.B}, H={w.H}, H_kv={w.H_kv}, N={getattr(w, 'N', None) or getattr(w, 'N_kv', None)}, "
            f"d={w.d}, {w.dtype}, {'causal' if w.causal else 'non-causal'}")
    lines = [f"# Kernel trace: {workload} ({what})", "",
             f"command (from the repository root): {cmd}", "",
             "| kernel | calls | average (us) | share of kernel time |", "|---|---|---|---|"]
    for name, calls, avg in sorted(rows, key=lambda r: -r[1] * r[2]):
        lines.append(f"| `{name}` | {calls} | {avg:.1f} | {100.0 * calls * avg / tot:.1f}% |")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def counter_rows(path):
    """(kernel, counter value) per dispatch of a rocprofv3 counter_collection.csv."""
    import csv
    with open(path, newline="") as f:
        return [(r["Kernel_Name"], float(r["Counter_Value"])) for r in csv.DictReader(f)]


SQ_PASS = ("SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_VALU", "SQ_INSTS_MFMA",
           "SQ_INSTS_VALU_TRANS_F32", "SQ_VALU_MFMA_COEXEC_CYCLES", "GRBM_GUI_ACTIVE")
LDS_PASS = ("SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES",
            "SQ_WAIT_ANY", "SQ_ACTIVE_INST_ANY", "GRBM_GUI_ACTIVE")
N_SIMD, N_XCD = 1024, 8


def counter_table(directory):
    """Per kernel of one rocprofv3 --kernel-trace --pmc run (its output directory):
    dispatches, median duration (us) and the median of each counter per dispatch."""
    import csv
    import glob
    import statistics
    cfiles = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    tfiles = glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True)
    dur = {}
    for tf in tfiles:
        with open(tf, newline="") as f:
            for r in csv.DictReader(f):
                dur[(tf, r["Dispatch_Id"])] = (r["Kernel_Name"], (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    per = {}
    for cf in cfiles:
        with open(cf, newline="") as f:
            for r in csv.DictReader(f):
                d = per.setdefault(r["Kernel_Name"], {}).setdefault(r["Dispatch_Id"], {})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    out = {}
    for k, disp in per.items():
        us = [v[1] for v in dur.values() if v[0] == k]
        names = sorted({c for d in disp.values() for c in d})
        out[k] = {"dispatches": len(disp), "us": statistics.median(us) if us else float("nan"),
                  **{c: statistics.median([d.get(c, 0.0) for d in disp.values()]) for c in names}}
    return out


def counter_summary_rows(tables):
    """Derived figures per (workload, kernel) from counter_table results."""
    rows = []
    for wname, tab in tables:
        for k, c in sorted(tab.items(), key=lambda kv: -kv[1]["us"] * kv[1]["dispatches"]):
            if not any(n in k for n in LIB_KERNELS):
                continue
            cyc = c.get("GRBM_GUI_ACTIVE", 0.0) / N_XCD
            r = {"workload": wname, "kernel": k.replace("void ", "").split("(")[0], "us": c["us"],
                 "clock_ghz": cyc / (c["us"] * 1e3) if c["us"] >= 20 and cyc else None}
            if "SQ_INSTS_MFMA" in c and cyc:
                mf = c["SQ_INSTS_MFMA"]
                r.update(mfma_busy=c["SQ_VALU_MFMA_BUSY_CYCLES"] / N_SIMD / cyc,
                         coexec=c["SQ_VALU_MFMA_COEXEC_CYCLES"] / N_SIMD / cyc,
                         mfma_insts=mf, valu_insts=c["SQ_INSTS_VALU"] - mf, exp_insts=c["SQ_INSTS_VALU_TRANS_F32"],
                         trans_share=c["SQ_INSTS_VALU_TRANS_F32"] * 16 / N_SIMD / cyc)
            if "SQ_INSTS_LDS" in c and cyc:
                r.update(lds_insts=c["SQ_INSTS_LDS"],
                         lds_conflict=c["SQ_LDS_BANK_CONFLICT"] / max(1.0, c["SQ_ACTIVE_INST_LDS"]),
                         lds_wait=c["SQ_WAIT_INST_LDS"] / max(1.0, c["SQ_WAVE_CYCLES"]),
                         any_wait=c["SQ_WAIT_ANY"] / max(1.0, c["SQ_WAVE_CYCLES"]))
            rows.append(r)
    return rows


def _placeholder(run):
    """'W=some/path/W_sq' -> 'W=<dir>/W_sq' (the summary names the run, not where it was written)."""
    w, _, d = run.partition("=")
    return f"{w}=<dir>/{os.path.basename(os.path.normpath(d))}"


def write_counter_summary(rows, path, runs):
    f3 = lambda v, fmt: "—" if v is None else fmt.format(v)
    lines = ["# Matrix-pipe use, instruction mix and LDS waits per kernel (rocprofv3 counters)", "",
             "commands (from the repository root), one run per workload W and counter pass:", "",
             "    rocprofv3 --kernel-trace --pmc " + " ".join(SQ_PASS) + " -d <dir>/W_sq -o c --output-format csv -- "
             "python3 bench.py --only W --steps 2 --warmup 0 --no-cpu-baseline --no-extra [--with-bwd]",
             "    rocprofv3 --kernel-trace --pmc " + " ".join(LDS_PASS) + " -d <dir>/W_lds (the same program, some W)",
             "    python3 bench.py --counter-summary " + " ".join(_placeholder(r) for r in runs) + " --summary-out <this file>", "",
             "How the columns are formed: kernel cycles = GRBM_GUI_ACTIVE / 8 (the counter sums the 8 XCDs); "
             "clock = kernel cycles / duration (not shown under 20 us); MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / "
             "1024 SIMDs / kernel cycles; co-issue = SQ_VALU_MFMA_COEXEC_CYCLES / 1024 / kernel cycles; "
             "instruction counts are totals over all waves (SQ_INSTS_VALU includes the MFMAs, subtracted here); "
             "exp share = SQ_INSTS_VALU_TRANS_F32 x 16 cycles (a quarter-rate wave64 op) / 1024 / kernel cycles, "
             "the fraction of every SIMD's time its transcendentals alone would take; LDS conflict = "
             "SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS; LDS wait and any wait = SQ_WAIT_INST_LDS and SQ_WAIT_ANY "
             "over SQ_WAVE_CYCLES (per-wave fractions). Durations are medians of the counter runs' kernel "
             "traces (collection slows kernels slightly).", "",
             "| workload | kernel | us | clock (GHz) | MFMA busy | MFMA+VALU co-issue | MFMA insts | other VALU insts "
             "| exp insts | exp share | LDS insts | LDS conflict | LDS wait | any wait |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {r['workload']} | `{r['kernel']}` | {r['us']:.1f} | {f3(r['clock_ghz'], '{:.2f}')} | "
                     f"{f3(r.get('mfma_busy'), '{:.1%}')} | {f3(r.get('coexec'), '{:.1%}')} | "
                     f"{f3(r.get('mfma_insts'), '{:.3g}')} | {f3(r.get('valu_insts'), '{:.3g}')} | "
                     f"{f3(r.get('exp_insts'), '{:.3g}')} | {f3(r.get('trans_share'), '{:.1%}')} | "
                     f"{f3(r.get('lds_insts'), '{:.3g}')} | {f3(r.get('lds_conflict'), '{:.1%}')} | "
                     f"{f3(r.get('lds_wait'), '{:.1%}')} | {f3(r.get('any_wait'), '{:.1%}')} |")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def compulsory_bytes(w):
    """Bytes a forward must move at least: Q, K, V (and fp8 scales) read once, O and LSE written once."""
    elt = {"f32": 4, "bf16": 2, "fp8": 1}[w.dtype]
    q = w.B * w.H * w.N * w.d * elt
    kv = 2 * w.B * w.H_kv * w.N * w.d * elt
    sc = 0 if w.dtype != "fp8" else 4 * ((w.N + 127) // 128) * (w.B * w.H + 2 * w.B * w.H_kv)
    out = w.B * w.H * w.N * w.d * (4 if w.dtype == "f32" else 2) + 4 * w.B * w.H * w.N
    return q + kv + sc, out


def traffic_entry(args):
    """HBM bytes per launch of a workload's dominant kernel from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by what the same counter reads
    for a plain 1 GiB device copy (which reads and writes 2^30 bytes)."""
    fetch, write, cfetch, cwrite = (counter_rows(p) for p in args.traffic)
    w = syn_workload(args.only)
    want = DOMINANT[args.only]
    avg = lambda rows: sum(v for k, v in rows if want in k) / max(1, sum(1 for k, _ in rows if want in k))
    cavg = lambda rows: sum(v for k, v in rows if "copyBuffer" in k) / max(1, sum(1 for k, _ in rows if "copyBuffer" in k))
    ff, wf = (1 << 30) / (cavg(cfetch) * 1024), (1 << 30) / (cavg(cwrite) * 1024)
    rd, wr = avg(fetch) * 1024 * ff, avg(write) * 1024 * wf
    comp_r, comp_w = compulsory_bytes(w)
    return {"workload": args.only, "kernel": want, "fetch_kib": avg(fetch), "write_kib": avg(write),
            "fetch_factor": ff, "write_factor": wf, "read_bytes": rd, "write_bytes": wr,
            "bytes_per_launch": rd + wr, "compulsory_read_bytes": comp_r, "compulsory_write_bytes": comp_w,
            "read_over_compulsory": rd / comp_r}


def main():
    args = parse()
    if args.counter_summary:
        tables = {}
        for spec in args.counter_summary:          # several passes of one workload merge per kernel
            wname, _, d = spec.partition("=")
            for k, c in counter_table(d).items():
                tables.setdefault(wname, {}).setdefault(k, {}).update({n: v for n, v in c.items()
                                                                       if n not in tables[wname].get(k, {})})
        rows = counter_summary_rows(list(tables.items()))
        if args.summary_out:
            write_counter_summary(rows, args.summary_out, args.counter_summary)
        print(json.dumps(rows))
        return
    if args.check_trace:
        rows = parse_kernel_stats(args.check_trace)
        res = check_kernels(rows, args.only or HEADLINE)
        if args.summary_out:
            write_summary(rows, args.summary_out, args.only or HEADLINE, args.summary_cmd)
        print(json.dumps({"trace": args.check_trace, "workload": args.only or HEADLINE, **res}))
        sys.exit(0 if res["ok"] else 1)
    if args.traffic:
        ent = traffic_entry(args)
        try:
            with open(TRAFFIC_FILE) as f:
                t = json.load(f)
        except (OSError, ValueError):
            t = {}
        if t.get("source_hash") != source_hash():
            t = {"source_hash": source_hash(), "kernels": {}}
        t["kernels"][kernel_name(syn_workload(args.only))] = ent
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(t, f, indent=1)
        if args.summary_out:
            mib = 1 << 20
            with open(args.summary_out, "w") as f:
                f.write(f"# HBM traffic per launch: {args.only}, `{ent['kernel']}...>`\n\n"
                        f"commands (from the repository root), one counter per run:\n\n"
                        f"    rocprofv3 --pmc FETCH_SIZE -d <dir> -o c --output-format csv -- python3 bench.py "
                        f"--only {args.only} --steps 2 --warmup 0 --no-cpu-baseline --no-extra\n"
                        f"    rocprofv3 --pmc WRITE_SIZE (the same program)\n"
                        f"    rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE -- python3 bench.py --copy-probe\n"
                        f"    python3 bench.py --only {args.only} --traffic <fetch csv> <write csv> <copy fetch csv> "
                        f"<copy write csv> --summary-out <this file>\n\n"
                        f"Calibration: a 1 GiB device copy reads 2^30 and writes 2^30 bytes; its FETCH_SIZE reads "
                        f"{(1 << 30) / ent['fetch_factor'] / 1024:.0f} KiB and its WRITE_SIZE "
                        f"{(1 << 30) / ent['write_factor'] / 1024:.0f} KiB per dispatch, so bytes = FETCH_SIZE x 1024 x "
                        f"{ent['fetch_factor']:.4f} and WRITE_SIZE x 1024 x {ent['write_factor']:.4f}.\n\n"
                        f"| FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | HBM read (MiB) | HBM write (MiB) | compulsory read (MiB) "
                        f"| compulsory write (MiB) | read / compulsory |\n|---|---|---|---|---|---|---|\n"
                        f"| {ent['fetch_kib']:.0f} | {ent['write_kib']:.0f} | {ent['read_bytes'] / mib:.1f} | "
                        f"{ent['write_bytes'] / mib:.1f} | {ent['compulsory_read_bytes'] / mib:.1f} | "
                        f"{ent['compulsory_write_bytes'] / mib:.1f} | {ent['read_over_compulsory']:.2f} |\n\n"
                        f"Kernel sources hash (bench.py source_hash): {source_hash()}\n")
        print(json.dumps(ent))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    dev = torch.device("cuda:0")
    import exact_tiled_attention_amd as fa
    fa.load_library()

    if args.copy_probe:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 5}))
        return

    import synthetic as syn
    if args.only in syn.KV_WORKLOADS:
        # decode alone (profiling runs): split + combine kernels per call
        c = KvCase(args.only, dev)
        rep = c.report(stats(time_launches(c.fwd, reps=args.steps, warmup=args.warmup, flush=True)))
        log(f"{args.only}: {rep}")
        print(json.dumps({"metric": "KV-cache read rate (GB/s) of the decode forward",
                          "value": rep["cache_GBps"], "unit": "GB/s", "n_gpus": 1,
                          "steps": args.steps, "warmup": args.warmup, "ms_per_step": rep["ms"],
                          "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
                          "config": {"workload": args.only}, "decode": rep}))
        return

    for table, cls in ((syn.BLOCKSPARSE_WORKLOADS, BlockSparseCase), (syn.MASKED_WORKLOADS, MaskedCase)):
        if args.only in table:
            c = cls(args.only, dev)
            rep = c.report(stats(time_launches(c.fwd, reps=args.steps, warmup=args.warmup, flush=True)))
            rep["bwd"] = c.bwd_report(dev)
            log(f"{args.only}: {rep}")
            print(json.dumps({"metric": "attention fwd TFLOP/s (visible pairs) and % of MI355X MFMA peak",
                              "value": rep["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
                              "warmup": args.warmup, "ms_per_step": rep["ms"], "higher_is_better": True,
                              "dtype": "bf16", "data": "synthetic", "config": {"workload": args.only},
                              "detail": rep}))
            return

    name = args.only or HEADLINE
    w0 = syn_workload(name)
    backward = bool(args.only) and (w0.backward or args.with_bwd)
    case = Case(name, dev, backward=backward, keep_cpu=not args.only and not args.no_cpu_baseline)
    step_flops = case.w.flops_fwd() + (case.w.flops_bwd() if backward else 0.0)
    log(f"timing {args.steps} steps of {name} after {args.warmup} warm-up steps")

    for _ in range(args.warmup):
        case.fwd()
        if backward:
            case.bwd()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    ev = {"fwd": [], "bwd": []}
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(st)
    for _ in range(args.steps):
        for direction, fn in (("fwd", case.fwd), ("bwd", case.bwd)):
            if direction == "bwd" and not backward:
                continue
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(st)
            fn()
            b.record(st)
            ev[direction].append((a, b))
    t_end.record(st)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    per = {k: [a.elapsed_time(b) for a, b in v] for k, v in ev.items() if v}
    ms_per_step = total_ms / args.steps
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    log(f"{ms_per_step:.4f} ms per step, {value:.1f} TFLOP/s")

    fwd_ms = sum(per["fwd"]) / len(per["fwd"])
    achieved = case.w.flops_fwd() / (fwd_ms * 1e-3) / 1e12
    tr = load_traffic().get(kernel_name(case.w))
    peak = PEAK_TFLOPS[case.w.dtype]
    roofline = {"bound": "mfma", "kernel": kernel_name(case.w), "workload": name,
                "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "avg_launch_ms": round(fwd_ms, 4),
                "traffic": tr["bytes_per_launch"] if tr else None,
                "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "traffic_detail": tr}
    if case.w.dtype == "fp8":
        # the PV product runs on the bf16 MFMA: 2/3 of the fp8 peak is the most
        # an fp8 QK^T + bf16 PV split can reach
        roofline["note"] = "QK^T on fp8 MFMA, PV on bf16 MFMA"
    timing = {d_: {**stats(v), "tflops": round((case.w.flops_fwd() if d_ == "fwd" else case.w.flops_bwd())
                                               / (median(v) * 1e-3) / 1e12, 2)} for d_, v in per.items()}

    kcheck = None
    if not args.only:
        rows = read_summary(HEADLINE_SUMMARY)
        kcheck = check_kernels(rows, name)
        kcheck["summary"] = os.path.relpath(HEADLINE_SUMMARY, ROOT)
        if kcheck["dominant_avg_us"]:
            kcheck["live_avg_us"] = round(fwd_ms * 1e3, 1)
            kcheck["live_over_summary"] = round(fwd_ms * 1e3 / kcheck["dominant_avg_us"], 3)
        log(f"kernel check: {kcheck}")

    cpu = None
    if not args.only and not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(case.x, case.w)
    del case
    torch.cuda.empty_cache()

    extra = {}
    if not args.no_extra and not args.only:
        for nm in EXTRA_FWD:
            log(f"extra: {nm}")
            c = Case(nm, dev)
            s_ = stats(time_launches(c.fwd, reps=REPS, warmup=WARMUP, flush=nm in SHORT_FWD))
            tf = c.w.flops_fwd() / (s_["ms"] * 1e-3) / 1e12
            extra[nm] = {"kernel": kernel_name(c.w), **s_, "tflops": round(tf, 2),
                         "frac_peak": round(tf / PEAK_TFLOPS[c.w.dtype], 4)}
            del c
            torch.cuda.empty_cache()
        fr = {nm: extra[nm]["frac_peak"] for nm in TARGET_SHAPES}
        extra["target"] = {"what": "causal bf16 forward, N >= 8192, d = 128, fraction of the dense bf16 "
                                   "MFMA peak at every shape", "shapes": fr, "target_min_frac": TARGET_FRAC,
                           "min_frac": min(fr.values()), "met": min(fr.values()) >= TARGET_FRAC}
        for nm in EXTRA_MASKED:
            log(f"extra: {nm}")
            c = MaskedCase(nm, dev)
            extra[nm] = c.report(stats(time_launches(c.fwd, reps=REPS, warmup=WARMUP, flush=nm in SHORT_FWD)))
            if nm == "W1":
                extra[nm + ".bwd"] = c.bwd_report(dev)
            del c
            torch.cuda.empty_cache()
        for nm in EXTRA_BLOCKSPARSE:
            log(f"extra: {nm}")
            c = BlockSparseCase(nm, dev)
            extra[nm] = c.report(stats(time_launches(c.fwd, reps=REPS, warmup=WARMUP, flush=nm in SHORT_FWD)))
            extra[nm]["bwd"] = c.bwd_report(dev)
            del c
            torch.cuda.empty_cache()
        for nm in EXTRA_KV:
            log(f"extra: {nm}")
            c = KvCase(nm, dev)
            extra[nm] = c.report(stats(time_launches(c.fwd, reps=REPS, warmup=WARMUP, flush=True)))
            del c
            torch.cuda.empty_cache()
        for nm in ("C2b", "C3"):
            log(f"extra: {nm} backward")
            c = Case(nm, dev, backward=True)
            c.fwd()
            s_ = stats(time_launches(c.bwd, reps=REPS, warmup=WARMUP, flush=True))
            tf = c.w.flops_bwd() / (s_["ms"] * 1e-3) / 1e12
            extra[nm + ".bwd"] = {"kernel": kernel_name(c.w, "bwd"), **s_, "tflops": round(tf, 2),
                                  "frac_peak": round(tf / PEAK_TFLOPS["bf16"], 4)}
            del c
            torch.cuda.empty_cache()
        log("extra: C4 forward + backward")
        c = Case("C4", dev, backward=True)
        sf = stats(time_launches(c.fwd, reps=REPS, warmup=WARMUP, flush=True))
        sb = stats(time_launches(c.bwd, reps=REPS, warmup=WARMUP, flush=True))
        extra["C4"] = {"fwd": {**sf, "tflops": round(c.w.flops_fwd() / (sf["ms"] * 1e-3) / 1e12, 2)},
                       "bwd": {**sb, "tflops": round(c.w.flops_bwd() / (sb["ms"] * 1e-3) / 1e12, 2)},
                       "fwd_bwd_tflops": round((c.w.flops_fwd() + c.w.flops_bwd())
                                               / ((sf["ms"] + sb["ms"]) * 1e-3) / 1e12, 2),
                       "bwd_frac_peak": round(c.w.flops_bwd() / (sb["ms"] * 1e-3) / 1e12
                                              / PEAK_TFLOPS["bf16"], 4)}
        del c
        torch.cuda.empty_cache()

    w = syn_workload(name)
    out = {
        "metric": "attention fwd/bwd TFLOP/s (causal-adjusted) and % of MI355X MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp8": "fp8_e4m3", "bf16": "bf16", "f32": "f32"}[w.dtype],
        "data": ("synthetic: seeded N(0,1) Q/K/V, block-quantised to OCP e4m3 with one fp32 scale "
                 "per 128-row block" if w.dtype == "fp8" else "synthetic: seeded N(0,1) Q/K/V"),
        "config": {"workload": name, "B": w.B, "H": w.H, "H_kv": w.H_kv, "N": w.N, "d": w.d,
                   "causal": w.causal, "dtype_in": w.dtype, "out": "f32" if w.dtype == "f32" else "bf16",
                   "backward": backward, "timing": timing,
                   "frac_of_peak": round(value / PEAK_TFLOPS[w.dtype], 4), "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernel_check": kcheck,
        "extra": extra,
        "source_hash": source_hash(),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
