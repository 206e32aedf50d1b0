"""Attention throughput on one MI355X: TFLOP/s (causal-adjusted) and % of MFMA peak.

One step = one forward pass over every case of the bf16 forward problem
(B=1, H=8, N=8192, d=64, causal and non-causal, plus its d=256 variant at
B=8, H=16, N=2048, causal), inputs resident in HBM.  FLOPs follow the
standard count: 4*B*H*N^2*d per forward, halved exactly when causal.

The JSON line also carries:
  roofline      the dominant kernel's algorithmic TFLOP/s (from HIP events
                around each of its launches inside the timed region) against
                the dense bf16 MFMA peak, and its HBM traffic per launch from
                the committed rocprofv3 counter summary when that summary was
                taken on the current kernel source (else null);
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same
                workload on this host's cores;
  extra         the other kernels measured the same way: the headline-size
                causal bf16 d=128 forward, the fp32 and fp8 forwards, the
                bf16 backward (fwd+bwd) at its full size, and the KV-cache
                (decode) forward as the rate it reads the cache at, against
                the 8 TB/s HBM peak, and the padded / sliding-window forward
                (FLOPs of the visible pairs only).
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
STEP = ["C2a", "C2a_nc", "C2b"]
EXTRA_FWD = ["Ta", "Ta_gqa", "Tb", "Tc", "C1", "C3", "C5"]
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
    return ap.parse_args()


class Case:
    """Device-resident inputs of one workload and a launcher for its kernels."""

    def __init__(self, name, dev, backward=False):
        import torch
        import synthetic as syn
        self.w = syn.WORKLOADS[name]
        x = syn.make_inputs(self.w, with_do=backward)
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

    def report(self, ms):
        gbs = self.w.cache_bytes(self.lens) / (ms * 1e-3) / 1e9
        return {"kernel": f"kvcache_bf16_d{self.w.d}", "ms": round(ms, 4),
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

    def report(self, ms):
        tf = self.w.flops_fwd(self.lens) / (ms * 1e-3) / 1e12
        return {"kernel": f"fwd_bf16_d{self.w.d}_masked", "ms": round(ms, 4), "tflops": round(tf, 2),
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
        ms = median(time_launches(fn, reps=5, warmup=1))
        tf = 2.5 * self.w.flops_fwd(self.lens) / (ms * 1e-3) / 1e12
        return {"kernel": f"bwd_bf16_d{self.w.d}_masked", "ms": round(ms, 4), "tflops": round(tf, 2),
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

    def report(self, ms):
        tf = self.w.flops_fwd(self.bm_cpu) / (ms * 1e-3) / 1e12
        return {"kernel": f"fwd_bf16_d{self.w.d}_blocksparse", "ms": round(ms, 4), "tflops": round(tf, 2),
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
        ms = median(time_launches(fn, reps=5, warmup=1))
        tf = 2.5 * self.w.flops_fwd(self.bm_cpu) / (ms * 1e-3) / 1e12
        return {"kernel": f"bwd_bf16_d{self.w.d}_blocksparse", "ms": round(ms, 4), "tflops": round(tf, 2),
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


def time_launches(fn, reps, warmup):
    """Per-launch durations (ms) from HIP events on the launching stream."""
    import torch
    for _ in range(warmup):
        fn()
    st = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        a.record(st)
        fn()
        b.record(st)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def median(xs):
    s = sorted(xs)
    n = len(s)
    return s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])


def load_traffic():
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return {}
    if t.get("source_hash") != source_hash():
        return {}
    return t.get("kernels", {})


def cpu_baseline(budget_s=20.0):
    """The oracle on a bounded sample: whole rows of the step's workloads."""
    import numpy as np
    import oracle
    import synthetic as syn
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    flops = 0.0
    t_total = 0.0
    done = []
    per_case = budget_s / len(STEP)
    for name in STEP:
        w = syn.WORKLOADS[name]
        x = syn.make_inputs(w, with_do=False)          # the step's own inputs, as the GPU sees them
        rows_done = heads = 0
        t0 = time.perf_counter()
        for b in range(w.B):
            for h in range(w.H):
                if time.perf_counter() - t0 >= per_case:
                    break
                kv = oracle.kv_head_of(h, w.H, w.H_kv)
                rows = np.arange(w.N)
                oracle.forward_rows(x["q_64"][b, h], x["k_64"][b, kv], x["v_64"][b, kv],
                                    x["scale"], w.causal, rows)
                vis = (rows + 1) if w.causal else np.full(rows.size, w.N)
                flops += float(np.sum(4.0 * w.d * vis))
                rows_done += rows.size
                heads += 1
        t_total += time.perf_counter() - t0
        done.append(f"{name}: {heads} of {w.B * w.H} heads")
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": "fp64 numpy oracle over whole heads (all rows, all visible keys) of each step "
                      "workload, heads taken in order until a per-workload time budget; " + "; ".join(done)
                      + f"; {t_total:.1f} s; TFLOP/s counts 4*d per visible (query,key) pair"}


def main():
    args = parse()
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
        xs = time_launches(c.fwd, reps=args.steps, warmup=args.warmup)
        rep = c.report(median(xs))
        log(f"{args.only}: {rep}")
        print(json.dumps({"metric": "KV-cache read rate (GB/s) of the decode forward",
                          "value": rep["cache_GBps"], "unit": "GB/s", "n_gpus": 1,
                          "steps": args.steps, "warmup": args.warmup, "ms_per_step": rep["ms"],
                          "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
                          "config": {"workload": args.only}, "decode": rep}))
        return

    if args.only in syn.BLOCKSPARSE_WORKLOADS:
        c = BlockSparseCase(args.only, dev)
        rep = c.report(median(time_launches(c.fwd, reps=args.steps, warmup=args.warmup)))
        rep["bwd"] = c.bwd_report(dev)
        log(f"{args.only}: {rep}")
        print(json.dumps({"metric": "attention fwd TFLOP/s (visible pairs) and % of MI355X MFMA peak",
                          "value": rep["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
                          "warmup": args.warmup, "ms_per_step": rep["ms"], "higher_is_better": True,
                          "dtype": "bf16", "data": "synthetic", "config": {"workload": args.only},
                          "blocksparse": rep}))
        return

    if args.only in syn.MASKED_WORKLOADS:
        c = MaskedCase(args.only, dev)
        xs = time_launches(c.fwd, reps=args.steps, warmup=args.warmup)
        rep = c.report(median(xs))
        rep["bwd"] = c.bwd_report(dev)
        log(f"{args.only}: {rep}")
        print(json.dumps({"metric": "attention fwd TFLOP/s (visible pairs) and % of MI355X MFMA peak",
                          "value": rep["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
                          "warmup": args.warmup, "ms_per_step": rep["ms"], "higher_is_better": True,
                          "dtype": "bf16", "data": "synthetic", "config": {"workload": args.only},
                          "masked": rep}))
        return

    names = [args.only] if args.only else STEP
    cases = [Case(n, dev, backward=(syn_workload(n).backward or args.with_bwd) and bool(args.only)) for n in names]
    step_flops = sum(c.w.flops_fwd() + (c.w.flops_bwd() if c.backward else 0.0) for c in cases)
    log(f"timing {args.steps} steps of {names} after {args.warmup} warm-up steps")

    for _ in range(args.warmup):
        for c in cases:
            c.fwd()
            if c.backward:
                c.bwd()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    per = {}          # (workload, direction) -> per-launch ms
    ev = []
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(st)
    for _ in range(args.steps):
        for c in cases:
            for direction, fn in (("fwd", c.fwd), ("bwd", c.bwd)):
                if direction == "bwd" and not c.backward:
                    continue
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(st)
                fn()
                b.record(st)
                ev.append(((c.w.name, direction), a, b))
    t_end.record(st)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    for key, a, b in ev:
        per.setdefault(key, []).append(a.elapsed_time(b))
    ms_per_step = total_ms / args.steps
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    log(f"{ms_per_step:.4f} ms per step, {value:.1f} TFLOP/s")

    # dominant kernel: the forward launch with the most time inside the timed region
    by_name = {c.w.name: c for c in cases}
    fwd_keys = [k for k in per if k[1] == "fwd"]
    dom_key = max(fwd_keys, key=lambda k: sum(per[k]))
    dom = by_name[dom_key[0]]
    dom_ms = sum(per[dom_key]) / len(per[dom_key])
    achieved = dom.w.flops_fwd() / (dom_ms * 1e-3) / 1e12
    tr = load_traffic().get(kernel_name(dom.w))
    traffic = tr["bytes_per_launch"] if tr else None
    roofline = {"bound": "mfma", "kernel": kernel_name(dom.w), "workload": dom.w.name,
                "achieved": round(achieved, 2), "peak": PEAK_TFLOPS[dom.w.dtype], "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_TFLOPS[dom.w.dtype], 4),
                "avg_launch_ms": round(dom_ms, 4),
                "traffic": traffic,
                "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "traffic_detail": tr}
    cases_out = {}
    for (name, direction), xs in per.items():
        w = by_name[name].w
        fl = w.flops_fwd() if direction == "fwd" else w.flops_bwd()
        cases_out[f"{name}.{direction}"] = {"ms_median": round(median(xs), 4),
                                            "tflops": round(fl / (median(xs) * 1e-3) / 1e12, 2)}

    extra = {}
    if not args.no_extra and not args.only:
        del cases
        torch.cuda.empty_cache()
        for name in EXTRA_FWD:
            log(f"extra: {name}")
            c = Case(name, dev)
            ms = median(time_launches(c.fwd, reps=10, warmup=2))
            tf = c.w.flops_fwd() / (ms * 1e-3) / 1e12
            extra[name] = {"kernel": kernel_name(c.w), "ms": round(ms, 4), "tflops": round(tf, 2),
                           "frac_peak": round(tf / PEAK_TFLOPS[c.w.dtype], 4)}
            del c
            torch.cuda.empty_cache()
        for name in EXTRA_MASKED:
            log(f"extra: {name}")
            c = MaskedCase(name, dev)
            extra[name] = c.report(median(time_launches(c.fwd, reps=10, warmup=2)))
            if name == "W1":
                extra[name + ".bwd"] = c.bwd_report(dev)
            del c
            torch.cuda.empty_cache()
        for name in EXTRA_BLOCKSPARSE:
            log(f"extra: {name}")
            c = BlockSparseCase(name, dev)
            extra[name] = c.report(median(time_launches(c.fwd, reps=10, warmup=2)))
            extra[name]["bwd"] = c.bwd_report(dev)
            del c
            torch.cuda.empty_cache()
        for name in EXTRA_KV:
            log(f"extra: {name}")
            c = KvCase(name, dev)
            extra[name] = c.report(median(time_launches(c.fwd, reps=20, warmup=3)))
            del c
            torch.cuda.empty_cache()
        for name in ("C2b", "C3"):
            log(f"extra: {name} backward")
            c = Case(name, dev, backward=True)
            c.fwd()
            ms_b = median(time_launches(c.bwd, reps=5, warmup=1))
            tf = c.w.flops_bwd() / (ms_b * 1e-3) / 1e12
            extra[name + ".bwd"] = {"kernel": kernel_name(c.w, "bwd"), "ms": round(ms_b, 4), "tflops": round(tf, 2),
                                    "frac_peak": round(tf / PEAK_TFLOPS["bf16"], 4)}
            del c
            torch.cuda.empty_cache()
        log("extra: C4 forward + backward")
        c = Case("C4", dev, backward=True)
        ms_f = median(time_launches(c.fwd, reps=10, warmup=2))
        ms_b = median(time_launches(c.bwd, reps=10, warmup=2))
        extra["C4"] = {"fwd_ms": round(ms_f, 4), "bwd_ms": round(ms_b, 4),
                       "fwd_tflops": round(c.w.flops_fwd() / (ms_f * 1e-3) / 1e12, 2),
                       "bwd_tflops": round(c.w.flops_bwd() / (ms_b * 1e-3) / 1e12, 2),
                       "fwd_bwd_tflops": round((c.w.flops_fwd() + c.w.flops_bwd())
                                               / ((ms_f + ms_b) * 1e-3) / 1e12, 2),
                       "bwd_frac_peak": round(c.w.flops_bwd() / (ms_b * 1e-3) / 1e12
                                              / PEAK_TFLOPS["bf16"], 4)}
        del c
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline and not args.only:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline()

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
        "dtype": cases[0].w.dtype if args.only else "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V, bf16 RNE)",
        "config": {"workload": "bf16 forward: B=1,H=8,N=8192,d=64 causal + non-causal; "
                               "B=8,H=16,N=2048,d=256 causal" if not args.only else args.only,
                   "cases": cases_out, "frac_of_bf16_peak": round(value / PEAK_TFLOPS["bf16"], 4),
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
        "source_hash": source_hash(),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
