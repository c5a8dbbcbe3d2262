"""Benchmark: attention forward TFLOP/s on one MI355X and fraction of dense MFMA peak.

One step = one pass of the hot path over one batch of synthetic input:
  * bf16 / fp32 workloads: one fa_fwd launch (query blocks x heads grid,
    K/V tiles through LDS, online softmax, epilogue);
  * the fp8 workload: one quantise+rotate launch for Q, K and V
    (fa_quant_rotate_fp8_qkv) and one fa_fwd_fp8 launch.
Inputs are resident in HBM before the timed region.  FLOPs counted:
4*B*H*N^2*d, halved when causal (masking waste and exps are not counted).

Prints exactly one JSON line on stdout; per-kernel details go to stderr.
The default workload is bf16 causal B=1 H=32 N=16384 d=128, the largest
workload that runs on one GPU; the same line also carries, under "extra",
bf16 causal B=4 H=16 N=2048 d=128 and the fp8 causal B=2 H=16 N=8192 d=128
workload (pre-pass and attention kernel timed apart), each with its own
roofline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import synthetic  # noqa: E402

PEAK_TFLOPS = {"bf16": 2516.6, "fp8": 5033.2, "f32": 157.3}  # MI355X dense, AMD spec
HBM_GBPS = 8000.0
KERNEL_SOURCE = {"bf16": "attn_bf16.hip", "f32": "attn_f32.hip", "fp8": "attn_fp8.hip"}


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(name: str) -> str:
    """Hash of a kernel's source file together with the device headers it includes."""
    h = hashlib.sha256()
    for f in (name, "fa_device.h", "launch.h"):
        h.update(open(os.path.join(ROOT, "exact_tiled_attention_18_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def hbm_traffic(workload: str, kernel_src: str):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary, or None when it is missing or the kernel changed since."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p))
    if rec.get("kernel_source_sha") != source_sha(kernel_src):
        return None
    return rec.get("bytes_per_launch")


def algorithmic_bytes(w) -> float:
    """One read of Q, K, V and one write of O and LSE (fp8: codes + scales + bf16 O)."""
    n = w.B * w.H * w.N * w.d
    lse = 4 * w.B * w.H * w.N
    if w.dtype == "f32":
        return 4 * 4 * n + lse
    if w.dtype == "bf16":
        return 4 * 2 * n + lse
    scales = 3 * 4 * w.B * w.H * ((w.N + 127) // 128)
    return 3 * n + scales + 2 * n + lse


def copy_calibration(fa, mib: int, dev) -> None:
    """The library's plain copy kernel over a known size (mib MiB read, mib MiB
    written), launched a few times so that a counter pass over this program can
    relate FETCH_SIZE / WRITE_SIZE to bytes actually moved."""
    x = torch.ones(mib << 20, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    for _ in range(3):
        fa.fa_calib_copy(x, y)
    torch.cuda.synchronize()
    del x, y


def calibrate(fa, dev) -> dict:
    """What the chip sustains in this process for the resources the kernels are priced
    against: MFMA-only kernels (bf16 and fp8; 3 wavefronts per SIMD, nothing but
    independent MFMAs), a 1 GiB streaming copy and a 1 GiB streaming read, each timed
    with HIP events after 0.2 s of warm-up."""
    def rate(fn, work: float, reps: int) -> float:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.2:
            fn()
            torch.cuda.synchronize()
        return work / time_loop(fn, reps)

    out = {}
    wgs, iters = 3 * 256, 20000  # three 4-wavefront workgroups per compute unit, all resident
    for kind in ("bf16", "fp8"):
        buf = torch.empty(wgs * 256, dtype=torch.float32, device=dev)
        flop = fa.fa_calib_mfma(kind, wgs, iters, out=buf)[1]
        r = rate(lambda k=kind, b=buf: fa.fa_calib_mfma(k, wgs, iters, out=b), flop, 10) / 1e12
        out[f"mfma_{kind}"] = {"tflops": round(r, 1), "frac_of_peak": round(r / PEAK_TFLOPS[kind], 4)}
    x = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    r = rate(lambda: fa.fa_calib_copy(x, y), 2.0 * (1 << 30), 20) / 1e9
    out["copy"] = {"gbs": round(r, 1), "frac_of_peak": round(r / HBM_GBPS, 4), "bytes": 2 * (1 << 30),
                   "note": "1 GiB read + 1 GiB written per launch"}
    del y
    sink = torch.empty(fa.CALIB_READ_OUT_WORDS, dtype=torch.int32, device=dev)
    r = rate(lambda: fa.fa_calib_read(x, out=sink), 1.0 * (1 << 30), 20) / 1e9
    out["read"] = {"gbs": round(r, 1), "frac_of_peak": round(r / HBM_GBPS, 4), "bytes": 1 << 30,
                   "note": "1 GiB read per launch"}
    del x, sink
    eprint("calibration: " + ", ".join(f"{k} {v.get('tflops', v.get('gbs'))}" for k, v in out.items()))
    return out


def _counter_rows(path: str):
    import csv
    if os.path.isdir(path):
        found = [os.path.join(r, f) for r, _, fs in os.walk(path) for f in fs if f.endswith("counter_collection.csv")]
        if len(found) != 1:
            raise SystemExit(f"expected one counter_collection.csv under {path}, found {found}")
        path = found[0]
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def _mean_counter(rows, counter: str, pick) -> tuple[float, int]:
    per_dispatch = {}
    for r in rows:
        if r["Counter_Name"] == counter and pick(r):
            per_dispatch[r["Dispatch_Id"]] = per_dispatch.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per_dispatch:
        raise SystemExit(f"no {counter} rows for the requested kernel")
    return sum(per_dispatch.values()) / len(per_dispatch), len(per_dispatch)


def write_traffic(workload: str, attn_tag: str, src: str, algorithmic: float, fetch_path: str, write_path: str,
                  copy_mib: int, commands: list[str], dst_dir: str | None = None) -> dict:
    """HBM bytes per launch of the kernel named attn_tag from two rocprofv3
    counter passes (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by
    what the same counter reads for the plain copy of copy_mib MiB in the same
    program."""
    is_attn = lambda r: attn_tag in r["Kernel_Name"]  # noqa: E731
    known = float(copy_mib << 20)
    out = {"workload": workload, "kernel": attn_tag,
           "kernel_source_sha": source_sha(src), "copy_bytes": known, "commands": commands}
    total = 0.0
    for counter, path in (("FETCH_SIZE", fetch_path), ("WRITE_SIZE", write_path)):
        rows = _counter_rows(path)
        # the calibration copies: the library's copy kernel (older runs: the runtime's
        # buffer-copy kernel at its largest grid; small copies of that kernel move the
        # inputs of the run)
        tag = "copy16_kernel" if any("copy16_kernel" in r["Kernel_Name"] for r in rows) else "copyBuffer"
        copies = [r for r in rows if tag in r["Kernel_Name"]]
        if not copies:
            raise SystemExit(f"no calibration-copy dispatches in {path}")
        grid = max(int(r["Grid_Size"]) for r in copies)
        is_copy = lambda r, g=grid: tag in r["Kernel_Name"] and int(r["Grid_Size"]) == g  # noqa: E731
        kib, n = _mean_counter(rows, counter, is_attn)
        ckib, cn = _mean_counter(rows, counter, is_copy)
        factor = known / (ckib * 1024.0)
        out[counter] = {"kernel_kib_per_dispatch": kib, "kernel_dispatches": n, "copy_kib_per_dispatch": ckib,
                        "copy_dispatches": cn, "factor": factor, "bytes_per_launch": kib * 1024.0 * factor}
        total += kib * 1024.0 * factor
    out["bytes_per_launch"] = total
    out["algorithmic_bytes_per_launch"] = algorithmic
    dst = os.path.join(dst_dir or os.path.join(ROOT, "profiles"), f"traffic_{workload}.json")
    with open(dst, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    return out


def make_step(fa, w, dev):
    q, k, v, signs = synthetic.workload_inputs(w)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    if w.dtype in ("f32", "bf16"):
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

        def step():
            fa.fa_fwd(q, k, v, causal=w.causal, scale=w.scale, o=o, lse=lse)
        return step, None
    sg = torch.from_numpy(signs).to(dev)
    nt = (w.N + 127) // 128
    q8 = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.uint8, device=dev)
    k8 = torch.empty_like(q8)
    v8t = torch.empty((w.B, w.H, w.d, fa.vt_cols(w.N)), dtype=torch.uint8, device=dev)
    qs, ks, vs = (torch.empty((w.B, w.H, nt), dtype=torch.float32, device=dev) for _ in range(3))
    o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

    def prepass():  # Q, K rotated, V transposed: one launch
        fa.fa_quant_rotate_fp8_qkv(q, k, v, sg, out=(q8, k8, v8t, qs, ks, vs))

    def attn():
        fa.fa_fwd_fp8(q8, k8, v8t, qs, ks, vs, causal=w.causal, scale=w.scale, o=o, lse=lse)

    def step():
        prepass()
        attn()
    return step, (prepass, attn)


def time_loop(fn, iters: int) -> float:
    """Seconds per call of fn, from HIP events on the stream the kernels run on."""
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(iters):
        fn()
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) / 1e3 / iters


def graph_time(fn, iters: int, reps: int = 20) -> float:
    """Seconds per call of fn with `iters` calls captured in one HIP graph and the graph
    replayed `reps` times: the GPU time of back-to-back steps without the host's
    per-launch cost (which bounds the plain loop for microsecond-scale launches)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(iters):
            fn()
    g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        g.replay()
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) / 1e3 / (iters * reps)


def warm_up(fn, steps: int, min_s: float) -> tuple[int, float]:
    """Untimed warm-up: at least `steps` calls of fn, continued until min_s seconds of
    back-to-back work have passed.  The chip raises its clock over tens of
    milliseconds of sustained load (a 20-step warm-up of a 100 us step ends well
    inside that ramp), so timing right after a short warm-up measures the ramp.
    Returns the number of calls made and the seconds they took."""
    t0 = time.perf_counter()
    n = 0
    for _ in range(steps):
        fn()
        n += 1
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < min_s:
        for _ in range(10):
            fn()
        n += 10
        torch.cuda.synchronize()
    return n, time.perf_counter() - t0


def extra_windows(fn, iters: int, n: int) -> list[float]:
    """Seconds per call of fn in n further windows of iters back-to-back calls (after
    the timed region; the reported value stays the timed region's)."""
    return [time_loop(fn, iters) for _ in range(n)]


def cold_cache_time(fn, iters: int, dev) -> float:
    """Median seconds of single calls of fn, each after a 512 MiB write that evicts the
    L2s and the 256 MB MALL, timed with HIP events around the call alone."""
    junk = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    s = torch.cuda.current_stream()
    times = []
    for i in range(iters):
        junk.fill_(i & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        fn()
        e1.record(s)
        e1.synchronize()
        times.append(e0.elapsed_time(e1) / 1e3)
    del junk
    return statistics.median(times)


def host_info() -> dict:
    """The host the oracle runs on: usable cores, BLAS library and threads, RAM."""
    info = {"cores_affinity": len(os.sched_getaffinity(0)), "blas": None, "blas_threads": None, "ram_gib": None}
    try:
        import threadpoolctl
        blas = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            info["blas"] = f"{blas[0].get('internal_api')} {blas[0].get('version')}"
            info["blas_threads"] = int(blas[0].get("num_threads", 1))
    except Exception:  # noqa: BLE001
        pass
    try:
        info["ram_gib"] = round(os.sysconf("SC_PAGE_SIZE") * os.sysconf("SC_PHYS_PAGES") / 2 ** 30, 1)
    except (ValueError, OSError):
        pass
    return info


def cpu_baseline(w, budget_s: float):
    """The fp64 oracle, timed on this host on a bounded sample of the workload's
    heads: whole heads, cycled until budget_s has passed (at least one).  The
    oracle materialises the full N x N score matrix, so it performs 4*N^2*d
    FLOPs per head even when causal; `value` uses the same counted FLOPs as the
    GPU line (halved for causal), `value_full_nxn` the FLOPs the oracle ran."""
    from oracle import attention as A

    hi = host_info()
    q, k, v, _ = synthetic.workload_inputs(w)
    heads = 0
    nbh = w.B * w.H
    t0 = time.perf_counter()
    while heads == 0 or time.perf_counter() - t0 < budget_s:  # cycle over the heads until the budget is spent
        b, h = divmod(heads % nbh, w.H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        A.reference(q[sl], k[sl], v[sl], w.causal, w.scale)
        heads += 1
    dt = time.perf_counter() - t0
    flops = w.flops() * heads / nbh
    full = 4.0 * w.N * w.N * w.d * heads
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": hi["blas_threads"] or 1,
            "kind": "oracle",
            "sample": f"{heads} whole-head evaluations ({heads / nbh:.3f} of the {nbh} heads) of {w.name}, "
                      f"full N x N fp64 oracle, {dt:.1f} s",
            "flop_basis": "counted FLOPs (4*B*H*N^2*d, halved when causal) of the heads evaluated; "
                          "the oracle itself computes the full N x N product",
            "value_full_nxn": round(full / dt / 1e12, 6),
            "cores_affinity": hi["cores_affinity"], "blas": hi["blas"], "blas_threads": hi["blas_threads"],
            "host_ram_gib": hi["ram_gib"], "seconds": round(dt, 2)}


class SclkSampler:
    """Samples the shader clock the driver reports (the starred level of
    pp_dpm_sclk, MHz) from a background thread while the GPU works; None when
    the file is not readable."""

    def __init__(self, period_s: float = 0.02):
        import glob
        import threading
        self.paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.samples: list[float] = []
        self.period = period_s
        self._stop = threading.Event()
        self._t = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        for p in self.paths:
            try:
                for line in open(p).read().splitlines():
                    if line.rstrip().endswith("*"):
                        return float(line.split(":")[1].strip().rstrip("*").strip().lower().rstrip("mhz"))
            except (OSError, ValueError, IndexError):
                continue
        return None

    def _run(self):
        while not self._stop.is_set():
            x = self._read()
            if x is not None:
                self.samples.append(x)
            time.sleep(self.period)

    def __enter__(self):
        if self.paths:
            self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._t.is_alive():
            self._t.join()

    def summary(self):
        if not self.samples:
            return None
        return {"mhz_median": statistics.median(self.samples), "mhz_min": min(self.samples),
                "mhz_max": max(self.samples), "samples": len(self.samples), "source": "pp_dpm_sclk (starred level)"}


def bench_backward(fa, w, dev, args):
    """One step = one fa_bwd call (delta, dQ, dK/dV kernels).  FLOPs counted as
    2.5x the forward's (five matrix products of the same size; the kernels
    recompute S and dP in both passes, which is not counted)."""
    if w.dtype != "bf16":
        raise SystemExit("the backward pass is provided for bf16 workloads")
    q, k, v, _ = synthetic.workload_inputs(w)
    do = synthetic.draw_qkv(w.B, w.H, w.N, w.d, seed=w.seed + 100, dtype="bf16")[0]
    q, k, v, do = (x.to(dev) for x in (q, k, v, do))
    o, lse = fa.fa_fwd(q, k, v, causal=w.causal, scale=w.scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    delta = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

    def step():
        fa.fa_bwd(q, k, v, o, do, lse, causal=w.causal, scale=w.scale, dq=dq, dk=dk, dv=dv, delta=delta)
    wn, ws = warm_up(step, args.warmup, args.min_warmup_s)
    sec = time_loop(step, args.steps)
    flops = 2.5 * w.flops()
    tflops = flops / sec / 1e12
    peak = PEAK_TFLOPS["bf16"]
    eprint(f"{w.name} backward: {sec * 1e6:.1f} us = {tflops:.1f} TFLOP/s = {tflops / peak:.1%} of {peak}")
    rec = {"metric": "attention bwd TFLOP/s at 1 MI355X (2.5x forward FLOPs)", "value": round(tflops, 2),
           "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": wn,
           "warmup_requested": args.warmup, "warmup_s": round(ws, 3),
           "ms_per_step": round(sec * 1e3, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic",
           "config": {"workload": w.name, "pass": "backward", "flops_per_step": flops},
           "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                        "frac": round(tflops / peak, 4), "traffic": None},
           "cpu_baseline": None}
    print(json.dumps(rec), flush=True)


DEFAULT_WORKLOAD = "bf16_causal_b1h32n16384d128"
EXTRA_WORKLOADS = ("bf16_causal_b4h16n2048d128", "fp8_causal_b2h16n8192d128_outliers")

DECODE = {"B": 4, "H": 16, "Nq": 16, "Nk": 16384, "d": 128, "n_splits": 8, "seed": 1200}


def split_kv_name() -> str:
    c = DECODE
    return f"split_kv_decode_b{c['B']}h{c['H']}nq{c['Nq']}nk{c['Nk']}d{c['d']}x{c['n_splits']}"


def split_kv_bytes() -> tuple[int, int]:
    """Algorithmic HBM bytes of the split launch (K and V once, Q once, the fp32
    partial outputs and LSEs written once) and of the merge (partials read once,
    O and LSE written once)."""
    c = DECODE
    B, H, Nq, Nk, d, n = c["B"], c["H"], c["Nq"], c["Nk"], c["d"], c["n_splits"]
    parts = n * B * H * Nq * (d + 1) * 4
    return 2 * B * H * Nk * d * 2 + B * H * Nq * d * 2 + parts, parts + B * H * Nq * (d * 2 + 4)


def bench_split_kv(fa, dev, args):
    """One step = a decode-shaped split-KV forward: the last Nq positions of a
    causal sequence of Nk keys, the keys cut into n_splits ranges, one
    fa_fwd_split launch for all ranges and one fa_merge.  The work is bound by
    reading K and V once (the scores are a few GFLOP), so the roofline is HBM;
    value counts the bytes of both launches over the step, the roofline those of
    the split launch (the dominant kernel) over its own time."""
    c = DECODE
    B, H, Nq, Nk, d, n = c["B"], c["H"], c["Nq"], c["Nk"], c["d"], c["n_splits"]
    q = synthetic.draw_qkv(B, H, Nq, d, seed=c["seed"], dtype="bf16")[0].to(dev)
    _, k, v = synthetic.draw_qkv(B, H, Nk, d, seed=c["seed"] + 1, dtype="bf16")
    k, v = k.to(dev), v.to(dev)
    o_parts = torch.empty((n, B, H, Nq, d), dtype=torch.float32, device=dev)
    lse_parts = torch.empty((n, B, H, Nq), dtype=torch.float32, device=dev)
    o = torch.empty((B, H, Nq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    scale = d ** -0.5

    def split():
        fa.fa_fwd_split(q, k, v, n, Nk - Nq, 0, Nk, True, scale, o_parts=o_parts, lse_parts=lse_parts)

    def merge():
        fa.fa_merge(o_parts, lse_parts, torch.bfloat16, o=o, lse=lse)

    def step():
        split()
        merge()
    wn, ws = warm_up(step, args.warmup, args.min_warmup_s)
    sec = time_loop(step, args.steps)
    k_sec = time_loop(split, args.steps)
    # the merge alone is shorter than one host call; its share is the step minus the split launch
    m_sec = sec - k_sec
    split_bytes, merge_bytes = split_kv_bytes()
    nbytes = split_bytes + merge_bytes
    gbs = nbytes / sec / 1e9
    k_gbs = split_bytes / k_sec / 1e9
    eprint(f"split-KV decode B{B} H{H} Nq{Nq} Nk{Nk} d{d} x{n}: step {sec * 1e6:.1f} us = {gbs:.0f} GB/s "
           f"= {gbs / HBM_GBPS:.1%} of {HBM_GBPS:.0f} GB/s; split launch {k_sec * 1e6:.1f} us = {k_gbs:.0f} GB/s "
           f"= {k_gbs / HBM_GBPS:.1%}; merge (step minus split launch) {m_sec * 1e6:.1f} us")
    rec = {"metric": "split-KV decode GB/s (K, V read once) at 1 MI355X", "value": round(gbs, 1), "unit": "GB/s",
           "n_gpus": 1, "steps": args.steps, "warmup": wn, "warmup_requested": args.warmup,
           "warmup_s": round(ws, 3), "ms_per_step": round(sec * 1e3, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": split_kv_name(), "causal": True, "bytes_per_step": nbytes},
           "roofline": {"bound": "hbm", "achieved": round(k_gbs, 1), "peak": HBM_GBPS, "unit": "GB/s",
                        "frac": round(k_gbs / HBM_GBPS, 4), "traffic": hbm_traffic(split_kv_name(), "attn_bf16.hip")},
           "cpu_baseline": None}
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20, help="untimed warm-up steps (at least)")
    ap.add_argument("--min-warmup-s", type=float, default=0.5,
                    help="keep warming up until this many seconds of back-to-back steps have run "
                         "(the clock ramps up under sustained load); 'warmup' in the output is the count run")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    choices=[w.name for w in synthetic.WORKLOADS])
    ap.add_argument("--no-extras", dest="extras", action="store_false",
                    help="with the default workload, do not add the N = 2048 and fp8 workloads under 'extra'")
    ap.add_argument("--extra-warmup-s", type=float, default=0.3,
                    help="minimum warm-up seconds of each extra workload")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--windows", type=int, default=5,
                    help="after the timed region, this many more windows of --steps steps (median and best reported)")
    ap.add_argument("--cold-cache", action="store_true",
                    help="also time single steps after a 512 MiB write that evicts L2 and MALL (forward workloads)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (fa_bwd) of a bf16 workload instead of the forward")
    ap.add_argument("--split-kv", action="store_true",
                    help="time a decode-shaped split-KV forward (one fa_fwd_split launch + fa_merge)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the steps replayed from a HIP graph (launch-bound workloads)")
    ap.add_argument("--no-calibration", dest="calibrate", action="store_false",
                    help="skip the MFMA-only and copy calibration kernels")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run a plain copy of this many MiB (for counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: turn two rocprofv3 --pmc outputs into profiles/traffic_<workload>.json")
    ap.add_argument("--traffic-command", action="append", default=[],
                    help="with --traffic-from: the profiler command lines, recorded in the JSON")
    args = ap.parse_args()
    if args.traffic_from:
        if args.copy_calibration_mib <= 0:
            raise SystemExit("--traffic-from needs --copy-calibration-mib (the size the counter runs copied)")
        if args.split_kv:
            name, tag, src, alg = split_kv_name(), "attn_decode_bf16_kernel", "attn_bf16.hip", split_kv_bytes()[0]
        else:
            w = synthetic.workload(args.workload)
            name, src, alg = w.name, KERNEL_SOURCE[w.dtype], algorithmic_bytes(w)
            tag = {"bf16": "attn_fwd_bf16_kernel", "f32": "attn_fwd_f32_kernel", "fp8": "attn_fwd_fp8_kernel"}[w.dtype]
        rec = write_traffic(name, tag, src, alg, *args.traffic_from, args.copy_calibration_mib, args.traffic_command)
        print(json.dumps(rec), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path shards heads and "
              "batches across GPUs with no exchange, so run it per GPU", file=sys.stderr)
        sys.exit(2)

    import exact_tiled_attention_18_amd as fa

    fa.load_library()
    dev = "cuda:0"
    w = synthetic.workload(args.workload)
    if args.copy_calibration_mib > 0:
        copy_calibration(fa, args.copy_calibration_mib, dev)
    if args.split_kv:
        bench_split_kv(fa, dev, args)
        return
    if args.backward:
        return bench_backward(fa, w, dev, args)
    with SclkSampler() as sclk:
        main_m = measure_forward(fa, w, dev, args.steps, args.warmup, args.min_warmup_s, args.windows,
                                 args.cold_cache, args.graph)
        extra = {}
        if args.extras and w.name == DEFAULT_WORKLOAD:
            for name in EXTRA_WORKLOADS:
                ew = synthetic.workload(name)
                m = measure_forward(fa, ew, dev, args.steps, args.warmup, args.extra_warmup_s, 0, False)
                extra[name] = forward_record(ew, m)
        calib = calibrate(fa, dev) if args.calibrate else None
    r = forward_record(w, main_m)
    if calib:
        for rr, ww in [(r, w)] + [(extra[n], synthetic.workload(n)) for n in extra]:
            sus = calib[f"mfma_{'fp8' if ww.dtype == 'fp8' else 'bf16'}"]["tflops"] if ww.dtype != "f32" else None
            if sus:
                rr["roofline"]["frac_of_sustained_mfma"] = round(rr["roofline"]["achieved"] / sus, 4)
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, args.cpu_budget)
    rec = {
        "metric": "attention fwd TFLOP/s at 1 MI355X and % of dense MFMA peak (bf16, fp8)",
        "value": r["value"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": main_m["warmup"], "warmup_requested": args.warmup, "warmup_s": main_m["warmup_s"],
        "ms_per_step": r["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": r["config"], "frac_of_peak": r["frac_of_peak"], "wall_s_timed": main_m["wall_s"],
        "windows": r["windows"], "cold_cache": r["cold_cache"], "graph": r.get("graph"),
        "roofline": r["roofline"], "cpu_baseline": cpu,
        "sclk": sclk.summary(),
        "calibration": calib,
        "extra": extra or None,
    }
    print(json.dumps(rec), flush=True)


def measure_forward(fa, w, dev, steps: int, warmup: int, min_warmup_s: float, windows: int, cold: bool,
                    graph: bool = False) -> dict:
    """Times `steps` back-to-back steps of a forward workload after the warm-up,
    then the attention kernel alone (and, for fp8, the pre-pass alone)."""
    step, parts = make_step(fa, w, dev)
    wn, ws = warm_up(step, warmup, min_warmup_s)
    t0 = time.perf_counter()
    sec = time_loop(step, steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    wins = sorted(extra_windows(step, steps, windows)) if windows > 0 else []
    cold_s = cold_cache_time(step, min(steps, 50), dev) if cold else None
    graph_s = graph_time(step, min(steps, 100)) if graph else None
    pre_sec = None
    if parts is None:
        k_sec = sec
    else:
        prepass, attn = parts
        pre_sec = time_loop(prepass, steps)
        k_sec = time_loop(attn, steps)
    return {"sec": sec, "k_sec": k_sec, "pre_sec": pre_sec, "wins": wins, "cold": cold_s, "graph": graph_s,
            "warmup": wn,
            "warmup_s": round(ws, 3), "wall_s": round(wall, 4), "steps": steps}


def forward_record(w, m: dict) -> dict:
    """The figures of one forward workload: step throughput, the attention kernel's
    roofline (and the fp8 pre-pass against HBM)."""
    sec, k_sec = m["sec"], m["k_sec"]
    tflops = w.flops() / sec / 1e12
    k_tflops = w.flops() / k_sec / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    eprint(f"{w.name}: step {sec * 1e6:.1f} us ({tflops:.1f} TFLOP/s); attention kernel {k_sec * 1e6:.1f} us "
           f"= {k_tflops:.1f} TFLOP/s = {k_tflops / peak:.1%} of {peak} TFLOP/s; algorithmic HBM "
           f"{algorithmic_bytes(w) / k_sec / 1e9:.0f} GB/s")
    rec = {"value": round(tflops, 2), "unit": "TFLOP/s", "ms_per_step": round(sec * 1e3, 5), "steps": m["steps"],
           "warmup": m["warmup"], "dtype": w.dtype,
           "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                      "scale": "1/sqrt(d)", "flops_per_step": w.flops()},
           "frac_of_peak": round(tflops / peak, 4),
           "roofline": {"bound": "mfma", "achieved": round(k_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                        "frac": round(k_tflops / peak, 4), "traffic": hbm_traffic(w.name, KERNEL_SOURCE[w.dtype]),
                        "kernel_ms": round(k_sec * 1e3, 5),
                        "algorithmic_bytes": algorithmic_bytes(w)},
           "windows": None, "cold_cache": None}
    wins = m["wins"]
    if wins:
        rec["windows"] = {
            "count": len(wins), "steps_each": m["steps"],
            "ms_per_step_median": round(statistics.median(wins) * 1e3, 5), "ms_per_step_best": round(wins[0] * 1e3, 5),
            "value_median": round(w.flops() / statistics.median(wins) / 1e12, 2),
            "value_best": round(w.flops() / wins[0] / 1e12, 2)}
    if m.get("graph") is not None:
        gs = m["graph"]
        eprint(f"{w.name}: graph replay {gs * 1e6:.2f} us per step ({w.flops() / gs / 1e12:.2f} TFLOP/s)")
        rec["graph"] = {"ms_per_step": round(gs * 1e3, 6), "value": round(w.flops() / gs / 1e12, 3),
                        "note": "min(steps, 100) steps captured in one HIP graph, replayed 20 times"}
    if m["cold"] is not None:
        rec["cold_cache"] = {"ms_per_step_median": round(m["cold"] * 1e3, 5),
                             "value": round(w.flops() / m["cold"] / 1e12, 2),
                             "note": "single launches, each after a 512 MiB write that evicts L2 and MALL"}
    if m["pre_sec"] is not None:
        pre_sec = m["pre_sec"]
        pre_bytes = 3 * (2 + 1) * w.B * w.H * w.N * w.d + 3 * 4 * w.B * w.H * ((w.N + 127) // 128)
        eprint(f"fp8 pre-pass: {pre_sec * 1e6:.1f} us for 3 tensors, {pre_bytes / pre_sec / 1e9:.0f} GB/s "
               f"({pre_bytes / pre_sec / 1e9 / HBM_GBPS:.1%} of 8 TB/s)")
        rec["prepass"] = {"ms": round(pre_sec * 1e3, 5), "bytes": pre_bytes,
                          "roofline": {"bound": "hbm", "achieved": round(pre_bytes / pre_sec / 1e9, 1),
                                       "peak": HBM_GBPS, "unit": "GB/s",
                                       "frac": round(pre_bytes / pre_sec / 1e9 / HBM_GBPS, 4)}}
    return rec


if __name__ == "__main__":
    main()
