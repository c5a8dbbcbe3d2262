"""Host logic of bench.py that needs no GPU: the HBM-traffic record built from two
counter passes, its staleness check against the kernel source, the algorithmic
byte counts and the refusal of more than one GPU."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import synthetic  # noqa: E402

FIELDS = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]


def _write_pass(path, counter, rows):
    os.makedirs(path)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(FIELDS, r[:3] + (counter,) + r[3:])))


def test_traffic_scales_each_counter_by_the_copy(tmp_path):
    mib = 64
    copy_kib = 2 * (mib << 10)  # the counter reads twice the bytes the copy moved: factor 1/2
    # two attention dispatches, each split over two counter instances; the calibration copy
    # at the largest grid; a small input copy of the same kernel that must be ignored
    fetch = [(1, "copyBuffer", 1024, 8.0), (2, "attn_fwd_bf16_kernel<128>", 4096, 300.0),
             (2, "attn_fwd_bf16_kernel<128>", 4096, 100.0), (3, "copyBuffer", 1 << 20, copy_kib),
             (4, "attn_fwd_bf16_kernel<128>", 4096, 500.0), (5, "copyBuffer", 1 << 20, copy_kib)]
    write = [(1, "copyBuffer", 1024, 8.0), (2, "attn_fwd_bf16_kernel<128>", 4096, 40.0),
             (3, "copyBuffer", 1 << 20, copy_kib / 2), (4, "attn_fwd_bf16_kernel<128>", 4096, 60.0)]
    _write_pass(str(tmp_path / "f"), "FETCH_SIZE", fetch)
    _write_pass(str(tmp_path / "w"), "WRITE_SIZE", write)
    rec = bench.write_traffic("wl_test", "attn_fwd_bf16_kernel", "attn_bf16.hip", 1234.0,
                              str(tmp_path / "f"), str(tmp_path / "w"), mib, ["cmd"], dst_dir=str(tmp_path))
    f, w = rec["FETCH_SIZE"], rec["WRITE_SIZE"]
    assert f["kernel_dispatches"] == 2 and f["kernel_kib_per_dispatch"] == 450.0
    assert f["copy_dispatches"] == 2 and f["factor"] == 0.5
    assert f["bytes_per_launch"] == 450.0 * 1024 * 0.5
    assert w["factor"] == 1.0 and w["bytes_per_launch"] == 50.0 * 1024
    assert rec["bytes_per_launch"] == f["bytes_per_launch"] + w["bytes_per_launch"]
    assert rec["algorithmic_bytes_per_launch"] == 1234.0
    assert json.load(open(tmp_path / "traffic_wl_test.json")) == rec


def test_traffic_is_null_when_the_kernel_source_changed(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    csrc = tmp_path / "exact_tiled_attention_18_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f, text in (("attn_bf16.hip", "kernel v1"), ("fa_device.h", "helpers v1"), ("launch.h", "args")):
        (csrc / f).write_text(text)
    (prof / "traffic_wl.json").write_text(json.dumps(
        {"kernel_source_sha": bench.source_sha("attn_bf16.hip"), "bytes_per_launch": 42.0}))
    assert bench.hbm_traffic("wl", "attn_bf16.hip") == 42.0
    (csrc / "fa_device.h").write_text("helpers v2")  # a shared device header counts as the kernel's source
    assert bench.hbm_traffic("wl", "attn_bf16.hip") is None
    assert bench.hbm_traffic("missing", "attn_bf16.hip") is None


def test_algorithmic_bytes():
    w = synthetic.workload("bf16_causal_b4h16n2048d128")
    n = 4 * 16 * 2048 * 128
    assert bench.algorithmic_bytes(w) == 4 * 2 * n + 4 * 4 * 16 * 2048  # Q, K, V read, O written; fp32 LSE
    w8 = synthetic.workload("fp8_causal_b2h16n8192d128_outliers")
    n8 = 2 * 16 * 8192 * 128
    assert bench.algorithmic_bytes(w8) == 3 * n8 + 3 * 4 * 2 * 16 * 64 + 2 * n8 + 4 * 2 * 16 * 8192
    split, merge = bench.split_kv_bytes()
    parts = 8 * 4 * 16 * 16 * 129 * 4
    assert split == 2 * 4 * 16 * 16384 * 128 * 2 + 4 * 16 * 16 * 128 * 2 + parts
    assert merge == parts + 4 * 16 * 16 * (128 * 2 + 4)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2 and "one GPU only" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("flag", [[], ["--split-kv"]])
def test_traffic_from_needs_the_copy_size(tmp_path, flag):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--traffic-from", str(tmp_path),
                        str(tmp_path)] + flag, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0 and "--copy-calibration-mib" in r.stderr


def test_warm_up_runs_at_least_the_steps_and_the_time(monkeypatch):
    # no GPU here: synchronisation is a no-op, and each "step" advances a fake clock
    monkeypatch.setattr(bench.torch.cuda, "synchronize", lambda: None)
    clock = {"t": 0.0}
    monkeypatch.setattr(bench.time, "perf_counter", lambda: clock["t"])
    calls = {"n": 0}

    def step(dt):
        def f():
            calls["n"] += 1
            clock["t"] += dt
        return f

    # long steps: the requested count already covers the minimum time
    n, s = bench.warm_up(step(0.1), 20, 0.5)
    assert n == calls["n"] == 20 and s == pytest.approx(2.0)
    # short steps: the count is topped up, in tens, until the minimum time has passed
    calls["n"] = 0
    clock["t"] = 0.0
    n, s = bench.warm_up(step(1e-4), 20, 0.5)
    assert n == calls["n"] and n >= 5000 and (n - 20) % 10 == 0 and s >= 0.5
    # no minimum time: exactly the requested count
    calls["n"] = 0
    n, _ = bench.warm_up(step(1e-4), 7, 0.0)
    assert n == calls["n"] == 7
