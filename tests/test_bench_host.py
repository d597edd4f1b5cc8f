"""Host-side pieces of bench.py (no GPU): the CPU baseline record the JSON
line carries -- the oracle timed on a bounded, fixed sample of query rows and
extrapolated to the whole forward by useful-pair count."""

import importlib.util
import os

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_cpu_baseline_record():
    bench = load_bench()
    g = torch.Generator().manual_seed(7)
    S, H, D = 512, 2, 16
    x = {n: torch.randn((1, S, H, D), generator=g) for n in ("q", "k", "v")}
    r = bench.cpu_baseline(x, 0.05, block=64, n_blocks=8)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["extrapolated"]
    assert r["value"] > 0 and r["cores"] == len(os.sched_getaffinity(0))
    # The extrapolation is the whole forward's useful flops at the sampled rate.
    full = 4.0 * D * 1 * H * S * (S + 1) / 2
    assert abs(r["extrapolated_full_forward_s"] * r["value"] * 1e12 - full) <= 1e-6 * full
    assert "blocks of 64 consecutive query rows" in r["sample"]
