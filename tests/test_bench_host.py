"""Host-side logic of bench.py, no GPU: the roofline block of each measured
workload, the traffic lookup tied to the kernel sources it was counted on,
the warm-up floor, and the CPU baseline's token sample."""
import json
import os
import sys
import time

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from speculative_decoding_draft_02_amd import workloads as W  # noqa: E402


def test_hbm_roofline_entry():
    r = {"GB_s": 6000.0, "kernel_us_avg": 25.0, "bytes_per_call": 150e6}
    e = bench.roofline_entry("prefill_bf16", r)
    assert (e["bound"], e["peak"], e["unit"]) == ("hbm", 8000.0, "GB/s")
    assert e["achieved"] == 6000.0
    assert e["frac"] == pytest.approx(0.75)
    assert e["kernel"] == bench.KERNELS["prefill_bf16"]
    assert e["kernel_us_avg"] == 25.0
    assert e["algorithmic_bytes_per_launch"] == 150e6


def test_kernel_rate_wins_over_step_rate():
    # the graph-replayed workloads carry both; the kernel's own rate is the
    # one the roofline compares with the peak
    e = bench.roofline_entry("decode_bf16", {"GB_s": 1500.0, "kernel_GB_s": 2000.0,
                                             "us_per_call": 3.0})
    assert e["achieved"] == 2000.0 and e["frac"] == pytest.approx(0.25)
    assert e["kernel_us_avg"] == 3.0


def test_mfma_roofline_entry():
    r = {"project_write_TFLOP_s": 1250.0, "project_write_us": 412.0, "gemm_flops": 515e9}
    e = bench.roofline_entry("project_prefill_bf16", r)
    assert (e["bound"], e["peak"], e["unit"]) == ("mfma", 2500.0, "TFLOP/s")
    assert e["frac"] == pytest.approx(0.5)
    assert e["traffic"] is None
    assert e["kernel_us_avg"] == 412.0 and e["algorithmic_flops_per_launch"] == 515e9
    assert e["kernel"] == bench.KERNELS["project_prefill_bf16"]


def test_no_roofline_without_a_rate():
    assert bench.roofline_entry("prefill_bf16", {}) is None


def test_every_reported_workload_names_its_kernel():
    reported = (W.NAMES[1:] + ["prefill_bf16_layer_slots", "prefill_bf16_tp4_shard"]
                + W.PROJECT_NAMES[1:] + W.INSERT_NAMES[1:])
    assert set(reported) <= set(bench.KERNELS)


def test_traffic_only_for_the_sources_it_was_counted_on(monkeypatch, tmp_path):
    (tmp_path / "profiles").mkdir()
    rec = {"kernel_source_hash": "0123456789abcdef", "bytes_per_launch": 165116271.9}
    (tmp_path / "profiles" / "traffic_prefill_bf16.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0123456789abcdef")
    assert bench.traffic_for("prefill_bf16") == rec["bytes_per_launch"]
    assert bench.traffic_for("prefill_fp8") is None          # never counted
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "fedcba9876543210")
    assert bench.traffic_for("prefill_bf16") is None         # sources changed since


def test_source_hash_follows_the_kernel_sources(monkeypatch, tmp_path):
    for p in bench.KERNEL_SOURCES:
        f = tmp_path / p
        f.parent.mkdir(parents=True, exist_ok=True)
        f.write_text("// " + p)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    (tmp_path / bench.KERNEL_SOURCES[0]).write_text("// changed")
    assert bench.kernel_source_hash() != h0


class _NoSync:
    @staticmethod
    def synchronize():
        pass


def test_warm_up_takes_the_count_or_the_floor(monkeypatch):
    monkeypatch.setattr(bench.torch, "cuda", _NoSync)
    seen = []
    assert bench.warm_up(seen.append, 5, floor_s=0.0) == 5
    assert seen == [0, 1, 2, 3, 4]
    seen.clear()
    t0 = time.perf_counter()
    n = bench.warm_up(seen.append, 0, floor_s=0.05)
    assert time.perf_counter() - t0 >= 0.05
    assert n == len(seen) >= 1 and seen == list(range(n))


def test_cpu_sample_is_a_token_prefix():
    full = W.make(0)
    n = full.num_ctx // 3
    wl = bench.token_prefix(full, n)
    assert wl.num_ctx == n
    assert np.array_equal(wl.all_kv, full.all_kv[:n])
    assert np.array_equal(wl.positions, full.positions[:n])
    assert np.array_equal(wl.slot_mapping, full.slot_mapping[..., :n])
    assert wl.cache_shape == full.cache_shape and wl.num_layers == full.num_layers
    assert 0 < wl.algorithmic_bytes() < full.algorithmic_bytes()
