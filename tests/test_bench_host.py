"""Host-side logic of bench.py (no GPU): work counts, traffic record, CLI."""

import importlib.util
import os
import subprocess
import sys

import numpy as np
import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location(
        "bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _pairs_by_mask(lq, lk, causal):
    """Visible (query, key) pairs counted from an explicit 0/1 mask."""
    i = np.arange(lq)[:, None]
    j = np.arange(lk)[None, :]
    mask = np.ones((lq, lk), dtype=bool)
    if causal:
        mask = j <= i + (lk - lq)        # bottom-right aligned
    return int(mask.sum())


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_visible_pairs_match_mask_count(name):
    bench = _bench()
    w = workloads.WORKLOADS[name]
    if w.varlen:
        lengths = workloads.make(name, seed=0)["lengths"]
        want = sum(_pairs_by_mask(n, n, w.causal) for n in lengths)
        assert bench.visible_pairs(w, lengths) == want
    else:
        want = w.batch * _pairs_by_mask(w.lq, w.lk, w.causal)
        assert bench.visible_pairs(w) == want


def test_headline_flops_and_bytes():
    bench = _bench()
    w = workloads.WORKLOADS["causal_b2h16"]
    # 4 * d * H * B * N (N + 1) / 2 for B2 H16 N2048 d64 causal
    assert 4.0 * w.d * w.hq * bench.visible_pairs(w) == 4 * 64 * 16 * 2 * 2048 * 2049 // 2
    inp = workloads.make("causal_b2h16", seed=0)
    # Q, K, V and O in fp16 plus one fp32 LSE per row
    assert bench.algorithmic_bytes(w, inp) == 4 * (2 * 16 * 2048 * 64 * 2) + 2 * 16 * 2048 * 4


def test_traffic_record_needs_matching_kernel_hash(tmp_path, monkeypatch):
    bench = _bench()
    src = tmp_path / "k.hpp"
    src.write_text("kernel v1")
    monkeypatch.setattr(bench, "KERNEL_SRCS", [str(src)])
    rec = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    import json
    rec.write_text(json.dumps({"kernel_sha256_16": bench.kernel_hash(),
                               "workloads": {"causal_b2h16": {"hbm_bytes_per_launch": 123}}}))
    assert bench.load_traffic("causal_b2h16") == 123
    assert bench.load_traffic("long_8k") is None
    src.write_text("kernel v2")                  # the kernel changed since
    assert bench.load_traffic("causal_b2h16") is None


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


@pytest.mark.gpu
@pytest.mark.parametrize("name,bound", [("tiny", "mfma"), ("rotary_gqa", "hbm")])
def test_bench_json_line_on_gpu(name, bound):
    """bench.py end to end: one JSON line with the contract's fields, a
    roofline entry and a passing parity record."""
    import json
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", name,
                          "--steps", "3", "--warmup", "1"],
                         capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-2000:]
    line = [x for x in res.stdout.splitlines() if x.startswith("{")][-1]
    rec = json.loads(line)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in rec, key
    assert rec["n_gpus"] == 1 and rec["steps"] == 3 and rec["config"]["workload"] == name
    roof = rec["roofline"]
    assert roof["bound"] == bound and roof["unit"] == ("TFLOP/s" if bound == "mfma" else "GB/s")
    assert rec["unit"] == roof["unit"] and rec["cpu_baseline"]["unit"] == roof["unit"]
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert rec["cpu_baseline"]["kind"] == "oracle" and rec["cpu_baseline"]["cores"] >= 1
    assert rec["parity"]["pass"]
    assert rec["cold"]["ms_per_launch_median"] > 0 and rec["cold"]["value"] > 0
    assert rec["device"]["cus"] >= 1


def test_batches_cover_exactly_the_timed_steps():
    bench = _bench()
    for steps in (1, 2, 3, 5, 7, 20, 200, 201):
        sizes = bench.batch_sizes(steps)
        assert sum(sizes) == steps and 1 <= len(sizes) <= 5
        assert max(sizes) - min(sizes) <= 1


def test_metric_labels():
    bench = _bench()
    labels = {n: bench.metric_label(w) for n, w in workloads.WORKLOADS.items()}
    # the headline keeps the metric string it is quoted on
    assert labels["causal_b2h16"] == ("attn fwd TFLOP/s + % of fp16 MFMA peak, "
                                      "B2 H16 N2048 d64 causal")
    assert len(set(labels.values())) == len(labels)
    assert labels["decode_gqa"].startswith("attn decode GB/s")
    assert "Hq32 Hkv8" in labels["gqa_causal"] and "causal" in labels["gqa_causal"]
    assert "Lq8192 Lk8192" in labels["long_8k"] and "bf16" in labels["long_8k"]
