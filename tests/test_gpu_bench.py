"""bench.py keeps its output contract: one JSON line with the metric, the
whole-job value, the roofline of the dominant kernel (the one with the most time per
step) and those of the gather, the projection and the gate under their own names,
the per-kernel breakdown, the sequential step order timed beside the look-ahead one,
and the oracle's CPU rate.  Runs the tiny workload in a child process
(a few seconds)."""
import json
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line_contract():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    out = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--config", "tiny",
                          "--steps", "3", "--warmup", "1", "--cpu-budget", "1"],
                         capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert out.returncode == 0, out.stderr[-2000:]
    lines = [ln for ln in out.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, out.stdout
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["value"] > 0
    assert d["value"] == pytest.approx(d["config"]["tokens_per_step"] / (d["ms_per_step"] * 1e-3), rel=1e-6)
    assert "workload" in d["config"]
    named = {"gather_dequant": d["roofline_gather"], "gemm": d["roofline_projection"],
             "gate_add": d["roofline_gate"]}
    for r in list(named.values()) + [d["roofline"]]:
        for k in ("bound", "achieved", "peak", "unit", "frac", "traffic", "avg_launch_ms"):
            assert k in r, k
        assert r["frac"] == pytest.approx(r["achieved"] / r["peak"])
    assert named["gather_dequant"]["bound"] == "hbm" and named["gate_add"]["bound"] == "hbm"
    # tiny's projection (512 tokens, 768 -> 256) does 118 flops per algorithmic byte, below
    # the ridge of 2.5 PFLOP/s over 8 TB/s (312.5): bound by HBM, against 8 TB/s
    assert named["gemm"]["bound"] == "hbm" and named["gemm"]["unit"] == "GB/s"
    # the dominant kernel: the named roofline with the longest launch
    longest = max(named.values(), key=lambda r: r["avg_launch_ms"])
    assert d["roofline"] == longest
    # the tiny workload is a many-token split-path call: the look-ahead order is timed,
    # and the sequential order beside it
    assert d["config"]["step_order"] == "lookahead"
    so = d["sequential_order"]
    assert so["value"] > 0 and so["ms_per_step"] > 0
    assert so["value"] == pytest.approx(d["config"]["tokens_per_step"] / (so["ms_per_step"] * 1e-3), rel=1e-6)
    assert set(so["kernels_ms"]) == set(d["kernels"])
    c = d["cpu_baseline"]
    for k in ("value", "unit", "cores", "kind", "sample"):
        assert k in c, k
    assert c["kind"] == "oracle" and c["cores"] >= 1 and c["value"] > 0

