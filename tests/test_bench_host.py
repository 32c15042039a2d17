"""Host-side logic of bench.py that runs without a GPU: the oracle baseline's
process pools (a bounded sample, one result per token or per slice of
requantised rows) and the failure path
(an error in a worker ends the run with that error instead of waiting), the
multi-GPU refusal, and the algorithmic byte count of the decode workload."""

import subprocess
import sys

import numpy as np
import pytest

import bench
import synth


def test_cpu_baseline_times_tokens():
    inp = synth.make_moe_inputs(synth.CONFIGS["tiny"])
    r = bench.cpu_baseline(inp, budget_s=2.0)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s"
    assert r["value"] > 0 and 1 <= r["cores"] <= 16


def test_cpu_baseline_worker_error_is_raised(monkeypatch):
    inp = synth.make_moe_inputs(synth.CONFIGS["tiny"])

    def broken(t):
        raise ImportError("oracle missing in the worker")

    monkeypatch.setattr(bench, "_oracle_token", broken)
    with pytest.raises(RuntimeError, match="failed in a worker"):
        bench.cpu_baseline(inp, budget_s=2.0)


def test_cpu_baseline_requant_counts_bytes():
    inp = synth.make_moe_inputs(synth.variant(synth.CONFIGS["decode16"], T=8, E=2))
    r = bench.cpu_baseline_requant(inp, budget_s=1.0)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s" and r["value"] > 0
    # every slice is 256 rows x K of codes and scales in and out
    assert "256 rows x K=6144" in r["sample"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr


def test_decode_algorithmic_bytes_count_active_experts():
    # the decode16 layer's compulsory bytes: 21 233 664 per active expert
    # (w13 and w2 codes and E4M3 scales) + 8 (two FP32 global scales), x and
    # out in bf16 (786 432 each), ids and router weights (T k 8 = 4 096)
    cfg = synth.CONFIGS["decode16"]
    ids, _ = synth.make_routing(cfg)
    ab = bench.algorithmic_bytes(cfg, ids)
    active = int(np.unique(ids).size)
    assert ab["active"] == active
    assert ab["whole"] == active * (21233664 + 8) + 786432 + 786432 + 4096
