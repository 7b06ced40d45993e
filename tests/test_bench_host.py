"""Host-side parts of bench.py: the one-GPU guard, the step's HBM fields and
the counter table lookups (no GPU: nothing here launches a kernel)."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from sparse_attention_index_amd import traffic  # noqa: E402
from workloads import case_config  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr


@pytest.mark.parametrize("workload", ["decode_16x4_32k", "decode_4x4_1m_planted", "decode_4x4_1m_mxfp4"])
def test_step_hbm_fields(workload):
    cfg = case_config(workload)
    kf = cfg.get("key_format", "fp8")
    lens, R, k = cfg["lengths"], cfg["R"], 2048
    step = traffic.decode_step_bytes(lens, R, k, kf)
    sec = 1e-4
    f = bench.step_hbm_fields(traffic, lens, R, k, kf, step, sec, workload)
    assert f["bytes"] == step
    assert f["frac"] == pytest.approx(step / sec / 1e9 / bench.HBM_PEAK_GBS)
    # the score round trip is 8 bytes per visible (row, token)
    rt = 8 * sum(traffic.visible(lens, R))
    assert f["frac_without_score_round_trip"] == pytest.approx((step - rt) / sec / 1e9 / bench.HBM_PEAK_GBS)
    # with counters for the current sources, the counted bytes cover the algorithmic ones (within the
    # counters' granularity); once a kernel source changes they are None until taken again
    if f["measured_bytes"] is None:
        assert f["measured_frac"] is None
    else:
        assert f["measured_bytes"] > 0.9 * step
        assert f["measured_frac"] == pytest.approx(f["measured_bytes"] / sec / 1e9 / bench.HBM_PEAK_GBS)


def test_counters_need_the_current_source(monkeypatch):
    assert bench.counters_for("score.hip", "no_such_workload") is None
    assert bench.measured_step_bytes("no_such_workload") is None
    # a changed kernel source invalidates its counter lines
    real = bench.kernel_source_hash
    monkeypatch.setattr(bench, "kernel_source_hash", lambda names: "0" * 16 if names[0] == "score.hip" else real(names))
    assert bench.counters_for("score.hip", "decode_16x4_32k") is None
    assert bench.measured_step_bytes("decode_16x4_32k") is None
