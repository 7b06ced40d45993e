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


def _step_kernels(cfg, filtered):
    R = cfg["R"]
    fmt = str(cfg.get("key_format", "fp8") == "mxfp4").lower()
    q8 = bool(cfg.get("fp8_query", False))
    qf = str(q8).lower()
    if filtered:
        ks = bench.sample_kernels(len(cfg["lengths"]) * R, R, fmt == "true", q8) + [
            f"score_kernel<{bench.score_rpw(R)},{qf},{fmt},true>", f"candidate_select_kernel<{fmt},{qf}>"]
    else:
        ks = [f"score_kernel<{bench.score_rpw(R, q8)},{qf},{fmt},false>", "topk_short_kernel<true>"]
    return ks + ["sparse_mla_kernel", "mla_combine_kernel"]


@pytest.mark.parametrize("workload", ["decode_16x4_32k", "decode_4x4_1m_planted", "decode_4x4_1m_mxfp4",
                                      "decode_4x4_1m_fp8q"])
def test_step_hbm_fields(workload):
    cfg = case_config(workload)
    kf = cfg.get("key_format", "fp8")
    lens, R, k = cfg["lengths"], cfg["R"], 2048
    filtered = max(lens) > bench.FILTER_MIN_CTX
    step = traffic.decode_step_bytes(lens, R, k, kf, round_trip=not filtered)
    no_rt = traffic.decode_step_bytes(lens, R, k, kf, round_trip=False)
    sec = 1e-4
    f = bench.step_hbm_fields(traffic, lens, R, k, kf, sec, workload, _step_kernels(cfg, filtered), filtered)
    assert f["bytes"] == step
    assert f["frac"] == pytest.approx(step / sec / 1e9 / bench.HBM_PEAK_GBS)
    # the score round trip is 8 bytes per visible (row, token), counted only on the stored path
    rt = 8 * sum(traffic.visible(lens, R))
    assert step - no_rt == (0 if filtered else rt)
    assert f["frac_without_score_round_trip"] == pytest.approx(no_rt / sec / 1e9 / bench.HBM_PEAK_GBS)
    # with counters for the current sources, the counted bytes cover the algorithmic ones (within the
    # counters' granularity); once a kernel source changes they are None until taken again
    if f["measured_bytes"] is None:
        assert f["measured_frac"] is None
    else:
        assert f["measured_bytes"] > 0.9 * step
        assert f["measured_frac"] == pytest.approx(f["measured_bytes"] / sec / 1e9 / bench.HBM_PEAK_GBS)


def test_the_filtered_step_is_charged_no_score_round_trip():
    lens, R, k = [1 << 20] * 4, 4, 2048
    full = traffic.decode_step_bytes(lens, R, k)
    filt = traffic.decode_step_bytes(lens, R, k, round_trip=False)
    assert full - filt == 8 * sum(traffic.visible(lens, R))
    assert traffic.filter_scorer_bytes(lens, R) == sum(lens) * 132 + 16 * traffic.Q_IDX_BYTES
    # E4M3 queries: 4 KB of codes and a 4-byte row scale per row instead of 8 KB of bf16
    assert traffic.filter_scorer_bytes(lens, R, q_fp8=True) == sum(lens) * 132 + 16 * (4096 + 4 + 64)


def test_counters_need_the_current_source(monkeypatch, tmp_path):
    assert bench.counters_for("score_kernel<1,false,false,true>", "no_such_workload") is None
    assert bench.measured_step_bytes("no_such_workload", ["sparse_mla_kernel"]) is None
    # a table with one line for the current sources is read back; a changed source invalidates it
    (tmp_path / "profiles").mkdir()
    h = bench.kernel_source_hash("mla.hip")
    (tmp_path / "profiles" / "hbm_counters.txt").write_text(
        f"# header\nmla.hip wl sparse_mla_kernel {h} 1000 24\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda name: h)  # the sources as they were
    assert bench.counters_for("sparse_mla_kernel", "wl") == 1024.0
    assert bench.measured_step_bytes("wl", ["sparse_mla_kernel"]) == 1024.0
    assert bench.measured_step_bytes("wl", ["sparse_mla_kernel", "mla_combine_kernel"]) is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda name: "0" * 16)
    assert bench.counters_for("sparse_mla_kernel", "wl") is None
    assert bench.measured_step_bytes("wl", ["sparse_mla_kernel"]) is None


def test_sample_kernel_names_follow_the_row_count():
    assert bench.sample_kernels(16, 4, False) == ["sample_score_kernel<false,128,2,false>", "sample_select_kernel"]
    assert bench.sample_kernels(64, 4, True) == ["sample_score_kernel<true,64,2,false>", "sample_select_kernel"]
    assert bench.sample_kernels(10, 10, False)[0] == "sample_score_rows_kernel<false,128,false>"
    assert bench.sample_kernels(16, 4, False, True)[0] == "sample_score_kernel<false,128,2,true>"


def test_counter_hash_follows_code_not_comments():
    a = "int f(int x) { return x + 1; }  // one\n/* note */\n"
    b = "int f(int x)\n{\n  return x + 1;  // other words\n}\n"
    c = "int f(int x) { return x + 2; }\n"
    assert bench._code_only(a) == bench._code_only(b) != bench._code_only(c)
    assert bench._code_only('const char* s = "// kept";') == 'constchar*s="//kept";'
