"""bench.py's host-side pieces, on the CPU: the one-GPU refusal, the algorithmic work that
the roofline divides by (pinned to the figures the trace summaries quote), the roofline's
bound rule, the traffic summary's source check, and the timing windows."""
import os
import subprocess
import sys

import pytest

import bench
import moe_synth as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout


def test_headline_gate_up_bytes():
    # 44 touched experts x (gate + up) x I x d bf16, the 8 token rows read once, the 64 h rows
    # written once
    w = bench.layer_work(S.OLMOE_BF16, 8, 44)
    assert w["gate_up_bytes"] == 44 * 2 * 1024 * 2048 * 2 + 8 * 2048 * 2 + 64 * 1024 * 2 == 369_262_592
    assert w["down_bytes"] == 44 * 2048 * 1024 * 2 + 64 * 1024 * 2 + 64 * 2048 * 2
    assert w["touched_groups"] == 44


def test_int8_gate_up_bytes_count_the_scales():
    w = bench.layer_work(S.OLMOE_I8, 8, 42)
    assert w["gate_up_bytes"] == 42 * (2 * 1024 * 2048 + 2 * 1024 * 4) + 8 * 2048 * 2 + 64 * 1024 * 2
    assert w["gate_up_bytes"] == 176_668_672


def test_prefill_flops_and_bound():
    wl = S.DEEPSEEK_BF16
    w = bench.layer_work(wl, 2048, wl.E)
    R = 2048 * 6 + 2 * 2048
    assert w["gate_up_flops"] == 2.0 * R * 2048 * 2 * 1408 == 188_978_561_024
    assert w["down_flops"] == 2.0 * R * 1408 * 2048
    # about 232 flop per byte, under the 312 of the ridge (2.5 PFLOP/s over 8 TB/s): the
    # larger of the two peak times is the HBM one
    assert w["gate_up_flops"] / w["gate_up_bytes"] < bench.MFMA_BF16_PEAK_TFS * 1e12 / (bench.HBM_PEAK_GBS * 1e9)
    assert not bench.mfma_bound(wl, 2048, w)


def test_traffic_only_while_the_sources_match(tmp_path, monkeypatch):
    name = "gemv_gateup_olmoe_bf16_T8.pmc.txt"
    got = bench.read_traffic(name)
    assert got is not None and got > 369_262_592  # counted bytes, at least the algorithmic ones
    text = open(os.path.join(bench.PROFILES, name)).read()
    stale = "\n".join(("sources_sha256 = " + "0" * 64) if ln.startswith("sources_sha256") else ln
                      for ln in text.splitlines())
    (tmp_path / name).write_text(stale)
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.read_traffic(name) is None
    assert bench.read_traffic("no_such_summary.pmc.txt") is None


@pytest.mark.parametrize("steps,per_step_ms,want", [(50, 0.03, 167), (50, 0.45, 50), (50, 0.1, 51)])
def test_timing_window(steps, per_step_ms, want):
    assert bench.window_steps(steps, per_step_ms) == want


def test_gate_tokens():
    assert bench.gate_tokens(1) == [0]
    assert bench.gate_tokens(2) == [0, 1]
    assert bench.gate_tokens(8) == [0, 4, 7]
