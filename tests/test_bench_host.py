"""Host-side checks of bench.py: the one-GPU contract and the per-unit work figures its roofline
divides by (no GPU needed)."""
import os
import subprocess
import sys

import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("name,flop", [("square256", 2 * 256 ** 3), ("square4096", 2 * 4096 ** 3),
                                       ("ragged", 2 * 1000 * 1537 * 999), ("gate_up", 4 * 4096 * 11008 * 4096),
                                       ("skinny", 2 * 16 * 28672 * 8192)])
def test_gemm_flops(name, flop):
    assert synth.WORKLOADS[name].flops() == flop


def test_algorithmic_bytes():
    # every operand read once, C written (and read when beta != 0)
    assert bench.algorithmic_bytes(synth.WORKLOADS["skinny"]) == 2 * 16 * 8192 + 2 * 8192 * 28672 + 4 * 16 * 28672 == 471_859_200
    assert bench.algorithmic_bytes(synth.WORKLOADS["square4096"]) == 3 * 2 * 4096 * 4096
    assert bench.algorithmic_bytes(synth.WORKLOADS["square4096_f32"]) == 3 * 4 * 4096 * 4096
    assert bench.algorithmic_bytes(synth.WORKLOADS["ragged"]) == 2 * (1000 * 999 + 999 * 1537) + 2 * 4 * 1000 * 1537
    assert bench.algorithmic_bytes(synth.WORKLOADS["gate_up"]) == 2 * 4096 * 4096 + 2 * 2 * 4096 * 11008 + 2 * 2 * 4096 * 11008
    assert bench.algorithmic_bytes(synth.WORKLOADS["gate_up_swiglu"]) == 2 * 4096 * 4096 + 2 * 2 * 4096 * 11008 + 2 * 4096 * 11008


def test_attention_and_norm_work():
    a = synth.ATTN_WORKLOADS["attention"]
    assert a.flops() == 4 * 64 * 4096 * 4096 * 128
    n = synth.NORM_WORKLOADS["rms_norm"]
    assert n.bytes() == n.M * n.D * 8 + n.D * 4


def test_traffic_lines_parse_and_follow_the_source_hash(tmp_path, monkeypatch):
    # a line is used only while its hash matches the workload's current kernel sources
    h = bench.kernel_source_hash("square4096")
    assert len(h) == 16 and h != bench.kernel_source_hash("attention")
    # same kernel sources, another instantiation: the plan summary keeps the hashes apart
    assert bench.workload_sources("square4096") == bench.workload_sources("gate_up")
    assert h != bench.kernel_source_hash("gate_up")
    assert "planner.cpp" in bench.workload_sources("ragged") and "planner.cpp" not in bench.workload_sources("attention")
    assert "prefetch=3" in bench.gemm_plan_summary("ragged")
    # each GEMM workload hashes the sources of the kernel family its plan selects
    assert "gemm_fast.hpp" in bench.workload_sources("square4096")
    assert "gemm_tiled.hpp" not in bench.workload_sources("square4096")
    assert "gemm_skinny.hip" in bench.workload_sources("skinny")
    assert "gemm_tiled.hpp" in bench.workload_sources("ragged")
    assert bench.kernel_source_hash("ragged") != h != bench.kernel_source_hash("skinny")
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic.md").write_text("# header\ntraffic square4096: 1234 %s\ntraffic skinny: 99 0000000000000000\n" % h)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda w: h)
    assert bench.measured_traffic("square4096") == 1234
    assert bench.measured_traffic("skinny") is None          # stale hash
    assert bench.measured_traffic("gate_up") is None         # no line


def test_graph_chunks_divide_the_timed_steps():
    """The timed steps replay a captured graph of S steps exactly steps / S times; S is even where
    an even divisor exists, so the skinny workload's two B buffers keep alternating across replays."""
    for steps in (1, 2, 5, 7, 20, 37, 100, 999, 1000):
        s = bench.graph_chunk(steps)
        assert 1 <= s <= 50 and steps % s == 0, steps
        if any(d % 2 == 0 and steps % d == 0 for d in range(2, 51)):
            assert s % 2 == 0, steps
    assert bench.graph_chunk(1000) == 50 and bench.graph_chunk(999) == 37


def test_peak_scaled_to_the_measured_clock():
    """The clock-scaled peak is the nominal peak times median gfx clock / maximum clock."""
    clock = {"gfx_mhz": [95.0, 1630.0, 1630.0], "settled_mhz": 1630.0, "max_mhz": 2400.0, "socket_power_w": [1267.0]}
    r = bench.at_clock(clock, 2516.6, 1239.0)
    assert r["gfx_mhz"] == 1630.0
    assert abs(r["peak_tflops"] - 2516.6 * 1630.0 / 2400.0) < 1e-9
    assert abs(r["frac"] - 1239.0 / r["peak_tflops"]) < 1e-12
    assert bench.at_clock(None, 2516.6, 1239.0) is None


def test_settled_clock_is_the_median_after_the_first_reading():
    assert bench.settled_clock([95.0, 1577.0, 1622.0]) == (1577.0 + 1622.0) / 2
    assert bench.settled_clock([95.0, 1630.0, 1600.0, 1640.0]) == 1630.0
    assert bench.settled_clock([1500.0]) == 1500.0
