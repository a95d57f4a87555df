"""bench.py's host-side logic, without a GPU: the one-GPU contract, the
counter summary's tie to the kernel sources, and the FLOP and byte counts
the roofline and the bandwidth figures divide by."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_attention_flops_are_the_causal_half():
    # Llama-3-8B layer at N = 2048: 2 * B * Hq * N^2 * D
    w = dict(B=1, Hq=32, Hkv=8, N=2048, D=128)
    assert bench.attn_flops(w) == 2 * 32 * 2048 ** 2 * 128 == 34359738368


def test_prerotation_bytes_read_and_write_q_and_k_once():
    w = dict(B=1, Hq=32, Hkv=8, N=2048, D=128, dtype="bf16")
    assert bench.prerot_bytes(w) == 2 * (32 + 8) * 2048 * 128 * 2  # 40 MiB
    assert bench.prerot_k_bytes(w) == 2 * 8 * 2048 * 128 * 2       # 8 MiB


def test_traffic_is_reported_only_for_the_sources_it_was_measured_on(tmp_path, monkeypatch):
    good = {"source_sha256": bench.attn_source_hash(), "read_bytes": 3.0e7, "write_bytes": 1.7e7}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(good))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic() == pytest.approx(4.7e7)
    f.write_text(json.dumps(dict(good, source_sha256="0" * 64)))
    assert bench.measured_traffic() is None



def _rows(gaps):
    # sweep rows whose fused time is (1 + gap) times the pre-rotation time
    return [{"N": n, "f": 100.0 * (1.0 + g), "p": 100.0} for n, g in gaps]


def test_crossover_is_the_log_linear_zero_of_the_relative_gap():
    r = bench.locate_crossover(_rows([(2048, -0.1), (4096, -0.1), (8192, 0.1), (16384, 0.2)]),
                               "f", "p")
    # the gap changes sign halfway between 4096 and 8192 on a log axis
    assert r["n_star"] == pytest.approx((4096 * 8192) ** 0.5)
    assert r["bracket"] == [4096, 8192]
    assert r["gaps_at_bracket"] == pytest.approx([-0.1, 0.1])
    assert r["winner_if_no_crossing"] is None


def test_crossover_reports_the_winner_when_the_sign_never_changes():
    pre = bench.locate_crossover(_rows([(2048, 0.01), (4096, 0.2)]), "f", "p")
    assert pre["n_star"] is None and pre["winner_if_no_crossing"] == "prerotate"
    fus = bench.locate_crossover(_rows([(2048, -0.3), (4096, -0.01)]), "f", "p")
    assert fus["n_star"] is None and fus["winner_if_no_crossing"] == "fused"


def test_gfx_clocks_are_read_per_xcd_from_the_amd_smi_json():
    text = json.dumps({"gpu_data": [{"gpu": 0, "clock": {
        "gfx_0": {"clk": {"value": 2170, "unit": "MHz"}, "max_clk": {"value": 2400}},
        "gfx_1": {"clk": {"value": 2118, "unit": "MHz"}},
        "mem_0": {"clk": {"value": 2000, "unit": "MHz"}},
        "gfx_2": {"clk": {"value": "N/A"}},
        "gfx_3": {"clk": {"value": 95}, "min_clk": {"value": 500}},
        "gfx_4": {"clk": {"value": 450}}}}]})
    # gfx_3 and gfx_4 sit below the lowest clock level: asleep, not slow
    assert bench.parse_gfx_clocks(text) == [2170.0, 2118.0]
    assert bench.parse_gfx_clocks("not json") == []
    assert bench.parse_gfx_clocks(json.dumps({"gpu_data": []})) == []
