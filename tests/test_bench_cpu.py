"""Host logic of bench.py with no GPU: the algorithmic byte and flop counts
per stage (and where the exact window's share is charged), the reading of the
committed counter summaries (only while the kernel sources hash the same),
and the step statistics."""
import os
import sys

import pytest

import synth

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_window_share_moves_between_stages(name):
    cfg = synth.CONFIGS[name]
    nb = 3
    b_att, f_att = bench.algorithmic(cfg, nb, "attend")
    b_sc, f_sc = bench.algorithmic(cfg, nb, "score")
    # the window's K and V rows (bf16) and its QK + PV flops, per sequence
    wb = 2 * cfg.n_heads_kv * cfg.window * cfg.head_dim * 2 * nb
    wf = 4.0 * cfg.n_heads_q * cfg.window * cfg.head_dim * nb
    assert b_att["attend"] - b_sc["attend"] == pytest.approx(wb)
    assert b_sc["score"] - b_att["score"] == pytest.approx(wb)
    assert f_att["attend"] - f_sc["attend"] == pytest.approx(wf)
    assert f_sc["score"] - f_att["score"] == pytest.approx(wf)
    assert sum(b_att.values()) == pytest.approx(sum(b_sc.values()))
    assert sum(f_att.values()) == pytest.approx(sum(f_sc.values()))


def test_benchmark_workload_bytes():
    # 262K context, batch 28: landmarks 1.877 GB per layer; the selected
    # chunks' stage 2.000 GB, 2.029 GB with the window
    cfg = synth.CONFIGS["c3_llama8b_262k"]
    b, _ = bench.algorithmic(cfg, 28, "attend")
    assert b["score"] == pytest.approx(1.877e9, rel=1e-3)
    assert b["attend"] == pytest.approx(2.029e9, rel=1e-3)
    b, _ = bench.algorithmic(cfg, 28, "score")
    assert b["attend"] == pytest.approx(2.000e9, rel=1e-3)


def test_counter_lines_follow_the_source_hash(tmp_path):
    h = bench.source_hash("attend")
    good = tmp_path / "t.txt"
    good.write_text(f"header\ntraffic attend c3_llama8b_262k 28 {h} 123456\n"
                    f"traffic score c3_llama8b_262k 28 0000000000000000 99\n")
    assert bench.measured_traffic("attend", "c3_llama8b_262k", 28, str(good)) == 123456.0
    assert bench.measured_traffic("score", "c3_llama8b_262k", 28, str(good)) is None  # stale hash
    assert bench.measured_traffic("attend", "c3_llama8b_262k", 16, str(good)) is None  # other batch
    assert bench.measured_traffic("attend", "c3_llama8b_262k", 28, str(tmp_path / "missing.txt")) is None


def test_source_hash_is_stable():
    h = bench.source_hash("merge")
    assert len(h) == 16 and h == bench.source_hash("merge")
    assert h != bench.source_hash("score")


def test_step_stats():
    st = bench.step_stats([3.0, 1.0, 2.0, 4.0, 5.0])
    assert st["median"] == 3.0 and st["n"] == 5
    assert st["p10"] <= st["median"] <= st["p90"]
