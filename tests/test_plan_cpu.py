"""The host's schedule of the selected chunks (lowram_decode_plan), with no
GPU: against its restatement in plan_util, and the invariants the kernels
rely on (the workspace reserve covers every plan's partial slots, groups hold
at least 2 tiles where a head has 2, the automatic choice rule)."""
import pytest

import synth
from long_context_decode_landmark_amd import native
from plan_util import pipe_plan

CASES = [
    ("c0", synth.C0, 1),
    ("c1_b1", synth.C1, 1),
    ("c1_b8", synth.C1, 8),
    ("c2_b4", synth.C2, 4),
    ("c3_b28", synth.C3, 28),
    ("c3_b4", synth.C3, 4),
    ("c4_b16", synth.C4, 16),
    ("ragged_b40", synth.C0.with_(name="ragged", ctx=4060, window=300, topk=45, rank=128), 40),
    ("multitile_b8", synth.C0.with_(name="multitile_b8", n_heads_q=32, n_heads_kv=8, rank=128, topk=250), 8),
    ("multitile_int4", synth.C4.with_(name="mt_int4", ctx=4096, window=64, n_layers=4, topk=200, rank=128), 8),
]
CUS = (256, 304, 100, 7, 1)


def tiles(cfg):
    return -(-min(cfg.topk, cfg.n_cand) // 16), -(-cfg.window // 128)


@pytest.mark.parametrize("n_cu", CUS)
@pytest.mark.parametrize("name,cfg,nb", CASES, ids=[c[0] for c in CASES])
def test_plan_matches_restatement(name, cfg, nb, n_cu):
    shape = native.make_shape(cfg, batch=nb)
    n, n_win = tiles(cfg)
    heads = nb * cfg.n_heads_kv
    auto, pipe, wave = (native.decode_plan(shape, n_cu, m) for m in (0, 1, 2))
    w, t, n_grp, most, several = pipe_plan(heads, n, n_cu)
    # the producer/consumer plan is the restated one
    assert pipe["kernel"] == 1
    assert (pipe["workgroups"], pipe["tiles_per_group"], pipe["groups_per_head"]) == (w, t, n_grp)
    assert pipe["partial_slots"] == 4 * n_grp + n_win
    assert t >= min(2, n)
    groups = heads * n_grp
    assert most <= -(-groups // w) * t  # the planner's bound on a workgroup's tiles
    # the 4-wave plan: one partial slot per tile
    assert wave["kernel"] == 2 and wave["workgroups"] == 0
    assert wave["partial_slots"] == n + n_win
    # the workspace reserve covers both kernels' slots
    assert auto["reserved_slots"] == 2 * n + 6 + n_win
    for pl in (auto, pipe, wave):
        assert pl["partial_slots"] <= pl["reserved_slots"]
    # automatic choice: the producer/consumer kernel once every CU gets more than two tiles
    assert auto["kernel"] == (1 if heads * n > 2 * n_cu else 2)
    assert auto == (pipe if auto["kernel"] == 1 else wave)
    # the window's tiles ride in the score launch beside the producer/consumer
    # kernel, in the 4-wave kernel's own grid otherwise
    assert pipe["window_kernel"] == (1 if n_win else 0)
    assert wave["window_kernel"] == (2 if n_win else 0)


def test_plan_of_the_benchmark_workload():
    # 262K context, batch 28 on 256 CUs: groups of 8 tiles, 8 per head, 7 per workgroup
    p = native.decode_plan(native.make_shape(synth.C3, batch=28), 256)
    assert p == {"kernel": 1, "workgroups": 256, "tiles_per_group": 8, "groups_per_head": 8,
                 "partial_slots": 4 * 8 + 2, "reserved_slots": 2 * 64 + 6 + 2, "window_kernel": 1}
    assert pipe_plan(28 * 8, 64)[3] == 56  # tiles per workgroup


def test_plan_window_without_prefix():
    # no compressed prefix yet: nothing is scored, the window runs in the 4-wave kernel's grid
    cfg = synth.C0.with_(name="window_only", ctx=64, window=64)
    p = native.decode_plan(native.make_shape(cfg, prefix_len=0, n_cand=0, n_resid=0), 256, 1)
    assert p["kernel"] == 0 and p["window_kernel"] == 2


def test_plan_rejects_bad_arguments():
    shape = native.make_shape(synth.C0)
    for n_cu, mode in ((0, 0), (-1, 0), (256, 3), (256, -1)):
        with pytest.raises(native.LowramError) as e:
            native.decode_plan(shape, n_cu, mode)
        assert e.value.status == -2  # LOWRAM_ERR_SHAPE
