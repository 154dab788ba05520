"""The decode step captured in a HIP graph (the way a serving loop replays it).

One lowram_decode_step is captured with torch.cuda.graph, then replayed
several times. Before each replay the program runs its own eager step with
other queries into another output (same workspace), clears the graph's
output and selection buffers, and synchronizes. Every replay must reproduce
the eager result bit for bit (the step is deterministic, and nothing in it
may depend on what an earlier call left in the workspace).

Both attention kernels are covered: a multi-tile case the library runs on the
producer/consumer kernel, and the small case it runs on the 4-wave kernel.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

from gpu_util import DEV, cache_to_device, up  # noqa: E402
from long_context_decode_landmark_amd import native  # noqa: E402
from oracle import fixture  # noqa: E402

CASES = {
    # 64 (sequence, KV head) pairs x 16 tiles: the producer/consumer kernel
    "multitile_b8": synth.C0.with_(name="multitile_b8", batch=8, n_heads_q=32, n_heads_kv=8, rank=128,
                                   topk=250, bias_std=0.1),
    # one sequence, two KV heads: the 4-wave kernel
    "c0": synth.C0,
}
REPLAYS = 4


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_eager(name):
    cfg = CASES[name]
    cache = fixture.build_layer(cfg, 0)
    dev = cache_to_device(cache)  # held for the whole test (the graph reads these buffers)
    t = native.make_cache(dev)
    q = up(cache["q"])
    q_other = torch.flip(q, dims=[1]).contiguous()  # other queries for the eager work in between
    shape = native.make_shape(cfg)
    ws = torch.empty(native.workspace_bytes(shape), dtype=torch.uint8, device=DEV)
    sel_shape = (cfg.batch, cfg.n_heads_kv, cfg.topk)

    out_e = torch.empty_like(q)
    sel_e = torch.empty(sel_shape, dtype=torch.int32, device=DEV)
    native.decode_step(shape, t, q, out_e, ws, sel_out=sel_e)
    torch.cuda.synchronize()

    out_g = torch.empty_like(q)
    sel_g = torch.empty(sel_shape, dtype=torch.int32, device=DEV)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        native.decode_step(shape, t, q, out_g, ws, sel_out=sel_g)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        native.decode_step(shape, t, q, out_g, ws, sel_out=sel_g)
    torch.cuda.synchronize()

    out_o = torch.empty_like(q)
    for r in range(REPLAYS):
        native.decode_step(shape, t, q_other, out_o, ws)  # eager work on the same workspace
        out_g.fill_(0)
        sel_g.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), out_e.view(torch.int16)), (name, r)
        assert torch.equal(sel_g, sel_e), (name, r)
    # the eager work itself differs from the captured step (other queries)
    assert not torch.equal(out_o.view(torch.int16), out_e.view(torch.int16))
    print(f"{name}: {REPLAYS} replays equal the eager step", flush=True)
