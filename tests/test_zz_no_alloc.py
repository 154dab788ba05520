"""lowram_decode_step_noalloc, the decode step on the library's fixed device
scratch (for callers that cannot allocate), against lowram_decode_step with a
caller-allocated workspace.  Both run the same kernels on the same inputs, so
outputs and selections must be identical; the outputs are also held to the
decode tolerance against the oracle on the selection.  Three calls in a row,
each on a smaller input than the one before: the scratch keeps the previous
call's contents, and nothing in it may leak into the next result.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

from gpu_util import DEV, cache_to_device, check_output, down_bf16, up  # noqa: E402
from long_context_decode_landmark_amd import native  # noqa: E402
from oracle import decode, fixture  # noqa: E402
from synth import device as sd  # noqa: E402


def both(cfg, tensors, q):
    """The step through both entry points; returns (out, sel) of each."""
    nb = q.shape[0]
    shape = native.make_shape(cfg, batch=nb)
    need = native.workspace_bytes(shape)
    assert need <= native.NOALLOC_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    cache = native.make_cache(tensors)
    res = []
    for noalloc in (False, True):
        # bf16 NaN bits: every element must be written
        out = torch.full(tuple(q.shape), 0x7FC0, dtype=torch.int16, device=DEV).view(q.dtype)
        sel = torch.full((nb, cfg.n_heads_kv, cfg.topk), -7, dtype=torch.int32, device=DEV)
        if noalloc:
            native.decode_step_noalloc(shape, cache, q, out, sel_out=sel)
        else:
            native.decode_step(shape, cache, q, out, ws, sel_out=sel)
        torch.cuda.synchronize()
        res.append((out, sel))
    return need, res


def test_noalloc_matches_the_workspace_step_on_successive_calls():
    # 1. a 262144-token batch of 4 drawn on the device (13 MB of scratch)
    cfg = synth.C3
    per = [sd.draw_layer(cfg, 500 + b, DEV) for b in range(4)]
    t = {k: torch.stack([p[k] for p in per]) for k in per[0]}
    t["coeff"] = torch.stack([sd.draw_coeff(cfg, 600 + b, DEV) for b in range(4)])
    desc = torch.empty((4, cfg.n_heads_kv, cfg.n_chunks), dtype=torch.int32, device=DEV)
    native.resid_chunk_desc(t["res_idx"], 4 * cfg.n_heads_kv, cfg.n_resid, cfg.n_chunks, cfg.chunk, desc)
    t["res_chunk_desc"] = desc
    q = sd.draw_queries(cfg, 4, 700, DEV)
    need, ((o1, s1), (o2, s2)) = both(cfg, t, q)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(s1, s2)
    assert np.all(np.isfinite(down_bf16(o2)))
    print(f"\nc3 batch 4: {need} bytes of scratch, identical to the workspace step", flush=True)
    del t, per, q
    sizes = [need]

    # 2. then smaller fixture caches, each also against the oracle
    for cfg in (synth.C0.with_(name="multitile_b8", batch=8, n_heads_q=32, n_heads_kv=8, rank=128, topk=250,
                               bias_std=0.1),
                synth.C0):
        cache = fixture.build_layer(cfg, 0)
        need, ((o1, s1), (o2, s2)) = both(cfg, cache_to_device(cache), up(cache["q"]))
        assert need < sizes[-1]
        sizes.append(need)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(s1, s2)
        ref, _ = decode.decode_step(cfg, cache, cache["q"], sel_override=s2.cpu().numpy())
        rel, mx = check_output(down_bf16(o2), ref, f"{cfg.name} (no-allocation step)")
        print(f"{cfg.name}: {need} bytes of scratch, identical to the workspace step; oracle rel {rel:.2e} "
              f"max {mx:.2e}", flush=True)
