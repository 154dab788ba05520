"""GPU parity at the full 262K sizes, in the launch configuration the benchmark times.

The whole batch (28 sequences at 262144 tokens, or 16 with int4 + eviction)
runs through lowram_decode_step in one call, as the benchmark runs it; each
sequence has its own seeded device-drawn cache.  The oracle then recomputes
sampled (sequence, KV head) slices one by one from the same arrays copied to
the host: selection within the tie band, that head's output within the
decode tolerance against the oracle re-run on the GPU's selection.  Every
output of the batch must be finite, and every selection ascending and full.
Every (sequence, KV head)'s selection is checked against the oracle's own
scores and top-k (tie band).  Every output is then checked by a property: the
4-wave kernel on the same batch selects the same chunks and agrees within
twice the tolerance (at these sizes the library runs the producer/consumer
kernel, whose workgroups switch heads inside their pipelines).

A third case has 40960 candidate chunks per head, more than the selection
kernel keeps in LDS (32768): it runs the variant that reads its keys from
the cache hierarchy.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

from gpu_util import DEV, MAX_ABS, REL_L2, check_output, check_selection, down_bf16  # noqa: E402
from long_context_decode_landmark_amd import native  # noqa: E402
from oracle import decode, steps  # noqa: E402
from synth import device as sd  # noqa: E402


def host(t):
    t = t.contiguous().cpu()
    if t.dtype in (torch.bfloat16, torch.int16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def draw_batch(cfg, nb, seed):
    """Distinct device caches for nb sequences (stacked on a batch axis)."""
    per = [sd.draw_layer(cfg, seed + b, DEV) for b in range(nb)]
    cache = {k: torch.stack([p[k] for p in per]) for k in per[0]}
    del per
    coeffs = [sd.draw_coeff(cfg, seed + 1000 + b, DEV) for b in range(nb)]
    if cfg.int4:
        cache["coeff"] = torch.stack([c[0] for c in coeffs])
        cache["coeff_scale"] = torch.stack([c[1] for c in coeffs])
    else:
        cache["coeff"] = torch.stack(coeffs)
    del coeffs
    desc = torch.empty((nb, cfg.n_heads_kv, cfg.n_chunks), dtype=torch.int32, device=DEV)
    native.resid_chunk_desc(cache["res_idx"], nb * cfg.n_heads_kv, cfg.n_resid, cfg.n_chunks, cfg.chunk, desc)
    cache["res_chunk_desc"] = desc
    return cache


def head_slice(cfg, cache, b, h):
    """Host copy of what the oracle reads for (sequence b, KV head h), as a 1 x 1 cache."""
    out = {}
    for k, v in cache.items():
        if k in ("coeff", "coeff_scale"):
            out[k] = host(v[b:b + 1])
        elif k != "res_chunk_desc":
            out[k] = host(v[b:b + 1, h:h + 1])
    return out


# 40960 chunks of 8 tokens per head (327680-token prefix plus a 256-token window)
WIDE = synth.C3.with_(name="wide_list_328k", batch=2, n_heads_q=8, n_heads_kv=2, ctx=327936)


@pytest.mark.parametrize("name,nb", [("c3_llama8b_262k", 28), ("c4_eq_int4_evict_262k", 16),
                                     ("wide_list_328k", 2)])
def test_full_size_sampled_heads(name, nb):
    cfg = WIDE if name == WIDE.name else synth.CONFIGS[name]
    if name == WIDE.name:
        assert cfg.n_cand > 32768
    g, keff = cfg.gqa, min(cfg.topk, cfg.n_cand)
    print(f"\n{name} batch {nb}: drawing caches", flush=True)
    cache = draw_batch(cfg, nb, seed=4242)
    q = sd.draw_queries(cfg, nb, 99, DEV)
    out = torch.empty_like(q)
    shape = native.make_shape(cfg, batch=nb)
    ws = torch.empty(native.workspace_bytes(shape), dtype=torch.uint8, device=DEV)
    sel = torch.full((nb, cfg.n_heads_kv, cfg.topk), -7, dtype=torch.int32, device=DEV)
    native.decode_step(shape, native.make_cache(cache), q, out, ws, sel_out=sel)
    torch.cuda.synchronize()
    got = down_bf16(out)
    sel_h = sel.cpu().numpy()
    assert np.all(np.isfinite(got))
    assert np.all(np.diff(sel_h[..., :keff], axis=-1) > 0)
    assert np.all(sel_h[..., keff:] == -1)
    print(f"{name}: step done, checking sampled heads", flush=True)

    q_h = host(q)
    # every head's selection against the oracle's own scores and top-k
    nflips = 0
    for b in range(nb):
        lm_b = host(cache["landmark"][b])
        cand_b = host(cache["cand_ids"][b]) if "cand_ids" in cache else None
        for h in range(cfg.n_heads_kv):
            sc = steps.landmark_scores(decode.widen(q_h[b, h * g:(h + 1) * g]), decode.widen(lm_b[h]))
            st = {"scores": sc, "sel": steps.select_topk(sc, cfg.topk, None if cand_b is None else cand_b[h])}
            if cand_b is not None:
                st["cand"] = cand_b[h]
            nflips += check_selection(cfg, {(0, 0): st}, sel_h[b:b + 1, h:h + 1], 0, 0)
        del lm_b
    print(f"{name}: every head's selection within the tie band of the oracle's ({nflips} tie flips)", flush=True)

    samples = sorted({(0, 0), (nb // 2, min(3, cfg.n_heads_kv - 1)), (nb - 1, cfg.n_heads_kv - 1)})
    for b, h in samples:
        sl = head_slice(cfg, cache, b, h)
        qs = decode.widen(q_h[b, h * g:(h + 1) * g])
        _, st = decode.decode_head(cfg, sl, qs, 0, 0)
        if "cand_ids" in sl:
            st["cand"] = sl["cand_ids"][0, 0]
        fake_sel = sel_h[b:b + 1, h:h + 1]
        nflip = check_selection(cfg, {(0, 0): st}, fake_sel, 0, 0)
        ref, _ = decode.decode_head(cfg, sl, qs, 0, 0, sel_override=sel_h[b, h])
        rel, mx = check_output(got[b, h * g:(h + 1) * g], ref, f"{name} b{b} h{h}")
        print(f"{name} b{b} h{h}: rel {rel:.2e} max {mx:.2e} flips {nflip}", flush=True)

    # Every head, by a property: the same batch through the other attention
    # kernel (LOWRAM_ATTEND=wave) must select the same chunks, and since each
    # kernel meets the decode tolerance against the oracle, the two outputs of
    # each (sequence, KV head) must agree within twice it.
    import os
    old = os.environ.get("LOWRAM_ATTEND")
    os.environ["LOWRAM_ATTEND"] = "wave"
    try:
        out_w = torch.empty_like(q)
        sel_w = torch.full_like(sel, -7)
        native.decode_step(shape, native.make_cache(cache), q, out_w, ws, sel_out=sel_w)
        torch.cuda.synchronize()
    finally:
        if old is None:
            os.environ.pop("LOWRAM_ATTEND", None)
        else:
            os.environ["LOWRAM_ATTEND"] = old
    assert torch.equal(sel_w, sel)
    a = got.reshape(nb, cfg.n_heads_kv, -1)
    w = down_bf16(out_w).reshape(nb, cfg.n_heads_kv, -1)
    rel = np.linalg.norm(a - w, axis=-1) / np.linalg.norm(w, axis=-1)
    mx = np.max(np.abs(a - w), axis=-1)
    print(f"{name}: every head against the 4-wave kernel: rel <= {rel.max():.2e}, max <= {mx.max():.2e}",
          flush=True)
    assert rel.max() <= 2 * REL_L2 and mx.max() <= 2 * MAX_ABS
