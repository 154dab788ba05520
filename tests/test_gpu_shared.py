"""GPU parity of the shared-prefix multi-query decode (lowram_decode_shared).

Q queries attend to one compressed context (every cache array for NB = 1,
read by all queries).  Each query's selection and output are checked against
the oracle's decode step of that query on the same single-context cache, by
the decode step's parity rule (selection within the tie band, output within
the decode tolerance against the oracle re-run on the GPU's selection).  The
shared call must also equal, bit for bit, lowram_decode_step on the context
replicated once per query.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

from gpu_util import DEV, check_output, check_selection, down_bf16, up  # noqa: E402
from long_context_decode_landmark_amd import native  # noqa: E402
from oracle import codecs, decode, fixture  # noqa: E402

CASES = {
    "c0_q5": (synth.C0, 1, 5),
    "ragged_q3": (synth.C0.with_(name="sh_ragged", ctx=4060, window=300, topk=45, rank=128, bias_std=0.1), 0, 3),
    "int4_evict_q4": (synth.C0.with_(name="sh_eq", rank=128, int4=True, evict=True, resid_frac=0.25, topk=48), 1, 4),
    "gqa8_q2": (synth.C0.with_(name="sh_g8", n_heads_q=16, rank=256, topk=40), 0, 2),
    "gqa16_q3": (synth.C0.with_(name="sh_g16", n_heads_q=32, rank=512, topk=70), 1, 3),
    "gqa2_q7": (synth.C0.with_(name="sh_g2", n_heads_q=4, topk=33), 0, 7),
    "gqa1_q9": (synth.C0.with_(name="sh_g1", n_heads_q=2, window=1, ctx=4033, topk=17), 1, 9),
}


def queries(cfg, layer, n):
    return np.stack([codecs.bf16_encode(synth.queries(cfg, 100 + i, layer)) for i in range(n)])


def run_shared(cfg, cache, q):
    nq = q.shape[0]
    t = {k: up(v) for k, v in cache.items() if k not in ("q", "needle")}
    qd = up(q)
    out = torch.empty_like(qd)
    shape = native.make_shape(cfg, batch=nq)
    ws = torch.empty(native.workspace_bytes(shape), dtype=torch.uint8, device=DEV)
    sel = torch.full((nq, cfg.n_heads_kv, cfg.topk), -7, dtype=torch.int32, device=DEV)
    native.decode_shared(shape, t, qd, out, ws, sel_out=sel)
    # the same queries against the context replicated once per query
    rep = {k: v.expand(nq, *v.shape[1:]).contiguous() for k, v in t.items()}
    out2 = torch.empty_like(qd)
    sel2 = torch.full_like(sel, -7)
    native.decode_step(shape, rep, qd, out2, ws, sel_out=sel2)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(sel, sel2)
    return down_bf16(out), sel.cpu().numpy()


@pytest.mark.parametrize("name", list(CASES))
def test_shared_context(name):
    cfg, layer, nq = CASES[name]
    cfg1 = cfg.with_(batch=1)
    cache = fixture.build_layer(cfg1, layer)
    q = queries(cfg, layer, nq)
    got, sel = run_shared(cfg, cache, q)
    flips, worst = 0, 0.0
    for i in range(nq):
        ref0, st = decode.decode_step(cfg1, cache, q[i:i + 1])
        if cache.get("cand_ids") is not None:
            for (b, h), s in st.items():
                s["cand"] = cache["cand_ids"][b, h]
        for h in range(cfg.n_heads_kv):
            flips += check_selection(cfg, st, sel[i:i + 1], 0, h)
        ref, _ = decode.decode_step(cfg1, cache, q[i:i + 1], sel_override=sel[i:i + 1])
        rel, mx = check_output(got[i:i + 1], ref, f"{name} query {i}")
        worst = max(worst, rel)
    print(f"\nshared {name}: {nq} queries, worst rel {worst:.2e}, flips {flips}", flush=True)


def test_shared_full_size_sampled():
    """A 262144-token context (one sequence's device-drawn cache) shared by 64
    queries: sampled (query, KV head) pairs against the oracle."""
    from synth import device as sd
    cfg, nq = synth.C3, 64
    g, keff = cfg.gqa, min(cfg.topk, cfg.n_cand)
    lay = sd.draw_layer(cfg, 5151, DEV)
    cache = {k: v[None] for k, v in lay.items()}
    cache["coeff"] = sd.draw_coeff(cfg, 6161, DEV)[None]
    desc = torch.empty((1, cfg.n_heads_kv, cfg.n_chunks), dtype=torch.int32, device=DEV)
    native.resid_chunk_desc(cache["res_idx"], cfg.n_heads_kv, cfg.n_resid, cfg.n_chunks, cfg.chunk, desc)
    cache["res_chunk_desc"] = desc
    q = sd.draw_queries(cfg, nq, 77, DEV)
    out = torch.empty_like(q)
    shape = native.make_shape(cfg, batch=nq)
    ws = torch.empty(native.workspace_bytes(shape), dtype=torch.uint8, device=DEV)
    sel = torch.full((nq, cfg.n_heads_kv, cfg.topk), -7, dtype=torch.int32, device=DEV)
    native.decode_shared(shape, native.make_cache(cache), q, out, ws, sel_out=sel)
    torch.cuda.synchronize()
    got = down_bf16(out)
    sel_h = sel.cpu().numpy()
    assert np.all(np.isfinite(got))
    assert np.all(np.diff(sel_h[..., :keff], axis=-1) > 0)

    def host(t):
        t = t.contiguous().cpu()
        if t.dtype in (torch.bfloat16, torch.int16):
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    q_h = host(q)
    for i, h in [(0, 0), (31, 3), (63, 7)]:
        sl = {k: (host(v) if k == "coeff" else host(v[:, h:h + 1])) for k, v in cache.items() if k != "res_chunk_desc"}
        qs = decode.widen(q_h[i, h * g:(h + 1) * g])
        _, st = decode.decode_head(cfg, sl, qs, 0, 0)
        nflip = check_selection(cfg, {(0, 0): st}, sel_h[i:i + 1, h:h + 1], 0, 0)
        ref, _ = decode.decode_head(cfg, sl, qs, 0, 0, sel_override=sel_h[i, h])
        rel, mx = check_output(got[i, h * g:(h + 1) * g], ref, f"shared c3 q{i} h{h}")
        print(f"shared c3 q{i} h{h}: rel {rel:.2e} max {mx:.2e} flips {nflip}", flush=True)
