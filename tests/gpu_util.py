"""Test helpers: move oracle-fixture caches to the GPU and apply the parity rule."""
import numpy as np
import torch

from long_context_decode_landmark_amd import native
from oracle import codecs, decode

DEV = torch.device("cuda:0")

# parity bar of the decode step
SEL_BAND = 1e-3      # relative band around the k-th score inside which set differences are ties
REL_L2 = 1e-2
MAX_ABS = 3e-2


def up(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV)
    return torch.from_numpy(a).to(DEV)


def down_bf16(t):
    """bf16 bits (int16 or bfloat16 tensor) -> fp64 numpy."""
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return codecs.bf16_decode(t.cpu().numpy().view(np.uint16))


def cache_to_device(cache):
    return {k: up(v) for k, v in cache.items() if k not in ("q", "needle")}


def run_gpu(cfg, cache, stages=False, nb=None, attend=None, pipe_cus=None):
    """Run the library on a fixture cache; returns (out fp64, sel, stage dict).

    attend: None (the library's own choice of kernel for the selected chunks),
    "pipe" (producer/consumer kernel) or "wave" (4-wave kernel); calls with
    stage outputs always take the 4-wave kernel.  pipe_cus: plan the
    producer/consumer kernel for that many CUs (fewer, longer workgroups)."""
    import os
    env = {"LOWRAM_ATTEND": attend, "LOWRAM_PIPE_CUS": None if pipe_cus is None else str(pipe_cus)}
    old = {k: os.environ.get(k) for k in env}
    for k, v in env.items():
        if v is not None:
            os.environ[k] = v
    try:
        return _run_gpu(cfg, cache, stages, nb)
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def _run_gpu(cfg, cache, stages, nb):
    nb = cache["q"].shape[0] if nb is None else nb
    t = cache_to_device(cache)
    q = up(cache["q"])
    out = torch.empty_like(q)
    shape = native.make_shape(cfg, batch=nb)
    ws = torch.empty(native.workspace_bytes(shape), dtype=torch.uint8, device=DEV)
    sel = torch.full((nb, cfg.n_heads_kv, cfg.topk), -7, dtype=torch.int32, device=DEV)
    st = {}
    if stages:
        keff = min(cfg.topk, cfg.n_cand)
        st["scores"] = torch.empty((nb, cfg.n_heads_kv, cfg.n_cand), dtype=torch.float32, device=DEV)
        for n in ("kpre", "kpost", "vhat"):
            st[n] = torch.empty((nb, cfg.n_heads_kv, keff * cfg.chunk, cfg.head_dim), dtype=torch.float32, device=DEV)
        native.decode_stages(shape, t, q, out, ws, sel_out=sel, **st)
    else:
        native.decode_step(shape, t, q, out, ws, sel_out=sel)
    torch.cuda.synchronize()
    return down_bf16(out), sel.cpu().numpy(), {k: v.cpu().numpy() for k, v in st.items()}


def check_selection(cfg, stages_oracle, sel_gpu, b, h):
    """Sets equal except chunks whose oracle score is within the tie band of the k-th."""
    s = stages_oracle[(b, h)]
    so = set(int(c) for c in s["sel"])
    sg = set(int(c) for c in sel_gpu[b, h] if c >= 0)
    keff = min(cfg.topk, cfg.n_cand)
    assert len(sg) == keff, (b, h, len(sg), keff)
    assert list(sel_gpu[b, h][:keff]) == sorted(sg), "GPU selection not ascending"
    assert all(c == -1 for c in sel_gpu[b, h][keff:])
    diff = so ^ sg
    if not diff:
        return 0
    scores = s["scores"]
    ids = np.arange(len(scores)) if "cand" not in s else s["cand"]
    by_id = {int(c): float(v) for c, v in zip(ids, scores)}
    sk = np.sort(scores)[::-1][keff - 1]
    band = SEL_BAND * abs(sk) if abs(sk) >= 1e-6 else 1e-6 * float(np.max(np.abs(scores)))
    for c in diff:
        assert abs(by_id[c] - sk) <= band, (b, h, c, by_id[c], sk)
    return len(diff)


def check_output(got, ref, what=""):
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    mx = float(np.max(np.abs(got - ref)))
    assert np.all(np.isfinite(got)), what
    assert rel <= REL_L2 and mx <= MAX_ABS, (what, rel, mx)
    return rel, mx


def oracle_with_cands(cfg, cache, stages):
    """Attach candidate ids to the oracle stages (eviction) for the tie check."""
    if cache.get("cand_ids") is not None:
        for (b, h), s in stages.items():
            s["cand"] = cache["cand_ids"][b, h]
    return stages


def full_parity(cfg, cache, stages=True, nb=None):
    """Run GPU + oracle on a cache and check selection, stages and output."""
    got, sel, st = run_gpu(cfg, cache, stages=stages, nb=nb)
    ref0, ost = decode.decode_step(cfg, cache, cache["q"])
    oracle_with_cands(cfg, cache, ost)
    nflip = 0
    for (b, h) in ost:
        nflip += check_selection(cfg, ost, sel, b, h)
    ref, ost2 = decode.decode_step(cfg, cache, cache["q"], sel_override=sel)
    rel, mx = check_output(got, ref, cfg.name)
    return dict(got=got, ref=ref, sel=sel, gpu_stages=st, oracle_stages=ost2, oracle_own_stages=ost, rel=rel,
                max_abs=mx, flips=nflip)
