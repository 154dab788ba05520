"""The select kernel bit for bit against the oracle's top-k, on exact ties.

Landmark rows repeat a few distinct rows (chunk c takes row c mod n_rows of
its head), so whole groups of chunks score exactly the same while distinct
scores next to the k-th stay far apart (checked: well beyond fp32 rounding).  The k highest
with ties to the lower chunk id are then unique and the GPU's fp32 scores
order them as the oracle's fp64 ones do: the selection must equal
steps.select_topk exactly, with no tie band.  The list lengths cover the
variant that keeps each thread's keys in registers at 32, 8 and 1 keys per
thread (32736, 5000 and 1000 candidates; 5000 is not a multiple of its
ranges), 8191 candidates at 8 per thread (the first list's last 16-byte piece
is partial, and the other lists start off 16-byte alignment, so their keys are
loaded one at a time), the variant that re-reads them from L2 (40960
candidates, 64 per thread), k above the candidate count, and a selection that
ends inside a group of up to ~5800 equal scores (7 distinct rows).
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

from gpu_util import DEV  # noqa: E402
from long_context_decode_landmark_amd import native  # noqa: E402
from oracle import decode, steps  # noqa: E402
from synth import device as sd  # noqa: E402
from test_gpu_fullsize import draw_batch, host  # noqa: E402


@pytest.mark.parametrize("name,n_cand,window,topk,n_rows", [
    ("regs_32_per_thread", 32736, 256, 1024, 7),
    ("regs_32_per_thread_60_rows", 32736, 256, 1024, 60),
    ("regs_8_per_thread_ragged", 5000, 64, 45, 11),
    ("regs_8_per_thread_unaligned", 8191, 64, 300, 13),
    ("regs_1_per_thread", 1000, 64, 32, 5),
    ("l2_64_per_thread", 40960, 256, 1024, 7),
    ("k_above_candidates", 300, 64, 512, 3),
])
def test_select_equals_oracle_topk_on_exact_ties(name, n_cand, window, topk, n_rows):
    nb = 2
    cfg = synth.C3.with_(name=f"select_{name}", batch=nb, n_heads_q=8, n_heads_kv=2, rank=64,
                         ctx=n_cand * synth.C3.chunk + window, window=window, topk=topk)
    assert cfg.n_cand == n_cand
    print(f"\n{name}: drawing", flush=True)
    cache = draw_batch(cfg, nb, seed=515)
    rows = torch.arange(n_cand, device=DEV) % n_rows
    cache["landmark"] = cache["landmark"][:, :, rows].contiguous()
    q = sd.draw_queries(cfg, nb, 616, DEV)
    out = torch.empty_like(q)
    shape = native.make_shape(cfg, batch=nb)
    ws = torch.empty(native.workspace_bytes(shape), dtype=torch.uint8, device=DEV)
    sel = torch.full((nb, cfg.n_heads_kv, topk), -7, dtype=torch.int32, device=DEV)
    native.decode_step(shape, native.make_cache(cache), q, out, ws, sel_out=sel)
    torch.cuda.synchronize()
    sel_h = sel.cpu().numpy()
    q_h, lm_h = host(q), host(cache["landmark"])
    g, keff = cfg.gqa, min(topk, n_cand)
    for b in range(nb):
        for h in range(cfg.n_heads_kv):
            sc = steps.landmark_scores(decode.widen(q_h[b, h * g:(h + 1) * g]), decode.widen(lm_h[b, h]))
            # the set depends only on how the k-th score T orders against its
            # neighbouring distinct values: those must be far apart
            distinct = np.unique(sc[:n_rows])
            assert len(distinct) == n_rows
            kth = np.sort(sc)[::-1][keff - 1]
            at = int(np.searchsorted(distinct, kth))
            for nb_ in (at - 1, at + 1):
                if 0 <= nb_ < len(distinct):
                    gap = abs(distinct[nb_] - kth) / max(abs(kth), 1e-30)
                    assert gap > 1e-4, f"rows next to the k-th score too close to order ({gap:.1e})"
            want = steps.select_topk(sc, topk)
            assert np.array_equal(sel_h[b, h, :keff], want), f"{name} b{b} h{h}"
            assert np.all(sel_h[b, h, keff:] == -1)
    print(f"{name}: {nb * cfg.n_heads_kv} lists equal to the oracle's top-{topk}", flush=True)


@pytest.mark.parametrize("name,n_cand,m_top", [
    ("exit_after_first_pass", 32736, 3),
    ("bin_at_the_lower_bound", 8192, 1),
    ("l2_exit_after_first_pass", 40960, 5),
])
def test_select_whole_bin(name, n_cand, m_top):
    """Landmark row c of a head is one base row times 2^(c mod 8) (exact in
    bf16, and every score is then exactly 2^(c mod 8) times one value in fp32
    too), so the 8 distinct scores differ in their exponent and each fills a
    first-pass bin of its own, with n_cand / 8 copies.  k is the number of
    chunks whose score is among the m_top highest: the bin of the k-th key
    holds exactly the keys still needed after the first pass.  At 32736 and
    40960 candidates (the register and L2 variants) the passes stop there; at
    8192 with m_top = 1 the lower bound on the k-th key equals that key, the
    bin starts below it, and all three passes run.  Either way the selection
    is every chunk of the m_top highest rows, equal to the oracle's top-k."""
    nb, n_rows = 2, 8
    cfg0 = synth.C3.with_(name=f"select_{name}", batch=nb, n_heads_q=8, n_heads_kv=2, rank=64,
                          ctx=n_cand * synth.C3.chunk + 64, window=64, topk=1024)
    assert cfg0.n_cand == n_cand and n_cand % n_rows == 0
    print(f"\n{name}: drawing", flush=True)
    cache = draw_batch(cfg0, nb, seed=717)
    scale = torch.pow(2.0, (torch.arange(n_cand, device=DEV) % n_rows).float()).to(torch.bfloat16)
    cache["landmark"] = (cache["landmark"][:, :, :1] * scale[None, None, :, None]).contiguous()
    q = sd.draw_queries(cfg0, nb, 818, DEV)
    topk = m_top * (n_cand // n_rows)
    cfg = cfg0.with_(topk=topk)
    out = torch.empty_like(q)
    shape = native.make_shape(cfg, batch=nb)
    ws = torch.empty(native.workspace_bytes(shape), dtype=torch.uint8, device=DEV)
    sel = torch.full((nb, cfg.n_heads_kv, topk), -7, dtype=torch.int32, device=DEV)
    native.decode_step(shape, native.make_cache(cache), q, out, ws, sel_out=sel)
    torch.cuda.synchronize()
    sel_h = sel.cpu().numpy()
    q_h, lm_h = host(q), host(cache["landmark"])
    g = cfg.gqa
    for b in range(nb):
        for h in range(cfg.n_heads_kv):
            sc = steps.landmark_scores(decode.widen(q_h[b, h * g:(h + 1) * g]), decode.widen(lm_h[b, h]))
            distinct = np.unique(sc)
            assert len(distinct) == n_rows and sc[0] != 0.0
            want = steps.select_topk(sc, topk)
            assert np.array_equal(np.sort(sc[want]), np.sort(sc[sc >= distinct[-m_top]]))  # whole groups
            assert np.array_equal(sel_h[b, h], want), f"{name} b{b} h{h}"
    print(f"{name}: {nb * cfg.n_heads_kv} lists equal to the oracle's top-{topk}", flush=True)
