"""GPU checks of the dense baseline and of the residual-descriptor helper.

dense_decode_step against the oracle's dense GQA attention (same tolerance
as the decode step), and lowram_resid_chunk_desc bit-exact against the
oracle side's descriptor construction, on seeded inputs.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

from gpu_util import DEV, check_output, down_bf16, up  # noqa: E402
from long_context_decode_landmark_amd import native  # noqa: E402
from oracle import compress, decode, fixture  # noqa: E402


def run_dense(cfg, k, v, q):
    nb = q.shape[0]
    kd, vd, qd = up(k), up(v), up(q)
    out = torch.empty_like(qd)
    ds = native.dense_shape(nb, cfg.ctx, cfg.n_heads_q, cfg.n_heads_kv, cfg.head_dim)
    ws = torch.empty(native.dense_workspace_bytes(ds), dtype=torch.uint8, device=DEV)
    native.dense_decode_step(ds, kd, vd, qd, out, ws)
    torch.cuda.synchronize()
    return down_bf16(out)


@pytest.mark.parametrize("name,over", [
    ("c0", {}),
    ("ragged_ctx", {"ctx": 5003, "window": 3}),      # context not a multiple of the 2048-token split
    ("gqa1", {"n_heads_q": 2}),
    ("gqa16_batch2", {"n_heads_q": 32, "batch": 2}),
])
def test_dense_matches_oracle(name, over):
    cfg = synth.C0.with_(name=f"dense_{name}", **over)
    k, v, q = fixture.dense_layer(cfg, 0)
    got = run_dense(cfg, k, v, q)
    ref = decode.dense_step(k, v, q, cfg.n_heads_kv)
    rel, mx = check_output(got, ref, name)
    print(f"dense {name}: rel {rel:.2e} max {mx:.2e}")


def test_dense_full_size_sampled_heads():
    """The 262144-token dense step at batch 8 (128 splits of 2048 tokens per
    head, the launch the benchmark times), K/V/q drawn as the benchmark draws
    them; sampled (sequence, KV head) slices against the oracle."""
    nb, T, hq, hkv, d = 8, 262144, 32, 8, 128
    g_ = torch.Generator(device=DEV)
    g_.manual_seed(77)
    k = torch.randn((nb, hkv, T, d), generator=g_, device=DEV, dtype=torch.bfloat16)
    v = torch.randn((nb, hkv, T, d), generator=g_, device=DEV, dtype=torch.bfloat16)
    q = torch.randn((nb, hq, d), generator=g_, device=DEV, dtype=torch.bfloat16)
    out = torch.empty_like(q)
    ds = native.dense_shape(nb, T, hq, hkv, d)
    ws = torch.empty(native.dense_workspace_bytes(ds), dtype=torch.uint8, device=DEV)
    native.dense_decode_step(ds, k, v, q, out, ws)
    torch.cuda.synchronize()
    got = down_bf16(out)
    assert np.all(np.isfinite(got))
    gq = hq // hkv
    bits = lambda t: t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    for b, h in [(0, 0), (3, 5), (7, 7)]:
        ref = decode.dense_step(bits(k[b:b + 1, h:h + 1]), bits(v[b:b + 1, h:h + 1]),
                                bits(q[b:b + 1, h * gq:(h + 1) * gq]), 1)
        rel, mx = check_output(got[b:b + 1, h * gq:(h + 1) * gq], ref, f"dense 262k b{b} h{h}")
        print(f"dense 262k b{b} h{h}: rel {rel:.2e} max {mx:.2e}", flush=True)
    del k, v
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n_chunks,n_resid,seed", [(5000, 625, 0), (4096, 0, 1), (777, 777 * 8, 2), (1, 3, 3),
                                                    (32736, 32736, 4)])
def test_resid_chunk_desc_matches_oracle(n_chunks, n_resid, seed):
    rng = np.random.default_rng(seed)
    n_lists = 3
    P = n_chunks * 8
    idx = np.stack([np.sort(rng.choice(P, size=n_resid, replace=False)) for _ in range(n_lists)]).astype(np.int32)
    ref = np.stack([compress.chunk_descriptors(idx[i], n_chunks, 8) for i in range(n_lists)])
    out = torch.full((n_lists, n_chunks), -1, dtype=torch.int32, device=DEV)
    native.resid_chunk_desc(up(idx), n_lists, n_resid, n_chunks, 8, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, ref)
