"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Every pin uses an independent formulation: a library routine (torch SDPA,
torch GELU, numpy lstsq, numpy stable argsort), a closed form (complex
rotation), a brute force on tiny inputs, or a whole-step invariant of the
method (full rank + all chunks + all residuals == dense attention).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings
from hypothesis import strategies as st

import synth
from oracle import codecs, compress, decode, fixture, steps

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------ codecs --
def test_bf16_golden():
    g = json.load(open(os.path.join(GOLDEN, "codecs.json")))
    for e in g["bf16"]:
        assert codecs.bf16_encode(np.array([e["x"]]))[0] == int(e["bits"], 16), e


def test_bf16_matches_torch_rne():
    x = np.random.default_rng(0).standard_normal(100000) * np.exp(np.random.default_rng(1).uniform(-20, 20, 100000))
    ours = codecs.bf16_encode(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(codecs.bf16_decode(ours), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())


def test_int4_golden():
    g = json.load(open(os.path.join(GOLDEN, "codecs.json")))["int4"]
    packed, sc = codecs.int4_encode(np.array(g["x"])[None, :])
    assert sc[0, 0] == int(g["scale_bits"], 16)
    assert [f"{b:02x}" for b in packed[0, :4]] == g["packed_first4"]
    assert list(codecs.int4_codes(packed)[0, :8]) == g["codes"]
    z, zs = codecs.int4_encode(np.zeros((1, 32)))
    assert zs[0, 0] == 0 and not z.any()


def test_int4_roundtrip_bound():
    x = np.random.default_rng(2).standard_normal((64, 256)) * 3
    p, s = codecs.int4_encode(x)
    y = codecs.int4_decode(p, s)
    scale = np.repeat(codecs.fp16_decode(s), 32, axis=-1)
    absmax = np.repeat(np.abs(x).reshape(64, 8, 32).max(-1), 32, axis=-1)
    assert np.all(np.abs(y - x) <= scale / 2 + absmax * 2.0 ** -10 + 1e-12)
    assert np.all(np.abs(codecs.int4_codes(p)) <= 7)


# -------------------------------------------------------------- RoPE --
def complex_rope(x, pos, theta):
    """RoPE as multiplication of z = x[:h] + i x[h:] by exp(i pos f)."""
    d = x.shape[1]
    h = d // 2
    f = np.exp(-(2.0 * np.arange(h) / d) * math.log(theta))
    z = (x[:, :h] + 1j * x[:, h:]) * np.exp(1j * np.outer(pos, f))
    return np.concatenate([z.real, z.imag], axis=1)


@pytest.mark.parametrize("theta", [1e4, 5e5, 1e6])
def test_rope_complex_form(theta):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((50, 128))
    pos = rng.integers(0, 262144, 50)
    assert np.allclose(steps.rope(x, pos, theta), complex_rope(x, pos, theta), atol=1e-9)


def test_rope_identity_norm_relative():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((20, 128))
    assert np.allclose(steps.rope(x, np.zeros(20), 5e5), x)
    y = steps.rope(x, rng.integers(0, 10 ** 5, 20), 5e5)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1))
    q, k = rng.standard_normal((1, 128)), rng.standard_normal((1, 128))
    for m, n in [(7, 3), (1000, 10), (262143, 100000)]:
        a = steps.rope(q, [m], 5e5) @ steps.rope(k, [n], 5e5).T
        b = steps.rope(q, [m - n], 5e5) @ k.T
        assert np.allclose(a, b, atol=1e-9)


def test_rope_angle_by_atan2():
    d, theta, t = 128, 1e4, 37
    x = np.zeros((d // 2, d))
    x[np.arange(d // 2), np.arange(d // 2)] = 1.0
    y = steps.rope(x, np.full(d // 2, t), theta)
    ang = np.arctan2(y[np.arange(d // 2), np.arange(d // 2) + d // 2], y[np.arange(d // 2), np.arange(d // 2)])
    want = np.mod(t * theta ** (-np.arange(0, d, 2) / d) + np.pi, 2 * np.pi) - np.pi
    assert np.allclose(ang, want, atol=1e-12)


# ------------------------------------------------------- GELU / MLP --
def test_gelu_against_math_erf_and_torch():
    xs = np.linspace(-9, 9, 2001)
    want = np.array([0.5 * v * (1 + math.erf(v / math.sqrt(2))) for v in xs])
    assert np.allclose(steps.gelu(xs), want, atol=1e-15, rtol=1e-14)
    t = torch.nn.functional.gelu(torch.from_numpy(xs), approximate="none").numpy()
    assert np.allclose(steps.gelu(xs), t, atol=1e-15, rtol=1e-14)


def test_value_mlp_against_torch_layers():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((33, 128))
    w1, b1, w2, b2 = rng.standard_normal((256, 128)) * .1, rng.standard_normal(256), rng.standard_normal((128, 256)) * .1, rng.standard_normal(128)
    l1, l2 = torch.nn.Linear(128, 256).double(), torch.nn.Linear(256, 128).double()
    with torch.no_grad():
        l1.weight[:], l1.bias[:], l2.weight[:], l2.bias[:] = map(torch.from_numpy, (w1, b1, w2, b2))
        ref = l2(torch.nn.GELU()(l1(torch.from_numpy(x)))).numpy()
    assert np.allclose(steps.value_mlp(x, w1, b1, w2, b2), ref, atol=1e-12)


# --------------------------------------------------------- attention --
def test_attend_against_torch_sdpa_gqa():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((8, 128))
    k = rng.standard_normal((2, 300, 128))
    v = rng.standard_normal((2, 300, 128))
    ours = np.stack([steps.attend(q[j], k[j // 4], v[j // 4], 1 / math.sqrt(128)) for j in range(8)])
    kk = torch.from_numpy(k).repeat_interleave(4, dim=0)
    vv = torch.from_numpy(v).repeat_interleave(4, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q)[:, None, :], kk, vv)[:, 0].numpy()
    assert np.allclose(ours, ref, atol=1e-12)


def test_attend_special_cases():
    rng = np.random.default_rng(7)
    v = rng.standard_normal((1, 16))
    assert np.allclose(steps.attend(rng.standard_normal(16), rng.standard_normal((1, 16)), v, 1.0), v[0])
    vv = rng.standard_normal((9, 16))
    assert np.allclose(steps.attend(np.zeros(16), rng.standard_normal((9, 16)), vv, 1.0), vv.mean(0))


def test_dense_step_against_sdpa():
    rng = np.random.default_rng(8)
    k = rng.standard_normal((2, 2, 100, 128))
    v = rng.standard_normal((2, 2, 100, 128))
    q = rng.standard_normal((2, 8, 128))
    ours = decode.dense_step(k, v, q, n_heads_kv=2)
    kk = torch.from_numpy(k).repeat_interleave(4, dim=1)
    vv = torch.from_numpy(v).repeat_interleave(4, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q)[:, :, None, :], kk, vv)[:, :, 0].numpy()
    assert np.allclose(ours, ref, atol=1e-12)


def test_decode_without_prefix_is_window_attention():
    """With no compressed prefix (a sequence still inside its first window)
    the decode step has nothing to score or rebuild: it is exact GQA
    attention of the queries over the window's keys and values."""
    cfg = synth.C0.with_(name="window_only", batch=2, ctx=40, window=40, topk=4)
    cache = fixture.build_layer(cfg, 0)
    out, st = decode.decode_step(cfg, cache, cache["q"])
    assert all(len(v["sel"]) == 0 for v in st.values())
    k = torch.from_numpy(decode.widen(cache["win_k"])).repeat_interleave(cfg.gqa, dim=1)
    v = torch.from_numpy(decode.widen(cache["win_v"])).repeat_interleave(cfg.gqa, dim=1)
    q = torch.from_numpy(decode.widen(cache["q"]))[:, :, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v)[:, :, 0].numpy()
    assert np.allclose(out, ref, atol=1e-12)


# ---------------------------------------------------- landmark / topk --
def test_landmark_scores_max_over_group():
    rng = np.random.default_rng(9)
    q, lm = rng.standard_normal((4, 128)), rng.standard_normal((50, 128))
    s = steps.landmark_scores(q, lm)
    for c in range(50):
        assert math.isclose(s[c], max(float(np.dot(q[j], lm[c])) for j in range(4)), rel_tol=1e-12, abs_tol=1e-12)


def topk_by_threshold(s, k):
    """Independent form: all scores above the k-th largest value, then the
    lowest-index ties at that value."""
    n = len(s)
    if k >= n:
        return np.arange(n)
    kth = np.sort(s)[::-1][k - 1]
    above = np.nonzero(s > kth)[0]
    ties = np.nonzero(s == kth)[0][: k - len(above)]
    return np.sort(np.concatenate([above, ties]))


@settings(max_examples=200, deadline=None)
@given(st.lists(st.integers(-5, 5), min_size=1, max_size=60), st.integers(1, 70))
def test_topk_with_ties_against_threshold_form(vals, k):
    s = np.array(vals, dtype=np.float64)
    got = steps.select_topk(s, k)
    assert np.array_equal(got, topk_by_threshold(s, k))
    order = np.argsort(-s, kind="stable")[: min(k, len(s))]
    assert np.array_equal(got, np.sort(order))


def test_topk_candidates_map_ids():
    s = np.array([3.0, 1.0, 3.0, 2.0])
    ids = np.array([4, 9, 11, 20])
    assert list(steps.select_topk(s, 2, ids)) == [4, 11]
    assert list(steps.select_topk(s, 9, ids)) == [4, 9, 11, 20]


# ------------------------------------------------ reconstruction etc. --
def test_reconstruct_is_orthogonal_projection():
    cfg = synth.C0
    B = synth.basis(cfg, 0, 0)
    assert np.allclose(B @ B.T, np.eye(cfg.rank), atol=1e-12)
    x = synth.exact_keys(cfg, 0, 0, 0, 300)
    c = compress.project(x, B)
    cols = synth.layer_cols(cfg, 1, 1)
    got = steps.reconstruct(c, compress.basis_block(B, cols))
    a, *_ = np.linalg.lstsq(B.T, x.T, rcond=None)
    want = (B.T @ a).T[:, cols]
    assert np.allclose(got, want, atol=1e-10)
    # the keys live in the latent subspace: projection leaves only the noise out
    err = np.linalg.norm(got - x[:, cols]) / np.linalg.norm(x[:, cols])
    assert err < 0.1


def test_landmarks_are_chunk_means_of_rotated_keys():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((64, 128))
    lm = compress.landmarks(x, 64, 8, 1e4)
    ref = complex_rope(x, np.arange(64), 1e4)
    for c in range(8):
        assert np.allclose(lm[c], sum(ref[8 * c + i] for i in range(8)) / 8, atol=1e-12)


def test_residual_select_brute_force_and_offsets():
    rng = np.random.default_rng(11)
    cfg = synth.C0
    w = synth.mlp_weights(cfg, 0, 0, 0)
    kp = rng.standard_normal((40, 128))
    v = rng.standard_normal((40, 128))
    v[[3, 17]] = steps.value_mlp(kp[[3, 17]], *w) + 5.0   # two tokens far off, equal error
    idx, rows = compress.residual_select(v, kp, *w, 5)
    errs = [float(np.linalg.norm(v[t] - steps.value_mlp(kp[t:t + 1], *w)[0])) for t in range(40)]
    brute = sorted(sorted(range(40), key=lambda t: (-errs[t], t))[:5])
    assert list(idx) == brute and 3 in idx and 17 in idx
    desc = compress.chunk_descriptors(idx, 5, 8)
    for c in range(5):
        first = sum(1 for t in idx if t < 8 * c)
        bits = sum(1 << (t - 8 * c) for t in idx if 8 * c <= t < 8 * c + 8)
        assert int(desc[c]) == (first << 8) | bits


def test_compress_from_kv_planted_residuals():
    """Values = torch MLP of the rebuilt keys + residuals planted on a known set.

    The rebuilt keys come from the orthogonal projection x B^T B (not the
    oracle's reconstruct); the MLP from torch layers; so the residual rows must
    come back exactly as planted, on exactly the planted tokens, and the
    landmarks / window from the complex-form rotation.
    """
    cfg = synth.C0.with_(name="planted", ctx=256, window=16, resid_frac=6 / 240)
    P, W = cfg.prefix, cfg.window
    assert cfg.n_resid == 6
    rng = np.random.default_rng(12)
    B = synth.basis(cfg, 0, 0)
    x = rng.standard_normal((cfg.ctx, cfg.group_dim))
    c = compress.project(x[:P], B)
    layer, h = 1, 1
    cols = synth.layer_cols(cfg, layer, h)
    k_pre = (x[:P] @ B.T @ B)[:, cols]
    w1, b1, w2, b2 = (np.asarray(a, np.float64) for a in synth.mlp_weights(cfg.with_(bias_std=0.2), 0, layer, h))
    tt = torch.from_numpy
    pred = torch.nn.functional.linear(torch.nn.functional.gelu(torch.nn.functional.linear(tt(k_pre), tt(w1), tt(b1))),
                                      tt(w2), tt(b2)).numpy()
    planted = np.array([3, 40, 41, 100, 177, 239])
    e = np.zeros((cfg.ctx, cfg.head_dim))
    e[planted] = rng.standard_normal((6, cfg.head_dim)) + 2.0
    v = np.concatenate([pred, rng.standard_normal((W, cfg.head_dim))]) + e
    out = compress.compress_from_kv(cfg, x[:, cols], v, c, compress.basis_block(B, cols), (w1, b1, w2, b2),
                                    exact=True)
    assert list(out["res_idx"]) == list(planted)
    assert np.allclose(out["res_val"], e[planted], atol=1e-9)
    rot = complex_rope(x[:, cols], np.arange(cfg.ctx), cfg.rope_theta)
    assert np.allclose(out["landmark"], rot[:P].reshape(-1, 8, cfg.head_dim).mean(axis=1), atol=1e-12)
    assert np.allclose(out["win_k"], rot[P:], atol=1e-12)
    assert np.array_equal(out["win_v"], v[P:])
    for ch in (0, 5, 12, 22, 29):
        first = int(np.sum(planted < 8 * ch))
        bits = sum(1 << int(t - 8 * ch) for t in planted if 8 * ch <= t < 8 * ch + 8)
        assert int(out["res_chunk_desc"][ch]) == (first << 8) | bits


# ------------------------------------------------ whole-step invariants --
def full_cfg():
    """Tiny workload where rank = G*Hkv*d, k = nC and every token has a residual."""
    return synth.C0.with_(name="ns1", ctx=512, window=32, rank=512, topk=10 ** 6, resid_frac=1.0,
                          bias_std=0.1)


def dense_reference(cfg, layer, exact=True):
    """Exact post-RoPE keys (complex form) and exact values of every token.

    The synthetic values come from the predictor's weights as stored (bf16
    unless exact), like the cache they are compared with.
    """
    ks, vs = [], []
    x = synth.exact_keys(cfg, 0, layer // cfg.group_layers)
    for h in range(cfg.n_heads_kv):
        xh = x[:, synth.layer_cols(cfg, layer, h)]
        ks.append(complex_rope(xh, np.arange(cfg.ctx), cfg.rope_theta))
        w = synth.mlp_weights(cfg, 0, layer, h)
        w = w if exact else [codecs.bf16_round(a) for a in w]
        vs.append(compress.exact_values(xh, *w, synth.value_noise(cfg, 0, layer, h), *synth.value_spikes(cfg, 0, layer, h)))
    return np.stack(ks)[None], np.stack(vs)[None]


@pytest.mark.parametrize("layer", [0, 1])
def test_ns1_full_rank_all_chunks_all_residuals_equals_dense(layer):
    cfg = full_cfg()
    cache = fixture.build_layer(cfg, layer, exact=True)
    out, st_ = decode.decode_step(cfg, cache, cache["q"])
    k, v = dense_reference(cfg, layer)
    kk = torch.from_numpy(k).repeat_interleave(cfg.gqa, dim=1)
    vv = torch.from_numpy(v).repeat_interleave(cfg.gqa, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(cache["q"])[:, :, None, :], kk, vv)[:, :, 0].numpy()
    assert np.max(np.abs(out - ref)) < 1e-10
    assert len(st_[(0, 0)]["sel"]) == cfg.n_chunks


def test_ns1_in_bf16_storage_within_rounding():
    cfg = full_cfg()
    cache = fixture.build_layer(cfg, 0)
    out, _ = decode.decode_step(cfg, cache, cache["q"])
    k, v = dense_reference(cfg, 0, exact=False)
    q = codecs.bf16_decode(cache["q"])
    ref = decode.dense_step(k, v, q, cfg.n_heads_kv)
    rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert rel < 1e-2, rel


def test_ns3_mlp_plus_residual_reproduces_values():
    cfg = full_cfg().with_(resid_frac=0.25)
    for exact in (True, False):
        cache = fixture.build_layer(cfg, 0, exact=exact)
        _, st_ = decode.decode_step(cfg, cache, cache["q"])
        _, v = dense_reference(cfg, 0, exact)
        for h in range(cfg.n_heads_kv):
            s = st_[(0, h)]
            ridx = cache["res_idx"][0, h]
            pos = np.nonzero(np.isin(s["tokens"], ridx))[0]
            assert len(pos) == len(ridx)
            got, want = s["v_hat"][pos], v[0, h][s["tokens"][pos]]
            if exact:
                assert np.max(np.abs(got - want)) < 1e-10
            else:
                r = want - steps.value_mlp(s["k_pre"][pos], *[codecs.bf16_decode(cache[n][0, h]) for n in ("w1", "b1", "w2", "b2")])
                assert np.all(np.abs(got - want) <= np.abs(r) * 2.0 ** -8 + 1e-12)


# ----------------------------- top-k smaller than the candidate count --
def subset_cfg(evict: bool, resid_frac: float = 1.0):
    """Full rank and exact storage as in full_cfg, but k below the number of
    candidates, so only a strict subset of the prefix is rebuilt (the review's
    keys paragraph: only the top-k chunks are rebuilt, at their positions)."""
    return full_cfg().with_(name="subset_ev" if evict else "subset", topk=7, evict=evict,
                            resid_frac=resid_frac)


def brute_topk(scores, ids, k):
    """Chunk ids whose score is beaten (or tied by a lower id) fewer than k times."""
    n = len(scores)
    keep = [int(ids[i]) for i in range(n)
            if sum(1 for j in range(n) if scores[j] > scores[i] or (scores[j] == scores[i] and ids[j] < ids[i])) < k]
    return sorted(keep)


def subset_reference(cfg, cache, layer):
    """Torch SDPA over the exact post-RoPE keys (complex form) and exact values
    of exactly the brute-force top-k chunks' tokens and the window."""
    k, v = dense_reference(cfg, layer)
    q = cache["q"][0]
    g, P, S = cfg.gqa, cfg.prefix, cfg.chunk
    out = np.zeros((1, cfg.n_heads_q, cfg.head_dim))
    sels = []
    for h in range(cfg.n_heads_kv):
        lm = cache["landmark"][0, h]
        ids = cache["cand_ids"][0, h] if cfg.evict else np.arange(cfg.n_chunks)
        s = [max(sum(float(q[j, i]) * float(lm[c, i]) for i in range(cfg.head_dim)) for j in range(h * g, (h + 1) * g))
             for c in range(len(lm))]
        sel = brute_topk(s, ids, cfg.topk)
        tok = [S * c + i for c in sel for i in range(S)] + list(range(P, cfg.ctx))
        kk = torch.from_numpy(k[0, h][tok])[None]
        vv = torch.from_numpy(v[0, h][tok])[None]
        qq = torch.from_numpy(q[h * g:(h + 1) * g])[:, None, :]
        out[0, h * g:(h + 1) * g] = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv)[:, 0].numpy()
        sels.append(sel)
    return out, sels


@pytest.mark.parametrize("evict", [False, True])
@pytest.mark.parametrize("layer", [0, 1])
def test_subset_full_rank_all_residuals_equals_sdpa_over_selected(layer, evict):
    cfg = subset_cfg(evict)
    assert cfg.topk < cfg.n_cand
    cache = fixture.build_layer(cfg, layer, exact=True)
    out, st_ = decode.decode_step(cfg, cache, cache["q"])
    ref, sels = subset_reference(cfg, cache, layer)
    for h in range(cfg.n_heads_kv):
        assert list(st_[(0, h)]["sel"]) == sels[h]
        assert sels[h] != list(range(cfg.topk))      # not simply the first chunks
    assert np.max(np.abs(out - ref)) < 1e-10


def _mut_rope_at_list_positions(mp):
    mp.setattr(decode, "rope", lambda x, pos, theta: steps.rope(x, np.arange(len(pos)), theta))


def _mut_residual_rows_by_list_index(mp):
    mp.setattr(decode, "residual_hits", lambda tokens, ridx: (np.arange(len(tokens)), np.arange(len(tokens))))


def _mut_dropped_chunk(mp):
    mp.setattr(decode, "select_topk", lambda s, k, c=None: steps.select_topk(s, k, c)[:-1])


def _mut_candidate_positions_as_ids(mp):
    mp.setattr(decode, "select_topk", lambda s, k, c=None: steps.select_topk(s, k, None))


@pytest.mark.parametrize("mutate,evict", [(_mut_rope_at_list_positions, False),
                                          (_mut_residual_rows_by_list_index, False),
                                          (_mut_dropped_chunk, False),
                                          (_mut_candidate_positions_as_ids, True)])
def test_subset_pin_catches_planted_mistakes(monkeypatch, mutate, evict):
    """Each planted mistake in the oracle's subset path fails the SDPA pin."""
    cfg = subset_cfg(evict)
    cache = fixture.build_layer(cfg, 1, exact=True)
    ref, _ = subset_reference(cfg, cache, 1)
    with monkeypatch.context() as mp:
        mutate(mp)
        bad, _ = decode.decode_step(cfg, cache, cache["q"])
    assert not np.max(np.abs(bad - ref)) < 1e-3


def _ns3_subset_check(cfg, cache, v, w):
    """Selected residual tokens come back as exact V; the other selected tokens
    as the torch MLP of their exact (full-rank) keys."""
    x = synth.exact_keys(cfg, 0, 0)
    _, st_ = decode.decode_step(cfg, cache, cache["q"])
    n_hit = n_miss = 0
    for h in range(cfg.n_heads_kv):
        s = st_[(0, h)]
        tok = s["tokens"]
        has = np.isin(tok, cache["res_idx"][0, h])
        tt = torch.from_numpy
        w1, b1, w2, b2 = (tt(np.asarray(a, np.float64)) for a in w[h])
        pred = torch.nn.functional.linear(torch.nn.functional.gelu(torch.nn.functional.linear(
            tt(x[tok][:, synth.layer_cols(cfg, 0, h)]), w1, b1)), w2, b2).numpy()
        if np.max(np.abs(s["v_hat"][has] - v[0, h][tok[has]]), initial=0) >= 1e-10:
            return False
        if np.max(np.abs(s["v_hat"][~has] - pred[~has]), initial=0) >= 1e-10:
            return False
        n_hit, n_miss = n_hit + has.sum(), n_miss + (~has).sum()
    assert n_hit > 0 and n_miss > 0
    return True


def test_ns3_subset_mlp_plus_residual_reproduces_values(monkeypatch):
    """NS-3 with k below the candidates and a quarter of the tokens holding
    residuals: the rows are found for a strict subset of the prefix."""
    cfg = subset_cfg(False, resid_frac=0.25)
    cache = fixture.build_layer(cfg, 0, exact=True)
    _, v = dense_reference(cfg, 0)
    w = [synth.mlp_weights(cfg, 0, 0, h) for h in range(cfg.n_heads_kv)]
    assert _ns3_subset_check(cfg, cache, v, w)
    # planted: the hit rows matched to the rebuilt tokens in list order
    with monkeypatch.context() as mp:
        mp.setattr(decode, "residual_hits",
                   lambda tokens, ridx: (np.arange(int(np.isin(ridx, tokens).sum())), np.nonzero(np.isin(ridx, tokens))[0]))
        assert not _ns3_subset_check(cfg, cache, v, w)


def test_eviction_that_evicts_nothing_is_the_plain_path():
    cfg = synth.C0
    cache = fixture.build_layer(cfg, 0)
    out0, _ = decode.decode_step(cfg, cache, cache["q"])
    c2 = dict(cache)
    c2["cand_ids"] = np.broadcast_to(np.arange(cfg.n_chunks, dtype=np.int32), (1, cfg.n_heads_kv, cfg.n_chunks)).copy()
    out1, _ = decode.decode_step(cfg, c2, cache["q"])
    assert np.array_equal(out0, out1)


def test_selection_override_matches_own_selection():
    cfg = synth.C0
    cache = fixture.build_layer(cfg, 1)
    out0, st_ = decode.decode_step(cfg, cache, cache["q"])
    sel = [[st_[(0, h)]["sel"] for h in range(cfg.n_heads_kv)]]
    out1, _ = decode.decode_step(cfg, cache, cache["q"], sel_override=sel)
    assert np.array_equal(out0, out1)


def test_needle_chunk_is_selected():
    cfg = synth.C2.with_(name="needle_small", batch=1, ctx=8192, window=128, n_layers=4, rank=128, topk=16)
    cache = fixture.build_layer(cfg, 1)
    _, st_ = decode.decode_step(cfg, cache, cache["q"])
    for h in range(cfg.n_heads_kv):
        assert cache["needle"][0, h] in st_[(0, h)]["sel"]


def test_int4_eviction_cache_decodes():
    cfg = synth.C4.with_(name="c4_small", batch=1, ctx=4096, window=64, n_layers=4, topk=32)
    cache = fixture.build_layer(cfg, 2)
    assert cache["coeff"].dtype == np.uint8 and cache["coeff"].shape == (1, cfg.prefix, cfg.rank // 2)
    assert cache["landmark"].shape[2] == cfg.n_cand == cfg.n_chunks - cfg.n_chunks // 2
    assert np.all(cache["cand_ids"][0, :, :4] == np.arange(4))
    out, st_ = decode.decode_step(cfg, cache, cache["q"])
    assert np.all(np.isfinite(out))
    for h in range(cfg.n_heads_kv):
        assert np.all(np.isin(st_[(0, h)]["sel"], cache["cand_ids"][0, h]))


def test_append_chunk_matches_a_longer_build():
    """Rolling the first window chunk into the prefix gives that chunk the
    landmark a build over the longer prefix gives it, and residuals exactly
    for the tokens whose error reaches the build threshold (brute force)."""
    cfg = synth.C0.with_(name="roll", ctx=512, window=64, resid_frac=0.125, bias_std=0.1)
    longer = cfg.with_(name="roll2", window=56)
    P, layer, h = cfg.prefix, 1, 0
    x = synth.exact_keys(cfg, 0, 0)
    B = synth.basis(cfg, 0, 0)
    cols = synth.layer_cols(cfg, layer, h)
    w = synth.mlp_weights(cfg.with_(bias_std=0.1), 0, layer, h)
    v = compress.exact_values(x[:, cols], *w, synth.value_noise(cfg, 0, layer, h), *synth.value_spikes(cfg, 0, layer, h))
    blk = compress.basis_block(B, cols)
    c = compress.project(x, B)
    base = compress.compress_from_kv(cfg, x[:, cols], v, c[:P], blk, w, exact=True)
    big = compress.compress_from_kv(longer, x[:, cols], v, c[:P + 8], blk, w, exact=True)
    app = compress.append_chunk(x[P:P + 8, cols], v[P:P + 8], c[P:P + 8], blk, *w, base["res_thresh"], P,
                                cfg.rope_theta)
    assert np.allclose(app["landmark"], big["landmark"][-1], atol=1e-12)
    assert np.allclose(app["landmark"], complex_rope(x[P:P + 8, cols], np.arange(P, P + 8), cfg.rope_theta).mean(0),
                       atol=1e-12)
    # brute force: the error of each new token against the build threshold
    pred = steps.value_mlp((c[P:P + 8] @ B)[:, cols], *w)
    errs = [float(np.linalg.norm(v[P + i] - pred[i])) for i in range(8)]
    assert list(app["keep"]) == [i for i in range(8) if errs[i] >= base["res_thresh"]]
    assert np.allclose(app["rows"], (v[P:P + 8] - pred)[app["keep"]], atol=1e-10)
    # the threshold is the nR-th largest prefix error
    assert np.sum(base["errors"] >= base["res_thresh"]) == cfg.n_resid


# ------------------------------------------------------------- basis fit --
def test_cholqr_equals_householder_qr():
    """Cholesky-QR equals LAPACK's Householder QR with the diagonal of R made positive."""
    from oracle import basis
    rng = np.random.default_rng(21)
    y = rng.standard_normal((300, 40)) @ np.diag(np.logspace(0, 2, 40))
    q, r = basis.cholqr(y)
    q2, r2 = np.linalg.qr(y)
    s = np.sign(np.diag(r2))
    assert np.allclose(q, q2 * s, atol=1e-10)
    assert np.allclose(r, s[:, None] * r2, atol=1e-9)


def test_randomized_basis_against_exact_svd():
    """On the synthetic keys (a 64-dimensional latent subspace plus noise) the
    randomised Cholesky-QR basis is orthonormal, contains the latent subspace
    (the SVD's top 64 directions) to within a small angle, and its projection
    error is within 1% of the SVD optimum, which it cannot beat (Eckart-Young)."""
    from oracle import basis
    cfg = synth.C0.with_(name="fit", rank=128)
    x = synth.exact_keys(cfg, 0, 0)[: cfg.prefix]
    rng = np.random.default_rng(22)
    omega = rng.standard_normal((cfg.prefix, cfg.rank))
    b_r = basis.randomized_cholqr(x, omega)
    b_s = basis.svd_basis(x, cfg.rank)
    assert np.allclose(b_r @ b_r.T, np.eye(cfg.rank), atol=1e-12)
    assert basis.max_angle(b_s[:64], b_r) < 1e-3
    e_r, e_s = basis.projection_error(x, b_r), basis.projection_error(x, b_s)
    assert e_s <= e_r + 1e-12
    assert e_r <= 1.05 * e_s
    # without the power pass the sketch is visibly worse; a second pass does not hurt
    b_0 = basis.randomized_cholqr(x, omega, power=0)
    assert basis.projection_error(x, b_0) > 1.2 * e_s and basis.max_angle(b_s[:64], b_0) > 1e-2
    b_2 = basis.randomized_cholqr(x, omega, power=2)
    assert basis.projection_error(x, b_2) <= e_r + 1e-12


def test_randomized_basis_downstream_decode():
    """Decode with a cache compressed in the randomised basis matches decode with
    the exact-SVD basis: both within bf16-scale distance of dense attention on
    the exact keys, and of each other."""
    from oracle import basis, fixture
    cfg = synth.C0.with_(name="fit2", ctx=1024, window=32, rank=128, topk=10 ** 6, resid_frac=1.0)
    layer = 1
    x = synth.exact_keys(cfg, 0, 0)
    rng = np.random.default_rng(23)
    omega = rng.standard_normal((cfg.prefix, cfg.rank))
    outs = {}
    for name, B in (("svd", basis.svd_basis(x[: cfg.prefix], cfg.rank)),
                    ("rand", basis.randomized_cholqr(x[: cfg.prefix], omega))):
        cache = fixture.build_layer_with_basis(cfg, layer, B)
        outs[name], _ = decode.decode_step(cfg, cache, cache["q"])
    k, v, q = fixture.dense_layer(cfg, layer)
    dense = decode.dense_step(codecs.bf16_decode(k), codecs.bf16_decode(v), codecs.bf16_decode(q), cfg.n_heads_kv)
    for name in outs:
        assert np.linalg.norm(outs[name] - dense) / np.linalg.norm(dense) < 2e-2, name
    assert np.linalg.norm(outs["svd"] - outs["rand"]) / np.linalg.norm(outs["svd"]) < 1e-2
