"""One LowRAM decode step, and the dense baseline, in plain fp64 (test infrastructure).

decode_step follows the order the LowRAM pages give for decoding
[review/keys; explainer/how "Selective reconstruction"; abstract]:

  1. candidates   every prefix chunk, or the survivors of an eviction mask
                  (the LowRAM-E / -EQ compositions of the review's tables)
  2. score        each candidate's landmark against the KV head's queries
  3. select       the top-k chunks
  4. rebuild      pre-RoPE keys of the selected tokens from coefficients x basis
  5. RoPE         rotate the rebuilt keys at their token positions
  6. values       value MLP on the rebuilt pre-RoPE keys, plus the stored
                  residual of every selected token that has one
  7. attend       GQA softmax attention of each query head over the selected
                  tokens and the exact recent window

Cache arrays are read in the layout the GPU library takes (one layer, batch
major); bf16 arrays arrive as uint16 bit patterns and are widened exactly,
float arrays (the exact-storage mode of the invariant tests) are used as is.
"""
from __future__ import annotations

import numpy as np

from . import codecs
from .steps import attend, landmark_scores, reconstruct, rope, select_topk, value_mlp


def widen(a) -> np.ndarray:
    """Stored array -> fp64: bf16 bit patterns are decoded, floats pass."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return codecs.bf16_decode(a)
    return a.astype(np.float64)


def coeff_rows(cfg, cache, b: int, tokens: np.ndarray) -> np.ndarray:
    """Coefficient rows C[t, :] of the given tokens (dequantised if int4)."""
    if cfg.int4:
        return codecs.int4_decode(cache["coeff"][b][tokens], cache["coeff_scale"][b][tokens])
    return widen(cache["coeff"][b][tokens])


def resid_rows(cfg, cache, b: int, h: int, rows: np.ndarray) -> np.ndarray:
    if cfg.int4:
        return codecs.int4_decode(cache["res_val"][b, h][rows], cache["res_scale"][b, h][rows])
    return widen(cache["res_val"][b, h][rows])


def residual_hits(tokens: np.ndarray, ridx: np.ndarray):
    """Which rebuilt tokens have a stored residual, and where it is stored.

    Returns (at, rows): tokens[at[n]] == ridx[rows[n]] for every stored row
    whose token is among ``tokens``; the row is found by the token id it
    names, never by its place in either list.
    """
    rows = np.nonzero(np.isin(ridx, tokens))[0]
    where = {int(t): i for i, t in enumerate(tokens)}
    at = np.array([where[int(t)] for t in ridx[rows]], dtype=np.int64)
    return at, rows


def decode_head(cfg, cache, q_b: np.ndarray, b: int, h: int, sel_override=None):
    """Decode step of one (sequence, KV head); returns (out [g][d], stages)."""
    g, S = cfg.gqa, cfg.chunk
    qg = q_b[h * g:(h + 1) * g]
    cand = cache.get("cand_ids")
    cand_h = None if cand is None else np.asarray(cand[b, h])
    lm = widen(cache["landmark"][b, h])

    scores = landmark_scores(qg, lm)                                     # step 2
    if sel_override is None:
        sel = select_topk(scores, cfg.topk, cand_h)                      # step 3
    else:
        sel = np.asarray(sel_override, dtype=np.int64)
        sel = np.sort(sel[sel >= 0])
    tokens = (sel[:, None] * S + np.arange(S)[None, :]).reshape(-1)

    k_pre = reconstruct(coeff_rows(cfg, cache, b, tokens), widen(cache["basis"][b, h]))  # step 4
    k_post = rope(k_pre, tokens, cfg.rope_theta)                         # step 5
    v_hat = value_mlp(k_pre, widen(cache["w1"][b, h]), widen(cache["b1"][b, h]),
                      widen(cache["w2"][b, h]), widen(cache["b2"][b, h]))  # step 6
    at, rows = residual_hits(tokens, np.asarray(cache["res_idx"][b, h]))
    if len(rows):
        v_hat[at] += resid_rows(cfg, cache, b, h, rows)

    keys = np.concatenate([k_post, widen(cache["win_k"][b, h])], axis=0)  # step 7
    vals = np.concatenate([v_hat, widen(cache["win_v"][b, h])], axis=0)
    scale = 1.0 / np.sqrt(cfg.head_dim)
    out = np.stack([attend(qg[j], keys, vals, scale) for j in range(g)])
    stages = dict(scores=scores, sel=sel, tokens=tokens, k_pre=k_pre, k_post=k_post, v_hat=v_hat)
    return out, stages


def decode_step(cfg, cache, q, sel_override=None, heads=None, batch=None):
    """Decode step of one layer for every sequence of the batch.

    q: [NB][Hq][d] post-RoPE queries (bf16 bits or floats).
    sel_override: optional [NB][Hkv][k] chunk ids (e.g. the GPU's selection)
    used instead of step 3.  heads / batch restrict the work to a subset;
    outputs of skipped entries are NaN.
    Returns (out [NB][Hq][d] fp64, stages[(b, h)]).
    """
    q = widen(q)
    nb = q.shape[0]
    out = np.full((nb, cfg.n_heads_q, cfg.head_dim), np.nan)
    stages = {}
    g = cfg.gqa
    for b in (range(nb) if batch is None else batch):
        for h in (range(cfg.n_heads_kv) if heads is None else heads):
            ov = None if sel_override is None else sel_override[b][h]
            o, st = decode_head(cfg, cache, q[b], b, h, ov)
            out[b, h * g:(h + 1) * g] = o
            stages[(b, h)] = st
    return out, stages


def dense_step(k, v, q, n_heads_kv: int, scale: float | None = None, batch=None):
    """Dense GQA decode over the full cache [NB][Hkv][T][d] (baseline).

    [review/motive]: GQA with a full KV cache, the uncompressed baseline the
    pages compare against.
    """
    q = widen(q)
    nb, hq, d = q.shape
    g = hq // n_heads_kv
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    out = np.full((nb, hq, d), np.nan)
    for b in (range(nb) if batch is None else batch):
        for h in range(n_heads_kv):
            kk, vv = widen(k[b, h]), widen(v[b, h])
            for j in range(h * g, (h + 1) * g):
                out[b, j] = attend(q[b, j], kk, vv, scale)
    return out
