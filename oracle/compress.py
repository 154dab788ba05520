"""Prefill side: write the compressed cache from exact keys and values (oracle).

The steps the LowRAM pages give for compression, as plain definitions:

  project     C = X B^T, the cross-layer low-rank coefficients of a
              layer-group's pre-RoPE keys [review/keys; explainer/how
              "Low-rank keys"].  Fitting the basis is out of scope: B is a
              seeded orthonormal basis.
  landmarks   per chunk of S prefix tokens, the mean of the exact post-RoPE
              keys [review/keys: mean keys as landmarks].
  values      the synthetic exact values V = MLP(X) + Laplace noise + spikes
              (workload recipe, not the method).
  residuals   R = V - MLP(K_pre) against the key decode rebuilds; keep the
              floor(rho P) tokens with the largest ||R||_2, ties to the lower
              index, stored in ascending token order [review/values;
              explainer/how "Residuals for difficult tokens"; abstract].
  window      the last W tokens exact: post-RoPE keys and values.
  eviction    survivors of a per-head mask; landmarks compacted to them
              (LowRAM-E / -EQ compositions of the review's tables).

``exact=True`` keeps every stored array in fp64 (the invariant tests); the
default stores bf16, or int4 group-32 codes for coefficients and residuals.
"""
from __future__ import annotations

import numpy as np

from . import codecs
from .steps import reconstruct, rope, value_mlp


def project(x_group: np.ndarray, basis: np.ndarray) -> np.ndarray:
    """C = X B^T (fp64)."""
    return np.asarray(x_group, np.float64) @ np.asarray(basis, np.float64).T


def basis_block(basis: np.ndarray, cols: slice) -> np.ndarray:
    """The (layer, head) block of B, transposed: [d][r], blk[i, m] = B[m, col(i)]."""
    return np.ascontiguousarray(np.asarray(basis)[:, cols].T)


def landmarks(x_pre: np.ndarray, prefix: int, chunk: int, theta: float) -> np.ndarray:
    """Mean post-RoPE key of each chunk of the prefix, [P/S][d]."""
    pos = np.arange(prefix)
    k_post = rope(np.asarray(x_pre[:prefix], np.float64), pos, theta)
    return k_post.reshape(prefix // chunk, chunk, k_post.shape[-1]).mean(axis=1)


def exact_values(x: np.ndarray, w1, b1, w2, b2, noise, spike_pos, spike_vals) -> np.ndarray:
    v = value_mlp(np.asarray(x, np.float64), w1, b1, w2, b2) + np.asarray(noise, np.float64)
    v[spike_pos] += spike_vals
    return v


def residuals(v_prefix: np.ndarray, k_pre_prefix: np.ndarray, w1, b1, w2, b2):
    """R_t = V_t - MLP(K_pre_t) and ||R_t||_2 of every prefix token."""
    r = np.asarray(v_prefix, np.float64) - value_mlp(k_pre_prefix, w1, b1, w2, b2)
    return r, np.sqrt(np.sum(r * r, axis=1))


def select_worst(err: np.ndarray, n_resid: int) -> np.ndarray:
    """The n_resid largest errors, ties to the lower index, ascending."""
    order = np.lexsort((np.arange(len(err)), -np.asarray(err)))   # by -err, then index
    return np.sort(order[:n_resid]).astype(np.int32)


def residual_threshold(err: np.ndarray, n_resid: int) -> float:
    """The error a token must reach to be kept: the n_resid-th largest error
    (0 when every token is kept, +inf when none is)."""
    err = np.asarray(err, np.float64)
    if n_resid == 0:
        return np.inf
    if n_resid >= len(err):
        return 0.0
    return float(np.sort(err)[::-1][n_resid - 1])


def append_chunk(x_new: np.ndarray, v_new: np.ndarray, c_new_dec: np.ndarray, blk, w1, b1, w2, b2,
                 tau: float, pos0: int, theta: float):
    """Window rollover: the S tokens at positions pos0 .. pos0+S-1 become a prefix chunk.

    x_new: their exact pre-RoPE keys [S][d]; v_new: exact values [S][d];
    c_new_dec: their coefficients as stored (decoded) [S][r]; blk: basis block
    [d][r].  Returns the chunk's landmark (mean post-RoPE key, as at build
    time), the offsets of the tokens whose residual error reaches the
    build-time threshold tau (the same test the build applied to the prefix:
    keep a residual when ||R|| is at least the nR-th largest error), their
    residual rows, and every token's error.
    """
    x_new = np.asarray(x_new, np.float64)
    S = x_new.shape[0]
    lm = rope(x_new, pos0 + np.arange(S), theta).mean(axis=0)
    r, err = residuals(v_new, reconstruct(c_new_dec, blk), w1, b1, w2, b2)
    keep = np.nonzero(err >= tau)[0].astype(np.int32)
    return dict(landmark=lm, keep=keep, rows=r[keep], errors=err)


def residual_select(v_prefix: np.ndarray, k_pre_prefix: np.ndarray, w1, b1, w2, b2, n_resid: int):
    """Indices (ascending) and rows of the n_resid worst-predicted prefix tokens."""
    r, err = residuals(v_prefix, k_pre_prefix, w1, b1, w2, b2)
    idx = select_worst(err, n_resid)
    return idx, r[idx]


def chunk_descriptors(idx: np.ndarray, n_chunks: int, chunk: int) -> np.ndarray:
    """Residual descriptor per chunk (cache layout, no method arithmetic).

    desc[c] = (number of residual tokens below c*S) << 8 | bitmask of the
    chunk's tokens c*S + i that have a residual (S <= 8).
    """
    idx = np.asarray(idx, np.int64)
    bounds = np.arange(n_chunks, dtype=np.int64) * chunk
    first = np.searchsorted(idx, bounds, side="left")
    mask = np.zeros(n_chunks, dtype=np.uint64)
    np.bitwise_or.at(mask, idx // chunk, np.left_shift(np.uint64(1), (idx % chunk).astype(np.uint64)))
    return ((first.astype(np.uint64) << np.uint64(8)) | mask).astype(np.uint32)


def _store(x, exact: bool):
    return np.asarray(x, np.float64) if exact else codecs.bf16_encode(x)


def store_coeff(c, int4: bool, exact: bool = False):
    """Coefficients as the cache stores them: fp64 (exact), int4 g32 (codes,
    scales) or bf16 bits."""
    if exact:
        return np.asarray(c, np.float64)
    return codecs.int4_encode(c) if int4 else codecs.bf16_encode(c)


def decode_coeff(coeff_stored, int4: bool, exact: bool = False) -> np.ndarray:
    if exact:
        return np.asarray(coeff_stored, np.float64)
    return codecs.int4_decode(*coeff_stored) if int4 else codecs.bf16_decode(coeff_stored)


def compress_from_kv(cfg, x_head: np.ndarray, v_head: np.ndarray, coeff_stored, blk_stored, mlp,
                     exact: bool = False):
    """Everything one (sequence, layer, KV head) stores, from its exact keys and values.

    x_head: exact pre-RoPE keys [T][d]; v_head: exact values [T][d];
    coeff_stored: the group's stored coefficients of the prefix tokens (bf16
    bits, int4 (codes, scales), or fp64 with exact=True); blk_stored: stored
    basis block [d][r]; mlp = (w1, b1, w2, b2) as stored.  The residual test
    runs against the keys decode rebuilds: stored coefficients x stored block.
    """
    P, S, W = cfg.prefix, cfg.chunk, cfg.window
    w = [np.asarray(a, np.float64) if exact else codecs.bf16_decode(a) for a in mlp]
    v = np.asarray(v_head, np.float64)
    c_dec = decode_coeff(coeff_stored, cfg.int4, exact)
    blk = np.asarray(blk_stored, np.float64) if exact else codecs.bf16_decode(blk_stored)
    k_pre = reconstruct(c_dec, blk)
    r, err = residuals(v[:P], k_pre, *w)
    idx = select_worst(err, cfg.n_resid)
    rows = r[idx]

    out = dict(
        landmark=_store(landmarks(x_head, P, S, cfg.rope_theta), exact),
        res_idx=idx,
        res_chunk_desc=chunk_descriptors(idx, cfg.n_chunks, S),
        win_k=_store(rope(x_head[P:], np.arange(P, P + W), cfg.rope_theta), exact),
        win_v=_store(v[P:], exact),
        errors=err,   # not stored by the cache: every prefix token's ||R||, for near-tie checks
        res_thresh=residual_threshold(err, cfg.n_resid),
    )
    if cfg.int4 and not exact:
        out["res_val"], out["res_scale"] = codecs.int4_encode(rows)
    else:
        out["res_val"] = _store(rows, exact)
    return out


def compress_head(cfg, x_head: np.ndarray, coeff_stored, blk_stored, mlp, noise, spikes,
                  exact: bool = False):
    """compress_from_kv with the synthetic exact values V = MLP(X) + noise + spikes."""
    w = [np.asarray(a, np.float64) if exact else codecs.bf16_decode(a) for a in mlp]
    v = exact_values(x_head, *w, noise, *spikes)
    return compress_from_kv(cfg, x_head, v, coeff_stored, blk_stored, mlp, exact=exact)


def compact_landmarks(lm: np.ndarray, survivors: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(lm)[np.asarray(survivors)])
