"""Assemble the compressed cache of one layer from the seeded draws (test infrastructure).

Draws come from ``synth`` (random numbers and the synthetic exact keys only);
every arithmetic step of compression is the oracle's own (``compress``).
Arrays come out in the layout the GPU library takes, batch major:

  coeff        [NB][P][r] bf16, or [NB][P][r/2] int4 + coeff_scale [NB][P][r/32] fp16
  basis        [NB][Hkv][d][r] bf16  (this layer's blocks of the group basis, transposed)
  landmark     [NB][Hkv][nCand][d] bf16
  cand_ids     [NB][Hkv][nCand] int32 (eviction only)
  w1 [NB][Hkv][H][d], b1 [NB][Hkv][H], w2 [NB][Hkv][d][H], b2 [NB][Hkv][d] bf16
  res_idx      [NB][Hkv][nR] int32 ascending
  res_val      [NB][Hkv][nR][d] bf16, or [..][nR][d/2] int4 + res_scale [..][nR][d/32]
  res_chunk_desc [NB][Hkv][nC] uint32 (first residual row << 8 | token bitmask)
  win_k, win_v [NB][Hkv][W][d] bf16
  q            [NB][Hq][d] bf16
"""
from __future__ import annotations

import functools

import numpy as np

import synth
from . import codecs
from .compress import basis_block, compact_landmarks, compress_head, project, store_coeff


def _key_dtype(cfg):
    return np.float64 if cfg.ctx <= 8192 else np.float32


@functools.lru_cache(maxsize=2)
def _group_state(cfg, b: int, grp: int, exact: bool):
    """Exact keys, basis and stored coefficients of one (sequence, group)."""
    x = synth.exact_keys(cfg, b, grp, dtype=_key_dtype(cfg))
    B = synth.basis(cfg, b, grp)
    c_st = store_coeff(project(x[: cfg.prefix], B), cfg.int4, exact)
    return x, B, c_st


_BASIS_OVERRIDE = {}


def build_layer_with_basis(cfg, layer: int, basis_rows: np.ndarray):
    """build_layer for batch element 0 with the group's basis replaced by
    ``basis_rows`` [r][D] (orthonormal rows), e.g. a fitted basis."""
    grp = layer // cfg.group_layers
    x = synth.exact_keys(cfg, 0, grp, dtype=_key_dtype(cfg))
    B = np.asarray(basis_rows, np.float64)
    _BASIS_OVERRIDE[(cfg, 0, grp)] = (x, B, store_coeff(project(x[: cfg.prefix], B), cfg.int4, False))
    try:
        return build_layer(cfg, layer, batch=[0])
    finally:
        _BASIS_OVERRIDE.pop((cfg, 0, grp), None)


def build_layer(cfg, layer: int, batch=None, exact: bool = False):
    """Compressed cache + queries of ``layer`` for the batch elements ``batch``."""
    batch = list(range(cfg.batch)) if batch is None else list(batch)
    G, Hkv = cfg.group_layers, cfg.n_heads_kv
    grp = layer // G
    per_b = []
    for b in batch:
        x, B, c_st = _BASIS_OVERRIDE.get((cfg, b, grp)) or _group_state(cfg, b, grp, exact)
        heads = []
        for h in range(Hkv):
            cols = synth.layer_cols(cfg, layer, h)
            blk = basis_block(B, cols)
            blk_st = blk if exact else codecs.bf16_encode(blk)
            mlp = synth.mlp_weights(cfg, b, layer, h)
            mlp_st = tuple(np.asarray(a, np.float64) if exact else codecs.bf16_encode(a) for a in mlp)
            noise = synth.value_noise(cfg, b, layer, h)
            spikes = synth.value_spikes(cfg, b, layer, h)
            hd = compress_head(cfg, np.asarray(x[:, cols], np.float64), c_st, blk_st, mlp_st,
                               noise, spikes, exact=exact)
            hd["basis"] = blk_st
            hd["w1"], hd["b1"], hd["w2"], hd["b2"] = mlp_st
            if cfg.evict:
                surv = synth.survivors(cfg, b, layer, h)
                hd["landmark"] = compact_landmarks(hd["landmark"], surv)
                hd["cand_ids"] = surv
            heads.append(hd)
        q = synth.queries(cfg, b, layer)
        if cfg.needle:
            cs = synth.needle_chunks(cfg, b, layer)
            rows = np.stack([codecs.bf16_decode(heads[h]["landmark"][cs[h]]) if not exact
                             else heads[h]["landmark"][cs[h]] for h in range(Hkv)])
            q = synth.plant_needle(q, cfg.gqa, rows)
        per_b.append((c_st, heads, q if exact else codecs.bf16_encode(q)))

    cache = {}
    if cfg.int4 and not exact:
        cache["coeff"] = np.stack([p[0][0] for p in per_b])
        cache["coeff_scale"] = np.stack([p[0][1] for p in per_b])
    else:
        cache["coeff"] = np.stack([p[0] for p in per_b])
    keys = ["basis", "landmark", "w1", "b1", "w2", "b2", "res_idx", "res_val",
            "res_chunk_desc", "win_k", "win_v"]
    if cfg.int4 and not exact:
        keys.append("res_scale")
    if cfg.evict:
        keys.append("cand_ids")
    for k in keys:
        cache[k] = np.ascontiguousarray(np.stack([np.stack([hd[k] for hd in p[1]]) for p in per_b]))
    cache["q"] = np.stack([p[2] for p in per_b])
    if cfg.needle:
        cache["needle"] = np.stack([synth.needle_chunks(cfg, b, layer) for b in batch])
    return cache


def dense_layer(cfg, layer: int, batch=None):
    """Exact bf16 dense cache K (post-RoPE), V [NB][Hkv][T][d] and q (baseline).

    The same synthetic model state the compressed cache is built from.
    """
    from .compress import exact_values
    from .steps import rope
    batch = list(range(cfg.batch)) if batch is None else list(batch)
    grp = layer // cfg.group_layers
    ks, vs, qs = [], [], []
    for b in batch:
        x = synth.exact_keys(cfg, b, grp, dtype=_key_dtype(cfg))
        kh, vh = [], []
        for h in range(cfg.n_heads_kv):
            xh = np.asarray(x[:, synth.layer_cols(cfg, layer, h)], np.float64)
            kh.append(codecs.bf16_encode(rope(xh, np.arange(cfg.ctx), cfg.rope_theta)))
            w = [codecs.bf16_round(a) for a in synth.mlp_weights(cfg, b, layer, h)]
            v = exact_values(xh, *w, synth.value_noise(cfg, b, layer, h), *synth.value_spikes(cfg, b, layer, h))
            vh.append(codecs.bf16_encode(v))
        ks.append(np.stack(kh))
        vs.append(np.stack(vh))
        qs.append(codecs.bf16_encode(synth.queries(cfg, b, layer)))
    return np.stack(ks), np.stack(vs), np.stack(qs)


def builder_expected(cfg, layer: int, x_bits, basis_bits, c_st, heads, values_bits, mlp_bits):
    """The oracle's compression of one sequence's builder inputs (given as bf16 bits).

    x_bits [T][D] group keys, basis_bits [r][D], c_st the stored coefficients
    of the prefix, heads the KV heads to compress, values_bits [len(heads)][T][d]
    and mlp_bits (per head: w1, b1, w2, b2) of those heads.  Arrays come out
    with a head axis in the order of ``heads``.
    """
    from .compress import compress_from_kv
    hexp = {}
    for i, h in enumerate(heads):
        cols = synth.layer_cols(cfg, layer, h)
        blk_st = basis_block(basis_bits, cols)
        hd = compress_from_kv(cfg, codecs.bf16_decode(x_bits[:, cols]), codecs.bf16_decode(values_bits[i]), c_st,
                              blk_st, mlp_bits[i])
        hd["basis"] = blk_st
        for k, v in hd.items():
            hexp.setdefault(k, []).append(v)
    return {k: np.stack(v) for k, v in hexp.items()}


def builder_io(cfg, layer: int, batch=None):
    """Inputs of the cache builder for ``layer`` and the cache the oracle builds from them.

    Inputs (bf16 bits, the layouts of lowram_build_coeff / lowram_build_layer):
      keys [NB][T][D] exact pre-RoPE keys of the layer's group, group_basis
      [NB][r][D], values [NB][Hkv][T][d] exact values of the layer, w1, b1, w2,
      b2 as in the cache.
    Expected: the oracle's compression (``compress``) run on exactly those
    bf16 inputs: coeff (+ coeff_scale), basis, landmark, res_idx, res_val
    (+ res_scale), res_chunk_desc, win_k, win_v, and ``errors`` [NB][Hkv][P],
    the oracle's ||R_t|| of every prefix token (for the near-tie rule).
    """
    from .compress import exact_values
    batch = list(range(cfg.batch)) if batch is None else list(batch)
    grp = layer // cfg.group_layers
    P, Hkv = cfg.prefix, cfg.n_heads_kv
    inp = {k: [] for k in ("keys", "group_basis", "values", "w1", "b1", "w2", "b2")}
    exp = {}
    for b in batch:
        x_bits = codecs.bf16_encode(synth.exact_keys(cfg, b, grp, dtype=_key_dtype(cfg)))
        B_bits = codecs.bf16_encode(synth.basis(cfg, b, grp))
        x = codecs.bf16_decode(x_bits)
        c_st = store_coeff(project(x[:P], codecs.bf16_decode(B_bits)), cfg.int4)
        mlp_bits = [tuple(codecs.bf16_encode(a) for a in synth.mlp_weights(cfg, b, layer, h)) for h in range(Hkv)]
        v_bits = np.stack([
            codecs.bf16_encode(exact_values(np.asarray(x[:, synth.layer_cols(cfg, layer, h)]),
                                            *[codecs.bf16_decode(a) for a in mlp_bits[h]],
                                            synth.value_noise(cfg, b, layer, h), *synth.value_spikes(cfg, b, layer, h)))
            for h in range(Hkv)])
        inp["keys"].append(x_bits)
        inp["group_basis"].append(B_bits)
        inp["values"].append(v_bits)
        for i, k in enumerate(("w1", "b1", "w2", "b2")):
            inp[k].append(np.stack([m[i] for m in mlp_bits]))
        e = builder_expected(cfg, layer, x_bits, B_bits, c_st, range(Hkv), v_bits, mlp_bits)
        if cfg.int4:
            e["coeff"], e["coeff_scale"] = c_st
        else:
            e["coeff"] = c_st
        for k, v in e.items():
            exp.setdefault(k, []).append(v)
    inp = {k: np.ascontiguousarray(np.stack(v)) for k, v in inp.items()}
    exp = {k: np.ascontiguousarray(np.stack(v)) for k, v in exp.items()}
    return inp, exp
