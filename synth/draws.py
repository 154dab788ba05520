"""Seeded random draws for the synthetic decode workloads.

This module only draws random numbers (and assembles the synthetic model
state from them: exact pre-RoPE keys as latents times a mixing matrix plus
noise, and an orthonormal key basis).  It holds none of the decode step's
arithmetic: no RoPE, no value MLP, no scoring, no selection, no attention.
Both the CPU oracle side and the GPU side of the tests read their inputs
from here.

Every array is regenerable on its own from (config, batch element, layer or
group, head, stream): each draw owns a ``numpy.random.SeedSequence`` with
entropy ``1000 + cfg_id`` and a spawn key naming the stream and indices.
"""
from __future__ import annotations

import numpy as np

from .configs import Config

# stream ids of the spawn keys
Z, MIX, NOISE, PAD, MLP, LAPLACE, SPIKE, QUERY, NEEDLE, EVICT, BIAS, BENCH = range(1, 13)

NOISE_BLOCK = 4096  # tokens per independently seeded noise block


def rng(cfg: Config, stream: int, *idx: int) -> np.random.Generator:
    key = (stream,) + tuple(int(i) for i in idx)
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(entropy=1000 + cfg.cfg_id, spawn_key=key)))


# ---------------------------------------------------------------- keys --
def latents(cfg: Config, b: int, grp: int, dtype=np.float64) -> np.ndarray:
    """Z ~ N(0, 1), shape [T][latent_dim], one draw per (sequence, group)."""
    return rng(cfg, Z, b, grp).standard_normal((cfg.ctx, cfg.latent_dim)).astype(dtype, copy=False)


def mixing(cfg: Config, b: int, grp: int) -> np.ndarray:
    """M, shape [latent_dim][G*Hkv*d], entries N(0, 1/latent_dim).

    The variance 1/latent_dim gives the exact key coordinates unit variance.
    """
    g = rng(cfg, MIX, b, grp)
    return g.standard_normal((cfg.latent_dim, cfg.group_dim)) / np.sqrt(cfg.latent_dim)


def key_noise(cfg: Config, b: int, grp: int, t0: int, t1: int, dtype=np.float64) -> np.ndarray:
    """N(0, key_noise_std) for tokens [t0, t1), columns G*Hkv*d.

    Drawn in independently seeded blocks of NOISE_BLOCK tokens so any token
    range can be produced without the rest.
    """
    out = np.empty((t1 - t0, cfg.group_dim), dtype=dtype)
    blk0, blk1 = t0 // NOISE_BLOCK, (t1 - 1) // NOISE_BLOCK
    for blk in range(blk0, blk1 + 1):
        a, e = blk * NOISE_BLOCK, min((blk + 1) * NOISE_BLOCK, cfg.ctx)
        vals = rng(cfg, NOISE, b, grp, blk).standard_normal((e - a, cfg.group_dim), dtype=np.float64
                                                             if dtype == np.float64 else np.float32)
        lo, hi = max(a, t0), min(e, t1)
        out[lo - t0:hi - t0] = vals[lo - a:hi - a] * cfg.key_noise_std
    return out


def exact_keys(cfg: Config, b: int, grp: int, t0: int = 0, t1: int | None = None,
               dtype=np.float64) -> np.ndarray:
    """Exact pre-RoPE keys X = Z M + noise of one layer-group, rows [t0, t1).

    Column layout: col(l, h, i) = (l * Hkv + h) * d + i, l the layer inside
    the group, h the KV head, i the head-dim coordinate.
    """
    t1 = cfg.ctx if t1 is None else t1
    zz = latents(cfg, b, grp, dtype)[t0:t1]
    m = mixing(cfg, b, grp).astype(dtype)
    return zz @ m + key_noise(cfg, b, grp, t0, t1, dtype)


def layer_cols(cfg: Config, layer: int, h: int) -> slice:
    """Columns of the group's concatenated keys that belong to (layer, head)."""
    li = layer % cfg.group_layers
    c0 = (li * cfg.n_heads_kv + h) * cfg.head_dim
    return slice(c0, c0 + cfg.head_dim)


def basis(cfg: Config, b: int, grp: int) -> np.ndarray:
    """Orthonormal key basis B, shape [r][G*Hkv*d] (rows orthonormal).

    QR of the mixing matrix's transpose, padded with N(0, 1) columns when the
    rank exceeds the latent dimension, so the basis always contains the
    latent subspace the keys live in.
    """
    m = mixing(cfg, b, grp)
    r = cfg.rank
    if r <= cfg.latent_dim:
        a = m.T[:, :r]
    else:
        pad = rng(cfg, PAD, b, grp).standard_normal((cfg.group_dim, r - cfg.latent_dim))
        a = np.concatenate([m.T, pad], axis=1)
    q, _ = np.linalg.qr(a)
    return np.ascontiguousarray(q[:, :r].T)


# -------------------------------------------------------------- values --
def mlp_weights(cfg: Config, b: int, layer: int, h: int):
    """Value-MLP weights of one (sequence, layer, KV head).

    W1 [H][d], W2 [d][H] (torch Linear orientation), Xavier-uniform with
    gain 1; biases N(0, bias_std) (zero in the named workloads).
    """
    d, hid = cfg.head_dim, cfg.mlp_hidden
    g = rng(cfg, MLP, b, layer, h)
    a = np.sqrt(6.0 / (d + hid))
    w1 = g.uniform(-a, a, size=(hid, d))
    w2 = g.uniform(-a, a, size=(d, hid))
    if cfg.bias_std > 0:
        gb = rng(cfg, BIAS, b, layer, h)
        b1 = gb.standard_normal(hid) * cfg.bias_std
        b2 = gb.standard_normal(d) * cfg.bias_std
    else:
        b1 = np.zeros(hid)
        b2 = np.zeros(d)
    return w1, b1, w2, b2


def value_noise(cfg: Config, b: int, layer: int, h: int, dtype=np.float64) -> np.ndarray:
    """Laplace(0, laplace_scale) noise on every token's value, [T][d]."""
    g = rng(cfg, LAPLACE, b, layer, h)
    return g.laplace(0.0, cfg.laplace_scale, size=(cfg.ctx, cfg.head_dim)).astype(dtype, copy=False)


def value_spikes(cfg: Config, b: int, layer: int, h: int):
    """round(spike_frac * T) distinct token positions (ascending) and N(0, 1) rows."""
    g = rng(cfg, SPIKE, b, layer, h)
    n = int(round(cfg.spike_frac * cfg.ctx))
    pos = np.sort(g.choice(cfg.ctx, size=n, replace=False))
    vals = g.standard_normal((n, cfg.head_dim))
    return pos, vals


# ------------------------------------------------------------- queries --
def queries(cfg: Config, b: int, layer: int) -> np.ndarray:
    """Post-RoPE queries of one (sequence, layer), N(0, 1), [Hq][d]."""
    return rng(cfg, QUERY, b, layer).standard_normal((cfg.n_heads_q, cfg.head_dim))


def needle_chunks(cfg: Config, b: int, layer: int) -> np.ndarray:
    """The planted chunk c* of each KV head, uniform over the candidates."""
    return rng(cfg, NEEDLE, b, layer).integers(0, cfg.n_chunks, size=cfg.n_heads_kv)


def plant_needle(q: np.ndarray, gqa: int, landmark_rows: np.ndarray) -> np.ndarray:
    """q_j <- q_j + |q_j| * L / |L| for each query head j of KV head h.

    landmark_rows[h] is the (stored) landmark of head h's planted chunk.
    """
    out = np.array(q, dtype=np.float64, copy=True)
    for h in range(landmark_rows.shape[0]):
        u = landmark_rows[h] / np.linalg.norm(landmark_rows[h])
        for j in range(h * gqa, (h + 1) * gqa):
            out[j] = out[j] + np.linalg.norm(out[j]) * u
    return out


# ------------------------------------------------------------ eviction --
def evicted_chunks(cfg: Config, b: int, layer: int, h: int) -> np.ndarray:
    """Chunk ids evicted for (b, layer, h): nC//2 of the non-sink chunks."""
    g = rng(cfg, EVICT, b, layer, h)
    perm = g.permutation(np.arange(cfg.n_sinks, cfg.n_chunks))
    return np.sort(perm[: cfg.n_chunks // 2])


def survivors(cfg: Config, b: int, layer: int, h: int) -> np.ndarray:
    keep = np.ones(cfg.n_chunks, dtype=bool)
    keep[evicted_chunks(cfg, b, layer, h)] = False
    return np.nonzero(keep)[0].astype(np.int32)
