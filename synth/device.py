"""Seeded random draws of full-size compressed caches, made on the GPU.

For timing at the 262K point the cache of a whole batch (185 GB at batch 28)
cannot come from the host-side fixture.  This module draws one (sequence,
layer) slice straight into device memory with a seeded torch generator, each
array from the distribution the structured fixture produces for it:

  coeff     first 64 of r coefficients N(0, 8^2) (the latent subspace carries
            all key energy), the rest N(0, 0.05^2); int4: codes uniform in
            [-7, 7] with group scales of matching magnitude
  basis     N(0, 1/64^2) (rows of an orthonormal 4096-dim basis)
  landmark  N(0, 0.35^2)
  w1, w2    Xavier-uniform, biases zero
  res_idx   a uniformly random subset of exactly nR prefix tokens, ascending
  res_val   N(0, 0.3^2)
  win_k/v   N(0, 1) / N(0, 0.5^2)
  cand_ids  the 4 sink chunks plus a uniformly random subset of the rest
  q         N(0, 1)

Bytes and flops of a decode step do not depend on the values, except through
the residual density of the selected chunks, which is the same (rho).  This
module holds none of the decode step's arithmetic.
"""
from __future__ import annotations

import torch

BF16 = torch.bfloat16


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, std, g, device, dtype=BF16):
    return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std).to(dtype)


def _pack_int4(codes: torch.Tensor) -> torch.Tensor:
    """int8 codes in [-7, 7], last axis even -> uint8 (even element in the low nibble)."""
    c = (codes.to(torch.int16) & 0xF).to(torch.uint8)
    return c[..., 0::2] | (c[..., 1::2] << 4)


def _fp16_bits(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.float16).view(torch.int16)


def draw_coeff(cfg, seed: int, device):
    """Coefficients of one (sequence, layer-group): bf16 [P][r], or (int4 [P][r/2], scales [P][r/32])."""
    g = _gen(seed, device)
    P, r = cfg.prefix, cfg.rank
    lat = min(64, r)
    if not cfg.int4:
        c = torch.empty((P, r), dtype=BF16, device=device)
        c[:, :lat] = _normal((P, lat), 8.0, g, device)
        if r > lat:
            c[:, lat:] = _normal((P, r - lat), 0.05, g, device)
        return c
    codes = torch.randint(-7, 8, (P, r), generator=g, device=device, dtype=torch.int8)
    scale = torch.empty((P, r // 32), dtype=torch.float32, device=device)
    scale[:, : lat // 32] = 8.0 * 2.5 / 7
    scale[:, lat // 32:] = 0.05 * 2.5 / 7
    scale *= torch.rand((P, r // 32), generator=g, device=device) * 0.5 + 0.75
    return _pack_int4(codes), _fp16_bits(scale)


def draw_layer(cfg, seed: int, device) -> dict:
    """Per-layer arrays of one sequence (no batch axis)."""
    g = _gen(seed, device)
    Hkv, d, H, r, P = cfg.n_heads_kv, cfg.head_dim, cfg.mlp_hidden, cfg.rank, cfg.prefix
    nR, W, nc = cfg.n_resid, cfg.window, cfg.n_cand
    a = (6.0 / (d + H)) ** 0.5
    t = {
        "basis": _normal((Hkv, d, r), 1.0 / 64, g, device),
        "landmark": _normal((Hkv, nc, d), 0.35, g, device),
        "w1": ((torch.rand((Hkv, H, d), generator=g, device=device) * 2 - 1) * a).to(BF16),
        "b1": torch.zeros((Hkv, H), dtype=BF16, device=device),
        "w2": ((torch.rand((Hkv, d, H), generator=g, device=device) * 2 - 1) * a).to(BF16),
        "b2": torch.zeros((Hkv, d), dtype=BF16, device=device),
        "win_k": _normal((Hkv, W, d), 1.0, g, device),
        "win_v": _normal((Hkv, W, d), 0.5, g, device),
    }
    idx = torch.empty((Hkv, nR), dtype=torch.int32, device=device)
    for h in range(Hkv):
        idx[h] = torch.sort(torch.randperm(P, generator=g, device=device)[:nR]).values.to(torch.int32)
    t["res_idx"] = idx
    if cfg.int4:
        codes = torch.randint(-7, 8, (Hkv, nR, d), generator=g, device=device, dtype=torch.int8)
        t["res_val"] = _pack_int4(codes)
        t["res_scale"] = _fp16_bits(torch.rand((Hkv, nR, d // 32), generator=g, device=device) * 0.05 + 0.08)
    else:
        t["res_val"] = _normal((Hkv, nR, d), 0.3, g, device)
    if cfg.evict:
        nC, ns = cfg.n_chunks, cfg.n_sinks
        cand = torch.empty((Hkv, nc), dtype=torch.int32, device=device)
        for h in range(Hkv):
            rest = torch.randperm(nC - ns, generator=g, device=device)[: nc - ns] + ns
            cand[h, :ns] = torch.arange(ns, device=device, dtype=torch.int32)
            cand[h, ns:] = torch.sort(rest).values.to(torch.int32)
        t["cand_ids"] = cand
    return t


def draw_queries(cfg, nb: int, seed: int, device) -> torch.Tensor:
    return _normal((nb, cfg.n_heads_q, cfg.head_dim), 1.0, _gen(seed, device), device)


def draw_build_inputs(cfg, seed: int, device, nb: int = 1, layers=None) -> dict:
    """Cache-builder inputs of nb sequences of one layer group, drawn on the GPU.

      keys         [NB][T][D] bf16: latents Z ~ N(0, 1) of dim 64 (drawn here)
                   times the group's host mixing matrix, plus N(0, 0.05^2)
      group_basis  [NB][r][D] bf16: the host fixture's orthonormal basis
      per layer l  values [NB][Hkv][T][d] ~ N(0, 0.5^2), and the host
                   fixture's MLP weights (w1, b1, w2, b2) of the layer
    Returned as {"keys", "group_basis", "layers": [dict per layer]}.
    """
    import numpy as np
    from . import draws
    g = _gen(seed, device)
    T, D, Hkv, d = cfg.ctx, cfg.group_dim, cfg.n_heads_kv, cfg.head_dim
    layers = list(range(cfg.group_layers)) if layers is None else list(layers)
    keys = torch.empty((nb, T, D), dtype=BF16, device=device)
    basis = torch.empty((nb, cfg.rank, D), dtype=BF16, device=device)
    for b in range(nb):
        m = torch.from_numpy(draws.mixing(cfg, b, 0)).to(device=device, dtype=torch.float32)
        for t0 in range(0, T, 32768):
            t1 = min(T, t0 + 32768)
            z = torch.randn((t1 - t0, cfg.latent_dim), generator=g, device=device, dtype=torch.float32)
            x = z @ m
            x += torch.randn(x.shape, generator=g, device=device, dtype=torch.float32) * cfg.key_noise_std
            keys[b, t0:t1] = x.to(BF16)
        basis[b] = torch.from_numpy(draws.basis(cfg, b, 0)).to(device=device, dtype=torch.float32).to(BF16)
    out = {"keys": keys, "group_basis": basis, "layers": []}
    for layer in layers:
        per = {"values": _normal((nb, Hkv, T, d), 0.5, g, device)}
        ws = [[draws.mlp_weights(cfg, b, layer, h) for h in range(Hkv)] for b in range(nb)]
        for i, name in enumerate(("w1", "b1", "w2", "b2")):
            a = np.stack([np.stack([ws[b][h][i] for h in range(Hkv)]) for b in range(nb)])
            per[name] = torch.from_numpy(a).to(device=device, dtype=torch.float32).to(BF16)
        out["layers"].append(per)
    return out
