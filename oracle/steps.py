"""Per-step definitions of the decode path, plain fp64 NumPy (test infrastructure).

Each function states one operation of LowRAM's decode step as its plain
mathematical definition.  Citations name the page and its paragraph:

  [review/keys]     LowRAM review (agihunt.info), paragraph on keys: xKV
                    cross-layer low-rank basis, RoPE undone before
                    compression, chunked prefix with mean-key landmarks,
                    top-k chunks rebuilt per query.
  [review/values]   same page, value-cache-amortisation paragraph and the
                    tagline: a small per-head MLP predicts values from keys,
                    residuals are stored only for the worst tokens.
  [explainer/how]   LowRAM explainer (cctest.ai), "How the method works".
  [review/motive]   same review, motivation paragraph: GQA, several query
                    heads share one KV head.
  [abstract]        LowRAM abstract.

Readings the pages leave open are stated where they are used.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf


# ---------------------------------------------------------------- RoPE --
def rope_freqs(d: int, theta: float) -> np.ndarray:
    """f_i = theta^(-2i/d), i < d/2 (fp64)."""
    i = np.arange(d // 2, dtype=np.float64)
    return theta ** (-2.0 * i / d)


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate rows x[t] (shape [n][d]) by the RoPE angles of positions pos[t].

    Rotate-half pairing (coordinates i and i + d/2), angle a = pos * f_i in
    fp64.  Keys are stored pre-RoPE and rotated again at their token
    positions when rebuilt [review/keys: RoPE is undone before compression].
    Reading: the rotate-half convention of the Llama / Mistral families.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    a = np.asarray(pos, dtype=np.float64)[:, None] * rope_freqs(d, theta)[None, :]
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[:, :h], x[:, h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=1)


# ---------------------------------------------------------- value MLP --
def gelu(x: np.ndarray) -> np.ndarray:
    """Exact GELU, x * (1 + erf(x / sqrt(2))) / 2 (the erf form, not tanh)."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def value_mlp(k_pre: np.ndarray, w1, b1, w2, b2) -> np.ndarray:
    """Amortised values V = W2 gelu(W1 k + b1) + b2, rows k = pre-RoPE keys.

    [review/values; explainer/how "Amortised values"]: a per-head key-to-value
    predictor; the pages call it a small MLP.  Reading: the input is the
    rebuilt pre-RoPE key (values carry no position).
    """
    hid = gelu(k_pre @ np.asarray(w1, np.float64).T + np.asarray(b1, np.float64))
    return hid @ np.asarray(w2, np.float64).T + np.asarray(b2, np.float64)


# ------------------------------------------------------------ landmarks --
def landmark_scores(q_group: np.ndarray, landmarks: np.ndarray) -> np.ndarray:
    """s[c] = max over the KV head's query heads j of q_j . L[c].

    [review/keys]: chunks are ranked against the current query by their mean
    key.  Reading: raw dot product (no 1/sqrt(d), no softmax), and a GQA
    group takes the maximum over its query heads.
    """
    return np.max(np.asarray(q_group, np.float64) @ np.asarray(landmarks, np.float64).T, axis=0)


def select_topk(scores: np.ndarray, k: int, cand_ids: np.ndarray | None = None) -> np.ndarray:
    """The k highest-scoring candidate chunks, returned in ascending chunk id.

    Ties go to the lower chunk id; with k >= candidates every candidate is
    taken.  cand_ids maps candidate position -> chunk id (identity when no
    eviction is applied).
    """
    n = len(scores)
    ids = np.arange(n) if cand_ids is None else np.asarray(cand_ids)
    order = sorted(range(n), key=lambda i: (-float(scores[i]), int(ids[i])))
    keep = order[: min(k, n)]
    return np.sort(ids[keep]).astype(np.int64)


# ------------------------------------------------------- reconstruction --
def reconstruct(coeff_rows: np.ndarray, basis_block: np.ndarray) -> np.ndarray:
    """Pre-RoPE keys rebuilt from their low-rank coefficients.

    K_pre[t, i] = sum_m C[t, m] * B[m, col(layer, head, i)]
    [review/keys; explainer/how "Low-rank keys"].  basis_block holds this
    (layer, head)'s columns of B transposed: basis_block[i, m] = B[m, col(i)].
    """
    return np.asarray(coeff_rows, np.float64) @ np.asarray(basis_block, np.float64).T


# ------------------------------------------------------------ attention --
def attend(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of one query row over keys/values, fp64.

    z_t = scale * q . k_t; p = exp(z - max z) / sum; out = p @ V.
    """
    z = scale * (np.asarray(keys, np.float64) @ np.asarray(q, np.float64))
    p = np.exp(z - np.max(z))
    p /= np.sum(p)
    return p @ np.asarray(values, np.float64)
