"""Fitting the layer group's key basis (oracle, test infrastructure).

LowRAM review (agihunt.info), key paragraph: the keys of adjacent layers
share one low-rank basis (xKV, an SVD basis of the group's concatenated
pre-RoPE keys), and a randomised Cholesky-QR replaces the exact SVD for a
reported 4x speed-up with no quality loss.  The pages give no further detail;
the plain reading implemented here:

  svd_basis        the exact fit: the top-r right singular vectors of X
                   [P][D] (rows of B), by LAPACK SVD.
  randomized_cholqr  a randomised range finder on the row space of X: the
                   sketch Y = X^T Omega (D x r, Omega [P][r] Gaussian, given
                   as an input), orthonormalised by Cholesky-QR, twice
                   (CholQR2: G = Y^T Y, R = chol(G) upper, Y <- Y R^-1; the
                   second pass restores the orthogonality the first loses to
                   rounding), then q power passes Y <- CholQR2(X^T (X Y)).
                   B = Y^T has orthonormal rows.  One power pass is the
                   default: without it the sketch of the synthetic keys
                   leaves the latent subspace ~0.1 rad away and the
                   projection error ~1.5x the SVD optimum; with it, within
                   1e-4 rad and a few per cent (the pages' "no quality loss").
                   Re-orthonormalising between passes keeps the Gram matrix
                   positive definite (X^T X X^T X Omega squares the spread of
                   the spectrum).

Quality measures used by the tests: principal angles between subspaces
(scipy), and the relative projection error ||X - X B^T B|| / ||X||, for which
the SVD basis is optimal (Eckart-Young).
"""
from __future__ import annotations

import numpy as np
import scipy.linalg


def svd_basis(x: np.ndarray, rank: int) -> np.ndarray:
    """Top-`rank` right singular vectors of x as rows [rank][D] (fp64)."""
    _, _, vt = np.linalg.svd(np.asarray(x, np.float64), full_matrices=False)
    return np.ascontiguousarray(vt[:rank])


def cholqr(y: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """One Cholesky-QR pass: y = Q R with R = chol(y^T y) upper triangular."""
    y = np.asarray(y, np.float64)
    g = y.T @ y
    r = np.linalg.cholesky(g).T                       # upper: g = r^T r
    q = scipy.linalg.solve_triangular(r, y.T, trans="T", lower=False).T   # q = y r^-1
    return q, r


def cholqr2(y: np.ndarray, passes: int = 2) -> np.ndarray:
    for _ in range(passes):
        y, _ = cholqr(y)
    return y


def randomized_cholqr(x: np.ndarray, omega: np.ndarray, power: int = 1, passes: int = 2) -> np.ndarray:
    """Basis rows [r][D] from the sketch X^T Omega (see the module docstring)."""
    x = np.asarray(x, np.float64)
    y = cholqr2(x.T @ np.asarray(omega, np.float64), passes)   # [D][r]
    for _ in range(power):
        y = cholqr2(x.T @ (x @ y), passes)
    return np.ascontiguousarray(y.T)


def projection_error(x: np.ndarray, basis: np.ndarray) -> float:
    """||X - X B^T B||_F / ||X||_F for orthonormal rows B."""
    x = np.asarray(x, np.float64)
    b = np.asarray(basis, np.float64)
    return float(np.linalg.norm(x - (x @ b.T) @ b) / np.linalg.norm(x))


def principal_angles(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Every principal angle (radians) between span(rows of a) and span(rows of b)."""
    return scipy.linalg.subspace_angles(np.asarray(a, np.float64).T, np.asarray(b, np.float64).T)


def max_angle(a: np.ndarray, b: np.ndarray) -> float:
    """Largest principal angle (radians) between span(rows of a) and span(rows of b).

    With fewer rows in a than in b this measures how far span(a) is from
    being contained in span(b).
    """
    return float(np.max(scipy.linalg.subspace_angles(np.asarray(a, np.float64).T, np.asarray(b, np.float64).T)))
