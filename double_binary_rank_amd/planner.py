"""Offline planning on the host (numpy): storage sizes, middle widths for a
bit budget, the per-channel importance and the channel gather used for
non-uniform middle widths.

None of this runs on the product path: it decides, once per model, which
middle channels each layer keeps (DBF summary, section 3, iterative
non-uniform pruning, read without data).  The binding in ``api.py`` only
moves the factors between the device and these functions; the sign packing
and unpacking themselves run in the HIP library.
"""
from __future__ import annotations

import numpy as np

__all__ = ["layer_bits", "rank_for_bits", "plan_channels", "channel_importance",
           "select_channels"]


def layer_bits(N: int, R: int, M: int, ell: int = 1) -> int:
    """Storage of one layer: N*R + R*M sign bits and 16-bit alpha, beta,
    gamma per term (DBF summary, Control Granular de Compresion)."""
    return N * R + R * M + 16 * ell * (N + R + M)


def rank_for_bits(N: int, M: int, bpw: float, ell: int = 1) -> int:
    """Largest middle width k whose storage is at most bpw bits per entry of
    the N x M matrix (fractional budgets allowed)."""
    k = int((bpw * N * M - 16 * ell * (N + M)) // (N + M + 16 * ell))
    while k > 0 and layer_bits(N, k, M, ell) > bpw * N * M:
        k -= 1
    while layer_bits(N, k + 1, M, ell) <= bpw * N * M:
        k += 1
    return max(k, 0)


def plan_channels(shapes, importances, budget_bits: float):
    """Non-uniform middle widths for a stack (DBF summary, section 3,
    iterative non-uniform pruning, read without data): drop the globally
    least important channel (ties: earlier layer, then lower index) until the
    stack's storage fits budget_bits.  shapes: (N, R, M) per layer (ell = 1);
    importances: host arrays of length R (``channel_importance``).  Returns
    the sorted kept channel indices of each layer (host int64 arrays; a
    layer may keep none)."""
    total = sum(layer_bits(N, R, M) for (N, R, M) in shapes)
    cand = sorted((float(v), li, r) for li, imp in enumerate(importances)
                  for r, v in enumerate(np.asarray(imp, dtype=np.float64)))
    dropped = [set() for _ in shapes]
    for _, li, r in cand:
        if total <= budget_bits:
            break
        N, _, M = shapes[li]
        dropped[li].add(r)
        total -= N + M + 16
    return [np.array([r for r in range(R) if r not in d], dtype=np.int64)
            for (N, R, M), d in zip(shapes, dropped)]


def channel_importance(alpha, beta, gamma) -> np.ndarray:
    """Per middle channel r of a one-term layer: |beta_r| ||alpha|| ||gamma||,
    the Frobenius norm of the channel's rank-1 term of the update whatever
    its signs (DBF summary, section 3: the middle dimension is pruned as
    channels).  alpha [1][N], beta [1][R], gamma [1][M] host arrays; returns
    float64 [R]."""
    a = np.asarray(alpha, dtype=np.float64).reshape(-1, np.shape(alpha)[-1])
    b = np.asarray(beta, dtype=np.float64).reshape(-1, np.shape(beta)[-1])
    g = np.asarray(gamma, dtype=np.float64).reshape(-1, np.shape(gamma)[-1])
    if a.shape[0] != 1 or b.shape[0] != 1 or g.shape[0] != 1:
        raise ValueError("channel importance is defined for ell = 1")
    return np.abs(b[0]) * np.sqrt(np.sum(a[0] * a[0])) * np.sqrt(np.sum(g[0] * g[0]))


def select_channels(S1, S2, beta, keep):
    """The factors restricted to the middle channels ``keep`` (sorted,
    distinct, in [0, R)): columns of S1 [N][R], rows of S2 [R][M] and
    entries of beta [ell][R].  Host arrays in, host arrays out."""
    keep = np.asarray(keep, dtype=np.int64).reshape(-1)
    R = np.shape(S1)[1]
    if keep.size == 0:
        raise ValueError("a layer needs at least one channel")
    if keep.min() < 0 or keep.max() >= R or np.any(np.diff(keep) <= 0):
        raise ValueError("keep must be sorted, distinct indices in [0, R)")
    return (np.ascontiguousarray(np.asarray(S1)[:, keep]), np.ascontiguousarray(np.asarray(S2)[keep]),
            np.ascontiguousarray(np.asarray(beta)[:, keep]))
