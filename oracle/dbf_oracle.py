"""fp64 reference of the double-binary-factorised (DBF) product.

TEST INFRASTRUCTURE ONLY: used by ``tests/``, the package smoke check and the
benchmark's CPU-baseline leg; never by the product path.  Plain, slow and
written to be checked against the pages by eye.  It imports numpy only.

Sources (web summaries; cited by title and section):

* [LoRDBA] "Resumen Tecnico: LoRDBA - Adaptacion Binaria Doble de Bajo Rango
  para Ajuste Fino en Dispositivos", section 2 "Metodologia: LoRDBA",
  "Arquitectura Central": the update is a sum over ell terms of
  diag(alpha_i) B1 diag(beta_i) B2 diag(gamma_i), with B1 in {+-1}^{N x R},
  B2 in {+-1}^{R x M}; signs take one bit each, scales are fp16.  Its
  "Pipeline de Entrenamiento" step 2 binarises a real latent with sign(H).
* [DBF] "Addition is almost all you need: Compressing large language models
  with double binary factorization", technical summary section 2
  "Formulacion Matematica": W ~ (a . A . m^T)(B . b^T) with A, B sign matrices
  and a, m, b fp16 vectors; "Calculo en la inferencia": X W^T is evaluated as
  ((((X . b^T) B^T) . m^T) A^T) . a^T, i.e. scale, sign-accumulate, scale,
  sign-accumulate, scale.

Notation used throughout: x is [T][M] (token rows, the X of [DBF]); S1 = B1
(= A) is [N][R]; S2 = B2 (= B) is [R][M]; alpha (= a) [ell][N], beta (= m)
[ell][R], gamma (= b) [ell][M].  The two pages agree for ell = 1 under
a = alpha, A = B1, m = beta, B = B2, b = gamma, k = R.

Readings where the pages are silent (each is listed in the design notes):
* signs are shared by the ell terms, only the scales carry the term index
  ([LoRDBA] indexes only alpha, beta, gamma);
* sign(h) is -1 for h < 0 and +1 otherwise (so sign(0) = +1, NaN -> +1);
* the ell terms are summed in ascending order; any order is exact in fp64 up
  to rounding;
* an unmerged adapter branch may be added onto an existing output
  (``y_old``); out-of-range adapter ids contribute nothing.

Parity: every function below is pinned by ``tests/test_oracle_pins.py``
(closed forms, a library Hadamard matrix, brute force on tiny shapes,
invariances, and the pages' printed storage figures).
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "sign_of_latent",
    "delta_w",
    "forward",
    "forward_loops",
    "forward_rows",
    "forward_transposed",
    "forward_multi_adapter",
    "backward",
    "soft_sign_slope",
    "svid",
    "admm_scaled_sign",
    "factorize",
    "rank_for_bits",
    "channel_importance",
    "prune_channels",
    "stage1",
    "fp16_rne",
    "max_norm_error",
    "sign_bits",
    "scale_bytes",
    "bits_per_weight",
    "compression_vs_fp16_lora",
]

# Row-block size used only to bound memory when a sign matrix is widened to
# float64; each output element is still one complete dot product.
_ROW_BLOCK = 2048


def _f64(a) -> np.ndarray:
    return np.asarray(a).astype(np.float64)


def _terms(alpha, beta, gamma):
    a, b, g = _f64(alpha), _f64(beta), _f64(gamma)
    if a.ndim == 1:
        a, b, g = a[None], b[None], g[None]
    if not (a.shape[0] == b.shape[0] == g.shape[0]):
        raise ValueError("alpha, beta, gamma must have the same number of terms")
    return a, b, g


def sign_of_latent(h) -> np.ndarray:
    """[LoRDBA] "Pipeline de Entrenamiento", step 2: B = sign(H).

    Reading: -1 where h < 0, +1 everywhere else (h = +0, -0 and NaN give +1).
    Returns int8."""
    h = np.asarray(h)
    return np.where(h < 0, -1, 1).astype(np.int8)


def delta_w(S1, S2, alpha, beta, gamma) -> np.ndarray:
    """[LoRDBA] "Arquitectura Central", the update equation written out:
    dW = sum_i diag(alpha_i) @ S1 @ diag(beta_i) @ S2 @ diag(gamma_i), [N][M]
    in float64 (dense; for small shapes)."""
    a, b, g = _terms(alpha, beta, gamma)
    s1, s2 = _f64(S1), _f64(S2)
    dw = np.zeros((s1.shape[0], s2.shape[1]))
    for i in range(a.shape[0]):
        dw += np.diag(a[i]) @ s1 @ np.diag(b[i]) @ s2 @ np.diag(g[i])
    return dw


def stage1(x, S2, beta_i, gamma_i) -> np.ndarray:
    """[DBF] "Calculo en la inferencia", the first three steps for one term:
    Z = ((X . gamma^T) S2^T) . beta^T, [T][R] float64."""
    v = _f64(x) * _f64(gamma_i)[None, :]
    R = np.asarray(S2).shape[0]
    u = np.empty((v.shape[0], R))
    for r0 in range(0, R, _ROW_BLOCK):
        u[:, r0:r0 + _ROW_BLOCK] = v @ _f64(S2[r0:r0 + _ROW_BLOCK]).T
    return u * _f64(beta_i)[None, :]


def forward(x, S1, S2, alpha, beta, gamma, y_old=None) -> np.ndarray:
    """[DBF] "Calculo en la inferencia" applied to every term of the [LoRDBA]
    sum: for each i (ascending)
        V = X . gamma_i,  U = V S2^T,  Z = U . beta_i,  W = Z S1^T,
        Y += W . alpha_i
    Returns Y [T][N] float64 (plus ``y_old`` when given, the unmerged adapter
    branch added onto a base output)."""
    a, b, g = _terms(alpha, beta, gamma)
    x = _f64(x)
    N = np.asarray(S1).shape[0]
    y = np.zeros((x.shape[0], N))
    for i in range(a.shape[0]):
        z = stage1(x, S2, b[i], g[i])
        w = np.empty_like(y)
        for n0 in range(0, N, _ROW_BLOCK):
            w[:, n0:n0 + _ROW_BLOCK] = z @ _f64(S1[n0:n0 + _ROW_BLOCK]).T
        y += w * a[i][None, :]
    if y_old is not None:
        y += _f64(y_old)
    return y


def forward_loops(x, S1, S2, alpha, beta, gamma) -> list:
    """The same product as ``forward`` with explicit Python loops and no
    library routine (tiny shapes only): y[t][n] = sum_i alpha_i[n] *
    sum_r S1[n][r] * beta_i[r] * sum_m S2[r][m] * gamma_i[m] * x[t][m]."""
    a, b, g = _terms(alpha, beta, gamma)
    xs = _f64(x).tolist()
    s1 = np.asarray(S1).astype(int).tolist()
    s2 = np.asarray(S2).astype(int).tolist()
    a, b, g = a.tolist(), b.tolist(), g.tolist()
    N, R, M = len(s1), len(s2), len(s2[0]) if s2 else 0
    out = []
    for xt in xs:
        row = [0.0] * N
        for i in range(len(a)):
            z = []
            for r in range(R):
                acc = 0.0
                for m in range(M):
                    acc += s2[r][m] * (g[i][m] * xt[m])
                z.append(acc * b[i][r])
            for n in range(N):
                acc = 0.0
                for r in range(R):
                    acc += s1[n][r] * z[r]
                row[n] += acc * a[i][n]
        out.append(row)
    return out


def forward_rows(x_rows, S1, S2, alpha, beta, gamma, n_idx) -> np.ndarray:
    """Sampled outputs: y[t][n] for the given token rows and output indices
    only.  Same steps as ``forward``; stage 2 is evaluated for the selected
    rows of S1.  Returns [len(x_rows)][len(n_idx)] float64."""
    a, b, g = _terms(alpha, beta, gamma)
    n_idx = np.asarray(n_idx)
    s1 = _f64(np.asarray(S1)[n_idx])
    y = np.zeros((np.asarray(x_rows).shape[0], len(n_idx)))
    for i in range(a.shape[0]):
        z = stage1(x_rows, S2, b[i], g[i])
        y += (z @ s1.T) * a[i][n_idx][None, :]
    return y


def forward_transposed(gvec, S1, S2, alpha, beta, gamma) -> np.ndarray:
    """The adjoint product dW^T g = sum_i diag(gamma_i) S2^T diag(beta_i)
    S1^T diag(alpha_i) g, for g [T][N]; returns [T][M] float64.  (The
    transpose of the [LoRDBA] update is again a DBF product with the roles of
    the two sign matrices and of alpha/gamma exchanged.)"""
    a, b, gm = _terms(alpha, beta, gamma)
    gv = _f64(gvec)
    out = np.zeros((gv.shape[0], np.asarray(S2).shape[1]))
    for i in range(a.shape[0]):
        p = (gv * a[i][None, :]) @ _f64(S1)
        p = p * b[i][None, :]
        out += (p @ _f64(S2)) * gm[i][None, :]
    return out


def soft_sign_slope(h, tau) -> np.ndarray:
    """[LoRDBA] "Pipeline de Entrenamiento", step 3: the backward pass lets the
    gradient through sign() with a soft-sign straight-through estimator under
    a temperature schedule.  Reading (the page gives no formula): the surrogate
    is tanh(h / tau), so d sign(h)/dh is replaced by its slope
    (1 - tanh(h / tau)^2) / tau; tau > 0 is the current temperature (the
    schedule belongs to the caller)."""
    th = np.tanh(_f64(h) / float(tau))
    return (1.0 - th * th) / float(tau)


def backward(x, gout, S1, S2, alpha, beta, gamma, H1=None, H2=None, tau=None) -> dict:
    """Backward pass of one layer for quantisation-aware training ([LoRDBA]
    "Pipeline de Entrenamiento", steps 3 and 4: the sign carriers and the
    scale vectors are trained together).  With G = dL/dY [T][N] for
    Y = forward(x, ...), and for each term i (ascending) the forward's steps
        V_i = X . gamma_i,  U_i = V_i S2^T,  Z_i = U_i . beta_i,  W_i = Z_i S1^T
    and the adjoint's steps (the transposed product)
        P_i = (G . alpha_i) S1,  Q_i = (P_i . beta_i) S2,
    the chain rule on the update equation ("Arquitectura Central") gives
        dalpha_i[n] = sum_t G[t,n] W_i[t,n]
        dbeta_i[r]  = sum_t U_i[t,r] P_i[t,r]
        dgamma_i[m] = sum_t X[t,m] Q_i[t,m]
        dX  = sum_i Q_i . gamma_i                       [T][M]
        dS1 = sum_i (G . alpha_i)^T Z_i                 [N][R]
        dS2 = sum_i (P_i . beta_i)^T V_i                [R][M]
    (the signs are shared by the terms, so their gradients sum over i).  With
    latents H1, H2 (S = sign(H)) and a temperature tau, the straight-through
    gradients are dH = dS * soft_sign_slope(H, tau).  Returns a dict of
    float64 arrays; dalpha, dbeta, dgamma are [ell][*]."""
    a, b, g = _terms(alpha, beta, gamma)
    x, G = _f64(x), _f64(gout)
    s1, s2 = _f64(S1), _f64(S2)
    ell = a.shape[0]
    out = {"dalpha": np.zeros_like(a), "dbeta": np.zeros_like(b), "dgamma": np.zeros_like(g),
           "dx": np.zeros_like(x), "dS1": np.zeros_like(s1), "dS2": np.zeros_like(s2)}
    for i in range(ell):
        v = x * g[i][None, :]
        u = v @ s2.T
        z = u * b[i][None, :]
        w = z @ s1.T
        ga = G * a[i][None, :]
        p = ga @ s1
        pb = p * b[i][None, :]
        q = pb @ s2
        out["dalpha"][i] = (G * w).sum(axis=0)
        out["dbeta"][i] = (u * p).sum(axis=0)
        out["dgamma"][i] = (x * q).sum(axis=0)
        out["dx"] += q * g[i][None, :]
        out["dS1"] += ga.T @ z
        out["dS2"] += pb.T @ v
    if H1 is not None:
        out["dH1"] = out["dS1"] * soft_sign_slope(H1, tau)
    if H2 is not None:
        out["dH2"] = out["dS2"] * soft_sign_slope(H2, tau)
    return out


def svid(Y):
    """[DBF] section 2 "Algoritmo de Optimizacion", the SVID projection: the
    sign of Y times the best rank-1 approximation of its magnitude |Y|.  The
    rank-1 factor is the top singular triplet (sigma, u, v) of |Y| (u, v >= 0:
    |Y| has no negative entry), split as u' = sqrt(sigma) u, v' = sqrt(sigma) v.
    Returns (u', S, v') with S = sign(Y) (h < 0 -> -1, else +1) as int8, so the
    projection is diag(u') S diag(v')."""
    Y = _f64(Y)
    S = np.where(Y < 0, -1, 1).astype(np.int8)
    uu, sig, vt = np.linalg.svd(np.abs(Y), full_matrices=False)
    u, v = uu[:, 0], vt[0]
    if u.sum() < 0:  # the singular pair is defined up to a joint sign
        u, v = -u, -v
    r = np.sqrt(sig[0])
    return r * u, S, r * v


def _svid_matrix(Y):
    u, S, v = svid(Y)
    return u[:, None] * S * v[None, :]


def admm_scaled_sign(W, F, side, Z, iters, rho0):
    """[DBF] "Algoritmo de Optimizacion", one alternating-minimisation half
    step: with the other factor F fixed, ADMM on
        min ||W - X F||^2 (side "A": X is N x k, F is k x M)  or
        min ||W - F X||^2 (side "B": X is k x M, F is N x k)
    subject to X in the set of scaled sign matrices diag(u) S diag(v), in the
    scaled form (dual U, penalty rho = rho0 * trace(G) / k with G the Gram
    matrix of F):
        X <- argmin_X ||W - X F||^2 + rho ||X - Z + U||^2   (a linear solve)
        Z <- SVID(X + U)
        U <- U + X - Z
    starting from the feasible Z given and U = 0.  Returns the final Z."""
    W, F, Z = _f64(W), _f64(F), _f64(Z)
    k = F.shape[0] if side == "A" else F.shape[1]
    G = F @ F.T if side == "A" else F.T @ F
    rho = rho0 * np.trace(G) / k
    reg = G + rho * np.eye(k)
    base = W @ F.T if side == "A" else F.T @ W  # N x k, or k x M
    U = np.zeros_like(Z)
    for _ in range(iters):
        rhs = base + rho * (Z - U)
        X = np.linalg.solve(reg, rhs.T).T if side == "A" else np.linalg.solve(reg, rhs)
        Z = _svid_matrix(X + U)
        U = U + X - Z
    return Z


def factorize(W, k, omega, outer, admm_iters, rho0=1.0, start=None):
    """[DBF] "Algoritmo de Optimizacion": W (N x M) ~ X Y with X = diag(a) A
    diag(m) (N x k) and Y = diag(r) B diag(b) (k x M), A and B sign matrices,
    by alternating minimisation (fix Y and solve for X, then fix X and solve
    for Y), each half step an ADMM run projecting with SVID.  Readings (the
    page gives the method, not its constants): the start is Y0 = SVID(omega W)
    for a Gaussian k x N sketch omega (drawn by the caller), X0 = 0; each half
    step starts its ADMM from the side's current value (X0's first run from
    SVID of the unconstrained least-squares solution) and ends on the
    projection Z, so both factors stay feasible; r is folded into m at the end.
    Returns dict(alpha=a, S1=A, beta=m*r, S2=B, gamma=b, rel_err), the
    factors of the layer y = diag(a) A diag(beta) B diag(b) x.  ``start``
    (X0, Y0), both scaled sign matrices, replaces the sketch start."""
    W = _f64(W)
    if start is None:
        Y = _svid_matrix(_f64(omega) @ W)
        X = None
    else:
        X, Y = _f64(start[0]), _f64(start[1])
    for _ in range(outer):
        if X is None:
            G = Y @ Y.T
            rho = rho0 * np.trace(G) / k
            X = _svid_matrix(np.linalg.solve(G + rho * np.eye(k), (W @ Y.T).T).T)
        X = admm_scaled_sign(W, Y, "A", X, admm_iters, rho0)
        Y = admm_scaled_sign(W, X, "B", Y, admm_iters, rho0)
    a, A, m = svid(X)
    r, B, b = svid(Y)
    rel = float(np.linalg.norm(W - (a[:, None] * A * (m * r)[None, :]) @ (B * b[None, :]))
                / np.linalg.norm(W))
    return {"alpha": a, "S1": A, "beta": m * r, "S2": B, "gamma": b, "rel_err": rel}


def forward_multi_adapter(x, ids, adapters, y_old=None) -> np.ndarray:
    """Per-token routing: y[t] = DBF_{ids[t]}(x[t]) when 0 <= ids[t] <
    len(adapters), otherwise 0 (or y_old[t] when a base output is given).
    ``adapters`` is a sequence of objects with S1, S2, alpha, beta, gamma."""
    x = _f64(x)
    ids = np.asarray(ids)
    N = np.asarray(adapters[0].S1).shape[0]
    y = np.zeros((x.shape[0], N)) if y_old is None else _f64(y_old).copy()
    for a_idx, ad in enumerate(adapters):
        rows = np.nonzero(ids == a_idx)[0]
        if rows.size == 0:
            continue
        y[rows] += forward(x[rows], ad.S1, ad.S2, ad.alpha, ad.beta, ad.gamma)
    return y


def fp16_rne(y) -> np.ndarray:
    """Round float64 results to fp16, nearest-even, overflow to +-inf
    (the pages store the scales in fp16; the output uses the same type)."""
    with np.errstate(over="ignore"):
        return np.asarray(y, dtype=np.float64).astype(np.float16)


def max_norm_error(y, y_ref) -> float:
    """max |y - y_ref| / max |y_ref| (0 when both are all-zero)."""
    y = _f64(y)
    y_ref = _f64(y_ref)
    den = np.max(np.abs(y_ref)) if y_ref.size else 0.0
    num = np.max(np.abs(y - y_ref)) if y_ref.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


def sign_bits(N: int, R: int, M: int) -> int:
    """[LoRDBA] "Eficiencia de Almacenamiento": one bit per sign entry of
    B1 (N x R) and B2 (R x M)."""
    return N * R + R * M


def scale_bytes(N: int, R: int, M: int, ell: int) -> int:
    """fp16 alpha_i (N), beta_i (R), gamma_i (M) for each of the ell terms."""
    return 2 * ell * (N + R + M)


def bits_per_weight(N: int, R: int, M: int, ell: int = 1) -> float:
    """Storage per entry of the N x M matrix the factors stand for
    ([DBF] "Control Granular de Compresion": the middle width k sets it)."""
    return (sign_bits(N, R, M) + 8 * scale_bytes(N, R, M, ell)) / (N * M)


def rank_for_bits(N: int, M: int, bpw: float, ell: int = 1) -> int:
    """[DBF] "Control Granular de Compresion": the middle width k sets the bits
    per weight, so a (fractional) budget picks k: the largest k >= 0 with
    bits_per_weight(N, k, M, ell) <= bpw, i.e. the floor of
    (bpw N M - 16 ell (N + M)) / (N + M + 16 ell)."""
    num = bpw * N * M - 16 * ell * (N + M)
    return max(0, int(math.floor(num / (N + M + 16 * ell))))


def channel_importance(alpha, beta, gamma) -> np.ndarray:
    """[DBF] section 3, "Poda Iterativa No Uniforme": the middle dimension is
    treated as channels and pruned by importance.  Reading (data-free, ell =
    1): channel r contributes the rank-1 term beta_r (alpha . S1[:, r])
    (S2[r, :] . gamma) to the update; its Frobenius norm, whatever the signs,
    is |beta_r| ||alpha|| ||gamma||, the importance used here."""
    a, b, g = _terms(alpha, beta, gamma)
    if a.shape[0] != 1:
        raise ValueError("channel importance is defined for ell = 1")
    return np.abs(b[0]) * np.linalg.norm(a[0]) * np.linalg.norm(g[0])


def prune_channels(shapes, importances, budget_bits):
    """[DBF] "Poda Iterativa No Uniforme" over a stack of layers: repeatedly
    drop the globally least important remaining channel (ties: lower layer,
    then lower channel index first) until the stack's storage (sign bits plus
    fp16 scales, ell = 1) fits budget_bits.  Dropping a channel of an N x M
    layer saves N + M sign bits and one 16-bit beta entry.  shapes is a list
    of (N, R, M); importances a list of length-R arrays.  Returns the kept
    channel indices per layer (sorted)."""
    keep = [np.ones(R, bool) for (_, R, _) in shapes]
    total = sum(sign_bits(N, R, M) + 8 * scale_bytes(N, R, M, 1) for (N, R, M) in shapes)
    order = sorted(((float(imp[r]), li, r) for li, imp in enumerate(importances)
                    for r in range(len(imp))))
    for _, li, r in order:
        if total <= budget_bits:
            break
        N, _, M = shapes[li]
        keep[li][r] = False
        total -= N + M + 16
    return [np.nonzero(k)[0] for k in keep]


def compression_vs_fp16_lora(N: int, R: int, M: int, ell: int = 1) -> float:
    """Footprint of an fp16 LoRA pair of rank R (16 R (N + M) bits) over the
    footprint of the binary adapter of the same rank."""
    return (16 * R * (N + M)) / (sign_bits(N, R, M) + 8 * scale_bytes(N, R, M, ell))
