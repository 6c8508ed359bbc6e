"""Plain fp64 CPU oracle of the per-matrix Muon update.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module: only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
call it. It shares no code with the HIP library (no kernels, headers, helpers or constant
tables); both sides only receive the same seeded inputs.

Every step is written out in float64 with NumPy, one library matmul per matrix product,
in the order the pages give, so that a reader can check it against them by eye.

Sources (three web pages on one subject):

* "MuonX: DMuon adjusts the multi-GPU division of labour, Gram NS lowers the compute"
  (Baidu Baige article on damodev.csdn.net), section 2 "why fewer but slower steps" and
  section 3.2 "Gram NS: fewer long matrix products".
* "DMuon: Efficient Distributed Muon Training with Near-Adam Overhead" (gist.science
  summary of the paper), technical summary section 1 (problem) and section 2.2
  (efficient Gram Newton-Schulz iteration).
* The X Square Robot DMuon announcement (agentren.cn), improvement 2 "shape-adaptive
  execution stack".

The pages do not print the Muon formulas. Readings taken where they are silent (each is
repeated where it is used):

* momentum is the heavy-ball sum ``M' = mu*M + G``; the Nesterov look-ahead is
  ``U = G + mu*M'`` (an EMA form only rescales U, which the normalisation cancels);
* tall matrices (rows > cols) are orthogonalised as their transpose, so the Gram matrix
  is always the small ``m' x m'`` one (the summary's section 2.2 states the saving for
  ``m < n``); a square matrix is not transposed;
* the normalisation is ``X0 = U / (||U||_F + eps)``;
* the quintic Newton-Schulz round with fixed coefficients (a, b, c) is
  ``A = X X^T; B = b*A + c*A^2; X <- a*X + B X``, the same coefficients every round;
* Gram segments: at each segment start ``R = X X^T`` is rebuilt and the transform Q
  restarts at I; every round forms ``A = Q R Q^T``, ``P = a*I + b*A + c*A^2``,
  ``Q <- P Q``; at the segment end ``X <- Q X``;
* the weight update is ``W' = W*(1 - lr*wd) - lr*O`` (decoupled decay, no extra scale).

Pins: ``tests/test_oracle.py`` checks every function here against closed forms (SVD of
an odd matrix polynomial, geometric series, rank-one inputs; the Frobenius normalisation
against singular values read off the spectrum of a rank-two and a full-rank input, where a
spectral-norm or other scaling gives different values), exact-arithmetic identities
(Gram = plain for any schedule, transpose and scale invariance), the singular-value band
the coefficients imply, the polar factor for the classical quintic, brute-force loops on
tiny inputs, and the FLOP counts the MuonX article prints for a 2560 x 9728 matrix.
"""

from __future__ import annotations

import numpy as np

# Quintic Newton-Schulz coefficients (a, b, c) used in Muon; the MuonX article (section
# 3.2) keeps "the existing fixed Muon coefficients" when it re-segments the iteration.
DEFAULT_COEFFS = (3.4445, -4.7750, 2.0315)
# 5 rounds split 2 + 2 + 1, Gram matrix rebuilt after rounds 2 and 4 (MuonX section 3.2).
DEFAULT_SEGMENTS = (2, 2, 1)


def as_f64(x) -> np.ndarray:
    """Read a stored array exactly into float64 (fp32 and bf16 values are exact in fp64)."""
    return np.array(x, dtype=np.float64, copy=True)


def momentum(G, M, mu: float, nesterov: bool = True):
    """Momentum smoothing of the gradient (MuonX article, section 2: Muon first smooths the
    gradient with momentum, then orthogonalises the update with Newton-Schulz).

    Returns ``(M_new, U)`` with ``M_new = mu*M + G`` and ``U = G + mu*M_new`` (Nesterov)
    or ``U = M_new``.
    """
    G = as_f64(G)
    M = as_f64(M)
    M_new = mu * M + G
    U = G + mu * M_new if nesterov else M_new
    return M_new, U


def orient(U):
    """Work on the short side: a matrix with more rows than columns is transposed so the
    Gram matrix X X^T is the smaller one (DMuon summary, section 2.2: the Gram form pays
    off for m < n). Returns ``(X, transposed)``."""
    U = as_f64(U)
    if U.shape[0] > U.shape[1]:
        return U.T.copy(), True
    return U, False


def frobenius_normalise(X, eps: float):
    """``X / (||X||_F + eps)``: bounds every singular value by 1 so the iteration stays in
    its convergence region."""
    X = as_f64(X)
    return X / (np.linalg.norm(X) + eps)


def ns_round(X, coeffs=DEFAULT_COEFFS):
    """One quintic Newton-Schulz round on the m x n iterate (MuonX article, sections 2 and
    3.2: every round needs products with the whole long matrix, two per round):
    ``A = X X^T``, ``B = b*A + c*A^2``, ``X <- a*X + B X``."""
    a, b, c = coeffs
    A = X @ X.T                      # long product 1 (m x n times n x m)
    B = b * A + c * (A @ A)          # square product
    return a * X + B @ X             # long product 2


def newton_schulz_plain(X0, coeffs=DEFAULT_COEFFS, rounds: int = 5):
    """Plain NS: ``rounds`` rounds of :func:`ns_round` directly on the long matrix."""
    X = as_f64(X0)
    for _ in range(rounds):
        X = ns_round(X, coeffs)
    return X


def newton_schulz_gram(X0, coeffs=DEFAULT_COEFFS, segments=DEFAULT_SEGMENTS):
    """Gram-space NS (MuonX article, section 3.2; DMuon summary, section 2.2).

    The iteration is moved into the m x m Gram space: per segment the Gram matrix
    ``R = X X^T`` is built once, the rounds accumulate an m x m transform Q, and only at
    the segment boundary is Q applied to the long matrix (``X <- Q X``). Q restarts at the
    identity in every segment. With ``X_k = Q_k X`` the plain round's ``A = X_k X_k^T``
    equals ``Q_k R Q_k^T``, so each round computes ``A = Q R Q^T`` (``= R`` in the first
    round, where Q is still I), ``P = a*I + b*A + c*A^2`` and ``Q <- P Q``.
    """
    a, b, c = coeffs
    X = as_f64(X0)
    m = X.shape[0]
    I = np.eye(m)
    for seg in segments:
        R = X @ X.T                              # long product: rebuild the Gram matrix
        Q = I
        for k in range(seg):
            A = R if k == 0 else (Q @ R) @ Q.T   # two square products after round 1
            P = a * I + b * A + c * (A @ A)      # square product
            Q = P if k == 0 else P @ Q           # square product after round 1
        X = Q @ X                                # long product: apply at the boundary
    return X


def weight_update(W, O, lr: float, wd: float):
    """Decoupled weight decay then the orthogonalised step: ``W*(1 - lr*wd) - lr*O``."""
    return as_f64(W) * (1.0 - lr * wd) - lr * as_f64(O)


def orthogonalise(U, *, eps=1e-7, coeffs=DEFAULT_COEFFS, mode="gram",
                  segments=DEFAULT_SEGMENTS, rounds=None):
    """Orientation, normalisation and NS for one momentum matrix; returns O in U's shape.

    ``mode`` is ``"plain"`` (``rounds`` rounds, default ``sum(segments)``) or ``"gram"``.
    """
    X, transposed = orient(U)
    X0 = frobenius_normalise(X, eps)
    if mode == "plain":
        n_rounds = int(sum(segments)) if rounds is None else int(rounds)
        O = newton_schulz_plain(X0, coeffs, n_rounds)
    elif mode == "gram":
        O = newton_schulz_gram(X0, coeffs, tuple(segments))
    else:
        raise ValueError(f"unknown mode {mode!r}")
    return O.T.copy() if transposed else O


def muon_step(W, G, M, *, lr=0.02, mu=0.95, wd=0.0, nesterov=True, eps=1e-7,
              coeffs=DEFAULT_COEFFS, mode="gram", segments=DEFAULT_SEGMENTS, rounds=None):
    """One Muon update of one 2-D weight: returns ``(W_new, M_new, O)`` in float64.

    Momentum, then orientation + Frobenius normalisation + Newton-Schulz, then the
    weight update. ``O`` (the orthogonalised update, shaped like W) is returned for
    diagnostics: with ``wd = 0``, ``W_new - W = -lr*O``.
    """
    M_new, U = momentum(G, M, mu, nesterov)
    O = orthogonalise(U, eps=eps, coeffs=coeffs, mode=mode, segments=segments, rounds=rounds)
    W_new = weight_update(W, O, lr, wd)
    return W_new, M_new, O
