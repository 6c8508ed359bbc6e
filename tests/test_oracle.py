"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these re-types the oracle's formulas: each compares it with an independent route
(an SVD closed form, a scalar recurrence on singular values, a geometric series, brute
force loops, exact-arithmetic identities, the FLOP counts the MuonX article prints), and
``test_planted_mistakes_are_caught`` checks that plausible slips in the oracle's NS code
fail those same checks.
"""

import json
import os

import numpy as np
import pytest

from oracle import flop_model
from oracle import muon as om

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
COEFFS = om.DEFAULT_COEFFS
CLASSICAL = (15.0 / 8.0, -10.0 / 8.0, 3.0 / 8.0)   # the textbook quintic polar iteration


def phi_iter(x, coeffs, rounds):
    """Scalar odd polynomial phi(x) = a x + b x^3 + c x^5 applied ``rounds`` times."""
    a, b, c = coeffs
    x = np.asarray(x, dtype=np.float64)
    for _ in range(rounds):
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def svd_closed_form(X0, coeffs, rounds):
    """An odd matrix polynomial acts on singular values only: U diag(phi^r(s)) V^T."""
    U, s, Vt = np.linalg.svd(X0, full_matrices=False)
    return (U * phi_iter(s, coeffs, rounds)) @ Vt


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / np.linalg.norm(np.asarray(b)))


def normalised(rng, m, n):
    X = rng.standard_normal((m, n))
    return X / np.linalg.norm(X)


SHAPES = [(8, 32), (16, 48), (33, 70), (64, 256), (50, 50)]


# ---------------------------------------------------------------- FLOP model (printed values)

def test_flop_model_matches_muonx_printed_counts():
    g = json.load(open(os.path.join(GOLDEN, "muonx_flop_counts_2560x9728.json")))
    rows, cols = g["rows"], g["cols"]
    tol = g["printed_precision"]
    assert flop_model.product_counts("plain") == (g["plain"]["long_products"], g["plain"]["square_products"])
    assert flop_model.product_counts("gram", tuple(g["gram"]["segments"])) == (
        g["gram"]["long_products"], g["gram"]["square_products"])
    plain = flop_model.dense_flops(rows, cols, "plain") / 1e12
    gram = flop_model.dense_flops(rows, cols, "gram", tuple(g["gram"]["segments"])) / 1e12
    assert abs(plain - g["plain"]["tflops"]) <= tol["tflops"]
    assert abs(gram - g["gram"]["tflops"]) <= tol["tflops"]
    assert abs(100.0 * (1.0 - gram / plain) - g["reduction_percent"]) <= tol["reduction_percent"]
    # orientation does not change the count (the tall form is the transpose)
    assert flop_model.dense_flops(cols, rows, "gram") == flop_model.dense_flops(rows, cols, "gram")


def test_flop_model_counts_the_oracle_products():
    """Count the matmuls the oracle actually performs and compare with the model."""
    rng = np.random.default_rng(7)
    m, n = 6, 20

    class Counter(np.ndarray):
        calls = []

        def __matmul__(self, other):
            a, b = np.asarray(self), np.asarray(other)
            Counter.calls.append((a.shape, b.shape))
            return np.ndarray.__matmul__(a, b).view(Counter)

        def __rmatmul__(self, other):
            a, b = np.asarray(other), np.asarray(self)
            Counter.calls.append((a.shape, b.shape))
            return np.ndarray.__matmul__(a, b).view(Counter)

    X0 = normalised(rng, m, n)
    for mode, segs in [("plain", (2, 2, 1)), ("gram", (2, 2, 1)), ("gram", (2, 3)), ("gram", (1, 1, 1, 1, 1))]:
        Counter.calls = []
        orig_eye, orig_asf = np.eye, om.as_f64
        try:
            om.as_f64 = lambda x: np.array(x, dtype=np.float64).view(Counter)
            om.np.eye = lambda k: orig_eye(k).view(Counter)
            if mode == "plain":
                om.newton_schulz_plain(X0, COEFFS, sum(segs))
            else:
                om.newton_schulz_gram(X0, COEFFS, segs)
        finally:
            om.as_f64, om.np.eye = orig_asf, orig_eye
        longs = sum(1 for (sa, sb) in Counter.calls if n in sa or n in sb)
        squares = len(Counter.calls) - longs
        assert (longs, squares) == flop_model.product_counts(mode, segs), (mode, segs, Counter.calls)


# ---------------------------------------------------------------- NS closed forms

@pytest.mark.parametrize("m,n", SHAPES)
def test_plain_matches_svd_closed_form(m, n):
    X0 = normalised(np.random.default_rng(m * 1000 + n), m, n)
    for coeffs, rounds in [(COEFFS, 5), (COEFFS, 3), (CLASSICAL, 4)]:
        assert rel(om.newton_schulz_plain(X0, coeffs, rounds), svd_closed_form(X0, coeffs, rounds)) < 1e-12


@pytest.mark.parametrize("segments", [(2, 2, 1), (2, 3), (1, 1, 1, 1, 1), (5,), (3, 2), (1, 4)])
@pytest.mark.parametrize("m,n", SHAPES)
def test_gram_equals_plain_and_closed_form(m, n, segments):
    X0 = normalised(np.random.default_rng(m * 7 + n), m, n)
    rounds = sum(segments)
    g = om.newton_schulz_gram(X0, COEFFS, segments)
    p = om.newton_schulz_plain(X0, COEFFS, rounds)
    assert rel(g, p) < 1e-10
    assert rel(g, svd_closed_form(X0, COEFFS, rounds)) < 1e-12


def test_gram_all_ones_schedule_is_plain():
    X0 = normalised(np.random.default_rng(3), 24, 80)
    g = om.newton_schulz_gram(X0, COEFFS, (1, 1, 1, 1, 1))
    assert rel(g, om.newton_schulz_plain(X0, COEFFS, 5)) < 1e-14


def test_singular_value_band():
    """Every output singular value is phi^5 of the input one, inside the band phi^5 maps
    [s_min, 1] into (sampled densely on the scalar polynomial)."""
    rng = np.random.default_rng(11)
    grid = np.linspace(1.55e-3, 1.0, 200001)
    band = phi_iter(grid, COEFFS, 5)
    lo, hi = band.min(), band.max()
    assert 0.68 < lo < 0.69 and 1.20 < hi < 1.21
    for m, n in [(32, 128), (64, 64), (40, 300)]:
        U, _ = np.linalg.qr(rng.standard_normal((m, m)))
        V, _ = np.linalg.qr(rng.standard_normal((n, m)))
        s = np.geomspace(1.0, 2e-3, m)
        X0 = (U * s) @ V.T
        X0 /= np.linalg.norm(X0)
        s_in = np.linalg.svd(X0, compute_uv=False)
        for mode in ("plain", "gram"):
            O = om.newton_schulz_plain(X0, COEFFS, 5) if mode == "plain" else om.newton_schulz_gram(X0, COEFFS)
            s_out = np.linalg.svd(O, compute_uv=False)
            assert np.allclose(np.sort(s_out), np.sort(phi_iter(s_in, COEFFS, 5)), rtol=1e-11, atol=1e-13)
            keep = s_in >= 1.55e-3
            sv = phi_iter(s_in[keep], COEFFS, 5)
            assert np.all(sv >= lo - 1e-12) and np.all(sv <= hi + 1e-12)


def test_polar_factor():
    """Classical quintic from a well-conditioned start reaches U V^T (numpy SVD); the
    Muon coefficients land within the band-implied distance of it."""
    rng = np.random.default_rng(5)
    m, n = 48, 160
    U, _ = np.linalg.qr(rng.standard_normal((m, m)))
    V, _ = np.linalg.qr(rng.standard_normal((n, m)))
    s = np.linspace(1.0, 0.1, m)
    X0 = (U * s) @ V.T
    X0 /= np.linalg.norm(X0)
    Us, _, Vts = np.linalg.svd(X0, full_matrices=False)
    polar = Us @ Vts
    assert rel(om.newton_schulz_gram(X0, CLASSICAL, (2, 2, 2, 2, 2, 2, 2, 2)), polar) < 1e-10
    assert rel(om.newton_schulz_plain(X0, CLASSICAL, 16), polar) < 1e-10
    s_in = np.linalg.svd(X0, compute_uv=False)
    bound = np.max(np.abs(phi_iter(s_in, COEFFS, 5) - 1.0))
    d = rel(om.newton_schulz_gram(X0), polar)
    assert d <= bound + 1e-12 and bound < 0.32


def test_rank_one_closed_form():
    rng = np.random.default_rng(2)
    u, v = rng.standard_normal(12), rng.standard_normal(40)
    G = np.outer(u, v)
    O = om.orthogonalise(G, eps=0.0)
    expect = phi_iter(1.0, COEFFS, 5) * np.outer(u / np.linalg.norm(u), v / np.linalg.norm(v))
    assert rel(O, expect) < 1e-13


def test_diagonal_input_is_scalar_iteration():
    d = np.array([0.7, 0.5, 0.3, 0.1, 0.01])
    X0 = np.zeros((5, 9))
    X0[np.arange(5), np.arange(5)] = d
    O = om.newton_schulz_gram(X0)
    expect = np.zeros_like(X0)
    expect[np.arange(5), np.arange(5)] = phi_iter(d, COEFFS, 5)
    assert np.max(np.abs(O - expect)) < 1e-14


# ---------------------------------------------------------------- invariances and brute force

def test_transpose_invariance():
    rng = np.random.default_rng(9)
    G = rng.standard_normal((30, 90))
    for mode in ("plain", "gram"):
        O_wide = om.orthogonalise(G, mode=mode)
        O_tall = om.orthogonalise(G.T, mode=mode)
        assert O_tall.shape == (90, 30)
        assert rel(O_tall, O_wide.T) < 1e-12


def test_square_is_not_transposed():
    X = np.arange(9.0).reshape(3, 3)
    Y, t = om.orient(X)
    assert not t and np.array_equal(Y, X)
    Y, t = om.orient(np.ones((4, 3)))
    assert t and Y.shape == (3, 4)


def test_scale_invariance():
    rng = np.random.default_rng(4)
    G = rng.standard_normal((20, 64))
    O1 = om.orthogonalise(G, eps=0.0)
    O2 = om.orthogonalise(37.5 * G, eps=0.0)
    assert rel(O2, O1) < 1e-12


def _loop_matmul(A, B):
    n, k = len(A), len(A[0])
    m = len(B[0])
    return [[sum(A[i][t] * B[t][j] for t in range(k)) for j in range(m)] for i in range(n)]


def test_brute_force_tiny():
    """Plain NS with pure-Python loops for every product on a 3 x 7 input."""
    rng = np.random.default_rng(1)
    X = normalised(rng, 3, 7)
    a, b, c = COEFFS
    Xl = X.tolist()
    for _ in range(5):
        Xt = [list(r) for r in zip(*Xl)]
        A = _loop_matmul(Xl, Xt)
        A2 = _loop_matmul(A, A)
        B = [[b * A[i][j] + c * A2[i][j] for j in range(3)] for i in range(3)]
        BX = _loop_matmul(B, Xl)
        Xl = [[a * Xl[i][j] + BX[i][j] for j in range(7)] for i in range(3)]
    assert np.max(np.abs(np.array(Xl) - om.newton_schulz_plain(X))) < 1e-13
    assert np.max(np.abs(np.array(Xl) - om.newton_schulz_gram(X))) < 1e-13


# ---------------------------------------------------------------- momentum and update

def test_momentum_geometric_series():
    """Constant G from M0 = 0: M_t = G (1 - mu^t) / (1 - mu); Nesterov U_t = G + mu M_t."""
    rng = np.random.default_rng(6)
    G = rng.standard_normal((4, 6))
    mu = 0.95
    M = np.zeros_like(G)
    for t in range(1, 8):
        M, U = om.momentum(G, M, mu, nesterov=True)
        geo = (1.0 - mu ** t) / (1.0 - mu)
        assert np.allclose(M, G * geo, rtol=1e-14, atol=0)
        assert np.allclose(U, G * (1.0 + mu * geo), rtol=1e-14, atol=0)
    M2, U2 = om.momentum(G, np.zeros_like(G), mu, nesterov=False)
    assert np.array_equal(M2, G) and np.array_equal(U2, G)


def test_update_identity_and_zero_gradient():
    rng = np.random.default_rng(8)
    W = rng.standard_normal((16, 40))
    G = rng.standard_normal((16, 40))
    M = np.zeros_like(G)
    W1, M1, O = om.muon_step(W, G, M, lr=0.02, wd=0.0)
    assert np.allclose(W1 - W, -0.02 * O, rtol=0, atol=1e-15)
    W2, _, O2 = om.muon_step(W, G, M, lr=0.02, wd=0.1)
    assert np.allclose(W2, W * (1 - 0.002) - 0.02 * O2, rtol=0, atol=1e-15)
    # zero gradient and zero momentum: the update vanishes, only decay acts
    W3, M3, O3 = om.muon_step(W, np.zeros_like(W), M, lr=0.02, wd=0.1)
    assert np.all(O3 == 0) and np.allclose(W3, W * (1 - 0.002))


def test_ema_momentum_gives_same_weights():
    """Reading check: the EMA form (1-mu) scales U, which the normalisation cancels."""
    rng = np.random.default_rng(12)
    W = rng.standard_normal((10, 30))
    Gs = [rng.standard_normal((10, 30)) for _ in range(3)]
    M = np.zeros_like(W)
    Me = np.zeros_like(W)
    for G in Gs:
        _, M, O = om.muon_step(W, G, M, eps=0.0)
        Me = 0.95 * Me + 0.05 * G
        Ue = 0.05 * G + 0.95 * Me
        Oe = om.orthogonalise(Ue, eps=0.0)
        assert rel(Oe, O) < 1e-12


# ---------------------------------------------------------------- the pins catch planted mistakes

def _plain_mutant(kind):
    a, b, c = COEFFS

    def ns(X0, coeffs=COEFFS, rounds=5):
        X = np.array(X0, dtype=np.float64)
        for _ in range(rounds):
            if kind == "gram_transposed":
                A = X.T @ X if X.shape[0] == X.shape[1] else X @ X.T
            else:
                A = X @ X.T
            if kind == "drop_c":
                B = b * A
            elif kind == "sign_b":
                B = -b * A + c * (A @ A)
            else:
                B = b * A + c * (A @ A)
            X = a * X + (X @ B if kind == "right_multiply" and X.shape[0] == X.shape[1] else B @ X)
        return X
    return ns


def _gram_mutant(kind):
    a, b, c = COEFFS

    def ns(X0, coeffs=COEFFS, segments=(2, 2, 1)):
        X = np.array(X0, dtype=np.float64)
        I = np.eye(X.shape[0])
        Q = I
        for seg in segments:
            R = X @ X.T
            if kind != "no_reset":
                Q = I
            for k in range(seg):
                if kind == "no_reset":
                    A = (Q @ R) @ Q.T
                elif kind == "QR_only":
                    A = R if k == 0 else Q @ R
                else:
                    A = R if k == 0 else (Q @ R) @ Q.T
                P = a * I + b * A + c * (A @ A)
                Q = P if (k == 0 and kind != "no_reset") else P @ Q
            X = Q @ X if kind != "stale_X" else Q @ X0
        return X
    return ns


@pytest.mark.parametrize("kind", ["drop_c", "sign_b", "gram_transposed", "right_multiply"])
def test_planted_mistakes_are_caught_plain(kind):
    rng = np.random.default_rng(21)
    X0 = normalised(rng, 12, 12)
    with np.errstate(all="ignore"):
        mut = _plain_mutant(kind)(X0, COEFFS, 5)
        err = rel(mut, svd_closed_form(X0, COEFFS, 5))
    assert not (err <= 1e-6)   # NaN or overflow also counts as caught


@pytest.mark.parametrize("kind", ["no_reset", "QR_only", "stale_X"])
def test_planted_mistakes_are_caught_gram(kind):
    rng = np.random.default_rng(22)
    X0 = normalised(rng, 12, 30)
    with np.errstate(all="ignore"):
        mut = _gram_mutant(kind)(X0, COEFFS, (2, 2, 1))
        err = rel(mut, om.newton_schulz_plain(X0, COEFFS, 5))
    assert not (err <= 1e-6)


# ---------------------------------------------------------------- Frobenius normalisation

def _rank_two(m=6, n=10, seed=0):
    rng = np.random.default_rng(seed)
    U, _ = np.linalg.qr(rng.standard_normal((m, 2)))
    V, _ = np.linalg.qr(rng.standard_normal((n, 2)))
    return (U * np.array([3.0, 4.0])) @ V.T


def test_frobenius_normalise_rank_two():
    """Singular values (3, 4): the Frobenius norm is 5, so X0 has singular values (0.6, 0.8);
    a spectral-norm scaling would give (0.75, 1). With eps = 5 the divisor is 5 + 5 = 10."""
    X = _rank_two()
    s = np.linalg.svd(om.frobenius_normalise(X, 0.0), compute_uv=False)
    assert np.allclose(s[:2], [0.8, 0.6], rtol=0, atol=1e-15) and np.all(s[2:] < 1e-15)
    s = np.linalg.svd(om.frobenius_normalise(X, 5.0), compute_uv=False)
    assert np.allclose(s[:2], [0.4, 0.3], rtol=0, atol=1e-15)
    s = np.linalg.svd(om.frobenius_normalise(X.T, 0.0), compute_uv=False)   # orientation-free
    assert np.allclose(s[:2], [0.8, 0.6], rtol=0, atol=1e-15)


def normalised_closed_form(G, coeffs, rounds):
    """O from the raw momentum: with G = U diag(s) V^T, X0 has singular values
    s / sqrt(sum s^2) (the Frobenius norm read off the spectrum, not computed from the
    entries) and NS maps them through phi^rounds."""
    U, s, Vt = np.linalg.svd(np.asarray(G, np.float64), full_matrices=False)
    return (U * phi_iter(s / np.sqrt(np.sum(s * s)), coeffs, rounds)) @ Vt


@pytest.mark.parametrize("shape", [(24, 80), (80, 24)])
@pytest.mark.parametrize("mode", ["plain", "gram"])
def test_orthogonalise_full_rank_closed_form(shape, mode):
    """Full rank with a spread spectrum (spectral norm well below the Frobenius norm), so any
    other normalisation changes every output singular value."""
    rng = np.random.default_rng(31)
    m, n = shape
    k = min(m, n)
    U, _ = np.linalg.qr(rng.standard_normal((m, k)))
    V, _ = np.linalg.qr(rng.standard_normal((n, k)))
    G = (U * np.geomspace(7.0, 0.05, k)) @ V.T
    O = om.orthogonalise(G, eps=0.0, mode=mode)
    assert O.shape == G.shape
    assert rel(O, normalised_closed_form(G, COEFFS, 5)) < 1e-12


@pytest.mark.parametrize("kind", ["spectral", "eps_in_square", "none", "max_abs"])
def test_planted_normalisation_mistakes_are_caught(kind, monkeypatch):
    slips = {
        "spectral": lambda X, eps: om.as_f64(X) / (np.linalg.norm(om.as_f64(X), 2) + eps),
        "eps_in_square": lambda X, eps: om.as_f64(X) / np.sqrt(np.sum(om.as_f64(X) ** 2) + eps),
        "none": lambda X, eps: om.as_f64(X),
        "max_abs": lambda X, eps: om.as_f64(X) / (np.max(np.abs(om.as_f64(X))) + eps),
    }
    monkeypatch.setattr(om, "frobenius_normalise", slips[kind])
    failures = 0
    checks = [test_frobenius_normalise_rank_two] + [
        (lambda mode=mode: test_orthogonalise_full_rank_closed_form((24, 80), mode)) for mode in ("plain", "gram")]
    for check in checks:
        try:
            check()
        except AssertionError:
            failures += 1
    assert failures > 0, kind
