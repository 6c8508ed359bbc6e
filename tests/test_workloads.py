"""Host-side checks of the seeded input generators (no GPU)."""

import numpy as np

from matrix_orthogonalising_optimizer_muon_amd import workloads as wl


def test_shapes_and_counts():
    assert wl.WORKLOADS["single_bf16_2560x9728"].elements == 2560 * 9728
    d = wl.WORKLOADS["decoder_d2048_24layers"]
    assert len(d.matrices) == 168 and d.steps == 3
    s = wl.WORKLOADS["small_batch_832"]
    assert len(s.matrices) == 832
    assert s.elements == 512 * 64 * 256 + 256 * 128 * 512 + 64 * 256 * 1024
    b = wl.WORKLOADS["dense_7b_28layers"]
    assert len(b.matrices) == 196
    assert b.elements == 28 * (2 * 3584 * 3584 + 2 * 512 * 3584 + 3 * 18944 * 3584)


def test_bf16_rounding_is_rne_and_exact():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1e-30, 3.0e38], dtype=np.float64)
    r = wl.round_to(x, "bf16")
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: RNE keeps the even mantissa (1.0)
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == 1.0 + 2 ** -6 and r[3] == -2.5
    bits = r.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)


def test_seeded_and_structured():
    w = wl.custom("t", [(40, 96)], structure="lowrank", rank=4)
    g1 = wl.gradient_np(w, 0, 0)
    g2 = wl.gradient_np(w, 0, 0)
    assert np.array_equal(g1, g2)
    assert not np.array_equal(g1, wl.gradient_np(w, 1, 0))
    s = np.linalg.svd(g1.astype(np.float64), compute_uv=False)
    # 4 strong directions (10, 5, 3.3, 2.5) above a noise floor near 0.01*(sqrt(96)+sqrt(40))
    assert s[3] > 2.0 and s[4] < 0.2
    b = wl.haar_basis(np.random.default_rng(0), 50, 6)
    assert np.allclose(b.T @ b, np.eye(6), atol=1e-12)
