"""Per-stage parity of the MFMA GEMM kernels (test-only entry point muon_debug_gemm)
against float64 products of the exact operand values the kernel consumed. Every product
is A B^T with both operands K-contiguous.

Tolerances: the output is rounded once to its storage type (fp16: 2^-11, bf16: 2^-8
relative) after fp32 accumulation, so each element is checked against
|ref| * 2 * u_out + K * 2^-22 * max|ref| (fp32 accumulation bound).
"""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from tests.gpu_util import rel  # noqa: E402


@pytest.fixture(scope="module")
def B():
    from matrix_orthogonalising_optimizer_muon_amd import binding
    return binding


@pytest.fixture(scope="module")
def ctx(B):
    c = B.muon_init(0)
    yield c
    B.muon_destroy(c)


def bf16_round(x):
    x32 = np.asarray(x, np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def f16_round(x):
    return np.asarray(x, np.float32).astype(np.float16).astype(np.float64)


def dev(a, dt):
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    return t.to(dt)


def host(t):
    return t.to(torch.float64).cpu().numpy()


def check_elems(got, ref, K, u_out):
    scale = np.max(np.abs(ref))
    bound = np.abs(ref) * 2 * u_out + K * 2.0 ** -22 * scale + 1e-30
    bad = np.abs(got - ref) > bound
    assert not bad.any(), (np.argwhere(bad)[:5], got[bad][:5], ref[bad][:5])


# tile configurations: 0 = 64x64, 1 = 128x128, 2 = 256x128 (apply only), 3 = 256x256;
# 4-7: the same tiles with direct global -> LDS loads; 8: 256x256 with 4 waves; 9, 10:
# 64 and 128 tiles with two k-groups; 11, 12: 256 and 128 (two k-groups) with 64-byte slices;
# 13: 256x192 (apply only); 14: 256x256 with 4 waves and 64-byte slices
SYM_TILES = [0, 1, 3, 4, 5, 7, 8, 9, 10, 11, 12, 14]
ALL_TILES = [0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14]
F32_TILES = [0, 1, 4, 5, 9, 10, 12]


@pytest.mark.parametrize("tile", SYM_TILES)
@pytest.mark.parametrize("M,K", [(64, 64), (192, 320), (256, 1024), (384, 128), (640, 192)])
def test_syrk_bf16(B, ctx, tile, M, K):
    rng = np.random.default_rng(M * 31 + K + tile)
    X = bf16_round(rng.standard_normal((M, K)))
    C = torch.empty((M, M), dtype=torch.float16, device="cuda")
    alpha = 0.25
    assert B.muon_debug_gemm(ctx, 0, "bf16", tile, M, M, K, dev(X, torch.bfloat16), None, None, C, alpha=alpha) == 0
    torch.cuda.synchronize()
    got = host(C)
    ref = alpha * (X @ X.T)
    check_elems(got, ref, K, 2.0 ** -11)
    assert np.array_equal(got, got.T)  # mirrored store: exactly symmetric


@pytest.mark.parametrize("tile", F32_TILES)
@pytest.mark.parametrize("M,K", [(128, 256), (320, 192)])
def test_syrk_f32(B, ctx, tile, M, K):
    rng = np.random.default_rng(M + K + tile)
    X = rng.standard_normal((M, K)).astype(np.float32).astype(np.float64)
    C = torch.empty((M, M), dtype=torch.float32, device="cuda")
    assert B.muon_debug_gemm(ctx, 0, "f32", tile, M, M, K, dev(X, torch.float32), None, None, C) == 0
    torch.cuda.synchronize()
    got = host(C)
    ref = X @ X.T
    check_elems(got, ref, K, 2.0 ** -24)
    assert np.array_equal(got, got.T)


@pytest.mark.parametrize("tile", SYM_TILES)
@pytest.mark.parametrize("ns,dt,u", [("bf16", torch.float16, 2.0 ** -11), ("f32", torch.float32, 2.0 ** -24)])
def test_square_poly(B, ctx, tile, ns, dt, u):
    if ns == "f32" and tile not in F32_TILES:
        pytest.skip("256x256 tiles are not built for fp32")
    M = 576
    rng = np.random.default_rng(tile)
    S = rng.standard_normal((M, M)) / np.sqrt(M)
    S = (S + S.T) / 2
    S = f16_round(S) if ns == "bf16" else S.astype(np.float32).astype(np.float64)
    A = dev(S, dt)
    C = torch.empty((M, M), dtype=dt, device="cuda")
    alpha, beta, gamma = 0.5, -1.25, 3.0
    assert B.muon_debug_gemm(ctx, 1, ns, tile, M, M, M, A, A, A, C, alpha=alpha, beta=beta, gamma=gamma) == 0
    torch.cuda.synchronize()
    got = host(C)
    ref = alpha * (S @ S.T) + beta * S + gamma * np.eye(M)
    check_elems(got, ref, M, u)
    assert np.array_equal(got, got.T)


@pytest.mark.parametrize("tile", SYM_TILES)
@pytest.mark.parametrize("M", [576, 1024])
def test_square_e_is_a_matches_copy(B, ctx, tile, M):
    """kind 1 with E = A itself (the direct-load kernels with 64-wide wave tiles then read
    E from A's slices in LDS during the main loop) and with E a separate copy of A: the
    same values enter the same arithmetic, so the outputs are bitwise equal, and both match
    the float64 reference. M = 576 leaves waves whose columns lie past the edge."""
    rng = np.random.default_rng(M + tile)
    S = rng.standard_normal((M, M)) / np.sqrt(M)
    S = f16_round((S + S.T) / 2)
    A = dev(S, torch.float16)
    A_copy = A.clone()
    C1 = torch.empty((M, M), dtype=torch.float16, device="cuda")
    C2 = torch.empty_like(C1)
    alpha, beta, gamma = -0.75, 2.5, 1.5
    assert B.muon_debug_gemm(ctx, 1, "bf16", tile, M, M, M, A, A, A, C1, alpha=alpha, beta=beta, gamma=gamma) == 0
    assert B.muon_debug_gemm(ctx, 1, "bf16", tile, M, M, M, A, A, A_copy, C2, alpha=alpha, beta=beta,
                             gamma=gamma) == 0
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)
    check_elems(host(C1), alpha * (S @ S.T) + beta * S + gamma * np.eye(M), M, 2.0 ** -11)


@pytest.mark.parametrize("tile", SYM_TILES)
@pytest.mark.parametrize("M,K", [(128, 576), (320, 192)])
def test_sym_long_fp16(B, ctx, tile, M, K):
    """kind 1 with A = B = X (M x K, K != M): the Gram product of the fp16 iterate."""
    rng = np.random.default_rng(M + 7 * K + tile)
    X = f16_round(rng.standard_normal((M, K)) * 4.0)
    Xd = dev(X, torch.float16)
    C = torch.empty((M, M), dtype=torch.float16, device="cuda")
    assert B.muon_debug_gemm(ctx, 1, "bf16", tile, M, M, K, Xd, Xd, None, C, alpha=1.0 / 256) == 0
    torch.cuda.synchronize()
    got = host(C)
    check_elems(got, (X @ X.T) / 256, K, 2.0 ** -11)
    assert np.array_equal(got, got.T)


@pytest.mark.parametrize("tile", ALL_TILES)
@pytest.mark.parametrize("M,N,K", [(128, 320, 192), (256, 1024, 256), (64, 64, 64), (384, 704, 320)])
def test_apply_fp16(B, ctx, tile, M, N, K):
    """kind 2: v = alpha A B^T + beta E^T; C = oscale v and C2 = oscale v^T (fp16)."""
    rng = np.random.default_rng(M + N + K + tile)
    Q = f16_round(rng.standard_normal((M, K)))
    XT = f16_round(rng.standard_normal((N, K)) * 8.0)
    ET = f16_round(rng.standard_normal((N, M)) * 8.0)
    C = torch.empty((M, N), dtype=torch.float16, device="cuda")
    C2 = torch.empty((N, M), dtype=torch.float16, device="cuda")
    alpha, beta, oscale = 1.0 / 64, 0.75 / 64, 64.0
    assert B.muon_debug_gemm(ctx, 2, "bf16", tile, M, N, K, dev(Q, torch.float16), dev(XT, torch.float16),
                             dev(ET, torch.float16), C, C2, alpha=alpha, beta=beta, oscale=oscale) == 0
    torch.cuda.synchronize()
    ref = oscale * (alpha * (Q @ XT.T) + beta * ET.T)
    got, got2 = host(C), host(C2)
    check_elems(got, ref, K, 2.0 ** -11)
    assert np.array_equal(got2, got.T)   # both layouts hold the same rounded values
    assert rel(got, ref) < 1e-3


@pytest.mark.parametrize("tile", F32_TILES)
def test_apply_f32(B, ctx, tile):
    M, N, K = 192, 448, 128
    rng = np.random.default_rng(tile + 5)
    Q = rng.standard_normal((M, K)).astype(np.float32).astype(np.float64)
    XT = rng.standard_normal((N, K)).astype(np.float32).astype(np.float64)
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    C2 = torch.empty((N, M), dtype=torch.float32, device="cuda")
    assert B.muon_debug_gemm(ctx, 2, "f32", tile, M, N, K, dev(Q, torch.float32), dev(XT, torch.float32),
                             None, C, C2, alpha=2.0, oscale=0.5) == 0
    torch.cuda.synchronize()
    got = host(C)
    ref = Q @ XT.T
    check_elems(got, ref, K, 2.0 ** -24)
    assert np.array_equal(host(C2), got.T)


def test_unavailable_tile_config(B, ctx):
    X = torch.zeros((64, 64), dtype=torch.float32, device="cuda")
    assert B.muon_debug_gemm(ctx, 0, "f32", 3, 64, 64, 64, X, None, None, X) == B.MUON_ERR_UNSUPPORTED
    assert B.muon_debug_gemm(ctx, 2, "f32", 2, 64, 64, 64, X, X, None, X) == B.MUON_ERR_UNSUPPORTED
    assert B.muon_debug_gemm(ctx, 0, "bf16", 2, 64, 64, 64, X, None, None, X) == B.MUON_ERR_ARG
    Y = torch.zeros((256, 256), dtype=torch.float32, device="cuda")
    assert B.muon_debug_gemm(ctx, 0, "bf16", 13, 256, 256, 64, Y, None, None, Y) == B.MUON_ERR_ARG
    assert B.muon_debug_gemm(ctx, 2, "f32", 13, 256, 192, 64, Y, Y, None, Y) == B.MUON_ERR_UNSUPPORTED
