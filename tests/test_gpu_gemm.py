"""Per-stage parity of the MFMA GEMM kernels (test-only entry point muon_debug_gemm)
against float64 products of the exact operand values the kernel consumed.

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


# tile configurations: 0 = 64x64, 1 = 128x128, 2 = 256x128 (apply only), 3 = 256x256
@pytest.mark.parametrize("tile", [0, 1, 3])
@pytest.mark.parametrize("M,K", [(64, 64), (192, 320), (256, 1024), (384, 128), (640, 192)])
def test_syrk_bf16(B, ctx, tile, M, K):
    rng = np.random.default_rng(M * 31 + K + tile)
    X = bf16_round(rng.standard_normal((M, K)))
    C = torch.empty((M, M), dtype=torch.float16, device="cuda")
    alpha = 0.25
    assert B.muon_debug_gemm(ctx, 0, "bf16", tile, M, M, K, dev(X, torch.bfloat16), None, None, C, alpha) == 0
    torch.cuda.synchronize()
    got = host(C)
    ref = alpha * (X @ X.T)
    check_elems(got, ref, K, 2.0 ** -11)
    assert np.array_equal(got, got.T)  # mirrored store: exactly symmetric


@pytest.mark.parametrize("tile", [0, 1])
@pytest.mark.parametrize("M,K", [(128, 256), (320, 192)])
def test_syrk_f32(B, ctx, tile, M, K):
    rng = np.random.default_rng(M + K + tile)
    X = rng.standard_normal((M, K)).astype(np.float32).astype(np.float64)
    C = torch.empty((M, M), dtype=torch.float32, device="cuda")
    assert B.muon_debug_gemm(ctx, 0, "f32", tile, M, M, K, dev(X, torch.float32), None, None, C, 1.0) == 0
    torch.cuda.synchronize()
    got = host(C)
    ref = X @ X.T
    check_elems(got, ref, K, 2.0 ** -24)
    assert np.array_equal(got, got.T)


@pytest.mark.parametrize("tile", [0, 1, 3])
@pytest.mark.parametrize("ns,dt,u", [("bf16", torch.float16, 2.0 ** -11), ("f32", torch.float32, 2.0 ** -24)])
def test_square_poly(B, ctx, tile, ns, dt, u):
    if ns == "f32" and tile == 3:
        pytest.skip("256x256 tiles are not built for fp32")
    M = 576
    rng = np.random.default_rng(tile)
    S = rng.standard_normal((M, M)) / np.sqrt(M)
    S = (S + S.T) / 2
    S = f16_round(S) if ns == "bf16" else S.astype(np.float32).astype(np.float64)
    A = dev(S, dt)
    C = torch.empty((M, M), dtype=dt, device="cuda")
    alpha, beta, gamma = 0.5, -1.25, 3.0
    assert B.muon_debug_gemm(ctx, 1, ns, tile, M, M, M, A, A, A, C, alpha, beta, gamma) == 0
    torch.cuda.synchronize()
    got = host(C)
    ref = alpha * (S @ S.T) + beta * S + gamma * np.eye(M)
    check_elems(got, ref, M, u)
    assert np.array_equal(got, got.T)


@pytest.mark.parametrize("tile", [0, 1, 2, 3])
@pytest.mark.parametrize("M,N,K", [(128, 320, 192), (256, 1024, 256), (64, 64, 64), (384, 704, 320)])
def test_apply_bf16(B, ctx, tile, M, N, K):
    rng = np.random.default_rng(M + N + K + tile)
    Q = f16_round(rng.standard_normal((M, K)))
    X = bf16_round(rng.standard_normal((K, N)) * 0.01)
    E = bf16_round(rng.standard_normal((M, N)) * 0.01)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    alpha, beta, bscale = 1.0 / 64, 0.75, 64.0
    assert B.muon_debug_gemm(ctx, 2, "bf16", tile, M, N, K, dev(Q, torch.float16), dev(X, torch.bfloat16),
                             dev(E, torch.bfloat16), C, alpha, beta, 0.0, bscale) == 0
    torch.cuda.synchronize()
    got = host(C)
    Xh = f16_round(X * bscale)  # the fp16 operand the kernel builds from bf16 X
    ref = alpha * (Q @ Xh) + beta * E
    check_elems(got, ref, K, 2.0 ** -8)
    assert rel(got, ref) < 4e-3


@pytest.mark.parametrize("tile", [0, 1])
def test_apply_f32(B, ctx, tile):
    M, N, K = 192, 448, 128
    rng = np.random.default_rng(tile + 5)
    Q = rng.standard_normal((M, K)).astype(np.float32).astype(np.float64)
    X = rng.standard_normal((K, N)).astype(np.float32).astype(np.float64)
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    assert B.muon_debug_gemm(ctx, 2, "f32", tile, M, N, K, dev(Q, torch.float32), dev(X, torch.float32),
                             None, C, 2.0, 0.0, 0.0, 0.5) == 0
    torch.cuda.synchronize()
    got = host(C)
    ref = 2.0 * (Q @ (X * 0.5))
    check_elems(got, ref, K, 2.0 ** -24)


def test_unavailable_tile_config(B, ctx):
    X = torch.zeros((64, 64), dtype=torch.float32, device="cuda")
    assert B.muon_debug_gemm(ctx, 0, "f32", 3, 64, 64, 64, X, None, None, X) == B.MUON_ERR_UNSUPPORTED
    assert B.muon_debug_gemm(ctx, 0, "bf16", 2, 64, 64, 64, X, None, None, X) == B.MUON_ERR_ARG
