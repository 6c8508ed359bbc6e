"""Stage-level parity through the test-only C entry point muon_debug_stage: the norm pass,
the momentum + normalised-iterate pass (both layouts, zero padding) and the fused W update,
each against float64 on the same stored inputs, element by element.

MuonX article, section 2: momentum, then orthogonalisation; the normalisation and the
update are the readings the oracle takes (X0 = U / (||U||_F + eps); W' = W (1 - lr wd) -
lr O). The oracle's own functions compute the references where it has them.
"""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from matrix_orthogonalising_optimizer_muon_amd import workloads as wl  # noqa: E402
from oracle import muon as om  # noqa: E402
from tests.gpu_util import to_dev, to_np  # noqa: E402

SHAPES = [(100, 300), (300, 100), (130, 130), (1, 17), (200, 1000), (1000, 200), (64, 64)]


@pytest.fixture(scope="module")
def B():
    from matrix_orthogonalising_optimizer_muon_amd import binding
    return binding


@pytest.fixture(scope="module")
def ctx(B):
    c = B.muon_init(0)
    yield c
    B.muon_destroy(c)


def up64(x):
    return (x + 63) // 64 * 64


def inputs(rows, cols, dtype, seed):
    rng = np.random.default_rng(seed)
    G = wl.round_to(rng.standard_normal((rows, cols)), dtype)
    M = wl.round_to(0.3 * rng.standard_normal((rows, cols)), dtype)
    W = wl.round_to(0.02 * rng.standard_normal((rows, cols)), "f32")
    return G, M, W


def workspace(rows, cols):
    return torch.empty(512 + ((rows * cols + 4095) // 4096 * 4 + 255) // 256 * 256, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("nesterov", [True, False])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES)
def test_norm_and_iterate(B, ctx, shape, dtype, nesterov):
    check_norm_and_iterate(B, ctx, shape, dtype, nesterov)


@pytest.mark.parametrize("shape", [(9000, 4001), (4001, 9000)])
def test_norm_and_iterate_large(B, ctx, shape):
    """G and M over 128 MB (36,009,000 bf16 elements each): the forms muon_step runs for
    large groups, four groups of 8 per thread in the norm pass (a partial last block:
    36,009,000 is not a multiple of 16384) and two 64 x 64 tiles per workgroup in the
    iterate pass (63 x 141 tiles, an odd count)."""
    check_norm_and_iterate(B, ctx, shape, "bf16", True)


def check_norm_and_iterate(B, ctx, shape, dtype, nesterov):
    rows, cols = shape
    G, M, _ = inputs(rows, cols, dtype, seed=rows * 7 + cols)
    hp = B.make_hparams(g_dtype=dtype, m_dtype=dtype, ns_dtype=dtype, nesterov=nesterov, momentum=0.9, eps=1e-7)
    Gd, Md = to_dev(G, dtype), to_dev(M, dtype)
    # the hyper-parameters as the library receives them (fp32)
    mu, eps = float(np.float32(0.9)), float(np.float32(1e-7))
    M_new_ref, U = om.momentum(G, M, mu, nesterov)
    X, transposed = om.orient(U)
    X0 = om.frobenius_normalise(X, eps)
    m, n = X.shape
    ws = workspace(rows, cols)
    # norm only: G and M are read, not written
    s = torch.zeros(1, device="cuda")
    rc, _ = B.muon_debug_stage(ctx, B.MUON_STAGE_NORM, (None, Gd, Md, rows, cols), hp, None, s, None, ws)
    torch.cuda.synchronize()
    assert rc == B.MUON_OK
    assert torch.equal(Md, to_dev(M, dtype))
    s_ref = 1.0 / (np.linalg.norm(U) + eps)
    assert abs(float(s.item()) - s_ref) <= 1e-5 * s_ref
    # momentum + iterate in both layouts
    xdt = torch.float16 if dtype == "bf16" else torch.float32
    Mp, Np = up64(m), up64(n)
    out = torch.full((Mp, Np), 7.0, dtype=xdt, device="cuda")     # padding must be overwritten with 0
    out2 = torch.full((Np, Mp), 7.0, dtype=xdt, device="cuda")
    rc, scale = B.muon_debug_stage(ctx, B.MUON_STAGE_ITERATE, (None, Gd, Md, rows, cols), hp, None, out, out2, ws)
    torch.cuda.synchronize()
    assert rc == B.MUON_OK
    Mg = to_np(Md)
    if dtype == "f32":
        assert np.all(np.abs(Mg - M_new_ref) <= 2.0 ** -23 * np.abs(M_new_ref))
    else:   # fp32 arithmetic, then one bf16 rounding: within one bf16 ulp of the exact value
        assert np.all(np.abs(Mg - M_new_ref) <= 2.0 ** -7 * np.abs(M_new_ref))
        assert np.mean(np.abs(Mg - wl.round_to(M_new_ref, "bf16")) > 0) < 1e-3
    if dtype == "f32":
        assert scale == 1.0
    assert scale >= 1.0 and scale == 2.0 ** round(np.log2(scale))
    Xg, XTg = to_np(out), to_np(out2)
    assert np.array_equal(XTg, Xg.T)
    assert np.all(Xg[m:, :] == 0) and np.all(Xg[:, n:] == 0)
    ref = scale * X0
    got = Xg[:m, :n]
    # U is formed in fp32 (an absolute error of a few fp32 ulps of |G| + |M| where terms
    # cancel), then scaled; the fp16 iterate adds one rounding (half an ulp, 2^-11)
    floor = 2.0 ** -21 * np.abs(ref).max()
    if dtype == "f32":
        assert np.all(np.abs(got - ref) <= 1e-6 * np.abs(ref) + floor)
    else:
        assert np.all(np.abs(got - ref) <= 2.0 ** -10 * np.abs(ref) + floor + 2.0 ** -24)


@pytest.mark.parametrize("wd", [0.0, 0.1])
@pytest.mark.parametrize("w_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ns", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES)
def test_weight_update(B, ctx, shape, ns, w_dtype, wd):
    rows, cols = shape
    rng = np.random.default_rng(rows * 13 + cols)
    m, n = min(rows, cols), max(rows, cols)
    Mp, Np = up64(m), up64(n)
    xdt = torch.float16 if ns == "bf16" else torch.float32
    cast = (lambda a: a.astype(np.float16).astype(np.float64)) if ns == "bf16" else (
        lambda a: a.astype(np.float32).astype(np.float64))
    Q = np.zeros((Mp, Mp))
    Q[:m, :m] = cast(rng.standard_normal((m, m)) / np.sqrt(m))
    # the iterate's scale: from the iterate stage on the same shape
    _, scale = B.muon_debug_stage(ctx, B.MUON_STAGE_ITERATE,
                                  (None, to_dev(np.zeros((rows, cols), np.float32), ns),
                                   to_dev(np.zeros((rows, cols), np.float32), ns), rows, cols),
                                  B.make_hparams(ns_dtype=ns, g_dtype=ns, m_dtype=ns), None,
                                  torch.zeros((Mp, Np), dtype=xdt, device="cuda"),
                                  torch.zeros((Np, Mp), dtype=xdt, device="cuda"), workspace(rows, cols))
    torch.cuda.synchronize()
    XT = np.zeros((Np, Mp))
    XT[:n, :m] = cast(scale * rng.standard_normal((n, m)) / np.sqrt(m * n))
    W = wl.round_to(0.02 * rng.standard_normal((rows, cols)), w_dtype)
    Wd = to_dev(W, w_dtype)
    hp = B.make_hparams(ns_dtype=ns, w_dtype=w_dtype, lr=0.02, weight_decay=wd)
    Qd = torch.from_numpy(Q).to("cuda").to(xdt)
    XTd = torch.from_numpy(XT).to("cuda").to(xdt)
    dummy = torch.empty(1, device="cuda")
    rc, _ = B.muon_debug_stage(ctx, B.MUON_STAGE_UPDATE, (Wd, None, None, rows, cols), hp, Qd, dummy, XTd,
                               workspace(rows, cols))
    torch.cuda.synchronize()
    assert rc == B.MUON_OK
    O = (Q[:m, :m] @ XT[:n, :m].T) / scale          # canonical m' x n'
    O_st = O.T if rows > cols else O
    ref = om.weight_update(W, O_st, 0.02, wd)
    got = to_np(Wd)
    step = 0.02 * np.abs(O_st).max()
    if w_dtype == "f32":
        assert np.all(np.abs(got - ref) <= 2.0 ** -23 * np.abs(ref) + 1e-4 * step)
    else:   # one bf16 rounding of W'
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-4 * step)


def test_stage_validation(B, ctx):
    hp = B.make_hparams()
    ws = workspace(64, 64)
    x = torch.zeros(64, 64, dtype=torch.bfloat16, device="cuda")
    out = torch.zeros(1, device="cuda")
    assert B.muon_debug_stage(ctx, 3, (None, x, x, 64, 64), hp, None, out, None, ws)[0] == B.MUON_ERR_ARG
    assert B.muon_debug_stage(ctx, B.MUON_STAGE_NORM, (None, None, x, 64, 64), hp, None, out, None, ws)[0] \
        == B.MUON_ERR_ARG
    assert B.muon_debug_stage(ctx, B.MUON_STAGE_UPDATE, (None, None, None, 64, 64), hp, x, out, x, ws)[0] \
        == B.MUON_ERR_ARG
    small = torch.empty(256, dtype=torch.uint8, device="cuda")
    assert B.muon_debug_stage(ctx, B.MUON_STAGE_NORM, (None, x, x, 64, 64), hp, None, out, None, small)[0] \
        == B.MUON_ERR_WORKSPACE
