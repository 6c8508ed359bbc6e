"""muon_step_static (the entry point over the library's static scratch, for callers that
cannot allocate) against muon_step on the same inputs, through the C ABI: two calls in a
row, the second with a smaller list, each bitwise equal to muon_step with the same tile
choices and within the bf16 bar of the fp64 oracle."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from matrix_orthogonalising_optimizer_muon_amd import workloads as wl  # noqa: E402
from oracle import muon as om  # noqa: E402
from tests.gpu_util import GpuState, rel, to_np  # noqa: E402


@pytest.fixture(scope="module")
def B():
    from matrix_orthogonalising_optimizer_muon_amd import binding
    return binding


def _run(B, ctx, w, hp, static):
    st = GpuState(w)
    st.load_gradients(0)
    mats = st.triples()
    if static:
        rc = B.muon_step_static(ctx, mats, hp)
    else:
        nbytes = B.muon_workspace_size(ctx, mats, hp)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
        rc = B.muon_step(ctx, mats, hp, ws.data_ptr(), nbytes)
    torch.cuda.synchronize()
    B.check(rc, "static" if static else "workspace")
    return st


def test_static_scratch_matches_workspace_entry(B):
    ctx = B.muon_init(0)
    try:
        hp = B.make_hparams(mode="gram")
        big = wl.custom("noalloc_big", [(512, 2048), (2048, 384), (300, 1000), (96, 320)],
                        structure="lowrank", rank=16, wid=301)
        small = wl.custom("noalloc_small", [(128, 640), (200, 72)], structure="lowrank", rank=8, wid=302)
        for w in (big, small):  # second call: a smaller list over the same scratch
            assert B.muon_workspace_size(ctx, [(0, 0, 0, s.rows, s.cols) for s in w.matrices], hp) \
                <= B.MUON_STATIC_SCRATCH_BYTES
            ref = _run(B, ctx, w, hp, static=False)   # measures the tiles the static call reuses
            got = _run(B, ctx, w, hp, static=True)
            for k, i in enumerate(got.indices):
                assert torch.equal(got.W[k], ref.W[k]), (w.name, i)
                assert torch.equal(got.M[k], ref.M[k]), (w.name, i)
                W0 = wl.weight_np(w, i).astype(np.float64)
                G = wl.gradient_np(w, 0, i).astype(np.float64)
                _, M_ref, O_ref = om.muon_step(W0, G, np.zeros_like(W0), mode="gram")
                O_gpu = (W0 - to_np(got.W[k])) / w.lr
                assert rel(O_gpu, O_ref) <= 2e-2, (w.name, i)
                assert np.array_equal(to_np(got.M[k]), M_ref)
    finally:
        B.muon_destroy(ctx)


def test_static_scratch_rejects_oversized_list(B):
    ctx = B.muon_init(0)
    try:
        hp = B.make_hparams()
        raw = [(0, 0, 0, 4096, 16384)] * 2     # about 0.8 GiB of workspace
        assert B.muon_workspace_size(ctx, raw, hp) > B.MUON_STATIC_SCRATCH_BYTES
        # real buffers of that size, so that nothing could be out of bounds even if launched
        mats = [(torch.zeros(4096, 16384, device="cuda"),
                 torch.zeros(4096, 16384, dtype=torch.bfloat16, device="cuda"),
                 torch.zeros(4096, 16384, dtype=torch.bfloat16, device="cuda")) for _ in range(2)]
        for W, _, _ in mats:
            W.fill_(0.25)
        torch.cuda.synchronize()
        assert B.muon_step_static(ctx, mats, hp) == B.MUON_ERR_WORKSPACE
        torch.cuda.synchronize()
        for W, _, M in mats:
            assert bool((W == 0.25).all()) and bool((M == 0).all())
    finally:
        B.muon_destroy(ctx)
