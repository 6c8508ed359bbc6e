"""muon_step captured into a HIP graph (torch.cuda.CUDAGraph) and replayed: every replay
must give the same W and M, bit for bit, as the same step run eagerly, also with other
eager work and synchronisations between replays. The step launches no memset; the tile
measurements happen on a warm-up of the same shapes before the capture."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from matrix_orthogonalising_optimizer_muon_amd import workloads as wl  # noqa: E402
from tests.gpu_util import GpuState, to_dev  # noqa: E402


@pytest.fixture(scope="module")
def B():
    from matrix_orthogonalising_optimizer_muon_amd import binding
    return binding


@pytest.mark.parametrize("shapes,mode", [
    ([(256, 1024), (128, 512), (512, 128), (64, 256), (192, 192)], "auto"),   # staged, 4 streams
    ([(64, 256), (100, 300), (128, 512)], "auto"),                             # single-workgroup
    ([(640, 2048)], "auto_schedule"),
])
def test_graph_replay_matches_eager(B, shapes, mode):
    w = wl.custom("graph", shapes, structure="lowrank", rank=8, wid=220, steps=3)
    ctx = B.muon_init(0)
    try:
        hp = B.make_hparams(mode=mode)
        eager, graphed = GpuState(w), GpuState(w)
        eager.load_gradients(0)
        nbytes = B.muon_workspace_size(ctx, eager.triples(), hp)
        ws_e = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        ws_g = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        # warm-up on separate buffers of the same shapes: tile measurements and streams
        warm = GpuState(w)
        warm.load_gradients(0)
        B.check(B.muon_step(ctx, warm.triples(), hp, ws_e.data_ptr(), nbytes), "warm-up")
        torch.cuda.synchronize()
        # capture one step on the graphed buffers (nothing executes during capture)
        graphed.load_gradients(0)
        arr = B.matrix_list(graphed.triples())
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                rc = B.muon_step(ctx, arr, hp, ws_g.data_ptr(), nbytes, torch.cuda.current_stream().cuda_stream,
                                 count=len(shapes))
        assert rc == 0
        torch.cuda.synchronize()
        noise = torch.randn(1 << 20, device="cuda")
        for s in range(3):
            eager.load_gradients(s)
            for k in range(len(shapes)):       # fresh gradients into the captured buffers
                graphed.G[k].copy_(to_dev(wl.gradient_np(w, s, k), w.g_dtype))
            B.check(B.muon_step(ctx, eager.triples(), hp, ws_e.data_ptr(), nbytes), "eager")
            g.replay()
            noise.mul_(1.0001).add_(0.5)        # unrelated eager work between replays
            torch.cuda.synchronize()
            for k in range(len(shapes)):
                assert torch.equal(eager.W[k], graphed.W[k]), (s, k)
                assert torch.equal(eager.M[k], graphed.M[k]), (s, k)
        del g
    finally:
        B.muon_destroy(ctx)
