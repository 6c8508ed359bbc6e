"""Parity at the full sizes of the two largest workloads, in the launch configuration
bench.py times: the whole matrix list in one muon_step (tiles already measured, so shape
groups run concurrently), checked on sampled matrices the oracle computes one by one.

Inputs are the workloads' device-side draws (workloads.gradient_torch / weight_torch);
the sampled matrices' inputs are copied to the host before the step and read exactly
(bf16 / fp32 values are exact in float64), so the oracle never sees a value the library
computed. Bars as in test_gpu_parity: O by relative Frobenius error <= 2e-2, M' to its
storage rounding. Besides whole layers, a seeded 10% sample of the other matrices is
checked; MUON_FULL_PARITY=1 checks every matrix (slow: tens of minutes of fp64 work on
the host).
"""

import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from matrix_orthogonalising_optimizer_muon_amd import workloads as wl  # noqa: E402
from oracle import flop_model  # noqa: E402
from oracle import muon as om  # noqa: E402
from tests.gpu_util import rel, to_np  # noqa: E402


@pytest.fixture(scope="module")
def B():
    from matrix_orthogonalising_optimizer_muon_amd import binding
    return binding


def mode_of(spec):
    g = flop_model.dense_flops(spec.rows, spec.cols, "gram")
    p = flop_model.dense_flops(spec.rows, spec.cols, "plain")
    return "gram" if g < p else "plain"


class FullRun:
    """The workload's whole list on the device, one context, bench.py's hyper-parameters."""

    def __init__(self, B, w):
        self.B, self.w = B, w
        self.ctx = B.muon_init(0)
        self.hp = B.make_hparams(lr=w.lr, momentum=w.mu, weight_decay=w.wd, mode="auto",
                                 w_dtype=w.w_dtype, g_dtype=w.g_dtype, m_dtype=w.m_dtype,
                                 ns_dtype=w.ns_dtype)
        self.reset()
        self.G = [wl.gradient_torch(w, 0, i) for i in range(len(w.matrices))]
        mats = list(zip(self.W, self.G, self.M))
        self.arr = B.matrix_list(mats, self.hp, 0)
        self.nbytes = B.muon_workspace_size(self.ctx, mats, self.hp)
        self.ws = torch.empty(self.nbytes, dtype=torch.uint8, device="cuda")
        self.step()            # measures every stage's tiles (as bench.py's warm-up does)
        self.reset()

    def reset(self):
        tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
        if not hasattr(self, "W"):
            self.W = [wl.weight_torch(self.w, i) for i in range(len(self.w.matrices))]
            self.M = [torch.zeros(s.rows, s.cols, dtype=tdt[self.w.m_dtype], device="cuda")
                      for s in self.w.matrices]
        else:
            for i in range(len(self.W)):
                self.W[i].copy_(wl.weight_torch(self.w, i))
                self.M[i].zero_()
        torch.cuda.synchronize()

    def load_gradients(self, step):
        for i in range(len(self.G)):
            self.G[i].copy_(wl.gradient_torch(self.w, step, i))
        torch.cuda.synchronize()

    def step(self):
        B = self.B
        B.check(B.muon_step(self.ctx, self.arr, self.hp, self.ws.data_ptr(), self.nbytes,
                            torch.cuda.current_stream().cuda_stream, count=len(self.W)), "muon_step")
        torch.cuda.synchronize()

    def close(self):
        self.B.muon_destroy(self.ctx)


def sample(w, layers, per_layer, checked_layers, extra=False):
    """Every matrix of `layers`, plus (extra=True) a seeded 10% sample of the matrices
    outside `checked_layers` (all the layers the workload's tests check in full), so the
    layer tests and the sample together cover distinct matrices. MUON_FULL_PARITY=1 checks
    every matrix instead."""
    if os.environ.get("MUON_FULL_PARITY") == "1":
        return list(range(len(w.matrices))) if extra else []
    idx = [l * per_layer + j for l in layers for j in range(per_layer)]
    if extra:
        done = {l * per_layer + j for l in checked_layers for j in range(per_layer)}
        rest = [i for i in range(len(w.matrices)) if i not in done]
        rng = np.random.default_rng(w.wid)
        idx += sorted(rng.choice(rest, size=(len(w.matrices) + 9) // 10, replace=False).tolist())
    return idx


def run_and_check(run, idx, steps):
    w = run.w
    W_o = {i: to_np(run.W[i]) for i in idx}
    M_o = {i: np.zeros_like(W_o[i]) for i in idx}
    worst = 0.0
    for s in range(steps):
        if s > 0:
            run.load_gradients(s)
        G_h = {i: to_np(run.G[i]) for i in idx}
        W_prev = {i: to_np(run.W[i]) for i in idx}
        run.step()
        for i in idx:
            spec = w.matrices[i]
            W_new, M_new, O_ref = om.muon_step(W_o[i], G_h[i], M_o[i], lr=w.lr, mu=w.mu, wd=w.wd,
                                               nesterov=True, eps=1e-7, mode=mode_of(spec))
            W_gpu, M_gpu = to_np(run.W[i]), to_np(run.M[i])
            e = rel((W_prev[i] - W_gpu) / w.lr, O_ref)
            worst = max(worst, e)
            assert e <= 2e-2, (w.name, spec.name, s, e)
            if s == 0:
                assert np.array_equal(M_gpu, M_new), (w.name, spec.name)
            else:
                assert rel(M_gpu, M_new) <= (s + 1) * 2.0 ** -8, (w.name, spec.name, s)
            W_o[i], M_o[i] = W_new, M_new
            if len(idx) > 16:  # the long seeded-sample runs report each matrix as it is checked
                print(f"[fullsize] {w.name} step {s}: {spec.name} O error {e:.3e}", flush=True)
        print(f"[fullsize] {w.name} step {s}: {len(idx)} matrices checked, worst O error {worst:.3e}",
              flush=True)
    return worst


@pytest.fixture(scope="module")
def decoder(B):
    run = FullRun(B, wl.WORKLOADS["decoder_d2048_24layers"])
    yield run
    run.close()


@pytest.fixture(scope="module")
def dense7b(B):
    run = FullRun(B, wl.WORKLOADS["dense_7b_28layers"])
    yield run
    run.close()


def test_decoder_24_layers_three_steps(decoder):
    """168 matrices (2048^2 plain, 8192x2048 / 2048x8192 Gram), 3 steps with momentum
    carried; layers 0 and 23 and a seeded 10% of the rest checked after every step."""
    run_and_check(decoder, sample(decoder.w, [0, 23], 7, [0, 23], extra=True), steps=3)


@pytest.mark.parametrize("layer", [0, 27])
def test_dense_7b_one_step(dense7b, layer):
    """196 matrices (3584^2 plain; 512x3584 and 3584x18944 / 18944x3584 Gram); every matrix
    of one layer checked; the layer-0 run also checks a seeded 10% of the other layers'
    matrices (20 of them: 34 distinct matrices over the two runs)."""
    dense7b.reset()
    run_and_check(dense7b, sample(dense7b.w, [layer], 7, [0, 27], extra=layer == 0), steps=1)
