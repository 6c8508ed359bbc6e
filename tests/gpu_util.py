"""Shared helpers of the GPU tests: upload seeded inputs, run the library, read back."""

from __future__ import annotations

import numpy as np
import torch

from matrix_orthogonalising_optimizer_muon_amd import binding as B
from matrix_orthogonalising_optimizer_muon_amd import workloads as wl

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 array holding values exact in `dtype` -> device tensor (exact conversion)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(TORCH_DT[dtype])


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def rel(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


class GpuState:
    """Device W, G, M for a workload (or a subset of its matrices)."""

    def __init__(self, w: wl.Workload, indices=None):
        self.w = w
        self.indices = list(range(len(w.matrices))) if indices is None else list(indices)
        self.W = [to_dev(wl.weight_np(w, i), w.w_dtype) for i in self.indices]
        self.M = [to_dev(wl.momentum0_np(w, i), w.m_dtype) for i in self.indices]
        self.G = [None] * len(self.indices)

    def load_gradients(self, step: int):
        for k, i in enumerate(self.indices):
            self.G[k] = to_dev(wl.gradient_np(self.w, step, i), self.w.g_dtype)

    def triples(self):
        return list(zip(self.W, self.G, self.M))


def run_step(ctx, state: GpuState, hp, check=True) -> int:
    mats = state.triples()
    nbytes = B.muon_workspace_size(ctx, mats, hp)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    rc = B.muon_step(ctx, mats, hp, ws.data_ptr(), nbytes)
    torch.cuda.synchronize()
    if check:
        B.check(rc, "muon_step")
    return rc
