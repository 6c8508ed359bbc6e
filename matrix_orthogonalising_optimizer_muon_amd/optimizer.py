"""Drop-in style wrapper: a context, the hyper-parameters, the matrix list and a
workspace tensor, so one Muon update of every registered 2-D weight is one call.

The DMuon announcement (agentren.cn, "three lines of code") and the MuonX article
(section 3.3) describe integration as: name the participating matrices, replace the
optimizer. Here: build ``MuonUpdate([(W, G, M), ...])`` once, call ``step()`` after
each backward. Only 2-D hidden weights belong here (MuonX section 2: embeddings and
biases stay on AdamW).
"""

from __future__ import annotations

import torch

from . import binding as B


class MuonUpdate:
    def __init__(self, mats, device: int | None = None, **hparams):
        self.device = torch.cuda.current_device() if device is None else int(device)
        self.ctx = B.muon_init(self.device)
        self.hp = B.make_hparams(**hparams)
        self.tensors = list(mats)
        self.count = len(self.tensors)
        self.arr = B.matrix_list(self.tensors)
        nbytes = B.muon_workspace_size(self.ctx, self.tensors, self.hp)
        self.workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8,
                                     device=f"cuda:{self.device}")
        self.workspace_bytes = nbytes

    def step(self, stream: torch.cuda.Stream | None = None) -> None:
        st = (stream or torch.cuda.current_stream(self.device)).cuda_stream
        B.check(B.muon_step(self.ctx, self.arr, self.hp, self.workspace.data_ptr(),
                            self.workspace_bytes, st, count=self.count), "muon_step")

    def plan(self, index: int) -> B.muon_plan_entry:
        return B.muon_plan_info(self.ctx, self.tensors, self.hp, index)

    def close(self) -> None:
        if self.ctx is not None:
            B.muon_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
