"""Drop-in style wrapper: a context, the hyper-parameters, the matrix list and a
workspace tensor, so one Muon update of every registered 2-D weight is one call.

The DMuon announcement (agentren.cn, "three lines of code") and the MuonX article
(section 3.3) describe integration as: name the participating matrices, replace the
optimizer. Here: build ``MuonUpdate([(W, G, M), ...])`` once, call ``step()`` after
each backward. The library keeps the tensors' addresses from construction on, so W, G
and M must stay the same tensors (G a persistent gradient buffer that each backward
fills, not a new ``.grad`` per step); ``MuonWithAdamW`` below takes the current ``.grad``
at every step instead. Only 2-D hidden weights belong here (MuonX section 2: embeddings
and biases stay on AdamW).
"""

from __future__ import annotations

import torch

from . import binding as B


class MuonUpdate:
    def __init__(self, mats, device: int | None = None, **hparams):
        self.tensors = list(mats)
        if device is None:
            device = self.tensors[0][0].device.index if self.tensors else torch.cuda.current_device()
        self.device = int(device)
        # Storage dtypes come from the tensors (every W alike, every G alike, every M alike);
        # a dtype also given by keyword must agree with them.
        for role, k in (("w_dtype", 0), ("g_dtype", 1), ("m_dtype", 2)):
            names = {_dtype_name(t[k].dtype) for t in self.tensors}
            if len(names) > 1:
                raise TypeError(f"mixed {role[0].upper()} dtypes {sorted(names)}: use one MuonUpdate per dtype")
            if names:
                got = names.pop()
                if hparams.get(role) not in (None, got):
                    raise TypeError(f"{role}={hparams[role]!r} but the tensors are {got}")
                hparams[role] = got
        self.hp = B.make_hparams(**hparams)
        self.count = len(self.tensors)
        # validates device, contiguity, shapes and dtypes before the context is created
        self.arr = B.matrix_list(self.tensors, self.hp, self.device)
        self.ctx = B.muon_init(self.device)
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
        if getattr(self, "ctx", None) is not None:
            B.muon_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _dtype_name(dt: torch.dtype) -> str:
    if dt == torch.float32:
        return "f32"
    if dt == torch.bfloat16:
        return "bf16"
    raise TypeError(f"parameters must be float32 or bfloat16, got {dt}")


class MuonWithAdamW(torch.optim.Optimizer):
    """torch.optim-style optimizer over a model's parameters: 2-D hidden weights go to the
    Muon update (``muon_step``), everything else -- embeddings, output heads, biases, norm
    weights -- to AdamW (``muon_adamw_step``), as the MuonX article (section 2) describes
    practice; integration is the announcement's "replace the optimizer".

    ``params``: an iterable of parameters or of ``(name, parameter)`` pairs. A 2-D parameter
    goes to AdamW when its name contains one of ``adamw_names``. All parameters must be on
    one GPU. All state (Muon momentum, AdamW moments and step counts, the Muon workspace)
    lives on that device; ``step()`` launches one ``muon_step`` per (weight dtype, gradient
    dtype) group and one ``muon_adamw_step`` per (weight dtype, gradient dtype, step count)
    on the current stream, with no host synchronisation. Parameters without a gradient are
    skipped for that step (an AdamW parameter's step count then does not advance, so its
    bias correction follows the steps it took part in).

    The two parameter groups carry their own ``"lr"`` (``lr`` for Muon, ``adamw_lr`` for
    AdamW), which ``step()`` reads every time, so ``torch.optim.lr_scheduler`` schedules
    both.
    """

    def __init__(self, params, *, lr: float = 0.02, momentum: float = 0.95, weight_decay: float = 0.0,
                 nesterov: bool = True, segments=(2, 2, 1), mode: str = "auto", ns_dtype: str = "bf16",
                 momentum_dtype: str = "bf16", adamw_lr: float = 3e-4, adamw_betas=(0.9, 0.95),
                 adamw_eps: float = 1e-8, adamw_weight_decay: float = 0.0,
                 adamw_names=("embed", "lm_head", "wte", "wpe", "head")):
        named = []
        for i, p in enumerate(params):
            named.append(p if isinstance(p, tuple) else (f"param{i}", p))
        muon, adamw = [], []
        for name, p in named:
            if not p.requires_grad:
                continue
            if p.ndim == 2 and not any(k in name for k in adamw_names):
                muon.append(p)
            else:
                adamw.append(p)
        defaults = dict(lr=lr)
        super().__init__([{"params": muon, "kind": "muon", "lr": lr},
                          {"params": adamw, "kind": "adamw", "lr": adamw_lr}], defaults)
        devices = {p.device for p in muon + adamw}
        if len(devices) > 1:
            raise ValueError(f"all parameters must be on one device, got {sorted(map(str, devices))}")
        self._muon_hp = dict(lr=lr, momentum=momentum, weight_decay=weight_decay, nesterov=nesterov,
                             segments=segments, mode=mode, ns_dtype=ns_dtype)
        self._adamw_hp = dict(lr=adamw_lr, beta1=adamw_betas[0], beta2=adamw_betas[1], eps=adamw_eps,
                              weight_decay=adamw_weight_decay)
        self._momentum_dtype = {"bf16": torch.bfloat16, "f32": torch.float32}[momentum_dtype]
        self._mdt = momentum_dtype
        dev = (muon + adamw)[0].device if (muon or adamw) else torch.device("cuda")
        self._ctx = B.muon_init(dev.index if dev.index is not None else torch.cuda.current_device())
        self._ws = None
        self._ws_bytes = 0
        for p in muon:
            self.state[p]["M"] = torch.zeros_like(p, dtype=self._momentum_dtype)
        for p in adamw:
            self.state[p]["m"] = torch.zeros_like(p, dtype=torch.float32)
            self.state[p]["v"] = torch.zeros_like(p, dtype=torch.float32)
            self.state[p]["step"] = 0

    def _workspace(self, nbytes: int, device) -> int:
        if self._ws is None or self._ws_bytes < nbytes:
            self._ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
            self._ws_bytes = nbytes
        return self._ws.data_ptr()

    @torch.no_grad()
    def step(self, closure=None):
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        stream = torch.cuda.current_stream().cuda_stream
        muon_group, adamw_group = self.param_groups
        # Muon: one call per (weight dtype, gradient dtype); the lr may be changed per step
        # through the group's "lr" entry, like torch schedulers do.
        by_dtype = {}
        for p in muon_group["params"]:
            if p.grad is None:
                continue
            by_dtype.setdefault((_dtype_name(p.dtype), _dtype_name(p.grad.dtype)), []).append(p)
        for (wd, gd), ps in by_dtype.items():
            hp = B.make_hparams(**{**self._muon_hp, "lr": muon_group["lr"]}, w_dtype=wd, g_dtype=gd,
                                m_dtype=self._mdt)
            mats = [(p, p.grad, self.state[p]["M"]) for p in ps]
            nbytes = B.muon_workspace_size(self._ctx, mats, hp)
            ws = self._workspace(nbytes, ps[0].device)
            B.check(B.muon_step(self._ctx, mats, hp, ws, nbytes, stream), "muon_step")
        # AdamW: one call per (weight dtype, gradient dtype, step count), all tensors of it
        # together (normally every tensor has taken every step: one call per dtype pair).
        by_key = {}
        for p in adamw_group["params"]:
            if p.grad is None:
                continue
            self.state[p]["step"] += 1
            key = (_dtype_name(p.dtype), _dtype_name(p.grad.dtype), self.state[p]["step"])
            by_key.setdefault(key, []).append(p)
        for (wd, gd, t), ps in by_key.items():
            hp = B.make_adamw_hparams(**{**self._adamw_hp, "lr": adamw_group["lr"]},
                                      step=t, w_dtype=wd, g_dtype=gd)
            ts = [(p, p.grad, self.state[p]["m"], self.state[p]["v"]) for p in ps]
            B.check(B.muon_adamw_step(self._ctx, ts, hp, stream), "muon_adamw_step")
        return loss

    def muon_parameters(self):
        return list(self.param_groups[0]["params"])

    def adamw_parameters(self):
        return list(self.param_groups[1]["params"])

    def __del__(self):
        try:
            if getattr(self, "_ctx", None) is not None:
                B.muon_destroy(self._ctx)
                self._ctx = None
        except Exception:
            pass
