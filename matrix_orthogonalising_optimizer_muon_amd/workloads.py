"""Seeded synthetic inputs for the Muon update: shapes, dtypes and value structure.

This module holds random-number generation only, none of the update's arithmetic. It is
the one piece of code that both the HIP path (tests, bench) and the fp64 oracle consume:
they receive the very same stored values.

Value recipes (the pages' workloads are private; these stand in for them):

* ``gaussian``: i.i.d. N(0, 1) gradient entries;
* ``lowrank``: ``U diag(s) V^T + N(0, noise^2)`` with Haar-random orthonormal U (rows x r)
  and V (cols x r) (QR of a Gaussian, column signs fixed by the sign of R's diagonal) and
  ``s_i = scale * i^(-decay)``; the MuonX article (section 2) describes momentum updates
  as dominated by a few directions;
* weights: ``0.02 * N(0, 1)``; momentum starts at zero.

Values are drawn in float64 and rounded (round-to-nearest-even) to the storage dtype; the
returned float32 arrays hold exactly the stored values, so the oracle reads them exactly.

Seeds: ``numpy.random.Generator(PCG64(SeedSequence([workload_id, step, index, role])))``
with role 0 = gradient noise / Gaussian gradient, 1 = weight, 2 = left basis, 3 = right
basis.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

ROLE_GRAD, ROLE_WEIGHT, ROLE_UBASIS, ROLE_VBASIS = 0, 1, 2, 3


@dataclass(frozen=True)
class MatrixSpec:
    name: str
    rows: int
    cols: int


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int                     # seed component
    matrices: tuple              # tuple[MatrixSpec]
    g_dtype: str = "bf16"        # gradient storage
    m_dtype: str = "bf16"        # momentum storage
    w_dtype: str = "f32"         # weight storage
    ns_dtype: str = "bf16"       # NS operand precision class ("bf16" path or "f32" path)
    structure: str = "lowrank"   # "gaussian" | "lowrank"
    rank: int = 0
    decay: float = 1.0
    scale: float = 10.0
    noise: float = 0.01
    steps: int = 1
    lr: float = 0.02
    mu: float = 0.95
    wd: float = 0.0
    description: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def elements(self) -> int:
        return sum(s.rows * s.cols for s in self.matrices)


def _decoder_layers(layers, d, ff, kv=None):
    out = []
    kv = d if kv is None else kv
    for l in range(layers):
        out += [MatrixSpec(f"L{l}.q", d, d), MatrixSpec(f"L{l}.k", kv, d),
                MatrixSpec(f"L{l}.v", kv, d), MatrixSpec(f"L{l}.o", d, d),
                MatrixSpec(f"L{l}.gate", ff, d), MatrixSpec(f"L{l}.up", ff, d),
                MatrixSpec(f"L{l}.down", d, ff)]
    return tuple(out)


WORKLOADS = {
    "single_fp32_256x1024": Workload(
        name="single_fp32_256x1024", wid=1, matrices=(MatrixSpec("w", 256, 1024),),
        g_dtype="f32", m_dtype="f32", w_dtype="f32", ns_dtype="f32", structure="gaussian",
        description="one fp32 256x1024 matrix, i.i.d. N(0,1) gradient, plain and Gram NS"),
    "single_bf16_2560x9728": Workload(
        name="single_bf16_2560x9728", wid=2, matrices=(MatrixSpec("w", 2560, 9728),),
        structure="lowrank", rank=64, decay=1.0,
        description="one bf16 2560x9728 momentum matrix, rank-64 gradient (s_i = 10/i) + N(0, 0.01^2)"),
    "decoder_d2048_24layers": Workload(
        name="decoder_d2048_24layers", wid=3, matrices=_decoder_layers(24, 2048, 8192),
        structure="lowrank", rank=32, decay=1.0, steps=3,
        description="24 decoder layers, d=2048, ff=8192: Q/K/V/O 2048^2, gate/up 8192x2048, "
                    "down 2048x8192; rank-32 gradients + noise, 3 steps with momentum carried"),
    "small_batch_832": Workload(
        name="small_batch_832", wid=4,
        matrices=tuple([MatrixSpec(f"a{i}", 64, 256) for i in range(512)]
                       + [MatrixSpec(f"b{i}", 128, 512) for i in range(256)]
                       + [MatrixSpec(f"c{i}", 256, 1024) for i in range(64)]),
        structure="gaussian",
        description="832 small bf16 matrices (512 x 64x256, 256 x 128x512, 64 x 256x1024), i.i.d. N(0,1)"),
    "dense_7b_28layers": Workload(
        name="dense_7b_28layers", wid=5, matrices=_decoder_layers(28, 3584, 18944, kv=512),
        structure="lowrank", rank=128, decay=0.8,
        description="28 decoder layers, hidden 3584, intermediate 18944, K/V 512x3584; "
                    "rank-128 gradients (s_i = 10 i^-0.8) + N(0, 0.01^2)"),
}


# Parameters of the 7B decoder shape set that stay with AdamW (MuonX article, section 2:
# embeddings, biases and similar parameters): token embedding and output head
# (vocabulary 152064 x hidden 3584, the untied head of the Qwen2.5-7B shape set), the
# q / k / v biases of 28 layers (3584, 512, 512) and 57 norm weights of 3584.
ADAMW_SETS = {
    "dense_7b_nonmatrix": (
        [("embed", 152064 * 3584), ("lm_head", 152064 * 3584)]
        + [(f"L{l}.{b}", n) for l in range(28) for b, n in (("q_bias", 3584), ("k_bias", 512), ("v_bias", 512))]
        + [(f"norm{i}", 3584) for i in range(57)]
    ),
}


def rng_for(w: Workload, step: int, index: int, role: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.wid, step, index, role])))


def round_to(x, dtype: str) -> np.ndarray:
    """Round float values to the storage dtype (RNE) and return them as float32."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        u = x32.view(np.uint32).astype(np.uint64)
        u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
        return u.astype(np.uint32).view(np.float32)
    raise ValueError(dtype)


def haar_basis(rng: np.random.Generator, n: int, r: int) -> np.ndarray:
    Z = rng.standard_normal((n, r))
    Qm, Rm = np.linalg.qr(Z)
    return Qm * np.sign(np.diag(Rm))


def gradient_np(w: Workload, step: int, index: int, spec: MatrixSpec | None = None) -> np.ndarray:
    """Gradient of matrix ``index`` at ``step`` as float32 holding the stored values."""
    spec = spec or w.matrices[index]
    rows, cols = spec.rows, spec.cols
    if w.structure == "gaussian":
        G = rng_for(w, step, index, ROLE_GRAD).standard_normal((rows, cols))
    else:
        r = min(w.rank, rows, cols)
        Ub = haar_basis(rng_for(w, step, index, ROLE_UBASIS), rows, r)
        Vb = haar_basis(rng_for(w, step, index, ROLE_VBASIS), cols, r)
        s = w.scale * np.arange(1, r + 1, dtype=np.float64) ** (-w.decay)
        G = (Ub * s) @ Vb.T
        G += w.noise * rng_for(w, step, index, ROLE_GRAD).standard_normal((rows, cols))
    return round_to(G, w.g_dtype)


def weight_np(w: Workload, index: int, spec: MatrixSpec | None = None) -> np.ndarray:
    spec = spec or w.matrices[index]
    W = 0.02 * rng_for(w, 0, index, ROLE_WEIGHT).standard_normal((spec.rows, spec.cols))
    return round_to(W, w.w_dtype)


def momentum0_np(w: Workload, index: int, spec: MatrixSpec | None = None) -> np.ndarray:
    spec = spec or w.matrices[index]
    return np.zeros((spec.rows, spec.cols), dtype=np.float32)


def custom(name: str, shapes, *, structure="gaussian", dtype="bf16", rank=8, decay=1.0,
           wid=100, steps=1) -> Workload:
    """A small workload of arbitrary shapes (tests: ragged sizes, edge cases)."""
    f32 = dtype == "f32"
    return Workload(name=name, wid=wid,
                    matrices=tuple(MatrixSpec(f"m{i}", r, c) for i, (r, c) in enumerate(shapes)),
                    g_dtype="f32" if f32 else "bf16", m_dtype="f32" if f32 else "bf16",
                    w_dtype="f32", ns_dtype="f32" if f32 else "bf16", structure=structure,
                    rank=rank, decay=decay, steps=steps)


def _haar_torch(Z):
    """Orthonormal factor of the QR decomposition of the Gaussian n x r matrix Z with R's
    diagonal positive (the same basis :func:`haar_basis` takes, as that factorisation is
    unique), by Cholesky QR: the r x r Gram matrix is formed on the device in float64, its
    Cholesky factor R^T computed on the host (NumPy), and Q = Z R^-1 on the device. Only
    products and element-wise kernels run on the device (Z is well conditioned for
    n >> r, so Cholesky QR keeps Q orthonormal to float64 rounding)."""
    import torch

    Z64 = Z.to(torch.float64)
    gram = (Z64.T @ Z64).cpu().numpy()
    Rinv = np.linalg.inv(np.linalg.cholesky(gram).T)      # upper-triangular R^-1
    return (Z64 @ torch.from_numpy(Rinv).to(Z.device)).to(torch.float32)


def gradient_torch(w: Workload, step: int, index: int, device="cuda", spec: MatrixSpec | None = None):
    """Device-side draw with the same recipe as :func:`gradient_np` (torch's generator,
    so not the same values): for timing runs of workloads too large to draw on the host.
    The Haar bases come from :func:`_haar_torch` (no device linear-algebra solver is
    called). Returns a tensor in the gradient's storage dtype."""
    import torch

    spec = spec or w.matrices[index]
    rows, cols = spec.rows, spec.cols
    gen = torch.Generator(device=device)
    gen.manual_seed(int(np.random.SeedSequence([w.wid, step, index, 7]).generate_state(1)[0]))
    if w.structure == "gaussian":
        G = torch.randn(rows, cols, generator=gen, device=device)
    else:
        r = min(w.rank, rows, cols)
        Ub = _haar_torch(torch.randn(rows, r, generator=gen, device=device))
        Vb = _haar_torch(torch.randn(cols, r, generator=gen, device=device))
        s = w.scale * torch.arange(1, r + 1, device=device, dtype=torch.float32) ** (-w.decay)
        G = (Ub * s) @ Vb.T
        G += w.noise * torch.randn(rows, cols, generator=gen, device=device)
    return G.to(torch.bfloat16 if w.g_dtype == "bf16" else torch.float32)


def weight_torch(w: Workload, index: int, device="cuda", spec: MatrixSpec | None = None):
    """Device-side initial weight, 0.02 * N(0, 1) from torch's generator (seeded per matrix),
    in the weight's storage dtype."""
    import torch

    spec = spec or w.matrices[index]
    gen = torch.Generator(device=device)
    gen.manual_seed(int(np.random.SeedSequence([w.wid, 0, index, 8]).generate_state(1)[0]))
    W = 0.02 * torch.randn(spec.rows, spec.cols, generator=gen, device=device)
    return W.to(torch.bfloat16 if w.w_dtype == "bf16" else torch.float32)
