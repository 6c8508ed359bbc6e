"""AdamW companion (muon_adamw_step) against the fp64 oracle (oracle/adamw.py), element
by element, over several steps; the oracle carries its own trajectory from the same seeded
inputs, its W rounded to the storage dtype after each step as the library stores it.

Bound per element: the kernel computes in fp32, so
    |W_gpu - W_ref| <= u_w |W_ref| + 1e-5 lr (1 + |q|)
with u_w = 2^-20 (fp32 W) or 2^-7 (bf16 W: one ulp, the two roundings either side of a tie) and
q = m_hat / (sqrt(v_hat) + eps) the oracle's step direction; v (fp32) within 1e-5 relative;
m within 1e-6 of the magnitudes summed into it (b1 |m| + (1 - b1) |g|, which may cancel).
"""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from matrix_orthogonalising_optimizer_muon_amd import workloads as wl  # noqa: E402
from oracle import adamw as oa  # noqa: E402

TDT = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def B():
    from matrix_orthogonalising_optimizer_muon_amd import binding
    return binding


@pytest.fixture(scope="module")
def ctx(B):
    c = B.muon_init(0)
    yield c
    B.muon_destroy(c)


def dev(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(TDT[dt])


def run(B, ctx, sizes, w_dtype, g_dtype, steps=3, misalign=(), seed=0, **hpkw):
    rng = np.random.default_rng(seed)
    lr = hpkw.get("lr", 2e-3)
    hpkw.setdefault("lr", lr)
    W_ref, m_ref, v_ref, state, keep = [], [], [], [], []
    mscale = [np.zeros(n) for n in sizes]
    for i, n in enumerate(sizes):
        W0 = wl.round_to(rng.standard_normal(n) * 0.05, w_dtype).astype(np.float64)
        off = 1 if i in misalign else 0          # a 1-element offset forces the scalar path
        Wb = torch.zeros(n + off, dtype=TDT[w_dtype], device="cuda")
        Wb[off:] = dev(W0, w_dtype)
        mb = torch.zeros(n + off, dtype=torch.float32, device="cuda")
        vb = torch.zeros(n + off, dtype=torch.float32, device="cuda")
        keep += [Wb, mb, vb]
        state.append([Wb[off:], None, mb[off:], vb[off:]])
        W_ref.append(W0); m_ref.append(np.zeros(n)); v_ref.append(np.zeros(n))
    for t in range(1, steps + 1):
        hp = B.make_adamw_hparams(step=t, w_dtype=w_dtype, g_dtype=g_dtype, **hpkw)
        Gs = [wl.round_to(rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 0), g_dtype).astype(np.float64)
              for n in sizes]
        for s, G in zip(state, Gs):
            s[1] = dev(G, g_dtype)
        tensors = [(s[0].data_ptr(), s[1].data_ptr(), s[2].data_ptr(), s[3].data_ptr(), n)
                   for s, n in zip(state, sizes)]
        assert B.muon_adamw_step(ctx, tensors, hp) == 0
        torch.cuda.synchronize()
        for k, (s, G) in enumerate(zip(state, Gs)):
            W_new, m_new, v_new = oa.adamw_step(W_ref[k], G, m_ref[k], v_ref[k], t, lr=hp.lr, beta1=hp.beta1,
                                                beta2=hp.beta2, eps=hp.eps, wd=hp.weight_decay)
            q = (m_new / (1 - hp.beta1 ** t)) / (np.sqrt(v_new / (1 - hp.beta2 ** t)) + hp.eps)
            W_new = wl.round_to(W_new, w_dtype).astype(np.float64)
            Wg = s[0].double().cpu().numpy()
            mg, vg = s[2].double().cpu().numpy(), s[3].double().cpu().numpy()
            u = 2.0 ** -20 if w_dtype == "f32" else 2.0 ** -7   # bf16: one ulp (2^-7 |W| >= ulp)
            bound = u * np.abs(W_new) + 1e-5 * lr * (1 + np.abs(q))
            bad = np.abs(Wg - W_new) > bound
            assert not bad.any(), (sizes[k], t, np.argwhere(bad)[:3], Wg[bad][:3], W_new[bad][:3])
            # m may cancel (beta1 m and (1 - beta1) g of opposite signs): its error is bounded
            # relative to the magnitudes summed into it, not to the result
            mscale[k] = hp.beta1 * mscale[k] + (1 - hp.beta1) * np.abs(G)
            assert np.all(np.abs(mg - m_new) <= 1e-6 * mscale[k] + 1e-30), (sizes[k], t)
            assert np.all(np.abs(vg - v_new) <= 1e-5 * np.abs(v_new) + 1e-30), (sizes[k], t)
            W_ref[k], m_ref[k], v_ref[k] = W_new, m_new, v_new


RAGGED = [1, 7, 8, 9, 2047, 2048, 2049, 3 * 2048 + 5, 100_000]


@pytest.mark.parametrize("w_dtype,g_dtype", [("f32", "bf16"), ("f32", "f32"), ("bf16", "bf16")])
def test_adamw_ragged(B, ctx, w_dtype, g_dtype):
    run(B, ctx, RAGGED, w_dtype, g_dtype, misalign={1, 4, 8}, weight_decay=0.1)


def test_adamw_many_tensors_and_empty(B, ctx):
    """More tensors than one launch carries (24), an empty tensor among them."""
    sizes = [int(n) for n in np.random.default_rng(5).integers(1, 5000, size=40)]
    sizes[13] = 0
    run(B, ctx, sizes, "f32", "bf16", steps=2)


def test_adamw_hyperparameters(B, ctx):
    run(B, ctx, [4096, 333], "f32", "f32", steps=4, lr=0.05, beta1=0.5, beta2=0.9, eps=1e-3, weight_decay=0.0)


def test_adamw_zero_gradient_is_decay_only(B, ctx):
    W = torch.full((5000,), 2.0, device="cuda")
    G = torch.zeros(5000, dtype=torch.bfloat16, device="cuda")
    m = torch.zeros(5000, device="cuda")
    v = torch.zeros(5000, device="cuda")
    hp = B.make_adamw_hparams(lr=0.1, weight_decay=0.5)
    assert B.muon_adamw_step(ctx, [(W, G, m, v)], hp) == 0
    torch.cuda.synchronize()
    assert torch.all(W == 2.0 * (1 - 0.1 * 0.5)) and torch.all(m == 0) and torch.all(v == 0)
