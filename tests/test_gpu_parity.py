"""End-to-end parity of muon_step (through the C ABI) against the fp64 oracle.

Compared quantities (the tolerances the method's precision allows):
  * O, the orthogonalised update, recovered as (W - W') / lr in float64 (wd = 0), by
    relative Frobenius error: <= 1e-4 on the fp32 path, <= 2e-2 on the bf16 path;
  * M', the new momentum: exact to the storage rounding (fp32: 1e-6, bf16: 2^-8 relative
    elementwise);
  * W' itself: W' = W - lr*O within the same bound scaled by lr.
Inputs come from the seeded generators both sides share; every GPU input value is exact
in its storage dtype and read exactly by the oracle.
"""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from matrix_orthogonalising_optimizer_muon_amd import workloads as wl  # noqa: E402
from oracle import muon as om  # noqa: E402
from tests.gpu_util import GpuState, rel, run_step, to_np  # noqa: E402

TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module")
def B():
    from matrix_orthogonalising_optimizer_muon_amd import binding
    return binding


@pytest.fixture(scope="module")
def ctx(B):
    c = B.muon_init(0)
    yield c
    B.muon_destroy(c)


def oracle_kwargs(w, hp_mode, segments, lr=None):
    return dict(lr=w.lr if lr is None else lr, mu=w.mu, wd=w.wd, nesterov=True, eps=1e-7,
                mode=hp_mode, segments=segments)


def check_step(B, ctx, w, indices=None, mode="gram", segments=(2, 2, 1), steps=1, gpu_mode=None,
               tol=None, mode_of=None):
    """Run `steps` steps on the GPU and in the oracle from the same seeded state and
    gradients; compare after each. The oracle carries its own float64 trajectory (its
    inputs are only the generators' values, never GPU results)."""
    tol = tol or TOL[w.ns_dtype]
    st = GpuState(w, indices)
    hp = B.make_hparams(lr=w.lr, momentum=w.mu, weight_decay=w.wd, segments=segments,
                        mode=gpu_mode or mode, w_dtype=w.w_dtype, g_dtype=w.g_dtype,
                        m_dtype=w.m_dtype, ns_dtype=w.ns_dtype)
    W_o = [wl.weight_np(w, i).astype(np.float64) for i in st.indices]
    M_o = [wl.momentum0_np(w, i).astype(np.float64) for i in st.indices]
    worst = 0.0
    for s in range(steps):
        st.load_gradients(s)
        W_prev = [to_np(x) for x in st.W]
        run_step(ctx, st, hp)
        for k, i in enumerate(st.indices):
            G = wl.gradient_np(w, s, i).astype(np.float64)
            m_k = mode_of(w.matrices[i]) if mode_of else mode
            W_new, M_new, O_ref = om.muon_step(W_o[k], G, M_o[k], **oracle_kwargs(w, m_k, segments))
            W_gpu, M_gpu = to_np(st.W[k]), to_np(st.M[k])
            assert np.all(np.isfinite(W_gpu)) and np.all(np.isfinite(M_gpu))
            O_gpu = (W_prev[k] - W_gpu) / w.lr
            e = rel(O_gpu, O_ref)
            worst = max(worst, e)
            assert e <= tol, (w.name, i, s, e)
            if s == 0:  # from M = 0 the new momentum is G itself: exact
                assert np.array_equal(M_gpu, M_new), (w.name, i)
            else:       # the stored momentum carries one storage rounding per step
                u = 2.0 ** -24 if w.m_dtype == "f32" else 2.0 ** -8
                assert rel(M_gpu, M_new) <= (s + 1) * u, (w.name, i, s)
            W_o[k], M_o[k] = W_new, M_new
    return worst


# ---------------------------------------------------------------- fp32 path (1e-4)

@pytest.mark.parametrize("mode", ["plain", "gram"])
def test_fp32_single_256x1024(B, ctx, mode):
    e = check_step(B, ctx, wl.WORKLOADS["single_fp32_256x1024"], mode=mode)
    print(f"[parity] fp32 256x1024 {mode}: O error {e:.3e}", flush=True)


@pytest.mark.parametrize("mode,segments", [("gram", (2, 3)), ("gram", (1, 1, 1, 1, 1)), ("gram", (5,)),
                                           ("plain", (3,))])
def test_fp32_schedules(B, ctx, mode, segments):
    w = wl.custom("f32sched", [(96, 200)], dtype="f32", wid=201)
    check_step(B, ctx, w, mode=mode, segments=segments)


def test_fp32_ragged_and_tall(B, ctx):
    w = wl.custom("f32ragged", [(100, 300), (300, 100), (130, 130), (1, 17), (65, 1000)], dtype="f32", wid=202)
    check_step(B, ctx, w, mode="gram")
    check_step(B, ctx, w, mode="plain")


# ---------------------------------------------------------------- bf16 path (2e-2)

@pytest.mark.parametrize("mode", ["plain", "gram"])
def test_bf16_lowrank_small(B, ctx, mode):
    w = wl.custom("bf16lr", [(256, 1024)], structure="lowrank", rank=16, wid=203)
    check_step(B, ctx, w, mode=mode)


def test_bf16_ragged_mixed_list(B, ctx):
    shapes = [(100, 300), (300, 100), (130, 130), (1, 17), (65, 1000), (192, 640), (64, 256), (256, 64)]
    w = wl.custom("bf16ragged", shapes, structure="gaussian", wid=204)
    check_step(B, ctx, w, mode="gram")
    check_step(B, ctx, w, mode="plain")


def test_bf16_auto_dispatch_multi_step(B, ctx):
    # decoder-like shapes (square -> plain, 4:1 -> Gram), momentum carried over 3 steps
    shapes = [(256, 256), (1024, 256), (256, 1024), (256, 256)]
    w = wl.custom("bf16dec", shapes, structure="lowrank", rank=8, wid=205, steps=3)
    mode_of = lambda s: "gram" if max(s.rows, s.cols) / min(s.rows, s.cols) > 1.5 else "plain"
    check_step(B, ctx, w, mode="gram", gpu_mode="auto", steps=3, mode_of=mode_of)


def test_bf16_weight_update_bf16_weights(B, ctx):
    """bf16-stored W: W' = bf16(W*(1 - lr*wd) - lr*O). The kernel rounds its fp32 W' once,
    so W' must be the oracle's W' rounded to bf16 except where the O error (about 3e-3 of
    lr*O, mostly far below a bf16 ulp of W) moves the value across a rounding boundary.
    Checked: every element within one ulp of bf16(oracle W') plus lr times the O bar (2e-2)
    of the largest |O| (the O error decides alone for weights near zero, whose ulp is
    tiny), and few elements off bf16(oracle W') at all (a CPU simulation with a 3e-3
    relative O error puts 6% of them one ulp off, 1e-2 puts 14%)."""
    w = wl.custom("bf16w", [(128, 384)], structure="gaussian", wid=206)
    w = wl.Workload(**{**w.__dict__, "w_dtype": "bf16"})
    st = GpuState(w)
    st.load_gradients(0)
    hp = B.make_hparams(w_dtype="bf16", mode="gram")
    run_step(ctx, st, hp)
    W0 = wl.weight_np(w, 0).astype(np.float64)
    G = wl.gradient_np(w, 0, 0).astype(np.float64)
    W_ref, _, O_ref = om.muon_step(W0, G, np.zeros_like(W0), mode="gram")
    W_gpu = to_np(st.W[0])
    W_ref_b = torch.from_numpy(W_ref).to(torch.bfloat16).double().numpy()
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(W_ref_b), 2.0 ** -126))) - 7)
    off = np.abs(W_gpu - W_ref_b)
    assert np.all(off <= ulp + w.lr * 2e-2 * np.abs(O_ref).max()), np.max(off / ulp)
    assert np.mean(off > 0) <= 0.15, np.mean(off > 0)


def test_bf16_2560x9728_full_size(B, ctx):
    """The 2560 x 9728 bf16 momentum matrix at full size, Gram 2+2+1 and plain."""
    w = wl.WORKLOADS["single_bf16_2560x9728"]
    e_gram = check_step(B, ctx, w, mode="gram")
    e_plain = check_step(B, ctx, w, mode="plain")
    print(f"[parity] 2560x9728: O error Gram 2+2+1 {e_gram:.3e}, plain {e_plain:.3e}", flush=True)
    assert e_gram <= 2e-2 and e_plain <= 2e-2


def test_bf16_auto_schedule(B, ctx):
    """Per-shape schedule: plain NS or Gram NS with k balanced segments. Every choice equals
    plain NS in exact arithmetic, so the oracle's plain update is the reference. Three steps:
    the first chooses by FLOP count, later ones by the measured stage times."""
    shapes = [(2560, 9728), (512, 2048), (384, 384), (1024, 256), (96, 700)]
    w = wl.custom("autosched", shapes, structure="lowrank", rank=16, wid=216, steps=3)
    check_step(B, ctx, w, mode="plain", gpu_mode="auto_schedule", steps=3)
    hp = B.make_hparams(mode="auto_schedule")
    raw = [(0, 0, 0, r, c) for r, c in shapes]
    for i in range(len(shapes)):
        e = B.muon_plan_info(ctx, raw, hp, i)
        assert sum(e.segments[:e.n_segments]) == 5


def test_auto_schedule_fixed_workspace(B):
    """A workspace sized once, before the first step measures any tile, serves every later
    step of the automatic schedule (whose plan may switch between plain and Gram NS once
    the stage times are measured), and the size it reports does not change."""
    c = B.muon_init(0)
    try:
        shapes = [(1984, 1984), (1472, 1472), (704, 2880), (2880, 704)]
        w = wl.custom("autows", shapes, structure="lowrank", rank=16, wid=217, steps=3)
        st = GpuState(w)
        hp = B.make_hparams(mode="auto_schedule")
        st.load_gradients(0)
        nbytes = B.muon_workspace_size(c, st.triples(), hp)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        for s in range(3):
            st.load_gradients(s)
            rc = B.muon_step(c, st.triples(), hp, ws.data_ptr(), nbytes)
            torch.cuda.synchronize()
            assert rc == B.MUON_OK, (s, B.muon_status_str(rc))
            assert B.muon_workspace_size(c, st.triples(), hp) == nbytes
        for x in st.W:
            assert torch.isfinite(x).all()
    finally:
        B.muon_destroy(c)


@pytest.mark.parametrize("segments", [(3, 2), (2, 3)])
def test_bf16_2560x9728_long_segments(B, ctx, segments):
    """The single long matrix with two Gram segments of 3 and 2 rounds (the schedule the
    per-shape choice takes for it) against the oracle's plain NS."""
    w = wl.WORKLOADS["single_bf16_2560x9728"]
    assert check_step(B, ctx, w, mode="plain", gpu_mode="gram", segments=segments) <= 2e-2


@pytest.mark.parametrize("mode", ["gram", "plain"])
def test_bf16_few_tiles(B, ctx, mode):
    """Single mid-size matrices with long K: fewer output tiles than the GPU has CUs, one
    of them tall (transposed)."""
    w = wl.custom("splitk", [(512, 4096), (2048, 384)], structure="lowrank", rank=16, wid=210)
    check_step(B, ctx, w, mode=mode)


def test_fp32_few_tiles(B, ctx):
    """The same on the fp32 path."""
    w = wl.custom("splitk32", [(256, 4096)], dtype="f32", wid=211)
    check_step(B, ctx, w, mode="gram")
    check_step(B, ctx, w, mode="plain")


def test_concurrent_groups(B, ctx):
    """Six shape groups: after the first step has measured their tiles, later steps run the
    groups on several streams. Results match the oracle over three steps, and are bitwise
    identical to a profiling context, which keeps every launch on one stream."""
    shapes = [(256, 1024), (128, 512), (512, 128), (64, 256), (192, 192), (96, 320), (448, 64)]
    w = wl.custom("lanes", shapes, structure="lowrank", rank=8, wid=212, steps=3)
    hp = B.make_hparams(mode="auto")
    warm = GpuState(w)
    warm.load_gradients(0)
    run_step(ctx, warm, hp)            # measures the tiles of every group
    mode_of = lambda s: "gram" if max(s.rows, s.cols) / min(s.rows, s.cols) > 1.5 else "plain"
    check_step(B, ctx, w, mode="gram", gpu_mode="auto", steps=3, mode_of=mode_of)
    prof = B.muon_init(0, B.MUON_FLAG_PROFILE)
    try:
        outs = []
        for c in (ctx, prof):
            st = GpuState(w)
            for s in range(3):
                st.load_gradients(s)
                run_step(c, st, hp)
            outs.append([x.clone() for x in st.W + st.M])
        for a, b in zip(*outs):
            assert torch.equal(a, b)
    finally:
        B.muon_destroy(prof)


def test_small_batch_832_full(B, ctx):
    w = wl.WORKLOADS["small_batch_832"]
    e = check_step(B, ctx, w, mode="gram", gpu_mode="auto")
    print(f"[parity] 832 matrices: worst O error {e:.3e}", flush=True)


@pytest.fixture(scope="module")
def ctx_staged(B):
    c = B.muon_init(0, B.MUON_FLAG_STAGED_ONLY)
    yield c
    B.muon_destroy(c)


@pytest.mark.parametrize("structure", ["gaussian", "lowrank"])
@pytest.mark.parametrize("mode", ["gram", "plain"])
def test_small_shapes_both_paths(B, ctx, ctx_staged, mode, structure):
    """Shapes the single-workgroup kernel takes (padded m' <= 128 and m' n' <= 64 Ki; 1 x 17
    up to 128 x 512 and 64 x 1024, tall and wide, ragged), on it and on the staged kernels:
    both within the bar of the oracle, over two steps with momentum carried. Gradients are
    i.i.d. (the small-matrix workload) or rank 4 (s_i = 10 / i) plus N(0, 0.01^2) noise:
    there Newton-Schulz lifts the noise directions, whose singular values are ~100x below
    the top one, to the size of the signal, so an error of a 16-bit rounding of U in them
    shows in O (rounding U to bf16 before the norm gave 0.9-1.7e-2 on these shapes)."""
    shapes = [(1, 17), (64, 256), (256, 64), (100, 300), (65, 500), (128, 128), (7, 129), (128, 512),
              (64, 1024), (1000, 60)]
    w = wl.custom("small_both", shapes, structure=structure, rank=4, wid=213, steps=2)
    hp = B.make_hparams(mode=mode)
    raw = [(0, 0, 0, r, c) for r, c in shapes]
    assert all(B.muon_plan_info(ctx, raw, hp, i).single_wg == 1 for i in range(len(shapes)))
    assert all(B.muon_plan_info(ctx_staged, raw, hp, i).single_wg == 0 for i in range(len(shapes)))
    e1 = check_step(B, ctx, w, mode=mode, steps=2)
    e2 = check_step(B, ctx_staged, w, mode=mode, steps=2)
    assert e1 <= 2e-2 and e2 <= 2e-2


@pytest.mark.parametrize("n", [48, 49])
@pytest.mark.parametrize("tall", [False, True])
def test_group_descriptor_paths(B, ctx_staged, n, tall):
    """A same-shape group of 48 matrices takes its descriptors in the momentum kernel's
    arguments (the kernel writes them to the workspace table for the later stages), one of
    49 from a table kernel; wide-only groups run the flat momentum kernel, groups with tall
    members the tiled one. Staged path, two steps, every matrix against the oracle."""
    shapes = [(96, 64) if tall and k % 3 == 0 else (64, 96) for k in range(n)]
    w = wl.custom("desc_paths", shapes, structure="gaussian", wid=230 + n + (100 if tall else 0), steps=2)
    raw = [(0, 0, 0, r, c) for r, c in shapes]
    hp = B.make_hparams(mode="gram")
    assert all(B.muon_plan_info(ctx_staged, raw, hp, i).single_wg == 0 for i in range(n))
    assert check_step(B, ctx_staged, w, mode="gram", steps=2) <= 2e-2


@pytest.mark.parametrize("segments", [(2, 3), (1, 1, 1, 1, 1), (3, 2), (1, 3, 1)])
def test_small_shapes_schedules(B, ctx, segments):
    w = wl.custom("small_sched", [(96, 320), (128, 512)], structure="gaussian", wid=214)
    check_step(B, ctx, w, mode="gram", segments=segments)


def test_small_bf16_weights(B, ctx):
    w = wl.custom("small_bf16w", [(64, 256), (300, 70)], structure="gaussian", wid=215)
    w = wl.Workload(**{**w.__dict__, "w_dtype": "bf16"})
    st = GpuState(w)
    st.load_gradients(0)
    run_step(ctx, st, B.make_hparams(w_dtype="bf16", mode="gram"))
    for k in range(2):
        W0 = wl.weight_np(w, k).astype(np.float64)
        G = wl.gradient_np(w, 0, k).astype(np.float64)
        W_ref, _, _ = om.muon_step(W0, G, np.zeros_like(W0), mode="gram")
        W_gpu = to_np(st.W[k])
        step = np.abs(W_ref - W0).max()
        assert np.all(np.abs(W_gpu - W_ref) <= 2.0 ** -9 * np.abs(W_ref) + 0.05 * step)
        assert rel(W_gpu - W0, W_ref - W0) < 0.1


# ---------------------------------------------------------------- edge cases

def test_zero_gradient_and_determinism(B, ctx):
    w = wl.custom("zero", [(64, 256), (300, 70)], structure="gaussian", wid=207)
    st = GpuState(w)
    st.G = [torch.zeros_like(m) for m in st.M]
    hp = B.make_hparams(weight_decay=0.1, mode="gram")
    W0 = [to_np(x) for x in st.W]
    run_step(ctx, st, hp)
    for k in range(2):
        Wn = to_np(st.W[k])
        assert np.all(np.isfinite(Wn))
        assert np.allclose(Wn, W0[k] * (1 - 0.02 * 0.1), rtol=1e-6, atol=0)
    # identical inputs -> bitwise identical outputs (fixed-order reductions); a first step
    # measures the tiles and stage times, from which the dispatcher's choice is fixed
    warm = GpuState(wl.custom("det", [(192, 640), (640, 192)], structure="lowrank", rank=4, wid=208))
    warm.load_gradients(0)
    run_step(ctx, warm, B.make_hparams())
    outs = []
    for _ in range(2):
        st2 = GpuState(wl.custom("det", [(192, 640), (640, 192)], structure="lowrank", rank=4, wid=208))
        st2.load_gradients(0)
        run_step(ctx, st2, B.make_hparams())
        outs.append([x.clone() for x in st2.W + st2.M])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_error_leaves_state_untouched(B, ctx):
    w = wl.custom("err", [(64, 256)], structure="gaussian", wid=209)
    st = GpuState(w)
    st.load_gradients(0)
    W0, M0 = st.W[0].clone(), st.M[0].clone()
    mats = st.triples()
    hp = B.make_hparams()
    nbytes = B.muon_workspace_size(ctx, mats, hp)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    assert B.muon_step(ctx, mats, hp, ws.data_ptr(), nbytes - 256) == B.MUON_ERR_WORKSPACE
    bad = B.make_hparams(momentum=1.5)
    assert B.muon_step(ctx, mats, bad, ws.data_ptr(), nbytes) == B.MUON_ERR_ARG
    torch.cuda.synchronize()
    assert torch.equal(st.W[0], W0) and torch.equal(st.M[0], M0)


def test_empty_list_is_a_noop(B, ctx):
    """count == 0 on a device context: MUON_OK, no workspace needed, nothing launched (a
    matrix the call does not name stays as it was)."""
    w = wl.custom("empty", [(64, 256)], structure="gaussian", wid=210)
    st = GpuState(w)
    st.load_gradients(0)
    W0, M0 = st.W[0].clone(), st.M[0].clone()
    arr = B.matrix_list(st.triples(), B.make_hparams())
    assert B.muon_workspace_size(ctx, [], B.make_hparams()) == 0
    assert B.muon_step(ctx, arr, B.make_hparams(), 0, 0, count=0) == B.MUON_OK
    torch.cuda.synchronize()
    assert torch.equal(st.W[0], W0) and torch.equal(st.M[0], M0)
