"""C-ABI checks that need no GPU: the library loads, exports every symbol the header
declares, validates every argument before touching a device, and plans as documented.

A host-only context (device -1) makes planning and validation callable on the CPU.
"""

import ctypes
import os
import re
import subprocess

import pytest

from oracle import flop_model

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon.h")
B = pytest.importorskip("matrix_orthogonalising_optimizer_muon_amd.binding")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(muon_[a-z_]+)\s*\(", text)))


def test_header_symbols_exported():
    names = declared_functions()
    assert "muon_step" in names and "muon_init" in names and len(names) >= 8
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (muon_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert getattr(lib, n) is not None


def test_header_constants_match_binding():
    text = open(HEADER).read()
    for name in ["MUON_OK", "MUON_ERR_ARG", "MUON_ERR_WORKSPACE", "MUON_ERR_DEVICE", "MUON_ERR_HIP",
                 "MUON_ERR_UNSUPPORTED", "MUON_F32", "MUON_BF16", "MUON_NS_AUTO", "MUON_NS_PLAIN",
                 "MUON_NS_GRAM", "MUON_MAX_SEGMENTS"]:
        m = re.search(rf"#define {name} (-?\d+)", text)
        assert m and int(m.group(1)) == getattr(B, name), name


def test_struct_layouts_match_c_compiler(tmp_path):
    """Field offsets and sizes of the header's structs, as gcc lays them out, equal the
    ctypes mirrors the binding uses."""
    structs = {"muon_matrix": B.muon_matrix, "muon_hparams": B.muon_hparams,
               "muon_plan_entry": B.muon_plan_entry, "muon_profile_entry": B.muon_profile_entry,
               "muon_adamw_tensor": B.muon_adamw_tensor, "muon_adamw_hparams": B.muon_adamw_hparams}
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(void){"]
    for name, cls in structs.items():
        lines.append(f'printf("{name} size %zu\\n", sizeof({name}));')
        for f, _ in cls._fields_:
            lines.append(f'printf("{name} {f} %zu\\n", offsetof({name}, {f}));')
    lines.append("return 0;}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", str(src), "-o", str(exe)], check=True)
    got = {}
    for line in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.splitlines():
        name, field, val = line.split()
        got[(name, field)] = int(val)
    for name, cls in structs.items():
        assert got[(name, "size")] == ctypes.sizeof(cls), name
        for f, _ in cls._fields_:
            assert got[(name, f)] == getattr(cls, f).offset, (name, f)


def test_defaults_and_status_strings():
    hp = B.muon_hparams_default()
    assert abs(hp.lr - 0.02) < 1e-9 and abs(hp.momentum - 0.95) < 1e-7 and hp.nesterov == 1
    assert (round(hp.a, 4), round(hp.b, 4), round(hp.c, 4)) == (3.4445, -4.775, 2.0315)
    assert hp.n_segments == 3 and list(hp.segments)[:3] == [2, 2, 1]
    assert hp.mode == B.MUON_NS_AUTO and hp.w_dtype == B.MUON_F32 and hp.ns_dtype == B.MUON_BF16
    for s in [0, -1, -2, -3, -4, -5]:
        assert B.muon_status_str(s).startswith("MUON_")
    assert "unknown" in B.muon_status_str(42)


@pytest.fixture(scope="module")
def hctx():
    ctx = B.muon_init(-1)
    yield ctx
    B.muon_destroy(ctx)


FAKE = 0x10000  # never dereferenced: host-only contexts launch nothing


def mats_of(shapes):
    return B.matrix_list([(FAKE, FAKE, FAKE, r, c) for r, c in shapes])


def step(ctx, shapes, hp=None, ws=FAKE * 256, wsb=1 << 40, count=None):
    hp = hp or B.make_hparams()
    arr = mats_of(shapes)
    n = len(shapes) if count is None else count
    return B._lib.muon_step(ctx, arr, n, ctypes.byref(hp), ctypes.c_void_p(ws), ctypes.c_size_t(wsb), None)


def test_profile_read_errors(hctx):
    n = ctypes.c_int(-1)
    buf = (B.muon_profile_entry * 4)()
    # context without the profiling flag
    assert B._lib.muon_profile_read(hctx, buf, 4, ctypes.byref(n)) == B.MUON_ERR_ARG
    assert B._lib.muon_profile_read(None, buf, 4, ctypes.byref(n)) == B.MUON_ERR_ARG
    pctx = B.muon_init(-1, B.MUON_FLAG_PROFILE)
    assert B.muon_profile_read(pctx) == []
    B.muon_destroy(pctx)


def test_init_errors():
    out = ctypes.c_void_p()
    assert B._lib.muon_init(None, 0, 0) == B.MUON_ERR_ARG
    assert B._lib.muon_init(ctypes.byref(out), -1, 16) == B.MUON_ERR_ARG
    assert B._lib.muon_init(ctypes.byref(out), 9999, 0) == B.MUON_ERR_DEVICE
    assert B._lib.muon_destroy(None) == B.MUON_OK


def test_validation_before_device(hctx):
    ok_shapes = [(64, 256)]
    # valid arguments reach the device check
    assert step(hctx, ok_shapes) == B.MUON_ERR_DEVICE
    assert step(hctx, [], count=0) == B.MUON_OK           # empty list is a no-op
    assert B._lib.muon_step(None, None, 0, None, None, 0, None) == B.MUON_ERR_ARG
    assert step(hctx, ok_shapes, count=-1) == B.MUON_ERR_ARG
    assert step(hctx, [(0, 256)]) == B.MUON_ERR_ARG
    assert step(hctx, [(64, -3)]) == B.MUON_ERR_ARG
    assert step(hctx, [(1 << 21, 4)]) == B.MUON_ERR_ARG
    arr = B.matrix_list([(0, FAKE, FAKE, 64, 256)])
    hp = B.make_hparams()
    assert B._lib.muon_step(hctx, arr, 1, ctypes.byref(hp), ctypes.c_void_p(FAKE * 256),
                            ctypes.c_size_t(1 << 40), None) == B.MUON_ERR_ARG
    bad = [dict(momentum=1.0), dict(momentum=-0.1), dict(eps=-1.0), dict(lr=float("nan")),
           dict(nesterov=2), dict(coeffs=(float("inf"), 0, 0)), dict(segments=[]),
           dict(segments=[2, 0, 1]), dict(segments=[1] * 9), dict(segments=[40, 30]),
           dict(mode=7), dict(w_dtype=5), dict(g_dtype=-1), dict(m_dtype=2), dict(ns_dtype=9)]
    for kw in bad:
        hp = B.make_hparams(**kw)
        if kw.get("segments") == []:
            hp.n_segments = 0
        assert step(hctx, ok_shapes, hp) == B.MUON_ERR_ARG, kw
    # fp16 Gram-space limit: a Gram segment longer than 3 rounds on the bf16 path
    assert step(hctx, ok_shapes, B.make_hparams(segments=[4, 1], mode="gram")) == B.MUON_ERR_UNSUPPORTED
    assert step(hctx, ok_shapes, B.make_hparams(segments=[4, 1], mode="auto")) == B.MUON_ERR_UNSUPPORTED
    assert step(hctx, ok_shapes, B.make_hparams(segments=[3, 2], mode="gram")) == B.MUON_ERR_DEVICE
    assert step(hctx, ok_shapes, B.make_hparams(segments=[9], mode="plain")) == B.MUON_ERR_DEVICE
    assert step(hctx, ok_shapes, B.make_hparams(segments=[9], mode="auto_schedule")) == B.MUON_ERR_DEVICE
    assert step(hctx, ok_shapes, B.make_hparams(segments=[9], mode="gram", ns_dtype="f32")) == B.MUON_ERR_DEVICE


def test_workspace_errors(hctx):
    shapes = [(64, 256), (300, 70)]
    need = B.muon_workspace_size(hctx, [(0, 0, 0, r, c) for r, c in shapes], B.make_hparams())
    assert need > 0 and need % 256 == 0
    assert step(hctx, shapes, ws=0) == B.MUON_ERR_WORKSPACE
    assert step(hctx, shapes, ws=FAKE * 256 + 16) == B.MUON_ERR_WORKSPACE
    assert step(hctx, shapes, wsb=need - 1) == B.MUON_ERR_WORKSPACE
    assert step(hctx, shapes, wsb=need) == B.MUON_ERR_DEVICE


B_TILE_COUNT = 15   # tile ids muon_debug_gemm documents: 0..14


def test_debug_gemm_validation(hctx):
    f = B._lib.muon_debug_gemm
    P = ctypes.c_void_p(FAKE)
    # f(ctx, kind, ns_dtype, tile_cfg, M, N, K, A, B, E, C, C2, alpha, beta, gamma, oscale, stream)
    assert f(hctx, 3, 1, 0, 64, 64, 64, P, P, None, P, None, 1.0, 0.0, 0.0, 1.0, None) == B.MUON_ERR_ARG
    assert f(hctx, 0, 1, B_TILE_COUNT, 64, 64, 64, P, P, None, P, None, 1.0, 0.0, 0.0, 1.0, None) == B.MUON_ERR_ARG
    assert f(hctx, 0, 1, 6, 256, 256, 64, P, P, None, P, None, 1.0, 0.0, 0.0, 1.0, None) == B.MUON_ERR_ARG
    assert f(hctx, 0, 1, 0, 64, 64, 100, P, P, None, P, None, 1.0, 0.0, 0.0, 1.0, None) == B.MUON_ERR_ARG
    assert f(hctx, 1, 1, 0, 64, 128, 64, P, P, None, P, None, 1.0, 0.0, 0.0, 1.0, None) == B.MUON_ERR_ARG
    assert f(hctx, 0, 1, 2, 256, 256, 64, P, P, None, P, None, 1.0, 0.0, 0.0, 1.0, None) == B.MUON_ERR_ARG
    assert f(hctx, 2, 1, 0, 64, 64, 64, P, P, None, None, None, 1.0, 0.0, 0.0, 1.0, None) == B.MUON_ERR_ARG
    assert f(hctx, 2, 1, 2, 64, 128, 64, P, P, None, P, None, 1.0, 0.0, 0.0, 1.0, None) == B.MUON_ERR_DEVICE


# ---------------------------------------------------------------- dispatcher / FLOP model

def plan(hctx, shapes, **kw):
    hp = B.make_hparams(**kw)
    raw = [(0, 0, 0, r, c) for r, c in shapes]
    return [B.muon_plan_info(hctx, raw, hp, i) for i in range(len(shapes))]


def test_plan_flops_match_oracle_model(hctx):
    shapes = [(2560, 9728), (9728, 2560), (64, 256), (300, 70), (2048, 2048), (512, 3584)]
    for segs in [(2, 2, 1), (2, 3), (1, 1, 1, 1, 1), (5,), (3, 1, 1)]:
        # segments longer than 3 rounds exist on the fp32 path only
        dt = dict(ns_dtype="f32", g_dtype="f32", m_dtype="f32") if max(segs) > 3 else {}
        for mode in ("plain", "gram"):
            for (r, c), e in zip(shapes, plan(hctx, shapes, segments=segs, mode=mode, **dt)):
                assert e.single_wg == 0   # a list with large shapes stays on the staged kernels
                assert e.mode == B.MODES[mode]
                assert e.dense_flops == pytest.approx(flop_model.dense_flops(r, c, mode, segs), rel=1e-12)
                m, n = min(r, c), max(r, c)
                assert (e.m, e.n, e.transposed) == (m, n, int(r > c))
                nl, ns = flop_model.product_counts(mode, segs)
                # symmetric outputs computed once: SYRK m'^2 n', squares m'^3, apply 2 m'^2 n'
                assert e.kernel_flops == pytest.approx((nl // 2) * 3.0 * m * m * n + ns * 1.0 * m ** 3, rel=1e-12)


def test_single_workgroup_choice(hctx):
    """Lists of small shapes only (padded m' <= 128, m' n' <= 64 Ki) run one workgroup per
    matrix, computing every product densely; one larger shape keeps the list staged."""
    small = [(64, 256), (300, 70), (1, 17), (128, 512), (1024, 64)]
    for i, e in enumerate(plan(hctx, small)):
        assert e.single_wg == 1 and (e.tile_sym, e.tile_apply) == (-1, -1)
        assert e.kernel_flops == pytest.approx(e.dense_flops, rel=1e-12)
    for extra in [(129, 512), (128, 576), (64, 1088)]:
        assert all(e.single_wg == 0 for e in plan(hctx, small + [extra]))
    staged = B.muon_init(-1, B.MUON_FLAG_STAGED_ONLY)
    try:
        assert all(e.single_wg == 0 for e in plan(staged, small))
    finally:
        B.muon_destroy(staged)
    assert all(e.single_wg == 0 for e in plan(hctx, small, ns_dtype="f32", g_dtype="f32", m_dtype="f32"))


def test_auto_dispatch_follows_flop_model(hctx):
    shapes = [(2048, 2048), (8192, 2048), (2048, 8192), (3584, 3584), (512, 3584), (18944, 3584),
              (64, 256), (100, 140), (100, 160), (2560, 9728)]
    for (r, c), e in zip(shapes, plan(hctx, shapes)):
        g = flop_model.dense_flops(r, c, "gram")
        p = flop_model.dense_flops(r, c, "plain")
        assert e.mode == (B.MUON_NS_GRAM if g < p else B.MUON_NS_PLAIN), (r, c)
    es = plan(hctx, shapes)
    assert es[0].mode == B.MUON_NS_PLAIN and es[1].mode == B.MUON_NS_GRAM and es[3].mode == B.MUON_NS_PLAIN
    # the crossover sits at n'/m' = 1.5 for segments 2+2+1
    assert es[7].mode == B.MUON_NS_PLAIN and es[8].mode == B.MUON_NS_GRAM


def test_grouping_by_canonical_shape(hctx):
    shapes = [(64, 256), (256, 64), (128, 512), (64, 256), (2048, 8192)]
    es = plan(hctx, shapes)
    assert es[0].group == es[1].group == es[3].group
    assert len({es[0].group, es[2].group, es[4].group}) == 3
    # largest work first
    assert es[4].group == 0


def test_workspace_size_is_deterministic_and_grows(hctx):
    hp = B.make_hparams()
    one = B.muon_workspace_size(hctx, [(0, 0, 0, 256, 1024)], hp)
    two = B.muon_workspace_size(hctx, [(0, 0, 0, 256, 1024)] * 2, hp)
    assert one == B.muon_workspace_size(hctx, [(0, 0, 0, 256, 1024)], hp)
    assert two > one
    f32 = B.muon_workspace_size(hctx, [(0, 0, 0, 256, 1024)], B.make_hparams(ns_dtype="f32"))
    assert f32 > one


# ---------------------------------------------------------------- tile cache file

def test_tune_cache_round_trip(hctx, tmp_path):
    """Choices loaded from a file are the ones plan_info reports and are written back
    unchanged (a host-only context keeps its own device key, so GPU runs are unaffected)."""
    src = tmp_path / "tune.txt"
    src.write_text("1 0 2560 2560 1 10 0.0305\n2 0 2560 9728 1 7\n\n0 0 2560 2560 1 5 -1\n"
                   "4 0 2560 2560 1 12 0.0925\n")
    assert B.muon_tune_load(hctx, str(src)) == 4
    e = B.muon_plan_info(hctx, [(0, 0, 0, 2560, 9728)], B.make_hparams(), 0)
    assert (e.tile_sym, e.tile_apply) == (10, 7)
    out = tmp_path / "out.txt"
    B.muon_tune_save(hctx, str(out))
    # the time is held as a float32
    got = sorted((tuple(map(int, l.split()[:6])), round(float(l.split()[6]), 6)) for l in out.read_text().splitlines())
    assert got == sorted([((0, 0, 2560, 2560, 1, 5), -1.0), ((1, 0, 2560, 2560, 1, 10), 0.0305),
                          ((2, 0, 2560, 9728, 1, 7), -1.0), ((4, 0, 2560, 2560, 1, 12), 0.0925)])


@pytest.mark.parametrize("text", [
    "1 0 2560 2560 1\n",            # missing field
    "1 0 2560 2560 1 10 3 4\n",     # extra field after the time
    "1 0 2560 2560 1 10 nan\n",     # time not finite
    "1 0 2560 2560 1 10 t\n",       # time not a number
    "3 0 2560 9728 1 7\n",          # the update stage shares the apply's choice
    "1 0 2560 9728 1 10\n",         # symmetric stage with m != n
    "1 0 2560 2560 1 6\n",          # 256x128 tile for a symmetric stage
    "2 1 2560 9728 1 7\n",          # 256 tile on the fp32 path
    "2 0 2500 9728 1 1\n",          # not a multiple of 64
    "2 0 2560 9728 0 1\n",          # empty batch
    "2 0 2560 9728 1 15\n",         # unknown tile
    "2 0 2560 9728 1 x\n",
])
def test_tune_cache_rejects_bad_files(hctx, tmp_path, text):
    f = tmp_path / "bad.txt"
    f.write_text("2 0 640 1280 3 1\n" + text)
    before = B.muon_plan_info(hctx, [(0, 0, 0, 640, 1280)] * 3, B.make_hparams(), 0).tile_apply
    with pytest.raises(B.MuonError):
        B.muon_tune_load(hctx, str(f))
    # nothing of the file was taken, also not its valid first line
    assert B.muon_plan_info(hctx, [(0, 0, 0, 640, 1280)] * 3, B.make_hparams(), 0).tile_apply == before
    with pytest.raises(B.MuonError):
        B.muon_tune_load(hctx, str(tmp_path / "missing.txt"))


# ---------------------------------------------------------------- per-shape schedule

def _expected_schedule(m, n, R, cap=3):
    """Cheapest of plain NS and Gram NS with k balanced segments (longer first), counted
    with the oracle's product counts and the kernels' cost per product (Gram product
    m'^2 n', apply 2 m'^2 n', m' x m' product m'^3); ties keep plain, then the larger k."""
    def cost(mode, segs):
        n_long, n_sq = flop_model.product_counts(mode, segs, rounds=R if mode == "plain" else None)
        return (n_long // 2) * (1.0 * m * m * n + 2.0 * m * m * n) + n_sq * 1.0 * m ** 3
    best, choice = cost("plain", (R,)), ("plain", (R,))
    for k in range(min(R, 8), -(-R // cap) - 1, -1):
        segs = tuple(R // k + (1 if i < R % k else 0) for i in range(k))
        c = cost("gram", segs)
        if c < best * (1 - 1e-9):
            best, choice = c, ("gram", segs)
    return choice


@pytest.mark.parametrize("segs", [(2, 2, 1), (5,), (1, 1, 1), (3, 4), (4, 4, 4, 4, 4)])
def test_auto_schedule_model_choice(hctx, segs):
    shapes = [(2560, 9728), (9728, 2560), (2048, 2048), (512, 3584), (3584, 18944), (300, 70), (1000, 1400)]
    R = sum(segs)
    mctx = B.muon_init(-1, B.MUON_FLAG_MODEL_ONLY)
    try:
        for (r, c), e in zip(shapes, plan(mctx, shapes, segments=segs, mode="auto_schedule")):
            m, n = min(r, c), max(r, c)
            mode, want = _expected_schedule(m, n, R)
            assert e.mode == B.MODES[mode], ((r, c), segs)
            got = tuple(e.segments[:e.n_segments])
            assert got == want, ((r, c), segs, got, want)
            assert sum(got) == R
            if mode == "gram":
                assert max(got) <= 3                      # bf16 path: fp16 Gram-space limit
                assert e.dense_flops == pytest.approx(flop_model.dense_flops(r, c, "gram", got), rel=1e-12)
    finally:
        B.muon_destroy(mctx)


def test_auto_schedule_examples(hctx):
    """Long rectangular shapes take the fewest segments, square ones plain NS."""
    mctx = B.muon_init(-1, B.MUON_FLAG_MODEL_ONLY)
    try:
        e = plan(mctx, [(2560, 9728), (2048, 2048)], mode="auto_schedule")
        assert (e[0].mode, tuple(e[0].segments[:e[0].n_segments])) == (B.MUON_NS_GRAM, (3, 2))
        assert (e[1].mode, tuple(e[1].segments[:e[1].n_segments])) == (B.MUON_NS_PLAIN, (5,))
        e = plan(mctx, [(2560, 9728)], mode="auto_schedule", segments=(4, 4, 4))
        assert tuple(e[0].segments[:e[0].n_segments]) == (3, 3, 3, 3)
        e = plan(mctx, [(2560, 9728)], mode="auto_schedule", segments=(4, 4, 4), ns_dtype="f32",
                 g_dtype="f32", m_dtype="f32")
        assert tuple(e[0].segments[:e[0].n_segments]) == (12,)
    finally:
        B.muon_destroy(mctx)


# ---------------------------------------------------------------- AdamW companion

def test_adamw_defaults_and_validation(hctx):
    hp = B.make_adamw_hparams()
    assert (hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.step) == pytest.approx(
        (1e-3, 0.9, 0.999, 1e-8, 0.01, 1))
    assert (hp.w_dtype, hp.g_dtype) == (B.MUON_F32, B.MUON_BF16)
    P = FAKE
    good = [(P, P, P, P, 1000), (0, 0, 0, 0, 0)]           # an empty tensor may hold nulls
    f = B._lib.muon_adamw_step
    arr = B.adamw_tensor_list(good)
    assert f(hctx, arr, 2, ctypes.byref(hp), None) == B.MUON_ERR_DEVICE   # valid; host-only ctx
    assert f(hctx, arr, 0, ctypes.byref(hp), None) == B.MUON_OK
    assert f(None, arr, 2, ctypes.byref(hp), None) == B.MUON_ERR_ARG
    assert f(hctx, None, 2, ctypes.byref(hp), None) == B.MUON_ERR_ARG
    assert f(hctx, arr, -1, ctypes.byref(hp), None) == B.MUON_ERR_ARG
    assert f(hctx, arr, 2, None, None) == B.MUON_ERR_ARG
    for bad in [[(P, P, P, P, -1)], [(P, 0, P, P, 10)], [(P, P, P, 0, 10)], [(0, P, P, P, 10)]]:
        assert f(hctx, B.adamw_tensor_list(bad), 1, ctypes.byref(hp), None) == B.MUON_ERR_ARG, bad
    for kw in [dict(beta1=1.0), dict(beta2=-0.1), dict(eps=-1e-8), dict(lr=float("nan")), dict(step=0),
               dict(weight_decay=float("inf")), dict(w_dtype=3), dict(g_dtype=-1)]:
        assert f(hctx, arr, 2, ctypes.byref(B.make_adamw_hparams(**kw)), None) == B.MUON_ERR_ARG, kw



def test_auto_schedule_workspace_covers_both_forms(hctx):
    """The automatic schedule may run plain NS before a shape's tiles are measured and Gram
    NS after: its workspace holds the Gram path's buffers whatever the plan, so a size
    taken once stays valid for every later step."""
    shapes = [(2048, 2048), (2560, 9728), (64, 256)]
    mats = [(0, 0, 0, r, c) for r, c in shapes]
    auto = B.muon_workspace_size(hctx, mats, B.make_hparams(mode="auto_schedule"))
    gram = B.muon_workspace_size(hctx, mats, B.make_hparams(mode="gram"))
    plain = B.muon_workspace_size(hctx, mats, B.make_hparams(mode="plain"))
    assert auto == gram > plain
    mctx = B.muon_init(-1, B.MUON_FLAG_MODEL_ONLY)
    try:
        e = plan(mctx, [(2048, 2048)], mode="auto_schedule")
        assert e[0].mode == B.MUON_NS_PLAIN            # plain for this shape, Gram-sized anyway
        assert B.muon_workspace_size(mctx, [(0, 0, 0, 2048, 2048)], B.make_hparams(mode="auto_schedule")) == \
            B.muon_workspace_size(mctx, [(0, 0, 0, 2048, 2048)], B.make_hparams(mode="gram"))
    finally:
        B.muon_destroy(mctx)


def test_binding_rejects_bad_tensors():
    """The binding hands tensors over as device pointers only when they are contiguous, on
    a GPU and in the hyper-parameters' storage dtypes; everything else raises before the
    library is called (checked here with host tensors, which can never be passed)."""
    import torch
    hp = B.make_hparams(w_dtype="f32", g_dtype="bf16", m_dtype="bf16")
    W = torch.zeros(4, 8)
    G = torch.zeros(4, 8, dtype=torch.bfloat16)
    M = torch.zeros(4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="not on a GPU"):
        B.matrix_list([(W, G, M)], hp)
    with pytest.raises(TypeError, match="dtype"):
        B.matrix_list([(W.to(torch.bfloat16), G, M)], hp)       # bf16 W where hp says f32
    with pytest.raises(TypeError, match="dtype"):
        B.matrix_list([(W, G.float(), M)], hp)
    with pytest.raises(ValueError, match="contiguous"):
        B.matrix_list([(torch.zeros(8, 4).t(), G, M)], hp)
    with pytest.raises(TypeError):
        B.matrix_list([(W, G, "M")], hp)
    ahp = B.make_adamw_hparams(w_dtype="f32", g_dtype="bf16")
    n = 16
    good = (torch.zeros(n), torch.zeros(n, dtype=torch.bfloat16), torch.zeros(n), torch.zeros(n))
    with pytest.raises(ValueError, match="not on a GPU"):
        B.adamw_tensor_list([good], ahp)
    with pytest.raises(TypeError, match="dtype"):
        B.adamw_tensor_list([(good[0], good[1], good[2].double(), good[3])], ahp)
    with pytest.raises(TypeError, match="dtype"):
        B.adamw_tensor_list([(good[0].to(torch.bfloat16),) + good[1:]], ahp)


def test_muon_update_takes_dtypes_from_tensors():
    """MuonUpdate reads the storage dtypes off the tensors and rejects a conflicting keyword
    or a mixed list before any device work."""
    import torch
    from matrix_orthogonalising_optimizer_muon_amd.optimizer import MuonUpdate
    W = torch.zeros(4, 8, dtype=torch.bfloat16)
    G = torch.zeros(4, 8, dtype=torch.bfloat16)
    M = torch.zeros(4, 8, dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="w_dtype"):
        MuonUpdate([(W, G, M)], device=0, w_dtype="f32")
    with pytest.raises(TypeError, match="mixed"):
        MuonUpdate([(W, G, M), (W.float(), G, M)], device=0)
    with pytest.raises(ValueError, match="not on a GPU"):    # dtypes agree; host tensors
        MuonUpdate([(W, G, M)], device=0)


def test_debug_stage_validation_on_host(hctx):
    """muon_debug_stage validates its arguments before touching a device: a host-only
    context gets MUON_ERR_DEVICE only for a valid call."""
    m = B.muon_matrix(8, 16, 24, 64, 100)      # non-null host-side stand-ins, never dereferenced
    hp = B.make_hparams()
    f = ctypes.c_float()
    assert B._lib.muon_debug_stage(hctx, 7, ctypes.byref(m), ctypes.byref(hp), None, ctypes.c_void_p(64),
                                   None, ctypes.byref(f), ctypes.c_void_p(256), 4096, None) == B.MUON_ERR_ARG
    assert B._lib.muon_debug_stage(hctx, 0, ctypes.byref(m), ctypes.byref(hp), None, ctypes.c_void_p(64),
                                   None, ctypes.byref(f), ctypes.c_void_p(256), 300, None) == B.MUON_ERR_WORKSPACE
    assert B._lib.muon_debug_stage(hctx, 0, ctypes.byref(m), ctypes.byref(hp), None, ctypes.c_void_p(64),
                                   None, ctypes.byref(f), ctypes.c_void_p(256), 4096, None) == B.MUON_ERR_DEVICE
    bad = B.make_hparams(momentum=2.0)
    assert B._lib.muon_debug_stage(hctx, 0, ctypes.byref(m), ctypes.byref(bad), None, ctypes.c_void_p(64),
                                   None, ctypes.byref(f), ctypes.c_void_p(256), 4096, None) == B.MUON_ERR_ARG


def test_plan_huge_operands_use_staged_tiles(hctx):
    """The direct-load kernels address a matrix's operands with 32-bit offsets: a shape whose
    padded iterate exceeds 4 GiB (32768 x 65600 fp16) is planned on register-staged tiles
    (ids 0-3); 32768 x 65472 (just under 2^32 bytes) keeps the direct-load ones."""
    staged = {0, 1, 2, 3}
    big, = plan(hctx, [(32768, 65600)], mode="gram")
    assert big.tile_sym in staged and big.tile_apply in staged
    ok, = plan(hctx, [(32768, 65472)], mode="gram")
    assert ok.tile_apply not in staged
