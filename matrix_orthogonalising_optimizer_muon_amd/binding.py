"""ctypes binding of ``libmuon_amd.so`` (the C ABI declared in ``include/muon.h``).

Argument marshalling only: the functions carry the C names and hand plain pointers,
sizes and structs to the library, where every step of the update runs in HIP kernels.
There is no fallback: if the library is missing this module raises on import.

torch is imported first so that the library binds to the HIP runtime torch already
loaded (same SONAME); device buffers and streams then come from torch tensors and
``torch.cuda.Stream`` objects.
"""

from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the process's HIP runtime before the library)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MUON_AMD_LIB", os.path.join(_HERE, "libmuon_amd.so"))

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libmuon_amd.so not found at {LIB_PATH}: build it first "
        "(python -m matrix_orthogonalising_optimizer_muon_amd.build)")

_lib = ctypes.CDLL(LIB_PATH)

# ---- constants (mirror include/muon.h) ----
MUON_OK = 0
MUON_ERR_ARG = -1
MUON_ERR_WORKSPACE = -2
MUON_ERR_DEVICE = -3
MUON_ERR_HIP = -4
MUON_ERR_UNSUPPORTED = -5
MUON_F32 = 0
MUON_BF16 = 1
MUON_NS_AUTO = 0
MUON_NS_PLAIN = 1
MUON_NS_GRAM = 2
MUON_NS_AUTO_SCHEDULE = 3
MUON_MAX_SEGMENTS = 8
MUON_FLAG_MODEL_ONLY = 1
MUON_FLAG_PROFILE = 2
MUON_FLAG_STAGED_ONLY = 4
MUON_FLAG_ONE_STREAM = 8

DTYPES = {"f32": MUON_F32, "bf16": MUON_BF16}
MODES = {"auto": MUON_NS_AUTO, "plain": MUON_NS_PLAIN, "gram": MUON_NS_GRAM,
         "auto_schedule": MUON_NS_AUTO_SCHEDULE}


class muon_matrix(ctypes.Structure):
    _fields_ = [("W", ctypes.c_void_p), ("G", ctypes.c_void_p), ("M", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


class muon_hparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("momentum", ctypes.c_float),
                ("weight_decay", ctypes.c_float), ("eps", ctypes.c_float),
                ("nesterov", ctypes.c_int32), ("a", ctypes.c_float), ("b", ctypes.c_float),
                ("c", ctypes.c_float), ("n_segments", ctypes.c_int32),
                ("segments", ctypes.c_int32 * MUON_MAX_SEGMENTS), ("mode", ctypes.c_int32),
                ("w_dtype", ctypes.c_int32), ("g_dtype", ctypes.c_int32),
                ("m_dtype", ctypes.c_int32), ("ns_dtype", ctypes.c_int32)]


class muon_plan_entry(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("n_segments", ctypes.c_int32),
                ("segments", ctypes.c_int32 * MUON_MAX_SEGMENTS), ("transposed", ctypes.c_int32),
                ("m", ctypes.c_int64), ("n", ctypes.c_int64), ("group", ctypes.c_int32),
                ("tile_sym", ctypes.c_int32), ("tile_apply", ctypes.c_int32),
                ("single_wg", ctypes.c_int32), ("dense_flops", ctypes.c_double),
                ("kernel_flops", ctypes.c_double)]


class muon_profile_entry(ctypes.Structure):
    _fields_ = [("stage", ctypes.c_char * 32), ("m", ctypes.c_int64), ("n", ctypes.c_int64),
                ("count", ctypes.c_int32), ("launches", ctypes.c_int32),
                ("tile", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("total_ms", ctypes.c_double), ("flops", ctypes.c_double),
                ("bytes", ctypes.c_double)]


class muon_adamw_tensor(ctypes.Structure):
    _fields_ = [("W", ctypes.c_void_p), ("G", ctypes.c_void_p), ("m", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("numel", ctypes.c_int64)]


class muon_adamw_hparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float), ("step", ctypes.c_int32),
                ("w_dtype", ctypes.c_int32), ("g_dtype", ctypes.c_int32)]


MUON_MAX_COST_POINTS = 16
MUON_MAX_PLAN_RANKS = 4096
MUON_PLAN_GREEDY = 1
MUON_PLAN_DEFAULT_NODES = 2000000


class muon_shape_cost(ctypes.Structure):
    _fields_ = [("n_points", ctypes.c_int32), ("batch", ctypes.c_int32 * MUON_MAX_COST_POINTS),
                ("ms", ctypes.c_double * MUON_MAX_COST_POINTS)]


_P = ctypes.c_void_p
_lib.muon_owner_plan.argtypes = [ctypes.POINTER(ctypes.c_int32), ctypes.c_int, ctypes.POINTER(muon_shape_cost),
                                 ctypes.c_int, ctypes.c_int, ctypes.c_uint32, ctypes.c_int64,
                                 ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_double),
                                 ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32)]
_lib.muon_owner_plan.restype = ctypes.c_int
_lib.muon_hparams_default.argtypes = [ctypes.POINTER(muon_hparams)]
_lib.muon_hparams_default.restype = None
_lib.muon_init.argtypes = [ctypes.POINTER(_P), ctypes.c_int, ctypes.c_uint32]
_lib.muon_init.restype = ctypes.c_int
_lib.muon_workspace_size.argtypes = [_P, ctypes.POINTER(muon_matrix), ctypes.c_int,
                                     ctypes.POINTER(muon_hparams), ctypes.POINTER(ctypes.c_size_t)]
_lib.muon_workspace_size.restype = ctypes.c_int
_lib.muon_step.argtypes = [_P, ctypes.POINTER(muon_matrix), ctypes.c_int,
                           ctypes.POINTER(muon_hparams), _P, ctypes.c_size_t, _P]
_lib.muon_step.restype = ctypes.c_int
_lib.muon_prepare.argtypes = [_P, ctypes.POINTER(muon_matrix), ctypes.c_int, ctypes.POINTER(muon_hparams),
                              _P, ctypes.c_size_t, _P, ctypes.POINTER(ctypes.c_double)]
_lib.muon_prepare.restype = ctypes.c_int
_lib.muon_step_static.argtypes = [_P, ctypes.POINTER(muon_matrix), ctypes.c_int,
                                  ctypes.POINTER(muon_hparams), _P]
_lib.muon_step_static.restype = ctypes.c_int
MUON_STATIC_SCRATCH_BYTES = 256 << 20
_lib.muon_plan_info.argtypes = [_P, ctypes.POINTER(muon_matrix), ctypes.c_int,
                                ctypes.POINTER(muon_hparams), ctypes.c_int,
                                ctypes.POINTER(muon_plan_entry)]
_lib.muon_plan_info.restype = ctypes.c_int
_lib.muon_debug_gemm.argtypes = [_P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                 ctypes.c_int64, ctypes.c_int64, _P, _P, _P, _P, _P, ctypes.c_float,
                                 ctypes.c_float, ctypes.c_float, ctypes.c_float, _P]
_lib.muon_debug_gemm.restype = ctypes.c_int
_lib.muon_debug_stage.argtypes = [_P, ctypes.c_int, ctypes.POINTER(muon_matrix), ctypes.POINTER(muon_hparams),
                                  _P, _P, _P, ctypes.POINTER(ctypes.c_float), _P, ctypes.c_size_t, _P]
_lib.muon_debug_stage.restype = ctypes.c_int
MUON_STAGE_NORM, MUON_STAGE_ITERATE, MUON_STAGE_UPDATE = 0, 1, 2
_lib.muon_profile_read.argtypes = [_P, ctypes.POINTER(muon_profile_entry), ctypes.c_int,
                                   ctypes.POINTER(ctypes.c_int)]
_lib.muon_profile_read.restype = ctypes.c_int
_lib.muon_tune_save.argtypes = [_P, ctypes.c_char_p]
_lib.muon_tune_save.restype = ctypes.c_int
_lib.muon_tune_load.argtypes = [_P, ctypes.c_char_p, ctypes.POINTER(ctypes.c_int)]
_lib.muon_tune_load.restype = ctypes.c_int
_lib.muon_adamw_hparams_default.argtypes = [ctypes.POINTER(muon_adamw_hparams)]
_lib.muon_adamw_hparams_default.restype = None
_lib.muon_adamw_step.argtypes = [_P, ctypes.POINTER(muon_adamw_tensor), ctypes.c_int,
                                 ctypes.POINTER(muon_adamw_hparams), _P]
_lib.muon_adamw_step.restype = ctypes.c_int
_lib.muon_destroy.argtypes = [_P]
_lib.muon_destroy.restype = ctypes.c_int
_lib.muon_status_str.argtypes = [ctypes.c_int]
_lib.muon_status_str.restype = ctypes.c_char_p


class MuonError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {muon_status_str(status)}")
        self.status = status


def check(status: int, where: str = "muon") -> None:
    if status != MUON_OK:
        raise MuonError(status, where)


def muon_status_str(status: int) -> str:
    return _lib.muon_status_str(int(status)).decode()


def muon_hparams_default() -> muon_hparams:
    hp = muon_hparams()
    _lib.muon_hparams_default(ctypes.byref(hp))
    return hp


def make_hparams(*, lr=None, momentum=None, weight_decay=None, eps=None, nesterov=None,
                 coeffs=None, segments=None, mode=None, w_dtype=None, g_dtype=None,
                 m_dtype=None, ns_dtype=None) -> muon_hparams:
    """Defaults from the library, with the given fields replaced (names as in muon.h)."""
    hp = muon_hparams_default()
    if lr is not None: hp.lr = lr
    if momentum is not None: hp.momentum = momentum
    if weight_decay is not None: hp.weight_decay = weight_decay
    if eps is not None: hp.eps = eps
    if nesterov is not None: hp.nesterov = int(nesterov)
    if coeffs is not None: hp.a, hp.b, hp.c = coeffs
    if segments is not None:
        segs = list(segments)
        hp.n_segments = len(segs)
        for i in range(MUON_MAX_SEGMENTS):
            hp.segments[i] = segs[i] if i < len(segs) else 0
    if mode is not None: hp.mode = MODES.get(mode, mode)
    if w_dtype is not None: hp.w_dtype = DTYPES.get(w_dtype, w_dtype)
    if g_dtype is not None: hp.g_dtype = DTYPES.get(g_dtype, g_dtype)
    if m_dtype is not None: hp.m_dtype = DTYPES.get(m_dtype, m_dtype)
    if ns_dtype is not None: hp.ns_dtype = DTYPES.get(ns_dtype, ns_dtype)
    return hp


TORCH_DTYPES = {MUON_F32: torch.float32, MUON_BF16: torch.bfloat16}


def _check_dtype(x, name: str, dtype_code: int | None) -> None:
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(x).__name__}")
    if dtype_code is not None and x.dtype != TORCH_DTYPES[dtype_code]:
        raise TypeError(f"{name} has dtype {x.dtype}, the hyper-parameters say {TORCH_DTYPES[dtype_code]}")


def _check_device_tensor(x, name: str, dtype_code: int | None, device: int | None) -> None:
    """A tensor handed to the library as a device pointer: contiguous, on a GPU (the
    context's device when given) and in the storage dtype the hyper-parameters name."""
    _check_dtype(x, name, dtype_code)
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if x.device.type != "cuda":
        raise ValueError(f"{name} is on {x.device}, not on a GPU")
    if device is not None and x.device.index != device:
        raise ValueError(f"{name} is on {x.device}, the context is on cuda:{device}")


def matrix_list(mats, hp: muon_hparams | None = None, device: int | None = None) -> ctypes.Array:
    """Build a ``muon_matrix[]`` from (W, G, M) torch tensors or (W, G, M, rows, cols)
    tuples of raw pointers. Tensors must be 2-D, contiguous, of one shape and on a GPU
    (``device`` when given); with ``hp`` their dtypes must be ``hp``'s w/g/m dtypes."""
    arr = (muon_matrix * max(1, len(mats)))()
    for i, t in enumerate(mats):
        if len(t) == 3:
            W, G, M = t
            codes = (hp.w_dtype, hp.g_dtype, hp.m_dtype) if hp is not None else (None, None, None)
            for x, name, code in zip((W, G, M), ("W", "G", "M"), codes):
                _check_dtype(x, f"matrix {i} {name}", code)
            for x, name, code in zip((W, G, M), ("W", "G", "M"), codes):
                _check_device_tensor(x, f"matrix {i} {name}", code, device)
                if x.dim() != 2:
                    raise ValueError(f"matrix {i} {name} must be 2-D")
            if not (W.shape == G.shape == M.shape):
                raise ValueError(f"matrix {i}: W, G, M shapes differ")
            if len({W.device, G.device, M.device}) != 1:
                raise ValueError(f"matrix {i}: W, G, M on different devices")
            arr[i] = muon_matrix(W.data_ptr(), G.data_ptr(), M.data_ptr(), W.shape[0], W.shape[1])
        else:
            W, G, M, r, c = t
            arr[i] = muon_matrix(W, G, M, r, c)
    return arr


def muon_init(device: int = 0, flags: int = 0) -> ctypes.c_void_p:
    ctx = ctypes.c_void_p()
    check(_lib.muon_init(ctypes.byref(ctx), int(device), int(flags)), "muon_init")
    return ctx


def muon_workspace_size(ctx, mats, hp: muon_hparams) -> int:
    arr = mats if isinstance(mats, ctypes.Array) else matrix_list(mats)
    n = len(mats)
    out = ctypes.c_size_t()
    check(_lib.muon_workspace_size(ctx, arr, n, ctypes.byref(hp), ctypes.byref(out)),
          "muon_workspace_size")
    return int(out.value)


def muon_step(ctx, mats, hp: muon_hparams, workspace_ptr: int, workspace_bytes: int,
              stream_ptr: int | None = None, count: int | None = None) -> int:
    """Enqueue one update; returns the status (use ``check`` to raise)."""
    arr = mats if isinstance(mats, ctypes.Array) else matrix_list(mats, hp)
    n = len(mats) if count is None else count
    if stream_ptr is None:
        stream_ptr = torch.cuda.current_stream().cuda_stream
    return _lib.muon_step(ctx, arr, n, ctypes.byref(hp), ctypes.c_void_p(workspace_ptr),
                          ctypes.c_size_t(workspace_bytes), ctypes.c_void_p(stream_ptr))


def muon_prepare(ctx, mats, hp: muon_hparams, workspace_ptr: int, workspace_bytes: int,
                 stream_ptr: int | None = None, count: int | None = None) -> float:
    """Measure the tiles of every stage of the list ahead of the first step (synthetic data in
    the workspace; W, G, M untouched) and return the time of one synthetic run in ms."""
    arr = mats if isinstance(mats, ctypes.Array) else matrix_list(mats)
    n = len(mats) if count is None else count
    if stream_ptr is None:
        stream_ptr = torch.cuda.current_stream().cuda_stream
    ms = ctypes.c_double()
    check(_lib.muon_prepare(ctx, arr, n, ctypes.byref(hp), ctypes.c_void_p(workspace_ptr),
                            ctypes.c_size_t(workspace_bytes), ctypes.c_void_p(stream_ptr), ctypes.byref(ms)),
          "muon_prepare")
    return ms.value


def muon_step_static(ctx, mats, hp: muon_hparams, stream_ptr: int | None = None,
                     count: int | None = None) -> int:
    """Enqueue one update over the library's static scratch (no workspace); returns the
    status (use ``check`` to raise)."""
    arr = mats if isinstance(mats, ctypes.Array) else matrix_list(mats, hp)
    n = len(mats) if count is None else count
    if stream_ptr is None:
        stream_ptr = torch.cuda.current_stream().cuda_stream
    return _lib.muon_step_static(ctx, arr, n, ctypes.byref(hp), ctypes.c_void_p(stream_ptr))


def muon_plan_info(ctx, mats, hp: muon_hparams, index: int) -> muon_plan_entry:
    arr = mats if isinstance(mats, ctypes.Array) else matrix_list(mats)
    out = muon_plan_entry()
    check(_lib.muon_plan_info(ctx, arr, len(mats), ctypes.byref(hp), int(index), ctypes.byref(out)),
          "muon_plan_info")
    return out


def muon_debug_gemm(ctx, kind, ns_dtype, tile, M, N, K, A, B, E, C, C2=None, alpha=1.0,
                    beta=0.0, gamma=0.0, oscale=1.0, stream_ptr=None) -> int:
    if stream_ptr is None:
        stream_ptr = torch.cuda.current_stream().cuda_stream
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    return _lib.muon_debug_gemm(ctx, int(kind), DTYPES.get(ns_dtype, ns_dtype), int(tile), M, N, K,
                                ptr(A), ptr(B), ptr(E), ptr(C), ptr(C2), alpha, beta, gamma, oscale,
                                ctypes.c_void_p(stream_ptr))


def muon_debug_stage(ctx, stage: int, mat, hp: muon_hparams, inp, out, out2, workspace,
                     stream_ptr=None) -> tuple:
    """One stage on one matrix (test-only). ``mat`` is (W, G, M) tensors (None allowed where
    the stage does not use them) plus rows, cols; the rest are tensors or None. Returns
    (status, scale)."""
    W, G, M, rows, cols = mat
    ptr = lambda t: None if t is None else t.data_ptr()
    m = muon_matrix(ptr(W), ptr(G), ptr(M), rows, cols)
    sc = ctypes.c_float()
    if stream_ptr is None:
        stream_ptr = torch.cuda.current_stream().cuda_stream
    rc = _lib.muon_debug_stage(ctx, int(stage), ctypes.byref(m), ctypes.byref(hp), ptr(inp), ptr(out), ptr(out2),
                               ctypes.byref(sc), ptr(workspace), workspace.numel() * workspace.element_size(),
                               ctypes.c_void_p(stream_ptr))
    return rc, sc.value


def muon_profile_read(ctx, capacity: int = 256) -> list:
    """Aggregated per-stage launch timings since the last read, as dicts."""
    buf = (muon_profile_entry * capacity)()
    n = ctypes.c_int()
    check(_lib.muon_profile_read(ctx, buf, capacity, ctypes.byref(n)), "muon_profile_read")
    return [dict(stage=e.stage.decode(), m=e.m, n=e.n, count=e.count, launches=e.launches,
                 tile=e.tile, total_ms=e.total_ms, flops=e.flops, bytes=e.bytes) for e in buf[:n.value]]


def muon_tune_save(ctx, path: str) -> None:
    check(_lib.muon_tune_save(ctx, os.fsencode(path)), "muon_tune_save")


def muon_tune_load(ctx, path: str) -> int:
    n = ctypes.c_int()
    check(_lib.muon_tune_load(ctx, os.fsencode(path), ctypes.byref(n)), "muon_tune_load")
    return n.value


def make_adamw_hparams(**kw) -> muon_adamw_hparams:
    """AdamW defaults from the library, with the given fields replaced (names as in muon.h;
    w_dtype / g_dtype accept "f32" / "bf16")."""
    hp = muon_adamw_hparams()
    _lib.muon_adamw_hparams_default(ctypes.byref(hp))
    for k, v in kw.items():
        if k in ("w_dtype", "g_dtype"):
            v = DTYPES.get(v, v)
        setattr(hp, k, v)
    return hp


def adamw_tensor_list(tensors, hp: muon_adamw_hparams | None = None, device: int | None = None) -> ctypes.Array:
    """Build a ``muon_adamw_tensor[]`` from (W, G, m, v) torch tensors (numel from W) or from
    (W, G, m, v, numel) raw pointer tuples. Tensors must be contiguous, on a GPU (``device``
    when given) and of one element count; m and v are fp32, and with ``hp`` W and G must be
    in its w/g dtypes."""
    arr = (muon_adamw_tensor * max(len(tensors), 1))()
    for i, t in enumerate(tensors):
        if len(t) == 5:
            arr[i] = muon_adamw_tensor(t[0], t[1], t[2], t[3], int(t[4]))
        else:
            W, G, m, v = t
            codes = (hp.w_dtype, hp.g_dtype) if hp is not None else (None, None)
            for x, name, code in ((W, "W", codes[0]), (G, "G", codes[1]), (m, "m", MUON_F32), (v, "v", MUON_F32)):
                _check_dtype(x, f"tensor {i} {name}", code)
            _check_device_tensor(W, f"tensor {i} W", codes[0], device)
            _check_device_tensor(G, f"tensor {i} G", codes[1], device)
            _check_device_tensor(m, f"tensor {i} m", MUON_F32, device)
            _check_device_tensor(v, f"tensor {i} v", MUON_F32, device)
            if not (W.numel() == G.numel() == m.numel() == v.numel()):
                raise ValueError(f"tensor {i}: W, G, m, v element counts differ")
            if len({W.device, G.device, m.device, v.device}) != 1:
                raise ValueError(f"tensor {i}: W, G, m, v on different devices")
            arr[i] = muon_adamw_tensor(W.data_ptr(), G.data_ptr(), m.data_ptr(), v.data_ptr(), W.numel())
    return arr


def muon_adamw_step(ctx, tensors, hp: muon_adamw_hparams, stream_ptr=None, count=None) -> int:
    arr = tensors if isinstance(tensors, ctypes.Array) else adamw_tensor_list(tensors, hp)
    n = len(tensors) if count is None else count
    if stream_ptr is None:
        stream_ptr = torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    return _lib.muon_adamw_step(ctx, arr, n, ctypes.byref(hp), stream_ptr)


def shape_cost(points) -> muon_shape_cost:
    """A ``muon_shape_cost`` from [(batch, ms), ...] measured points."""
    c = muon_shape_cost()
    c.n_points = len(points)
    for i, (b, ms) in enumerate(points):
        c.batch[i] = int(b)
        c.ms[i] = float(ms)
    return c


def muon_owner_plan(shape_of, costs, ranks: int, greedy: bool = False, max_nodes: int = 0) -> dict:
    """Owner map of matrices (shape ids ``shape_of``) over ``ranks`` ranks from per-shape
    measured costs (a list of [(batch, ms), ...] or ``muon_shape_cost``). Returns a dict with
    ``owner`` (list), ``rank_ms`` (list), ``makespan_ms`` and ``optimal``."""
    n = len(shape_of)
    so = (ctypes.c_int32 * max(n, 1))(*shape_of)
    cs = (muon_shape_cost * max(len(costs), 1))(
        *[c if isinstance(c, muon_shape_cost) else shape_cost(c) for c in costs])
    owner = (ctypes.c_int32 * max(n, 1))()
    rank_ms = (ctypes.c_double * max(ranks, 1))()
    mk = ctypes.c_double()
    opt = ctypes.c_int32()
    check(_lib.muon_owner_plan(so, n, cs, len(costs), int(ranks), MUON_PLAN_GREEDY if greedy else 0,
                               int(max_nodes), owner, rank_ms, ctypes.byref(mk), ctypes.byref(opt)),
          "muon_owner_plan")
    return {"owner": list(owner[:n]), "rank_ms": list(rank_ms[:ranks]), "makespan_ms": mk.value,
            "optimal": bool(opt.value)}


def muon_destroy(ctx) -> int:
    return _lib.muon_destroy(ctx)


def exported_symbols() -> list:
    """Names of the C entry points this binding resolved (each must exist in the .so)."""
    return [n for n in ("muon_hparams_default", "muon_init", "muon_workspace_size", "muon_step", "muon_step_static", "muon_prepare",
                        "muon_plan_info", "muon_debug_gemm", "muon_debug_stage", "muon_profile_read", "muon_tune_save",
                        "muon_tune_load", "muon_adamw_hparams_default", "muon_adamw_step",
                        "muon_destroy", "muon_status_str", "muon_owner_plan")
            if hasattr(_lib, n)]
