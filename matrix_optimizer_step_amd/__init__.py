"""Python binding of libmatopt: the owner-local Muon step and the RMNP comparator
as hand-written HIP kernels for MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the library's
kernels.  torch supplies device memory (tensors, the workspace) and the current
stream; nothing here computes.  If ``libmatopt.so`` has not been built, every
entry point raises ``MatoptError`` -- there is no fallback.

Entry points mirror the C ABI (``include/matopt.h``):

* ``muon_step_batched(weights, grads, moms, mu, lr, ns_steps, coeffs, eps)``
* ``rmnp_step_batched(weights, grads, moms, mu, lr, eps)``
* ``ns_orthogonalize_batched(xs, out_dtype, ns_steps, coeffs, eps)``
* ``workspace_bytes(shapes, dtype)``, ``profile_enable``, ``profile_read``,
  ``counters``
"""
from __future__ import annotations

import collections
import ctypes
import os
import threading

import torch

__all__ = ["MatoptError", "lib", "workspace_bytes", "muon_step_batched",
           "muon_step_batched_wd", "muon_step_batched_noalloc", "rmnp_step_batched", "rmnp_colcut_partial_batched",
           "rmnp_colcut_apply_batched", "adamw_step_batched", "flat_views", "ns_orthogonalize_batched", "profile_enable",
           "profile_read", "profile_read_clock", "counters", "mfma_probe", "PROFILE_CLASSES", "COUNTERS",
           "LIB_PATH", "EXPORTS"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmatopt.so")

F32, BF16, BF16_SPLIT = 0, 1, 2
PROFILE_CLASSES = ("prep", "finalize", "gram", "poly", "apply", "scale_out", "rmnp",
                   "colcut_partial", "colcut_apply", "adamw", "bind")
COUNTERS = ("plan_builds", "device_allocs", "device_frees", "bind_launches")

# Defaults printed on the pages (blog post appendix).
NS_COEFFS = (3.4445, -4.7750, 2.0315)


class MatoptError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name}: {detail}")
        self.status = status
        self.name = name
        self.detail = detail


class _Vec(ctypes.Structure):
    _fields_ = [("p", ctypes.c_void_p), ("g", ctypes.c_void_p), ("m", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("n", ctypes.c_int64)]


class _Mat(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("g", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


_vp, _i32, _i64, _f32, _sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                              ctypes.c_float, ctypes.c_size_t)

# symbol -> (restype, argtypes); every function include/matopt.h declares
EXPORTS = {
    "matopt_workspace_bytes": (_sz, [ctypes.POINTER(_i64), ctypes.POINTER(_i64), _i32, _i32]),
    "muon_step_batched": (_i32, [ctypes.POINTER(_Mat), _i32, _i32, _f32, _f32, _i32, _f32,
                                 _f32, _f32, _f32, _vp, _sz, _vp]),
    "muon_step_batched_wd": (_i32, [ctypes.POINTER(_Mat), _i32, _i32, _f32, _f32, _f32, _i32,
                                    _f32, _f32, _f32, _f32, _vp, _sz, _vp]),
    "muon_step_batched_noalloc": (_i32, [ctypes.POINTER(_Mat), _i32, _i32, _f32, _f32, _i32,
                                         _f32, _f32, _f32, _f32, _vp]),
    "rmnp_step_batched": (_i32, [ctypes.POINTER(_Mat), _i32, _i32, _f32, _f32, _f32, _vp]),
    "adamw_step_batched": (_i32, [ctypes.POINTER(_Vec), _i32, _i32, _f32, _f32, _f32, _f32, _f32,
                                  _i32, _vp]),
    "rmnp_colcut_partial_batched": (_i32, [ctypes.POINTER(_Mat), _i32, _i32, _f32, _vp, _vp]),
    "rmnp_colcut_apply_batched": (_i32, [ctypes.POINTER(_Mat), _i32, _i32, _f32, _f32, _vp,
                                         ctypes.POINTER(_i64), _vp]),
    "ns_orthogonalize_batched": (_i32, [ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                        ctypes.POINTER(_i64), ctypes.POINTER(_i64), _i32,
                                        _i32, _i32, _i32, _f32, _f32, _f32, _f32, _vp, _sz,
                                        _vp]),
    "matopt_status_string": (ctypes.c_char_p, [_i32]),
    "matopt_last_error_detail": (ctypes.c_char_p, []),
    "matopt_version": (_i32, []),
    "matopt_profile_enable": (_i32, [_i32]),
    "matopt_profile_read": (_i32, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64)]),
    "matopt_counters": (_i32, [ctypes.POINTER(_i64), _i32]),
    "matopt_profile_read_clock": (_i32, [ctypes.POINTER(ctypes.c_double)]),
    "matopt_mfma_probe": (_i32, [_i32, _i32, _vp, _vp, _i32, _i32, _vp, _vp]),
}

_lib = None
_lock = threading.Lock()


def lib():
    """The loaded ``libmatopt.so`` (ctypes), with argument types set."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise MatoptError(-1, "MATOPT_NOT_BUILT",
                                  f"{LIB_PATH} is missing; run __graft_entry__.build() or "
                                  "python -m matrix_optimizer_step_amd.build")
            L = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in EXPORTS.items():
                f = getattr(L, name)
                f.restype = res
                f.argtypes = args
            _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        L = lib()
        name = L.matopt_status_string(status).decode()
        detail = L.matopt_last_error_detail().decode()
        raise MatoptError(status, name, detail)


def _dt(dtype, precision: str = "default") -> int:
    """Library dtype code of a tensor dtype; precision="split" selects the
    split-precision Newton-Schulz path for bfloat16 (MATOPT_BF16_SPLIT)."""
    if precision not in ("default", "split"):
        raise ValueError(f"precision must be 'default' or 'split', got {precision!r}")
    if dtype == torch.bfloat16:
        return BF16_SPLIT if precision == "split" else BF16
    if dtype == torch.float32:
        if precision == "split":
            raise ValueError("precision='split' applies to bfloat16 tensors only")
        return F32
    raise TypeError(f"unsupported dtype {dtype} (bfloat16 or float32)")


def _check_dev(t, what: str, device=None):
    """A CUDA (HIP) tensor, on ``device`` when given: a host pointer must never
    reach a kernel."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{what} must be a CUDA (HIP) tensor")
    if device is not None and t.device != torch.device(device):
        raise TypeError(f"{what} is on {t.device}, expected {device}")


def _check_mat(t: torch.Tensor, what: str, dtype=None):
    _check_dev(t, what)
    if t.dim() != 2:
        raise ValueError(f"{what} must be 2-D, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what} has dtype {t.dtype}, expected {dtype}")


def _stream_ptr(device, stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return int(s.cuda_stream)


def workspace_bytes(shapes, dtype, precision="default") -> int:
    n = len(shapes)
    rows = (_i64 * max(n, 1))(*[int(r) for r, _ in shapes])
    cols = (_i64 * max(n, 1))(*[int(c) for _, c in shapes])
    return int(lib().matopt_workspace_bytes(rows, cols, n, _dt(dtype, precision)))


# Workspaces allocated by the binding, most recently used last; at most
# _WS_CACHE_CAP of them are kept (an evicted one goes back to torch's caching
# allocator once the last call that used it is no longer referenced).
_WS_CACHE_CAP = 4
_ws_cache: "collections.OrderedDict" = collections.OrderedDict()


def _workspace(device, dtype, shapes, workspace, precision="default"):
    need = workspace_bytes(shapes, dtype, precision)
    if workspace is not None:
        _check_dev(workspace, "workspace", device)
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        if workspace.numel() * workspace.element_size() < need:
            raise ValueError(f"workspace too small: need {need} bytes")
        return workspace.data_ptr(), workspace.numel() * workspace.element_size(), workspace
    key = (str(device), _dt(dtype, precision), tuple(shapes))
    ws = _ws_cache.pop(key, None)
    if ws is None:
        ws = torch.empty(need + 256, dtype=torch.uint8, device=device)
    _ws_cache[key] = ws
    while len(_ws_cache) > _WS_CACHE_CAP:
        _ws_cache.popitem(last=False)
    base = ws.data_ptr()
    off = (-base) % 256
    return base + off, need, ws


def clear_workspace_cache():
    _ws_cache.clear()


def _mats(weights, grads, moms):
    if not (len(weights) == len(grads) == len(moms)):
        raise ValueError("weights, grads and moms must have the same length")
    n = len(weights)
    arr = (_Mat * max(n, 1))()
    dtype = weights[0].dtype if n else torch.bfloat16
    for i, (w, g, v) in enumerate(zip(weights, grads, moms)):
        _check_mat(w, f"weights[{i}]", dtype)
        _check_mat(g, f"grads[{i}]", dtype)
        _check_mat(v, f"moms[{i}]", dtype)
        if not (w.shape == g.shape == v.shape):
            raise ValueError(f"matrix {i}: W, G, V shapes differ")
        arr[i] = _Mat(w.data_ptr(), g.data_ptr(), v.data_ptr(), w.shape[0], w.shape[1])
    return arr, n, dtype


def muon_step_batched(weights, grads, moms, mu=0.95, lr=0.02, ns_steps=5,
                      coeffs=NS_COEFFS, eps=1e-7, workspace=None, stream=None,
                      precision="default"):
    """One Muon step on every (W, G, V) triple; W and V are updated in place.
    precision="split" (bfloat16 only): the split-precision iterate."""
    arr, n, dtype = _mats(weights, grads, moms)
    if n == 0:
        return
    device = weights[0].device
    shapes = [tuple(w.shape) for w in weights]
    wp, wb, _keep = _workspace(device, dtype, shapes, workspace, precision)
    a, b, c = coeffs
    _check(lib().muon_step_batched(arr, n, _dt(dtype, precision), mu, lr, ns_steps, a, b, c,
                                   eps, wp, wb, _stream_ptr(device, stream)))


def muon_step_batched_wd(weights, grads, moms, mu=0.5, lr=1e-3, wd=1e-2, ns_steps=2,
                         coeffs=NS_COEFFS, eps=1e-7, workspace=None, stream=None,
                         precision="default"):
    """The Muon step with decoupled weight decay, W <- W - lr*(wd*W + s*O); the
    defaults are the MatrixFSDP paper's training configuration (section 5.1)."""
    arr, n, dtype = _mats(weights, grads, moms)
    if n == 0:
        return
    device = weights[0].device
    shapes = [tuple(w.shape) for w in weights]
    wp, wb, _keep = _workspace(device, dtype, shapes, workspace, precision)
    a, b, c = coeffs
    _check(lib().muon_step_batched_wd(arr, n, _dt(dtype, precision), mu, lr, wd, ns_steps, a, b,
                                      c, eps, wp, wb, _stream_ptr(device, stream)))


def muon_step_batched_noalloc(weights, grads, moms, mu=0.95, lr=0.02, ns_steps=5,
                              coeffs=NS_COEFFS, eps=1e-7, stream=None, precision="default"):
    """The Muon step without a workspace and without any allocation: the
    library's per-GPU device scratch array (MATOPT_NOALLOC_SCRATCH_BYTES) holds
    workspace and tables; shape lists that do not fit raise MatoptError
    (MATOPT_ERR_WORKSPACE).  Nothing is allocated here either."""
    arr, n, dtype = _mats(weights, grads, moms)
    if n == 0:
        return
    device = weights[0].device
    a, b, c = coeffs
    _check(lib().muon_step_batched_noalloc(arr, n, _dt(dtype, precision), mu, lr, ns_steps, a, b,
                                           c, eps, _stream_ptr(device, stream)))


def rmnp_step_batched(weights, grads, moms, mu=0.95, lr=0.02, eps=1e-12, stream=None):
    """One RMNP step on every (W, G, V) triple; W and V are updated in place."""
    arr, n, dtype = _mats(weights, grads, moms)
    if n == 0:
        return
    device = weights[0].device
    _check(lib().rmnp_step_batched(arr, n, _dt(dtype), mu, lr, eps,
                                   _stream_ptr(device, stream)))


def _colcut_mats(weights, moms, others, what):
    n = len(moms)
    if n == 0:
        return None, 0, None
    dtype = moms[0].dtype
    arr = (_Mat * n)()
    for i, v in enumerate(moms):
        _check_mat(v, f"moms[{i}]", dtype)
        o = others[i]
        _check_mat(o, f"{what}[{i}]", dtype)
        if o.shape != v.shape:
            raise ValueError(f"{what}[{i}] shape differs from moms[{i}]")
        w = o.data_ptr() if what == "weights" else None
        g = o.data_ptr() if what == "grads" else None
        arr[i] = _Mat(w, g, v.data_ptr(), v.shape[0], v.shape[1])
    return arr, n, dtype


def rmnp_colcut_partial_batched(grads, moms, rowsq=None, mu=0.95, stream=None):
    """Column-cut RMNP, first local half: V <- mu V + G on each column slice and
    the float32 row sums of squares of the stored slices, concatenated over the
    matrices into ``rowsq`` (allocated if not given).  Returns ``rowsq``; sum it
    over the ranks holding the other slices before the apply half."""
    arr, n, dtype = _colcut_mats(None, moms, grads, "grads")
    if n == 0:
        return rowsq
    device = moms[0].device
    total = sum(v.shape[0] for v in moms)
    if rowsq is None:
        rowsq = torch.empty(total, dtype=torch.float32, device=device)
    _check_dev(rowsq, "rowsq", device)
    if rowsq.dtype != torch.float32 or rowsq.numel() < total or not rowsq.is_contiguous():
        raise ValueError("rowsq must be a contiguous float32 tensor of sum(rows) entries")
    _check(lib().rmnp_colcut_partial_batched(arr, n, _dt(dtype), mu, rowsq.data_ptr(),
                                             _stream_ptr(device, stream)))
    return rowsq


def rmnp_colcut_apply_batched(weights, moms, rowsq, full_cols=None, lr=0.02, eps=1e-7,
                              stream=None):
    """Column-cut RMNP, second local half: W <- W - lr s V / max(sqrt(rowsq), eps)
    on each column slice, with s from the whole matrix's shape (rows x
    full_cols[i]; default: the slice's own width)."""
    arr, n, dtype = _colcut_mats(weights, moms, weights, "weights")
    if n == 0:
        return
    device = moms[0].device
    total = sum(v.shape[0] for v in moms)
    _check_dev(rowsq, "rowsq", device)
    if rowsq.dtype != torch.float32 or rowsq.numel() < total or not rowsq.is_contiguous():
        raise ValueError("rowsq must be a contiguous float32 tensor of sum(rows) entries")
    fc = None if full_cols is None else (_i64 * n)(*full_cols)
    _check(lib().rmnp_colcut_apply_batched(arr, n, _dt(dtype), lr, eps, rowsq.data_ptr(), fc,
                                           _stream_ptr(device, stream)))


def flat_views(flat: torch.Tensor, shapes):
    """Views of consecutive pieces of one contiguous 1-D tensor, one per shape:
    the layout that lets a whole non-2D tail go through adamw_step_batched as
    one tensor.  Keep the tail's parameters (and gradients, and moments) as
    such views -- e.g. ``param.data = view`` -- and pass the flat tensors: the
    kernel time is the same as for separate tensors, but the call marshals one
    tensor instead of hundreds (GPT-2 Large's 290-tensor tail: ~14 us of wall
    time instead of ~600 us)."""
    if flat.dim() != 1 or not flat.is_contiguous():
        raise ValueError("flat must be a contiguous 1-D tensor")
    sizes = []
    for shp in shapes:
        n = 1
        for d in shp:
            n *= int(d)
        sizes.append(n)
    if sum(sizes) > flat.numel():
        raise ValueError(f"the shapes need {sum(sizes)} elements, flat has {flat.numel()}")
    views, off = [], 0
    for shp, n in zip(shapes, sizes):
        views.append(flat[off:off + n].view(*shp))
        off += n
    return views


def adamw_step_batched(params, grads, exp_avgs, exp_avg_sqs, step, lr=1e-3, betas=(0.9, 0.999),
                       eps=1e-8, wd=1e-2, stream=None):
    """One AdamW step on every (p, g, m, v) of the non-2D tail (contiguous tensors
    of any shape, treated as flat): p and g in bf16 or float32, m and v float32,
    all updated in place but g.  ``step`` counts steps including this one.  The
    defaults are the MatrixFSDP paper's AdamW settings (section 5.1).  A tail of
    many small tensors is best kept as views into one flat tensor of each kind
    (``flat_views``) and passed as one tensor: the per-tensor marshalling here
    costs about 2 us of host time per tensor."""
    n = len(params)
    if n == 0:
        return
    dtype = params[0].dtype
    device = params[0].device
    arr = (_Vec * n)()
    for i, (p, g, m, v) in enumerate(zip(params, grads, exp_avgs, exp_avg_sqs)):
        for t, what, dt in ((p, "params", dtype), (g, "grads", dtype),
                            (m, "exp_avgs", torch.float32), (v, "exp_avg_sqs", torch.float32)):
            if not isinstance(t, torch.Tensor) or not t.is_cuda:
                raise ValueError(f"{what}[{i}] must be a CUDA tensor")
            if t.dtype != dt or not t.is_contiguous():
                raise ValueError(f"{what}[{i}] must be a contiguous {dt} tensor")
            if t.numel() != p.numel():
                raise ValueError(f"{what}[{i}] has {t.numel()} elements, params[{i}] {p.numel()}")
        arr[i] = _Vec(p.data_ptr(), g.data_ptr(), m.data_ptr(), v.data_ptr(), p.numel())
    b1, b2 = betas
    _check(lib().adamw_step_batched(arr, n, _dt(dtype), lr, b1, b2, eps, wd, int(step),
                                    _stream_ptr(device, stream)))


def ns_orthogonalize_batched(xs, out_dtype=torch.float32, ns_steps=5, coeffs=NS_COEFFS,
                             eps=1e-7, outs=None, workspace=None, stream=None,
                             precision="default"):
    """Newton-Schulz only: returns (or fills ``outs`` with) O for every x.
    precision="split" (bfloat16 inputs only): the split-precision iterate."""
    n = len(xs)
    if n == 0:
        return []
    in_dtype = xs[0].dtype
    device = xs[0].device
    for i, x in enumerate(xs):
        _check_mat(x, f"xs[{i}]", in_dtype)
    if outs is None:
        outs = [torch.empty(x.shape, dtype=out_dtype, device=device) for x in xs]
    for i, (x, o) in enumerate(zip(xs, outs)):
        _check_mat(o, f"outs[{i}]", out_dtype)
        if o.shape != x.shape:
            raise ValueError(f"outs[{i}] shape differs from xs[{i}]")
    shapes = [tuple(x.shape) for x in xs]
    wp, wb, _keep = _workspace(device, in_dtype, shapes, workspace, precision)
    xp = (_vp * n)(*[x.data_ptr() for x in xs])
    op = (_vp * n)(*[o.data_ptr() for o in outs])
    rows = (_i64 * n)(*[s[0] for s in shapes])
    cols = (_i64 * n)(*[s[1] for s in shapes])
    a, b, c = coeffs
    _check(lib().ns_orthogonalize_batched(xp, op, rows, cols, n, _dt(in_dtype, precision),
                                          _dt(out_dtype),
                                          ns_steps, a, b, c, eps, wp, wb,
                                          _stream_ptr(device, stream)))
    return outs


def profile_enable(on: bool = True):
    _check(lib().matopt_profile_enable(1 if on else 0))


def profile_read() -> dict:
    """Accumulated kernel milliseconds and launch counts per class (resets them)."""
    k = len(PROFILE_CLASSES)
    ms = (ctypes.c_double * k)()
    n = (_i64 * k)()
    _check(lib().matopt_profile_read(ms, n))
    return {name: (ms[i], n[i]) for i, name in enumerate(PROFILE_CLASSES)}


def profile_read_clock() -> dict:
    """Shader clock (MHz) per kernel class of the bf16 GEMM launches made while
    profiling was on (resets the counters); classes without data are left out."""
    k = len(PROFILE_CLASSES)
    mhz = (ctypes.c_double * k)()
    _check(lib().matopt_profile_read_clock(mhz))
    return {name: mhz[i] for i, name in enumerate(PROFILE_CLASSES) if mhz[i] > 0}


def mfma_probe(form: int, from_lds: bool, src: torch.Tensor, out: torch.Tensor,
               clk: torch.Tensor, iters: int, workgroups: int, stream=None):
    """Enqueue the MFMA rate probe (matopt_mfma_probe, a measurement aid):
    ``src`` 49152 bf16 operand values, ``out`` workgroups * 512 float32 values,
    ``clk`` two int64 tick accumulators (added to), all on one GPU."""
    for t, what, dt, n in ((src, "src", torch.bfloat16, 49152),
                           (out, "out", torch.float32, workgroups * 512),
                           (clk, "clk", torch.int64, 2)):
        _check_dev(t, what, src.device)
        if t.dtype != dt or not t.is_contiguous() or t.numel() < n:
            raise ValueError(f"{what} must be a contiguous {dt} tensor of at least {n} elements")
    _check(lib().matopt_mfma_probe(int(form), 1 if from_lds else 0, src.data_ptr(), out.data_ptr(),
                                   int(iters), int(workgroups), clk.data_ptr(),
                                   _stream_ptr(src.device, stream)))


def counters() -> dict:
    """The library's cumulative plan-cache diagnostics (see matopt_counters)."""
    k = len(COUNTERS)
    out = (_i64 * k)()
    _check(lib().matopt_counters(out, k))
    return {name: int(out[i]) for i, name in enumerate(COUNTERS)}
