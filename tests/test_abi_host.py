"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function ``include/matopt.h`` declares,
and reject invalid arguments synchronously -- before any device call -- with the
documented status codes.  Pointers used here are never dereferenced: every case
fails validation first.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "matopt.h")

OK, NULL, SHAPE, DTYPE, PARAM, WORKSPACE, ALIAS, ALIGN = range(8)


@pytest.fixture(scope="module")
def L():
    import matrix_optimizer_step_amd as m
    if not os.path.exists(m.LIB_PATH):
        pytest.fail("libmatopt.so is not built (run __graft_entry__.build())")
    return m.lib()


@pytest.fixture(scope="module")
def mod():
    import matrix_optimizer_step_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)
    keep = [n for n in names if n.startswith("matopt_") or "_batched" in n]
    return sorted(set(keep))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("muon_step_batched", "muon_step_batched_wd", "rmnp_step_batched",
              "ns_orthogonalize_batched",
              "matopt_workspace_bytes", "matopt_status_string", "matopt_last_error_detail"):
        assert n in names


def test_library_exports_every_declared_symbol(L, mod):
    for n in declared_functions():
        assert hasattr(L, n), f"libmatopt.so does not export {n}"
        assert n in mod.EXPORTS, f"binding does not wrap {n}"


def test_status_strings(L):
    assert L.matopt_status_string(0) == b"MATOPT_OK"
    assert L.matopt_status_string(6) == b"MATOPT_ERR_ALIAS"
    assert L.matopt_version() >= 10000


def _ws(L, shapes, dt):
    n = len(shapes)
    rows = (ctypes.c_int64 * n)(*[s[0] for s in shapes])
    cols = (ctypes.c_int64 * n)(*[s[1] for s in shapes])
    return L.matopt_workspace_bytes(rows, cols, n, dt)


def test_workspace_bytes_monotone_and_padded(L):
    a = _ws(L, [(256, 512)], 1)
    b = _ws(L, [(256, 512), (300, 700)], 1)
    c = _ws(L, [(1280, 5120)], 1)
    assert 0 < a < b < c
    # bf16: 2 iterates 256x512 + A,B 256x256 (2 bytes) + partials/xs
    assert a >= 2 * 256 * 512 * 2 + 2 * 256 * 256 * 2
    # tall and wide of the same size need the same workspace, but for the prep
    # partials (one float per prep tile; a transposed bf16 matrix has half as
    # many, 64 x 128 tiles)
    tall = _ws(L, [(5120, 1280)], 1)
    assert 0 <= c - tall <= (1280 * 5120 // 4096 * 4 + 255) // 256 * 256
    # fp32 pads to 64, bf16 to 256
    assert _ws(L, [(65, 65)], 0) >= 2 * 128 * 128 * 4
    assert _ws(L, [(0, 5)], 1) == 0
    assert _ws(L, [(5, 5)], 7) == 0


def _mats(mod, specs):
    arr = (mod._Mat * len(specs))()
    for i, (w, g, v, r, c) in enumerate(specs):
        arr[i] = mod._Mat(w, g, v, r, c)
    return arr


BASE = 1 << 40   # fake, never dereferenced


def _muon(L, arr, n, dt=1, ns=5, mu=0.95, lr=0.02, eps=1e-7, ws=BASE * 8, wsb=1 << 40):
    return L.muon_step_batched(arr, n, dt, mu, lr, ns, 3.4445, -4.775, 2.0315, eps, ws, wsb, None)


def test_muon_argument_errors(L, mod):
    good = [(BASE, BASE + (1 << 30), BASE + (2 << 30), 64, 128)]
    arr = _mats(mod, good)
    assert _muon(L, arr, 0) == OK                       # count 0 is a no-op
    assert _muon(L, arr, -1) == PARAM
    assert _muon(L, None, 1) == NULL
    assert _muon(L, arr, 1, dt=5) == DTYPE
    assert _muon(L, arr, 1, ns=-1) == PARAM
    assert _muon(L, arr, 1, ns=65) == PARAM
    assert _muon(L, arr, 1, mu=float("nan")) == PARAM
    assert _muon(L, arr, 1, lr=float("inf")) == PARAM
    assert _muon(L, arr, 1, eps=-1.0) == PARAM
    assert _muon(L, _mats(mod, [(0, BASE, BASE + (1 << 30), 4, 4)]), 1) == NULL
    assert _muon(L, _mats(mod, [(BASE, BASE + (1 << 30), BASE + (2 << 30), 0, 4)]), 1) == SHAPE
    assert _muon(L, _mats(mod, [(BASE + 8, BASE + (1 << 30), BASE + (2 << 30), 4, 4)]), 1) == ALIGN
    assert _muon(L, arr, 1, ws=0) == WORKSPACE
    assert _muon(L, arr, 1, wsb=16) == WORKSPACE
    assert _muon(L, arr, 1, ws=BASE * 8 + 16) == ALIGN
    # W == V, and G overlapping the next matrix's W
    assert _muon(L, _mats(mod, [(BASE, BASE + (1 << 30), BASE, 64, 128)]), 1) == ALIAS
    two = [(BASE, BASE + (1 << 30), BASE + (2 << 30), 64, 128),
           (BASE + (1 << 30) + 64, BASE + (3 << 30), BASE + (4 << 30), 64, 128)]
    assert _muon(L, _mats(mod, two), 2) == ALIAS
    # workspace overlapping an input
    assert _muon(L, arr, 1, ws=BASE + (2 << 30) - 256 * 4) == ALIAS
    detail = L.matopt_last_error_detail().decode()
    assert "overlaps" in detail


def test_muon_wd_argument_errors(L, mod):
    arr = _mats(mod, [(BASE, BASE + (1 << 30), BASE + (2 << 30), 64, 128)])

    def call(n=1, wd=1e-2, ns=2, ws=BASE * 8):
        return L.muon_step_batched_wd(arr, n, 1, 0.5, 1e-3, wd, ns, 3.4445, -4.775, 2.0315,
                                      1e-7, ws, 1 << 40, None)
    assert call(n=0) == OK
    assert call(wd=float("nan")) == PARAM
    assert call(wd=float("-inf")) == PARAM
    assert call(ns=65) == PARAM
    assert call(ws=0) == WORKSPACE
    assert call(wd=float("inf")) == PARAM
    assert "weight decay" in L.matopt_last_error_detail().decode()


def test_rmnp_colcut_argument_errors(L, mod):
    # partial: G and V used, W may be NULL; apply: W and V used, G may be NULL
    part = _mats(mod, [(0, BASE + (1 << 30), BASE + (2 << 30), 64, 128)])
    rowsq = BASE + (5 << 30)
    assert L.rmnp_colcut_partial_batched(part, 0, 1, 0.9, rowsq, None) == OK
    assert L.rmnp_colcut_partial_batched(part, 1, 1, 0.9, None, None) == NULL
    assert L.rmnp_colcut_partial_batched(part, 1, 1, 0.9, rowsq + 2, None) == ALIGN
    assert L.rmnp_colcut_partial_batched(part, 1, 1, float("nan"), rowsq, None) == PARAM
    # rowsq overlapping V
    assert L.rmnp_colcut_partial_batched(part, 1, 1, 0.9, BASE + (2 << 30) + 64, None) == ALIAS
    app = _mats(mod, [(BASE, 0, BASE + (2 << 30), 64, 128)])
    fc = (ctypes.c_int64 * 1)(100)   # narrower than the slice
    assert L.rmnp_colcut_apply_batched(app, 1, 1, 0.02, 1e-7, rowsq, fc, None) == SHAPE
    assert L.rmnp_colcut_apply_batched(app, 1, 1, 0.02, -1.0, rowsq, None, None) == PARAM
    assert L.rmnp_colcut_apply_batched(part, 1, 1, 0.02, 1e-7, rowsq, None, None) == NULL


def test_adamw_argument_errors(L, mod):
    arr = (mod._Vec * 1)(mod._Vec(BASE, BASE + (1 << 30), BASE + (2 << 30), BASE + (3 << 30), 1000))

    def call(n=1, b1=0.9, b2=0.999, eps=1e-8, step=1, a=arr):
        return L.adamw_step_batched(a, n, 1, 1e-3, b1, b2, eps, 1e-2, step, None)
    assert call(n=0) == OK
    assert call(step=0) == PARAM
    assert call(b1=1.0) == PARAM
    assert call(b2=-0.1) == PARAM
    assert call(eps=float("nan")) == PARAM
    bad = (mod._Vec * 1)(mod._Vec(BASE, BASE + 8, BASE + (2 << 30), BASE + (3 << 30), 1000))
    assert call(a=bad) == ALIGN
    ali = (mod._Vec * 1)(mod._Vec(BASE, BASE + 512, BASE + (2 << 30), BASE + (3 << 30), 1000))
    assert call(a=ali) == ALIAS   # g starts inside p (1000 bf16 = 2000 bytes)
    zero = (mod._Vec * 1)(mod._Vec(BASE, BASE + (1 << 30), BASE + (2 << 30), BASE + (3 << 30), 0))
    assert call(a=zero) == SHAPE


def test_rmnp_argument_errors(L, mod):
    arr = _mats(mod, [(BASE, BASE + (1 << 30), BASE + (2 << 30), 64, 128)])
    assert L.rmnp_step_batched(arr, 0, 1, 0.95, 0.02, 1e-12, None) == OK
    assert L.rmnp_step_batched(arr, 1, 9, 0.95, 0.02, 1e-12, None) == DTYPE
    assert L.rmnp_step_batched(arr, 1, 1, 0.95, 0.02, -1.0, None) == PARAM
    assert L.rmnp_step_batched(None, 1, 1, 0.95, 0.02, 1e-12, None) == NULL
    bad = _mats(mod, [(BASE, BASE, BASE + (2 << 30), 64, 128)])
    assert L.rmnp_step_batched(bad, 1, 1, 0.95, 0.02, 1e-12, None) == ALIAS


def test_ns_argument_errors(L, mod):
    vp = ctypes.c_void_p
    x = (vp * 1)(BASE)
    o = (vp * 1)(BASE + (1 << 30))
    rows = (ctypes.c_int64 * 1)(64)
    cols = (ctypes.c_int64 * 1)(100)

    def call(xx=x, oo=o, in_dt=1, out_dt=0, ns=5, ws=BASE * 8, wsb=1 << 40):
        return L.ns_orthogonalize_batched(xx, oo, rows, cols, 1, in_dt, out_dt, ns, 3.4445,
                                          -4.775, 2.0315, 1e-7, ws, wsb, None)
    assert call(out_dt=3) == DTYPE
    assert call(in_dt=3) == DTYPE
    assert call(xx=None) == NULL
    assert call(ns=100) == PARAM
    assert call(wsb=0) == WORKSPACE
    assert call(oo=(vp * 1)(BASE + 64)) == ALIAS


def test_binding_rejects_cpu_tensors(mod):
    import torch
    w = torch.zeros(4, 4, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        mod.muon_step_batched([w], [w.clone()], [w.clone()])


def test_flat_views_cover_one_buffer(mod):
    import torch
    flat = torch.arange(3 + 12 + 5, dtype=torch.float32)
    v = mod.flat_views(flat, [(3,), (3, 4), (5,)])
    assert [tuple(t.shape) for t in v] == [(3,), (3, 4), (5,)]
    assert v[1][0, 0].item() == 3 and v[2][-1].item() == 19
    v[1].zero_()
    assert flat[3:15].abs().sum().item() == 0     # views, not copies
    import pytest
    with pytest.raises(ValueError):
        mod.flat_views(flat, [(30,)])


def test_mfma_probe_argument_errors(L, mod):
    def call(form=16, lds=0, src=BASE, out=BASE + (1 << 30), iters=8, wg=4, clk=BASE + (2 << 30)):
        return L.matopt_mfma_probe(form, lds, src, out, iters, wg, clk, None)
    assert call(src=None) == NULL
    assert call(clk=None) == NULL
    assert call(form=8) == PARAM
    assert call(iters=7) == PARAM
    assert call(iters=0) == PARAM
    assert call(wg=0) == PARAM
    assert call(out=BASE + 8) == ALIGN
    import torch
    with pytest.raises(TypeError):
        mod.mfma_probe(16, False, torch.zeros(49152, dtype=torch.bfloat16),
                       torch.zeros(512), torch.zeros(2, dtype=torch.int64), 2, 1)
