"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Tolerances (relative Frobenius error per matrix, max over matrices):
* float32 path: <= 1e-4 against the exact float64 oracle.
* bf16 path: the orthogonalized direction O (read out in float32 through
  ns_orthogonalize_batched) <= 2e-2 against the oracle's bf16 storage model and
  against the exact oracle on Gaussian inputs.
* stored momentum: bit-identical to the oracle's single rounding of mu*V+G.
* stored weights: within 1 ulp of round(W - lr*sqrt(max(1,r/c))*O_gpu), where
  O_gpu is the GPU's own float32 direction for the GPU's own V (the kernels are
  deterministic, so this isolates the update); bit-identical to the single
  rounding of W + upd*O_gpu when upd is formed in float32 as the kernel does.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.helpers import f64, relF, ulp_distance

pytestmark = pytest.mark.gpu

COEFFS = oracle.NS_COEFFS


@pytest.fixture(scope="module")
def mo():
    import matrix_optimizer_step_amd as m
    m.lib()   # raises if the library is missing: no fallback
    return m


def _dev(ts):
    return [t.to("cuda") for t in ts]


def _inputs(wl, idx=None):
    trip = workloads.workload_inputs(wl, idx)
    W = _dev([t[0] for t in trip])
    V = _dev([t[1] for t in trip])
    G = _dev([t[2] for t in trip])
    return W, V, G


def _expect_w(w_old, o_gpu, lr, dtype, wd=0.0):
    r, c = w_old.shape
    s = oracle.update_scale(r, c)
    w = f64(w_old)
    ref = w - oracle.f32_param(lr) * (oracle.f32_param(wd) * w + s * f64(o_gpu))
    st = "bf16" if dtype == torch.bfloat16 else "f32"
    return oracle.round_storage(ref, st)


def _check_w(w_new, w_old, o_gpu, lr, wd=0.0):
    exp = _expect_w(w_old, o_gpu, lr, w_new.dtype, wd)
    got = f64(w_new)
    exp_t = torch.from_numpy(exp).to(w_new.dtype)
    d = ulp_distance(w_new.cpu(), exp_t)
    assert d.max() <= 1, f"W off by {d.max()} ulp"
    assert (d == 0).mean() >= 0.999
    return float(np.abs(got - exp).max())


def _check_w_rmnp(w, exp, upd):
    """RMNP weights against the oracle: bf16 within 1 ulp (99% exact).  float32:
    the row norm is summed in float32 (relative error ~1e-7 of the update);
    where W - lr*s*u cancels towards zero an ulp of the result is far smaller
    than that, so the bound is one ulp of the result plus 1e-6 of the update."""
    if w.dtype == torch.bfloat16:
        d = ulp_distance(w.cpu(), torch.from_numpy(exp).to(w.dtype))
        assert d.max() <= 1, (w.shape, d.max())
        assert (d == 0).mean() >= 0.99
    else:
        err = np.abs(f64(w) - exp)
        allowed = (np.spacing(np.abs(exp).astype(np.float32)).astype(np.float64)
                   + 1e-6 * np.abs(upd))
        assert (err <= allowed).all(), (w.shape, float((err / allowed).max()))


def _check_v(v_new, v_old, g, mu):
    st = "bf16" if v_new.dtype == torch.bfloat16 else "f32"
    exp = oracle.momentum(f64(v_old), f64(g), mu, st)
    d = ulp_distance(v_new.cpu(), torch.from_numpy(exp).to(v_new.dtype))
    # one correctly rounded fma on both sides: bit-exact
    assert d.max() == 0, f"V differs in {(d > 0).mean():.2%} of elements"


# --------------------------------------------------------------------------
# Newton-Schulz direction
# --------------------------------------------------------------------------

BF16_SHAPES = [(700, 1300), (1300, 700), (256, 256), (513, 1030), (1, 64), (64, 1),
               (37, 45), (8, 8), (1, 1), (300, 2000)]


# Shapes of BF16_SHAPES exempt from the 2e-2 gate against the exact iteration,
# with the reason.  This 8x8 Gaussian draw (seed 11, index 7) is
# ill-conditioned: its smallest singular value is 1.7e-4 of the Frobenius norm,
# on the steep part of the quintic's fifth iterate (gain up to a^5 ~ 485), and
# with only 8 singular values that one direction carries an eighth of |O|^2, so
# bf16 storage of the iterates costs ~3e-2 against the exact iteration.  It is
# gated instead against the storage model (2e-2) and against the appendix
# routine run in its own bf16 precision (no farther from the exact iteration).
EXACT_GATE_EXEMPT = {(8, 8): "ill-conditioned draw: sigma_min = 1.7e-4 |X0|_F"}


def test_ns_bf16_ragged_batch(mo):
    wl = workloads.small_case("ns_bf16", BF16_SHAPES, seed=11, v_std=1.0, g_std=1.0)
    _, V, _ = _inputs(wl)
    O = mo.ns_orthogonalize_batched(V, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for shape, v, o in zip(BF16_SHAPES, V, O):
        x = f64(v)
        exact = oracle.ns_orthogonalize(x)
        em = relF(f64(o), oracle.ns_orthogonalize(x, rounding="bf16"))
        ee = relF(f64(o), exact)
        ep = relF(oracle.ns_orthogonalize_page_bf16(x), exact)
        print(f"{shape}: relF(O) vs bf16 model {em:.2e}, vs exact {ee:.2e} "
              f"(appendix routine in bf16 vs exact {ep:.2e})", flush=True)
        assert em <= 2e-2
        if shape in EXACT_GATE_EXEMPT:
            assert ee <= ep
        else:
            assert ee <= 2e-2, f"{shape}: {ee:.3e} against the exact iteration"


def _illcond_small():
    """The ill-conditioned set's matrices with max side <= 512 (singular values
    log-uniform in [1e-4, 1]) and their stored momenta."""
    wl = workloads.get("ragged_illcond_64")
    idx = [i for i, s in enumerate(wl.shapes) if max(s) <= 512]
    trip = workloads.workload_inputs(wl, idx)
    return [wl.shapes[i] for i in idx], [t[2].to("cuda") for t in trip]


def test_ns_split_precision_meets_exact_tolerance(mo):
    """The split-precision path (precision="split") against the exact
    iteration at the bf16 path's tolerance, 2e-2, on every shape -- the
    ill-conditioned 8x8 draw and the ill-conditioned set included -- and
    against its own storage model."""
    wl = workloads.small_case("ns_bf16", BF16_SHAPES, seed=11, v_std=1.0, g_std=1.0)
    _, V, _ = _inputs(wl)
    shapes_ic, V_ic = _illcond_small()
    shapes = list(BF16_SHAPES) + shapes_ic
    O = mo.ns_orthogonalize_batched(V + V_ic, out_dtype=torch.float32, precision="split")
    O_plain = mo.ns_orthogonalize_batched(V + V_ic, out_dtype=torch.float32)
    torch.cuda.synchronize()
    worst = 0.0
    for shape, v, o, op in zip(shapes, V + V_ic, O, O_plain):
        x = f64(v)
        exact = oracle.ns_orthogonalize(x)
        ee = relF(f64(o), exact)
        em = relF(f64(o), oracle.ns_orthogonalize(x, rounding="bf16_split"))
        ep = relF(f64(op), exact)
        print(f"{shape}: split vs exact {ee:.2e} (plain bf16 {ep:.2e}), vs split model {em:.2e}",
              flush=True)
        assert ee <= 2e-2, f"{shape}: {ee:.3e} against the exact iteration"
        assert em <= 2e-2
        worst = max(worst, ee)
    print(f"worst split-precision error against the exact iteration: {worst:.2e}", flush=True)


def test_muon_step_split_precision(mo):
    """The Muon step in split precision: momentum bit-exact, the update a single
    rounding of W - lr*s*O with O the split path's own direction, O within 2e-2
    of the exact iteration."""
    shapes = [(700, 1300), (1300, 700), (256, 256), (37, 45), (1, 300), (300, 1)]
    wl = workloads.small_case("muon_split", shapes, seed=27)
    W, V, G = _inputs(wl)
    W0, V0 = [w.clone() for w in W], [v.clone() for v in V]
    mo.muon_step_batched(W, G, V, mu=0.95, lr=0.02, ns_steps=5, precision="split")
    O = mo.ns_orthogonalize_batched(V, out_dtype=torch.float32, precision="split")
    torch.cuda.synchronize()
    for w, w0, v, v0, g, o in zip(W, W0, V, V0, G, O):
        _check_v(v, v0, g, 0.95)
        _check_w(w, w0, o, 0.02)
        assert relF(f64(o), oracle.ns_orthogonalize(f64(v))) <= 2e-2


# Gram and polynomial tables of this batch differ in length (72 and 48 entries:
# both are packed longest-unit-first, with K = n and K = m per tile), so it
# checks that each stage launches exactly its own table.
MIXED_SHAPES = [(384, 3072), (512, 256), (512, 1024), (512, 128), (512, 2048), (128, 512),
                (1024, 256), (768, 768), (128, 128), (768, 768), (768, 1536), (2048, 512),
                (768, 1536), (384, 384), (512, 512)]


def test_ns_bf16_mixed_batch_stage_tables_differ(mo):
    wl = workloads.small_case("mixed", MIXED_SHAPES, seed=21, v_std=1.0)
    _, V, _ = _inputs(wl)
    O = mo.ns_orthogonalize_batched(V, out_dtype=torch.float32)
    torch.cuda.synchronize()
    errs = [relF(f64(o), oracle.ns_orthogonalize(f64(v), rounding="bf16")) for v, o in zip(V, O)]
    print("mixed batch relF vs bf16 model", np.round(errs, 5))
    assert max(errs) <= 2e-2
    alone = [mo.ns_orthogonalize_batched([v], out_dtype=torch.float32)[0] for v in V]
    torch.cuda.synchronize()
    for o, a in zip(O, alone):
        assert torch.equal(o, a)


# Every matrix padded to m = 512 rows, so every apply tile has K = 512 and the
# non-final applies run as the persistent kernel (one workgroup per CU walking
# its XCD stream: 552 tiles here, two or three per workgroup).  Adding a matrix
# of another height makes the launch take one tile per workgroup instead.
SAME_K_SHAPES = [(512, 8192)] * 6 + [(300, 8192), (8192, 512), (512, 4096), (512, 1000)]


@pytest.mark.parametrize("precision", ["default", "split"])
def test_persistent_apply_matches_one_tile_per_workgroup(mo, precision):
    wl = workloads.small_case("same_k", SAME_K_SHAPES + [(256, 256)], seed=31, v_std=1.0)
    _, V, _ = _inputs(wl)
    n = len(SAME_K_SHAPES)
    O_persist = mo.ns_orthogonalize_batched(V[:n], out_dtype=torch.float32, precision=precision)
    O_tiles = mo.ns_orthogonalize_batched(V, out_dtype=torch.float32, precision=precision)
    torch.cuda.synchronize()
    for a, b in zip(O_persist, O_tiles[:n]):
        assert torch.equal(a, b)
    for i in (6, 7, 9):
        x = f64(V[i])
        ee = relF(f64(O_persist[i]), oracle.ns_orthogonalize(x))
        rounding = "bf16_split" if precision == "split" else "bf16"
        em = relF(f64(O_persist[i]), oracle.ns_orthogonalize(x, rounding=rounding))
        print(f"{SAME_K_SHAPES[i]} ({precision}): relF(O) vs exact {ee:.2e}, vs model {em:.2e}",
              flush=True)
        assert ee <= 2e-2 and em <= 2e-2


F32_SHAPES = [(256, 512), (150, 333), (333, 150), (64, 64), (1, 7), (7, 1), (65, 129)]


def test_ns_f32_ragged_batch(mo):
    wl = workloads.small_case("ns_f32", F32_SHAPES, dtype="f32", seed=12, v_std=1.0)
    _, V, _ = _inputs(wl)
    O = mo.ns_orthogonalize_batched(V, out_dtype=torch.float32)
    torch.cuda.synchronize()
    errs = [relF(f64(o), oracle.ns_orthogonalize(f64(v))) for v, o in zip(V, O)]
    print("f32 relF vs exact", np.round(errs, 8))
    assert max(errs) <= 1e-4


# Both matrices pad to m = 512: every non-final apply runs as the persistent
# kernel, and seven steps take each iterate buffer through it three times.
@pytest.mark.parametrize("precision", ["default", "split"])
@pytest.mark.parametrize("steps", [0, 1, 2, 7])
def test_ns_step_counts(mo, steps, precision):
    wl = workloads.small_case("ns_steps", [(300, 500), (500, 300)], seed=13, v_std=1.0)
    _, V, _ = _inputs(wl)
    O = mo.ns_orthogonalize_batched(V, out_dtype=torch.float32, ns_steps=steps,
                                    precision=precision)
    torch.cuda.synchronize()
    rounding = "bf16_split" if precision == "split" else "bf16"
    for v, o in zip(V, O):
        ref = oracle.ns_orthogonalize(f64(v), steps=steps, rounding=rounding)
        assert relF(f64(o), ref) <= (1e-6 if steps == 0 else 2e-2)
        if steps:
            assert relF(f64(o), oracle.ns_orthogonalize(f64(v), steps=steps)) <= 2e-2


# Coefficients other than the default quintic reach the kernels unchanged: the
# classic cubic (c = 0, the polynomial is a I + b A), the quintic with the
# flattest fixed point at 1 (15/8, -10/8, 3/8), and a quintic with fixed point
# 1 and a negative slope there (3, -3.2, 1.2).  Wide, tall (transposed) and
# aligned (read in place) matrices, in both precisions.
OTHER_COEFFS = [(1.5, -0.5, 0.0), (1.875, -1.25, 0.375), (3.0, -3.2, 1.2)]


@pytest.mark.parametrize("coeffs", OTHER_COEFFS, ids=["cubic", "quintic-flat", "quintic-oscillating"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ns_other_coefficients(mo, coeffs, dtype):
    shapes = [(300, 700), (520, 260), (256, 256)]
    wl = workloads.small_case("ns_coeffs", shapes, dtype=dtype, seed=17, v_std=1.0)
    _, V, _ = _inputs(wl)
    O = mo.ns_orthogonalize_batched(V, out_dtype=torch.float32, coeffs=coeffs)
    torch.cuda.synchronize()
    for shape, v, o in zip(shapes, V, O):
        x = f64(v)
        ee = relF(f64(o), oracle.ns_orthogonalize(x, coeffs=coeffs))
        if dtype == "f32":
            assert ee <= 1e-4, (shape, ee)
        else:
            em = relF(f64(o), oracle.ns_orthogonalize(x, coeffs=coeffs, rounding="bf16"))
            print(f"{coeffs} {shape}: relF(O) vs bf16 model {em:.2e}, vs exact {ee:.2e}", flush=True)
            assert em <= 2e-2 and ee <= 2e-2, (shape, em, ee)


def test_ns_bf16_output_dtype(mo):
    wl = workloads.small_case("ns_out", [(512, 768)], seed=14, v_std=1.0)
    _, V, _ = _inputs(wl)
    O32 = mo.ns_orthogonalize_batched(V, out_dtype=torch.float32)
    O16 = mo.ns_orthogonalize_batched(V, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(O32[0].to(torch.bfloat16), O16[0])


def test_ns_zero_matrix(mo):
    z = [torch.zeros(300, 700, dtype=torch.bfloat16, device="cuda"),
         torch.zeros(40, 9, dtype=torch.float32, device="cuda")]
    o = mo.ns_orthogonalize_batched(z[:1])
    o2 = mo.ns_orthogonalize_batched(z[1:])
    torch.cuda.synchronize()
    assert not o[0].any() and not o2[0].any()


def test_ns_batch_invariance_and_determinism(mo):
    wl = workloads.small_case("inv", [(600, 900), (900, 600), (256, 1024), (33, 77)],
                              seed=15, v_std=1.0)
    _, V, _ = _inputs(wl)
    full = mo.ns_orthogonalize_batched(V)
    again = mo.ns_orthogonalize_batched(V)
    alone = [mo.ns_orthogonalize_batched([v])[0] for v in V]
    torch.cuda.synchronize()
    for f, a, s in zip(full, again, alone):
        assert torch.equal(f, a)
        assert torch.equal(f, s)


def test_ns_transpose_equivariance(mo):
    # O(V^T) = O(V)^T.  The two calls sum the Frobenius norm in different tile
    # orders, so the scale may differ in its last bit: compare within tolerance.
    for dtype, tol in ((torch.bfloat16, 2e-2), (torch.float32, 1e-5)):
        v = torch.randn(400, 900, device="cuda").to(dtype)
        vt = v.t().contiguous()
        o = mo.ns_orthogonalize_batched([v])[0]
        ot = mo.ns_orthogonalize_batched([vt])[0]
        torch.cuda.synchronize()
        assert relF(f64(ot), f64(o).T) <= tol


# --------------------------------------------------------------------------
# full Muon step
# --------------------------------------------------------------------------

def test_muon_step_f32_single_256x512(mo):
    wl = workloads.get("single_f32_256x512")
    W, V, G = _inputs(wl)
    W0, V0 = [w.clone() for w in W], [v.clone() for v in V]
    mo.muon_step_batched(W, G, V, mu=wl.mu, lr=wl.lr, ns_steps=wl.ns_steps)
    torch.cuda.synchronize()
    w_ref, v_ref, o_ref = oracle.muon_step(f64(W0[0]), f64(G[0]), f64(V0[0]), mu=wl.mu,
                                           lr=wl.lr, dtype="f32")
    _check_v(V[0], V0[0], G[0], wl.mu)
    dw = f64(W[0]) - f64(W0[0])
    dw_ref = -oracle.f32_param(wl.lr) * oracle.update_scale(256, 512) * o_ref
    err = relF(dw, dw_ref)
    print("C1 relF(dW)", err)
    assert err <= 1e-4


def test_muon_step_bf16_ragged(mo):
    shapes = [(700, 1300), (1300, 700), (256, 256), (37, 45), (1, 300), (300, 1)]
    wl = workloads.small_case("muon_bf16", shapes, seed=17)
    W, V, G = _inputs(wl)
    W0, V0 = [w.clone() for w in W], [v.clone() for v in V]
    mo.muon_step_batched(W, G, V, mu=0.95, lr=0.02, ns_steps=5)
    O = mo.ns_orthogonalize_batched(V, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for w, w0, v, v0, g, o in zip(W, W0, V, V0, G, O):
        _check_v(v, v0, g, 0.95)
        _check_w(w, w0, o, 0.02)
        ref = oracle.ns_orthogonalize(f64(v), rounding="bf16")
        assert relF(f64(o), ref) <= 2e-2


def test_muon_fused_update_rounds_once_bitwise(mo):
    """The fused bf16 weight update stores the single nearest-even rounding of
    W + upd*O bit for bit, where upd = -lr*sqrt(max(1, r/c)) is formed in
    float32 as the kernel forms it and O is the GPU's own float32 direction
    for the updated V.  The shapes (full and ragged tiles, both orientations)
    hold millions of weights, so float32 sums that fall exactly on a bfloat16
    midpoint -- the case that needs the float64 tie-break -- occur and are
    counted."""
    shapes = [(1280, 5120), (5120, 1280), (1000, 3000)]
    wl = workloads.small_case("muon_fused_round", shapes, seed=23)
    W, V, G = _inputs(wl)
    W0 = [w.clone() for w in W]
    lr = 0.02
    mo.muon_step_batched(W, G, V, mu=0.95, lr=lr, ns_steps=5)
    O = mo.ns_orthogonalize_batched(V, out_dtype=torch.float32)
    torch.cuda.synchronize()
    midpoints = 0
    for w, w0, o in zip(W, W0, O):
        r, c = w.shape
        upd = np.float32(-(np.float32(lr) * np.float32(np.sqrt(max(1.0, r / c)))))
        exact = f64(w0) + float(upd) * f64(o)
        s32 = exact.astype(np.float32)
        midpoints += int(((s32.view(np.uint32) & 0xFFFF) == 0x8000).sum())
        got = f64(w)
        exp = oracle.round_bf16(exact)
        bad = int((got != exp).sum())
        assert bad == 0, f"{w.shape}: {bad} weights differ from the single rounding"
    assert midpoints > 0, "no float32 result fell on a bfloat16 midpoint"


def test_muon_step_ns_steps_zero_and_lr_zero(mo):
    wl = workloads.small_case("muon0", [(128, 640), (640, 128)], seed=18)
    W, V, G = _inputs(wl)
    W0 = [w.clone() for w in W]
    mo.muon_step_batched(W, G, V, ns_steps=0, lr=0.5)
    O = mo.ns_orthogonalize_batched(V, ns_steps=0)
    torch.cuda.synchronize()
    for w, w0, v, o in zip(W, W0, V, O):
        ref = f64(v) / (np.linalg.norm(f64(v)) + oracle.f32_param(1e-7))
        assert relF(f64(o), ref) <= 1e-6
        _check_w(w, w0, o, 0.5)
    W1 = [w.clone() for w in W]
    mo.muon_step_batched(W, G, V, lr=0.0)
    torch.cuda.synchronize()
    for w, w1 in zip(W, W1):
        assert torch.equal(w, w1)


# MatrixFSDP section 5.1 trains with momentum 0.5, two Newton-Schulz steps and
# weight decay 1e-2 at lr 1e-3; the second case makes the decay large enough to
# move most bf16 weights.
@pytest.mark.parametrize("lr,wd", [(1e-3, 1e-2), (0.05, 0.5)])
@pytest.mark.parametrize("precision", ["default", "split"])
def test_muon_wd_training_config_bf16(mo, lr, wd, precision):
    shapes = [(700, 1300), (1300, 700), (256, 256), (37, 45), (1, 300), (300, 1)]
    wl = workloads.small_case("muon_wd", shapes, seed=23)
    W, V, G = _inputs(wl)
    W0, V0 = [w.clone() for w in W], [v.clone() for v in V]
    mo.muon_step_batched_wd(W, G, V, mu=0.5, lr=lr, wd=wd, ns_steps=2, precision=precision)
    O = mo.ns_orthogonalize_batched(V, out_dtype=torch.float32, ns_steps=2, precision=precision)
    torch.cuda.synchronize()
    rounding = "bf16_split" if precision == "split" else "bf16"
    moved = 0
    for w, w0, v, v0, g, o in zip(W, W0, V, V0, G, O):
        _check_v(v, v0, g, 0.5)
        _check_w(w, w0, o, lr, wd)
        ref = oracle.ns_orthogonalize(f64(v), steps=2, rounding=rounding)
        assert relF(f64(o), ref) <= 2e-2
        moved += int((w != w0).sum())
    assert moved > 0


def test_muon_wd_zero_is_the_plain_step(mo):
    for dtype, shapes in (("bf16", [(512, 1280), (1280, 512), (37, 45)]),
                          ("f32", [(256, 512), (65, 129)])):
        wl = workloads.small_case("wd0", shapes, dtype=dtype, seed=24)
        W1, V1, G = _inputs(wl)
        W2, V2 = [w.clone() for w in W1], [v.clone() for v in V1]
        mo.muon_step_batched(W1, G, V1, mu=0.9, lr=0.03, ns_steps=3)
        mo.muon_step_batched_wd(W2, G, V2, mu=0.9, lr=0.03, wd=0.0, ns_steps=3)
        torch.cuda.synchronize()
        for a, b in zip(W1 + V1, W2 + V2):
            assert torch.equal(a, b)


def test_muon_wd_f32_and_ns_steps_zero(mo):
    # float32 storage (vector and ragged-width rows), then the ns_steps == 0 path
    wl = workloads.small_case("wd_f32", [(256, 512), (65, 129)], dtype="f32", seed=25)
    W, V, G = _inputs(wl)
    W0, V0 = [w.clone() for w in W], [v.clone() for v in V]
    mo.muon_step_batched_wd(W, G, V, mu=0.5, lr=0.05, wd=0.5, ns_steps=2)
    O = mo.ns_orthogonalize_batched(V, out_dtype=torch.float32, ns_steps=2)
    torch.cuda.synchronize()
    for w, w0, v, v0, g, o in zip(W, W0, V, V0, G, O):
        _check_v(v, v0, g, 0.5)
        _check_w(w, w0, o, 0.05, 0.5)
        assert relF(f64(o), oracle.ns_orthogonalize(f64(v), steps=2)) <= 1e-4
    wl = workloads.small_case("wd_ns0", [(128, 640), (640, 128), (33, 70)], seed=26)
    W, V, G = _inputs(wl)
    W0 = [w.clone() for w in W]
    mo.muon_step_batched_wd(W, G, V, mu=0.5, lr=0.05, wd=0.5, ns_steps=0)
    O = mo.ns_orthogonalize_batched(V, ns_steps=0)
    torch.cuda.synchronize()
    for w, w0, o in zip(W, W0, O):
        _check_w(w, w0, o, 0.05, 0.5)


def test_muon_step_zero_inputs(mo):
    z = lambda: torch.zeros(256, 512, dtype=torch.bfloat16, device="cuda")
    w = torch.randn(256, 512, device="cuda").to(torch.bfloat16)
    w0 = w.clone()
    v, g = z(), z()
    mo.muon_step_batched([w], [g], [v])
    torch.cuda.synchronize()
    assert torch.equal(w, w0) and not v.any()


def test_muon_step_deterministic_and_batch_invariant(mo):
    shapes = [(512, 1280), (1280, 512), (256, 768)]
    wl = workloads.small_case("det", shapes, seed=19)
    runs = []
    for batch in (True, False):
        W, V, G = _inputs(wl)
        if batch:
            mo.muon_step_batched(W, G, V)
        else:
            for i in range(len(W)):
                mo.muon_step_batched([W[i]], [G[i]], [V[i]])
        torch.cuda.synchronize()
        runs.append((W, V))
    W, V, G = _inputs(wl)
    mo.muon_step_batched(W, G, V)
    torch.cuda.synchronize()
    for a, b, c in zip(runs[0][0], runs[1][0], W):
        assert torch.equal(a, b) and torch.equal(a, c)
    for a, b in zip(runs[0][1], runs[1][1]):
        assert torch.equal(a, b)


def test_muon_two_steps_resume(mo):
    """k steps, save (W, V), reload, k more == 2k uninterrupted (same gradients)."""
    wl = workloads.small_case("resume", [(384, 640)], seed=20)
    W, V, G = _inputs(wl)
    Wa, Va = [W[0].clone()], [V[0].clone()]
    for _ in range(4):
        mo.muon_step_batched(Wa, G, Va)
    Wb, Vb = [W[0].clone()], [V[0].clone()]
    for _ in range(2):
        mo.muon_step_batched(Wb, G, Vb)
    torch.cuda.synchronize()
    Wc, Vc = [Wb[0].cpu().clone().cuda()], [Vb[0].cpu().clone().cuda()]
    for _ in range(2):
        mo.muon_step_batched(Wc, G, Vc)
    torch.cuda.synchronize()
    assert torch.equal(Wa[0], Wc[0]) and torch.equal(Va[0], Vc[0])


# --------------------------------------------------------------------------
# RMNP
# --------------------------------------------------------------------------

# widths that reach every register-resident variant in both dtypes (rows of
# one wave with 1, 2, 4 and 8 chunks per lane, of a workgroup with 4, 8 and 16)
# with lanes past the row's end, and the streaming variant
RMNP_SHAPES = [(96, 1280), (40, 5120), (8, 27648), (3, 40000), (50, 45), (64, 8),
               (200, 64), (17, 3000), (9, 400), (11, 1000), (5, 12000)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rmnp_step(mo, dtype):
    wl = workloads.small_case("rmnp", RMNP_SHAPES, dtype=dtype, seed=21)
    W, V, G = _inputs(wl)
    W0, V0 = [w.clone() for w in W], [v.clone() for v in V]
    mo.rmnp_step_batched(W, G, V, mu=0.95, lr=0.02, eps=1e-12)
    torch.cuda.synchronize()
    for w, w0, v, v0, g in zip(W, W0, V, V0, G):
        _check_v(v, v0, g, 0.95)
        u = oracle.rmnp_direction(f64(v))
        r, c = w.shape
        exp = oracle.round_storage(f64(w0) - oracle.f32_param(0.02) * oracle.update_scale(r, c) * u,
                                   dtype)
        _check_w_rmnp(w, exp, oracle.f32_param(0.02) * oracle.update_scale(r, c) * u)


def test_rmnp_row_split_invariance_bitwise(mo):
    wl = workloads.small_case("split", [(384, 512)], seed=22)
    W, V, G = _inputs(wl)
    Ws = [W[0][a:b].clone() for a, b in ((0, 100), (100, 250), (250, 384))]
    Vs = [V[0][a:b].clone() for a, b in ((0, 100), (100, 250), (250, 384))]
    Gs = [G[0][a:b].clone() for a, b in ((0, 100), (100, 250), (250, 384))]
    mo.rmnp_step_batched(W, G, V)
    mo.rmnp_step_batched(Ws, Gs, Vs)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(Ws), W[0])
    assert torch.equal(torch.cat(Vs), V[0])


def test_rmnp_zero_row(mo):
    w = torch.randn(8, 1024, device="cuda").to(torch.bfloat16)
    v = torch.randn(8, 1024, device="cuda").to(torch.bfloat16)
    g = torch.randn(8, 1024, device="cuda").to(torch.bfloat16)
    v[3].zero_()
    g[3].zero_()
    w0 = w.clone()
    mo.rmnp_step_batched([w], [g], [v])
    torch.cuda.synchronize()
    assert torch.equal(w[3], w0[3])
    assert not torch.equal(w[2], w0[2])


# --------------------------------------------------------------------------
# Column-cut RMNP (local halves); two ranks simulated on one GPU
# --------------------------------------------------------------------------

COLCUT = [((300, 1000), [0, 400, 1000]), ((1280, 640), [0, 320, 640]), ((37, 45), [0, 13, 45]),
          ((64, 8), [0, 8, 8]), ((5, 3000), [0, 1496, 3000])]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rmnp_colcut_two_slices(mo, dtype):
    shapes = [sh for sh, _ in COLCUT]
    wl = workloads.small_case("colcut", shapes, dtype=dtype, seed=31, v_std=1.0, g_std=1.0)
    W, V, G = _inputs(wl)
    tdt = W[0].dtype
    ranks = []
    for k in range(2):
        sl = [(a[k], a[k + 1]) for _, a in COLCUT]
        ranks.append({
            # copies (a slice spanning every column would otherwise alias the whole)
            "W": [w[:, a:b].clone() for w, (a, b) in zip(W, sl) if b > a],
            "V": [v[:, a:b].clone() for v, (a, b) in zip(V, sl) if b > a],
            "G": [g[:, a:b].clone() for g, (a, b) in zip(G, sl) if b > a],
            "full": [sh[1] for (sh, _), (a, b) in zip(COLCUT, sl) if b > a],
            "idx": [i for i, (a, b) in enumerate(sl) if b > a]})
    for r in ranks:
        r["W0"] = [w.clone() for w in r["W"]]
        r["V0"] = [v.clone() for v in r["V"]]
        r["rowsq"] = mo.rmnp_colcut_partial_batched(r["G"], r["V"], mu=0.9)
    torch.cuda.synchronize()
    # the all-reduce over the ranks, as a host-side sum of each row's partials
    total = {}
    for r in ranks:
        off = 0
        for i, v in zip(r["idx"], r["V"]):
            part = r["rowsq"][off:off + v.shape[0]]
            total[i] = part.clone() if i not in total else total[i] + part
            off += v.shape[0]
    for r in ranks:
        r["sum"] = torch.cat([total[i] for i in r["idx"]])
        mo.rmnp_colcut_apply_batched(r["W"], r["V"], r["sum"], full_cols=r["full"], lr=0.3,
                                     eps=1e-7)
    torch.cuda.synchronize()
    st = "bf16" if dtype == "bf16" else "f32"
    for r in ranks:
        off = 0
        for w, w0, v, v0, g, fc in zip(r["W"], r["W0"], r["V"], r["V0"], r["G"], r["full"]):
            rows = v.shape[0]
            _check_v(v, v0, g, 0.9)
            v_new, rowsq = oracle.rmnp_colcut_partial(f64(v0), f64(g), mu=0.9, dtype=st)
            got = r["rowsq"][off:off + rows].double().cpu().numpy()
            np.testing.assert_allclose(got, rowsq, rtol=2e-6, atol=0)
            tot = r["sum"][off:off + rows].double().cpu().numpy()
            exp = oracle.rmnp_colcut_apply(f64(w0), v_new, tot, lr=0.3, eps=1e-7, full_cols=fc,
                                           dtype=st)
            upd = (oracle.f32_param(0.3) * oracle.update_scale(rows, fc) * v_new
                   / np.maximum(np.sqrt(tot), oracle.f32_param(1e-7))[:, None])
            _check_w_rmnp(w, exp, upd)
            off += rows
    # recombined slices against the row-local step on the whole matrices
    for i, (sh, _) in enumerate(COLCUT):
        parts = [r["W"][r["idx"].index(i)] for r in ranks if i in r["idx"]]
        w_full = torch.cat(parts, dim=1).cpu()
        w_ref, _, u = oracle.rmnp_step(f64(W[i]), f64(G[i]), f64(V[i]), mu=0.9, lr=0.3, eps=1e-7,
                                       dtype=st)
        _check_w_rmnp(w_full, w_ref, oracle.f32_param(0.3) * oracle.update_scale(*sh) * u)


# --------------------------------------------------------------------------
# AdamW for the non-2D tail
# --------------------------------------------------------------------------

ADAMW_LENS = [1280, 1280, 3840, 1280, 5120, 1280, 7, 1, 1000, 4099, 2048, 2049]


@pytest.mark.parametrize("dtype,step", [("bf16", 1), ("bf16", 7), ("f32", 7)])
def test_adamw_ragged_tail(mo, dtype, step):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    gen = torch.Generator().manual_seed(40 + step)
    P = [torch.randn(n, generator=gen).to(tdt) for n in ADAMW_LENS]
    G = [(torch.randn(n, generator=gen) * 0.1).to(tdt) for n in ADAMW_LENS]
    if step == 1:
        M = [torch.zeros(n) for n in ADAMW_LENS]
        Vs = [torch.zeros(n) for n in ADAMW_LENS]
    else:
        M = [torch.randn(n, generator=gen) * 0.01 for n in ADAMW_LENS]
        Vs = [torch.rand(n, generator=gen) * 1e-3 for n in ADAMW_LENS]
    dP, dG, dM, dV = ([t.cuda() for t in L] for L in (P, G, M, Vs))
    mo.adamw_step_batched(dP, dG, dM, dV, step, lr=1e-3, betas=(0.9, 0.999), eps=1e-8, wd=1e-2)
    torch.cuda.synchronize()
    for p0, g, m0, v0, p1, m1, v1 in zip(P, G, M, Vs, dP, dM, dV):
        pe, me, ve = oracle.adamw_step(f64(p0), f64(g), f64(m0), f64(v0), step, lr=1e-3,
                                       beta1=0.9, beta2=0.999, eps=1e-8, wd=1e-2, dtype=dtype)
        # the moments: one float64 expression in the same order, one rounding
        assert torch.equal(m1.cpu(), torch.from_numpy(me).float())
        assert torch.equal(v1.cpu(), torch.from_numpy(ve).float())
        if dtype == "bf16":
            d = ulp_distance(p1.cpu(), torch.from_numpy(pe).to(tdt))
            assert d.max() <= 1 and (d == 0).mean() >= 0.99
        else:
            upd = np.abs(f64(p0) - oracle.adamw_step(f64(p0), f64(g), f64(m0), f64(v0), step,
                                                      dtype="f64")[0])
            err = np.abs(f64(p1) - pe)
            allowed = np.spacing(np.abs(pe).astype(np.float32)).astype(np.float64) + 1e-9 * upd
            assert (err <= allowed).all()


def test_adamw_flat_tail_equals_separate_tensors(mo):
    """The tail as views into one flat tensor of each kind (flat_views), passed
    as one tensor, gives the bits of the same tensors passed one by one."""
    gen = torch.Generator().manual_seed(77)
    lens = ADAMW_LENS
    shapes = [(n,) for n in lens]
    total = sum(lens)
    fp = torch.randn(total, generator=gen).bfloat16().cuda()
    fg = (torch.randn(total, generator=gen) * 0.1).bfloat16().cuda()
    fm = (torch.randn(total, generator=gen) * 0.01).cuda()
    fv = (torch.rand(total, generator=gen) * 1e-3).cuda()
    sep = [[t.clone() for t in mo.flat_views(f, shapes)] for f in (fp, fg, fm, fv)]
    mo.adamw_step_batched(*sep, 3)
    mo.adamw_step_batched([fp], [fg], [fm], [fv], 3)
    torch.cuda.synchronize()
    for flat, parts in ((fp, sep[0]), (fm, sep[2]), (fv, sep[3])):
        for view, part in zip(mo.flat_views(flat, shapes), parts):
            assert torch.equal(view, part)
