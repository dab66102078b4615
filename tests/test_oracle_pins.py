"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: closed forms
(the action of one Newton-Schulz step on singular values, rank-1 and
diagonal-Gram constructions, the cubic polar iteration), library routines
(LAPACK SVD through numpy, torch's bfloat16 conversion and row normalisation),
invariances, and the constants and ledger the blog post prints
(``tests/golden/``).  Inputs are small so the whole file runs in seconds.
"""

import json
import os

import numpy as np
import torch
import pytest

import oracle
from oracle import (NS_COEFFS, f32_param, momentum, ns_orthogonalize,
                    ns_orthogonalize_page_form, ns_orthogonalize_page_bf16, split_bf16, muon_step, rmnp_direction,
                    rmnp_step, round_bf16, round_storage)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
A, B, C = (f32_param(t) for t in NS_COEFFS)


def relF(x, y):
    return np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-300)


def p(s, k=1, a=A, b=B, c=C):
    """k-fold scalar map of one Newton-Schulz step on a singular value."""
    s = np.asarray(s, np.float64)
    for _ in range(k):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def svd_closed_form(x, k, eps=1e-7, coeffs=NS_COEFFS):
    """``X0 = U S V^T`` (LAPACK) => k Newton-Schulz steps give ``U p^k(S) V^T``,
    because ``X X^T = U S^2 U^T`` makes every step act on S alone."""
    a, b, c = (f32_param(t) for t in coeffs)
    x = np.asarray(x, np.float64)
    x0 = x / (np.linalg.norm(x) + f32_param(eps))
    u, s, vt = np.linalg.svd(x0, full_matrices=False)
    return (u * p(s, k, a, b, c)[None, :]) @ vt


def rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------
# golden constants and ledger printed on the pages
# --------------------------------------------------------------------------

def test_constants_match_page_appendix():
    g = json.load(open(os.path.join(GOLDEN, "ns_constants.json")))
    assert tuple(g["ns_coefficients"]) == oracle.NS_COEFFS
    assert g["ns_steps"] == oracle.NS_STEPS
    assert g["ns_eps"] == oracle.NS_EPS
    assert g["momentum"] == oracle.MOMENTUM
    assert g["rmnp_row_norm_clamp"]["value"] == oracle.RMNP_EPS


def test_gpt2_large_workload_matches_page_ledger():
    import workloads
    g = json.load(open(os.path.join(GOLDEN, "gpt2_large_ledger.json")))
    wl = workloads.get("gpt2_large_144")
    assert len(wl.shapes) == g["matrices"]
    assert round(wl.numel / 1e6) == g["params_millions_rounded"]
    gather = sum(7 / 8 * r * c * 2 for r, c in wl.shapes) / 2 ** 20
    assert round(gather) == g["gather_mib_per_gpu_8way_rounded"]
    assert 5120 * 1280 * 2 / 2 ** 20 == g["c_fc_bf16_mib"]
    assert (5120, 1280) in wl.shapes
    # page rows ([out, in]) are this workload's columns
    sum_rows_page = sum(c for _, c in wl.shapes)
    assert abs(sum_rows_page - g["row_vector_len_approx"]) <= \
        g["row_vector_len_rel_tol"] * g["row_vector_len_approx"]


# --------------------------------------------------------------------------
# storage rounding
# --------------------------------------------------------------------------

def test_round_bf16_matches_torch_on_fp32_values():
    torch = pytest.importorskip("torch")
    r = rng(0)
    x = np.concatenate([
        r.standard_normal(20000).astype(np.float32),
        (r.standard_normal(20000) * 1e-3).astype(np.float32),
        (r.standard_normal(2000) * 1e30).astype(np.float32),
    ])
    # constructed ties: low 16 bits exactly 0x8000 (odd and even kept parts)
    bits = r.integers(0x3F000000 >> 16, 0x4100, size=4000).astype(np.uint32) << 16
    ties = (bits | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties, np.float32([0.0, -0.0, 1.0])])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = round_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_round_bf16_is_direct_from_float64():
    # 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7: ties to even -> 1.
    assert round_bf16(1 + 2.0 ** -8) == 1.0
    # 1 + 3*2^-8 is the midpoint of 1+2^-7 (odd) and 1+2^-6 (even) -> 1+2^-6.
    assert round_bf16(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6
    # Just above the midpoint rounds up even though a float32 hop would tie.
    assert round_bf16(1 + 2.0 ** -8 + 2.0 ** -40) == 1 + 2.0 ** -7
    assert round_bf16(-(1 + 2.0 ** -8 + 2.0 ** -40)) == -(1 + 2.0 ** -7)
    # carry into the exponent
    assert round_bf16(2.0 - 2.0 ** -9) == 2.0
    assert np.isnan(round_bf16(np.nan)) and round_bf16(np.inf) == np.inf


def test_round_storage_f32_is_float32():
    x = rng(1).standard_normal(1000)
    np.testing.assert_array_equal(round_storage(x, "f32"),
                                  x.astype(np.float32).astype(np.float64))


# --------------------------------------------------------------------------
# Newton-Schulz: closed forms
# --------------------------------------------------------------------------

SHAPES = [(1, 1), (1, 5), (5, 1), (8, 16), (16, 8), (32, 64), (64, 64), (3, 200),
          (200, 3), (48, 20)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("k", [0, 1, 2, 5])
def test_ns_matches_svd_closed_form(shape, k):
    x = rng(hash(shape) % 1000 + k).standard_normal(shape)
    got = ns_orthogonalize(x, steps=k)
    ref = svd_closed_form(x, k)
    assert relF(got, ref) <= 1e-12


def test_ns_band_of_singular_values_gaussian_256x512():
    # sup over [0,1] of p^5 is 1.20237...; every singular value above 0.0015
    # maps into [0.6818, 1.2024] (scalar map of the printed coefficients).
    grid = np.linspace(0, 1, 200001)
    sup = p(grid, 5).max()
    assert 1.2023 < sup < 1.2025
    x = rng(2).standard_normal((256, 512))
    s_in = np.linalg.svd(x / (np.linalg.norm(x) + 1e-7), compute_uv=False)
    assert s_in.min() > 0.0015
    s = np.linalg.svd(ns_orthogonalize(x), compute_uv=False)
    assert s.max() <= sup + 1e-12
    assert s.min() >= 0.6818 - 1e-12


def test_ns_cubic_coefficients_converge_to_polar_factor():
    # (1.5, -0.5, 0) is the classic cubic iteration for the polar factor U V^T.
    r = rng(3)
    u, _ = np.linalg.qr(r.standard_normal((24, 24)))
    v, _ = np.linalg.qr(r.standard_normal((40, 24)))
    s = np.linspace(0.1, 1.0, 24)
    x = (u * s) @ v.T
    got = ns_orthogonalize(x, steps=40, coeffs=(1.5, -0.5, 0.0))
    assert relF(got, u @ v.T) <= 1e-12


def test_ns_quintic_within_convergence_band_of_polar_factor():
    r = rng(4)
    u, _ = np.linalg.qr(r.standard_normal((16, 16)))
    v, _ = np.linalg.qr(r.standard_normal((48, 16)))
    s = np.linspace(0.2, 2.0, 16)
    x = (u * s) @ v.T
    sh = np.linalg.svd(x / (np.linalg.norm(x) + 1e-7), compute_uv=False)
    bound = np.abs(p(sh, 5) - 1).max()
    err = np.linalg.norm(ns_orthogonalize(x) - u @ v.T, 2)
    assert err <= bound + 1e-12
    assert bound < 0.32


def test_ns_rank_one_closed_form():
    r = rng(5)
    a = r.standard_normal(7)
    b = r.standard_normal(11)
    x = np.outer(a, b)
    nu = np.linalg.norm(a) * np.linalg.norm(b)
    sig = nu / (nu + f32_param(1e-7))
    ref = p(sig, 5) * np.outer(a / np.linalg.norm(a), b / np.linalg.norm(b))
    assert relF(ns_orthogonalize(x), ref) <= 1e-13
    # trajectory of the scalar map from sigma = 1
    traj = [1.0]
    for _ in range(5):
        traj.append(float(p(traj[-1])))
    np.testing.assert_allclose(traj[1:], [0.701, 1.11362, 0.72071, 1.08997, 0.69644],
                               atol=1e-5)
    # 1x1 matrix: O = p^5(|v|/(|v|+eps)) * sign(v)
    for val in (3.0, -0.25):
        o = ns_orthogonalize(np.array([[val]]))
        assert abs(o[0, 0] - np.sign(val) * p(abs(val) / (abs(val) + f32_param(1e-7)), 5)) < 1e-14


def test_ns_page_association_equals_factored_form():
    for shape in [(16, 40), (40, 16), (33, 33)]:
        x = rng(6).standard_normal(shape)
        assert relF(ns_orthogonalize(x), ns_orthogonalize_page_form(x)) <= 1e-13


def _torch_bf16_page_routine(x, steps=5, eps=1e-7):
    """The appendix association run with torch's own bfloat16 CPU tensor
    arithmetic (an independent implementation of bf16 rounding: float32
    arithmetic per operation, then round to nearest even)."""
    a, b, c = (np.float32(t) for t in (3.4445, -4.7750, 2.0315))
    X = torch.from_numpy(x).to(torch.bfloat16)
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.t().contiguous()
    X = X / (X.norm() + eps)
    for _ in range(steps):
        A = X @ X.t().contiguous()
        AX = A @ X
        X = float(a) * X + float(b) * AX + float(c) * (A @ AX)
    if tall:
        X = X.t()
    return X.to(torch.float64).numpy()


@pytest.mark.parametrize("shape", [(48, 80), (80, 48), (64, 64)])
def test_page_bf16_model_matches_torch_bf16_arithmetic(shape):
    """The bf16 model of the appendix routine against torch's bf16 tensor ops
    on the same input: the same rounding points give results far closer to
    each other than either is to the exact iteration (a dropped or extra
    rounding point, or a wrong association, would not)."""
    rng = np.random.default_rng(41)
    x = rng.standard_normal(shape)
    mine = ns_orthogonalize_page_bf16(x)
    ref = _torch_bf16_page_routine(x)
    exact = ns_orthogonalize(x)
    d_mine, d_ref = relF(mine, exact), relF(ref, exact)
    assert 1e-2 <= d_mine <= 5e-2 and 1e-2 <= d_ref <= 5e-2
    assert relF(mine, ref) <= 0.35 * min(d_mine, d_ref)


def test_split_bf16_carries_sixteen_bits():
    """hi + lo reproduces every value of at most 15 significant bits exactly,
    and any value within 2^-17 of its magnitude (hi is off by at most 2^-9,
    lo by 2^-9 of that)."""
    rng = np.random.default_rng(43)
    m = rng.integers(-(2 ** 15) + 1, 2 ** 15, 20000).astype(np.float64)
    x = np.ldexp(m, rng.integers(-40, 10, m.size))
    assert np.array_equal(split_bf16(x), x)
    y = rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))
    assert (np.abs(split_bf16(y) - y) <= 2.0 ** -17 * np.abs(y)).all()
    assert (round_bf16(y) != y).mean() > 0.99   # the high part alone is not enough


def _illconditioned(rng, m, n, lo=1e-4):
    """U diag(s) V^T with orthonormal U, V (QR of Gaussians) and singular values
    log-uniform in [lo, 1]."""
    k = min(m, n)
    u = np.linalg.qr(rng.standard_normal((m, k)))[0]
    v = np.linalg.qr(rng.standard_normal((n, k)))[0]
    s = np.exp(rng.uniform(np.log(lo), 0.0, k))
    return (u * s) @ v.T


@pytest.mark.parametrize("shape", [(64, 128), (128, 96), (48, 48)])
def test_split_model_reaches_exact_tolerance_where_bf16_cannot(shape):
    """On ill-conditioned inputs the bf16 storage model lies several 1e-2 from
    the exact iteration (pinned by the SVD closed form); carrying the iterate
    as hi + lo into the products with X brings it within 2e-2 -- a dropped low
    part would leave it at the bf16 level."""
    rng = np.random.default_rng(47)
    x = _illconditioned(rng, *shape)
    exact = ns_orthogonalize(x)
    e_bf16 = relF(ns_orthogonalize(x, rounding="bf16"), exact)
    e_split = relF(ns_orthogonalize(x, rounding="bf16_split"), exact)
    assert e_bf16 >= 2.5e-2
    assert e_split <= 1.5e-2
    # one step has no stored iterate yet: the split model is the bf16 model
    assert np.array_equal(ns_orthogonalize(x, steps=1, rounding="bf16_split"),
                          ns_orthogonalize(x, steps=1, rounding="bf16"))


def test_ns_transpose_equivariance():
    for shape in [(12, 30), (30, 12), (1, 9)]:
        x = rng(7).standard_normal(shape)
        assert np.array_equal(ns_orthogonalize(x.T), ns_orthogonalize(x).T)
    # the tall branch agrees with the closed form of the untransposed matrix
    x = rng(8).standard_normal((50, 20))
    assert relF(ns_orthogonalize(x), svd_closed_form(x, 5)) <= 1e-12


def test_ns_orthogonal_invariance():
    r = rng(9)
    x = r.standard_normal((20, 36))
    q1, _ = np.linalg.qr(r.standard_normal((20, 20)))
    q2, _ = np.linalg.qr(r.standard_normal((36, 36)))
    lhs = ns_orthogonalize(q1 @ x @ q2)
    rhs = q1 @ ns_orthogonalize(x) @ q2
    assert relF(lhs, rhs) <= 1e-12


def test_diagonal_gram_links_muon_and_rmnp():
    # V = diag(d) Q with orthonormal rows: V V^T is diagonal, and Muon's
    # direction is row-wise RMNP scaled by p^k of each row's singular value.
    r = rng(10)
    q, _ = np.linalg.qr(r.standard_normal((40, 12)))
    q = q.T                                  # 12 x 40, orthonormal rows
    d = r.uniform(0.5, 2.0, 12) * np.sign(r.standard_normal(12))
    v = d[:, None] * q
    gram = v @ v.T
    assert np.abs(gram - np.diag(np.diag(gram))).max() < 1e-13
    sig = np.abs(d) / (np.linalg.norm(d) + f32_param(1e-7))
    o = ns_orthogonalize(v)
    u = rmnp_direction(v)
    assert relF(o, p(sig, 5)[:, None] * u) <= 1e-13
    # with the cubic polar iteration both directions coincide
    o_polar = ns_orthogonalize(v, steps=60, coeffs=(1.5, -0.5, 0.0))
    assert relF(o_polar, u) <= 1e-12


def test_ns_zero_matrix():
    o = ns_orthogonalize(np.zeros((4, 9)))
    assert np.array_equal(o, np.zeros((4, 9)))


def test_ns_steps_zero_is_normalisation():
    x = rng(11).standard_normal((6, 10))
    ref = x / (np.linalg.norm(x) + f32_param(1e-7))
    assert relF(ns_orthogonalize(x, steps=0), ref) <= 1e-15
    assert relF(ns_orthogonalize(x, steps=0, rounding="bf16"), ref) <= 1e-15


# --------------------------------------------------------------------------
# bf16 storage model
# --------------------------------------------------------------------------

def test_bf16_model_rounds_exactly_a_b_and_iterates():
    # x has orthonormal rows scaled by 1 (4 of 8 unit columns), ||x||_F = 2 and
    # eps = 0, so the Frobenius scale is exactly 1/2 and X X^T = I.  One step:
    # A = I/4 (bf16-exact), B = (a + b/4 + c/16) I (rounded to bf16), and the
    # last iterate 0.5 * B x is not rounded.
    x = np.zeros((4, 8))
    x[np.arange(4), [1, 3, 5, 7]] = 1.0
    model = ns_orthogonalize(x, steps=1, eps=0.0, rounding="bf16")
    p1 = A + B * 0.25 + C * 0.0625
    b_model = round_bf16(p1)
    assert b_model != p1
    assert np.array_equal(model, 0.5 * b_model * x)
    exact = ns_orthogonalize(x, steps=1, eps=0.0)
    assert np.allclose(exact, 0.5 * p1 * x, rtol=1e-15, atol=0)
    # two steps: the first iterate is rounded to bf16 before the second step
    x1 = round_bf16(0.5 * b_model)
    a2 = round_bf16(x1 * x1)
    b2 = round_bf16(A + B * a2 + C * a2 * a2)
    ref2 = (b2 * x1) * x
    assert np.array_equal(ns_orthogonalize(x, steps=2, eps=0.0, rounding="bf16"), ref2)


def test_bf16_model_close_to_exact_on_gaussian():
    x = round_bf16(rng(12).standard_normal((64, 192)) * 1e-3)
    e = ns_orthogonalize(x)
    m = ns_orthogonalize(x, rounding="bf16")
    err = relF(m, e)
    assert 1e-4 < err < 2e-2


# --------------------------------------------------------------------------
# full Muon step
# --------------------------------------------------------------------------

def test_momentum_heavy_ball_and_mu_zero():
    r = rng(13)
    v = r.standard_normal((5, 7))
    g = r.standard_normal((5, 7))
    got = momentum(v, g, 0.95, "f32")
    ref = (np.float64(np.float32(0.95)) * v + g).astype(np.float32).astype(np.float64)
    assert np.array_equal(got, ref)
    gb = round_bf16(g)
    assert np.array_equal(momentum(v, gb, 0.0, "bf16"), gb)


@pytest.mark.parametrize("shape,scale", [((8, 2), 2.0), ((2, 8), 1.0), ((18, 2), 3.0),
                                         ((6, 6), 1.0)])
def test_muon_step_update_and_scale(shape, scale):
    r = rng(14)
    w = r.standard_normal(shape) * 0.02
    v = r.standard_normal(shape)
    g = r.standard_normal(shape)
    w_new, v_new, o = muon_step(w, g, v, mu=0.9, lr=0.5, dtype="f32")
    v_ref = (np.float64(np.float32(0.9)) * v + g).astype(np.float32).astype(np.float64)
    assert np.array_equal(v_new, v_ref)
    o_ref = svd_closed_form(v_ref, 5)
    assert relF(o, o_ref) <= 1e-12
    w_ref = (w - 0.5 * scale * o).astype(np.float32).astype(np.float64)
    np.testing.assert_allclose(w_new, w_ref, rtol=0, atol=1e-6)


def test_muon_step_lr_zero_leaves_weights():
    r = rng(15)
    w = round_bf16(r.standard_normal((6, 9)) * 0.02)
    w_new, _, _ = muon_step(w, r.standard_normal((6, 9)), r.standard_normal((6, 9)),
                            lr=0.0, dtype="bf16")
    assert np.array_equal(w_new, w)


def test_muon_step_zero_momentum_and_gradient():
    w = round_bf16(rng(16).standard_normal((5, 11)) * 0.02)
    z = np.zeros((5, 11))
    w_new, v_new, o = muon_step(w, z, z, dtype="bf16")
    assert not v_new.any() and not o.any()
    assert np.array_equal(w_new, w)


def test_muon_step_weight_decay_alone_scales_weights():
    # zero momentum and gradient: O = 0, so the step is W (1 - lr wd), one
    # rounding; lr = wd = 0.5 makes the factor 0.75 exact.  Expected from
    # torch's own bfloat16 conversion.
    torch = pytest.importorskip("torch")
    w = torch.from_numpy(rng(40).standard_normal((7, 12)) * 0.02).to(torch.bfloat16)
    z = np.zeros((7, 12))
    w_new, _, o = muon_step(w.double().numpy(), z, z, lr=0.5, wd=0.5, dtype="bf16")
    assert not o.any()
    exp = (w.double() * 0.75).to(torch.bfloat16).double().numpy()
    assert np.array_equal(w_new, exp)


@pytest.mark.parametrize("shape,scale", [((8, 2), 2.0), ((2, 8), 1.0)])
def test_muon_step_weight_decay_is_decoupled(shape, scale):
    # W_new = W - lr (wd W + s O) with O from the SVD closed form: the decay
    # multiplies W by lr*wd and is added to the scaled direction, not to it
    # before orthogonalisation.
    r = rng(41)
    w = r.standard_normal(shape) * 0.02
    v = r.standard_normal(shape)
    g = r.standard_normal(shape)
    w_new, v_new, _ = muon_step(w, g, v, mu=0.5, lr=0.25, wd=0.5, steps=2, dtype="f32")
    o_ref = svd_closed_form(v_new, 2)
    w_ref = (w - 0.25 * (0.5 * w + scale * o_ref)).astype(np.float32).astype(np.float64)
    np.testing.assert_allclose(w_new, w_ref, rtol=0, atol=1e-6)
    w0, _, _ = muon_step(w, g, v, mu=0.5, lr=0.25, wd=0.0, steps=2, dtype="f32")
    np.testing.assert_allclose(w_new - w0, -0.125 * w, rtol=0, atol=1e-6)


# --------------------------------------------------------------------------
# RMNP
# --------------------------------------------------------------------------

def test_rmnp_unit_rows_and_library_normalize():
    torch = pytest.importorskip("torch")
    x = rng(17).standard_normal((30, 70))
    u = rmnp_direction(x)
    np.testing.assert_allclose(np.linalg.norm(u, axis=1), 1.0, atol=1e-15)
    ref = torch.nn.functional.normalize(torch.from_numpy(x), p=2, dim=-1).numpy()
    assert np.abs(u - ref).max() <= 1e-15


def test_rmnp_row_split_invariance_exact():
    # the blog post's exactness check: 512x384, 8 row shards, max |diff| = 0
    x = np.random.default_rng(7).standard_normal((512, 384))
    full = rmnp_direction(x)
    for k in range(8):
        sl = slice(k * 64, (k + 1) * 64)
        assert np.array_equal(rmnp_direction(x[sl]), full[sl])


def test_rmnp_zero_row_gives_zero_update():
    r = rng(18)
    w = round_bf16(r.standard_normal((4, 16)) * 0.02)
    v = round_bf16(r.standard_normal((4, 16)))
    g = round_bf16(r.standard_normal((4, 16)))
    v[2] = 0.0
    g[2] = 0.0
    w_new, v_new, u = rmnp_step(w, g, v, dtype="bf16")
    assert not u[2].any()
    assert np.array_equal(w_new[2], w[2])
    np.testing.assert_allclose(np.linalg.norm(u[[0, 1, 3]], axis=1), 1.0, atol=1e-15)


def test_rmnp_step_scale_tall():
    r = rng(19)
    w = r.standard_normal((32, 8)) * 0.02
    v = r.standard_normal((32, 8))
    g = r.standard_normal((32, 8))
    w_new, v_new, u = rmnp_step(w, g, v, mu=0.95, lr=0.1, dtype="f32")
    ref = (w - 0.1 * 2.0 * v_new / np.linalg.norm(v_new, axis=1, keepdims=True))
    np.testing.assert_allclose(w_new, ref.astype(np.float32), rtol=0, atol=1e-7)


# --------------------------------------------------------------------------
# Column-cut RMNP (local halves)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("shape,cuts", [((12, 40), [0, 7, 20, 40]), ((40, 12), [0, 5, 12]),
                                        ((9, 9), [0, 9])])
def test_rmnp_colcut_slices_reproduce_the_row_local_step(shape, cuts):
    # A row's squared norm is the sum of its slices' squared norms: partials
    # summed over the slices, then each slice updated with the whole matrix's
    # scale, give the row-local RMNP step (pinned against torch's normalize).
    r = rng(50)
    w = r.standard_normal(shape) * 0.02
    v = r.standard_normal(shape)
    g = r.standard_normal(shape)
    parts = [oracle.rmnp_colcut_partial(v[:, a:b], g[:, a:b], mu=0.9, dtype="f32")
             for a, b in zip(cuts[:-1], cuts[1:])]
    rowsq = sum(pp[1] for pp in parts)
    w_cut = np.concatenate([oracle.rmnp_colcut_apply(w[:, a:b], pp[0], rowsq, lr=0.3,
                                                     eps=1e-7, full_cols=shape[1], dtype="f32")
                            for (a, b), pp in zip(zip(cuts[:-1], cuts[1:]), parts)], axis=1)
    w_ref, v_ref, _ = oracle.rmnp_step(w, g, v, mu=0.9, lr=0.3, eps=1e-7, dtype="f32")
    assert np.array_equal(np.concatenate([pp[0] for pp in parts], axis=1), v_ref)
    np.testing.assert_allclose(w_cut, w_ref, rtol=0, atol=1e-7)


def test_rmnp_colcut_clamp_and_zero_row():
    # rowsq = 0 leaves W; a norm below the 1e-7 clamp divides by 1e-7 exactly
    w = np.array([[0.5, -0.25], [0.125, 1.0]])
    v = np.array([[0.0, 0.0], [3e-9, 4e-9]])   # second row norm 5e-9 < 1e-7
    rowsq = np.array([0.0, 25e-18])
    out = oracle.rmnp_colcut_apply(w, v, rowsq, lr=0.5, eps=1e-7, dtype="f32")
    eps = float(np.float32(1e-7))
    exp = np.array([[0.5, -0.25], [0.125 - 0.5 * 3e-9 / eps, 1.0 - 0.5 * 4e-9 / eps]])
    np.testing.assert_allclose(out, exp.astype(np.float32), rtol=0, atol=1e-7)


# --------------------------------------------------------------------------
# AdamW for the non-2D tail
# --------------------------------------------------------------------------

@pytest.mark.parametrize("step", [1, 7])
def test_adamw_matches_torch_adamw_in_float64(step):
    # the standard form as torch.optim.AdamW computes it (single-tensor path),
    # with the same float32 hyperparameters, mid-run state for step > 1
    torch = pytest.importorskip("torch")
    r = rng(60)
    p0 = r.standard_normal(257)
    g = r.standard_normal(257) * 0.1
    m0 = r.standard_normal(257) * 0.01 if step > 1 else np.zeros(257)
    v0 = np.abs(r.standard_normal(257)) * 1e-3 if step > 1 else np.zeros(257)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=1e-2)
    f = {k: f32_param(x) for k, x in hp.items()}
    prm = torch.nn.Parameter(torch.tensor(p0, dtype=torch.float64))
    prm.grad = torch.tensor(g, dtype=torch.float64)
    opt = torch.optim.AdamW([prm], lr=f["lr"], betas=(f["beta1"], f["beta2"]), eps=f["eps"],
                            weight_decay=f["wd"], foreach=False)
    opt.state[prm] = {"step": torch.tensor(float(step - 1)),
                      "exp_avg": torch.tensor(m0, dtype=torch.float64),
                      "exp_avg_sq": torch.tensor(v0, dtype=torch.float64)}
    opt.step()
    p_new, m_new, v_new = oracle.adamw_step(p0, g, m0, v0, step, dtype="f64", **hp)
    np.testing.assert_allclose(m_new, opt.state[prm]["exp_avg"].numpy(), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(v_new, opt.state[prm]["exp_avg_sq"].numpy(), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(p_new, prm.detach().numpy(), rtol=1e-13, atol=0)


def test_adamw_first_step_is_a_signed_step():
    # t = 1 from zero state and no decay: m_hat = g, v_hat = g^2, so the
    # update is lr g / (|g| + eps)
    g = np.array([3.0, -0.5, 1e-9, 0.0])
    p0 = np.array([1.0, 2.0, -3.0, 4.0])
    p_new, m_new, v_new = oracle.adamw_step(p0, g, np.zeros(4), np.zeros(4), 1, lr=0.5, wd=0.0,
                                            eps=1e-8, dtype="f64")
    eps = f32_param(1e-8)
    b1 = f32_param(0.9)
    np.testing.assert_allclose(m_new, (1 - b1) * g, rtol=1e-15)
    np.testing.assert_allclose(p0 - p_new, 0.5 * g / (np.abs(g) + eps), rtol=1e-12, atol=1e-300)
