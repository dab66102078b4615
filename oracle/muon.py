"""Oracle: the owner-local Muon step and the RMNP comparator, in float64 numpy.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the product path never
imports this module.

What is computed, and where the pages define it
------------------------------------------------
Blog post "Optimizers In A Sharded World: Muon's O(mn) Vs RMNP's Zero":

* Section 1: momentum is heavy ball, ``V_t = mu * V_{t-1} + G_t``; Muon's target
  direction is the orthogonalized ``(V V^T)^{-1/2} V``, approximated by five
  Newton-Schulz iterations of three matrix products each; RMNP's direction
  divides each row of ``V_t`` by its L2 norm.
* Appendix "The Code That Ran": the Newton-Schulz routine (coefficients
  (3.4445, -4.7750, 2.0315), 5 steps, ``eps = 1e-7`` added to the Frobenius
  norm, transpose when rows > cols and back at the end); the ``muon_sc`` step
  (momentum in place, Newton-Schulz on the updated momentum, update scaled by
  ``sqrt(max(1, rows/cols))``); the ``rmnp_local`` step (momentum in place,
  fp32 row normalisation with the library default ``max(||v||, 1e-12)``
  clamp, the same update scale).

* Section 3, the column-cut layout, and the appendix's ``rmnp_colcut``: each
  rank holds a column slice of every matrix, computes one partial sum of
  squares per row of its updated momentum slice, the partials of all matrices
  are summed over the ranks, and each slice is divided by the clamped root
  (``max(sqrt(.), 1e-7)``).  ``rmnp_colcut_partial`` and ``rmnp_colcut_apply``
  are the two local halves on one slice; the sum over ranks happens between
  them.

MatrixFSDP (arXiv 2607.05895), section 3 and section 4.4: each owner applies
this update to the whole 2D matrices it owns, independently per matrix; there
is no cross-matrix coupling, which is why every function below works on one
matrix at a time.  Section 5.1: the training configuration adds weight decay
1e-2 (with momentum 0.5 and two Newton-Schulz steps); ``muon_step`` takes it
as decoupled decay, ``W - lr (wd W + s O)``.  The same section puts the
non-2D tail on AdamW (``adamw_step``, the standard form; its formula is not on
the pages).

Readings taken where the pages leave a step open (each is listed in the design
notes with its reason):

* The iteration is written in the factored form ``A = X X^T``,
  ``B = p(A) = a I + b A + c A A``, ``X = B X`` -- the quintic polynomial in A,
  then its product with X.  The appendix associates the same polynomial the
  other way, applying A to X and then to that product (``a X + b (A X) +
  c A (A X)``); the two agree in exact arithmetic, which
  ``ns_orthogonalize_page_form`` pins.  ``ns_orthogonalize_page_bf16`` is that
  association in the appendix routine's own precision (bf16 tensors, each
  result rounded), the yardstick for what bf16 storage costs on a given input.
* Scalar parameters are the float32 values a caller passes through the C ABI,
  widened exactly to float64 (``f32_param``).
* Momentum is rounded once to the storage dtype (the page rounds twice, once per
  in-place op); the update ``W - lr*s*O`` is rounded once.
* Newton-Schulz consumes the *stored* updated momentum.
* ``rounding="bf16"`` is the bf16 storage model: the tensors a bf16 engine keeps
  in bf16 between matrix products are rounded to bf16 (round to nearest even) at
  exactly those points -- A, the polynomial B = p(A) (with a on its diagonal)
  and every iterate except the last -- while the Frobenius scale
  ``1/(||V||+eps)`` is carried as an exact factor into the first iteration's
  products instead of being rounded into a bf16 copy of V.  All accumulation
  stays float64.  ``rounding="exact"`` rounds nothing.
* ``rounding="bf16_split"`` is the same model with each iterate after the first
  kept as a bf16 high part plus a bf16 low part (``split_bf16``): the Gram
  reads the high part alone, the product ``B X`` both parts.

Parity status
-------------
Every public function here is pinned by ``tests/test_oracle_pins.py`` against
closed forms (the SVD action of the iteration on singular values, the rank-1
trajectory, the cubic polar iteration, orthogonal and transpose equivariance,
the diagonal-Gram identity linking Muon and RMNP, degenerate parameters, exact
row-split invariance of RMNP) and against library routines (numpy/LAPACK SVD,
torch's bfloat16 conversion).  No function is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

# Constants printed in the blog post's appendix ("The Code That Ran").
NS_COEFFS = (3.4445, -4.7750, 2.0315)
NS_STEPS = 5
NS_EPS = 1e-7
MOMENTUM = 0.95
# The row normalisation in the appendix calls the library default clamp.
RMNP_EPS = 1e-12
# The column-cut RMNP listing clamps the all-reduced norm at 1e-7.
RMNP_COLCUT_EPS = 1e-7


def f32_param(p: float) -> float:
    """The float32 value of a scalar parameter, widened exactly to float64."""
    return float(np.float32(p))


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def round_bf16(x) -> np.ndarray:
    """Nearest bfloat16 value of each entry (ties to even), returned as float64.

    bfloat16 keeps 8 significant bits.  ``frexp`` writes ``x = m * 2**e`` with
    ``0.5 <= |m| < 1``; ``m * 256`` then has 8 integer bits and ``rint`` rounds it
    half-to-even.  A carry to ``|m| = 1`` is exact under ``ldexp``.  Valid for the
    normal bfloat16 range (|x| >= 2**-126); zeros, infinities and NaN pass
    through.  Subnormal and overflowing magnitudes never occur in this workload.
    """
    x = _f64(x)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def round_storage(x, dtype: str) -> np.ndarray:
    """Round to the storage dtype ('bf16' or 'f32'); returned as float64."""
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return _f64(x).astype(np.float32).astype(np.float64)
    raise ValueError(f"unknown storage dtype {dtype!r}")


def split_bf16(x) -> np.ndarray:
    """``hi + lo`` with ``hi`` the nearest bfloat16 of each entry and ``lo`` the
    nearest bfloat16 of ``x - hi``: about 16 significant bits."""
    hi = round_bf16(x)
    return hi + round_bf16(_f64(x) - hi)


def momentum(v, g, mu: float, dtype: str) -> np.ndarray:
    """Heavy-ball momentum ``V_t = mu V_{t-1} + G_t`` (blog post, section 1),
    rounded once to the storage dtype."""
    return round_storage(f32_param(mu) * _f64(v) + _f64(g), dtype)


def frobenius_scale(v, eps: float = NS_EPS) -> float:
    """``1 / (||V||_F + eps)``: the normalisation that opens the appendix's
    Newton-Schulz routine (eps added to the norm, not a clamp)."""
    v = _f64(v)
    return 1.0 / (float(np.sqrt(np.sum(v * v))) + f32_param(eps))


def update_scale(rows: int, cols: int) -> float:
    """``sqrt(max(1, rows/cols))`` on the matrix's own shape (appendix, the
    ``muon_sc`` and ``rmnp_local`` steps)."""
    return float(np.sqrt(max(1.0, rows / cols)))


def ns_orthogonalize(x, steps: int = NS_STEPS, coeffs=NS_COEFFS,
                     eps: float = NS_EPS, rounding: str = "exact") -> np.ndarray:
    """Newton-Schulz orthogonalization of one matrix (appendix routine, factored).

    1. ``X0 = x / (||x||_F + eps)``.
    2. If rows > cols (strict), work on the transpose.
    3. ``steps`` times: ``A = X X^T``; ``B = a I + b A + c A A``; ``X = B X``.
    4. Transpose back.

    ``rounding="bf16"`` applies the bf16 storage model described in the module
    header, ``rounding="bf16_split"`` its split-iterate variant; the returned
    matrix (the last iterate) is never rounded.
    """
    if rounding not in ("exact", "bf16", "bf16_split"):
        raise ValueError(rounding)
    a, b, c = (f32_param(t) for t in coeffs)
    x = _f64(x)
    rows, cols = x.shape
    scale = frobenius_scale(x, eps)
    tall = rows > cols
    X = x.T if tall else x
    if rounding == "exact":
        X = X * scale
        s = 1.0
    else:
        s = scale  # carried exactly into the first iteration's products
    eye = np.eye(X.shape[0])
    rounded = rounding != "exact"
    for k in range(steps):
        Xg = Xb = X
        if rounding == "bf16_split" and k > 0:   # the stored iterate: hi, and hi + lo
            Xg = round_bf16(X)
            Xb = split_bf16(X)
        A = (s * s) * (Xg @ Xg.T)
        if rounded:
            A = round_bf16(A)
        B = a * eye + b * A + c * (A @ A)
        if rounded:
            B = round_bf16(B)
        Xn = s * (B @ Xb)
        if rounding == "bf16" and k < steps - 1:
            Xn = round_bf16(Xn)
        X = Xn
        s = 1.0
    X = s * X  # only ns_steps == 0 leaves the scale unapplied
    return X.T if tall else X


def ns_orthogonalize_page_form(x, steps: int = NS_STEPS, coeffs=NS_COEFFS,
                               eps: float = NS_EPS) -> np.ndarray:
    """The iteration with the polynomial associated as the appendix associates
    it: each step applies ``X -> a X + b (A X) + c A (A X)`` with ``A = X X^T``,
    so A meets X twice and no product of A with itself is formed (exact
    arithmetic; normalisation and transposes as in ``ns_orthogonalize``)."""
    a, b, c = (f32_param(t) for t in coeffs)
    x = _f64(x)
    tall = x.shape[0] > x.shape[1]
    X = (x.T if tall else x) * frobenius_scale(x, eps)
    for _ in range(steps):
        A = X @ X.T
        AX = A @ X
        X = a * X + b * AX + c * (A @ AX)
    return X.T if tall else X


def ns_orthogonalize_page_bf16(x, steps: int = NS_STEPS, coeffs=NS_COEFFS,
                               eps: float = NS_EPS) -> np.ndarray:
    """``ns_orthogonalize_page_form`` in the precision the appendix runs it:
    the input cast to bf16, and every tensor the routine produces rounded to
    bf16 -- the norm, the normalised X, A, A X, A (A X), each of the three
    scaled terms and the two sums (products accumulate exactly here, in
    float64, before their one rounding).  Only used to measure how far a
    bf16 implementation of the method itself lies from the exact iteration on
    a given input; the returned matrix is the last rounded iterate."""
    r = round_bf16
    a, b, c = (f32_param(t) for t in coeffs)
    x = r(_f64(x))
    tall = x.shape[0] > x.shape[1]
    X = x.T if tall else x
    X = r(X / r(r(np.sqrt(np.sum(X * X))) + f32_param(eps)))
    for _ in range(steps):
        A = r(X @ X.T)
        AX = r(A @ X)
        AAX = r(A @ AX)
        X = r(r(r(a * X) + r(b * AX)) + r(c * AAX))
    return X.T if tall else X


def muon_step(w, g, v, mu: float = MOMENTUM, lr: float = 0.02,
              steps: int = NS_STEPS, coeffs=NS_COEFFS, eps: float = NS_EPS,
              dtype: str = "bf16", rounding: str = "exact", wd: float = 0.0):
    """One owner-local Muon step on one whole matrix.

    ``V_new = round(mu V + G)``; ``O = NS(V_new)``;
    ``W_new = round(W - lr * (wd * W + sqrt(max(1, rows/cols)) * O))``.
    ``wd`` is decoupled weight decay, 0 in the blog post's step; the MatrixFSDP
    paper trains with weight decay 1e-2, momentum 0.5 and two Newton-Schulz
    steps (section 5.1), and decoupled is the reading taken for "weight decay"
    there (the decay scales W by lr*wd, apart from the orthogonalized direction).
    Returns ``(W_new, V_new, O)`` as float64 arrays.
    """
    w = _f64(w)
    v_new = momentum(v, g, mu, dtype)
    o = ns_orthogonalize(v_new, steps, coeffs, eps, rounding)
    rows, cols = w.shape
    s = update_scale(rows, cols)
    lr64 = f32_param(lr)
    w_new = round_storage(w - lr64 * (f32_param(wd) * w + s * o), dtype)
    return w_new, v_new, o


def rmnp_direction(v, eps: float = RMNP_EPS) -> np.ndarray:
    """RMNP direction: each row divided by ``max(||row||_2, eps)``
    (blog post, section 1; the clamp is the library default the appendix uses)."""
    v = _f64(v)
    nrm = np.sqrt(np.sum(v * v, axis=1))
    return v / np.maximum(nrm, f32_param(eps))[:, None]


def rmnp_step(w, g, v, mu: float = MOMENTUM, lr: float = 0.02,
              eps: float = RMNP_EPS, dtype: str = "bf16"):
    """One RMNP step on one matrix: momentum, row-normalized direction, update
    scaled by ``sqrt(max(1, rows/cols))`` (appendix, ``rmnp_local``).
    Returns ``(W_new, V_new, U)``."""
    w = _f64(w)
    v_new = momentum(v, g, mu, dtype)
    u = rmnp_direction(v_new, eps)
    rows, cols = w.shape
    s = update_scale(rows, cols)
    w_new = round_storage(w - f32_param(lr) * s * u, dtype)
    return w_new, v_new, u


def rmnp_colcut_partial(v, g, mu: float = MOMENTUM, dtype: str = "bf16"):
    """Column-cut RMNP, the local half on one column slice (blog post, section 3,
    the column-cut layout; appendix ``rmnp_colcut``): momentum on the slice, then
    one partial sum of squares per row of the stored slice.  The row's squared
    norm is the sum of these partials over the slices of the row.
    Returns ``(V_new, rowsq)``."""
    v_new = momentum(v, g, mu, dtype)
    return v_new, np.sum(v_new * v_new, axis=1)


def rmnp_colcut_apply(w, v_new, rowsq, lr: float = 0.02, eps: float = RMNP_COLCUT_EPS,
                      full_cols: int | None = None, dtype: str = "bf16") -> np.ndarray:
    """The update of one column slice once the row sums of squares are summed
    over all slices: ``W - lr sqrt(max(1, rows/full_cols)) V / max(sqrt(rowsq), eps)``
    with the whole matrix's shape in the scale (rows x full_cols) and one
    rounding.  The column-cut listing clamps the norm at 1e-7."""
    w = _f64(w)
    rows, cols = w.shape
    s = update_scale(rows, cols if full_cols is None else full_cols)
    u = _f64(v_new) / np.maximum(np.sqrt(_f64(rowsq)), f32_param(eps))[:, None]
    return round_storage(w - f32_param(lr) * s * u, dtype)


def adamw_step(p, g, m, v, step: int, lr: float = 1e-3, beta1: float = 0.9,
               beta2: float = 0.999, eps: float = 1e-8, wd: float = 1e-2,
               dtype: str = "bf16"):
    """AdamW on one non-2D tensor of the owner's tail.  MatrixFSDP section 5.1
    puts LayerNorm weights and other non-2D tensors on AdamW with lr 1e-3,
    weight decay 1e-2, betas (0.9, 0.999), eps 1e-8 and no schedule; the update
    itself is not written on the pages, so this is the standard decoupled form
    (Loshchilov and Hutter's AdamW, as torch.optim.AdamW computes it):

        m = beta1 m + (1 - beta1) g            (stored as float32)
        v = beta2 v + (1 - beta2) g^2          (stored as float32)
        p = p - lr wd p - lr/(1 - beta1^t) m / (sqrt(v)/sqrt(1 - beta2^t) + eps)

    using the stored m and v in the last line, rounded once to ``dtype``
    ('bf16', 'f32', or 'f64' for no rounding).  ``step`` is t >= 1, the count
    of steps including this one.  Returns ``(p_new, m_new, v_new)``."""
    p, g, m, v = _f64(p), _f64(g), _f64(m), _f64(v)
    b1, b2 = f32_param(beta1), f32_param(beta2)
    m_new = b1 * m + (1.0 - b1) * g
    v_new = b2 * v + (1.0 - b2) * g * g
    if dtype != "f64":
        m_new = round_storage(m_new, "f32")
        v_new = round_storage(v_new, "f32")
    lr64 = f32_param(lr)
    bc1 = 1.0 - b1 ** step
    bc2 = 1.0 - b2 ** step
    denom = np.sqrt(v_new) / np.sqrt(bc2) + f32_param(eps)
    p_new = p - lr64 * f32_param(wd) * p - (lr64 / bc1) * m_new / denom
    if dtype != "f64":
        p_new = round_storage(p_new, dtype)
    return p_new, m_new, v_new
