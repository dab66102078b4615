"""GPU parity at the largest shapes the boundary accepts (a side of 2^20, or
rows x cols up to 2^32 elements), where every offset into the caller's
matrices and the workspace needs 64 bits.

Such a matrix is far beyond the float64 oracle, so each one carries a few
small Gaussian blocks with pairwise disjoint rows and columns, zero
elsewhere, placed at the start, the middle and the very end of the matrix.
The Newton-Schulz iteration acts on such a matrix block by block: X X^T is
block diagonal, so is every polynomial of it, and rows and columns that are
zero stay zero; the Frobenius scale is that of the blocks alone.  The
expected result is therefore the oracle's iteration on the small
block-diagonal matrix made of the same blocks, computed exactly.

One Muon step per shape (momentum, Newton-Schulz, fused weight update), in
bf16 storage at every shape and in float32 at the longest side:
* V: the blocks bit-exact against the oracle's momentum, zero elsewhere;
* W: zero on the blocks before the step, so that afterwards they hold
  round(-lr * sqrt(max(1, rows/cols)) * O) and O can be read back, compared
  with the oracle at relative Frobenius error <= 2e-2 (bf16) or 1e-4
  (float32); a constant elsewhere,
  which must be untouched bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.helpers import f64, relF, ulp_distance

pytestmark = pytest.mark.gpu

W_FILL = 0.015625   # exact in bfloat16
MU, LR = 0.95, 0.02

# (rows, cols, blocks as (row0, col0, height, width)); rows and columns of the
# blocks are pairwise disjoint
CASES = [
    # largest square under 2^32 elements; padded to 65536 (a ragged last tile)
    (65535, 65535, [(0, 0, 40, 24), (32000, 40000, 33, 57), (65535 - 35, 65535 - 29, 35, 29)]),
    # 2^32 elements, longest side 2^20, transposed inside the library
    (1 << 20, 4096, [(0, 100, 64, 32), (1 << 19, 2000, 48, 40), ((1 << 20) - 50, 4096 - 20, 50, 20)]),
    # the same wide: X0 read in place, a 2^20-long K loop in the Gram
    (4096, 1 << 20, [(0, 0, 30, 70), (2048, 600000, 25, 60), (4096 - 22, (1 << 20) - 45, 22, 45)]),
    # one row of 2^20 elements
    (1, 1 << 20, [(0, (1 << 20) - 300, 1, 300)]),
]


@pytest.fixture(scope="module")
def mo():
    import matrix_optimizer_step_amd as m
    m.lib()   # raises if the library is missing: no fallback
    return m


def _block_diag(mats):
    r = sum(m.shape[0] for m in mats)
    c = sum(m.shape[1] for m in mats)
    out = np.zeros((r, c))
    i = j = 0
    for m in mats:
        out[i:i + m.shape[0], j:j + m.shape[1]] = m
        i += m.shape[0]
        j += m.shape[1]
    return out


# float32 storage at the largest side (float32 products throughout)
CASES_F32 = [CASES[1], CASES[3]]
TOL = {"bf16": 2e-2, "f32": 1e-4}


@pytest.mark.parametrize("dt,rows,cols,blocks",
                         [("bf16",) + c for c in CASES] + [("f32",) + c for c in CASES_F32],
                         ids=[f"bf16-{r}x{c}" for r, c, _ in CASES]
                         + [f"f32-{r}x{c}" for r, c, _ in CASES_F32])
def test_block_matrix_at_maximum_size(mo, dt, rows, cols, blocks):
    print(f"[maxsize] {dt} {rows} x {cols}, {len(blocks)} blocks", flush=True)
    rng = np.random.default_rng(rows * 7 + cols)
    dev = "cuda"
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    W = torch.full((rows, cols), W_FILL, dtype=tdt, device=dev)
    G = torch.zeros((rows, cols), dtype=tdt, device=dev)
    V = torch.zeros((rows, cols), dtype=tdt, device=dev)
    g_blk, v_blk = [], []
    for (r0, c0, h, w) in blocks:
        g = torch.from_numpy(rng.standard_normal((h, w))).to(tdt)
        v = torch.from_numpy(rng.standard_normal((h, w))).to(tdt)
        G[r0:r0 + h, c0:c0 + w] = g.to(dev)
        V[r0:r0 + h, c0:c0 + w] = v.to(dev)
        W[r0:r0 + h, c0:c0 + w] = 0
        g_blk.append(g)
        v_blk.append(v)
    ws = torch.empty(mo.workspace_bytes([(rows, cols)], tdt), dtype=torch.uint8, device=dev)
    mo.muon_step_batched([W], [G], [V], mu=MU, lr=LR, ns_steps=5, workspace=ws)
    torch.cuda.synchronize()
    del ws, G
    print("[maxsize] step done on the GPU", flush=True)

    # momentum: bit-exact on the blocks, zero elsewhere
    v_new = []
    for (r0, c0, h, w), v0, g in zip(blocks, v_blk, g_blk):
        exp = oracle.momentum(f64(v0), f64(g), MU, dt)
        got = V[r0:r0 + h, c0:c0 + w].cpu()
        assert ulp_distance(got, torch.from_numpy(exp).to(tdt)).max() == 0
        v_new.append(exp)
        V[r0:r0 + h, c0:c0 + w] = 0
    assert int(torch.count_nonzero(V)) == 0, "momentum written outside the blocks"
    del V

    # the update on the blocks against the exact iteration on the compact matrix
    o_exp = oracle.ns_orthogonalize(_block_diag(v_new))
    step = oracle.f32_param(LR) * oracle.update_scale(rows, cols)
    i = j = 0
    got_all, exp_all = [], []
    for (r0, c0, h, w) in blocks:
        got = -f64(W[r0:r0 + h, c0:c0 + w]) / step
        exp = o_exp[i:i + h, j:j + w]
        got_all.append(got.ravel())
        exp_all.append(exp.ravel())
        # the rest of the compact matrix's rows and columns of this block is zero
        assert np.all(o_exp[i:i + h, :j] == 0) and np.all(o_exp[i:i + h, j + w:] == 0)
        i += h
        j += w
        W[r0:r0 + h, c0:c0 + w] = W_FILL
    err = relF(np.concatenate(got_all), np.concatenate(exp_all))
    print(f"[maxsize] {dt} {rows} x {cols}: relF(O) vs exact {err:.2e}", flush=True)
    assert err <= TOL[dt]
    assert bool(torch.all(W == W_FILL)), "W changed outside the blocks"
    del W
    torch.cuda.empty_cache()
