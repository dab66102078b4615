"""Seeded synthetic inputs for the Muon / RMNP step (shared by tests, bench, smoke).

This module holds no arithmetic of the method: it only lists matrix shapes and
draws seeded random inputs, which both the HIP path and the CPU oracle consume.

Every matrix ``i`` of a workload has its own numpy PCG64 stream seeded with
``SeedSequence([seed, i])``, so one matrix can be regenerated alone (sampled
parity checks) and a whole set can be drawn in parallel.  From that stream the
weight ``W``, the prior momentum ``V`` and the gradient ``G`` are drawn in that
order (the order the blog post's benchmark state draws them), each as float32
``standard_normal * std`` and then rounded to the storage dtype by torch's own
conversion (round to nearest even).  ``N(0, s)`` means standard deviation ``s``.

Workloads (shapes are rows x cols of the stored matrix):

* ``single_f32_256x512``: one fp32 256x512 matrix, G and V ~ N(0,1), W ~ N(0,0.02).
* ``gpt2_large_144``: GPT-2 Large's 144 matrices, 36 layers x {1280x3840,
  1280x1280, 1280x5120, 5120x1280} (hidden 1280; the blog post's GPT-2 Large
  set, in [in, out] orientation), bf16, G and V ~ N(0,1e-3), W ~ N(0,0.02).
* ``llama3_8b_share_28``: 4 layers x {4096x4096 Q, 1024x4096 K, 1024x4096 V,
  4096x4096 O, 14336x4096 gate, 14336x4096 up, 4096x14336 down}, bf16.
* ``ragged_illcond_64``: 64 matrices with power-of-two sides in [128, 8192] and
  aspect ratio within 8:1 either way; each G is ``U diag(s) V^T + 1e-4 noise``
  with random orthogonal U, V (columns of randomly signed Hadamard matrices,
  exactly orthonormal) and singular values log-uniform in [1e-4, 1]; prior
  momentum is zero so the momentum keeps that spectrum; bf16.
* ``qwen32b_share_14``: 2 layers x {5120x5120 Q, 1024x5120 K, 1024x5120 V,
  5120x5120 O, 27648x5120 gate, 27648x5120 up, 5120x27648 down}, bf16.
* ``square_sweep(s)``: one s x s bf16 matrix, s in 1024 .. 8192 (the blog
  post's single-matrix size sweep).
"""

from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get", "matrix_inputs", "workload_inputs",
           "small_case", "square_sweep", "SWEEP_SIZES"]


@dataclass(frozen=True)
class Workload:
    name: str
    shapes: tuple            # ((rows, cols), ...)
    dtype: str               # "bf16" or "f32"
    seed: int
    w_std: float = 0.02
    v_std: float = 1e-3
    g_std: float = 1e-3
    mu: float = 0.95
    lr: float = 0.02
    ns_steps: int = 5
    kind: str = "gaussian"   # or "illcond"
    meta: dict = field(default_factory=dict, compare=False)

    @property
    def numel(self) -> int:
        return sum(r * c for r, c in self.shapes)


def _gpt2_large():
    h = 1280
    layer = ((h, 3 * h), (h, h), (h, 4 * h), (4 * h, h))
    return tuple(layer) * 36


def _llama3_8b_share():
    layer = ((4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096),
             (14336, 4096), (14336, 4096), (4096, 14336))
    return tuple(layer) * 4


def _qwen32b_share():
    layer = ((5120, 5120), (1024, 5120), (1024, 5120), (5120, 5120),
             (27648, 5120), (27648, 5120), (5120, 27648))
    return tuple(layer) * 2


def ragged_shapes(seed: int, count: int = 64, lo_exp: int = 7, hi_exp: int = 13):
    """Power-of-two sides in [2**lo_exp, 2**hi_exp], aspect ratio <= 8 either way:
    for each matrix a row count drawn uniformly from the sides, then a column
    count drawn uniformly from the sides within a factor 8 of it, from one
    PCG64 stream seeded with ``seed`` (seed 4 gives 671,924,224 elements, five
    8192 x 8192 matrices and 18 tall ones)."""
    rng = np.random.default_rng(seed)
    sides = [1 << e for e in range(lo_exp, hi_exp + 1)]
    out = []
    for _ in range(count):
        r = int(rng.choice(sides))
        allowed = [s for s in sides if r <= 8 * s and s <= 8 * r]
        c = int(rng.choice(allowed))
        out.append((r, c))
    return tuple(out)


WORKLOADS = {
    "single_f32_256x512": Workload("single_f32_256x512", ((256, 512),), "f32",
                                   seed=0, w_std=0.02, v_std=1.0, g_std=1.0),
    "gpt2_large_144": Workload("gpt2_large_144", _gpt2_large(), "bf16", seed=1337),
    "llama3_8b_share_28": Workload("llama3_8b_share_28", _llama3_8b_share(), "bf16",
                                   seed=8),
    "ragged_illcond_64": Workload("ragged_illcond_64", ragged_shapes(4), "bf16",
                                  seed=4, v_std=0.0, kind="illcond"),
    "qwen32b_share_14": Workload("qwen32b_share_14", _qwen32b_share(), "bf16",
                                 seed=32),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def small_case(name: str, shapes, dtype="bf16", seed=123, kind="gaussian",
               v_std=1e-3, g_std=1e-3, w_std=0.02) -> Workload:
    """An ad-hoc workload (tests: ragged tails, tiny and edge shapes)."""
    return Workload(name, tuple(tuple(s) for s in shapes), dtype, seed,
                    w_std=w_std, v_std=v_std, g_std=g_std, kind=kind)


SWEEP_SIZES = (1024, 2048, 4096, 8192)


def square_sweep(s: int) -> Workload:
    """One s x s bf16 matrix of the blog post's single-matrix size sweep (sides
    1024 .. 8192): W ~ N(0, 0.02), G and V ~ N(0, 1e-3), seed 1000 + s."""
    return small_case(f"square_sweep_{s}", [(s, s)], seed=1000 + s)


def _to_storage(a32: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t.clone()


def _orthonormal_columns(rng, n: int, k: int) -> np.ndarray:
    """An n x k float32 matrix with exactly orthonormal columns (n a power of
    two): k columns, picked at random, of the Sylvester-Hadamard matrix with
    random row and column signs, scaled by 1/sqrt(n) -- a random orthogonal
    factor that costs no factorisation."""
    from scipy.linalg import hadamard
    cols = rng.permutation(n)[:k]
    h = hadamard(n, dtype=np.int8)[:, cols].astype(np.float32)
    rs = rng.choice(np.array([-1.0, 1.0], np.float32), n)
    cs = rng.choice(np.array([-1.0, 1.0], np.float32), k)
    return h * (rs[:, None] * cs[None, :] / np.float32(np.sqrt(n)))


def _illcond(rng, r, c):
    """U diag(s) V^T + 1e-4 N(0,1): orthonormal U (r x k), V (c x k),
    k = min(r, c), singular values log-uniform in [1e-4, 1]."""
    k = min(r, c)
    u = _orthonormal_columns(rng, r, k)
    v = _orthonormal_columns(rng, c, k)
    s = np.exp(rng.uniform(np.log(1e-4), 0.0, k)).astype(np.float32)
    return (u * s[None, :]) @ v.T + np.float32(1e-4) * rng.standard_normal((r, c), dtype=np.float32)


def matrix_inputs(wl: Workload, i: int):
    """(W, V_prev, G) of matrix ``i`` as CPU torch tensors in the storage dtype."""
    r, c = wl.shapes[i]
    rng = np.random.default_rng(np.random.SeedSequence([wl.seed, i]))
    w = rng.standard_normal((r, c), dtype=np.float32) * np.float32(wl.w_std)
    if wl.kind == "illcond":
        v = np.zeros((r, c), np.float32)
        g = _illcond(rng, r, c).astype(np.float32)
    else:
        v = rng.standard_normal((r, c), dtype=np.float32) * np.float32(wl.v_std)
        g = rng.standard_normal((r, c), dtype=np.float32) * np.float32(wl.g_std)
    return (_to_storage(w, wl.dtype), _to_storage(v, wl.dtype),
            _to_storage(g, wl.dtype))


def workload_inputs(wl: Workload, indices=None, threads: int | None = None):
    """Inputs of several matrices (default: all), drawn in parallel."""
    idx = list(range(len(wl.shapes))) if indices is None else list(indices)
    if threads is None:
        threads = max(1, min(16, len(os.sched_getaffinity(0))))
    if len(idx) <= 1 or threads == 1:
        return [matrix_inputs(wl, i) for i in idx]
    with _cf.ThreadPoolExecutor(threads) as ex:
        return list(ex.map(lambda i: matrix_inputs(wl, i), idx))
