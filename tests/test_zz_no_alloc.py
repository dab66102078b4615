"""The allocation-free Muon step (muon_step_batched_noalloc) against the
workspace entry point muon_step_batched: the same kernels on the same inputs,
so the results must be bit-identical -- on two calls in a row, the second with
a smaller input (the scratch array keeps the first call's contents), in bf16
and in float32, and once in split precision.  The calls build no plan and allocate nothing on the device.
A shape list beyond the scratch array is rejected before anything runs.

Under HIP graph capture (the callers this entry point is for): one step
captured on fixed tensors and replayed several times, with eager work and
synchronisations between the replays, gives on every replay the bits of the
same step run eagerly."""
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mo():
    import matrix_optimizer_step_amd as m
    m.lib()   # raises if the library is missing: no fallback
    return m


def _inputs(shapes, seed, dtype="bf16"):
    wl = workloads.small_case("noalloc", shapes, dtype=dtype, seed=seed, v_std=1e-3, g_std=1e-3)
    trip = workloads.workload_inputs(wl)
    return ([t[0].cuda() for t in trip], [t[1].cuda() for t in trip],
            [t[2].cuda() for t in trip])


CALLS = [
    ("bf16", [(1280, 1280), (300, 700), (700, 300), (256, 512), (1280, 3840)]),
    ("bf16", [(256, 512), (37, 45)]),          # smaller than the first
    ("f32", [(256, 512)]),                      # the float32 single-matrix case
    ("bf16", [(512, 1280), (300, 700)]),        # split precision (below)
]
SPLIT_CALL = 3


def test_noalloc_bit_identical_to_workspace_step(mo):
    for k, (dt, shapes) in enumerate(CALLS):
        print(f"[noalloc] call {k}: {dt} {shapes}", flush=True)
        W, V, G = _inputs(shapes, seed=200 + k, dtype=dt)
        Wr, Vr = [w.clone() for w in W], [v.clone() for v in V]
        Wn, Vn = [w.clone() for w in W], [v.clone() for v in V]
        prec = "split" if k == SPLIT_CALL else "default"
        mo.muon_step_batched(Wr, G, Vr, precision=prec)
        torch.cuda.synchronize()
        before = mo.counters()
        mo.muon_step_batched_noalloc(Wn, G, Vn, precision=prec)
        torch.cuda.synchronize()
        after = mo.counters()
        assert after["plan_builds"] == before["plan_builds"]
        assert after["device_allocs"] == before["device_allocs"]
        for a, b in zip(Wr + Vr, Wn + Vn):
            assert torch.equal(a, b)


def test_noalloc_rejects_shapes_beyond_the_scratch(mo):
    shapes = [(4096, 4096)] * 4
    W = [torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    with pytest.raises(mo.MatoptError) as ei:
        mo.muon_step_batched_noalloc(W, [w.clone() for w in W], [w.clone() for w in W])
    assert ei.value.name == "MATOPT_ERR_WORKSPACE"
    assert "scratch" in ei.value.detail


@pytest.mark.parametrize("dt,shapes", [("f32", [(256, 512)]),
                                       ("bf16", [(300, 700), (700, 300), (256, 512)])])
def test_noalloc_step_replays_from_a_captured_graph(mo, dt, shapes):
    print(f"[noalloc graph] {dt} {shapes}", flush=True)
    W0, V0, G = _inputs(shapes, seed=300, dtype=dt)
    W, V = [w.clone() for w in W0], [v.clone() for v in V0]
    mo.muon_step_batched_noalloc(W, G, V)          # eager reference
    torch.cuda.synchronize()
    We, Ve = [w.clone() for w in W], [v.clone() for v in V]

    def reset():
        for w, w0 in zip(W, W0):
            w.copy_(w0)
        for v, v0 in zip(V, V0):
            v.copy_(v0)
        torch.cuda.synchronize()

    reset()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mo.muon_step_batched_noalloc(W, G, V)
    torch.cuda.synchronize()
    for rep in range(3):
        reset()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(W + V, We + Ve):
            assert torch.equal(a, b), f"replay {rep}"
        # eager work between replays, on the same scratch array
        Wx, Vx = [w.clone() for w in W0], [v.clone() for v in V0]
        mo.muon_step_batched_noalloc(Wx, G, Vx)
        torch.cuda.synchronize()
