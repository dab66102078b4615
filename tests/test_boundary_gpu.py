"""GPU tests of the C-ABI boundary's plan cache and workspace contract.

* A plan depends on the list of shapes only: steps whose W, G, V (and
  workspace) are freshly allocated every time give bit-identical results to
  steps on the same tensors, and build no plan, allocate nothing on the device
  and leave the host free to return while the stream is still busy.
* Calls of one plan on two streams are chained on the device.
* More than 64 shape lists evict plans; evicted plans are freed once idle.
* The workspace contents on entry are irrelevant: a workspace filled with NaN
  gives the bits of a zeroed one (every workspace byte a launch reads was
  written earlier in the same call; the padding is rewritten as zeros).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.helpers import f64, relF

pytestmark = pytest.mark.gpu

SHAPES = [(300, 700), (700, 300), (256, 512), (1280, 1280), (37, 45)]


@pytest.fixture(scope="module")
def mo():
    import matrix_optimizer_step_amd as m
    m.lib()   # raises if the library is missing: no fallback
    return m


def _inputs(shapes, seed, dtype="bf16"):
    wl = workloads.small_case("boundary", shapes, dtype=dtype, seed=seed, v_std=1e-3, g_std=1e-3)
    trip = workloads.workload_inputs(wl)
    return ([t[0].cuda() for t in trip], [t[1].cuda() for t in trip],
            [t[2].cuda() for t in trip])


def _delta(mo, before):
    after = mo.counters()
    return {k: after[k] - before[k] for k in after}


def test_fresh_pointers_every_step_match_stable_pointers(mo):
    W0, V0, _ = _inputs(SHAPES, seed=71)
    grads = [_inputs(SHAPES, seed=80 + k)[2] for k in range(5)]
    # stable pointers: the same W, V, G tensors every step (G refilled in place)
    Ws = [w.clone() for w in W0]
    Vs = [v.clone() for v in V0]
    Gs = [g.clone() for g in grads[0]]
    for k in range(5):
        for g, src in zip(Gs, grads[k]):
            g.copy_(src)
        mo.muon_step_batched(Ws, Gs, Vs)
    torch.cuda.synchronize()
    # fresh pointers: every step new W, V, G tensors and a new workspace
    before = mo.counters()
    Wf = [w.clone() for w in W0]
    Vf = [v.clone() for v in V0]
    need = mo.workspace_bytes([tuple(w.shape) for w in W0], torch.bfloat16)
    for k in range(5):
        Wf = [w.clone() for w in Wf]
        Vf = [v.clone() for v in Vf]
        Gf = [g.clone() for g in grads[k]]
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        mo.muon_step_batched(Wf, Gf, Vf, workspace=ws)
    torch.cuda.synchronize()
    d = _delta(mo, before)
    print("counters over 5 fresh-pointer steps:", d, flush=True)
    assert d["plan_builds"] == 0 and d["device_allocs"] == 0 and d["device_frees"] == 0
    assert d["bind_launches"] == 5
    for a, b in zip(Ws, Wf):
        assert torch.equal(a, b)
    for a, b in zip(Vs, Vf):
        assert torch.equal(a, b)


def test_call_returns_while_stream_busy(mo):
    """No host synchronisation inside a call: with a long queue of work ahead
    of it on the stream, a step with pointers the plan has never seen returns
    before the stream has drained."""
    W, V, G = _inputs(SHAPES, seed=91)
    mo.muon_step_batched(W, G, V)          # the plan for these shapes exists now
    torch.cuda.synchronize()
    W2 = [w.clone() for w in W]
    V2 = [v.clone() for v in V]
    G2 = [g.clone() for g in G]
    need = mo.workspace_bytes([tuple(w.shape) for w in W], torch.bfloat16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    a = torch.randn(4096, 4096, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(4096, 4096, device="cuda", dtype=torch.bfloat16)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    for _ in range(400):                   # ~0.1 s of queued products
        c = a @ b
    mo.muon_step_batched(W2, G2, V2, workspace=ws)
    busy = not stream.query()
    torch.cuda.synchronize()
    del c
    assert busy, "the stream had drained when the call returned: the call synchronised"


def test_rmnp_and_adamw_fresh_pointers(mo):
    W0, V0, G0 = _inputs(SHAPES, seed=101)
    Ws, Vs = [w.clone() for w in W0], [v.clone() for v in V0]
    for _ in range(3):
        mo.rmnp_step_batched(Ws, G0, Vs)
    torch.cuda.synchronize()
    before = mo.counters()
    Wf, Vf = [w.clone() for w in W0], [v.clone() for v in V0]
    for _ in range(3):
        Wf = [w.clone() for w in Wf]
        Vf = [v.clone() for v in Vf]
        mo.rmnp_step_batched(Wf, [g.clone() for g in G0], Vf)
    torch.cuda.synchronize()
    d = _delta(mo, before)
    assert d["plan_builds"] == 0 and d["device_allocs"] == 0
    for a, b in zip(Ws + Vs, Wf + Vf):
        assert torch.equal(a, b)
    # AdamW on a two-tensor tail
    lens = [1000, 4096]
    p0 = [torch.randn(n, device="cuda").bfloat16() for n in lens]
    g0 = [(torch.randn(n, device="cuda") * 0.1).bfloat16() for n in lens]
    ps, ms, vs = [p.clone() for p in p0], [torch.zeros(n, device="cuda") for n in lens], \
        [torch.zeros(n, device="cuda") for n in lens]
    for t in range(1, 4):
        mo.adamw_step_batched(ps, g0, ms, vs, t)
    torch.cuda.synchronize()
    pf, mf, vf = [p.clone() for p in p0], [torch.zeros(n, device="cuda") for n in lens], \
        [torch.zeros(n, device="cuda") for n in lens]
    for t in range(1, 4):
        pf, mf, vf = [x.clone() for x in pf], [x.clone() for x in mf], [x.clone() for x in vf]
        mo.adamw_step_batched(pf, [g.clone() for g in g0], mf, vf, t)
    torch.cuda.synchronize()
    for a, b in zip(ps + ms + vs, pf + mf + vf):
        assert torch.equal(a, b)


def test_two_streams_share_a_plan(mo):
    """One shape list on two streams, back to back without host
    synchronisation: the second call waits on the device for the first."""
    W, V, G = _inputs(SHAPES, seed=111)
    Wa, Va = [w.clone() for w in W], [v.clone() for v in V]
    Wb, Vb = [w.clone() for w in W], [v.clone() for v in V]
    mo.rmnp_step_batched(Wa, G, Va)          # reference on the current stream
    mo.muon_step_batched(Wa, G, Va)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    ws1 = torch.empty(mo.workspace_bytes(SHAPES, torch.bfloat16), dtype=torch.uint8, device="cuda")
    ws2 = torch.empty_like(ws1)
    Wc, Vc = [w.clone() for w in W], [v.clone() for v in V]
    torch.cuda.synchronize()
    with torch.cuda.stream(s1):
        mo.rmnp_step_batched(Wb, G, Vb)      # rmnp plan: descriptor slot in the plan
        mo.muon_step_batched(Wb, G, Vb, workspace=ws1)
    with torch.cuda.stream(s2):
        mo.rmnp_step_batched(Wc, G, Vc)      # same plans, other stream, other tensors
        mo.muon_step_batched(Wc, G, Vc, workspace=ws2)
    torch.cuda.synchronize()
    for a, b, c in zip(Wa + Va, Wb + Vb, Wc + Vc):
        assert torch.equal(a, b) and torch.equal(a, c)


def test_plan_eviction_frees_idle_plans(mo):
    before = mo.counters()
    xs = []
    for i in range(70):   # 70 distinct shape lists: more than the 64 cached plans
        x = torch.randn(8, 16 + i, device="cuda").bfloat16()
        o = mo.ns_orthogonalize_batched([x], out_dtype=torch.float32)[0]
        xs.append((x, o))
    torch.cuda.synchronize()
    # a further call sweeps the retired plans, now idle
    mo.ns_orthogonalize_batched([torch.randn(8, 200, device="cuda").bfloat16()])
    torch.cuda.synchronize()
    d = _delta(mo, before)
    print("eviction counters:", d, flush=True)
    assert d["plan_builds"] == 71
    assert d["device_frees"] >= 6
    # the cache still computes correctly after evictions
    for x, o in xs[:3] + xs[-3:]:
        ref = oracle.ns_orthogonalize(f64(x), rounding="bf16")
        assert relF(f64(o), ref) <= 2e-2
        again = mo.ns_orthogonalize_batched([x], out_dtype=torch.float32)[0]
        torch.cuda.synchronize()
        assert torch.equal(again, o)


@pytest.mark.parametrize("dtype,precision", [("bf16", "default"), ("f32", "default"),
                                             ("bf16", "split")])
def test_nan_poisoned_workspace(mo, dtype, precision):
    shapes = SHAPES if dtype == "bf16" else [(300, 700), (700, 300), (64, 64), (37, 45)]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    W, V, G = _inputs(shapes, seed=121, dtype=dtype)
    need = mo.workspace_bytes(shapes, tdt, precision=precision)
    clean = torch.zeros(need, dtype=torch.uint8, device="cuda")
    poison = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")   # NaN in bf16 and f32
    Wc, Vc = [w.clone() for w in W], [v.clone() for v in V]
    Wp, Vp = [w.clone() for w in W], [v.clone() for v in V]
    mo.muon_step_batched(Wc, G, Vc, workspace=clean, precision=precision)
    mo.muon_step_batched(Wp, G, Vp, workspace=poison, precision=precision)
    Oc = mo.ns_orthogonalize_batched(Vc, out_dtype=torch.float32, workspace=clean.zero_(),
                                     precision=precision)
    Op = mo.ns_orthogonalize_batched(Vc, out_dtype=torch.float32,
                                     workspace=poison.fill_(0xFF), precision=precision)
    torch.cuda.synchronize()
    for a, b in zip(Wc + Vc, Wp + Vp):
        assert torch.isfinite(b.float()).all()
        assert torch.equal(a, b)
    for a, b in zip(Oc, Op):
        assert torch.isfinite(b).all()
        assert torch.equal(a, b)
