"""The MFMA rate probe (a measurement aid, matopt_mfma_probe) runs to
completion on both MFMA forms and operand sources: every thread's sum is
finite, all-zero operands give exactly zero, and the clock counters advance."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("form", [16, 32])
@pytest.mark.parametrize("lds", [False, True])
def test_probe_runs(form, lds):
    import matrix_optimizer_step_amd as mo
    print(f"[probe] form {form} lds {lds}", flush=True)
    g = torch.Generator().manual_seed(1)
    src = torch.randn(49152, generator=g).to(torch.bfloat16).cuda()
    out = torch.full((4 * 512,), float("nan"), device="cuda")
    clk = torch.zeros(2, dtype=torch.int64, device="cuda")
    mo.mfma_probe(form, lds, src, out, clk, 4, 4)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    c = clk.cpu().tolist()
    assert c[0] > 0 and c[1] > 0
    mo.mfma_probe(form, lds, torch.zeros_like(src), out, clk, 2, 4)
    torch.cuda.synchronize()
    assert bool((out == 0).all())
