"""CPU oracle for the owner-local Muon step and the RMNP comparator.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP library (``matrix_optimizer_step_amd``) and imports nothing from it.

Everything is plain numpy in float64.  Matrix products use numpy's ``@`` (a
library primitive); there is no blocking, fusion, symmetry trick or reordering
beyond what the algorithm states, so each function can be checked against the
pages by eye.

Sources (cited by page title and section):

* "Optimizers In A Sharded World: Muon's O(mn) Vs RMNP's Zero" (blog post):
  section 1 (heavy-ball momentum, the Muon target direction, the RMNP row
  direction), section 3 (the column-cut layout's row sums), section 8
  (summary), and the appendix "The Code That Ran" (the five-step Newton-Schulz
  routine, the ``rmnp_local``, ``rmnp_colcut`` and ``muon_sc`` steps with their
  update scale).
* "MatrixFSDP" (arXiv 2607.05895), section 3 and section 4.4: the owner runs
  the whole-matrix Newton-Schulz update locally on each matrix it owns;
  section 5.1: the training configuration (weight decay, momentum 0.5, two
  Newton-Schulz steps).

Parity status of every function is listed in ``oracle/muon.py``'s header.
"""

from .muon import (  # noqa: F401
    NS_COEFFS,
    NS_STEPS,
    NS_EPS,
    MOMENTUM,
    RMNP_EPS,
    RMNP_COLCUT_EPS,
    f32_param,
    round_bf16,
    round_storage,
    momentum,
    frobenius_scale,
    update_scale,
    ns_orthogonalize,
    ns_orthogonalize_page_form,
    ns_orthogonalize_page_bf16,
    split_bf16,
    muon_step,
    rmnp_direction,
    rmnp_step,
    rmnp_colcut_partial,
    rmnp_colcut_apply,
    adamw_step,
)
