"""Host model of the bf16 GEMM K-loop pipeline (ns_gemm_bf16.hip), checked on
the CPU for every K length and diagonal split the workloads reach.

Every wave of a workgroup runs the same program: DMA instructions that copy a
K step's operand tiles from HBM into one of NS = 5 LDS stages (stage of step t
= t mod NS), waits on its own DMA count (s_waitcnt vmcnt(n): all but the n
most recent DMA instructions of the wave have landed), workgroup barriers,
fragment reads of a stage, and the MFMAs that consume those fragments.  The
model writes each schedule's program as the kernel's loops emit it --

  kloop   (Gram and polynomial: prologue, steady steps with the Q half of the
           DMA of step t+3 before the barrier and the P half of step t+4 after
           it, three drain steps), with the k-major -> row-major switch of P at
           bP and of Q at bQ;
  kloop2  (apply: the DMA of steps s and s+1 issued back to back, Q of an even
           pair before the barrier of its even step, P after the barrier of
           its odd step), with P's switch at bP;
  diag    (a diagonal tile: P panel only);
  pair    (a diagonal pair: both panels, the kloop schedule)

-- and checks that
  * every stage read sees its step's DMA landed for every wave (the reading
    wave waited for its own DMA, and every wave waited before the barrier
    that precedes the read);
  * no DMA overwrites a stage before every wave has consumed the step it held
    (consumption happens at the MFMA; a barrier must separate it from the
    DMA issue);
  * every step's tile is read in the layout its DMA wrote;
  * every step is issued, read and multiplied exactly once per sub-step.
"""
import pytest

NS = 5          # LDS stages
BPW = 2         # DMA instructions per wave, operand and step (eight waves)
DPS = 2 * BPW   # DMA instructions per wave and step (P and Q)


class Program:
    """The event list of one wave."""

    def __init__(self, km_p, km_q):
        self.ev = []
        self.km_p, self.km_q = km_p, km_q   # step -> k-major layout of the DMA

    def issue(self, op, t):
        km = (self.km_p if op == "P" else self.km_q)(t)
        for _ in range(BPW):
            self.ev.append(("issue", op, t, t % NS, km))

    def wait(self, n):
        self.ev.append(("wait", n))

    def barrier(self):
        self.ev.append(("barrier",))

    def read(self, t, kk, p_km, q_km, ops="PQ"):
        self.ev.append(("read", t, t % NS, kk, p_km, q_km, ops))

    def mfma(self, t, kk):
        self.ev.append(("mfma", t, kk))


def check(prog, nk, ops="PQ"):
    """Verify the invariants of one wave program (all waves run it)."""
    issued = []        # DMA instructions in issue order: (op, t, stage, km)
    by_step = {}       # step -> indices into `issued`
    landed = 0         # instructions [0, landed) known landed at the last wait
    landed_at_barrier = 0
    barriers = 0
    consumed_before_barrier = {}   # (t, kk) -> barrier count when its MFMA ran
    read_steps = {}
    mfma_steps = set()
    for ev in prog.ev:
        kind = ev[0]
        if kind == "issue":
            _, op, t, s, km = ev
            prev = t - NS
            if prev >= 0:
                # the previous occupant of this stage must have been consumed
                # (both sub-steps) before a barrier that this issue follows
                for kk in (0, 1):
                    b = consumed_before_barrier.get((prev, kk))
                    assert b is not None and b < barriers, \
                        f"DMA {op}({t}) into stage {s} before step {prev} sub-step {kk} was consumed"
            by_step.setdefault(t, []).append(len(issued))
            issued.append((op, t, s, km))
        elif kind == "wait":
            landed = max(landed, len(issued) - ev[1])
        elif kind == "barrier":
            landed_at_barrier = landed
            barriers += 1
        elif kind == "read":
            _, t, s, kk, p_km, q_km, rops = ev
            need = [i for i in by_step.get(t, []) if issued[i][0] in rops]
            assert len(need) == BPW * len(rops), f"step {t}: {len(need)} DMA instructions issued"
            # every wave: landed before the last barrier; this wave: landed now
            assert max(need) < landed_at_barrier <= landed, \
                f"read of step {t} sub-step {kk} before its DMA landed"
            for i in need:
                op, _, st, km = issued[i]
                assert st == s, "read from another stage than the DMA wrote"
                assert km == (p_km if op == "P" else q_km), \
                    f"step {t}: {op} read in the other layout than its DMA wrote"
            read_steps.setdefault(t, set()).add(kk)
        elif kind == "mfma":
            _, t, kk = ev
            assert kk in read_steps.get(t, set()), f"MFMA of step {t} sub-step {kk} before its read"
            assert (t, kk) not in mfma_steps
            mfma_steps.add((t, kk))
            consumed_before_barrier[(t, kk)] = barriers
    assert mfma_steps == {(t, kk) for t in range(nk) for kk in (0, 1)}
    for op in ops:
        assert sorted(t for (o, t, _, _) in issued if o == op) == \
            sorted(t for t in range(nk) for _ in range(BPW))


# ------------------------------------------------------------------ schedules
def kloop_program(nk, bP, bQ, qs):
    """kloop: P k-major for t < bP, Q k-major for t < bQ when qs (polynomial)."""
    km_p = lambda t: t < bP
    km_q = lambda t: qs and t < bQ
    p = Program(km_p, km_q)
    lay = lambda t: (km_p(t), km_q(t))
    # prologue: steps 0 .. NS-3 both halves, P of step NS-2
    for t in range(NS - 2):
        p.issue("P", t)
        p.issue("Q", t)
    p.issue("P", NS - 2)
    p.wait(DPS * (NS - 3) + DPS // 2)
    p.barrier()
    p.read(0, 0, *lay(0))

    def step(t, vmw, dq, dp):
        p.read(t, 1, *lay(t))
        if dq:
            p.issue("Q", t + NS - 2)
        p.mfma(t, 0)
        p.wait(vmw)
        p.barrier()
        if dp:
            p.issue("P", t + NS - 1)
        if t + 1 < nk:
            p.read(t + 1, 0, *lay(t + 1))
        p.mfma(t, 1)

    t = 0
    while t < nk - NS + 1:
        step(t, 4 * BPW, True, True)
        t += 1
    step(t, DPS * 2, True, False)
    step(t + 1, DPS, False, False)
    step(t + 2, 0, False, False)
    # the last step: its sub-step-1 fragments, then both MFMAs
    p.read(nk - 1, 1, *lay(nk - 1))
    p.mfma(nk - 1, 0)
    p.mfma(nk - 1, 1)
    return p


def kloop2_program(nk, bP):
    """kloop2 (paired DMA): P k-major for t < bP, Q k-major throughout."""
    km_p = lambda t: t < bP
    km_q = lambda t: True
    p = Program(km_p, km_q)
    lay = lambda t: (km_p(t), km_q(t))
    p.issue("P", 0)
    p.issue("Q", 0)
    p.issue("P", 1)
    p.issue("Q", 1)
    p.issue("P", 2)
    p.issue("P", 3)
    p.wait(2 * DPS)
    p.barrier()
    p.read(0, 0, *lay(0))

    def step2(t, vmw, qpair, ppair):
        p.read(t, 1, *lay(t))
        if qpair:
            p.issue("Q", t + 2)
            p.issue("Q", t + 3)
        p.mfma(t, 0)
        p.wait(vmw)
        p.barrier()
        if ppair:
            p.issue("P", t + 3)
            p.issue("P", t + 4)
        if t + 1 < nk:
            p.read(t + 1, 0, *lay(t + 1))
        p.mfma(t, 1)

    t = 0
    while t < nk - 4:
        step2(t, 2 * DPS, True, False)
        step2(t + 1, BPW, False, True)
        t += 2
    step2(t, 2 * DPS, True, False)
    step2(t + 1, BPW, False, False)
    step2(t + 2, 0, False, False)
    p.read(nk - 1, 1, *lay(nk - 1))
    p.mfma(nk - 1, 0)
    p.mfma(nk - 1, 1)
    return p


def diag_program(nk, bP):
    """A diagonal tile: the P panel only, k-major for t < bP."""
    km_p = lambda t: t < bP
    p = Program(km_p, lambda t: False)
    lay = lambda t: (km_p(t), False)
    for t in range(NS - 1):
        p.issue("P", t)
    p.wait(BPW * (NS - 2))
    p.barrier()
    p.read(0, 0, *lay(0), ops="P")

    def step(t, vmw, dp):
        p.read(t, 1, *lay(t), ops="P")
        p.mfma(t, 0)
        p.wait(vmw)
        p.barrier()
        if dp:
            p.issue("P", t + NS - 1)
        if t + 1 < nk:
            p.read(t + 1, 0, *lay(t + 1), ops="P")
        p.mfma(t, 1)

    t = 0
    while t < nk - NS + 1:
        step(t, 2 * BPW, True)
        t += 1
    step(t, 2 * BPW, False)
    step(t + 1, BPW, False)
    step(t + 2, 0, False)
    p.read(nk - 1, 1, *lay(nk - 1), ops="P")
    p.mfma(nk - 1, 0)
    p.mfma(nk - 1, 1)
    return p


def pair_program(nk):
    """A diagonal pair: both panels row-major, the kloop schedule with the
    prologue waiting for BPW fewer instructions."""
    p = kloop_program(nk, 0, 0, False)
    # the pair's prologue wait is DPS*(NS-3) + BPW (the same count: DPS/2 == BPW)
    assert DPS // 2 == BPW
    return p


# ------------------------------------------------------------------ cases
# K steps of 32 the workloads reach.  Gram: K = n, 256 .. 27648 (the 32B-class
# share's 5120 x 27648 matrices: 864 steps).  Polynomial, apply and diagonal
# tiles: K = m <= 8192 (256 steps), the split-precision apply twice that.
GRAM_NKS = [8, 10, 12, 16, 24, 32, 40, 48, 64, 80, 120, 128, 160, 256, 448, 512, 864]
M_NKS = [8, 16, 24, 32, 40, 48, 64, 80, 128, 160, 256]


@pytest.mark.parametrize("nk", GRAM_NKS)
def test_gram_schedule(nk):
    check(kloop_program(nk, 0, 0, False), nk)


@pytest.mark.parametrize("nk", M_NKS)
def test_polynomial_schedule_every_split(nk):
    # tile (ti, tj), ti < tj: P k-major before bP = 8 ti, Q before bQ = 8 tj,
    # both at most nk - 8 (the diagonal tiles go through diag_program)
    for bp in range(0, nk - 7, 8):
        for bq in range(bp + 8, nk - 7, 8):
            check(kloop_program(nk, bp, bq, True), nk)


@pytest.mark.parametrize("nk", M_NKS + [2 * n for n in M_NKS])
def test_apply_schedule_every_split(nk):
    # P (B rows) k-major before its diagonal block, bP = 8 ti <= nk - 8; the
    # split-precision apply runs K twice with bP = 0
    for bp in range(0, nk - 7, 8):
        check(kloop2_program(nk, bp), nk)


@pytest.mark.parametrize("nk", M_NKS)
def test_diagonal_tile_schedule_every_split(nk):
    for bp in range(0, nk - 7, 8):
        check(diag_program(nk, bp), nk, ops="P")


@pytest.mark.parametrize("nk", GRAM_NKS)
def test_diagonal_pair_schedule(nk):
    check(pair_program(nk), nk)


def test_model_catches_a_short_wait():
    """A wait that leaves one more DMA instruction in flight must be caught."""
    p = kloop_program(40, 0, 0, False)
    for i, ev in enumerate(p.ev):
        if ev[0] == "wait" and ev[1] == 4 * BPW:
            p.ev[i] = ("wait", 4 * BPW + 2)
            break
    with pytest.raises(AssertionError):
        check(p, 40)


def test_model_catches_an_early_dma():
    """A DMA issued before the barrier that frees its stage must be caught:
    P of step NS refills the stage of step 0, whose second sub-step is
    consumed after the barrier of step 0; moved before the barrier of step 1
    it would overwrite fragments other waves may still be reading."""
    p = kloop_program(40, 0, 0, False)
    first = next(i for i, ev in enumerate(p.ev) if ev[0] == "issue" and ev[1] == "P" and ev[2] == NS)
    j = first - 1
    while p.ev[j][0] != "barrier":
        j -= 1
    moved = [p.ev.pop(first) for _ in range(BPW)]
    for k, e in enumerate(moved):
        p.ev.insert(j + k, e)
    with pytest.raises(AssertionError):
        check(p, 40)


def test_model_catches_a_layout_mismatch():
    p = kloop_program(40, 16, 24, True)
    for i, ev in enumerate(p.ev):
        if ev[0] == "read" and ev[1] == 15 and ev[3] == 0:
            p.ev[i] = ev[:4] + (False,) + ev[5:]   # P of step 15 read as row-major
            break
    with pytest.raises(AssertionError):
        check(p, 40)
