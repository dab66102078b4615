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
  pair    (a diagonal pair: both panels, the kloop schedule);
  persist (the persistent apply: kloop2 tiles back to back, the next tile's
           prologue DMA issued after a barrier that follows the last MFMAs,
           then the finished tile's stores, which the next tile's first two
           waits let stay in flight)

The 16 x 16 x 32 forms of these loops (kloop16, kloop16_rest, the diagonal
pair on slabs) emit the same events per step: the two halves of a step take
the places of its two k16 sub-steps (the first half's reads, of this step's
stage, before the barrier; the second half's, of the next step's stage, after
it), with the same DMA, waits and barriers, so the model covers them too.

-- and checks that
  * every stage read sees its step's DMA landed for every wave (the reading
    wave waited for its own DMA, and every wave waited before the barrier
    that precedes the read);
  * no DMA overwrites a stage before every wave has consumed the step it held
    (consumption happens at the MFMA; a barrier must separate it from the
    DMA issue);
  * every step's tile is read in the layout its DMA wrote;
  * every step is issued, read and multiplied exactly once per sub-step;
  * a wait that lets stores stay in flight still covers the DMA it guards
    (stores count in the same vmcnt as the DMA, in issue order).
"""
import pytest

NS = 5          # LDS stages
BPW = 2         # DMA instructions per wave, operand and step (eight waves)
DPS = 2 * BPW   # DMA instructions per wave and step (P and Q)


class Program:
    """The event list of one wave.  A step is keyed (tile, t): the persistent
    apply runs several tiles' K loops in one program; stage of step t = t mod
    NS within each tile."""

    def __init__(self, km_p, km_q):
        self.ev = []
        self.tile = 0
        self.km_p, self.km_q = km_p, km_q   # step -> k-major layout of the DMA

    def next_tile(self, km_p, km_q):
        self.tile += 1
        self.km_p, self.km_q = km_p, km_q

    def issue(self, op, t):
        km = (self.km_p if op == "P" else self.km_q)(t)
        for _ in range(BPW):
            self.ev.append(("issue", op, (self.tile, t), t % NS, km))

    def store(self, n):
        """n vector memory stores: counted by the waits like DMA instructions."""
        for _ in range(n):
            self.ev.append(("store",))

    def wait(self, n):
        self.ev.append(("wait", n))

    def barrier(self):
        self.ev.append(("barrier",))

    def read(self, t, kk, p_km, q_km, ops="PQ"):
        self.ev.append(("read", (self.tile, t), t % NS, kk, p_km, q_km, ops))

    def mfma(self, t, kk):
        self.ev.append(("mfma", (self.tile, t), kk))


def check(prog, nk, ops="PQ"):
    """Verify the invariants of one wave program (all waves run it).  nk: the
    K steps of each tile (an int: one tile; a list: one entry per tile)."""
    nks = nk if isinstance(nk, list) else [nk]
    issued = []        # vector memory instructions in issue order: (op, key, stage, km)
    by_step = {}       # step key -> indices into `issued`
    owner = {}         # stage -> key of the step its last DMA brought in
    landed = 0         # instructions [0, landed) known landed at the last wait
    landed_at_barrier = 0
    barriers = 0
    consumed_before_barrier = {}   # (key, kk) -> barrier count when its MFMA ran
    read_steps = {}
    mfma_steps = set()
    for ev in prog.ev:
        kind = ev[0]
        if kind == "issue":
            _, op, key, s, km = ev
            prev = owner.get(s)
            if prev is not None and prev != key:
                # the previous occupant of this stage must have been consumed
                # (both sub-steps) before a barrier that this issue follows
                for kk in (0, 1):
                    b = consumed_before_barrier.get((prev, kk))
                    assert b is not None and b < barriers, \
                        f"DMA {op}{key} into stage {s} before step {prev} sub-step {kk} was consumed"
            owner[s] = key
            by_step.setdefault(key, []).append(len(issued))
            issued.append((op, key, s, km))
        elif kind == "store":
            issued.append(("S", None, None, None))
        elif kind == "wait":
            landed = max(landed, len(issued) - ev[1])
        elif kind == "barrier":
            landed_at_barrier = landed
            barriers += 1
        elif kind == "read":
            _, key, s, kk, p_km, q_km, rops = ev
            need = [i for i in by_step.get(key, []) if issued[i][0] in rops]
            assert len(need) == BPW * len(rops), f"step {key}: {len(need)} DMA instructions issued"
            # every wave: landed before the last barrier; this wave: landed now
            assert max(need) < landed_at_barrier <= landed, \
                f"read of step {key} sub-step {kk} before its DMA landed"
            for i in need:
                op, _, st, km = issued[i]
                assert st == s, "read from another stage than the DMA wrote"
                assert km == (p_km if op == "P" else q_km), \
                    f"step {key}: {op} read in the other layout than its DMA wrote"
            read_steps.setdefault(key, set()).add(kk)
        elif kind == "mfma":
            _, key, kk = ev
            assert kk in read_steps.get(key, set()), f"MFMA of step {key} sub-step {kk} before its read"
            assert (key, kk) not in mfma_steps
            mfma_steps.add((key, kk))
            consumed_before_barrier[(key, kk)] = barriers
    assert mfma_steps == {((i, t), kk) for i, n in enumerate(nks) for t in range(n) for kk in (0, 1)}
    for op in ops:
        for i, n in enumerate(nks):
            assert sorted(key[1] for (o, key, _, _) in issued if o == op and key[0] == i) == \
                sorted(t for t in range(n) for _ in range(BPW))


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


def kloop2_issue_prologue(p):
    p.issue("P", 0)
    p.issue("Q", 0)
    p.issue("P", 1)
    p.issue("Q", 1)
    p.issue("P", 2)
    p.issue("P", 3)


def kloop2_rest(p, nk, lay, xw=0):
    """Everything after the prologue DMA; xw: stores that may stay in flight
    at the waits of steps -1 and 0 (the persistent apply's previous tile)."""
    p.wait(2 * DPS + xw)
    p.barrier()
    p.read(0, 0, *lay(0))

    def step2(t, vmw, qpair, ppair):
        p.read(t, 1, *lay(t))
        if qpair:
            p.issue("Q", t + 2)
            p.issue("Q", t + 3)
        p.mfma(t, 0)
        p.wait(vmw + (xw if t == 0 else 0))
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


def kloop2_program(nk, bP):
    """kloop2 (paired DMA): P k-major for t < bP, Q k-major throughout."""
    km_p = lambda t: t < bP
    km_q = lambda t: True
    p = Program(km_p, km_q)
    kloop2_issue_prologue(p)
    kloop2_rest(p, nk, lambda t: (km_p(t), km_q(t)))
    return p


XW = 16   # stores the persistent apply lets stay in flight (bf16 iterate: 2 per 32 x 32 block)


def persist_program(tiles, nst, xw=XW):
    """The persistent apply: tiles = [(nk, bP), ...] run back to back.  After a
    tile's last MFMAs: every wave waits for its LDS reads and passes a barrier,
    the next tile's prologue DMA is issued, then the finished tile's nst
    stores; the next K loop lets xw of them stay in flight."""
    def lays(bp):
        return (lambda t: t < bp), (lambda t: True)

    km_p, km_q = lays(tiles[0][1])
    p = Program(km_p, km_q)
    kloop2_issue_prologue(p)
    pend = False
    for i, (nk, bp) in enumerate(tiles):
        km_p, km_q = lays(bp)
        kloop2_rest(p, nk, lambda t, a=km_p, b=km_q: (a(t), b(t)), xw if pend else 0)
        if i + 1 < len(tiles):
            p.barrier()
            p.next_tile(*lays(tiles[i + 1][1]))
            kloop2_issue_prologue(p)
        p.store(nst)
        pend = True
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


@pytest.mark.parametrize("nk", M_NKS + [2 * n for n in M_NKS])
def test_persistent_apply_schedule(nk):
    # consecutive tiles of one matrix (every split of the first, the diagonal
    # one next) and a change of K between tiles; bf16 (16 stores per tile)
    # and split-precision (32) iterates
    for nst in (XW, 2 * XW):
        for bp in range(0, nk - 7, 8):
            tiles = [(nk, bp), (nk, min(bp + 8, nk - 8)), (8, 0), (nk, 0)]
            check(persist_program(tiles, nst), [t[0] for t in tiles])


def test_model_catches_too_few_stores_for_the_allowance():
    """The allowance is only sound when at least that many stores followed
    the prologue: with fewer, step 0's DMA may still be in flight."""
    tiles = [(40, 0), (40, 8)]
    with pytest.raises(AssertionError):
        check(persist_program(tiles, XW - 4), [40, 40])


def test_model_catches_a_prologue_before_the_barrier():
    """The next tile's prologue overwrites stages the last steps were read
    from: without the barrier after the last MFMAs it must be caught."""
    tiles = [(40, 0), (40, 0)]
    p = persist_program(tiles, XW)
    # drop the barrier that precedes tile 1's first DMA
    first = next(i for i, ev in enumerate(p.ev) if ev[0] == "issue" and ev[2][0] == 1)
    j = first - 1
    while p.ev[j][0] != "barrier":
        j -= 1
    del p.ev[j]
    with pytest.raises(AssertionError):
        check(p, [40, 40])


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
    first = next(i for i, ev in enumerate(p.ev) if ev[0] == "issue" and ev[1] == "P" and ev[2] == (0, NS))
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
        if ev[0] == "read" and ev[1] == (0, 15) and ev[3] == 0:
            p.ev[i] = ev[:4] + (False,) + ev[5:]   # P of step 15 read as row-major
            break
    with pytest.raises(AssertionError):
        check(p, 40)
