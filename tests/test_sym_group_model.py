"""Host emulation of the sweep-group protocol for the symmetric reduction
(no GPU): the group kernel's rules (rows released between groups through
X_g, in-group waits of d half-cycles, floors, a ring of W rows) with the
symmetric half-cycle as the unit of work: half 2k forms cycle k's reflector
and applies it to the pivot row and the row segments above the block, half
2k+1 applies it to the block and the column segments (the reflector passes
between the two halves in the wave's registers).

As in test_group_model.py, the real cycle arithmetic runs (numpy, the same
code for both sides) under random interleavings of every enabled action,
each group on private copies of its rows (as in LDS) that reach the shared
matrix only through write-backs, and the test checks that the result equals
the sequential reduction to the bit and that no interleaving deadlocks with
the ring size the library computes (re-derived here).
"""
import numpy as np
import pytest

from refs import pass_list


def cycles_of(n, b, t, R):
    last = n - 2 - R - (b - t)
    return 0 if last < 0 else last // b + 1


def lag(b, t):
    """Half-cycles of separation (d)."""
    bp = b - t
    return 2 if bp >= 3 else (3 if bp == 2 else 4)


def cyc_geom(n, b, t, R, k):
    c = R + (b - t) + k * b
    ch = min(c + t, n - 1)
    p = R if k == 0 else c - b
    return c, ch, p


def half_rows(n, b, t, R, q):
    """Rows half q of sweep R touches: half 2k = rows p..c-1 (pivot row and
    the row segments), half 2k+1 = rows c..ch (block, column segments)."""
    c, ch, p = cyc_geom(n, b, t, R, q // 2)
    return (p, c - 1) if q % 2 == 0 else (c, ch)


def half_floor(n, b, t, R, q, K):
    """Lowest row sweep R still touches after q halves."""
    if q >= 2 * K:
        return n
    c, ch, p = cyc_geom(n, b, t, R, q // 2)
    return p if q % 2 == 0 else c


def prep_a(rows, n, b, t, R, q):
    """First part of half A (q even): the reflector from pivot row p at
    columns c..ch, and the pivot's final values (beta, then zeros)."""
    c, ch, p = cyc_geom(n, b, t, R, q // 2)
    x = rows[p][c:ch + 1].copy()
    s = float(np.dot(x[1:], x[1:]))
    refl = None
    if s != 0.0:
        alpha = x[0]
        nrm = np.sqrt(alpha * alpha + s)
        beta = -nrm if alpha >= 0 else nrm
        tau = (beta - alpha) / beta
        v = x / (alpha - beta)
        v[0] = 1.0
        refl = (tau, v)
        rows[p][c] = beta
    rows[p][c + 1:ch + 1] = 0.0
    return refl


def do_half(rows, refl, n, b, t, R, q, pre=False):
    """Half q of sweep R on dense upper rows; refl carries v and tau from
    half 2k to half 2k+1 (as the wave's registers do).  pre: half A's first
    part (prep_a) has already run and refl[R] holds its result."""
    c, ch, p = cyc_geom(n, b, t, R, q // 2)
    m = ch - c + 1
    if q % 2 == 0:
        if not pre:
            refl[R] = prep_a(rows, n, b, t, R, q)
        if refl[R] is not None:
            tau, v = refl[R]
            for i in range(p + 1, c):
                a = rows[i][c:ch + 1]
                w = tau * (a[0] + float(np.dot(a[1:], v[1:])))
                a[0] -= w
                a[1:] -= w * v[1:]
        return
    if refl[R] is None:
        return
    tau, v = refl[R]
    for j in range(ch + 1, min(ch + b, n - 1) + 1):
        a = np.array([rows[c + i][j] for i in range(m)])
        w = tau * (a[0] + float(np.dot(a[1:], v[1:])))
        a[0] -= w
        a[1:] -= w * v[1:]
        for i in range(m):
            rows[c + i][j] = a[i]
    B = np.array([[rows[c + min(i, j)][c + max(i, j)] for j in range(m)] for i in range(m)])
    y = tau * (B @ v)
    alpha2 = -(0.5 * tau) * float(y @ v)
    z = y + alpha2 * v
    for i in range(m):
        for j in range(i, m):
            rows[c + i][c + j] = B[i, j] - v[i] * z[j] - z[i] * v[j]


def sequential(A, b, t):
    n = A.shape[0]
    rows = {i: A[i].copy() for i in range(n)}
    refl = {}
    for R in range(max(n - (b - t) - 1, 0)):
        for q in range(2 * cycles_of(n, b, t, R)):
            do_half(rows, refl, n, b, t, R, q)
    return np.array([rows[i] for i in range(n)])


def sym_group_ring_rows(n, b, t, G):
    """The library's ring size (bb_plan.hpp sym_group_ring_rows), re-derived."""
    ns = max(n - (b - t) - 1, 0)
    d = lag(b, t)
    need = 0
    for R0 in range(0, ns, G):
        Gg = min(G, ns - R0)
        K2 = [2 * cycles_of(n, b, t, R0 + j) for j in range(Gg)]
        steps = max(K2[j] + j * d for j in range(Gg))
        for q0 in range(steps):
            hi, fl = -1, n
            for j in range(Gg):
                qa = q0 - j * (d - 1)
                if 0 <= qa < K2[j]:
                    hi = max(hi, half_rows(n, b, t, R0 + j, qa)[1])
                qb = q0 - j * d
                if qb < 0:
                    fl = min(fl, R0 + j)
                elif qb < K2[j]:
                    fl = min(fl, half_rows(n, b, t, R0 + j, qb)[0])
            if hi >= 0:
                need = max(need, hi - fl + 1)
    return need


class Group:
    def __init__(self, g, G, ns, n, b, t, p=0):
        self.g, self.R0, self.b, self.t, self.p = g, g * G, b, t, p
        self.Gg = min(G, ns - self.R0)
        self.K = [2 * cycles_of(n, b, t, self.R0 + j) for j in range(self.Gg)]
        self.Kp = [2 * cycles_of(n, b, t, self.R0 + j - 1) if j > 0 else 0 for j in range(self.Gg)]
        self.refl = {}
        self.prog = [0] * self.Gg
        self.done = [0] * self.Gg
        self.floor = [self.R0 + j for j in range(self.Gg)]
        self.loaded = self.written = self.R0
        self.X = 0
        self.lds = {}
        self.pre = [False] * self.Gg
        self.st = [0] * self.Gg          # published steps


def emulate(A, b, t, G, W, rng, max_live=None, d=None, early=False, first=2, all_marks=False, steps=None):
    """One pass (b, t): see emulate_run."""
    return emulate_run(A, [(b, t)], G, W, rng, max_live=max_live, d=d, early=early, first=first,
                       all_marks=all_marks, steps=steps)


def emulate_run(A, passes, G, W, rng, max_live=None, d=None, early=False, first=2, all_marks=False, steps=None,
                cross=True, batch=None):
    """A run of passes in one launch: the groups of every pass in one claim
    order, pass by pass (max_live of them resident at a time; G, sweeps per
    group, one for all passes or one per pass).  The first group of a pass
    after the first loads rows [loaded, want), want = loaded + batch, only
    below X of the previous pass's group that owns row want - 1 (cross =
    False plants a mistake: it loads without waiting).
    early: a sweep runs half A's first part (reflector and pivot) as soon
    as it has published the half before it, ahead of its waits (the kernel's
    schedule), for every half A from half `first` on (2; 0 plants a mistake:
    half 0's pivot row comes from the predecessor), and for b' <= 2 (or every
    b' with all_marks) publishes that first part as a step.  Progress counts
    steps, two per half; half q waits for min(2q + steps, all) steps of the
    predecessor, steps = 2d - 1 with first-part steps, else 2d (d: the lag
    in halves, default lag(b, t))."""
    n = A.shape[0]
    batch = batch or n
    Gs = G if isinstance(G, (list, tuple)) else [G] * len(passes)
    mem = {i: A[i].copy() for i in range(n)}
    groups, first_of = [], []
    for p, (b, t) in enumerate(passes):
        ns = max(n - (b - t) - 1, 0)
        first_of.append(len(groups))
        groups += [Group(g, Gs[p], ns, n, b, t, p) for g in range((ns + Gs[p] - 1) // Gs[p])]
    first_of.append(len(groups))
    started = 0 if max_live else len(groups)

    def xprev(gr, want):
        if gr.p == 0 and gr.g == 0:
            return n
        if gr.g > 0:
            return groups[first_of[gr.p] + gr.g - 1].X
        if not cross:
            return n
        lo, hi = first_of[gr.p - 1], first_of[gr.p]
        if lo == hi:
            return n
        return groups[lo + min((want - 1) // Gs[gr.p - 1], hi - lo - 1)].X

    while True:
        live = [gr for gr in groups[:started] if gr.X < n]
        if max_live and len(live) < max_live and started < len(groups):
            started += 1
            continue
        if not live:
            break
        acts = []
        for gr in live:
            b, t = gr.b, gr.t
            L = lag(b, t) if d is None else d   # half-cycles
            mark = early and (b - t <= 2 or all_marks)
            LS = (2 * L - 1 if mark else 2 * L) if steps is None else steps
            for j in range(gr.Gg):
                q = gr.done[j]
                if early and q == gr.prog[j] and q % 2 == 0 and first <= q < gr.K[j] and not gr.pre[j]:
                    acts.append(("prep", gr, j))
                if q == gr.prog[j] and q < gr.K[j] and (not early or q % 2 or q < first or gr.pre[j]):
                    lo, hi = half_rows(n, b, t, gr.R0 + j, q)
                    pred_ok = j == 0 or gr.st[j - 1] >= min(2 * q + LS, 2 * gr.Kp[j])
                    if pred_ok and gr.loaded > hi:
                        acts.append(("cycle", gr, j))
                elif gr.done[j] == gr.prog[j] + 1:
                    final = gr.done[j] == gr.K[j]
                    if not final or j == 0 or gr.st[j - 1] >= 2 * gr.Kp[j]:
                        acts.append(("publish", gr, j))
            dead = min(gr.floor) if gr.Gg else n
            if min(dead, gr.loaded) > gr.written:
                acts.append(("writeback", gr, None))
            want = min(n, gr.loaded + batch)
            if min(xprev(gr, want), gr.written + W, want) > gr.loaded:
                acts.append(("load", gr, None))
            if gr.written > max(gr.X, gr.R0):             # X moves only past rows written back
                acts.append(("announce", gr, None))
        if not acts:
            raise RuntimeError("deadlock")
        kind, gr, j = acts[rng.integers(len(acts))]
        b, t = gr.b, gr.t
        if kind == "cycle":
            R, q = gr.R0 + j, gr.done[j]
            lo, hi = half_rows(n, b, t, R, q)
            assert all(i in gr.lds for i in range(lo, hi + 1)) and lo >= gr.written
            do_half(gr.lds, gr.refl, n, b, t, R, q, pre=gr.pre[j])
            gr.pre[j] = False
            gr.done[j] += 1
        elif kind == "prep":
            R, q = gr.R0 + j, gr.done[j]
            c, ch, p = cyc_geom(n, b, t, R, q // 2)
            assert p in gr.lds and p >= gr.written
            gr.refl[R] = prep_a(gr.lds, n, b, t, R, q)
            gr.pre[j] = True
            if early and (b - t <= 2 or all_marks):
                gr.st[j] = 2 * q + 1
        elif kind == "publish":
            q = gr.done[j]
            gr.floor[j] = half_floor(n, b, t, gr.R0 + j, q, gr.K[j] // 2)
            gr.prog[j] = q
            gr.st[j] = 2 * q
        elif kind == "writeback":
            wb = min(min(gr.floor), gr.loaded)
            for i in range(gr.written, wb):
                mem[i] = gr.lds.pop(i).copy()
            gr.written = wb
        elif kind == "load":
            want = min(n, gr.loaded + batch)
            lim = min(xprev(gr, want), gr.written + W, want)
            for i in range(gr.loaded, lim):
                gr.lds[i] = mem[i].copy()
            gr.loaded = lim
            assert len(gr.lds) <= W
        else:
            gr.X = gr.written
    return np.array([mem[i] for i in range(n)])


SHAPES = [(40, 8, 3, 2), (40, 8, 3, 3), (36, 6, 5, 3), (45, 6, 2, 4), (30, 4, 1, 3), (33, 7, 6, 5), (50, 10, 4, 2)]


@pytest.mark.parametrize("early", [False, True])
@pytest.mark.parametrize("n,bw,tw,G", SHAPES)
def test_sym_group_protocol_matches_sequential(n, bw, tw, G, early):
    rng = np.random.default_rng(n * 10 + bw)
    A = np.triu(np.tril(rng.standard_normal((n, n)), bw))   # upper rows of a symmetric band
    for (b, t) in pass_list(bw, tw):
        ref = sequential(A, b, t)
        W = sym_group_ring_rows(n, b, t, G)
        for trial in range(3):
            out = emulate(A, b, t, G, W, np.random.default_rng(trial), max_live=(None if trial == 0 else 2),
                          early=early)
            assert np.array_equal(out, ref), (b, t, trial)
        A = ref
    T = A
    assert np.all(np.triu(T, 2) == 0)


def test_cycle_is_the_oracles():
    # the emulation's numpy cycle reduces to the same tridiagonal as the
    # symmetric oracle (up to rounding: different summation order)
    import oracle
    n, bw, tw = 30, 6, 2
    rng = np.random.default_rng(5)
    band = rng.standard_normal((n, bw + 1))
    A = np.zeros((n, n))
    for i in range(n):
        for o in range(bw + 1):
            if i + o < n:
                A[i, i + o] = band[i, o]
    for (b, t) in pass_list(bw, tw):
        A = sequential(A, b, t)
    d, e = oracle.sym_reduce(band, bw, tw)
    assert np.allclose(np.diag(A), d, atol=1e-12) and np.allclose(np.abs(np.diag(A, 1)), np.abs(e), atol=1e-12)


def test_emulation_detects_a_broken_rule():
    # one half-cycle less of separation inside the groups gives wrong results
    n, bw, tw, G = 40, 8, 3, 4
    rng = np.random.default_rng(3)
    A = np.triu(np.tril(rng.standard_normal((n, n)), bw))
    b, t = pass_list(bw, tw)[0]
    ref = sequential(A, b, t)
    W = sym_group_ring_rows(n, b, t, G)
    bad = 0
    for trial in range(6):
        try:
            out = emulate(A, b, t, G, W + 8, np.random.default_rng(trial), d=lag(b, t) - 1)
        except (RuntimeError, AssertionError):
            bad += 1
            continue
        bad += not np.array_equal(out, ref)
    assert bad > 0


def test_emulation_detects_an_early_first_pivot():
    # forming half 0's reflector before the wait (its pivot row R is still
    # updated by the predecessor) gives wrong results
    n, bw, tw, G = 40, 8, 3, 3
    rng = np.random.default_rng(7)
    A = np.triu(np.tril(rng.standard_normal((n, n)), bw))
    b, t = pass_list(bw, tw)[0]
    ref = sequential(A, b, t)
    W = sym_group_ring_rows(n, b, t, G)
    bad = 0
    for trial in range(6):
        try:
            out = emulate(A, b, t, G, W, np.random.default_rng(trial), early=True, first=0)
        except (RuntimeError, AssertionError):
            bad += 1
            continue
        bad += not np.array_equal(out, ref)
    assert bad > 0


@pytest.mark.parametrize("n,bw,tw,G", [(40, 16, 15, 3), (48, 16, 14, 3), (40, 8, 3, 3), (50, 10, 4, 2)])
def test_emulation_detects_a_short_wait(n, bw, tw, G):
    # one step less than the kernel waits for gives wrong results (first-part
    # steps published for every b', to show that b' >= 3 must not use them)
    rng = np.random.default_rng(9)
    A = np.triu(np.tril(rng.standard_normal((n, n)), bw))
    b, t = pass_list(bw, tw)[0]
    ref = sequential(A, b, t)
    W = sym_group_ring_rows(n, b, t, G) + 8
    ls = 2 * lag(b, t) - 1 if b - t <= 2 else 2 * lag(b, t)
    bad = 0
    for trial in range(6):
        try:
            out = emulate(A, b, t, G, W, np.random.default_rng(trial), early=True, all_marks=True, steps=ls - 1)
        except (RuntimeError, AssertionError):
            bad += 1
            continue
        bad += not np.array_equal(out, ref)
    assert bad > 0


@pytest.mark.parametrize("n,bw,tw,G", [(40, 8, 3, [2, 3, 2]), (36, 6, 2, 3), (45, 12, 5, [3, 2, 4]), (30, 9, 8, 2)])
def test_sym_run_of_passes_matches_sequential(n, bw, tw, G):
    # every pass in one launch: a pass's first group loads each row once the
    # previous pass's group that owns it has released it
    rng = np.random.default_rng(n * 3 + bw)
    A = np.triu(np.tril(rng.standard_normal((n, n)), bw))
    passes = pass_list(bw, tw)
    Gs = G if isinstance(G, list) else [G] * len(passes)
    Gs = (Gs * len(passes))[:len(passes)]
    ref = A
    for (b, t) in passes:
        ref = sequential(ref, b, t)
    W = max(sym_group_ring_rows(n, b, t, g) for (b, t), g in zip(passes, Gs)) + 2
    for trial in range(3):
        out = emulate_run(A, passes, Gs, W, np.random.default_rng(trial), early=True, batch=[3, 5, 64][trial],
                          max_live=[None, 2, 3][trial])
        assert np.array_equal(out, ref), trial


def test_sym_run_detects_a_missing_cross_pass_wait():
    n, bw, tw = 40, 8, 3
    rng = np.random.default_rng(6)
    A = np.triu(np.tril(rng.standard_normal((n, n)), bw))
    passes = pass_list(bw, tw)
    ref = A
    for (b, t) in passes:
        ref = sequential(ref, b, t)
    W = max(sym_group_ring_rows(n, b, t, 2) for (b, t) in passes) + 2
    bad = 0
    for trial in range(5):
        try:
            out = emulate_run(A, passes, 2, W, np.random.default_rng(trial), early=True, batch=4, cross=False)
        except (RuntimeError, AssertionError):
            bad += 1
            continue
        bad += not np.array_equal(out, ref)
    assert bad > 0
