"""Host emulation of the sweep-group protocol (no GPU).

The group kernel runs G consecutive sweeps of a pass in one workgroup on a
ring of W band rows in LDS; groups hand rows to each other through memory:

  * group g loads row i only once X_{g-1} > i, and publishes
    X_g = min(rows written back, X_{g-1});
  * sweep j of a group starts half-cycle q once sweep j-1 has completed
    min(q + d, all of its) half-cycles, and publishes its final count only
    after sweep j-1's final count;
  * every sweep publishes the lowest row it will still touch; the auxiliary
    wave writes back rows below the group's minimum and reuses their slots,
    loading at most W rows ahead of the lowest live row.

This test executes the real half-cycle arithmetic (plain numpy, the same
code for both sides) under random interleavings of every enabled action of
every group -- each group's rows living in its own private copy, as in LDS,
and only reaching the shared matrix through write-backs -- and checks that:
  * the result equals the sequential reduction to the bit (every dependence
    between sweeps is honoured, no update is lost or read stale);
  * the emulation never deadlocks with the ring size the library computes
    (group_ring_rows, re-derived here).
"""
import numpy as np
import pytest

from refs import cycles_of_sweep, pass_list


def lag(b, t):
    bp = b - t
    return 2 if bp >= 3 else (3 if bp == 2 else 4)


def half_geom(n, b, t, R, q):
    k, h = q // 2, q % 2
    c = R + (b - t) + k * b
    ch = min(c + t, n - 1)
    r = R if k == 0 else c - b
    jend = min(c + t + b, n - 1)
    return h, r, c, ch, jend


def house(x):
    alpha = x[0]
    s = float(np.sum(x[1:] * x[1:])) if len(x) > 1 else 0.0
    if s == 0.0:
        return None
    nrm = np.sqrt(alpha * alpha + s)
    beta = -nrm if alpha >= 0 else nrm
    return beta, (beta - alpha) / beta, 1.0 / (alpha - beta)


def do_half(rows, n, b, t, R, q):
    """One half-cycle on a dict row -> dense row (modified in place)."""
    h, r, c, ch, jend = half_geom(n, b, t, R, q)
    if h == 0:
        x = rows[r][c:ch + 1].copy()
        hh = house(x)
        if hh is not None:
            beta, tau, inv = hh
            v = x * inv
            for i in range(r + 1, ch + 1):
                a = rows[i][c:ch + 1]
                w = a[0] + float(np.dot(a[1:], x[1:])) * inv
                a[0] -= tau * w
                a[1:] -= tau * w * v[1:]
            rows[r][c] = beta
        rows[r][c + 1:ch + 1] = 0.0
    else:
        y = np.array([rows[i][c] for i in range(c, ch + 1)])
        hh = house(y)
        if hh is not None:
            beta, tau, inv = hh
            v = y * inv
            for col in range(c + 1, jend + 1):
                a = np.array([rows[i][col] for i in range(c, ch + 1)])
                w = a[0] + float(np.dot(a[1:], y[1:])) * inv
                a[0] -= tau * w
                a[1:] -= tau * w * v[1:]
                for ii, i in enumerate(range(c, ch + 1)):
                    rows[i][col] = a[ii]
            rows[c][c] = beta
        for i in range(c + 1, ch + 1):
            rows[i][c] = 0.0


def sequential(A, b, t):
    n = A.shape[0]
    rows = {i: A[i].copy() for i in range(n)}
    for R in range(max(n - (b - t) - 1, 0)):
        for q in range(2 * cycles_of_sweep(n, b, t, R)):
            do_half(rows, n, b, t, R, q)
    return np.array([rows[i] for i in range(n)])


def half_rows(n, b, t, R, q):
    h, r, c, ch, _ = half_geom(n, b, t, R, q)
    return (r if h == 0 else c), ch


def group_ring_rows(n, b, t, G):
    """The library's ring size (bb_plan.hpp group_ring_rows), re-derived."""
    ns = max(n - (b - t) - 1, 0)
    d = lag(b, t)
    need = 0
    for R0 in range(0, ns, G):
        Gg = min(G, ns - R0)
        K = [cycles_of_sweep(n, b, t, R0 + j) for j in range(Gg)]
        steps = max(2 * K[j] + j * d for j in range(Gg))
        for q0 in range(steps):
            hi, fl = -1, n
            for j in range(Gg):
                qa = q0 - j * (d - 1)
                if 0 <= qa < 2 * K[j]:
                    hi = max(hi, half_rows(n, b, t, R0 + j, qa)[1])
                qb = q0 - j * d
                if qb < 0:
                    fl = min(fl, R0 + j)
                elif qb < 2 * K[j]:
                    fl = min(fl, half_rows(n, b, t, R0 + j, qb)[0])
            if hi >= 0:
                need = max(need, hi - fl + 1)
    return need


class Group:
    def __init__(self, g, G, ns, n, b, t):
        self.g, self.R0 = g, g * G
        self.Gg = min(G, ns - self.R0)
        self.K = [cycles_of_sweep(n, b, t, self.R0 + j) for j in range(self.Gg)]
        self.Kp = [cycles_of_sweep(n, b, t, self.R0 + j - 1) if j > 0 else 0 for j in range(self.Gg)]
        self.prog = [0] * self.Gg          # published half-cycles
        self.done = [0] * self.Gg          # executed half-cycles
        self.floor = [self.R0 + j for j in range(self.Gg)]
        self.loaded = self.written = self.R0
        self.X = 0
        self.lds = {}


def emulate(A, b, t, G, W, rng, max_live=None, wait_for_prev=True):
    n = A.shape[0]
    d = lag(b, t)
    ns = max(n - (b - t) - 1, 0)
    mem = {i: A[i].copy() for i in range(n)}
    groups = [Group(g, G, ns, n, b, t) for g in range((ns + G - 1) // G)]
    started = 0 if max_live else len(groups)

    def xprev(gr):
        return n if gr.g == 0 or not wait_for_prev else groups[gr.g - 1].X

    def finished(gr):
        return gr.X >= n

    while True:
        live = [gr for gr in groups[:started] if not finished(gr)] if max_live else \
            [gr for gr in groups if not finished(gr)]
        if max_live and len(live) < max_live and started < len(groups):
            started += 1
            continue
        if not live:
            break
        actions = []
        for gr in live:
            for j in range(gr.Gg):
                q = gr.done[j]
                if q == gr.prog[j] and q < 2 * gr.K[j]:   # ready to run half q
                    lo, hi = half_rows(n, b, t, gr.R0 + j, q)
                    pred_ok = j == 0 or gr.prog[j - 1] >= min(q + d, 2 * gr.Kp[j])
                    if pred_ok and gr.loaded > hi:
                        actions.append(("half", gr, j))
                elif gr.done[j] == gr.prog[j] + 1:         # executed, not yet published
                    final = gr.done[j] == 2 * gr.K[j]
                    if not final or j == 0 or gr.prog[j - 1] >= 2 * gr.Kp[j]:
                        actions.append(("publish", gr, j))
            dead = min(gr.floor) if gr.Gg else n
            if min(dead, gr.loaded) > gr.written:
                actions.append(("writeback", gr, None))
            lim = min(xprev(gr), gr.written + W, n)
            if lim > gr.loaded:
                actions.append(("load", gr, None))
            if min(gr.written, xprev(gr)) > gr.X:
                actions.append(("announce", gr, None))
        if not actions:
            raise RuntimeError("deadlock")
        kind, gr, j = actions[rng.integers(len(actions))]
        if kind == "half":
            R, q = gr.R0 + j, gr.done[j]
            lo, hi = half_rows(n, b, t, R, q)
            assert all(i in gr.lds for i in range(lo, hi + 1))
            assert lo >= gr.written   # never touches a row already handed on
            do_half(gr.lds, n, b, t, R, q)
            gr.done[j] += 1
        elif kind == "publish":
            q = gr.done[j]
            gr.floor[j] = half_geom(n, b, t, gr.R0 + j, q - 1)[2] if q < 2 * gr.K[j] else n
            gr.prog[j] = q
        elif kind == "writeback":
            wb = min(min(gr.floor), gr.loaded)
            for i in range(gr.written, wb):
                mem[i] = gr.lds.pop(i).copy()
            gr.written = wb
        elif kind == "load":
            lim = min(xprev(gr), gr.written + W, n)
            for i in range(gr.loaded, lim):
                gr.lds[i] = mem[i].copy()
            gr.loaded = lim
            assert len(gr.lds) <= W
        else:
            gr.X = min(gr.written, xprev(gr))
    return np.array([mem[i] for i in range(n)])


SHAPES = [(40, 8, 3, 2), (40, 8, 3, 4), (48, 16, 15, 3), (50, 12, 4, 3), (45, 6, 5, 4), (36, 9, 8, 2),
          (60, 10, 2, 3), (30, 4, 2, 5), (33, 7, 6, 8), (24, 16, 5, 2)]


@pytest.mark.parametrize("n,bw,tw,G", SHAPES)
def test_group_protocol_matches_sequential(n, bw, tw, G):
    rng = np.random.default_rng(n * 100 + bw)
    A = np.triu(np.tril(rng.standard_normal((n, n)), bw))
    for (b, t) in pass_list(bw, tw):
        ref = sequential(A, b, t)
        W = group_ring_rows(n, b, t, G)
        for trial in range(3):
            out = emulate(A, b, t, G, W, np.random.default_rng(trial), max_live=(None if trial == 0 else 2))
            assert np.array_equal(out, ref), (b, t, trial)
        A = ref


def test_ring_rows_of_the_headline_passes():
    # LDS budget: the library keeps the ring within 158 KiB (stride 100 fp32 = 400 B/row)
    rows = {(b, t): group_ring_rows(2000, b, t, G) for (b, t, G) in [(64, 16, 4), (48, 16, 6), (32, 16, 8),
                                                                       (16, 15, 8)]}
    assert all(r * 400 <= 158 * 1024 for r in rows.values()), rows


def test_emulation_detects_a_broken_rule():
    # the same emulation with one planted mistake -- groups load rows without
    # waiting for their predecessor to release them -- gives wrong results
    n, b, t, G = 40, 8, 3, 2
    rng = np.random.default_rng(1)
    A = np.triu(np.tril(rng.standard_normal((n, n)), b))
    ref = sequential(A, b, t)
    W = group_ring_rows(n, b, t, G)
    bad = sum(not np.array_equal(emulate(A, b, t, G, W, np.random.default_rng(trial), wait_for_prev=False), ref)
              for trial in range(5))
    assert bad > 0
