"""Host model of the persistent scheduler's wait rule (no GPU).

Each sweep runs its half-cycles in order (2k: row half, 2k+1: column half).
Before half h of cycle k, sweep R waits until sweep R-1 has completed

    need(R, k, h) = min(2k + h + d(b'), all of R-1's half-cycles),
    d = 2 (b' >= 3), 3 (b' = 2), 4 (b' = 1)

(the kernel's half_cycles_needed), and a sweep publishes its final count only
once its predecessor has published its own, so "R-1 complete" implies "every
earlier sweep complete".  The test enumerates, for small shapes, every pair
of half-cycles that touch a common entry and checks that the one earlier in
the sequential order is guaranteed to finish first through the chain of
waits -- so any schedule obeying the rule computes the sequential result.  It
also shows that the rule cannot be loosened: without the transitive
completion, or with a smaller lag for b' = 2 or b' = 1, conflicts go
unordered.
"""
import pytest

from refs import cycles_of_sweep, pass_list


def half_cells(n, b, t, R, k, h):
    bp = b - t
    c = R + bp + k * b
    ch = min(c + t, n - 1)
    r = R if k == 0 else c - b
    s = set()
    if h == 0:
        s.update((r, j) for j in range(c, ch + 1))
        s.update((i, j) for i in range(r + 1, ch + 1) for j in range(c, ch + 1))
    else:
        s.update((i, j) for i in range(c, ch + 1) for j in range(c, min(c + t + b, n - 1) + 1))
    return s


def rule(b, t, k, h, kprev, lag=None):
    bp = b - t
    d = lag if lag is not None else (2 if bp >= 3 else (3 if bp == 2 else 4))
    return min(2 * k + h + d, 2 * kprev)


def uncovered_conflicts(n, b, t, lag=None, completion=True):
    bp = b - t
    ns = max(n - bp - 1, 0)
    K = [cycles_of_sweep(n, b, t, R) for R in range(ns)]
    cells = {(R, q): half_cells(n, b, t, R, q // 2, q % 2) for R in range(ns) for q in range(2 * K[R])}

    def need(R, q):
        return rule(b, t, q // 2, q % 2, K[R - 1], lag)

    bad = 0
    for R in range(1, ns):
        for q in range(2 * K[R]):
            done = {}  # sweep -> number of its half-cycles guaranteed complete
            Rp, w = R - 1, need(R, q)
            while Rp >= 0 and w > 0:
                if completion and w == 2 * K[Rp]:
                    done.update({x: 2 * K[x] for x in range(Rp + 1)})
                    break
                done[Rp] = w
                if Rp == 0:
                    break
                w = need(Rp, w - 1)
                Rp -= 1
            for Rp in range(R):
                for qp in range(2 * K[Rp]):
                    if done.get(Rp, 0) <= qp and cells[(Rp, qp)] & cells[(R, q)]:
                        bad += 1
    return bad


SHAPES = [(200, 64, 16), (150, 48, 16), (120, 16, 8), (100, 18, 15), (96, 64, 16), (90, 48, 16), (80, 32, 16), (70, 16, 15), (60, 3, 1), (50, 4, 2), (77, 8, 6),
          (90, 12, 4), (60, 10, 1), (45, 5, 3), (64, 33, 32), (40, 39, 13), (17, 16, 5), (50, 2, 1)]


@pytest.mark.parametrize("n,b,t", sorted({(n, bb, tt) for (n, bw, tw) in SHAPES for (bb, tt) in pass_list(bw, tw)}))
def test_wait_rule_orders_every_conflict(n, b, t):
    assert uncovered_conflicts(n, b, t) == 0


def test_rule_cannot_be_loosened():
    # without the transitive completion the cap at "all of R-1" is unsound
    assert uncovered_conflicts(120, 16, 8, completion=False) > 0
    assert uncovered_conflicts(100, 18, 15, completion=False) > 0
    # lag 2 is not enough for b' = 2
    assert uncovered_conflicts(50, 4, 2, lag=2) > 0
    # lag 3 is not enough for b' = 1
    assert uncovered_conflicts(50, 2, 1, lag=3) > 0
