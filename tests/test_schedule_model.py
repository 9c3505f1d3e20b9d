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


# ---- Early and late parts of a half (persistent kernel, b' >= 4) ----------
#
# In an interior cycle (k >= 1, full blocks) of a pass with b' >= 4, the
# predecessor's next half touches only t + 1 rows of a row half's block (rows
# c-1 .. c+t-1, its column half of cycle k) and only t + 1 columns of a column
# half's block (columns c+b-1 .. c+b+t-1, its row half of cycle k+1).  The rest
# of the block (the early part) needs one half less of the predecessor: the
# kernel may run it before the half's usual wait, and the rest (the late part)
# after it.  With b' = 3 the early part can meet a half of the sweep three
# back that the weaker wait no longer orders (a scan of every shape with
# b <= 40 finds b' = 3 the only failing case), so the split needs b' >= 4.

def split_parts(n, b, t, R, q, min_bp=4):
    """(early cells, late cells) of half q of sweep R, or None when the half
    runs whole (first cycle, truncated blocks, b' < min_bp)."""
    k, h = q // 2, q % 2
    c = R + (b - t) + k * b
    if b - t < min_bp or k == 0 or R == 0 or c + t + b > n - 1:
        return None
    cells = half_cells(n, b, t, R, k, h)
    if h == 0:
        late = {(i, j) for (i, j) in cells if c - 1 <= i <= c + t - 1}
    else:
        late = {(i, j) for (i, j) in cells if c + b - 1 <= j <= c + b + t - 1}
    return cells - late, late


def uncovered_split_conflicts(n, b, t, early_lag=1, min_bp=4):
    """Conflicts left unordered when the early part of a split half waits for
    q + early_lag halves of the predecessor instead of q + d, and the late
    part for the usual q + d."""
    bp = b - t
    ns = max(n - bp - 1, 0)
    K = [cycles_of_sweep(n, b, t, R) for R in range(ns)]
    ops = {}  # (R, q) -> [(cells, need on R-1)]
    for R in range(ns):
        for q in range(2 * K[R]):
            full = rule(b, t, q // 2, q % 2, K[R - 1]) if R > 0 else 0
            sp = split_parts(n, b, t, R, q, min_bp)
            if sp is None:
                ops[(R, q)] = [(half_cells(n, b, t, R, q // 2, q % 2), full)]
            else:
                ops[(R, q)] = [(sp[0], min(q + early_lag, 2 * K[R - 1])), (sp[1], full)]
    cells = {key: set().union(*[c for c, _ in v]) for key, v in ops.items()}

    def need_whole(R, q):  # what half q of R waited for on R-1, all parts done
        return max(w for _, w in ops[(R, q)])

    bad = 0
    for R in range(1, ns):
        for q in range(2 * K[R]):
            for (cs, w0) in ops[(R, q)]:
                done = {}
                Rp, w = R - 1, w0
                while Rp >= 0 and w > 0:
                    if w == 2 * K[Rp]:
                        done.update({x: 2 * K[x] for x in range(Rp + 1)})
                        break
                    done[Rp] = w
                    if Rp == 0:
                        break
                    w = need_whole(Rp, w - 1)
                    Rp -= 1
                for Rp in range(R):
                    for qp in range(2 * K[Rp]):
                        if done.get(Rp, 0) <= qp and cells[(Rp, qp)] & cs:
                            bad += 1
    return bad


@pytest.mark.parametrize("n,b,t", [(200, 64, 16), (150, 48, 16), (120, 32, 16), (100, 18, 15), (90, 12, 4),
                                   (130, 40, 8), (96, 20, 16), (80, 7, 3), (300, 128, 32), (400, 96, 32),
                                   (120, 19, 15)])
def test_early_part_needs_one_half_less(n, b, t):
    assert uncovered_split_conflicts(n, b, t) == 0


def test_early_part_cannot_start_two_halves_early():
    # the early part still needs the predecessor's previous half
    assert uncovered_split_conflicts(200, 64, 16, early_lag=0) > 0


def test_split_needs_target_band_of_four():
    # with b' = 3 a sweep further back still overlaps the early part
    assert uncovered_split_conflicts(100, 18, 15, min_bp=3) > 0
    assert uncovered_split_conflicts(40, 4, 1, min_bp=3) > 0


# ---- Publishing a half's early part (persistent kernel) ------------------
#
# A half publishes step 2p + 1 once every earlier half is done and its
# pivot and the t + 1 rows (row half) or columns (column half) after it are
# stored, and the sweep's final count once it is done; half q of sweep R
# waits for min(2(q + d - 1) + 1, all) steps of sweep R-1 (the kernel's
# steps_needed): the early part of R-1's half q + d - 1 instead of the whole
# half.  The rest of a half is read before its early part is published and
# written after, so it must meet nothing the successor touches.

def part_cells(n, b, t, R, q, part, early):
    """Cells of half q of sweep R in its early part (part 0: the pivot and
    offsets 1..early) or the rest (part 1)."""
    k, h = q // 2, q % 2
    c = R + (b - t) + k * b
    ch = min(c + t, n - 1)
    r = R if k == 0 else c - b
    jend = min(c + t + b, n - 1)
    s = set()
    if h == 0:
        for i in range(r, ch + 1):
            if (i - r <= early) == (part == 0):
                s.update((i, j) for j in range(c, ch + 1))
    else:
        for j in range(c, jend + 1):
            if (j - c <= early) == (part == 0):
                s.update((i, j) for i in range(c, ch + 1))
    return s


def uncovered_partial_conflicts(n, b, t, early=None, extra=0):
    """Conflicts left unordered under the early-part rule; early: offsets in
    the early part (t + 1; fewer plants a mistake), extra: steps added to
    every wait (-1 plants a mistake)."""
    early = t + 1 if early is None else early
    bp = b - t
    d = 2 if bp >= 3 else (3 if bp == 2 else 4)
    ns = max(n - bp - 1, 0)
    K = [cycles_of_sweep(n, b, t, R) for R in range(ns)]
    cells = {(R, 2 * q + p): part_cells(n, b, t, R, q, p, early)
             for R in range(ns) for q in range(2 * K[R]) for p in (0, 1)}

    def need(R, q):
        return min(2 * (q + d - 1) + 1 + extra, 4 * K[R - 1])

    bad = 0
    for R in range(1, ns):
        for q in range(2 * K[R]):
            done = {}  # sweep -> steps guaranteed published (ops 0..w-1 done)
            Rp, w = R - 1, need(R, q)
            while Rp >= 0 and w > 0:
                if w == 4 * K[Rp]:
                    done.update({x: 4 * K[x] for x in range(Rp + 1)})
                    break
                done[Rp] = w
                if Rp == 0:
                    break
                w = need(Rp, (w - 1) // 2)
                Rp -= 1
            mine = cells[(R, 2 * q)] | cells[(R, 2 * q + 1)]
            for Rp in range(R):
                for op in range(4 * K[Rp]):
                    if done.get(Rp, 0) <= op and cells[(Rp, op)] & mine:
                        bad += 1
    return bad


PARTIAL_SHAPES = [(150, 48, 16), (120, 16, 8), (100, 18, 15), (90, 12, 4), (60, 10, 1), (50, 4, 2), (64, 33, 32),
                  (40, 39, 13), (17, 16, 5), (50, 2, 1), (160, 64, 32)]


@pytest.mark.parametrize("n,b,t", sorted({(n, bb, tt) for (n, bw, tw) in PARTIAL_SHAPES
                                          for (bb, tt) in pass_list(bw, tw)}))
def test_early_part_publication_orders_every_conflict(n, b, t):
    assert uncovered_partial_conflicts(n, b, t) == 0


def test_early_part_publication_cannot_be_loosened():
    # one row or column fewer in the early part (b' >= 3) ...
    assert uncovered_partial_conflicts(120, 16, 8, early=8) > 0
    assert uncovered_partial_conflicts(100, 18, 15, early=15) > 0
    # ... or one step less of the predecessor, at every lag
    assert uncovered_partial_conflicts(120, 16, 8, extra=-1) > 0
    assert uncovered_partial_conflicts(50, 4, 2, extra=-1) > 0
    assert uncovered_partial_conflicts(50, 2, 1, extra=-1) > 0
