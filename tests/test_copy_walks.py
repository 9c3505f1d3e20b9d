"""Host models of the add-only index walks in the copy loops (no GPU).

Two kernels step through their copies with adds instead of a division per
element; the GPU parity tests check the kernels' results, and these tests
check the identity each walk relies on, over the shapes the kernels meet:

* the group kernel's window walk (loader and writer of windowed rings): lane
  l visits 16-byte chunks l, l + 64, ... of ring rows stored back to back
  (rc chunks per row); 64 = q rc + s, so a step adds q rows and s chunks,
  plus one row when the chunk's place in its row reaches rc.  The offset it
  keeps must equal the direct one, (lo + c // rc) * row_bytes + w0 +
  16 (c % rc);
* the persistent kernel's element stores of a staged row half: thread t of
  nt visits elements t, t + nt, ... of the (nr - 1) x m block (row 1 + e // m,
  entry e % m), eight at a time, first below the early part's end ep and then
  on, continuing the same walk; every element must be visited exactly once.
"""
import pytest


def direct_offset(row_bytes, w0, rb, lo, e):
    c = e // 16
    i = c // (rb // 16)
    return (lo + i) * row_bytes + w0 + (e - i * rb)


def window_walk(row_bytes, w0, rb, lo, nbytes, lane):
    rc = rb // 16
    q, s = 64 // rc, 64 % rc
    i0 = lane // rc
    r = lane - i0 * rc
    at = (lo + i0) * row_bytes + w0 + 16 * r
    d0, d1 = q * row_bytes + 16 * s, row_bytes - 16 * rc
    out = []
    for off in range(0, nbytes, 1024):
        if off + 16 * lane < nbytes:
            out.append((off + 16 * lane, at))
        r += s
        at += d0
        if r >= rc:
            r -= rc
            at += d1
    return out


# window widths of the windowed passes (384, 528, 656 bytes in fp32, 768 in
# fp64) and every other multiple of 16 up to 1264 bytes
WIDTHS = sorted({384, 528, 656, 768} | {16 * k for k in range(1, 80, 3)})


@pytest.mark.parametrize("rb", WIDTHS)
def test_window_walk_matches_direct_offsets(rb):
    for row_bytes, w0, lo, rows in [(rb, 0, 0, 1), (rb + 16, 16, 7, 5), (rb + 640, 96, 12345, 37), (2 * rb, rb, 65000, 96)]:
        nbytes = rows * rb
        for lane in range(64):
            for e, at in window_walk(row_bytes, w0, rb, lo, nbytes, lane):
                assert at == direct_offset(row_bytes, w0, rb, lo, e), (rb, row_bytes, lo, rows, lane, e)


def element_walk(nt, m, ne, ep):
    seen = {}
    for tid in range(nt):
        qs, ss = nt // m, nt % m
        i = 1 + tid // m
        j = tid - (i - 1) * m
        e = tid

        def step():
            nonlocal e, i, j
            e += nt
            j += ss
            i += qs
            if j >= m:
                j -= m
                i += 1

        for lim in (ep, ne):
            while e + 7 * nt < lim:
                for _ in range(8):
                    assert (i, j) == (1 + e // m, e % m)
                    seen[e] = seen.get(e, 0) + 1
                    step()
            while e < lim:
                assert (i, j) == (1 + e // m, e % m)
                seen[e] = seen.get(e, 0) + 1
                step()
    return seen


@pytest.mark.parametrize("nt", [64, 128, 256])
def test_element_walk_covers_each_element_once(nt):
    for m in (1, 2, 7, 16, 17, 31, 32, 33, 65):
        for nr in (1, 2, 33, 97, 161, 289):
            for early in (0, 1, 17, 33, 1000):
                ne, ep = (nr - 1) * m, min(early, nr - 1) * m
                seen = element_walk(nt, m, ne, ep)
                assert sorted(seen) == list(range(ne)) and set(seen.values()) <= {1}, (nt, m, nr, early)


def staged_chunk_walk(nt, CH, nr, rstep, o0):
    """The persistent kernel's staged loads: wave w's lanes copy chunks
    e0 + lane, e0 = 64 w, 64 w + nt, ... (whole waves unmasked, then one
    partial); thread tid keeps (row, chunk) and the row's memory offset by
    adds.  Returns {chunk: source offset}."""
    nch = nr * CH
    got = {}
    qc, sc = nt // CH, nt % CH
    for tid in range(nt):
        lane = tid % 64
        ci, cc = tid // CH, tid % CH
        srow = o0 + ci * rstep
        e0 = tid - lane
        while e0 + 64 <= nch:
            assert e0 + lane not in got
            got[e0 + lane] = (srow & ~15) + cc * 16
            cc += sc
            srow += qc * rstep
            if cc >= CH:
                cc -= CH
                srow += rstep
            e0 += nt
        if e0 < nch and e0 + lane < nch:
            assert e0 + lane not in got
            got[e0 + lane] = (srow & ~15) + cc * 16
    return got


@pytest.mark.parametrize("nt", [64, 128, 192, 256])
def test_staged_chunk_walk_matches_division(nt):
    for CH in (3, 5, 9, 17):
        for nr in (1, 2, 33, 97, 129, 161, 289):
            for rstep, o0 in ((1292, 4), (1288, 8), (3000, 0), (2584, 16)):
                got = staged_chunk_walk(nt, CH, nr, rstep, o0)
                assert sorted(got) == list(range(nr * CH))
                for e, src in got.items():
                    i = e // CH
                    assert src == ((o0 + i * rstep) & ~15) + (e - i * CH) * 16, (nt, CH, nr, e)
