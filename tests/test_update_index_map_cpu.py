"""The store map of the writing update kernels, replayed on the host.

k_update's vector path (projection, Muon's decayed update) walks W in units
of 4 columns x a row pair, two units per thread per pass, and issues its
loads and stores unconditionally: a slot past the end of the matrix or of
the block's range reuses the address of a live unit. This test replays the
kernel's index arithmetic for every block and thread, exactly as the kernel
writes it, and checks that

  * the live units of all threads cover every 4-column group of every row
    exactly once, and
  * every store a thread issues lands in one of its own live groups (so no
    two threads ever write the same bytes, and a reused slot rewrites a
    value its own thread computed).

A mistake in the reuse rule (taking the row from one slot and the column
from another) is planted in the replay below and must be caught.

The block counts follow the library's launch descriptors: one-shot blocks
of 2 x 256 units for the writing updates, and up to 256 blocks per matrix
(16384 elements each) for the trial norm, whose loads take the same path.
"""
from __future__ import annotations

import pytest

THREADS = 256
ELEMS_PER_BLOCK = 16384
MAX_PARTIALS = 256


def chunk_range(n, bpm, c):
    ln = (n + bpm - 1) // bpm
    ln = (ln + 3) & ~3
    lo = c * ln
    hi = min(lo + ln, n)
    return min(lo, n), hi


def oneshot_bpm(rows, cols):
    units = ((rows + 1) // 2) * ((cols + 3) // 4)
    return max(1, (units + 2 * THREADS - 1) // (2 * THREADS))


def stream_bpm(rows, cols):
    n = rows * cols
    return max(1, min((n + ELEMS_PER_BLOCK - 1) // ELEMS_PER_BLOCK, MAX_PARTIALS))


def replay(rows, cols, bpm, planted=False):
    """(owner of each live (row, 4-column group), list of violations)."""
    assert cols % 4 == 0
    cq = cols // 4
    npairs = (rows + 1) // 2
    owner = {}
    bad = []
    dpr, dq = THREADS // cq, THREADS - (THREADS // cq) * cq
    for c in range(bpm):
        u0, u1 = chunk_range(npairs * cq, bpm, c)
        for t in range(THREADS):
            u = u0 + t
            pr, q = divmod(u, cq)
            while u < u1:
                prs = [pr, pr + dpr]
                qs = [q, q + dq]
                if qs[1] >= cq:
                    qs[1] -= cq
                    prs[1] += 1
                has1 = u + THREADS < u1
                mine = set()
                stores = []
                for j in range(2):
                    for h in range(2):
                        unit = j == 0 or has1
                        r = 2 * prs[j] + h
                        live = unit and r < rows
                        if planted:  # row of slot 0 with the column of slot j
                            rl = r if live else 2 * prs[0]
                            cl = qs[j] if unit else qs[0]
                        else:
                            rl = r if live else 2 * (prs[j] if unit else prs[0])
                            cl = qs[j] if unit else qs[0]
                        if live:
                            key = (r, qs[j])
                            if key in owner:
                                bad.append(("twice", key))
                            owner[key] = (c, t)
                            mine.add(key)
                        stores.append((rl, cl))
                for s in stores:
                    if s not in mine:
                        bad.append(("foreign store", (c, t), s))
                pr = prs[1] + dpr
                q = qs[1] + dq
                if q >= cq:
                    q -= cq
                    pr += 1
                u += 2 * THREADS
    return owner, bad


SHAPES = [(129, 2052), (1001, 1200), (37, 52), (1, 64), (3, 4), (2, 1024), (7, 260), (513, 1028),
          (2048, 512), (65, 4096)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("kind", ["oneshot", "stream"])
def test_every_store_lands_in_the_threads_own_groups(shape, kind):
    rows, cols = shape
    bpm = oneshot_bpm(rows, cols) if kind == "oneshot" else stream_bpm(rows, cols)
    owner, bad = replay(rows, cols, bpm)
    assert not bad, bad[:5]
    assert len(owner) == rows * (cols // 4)
    assert set(owner) == {(r, q) for r in range(rows) for q in range(cols // 4)}


def test_planted_mistake_is_caught():
    # the reuse rule that mixes slot 0's row with slot 1's column writes
    # groups of other threads on odd row counts with many columns
    for rows, cols in ((129, 2052), (1001, 1200)):
        _, bad = replay(rows, cols, oneshot_bpm(rows, cols), planted=True)
        assert any(b[0] == "foreign store" for b in bad), (rows, cols)
