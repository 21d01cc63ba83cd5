"""The split-KV decode's work decomposition, modelled on the CPU.

The decode's first pass cuts the global page list (the (sequence, KV head)
units in order, each with its sequence's pages) into W equal contiguous
ranges, [w T / W, (w + 1) T / W); each (work-group w, unit u) pair that
overlaps writes record w + u; the second pass finds the work-groups of unit u
as floor(((x + 1) W - 1) / T) for its first and last page x. These tests check
the arithmetic: every page is covered once, record indices are unique and
below W + U, and the second pass finds exactly the work-groups that wrote.
"""
import numpy as np
import pytest


def ranges(T, W):
    return [(w * T // W, (w + 1) * T // W) for w in range(W)]


def wg_of(x, T, W):
    return ((x + 1) * W - 1) // T


def decompose(pages, H_kv, W):
    units = [(b, g, n) for b, n in enumerate(pages) for g in range(H_kv)]
    base, starts = 0, []
    for _, _, n in units:
        starts.append(base)
        base += n
    T = base
    written = {}
    for w, (s, e) in enumerate(ranges(T, W)):
        assert e > s, "every work-group gets a page"
        for u, (_, _, n) in enumerate(units):
            lo, hi = max(s, starts[u]), min(e, starts[u] + n)
            if lo < hi:
                r = w + u
                assert r not in written, "record written twice"
                written[r] = (w, u, lo, hi)
    return units, starts, T, written


@pytest.mark.parametrize("seed", range(40))
def test_decomposition(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 9))
    H_kv = int(rng.integers(1, 5))
    pages = rng.integers(0, 40, size=B)
    pages[rng.random(B) < 0.2] = 0  # invalid lengths have no pages
    if pages.sum() == 0:
        pages[0] = 1
    T = int(pages.sum()) * H_kv
    W = int(rng.integers(1, T + 1))
    units, starts, T2, written = decompose(pages.tolist(), H_kv, W)
    assert T2 == T
    assert all(r < W + len(units) for r in written)
    covered = np.zeros(T, int)
    for w, u, lo, hi in written.values():
        covered[lo:hi] += 1
    assert np.all(covered == 1)
    for u, (_, _, n) in enumerate(units):
        if n == 0:
            continue
        w0, w1 = wg_of(starts[u], T, W), wg_of(starts[u] + n - 1, T, W)
        found = {r - u for r in range(w0 + u, w1 + u + 1)}
        wrote = {w for (w, uu, _, _) in written.values() if uu == u}
        assert found == wrote
        # the pages of the unit's records add up to the unit
        assert sum(hi - lo for (w, uu, lo, hi) in written.values() if uu == u) == n


def test_wg_of_is_the_range_owner():
    for T in range(1, 60):
        for W in range(1, T + 1):
            for w, (s, e) in enumerate(ranges(T, W)):
                for x in range(s, e):
                    assert wg_of(x, T, W) == w
