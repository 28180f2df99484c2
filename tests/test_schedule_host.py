"""Host logic: the attention-schedule property check used by the GPU tests.

A plain Python construction of the documented schedule (each XCD owns the
rows whose work midpoint falls in its eighth, longest first; surplus rows,
shortest first from the owner's view, fill other XCDs' spare positions) must
pass ``check_schedule``; schedules that break one property must not.
"""
import numpy as np
import pytest

from parity_util import XCDS, check_schedule


def build_schedule(lens):
    lens = np.asarray(lens, dtype=np.int64)
    n = lens.size
    rp = np.concatenate([[0], np.cumsum(lens)])
    owner = np.minimum((2 * rp[:-1] + lens) * XCDS // (2 * rp[-1]), XCDS - 1)
    P = np.argsort(-lens, kind="stable")
    cap = [n // XCDS + (1 if x < n % XCDS else 0) for x in range(XCDS)]
    slots = [[] for _ in range(XCDS)]
    surplus = []
    for r in P:
        x = owner[r]
        (slots[x] if len(slots[x]) < cap[x] else surplus).append(int(r))
    for x in range(XCDS):
        while len(slots[x]) < cap[x]:
            slots[x].append(surplus.pop(0))
    order = np.empty(n, dtype=np.int64)
    for x in range(XCDS):
        order[x::XCDS] = slots[x]
    return order, rp


def _lens(seed, H=8, nb=37):
    rng = np.random.default_rng(seed)
    k = rng.choice([1, 2, 5, nb], size=H)
    I = np.arange(nb)
    return (np.minimum(k[:, None], I[None, :] + 1) + (rng.random((H, nb)) < 0.3)).reshape(-1)


@pytest.mark.parametrize("seed", range(5))
def test_documented_schedule_passes(seed):
    order, rp = build_schedule(_lens(seed))
    check_schedule(order, rp)


def test_small_and_ragged_counts():
    for n in (1, 3, 8, 9, 15):
        order, rp = build_schedule(np.arange(1, n + 1)[::-1])
        check_schedule(order, rp)


def test_violations_are_caught():
    order, rp = build_schedule(_lens(7))
    bad = order.copy()
    bad[[0, 1]] = bad[[1, 0]]                 # two rows trade XCDs
    with pytest.raises(AssertionError):
        check_schedule(bad, rp)
    bad = order.copy()
    bad[[0, 8]] = bad[[8, 0]]                 # same XCD, shorter row first
    lens = np.diff(rp)
    if lens[bad[0]] != lens[bad[8]]:
        with pytest.raises(AssertionError):
            check_schedule(bad, rp)
    bad = order.copy()
    bad[-1] = bad[0]                          # not a permutation
    with pytest.raises(AssertionError):
        check_schedule(bad, rp)
    lens_order = np.argsort(-np.diff(rp), kind="stable")   # the old longest-first order
    with pytest.raises(AssertionError):
        check_schedule(lens_order, rp)
