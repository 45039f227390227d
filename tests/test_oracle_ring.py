"""Pins for the oracle's ring model (CPU only): brute force against a deque of frame
ids, for random roll sequences, plus the error cases."""
from collections import deque

import numpy as np
import pytest

from oracle.ring import RingError, RingModel


class DequeWindow:
    """Independent model: the window is a deque of the newest W distinct frame ids."""

    def __init__(self, W):
        self.W = W
        self.frames = deque(maxlen=W)
        self.written = {}  # frame -> write serial

    def roll(self, t0, n, serial):
        for t in range(t0, t0 + n):
            if t not in self.frames:
                self.frames.append(t)  # maxlen drops the oldest
            self.written[t] = serial


@pytest.mark.parametrize("W", [1, 2, 5, 21])
def test_random_roll_sequences_match_deque(W):
    rng = np.random.default_rng(W)
    for seq in range(2500 if W != 21 else 500):
        ring = RingModel(W)
        dq = DequeWindow(W)
        start = int(rng.integers(0, 50))
        serial = 0
        for _ in range(int(rng.integers(1, 12))):
            if ring.count == 0:
                t0 = start
            else:
                t0 = int(rng.integers(ring.first, ring.first + ring.count + 1))
            n = int(rng.integers(1, W + 1))
            ring.roll(t0, n, [serial] * n)
            dq.roll(t0, n, serial)
            serial += 1
            assert ring.window() == list(dq.frames)
            # every window frame sits in slot t % W with the latest data written for it
            for t in dq.frames:
                s = t % W
                assert ring.slot_frame[s] == t
                assert ring.slot_data[s] == dq.written[t]


def test_eviction_is_oldest_and_only_on_full_append():
    r = RingModel(3)
    assert r.roll(0, 3) == []
    assert (r.first, r.count) == (0, 3)
    assert r.roll(3, 1) == [0]
    assert (r.first, r.count) == (1, 3)
    assert r.roll(2, 3) == [1]  # frames 2,3 in place, 4 appended -> evicts 1
    assert r.window() == [2, 3, 4]


def test_untouched_slots_keep_contents():
    r = RingModel(5)
    r.roll(0, 5, list("abcde"))
    r.roll(5, 1, ["f"])
    assert r.slot_data == ["f", "b", "c", "d", "e"]


@pytest.mark.parametrize("t0,n", [(-1, 1), (6, 1), (2, 0), (2, 6)])
def test_invalid_rolls_rejected_without_change(t0, n):
    r = RingModel(5)
    r.roll(0, 5)
    with pytest.raises(RingError):
        r.roll(t0, n)
    assert (r.first, r.count) == (0, 5)


def test_empty_ring_starts_anywhere():
    r = RingModel(4)
    r.roll(1000, 2)
    assert r.window() == [1000, 1001]
    assert r.contains(1000, 2) and not r.contains(999, 2) and not r.contains(1001, 2)
