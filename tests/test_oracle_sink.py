"""Pins of the StreamingLLM sink + recent oracle: hand-worked table and deque simulation."""
import numpy as np
import pytest

from oracle import sink as ref
from tests import golden_io as gio


def test_worked_example():
    g = gio.load("sink_worked.txt")
    s, r = int(g["n_sink"][0]), int(g["n_recent"][0])
    for t in range(1, 9):
        assert ref.kept_positions(t, s, r) == gio.ints(g[f"kept_{t}"])
    assert [ref.slot_of(p, s, r) for p in range(8)] == gio.ints(g["slots"])
    assert ref.kept_positions(2000, 4, 1020) == gio.ints(g["kept_s4_r1020_len2000"])


@pytest.mark.parametrize("s,r", [(0, 1), (0, 5), (1, 1), (4, 3), (4, 1020), (2, 7)])
def test_closed_form_matches_simulation(s, r):
    for length in list(range(0, 40)) + [1023, 1024, 1025, 3000]:
        assert ref.kept_positions(length, s, r) == ref.simulate(length, s, r)


@pytest.mark.parametrize("s,r", [(4, 6), (1, 3), (0, 4)])
def test_ring_holds_exactly_the_kept_positions(s, r):
    for length in range(1, 30):
        rows = [np.full(3, p) for p in range(length)]
        slot_rows, slot_pos = ref.ring_after(rows, s, r)
        held = sorted(p for p in slot_pos if p >= 0)
        assert held == ref.kept_positions(length, s, r)
        for sr, p in zip(slot_rows, slot_pos):
            if p >= 0:
                assert np.all(sr == p)


def test_window_attention_is_zero_sinks():
    """With no sinks the cache is a plain sliding window (the page's failing baseline)."""
    for length in range(50):
        assert ref.kept_positions(length, 0, 8) == list(range(max(0, length - 8), length))


def test_cache_positions_worked_example():
    g = gio.load("sink_worked.txt")
    s, r = int(g["n_sink"][0]), int(g["n_recent"][0])
    n = 0
    for key, toks in g.items():
        if key.startswith("cachepos_"):
            assert ref.cache_positions(int(key.split("_")[1]), s, r) == gio.ints(toks), key
            n += 1
    assert n == 7


@pytest.mark.parametrize("s,r", [(0, 1), (0, 5), (1, 1), (4, 3), (2, 7), (4, 1020)])
def test_cache_positions_follow_the_deque(s, r):
    """The same positions from the inference flow simulated as a deque: the held tokens in the
    order the deque keeps them (sinks, then recent oldest first) are numbered 0, 1, 2, ..."""
    from collections import deque

    for length in list(range(1, 40)) + [1023, 1024, 1025, 1030, 2500]:
        sinks, recent = [], deque()
        for p in range(length):
            if len(sinks) < s:
                sinks.append(p)
                continue
            recent.append(p)
            if len(recent) > r:
                recent.popleft()
        order = sinks + list(recent)
        by_pos = {p: i for i, p in enumerate(order)}
        got = ref.cache_positions(length, s, r)
        for slot, cp in enumerate(got):
            if cp < 0:
                assert slot >= length  # slots fill in order: an empty slot is one never reached
                continue
            held = order[cp]
            assert ref.slot_of(held, s, r) == slot and by_pos[held] == cp
        held_slots = sorted(c for c in got if c >= 0)
        assert held_slots == list(range(min(length, s + r)))  # a permutation of 0 .. n_held-1


def test_cache_positions_closed_forms():
    for length in range(1, 30):
        cp = ref.cache_positions(length, 4, 6)
        if length <= 10:  # nothing evicted yet: inside the cache a token keeps its own position
            assert cp[:length] == list(range(length))
        assert cp[:min(length, 4)] == list(range(min(length, 4)))  # sinks keep theirs for good
        newest = ref.slot_of(length - 1, 4, 6)
        assert cp[newest] == min(length, 10) - 1  # the newest token takes the last position
