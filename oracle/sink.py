"""CPU oracle for the StreamingLLM attention-sink + recent-window cache.

TEST INFRASTRUCTURE. Only the tests, the smoke check in ``__graft_entry__`` and
the CPU-baseline leg of ``bench.py`` may import this module. The GPU library
never calls it, and this module shares no code with the GPU path.

Source: the abeam.tech summary of "Efficient Streaming Language Models with
Attention Sinks" (the StreamingLLM page), section 技術の仕組み (how it works),
subsections キャッシュ構造 (cache structure: a few permanent sink tokens from
the start of the stream plus a recent window of fixed length) and 推論の流れ
(inference flow: each new token enters the recent region, the oldest recent
token leaves once the window is full, sink tokens never leave).

Readings adopted where the page is silent:
  * the cache stores the sinks in slots 0 .. s-1 and the recent window as a
    ring of r slots after them, so the position p >= s lives in slot
    s + (p - s) mod r;
  * the position a held token takes inside the cache (the position the model's
    positional encoding would use while streaming) is its rank among the held
    tokens in the order the inference flow keeps them: the sinks in arrival
    order, then the recent window from oldest to newest. Positions then stay
    below s + r however long the stream runs, which is what a cache of constant
    size (cache structure subsection) streaming millions of tokens (section
    実験と結果, the 4M-token result) needs; the newest token always takes the
    last position.
"""
from collections import deque


def kept_positions(length, n_sink, n_recent):
    """Absolute positions held after ``length`` tokens, ascending (closed form)."""
    sinks = list(range(min(n_sink, length)))
    recent = list(range(max(n_sink, length - n_recent), length))
    return sinks + recent


def slot_of(pos, n_sink, n_recent):
    """Cache slot of absolute position ``pos`` in the sink + ring layout."""
    if pos < n_sink:
        return pos
    return n_sink + (pos - n_sink) % n_recent


def simulate(length, n_sink, n_recent):
    """Token-by-token simulation of the inference flow (deque of recent tokens).

    The first ``n_sink`` tokens go to the sink region and stay; every later token
    joins the recent region, which drops its oldest member once it holds more
    than ``n_recent``. Returns the held positions, ascending.
    """
    sinks, recent = [], deque()
    for p in range(length):
        if len(sinks) < n_sink:
            sinks.append(p)
            continue
        recent.append(p)
        if len(recent) > n_recent:
            recent.popleft()
    return sorted(sinks + list(recent))


def ring_after(rows, n_sink, n_recent):
    """Slot contents after writing ``rows[p]`` for p = 0 .. len(rows)-1 in order.

    Returns (slot_rows, slot_pos) lists of length n_sink + n_recent; unwritten
    slots hold None and position -1.
    """
    n_slots = n_sink + n_recent
    slot_rows = [None] * n_slots
    slot_pos = [-1] * n_slots
    for p, row in enumerate(rows):
        s = slot_of(p, n_sink, n_recent)
        slot_rows[s] = row
        slot_pos[s] = p
    return slot_rows, slot_pos


def cache_positions(length, n_sink, n_recent):
    """Position inside the cache of the token each slot holds after ``length`` tokens, slot by slot
    (-1 for a slot not yet written): the token's rank in the held order, sinks first, then the recent
    tokens oldest to newest. The slots are filled by writing the tokens in order (ring_after)."""
    _, slot_pos = ring_after(list(range(length)), n_sink, n_recent)
    rank = {p: i for i, p in enumerate(kept_positions(length, n_sink, n_recent))}
    return [rank[p] if p >= 0 else -1 for p in slot_pos]
