"""CPU oracle of the KV-selection hot path (SnapKV, H2O, StreamingLLM).

TEST INFRASTRUCTURE ONLY. Plain, slow float64 numpy written from the three
summary pages; it checks the GPU library and is never called by it. Only the
tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import it. It shares no code with the GPU path; the seeded input generators in
``synthetic`` are the only common module.

Parity unpinned (no external fixture can fix them; they are conventions of
this oracle, pinned only by self-consistency and the invariants in the tests):
the 1/sqrt(D) score scale, the tie rules, the pooling edges and the H2O
prompt-score initialisation.
"""
from . import snapkv, h2o, sink, attention

__all__ = ["snapkv", "h2o", "sink", "attention"]
