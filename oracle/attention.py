"""CPU oracle for decode-time attention over a compacted or windowed KV cache.

TEST INFRASTRUCTURE. Only the tests, the smoke check in ``__graft_entry__`` and
the CPU-baseline leg of ``bench.py`` may import this module. The GPU library
never calls it, and this module shares no code with the GPU path.

Sources:
  * the SnapKV page, section 技術の仕組み (how it works), processing flow
    step 4: once the cache is compressed, every later generation step attends
    over the compressed cache only (kept prefix rows followed by the window);
  * the StreamingLLM page, section 推論の流れ (inference flow): the attention of
    each next token is computed over the sink tokens and the recent tokens only.

The attention itself is the scaled dot-product softmax with the same 1/sqrt(D)
reading as the SnapKV scores: o = sum_j softmax_j(q.k_j / sqrt(D)) v_j over the
cached rows. No positional re-encoding happens inside the cache (the pages are
silent on it), so the result does not depend on the order of the rows.
Float64 throughout.
"""
import numpy as np

from .snapkv import to_f64


def scores(q, k):
    """q [D], k [n, D] (float64): q.k_j / sqrt(D) for every cached row."""
    return (k @ q) / np.sqrt(q.shape[-1])


def softmax(s):
    """Softmax of a score vector (shifted by its max; the result is unchanged)."""
    e = np.exp(s - s.max())
    return e / e.sum()


def decode_head(q, k, v, dtype):
    """Attention output of one query over one head's cached rows.

    q: [D]; k, v: [n, D], n >= 1; values stored as ``dtype`` (bf16 bits, fp32 or fp64).
    Returns o [D] float64.
    """
    qf, kf, vf = to_f64(q, dtype), to_f64(k, dtype), to_f64(v, dtype)
    return softmax(scores(qf, kf)) @ vf


def decode(q, k, v, n, dtype):
    """Every (b, h): q [B,H,D], k/v [B,H,>=n,D]; attention over rows 0..n-1. Returns [B,H,D]."""
    B, H, D = q.shape
    out = np.empty((B, H, D), np.float64)
    for b in range(B):
        for h in range(H):
            out[b, h] = decode_head(q[b, h], k[b, h, :n], v[b, h, :n], dtype)
    return out
