"""CPU oracle for SnapKV prompt-KV selection and compaction (one attention layer).

TEST INFRASTRUCTURE. Only the tests, the smoke check in ``__graft_entry__`` and
the CPU-baseline leg of ``bench.py`` may import this module. The GPU library
never calls it, and this module shares no code with the GPU path.

Source: the abeam.tech summary of "SnapKV: LLM Knows What You are Looking for
Before Generation" (the SnapKV page), section 技術の仕組み (how it works),
subsection 処理の流れ (processing flow), steps 1-4, and the glossary entries
for Observation Window, Prefix and Pooling. Every step below works on one
(batch, head) pair at a time, in float64, with plain numpy.

Readings adopted where the page is silent (each is listed in the design notes):
  * scores are the layer's scaled dot product q.k / sqrt(D);
  * each window query's softmax runs over every key it can see: the whole
    prefix plus the window keys up to its own position (causal inside the
    window); only prefix columns are voted on;
  * the vote of a prefix position is the plain sum over the window queries;
  * the pooling is a max-pool of odd width p, stride 1, over the prefix vote
    vector only, with out-of-range neighbours ignored; the averaging variant
    takes the mean of the same in-range neighbours;
  * the budget counts the window, so budget - window prefix positions are kept;
    equal pooled scores are broken toward the lower position; kept positions
    come out in ascending order, followed by the window.
"""
import numpy as np


def window_scores(q_win, k):
    """Scaled scores of the window queries against every prompt key, causal inside the window.

    Processing flow step 1: the last ``w`` prompt queries look at the prompt keys,
    head by head. Query ``i`` of the window sits at absolute position ``t0 + i``
    (``t0 = L - w``) and sees keys ``0 .. t0 + i``; invisible entries are -inf.

    q_win: [w, D] float64; k: [L, D] float64. Returns S [w, L].
    """
    w, D = q_win.shape
    L = k.shape[0]
    t0 = L - w
    S = (q_win @ k.T) / np.sqrt(D)
    for i in range(w):
        S[i, t0 + i + 1:] = -np.inf
    return S


def row_softmax(S):
    """Softmax of every row over its visible entries.

    Returns (P, m, l) with m the row maximum and l the sum of exp(S - m), so
    that P = exp(S - m) / l.
    """
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    return E / l, m[:, 0], l[:, 0]


def vote(P, t0):
    """Processing flow step 2 (voting): add up, for each prefix position, the
    attention weights it receives from all window queries of this head."""
    return P[:, :t0].sum(axis=0)


def max_pool(v, p):
    """Processing flow step 3 (pooling): 1D max-pool of odd width p, stride 1.

    pooled[j] = max(v[j + d]) over |d| <= p // 2 with 0 <= j + d < len(v).
    A high-vote position lifts its neighbours, so a phrase is kept whole.
    """
    r = p // 2
    # Out-of-range neighbours are ignored: pad with -inf, which never wins a max.
    padded = np.concatenate([np.full(r, -np.inf), v, np.full(r, -np.inf)])
    return np.lib.stride_tricks.sliding_window_view(padded, p).max(axis=1)


def avg_pool(v, p):
    """Processing flow step 3 with an averaging 1D pooling of odd width p, stride 1.

    pooled[j] = mean(v[j + d]) over |d| <= p // 2 with 0 <= j + d < len(v): the
    out-of-range neighbours are ignored (not counted), as for the max-pool, so a
    window at either end averages fewer votes.
    """
    r = p // 2
    # Out-of-range neighbours are ignored: pad with NaN and take the mean of the rest.
    padded = np.concatenate([np.full(r, np.nan), v, np.full(r, np.nan)])
    return np.nanmean(np.lib.stride_tricks.sliding_window_view(padded, p), axis=1)


POOLS = {"max": max_pool, "avg": avg_pool}


def top_positions(pooled, n_keep):
    """Choose the ``n_keep`` prefix positions with the largest pooled score.

    Ties go to the lower position. The result is returned in ascending order.
    """
    n = pooled.shape[0]
    order = np.lexsort((np.arange(n), -pooled))  # pooled descending, then position ascending
    return np.sort(order[:n_keep])


def gather_concat(x, idx, t0):
    """Processing flow step 4: selected prefix rows followed by the window rows.

    Works on raw element arrays (float32 or bfloat16 bit patterns); it is a copy.
    """
    return np.concatenate([x[idx], x[t0:]], axis=0)


def to_f64(x, dtype):
    """Exact widening of the stored input values (float64, float32, or uint16 bfloat16 bits)."""
    if dtype == "fp64":
        return np.asarray(x, dtype=np.float64)
    if dtype == "bf16":
        return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
            np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def compress_head(q_win, k, v, budget, pool_kernel, dtype, pool_type="max"):
    """SnapKV compression of one head.

    q_win: [w, D] window queries; k, v: [L, D]; values stored as ``dtype``;
    ``pool_type`` "max" (max_pool) or "avg" (avg_pool).
    Returns a dict with scores-derived intermediates and the compacted cache:
      P [w, L], m [w], l [w]   softmax of the window rows (natural-exp domain)
      vote [t0], pooled [t0]   float64
      idx [budget - w]         kept prefix positions, ascending (int64)
      k_out, v_out [budget, D] raw copies in the input's storage type
    """
    w = q_win.shape[0]
    L = k.shape[0]
    t0 = L - w
    if not (1 <= w < budget < L):
        raise ValueError("need 1 <= window < budget < L")
    if pool_kernel < 1 or pool_kernel % 2 == 0:
        raise ValueError("pool_kernel must be odd and >= 1")
    S = window_scores(to_f64(q_win, dtype), to_f64(k, dtype))
    P, m, l = row_softmax(S)
    vt = vote(P, t0)
    pooled = POOLS[pool_type](vt, pool_kernel)
    idx = top_positions(pooled, budget - w)
    return dict(P=P, m=m, l=l, vote=vt, pooled=pooled, idx=idx,
                k_out=gather_concat(k, idx, t0), v_out=gather_concat(v, idx, t0))


def compress(q, k, v, window, budget, pool_kernel, dtype, heads=None, pool_type="max", lengths=None):
    """SnapKV compression of a whole layer; every (batch, head) is independent.

    q: [B, H, q_len, D] (its last ``window`` rows are the observation window);
    k, v: [B, H, L, D]. ``heads`` optionally restricts the work to a list of
    (b, h) pairs. ``lengths`` (optional, [B]) makes the batch ragged: sequence
    b is the prompt k[b, :, :lengths[b]], v[b, :, :lengths[b]], and its window
    queries are still q's last ``window`` rows. Returns {(b, h): compress_head(...)}.
    """
    B, H, L = k.shape[:3]
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    out = {}
    for b, h in pairs:
        Lb = L if lengths is None else int(lengths[b])
        qw = q[b, h, q.shape[2] - window:]
        out[(b, h)] = compress_head(qw, k[b, h, :Lb], v[b, h, :Lb], budget, pool_kernel, dtype, pool_type)
    return out


def compress_layers(q, k, v, window, budget, pool_kernel, dtype, pool_type="max", lengths=None):
    """All layers of one prompt: q [n_layers, B, H, q_len, D], k and v [n_layers, B, H, L, D]; each layer
    is compressed on its own (the method runs once per attention layer). Returns a list of compress(...)."""
    return [compress(q[l], k[l], v[l], window, budget, pool_kernel, dtype, pool_type=pool_type, lengths=lengths)
            for l in range(k.shape[0])]
