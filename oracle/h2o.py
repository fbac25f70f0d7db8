"""CPU oracle for the H2O heavy-hitter + recent KV-cache policy.

TEST INFRASTRUCTURE. Only the tests, the smoke check in ``__graft_entry__`` and
the CPU-baseline leg of ``bench.py`` may import this module. The GPU library
never calls it, and this module shares no code with the GPU path.

Source: the abeam.tech summary of "H2O: Heavy-Hitter Oracle for Efficient
Generative Inference of Large Language Models" (the H2O page), section
技術の仕組み (how it works), subsections 何を残すのか (what is kept) and
処理の流れ (processing flow), plus the glossary entries for attention score,
heavy hitter and local statistics. One (batch, head) pair at a time, float64.

Readings adopted where the page is silent (each is listed in the design notes):
  * every head keeps its own token set;
  * a decode step first appends the new token (score 0), attends with the new
    query over every cached token including itself, adds each token's
    probability to its cumulative score, and only then evicts;
  * recent tokens are those at positions >= len - n_recent (len counts the new
    token); the cache budget is n_heavy + n_recent; when the cache holds more
    than that, every recent token stays and the remaining budget goes to the
    other tokens with the largest cumulative score, equal scores favouring the
    newer position;
  * before decoding, each prompt token's score is the sum of the causal
    prompt attention it received (the attention observed so far), and the same
    eviction rule cuts the prompt cache to the budget at the prompt length.
"""
import numpy as np

from .snapkv import to_f64


class HeadState:
    """Cached tokens of one head: positions, cumulative scores, raw key/value rows."""

    def __init__(self, pos, acc, k, v):
        self.pos = np.asarray(pos, dtype=np.int64)
        self.acc = np.asarray(acc, dtype=np.float64)
        self.k = np.asarray(k)
        self.v = np.asarray(v)

    def copy(self):
        return HeadState(self.pos.copy(), self.acc.copy(), self.k.copy(), self.v.copy())

    def __len__(self):
        return self.pos.shape[0]


def evict(pos, acc, length, n_heavy, n_recent):
    """Boolean keep-mask under the heavy-hitter + recent rule.

    What-is-kept subsection: recent tokens are always kept; the rest of the
    budget n_heavy + n_recent goes to the tokens with the largest cumulative
    attention (ties: newer position first). No eviction while the cache fits.
    """
    n = pos.shape[0]
    budget = n_heavy + n_recent
    keep = np.ones(n, dtype=bool)
    if n <= budget:
        return keep
    recent = pos >= length - n_recent
    cand = np.flatnonzero(~recent)
    n_fill = budget - int(recent.sum())
    order = np.lexsort((-pos[cand], -acc[cand]))  # acc descending, then pos descending
    keep[:] = recent
    keep[cand[order[:n_fill]]] = True
    return keep


def step_head(st, q, k_new, v_new, length, n_heavy, n_recent, dtype):
    """One decode step of one head (processing-flow subsection).

    ``length`` counts every token seen, the new one included, so the new token's
    position is length - 1. Returns (new_state, p, o): p are the attention
    probabilities over the pre-eviction cache (in its slot order, the new token
    last) and o = sum_j p_j v_j.
    """
    pos = np.append(st.pos, length - 1)
    acc = np.append(st.acc, 0.0)
    K = np.concatenate([st.k, np.asarray(k_new)[None]], axis=0)
    V = np.concatenate([st.v, np.asarray(v_new)[None]], axis=0)
    D = K.shape[1]
    s = to_f64(K, dtype) @ to_f64(q, dtype) / np.sqrt(D)
    e = np.exp(s - s.max())
    p = e / e.sum()
    acc = acc + p
    o = p @ to_f64(V, dtype)
    keep = evict(pos, acc, length, n_heavy, n_recent)
    return HeadState(pos[keep], acc[keep], K[keep], V[keep]), p, o


def prefill_head(q, k, v, n_heavy, n_recent, dtype):
    """Initial state of one head after the prompt.

    Score of prompt token j = sum over prompt queries i >= j of the causal
    softmax weight P[i, j]; then the eviction rule at length = prompt length.
    Returns (state, colsum) where colsum [Lp] is the score before eviction.
    """
    qf, kf = to_f64(q, dtype), to_f64(k, dtype)
    Lp, D = kf.shape
    S = qf @ kf.T / np.sqrt(D)
    S[np.triu_indices(Lp, 1)] = -np.inf
    E = np.exp(S - S.max(axis=1, keepdims=True))
    P = E / E.sum(axis=1, keepdims=True)
    colsum = P.sum(axis=0)
    pos = np.arange(Lp, dtype=np.int64)
    keep = evict(pos, colsum, Lp, n_heavy, n_recent)
    return HeadState(pos[keep], colsum[keep], np.asarray(k)[keep], np.asarray(v)[keep]), colsum
