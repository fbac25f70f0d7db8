"""Pins of the SnapKV oracle against things other than itself.

Each test fixes the oracle to an external fact: a hand-worked example with exact
fractions (tests/golden/snapkv_worked.txt), a closed form, a library routine it
does not call (torch CPU softmax / attention / max_pool1d), brute force over all
subsets, or an invariant the method guarantees. Together they catch a dropped
term, a wrong sign, an off-by-one in the causal boundary, a transposed operand,
a wrong scale, mean-instead-of-sum voting, the wrong pooling width, and the
wrong tie or output order.
"""
import itertools

import numpy as np
import pytest

from oracle import snapkv as ref
from tests import golden_io as gio

torch = pytest.importorskip("torch")


def _worked():
    g = gio.load("snapkv_worked.txt")
    D, L, w = int(g["D"][0]), int(g["L"][0]), int(g["window"][0])
    a, b = np.array(gio.nums(g["a"])), np.array(gio.nums(g["b"]))
    q = np.zeros((w, D))
    q[0, 0] = 2.0
    q[1, 1] = 2.0
    k = np.zeros((L, D))
    k[:, 0] = np.log(a)
    k[:, 1] = np.log(b)
    v = np.arange(L * D, dtype=np.float64).reshape(L, D)
    return g, q, k, v


def test_worked_example_softmax_and_stats():
    g, q, k, v = _worked()
    S = ref.window_scores(q, k)
    P, m, l = ref.row_softmax(S)
    np.testing.assert_allclose(P[0], gio.nums(g["P0"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(P[1], gio.nums(g["P1"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(m, gio.nums(g["m"]), rtol=1e-14)
    np.testing.assert_allclose(l, gio.nums(g["l"]), rtol=1e-14)


def test_worked_example_vote_pool_topk():
    g, q, k, v = _worked()
    t0 = k.shape[0] - q.shape[0]
    P, _, _ = ref.row_softmax(ref.window_scores(q, k))
    vt = ref.vote(P, t0)
    np.testing.assert_allclose(vt, gio.nums(g["vote"]), atol=1e-14)
    for p in (1, 3, 5):
        np.testing.assert_allclose(ref.max_pool(vt, p), gio.nums(g[f"pooled_p{p}"]), atol=1e-14)
    for key, toks in g.items():
        if not key.startswith("idx_"):
            continue
        _, pk, bk = key.split("_")
        p, budget = int(pk[1:]), int(bk[1:])
        out = ref.compress_head(q, k, v, budget, p, "fp64")
        assert out["idx"].tolist() == gio.ints(toks), key


def _rand_head(seed, w, L, D, scale=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((w, D)) * scale, rng.standard_normal((L, D)) * scale,
            rng.standard_normal((L, D)))


@pytest.mark.parametrize("w,L,D", [(1, 9, 4), (4, 20, 8), (16, 100, 64), (32, 300, 128)])
def test_softmax_matches_torch_attention(w, L, D):
    """The oracle's weights, applied to V, equal torch's scaled-dot-product attention
    with the same causal-in-window mask (library routine; default scale 1/sqrt(D))."""
    q, k, v = _rand_head(w * 1000 + L, w, L, D, scale=1.5)
    P, _, _ = ref.row_softmax(ref.window_scores(q, k))
    t0 = L - w
    mask = torch.zeros(w, L, dtype=torch.bool)
    for i in range(w):
        mask[i, : t0 + i + 1] = True
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=mask[None])[0].numpy()
    np.testing.assert_allclose(P @ v, out, rtol=1e-10, atol=1e-12)
    ts = torch.softmax(torch.from_numpy(q @ k.T / np.sqrt(D)).masked_fill(~mask, -np.inf), dim=1)
    np.testing.assert_allclose(P, ts.numpy(), rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("w,L", [(1, 5), (3, 10), (16, 512), (32, 2000)])
def test_zero_queries_closed_form(w, L):
    """Q = 0: every visible weight of row i equals 1/(t0+i+1); every prefix vote is
    sum_i 1/(t0+i+1); with all pooled scores tied, the lowest positions are kept."""
    D = 8
    t0 = L - w
    q = np.zeros((w, D))
    k = np.random.default_rng(1).standard_normal((L, D))
    P, _, _ = ref.row_softmax(ref.window_scores(q, k))
    for i in range(w):
        np.testing.assert_allclose(P[i, : t0 + i + 1], 1.0 / (t0 + i + 1), rtol=1e-13)
        assert np.all(P[i, t0 + i + 1:] == 0)
    expect = sum(1.0 / (t0 + i + 1) for i in range(w))
    np.testing.assert_allclose(ref.vote(P, t0), expect, rtol=1e-13)
    budget = min(L - 1, w + max(1, t0 // 3))
    out = ref.compress_head(q, k, k, budget, 3, "fp64")
    assert out["idx"].tolist() == list(range(budget - w))


def test_rows_sum_to_one_and_votes_total_window():
    w, L, D = 8, 200, 16
    q, k, v = _rand_head(7, w, L, D, scale=2.0)
    P, _, _ = ref.row_softmax(ref.window_scores(q, k))
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=1e-13)
    t0 = L - w
    vt = ref.vote(P, t0)
    assert np.all(vt >= 0) and vt.sum() <= w + 1e-12
    # prefix votes plus the window columns' weights account for every row exactly once
    np.testing.assert_allclose(vt.sum() + P[:, t0:].sum(), w, rtol=1e-13)


@pytest.mark.parametrize("p", [1, 3, 5, 7, 9])
def test_max_pool_matches_torch(p):
    v = np.random.default_rng(p).random(301)
    got = ref.max_pool(v, p)
    want = torch.nn.functional.max_pool1d(torch.from_numpy(v)[None, None], p, stride=1,
                                          padding=p // 2)[0, 0].numpy()
    np.testing.assert_array_equal(got, want)
    assert np.all(got >= v)
    if p == 1:
        np.testing.assert_array_equal(got, v)


def _brute_topk(pooled, n_keep):
    """Best subset by brute force: largest total score, then the lexicographically
    smallest ascending position list."""
    best, best_key = None, None
    for sub in itertools.combinations(range(len(pooled)), n_keep):
        key = (-sum(pooled[list(sub)]), sub)
        if best_key is None or key < best_key:
            best, best_key = sub, key
    return list(best)


@pytest.mark.parametrize("seed", range(12))
def test_topk_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(4, 13))
    n_keep = int(rng.integers(1, n))
    # few distinct values so ties at the boundary are common
    pooled = rng.integers(0, 4, size=n).astype(np.float64) / 4
    assert ref.top_positions(pooled, n_keep).tolist() == _brute_topk(pooled, n_keep)


def test_topk_matches_stable_sort():
    rng = np.random.default_rng(3)
    pooled = np.round(rng.random(5000), 2)
    n_keep = 777
    order = np.argsort(-pooled, kind="stable")  # library stable sort: equal keys keep index order
    assert ref.top_positions(pooled, n_keep).tolist() == sorted(order[:n_keep].tolist())


@pytest.mark.parametrize("p", [1, 3, 7])
def test_planted_spike_keeps_neighbourhood(p):
    """One dominant key at j*: its whole pooling neighbourhood is kept when the
    budget has room for it (pooling keeps a phrase together)."""
    w, L, D = 4, 400, 32
    q, k, v = _rand_head(11, w, L, D)
    u = q.mean(axis=0)
    j = 123
    k[j] += 40.0 * u / np.linalg.norm(u)
    out = ref.compress_head(q, k, v, budget=w + p, pool_kernel=p, dtype="fp64")
    assert out["idx"].tolist() == list(range(j - p // 2, j + p // 2 + 1))


def test_gather_is_a_bit_copy_in_order():
    w, L, D = 8, 300, 64
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2 ** 16, size=(L, D), dtype=np.uint16)
    bits &= np.uint16(0x7F7F)  # finite bf16 values
    q = rng.integers(0, 2 ** 16, size=(w, D), dtype=np.uint16) & np.uint16(0x3F7F)
    out = ref.compress_head(q, bits, bits[::-1].copy(), budget=40, pool_kernel=5, dtype="bf16")
    idx, t0 = out["idx"], L - w
    assert len(idx) == 32 and np.all(np.diff(idx) > 0) and idx.max() < t0
    np.testing.assert_array_equal(out["k_out"][:32], bits[idx])
    np.testing.assert_array_equal(out["k_out"][32:], bits[t0:])
    np.testing.assert_array_equal(out["v_out"][32:], bits[::-1][t0:])


def test_heads_are_independent():
    """Permuting heads permutes the outputs (each head selects on its own)."""
    B, H, w, L, D = 1, 3, 4, 64, 8
    rng = np.random.default_rng(9)
    q = rng.standard_normal((B, H, w, D))
    k = rng.standard_normal((B, H, L, D))
    v = rng.standard_normal((B, H, L, D))
    a = ref.compress(q, k, v, w, 20, 3, "fp64")
    perm = [2, 0, 1]
    b = ref.compress(q[:, perm], k[:, perm], v[:, perm], w, 20, 3, "fp64")
    for new_h, old_h in enumerate(perm):
        assert a[(0, old_h)]["idx"].tolist() == b[(0, new_h)]["idx"].tolist()


def test_rejects_bad_arguments():
    q, k, v = _rand_head(0, 4, 20, 8)
    with pytest.raises(ValueError):
        ref.compress_head(q, k, v, budget=4, pool_kernel=3, dtype="fp64")   # budget <= window
    with pytest.raises(ValueError):
        ref.compress_head(q, k, v, budget=20, pool_kernel=3, dtype="fp64")  # budget >= L
    with pytest.raises(ValueError):
        ref.compress_head(q, k, v, budget=10, pool_kernel=4, dtype="fp64")  # even kernel


def test_worked_example_average_pooling():
    """Hand-worked means over in-range neighbours (tests/golden/snapkv_worked.txt) and the kept sets
    they give."""
    g, q, k, v = _worked()
    t0 = k.shape[0] - q.shape[0]
    vt = ref.vote(ref.row_softmax(ref.window_scores(q, k))[0], t0)
    for p in (1, 3, 5):
        np.testing.assert_allclose(ref.avg_pool(vt, p), gio.nums(g[f"pooled_avg_p{p}"]), atol=1e-14)
    n = 0
    for key, toks in g.items():
        if key.startswith("idxavg_"):
            _, pk, bk = key.split("_")
            out = ref.compress_head(q, k, v, int(bk[1:]), int(pk[1:]), "fp64", pool_type="avg")
            assert out["idx"].tolist() == gio.ints(toks), key
            n += 1
    assert n == 8


@pytest.mark.parametrize("p", [1, 3, 5, 7, 9, 17, 65])
def test_avg_pool_matches_torch(p):
    """Same as torch's avg_pool1d with zero padding left out of the count (count_include_pad=False)."""
    rng = np.random.default_rng(p)
    for n in (1, 2, p // 2, p, 3 * p + 1, 200):
        if n < 1:
            continue
        v = rng.random(n)
        want = torch.nn.functional.avg_pool1d(torch.from_numpy(v)[None, None], kernel_size=p, stride=1,
                                              padding=p // 2, count_include_pad=False)[0, 0].numpy()
        if p // 2 > 0 and n < p // 2:  # torch needs at least one in-range value per window, as we do
            continue
        np.testing.assert_allclose(ref.avg_pool(v, p), want, rtol=1e-12, atol=0)


def test_avg_pool_closed_forms():
    rng = np.random.default_rng(0)
    v = rng.random(50)
    np.testing.assert_array_equal(ref.avg_pool(v, 1), v)                     # width 1: identity
    np.testing.assert_allclose(ref.avg_pool(np.full(30, 0.3), 7), 0.3)        # constant stays constant
    spike = np.zeros(40)
    spike[20] = 7.0                                                           # interior spike: 7 / p around it
    np.testing.assert_allclose(ref.avg_pool(spike, 5)[18:23], 7.0 / 5)
    assert np.all(ref.avg_pool(spike, 5)[:18] == 0) and np.all(ref.avg_pool(spike, 5)[23:] == 0)
    edge = np.zeros(40)
    edge[0] = 6.0                                                             # edge spike: fewer neighbours
    np.testing.assert_allclose(ref.avg_pool(edge, 5)[:3], [6.0 / 3, 6.0 / 4, 6.0 / 5])
    assert ref.avg_pool(v, 5).sum() <= v.sum() * 1.0000001 * 5 / 3            # a mean never exceeds the max
    assert np.all(ref.avg_pool(v, 9) <= ref.max_pool(v, 9) + 1e-15)


def test_zero_queries_average_pooling_ties():
    """Q = 0 gives equal votes, so the averages are equal too (up to rounding of equal sums) and the
    kept set is decided by the positions: with exactly equal votes every mean is the same value."""
    w, L, D, budget = 4, 60, 8, 20
    rng = np.random.default_rng(1)
    k = rng.standard_normal((L, D))
    out = ref.compress_head(np.zeros((w, D)), k, k, budget, 5, "fp64", pool_type="avg")
    np.testing.assert_allclose(out["pooled"], out["vote"][0], rtol=1e-14)


def test_ragged_lengths_ignore_padding():
    """A ragged batch: sequence b sees only its first lengths[b] keys; whatever lies in the padding
    beyond does not change its result, and the result is that of the truncated prompt."""
    B, H, L, D, w, budget = 3, 2, 90, 16, 4, 20
    rng = np.random.default_rng(7)
    q = rng.standard_normal((B, H, w, D))
    k = rng.standard_normal((B, H, L, D))
    v = rng.standard_normal((B, H, L, D))
    lengths = [90, 41, 64]
    a = ref.compress(q, k, v, w, budget, 5, "fp64", lengths=lengths)
    k2, v2 = k.copy(), v.copy()
    for b, n in enumerate(lengths):
        k2[b, :, n:] = 50.0 * rng.standard_normal((H, L - n, D))  # loud padding
        v2[b, :, n:] = -9.0
    c = ref.compress(q, k2, v2, w, budget, 5, "fp64", lengths=lengths)
    for b, n in enumerate(lengths):
        for h in range(H):
            assert a[(b, h)]["idx"].tolist() == c[(b, h)]["idx"].tolist()
            np.testing.assert_array_equal(a[(b, h)]["vote"], c[(b, h)]["vote"])
            assert a[(b, h)]["vote"].shape == (n - w,)
            np.testing.assert_array_equal(a[(b, h)]["k_out"][-w:], k[b, h, n - w:n])  # its own window
            t = ref.compress_head(q[b, h], k[b, h, :n], v[b, h, :n], budget, 5, "fp64")
            assert t["idx"].tolist() == a[(b, h)]["idx"].tolist()


def test_layers_are_independent():
    """compress_layers runs every layer on its own: permuting the layers permutes the results."""
    NL, B, H, L, D, w, budget = 3, 2, 2, 70, 8, 4, 16
    rng = np.random.default_rng(9)
    q = rng.standard_normal((NL, B, H, w, D))
    k = rng.standard_normal((NL, B, H, L, D))
    v = rng.standard_normal((NL, B, H, L, D))
    out = ref.compress_layers(q, k, v, w, budget, 3, "fp64", pool_type="avg")
    perm = [2, 0, 1]
    outp = ref.compress_layers(q[perm], k[perm], v[perm], w, budget, 3, "fp64", pool_type="avg")
    for i, l in enumerate(perm):
        for bh in out[l]:
            assert out[l][bh]["idx"].tolist() == outp[i][bh]["idx"].tolist()
            np.testing.assert_array_equal(out[l][bh]["pooled"], outp[i][bh]["pooled"])
