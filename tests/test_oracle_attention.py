"""Pins of the decode-attention oracle: closed forms, invariances and a direct evaluation."""
import numpy as np
import pytest

from oracle import attention as ref
import synthetic as syn


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_zero_query_is_the_mean_of_the_values():
    """q = 0: every score is 0, every weight 1/n, so o is the plain mean of V (closed form)."""
    v = _rand((37, 16), 0)
    o = ref.decode_head(np.zeros(16), _rand((37, 16), 1), v, "fp64")
    np.testing.assert_allclose(o, v.mean(0), rtol=0, atol=1e-14)


def test_single_row_returns_its_value():
    k, v = _rand((1, 8), 2), _rand((1, 8), 3)
    np.testing.assert_array_equal(ref.decode_head(_rand(8, 4), k, v, "fp64"), v[0])


def test_dominant_key_selects_its_value():
    """One key 60 logits ahead of the rest (other weights ~1e-25): o equals its value to 1e-12."""
    D = 32
    q = _rand(D, 5)
    k = _rand((50, D), 6) * 0.1
    k[17] = q / np.linalg.norm(q) * (60.0 * np.sqrt(D) / np.linalg.norm(q))
    v = _rand((50, D), 7)
    np.testing.assert_allclose(ref.decode_head(q, k, v, "fp64"), v[17], rtol=1e-12, atol=1e-12)


def test_two_equal_keys_average():
    """Two identical keys and all others far below: o is the average of their two values."""
    D = 8
    q = np.ones(D)
    k = np.full((5, D), -10.0)
    k[1] = k[3] = np.full(D, 10.0)
    v = _rand((5, D), 8)
    np.testing.assert_allclose(ref.decode_head(q, k, v, "fp64"), 0.5 * (v[1] + v[3]), rtol=1e-12, atol=1e-12)


def test_matches_direct_exponential_sum():
    """Against exp(s)/sum(exp(s)) written out with math.exp per term and no max shift."""
    import math
    D, n = 16, 23
    q, k, v = _rand(D, 9), _rand((n, D), 10), _rand((n, D), 11)
    w = [math.exp(sum(q[d] * k[j, d] for d in range(D)) / math.sqrt(D)) for j in range(n)]
    tot = math.fsum(w)
    o = [math.fsum(w[j] * v[j, d] for j in range(n)) / tot for d in range(D)]
    np.testing.assert_allclose(ref.decode_head(q, k, v, "fp64"), o, rtol=1e-12, atol=1e-14)


def test_row_order_does_not_matter():
    D, n = 16, 40
    q, k, v = _rand(D, 12), _rand((n, D), 13), _rand((n, D), 14)
    perm = np.random.default_rng(15).permutation(n)
    np.testing.assert_allclose(ref.decode_head(q, k, v, "fp64"), ref.decode_head(q, k[perm], v[perm], "fp64"),
                               rtol=1e-13, atol=1e-14)


def test_output_is_a_convex_combination():
    D, n = 8, 100
    q, k, v = _rand(D, 16) * 3, _rand((n, D), 17), _rand((n, D), 18)
    p = ref.softmax(ref.scores(q, k))
    assert abs(p.sum() - 1.0) < 1e-14 and (p > 0).all()
    o = ref.decode_head(q, k, v, "fp64")
    assert (o <= v.max(0) + 1e-12).all() and (o >= v.min(0) - 1e-12).all()


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_stored_values_are_widened_exactly(dtype):
    """bf16 bits / fp32 inputs give the same result as their exact float64 values."""
    D, n = 16, 9
    q, k, v = (_rand(s, 19 + i).astype(np.float32) for i, s in enumerate([(D,), (n, D), (n, D)]))
    if dtype == "bf16":
        q, k, v = (syn.f32_to_bf16_bits(x) for x in (q, k, v))
        wq, wk, wv = (syn.bf16_bits_to_f32(x).astype(np.float64) for x in (q, k, v))
    else:
        wq, wk, wv = (x.astype(np.float64) for x in (q, k, v))
    np.testing.assert_array_equal(ref.decode_head(q, k, v, dtype), ref.decode_head(wq, wk, wv, "fp64"))


def test_decode_loops_over_heads():
    B, H, D, n = 2, 3, 8, 5
    q, k, v = _rand((B, H, D), 20), _rand((B, H, n + 2, D), 21), _rand((B, H, n + 2, D), 22)
    out = ref.decode(q, k, v, n, "fp64")
    for b in range(B):
        for h in range(H):
            np.testing.assert_array_equal(out[b, h], ref.decode_head(q[b, h], k[b, h, :n], v[b, h, :n], "fp64"))
