"""Pins of the H2O oracle: hand-worked example, closed forms, conservation, torch softmax."""
import numpy as np
import pytest

from oracle import h2o as ref
from tests import golden_io as gio

torch = pytest.importorskip("torch")


def _empty(D, dtype=np.float64):
    return ref.HeadState(np.zeros(0, np.int64), np.zeros(0), np.zeros((0, D), dtype),
                         np.zeros((0, D), dtype))


def _parse_state(toks):
    pos, acc = [], []
    for t in toks:
        p, a = t.split(":")
        pos.append(int(p))
        acc.append(gio.num(a))
    return pos, acc


def test_worked_example():
    g = gio.load("h2o_worked.txt")
    D = int(g["D"][0])
    a = gio.nums(g["a"])
    hh, r = int(g["n_heavy"][0]), int(g["n_recent"][0])
    q = np.array([2.0, 0, 0, 0])
    st = _empty(D)
    for t in range(1, len(a) + 1):
        k_new = np.array([np.log(a[t - 1]), 0, 0, 0])
        v_new = np.array([t - 1, 1.0, 0, 0])
        st, p, o = ref.step_head(st, q, k_new, v_new, t, hh, r, "fp64")
        pos, acc = _parse_state(g[f"state_{t}"])
        order = np.argsort(st.pos)
        assert st.pos[order].tolist() == pos
        np.testing.assert_allclose(st.acc[order], acc, rtol=1e-13)
    np.testing.assert_allclose(o, gio.nums(g["o_5"]), atol=1e-13)


def test_worked_evicted_scores_and_conservation():
    g = gio.load("h2o_worked.txt")
    a = gio.nums(g["a"])
    q = np.array([2.0, 0, 0, 0])
    st = _empty(4)
    evicted = {}
    for t in range(1, len(a) + 1):
        k_new = np.array([np.log(a[t - 1]), 0, 0, 0])
        pre_pos = np.append(st.pos, t - 1)
        st2, p, _ = ref.step_head(st, q, k_new, np.zeros(4), t, 1, 1, "fp64")
        acc_full = np.append(st.acc, 0.0) + p
        for j, x in zip(pre_pos, acc_full):
            if j not in st2.pos:
                evicted[int(j)] = (x, t)
        st = st2
    for tok in g["evicted"]:
        pa, rest = tok.split(":")
        val, at = rest.rstrip("]").split("[")
        got_val, got_at = evicted[int(pa)]
        assert got_at == int(at)
        np.testing.assert_allclose(got_val, gio.num(val), rtol=1e-13)
    # every attention row sums to one: all score ever handed out equals the step count
    total = st.acc.sum() + sum(x for x, _ in evicted.values())
    np.testing.assert_allclose(total, len(a), rtol=1e-13)


def test_tie_rule_on_hand_scores():
    g = gio.load("h2o_worked.txt")
    acc = np.array(gio.nums(g["tie_acc"]))
    pos = np.arange(4)
    for key, hh, r in (("tie_keep_h1_r1", 1, 1), ("tie_keep_h2_r1", 2, 1), ("tie_keep_h1_r2", 1, 2)):
        keep = ref.evict(pos, acc, 4, hh, r)
        assert np.flatnonzero(keep).tolist() == gio.ints(g[key]), key


def _run(seed, steps, D, hh_fn, r_fn, scale=1.0):
    rng = np.random.default_rng(seed)
    st = _empty(D)
    hist = []
    Q, Kx = [], []
    for t in range(1, steps + 1):
        q = rng.standard_normal(D) * scale
        k = rng.standard_normal(D) * scale
        v = rng.standard_normal(D)
        Q.append(q)
        Kx.append(k)
        pre = st
        st, p, o = ref.step_head(st, q, k, v, t, hh_fn(t), r_fn(t), "fp64")
        hist.append((pre, p, st))
    return st, hist, np.array(Q), np.array(Kx)


def test_no_heavy_is_window_attention():
    """n_heavy = 0: the cache is exactly the last n_recent positions (closed form)."""
    st, hist, _, _ = _run(1, 60, 8, lambda t: 0, lambda t: 7)
    for t, (_, _, s) in enumerate(hist, start=1):
        assert sorted(s.pos.tolist()) == list(range(max(0, t - 7), t))


def test_large_budget_equals_causal_column_sums():
    """A budget that never binds: no eviction, and every token's score equals the
    column sum of the causal attention of the whole sequence (torch softmax)."""
    T, D = 50, 16
    st, hist, Q, K = _run(2, T, D, lambda t: 1000, lambda t: 1000, scale=1.3)
    assert sorted(st.pos.tolist()) == list(range(T))
    S = torch.from_numpy(Q @ K.T / np.sqrt(D))
    S = S.masked_fill(torch.triu(torch.ones(T, T, dtype=torch.bool), 1), -np.inf)
    colsum = torch.softmax(S, dim=1).sum(dim=0).numpy()
    order = np.argsort(st.pos)
    np.testing.assert_allclose(st.acc[order], colsum, rtol=1e-12)


def test_kept_count_and_recent_always_kept():
    st, hist, _, _ = _run(3, 120, 8, lambda t: t // 10, lambda t: t // 10)
    for t, (pre, p, s) in enumerate(hist, start=1):
        n_before = len(pre) + 1
        budget = 2 * (t // 10)
        assert len(s) == min(n_before, budget) if n_before > budget else len(s) == n_before
        r = t // 10
        assert set(range(t - r, t)) <= set(s.pos.tolist())
        np.testing.assert_allclose(p.sum(), 1.0, rtol=1e-13)


def test_score_is_sum_of_step_probabilities():
    """For a surviving token, its score equals the sum of the probabilities it got."""
    st, hist, _, _ = _run(4, 80, 8, lambda t: t // 5, lambda t: t // 10)
    # direct bookkeeping, step by step
    sums = {}
    for t, (pre, p, s) in enumerate(hist, start=1):
        pos_all = np.append(pre.pos, t - 1)
        for j, x in zip(pos_all, p):
            sums[int(j)] = sums.get(int(j), 0.0) + x
    for j, a in zip(st.pos, st.acc):
        np.testing.assert_allclose(a, sums[int(j)], rtol=1e-12)


def test_prefill_equals_stepping_from_empty():
    """Prompt scores (causal column sums) equal running the decode step over the prompt
    with a budget that never binds; with a binding budget, the eviction keeps the
    recent tail and the top remaining scores."""
    Lp, D = 40, 8
    rng = np.random.default_rng(6)
    q, k, v = (rng.standard_normal((Lp, D)) for _ in range(3))
    st, colsum = ref.prefill_head(q, k, v, 10 ** 6, 10 ** 6, "fp64")
    s2 = _empty(D)
    for t in range(1, Lp + 1):
        s2, _, _ = ref.step_head(s2, q[t - 1], k[t - 1], v[t - 1], t, 10 ** 6, 10 ** 6, "fp64")
    np.testing.assert_allclose(np.sort(st.pos), np.arange(Lp))
    np.testing.assert_allclose(s2.acc[np.argsort(s2.pos)], colsum, rtol=1e-12)
    st3, _ = ref.prefill_head(q, k, v, 4, 4, "fp64")
    assert set(range(Lp - 4, Lp)) <= set(st3.pos.tolist()) and len(st3) == 8
    rest = [j for j in np.argsort(-colsum, kind="stable") if j < Lp - 4][:4]
    assert set(rest) <= set(st3.pos.tolist())


def _bf16_bits_via_torch(x32):
    """bf16 bit patterns of float32 values, rounded by torch (a library the oracle does not call)."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16)


def test_widening_matches_torch_and_known_encodings():
    """The oracle's exact widening of stored inputs: bf16 bit patterns against torch's own widening and
    a few encodings fixed by the bfloat16 format (sign, 8-bit exponent, 7-bit fraction), fp32 unchanged."""
    import torch

    from oracle.snapkv import to_f64

    known = {0x3F80: 1.0, 0xC000: -2.0, 0x3F81: 1.0 + 2.0 ** -7, 0x0000: 0.0, 0x8000: -0.0,
             0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127, 0x0001: 2.0 ** -133, 0x4049: 3.140625}
    bits = np.array(list(known), np.uint16)
    got = to_f64(bits, "bf16")
    np.testing.assert_array_equal(got, np.array(list(known.values())))
    rng = np.random.default_rng(3)
    x = _bf16_bits_via_torch(rng.standard_normal(4096).astype(np.float32) * 10)
    via_torch = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(to_f64(x, "bf16"), via_torch)
    f = rng.standard_normal(100).astype(np.float32)
    np.testing.assert_array_equal(to_f64(f, "fp32"), f.astype(np.float64))
    assert to_f64(f, "fp32").dtype == np.float64


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_step_and_prefill_on_stored_types_equal_fp64_on_widened_values(dtype):
    """step_head / prefill_head on bf16 bit patterns or fp32 arrays give exactly what the fp64 run gives on
    the same values widened by torch (so the stored-type branch neither drops, shifts nor masks bits)."""
    import torch

    rng = np.random.default_rng(11 if dtype == "bf16" else 12)
    Lp, D, steps = 40, 64, 12
    x = rng.standard_normal((3, Lp + steps, D)).astype(np.float32)
    if dtype == "bf16":
        stored = _bf16_bits_via_torch(x)
        wide = torch.from_numpy(stored.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    else:
        stored = x
        wide = torch.from_numpy(x).to(torch.float64).numpy()
    q, k, v = stored
    qw, kw, vw = wide
    st_s, col_s = ref.prefill_head(q[:Lp], k[:Lp], v[:Lp], 6, 5, dtype)
    st_w, col_w = ref.prefill_head(qw[:Lp], kw[:Lp], vw[:Lp], 6, 5, "fp64")
    np.testing.assert_array_equal(col_s, col_w)
    np.testing.assert_array_equal(st_s.pos, st_w.pos)
    np.testing.assert_array_equal(st_s.acc, st_w.acc)
    for t in range(steps):
        length = Lp + t + 1
        st_s, p_s, o_s = ref.step_head(st_s, q[length - 1], k[length - 1], v[length - 1], length, 6, 5, dtype)
        st_w, p_w, o_w = ref.step_head(st_w, qw[length - 1], kw[length - 1], vw[length - 1], length, 6, 5, "fp64")
        np.testing.assert_array_equal(p_s, p_w)
        np.testing.assert_array_equal(o_s, o_w)
        np.testing.assert_array_equal(st_s.pos, st_w.pos)
        np.testing.assert_array_equal(st_s.acc, st_w.acc)
    # the kept rows are the stored rows themselves (raw bits), not widened copies
    assert st_s.k.dtype == stored.dtype
