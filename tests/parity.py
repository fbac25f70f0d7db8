"""Parity criteria between the GPU library and the CPU oracle.

Selection (SnapKV top-k, H2O eviction) is decided by floating-point scores that
the GPU computes in float32 and the oracle in float64. Following the
acceptance rule for this path:
  * where the oracle's last kept and first dropped scores differ by more than
    REL (1e-3, relative), the GPU's kept set must equal the oracle's exactly;
  * otherwise (a near-tie) the GPU set must still be a valid top-k within REL:
    it keeps every score above s_k (1 + REL) and drops every score below
    s_k+1 (1 - REL), with the right count, sorted and unique;
  * gathered rows are bit-exact copies of the rows the GPU selected;
  * votes / softmax / scores within 2e-3 absolute (fp32 accumulation of bf16
    products). A tighter relative bound, 1e-4 |ref| + 1e-9, is also enforced: the
    fp32 path's error (rounded dot products, 2^x on the hardware unit, sums of up
    to a few hundred terms per lane before the merge) stays near 1e-6 relative.
"""
import numpy as np
import torch

REL = 1e-3
VOTE_ABS = 2e-3
VOTE_REL = 1e-4
VOTE_FLOOR = 1e-9
# A tighter band for the kept set, implied by the bound above: when every GPU
# pooled score is within VOTE_REL |ref| + VOTE_FLOOR of the oracle's, two
# positions whose oracle scores differ by more than ~2 VOTE_REL relative (plus
# the floor over scores near 1e-5) keep their order on the GPU, so only
# positions within REL_TIGHT of the threshold may be chosen differently.
REL_TIGHT = 3e-4


def to_device(arr, dtype):
    """numpy float32 array or uint16 bf16 bits -> contiguous GPU tensor."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.cuda()


def to_host_bits(t):
    """GPU tensor -> numpy raw element array (uint16 bits for bf16, float32 otherwise)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def assert_close_votes(got, ref, what="vote", scale=None):
    """|got - ref| <= 2e-3 and <= 1e-4 * scale + 1e-9, with scale = |ref| by default.
    For a sum with cancellation (an attention output), pass scale = sum_j p_j |v_j|."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    if got.size == 0:
        return
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    worst = int(np.argmax(err))
    assert err.max() <= VOTE_ABS, f"{what}: abs err {err.max():.3g} at {worst}"
    bound = VOTE_REL * (np.abs(ref) if scale is None else np.asarray(scale, np.float64)) + VOTE_FLOOR
    bad = np.flatnonzero(err > bound)
    assert bad.size == 0, (f"{what}: {bad.size} values beyond rel {VOTE_REL}; first at {bad[0]}: "
                           f"got {got[bad[0]]!r} ref {ref[bad[0]]!r}")


def check_topk(pooled_ref, idx_ref, idx_gpu, rel=REL):
    """Check a GPU kept-position list against the oracle's scores. Returns
    'exact' when the oracle's k-th/(k+1)-th gap decides the set, else 'near-tie'."""
    idx_gpu = np.asarray(idx_gpu, np.int64)
    kk = len(idx_ref)
    n = len(pooled_ref)
    assert idx_gpu.shape == (kk,), f"expected {kk} indices, got {idx_gpu.shape}"
    assert np.all(idx_gpu >= 0) and np.all(idx_gpu < n), "index out of range"
    assert np.all(np.diff(idx_gpu) > 0), "indices must be strictly ascending (sorted, unique)"
    s = np.sort(pooled_ref)[::-1]
    s_k = s[kk - 1]
    s_k1 = s[kk] if kk < n else -np.inf
    if s_k - s_k1 > rel * abs(s_k):
        assert np.array_equal(idx_gpu, idx_ref), (
            f"clear gap but sets differ: {np.setdiff1d(idx_ref, idx_gpu)[:8]} missing, "
            f"{np.setdiff1d(idx_gpu, idx_ref)[:8]} extra")
        return "exact"
    kept = np.zeros(n, bool)
    kept[idx_gpu] = True
    must_keep = pooled_ref > s_k * (1 + rel)
    must_drop = pooled_ref < s_k1 * (1 - rel)
    assert np.all(kept[must_keep]), "a clearly-above-threshold position was dropped"
    assert not np.any(kept[must_drop]), "a clearly-below-threshold position was kept"
    return "near-tie"


def check_gather(k_out, v_out, k_in, v_in, idx_gpu, t0):
    """Output rows are bit copies: kept prefix rows, then the window rows."""
    kk = len(idx_gpu)
    np.testing.assert_array_equal(k_out[:kk], k_in[idx_gpu])
    np.testing.assert_array_equal(v_out[:kk], v_in[idx_gpu])
    np.testing.assert_array_equal(k_out[kk:], k_in[t0:])
    np.testing.assert_array_equal(v_out[kk:], v_in[t0:])


def check_topk_self(pooled_gpu, idx_gpu, kk):
    """The GPU's kept list is exactly the top-kk of the GPU's own pooled scores under the tie rule
    (larger score first, equal scores: lower position first), ascending. Integer work on the GPU's
    float32 values, so it must hold bit for bit at any size, near-ties and plateaus included."""
    p = np.asarray(pooled_gpu, np.float32)
    idx_gpu = np.asarray(idx_gpu, np.int64)
    n = p.shape[0]
    assert idx_gpu.shape == (kk,), f"expected {kk} indices, got {idx_gpu.shape}"
    assert np.all(np.diff(idx_gpu) > 0), "indices must be strictly ascending"
    assert idx_gpu[0] >= 0 and idx_gpu[-1] < n, "index out of range"
    # the kk-th largest key (score desc, position asc): everything strictly above
    # the threshold score is kept, and among positions equal to it the lowest ones
    thr = np.partition(p, n - kk)[n - kk]
    above = np.flatnonzero(p > thr)
    equal = np.flatnonzero(p == thr)
    want = np.sort(np.concatenate([above, equal[:kk - above.size]]))
    assert np.array_equal(idx_gpu, want), (
        f"not the top-{kk} of the GPU's own scores: {np.setdiff1d(want, idx_gpu)[:8]} missing, "
        f"{np.setdiff1d(idx_gpu, want)[:8]} extra")
