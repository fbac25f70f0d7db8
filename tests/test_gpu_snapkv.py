"""GPU parity of kvc_snapkv_compress (through the C ABI) against the CPU oracle."""
import numpy as np
import pytest
import torch

import kv_cache_compression_02_amd as kvc
import synthetic as syn
from oracle import snapkv as ref
from tests import parity as par

pytestmark = pytest.mark.gpu

SCHEDULES = {"two_pass": kvc.SNAPKV_TWO_PASS, "single_pass": kvc.SNAPKV_SINGLE_PASS}


@pytest.fixture(params=list(SCHEDULES))
def schedule(request):
    """Both score schedules; SINGLE_PASS falls back to TWO_PASS where it cannot run (fp32, long heads)."""
    return SCHEDULES[request.param]


def _run(q, k, v, wl_window, budget, pool, dtype, schedule=kvc.SNAPKV_AUTO, want_vote=True, want_pooled=True, **kw):
    if "workspace" not in kw:
        B, H, L, D = k.shape
        n = kvc.snapkv_workspace_bytes(B, H, L, D, wl_window, budget, pool, k.dtype)
        kw["workspace"] = torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda")  # garbage on entry
    with kvc.snapkv_schedule(schedule):
        res = kvc.snapkv_compress(q, k, v, wl_window, budget, pool, want_pooled=want_pooled, want_vote=want_vote,
                                  **kw)
    torch.cuda.synchronize()
    ran = kvc.snapkv_last_schedule()
    print(f"[snapkv] schedule asked {schedule} ran {ran} ({kvc.snapkv_last_score_kernel()})", flush=True)
    if dtype == "fp32" or schedule == kvc.SNAPKV_TWO_PASS:
        assert ran == kvc.SNAPKV_TWO_PASS
    return res


# Inputs of the last named workload and the oracle's results on them, kept across the two
# schedules (the 380K layer takes about a minute to generate and as long to run through the oracle).
_CACHE = {}


def _batch(wl):
    if _CACHE.get("wl") != wl:
        _CACHE.clear()
        _CACHE["wl"] = wl
        _CACHE["batch"] = syn.snapkv_batch(wl)
    return _CACHE["batch"]


def _oracle(qn, kn, vn, b, h, window, budget, pool, dtype, cache_key=None):
    key = (cache_key, b, h, window, budget, pool)
    r = _CACHE.get(key) if cache_key is not None else None
    if r is None:
        r = ref.compress_head(qn[b, h, qn.shape[2] - window:], kn[b, h], vn[b, h], budget, pool, dtype)
        r = {n: r[n] for n in ("vote", "pooled", "idx", "k_out", "v_out")}  # the [w, L] softmax is not kept
        if cache_key is not None:
            _CACHE[key] = r
    return r


def _compare(qn, kn, vn, res, window, budget, pool, dtype, heads=None, cache_key=None):
    """Compare GPU results with the oracle on the given (b, h) pairs (default: all). Returns the
    per-head classification of the kept set under the 1e-3 rule ('exact' / 'near-tie'); every
    head is also held to the tighter band parity.REL_TIGHT and, when the pooled scores were
    returned, to the bit-exact rule that its kept list is the top-k of its own pooled scores."""
    B, H, L, D = kn.shape
    t0 = L - window
    idx = res.idx.cpu().numpy()
    k_out = par.to_host_bits(res.k)
    v_out = par.to_host_bits(res.v)
    vote = res.vote.cpu().numpy() if res.vote is not None else None
    pooled = res.pooled.cpu().numpy() if res.pooled is not None else None
    pairs = heads or [(b, h) for b in range(B) for h in range(H)]
    kinds = []
    for b, h in pairs:
        r = _oracle(qn, kn, vn, b, h, window, budget, pool, dtype, cache_key)
        if vote is not None:
            par.assert_close_votes(vote[b, h], r["vote"], f"vote[{b},{h}]")
        if pooled is not None:
            par.assert_close_votes(pooled[b, h], r["pooled"], f"pooled[{b},{h}]")
            par.check_topk_self(pooled[b, h], idx[b, h], budget - window)
        kinds.append(par.check_topk(r["pooled"], r["idx"], idx[b, h]))
        par.check_topk(r["pooled"], r["idx"], idx[b, h], rel=par.REL_TIGHT)
        par.check_gather(k_out[b, h], v_out[b, h], kn[b, h], vn[b, h], idx[b, h], t0)
        if kinds[-1] == "exact":
            np.testing.assert_array_equal(k_out[b, h], r["k_out"])
            np.testing.assert_array_equal(v_out[b, h], r["v_out"])
    return kinds


def _report(name, kinds, n_heads):
    """Log how many heads the 1e-3 rule compared exactly and how many as near-ties, and check that
    every head was compared."""
    ex, nt = kinds.count("exact"), kinds.count("near-tie")
    print(f"[snapkv] {name}: {ex} exact, {nt} near-tie heads of {n_heads} compared", flush=True)
    assert ex + nt == len(kinds) == n_heads


def _workload(wl, heads=None, schedule=kvc.SNAPKV_AUTO, want_vote=True, want_pooled=True):
    print(f"[snapkv] workload {wl.name} B{wl.B} H{wl.H} D{wl.D} L{wl.L} w{wl.window} "
          f"C{wl.budget} p{wl.pool_kernel} {wl.dtype} schedule {schedule}", flush=True)
    qn, kn, vn = _batch(wl)
    q, k, v = (par.to_device(x, wl.dtype) for x in (qn, kn, vn))
    res = _run(q, k, v, wl.window, wl.budget, wl.pool_kernel, wl.dtype, schedule, want_vote=want_vote,
               want_pooled=want_pooled)
    del q, k, v
    kinds = _compare(qn, kn, vn, res, wl.window, wl.budget, wl.pool_kernel, wl.dtype, heads, cache_key=wl)
    _report(wl.name, kinds, len(heads) if heads else wl.B * wl.H)
    return kinds


def test_tiny_fp32_full(schedule):
    _workload(syn.SNAPKV_WORKLOADS["tiny-fp32"], schedule=schedule)


def test_16k_shape_ragged_small(schedule):
    # several MFMA chunks, pooling chunks and a ragged tail (L - w = 2968)
    _workload(syn.SNAPKV_WORKLOADS["16k-bf16"].with_(L=3000, H=4), schedule=schedule)


def test_16k_full_all_heads(schedule):
    _workload(syn.SNAPKV_WORKLOADS["16k-bf16"], schedule=schedule)
    assert kvc.snapkv_last_select_kernel() == "snap_select_head"
    if schedule == kvc.SNAPKV_SINGLE_PASS:
        assert kvc.snapkv_last_schedule() == kvc.SNAPKV_SINGLE_PASS


def test_131k_full_all_heads(schedule):
    _workload(syn.SNAPKV_WORKLOADS["131k-bf16"], schedule=schedule)
    if schedule == kvc.SNAPKV_SINGLE_PASS:
        assert kvc.snapkv_last_schedule() == kvc.SNAPKV_SINGLE_PASS


def test_131k_no_optional_outputs_all_heads(schedule):
    """No vote or pooled output (the benchmark's call): raw votes live in the workspace only."""
    _workload(syn.SNAPKV_WORKLOADS["131k-bf16"], want_vote=False, want_pooled=False, schedule=schedule)
    assert kvc.snapkv_last_select_kernel() == "snap_select"


def test_380k_full_all_heads(schedule):
    _workload(syn.SNAPKV_WORKLOADS["380k-bf16"], schedule=schedule)
    if schedule == kvc.SNAPKV_SINGLE_PASS:
        assert kvc.snapkv_last_score_kernel() == "snap_wave_bf16"


def test_600k_global_bitmap():
    """A prefix longer than the selection keeps in LDS (N > 524288 positions: the bitmap stays in
    device memory and every output is compacted from it); heads of 600K keys span more rounds than
    the single pass allows, so both schedules run two passes."""
    wl = syn.SNAPKV_WORKLOADS["380k-bf16"].with_(name="600k-bf16", L=600000, H=2, seed=20266)
    _workload(wl)
    assert kvc.snapkv_last_schedule() == kvc.SNAPKV_TWO_PASS


def test_short_heads_straddling_rounds(schedule):
    """52 heads of 10000 keys (40 tile groups each, not a divisor of a round's 256): heads such as
    head 6 start at the end of one round and finish at the start of the next, so two ranges of
    workgroups count for them; the layer ends in a partial round."""
    wl = syn.SnapKVWorkload(name="short-straddle", B=1, H=52, D=128, L=10000, window=32, budget=512,
                            pool_kernel=7, dtype="bf16", n_spans=8, span_len=6, span_boost=1.5, seed=5252)
    _workload(wl, heads=[(0, 0), (0, 6), (0, 32), (0, 51)], schedule=schedule)
    if schedule == kvc.SNAPKV_SINGLE_PASS:
        assert kvc.snapkv_last_score_kernel() == "snap_wave_bf16"


def test_short_heads_d64_sampled_heads(schedule):
    """32 heads of 16K keys at head dim 64: under the single pass, the independent-wave kernel's
    short-head form at D = 64 (each workgroup one head per round)."""
    wl = syn.SnapKVWorkload(name="short-d64", B=1, H=32, D=64, L=16384, window=32, budget=1024, pool_kernel=7,
                            dtype="bf16", n_spans=12, span_len=8, span_boost=1.5, seed=1664)
    _workload(wl, heads=[(0, 0), (0, 13), (0, 31)], schedule=schedule)
    if schedule == kvc.SNAPKV_SINGLE_PASS:
        assert kvc.snapkv_last_score_kernel() == "snap_wave_bf16"


EDGE = [
    # dtype, D, window, L, budget, pool
    ("bf16", 64, 1, 100, 2, 1),
    ("bf16", 128, 32, 70, 33, 3),        # one kept prefix position
    ("bf16", 128, 32, 1057, 1056, 65),   # keeps all but one prefix position; widest pool
    ("bf16", 128, 17, 5000, 300, 5),
    ("bf16", 64, 32, 4097, 600, 7),
    ("fp32", 128, 8, 777, 100, 9),
    ("fp32", 64, 32, 300, 64, 3),
    ("fp32", 64, 16, 513, 128, 5),
]


@pytest.mark.parametrize("dtype,D,w,L,budget,pool", EDGE)
def test_edge_shapes(dtype, D, w, L, budget, pool, schedule):
    wl = syn.SnapKVWorkload(name=f"edge-{dtype}-{D}-{w}-{L}", B=1, H=3, D=D, L=L, window=w, budget=budget,
                            pool_kernel=pool, dtype=dtype, n_spans=2, span_len=3, span_boost=2.0,
                            seed=777 + L)
    _workload(wl, schedule=schedule)


@pytest.mark.parametrize("L,w,pool", [(6000, 32, 7), (6000, 32, 9), (6000, 32, 11), (5002, 17, 5), (3000, 8, 1)])
def test_no_optional_outputs(L, w, pool, schedule):
    """Only the kept indices and rows asked for (no votes, no pooled scores): the
    path where the selection pools the raw votes itself (radius <= 4), reads
    pooled scores the pooling kernel stored only for it (larger radii), or
    takes scalar loads (prefix length not a multiple of 4)."""
    wl = syn.SnapKVWorkload(name=f"noout-{L}-{w}-{pool}", B=1, H=5, D=128, L=L, window=w, budget=400,
                            pool_kernel=pool, dtype="bf16", n_spans=6, span_len=5, span_boost=1.5, seed=4242 + pool)
    qn, kn, vn = syn.snapkv_batch(wl)
    q, k, v = par.to_device(qn, "bf16"), par.to_device(kn, "bf16"), par.to_device(vn, "bf16")
    print(f"[snapkv] no optional outputs L{L} w{w} p{pool} schedule {schedule}", flush=True)
    res = _run(q, k, v, wl.window, wl.budget, wl.pool_kernel, "bf16", schedule, want_vote=False, want_pooled=False)
    assert res.vote is None and res.pooled is None
    kinds = _compare(qn, kn, vn, res, wl.window, wl.budget, wl.pool_kernel, "bf16")
    print(f"[snapkv] {wl.name}: {kinds.count('exact')} exact, {kinds.count('near-tie')} near-tie heads", flush=True)


@pytest.mark.parametrize("pool", [7, 17])
def test_single_pass_residency_fallback(pool):
    """The score kernel's residency check forced to fail from the host (it waits
    for one workgroup more than its grid has, briefly): the kernel flags every
    head, the pooling kernel (register windows for p = 7, the LDS path for
    p = 17) computes all votes exactly, and the results still match the oracle."""
    wl = syn.SNAPKV_WORKLOADS["16k-bf16"].with_(B=1, H=2, L=70000, budget=1200, pool_kernel=pool)
    lib = kvc.library()
    prev = lib.kvc_snapkv_force_residency_fallback(1)
    try:
        _workload(wl, schedule=kvc.SNAPKV_SINGLE_PASS)
        assert kvc.snapkv_last_score_kernel() == "snap_wave_bf16"
    finally:
        lib.kvc_snapkv_force_residency_fallback(prev)


def test_single_pass_residency_fallback_fused_select():
    """The same at the 16K layer's shape, where the per-head selection kernel also does the pooling
    kernel's work (no pooling kernel is launched): each selection workgroup recomputes its flagged
    head's votes exactly before pooling and counting them."""
    wl = syn.SNAPKV_WORKLOADS["16k-bf16"]
    lib = kvc.library()
    prev = lib.kvc_snapkv_force_residency_fallback(1)
    try:
        _workload(wl, heads=[(0, 0), (0, 17), (1, 31)], schedule=kvc.SNAPKV_SINGLE_PASS)
        assert kvc.snapkv_last_score_kernel() == "snap_wave_bf16"
        assert kvc.snapkv_last_select_kernel() == "snap_select_head"
    finally:
        lib.kvc_snapkv_force_residency_fallback(prev)


@pytest.mark.parametrize("pool", [7, 17])
def test_single_pass_wait_timeout(pool):
    """The independent-wave kernel's cross-worker waits given a limit of zero polls from the host: a
    head's finisher gives up before publishing and every vote that would wait gives up at once, each
    recording a failure code in the status word. The kernel still exits; the pooling kernel reads the
    status word and recomputes every head's votes exactly, so the results match the oracle and the
    votes equal, bit for bit, those of the residency fallback (the same exact path)."""
    wl = syn.SNAPKV_WORKLOADS["16k-bf16"].with_(B=1, H=2, L=70000, budget=1200, pool_kernel=pool)
    qn, kn, vn = _batch(wl)
    q, k, v = (par.to_device(x, "bf16") for x in (qn, kn, vn))
    lib = kvc.library()
    print(f"[snapkv] forced wait timeout, p{pool}", flush=True)
    prev = lib.kvc_snapkv_force_wait_timeout(1)
    try:
        forced = _run(q, k, v, wl.window, wl.budget, pool, "bf16", kvc.SNAPKV_SINGLE_PASS)
        assert kvc.snapkv_last_score_kernel() == "snap_wave_bf16"
    finally:
        lib.kvc_snapkv_force_wait_timeout(prev)
    prev = lib.kvc_snapkv_force_residency_fallback(1)
    try:
        fallback = _run(q, k, v, wl.window, wl.budget, pool, "bf16", kvc.SNAPKV_SINGLE_PASS)
    finally:
        lib.kvc_snapkv_force_residency_fallback(prev)
    normal = _run(q, k, v, wl.window, wl.budget, pool, "bf16", kvc.SNAPKV_SINGLE_PASS)
    assert torch.equal(forced.vote, fallback.vote) and torch.equal(forced.idx, fallback.idx)
    assert not torch.equal(forced.vote, normal.vote), "the exact recomputation did not run"
    _report(f"wait-timeout-p{pool}", _compare(qn, kn, vn, forced, wl.window, wl.budget, pool, "bf16",
                                              cache_key=wl), wl.B * wl.H)


@pytest.mark.parametrize("name,H,L", [("16k-bf16", 32, 8000), ("16k-bf16", 32, 9000), ("16k-bf16", 26, 10000),
                                      ("16k-bf16", 32, 16384), ("131k-bf16", 32, 131072)])
def test_single_pass_waits_end_in_time(name, H, L):
    """Every bounded wait of the independent-wave kernel ends in time on ordinary inputs: the status
    word reads 0 after the call and the residency gate passed, so the votes come from the single
    pass itself, not from the exact fallback (which would give the same kept positions, only
    slower). With 256 workgroups of 8 waves, 64 heads of 8000 keys (256 tiles) put 8 whole heads
    in each round, so a workgroup's head advances by 8 from round to round and one wave merges
    every round's sums; at 9000 keys (288 tiles) the advance is 7 or 8; at 10000 keys (320 tiles)
    6 or 7; the 16K and 131K layers have other step patterns (4 heads a round, and heads longer
    than a round). Two heads of the short-head shapes are also checked against the oracle."""
    wl = syn.SNAPKV_WORKLOADS[name].with_(H=H, L=L)
    qn, kn, vn = _batch(wl)
    q, k, v = (par.to_device(x, "bf16") for x in (qn, kn, vn))
    B, _, _, D = k.shape
    n = kvc.snapkv_workspace_bytes(B, H, L, D, wl.window, wl.budget, wl.pool_kernel, k.dtype)
    off = kvc.snapkv_status_offset(B, H, L, D, wl.window, wl.budget, wl.pool_kernel, k.dtype)
    assert 0 < off and off + 12 <= n and off % 4 == 0
    ws = torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda")
    for rep in range(3):
        print(f"[snapkv] status word {name} B{B} H{H} L{L} call {rep}", flush=True)
        res = _run(q, k, v, wl.window, wl.budget, wl.pool_kernel, "bf16", kvc.SNAPKV_SINGLE_PASS, workspace=ws)
        assert kvc.snapkv_last_score_kernel() == "snap_wave_bf16"
        words = ws[off:off + 12].view(torch.int32).cpu().tolist()
        assert words[0] == 0 and words[2] == 1, f"status word {words[0]}, gate {words[1:]}"
        # pooling inside the selection: one workgroup per head, or (131K: 8 workgroups for each of
        # 32 heads, one per compute unit) the head's workgroups together
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        want = "snap_select_head" if L - wl.window <= 16384 else "snap_select" if cus >= 256 else None
        if want:
            assert kvc.snapkv_last_pool_kernel() == want
    if L < 20000:
        _report(f"waits-{L}", _compare(qn, kn, vn, res, wl.window, wl.budget, wl.pool_kernel, "bf16",
                                       heads=[(0, 0), (B - 1, H - 1)]), 2)


def test_single_pass_two_finishers_per_workgroup():
    """More heads than workgroups (9 x 32 = 288 heads of 16K keys on 256 workgroups): head g is
    finished by wave 0 of workgroup g and head g + 256 by its wave 1, which share a staging buffer
    (taken by compare-and-swap). The waits end in time and sampled heads of both finishers match
    the oracle."""
    wl = syn.SNAPKV_WORKLOADS["16k-bf16"].with_(B=9)
    qn, kn, vn = _batch(wl)
    q, k, v = (par.to_device(x, "bf16") for x in (qn, kn, vn))
    B, H, L, D = k.shape
    n = kvc.snapkv_workspace_bytes(B, H, L, D, wl.window, wl.budget, wl.pool_kernel, k.dtype)
    off = kvc.snapkv_status_offset(B, H, L, D, wl.window, wl.budget, wl.pool_kernel, k.dtype)
    ws = torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda")
    print(f"[snapkv] two finishers per workgroup B{B} H{H} L{L}", flush=True)
    res = _run(q, k, v, wl.window, wl.budget, wl.pool_kernel, "bf16", kvc.SNAPKV_SINGLE_PASS, workspace=ws)
    assert kvc.snapkv_last_score_kernel() == "snap_wave_bf16"
    words = ws[off:off + 12].view(torch.int32).cpu().tolist()
    assert words[0] == 0 and words[2] == 1, f"status word {words[0]}, gate {words[1:]}"
    del q, k, v
    heads = [(0, 0), (0, 1), (8, 0), (8, 31)]  # heads 0, 1 (wave 0) and 256, 287 (wave 1)
    _report("two-finishers", _compare(qn, kn, vn, res, wl.window, wl.budget, wl.pool_kernel, "bf16", heads=heads),
            len(heads))


def test_single_pass_many_heads_unaligned():
    """Heads whose units straddle device-wide rounds (B*H*units not a multiple of the grid)."""
    wl = syn.SNAPKV_WORKLOADS["16k-bf16"].with_(B=3, H=7, L=70001, budget=1500)
    _workload(wl, heads=[(0, 0), (1, 3), (2, 6)], schedule=kvc.SNAPKV_SINGLE_PASS)
    assert kvc.snapkv_last_schedule() == kvc.SNAPKV_SINGLE_PASS


@pytest.mark.parametrize("L,C", [(2000, 300), (12000, 1024), (70000, 2048), (600000, 1024)])
def test_zero_queries_exact_ties(L, C, schedule):
    """Q = 0 makes every vote equal: the tie rule alone decides, so the kept set is 0..k-1.
    Every prefix position then shares the threshold bin. At L = 12000 one workgroup selects each
    head and its 11968 candidates overflow its LDS list into the head's device list; at
    L = 70000 several workgroups select each head and their lists overflow the same way; both
    rank with several radix passes over the position bits before the direct rank. At
    L = 600000 the bitmap also lives in device memory (N > 524288)."""
    B, H, D, w = 1, 2, 128, 32
    print(f"[snapkv] zero queries L{L} C{C} schedule {schedule}", flush=True)
    rng = np.random.default_rng(L)
    kn = syn.f32_to_bf16_bits(rng.standard_normal((B, H, L, D), dtype=np.float32))
    qn = np.zeros((B, H, w, D), np.uint16)
    q, k = par.to_device(qn, "bf16"), par.to_device(kn, "bf16")
    res = _run(q, k, k, w, C, 7, "bf16", schedule)
    idx = res.idx.cpu().numpy()
    for h in range(H):
        assert idx[0, h].tolist() == list(range(C - w))
    vote = res.vote.cpu().numpy()
    assert np.all(vote == vote[:, :, :1]), "equal votes expected bit for bit"
    _report(f"zero-queries-{L}", _compare(qn, kn, kn, res, w, C, 7, "bf16"), B * H)


class _SplitSelect:
    """Forces the several-workgroups-per-head selection while active (mode 2: and the single pass's
    separate pooling kernel)."""

    def __init__(self, mode=1):
        self.mode = mode

    def __enter__(self):
        self.prev = kvc.library().kvc_snapkv_force_split_select(self.mode)

    def __exit__(self, *exc):
        kvc.library().kvc_snapkv_force_split_select(self.prev)


@pytest.mark.parametrize("L,C", [(2000, 300), (70000, 2048)])
def test_zero_queries_exact_ties_split_select(L, C):
    """The tie rule through the split selection (at L = 70000 the candidates overflow each
    workgroup's LDS list into the head's device list)."""
    B, H, D, w = 1, 2, 128, 32
    print(f"[snapkv] zero queries, split selection, L{L} C{C}", flush=True)
    rng = np.random.default_rng(L + 1)
    kn = syn.f32_to_bf16_bits(rng.standard_normal((B, H, L, D), dtype=np.float32))
    qn = np.zeros((B, H, w, D), np.uint16)
    q, k = par.to_device(qn, "bf16"), par.to_device(kn, "bf16")
    with _SplitSelect():
        res = _run(q, k, k, w, C, 7, "bf16")
        assert kvc.snapkv_last_select_kernel() == "snap_select"
    idx = res.idx.cpu().numpy()
    for h in range(H):
        assert idx[0, h].tolist() == list(range(C - w))


@pytest.mark.parametrize("name,L,pool", [("16k-bf16", None, 7), ("16k-bf16", None, 13), ("131k-bf16", 16416, 7),
                                          ("16k-bf16", 9000, 5), ("131k-bf16", 70000, 7)])
def test_select_forms_agree(name, L, pool):
    """One workgroup per head (heads of at most 16384 prefix positions) and several per head keep
    the same positions, bit for bit, on the same votes (both schedules' votes: the selection reads
    raw votes and pools them itself for a max-pool of radius <= 4, else the pooling kernel's
    stored scores). Under the single pass with a max-pool of radius <= 4 the selection also does
    the pooling kernel's work (pooled output and histogram), which is then not launched: the
    per-head form alone, the split form with the head's workgroups adding to one histogram and
    meeting on it; the split form with the separate pooling kernel is the third form compared.
    Their pooled scores agree bit for bit."""
    wl = syn.SNAPKV_WORKLOADS[name].with_(pool_kernel=pool)
    if L is not None:
        wl = wl.with_(L=L, name=f"{name}-L{L}")
    print(f"[snapkv] selection forms on {wl.name} p{pool}", flush=True)
    qn, kn, vn = _batch(wl.with_(pool_kernel=syn.SNAPKV_WORKLOADS[name].pool_kernel))
    q, k, v = (par.to_device(x, wl.dtype) for x in (qn, kn, vn))
    short = wl.L - wl.window <= 16384
    for schedule in (kvc.SNAPKV_SINGLE_PASS, kvc.SNAPKV_TWO_PASS):
        single = schedule == kvc.SNAPKV_SINGLE_PASS
        fused = single and pool <= 9
        runs = []
        for mode in (0, 1, 2):
            with _SplitSelect(mode):
                runs.append(_run(q, k, v, wl.window, wl.budget, pool, wl.dtype, schedule, want_vote=True,
                                 want_pooled=True))
                per_head = mode == 0 and short
                assert kvc.snapkv_last_select_kernel() == ("snap_select_head" if per_head else "snap_select")
                want_pool = ("snap_select_head" if per_head else "snap_select" if mode < 2 else "snap_pool") \
                    if fused else "snap_pool" if single else "snap_votes_bf16"
                assert kvc.snapkv_last_pool_kernel() == want_pool
        a = runs[0]
        for b in runs[1:]:
            assert torch.equal(a.vote, b.vote) and torch.equal(a.pooled, b.pooled)  # deterministic votes
            assert torch.equal(a.idx, b.idx)
            assert torch.equal(a.k, b.k) and torch.equal(a.v, b.v)
        pooled, idx = a.pooled.cpu().numpy(), a.idx.cpu().numpy()
        for bb in range(wl.B):
            for h in range(wl.H):
                par.check_topk_self(pooled[bb, h], idx[bb, h], wl.budget - wl.window)


def test_planted_spike_neighbourhood(schedule):
    B, H, L, D, w, p = 1, 1, 3000, 128, 32, 7
    rng = np.random.default_rng(1)
    q32 = rng.standard_normal((B, H, w, D), dtype=np.float32)
    k32 = rng.standard_normal((B, H, L, D), dtype=np.float32)
    u = q32[0, 0].mean(0)
    j = 1234
    k32[0, 0, j] += 30.0 * u / np.linalg.norm(u)
    qn, kn = syn.f32_to_bf16_bits(q32), syn.f32_to_bf16_bits(k32)
    res = _run(par.to_device(qn, "bf16"), par.to_device(kn, "bf16"), par.to_device(kn, "bf16"), w, w + p, p,
               "bf16", schedule)
    assert res.idx[0, 0].cpu().tolist() == list(range(j - 3, j + 4))


def test_strided_inputs(schedule):
    """q_len > window and K/V row strides wider than D (views into padded buffers)."""
    B, H, L, D, w, C, p = 2, 3, 2500, 128, 32, 256, 7
    rng = np.random.default_rng(2)
    qbig = syn.f32_to_bf16_bits(rng.standard_normal((B, H, 48, D), dtype=np.float32))
    kbig = syn.f32_to_bf16_bits(rng.standard_normal((B, H, L, D + 64), dtype=np.float32))
    vbig = syn.f32_to_bf16_bits(rng.standard_normal((B, H, L, D + 64), dtype=np.float32))
    qd, kd, vd = (par.to_device(x, "bf16") for x in (qbig, kbig, vbig))
    k, v = kd[..., :D], vd[..., :D]
    assert k.stride(2) == D + 64
    res = _run(qd, k, v, w, C, p, "bf16", schedule)
    _compare(qbig, np.ascontiguousarray(kbig[..., :D]), np.ascontiguousarray(vbig[..., :D]), res, w, C, p,
             "bf16")


def test_deterministic_and_workspace_reuse(schedule):
    wl = syn.SNAPKV_WORKLOADS["16k-bf16"].with_(L=6000, H=4)
    qn, kn, vn = syn.snapkv_batch(wl)
    q, k, v = (par.to_device(x, "bf16") for x in (qn, kn, vn))
    nbytes = kvc.snapkv_workspace_bytes(wl.B, wl.H, wl.L, wl.D, wl.window, wl.budget, wl.pool_kernel,
                                        torch.bfloat16)
    ws = torch.full((nbytes,), 0xAB, dtype=torch.uint8, device="cuda")  # garbage on entry
    a = _run(q, k, v, wl.window, wl.budget, wl.pool_kernel, "bf16", schedule, workspace=ws)
    # a different input through the same workspace, then the first again
    wl2 = wl.with_(seed=wl.seed + 1)
    qn2, kn2, vn2 = syn.snapkv_batch(wl2)
    q2, k2, v2 = (par.to_device(x, "bf16") for x in (qn2, kn2, vn2))
    b = _run(q2, k2, v2, wl.window, wl.budget, wl.pool_kernel, "bf16", schedule, workspace=ws)
    c = _run(q, k, v, wl.window, wl.budget, wl.pool_kernel, "bf16", schedule, workspace=ws)
    assert torch.equal(a.idx, c.idx) and torch.equal(a.vote, c.vote) and torch.equal(a.k, c.k)
    _compare(qn2, kn2, vn2, b, wl.window, wl.budget, wl.pool_kernel, "bf16")


def test_prepared_call_matches():
    """A SnapKVCall (arguments checked and marshalled once) gives what snapkv_compress gives, bit for
    bit, call after call, with the inputs' contents changed between calls."""
    wl = syn.SNAPKV_WORKLOADS["16k-bf16"].with_(B=1, H=4, L=20000, budget=1500)
    qn, kn, vn = syn.snapkv_batch(wl)
    q, k, v = (par.to_device(x, "bf16") for x in (qn, kn, vn))
    B, H, L, D = k.shape
    n = kvc.snapkv_workspace_bytes(B, H, L, D, wl.window, wl.budget, wl.pool_kernel, k.dtype)
    ws = torch.empty((n,), dtype=torch.uint8, device="cuda")
    call = kvc.SnapKVCall(q, k, v, wl.window, wl.budget, wl.pool_kernel, want_vote=True, want_pooled=True,
                          workspace=ws)
    print("[snapkv] prepared call", flush=True)
    for rep in range(3):
        if rep == 2:
            k.mul_(-1.0)  # new contents, same buffers
        got = call()
        torch.cuda.synchronize()
        want = kvc.snapkv_compress(q, k, v, wl.window, wl.budget, wl.pool_kernel, want_vote=True, want_pooled=True)
        torch.cuda.synchronize()
        for a, b in zip(got, want):
            assert torch.equal(a, b)
    bad = kvc.SnapKVCall(q, k, v, wl.window, wl.budget, wl.pool_kernel, workspace=ws[: n // 2])
    with pytest.raises(kvc.KvcError):
        bad()


def test_error_statuses():
    B, H, L, D = 1, 2, 512, 128
    k = torch.zeros((B, H, L, D), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kvc.KvcError) as e:
        kvc.snapkv_compress(k, k, k, 32, 512, 7)  # budget >= L
    assert e.value.status == kvc.KVC_ERR_INVALID_ARG
    with pytest.raises(kvc.KvcError) as e:
        kvc.snapkv_compress(k, k, k, 40, 100, 7)  # window > 32
    assert e.value.status == kvc.KVC_ERR_UNSUPPORTED
    with pytest.raises(kvc.KvcError) as e:
        kvc.snapkv_compress(k, k, k, 32, 100, 7, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert e.value.status == kvc.KVC_ERR_WORKSPACE
    with pytest.raises(kvc.KvcError) as e:
        kvc.snapkv_compress(k, k, k, 32, 100, 4)  # even pool kernel
    assert e.value.status == kvc.KVC_ERR_INVALID_ARG


def test_schedules_agree():
    """Both schedules on one input: same kept set up to near-ties, votes within rounding."""
    wl = syn.SNAPKV_WORKLOADS["16k-bf16"].with_(L=9000, H=4)
    qn, kn, vn = syn.snapkv_batch(wl)
    q, k, v = (par.to_device(x, "bf16") for x in (qn, kn, vn))
    a = _run(q, k, v, wl.window, wl.budget, wl.pool_kernel, "bf16", kvc.SNAPKV_TWO_PASS)
    b = _run(q, k, v, wl.window, wl.budget, wl.pool_kernel, "bf16", kvc.SNAPKV_SINGLE_PASS)
    assert kvc.snapkv_last_schedule() == kvc.SNAPKV_SINGLE_PASS
    va, vb = a.vote.cpu().numpy(), b.vote.cpu().numpy()
    for h in range(wl.H):
        par.assert_close_votes(vb[0, h], va[0, h].astype(np.float64), f"vote[0,{h}] single vs two-pass")
    same = (a.idx == b.idx).float().mean().item()
    assert same > 0.99, same


@pytest.mark.parametrize("L,kernel", [(9000, "snap_coop_bf16"), (70000, "snap_wave_bf16")])
def test_single_pass_logit_overflow(L, kernel):
    """A key scoring 2^180 above window row 0's reference flags the head: its normalisers
    come from the exact merge of per-unit / per-workgroup partials instead of the
    fixed-point accumulators, and the votes still match the oracle."""
    B, H, D, w, C, p = 1, 2, 128, 32, 400, 7
    rng = np.random.default_rng(5)
    q32 = rng.standard_normal((B, H, w, D), dtype=np.float32)
    k32 = rng.standard_normal((B, H, L, D), dtype=np.float32)
    j = 5000
    for h in range(H):
        u = q32[0, h, 0]
        k32[0, h, j] = 130.0 * u / np.linalg.norm(u)  # row 0: score ~ 1.44 * 130 in log2 units
    qn, kn = syn.f32_to_bf16_bits(q32), syn.f32_to_bf16_bits(k32)
    vn = syn.f32_to_bf16_bits(rng.standard_normal((B, H, L, D), dtype=np.float32))
    q, k, v = (par.to_device(x, "bf16") for x in (qn, kn, vn))
    print(f"[snapkv] overflow case L{L}", flush=True)
    res = _run(q, k, v, w, C, p, "bf16", kvc.SNAPKV_SINGLE_PASS)
    assert kvc.snapkv_last_schedule() == kvc.SNAPKV_SINGLE_PASS
    assert kvc.snapkv_last_score_kernel() == kernel
    _compare(qn, kn, vn, res, w, C, p, "bf16")


def test_single_pass_kernel_choice():
    """Long prompts take the independent-wave kernel, short ones the lockstep one
    (when the single pass is asked for)."""
    for L, kernel in ((3000, "snap_coop_bf16"), (131072, "snap_wave_bf16")):
        B, H, D = 1, 2, 128
        q = torch.zeros((B, H, 32, D), dtype=torch.bfloat16, device="cuda")
        k = torch.zeros((B, H, L, D), dtype=torch.bfloat16, device="cuda")
        _run(q, k, k, 32, 256, 7, "bf16", kvc.SNAPKV_SINGLE_PASS)
        assert kvc.snapkv_last_score_kernel() == kernel, (L, kvc.snapkv_last_score_kernel())
    _run(q, k, k, 32, 256, 7, "bf16", kvc.SNAPKV_TWO_PASS)
    assert kvc.snapkv_last_score_kernel() == "snap_stats_bf16+snap_votes_bf16"
    # AUTO: the independent-wave kernel where it runs, else two passes (380000 keys: a head
    # spans six rounds, the most the nine-round vote lag allows)
    for L, kernel in ((3000, "snap_stats_bf16+snap_votes_bf16"), (131072, "snap_wave_bf16"),
                      (380000, "snap_wave_bf16")):
        q = torch.zeros((1, 2, 32, 128), dtype=torch.bfloat16, device="cuda")
        k = torch.zeros((1, 2, L, 128), dtype=torch.bfloat16, device="cuda")
        _run(q, k, k, 32, 256, 7, "bf16", kvc.SNAPKV_AUTO)
        assert kvc.snapkv_last_score_kernel() == kernel, (L, kvc.snapkv_last_score_kernel())
    # heads shorter than a round of the independent-wave kernel (512 tiles against 2048 workers):
    # its short-head form once the layer fills eight rounds (32 heads of 16K keys), else two passes
    for H, kernel in ((32, "snap_wave_bf16"), (8, "snap_stats_bf16+snap_votes_bf16")):
        q = torch.zeros((1, H, 32, 128), dtype=torch.bfloat16, device="cuda")
        k = torch.zeros((1, H, 16384, 128), dtype=torch.bfloat16, device="cuda")
        _run(q, k, k, 32, 1024, 7, "bf16", kvc.SNAPKV_AUTO)
        assert kvc.snapkv_last_score_kernel() == kernel, (H, kvc.snapkv_last_score_kernel())


def test_schedule_setting_rejects_unknown():
    with pytest.raises(ValueError):
        with kvc.snapkv_schedule(7):
            pass
