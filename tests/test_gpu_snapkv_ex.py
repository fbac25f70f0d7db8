"""GPU parity of kvc_snapkv_compress_ex (through the C ABI) against the CPU oracle: the average-pool
variant, ragged batches (per-sequence prompt lengths, pooled/vote rows packed) and all layers of a
prompt in one call (folded into one batch when the layers are stacked, else layer by layer)."""
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
    return SCHEDULES[request.param]


def _check_head(qw, kh, vh, Lb, budget, pool, dtype, pool_type, idx, k_out, v_out, vote=None, pooled=None):
    """One head against the oracle on its own prompt (its first Lb keys); returns 'exact' / 'near-tie'."""
    w = qw.shape[0]
    r = ref.compress_head(qw, kh[:Lb], vh[:Lb], budget, pool, dtype, pool_type=pool_type)
    if vote is not None:
        par.assert_close_votes(vote, r["vote"], "vote")
    if pooled is not None:
        par.assert_close_votes(pooled, r["pooled"], "pooled")
        par.check_topk_self(pooled, idx, budget - w)
    kind = par.check_topk(r["pooled"], r["idx"], idx)
    par.check_topk(r["pooled"], r["idx"], idx, rel=par.REL_TIGHT)
    par.check_gather(k_out, v_out, kh[:Lb], vh[:Lb], idx, Lb - w)
    if kind == "exact":
        np.testing.assert_array_equal(k_out, r["k_out"])
    return kind


def _run(q, k, v, w, budget, pool_kernel, schedule, **kw):
    with kvc.snapkv_schedule(schedule):
        res = kvc.snapkv_compress_ex(q, k, v, w, budget, pool_kernel, want_pooled=True, want_vote=True, **kw)
    torch.cuda.synchronize()
    print(f"[snapkv-ex] schedule {schedule} ran {kvc.snapkv_last_schedule()} ({kvc.snapkv_last_score_kernel()})",
          flush=True)
    return res


def _host(res):
    return (res.idx.cpu().numpy(), par.to_host_bits(res.k), par.to_host_bits(res.v), res.vote.cpu().numpy(),
            res.pooled.cpu().numpy())


@pytest.mark.parametrize("L,p,H", [(6000, 1, 3), (6000, 3, 3), (6000, 7, 3), (5002, 17, 3), (70000, 7, 2),
                                   (70000, 17, 2)])
def test_avg_pool(L, p, H, schedule):
    """Average pooling: the two-pass vote kernels pool in LDS, the single pass's pooling kernel from
    register windows (p <= 15) or LDS, and the selection reads the stored averages."""
    wl = syn.SnapKVWorkload(name=f"avg-{L}-{p}", B=1, H=H, D=128, L=L, window=32, budget=700, pool_kernel=p,
                            dtype="bf16", n_spans=6, span_len=5, span_boost=1.5, seed=600 + p + L)
    print(f"[snapkv-ex] avg pool L{L} p{p} H{H} schedule {schedule}", flush=True)
    qn, kn, vn = syn.snapkv_batch(wl)
    res = _run(*(par.to_device(x, "bf16") for x in (qn, kn, vn)), 32, 700, p, schedule, pool="avg")
    if schedule == kvc.SNAPKV_SINGLE_PASS and L == 70000:
        assert kvc.snapkv_last_score_kernel() == "snap_wave_bf16"
    idx, ko, vo, vote, pooled = _host(res)
    kinds = [_check_head(qn[0, h], kn[0, h], vn[0, h], L, 700, p, "bf16", "avg", idx[0, h], ko[0, h], vo[0, h],
                         vote[0, h], pooled[0, h]) for h in range(H)]
    print(f"[snapkv-ex] avg p{p} L{L}: {kinds.count('exact')} exact, {kinds.count('near-tie')} near-tie", flush=True)


def test_avg_pool_fp32_tiny():
    wl = syn.SNAPKV_WORKLOADS["tiny-fp32"]
    qn, kn, vn = syn.snapkv_batch(wl)
    res = _run(*(par.to_device(x, "fp32") for x in (qn, kn, vn)), wl.window, wl.budget, wl.pool_kernel,
               kvc.SNAPKV_AUTO, pool="avg")
    idx, ko, vo, vote, pooled = _host(res)
    for h in range(wl.H):
        _check_head(qn[0, h], kn[0, h], vn[0, h], wl.L, wl.budget, wl.pool_kernel, "fp32", "avg", idx[0, h], ko[0, h],
                    vo[0, h], vote[0, h], pooled[0, h])


@pytest.mark.parametrize("pool_type", ["max", "avg"])
def test_ragged_batch(pool_type, schedule):
    """Three sequences padded to 9000 keys with lengths 9000, 5000 and 7321: each is compressed over its
    own prompt, its window being its own last 32 positions; pooled/vote rows come back packed."""
    B, H, L, D, w, budget, p = 3, 4, 9000, 128, 32, 600, 7
    lengths = [9000, 5000, 7321]
    rng = np.random.default_rng(31)
    qn = syn.f32_to_bf16_bits(rng.standard_normal((B, H, w, D), dtype=np.float32))
    kn = syn.f32_to_bf16_bits(rng.standard_normal((B, H, L, D), dtype=np.float32))
    vn = syn.f32_to_bf16_bits(rng.standard_normal((B, H, L, D), dtype=np.float32))
    for b, n in enumerate(lengths):  # loud padding: it must not matter
        kn[b, :, n:] = syn.f32_to_bf16_bits(np.full((H, L - n, D), 40.0, np.float32))
    print(f"[snapkv-ex] ragged {lengths} {pool_type} schedule {schedule}", flush=True)
    res = _run(*(par.to_device(x, "bf16") for x in (qn, kn, vn)), w, budget, p, schedule, pool=pool_type,
               lengths=lengths)
    idx, ko, vo, vote, pooled = _host(res)
    assert vote.shape == (H * sum(n - w for n in lengths),)
    off = 0
    for b, n in enumerate(lengths):
        for h in range(H):
            sl = slice(off, off + n - w)
            _check_head(qn[b, h], kn[b, h], vn[b, h], n, budget, p, "bf16", pool_type, idx[b, h], ko[b, h], vo[b, h],
                        vote[sl], pooled[sl])
            off += n - w
    assert off == vote.shape[0]


@pytest.mark.parametrize("stacked", [True, False])
def test_layers_in_one_call(stacked, schedule):
    """Three layers of B2 H4 L4000 in one call: stacked in front of the batch axis they run as one
    batch of six sequences; as a strided view (every layer followed by padding) layer by layer."""
    NL, B, H, L, D, w, budget, p = 3, 2, 4, 4000, 128, 32, 300, 7
    rng = np.random.default_rng(77 + stacked)
    lead = B if stacked else B + 1
    qn = syn.f32_to_bf16_bits(rng.standard_normal((NL, lead, H, w, D), dtype=np.float32))
    kn = syn.f32_to_bf16_bits(rng.standard_normal((NL, lead, H, L, D), dtype=np.float32))
    vn = syn.f32_to_bf16_bits(rng.standard_normal((NL, lead, H, L, D), dtype=np.float32))
    q, k, v = (par.to_device(x, "bf16")[:, :B] for x in (qn, kn, vn))
    assert (k.stride(0) == B * k.stride(1)) == stacked
    print(f"[snapkv-ex] {NL} layers stacked={stacked} schedule {schedule}", flush=True)
    res = _run(q, k, v, w, budget, p, schedule)
    idx, ko, vo, vote, pooled = _host(res)
    assert idx.shape == (NL, B, H, budget - w) and ko.shape == (NL, B, H, budget, D)
    for l in range(NL):
        for b in range(B):
            for h in range(H):
                _check_head(qn[l, b, h], kn[l, b, h], vn[l, b, h], L, budget, p, "bf16", "max", idx[l, b, h],
                            ko[l, b, h], vo[l, b, h], vote[l, b, h], pooled[l, b, h])


def test_layers_ragged_avg():
    """Two layers, a ragged batch of two and average pooling together."""
    NL, B, H, L, D, w, budget, p = 2, 2, 3, 3000, 64, 16, 200, 5
    lengths = [2100, 3000]
    rng = np.random.default_rng(5)
    qn = syn.f32_to_bf16_bits(rng.standard_normal((NL, B, H, w, D), dtype=np.float32))
    kn = syn.f32_to_bf16_bits(rng.standard_normal((NL, B, H, L, D), dtype=np.float32))
    vn = syn.f32_to_bf16_bits(rng.standard_normal((NL, B, H, L, D), dtype=np.float32))
    res = _run(*(par.to_device(x, "bf16") for x in (qn, kn, vn)), w, budget, p, kvc.SNAPKV_AUTO, pool="avg",
               lengths=lengths)
    idx, ko, vo, vote, pooled = _host(res)
    off = 0
    for l in range(NL):
        for b, n in enumerate(lengths):
            for h in range(H):
                sl = slice(off, off + n - w)
                _check_head(qn[l, b, h], kn[l, b, h], vn[l, b, h], n, budget, p, "bf16", "avg", idx[l, b, h],
                            ko[l, b, h], vo[l, b, h], vote[sl], pooled[sl])
                off += n - w


def test_16k_layers_fold_into_the_single_pass():
    """Four layers of the 16K batch-2 workload in one call: 256 heads of 16K keys fill the independent-wave
    kernel's short-head form; sampled heads of every layer checked."""
    wl = syn.SNAPKV_WORKLOADS["16k-bf16"]
    NL = 4
    layers = [syn.snapkv_batch(wl.with_(seed=wl.seed + 100 * l)) for l in range(NL)]
    qn, kn, vn = (np.stack([x[i] for x in layers]) for i in range(3))
    res = _run(*(par.to_device(x, "bf16") for x in (qn, kn, vn)), wl.window, wl.budget, wl.pool_kernel,
               kvc.SNAPKV_AUTO)
    assert kvc.snapkv_last_score_kernel() == "snap_wave_bf16"
    idx, ko, vo, vote, pooled = _host(res)
    for l in range(NL):
        for b, h in ((0, 0), (1, 31), (l % 2, 7 + l)):
            _check_head(qn[l, b, h], kn[l, b, h], vn[l, b, h], wl.L, wl.budget, wl.pool_kernel, "bf16", "max",
                        idx[l, b, h], ko[l, b, h], vo[l, b, h], vote[l, b, h], pooled[l, b, h])


def test_ex_error_statuses():
    k = torch.zeros((2, 2, 512, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kvc.KvcError) as e:  # a length not above the budget
        kvc.snapkv_compress_ex(k, k, k, 32, 300, 7, lengths=[512, 300])
    assert e.value.status == kvc.KVC_ERR_INVALID_ARG
    with pytest.raises(kvc.KvcError) as e:  # a length beyond L
        kvc.snapkv_compress_ex(k, k, k, 32, 300, 7, lengths=[513, 400])
    assert e.value.status == kvc.KVC_ERR_INVALID_ARG
    lib = kvc.library()
    assert lib.kvc_snapkv_workspace_bytes_ex(0, 1, 1, 512, 128, 32, 300, 7, kvc.KVC_BF16, 0) == 0
    st = lib.kvc_snapkv_compress_ex(None, 512, kvc.Strides(0, 0, 0), 0, None, None, kvc.Strides(0, 0, 0), 0, 1, 1,
                                    1, 512, 128, None, 32, 300, 7, 5, kvc.KVC_BF16, None, None, None, None, None,
                                    None, 0, None)
    assert st == kvc.KVC_ERR_INVALID_ARG
