"""GPU parity of kvc_decode_attention (through the C ABI) against the CPU oracle."""
import numpy as np
import pytest
import torch

import kv_cache_compression_02_amd as kvc
import synthetic as syn
from oracle import attention as ref
from oracle import sink as sink_ref
from oracle import snapkv as snap_ref
from tests import parity as par

pytestmark = pytest.mark.gpu


def _rand(shape, seed, dtype):
    x = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    return syn.f32_to_bf16_bits(x) if dtype == "bf16" else x


def _expect(qh, kh, vh, dtype):
    """Oracle output of one head and the tolerance scale sum_j p_j |v_j|."""
    qf, kf, vf = (snap_ref.to_f64(x, dtype) for x in (qh, kh, vh))
    p = ref.softmax(ref.scores(qf, kf))
    return p @ vf, p @ np.abs(vf)


def _check(qn, kn, vn, n, dtype, got, heads=None, what="o"):
    B, H, D = qn.shape
    got = got.cpu().numpy()
    pairs = heads or [(b, h) for b in range(B) for h in range(H)]
    for b, h in pairs:
        o, scale = _expect(qn[b, h], kn[b, h, :n, :D], vn[b, h, :n, :D], dtype)
        par.assert_close_votes(got[b, h], o, f"{what}[{b},{h}]", scale=scale)


CASES = [
    # B, H, N (rows held), n (rows attended), D, dtype
    (1, 4, 1, 1, 64, "bf16"),        # a single row
    (1, 4, 7, 7, 128, "bf16"),       # fewer rows than one wave load
    (2, 3, 300, 300, 128, "bf16"),   # two chunks, ragged tail
    (2, 3, 600, 513, 128, "bf16"),   # n < rows held
    (1, 4, 256, 256, 64, "bf16"),    # exactly one chunk
    (2, 2, 1000, 1000, 64, "fp32"),
    (1, 3, 257, 257, 128, "fp32"),   # one row into the second chunk
    (1, 2, 5000, 4999, 128, "fp32"),
    (16, 32, 700, 700, 128, "bf16"),   # enough heads for 256-row chunks, ragged
    (16, 32, 700, 650, 64, "fp32"),
]


@pytest.mark.parametrize("B,H,N,n,D,dtype", CASES)
def test_random_shapes(B, H, N, n, D, dtype):
    print(f"[decode] B{B} H{H} N{N} n{n} D{D} {dtype}", flush=True)
    qn, kn, vn = _rand((B, H, D), 1 + N, dtype), _rand((B, H, N, D), 2 + N, dtype), _rand((B, H, N, D), 3 + N, dtype)
    q, k, v = (par.to_device(x, dtype) for x in (qn, kn, vn))
    _check(qn, kn, vn, n, dtype, kvc.decode_attention(q, k, v, n))


def test_strided_rows_and_garbage_workspace():
    """K/V views into wider padded rows, q a view, and a garbage-filled workspace."""
    B, H, N, D = 2, 3, 700, 128
    qn = _rand((B, H, 2 * D), 11, "bf16")
    kn, vn = _rand((B, H, N, D + 64), 12, "bf16"), _rand((B, H, N, D + 64), 13, "bf16")
    qd, kd, vd = (par.to_device(x, "bf16") for x in (qn, kn, vn))
    q, k, v = qd[..., :D], kd[..., :D], vd[..., :D]
    ws = torch.full((kvc.decode_attention_workspace_bytes(B, H, N, D),), 0x5A, dtype=torch.uint8, device="cuda")
    got = kvc.decode_attention(q, k, v, workspace=ws)
    _check(np.ascontiguousarray(qn[..., :D]), kn, vn, N, "bf16", got)


def test_peaked_and_flat_attention():
    """Q = 0 (every weight equal: the mean of V) and one key far ahead of the rest."""
    B, H, N, D = 1, 2, 900, 128
    kn, vn = _rand((B, H, N, D), 21, "bf16"), _rand((B, H, N, D), 22, "bf16")
    qn = np.zeros((B, H, D), np.uint16)
    q, k, v = (par.to_device(x, "bf16") for x in (qn, kn, vn))
    got = kvc.decode_attention(q, k, v).cpu().numpy()
    mean = syn.bf16_bits_to_f32(vn).astype(np.float64).mean(2)
    np.testing.assert_allclose(got, mean, rtol=0, atol=1e-5)
    # a planted key: its weight dominates
    q32 = np.random.default_rng(23).standard_normal((B, H, D), dtype=np.float32)
    k32 = syn.bf16_bits_to_f32(kn).copy()
    k32[0, 1, 777] = 4.0 * q32[0, 1] / np.linalg.norm(q32[0, 1]) * np.sqrt(D)
    qn2, kn2 = syn.f32_to_bf16_bits(q32), syn.f32_to_bf16_bits(k32)
    q2, k2 = par.to_device(qn2, "bf16"), par.to_device(kn2, "bf16")
    _check(qn2, kn2, vn, N, "bf16", kvc.decode_attention(q2, k2, v))


def test_over_snapkv_compressed_cache():
    """The generation step after compression: attend over kvc_snapkv_compress's K', V'."""
    wl = syn.SNAPKV_WORKLOADS["16k-bf16"].with_(L=6000, H=4)
    qn, kn, vn = syn.snapkv_batch(wl)
    q, k, v = (par.to_device(x, "bf16") for x in (qn, kn, vn))
    res = kvc.snapkv_compress(q, k, v, wl.window, wl.budget, wl.pool_kernel)
    qd = _rand((wl.B, wl.H, wl.D), 31, "bf16")
    got = kvc.decode_attention(par.to_device(qd, "bf16"), res.k, res.v).cpu().numpy()
    # the oracle attends over its own compressed rows; where its kept set equals the
    # GPU's (the rows are then the same, bit for bit) the outputs must agree
    idx = res.idx.cpu().numpy()
    compared = 0
    for b in range(wl.B):
        for h in range(wl.H):
            r = snap_ref.compress_head(qn[b, h, -wl.window:], kn[b, h], vn[b, h], wl.budget, wl.pool_kernel, "bf16")
            if np.array_equal(r["idx"], idx[b, h]):
                o, scale = _expect(qd[b, h], r["k_out"], r["v_out"], "bf16")
                par.assert_close_votes(got[b, h], o, f"o[{b},{h}]", scale=scale)
                compared += 1
    assert compared >= (wl.B * wl.H * 3) // 4, compared


def test_over_sink_ring():
    """A StreamingLLM step: attend over the sink + recent ring (slots in ring order)."""
    B, H, D, s, r = 2, 3, 128, 4, 60
    cache = kvc.SinkCache(B, H, D, s, r)
    rows_k, rows_v = [], []
    for t in range(150):
        kt, vt = _rand((B, H, D), 100 + t, "bf16"), _rand((B, H, D), 400 + t, "bf16")
        rows_k.append(kt)
        rows_v.append(vt)
        cache.append(par.to_device(kt, "bf16"), par.to_device(vt, "bf16"))
        if t in (2, 63, 64, 149):
            n = min(t + 1, s + r)
            qd = _rand((B, H, D), 700 + t, "bf16")
            got = kvc.decode_attention(par.to_device(qd, "bf16"), cache.k, cache.v, n).cpu().numpy()
            kept = sink_ref.kept_positions(t + 1, s, r)
            for b in range(B):
                for h in range(H):
                    kk = np.stack([rows_k[p][b, h] for p in kept])
                    vv = np.stack([rows_v[p][b, h] for p in kept])
                    o, scale = _expect(qd[b, h], kk, vv, "bf16")
                    par.assert_close_votes(got[b, h], o, f"ring t{t} [{b},{h}]", scale=scale)


def test_decode_shapes_sampled():
    """The two shapes the bench times: the 131K layer's compacted cache and the decode layer's ring."""
    for B, H, N in ((1, 32, 2048), (64, 32, 1024)):
        print(f"[decode] B{B} H{H} N{N}", flush=True)
        qn, kn, vn = _rand((B, H, 128), 41 + B, "bf16"), _rand((B, H, N, 128), 42 + B, "bf16"), \
            _rand((B, H, N, 128), 43 + B, "bf16")
        got = kvc.decode_attention(*(par.to_device(x, "bf16") for x in (qn, kn, vn)))
        heads = [(0, 0), (0, H - 1), (B - 1, 7)]
        _check(qn, kn, vn, N, "bf16", got, heads=heads)


def test_error_statuses():
    q = torch.zeros((1, 2, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 2, 300, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kvc.KvcError) as e:
        kvc.decode_attention(q, k, k, 0)
    assert e.value.status == kvc.KVC_ERR_INVALID_ARG
    with pytest.raises(kvc.KvcError) as e:
        kvc.decode_attention(q, k, k, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert e.value.status == kvc.KVC_ERR_WORKSPACE
