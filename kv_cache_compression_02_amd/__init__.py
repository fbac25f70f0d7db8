"""kvc: attention-score-guided KV-cache selection and compaction on AMD MI355X.

Python binding of ``libkvc.so`` (the HIP kernels behind the C ABI declared in
``include/kvc.h``). This module only marshals arguments: it takes torch device
tensors, passes their pointers, strides and the current HIP stream to the
library, and allocates outputs and workspaces with torch. Every step of the
computation runs in the library's kernels. There is no CPU fallback: when the
library is missing or a call fails, an exception is raised.

Entry points (same names as the C ABI, without the ``kvc_`` prefix):
  snapkv_compress     SnapKV prompt compression of one layer
  snapkv_workspace_bytes
  H2OCache.prefill    H2O prompt scores + first eviction (kvc_h2o_prefill)
  H2OCache.step       H2O decode step (kvc_h2o_step)
  SinkCache.append    StreamingLLM sink + recent ring (kvc_sink_recent)
"""
import contextlib
import ctypes
import os
from collections import namedtuple

import torch

__all__ = [
    "KvcError", "library", "library_path", "snapkv_workspace_bytes", "snapkv_compress",
    "SnapKVResult", "H2OCache", "SinkCache", "KVC_F32", "KVC_BF16", "EXPORTED_SYMBOLS", "KVC_POOL_MAX",
    "KVC_POOL_AVG", "snapkv_workspace_bytes_ex", "snapkv_compress_ex", "snapkv_status_offset",
    "snapkv_last_pool_kernel", "SnapKVCall",
    "SNAPKV_AUTO", "SNAPKV_TWO_PASS", "SNAPKV_SINGLE_PASS", "snapkv_schedule", "snapkv_last_schedule",
    "decode_attention_workspace_bytes", "decode_attention", "decode_attention_noalloc",
]

KVC_OK, KVC_ERR_INVALID_ARG, KVC_ERR_UNSUPPORTED, KVC_ERR_WORKSPACE, KVC_ERR_HIP = range(5)
KVC_F32, KVC_BF16 = 0, 1
KVC_POOL_MAX, KVC_POOL_AVG = 0, 1
_POOLS = {"max": KVC_POOL_MAX, "avg": KVC_POOL_AVG}
SNAPKV_AUTO, SNAPKV_TWO_PASS, SNAPKV_SINGLE_PASS = 0, 1, 2
_STATUS_NAMES = {1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "WORKSPACE", 4: "HIP"}

EXPORTED_SYMBOLS = (
    "kvc_last_error", "kvc_version", "kvc_snapkv_workspace_bytes", "kvc_snapkv_compress",
    "kvc_h2o_step", "kvc_sink_recent", "kvc_snapkv_set_phase_events", "kvc_h2o_prefill",
    "kvc_h2o_prefill_workspace_bytes", "kvc_snapkv_set_schedule", "kvc_snapkv_last_schedule",
    "kvc_snapkv_last_score_kernel", "kvc_snapkv_force_residency_fallback", "kvc_snapkv_force_wait_timeout",
    "kvc_snapkv_force_split_select", "kvc_snapkv_last_select_kernel",
    "kvc_decode_attention_workspace_bytes", "kvc_decode_attention", "kvc_measure_stream_read",
    "kvc_decode_attention_noalloc", "kvc_snapkv_workspace_bytes_ex", "kvc_snapkv_compress_ex",
    "kvc_sink_cache_positions", "kvc_snapkv_status_offset", "kvc_snapkv_last_pool_kernel",
)

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path():
    return os.path.join(_HERE, "libkvc.so")


class KvcError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"kvc {_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class Strides(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("h", ctypes.c_int64), ("t", ctypes.c_int64)]


class _H2OCacheC(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("pos", ctypes.c_void_p),
        ("acc", ctypes.c_void_p), ("B", ctypes.c_int), ("H", ctypes.c_int), ("D", ctypes.c_int),
        ("cap", ctypes.c_int), ("n", ctypes.c_int), ("len", ctypes.c_int64), ("dt", ctypes.c_int),
    ]


_lib = None


def library():
    """Load libkvc.so (built in-tree by ``python -m kv_cache_compression_02_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with python -m kv_cache_compression_02_amd.build")
    L = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    L.kvc_last_error.restype = ctypes.c_char_p
    L.kvc_last_error.argtypes = []
    L.kvc_version.restype = i32
    L.kvc_version.argtypes = []
    L.kvc_snapkv_workspace_bytes.restype = sz
    L.kvc_snapkv_workspace_bytes.argtypes = [i32] * 7 + [i32]
    L.kvc_snapkv_compress.restype = i32
    L.kvc_snapkv_compress.argtypes = [
        vp, i32, Strides, vp, vp, Strides, i32, i32, i32, i32, i32, i32, i32, i32,
        vp, vp, vp, vp, vp, vp, sz, vp]
    L.kvc_snapkv_workspace_bytes_ex.restype = sz
    L.kvc_snapkv_workspace_bytes_ex.argtypes = [i32] * 8 + [i32, i32]
    L.kvc_snapkv_compress_ex.restype = i32
    L.kvc_snapkv_compress_ex.argtypes = [
        vp, i32, Strides, i64, vp, vp, Strides, i64, i32, i32, i32, i32, i32, vp, i32, i32, i32, i32, i32,
        vp, vp, vp, vp, vp, vp, sz, vp]
    L.kvc_h2o_step.restype = i32
    L.kvc_h2o_step.argtypes = [ctypes.POINTER(_H2OCacheC), vp, vp, vp, i32, i32, vp, vp]
    L.kvc_h2o_prefill_workspace_bytes.restype = sz
    L.kvc_h2o_prefill_workspace_bytes.argtypes = [i32, i32, i32]
    L.kvc_h2o_prefill.restype = i32
    L.kvc_h2o_prefill.argtypes = [ctypes.POINTER(_H2OCacheC), vp, Strides, vp, vp, Strides, i32, i32, i32,
                                  vp, sz, vp]
    L.kvc_snapkv_set_phase_events.restype = None
    L.kvc_snapkv_set_phase_events.argtypes = [vp, i32]
    L.kvc_decode_attention_workspace_bytes.restype = sz
    L.kvc_decode_attention_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.kvc_decode_attention.restype = i32
    L.kvc_decode_attention.argtypes = [vp, Strides, vp, vp, Strides, i32, i32, i32, i32, i32, vp, vp, sz, vp]
    L.kvc_snapkv_set_schedule.restype = i32
    L.kvc_snapkv_set_schedule.argtypes = [i32]
    L.kvc_snapkv_last_schedule.restype = i32
    L.kvc_snapkv_last_schedule.argtypes = []
    L.kvc_snapkv_last_score_kernel.restype = ctypes.c_char_p
    L.kvc_snapkv_last_score_kernel.argtypes = []
    L.kvc_snapkv_force_split_select.restype = i32
    L.kvc_snapkv_force_split_select.argtypes = [i32]
    L.kvc_snapkv_last_select_kernel.restype = ctypes.c_char_p
    L.kvc_snapkv_last_select_kernel.argtypes = []
    L.kvc_snapkv_status_offset.restype = i64
    L.kvc_snapkv_last_pool_kernel.restype = ctypes.c_char_p
    L.kvc_snapkv_last_pool_kernel.argtypes = []
    L.kvc_snapkv_status_offset.argtypes = [i32] * 7 + [i32]
    L.kvc_decode_attention_noalloc.restype = i32
    L.kvc_decode_attention_noalloc.argtypes = [vp, Strides, vp, vp, Strides, i32, i32, i32, i32, i32, vp, vp]
    L.kvc_measure_stream_read.restype = i32
    L.kvc_measure_stream_read.argtypes = [vp, sz, i32, vp, vp]
    L.kvc_sink_cache_positions.restype = i32
    L.kvc_sink_cache_positions.argtypes = [vp, i64, i32, i32, vp, vp]
    L.kvc_sink_recent.restype = i32
    L.kvc_sink_recent.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, i32, i32, vp, vp]
    _lib = L
    return L


def _check(status):
    if status != KVC_OK:
        raise KvcError(status, library().kvc_last_error().decode())


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return KVC_BF16
    if t.dtype == torch.float32:
        return KVC_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.bfloat16 or torch.float32")


def _dev(t, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if t.stride(-1) != 1:
        raise ValueError(f"{name}: the last (head_dim) axis must be contiguous")
    return t


def _check_out(t, name, shape, dtype, device):
    """A caller-supplied output: contiguous, of the documented shape and dtype, on the inputs' device."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the inputs on {device}")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} of shape {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _strides4(t):
    return Strides(t.stride(0), t.stride(1), t.stride(2))


def snapkv_workspace_bytes(B, H, L, D, window, budget, pool_kernel, dtype):
    code = KVC_BF16 if dtype == torch.bfloat16 else KVC_F32
    return int(library().kvc_snapkv_workspace_bytes(B, H, L, D, window, budget, pool_kernel, code))


def snapkv_status_offset(B, H, L, D, window, budget, pool_kernel, dtype):
    """Byte offset of the single pass's three status words in a workspace of
    snapkv_workspace_bytes(...) bytes, -1 if that layout has none (testing)."""
    code = KVC_BF16 if dtype == torch.bfloat16 else KVC_F32
    return int(library().kvc_snapkv_status_offset(B, H, L, D, window, budget, pool_kernel, code))


SnapKVResult = namedtuple("SnapKVResult", "k v idx pooled vote")


@contextlib.contextmanager
def snapkv_schedule(schedule):
    """Run the enclosed snapkv_compress calls (this thread) under ``schedule``
    (SNAPKV_AUTO, SNAPKV_TWO_PASS or SNAPKV_SINGLE_PASS; kvc_snapkv_set_schedule)."""
    prev = library().kvc_snapkv_set_schedule(int(schedule))
    if prev < 0:
        raise ValueError(f"unknown SnapKV schedule {schedule!r}")
    try:
        yield
    finally:
        library().kvc_snapkv_set_schedule(prev)


def snapkv_last_schedule():
    """Schedule the last successful snapkv_compress call on this thread ran (0 if none)."""
    return int(library().kvc_snapkv_last_schedule())


def snapkv_last_score_kernel():
    """Kernel name(s) that computed the scores in the last successful snapkv_compress call."""
    return library().kvc_snapkv_last_score_kernel().decode()


def snapkv_last_select_kernel():
    """Selection kernel the last snapkv_compress call launched."""
    return library().kvc_snapkv_last_select_kernel().decode()


def snapkv_last_pool_kernel():
    """Kernel that pooled the votes and counted their histogram in the last snapkv_compress call."""
    return library().kvc_snapkv_last_pool_kernel().decode()


def _snapkv_args(q, k, v, window, budget, pool_kernel, want_pooled, want_vote, workspace, out):
    """Checks and marshals one kvc_snapkv_compress call: returns (arguments, SnapKVResult)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n)
        if t.dim() != 4:
            raise ValueError(f"{n} must be 4-D [B, H, T, D]")
    if k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("k and v must have the same shape and strides")
    if q.dtype != k.dtype or v.dtype != k.dtype:
        raise TypeError("q, k, v must share one dtype")
    B, H, L, D = k.shape
    dt = _dtype_code(k)
    dev = k.device
    if q.device != dev or v.device != dev:
        raise ValueError("q, k, v must be on one device")
    if (q.shape[0], q.shape[1], q.shape[3]) != (B, H, D):
        raise ValueError(f"q must be [B, H, q_len, D] = [{B}, {H}, *, {D}], got {tuple(q.shape)}")
    if q.shape[2] < window:
        raise ValueError(f"q holds {q.shape[2]} rows, fewer than the window {window}")
    n_keep, n_pre = max(budget - window, 0), max(L - window, 0)
    if out is None:
        k_out = torch.empty((B, H, budget, D), dtype=k.dtype, device=dev)
        v_out = torch.empty_like(k_out)
        idx = torch.empty((B, H, n_keep), dtype=torch.int32, device=dev)
        pooled = torch.empty((B, H, n_pre), dtype=torch.float32, device=dev) if want_pooled else None
        vote = torch.empty((B, H, n_pre), dtype=torch.float32, device=dev) if want_vote else None
    else:
        k_out, v_out, idx, pooled, vote = out
        _check_out(k_out, "out.k", (B, H, budget, D), k.dtype, dev)
        _check_out(v_out, "out.v", (B, H, budget, D), k.dtype, dev)
        _check_out(idx, "out.idx", (B, H, n_keep), torch.int32, dev)
        if pooled is not None:
            _check_out(pooled, "out.pooled", (B, H, n_pre), torch.float32, dev)
        if vote is not None:
            _check_out(vote, "out.vote", (B, H, n_pre), torch.float32, dev)
    if workspace is not None:
        _check_out(workspace, "workspace", (workspace.numel(),), torch.uint8, dev)
    if workspace is None:
        nbytes = snapkv_workspace_bytes(B, H, L, D, window, budget, pool_kernel, k.dtype)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    args = (_ptr(q), q.shape[2], _strides4(q), _ptr(k), _ptr(v), _strides4(k), B, H, L, D,
            window, budget, pool_kernel, dt, _ptr(k_out), _ptr(v_out), _ptr(idx), _ptr(pooled),
            _ptr(vote), _ptr(workspace), workspace.numel(), _stream())
    # the tensors stay referenced by the result (and the workspace by the caller or the call object)
    return args, SnapKVResult(k_out, v_out, idx, pooled, vote), workspace


def snapkv_compress(q, k, v, window, budget, pool_kernel, *, want_pooled=False, want_vote=False,
                    workspace=None, out=None):
    """SnapKV compression of one layer (kvc_snapkv_compress).

    q: [B, H, q_len, D] (last ``window`` rows used); k, v: [B, H, L, D] with the same
    strides; bf16 or fp32 on the GPU. Returns SnapKVResult(k [B,H,budget,D],
    v [B,H,budget,D], idx int32 [B,H,budget-window], pooled, vote) where pooled/vote
    are float32 [B,H,L-window] or None. ``workspace`` (uint8 tensor) and ``out``
    (a SnapKVResult of preallocated tensors) may be passed to avoid allocations.
    """
    args, res, _ = _snapkv_args(q, k, v, window, budget, pool_kernel, want_pooled, want_vote, workspace, out)
    _check(library().kvc_snapkv_compress(*args))
    return res


class SnapKVCall:
    """One kvc_snapkv_compress call with its arguments checked and marshalled once, for loops that
    compress into the same buffers again and again: calling the object enqueues the compression
    (the same kernels as snapkv_compress) on the stream that was current when it was made, and
    returns its SnapKVResult. The tensors must stay where they are between calls; their contents
    may change."""

    def __init__(self, q, k, v, window, budget, pool_kernel, *, want_pooled=False, want_vote=False,
                 workspace=None, out=None):
        self._args, self.result, self._ws = _snapkv_args(q, k, v, window, budget, pool_kernel, want_pooled,
                                                         want_vote, workspace, out)
        self._inputs = (q, k, v)
        self._fn = library().kvc_snapkv_compress

    def __call__(self):
        st = self._fn(*self._args)
        if st != KVC_OK:
            raise KvcError(st, library().kvc_last_error().decode())
        return self.result


def snapkv_workspace_bytes_ex(n_layers, B, H, L, D, window, budget, pool_kernel, dtype, ragged=False):
    code = KVC_BF16 if dtype == torch.bfloat16 else KVC_F32
    return int(library().kvc_snapkv_workspace_bytes_ex(n_layers, B, H, L, D, window, budget, pool_kernel, code,
                                                       int(bool(ragged))))


def snapkv_compress_ex(q, k, v, window, budget, pool_kernel, *, pool="max", lengths=None, want_pooled=False,
                       want_vote=False, workspace=None, out=None):
    """kvc_snapkv_compress_ex: the pooling operator ("max" or "avg"), all layers of a prompt in one call and
    ragged batches.

    q: [B, H, q_len, D] or [n_layers, B, H, q_len, D] (the last ``window`` rows of each sequence's q are its
    window queries); k, v: [B, H, L, D] or [n_layers, B, H, L, D] with the same strides. ``lengths``: optional
    sequence of B prompt lengths (budget < length <= L). Returns SnapKVResult with k, v [n_layers, B, H,
    budget, D], idx [n_layers, B, H, budget - window] (the layer axis dropped for 4-D inputs) and pooled /
    vote float32: [n_layers, B, H, L - window] without lengths, else packed 1-D (per layer, per sequence,
    H rows of lengths[b] - window).
    """
    if pool not in _POOLS:
        raise ValueError(f"pool must be one of {sorted(_POOLS)}")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n)
    layered = k.dim() == 5
    if q.dim() != k.dim() or k.dim() not in (4, 5):
        raise ValueError("q, k, v must all be 4-D [B, H, T, D] or all 5-D [n_layers, B, H, T, D]")
    if k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("k and v must have the same shape and strides")
    if q.dtype != k.dtype or v.dtype != k.dtype:
        raise TypeError("q, k, v must share one dtype")
    if q.device != k.device or v.device != k.device:
        raise ValueError("q, k, v must be on one device")
    q5, k5 = (q, k) if layered else (q.unsqueeze(0), k.unsqueeze(0))
    NL, B, H, L, D = k5.shape
    if (q5.shape[0], q5.shape[1], q5.shape[2], q5.shape[4]) != (NL, B, H, D):
        raise ValueError(f"q must be [{NL}, {B}, {H}, *, {D}] like k, got {tuple(q.shape)}")
    if q5.shape[3] < window:
        raise ValueError(f"q holds {q5.shape[3]} rows, fewer than the window {window}")
    dt = _dtype_code(k)
    dev = k.device
    lens = None
    if lengths is not None:
        lengths = [int(x) for x in lengths]
        if len(lengths) != B:
            raise ValueError(f"lengths must hold {B} values")
        lens = (ctypes.c_int32 * B)(*lengths)
        n_pre = NL * H * sum(max(x - window, 0) for x in lengths)
        pv_shape = (n_pre,)
    else:
        pv_shape = (NL, B, H, max(L - window, 0)) if layered else (B, H, max(L - window, 0))
    lead = (NL, B, H) if layered else (B, H)
    n_keep = max(budget - window, 0)
    if out is None:
        k_out = torch.empty(lead + (budget, D), dtype=k.dtype, device=dev)
        v_out = torch.empty_like(k_out)
        idx = torch.empty(lead + (n_keep,), dtype=torch.int32, device=dev)
        pooled = torch.empty(pv_shape, dtype=torch.float32, device=dev) if want_pooled else None
        vote = torch.empty(pv_shape, dtype=torch.float32, device=dev) if want_vote else None
    else:
        k_out, v_out, idx, pooled, vote = out
        _check_out(k_out, "out.k", lead + (budget, D), k.dtype, dev)
        _check_out(v_out, "out.v", lead + (budget, D), k.dtype, dev)
        _check_out(idx, "out.idx", lead + (n_keep,), torch.int32, dev)
        if pooled is not None:
            _check_out(pooled, "out.pooled", pv_shape, torch.float32, dev)
        if vote is not None:
            _check_out(vote, "out.vote", pv_shape, torch.float32, dev)
    if workspace is None:
        nbytes = snapkv_workspace_bytes_ex(NL, B, H, L, D, window, budget, pool_kernel, k.dtype, lens is not None)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    else:
        _check_out(workspace, "workspace", (workspace.numel(),), torch.uint8, dev)
    qs = Strides(q5.stride(1), q5.stride(2), q5.stride(3))
    ks = Strides(k5.stride(1), k5.stride(2), k5.stride(3))
    _check(library().kvc_snapkv_compress_ex(
        _ptr(q), q5.shape[3], qs, q5.stride(0), _ptr(k), _ptr(v), ks, k5.stride(0), NL, B, H, L, D,
        ctypes.cast(lens, ctypes.c_void_p) if lens is not None else None, window, budget, pool_kernel, _POOLS[pool],
        dt, _ptr(k_out), _ptr(v_out), _ptr(idx), _ptr(pooled), _ptr(vote), _ptr(workspace), workspace.numel(),
        _stream()))
    return SnapKVResult(k_out, v_out, idx, pooled, vote)


def decode_attention_workspace_bytes(B, H, n, D):
    return int(library().kvc_decode_attention_workspace_bytes(B, H, n, D))


def decode_attention(q, k, v, n=None, *, workspace=None, out=None):
    """Attention of one query per head over the first ``n`` cached rows (kvc_decode_attention).

    q: [B, H, D]; k, v: [B, H, N, D] with the same strides (D contiguous), bf16 or fp32 on
    the GPU; ``n`` defaults to N. Returns float32 [B, H, D] (``out`` if given, contiguous).
    """
    _dev(q, "q"), _dev(k, "k"), _dev(v, "v")
    if q.dim() != 3 or k.dim() != 4:
        raise ValueError("q must be [B, H, D] and k, v [B, H, N, D]")
    if k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("k and v must have the same shape and strides")
    if q.dtype != k.dtype or v.dtype != k.dtype:
        raise TypeError("q, k, v must share one dtype")
    B, H, N, D = k.shape
    if tuple(q.shape) != (B, H, D):
        raise ValueError("q must be [B, H, D] matching k")
    n = N if n is None else int(n)
    if n > N:  # (n < 1 is the library's INVALID_ARG)
        raise ValueError(f"n = {n} exceeds the {N} rows of k and v")
    if q.device != k.device or v.device != k.device:
        raise ValueError("q, k, v must be on one device")
    if out is None:
        out = torch.empty((B, H, D), dtype=torch.float32, device=k.device)
    else:
        _check_out(out, "out", (B, H, D), torch.float32, k.device)
    if workspace is None:
        nbytes = decode_attention_workspace_bytes(B, H, n, D)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=k.device)
    _check(library().kvc_decode_attention(
        _ptr(q), Strides(q.stride(0), q.stride(1), 0), _ptr(k), _ptr(v), _strides4(k), B, H, n, D,
        _dtype_code(k), _ptr(out), _ptr(workspace), workspace.numel(), _stream()))
    return out


def decode_attention_noalloc(q, k, v, n, out):
    """decode_attention without a workspace (kvc_decode_attention_noalloc): the library's static
    scratch holds the partials, so neither this call nor the library allocates; ``out`` (float32
    [B, H, D], contiguous) is the caller's. Overlapping calls on one GPU race on that scratch."""
    _dev(q, "q"), _dev(k, "k"), _dev(v, "v")
    if q.dim() != 3 or k.dim() != 4:
        raise ValueError("q must be [B, H, D] and k, v [B, H, N, D]")
    if k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("k and v must have the same shape and strides")
    if q.dtype != k.dtype or v.dtype != k.dtype:
        raise TypeError("q, k, v must share one dtype")
    B, H, N, D = k.shape
    if tuple(q.shape) != (B, H, D) or q.device != k.device or v.device != k.device:
        raise ValueError("q must be [B, H, D] matching k, on k's device")
    if int(n) > N:
        raise ValueError(f"n = {n} exceeds the {N} rows of k and v")
    _check_out(out, "out", (B, H, D), torch.float32, k.device)
    _check(library().kvc_decode_attention_noalloc(
        _ptr(q), Strides(q.stride(0), q.stride(1), 0), _ptr(k), _ptr(v), _strides4(k), B, H, int(n), D,
        _dtype_code(k), _ptr(out), _stream()))
    return out


class H2OCache:
    """Device-resident H2O cache of one layer (kvc_h2o_cache) and its step call."""

    def __init__(self, B, H, D, cap, dtype=torch.bfloat16, device="cuda"):
        self.k = torch.zeros((B, H, cap, D), dtype=dtype, device=device)
        self.v = torch.zeros_like(self.k)
        self.pos = torch.full((B, H, cap), -1, dtype=torch.int32, device=device)
        self.acc = torch.zeros((B, H, cap), dtype=torch.float32, device=device)
        self._c = _H2OCacheC(self.k.data_ptr(), self.v.data_ptr(), self.pos.data_ptr(),
                             self.acc.data_ptr(), B, H, D, cap, 0, 0, _dtype_code(self.k))

    @property
    def n(self):
        return self._c.n

    @property
    def length(self):
        return self._c.len

    def prefill(self, q, k, v, n_heavy, n_recent, workspace=None):
        """Initial state from a prompt (kvc_h2o_prefill); q, k, v: [B, H, prompt_len, D]."""
        for t, n in ((q, "q"), (k, "k"), (v, "v")):
            _dev(t, n)
            if t.dim() != 4 or t.dtype != self.k.dtype:
                raise ValueError(f"{n} must be 4-D [B, H, T, D] with the cache's dtype")
        if k.shape != v.shape or k.stride() != v.stride() or q.shape != k.shape:
            raise ValueError("q, k, v must share one shape, and k, v one set of strides")
        B, H, Lp, D = k.shape
        if (B, H, D) != (self.k.shape[0], self.k.shape[1], self.k.shape[3]) or k.device != self.k.device:
            raise ValueError(f"prompt [B, H, *, D] = {tuple(k.shape)} does not match the cache "
                             f"{tuple(self.k.shape)} on {self.k.device}")
        if workspace is None:
            nbytes = int(library().kvc_h2o_prefill_workspace_bytes(B, H, Lp))
            workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=k.device)
        _check(library().kvc_h2o_prefill(ctypes.byref(self._c), _ptr(q), _strides4(q), _ptr(k), _ptr(v),
                                         _strides4(k), Lp, n_heavy, n_recent, _ptr(workspace),
                                         workspace.numel(), _stream()))

    def step(self, q, k_new, v_new, n_heavy, n_recent, attn_out=None):
        """One decode step for every head; q, k_new, v_new: [B, H, D] contiguous."""
        B, H, _, D = self.k.shape
        for t, n in ((q, "q"), (k_new, "k_new"), (v_new, "v_new")):
            _dev(t, n)
            if not t.is_contiguous() or t.dtype != self.k.dtype:
                raise ValueError(f"{n} must be contiguous with the cache's dtype")
            _check_out(t, n, (B, H, D), self.k.dtype, self.k.device)
        if attn_out is not None:
            _check_out(attn_out, "attn_out", (B, H, D), torch.float32, self.k.device)
        _check(library().kvc_h2o_step(ctypes.byref(self._c), _ptr(q), _ptr(k_new), _ptr(v_new),
                                      n_heavy, n_recent, _ptr(attn_out), _stream()))
        return attn_out


class SinkCache:
    """StreamingLLM sink + recent ring of one layer (kvc_sink_recent)."""

    def __init__(self, B, H, D, n_sink, n_recent, dtype=torch.bfloat16, device="cuda"):
        self.B, self.H, self.D = B, H, D
        self.n_sink, self.n_recent = n_sink, n_recent
        slots = n_sink + n_recent
        self.k = torch.zeros((B, H, slots, D), dtype=dtype, device=device)
        self.v = torch.zeros_like(self.k)
        self.slot_pos = torch.full((slots,), -1, dtype=torch.int32, device=device)
        self.kept = torch.empty((slots,), dtype=torch.int32, device=device)
        self.length = 0

    def append(self, k_new, v_new):
        """Write one new token ([B, H, D] contiguous); return the held positions, ascending."""
        for t, n in ((k_new, "k_new"), (v_new, "v_new")):
            _dev(t, n)
            _check_out(t, n, (self.B, self.H, self.D), self.k.dtype, self.k.device)
        self.length += 1
        n_kept = min(self.length, self.n_sink + self.n_recent)
        _check(library().kvc_sink_recent(
            _ptr(self.k), _ptr(self.v), _ptr(self.slot_pos), _ptr(k_new), _ptr(v_new),
            self.length, self.n_sink, self.n_recent, self.B, self.H, self.D,
            _dtype_code(self.k), _ptr(self.kept), _stream()))
        return self.kept[:n_kept]

    def cache_positions(self, out=None):
        """Position inside the cache of each slot's token ([n_sink + n_recent] int32, -1 for an empty slot;
        kvc_sink_cache_positions): the positions a positional encoding would give the cached keys."""
        if self.length < 1:
            raise ValueError("the cache holds no token yet")
        slots = self.n_sink + self.n_recent
        if out is None:
            out = torch.empty((slots,), dtype=torch.int32, device=self.k.device)
        else:
            _check_out(out, "out", (slots,), torch.int32, self.k.device)
        _check(library().kvc_sink_cache_positions(_ptr(self.slot_pos), self.length, self.n_sink, self.n_recent,
                                                  _ptr(out), _stream()))
        return out
