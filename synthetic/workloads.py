"""Named synthetic workloads shaped like the pages' experiments.

SnapKV workloads (one attention layer, multi-head, keys/values [B,H,L,D]):

  tiny-fp32      B1  H4  D64  L512     w16 C128  p5  fp32, 3 spans x 4 tokens, boost 2.0
  16k-bf16       B2  H32 D128 L16384   w32 C1024 p7  bf16, 20 spans x 8 tokens, boost 1.5,
                                                        first 4 keys +3.0 (sink-like)
  131k-bf16      B1  H32 D128 L131072  w32 C2048 p7  bf16, 64 spans x 8 tokens,
                                                        boost 1.5*z, z ~ Zipf(1.1) on 1..64, sinks
  380k-bf16      B1  H32 D128 L380000  w32 C1024 p7  bf16, one 16-token needle at a depth
                                                        uniform in [0.05, 0.95], boost 1.5*z, sinks

H2O / StreamingLLM decode workload:

  opt6.7b-decode B64 H32 D128, 2048-token prompt, 2048 decode steps, bf16; 5% of prompt
                 keys carry a persistent +1.5 bias on every element; per-step q/k/v ~ N(0,1);
                 budget = len//10 heavy hitters + len//10 recent; sink 4 + recent 1020 ring.

The shapes follow the SnapKV summary page (section on experiments: the 16K,
batch-2 speed test, the 131K batch-2 memory test, the 380K needle test with a
1024-token prompt KV) and the H2O summary page (section on system performance:
OPT-6.7B, 2048 prompt + 2048 generated tokens, 20% heavy hitters). The public
datasets those pages measure on are not used: these generators stand in for
them by shape only.

A boost adds ``magnitude * u_hat`` to every key of a span, where ``u_hat`` is the
unit vector along the mean of that head's window queries (after bf16 rounding),
so the window queries attend to the span more than to the Gaussian background.
"""
from dataclasses import dataclass, replace

import numpy as np

from .bf16 import f32_to_bf16_bits, bf16_bits_to_f32


@dataclass(frozen=True)
class SnapKVWorkload:
    name: str
    B: int
    H: int
    D: int
    L: int
    window: int
    budget: int
    pool_kernel: int
    dtype: str            # "fp32" or "bf16"
    n_spans: int
    span_len: int
    span_boost: float     # constant magnitude, or the base multiplying z
    zipf_a: float = 0.0   # > 0: magnitude = span_boost * z, z ~ Zipf(zipf_a) on 1..zipf_max
    zipf_max: int = 64
    sink_boost: float = 0.0
    n_sink_boost: int = 4
    needle_depth: tuple = ()  # (lo, hi): single span starting at depth U[lo, hi] * L
    seed: int = 0

    def with_(self, **kw):
        return replace(self, **kw)

    @property
    def prefix_len(self):
        return self.L - self.window

    @property
    def n_keep_prefix(self):
        return self.budget - self.window


@dataclass(frozen=True)
class H2OWorkload:
    name: str
    B: int
    H: int
    D: int
    prompt_len: int
    steps: int
    heavy_div: int = 10   # n_heavy = len // heavy_div
    recent_div: int = 10  # n_recent = len // recent_div
    bias_frac: float = 0.05
    bias: float = 1.5
    n_sink: int = 4
    sink_recent: int = 1020
    dtype: str = "bf16"
    seed: int = 0

    def with_(self, **kw):
        return replace(self, **kw)

    def n_heavy(self, length):
        return length // self.heavy_div

    def n_recent(self, length):
        return length // self.recent_div

    @property
    def cap(self):
        # Largest cache the loop ever holds: the budget at the final length plus
        # the token appended before eviction.
        final = self.prompt_len + self.steps
        return self.n_heavy(final) + self.n_recent(final) + 1


SNAPKV_WORKLOADS = {
    "tiny-fp32": SnapKVWorkload(
        name="tiny-fp32", B=1, H=4, D=64, L=512, window=16, budget=128, pool_kernel=5,
        dtype="fp32", n_spans=3, span_len=4, span_boost=2.0, seed=20261),
    "16k-bf16": SnapKVWorkload(
        name="16k-bf16", B=2, H=32, D=128, L=16384, window=32, budget=1024, pool_kernel=7,
        dtype="bf16", n_spans=20, span_len=8, span_boost=1.5, sink_boost=3.0, seed=20262),
    "131k-bf16": SnapKVWorkload(
        name="131k-bf16", B=1, H=32, D=128, L=131072, window=32, budget=2048, pool_kernel=7,
        dtype="bf16", n_spans=64, span_len=8, span_boost=1.5, zipf_a=1.1, sink_boost=3.0,
        seed=20263),
    "380k-bf16": SnapKVWorkload(
        name="380k-bf16", B=1, H=32, D=128, L=380000, window=32, budget=1024, pool_kernel=7,
        dtype="bf16", n_spans=1, span_len=16, span_boost=1.5, zipf_a=1.1, sink_boost=3.0,
        needle_depth=(0.05, 0.95), seed=20265),
}

H2O_WORKLOADS = {
    "opt6.7b-decode": H2OWorkload(
        name="opt6.7b-decode", B=64, H=32, D=128, prompt_len=2048, steps=2048, seed=20264),
}


def _rng(seed, *key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=seed, spawn_key=key)))


def _encode(x32, dtype):
    if dtype == "fp32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    return f32_to_bf16_bits(x32)


def _decode(arr, dtype):
    if dtype == "fp32":
        return arr.astype(np.float32)
    return bf16_bits_to_f32(arr)


def _zipf_truncated(rng, n, a, zmax):
    z = np.arange(1, zmax + 1, dtype=np.float64)
    pmf = z ** (-a)
    pmf /= pmf.sum()
    return rng.choice(z, size=n, p=pmf)


def snapkv_head(wl: SnapKVWorkload, b: int, h: int):
    """Window queries [w,D], keys [L,D], values [L,D] of head (b, h).

    Returns float32 arrays for an fp32 workload, uint16 bfloat16 bits otherwise.
    Draw order: window queries, keys, values, span starts, span magnitudes.
    """
    rng = _rng(wl.seed, 0, b, h)
    w, D, L = wl.window, wl.D, wl.L
    q32 = rng.standard_normal((w, D), dtype=np.float32)
    k32 = rng.standard_normal((L, D), dtype=np.float32)
    v32 = rng.standard_normal((L, D), dtype=np.float32)
    q = _encode(q32, wl.dtype)

    hi = L - w - wl.span_len
    if wl.needle_depth:
        lo_d, hi_d = wl.needle_depth
        depth = rng.uniform(lo_d, hi_d, size=wl.n_spans)
        starts = np.clip((depth * L).astype(np.int64), 0, hi)
    else:
        starts = rng.integers(0, hi + 1, size=wl.n_spans)
    if wl.zipf_a > 0:
        mags = wl.span_boost * _zipf_truncated(rng, wl.n_spans, wl.zipf_a, wl.zipf_max)
    else:
        mags = np.full(wl.n_spans, wl.span_boost)

    u = _decode(q, wl.dtype).astype(np.float64).mean(axis=0)
    u_hat = (u / np.linalg.norm(u)).astype(np.float32)
    for s0, m in zip(starts, mags):
        k32[s0:s0 + wl.span_len] += np.float32(m) * u_hat
    if wl.sink_boost:
        k32[:wl.n_sink_boost] += np.float32(wl.sink_boost) * u_hat

    return q, _encode(k32, wl.dtype), _encode(v32, wl.dtype)


def snapkv_spans(wl: SnapKVWorkload, b: int, h: int):
    """Start positions of the planted spans of head (b, h) (same draws as snapkv_head)."""
    rng = _rng(wl.seed, 0, b, h)
    w, D, L = wl.window, wl.D, wl.L
    rng.standard_normal((w, D), dtype=np.float32)
    rng.standard_normal((L, D), dtype=np.float32)
    rng.standard_normal((L, D), dtype=np.float32)
    hi = L - w - wl.span_len
    if wl.needle_depth:
        depth = rng.uniform(*wl.needle_depth, size=wl.n_spans)
        return np.clip((depth * L).astype(np.int64), 0, hi)
    return rng.integers(0, hi + 1, size=wl.n_spans)


def snapkv_batch(wl: SnapKVWorkload):
    """Whole-layer inputs: q [B,H,w,D], k and v [B,H,L,D] (float32 or uint16 bf16 bits)."""
    dt = np.float32 if wl.dtype == "fp32" else np.uint16
    q = np.empty((wl.B, wl.H, wl.window, wl.D), dt)
    k = np.empty((wl.B, wl.H, wl.L, wl.D), dt)
    v = np.empty((wl.B, wl.H, wl.L, wl.D), dt)
    for b in range(wl.B):
        for h in range(wl.H):
            q[b, h], k[b, h], v[b, h] = snapkv_head(wl, b, h)
    return q, k, v


def h2o_prompt_head(wl: H2OWorkload, b: int, h: int):
    """Prompt queries, keys, values [Lp, D] of head (b, h), plus the biased key positions.

    Draw order: q, k, v, then the biased positions (chosen without replacement).
    The bias adds ``wl.bias`` to every element of those keys.
    """
    rng = _rng(wl.seed, 0, b, h)
    Lp, D = wl.prompt_len, wl.D
    q32 = rng.standard_normal((Lp, D), dtype=np.float32)
    k32 = rng.standard_normal((Lp, D), dtype=np.float32)
    v32 = rng.standard_normal((Lp, D), dtype=np.float32)
    biased = np.sort(rng.choice(Lp, size=int(wl.bias_frac * Lp), replace=False))
    k32[biased] += np.float32(wl.bias)
    return _encode(q32, wl.dtype), _encode(k32, wl.dtype), _encode(v32, wl.dtype), biased


def h2o_prompt_batch(wl: H2OWorkload):
    """Prompt q, k, v [B,H,Lp,D] for every head."""
    dt = np.float32 if wl.dtype == "fp32" else np.uint16
    shape = (wl.B, wl.H, wl.prompt_len, wl.D)
    q, k, v = np.empty(shape, dt), np.empty(shape, dt), np.empty(shape, dt)
    for b in range(wl.B):
        for h in range(wl.H):
            q[b, h], k[b, h], v[b, h], _ = h2o_prompt_head(wl, b, h)
    return q, k, v


def h2o_step_inputs(wl: H2OWorkload, step: int):
    """Fresh decode-step q, k, v [B,H,D] for generated token ``step`` (0-based)."""
    rng = _rng(wl.seed, 1, step)
    shape = (wl.B, wl.H, wl.D)
    out = [rng.standard_normal(shape, dtype=np.float32) for _ in range(3)]
    return tuple(_encode(x, wl.dtype) for x in out)
