#!/usr/bin/env python3
"""Benchmark of the KV-selection hot path on one MI355X.

Default run (N = 1 GPU):
  * SnapKV compression of one 131K-token layer (B1 H32 D128 L131072, window 32,
    budget 2048, max-pool 7, bf16): a step is one full kvc_snapkv_compress call
    (window scores, softmax normalisers, vote, pool, top-k, gather) over inputs
    already resident in HBM. value = prompt tokens compressed per second.
  * The other SnapKV layers (tiny fp32, 16K batch 2, 380K) are timed the same
    way and reported under "workloads", each with its own roofline.
  * Consecutive steps rotate over enough device copies of K and V that a step
    never finds the previous step's K in the 256 MB infinity cache (MALL).
  * The timed steps of a layer come after its warmup steps and its untimed
    instrumented passes (kernel and phase events), so that they run at the
    clocks the GPU holds under sustained load.
  * The H2O + StreamingLLM decode loop of an OPT-6.7B-shaped layer (B64 H32
    D128, 2048-token prompt then 2048 decode steps, budget len//10 heavy +
    len//10 recent, sink 4 + recent 1020 ring) is measured as a second object.
  * The CPU oracle is timed on bounded samples of the same workloads.

Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12  # MI355X HBM3E, bytes/s
PHASES = ["zero", "stats", "merge", "votes", "select", "gather"]
# the same boundaries under the single-pass schedule: the preparation kernel,
# the score kernel, (nothing), pooling + histogram, then the shared phases
PHASES_SINGLE = ["prep", "score", "none", "pool", "select", "gather"]
SCHEDULES = {"auto": 0, "two-pass": 1, "single-pass": 2}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="131k-bf16")
    ap.add_argument("--schedule", choices=sorted(SCHEDULES), default="auto",
                    help="SnapKV score schedule (auto: single pass where it can run)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU-oracle sample")
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--skip-h2o", action="store_true")
    ap.add_argument("--h2o-steps", type=int, default=2048, help="timed decode steps (<= 2048)")
    ap.add_argument("--skip-extra", action="store_true", help="only the 131K layer (no tiny / 16K / 380K lines)")
    ap.add_argument("--extra-steps", type=int, default=10, help="timed steps of each extra SnapKV layer")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    return ap.parse_args()


class HipEvents:
    """hipEvent_t handles from libamdhip64 (timing on the library's stream)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(h)) == 0
            arr[i] = h
        return arr

    def record(self, ev, stream):
        assert self.hip.hipEventRecord(ev, stream) == 0

    def ms(self, a, b):
        out = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), a, b) == 0
        return out.value


def source_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "kv_cache_compression_02_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, sources):
    """Per-launch HBM bytes of `kernel` from the committed counter summary, if the
    kernel source has not changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_digest:\s*([0-9a-f]+)", text)
    b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not b or m.group(1) != source_digest(*sources):
        return None
    return float(b.group(1))


def snapkv_bytes(wl):
    """Algorithmic HBM bytes of one compression: K read once, the window queries,
    the kept K/V rows read and written, the kept indices."""
    es = 2 if wl.dtype == "bf16" else 4
    BH = wl.B * wl.H
    k_read = BH * wl.L * wl.D * es
    q_read = BH * wl.window * wl.D * es
    gather = 4 * BH * wl.budget * wl.D * es
    idx = 4 * BH * (wl.budget - wl.window)
    # a score kernel's share: K once and the window queries (votes and row
    # statistics are workspace and not counted); the two-pass vote pass reads
    # the prefix keys again
    return dict(total=k_read + q_read + gather + idx, stats=k_read + q_read,
                votes=BH * (wl.L - wl.window) * wl.D * es + q_read,
                score=k_read + q_read, gather=gather + idx)


MALL_BYTES = 256 << 20


def n_copies(wl):
    """Device copies of K and V the timed steps rotate over: enough that at least twice the MALL's
    256 MB of other keys is read between two reads of one copy."""
    es = 2 if wl.dtype == "bf16" else 4
    k_bytes = wl.B * wl.H * wl.L * wl.D * es
    return 1 + -(-2 * MALL_BYTES // k_bytes)


def put_host(x, dtype):
    import numpy as np
    import torch

    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def bench_snapkv(wl, args, ev, steps, warmup, detail=True, keep_host=False):
    """Time kvc_snapkv_compress on one layer: after `warmup` calls, `steps` calls with events around
    the score kernel(s) only (the dominant kernel's launch time), with `detail` the same calls again
    with every phase boundary marked (both untimed for the step), then `steps` calls back to back
    with no events in the stream (the step time)."""
    import torch

    import kv_cache_compression_02_amd as kvc
    import synthetic as syn

    log(f"generating {wl.name}: B{wl.B} H{wl.H} D{wl.D} L{wl.L} w{wl.window} C{wl.budget} p{wl.pool_kernel}")
    t = time.time()
    qn, kn, vn = syn.snapkv_batch(wl)
    log(f"generated in {time.time() - t:.1f}s")
    ncp = n_copies(wl)
    q = put_host(qn, wl.dtype)
    k0, v0 = put_host(kn, wl.dtype), put_host(vn, wl.dtype)
    if not keep_host:
        del kn, vn
        kn = vn = None
    ks, vs = [k0], [v0]
    for _ in range(ncp - 1):
        ks.append(k0.clone())
        vs.append(v0.clone())
    log(f"{ncp} device copies of K and V ({ncp * 2 * k0.numel() * k0.element_size() / 2**30:.2f} GiB)")
    B, H, L, D = k0.shape
    out = kvc.SnapKVResult(torch.empty((B, H, wl.budget, D), dtype=k0.dtype, device="cuda"),
                           torch.empty((B, H, wl.budget, D), dtype=k0.dtype, device="cuda"),
                           torch.empty((B, H, wl.budget - wl.window), dtype=torch.int32, device="cuda"),
                           None, None)
    ws = torch.empty(kvc.snapkv_workspace_bytes(B, H, L, D, wl.window, wl.budget, wl.pool_kernel, k0.dtype),
                     dtype=torch.uint8, device="cuda")
    lib = kvc.library()
    n_ev = len(PHASES) + 1

    # one prepared call per K/V copy: arguments checked and marshalled once, each call enqueues the
    # whole compression (kvc_snapkv_compress) as snapkv_compress would
    prepared = [kvc.SnapKVCall(q, ks[c], vs[c], wl.window, wl.budget, wl.pool_kernel, workspace=ws, out=out)
                for c in range(ncp)]

    def call(i):
        prepared[i % ncp]()

    def set_events(arr):
        lib.kvc_snapkv_set_phase_events(ctypes.cast(arr, ctypes.c_void_p) if arr is not None else None,
                                        n_ev if arr is not None else 0)

    lib.kvc_snapkv_set_schedule(SCHEDULES[args.schedule])
    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    single = kvc.snapkv_last_schedule() == kvc.SNAPKV_SINGLE_PASS
    score_kernel = kvc.snapkv_last_score_kernel()
    pool_kernel = kvc.snapkv_last_pool_kernel()
    # the per-head selection kernel pools and counts itself: no pooling kernel between marks 3 and 4
    fused_pool = single and pool_kernel in ("snap_select_head", "snap_select")
    phases = PHASES_SINGLE if single else PHASES
    if fused_pool:
        phases = [("none_pool" if p == "pool" else p) for p in phases]
    passes = ("score", "pool") if single else ("stats", "votes")
    log(f"schedule: {'single pass' if single else 'two passes'} ({score_kernel}; pooling in {pool_kernel})")
    # Untimed instrumented passes first (the timed steps then start with the
    # GPU at the clocks it holds under sustained load, as in a serving loop:
    # the first ~10 ms of work after an idle period run a few percent slower).
    # The steps with events around the score passes only (boundaries 1 to 4):
    # 1 -> 2 is the statistics pass or the single score kernel, 3 -> 4 the
    # vote pass or the pooling kernel.
    timed = [ev.create(4) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        arr = (ctypes.c_void_p * n_ev)()
        arr[1], arr[2], arr[3], arr[4] = timed[i]
        set_events(arr)
        call(i)
    torch.cuda.synchronize()
    set_events(None)
    kern_ms = {passes[0]: sum(ev.ms(e[0], e[1]) for e in timed) / steps,
               passes[1]: sum(ev.ms(e[2], e[3]) for e in timed) / steps}
    if fused_pool:
        del kern_ms["pool"]
    phase_ms = None
    if detail:
        # every phase boundary, for the breakdown only
        events = [ev.create(n_ev) for _ in range(steps)]
        for i in range(steps):
            set_events(events[i])
            call(i)
        torch.cuda.synchronize()
        set_events(None)
        phase_ms = {p: sum(ev.ms(e[j], e[j + 1]) for e in events) / steps for j, p in enumerate(phases)}
        # (single pass: nothing runs between marks 2 and 3, nor between 3 and 4 where the
        # selection pools; such an interval is the events' own cost)
        phase_ms.pop("none", None)
        phase_ms.pop("none_pool", None)
    # Timed region: the steps back to back with no events in the stream (a
    # recorded event between two kernels costs the GPU several microseconds).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        call(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    lib.kvc_snapkv_set_schedule(0)
    step_ms = elapsed / steps * 1e3
    nbytes = snapkv_bytes(wl)
    dominant = "score" if single else max(("stats", "votes"), key=lambda p: kern_ms[p])
    dom_bytes = nbytes[dominant]
    achieved = dom_bytes / (kern_ms[dominant] * 1e-3)
    suffix = "bf16" if wl.dtype == "bf16" else "f32"
    kernel_name = score_kernel if single else f"snap_{dominant}_{suffix}"
    traffic = load_traffic(kernel_name, ["snapkv.hip", "common.hpp"])
    log(f"{wl.name}: step {step_ms:.4f} ms, {nbytes['total'] / (step_ms * 1e-3) / PEAK_HBM:.3f} of HBM peak; "
        f"{kernel_name} {kern_ms[dominant] * 1e3:.1f} us" +
        ("; phases (ms): " + ", ".join(f"{p} {v:.4f}" for p, v in phase_ms.items()) if phase_ms else ""))
    res = dict(
        wl=wl, step_ms=step_ms, elapsed=elapsed, steps=steps, copies=ncp,
        value=B * L * steps / elapsed,
        path_gbps=nbytes["total"] / (step_ms * 1e-3) / 1e9,
        roofline={"bound": "hbm", "achieved": achieved / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                  "frac": achieved / PEAK_HBM, "traffic": traffic, "kernel": kernel_name,
                  "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_ms": kern_ms[dominant],
                  "score_pass_ms": kern_ms},
        phase_ms=phase_ms, alg_bytes=nbytes["total"], schedule="single-pass" if single else "two-pass",
        pool_kernel=pool_kernel,
        host=(qn, kn, vn) if keep_host else None)
    if detail:
        # decode attention over the compressed cache, rotated over enough copies of it (K' and V')
        # that the calls do not re-read it from the L2 / MALL
        res["decode_attention"] = time_decode(
            kvc, ev, q[:, :, -1].contiguous(), out.k, out.v, wl.budget, 200,
            f"SnapKV-compressed {wl.name} layer B{B} H{H} {wl.budget} rows")
    del ks, vs, q, out, ws
    torch.cuda.empty_cache()
    return res


def workload_line(res):
    """The JSON object of one SnapKV layer."""
    wl = res["wl"]
    return {
        "config": {"workload": f"snapkv-{wl.name}", "batch": wl.B, "heads": wl.H, "head_dim": wl.D,
                   "prompt_len": wl.L, "window": wl.window, "budget": wl.budget, "pool_kernel": wl.pool_kernel,
                   "dtype": wl.dtype, "schedule": res["schedule"]},
        "value": res["value"], "unit": "tokens/s", "ms_per_step": res["step_ms"], "steps": res["steps"],
        "kv_copies_rotated": res["copies"],
        "hbm_gbps_path": res["path_gbps"], "hbm_frac_path": res["path_gbps"] * 1e9 / PEAK_HBM,
        "algorithmic_bytes_per_step": res["alg_bytes"], "roofline": res["roofline"],
        "pooling_kernel": res["pool_kernel"],
    }


def blas_threads():
    try:
        import threadpoolctl

        return max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()), default=1)
    except Exception:  # threadpoolctl missing: report the affinity only
        return None


def cpu_snapkv(wl, seconds, host=None, threads=None):
    """The oracle on a bounded sample of a SnapKV layer: whole heads, in order, cycling over the
    layer until `seconds` have passed; scaled to one layer. `threads` caps the BLAS threads."""
    import contextlib

    import synthetic as syn
    from oracle import snapkv as ref

    ctx = contextlib.nullcontext()
    if threads is not None:
        import threadpoolctl

        ctx = threadpoolctl.threadpool_limits(limits=threads)
    heads = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    done = 0
    with ctx:
        used = blas_threads()
        t0 = time.perf_counter()
        while True:
            b, h = heads[done % len(heads)]
            if host is not None:
                qh, kh, vh = host[0][b, h], host[1][b, h], host[2][b, h]
            else:
                tg = time.perf_counter()
                qh, kh, vh = syn.snapkv_head(wl, b, h)
                t0 += time.perf_counter() - tg  # generation is not the oracle's time
            ref.compress_head(qh, kh, vh, wl.budget, wl.pool_kernel, wl.dtype)
            done += 1
            if time.perf_counter() - t0 > seconds:
                break
        t = time.perf_counter() - t0
    full_layer_s = t * len(heads) / done
    cores = len(os.sched_getaffinity(0))
    log(f"cpu oracle {wl.name}: {done} head compressions ({done / len(heads):.2f} layers) in {t:.1f}s, "
        f"{used} BLAS threads")
    return {"value": wl.B * wl.L / full_layer_s, "unit": "tokens/s", "cores": used or cores, "kind": "oracle",
            "affinity_cores": cores,
            "sample": f"{done} whole-head compressions cycling over the {len(heads)} heads of the {wl.name} "
                      f"layer (fp64 numpy, {used} BLAS threads), {t:.1f}s; scaled to one layer"}


def cpu_h2o(seconds, n_heads=4, steps=256):
    """The H2O oracle on a sample of the decode workload: `n_heads` heads from their own prompt
    prefill, then up to `steps` decode steps each (bounded by `seconds`); per-step time scaled to
    all B x H heads. Labelled per step: the sample covers the first decode steps only."""
    import numpy as np

    import synthetic as syn
    from oracle import h2o as ref

    wl = syn.H2O_WORKLOADS["opt6.7b-decode"]
    Lp = wl.prompt_len
    heads = [(b, (7 * b) % wl.H) for b in range(0, wl.B, wl.B // n_heads)][:n_heads]
    used = blas_threads()
    t_pf = 0.0
    states = {}
    for b, h in heads:
        q, k, v, _ = syn.h2o_prompt_head(wl, b, h)
        t = time.perf_counter()
        states[(b, h)], _ = ref.prefill_head(q, k, v, wl.n_heavy(Lp), wl.n_recent(Lp), wl.dtype)
        t_pf += time.perf_counter() - t
    t_steps, done = 0.0, 0
    for s_ in range(steps):
        x = syn.h2o_step_inputs(wl, s_)
        length = Lp + s_ + 1
        t = time.perf_counter()
        for b, h in heads:
            states[(b, h)], _, _ = ref.step_head(states[(b, h)], x[0][b, h], x[1][b, h], x[2][b, h], length,
                                                 wl.n_heavy(length), wl.n_recent(length), wl.dtype)
        t_steps += time.perf_counter() - t
        done += 1
        if t_steps + t_pf > seconds:
            break
    per_step_all = t_steps / done * (wl.B * wl.H) / len(heads)
    log(f"cpu oracle h2o: {len(heads)} heads, prefill {t_pf:.1f}s, {done} steps {t_steps:.2f}s")
    return {"value": wl.B / per_step_all, "unit": "decode tokens/s (per step)", "cores": used,
            "kind": "oracle", "prefill_s_all_heads": t_pf * wl.B * wl.H / len(heads),
            "sample": f"{len(heads)} of the {wl.B * wl.H} heads of {wl.name}: the oracle's prompt prefill, then the "
                      f"first {done} decode steps; per-step time scaled to all heads (per step, not the whole "
                      f"2048-step loop)"}


def time_decode(kvc, ev, q, k, v, n, reps, label):
    """kvc_decode_attention over the first n rows of k/v: average time of `reps` back-to-back
    calls bracketed by two events on the library's stream, and its HBM roofline (K and V rows
    read once, q read, the fp32 output written). The calls rotate over enough copies of the
    cache that at least twice the MALL's 256 MB of other rows is read between two reads of one
    copy, so that the figure is an HBM one even for a small (compressed) cache."""
    import torch

    B, H, _, D = k.shape
    es = k.element_size()
    cache_bytes = 2 * B * H * n * D * es
    ncp = 1 + -(-2 * MALL_BYTES // cache_bytes)
    ks = [k] + [k[:, :, :n].clone() for _ in range(ncp - 1)]
    vs = [v] + [v[:, :, :n].clone() for _ in range(ncp - 1)]
    ws = torch.empty(max(kvc.decode_attention_workspace_bytes(B, H, n, D), 16), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
    for i in range(3):
        kvc.decode_attention(q, ks[i % ncp], vs[i % ncp], n, workspace=ws, out=out)
    torch.cuda.synchronize()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    e = ev.create(2)
    ev.record(e[0], stream)
    for i in range(reps):
        kvc.decode_attention(q, ks[i % ncp], vs[i % ncp], n, workspace=ws, out=out)
    ev.record(e[1], stream)
    torch.cuda.synchronize()
    ms = ev.ms(e[0], e[1]) / reps
    nbytes = B * H * (2 * n * D * es + D * es + D * 4)
    gbps = nbytes / (ms * 1e-3) / 1e9
    log(f"decode attention, {label}: {ms * 1e3:.1f} us per call, {gbps:.0f} GB/s ({ncp} cache copies rotated)")
    del ks, vs
    return {"cache": label, "ms_per_call": ms, "calls": reps, "algorithmic_bytes": nbytes,
            "cache_copies_rotated": ncp,
            "roofline": {"bound": "hbm", "achieved": gbps, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                         "frac": gbps * 1e9 / PEAK_HBM, "kernel": "decode_partial + decode_merge"}}


def bench_h2o(args, ev):
    import numpy as np
    import torch

    import kv_cache_compression_02_amd as kvc
    import synthetic as syn

    wl = syn.H2O_WORKLOADS["opt6.7b-decode"]
    B, H, D, Lp = wl.B, wl.H, wl.D, wl.prompt_len
    steps = min(args.h2o_steps, wl.steps)
    log(f"h2o: generating the {B}x{H} prompt of {Lp} tokens")
    prompt = np.empty((3, B, H, Lp, D), np.uint16)
    for b in range(B):
        for h in range(H):
            q_, k_, v_, _ = syn.h2o_prompt_head(wl, b, h)
            prompt[0, b, h], prompt[1, b, h], prompt[2, b, h] = q_, k_, v_
    pdev = torch.from_numpy(prompt.view(np.int16)).view(torch.bfloat16).cuda()
    del prompt
    # decode-step inputs drawn on the GPU (seeded; same N(0,1) law as the host generator)
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.seed)
    dec = torch.randn((steps, 3, B, H, D), generator=g, device="cuda").to(torch.bfloat16)
    cache = kvc.H2OCache(B, H, D, wl.cap)
    sink = kvc.SinkCache(B, H, D, wl.n_sink, wl.sink_recent)
    torch.cuda.synchronize()
    t_pf = time.perf_counter()
    cache.prefill(pdev[0], pdev[1], pdev[2], wl.n_heavy(Lp), wl.n_recent(Lp))
    torch.cuda.synchronize()
    prefill_ms = (time.perf_counter() - t_pf) * 1e3
    log(f"h2o: prompt prefill {prefill_ms:.2f} ms; filling the sink ring with the prompt (untimed)")
    for t in range(Lp):
        sink.append(pdev[1, :, :, t].contiguous(), pdev[2, :, :, t].contiguous())
    torch.cuda.synchronize()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    evs = ev.create(3 * steps)
    ns = []
    t0 = time.perf_counter()
    for s in range(steps):
        length = Lp + s + 1
        ns.append(cache.n + 1)
        ev.record(evs[3 * s], stream)
        cache.step(dec[s, 0], dec[s, 1], dec[s, 2], wl.n_heavy(length), wl.n_recent(length))
        ev.record(evs[3 * s + 1], stream)
        sink.append(dec[s, 1], dec[s, 2])
        ev.record(evs[3 * s + 2], stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    h2o_ms = [ev.ms(evs[3 * s], evs[3 * s + 1]) for s in range(steps)]
    sink_ms = [ev.ms(evs[3 * s + 1], evs[3 * s + 2]) for s in range(steps)]
    es = 2
    # per (b,h): N rows of K (D*es), score read+write (8 B) and position read (4 B), plus q,
    # new k/v read and written (5 rows)
    step_bytes = [B * H * (N * (D * es + 12) + 5 * D * es) for N in ns]
    kern_s = sum(h2o_ms) * 1e-3
    achieved = sum(step_bytes) / kern_s
    # decode attention (the generation step over the policies' caches) with the last step's queries
    q_last = dec[steps - 1, 0]
    dec_att = [time_decode(kvc, ev, q_last, sink.k, sink.v, min(sink.length, wl.n_sink + wl.sink_recent), 20,
                           f"sink + recent ring B{B} H{H} {wl.n_sink}+{wl.sink_recent} slots"),
               time_decode(kvc, ev, q_last, cache.k, cache.v, cache.n, 20,
                           f"H2O cache B{B} H{H} {cache.n} slots")]
    return {
        "workload": f"{wl.name}: B{B} H{H} D{D}, prompt {Lp} (GPU prompt-score prefill, untimed) then "
                    f"{steps} decode steps, "
                    f"budget len//10 heavy + len//10 recent, sink {wl.n_sink} + recent {wl.sink_recent}",
        "decode_tokens_per_s": B * steps / elapsed,
        "ms_per_step_wall": elapsed / steps * 1e3,
        "h2o_step_ms": kern_s / steps * 1e3,
        "sink_step_ms": sum(sink_ms) / steps,
        "decode_tokens_per_s_kernels": B * steps / (kern_s + sum(sink_ms) * 1e-3),
        "roofline": {"bound": "hbm", "achieved": achieved / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM, "traffic": load_traffic("h2o_step_kernel", ["h2o.hip", "common.hpp"]),
                     "kernel": "h2o_step_kernel", "algorithmic_bytes_per_launch": sum(step_bytes) / steps,
                     "avg_launch_ms": kern_s / steps * 1e3},
        "prefill_ms": prefill_ms,
        "decode_attention": dec_att,
        "inputs": "prompt from the seeded host generator; decode q/k/v drawn on the GPU with a seeded "
                  "torch generator (N(0,1), bf16)",
    }


def stream_peak(ev):
    """What this GPU streams over a 1 GiB buffer (4x the MALL): a torch device copy (bytes read plus
    bytes written; the stream-copy peak), and the library's plain streaming-read kernel
    (kvc_measure_stream_read: bytes read; the best of a few workgroups-per-CU settings), each
    over 10 launches bracketed by events on the stream they run on."""
    import torch

    import kv_cache_compression_02_amd as kvc

    n = 1 << 30
    a = torch.empty(n // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    lib = kvc.library()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def read(per_cu):
        st = lib.kvc_measure_stream_read(ctypes.c_void_p(a.data_ptr()), n, per_cu, ctypes.c_void_p(sink.data_ptr()),
                                         stream)
        assert st == 0, lib.kvc_last_error().decode()

    def timed(fn, reps=10):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e = ev.create(2)
        ev.record(e[0], stream)
        for _ in range(reps):
            fn()
        ev.record(e[1], stream)
        torch.cuda.synchronize()
        return ev.ms(e[0], e[1]) / reps * 1e-3

    out = {"copy_gbps": 2 * n / timed(lambda: b.copy_(a)) / 1e9}
    reads = {per_cu: n / timed(lambda: read(per_cu)) / 1e9 for per_cu in (2, 4, 8, 16)}
    best = max(reads, key=reads.get)
    out["read_gbps"] = reads[best]
    out["read_gbps_by_workgroups_per_cu"] = reads
    del a, b
    torch.cuda.empty_cache()
    out["bytes"] = n
    out["kernels"] = ("torch copy_ (read + write counted); kvc_measure_stream_read (plain 16-byte nontemporal "
                      "loads, grid-stride, 4 in flight per thread; read only), 10 launches each")
    return out


def calibrate_copy():
    import torch

    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n, "launches": 3}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (the path shards over "
              "(batch, head) with no exchange; run one process per GPU)", file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    if args.calibrate_copy:
        calibrate_copy()
        return
    ev = HipEvents()
    import synthetic as syn

    wl = syn.SNAPKV_WORKLOADS[args.workload]
    res = bench_snapkv(wl, args, ev, args.steps, args.warmup, detail=True, keep_host=not args.skip_cpu)
    line = {
        "metric": "prompt tokens compressed/s per layer (all heads); HBM GB/s as % of peak",
        "value": res["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": f"snapkv-{wl.name}", "batch": wl.B, "heads": wl.H, "head_dim": wl.D,
                   "prompt_len": wl.L, "window": wl.window, "budget": wl.budget,
                   "pool_kernel": wl.pool_kernel, "schedule": res["schedule"]},
        "hbm_gbps_path": res["path_gbps"],
        "hbm_frac_path": res["path_gbps"] * 1e9 / PEAK_HBM,
        "algorithmic_bytes_per_step": res["alg_bytes"],
        "kv_copies_rotated": res["copies"],
        "roofline": res["roofline"],
        "phase_ms": res["phase_ms"],
        "pooling_kernel": res["pool_kernel"],
        "decode_attention_compressed": res["decode_attention"],
    }
    sp = stream_peak(ev)
    sp["score_kernel_frac_of_read"] = res["roofline"]["achieved"] / sp["read_gbps"]
    sp["path_frac_of_read"] = res["path_gbps"] / sp["read_gbps"]
    line["measured_stream"] = sp
    log(f"stream peak: copy {sp['copy_gbps']:.0f} GB/s, read {sp['read_gbps']:.0f} GB/s")
    host = res.pop("host")
    extra = {}
    if not args.skip_extra:
        for name in ("tiny-fp32", "16k-bf16", "380k-bf16"):
            if name == wl.name:
                continue
            r = bench_snapkv(syn.SNAPKV_WORKLOADS[name], args, ev, args.extra_steps, 2, detail=False,
                             keep_host=not args.skip_cpu and name != "380k-bf16")
            extra[name] = r
        line["workloads"] = {n: workload_line(r) for n, r in extra.items()}
    if not args.skip_cpu:
        line["cpu_baseline"] = cpu_snapkv(wl, args.cpu_seconds, host)
        cpu = {}
        short = min(args.cpu_seconds, 6.0)
        for name, r in extra.items():
            cpu[name] = cpu_snapkv(r["wl"], short, r["host"])
            if name in ("tiny-fp32", "16k-bf16"):
                cpu[name + " (1 thread)"] = cpu_snapkv(r["wl"], short, r["host"], threads=1)
        if not args.skip_h2o:
            cpu["opt6.7b-decode"] = cpu_h2o(short)
        line["cpu_baselines"] = cpu
    else:
        line["cpu_baseline"] = None
    del res, host, extra
    if not args.skip_h2o:
        line["h2o_sink"] = bench_h2o(args, ev)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
