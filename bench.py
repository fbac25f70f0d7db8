#!/usr/bin/env python3
"""Benchmark of the KV-selection hot path on one MI355X.

Default run (N = 1 GPU):
  * SnapKV compression of one 131K-token layer (B1 H32 D128 L131072, window 32,
    budget 2048, max-pool 7, bf16): a step is one full kvc_snapkv_compress call
    (window scores, two-pass softmax, vote, pool, top-k, gather) over inputs
    already resident in HBM. value = prompt tokens compressed per second.
  * The H2O + StreamingLLM decode loop of an OPT-6.7B-shaped layer (B64 H32
    D128, 2048-token prompt then 2048 decode steps, budget len//10 heavy +
    len//10 recent, sink 4 + recent 1020 ring) is measured as a second object.
  * The CPU oracle is timed on a bounded sample of the same SnapKV workload.

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
    votes_out = 4 * BH * (wl.L - wl.window)
    return dict(total=k_read + q_read + gather + idx, stats=k_read + q_read,
                votes=BH * (wl.L - wl.window) * wl.D * es + q_read,
                score=k_read + q_read + votes_out, gather=gather + idx)


def bench_snapkv(args, ev):
    import numpy as np
    import torch

    import kv_cache_compression_02_amd as kvc
    import synthetic as syn

    wl = syn.SNAPKV_WORKLOADS[args.workload]
    log(f"generating {wl.name}: B{wl.B} H{wl.H} D{wl.D} L{wl.L} w{wl.window} C{wl.budget} p{wl.pool_kernel}")
    t = time.time()
    qn, kn, vn = syn.snapkv_batch(wl)
    log(f"generated in {time.time() - t:.1f}s")

    def put(x):
        if wl.dtype == "bf16":
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()

    q, k, v = put(qn), put(kn), put(vn)
    B, H, L, D = k.shape
    out = kvc.SnapKVResult(torch.empty((B, H, wl.budget, D), dtype=k.dtype, device="cuda"),
                           torch.empty((B, H, wl.budget, D), dtype=k.dtype, device="cuda"),
                           torch.empty((B, H, wl.budget - wl.window), dtype=torch.int32, device="cuda"),
                           None, None)
    ws = torch.empty(kvc.snapkv_workspace_bytes(B, H, L, D, wl.window, wl.budget, wl.pool_kernel, k.dtype),
                     dtype=torch.uint8, device="cuda")
    lib = kvc.library()
    n_ev = len(PHASES) + 1

    def call():
        kvc.snapkv_compress(q, k, v, wl.window, wl.budget, wl.pool_kernel, workspace=ws, out=out)

    def set_events(arr):
        lib.kvc_snapkv_set_phase_events(ctypes.cast(arr, ctypes.c_void_p) if arr is not None else None,
                                        n_ev if arr is not None else 0)

    lib.kvc_snapkv_set_schedule(SCHEDULES[args.schedule])
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    single = kvc.snapkv_last_schedule() == kvc.SNAPKV_SINGLE_PASS
    score_kernel = kvc.snapkv_last_score_kernel()
    phases = PHASES_SINGLE if single else PHASES
    passes = ("score", "pool") if single else ("stats", "votes")
    log(f"schedule: {'single pass' if single else 'two passes'} ({score_kernel})")
    # Timed region: K steps back to back with no events in the stream (a
    # recorded event between two kernels costs the GPU several microseconds).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        call()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # The same K steps again with events around the score passes only
    # (boundaries 1 to 4): 1 -> 2 is the statistics pass or the single score
    # kernel, 3 -> 4 the vote pass or the pooling kernel.
    timed = [ev.create(4) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        arr = (ctypes.c_void_p * n_ev)()
        arr[1], arr[2], arr[3], arr[4] = timed[i]
        set_events(arr)
        call()
    torch.cuda.synchronize()
    set_events(None)
    kern_ms = {passes[0]: sum(ev.ms(e[0], e[1]) for e in timed) / args.steps,
               passes[1]: sum(ev.ms(e[2], e[3]) for e in timed) / args.steps}
    # Untimed instrumented pass: every phase boundary, for the breakdown only.
    events = [ev.create(n_ev) for _ in range(args.steps)]
    for i in range(args.steps):
        set_events(events[i])
        call()
    torch.cuda.synchronize()
    set_events(None)
    lib.kvc_snapkv_set_schedule(0)
    dec_att = time_decode(kvc, ev, q[:, :, -1].contiguous(), out.k, out.v, wl.budget, 200,
                          f"SnapKV-compressed {wl.name} layer B{B} H{H} {wl.budget} rows")
    phase_ms = {p: sum(ev.ms(e[j], e[j + 1]) for e in events) / args.steps for j, p in enumerate(phases)}
    # (single pass: nothing runs between marks 2 and 3; that interval is the events' own cost)
    phase_ms.pop("none", None)
    phases = [p for p in phases if p != "none"]
    step_ms = elapsed / args.steps * 1e3
    nbytes = snapkv_bytes(wl)
    dominant = "score" if single else max(("stats", "votes"), key=lambda p: kern_ms[p])
    dom_bytes = nbytes[dominant]
    achieved = dom_bytes / (kern_ms[dominant] * 1e-3)
    suffix = "bf16" if wl.dtype == "bf16" else "f32"
    kernel_name = score_kernel if single else f"snap_{dominant}_{suffix}"
    traffic = load_traffic(kernel_name, ["snapkv.hip", "common.hpp"])
    log(f"step {step_ms:.3f} ms; phases (ms): " + ", ".join(f"{p} {phase_ms[p]:.4f}" for p in phases))
    return dict(
        wl=wl, qn=qn, kn=kn, vn=vn, step_ms=step_ms, elapsed=elapsed,
        value=B * L * args.steps / elapsed,
        path_gbps=nbytes["total"] / (step_ms * 1e-3) / 1e9,
        roofline={"bound": "hbm", "achieved": achieved / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                  "frac": achieved / PEAK_HBM, "traffic": traffic, "kernel": kernel_name,
                  "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_ms": kern_ms[dominant],
                  "score_pass_ms": kern_ms},
        phase_ms=phase_ms, alg_bytes=nbytes["total"], schedule="single-pass" if single else "two-pass",
        decode_attention=dec_att)


def cpu_baseline(res, seconds):
    """The oracle on a bounded sample of the same workload (whole heads, in order)."""
    from oracle import snapkv as ref

    wl = res["wl"]
    try:
        import threadpoolctl
        blas = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()), default=1)
    except Exception:  # threadpoolctl missing: report the affinity only
        blas = None
    cores = len(os.sched_getaffinity(0))
    heads = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    done = 0
    t0 = time.perf_counter()
    # whole heads, cycling over the layer, until the time budget is spent
    while True:
        b, h = heads[done % len(heads)]
        ref.compress_head(res["qn"][b, h], res["kn"][b, h], res["vn"][b, h], wl.budget, wl.pool_kernel, wl.dtype)
        done += 1
        if time.perf_counter() - t0 > seconds:
            break
    t = time.perf_counter() - t0
    full_layer_s = t * len(heads) / done
    log(f"cpu oracle: {done} head compressions ({done / len(heads):.2f} layers) in {t:.1f}s")
    return {"value": wl.B * wl.L / full_layer_s, "unit": "tokens/s", "cores": blas or cores,
            "kind": "oracle", "affinity_cores": cores,
            "sample": f"{done} whole-head compressions cycling over the {len(heads)} heads of the {wl.name} "
                      f"layer (fp64 numpy, BLAS threads as reported), {t:.1f}s; scaled to one layer"}


def time_decode(kvc, ev, q, k, v, n, reps, label):
    """kvc_decode_attention over the first n rows of k/v: average time of `reps` back-to-back
    calls bracketed by two events on the library's stream, and its HBM roofline (K and V rows
    read once, q read, the fp32 output written)."""
    import torch

    B, H, _, D = k.shape
    es = k.element_size()
    ws = torch.empty(max(kvc.decode_attention_workspace_bytes(B, H, n, D), 16), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
    for _ in range(3):
        kvc.decode_attention(q, k, v, n, workspace=ws, out=out)
    torch.cuda.synchronize()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    e = ev.create(2)
    ev.record(e[0], stream)
    for _ in range(reps):
        kvc.decode_attention(q, k, v, n, workspace=ws, out=out)
    ev.record(e[1], stream)
    torch.cuda.synchronize()
    ms = ev.ms(e[0], e[1]) / reps
    nbytes = B * H * (2 * n * D * es + D * es + D * 4)
    gbps = nbytes / (ms * 1e-3) / 1e9
    log(f"decode attention, {label}: {ms * 1e3:.1f} us per call, {gbps:.0f} GB/s")
    return {"cache": label, "ms_per_call": ms, "calls": reps, "algorithmic_bytes": nbytes,
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


def stream_peak():
    """What this GPU streams with plain library kernels: a 1 GiB device copy (bytes read plus
    bytes written; the stream-copy peak) and a 1 GiB sum (a library reduction: bytes read), each
    timed over 10 launches with torch events on torch's own stream."""
    import torch

    n = 1 << 30
    a = torch.empty(n // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
        torch.sum(a)
    torch.cuda.synchronize()
    reps = 10
    out = {}
    for name, fn, nbytes in (("copy", lambda: b.copy_(a), 2 * n), ("read", lambda: torch.sum(a), n)):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        e.synchronize()
        out[f"{name}_gbps"] = nbytes * reps / (s.elapsed_time(e) * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    out["bytes"] = n
    out["kernels"] = "torch copy_ (read + write counted) and torch.sum (a reduction; read), 10 launches each"
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
    res = bench_snapkv(args, ev)
    wl = res["wl"]
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
        "roofline": res["roofline"],
        "phase_ms": res["phase_ms"],
        "decode_attention_compressed": res["decode_attention"],
    }
    sp = stream_peak()
    sp["score_kernel_frac_of_copy"] = res["roofline"]["achieved"] / sp["copy_gbps"]
    line["measured_stream"] = sp
    log(f"stream peak: copy {sp['copy_gbps']:.0f} GB/s, read {sp['read_gbps']:.0f} GB/s")
    if not args.skip_cpu:
        line["cpu_baseline"] = cpu_baseline(res, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    del res
    if not args.skip_h2o:
        line["h2o_sink"] = bench_h2o(args, ev)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
