#!/usr/bin/env python3
"""Throughput of packed draft-token verification on one MI355X.

One step is one pass of the whole verification path over one batch of
synthetic input: every verify row streamed once from HBM and reduced or
sampled, the per-request prefix-accept scan, compaction of emitted tokens by
device offsets, and (where the workload has draft logits) the draft
confidence of every draft row. The default workload is the EAGLE-shaped
greedy batch the headline metric is quoted on (B=128 requests, K=4 drafts,
V=152064, bf16 logits). Inputs are resident in HBM before timing starts and
rotate over enough copies (>= 1 GiB) that no step reads from the 256 MB
Infinity Cache.

Prints one JSON line on stdout. `roofline` rates the dominant kernel's
algorithmic bytes per launch against the 8 TB/s HBM peak, with the
per-launch duration from HIP events around each launch in the timed region;
`cpu_baseline` times the float64 CPU oracle on the same kind of input.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
ROTATE_BYTES = 1 << 30
KERNEL_SOURCES = ("csrc/device.hpp", "csrc/row_stream.hpp", "csrc/sampled_row.hpp", "csrc/verify_common.hpp",
                  "csrc/verify.hip", "csrc/sampled.hip", "csrc/confidence.hip", "csrc/kernels.hpp")


def kernel_source_sha():
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "draft_token_verification_packed_amd")
    for rel in KERNEL_SOURCES:
        p = os.path.join(pkg, rel)
        if os.path.exists(p):
            h.update(rel.encode())
            h.update(open(p, "rb").read())
    return h.hexdigest()


def measured_traffic(kernel, workload_tag):
    """HBM bytes per launch from committed rocprofv3 PMC runs, if still valid."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        entries = json.load(open(p))
    except ValueError:
        return None
    e = entries.get("%s/%s" % (kernel, workload_tag))
    if not e or e.get("kernel_source_sha") != kernel_source_sha():
        return None
    return e.get("bytes_per_launch")


def upload(torch, arr):
    import numpy as np
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def build_steps(vsv, torch, wl):
    """One list of prepared calls per rotating copy of the inputs.

    Returns (steps, kernels): steps[c] is the call list for copy c, kernels
    names each call's kernel and its algorithmic bytes per launch.
    """
    es = 2 if wl.dtype == 1 else 4
    verify_bytes = wl.R * wl.V * es
    conf_bytes = wl.D * wl.V * es
    step_bytes = verify_bytes + conf_bytes
    ncopy = max(1, math.ceil(ROTATE_BYTES / step_bytes))
    off, own, dr = upload(torch, wl.offsets), upload(torch, wl.owner), upload(torch, wl.drafts)
    base = upload(torch, wl.logits)
    dbase = upload(torch, wl.draft_logits) if wl.D else None
    sel = upload(torch, wl.selected) if wl.D else None
    if wl.sampled:
        params = [upload(torch, a) for a in (wl.temperature, wl.top_k, wl.top_p, wl.min_p)]
    steps = []
    for c in range(ncopy):
        logits = base if c == 0 else base.clone()
        calls = []
        if wl.sampled:
            call, _ = vsv.prepare_sampled(logits, off, own, dr, *params, wl.seed, wl.offset)
        else:
            call, _ = vsv.prepare_greedy(logits, off, own, dr, relaxed_topk=wl.relaxed_topk)
        calls.append(call)
        if wl.D:
            dl = dbase if c == 0 else dbase.clone()
            ccall, _ = vsv.prepare_confidence(dl, sel)
            calls.append(ccall)
        steps.append(calls)
    # greedy batches with between half as many rows as CUs and as many run
    # one persistent workgroup per CU, the others one workgroup per row or
    # half row (the library's launch rule)
    cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    greedy = "verify_greedy_kernel" if 2 * wl.R >= cus and wl.R <= cus else "verify_greedy_rows_kernel"
    kernels = [("verify_sampled_kernel" if wl.sampled else greedy, verify_bytes)]
    if wl.D:
        kernels.append(("confidence_kernel", conf_bytes))
    return steps, kernels, ncopy, step_bytes


def cpu_baseline(wl, budget_s=12.0):
    """Oracle (float64 NumPy, one process) on whole requests of the workload."""
    import numpy as np
    import oracle
    t0 = time.perf_counter()
    rows = 0
    passes = 0
    # one pass over the whole batch is seconds; repeat within the budget
    while True:
        if wl.sampled:
            oracle.verify_sampled(wl.logits, wl.dtype, wl.V, wl.offsets, wl.owner, wl.drafts,
                                  wl.temperature, wl.top_k, wl.top_p, wl.min_p, wl.seed, wl.offset)
        else:
            oracle.verify_greedy(wl.logits, wl.dtype, wl.V, wl.offsets, wl.owner, wl.drafts,
                                 relaxed_topk=wl.relaxed_topk)
        if wl.D:
            oracle.draft_confidence(wl.draft_logits, wl.dtype, wl.V, wl.selected)
        rows += wl.R
        passes += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return dict(value=rows / dt, unit="rows/s", cores=1, kind="oracle",
                sample="%d full pass(es) over the %d-row batch (%s), %.1f s, single process"
                       % (passes, wl.R, "plus its draft rows" if wl.D else "verify rows only", dt))


def bench_allocate(args, vsv, torch):
    """Adaptive verify allocation at the large mixed batch's shape (B=512,
    K=7, budget G = B + B * K / 2 rows), scores from the seeded generator.
    One workgroup; the kernel is latency-bound, so the line reports its
    launch time, with its algorithmic bytes against HBM for reference."""
    import numpy as np
    import synth
    from oracle.allocate import allocate_verify
    B, K = 512, 7
    G = B + (B * K) // 2
    conf, drafts = synth.scores(B, K, 1006, "confidence")
    c, d = upload(torch, conf), upload(torch, drafts)
    call, out = vsv.prepare_allocate(c, d, B, K, G)
    for _ in range(args.warmup):
        call.run()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(args.steps):
        call.run()
    ev[1].record()
    torch.cuda.synchronize()
    us = ev[0].elapsed_time(ev[1]) * 1e3 / args.steps
    ref = allocate_verify(conf, drafts, B, K, G)
    assert np.array_equal(out["verify_len"].cpu().numpy(), ref["verify_len"]), "allocation differs from the oracle"
    # scores and drafts read; lengths, offsets, owners, sources, packed drafts, products written
    nbytes = 4 * (2 * B * K + B + (B + 1) + 2 * G + (G - B) + B * K)
    achieved = nbytes / (us * 1e-6) / 1e9
    line = dict(metric="adaptive verify allocation latency, B=512 K=7 G=2304", value=us, unit="us",
                n_gpus=1, steps=args.steps, warmup=args.warmup, ms_per_step=us * 1e-3, higher_is_better=False,
                scaling="weak", vs_baseline=None, dtype="f32", data="synthetic",
                config=dict(workload="adaptive verify allocation, B=512 K=7 G=2304, confidence-shaped scores",
                            B=B, K=K, G=G, score_seed=1006),
                roofline=dict(bound="hbm", kernel="allocate_kernel", achieved=achieved, peak=HBM_PEAK_GBPS,
                              unit="GB/s", frac=achieved / HBM_PEAK_GBPS, traffic=None, bytes_per_launch=nbytes,
                              launch_us=us, note="one workgroup: bound by latency, not bandwidth"))
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < 10.0:
            allocate_verify(conf, drafts, B, K, G)
            n += 1
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = dict(value=dt / n * 1e6, unit="us", cores=1, kind="oracle",
                                    sample="%d allocations of the same batch, %.1f s, single process" % (n, dt))
    print(json.dumps(line), flush=True)
    return 0


def bench_probabilistic(args, vsv, torch):
    """Verification with probabilistic drafts on the large mixed batch (B=512,
    K=7, V=152064 bf16: even requests greedy, odd ones T = 0.7 and top_p
    0.95), each draft row the draft law at the request's temperature. The
    kernel is the exact, multi-pass one, so the line caps the launches at 3
    warm-up and 20 timed ones."""
    import numpy as np
    import synth
    wl = synth.make("mixed")
    B, R, V = wl.B, wl.R, wl.V
    td = wl.temperature.astype(np.float32)
    dev = [upload(torch, a) for a in (wl.logits, wl.offsets, wl.owner, wl.drafts, wl.draft_logits,
                                      wl.temperature, wl.top_k, wl.top_p, wl.min_p, td)]
    x, off, own, dr, y, T, TK, TP, MP, TD = dev
    warm, steps = min(args.warmup, 3), min(args.steps, 20)

    def call():
        return vsv.verify_probabilistic(x, off, own, dr, y, T, TK, TP, MP, TD, wl.seed, wl.offset, vocab=V)
    for _ in range(warm):
        call()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(steps):
        out = call()
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    assert int(out["error_flag"].item()) == 0
    nbytes = (R + wl.D) * V * 2     # every target and draft row read once
    achieved = nbytes / (ms * 1e-3) / 1e9
    line = dict(metric="probabilistic-draft verified rows/sec, B=512 K=7 V=152064", value=R / (ms * 1e-3),
                unit="rows/s", n_gpus=1, steps=steps, warmup=warm, ms_per_step=ms, higher_is_better=True,
                scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic",
                config=dict(workload="probabilistic-draft verify, " + wl.name.split(", ", 1)[1], B=B, R=R, D=wl.D,
                            V=V, draft_temperature="the request's target temperature", data_seed=wl._spec["data_seed"],
                            philox_seed=wl.seed),
                roofline=dict(bound="hbm", kernel="verify_probabilistic_kernel", achieved=achieved,
                              peak=HBM_PEAK_GBPS, unit="GB/s", frac=achieved / HBM_PEAK_GBPS, traffic=None,
                              bytes_per_launch=nbytes, launch_us=ms * 1e3,
                              note="exact multi-pass kernel: bound by its passes over rows held in the caches"))
    if not args.no_cpu_baseline:
        from oracle.probabilistic import verify_probabilistic
        t0 = time.perf_counter()
        rows, n = 0, 0
        while time.perf_counter() - t0 < 12.0 and n < B:
            r0, r1 = int(wl.offsets[n]), int(wl.offsets[n + 1])
            sub = slice(n, n + 1)
            verify_probabilistic(wl.logits[r0:r1], wl.dtype, V, np.array([0, r1 - r0], dtype=np.int32),
                                 np.zeros(r1 - r0, dtype=np.int32), wl.drafts[r0 - n:r1 - n - 1],
                                 wl.draft_logits[r0 - n:r1 - n - 1], wl.temperature[sub], wl.top_k[sub],
                                 wl.top_p[sub], wl.min_p[sub], td[sub], wl.seed, wl.offset)
            rows += r1 - r0
            n += 1
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = dict(value=rows / dt, unit="rows/s", cores=1, kind="oracle",
                                    sample="first %d requests (%d rows) one by one, %.1f s, single process"
                                    % (n, rows, dt))
    print(json.dumps(line), flush=True)
    return 0


def bench_goodput(args, vsv):
    """Goodput step selection per completed batch (host code): observe one
    batch of B=512 requests with up to 7 verified drafts, then pick the next
    step count, on a drifting synthetic acceptance history; the oracle is
    timed beside it on the same history."""
    import numpy as np
    from oracle.goodput import GoodputController
    rng = np.random.default_rng(1007)
    S, B, n = 7, 512, 2000
    hist = []
    for t in range(n):
        k = rng.integers(1, S + 1, B)
        p = 0.55 + 0.35 * np.sin(t / 50.0)
        a = np.minimum(rng.geometric(1.0 - p, B) - 1, k)
        hist.append((a.astype(np.int32), k.astype(np.int32)))
    cost = 10.0 + 1.5 * np.arange(1, S + 1)
    import ctypes
    g = vsv.Goodput(S)
    L = vsv.lib()
    st = ctypes.byref(g.state)
    ptrs = [(a.ctypes.data_as(ctypes.c_void_p), k.ctypes.data_as(ctypes.c_void_p)) for a, k in hist]
    cost = np.ascontiguousarray(cost, dtype=np.float64)
    pc = cost.ctypes.data_as(ctypes.c_void_p)
    out = ctypes.c_int32(0)
    po = ctypes.byref(out)
    steps = []
    t0 = time.perf_counter()
    for pa, pk in ptrs:
        if L.vsv_goodput_observe(st, pa, pk, B) != 0 or L.vsv_goodput_step(st, pc, B, po) != 0:
            raise RuntimeError("goodput call failed")
        steps.append(out.value)
    dt = time.perf_counter() - t0
    line = dict(metric="goodput step selection per batch (host), B=512 S=7", value=dt / n * 1e6, unit="us",
                n_gpus=0, steps=n, warmup=0, ms_per_step=dt / n * 1e3, higher_is_better=False, scaling="weak",
                vs_baseline=None, dtype="f64", data="synthetic",
                config=dict(workload="goodput step selection, B=512 max_steps=7, window 20, re-score every 5",
                            B=B, max_steps=S, batches=n, switches=int(np.count_nonzero(np.diff(steps)))),
                note="host code: the two C calls per batch through ctypes with arguments prepared beforehand")
    if not args.no_cpu_baseline:
        ref = GoodputController(S)
        t0 = time.perf_counter()
        ref_steps = []
        for a, k in hist:
            ref.observe(a, k)
            ref_steps.append(ref.step(cost, B))
        rdt = time.perf_counter() - t0
        assert ref_steps == steps, "goodput decisions differ from the oracle"
        line["cpu_baseline"] = dict(value=rdt / n * 1e6, unit="us", cores=1, kind="oracle",
                                    sample="the same %d batches, %.1f s, single process" % (n, rdt))
    print(json.dumps(line), flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    # the GPU needs tens of milliseconds of sustained work before its clocks
    # settle: with a short warm-up the first timed launches run 5-10 % slow
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default="eagle", choices=["tiny", "eagle", "ragged", "relaxed", "mixed"],
                    help="synthetic batch: tiny greedy B=4 K=4 V=1024 fp32; eagle greedy B=128 K=4 "
                         "V=152064 bf16 (default); ragged sampled B=128 K~U{0..7} fp32; relaxed top-4 + "
                         "confidence B=128 K=4 bf16; mixed sampled + confidence B=512 K=7 bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--goodput", action="store_true",
                    help="time goodput step selection (host code, B=512, 7 steps) instead of verification")
    ap.add_argument("--probabilistic", action="store_true",
                    help="time verification with probabilistic drafts on the mixed B=512 K=7 batch instead")
    ap.add_argument("--allocate", action="store_true",
                    help="time adaptive verify allocation (B=512, K=7) instead of verification")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB --steps times (calibrates "
                         "the profiler's FETCH_SIZE / WRITE_SIZE counters against a known byte count)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this library verifies on one GPU; --gpus %d is not supported "
              "(requests shard across GPUs without collectives, see the design notes)" % max(args.gpus, world),
              file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import synth
    import draft_token_verification_packed_amd as vsv

    if args.goodput:
        vsv.lib()
        return bench_goodput(args, vsv)
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps(dict(copy_probe_bytes=n, launches=args.steps)), flush=True)
        return 0
    vsv.lib()
    if args.allocate:
        return bench_allocate(args, vsv, torch)
    if args.probabilistic:
        return bench_probabilistic(args, vsv, torch)
    print("[bench] generating workload %s" % args.workload, file=sys.stderr, flush=True)
    wl = synth.make(args.workload)
    steps, kernels, ncopy, step_bytes = build_steps(vsv, torch, wl)
    torch.cuda.synchronize()
    print("[bench] %d input copies, %.1f MB per step" % (ncopy, step_bytes / 1e6), file=sys.stderr, flush=True)

    for k in range(args.warmup):
        for call in steps[k % ncopy]:
            call.run()
    torch.cuda.synchronize()

    # The calls of one step are independent (verification reads the target
    # rows, confidence the draft rows), so the timed region issues each call's
    # K launches back to back: the same work as K steps, and the event between
    # two runs gives that kernel's average launch duration on its own stream.
    ncall = len(steps[0])
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(ncall + 1)]
    torch.cuda.synchronize()
    bounds[0].record()
    for c in range(ncall):
        for k in range(args.steps):
            steps[k % ncopy][c].run()
        bounds[c + 1].record()
    torch.cuda.synchronize()
    total_ms = bounds[0].elapsed_time(bounds[ncall])
    per_kernel_ms = [bounds[c].elapsed_time(bounds[c + 1]) / args.steps for c in range(ncall)]
    ms = total_ms / args.steps
    print("[bench] %.2f us/step; per kernel %s us" % (ms * 1e3, ["%.2f" % (t * 1e3) for t in per_kernel_ms]),
          file=sys.stderr, flush=True)

    slow = None
    if wl.sampled:
        slow = int(steps[0][0]._keep[2]["slow_rows"].item())  # rows sent to the exact path, summed over calls
    dom = max(range(ncall), key=lambda c: kernels[c][1])
    kname, kbytes = kernels[dom]
    kms = per_kernel_ms[dom]
    achieved = kbytes / (kms * 1e-3) / 1e9
    traffic = measured_traffic(kname, args.workload)
    line = dict(
        metric="verified rows/sec and achieved HBM GB/s (% of peak), B=128 K=4 V=152064",
        value=wl.R / (ms * 1e-3), unit="rows/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=ms, higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="bf16" if wl.dtype == 1 else "f32", data="synthetic",
        hbm_gbps=step_bytes / (ms * 1e-3) / 1e9, hbm_frac=step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        config=dict(workload=wl.name, key=args.workload, B=wl.B, R=wl.R, D=wl.D, V=wl.V,
                    K=None if wl._spec["K"] is None else int(wl._spec["K"]),
                    relaxed_topk=wl.relaxed_topk, sampled=bool(wl.sampled), input_copies=ncopy,
                    bytes_per_step=step_bytes, data_seed=wl._spec["data_seed"], philox_seed=wl.seed,
                    slow_rows_first_copy=slow),
        roofline=dict(bound="hbm", kernel=kname, achieved=achieved, peak=HBM_PEAK_GBPS, unit="GB/s",
                      frac=achieved / HBM_PEAK_GBPS, traffic=traffic, bytes_per_launch=kbytes,
                      launch_us=kms * 1e3),
    )
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
