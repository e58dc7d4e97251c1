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
SPREAD_BLOCK = 10
ROTATE_BYTES = 1 << 30
KERNEL_SOURCES = ("csrc/device.hpp", "csrc/row_stream.hpp", "csrc/sampled_row.hpp", "csrc/verify_common.hpp",
                  "csrc/verify.hip", "csrc/sampled.hip", "csrc/confidence.hip", "csrc/kernels.hpp",
                  "csrc/row_queue.hpp", "csrc/probabilistic.hip", "csrc/probabilistic.hpp")


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


def metric_name(wl):
    """BASELINE's headline metric, named for the shape actually run."""
    K = wl._spec["K"]
    shape = "B=%d %s V=%d" % (wl.B, "K=%d" % K if K is not None else "K~U{0..%d}" % wl._spec["Kmax"], wl.V)
    return "verified rows/sec and achieved HBM GB/s (% of peak), " + shape


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
    kernels = [("verify_sampled_kernel" if wl.sampled else "verify_greedy_rows_kernel", verify_bytes)]
    if wl.D:
        kernels.append(("confidence_kernel", conf_bytes))
    return steps, kernels, ncopy, step_bytes


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cores():
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    # the GPU host's share is at most 16 cores per GPU
    return max(1, min(n, 16))


def request_args(wl, i):
    """The oracle's arguments for request i on its own (rows, drafts,
    parameters, and its Philox uniforms keyed by its batch index)."""
    r0, r1 = int(wl.offsets[i]), int(wl.offsets[i + 1])
    a = dict(i=i, logits=wl.logits[r0:r1], dtype=wl.dtype, V=wl.V, drafts=wl.drafts[r0 - i:r1 - i - 1],
             sampled=bool(wl.sampled), relaxed=wl.relaxed_topk, seed=wl.seed, offset=wl.offset,
             draft_logits=None if wl.D == 0 else wl.draft_logits[r0 - i:r1 - i - 1])
    if wl.sampled:
        a.update(T=wl.temperature[i:i + 1], TK=wl.top_k[i:i + 1], TP=wl.top_p[i:i + 1], MP=wl.min_p[i:i + 1])
    return a


def oracle_request(a):
    """One request through the oracle: verification of its rows (and draft
    confidence of its draft rows). Runs in the bench process or a pool worker;
    imports only NumPy and the oracle."""
    import numpy as np
    import oracle
    n = a["logits"].shape[0]
    off = np.array([0, n], dtype=np.int32)
    if a["sampled"]:
        us = {(0, j): oracle.row_uniform(a["seed"], a["i"], j, a["offset"]) for j in range(n)}
        ref = oracle.verify_sampled(a["logits"], a["dtype"], a["V"], off, None, a["drafts"], a["T"], a["TK"], a["TP"],
                                    a["MP"], a["seed"], a["offset"], uniforms=us)
    else:
        ref = oracle.verify_greedy(a["logits"], a["dtype"], a["V"], off, None, a["drafts"], relaxed_topk=a["relaxed"])
    if a["draft_logits"] is not None:
        ref["confidence"], ref["confidence_lse"] = oracle.draft_confidence(a["draft_logits"], a["dtype"], a["V"],
                                                                           a["drafts"])
    return ref


def margin_request(a):
    """True if a sampled row of the request lies within the tie margins (its
    outcome would then hinge on rounding, so it is left out of the check)."""
    import numpy as np
    import oracle
    if not a["sampled"] or float(np.float32(a["T"][0])) == 0.0:
        return False
    T = float(np.float32(a["T"][0]))
    for j in range(a["logits"].shape[0]):
        x = oracle.row_f64(a["logits"], a["dtype"], j, a["V"])
        u = oracle.row_uniform(a["seed"], a["i"], j, a["offset"])
        tp, um, mp = oracle.sampled_row_margins(x, T, int(a["TK"][0]), float(np.float32(a["TP"][0])),
                                                float(np.float32(a["MP"][0])), u)
        if tp < 2e-7 or um < 2e-7 or mp < 1e-9:
            return True
    return False


_POOL_WL = None


def _pool_init(meta, names):
    """Pool worker set-up: attach to the shared logits blocks (no copy) and
    rebuild a light view of the workload."""
    import types
    from multiprocessing import shared_memory
    import numpy as np
    import oracle  # noqa: F401  (imported once per worker, not per task)
    global _POOL_WL
    wl = types.SimpleNamespace(**meta)
    blocks = []
    for field, (name, shape, dtype) in names.items():
        shm = shared_memory.SharedMemory(name=name)
        blocks.append(shm)
        setattr(wl, field, np.ndarray(shape, dtype=dtype, buffer=shm.buf))
    wl._blocks = blocks
    _POOL_WL = wl


def _pool_task(i):
    a = request_args(_POOL_WL, i)
    oracle_request(a)
    return a["logits"].shape[0] + (0 if a["draft_logits"] is None else a["draft_logits"].shape[0])


def pool_rate(wl, cores, budget_s):
    """Oracle rows/s over `cores` worker processes split by request: the
    logits sit in shared memory, tasks are request indices, and whole
    rounds of requests are issued until budget_s has passed."""
    import multiprocessing
    from multiprocessing import shared_memory
    import numpy as np
    shms, names = [], {}
    try:
        for field in ("logits", "draft_logits"):
            arr = getattr(wl, field)
            if arr is None:
                continue
            shm = shared_memory.SharedMemory(create=True, size=max(1, arr.nbytes))
            shms.append(shm)
            np.ndarray(arr.shape, dtype=arr.dtype, buffer=shm.buf)[...] = arr
            names[field] = (shm.name, arr.shape, arr.dtype.str)
        meta = dict(B=wl.B, V=wl.V, D=wl.D, dtype=wl.dtype, offsets=wl.offsets, drafts=wl.drafts,
                    sampled=wl.sampled, relaxed_topk=wl.relaxed_topk, seed=wl.seed, offset=wl.offset,
                    temperature=wl.temperature, top_k=wl.top_k, top_p=wl.top_p, min_p=wl.min_p,
                    draft_logits=None)
        ctx = multiprocessing.get_context("spawn")
        pool = ctx.Pool(cores, initializer=_pool_init, initargs=(meta, names))
        try:
            pool.map(_pool_task, range(min(cores, wl.B)))          # start-up, not timed
            rows, n, nxt = 0, 0, 0
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < budget_s:
                chunk = [(nxt + k) % wl.B for k in range(4 * cores)]
                nxt = (nxt + 4 * cores) % wl.B
                rows += sum(pool.map(_pool_task, chunk, chunksize=1))
                n += len(chunk)
            dt = time.perf_counter() - t0
            # workers leave on their own (no signal): under a profiler that
            # hooks signals, terminated workers have failed to exit
            pool.close()
        except BaseException:
            pool.terminate()
            raise
        finally:
            pool.join()
    finally:
        for shm in shms:
            shm.close()
            shm.unlink()
    return rows / dt, n, rows, dt


def compare_request(wl, i, ref, gpu):
    """Mismatches between the oracle's result for request i and the GPU's."""
    import numpy as np
    r0, r1 = int(wl.offsets[i]), int(wl.offsets[i + 1])
    bad = []
    if int(gpu["accepted_len"][i]) != int(ref["accepted_len"][0]):
        bad.append("accepted_len")
    if int(gpu["next_token"][i]) != int(ref["next_token"][0]):
        bad.append("next_token")
    if not np.array_equal(gpu["row_token"][r0:r1], ref["row_token"]):
        bad.append("row_token")
    lse, want = gpu["row_lse"][r0:r1].astype(np.float64), ref["row_lse"]
    if not np.all(np.abs(lse - want) <= 1e-5 * np.maximum(1.0, np.abs(want))):
        bad.append("row_lse")
    o = int(gpu["out_offsets"][i])
    n = int(ref["out_offsets"][1])
    if int(gpu["out_offsets"][i + 1]) - o != n or not np.array_equal(gpu["out_tokens"][o:o + n], ref["out_tokens"]):
        bad.append("out_tokens")
    if "confidence" in ref:
        c = gpu["confidence"][r0 - i:r1 - i - 1].astype(np.float64)
        if not np.all(np.abs(c - ref["confidence"]) <= 1e-5 * ref["confidence"]):
            bad.append("confidence")
    return bad


def cpu_baseline(wl, gpu, budget_s=10.0):
    """The float64 oracle on the host cores, and the parity check.

    Single process: whole requests in batch order until about budget_s of CPU
    work (repeating whole passes if the batch takes less). Pool: the same
    oracle over len(sched_getaffinity) worker processes (at most 16), split by
    request, for about budget_s (pool_rate). Every request the single-process leg ran first is compared with
    the GPU's outputs of the first input copy (`gpu`, host arrays): bit-exact
    tokens, lengths and compacted output, log-sum-exp and confidence within
    1e-5 relative; sampled requests with a row inside the tie margins are
    left out of that check and counted."""
    import multiprocessing
    import numpy as np
    t0 = time.perf_counter()
    rows, done, mismatched, margin_skipped = 0, 0, [], 0
    checked = set()
    while True:
        i = done % wl.B
        a = request_args(wl, i)
        ref = oracle_request(a)
        rows += a["logits"].shape[0] + (0 if a["draft_logits"] is None else a["draft_logits"].shape[0])
        done += 1
        if i not in checked:
            checked.add(i)
            bad = compare_request(wl, i, ref, gpu)
            if bad:
                if margin_request(a):
                    margin_skipped += 1
                else:
                    mismatched.append((i, bad))
        if time.perf_counter() - t0 >= budget_s:
            break
    dt1 = time.perf_counter() - t0
    single = rows / dt1
    cores = host_cores()
    rate, n_pool, prow, dt2 = pool_rate(wl, cores, budget_s)
    unit_rows = "verify + draft rows" if wl.D else "verify rows"
    return dict(
        value=rate, unit="rows/s", cores=cores, kind="oracle", cpu=cpu_model(),
        single_core_value=single,
        sample="%d requests (%d %s) over a pool of %d processes split by request, %.1f s; single process: "
               "%d requests in %.1f s" % (n_pool, prow, unit_rows, cores, dt2, done, dt1),
        parity=dict(requests_checked=len(checked), requests_mismatched=len(mismatched),
                    margin_skipped=margin_skipped, first_mismatches=mismatched[:5],
                    checked="accepted_len, next_token, row_token, compacted tokens bit-exact; row_lse%s within "
                            "1e-5 relative" % (" and confidence" if wl.D else "")),
    )


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
    slow = int(out["slow_rows"].item())     # rows of the last launch that took the whole-row path
    # every target row read once, and the draft rows of sampled requests (a
    # greedy target's law is a point mass: its drafts are decided without q)
    d_sampled = int(sum(int(wl.offsets[i + 1] - wl.offsets[i]) - 1 for i in range(B) if wl.temperature[i] > 0))
    nbytes = (R + d_sampled) * V * 2
    achieved = nbytes / (ms * 1e-3) / 1e9
    line = dict(metric="probabilistic-draft verified rows/sec, B=512 K=7 V=152064", value=R / (ms * 1e-3),
                unit="rows/s", n_gpus=1, steps=steps, warmup=warm, ms_per_step=ms, higher_is_better=True,
                scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic",
                config=dict(workload="probabilistic-draft verify, " + wl.name.split(", ", 1)[1], B=B, R=R, D=wl.D,
                            draft_rows_read=d_sampled,
                            V=V, draft_temperature="the request's target temperature", data_seed=wl._spec["data_seed"],
                            philox_seed=wl.seed, slow_rows_last_launch=slow),
                roofline=dict(bound="hbm", kernel="verify_probabilistic_kernel", achieved=achieved,
                              peak=HBM_PEAK_GBPS, unit="GB/s", frac=achieved / HBM_PEAK_GBPS,
                              traffic=measured_traffic("verify_probabilistic_kernel", "probabilistic"),
                              bytes_per_launch=nbytes, launch_us=ms * 1e3,
                              note="each verify row streamed once, then its draft row; sampled rows re-read "
                                   "their candidate vectors"))
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

    # The first copy's outputs, before any timing: the CPU-baseline leg
    # compares them with the oracle's.
    for call in steps[0]:
        call.run()
    torch.cuda.synchronize()
    res = steps[0][0]._keep[2]
    gpu = {k: res[k].cpu().numpy() for k in ("accepted_len", "next_token", "out_offsets", "out_tokens",
                                             "row_token", "row_lse", "error_flag")}
    if wl.D:
        gpu["confidence"] = steps[0][1]._keep[2][0].cpu().numpy()
    slow = int(res["slow_rows"].item()) if wl.sampled else None
    baseline = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle and checking the first copy against it", file=sys.stderr, flush=True)
        baseline = cpu_baseline(wl, gpu)
        par = baseline["parity"]
        print("[bench] parity: %d requests checked, %d mismatched, %d inside the tie margins"
              % (par["requests_checked"], par["requests_mismatched"], par["margin_skipped"]),
              file=sys.stderr, flush=True)
        if par["requests_mismatched"] or int(gpu["error_flag"][0]) != 0:
            print("[bench] GPU outputs differ from the oracle: %s" % par["first_mismatches"], file=sys.stderr)
            return 3

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
    # The spread of launch times: a second pass with an event after every
    # SPREAD_BLOCK launches (an event between every two launches would add
    # its own gap to each); median, p10 and p90 of the block means.
    spread = []
    nblk = max(1, args.steps // SPREAD_BLOCK)
    for c in range(ncall):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(nblk + 1)]
        ev[0].record()
        for b in range(nblk):
            for k in range(b * SPREAD_BLOCK, (b + 1) * SPREAD_BLOCK):
                steps[k % ncopy][c].run()
            ev[b + 1].record()
        torch.cuda.synchronize()
        t = sorted(ev[b].elapsed_time(ev[b + 1]) * 1e3 / SPREAD_BLOCK for b in range(nblk))
        pick = lambda q: t[min(len(t) - 1, int(round(q * (len(t) - 1))))]
        spread.append(dict(median=pick(0.5), p10=pick(0.1), p90=pick(0.9), block=SPREAD_BLOCK))
    print("[bench] %.2f us/step; per kernel %s us; medians %s us" % (
        ms * 1e3, ["%.2f" % (t * 1e3) for t in per_kernel_ms], ["%.2f" % d["median"] for d in spread]),
        file=sys.stderr, flush=True)

    dom = max(range(ncall), key=lambda c: kernels[c][1])
    kname, kbytes = kernels[dom]
    kms = per_kernel_ms[dom]
    achieved = kbytes / (kms * 1e-3) / 1e9
    traffic = measured_traffic(kname, args.workload)
    step_median_us = sum(d["median"] for d in spread)
    line = dict(
        metric=metric_name(wl),
        value=wl.R / (ms * 1e-3), unit="rows/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=ms, higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="bf16" if wl.dtype == 1 else "f32", data="synthetic",
        hbm_gbps=step_bytes / (ms * 1e-3) / 1e9, hbm_frac=step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        step_us=dict(mean=ms * 1e3, median=step_median_us, per_kernel=[
            dict(kernel=kernels[c][0], mean=per_kernel_ms[c] * 1e3, **spread[c]) for c in range(ncall)]),
        rows_per_s_at_median=wl.R / (step_median_us * 1e-6),
        config=dict(workload=wl.name, key=args.workload, B=wl.B, R=wl.R, D=wl.D, V=wl.V,
                    K=None if wl._spec["K"] is None else int(wl._spec["K"]),
                    relaxed_topk=wl.relaxed_topk, sampled=bool(wl.sampled), input_copies=ncopy,
                    bytes_per_step=step_bytes, data_seed=wl._spec["data_seed"], philox_seed=wl.seed,
                    slow_rows_first_copy=slow),
        roofline=dict(bound="hbm", kernel=kname, achieved=achieved, peak=HBM_PEAK_GBPS, unit="GB/s",
                      frac=achieved / HBM_PEAK_GBPS, traffic=traffic, bytes_per_launch=kbytes,
                      launch_us=kms * 1e3, launch_us_median=spread[dom]["median"],
                      launch_us_p10=spread[dom]["p10"], launch_us_p90=spread[dom]["p90"]),
    )
    if baseline is not None:
        line["cpu_baseline"] = baseline
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
