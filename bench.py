"""Benchmark: KV bytes moved per second by kvx backup (GPU pool -> pinned host)
and restore (pinned host -> other GPU pages, with per-layer publish) on one
MI355X.

Default workload: the mixed hit/miss stream over a bf16 pool of 32 layers,
K+V, 8 KV heads, head_dim 128, page size 64 and 8192 pages (64 GiB). It
stands in for the alternating storage-hit / storage-miss benchmark of the
PP-prefetch-ticket PR (128 requests, concurrency 4, 16,384-token inputs;
[TICKET] "Benchmark / Setup"). One step = that whole stream: 128 requests of
256 fragmented pages (16,384 tokens, 2 GiB each), alternating BACKUP (a
miss: gather the request's pages into a pinned host buffer) and RESTORE (a
hit: scatter a primed host copy into 256 other pages, publishing every
layer into a ready object), then the host polls the ready prefix until every
restore of the step is published. Each call runs validation and run planning
on the host and then the zero-copy gather or scatter kernel over the host
link.

Headline schedule: every request its own zero-copy call, round-robin over
four streams, so four requests are in flight (two backups and two restores)
and both directions of the host link carry data together; the library sizes
each kernel's grid by the other streams' host-link calls in flight and their
direction. Also reported: the same stream with each backup paired with the
restore after it in one kvx_exchange launch (pairs on two streams), the
four-stream schedule on the staged path, through the submission ring's
executor, the device pack/unpack kernels against the HBM roofline, the
pinned memcpy peaks, the Llama-3-8B-shaped one-request step and the CPU
oracle on a bounded sample (a baseline only).

value = 128 x 2 GiB x steps / wall time of the steps (GB = 1e9 B). The pool
is resident in HBM when the timed region starts; crossing the host link is
part of the method (the host tier is where BACKUP writes and RESTORE reads).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--schedule exchange|streams]
       [--workload mixed|llama8b|mla_fp8|trtllm_hnd|tiny|token_pages] [--no-cpu-baseline] [--kernel-only]
       [--no-extras] [--all-workloads] [--set OPTION=VALUE]
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

GB = 1e9
HBM_PEAK_GBS = 8000.0     # MI355X published HBM3E bandwidth
PCIE_PEAK_GBS = 64.0      # MI355X host interface, PCIe 5.0 x16, published per-direction rate


def pcie_protocol_bound(payload=256, write_overhead=24, completion_overhead=20, request_bytes=24):
    """The host link's transaction-layer bound in GB/s, before link-layer
    acknowledgement and flow-control packets. PCIe 5.0 x16 signals at 32
    GT/s on 16 lanes with 128b/130b coding: 63.0 GB/s each way. Data moves
    in packets of `payload` bytes: a posted write (the backup's stores into
    host memory) adds 4 bytes of start token, a 16-byte header and a 4-byte
    CRC; a completion with data (the restore's loads from host memory) a
    12-byte header instead; each read request is a 24-byte packet on the
    link towards the host, one per completion. With both directions busy
    that link carries the backup's writes and the restore's requests."""
    raw = 32e9 * 16 / 8 * 128 / 130 / GB
    d2h = raw * payload / (payload + write_overhead)
    h2d = raw * payload / (payload + completion_overhead)
    each = min(raw * payload / (payload + write_overhead + request_bytes), h2d)
    return {"d2h": round(d2h, 2), "h2d": round(h2d, 2), "both_directions": round(2 * each, 2),
            "assumes": f"PCIe 5.0 x16, 128b/130b, {payload} B payload per packet, "
                       f"{write_overhead} B per write, {completion_overhead} B per completion, "
                       f"one {request_bytes} B read request per completion, no link-layer packets"}


# pages one move-kernel launch carries in its arguments; a longer page list
# goes to device memory and one launch serves the call (KVX_OPT_DEVICE_LISTS;
# the exception, plain device-memory kernels of units under 32 KiB, is no
# workload here), else the call is split into equal launches and the roofline
# figures of such a call are per call
PAGES_PER_LAUNCH = 448

# HBM bytes per launch of the roofline kernel from the two rocprofv3 --pmc runs
# (FETCH_SIZE, WRITE_SIZE, scaled by a plain device copy in the same run; see
# profiles/pack_kernel_<workload>.txt). Valid only for the kernel source they
# were taken on: reported as null once kernels.hip changes.
MEASURED_TRAFFIC = {
    "mixed": {"kernels_hip_sha256": "aff0f2d369a8c53df0c3f40de64881e63b4fab8f214273fbbe41d29b0b9bf0b4",
            "bytes_per_launch": 4295192767},
    "llama8b": {"kernels_hip_sha256": "aff0f2d369a8c53df0c3f40de64881e63b4fab8f214273fbbe41d29b0b9bf0b4",
              "bytes_per_launch": 4295191652},
    "mla_fp8": {"kernels_hip_sha256": "aff0f2d369a8c53df0c3f40de64881e63b4fab8f214273fbbe41d29b0b9bf0b4",
              "bytes_per_launch": 1151511736},
    "trtllm_hnd": {"kernels_hip_sha256": "aff0f2d369a8c53df0c3f40de64881e63b4fab8f214273fbbe41d29b0b9bf0b4",
                 "bytes_per_launch": 4295389723},
    "token_pages": {"kernels_hip_sha256": "aff0f2d369a8c53df0c3f40de64881e63b4fab8f214273fbbe41d29b0b9bf0b4",
                  "bytes_per_launch": 4306347663},
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def median(xs):
    return statistics.median(xs) if xs else float("nan")


def measured_traffic(workload):
    """Counter traffic of the roofline kernel for this workload, if it was
    taken on the kernel source in the tree."""
    m = MEASURED_TRAFFIC.get(workload)
    if not m or not m["kernels_hip_sha256"]:
        return None
    import hashlib
    try:
        with open(os.path.join(ROOT, "paged_kv_offload_amd", "csrc", "kernels.hip"), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() == m["kernels_hip_sha256"]:
                return m["bytes_per_launch"]
    except OSError:
        pass
    return None


class Timer:
    """HIP events on one stream (torch.cuda.Event records on the stream it is
    given, the stream the kernels run on)."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def ev(self):
        return self.torch.cuda.Event(enable_timing=True)

    def timed(self, fn, reps, s=None):
        """Per-repetition durations (s) of fn, each between two events."""
        s = s or self.stream
        out = []
        for _ in range(reps):
            a, b = self.ev(), self.ev()
            a.record(s)
            fn()
            b.record(s)
            b.synchronize()
            out.append(a.elapsed_time(b) / 1e3)
        return out

    def batched(self, fn, reps, per=10, s=None):
        """Per-launch durations (s): events around `per` back-to-back calls,
        `reps` times. The host work of each call overlaps the previous
        kernel, so the average is the kernel's own duration."""
        s = s or self.stream
        out = []
        for _ in range(reps):
            a, b = self.ev(), self.ev()
            a.record(s)
            for _ in range(per):
                fn()
            b.record(s)
            b.synchronize()
            out.append(a.elapsed_time(b) / 1e3 / per)
        return out

    def stats(self, fn, warm=2, reps=10):
        """(median, best) of `reps` timed calls after `warm` untimed ones."""
        self.timed(fn, warm)
        t = self.timed(fn, reps)
        return median(t), min(t)


def make_pool(K, synth, torch, w):
    """The workload's allocation on cuda:0, filled from the seeded generator,
    and the pool registered on it."""
    alloc = torch.empty(w.alloc_bytes, dtype=torch.uint8, device="cuda")
    synth.fill_alloc_gpu(alloc.data_ptr(), w, w.seed)
    dt = {1: torch.uint8, 2: torch.bfloat16}[w.dtype_bytes]
    t = alloc[w.byte_offset:w.byte_offset + w.pool_bytes].view(dt).view(*w.tensor_shape())
    lay = K.make_layout(w.outer, w.inner, w.num_pages, w.num_layers, w.num_kv, w.page_size,
                        w.num_heads, w.head_dim)
    torch.cuda.synchronize()
    return alloc, K.register_tensor(t, lay, 1)


def device_kernels(T, K, torch, w, pool, src, dst, reps):
    """The device pack and unpack kernels on one request (device path), the
    unpack publishing every layer, and torch's D2D copy of the same bytes;
    read + write bytes over the per-launch duration (HIP events around
    back-to-back launches on the kernels' stream)."""
    P = w.payload_bytes(len(src))
    dev = torch.empty(P, dtype=torch.uint8, device="cuda")
    ready = K.kvx_ready_create(w.num_layers, 1)

    def pack():
        K.kvx_backup(pool, src, dev, P, 0, w.num_layers, T.stream, K.KVX_PATH_DEVICE)

    def unpack():
        K.kvx_restore(pool, dev, P, dst, 0, w.num_layers, None, 0, T.stream, K.KVX_PATH_DEVICE)

    def unpack_publish():
        K.kvx_restore(pool, dev, P, dst, 0, w.num_layers, ready, 0, T.stream, K.KVX_PATH_DEVICE)

    out = {}
    for name, fn in (("pack", pack), ("unpack", unpack), ("unpack_publish", unpack_publish)):
        T.timed(fn, 3)
        t = T.batched(fn, reps)
        out[name] = {"gbs": round(2 * P / median(t) / GB, 1), "best_gbs": round(2 * P / min(t) / GB, 1),
                     "frac": round(2 * P / median(t) / GB / HBM_PEAK_GBS, 4),
                     "avg_launch_ms": round(median(t) * 1e3, 4)}
    K.kvx_ready_destroy(ready)
    copy = torch.empty(P, dtype=torch.uint8, device="cuda")
    with torch.cuda.stream(T.stream):
        T.timed(lambda: copy.copy_(dev), 2)
        t = T.timed(lambda: copy.copy_(dev), 5)
    out["d2d_copy_gbs"] = round(2 * P / median(t) / GB, 1)
    del dev, copy
    log(f"device kernels, {w.name}: " + ", ".join(
        f"{k} {v['gbs'] if isinstance(v, dict) else v} GB/s" for k, v in out.items()))
    return out


def memcpy_peaks(T, torch, s2):
    """Pinned hipMemcpyAsync peaks, 1 GiB: D2H and H2D (median of 10 each)
    and both directions at once on two streams (median of 5)."""
    n = 1 << 30
    pin, pin2 = (torch.empty(n, dtype=torch.uint8, pin_memory=True) for _ in range(2))
    dev1, dev2 = (torch.empty(n, dtype=torch.uint8, device="cuda") for _ in range(2))
    with torch.cuda.stream(T.stream):
        T.timed(lambda: pin.copy_(dev1, non_blocking=True), 2)
        t_d2h = T.timed(lambda: pin.copy_(dev1, non_blocking=True), 10)
        t_h2d = T.timed(lambda: dev1.copy_(pin, non_blocking=True), 10)
    both = []
    for _ in range(5):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(T.stream):
            pin.copy_(dev1, non_blocking=True)
        with torch.cuda.stream(s2):
            dev2.copy_(pin2, non_blocking=True)
        torch.cuda.synchronize()
        both.append(time.perf_counter() - t0)
    del pin, pin2, dev1, dev2
    peaks = {"d2h": round(n / median(t_d2h) / GB, 2), "h2d": round(n / median(t_h2d) / GB, 2),
             "both_directions": round(2 * n / median(both) / GB, 2)}
    log(f"pinned memcpy peaks: {peaks}")
    return peaks


# ---------------------------------------------------------------------------
# the mixed hit/miss stream (default)
# ---------------------------------------------------------------------------
def mixed_main(args, options):
    import numpy as np
    import torch

    import synth
    from paged_kv_offload_amd import kvx as K
    from synth.workloads import WORKLOADS, mixed_schedule

    w = WORKLOADS["mixed"]
    NL, n = w.num_layers, w.pages_per_request
    P = w.payload_bytes()
    R = 128
    ZC = K.KVX_PATH_ZEROCOPY
    sched = mixed_schedule(w, R)
    perm = synth.page_perm(w.seed, w.num_pages)
    stream = torch.cuda.Stream()
    T = Timer(torch, stream)
    log(f"workload {w.name}: pool {w.pool_bytes / 2**30:.0f} GiB, {R} requests of "
        f"{P / 2**30:.2f} GiB per step")
    alloc, pool = make_pool(K, synth, torch, w)

    # ---- HBM roofline: the pack kernel on the stream's first request ----
    kern = device_kernels(T, K, torch, w, pool, sched[0][1], sched[1][1], max(args.steps, 10))
    roofline = {"bound": "hbm",
                "kernel": f"kvx_move_kernel<GATHER> (device pack of one {P / 2**30:.0f} GiB request "
                          f"of the mixed stream: 32 layers x K,V x 256 fragmented 128 KiB pieces)",
                "achieved": kern["pack"]["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": kern["pack"]["frac"], "traffic": measured_traffic(w.name),
                "algorithmic_bytes_per_launch": 2 * P,
                "avg_launch_ms": kern["pack"]["avg_launch_ms"]}
    if args.kernel_only:
        print(json.dumps({"roofline": roofline, "device_kernels": kern, "options": options}), flush=True)
        return

    # ---- host buffers: four primed restore sources, four rotating backup targets ----
    bufs = [K.HostBuffer(P) for _ in range(8)]
    for r in range(4):
        K.kvx_backup(pool, np.ascontiguousarray(perm[n * r:n * (r + 1)]), bufs[r].ptr, P, 0, NL,
                     stream, ZC)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(4)]
    peaks = memcpy_peaks(T, torch, streams[1])
    proto = pcie_protocol_bound()

    # ---- the paired schedule: backup k + restore k+1 in one kvx_exchange ----
    pairs = [(sched[k][1], sched[k + 1][1]) for k in range(0, R, 2)]
    assert all(sched[k][0] == "backup" and sched[k + 1][0] == "restore" for k in range(0, R, 2))
    ready_x = K.kvx_ready_create(2 * NL, 1)     # slots [0, NL): stream 0's restores; [NL, 2NL): stream 1's
    published = {"x": 0, "s": 0, "r": 0}        # pages published so far into each slot of each object

    def exchange_pass(marks=None):
        for i, (ib, ir) in enumerate(pairs):
            s = streams[i % 2]
            if marks is not None:
                e0 = T.ev()
                e0.record(s)
            K.kvx_exchange(pool, ib, bufs[4 + i % 4].ptr, P, (0, NL), bufs[i % 4].ptr, P, ir, (0, NL),
                           ready_x, NL * (i % 2), s, ZC)
            if marks is not None:
                e1 = T.ev()
                e1.record(s)
                marks.append((e0, e1))
        published["x"] += len(pairs) // 2 * n
        while K.kvx_ready_prefix(ready_x) < published["x"]:    # the consumers' view of completion
            pass

    # ---- the headline schedule: every request its own call, four streams ----
    ready_s = K.kvx_ready_create(2 * NL, 1)     # restores run on streams 1 and 3

    def streams_pass(bpath, rpath):
        nb = nr = 0
        for k, (kind, ids) in enumerate(sched):
            s = streams[k % 4]
            if kind == "backup":
                K.kvx_backup(pool, ids, bufs[4 + nb % 4].ptr, P, 0, NL, s, bpath)
                nb += 1
            else:
                K.kvx_restore(pool, bufs[nr % 4].ptr, P, ids, 0, NL, ready_s, NL * ((k % 4) // 2), s,
                              rpath)
                nr += 1
        published["s"] += R // 4 * n
        while K.kvx_ready_prefix(ready_s) < published["s"]:
            pass

    def run(pass_fn, steps, warmup):
        for _ in range(warmup):
            pass_fn()
        torch.cuda.synchronize()
        marks = []
        t0 = time.perf_counter()
        for _ in range(steps):
            pass_fn(marks) if pass_fn is exchange_pass else pass_fn()
        torch.cuda.synchronize()
        return time.perf_counter() - t0, marks

    if args.schedule == "exchange":
        head_fn = exchange_pass
        schedule = ("each backup paired with the restore after it in one kvx_exchange launch, pairs "
                    "alternating over two streams (4 requests in flight); zero-copy; restores publish "
                    "every layer; the host polls the ready prefix until the step's restores are published")
    else:
        head_fn = lambda marks=None: streams_pass(ZC, ZC)  # noqa: E731
        schedule = ("every request its own zero-copy call, round-robin over four streams (4 in flight: "
                    "two backups, two restores; the library holds the kernels that write host memory "
                    "to 6 workgroups and those that read it to 18 in total while both directions are "
                    "in flight); restores publish every layer; the host polls the ready prefix until "
                    "the step's restores are published")
    wall, marks = run(head_fn, args.steps, args.warmup)
    value = R * P * args.steps / wall / GB
    ms_per_step = wall / args.steps * 1e3
    log(f"mixed stream ({args.schedule}): {ms_per_step:.1f} ms per step -> {value:.2f} GB/s")

    link = {"bound": "host link (PCIe 5.0 x16, both directions at once)",
            "achieved": round(value, 2), "unit": "GB/s", "peak": 2 * PCIE_PEAK_GBS,
            "frac": round(value / (2 * PCIE_PEAK_GBS), 4),
            "protocol_bound": proto,
            "frac_of_protocol_bound": round(value / proto["both_directions"], 4),
            "measured_memcpy_peak": peaks,
            "frac_of_measured_memcpy_both_directions": round(value / peaks["both_directions"], 4)}
    if marks:
        per = [a.elapsed_time(b) / 1e3 for a, b in marks]
        link["exchange_launch_ms"] = {"median": round(median(per) * 1e3, 3),
                                      "best": round(min(per) * 1e3, 3),
                                      "two_launches_in_flight": True,
                                      "bytes_per_launch": 2 * P}
    result = {
        "metric": "KV GB/s moved (backup D2H, restore H2D) + % of HBM / host-link roofline",
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "config": {"workload": w.description, "requests_per_step": R, "in_flight": 4,
                   "pages_per_request": n, "layers": NL, "payload_bytes_per_request": P,
                   "bytes_per_step": R * P, "path": "zerocopy", "schedule": schedule,
                   "hw_queues": os.environ.get("GPU_MAX_HW_QUEUES", "runtime default"),
                   "options": options},
        "roofline": roofline,
        "device_kernels": kern,
        "link_roofline": link,
    }

    if not args.no_extras:
        other = {}
        # the other way of running the same stream, one warm-up pass and two timed
        for name, fn in ((("streams_zerocopy", lambda m=None: streams_pass(ZC, ZC))
                          if args.schedule == "exchange" else ("exchange_paired", exchange_pass)),
                         ("streams_staged", lambda m=None: streams_pass(K.KVX_PATH_STAGED,
                                                                        K.KVX_PATH_STAGED))):
            wl, _ = run(fn, 2, 1)
            other[name] = round(R * P * 2 / wl / GB, 2)
            log(f"mixed stream, {name}: {other[name]} GB/s")
        # the same stream as descriptors through a submission ring, served on
        # one stream by the library's executor (it pairs a backup with the
        # restore after it by itself)
        ready_r = K.kvx_ready_create(NL, 1)
        rname = f"/kvx-bench-{os.getpid()}"
        ring = K.kvx_ring_create(rname, 256, 1)
        srv = K.kvx_ring_open(rname)
        rbufs, rsizes = [b.ptr for b in bufs], [P] * len(bufs)

        def ring_pass(m=None):
            nb = nr = 0
            for k, (kind, ids) in enumerate(sched):
                if kind == "backup":
                    q = K.make_sqe(K.KVX_OP_BACKUP, k, 1, 0, 4 + nb % 4, ids, 0, NL, ZC)
                    nb += 1
                else:
                    q = K.make_sqe(K.KVX_OP_RESTORE, k, 1, 0, nr % 4, ids, 0, NL, ZC, ready_slot_base=0)
                    nr += 1
                K.kvx_ring_submit(ring, q)
            done = []
            while len(done) < len(sched):
                K.kvx_ring_serve(srv, [pool], rbufs, rsizes, ready_r, streams[0], 256)
                done += K.kvx_ring_reap(ring, 256)
                time.sleep(0.0002)
            assert all(c[2] == 0 for c in done), [c for c in done if c[2] != 0][:3]
            published["r"] += R // 2 * n
            assert K.kvx_ready_prefix(ready_r) == published["r"]

        wl, _ = run(ring_pass, 2, 1)
        other["ring_executor_paired"] = round(R * P * 2 / wl / GB, 2)
        log(f"mixed stream, ring executor: {other['ring_executor_paired']} GB/s")
        K.kvx_ring_close(srv)
        K.kvx_ring_close(ring)
        K.kvx_ready_destroy(ready_r)
        result["other_schedules_gbs"] = other

    K.kvx_ready_destroy(ready_x)
    K.kvx_ready_destroy(ready_s)
    for b in bufs:
        b.free()
    K.kvx_unregister_pool(pool)
    del alloc
    torch.cuda.empty_cache()

    if not args.no_extras:
        # the Llama-3-8B-shaped one-request step (layer-pipelined exchange)
        sub = argparse.Namespace(**vars(args))
        sub.steps, sub.warmup, sub.schedule, sub.no_extras = min(args.steps, 10), 2, "exchange", True
        result["llama8b_request_step"] = single_main(sub, options, WORKLOADS["llama8b"], quiet=True)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w)
        log(f"cpu baseline: {result['cpu_baseline']}")
        result["cpu_baseline_all_cores"] = cpu_baseline_all_cores(w)
        log(f"cpu baseline, all cores: {result['cpu_baseline_all_cores']}")
    print(json.dumps(result), flush=True)


# ---------------------------------------------------------------------------
# one request of a single-request workload (llama8b, mla_fp8, trtllm_hnd, tiny)
# ---------------------------------------------------------------------------
def single_main(args, options, w, quiet=False):
    """One step = BACKUP of one request to pinned host memory and its RESTORE
    into other pages with per-layer publish, then the ready-prefix poll.
    Schedule "exchange": the backup of layer 0, then one kvx_exchange per
    layer that backs up layer l + 1 while it restores layer l (the restore
    reads what the previous launch wrote), then the restore of the last
    layer; zero-copy. Schedule "streams" runs the serial form: backup of
    every layer, then restore of every layer. Returns the result (quiet) or
    prints it."""
    import numpy as np
    import torch

    import synth
    from paged_kv_offload_amd import kvx as K

    n = w.pages_per_request
    P = w.payload_bytes(n)
    perm = synth.page_perm(w.seed, w.num_pages)
    src = np.ascontiguousarray(perm[:n])
    dst = np.ascontiguousarray(perm[n:2 * n])
    stream = torch.cuda.Stream()
    T = Timer(torch, stream)
    log(f"workload {w.name}: pool {w.pool_bytes / 2**30:.1f} GiB, payload {P / 2**30:.2f} GiB/op")
    alloc, pool = make_pool(K, synth, torch, w)
    kern = device_kernels(T, K, torch, w, pool, src, dst, max(args.steps, 10))
    roofline = {"bound": "hbm",
                "kernel": f"kvx_move_kernel<GATHER> (pack of one {P / 2**30:.2f} GiB {w.name} request, "
                          f"device path)",
                "achieved": kern["pack"]["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": kern["pack"]["frac"], "traffic": measured_traffic(w.name),
                "algorithmic_bytes_per_launch": 2 * P, "avg_launch_ms": kern["pack"]["avg_launch_ms"],
                "launches_per_call": 1 if K.kvx_get_option(K.KVX_OPT_DEVICE_LISTS) else -(-n // PAGES_PER_LAUNCH)}
    if args.kernel_only:
        print(json.dumps({"roofline": roofline, "device_kernels": kern, "options": options}), flush=True)
        return None

    sb = torch.cuda.Stream()
    peaks = memcpy_peaks(T, torch, sb)
    host = K.HostBuffer(P)
    ready = K.kvx_ready_create(w.num_layers, 1)
    layer_bytes = P // w.num_layers
    published = [0]

    def serial_step(marks=None, path=K.KVX_PATH_ZEROCOPY):
        e = [T.ev() for _ in range(3)] if marks is not None else None
        if e:
            e[0].record(stream)
        K.kvx_backup(pool, src, host.ptr, P, 0, w.num_layers, stream, path)
        if e:
            e[1].record(stream)
        K.kvx_restore(pool, host.ptr, P, dst, 0, w.num_layers, ready, 0, stream, path)
        if e:
            e[2].record(stream)
            marks.append(e)
        published[0] += n
        while K.kvx_ready_prefix(ready) < published[0]:    # the consumer's view of completion
            pass

    def exchange_step(marks=None):
        e = [T.ev() for _ in range(4)] if marks is not None else None
        if e:
            e[0].record(stream)
        K.kvx_backup(pool, src, host.ptr, P, 0, 1, stream, K.KVX_PATH_ZEROCOPY)
        if e:
            e[1].record(stream)
        for l in range(1, w.num_layers):
            K.kvx_exchange(pool, src, host.ptr, P, (l, l + 1), host.ptr, P, dst, (l - 1, l), ready,
                           0, stream, K.KVX_PATH_ZEROCOPY)
        if e:
            e[2].record(stream)
        K.kvx_restore(pool, host.ptr, P, dst, w.num_layers - 1, w.num_layers, ready, 0, stream,
                      K.KVX_PATH_ZEROCOPY)
        if e:
            e[3].record(stream)
            marks.append(e)
        published[0] += n
        while K.kvx_ready_prefix(ready) < published[0]:
            pass

    def run(step_fn, steps, warmup):
        marks = []
        for _ in range(warmup):
            step_fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step_fn(marks)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, marks

    if args.schedule == "exchange" and w.num_layers > 1:
        wall, marks = run(exchange_step, args.steps, args.warmup)
        per = [m[1].elapsed_time(m[2]) / 1e3 / (w.num_layers - 1) for m in marks]
        step = {"exchange_launch_ms": round(median(per) * 1e3, 4),
                "exchange_achieved": round(2 * layer_bytes / median(per) / GB, 2),
                "exchange_best": round(2 * layer_bytes / min(per) / GB, 2)}
        schedule = ("layer-pipelined: backup of layer 0, then one kvx_exchange per layer (backup of "
                    "layer l+1 and restore of layer l in one launch), then restore of the last layer; "
                    "zero-copy; the host waits for the ready prefix")
    else:
        wall, marks = run(serial_step, args.steps, args.warmup)
        t_bk = [m[0].elapsed_time(m[1]) / 1e3 for m in marks]
        t_rs = [m[1].elapsed_time(m[2]) / 1e3 for m in marks]
        step = {"backup_gbs": round(P / median(t_bk) / GB, 2), "backup_best": round(P / min(t_bk) / GB, 2),
                "restore_gbs": round(P / median(t_rs) / GB, 2), "restore_best": round(P / min(t_rs) / GB, 2)}
        schedule = "backup then restore (zero-copy), the host waits for the ready prefix"
    value = 2 * P * args.steps / wall / GB
    ms = wall / args.steps * 1e3
    log(f"{w.name} step: {ms:.2f} ms -> {value:.2f} GB/s")
    result = {
        "metric": "KV GB/s moved (backup D2H, restore H2D) + % of HBM / host-link roofline",
        "value": round(value, 3), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
        "config": {"workload": w.description, "pages_per_request": n, "layers": w.num_layers,
                   "payload_bytes_per_op": P, "path": "zerocopy", "schedule": schedule,
                   "options": options},
        "roofline": roofline,
        "device_kernels": kern,
        "link_roofline": {"bound": "host link (PCIe 5.0 x16)", "unit": "GB/s",
                          "peak_both_directions": 2 * PCIE_PEAK_GBS, "step": step,
                          "measured_memcpy_peak": peaks, "protocol_bound": pcie_protocol_bound()},
    }

    if not args.no_extras:
        # each host path per direction: 2 warm-up and 10 timed calls, median and best
        per_path = {}
        for name, pth in (("staged", K.KVX_PATH_STAGED), ("zerocopy", K.KVX_PATH_ZEROCOPY)):
            b = lambda: K.kvx_backup(pool, src, host.ptr, P, 0, w.num_layers, stream, pth)  # noqa
            r = lambda: K.kvx_restore(pool, host.ptr, P, dst, 0, w.num_layers, None, 0,  # noqa
                                      stream, pth)
            tb, tb_best = T.stats(b)
            tr, tr_best = T.stats(r)
            per_path[name] = {"backup_gbs": round(P / tb / GB, 2), "backup_best": round(P / tb_best / GB, 2),
                              "backup_frac_d2h_peak": round(P / tb / GB / peaks["d2h"], 4),
                              "restore_gbs": round(P / tr / GB, 2), "restore_best": round(P / tr_best / GB, 2),
                              "restore_frac_h2d_peak": round(P / tr / GB / peaks["h2d"], 4)}
            log(f"{name}: {per_path[name]}")
        result["link_roofline"]["per_path"] = per_path
        # layer-0-ready latency of a restore: the CPU polls layer 0's count
        lat = {}
        for name, pth in (("staged", K.KVX_PATH_STAGED), ("zerocopy", K.KVX_PATH_ZEROCOPY)):
            torch.cuda.synchronize()
            base = K.kvx_layer_ready(ready, 0)
            t0 = time.perf_counter()
            K.kvx_restore(pool, host.ptr, P, dst, 0, w.num_layers, ready, 0, stream, pth)
            while K.kvx_layer_ready(ready, 0) < base + n:
                pass
            t_l0 = time.perf_counter() - t0
            published[0] += n
            while K.kvx_ready_prefix(ready) < published[0]:
                pass
            t_all = time.perf_counter() - t0
            stream.synchronize()
            lat[name] = {"layer0_ms": round(t_l0 * 1e3, 3), "all_layers_ms": round(t_all * 1e3, 3)}
        result["restore_ready_latency"] = lat
        log(f"restore ready latency: {lat}")

    K.kvx_ready_destroy(ready)
    K.kvx_unregister_pool(pool)
    host.free()
    del alloc
    torch.cuda.empty_cache()
    if quiet:
        return result
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w)
        result["cpu_baseline_all_cores"] = cpu_baseline_all_cores(w)
    print(json.dumps(result), flush=True)
    return None


# ---------------------------------------------------------------------------
# --all-workloads: one line per other workload
# ---------------------------------------------------------------------------
def all_workloads():
    """One JSON line per workload with the figures that workload is measured
    by (latency for the tiny pool, layer-0-ready latency for the layer-wise
    MLA restore, HND conversion rates for the TRT-LLM pool, aggregate rate
    with four requests in flight for the mixed stream)."""
    import numpy as np
    import torch

    import synth
    from paged_kv_offload_amd import kvx as K
    from synth.workloads import WORKLOADS, mixed_schedule, request_pair

    stream = torch.cuda.Stream()
    paths = {"staged": K.KVX_PATH_STAGED, "zerocopy": K.KVX_PATH_ZEROCOPY}

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def timed(fn, reps, s=stream):
        out = []
        for _ in range(reps):
            a, b = ev(), ev()
            a.record(s)
            fn()
            b.record(s)
            b.synchronize()
            out.append(a.elapsed_time(b) / 1e3)
        return out

    def batched(fn, reps, per=10, s=stream):
        out = []
        for _ in range(reps):
            a, b = ev(), ev()
            a.record(s)
            for _ in range(per):
                fn()
            b.record(s)
            b.synchronize()
            out.append(a.elapsed_time(b) / 1e3 / per)
        return out

    def make_pool(w):
        alloc = torch.empty(w.alloc_bytes, dtype=torch.uint8, device="cuda")
        synth.fill_alloc_gpu(alloc.data_ptr(), w, w.seed)
        dt = {1: torch.uint8, 2: torch.bfloat16}[w.dtype_bytes]
        t = alloc[w.byte_offset:w.byte_offset + w.pool_bytes].view(dt).view(*w.tensor_shape())
        lay = K.make_layout(w.outer, w.inner, w.num_pages, w.num_layers, w.num_kv, w.page_size,
                            w.num_heads, w.head_dim)
        torch.cuda.synchronize()
        return alloc, K.register_tensor(t, lay, 1)

    def device_rates(w, pool, src, dst, P):
        dev = torch.empty(P, dtype=torch.uint8, device="cuda")
        pk = lambda: K.kvx_backup(pool, src, dev, P, 0, w.num_layers, stream, K.KVX_PATH_DEVICE)  # noqa
        up = lambda: K.kvx_restore(pool, dev, P, dst, 0, w.num_layers, None, 0, stream,  # noqa
                                   K.KVX_PATH_DEVICE)
        # batches of back-to-back launches between the events (the kernel's
        # own duration, as in the main roofline)
        timed(pk, 3)
        tp = median(batched(pk, 5))
        timed(up, 3)
        tu = median(batched(up, 5))
        del dev
        return {"pack_gbs": round(2 * P / tp / GB, 1), "pack_frac": round(2 * P / tp / GB / HBM_PEAK_GBS, 4),
                "unpack_gbs": round(2 * P / tu / GB, 1),
                "unpack_frac": round(2 * P / tu / GB / HBM_PEAK_GBS, 4)}

    # ---- tiny: latency of one call, launch-bound and cache-resident ----
    w = WORKLOADS["tiny"]
    n = w.pages_per_request
    P = w.payload_bytes(n)
    src, dst = request_pair(w)
    alloc, pool = make_pool(w)
    host = K.HostBuffer(P)
    ready = K.kvx_ready_create(w.num_layers, 1)
    dev = torch.empty(P, dtype=torch.uint8, device="cuda")
    res = {"workload": w.description, "payload_bytes_per_op": P, "unit": "us"}
    for name, pth, buf in (("zerocopy", K.KVX_PATH_ZEROCOPY, host.ptr),
                           ("staged", K.KVX_PATH_STAGED, host.ptr),
                           ("device", K.KVX_PATH_DEVICE, dev.data_ptr())):
        b = lambda: K.kvx_backup(pool, src, buf, P, 0, w.num_layers, stream, pth)  # noqa
        r = lambda: K.kvx_restore(pool, buf, P, dst, 0, w.num_layers, ready, 0, stream, pth)  # noqa
        timed(b, 5)
        timed(r, 5)
        wall_b, wall_r = [], []
        for _ in range(50):
            t0 = time.perf_counter()
            b()
            stream.synchronize()
            wall_b.append(time.perf_counter() - t0)
            K.kvx_ready_reset(ready)
            t0 = time.perf_counter()
            r()
            while K.kvx_ready_prefix(ready) < n:
                pass
            wall_r.append(time.perf_counter() - t0)
            stream.synchronize()
        res[name] = {"backup_gpu_us": round(median(timed(b, 50)) * 1e6, 1),
                     "restore_gpu_us": round(median(timed(r, 50)) * 1e6, 1),
                     "backup_call_to_done_us": round(median(wall_b) * 1e6, 1),
                     "restore_call_to_ready_us": round(median(wall_r) * 1e6, 1)}
    # the same calls as descriptors through a submission / completion ring,
    # served in this process: submit to completion reaped
    name = f"/kvx-bench-{os.getpid()}"
    ring = K.kvx_ring_create(name, 64, 1)
    srv = K.kvx_ring_open(name)
    rb = K.make_sqe(K.KVX_OP_BACKUP, 1, 1, 0, 0, src, 0, w.num_layers, K.KVX_PATH_ZEROCOPY)
    rr = K.make_sqe(K.KVX_OP_RESTORE, 2, 1, 0, 0, dst, 0, w.num_layers, K.KVX_PATH_ZEROCOPY)

    def through_ring(q):
        K.kvx_ring_submit(ring, q)
        while True:
            K.kvx_ring_serve(srv, [pool], [host.ptr], [P], None, stream)
            got = K.kvx_ring_reap(ring, 4)
            if got:
                assert got[0][2] == 0, got
                return

    lat = {"backup": [], "restore": []}
    for k in range(60):
        for key, q in (("backup", rb), ("restore", rr)):
            t0 = time.perf_counter()
            through_ring(q)
            if k >= 10:
                lat[key].append(time.perf_counter() - t0)
    # 64 descriptors in flight at once (launches queue on the stream);
    # median of 5 batches
    t_batches = []
    for _ in range(5):
        t0 = time.perf_counter()
        for k in range(64):
            K.kvx_ring_submit(ring, rb if k % 2 == 0 else rr)
        done = 0
        while done < 64:
            K.kvx_ring_serve(srv, [pool], [host.ptr], [P], None, stream)
            done += len(K.kvx_ring_reap(ring, 64))
        t_batches.append(time.perf_counter() - t0)
    t_batch = median(t_batches)
    K.kvx_ring_close(srv)
    K.kvx_ring_close(ring)
    res["ring_zerocopy"] = {"backup_submit_to_completion_us": round(median(lat["backup"]) * 1e6, 1),
                            "restore_submit_to_completion_us": round(median(lat["restore"]) * 1e6, 1),
                            "ops_per_s_64_in_flight": round(64 / t_batch, 0)}
    print(json.dumps({"tiny": res}), flush=True)
    K.kvx_ready_destroy(ready)
    K.kvx_unregister_pool(pool)
    host.free()
    del alloc, dev

    # ---- mla: four requests, layer-wise restore, layer-0-ready latency ----
    w = WORKLOADS["mla_fp8"]
    n = w.pages_per_request
    P = w.payload_bytes(n)
    alloc, pool = make_pool(w)
    host = K.HostBuffer(P)
    ready = K.kvx_ready_create(w.num_layers, 1)
    res = {"workload": w.description, "payload_bytes_per_op": P}
    res.update(device_rates(w, pool, *request_pair(w, 0), P))
    consumer = torch.cuda.Stream()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for name, pth in paths.items():
        per = []
        for r in range(4):
            src, dst = request_pair(w, r)
            tb = median(timed(lambda: K.kvx_backup(pool, src, host.ptr, P, 0, w.num_layers,
                                                   stream, pth), 2))
            # a CPU consumer polls layer 0's count, then the prefix; a GPU
            # consumer on its own stream waits for layer 0 with the bounded
            # wait kernel (its end is timed against the restore's start)
            K.kvx_ready_reset(ready)
            torch.cuda.synchronize()
            e_start, e_gpu = ev(), ev()
            t0 = time.perf_counter()
            e_start.record(stream)
            K.kvx_restore(pool, host.ptr, P, dst, 0, w.num_layers, ready, 0, stream, pth)
            K.kvx_ready_wait_gpu(ready, 0, n, consumer, 10_000_000, status.data_ptr())
            e_gpu.record(consumer)
            while K.kvx_layer_ready(ready, 0) < n:
                pass
            t_l0 = time.perf_counter() - t0
            while K.kvx_ready_prefix(ready) < n:
                pass
            t_all = time.perf_counter() - t0
            torch.cuda.synchronize()
            assert int(status.item()) == 1, "the GPU consumer gave up waiting for layer 0"
            per.append((P / tb / GB, t_l0, t_all, e_start.elapsed_time(e_gpu) / 1e3))
        res[name] = {"backup_gbs": round(median([x[0] for x in per]), 2),
                     "layer0_ready_ms": round(median([x[1] for x in per]) * 1e3, 3),
                     "gpu_consumer_layer0_ms": round(median([x[3] for x in per]) * 1e3, 3),
                     "all_layers_ready_ms": round(median([x[2] for x in per]) * 1e3, 3),
                     "restore_gbs": round(P / median([x[2] for x in per]) / GB, 2)}
    print(json.dumps({"mla_fp8": res}), flush=True)
    K.kvx_ready_destroy(ready)
    K.kvx_unregister_pool(pool)
    host.free()
    del alloc
    torch.cuda.empty_cache()

    # ---- trtllm: head-major pool at a byte offset ----
    w = WORKLOADS["trtllm_hnd"]
    n = w.pages_per_request
    P = w.payload_bytes(n)
    src, dst = request_pair(w)
    alloc, pool = make_pool(w)
    host = K.HostBuffer(P)
    res = {"workload": w.description, "payload_bytes_per_op": P}
    res.update(device_rates(w, pool, src, dst, P))
    for name, pth in paths.items():
        b = lambda: K.kvx_backup(pool, src, host.ptr, P, 0, w.num_layers, stream, pth)  # noqa
        r = lambda: K.kvx_restore(pool, host.ptr, P, dst, 0, w.num_layers, None, 0, stream, pth)  # noqa
        timed(b, 1)
        timed(r, 1)
        res[name] = {"backup_gbs": round(P / median(timed(b, 3)) / GB, 2),
                     "restore_gbs": round(P / median(timed(r, 3)) / GB, 2)}
    print(json.dumps({"trtllm_hnd": res}), flush=True)
    K.kvx_unregister_pool(pool)
    host.free()
    del alloc
    torch.cuda.empty_cache()

    # ---- host tier: the llama8b request through slot-addressed host pools ----
    w = WORKLOADS["llama8b"]
    n, S = w.pages_per_request, 1024
    P, HB = w.payload_bytes(n), w.payload_bytes(S)
    alloc, pool = make_pool(w)
    rng = np.random.default_rng(w.seed + 70)
    res = {"workload": w.description + f"; host tier of {S} slots", "payload_bytes_per_op": P}
    host = K.HostBuffer(HB)
    dev = torch.empty(HB, dtype=torch.uint8, device="cuda")
    for name, pth, buf in (("zerocopy", K.KVX_PATH_ZEROCOPY, host.ptr),
                           ("device", K.KVX_PATH_DEVICE, dev.data_ptr())):
        src, dst = request_pair(w)
        slots = rng.permutation(S)[:n].astype(np.int32)
        b = lambda: K.kvx_backup_slots(pool, src, slots, buf, HB, S, 0, w.num_layers, stream, pth)  # noqa
        r = lambda: K.kvx_restore_slots(pool, buf, HB, S, slots, dst, 0, w.num_layers, None, 0,  # noqa
                                        stream, pth)
        timed(b, 2)
        timed(r, 2)
        if pth == K.KVX_PATH_DEVICE:
            tb, tr = median(batched(b, 3)), median(batched(r, 3))
        else:
            tb, tr = median(timed(b, 5)), median(timed(r, 5))
        if pth == K.KVX_PATH_DEVICE:
            res[name] = {"backup_slots_gbs": round(2 * P / tb / GB, 1),
                         "backup_slots_frac_hbm": round(2 * P / tb / GB / HBM_PEAK_GBS, 4),
                         "restore_slots_gbs": round(2 * P / tr / GB, 1),
                         "restore_slots_frac_hbm": round(2 * P / tr / GB / HBM_PEAK_GBS, 4)}
        else:
            res[name] = {"backup_slots_gbs": round(P / tb / GB, 2),
                         "restore_slots_gbs": round(P / tr / GB, 2)}
    del dev
    # write-through: eight requests in a row, each reserved, backed up and
    # committed; from the fifth on the tier is full and evicts a request's
    # worth of entries per call
    tier = K.kvx_tier_create(S, 1)
    perm = synth.page_perm(w.seed + 71, w.num_pages)
    t_res, evicted = [], 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for r in range(8):
        pages = perm[r * n:(r + 1) * n]
        keys = np.arange(r * n, (r + 1) * n, dtype=np.uint64) + 1
        c0 = time.perf_counter()
        sl, ev_keys = K.kvx_tier_backup(tier, pool, keys, pages, host.ptr, HB, stream,
                                        K.KVX_PATH_ZEROCOPY)
        t_res.append(time.perf_counter() - c0)
        evicted += ev_keys.size
        stream.synchronize()
        K.kvx_tier_commit(tier, sl)
    wall = time.perf_counter() - t0
    res["write_through"] = {"requests": 8, "gbs": round(8 * P / wall / GB, 2),
                            "evicted_entries": int(evicted),
                            "call_enqueue_us": round(median(t_res) * 1e6, 1)}
    # a miss stored while a hit is loaded: kvx_tier_exchange backs up a new
    # request (evicting a request's worth of entries) while it restores a
    # resident one into other pages, both directions at once
    rates = []
    hkeys = np.arange(7 * n, 8 * n, dtype=np.uint64) + 1     # the last request is resident
    for r in range(6):
        nkeys = np.arange((8 + r) * n, (9 + r) * n, dtype=np.uint64) + 1
        stream.synchronize()
        t0 = time.perf_counter()
        bsl, _, rsl = K.kvx_tier_exchange(tier, pool, nkeys, perm[:n], hkeys, perm[n:2 * n], host.ptr,
                                          HB, None, 0, stream, K.KVX_PATH_ZEROCOPY)
        stream.synchronize()
        rates.append(2 * P / (time.perf_counter() - t0) / GB)
        assert (rsl >= 0).all(), "a resident request missed"
        K.kvx_tier_commit(tier, bsl)
        K.kvx_tier_release(tier, rsl)
        K.kvx_tier_invalidate(tier, nkeys)              # room for the next round's request
    res["tier_exchange"] = {"gbs": round(median(rates[1:]), 2), "bytes_per_call": 2 * P}
    K.kvx_tier_destroy(tier)
    print(json.dumps({"host_tier": res}), flush=True)
    log(f"host tier: {res}")
    host.free()
    K.kvx_unregister_pool(pool)
    del alloc
    torch.cuda.empty_cache()


def cpu_baseline(w, budget_s: float = 12.0):
    """The oracle's backup + restore byte loops, single-threaded, on a host
    pool with the workload's piece shape and request size (n fragmented
    pages) but 2n pages and at most 4 layers; one layer per pass, passes
    repeated until about budget_s seconds of CPU work."""
    import numpy as np

    import oracle
    import synth

    n = w.pages_per_request
    nl = min(w.num_layers, 4)
    sample = w.scaled(num_pages=2 * n, num_layers=nl)
    L = oracle_layout_of(oracle, sample)
    # only the shape matters for the timing; the bytes are a constant pattern
    alloc = np.full(sample.pool_bytes, 0x5A, dtype=np.uint8)
    perm = synth.page_perm(w.seed, 2 * n)
    src, dst = perm[:n].copy(), perm[n:].copy()
    host = np.zeros(sample.host_bytes(n), dtype=np.uint8)
    moved, t, passes = 0, 0.0, 0
    while t < budget_s:
        l = passes % nl
        t0 = time.perf_counter()
        oracle.backup(L, alloc, src, l, l + 1, host=host)
        oracle.restore(L, alloc, host, dst, l, l + 1, out=alloc)
        t += time.perf_counter() - t0
        moved += 2 * sample.num_kv * n * sample.piece_bytes
        passes += 1
    gbs = moved / t / GB
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{passes} single-layer backup+restore passes of {n} fragmented pages x "
                      f"{sample.num_kv} x {sample.piece_bytes} B pieces on a {2 * n}-page, "
                      f"{nl}-layer host pool ({moved / GB:.2f} GB moved in {t:.1f} s)",
            "cpu_model": cpu_model()}


def oracle_layout_of(oracle, w):
    return oracle.Layout(outer=tuple({"page": oracle.PAGE, "layer": oracle.LAYER,
                                      "kv": oracle.KV}[a] for a in w.outer),
                         inner=oracle.NHD if w.inner == "NHD" else oracle.HND,
                         num_pages=w.num_pages, num_layers=w.num_layers, num_kv=w.num_kv,
                         page_size=w.page_size, num_heads=w.num_heads, head_dim=w.head_dim,
                         dtype_bytes=w.dtype_bytes)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_all_cores(w, budget_s: float = 8.0, max_threads: int = 16):
    """The oracle from one host thread per core (the process's affinity set,
    at most max_threads) over the (layer, kv, page) pieces of ONE host pool
    and one request: thread k takes every threads-th page of the request and
    runs backup + restore passes of its pages' pieces in every layer and kv
    (the slot-addressed oracle calls, each page to its own slot of the
    request's packed buffer, so no two threads touch the same bytes) for
    about budget_s seconds. The oracle's C functions run without the
    interpreter lock, so the threads run in parallel; the oracle itself is
    unchanged."""
    import threading

    import numpy as np

    import oracle
    import synth

    n = w.pages_per_request
    # every thread gets at least one page of the request
    threads = max(1, min(max_threads, len(os.sched_getaffinity(0)), n))
    sample = w.scaled(num_pages=2 * n, num_layers=4)
    NL = sample.num_layers
    L = oracle_layout_of(oracle, sample)
    alloc = np.full(sample.pool_bytes, 0x5A, dtype=np.uint8)
    host = np.zeros(sample.host_bytes(n), dtype=np.uint8)
    perm = synth.page_perm(w.seed, 2 * n)
    src, dst = perm[:n].copy(), perm[n:].copy()
    mine = [np.arange(k, n, threads, dtype=np.int32) for k in range(threads)]
    passes = [0] * threads
    start = threading.Barrier(threads + 1)
    stop = threading.Event()

    def worker(k):
        slots = mine[k]
        s_ids, d_ids = src[slots].copy(), dst[slots].copy()
        start.wait()
        while not stop.is_set():
            oracle.backup_slots(L, alloc, s_ids, slots, n, 0, NL, host=host)
            oracle.restore_slots(L, alloc, host, slots, d_ids, n, 0, NL, out=alloc)
            passes[k] += 1

    ths = [threading.Thread(target=worker, args=(k,)) for k in range(threads)]
    for th in ths:
        th.start()
    start.wait()
    t0 = time.perf_counter()
    time.sleep(budget_s)
    stop.set()
    for th in ths:
        th.join()
    t = time.perf_counter() - t0     # includes each thread finishing its last pass
    moved = sum(2 * NL * sample.num_kv * len(mine[k]) * sample.piece_bytes * passes[k] for k in range(threads))
    return {"value": round(moved / t / GB, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"backup+restore passes of one {n}-page request ({sample.num_kv} x "
                      f"{sample.piece_bytes} B pieces, {NL} layers) over one {2 * n}-page host pool, "
                      f"the request's pages dealt out to {threads} threads, each moving its pages' "
                      f"pieces in every layer ({sum(passes)} thread passes, {moved / GB:.2f} GB moved "
                      f"in {t:.1f} s)",
            "cpu_model": cpu_model()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="mixed",
                    help="mixed (the 128-request hit/miss stream, default) or a single-request "
                         "workload: llama8b, mla_fp8, trtllm_hnd, tiny, token_pages (the llama8b "
                         "shape at one token per page)")
    ap.add_argument("--schedule", choices=["exchange", "streams"], default=None,
                    help="mixed: streams (default) = one call per request on four streams, exchange = "
                         "backup + next restore in one kvx_exchange on two streams; single-request "
                         "workloads: exchange (default) = layer-pipelined, streams = serial backup then "
                         "restore")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the other schedules, the per-path rates and the latency legs")
    ap.add_argument("--kernel-only", action="store_true",
                    help="time only the device pack/unpack kernels (for counter runs)")
    ap.add_argument("--set", action="append", default=[], metavar="OPTION=VALUE",
                    help="kvx_set_option before timing, e.g. --set hnd_lds=0 (names of the "
                         "KVX_OPT_* constants, lower case); recorded in config.options")
    ap.add_argument("--all-workloads", action="store_true",
                    help="instead of the headline, print one line per other workload with its own "
                         "figures (tiny: latency; mla: layer-0-ready; trtllm: HND rates; host tier)")
    args = ap.parse_args()
    if args.schedule is None:
        args.schedule = "streams" if args.workload == "mixed" and not args.all_workloads else "exchange"
    if args.gpus != 1:
        print(json.dumps({"error": "kvx moves KV between one GPU and its host tier; this benchmark "
                                   "measures one GPU (run with --gpus 1)"}), flush=True)
        sys.exit(2)

    # The mixed stream keeps requests in flight on several streams. HIP gives
    # a process 4 hardware queues by default and streams share them
    # round-robin; with the default stream, five streams would put two
    # requests on one queue, and those run one after the other.
    try:
        queues = int(os.environ.get("GPU_MAX_HW_QUEUES", "4"))
    except ValueError:
        queues = 4
    if queues < 8:
        os.environ["GPU_MAX_HW_QUEUES"] = "8"   # read by the HIP runtime when torch loads it

    import torch

    from paged_kv_offload_amd import kvx as K
    from synth.workloads import WORKLOADS

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    K.lib()
    options = {}
    for item in args.set:
        name, _, value = item.partition("=")
        const = getattr(K, "KVX_OPT_" + name.upper(), None)
        if const is None or not value.lstrip("-").isdigit():
            print(json.dumps({"error": f"--set {item}: unknown option or non-integer value"}), flush=True)
            sys.exit(2)
        K.kvx_set_option(const, int(value))
        options[name.lower()] = int(value)
    if args.all_workloads:
        all_workloads()
    elif args.workload == "mixed":
        mixed_main(args, options)
    else:
        single_main(args, options, WORKLOADS[args.workload])


if __name__ == "__main__":
    main()
