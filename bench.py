"""Benchmark: KV bytes moved per second by kvx backup (GPU pool -> pinned host)
and restore (pinned host -> other GPU pages, with per-layer publish) on one
MI355X.

One step = the whole hot path over one request of the Llama-3-8B-shaped bf16
pool (32 layers, K+V, 8 KV heads, head_dim 128, page size 64, 2048 pages):
BACKUP of 256 fragmented pages (16,384 tokens, 2 GiB) to pinned host memory
(validation + run planning, then the gather kernel writing the packed buffer
over the host link), RESTORE of that buffer into 256 other pages with
per-layer publish, and the ready-prefix query, which the host polls until
the whole request is published.

The default schedule is layer-pipelined on the zero-copy path: the backup of
layer 0, then 31 kvx_exchange launches that each back up layer l + 1 while
they restore layer l (the restore reads what the previous launch wrote),
then the restore of layer 31. It moves the same bytes, with the same
results, as the serial schedule (--schedule serial: backup of every layer,
then restore of every layer, on --path), but keeps both directions of the
host link busy at once.

value = 2 x 2 GiB x steps / wall time of the steps (GB = 1e9 B). The pool is
resident in HBM when the timed region starts; crossing the host link is
part of the method (the host tier is where BACKUP writes and RESTORE reads).

Also reported: the device pack/unpack kernels alone against the HBM peak
(the roofline), the step's kernels against the host link (link_roofline,
with the pinned hipMemcpyAsync peaks measured in the same run), the other
schedule, both host paths per direction, layer-pipelined schedules on two
streams, the layer-0-ready latency, and the CPU oracle on a bounded sample
(a baseline only).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--schedule exchange|serial]
       [--path staged|zerocopy] [--no-cpu-baseline] [--kernel-only] [--no-extras]
       [--all-workloads]
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


# HBM bytes per launch of the roofline kernel from the two rocprofv3 --pmc runs
# (FETCH_SIZE, WRITE_SIZE, scaled by a plain 2 GiB device copy in the same
# run; see profiles/pack_kernel_llama8b.txt). Valid only for the kernel source
# they were taken on: reported as null once kernels.hip changes.
MEASURED_TRAFFIC = {"workload": "llama8b", "kernels_hip_sha256": "164fbcb2bd67b348945947576205716d4e5aa6b50254fa098284582380e27001",
                    "bytes_per_launch": 4295172094}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def median(xs):
    return statistics.median(xs) if xs else float("nan")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--schedule", choices=["exchange", "serial"], default="exchange",
                    help="exchange: layer-pipelined kvx_exchange launches (zero-copy); serial: "
                         "backup then restore on --path")
    ap.add_argument("--path", choices=["staged", "zerocopy"], default="zerocopy",
                    help="host path of the serial schedule")
    ap.add_argument("--workload", default="llama8b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the per-path, pipelined and latency measurements")
    ap.add_argument("--kernel-only", action="store_true",
                    help="time only the device pack/unpack kernels (for counter runs)")
    ap.add_argument("--set", action="append", default=[], metavar="OPTION=VALUE",
                    help="kvx_set_option before timing, e.g. --set hnd_lds=0 (names of the "
                         "KVX_OPT_* constants, lower case); recorded in config.options")
    ap.add_argument("--all-workloads", action="store_true",
                    help="instead of the headline step, print one line per workload with its own "
                         "figures (tiny: latency; mla: layer-0-ready; trtllm: HND rates; mixed: "
                         "4 streams in flight)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "kvx moves KV between one GPU and its host tier; this benchmark "
                                   "measures one GPU (run with --gpus 1)"}), flush=True)
        sys.exit(2)

    if args.all_workloads:
        # The mixed leg keeps four requests in flight on four streams. HIP
        # gives a process 4 hardware queues by default and streams share
        # them round-robin; with the default stream that is five streams, so
        # two requests would share a queue and run one after the other.
        try:
            queues = int(os.environ.get("GPU_MAX_HW_QUEUES", "4"))
        except ValueError:
            queues = 4
        if queues < 8:
            os.environ["GPU_MAX_HW_QUEUES"] = "8"   # read by the HIP runtime when torch loads it

    import numpy as np
    import torch

    import synth
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
        return
    w = WORKLOADS[args.workload]
    n = w.pages_per_request
    P = w.payload_bytes(n)
    perm = synth.page_perm(w.seed, w.num_pages)
    src = np.ascontiguousarray(perm[:n])
    dst = np.ascontiguousarray(perm[n:2 * n])
    stream = torch.cuda.Stream()
    log(f"workload {w.name}: pool {w.pool_bytes / 2**30:.1f} GiB, payload {P / 2**30:.2f} GiB/op")

    # ---- pool in HBM, filled from the seeded generator ----
    alloc = torch.empty(w.alloc_bytes, dtype=torch.uint8, device="cuda")
    synth.fill_alloc_gpu(alloc.data_ptr(), w, w.seed)
    dt = {1: torch.uint8, 2: torch.bfloat16}[w.dtype_bytes]
    pool_t = alloc[w.byte_offset:w.byte_offset + w.pool_bytes].view(dt).view(*w.tensor_shape())
    layout = K.make_layout(w.outer, w.inner, w.num_pages, w.num_layers, w.num_kv, w.page_size,
                           w.num_heads, w.head_dim)
    pool = K.register_tensor(pool_t, layout, 1)
    dev_packed = torch.empty(P, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def timed(fn, reps, s=stream):
        """Per-repetition durations (s) from HIP events on stream s."""
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
        """Per-launch durations (s): HIP events on stream s around `per`
        back-to-back calls, `reps` times."""
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

    # ---- device pack / unpack kernels alone (HBM roofline) ----
    # one launch packs the whole request: 32 layers x 2 x 256 pieces of 128 KiB
    def pack():
        K.kvx_backup(pool, src, dev_packed, P, 0, w.num_layers, stream, K.KVX_PATH_DEVICE)

    def unpack():
        K.kvx_restore(pool, dev_packed, P, dst, 0, w.num_layers, None, 0, stream,
                      K.KVX_PATH_DEVICE)

    # events bracket a batch of back-to-back launches, so the host work of
    # each call overlaps the previous kernel and the per-launch average is
    # the kernel's own duration (what the kernel trace reports)
    kreps = max(args.steps, 10)
    timed(pack, 3)
    t_pack = batched(pack, kreps)
    timed(unpack, 3)
    t_unpack = batched(unpack, kreps)
    pack_gbs = 2 * P / median(t_pack) / GB
    unpack_gbs = 2 * P / median(t_unpack) / GB
    # the same unpack publishing every layer into a ready object (the
    # queue-driven kernel: one count per layer and block of units)
    ready_k = K.kvx_ready_create(w.num_layers, 1)

    def unpack_publish():
        K.kvx_restore(pool, dev_packed, P, dst, 0, w.num_layers, ready_k, 0, stream,
                      K.KVX_PATH_DEVICE)

    timed(unpack_publish, 3)
    t_unpack_pub = batched(unpack_publish, kreps)
    K.kvx_ready_destroy(ready_k)
    unpack_pub_gbs = 2 * P / median(t_unpack_pub) / GB
    log(f"device pack {median(t_pack) * 1e3:.3f} ms = {pack_gbs:.0f} GB/s (read+write); "
        f"unpack {median(t_unpack) * 1e3:.3f} ms = {unpack_gbs:.0f} GB/s; "
        f"unpack with per-layer publish {unpack_pub_gbs:.0f} GB/s")

    # a plain device-to-device copy of the same byte count (the in-run
    # achievable line, and the calibration kernel for the traffic counters)
    d2d_a = torch.empty(P, dtype=torch.uint8, device="cuda")
    with torch.cuda.stream(stream):
        timed(lambda: d2d_a.copy_(dev_packed), 2)
        t_d2d = timed(lambda: d2d_a.copy_(dev_packed), 5)
    d2d_gbs = 2 * P / median(t_d2d) / GB
    del d2d_a
    log(f"D2D copy {d2d_gbs:.0f} GB/s (read+write)")
    traffic = None
    try:
        import hashlib
        with open(os.path.join(ROOT, "paged_kv_offload_amd", "csrc", "kernels.hip"), "rb") as f:
            if (hashlib.sha256(f.read()).hexdigest() == MEASURED_TRAFFIC["kernels_hip_sha256"]
                    and w.name == MEASURED_TRAFFIC["workload"]):
                traffic = MEASURED_TRAFFIC["bytes_per_launch"]
    except OSError:
        pass
    roofline = {"bound": "hbm",
                "kernel": f"kvx_move_kernel<GATHER> (pack of one {P / 2**30:.2f} GiB {w.name} request, "
                          f"device path)",
                "achieved": round(pack_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(pack_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": 2 * P,
                "avg_launch_ms": round(median(t_pack) * 1e3, 4)}
    if args.kernel_only:
        print(json.dumps({"roofline": roofline, "unpack_gbs": round(unpack_gbs, 1),
                          "unpack_publish_gbs": round(unpack_pub_gbs, 1),
                          "d2d_copy_gbs": round(d2d_gbs, 1), "options": options}), flush=True)
        return

    # ---- pinned host-link peaks: 1 GiB hipMemcpyAsync, median of 10 ----
    peak_bytes = 1 << 30
    pin = torch.empty(peak_bytes, dtype=torch.uint8, pin_memory=True)
    pin2 = torch.empty(peak_bytes, dtype=torch.uint8, pin_memory=True)
    dev1 = torch.empty(peak_bytes, dtype=torch.uint8, device="cuda")
    dev2 = torch.empty(peak_bytes, dtype=torch.uint8, device="cuda")
    sb = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        timed(lambda: pin.copy_(dev1, non_blocking=True), 2)
        t_d2h = timed(lambda: pin.copy_(dev1, non_blocking=True), 10)
        t_h2d = timed(lambda: dev1.copy_(pin, non_blocking=True), 10)
    bidir = []
    for _ in range(5):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(stream):
            pin.copy_(dev1, non_blocking=True)
        with torch.cuda.stream(sb):
            dev2.copy_(pin2, non_blocking=True)
        torch.cuda.synchronize()
        bidir.append(time.perf_counter() - t0)
    d2h_peak = peak_bytes / median(t_d2h) / GB
    h2d_peak = peak_bytes / median(t_h2d) / GB
    bidir_peak = 2 * peak_bytes / median(bidir) / GB
    del pin, pin2, dev1, dev2
    log(f"pinned memcpy peak: D2H {d2h_peak:.1f} GB/s, H2D {h2d_peak:.1f} GB/s, "
        f"both directions at once {bidir_peak:.1f} GB/s")

    # ---- the step ----
    host = K.HostBuffer(P)
    ready = K.kvx_ready_create(w.num_layers, 1)
    path = {"staged": K.KVX_PATH_STAGED, "zerocopy": K.KVX_PATH_ZEROCOPY}[args.path]
    layer_bytes = P // w.num_layers

    # Serial schedule: BACKUP of every layer, then RESTORE of every layer.
    # HIP events on the stream the kernels run on bracket the backup and the
    # restore (on the zero-copy path each call is one kernel launch).
    def serial_step(marks=None, path=path):
        K.kvx_ready_reset(ready)
        e = [ev() for _ in range(3)] if marks is not None else None
        if e:
            e[0].record(stream)
        K.kvx_backup(pool, src, host.ptr, P, 0, w.num_layers, stream, path)
        if e:
            e[1].record(stream)
        K.kvx_restore(pool, host.ptr, P, dst, 0, w.num_layers, ready, 0, stream, path)
        if e:
            e[2].record(stream)
            marks.append(e)
        while K.kvx_ready_prefix(ready) < n:    # the consumer's view of completion
            pass

    # Layer-pipelined schedule on the zero-copy path: BACKUP of layer 0, then
    # one kvx_exchange per layer that backs up layer l + 1 while it restores
    # layer l (the restore reads what the previous launch wrote), then the
    # RESTORE of the last layer. Same bytes, same results, per-layer publish;
    # both directions of the host link carry data at once.
    def exchange_step(marks=None):
        K.kvx_ready_reset(ready)
        e = [ev() for _ in range(4)] if marks is not None else None
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
        while K.kvx_ready_prefix(ready) < n:
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

    serial_peak = 2 / (1 / d2h_peak + 1 / h2d_peak)

    def serial_report(wall, marks, steps):
        t_bk = median([m[0].elapsed_time(m[1]) / 1e3 for m in marks])
        t_rs = median([m[1].elapsed_time(m[2]) / 1e3 for m in marks])
        t_bk_best = min(m[0].elapsed_time(m[1]) / 1e3 for m in marks)
        t_rs_best = min(m[1].elapsed_time(m[2]) / 1e3 for m in marks)
        gbs = 2 * P * steps / wall / GB
        return gbs, {
            "gbs": round(gbs, 3), "ms_per_step": round(wall / steps * 1e3, 3),
            "backup_achieved": round(P / t_bk / GB, 2), "restore_achieved": round(P / t_rs / GB, 2),
            "backup_best": round(P / t_bk_best / GB, 2), "restore_best": round(P / t_rs_best / GB, 2),
            "backup_frac_of_pcie": round(P / t_bk / GB / PCIE_PEAK_GBS, 4),
            "restore_frac_of_pcie": round(P / t_rs / GB / PCIE_PEAK_GBS, 4),
            "backup_frac_of_measured": round(P / t_bk / GB / d2h_peak, 4),
            "restore_frac_of_measured": round(P / t_rs / GB / h2d_peak, 4),
            "frac_of_serial_measured_peak": round(gbs / serial_peak, 4)}

    def exchange_report(wall, marks, steps):
        per = [m[1].elapsed_time(m[2]) / 1e3 / (w.num_layers - 1) for m in marks]
        t_x, t_x_best = median(per), min(per)
        t_b0 = median([m[0].elapsed_time(m[1]) / 1e3 for m in marks])
        t_rl = median([m[2].elapsed_time(m[3]) / 1e3 for m in marks])
        gbs = 2 * P * steps / wall / GB
        both = 2 * PCIE_PEAK_GBS
        return gbs, {
            "gbs": round(gbs, 3), "ms_per_step": round(wall / steps * 1e3, 3),
            "exchange_launch_ms": round(t_x * 1e3, 4),
            "exchange_achieved": round(2 * layer_bytes / t_x / GB, 2),
            "exchange_best": round(2 * layer_bytes / t_x_best / GB, 2),
            "exchange_frac_of_pcie_both_directions": round(2 * layer_bytes / t_x / GB / both, 4),
            "exchange_frac_of_measured_both_directions": round(2 * layer_bytes / t_x / GB / bidir_peak, 4),
            "first_backup_gbs": round(layer_bytes / t_b0 / GB, 2),
            "last_restore_gbs": round(layer_bytes / t_rl / GB, 2)}

    if args.schedule == "exchange":
        wall, marks = run(exchange_step, args.steps, args.warmup)
        value, main_rep = exchange_report(wall, marks, args.steps)
        schedule = ("layer-pipelined: backup of layer 0, then one kvx_exchange per layer (backup of "
                    "layer l+1 and restore of layer l in one launch), then restore of the last "
                    "layer; zero-copy; the host waits for the ready prefix")
        path_name = "zerocopy"
    else:
        wall, marks = run(serial_step, args.steps, args.warmup)
        value, main_rep = serial_report(wall, marks, args.steps)
        schedule = "backup then restore, host waits for the ready prefix"
        path_name = args.path
    ms_per_step = wall / args.steps * 1e3
    log(f"step ({args.schedule}, {path_name}): {ms_per_step:.2f} ms -> {value:.2f} GB/s")

    if args.schedule == "exchange":
        link = {"bound": "host link (PCIe 5.0 x16, both directions at once)",
                "kernels": "the step's kvx_exchange launches (zero-copy backup of one layer and restore "
                           "of another in each), HIP events in the timed region",
                "achieved": main_rep["exchange_achieved"], "best": main_rep["exchange_best"],
                "unit": "GB/s", "peak": 2 * PCIE_PEAK_GBS,
                "frac": main_rep["exchange_frac_of_pcie_both_directions"],
                "frac_of_measured_both_directions": main_rep["exchange_frac_of_measured_both_directions"],
                "step": main_rep}
    else:
        link = {"bound": "host link (PCIe 5.0 x16)",
                "kernels": f"the step's {path_name} backup and restore, HIP events in the timed region",
                "unit": "GB/s", "peak": PCIE_PEAK_GBS, "step": main_rep}
    link["measured_memcpy_peak"] = {"d2h": round(d2h_peak, 2), "h2d": round(h2d_peak, 2),
                                    "both_directions": round(bidir_peak, 2)}
    proto = pcie_protocol_bound()
    link["protocol_bound"] = proto
    if args.schedule == "exchange":
        link["frac_of_protocol_bound"] = round(main_rep["exchange_achieved"] / proto["both_directions"], 4)

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
        "config": {"workload": w.description, "pages_per_request": n, "layers": w.num_layers,
                   "payload_bytes_per_op": P, "path": path_name, "schedule": schedule,
                   "options": options},
        "roofline": roofline,
        "unpack_roofline": {"achieved": round(unpack_gbs, 1), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(unpack_gbs / HBM_PEAK_GBS, 4),
                            "with_per_layer_publish": {
                                "achieved": round(unpack_pub_gbs, 1),
                                "frac": round(unpack_pub_gbs / HBM_PEAK_GBS, 4)}},
        "d2d_copy_gbs": round(d2d_gbs, 1),
        "link_roofline": link,
    }

    if not args.no_extras:
        # the other schedule, same number of steps
        if args.schedule == "exchange":
            wall2, marks2 = run(lambda m=None: serial_step(m, K.KVX_PATH_ZEROCOPY), args.steps, 1)
            _, rep2 = serial_report(wall2, marks2, args.steps)
            result["link_roofline"]["serial_step_zerocopy"] = rep2
        else:
            wall2, marks2 = run(exchange_step, args.steps, 1)
            _, rep2 = exchange_report(wall2, marks2, args.steps)
            result["link_roofline"]["exchange_step"] = rep2
        log(f"other schedule: {rep2['gbs']} GB/s")

    if not args.no_extras:
        extras = {}
        for name, pth in (("staged", K.KVX_PATH_STAGED), ("zerocopy", K.KVX_PATH_ZEROCOPY)):
            b = lambda: K.kvx_backup(pool, src, host.ptr, P, 0, w.num_layers, stream, pth)  # noqa
            r = lambda: K.kvx_restore(pool, host.ptr, P, dst, 0, w.num_layers, ready, 0,  # noqa
                                      stream, pth)
            timed(b, 1)
            tb = timed(b, 3)
            timed(r, 1)
            tr = timed(r, 3)
            extras[name] = {"backup_gbs": round(P / median(tb) / GB, 2),
                            "backup_frac_d2h_peak": round(P / median(tb) / GB / d2h_peak, 4),
                            "restore_gbs": round(P / median(tr) / GB, 2),
                            "restore_frac_h2d_peak": round(P / median(tr) / GB / h2d_peak, 4)}
            log(f"{name}: backup {extras[name]['backup_gbs']} GB/s, "
                f"restore {extras[name]['restore_gbs']} GB/s")
        result["link_roofline"]["per_path"] = extras

        # layer-pipelined: restore of layer group g runs on a second stream
        # while group g+1 is backed up, so both link directions carry data
        def pipelined(pth, group=2):
            K.kvx_ready_reset(ready)
            for l0 in range(0, w.num_layers, group):
                l1 = min(w.num_layers, l0 + group)
                K.kvx_backup(pool, src, host.ptr, P, l0, l1, stream, pth)
                e = torch.cuda.Event()
                e.record(stream)
                sb.wait_event(e)
                K.kvx_restore(pool, host.ptr, P, dst, l0, l1, ready, 0, sb, pth)
            while K.kvx_ready_prefix(ready) < n:
                pass
        pipe = {}
        for name, pth in (("staged", K.KVX_PATH_STAGED), ("zerocopy", K.KVX_PATH_ZEROCOPY)):
            pipelined(pth)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(3):
                pipelined(pth)
            torch.cuda.synchronize()
            pipe[name] = round(2 * P * 3 / (time.perf_counter() - t0) / GB, 2)
        # the same schedule in one stream with kvx_exchange: each launch
        # backs up layer group g + 1 while it restores group g
        def exchanged(group):
            K.kvx_ready_reset(ready)
            G = (w.num_layers + group - 1) // group
            rng = lambda g: (g * group, min(w.num_layers, (g + 1) * group))  # noqa: E731
            K.kvx_backup(pool, src, host.ptr, P, *rng(0), stream, K.KVX_PATH_ZEROCOPY)
            for g in range(1, G):
                K.kvx_exchange(pool, src, host.ptr, P, rng(g), host.ptr, P, dst, rng(g - 1),
                               ready, 0, stream, K.KVX_PATH_ZEROCOPY)
            K.kvx_restore(pool, host.ptr, P, dst, *rng(G - 1), ready, 0, stream,
                          K.KVX_PATH_ZEROCOPY)
            while K.kvx_ready_prefix(ready) < n:
                pass
        for group in (1, 2, 4):
            exchanged(group)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(3):
                exchanged(group)
            torch.cuda.synchronize()
            pipe[f"zerocopy_exchange_group{group}"] = round(2 * P * 3 / (time.perf_counter() - t0) / GB, 2)
        result["layer_pipelined_gbs"] = pipe
        log(f"layer-pipelined step: {pipe}")

        # layer-0-ready latency of a restore: the CPU polls layer 0's count
        lat = {}
        for name, pth in (("staged", K.KVX_PATH_STAGED), ("zerocopy", K.KVX_PATH_ZEROCOPY)):
            K.kvx_ready_reset(ready)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            K.kvx_restore(pool, host.ptr, P, dst, 0, w.num_layers, ready, 0, stream, pth)
            while K.kvx_layer_ready(ready, 0) < n:
                pass
            t_l0 = time.perf_counter() - t0
            while K.kvx_ready_prefix(ready) < n:
                pass
            t_all = time.perf_counter() - t0
            stream.synchronize()
            lat[name] = {"layer0_ms": round(t_l0 * 1e3, 3), "all_layers_ms": round(t_all * 1e3, 3)}
        result["restore_ready_latency"] = lat
        log(f"restore ready latency: {lat}")

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w)
        log(f"cpu baseline: {result['cpu_baseline']}")
        result["cpu_baseline_all_cores"] = cpu_baseline_all_cores(w)
        log(f"cpu baseline, all cores: {result['cpu_baseline_all_cores']}")
    print(json.dumps(result), flush=True)

    K.kvx_ready_destroy(ready)
    K.kvx_unregister_pool(pool)
    host.free()


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

    # ---- mixed: 128 alternating requests, four in flight on four streams ----
    w = WORKLOADS["mixed"]
    P = w.payload_bytes()
    alloc, pool = make_pool(w)
    perm = synth.page_perm(w.seed, w.num_pages)
    prime = [np.ascontiguousarray(perm[256 * r:256 * (r + 1)]) for r in range(4)]
    slots = [K.HostBuffer(P) for _ in range(8)]
    streams = [torch.cuda.Stream() for _ in range(4)]
    for r in range(4):
        K.kvx_backup(pool, prime[r], slots[r].ptr, P, 0, w.num_layers, streams[0],
                     K.KVX_PATH_ZEROCOPY)
    torch.cuda.synchronize()
    sched = mixed_schedule(w, 128)
    res = {"workload": w.description, "requests": 128, "in_flight": 4,
           "bytes_total": 128 * P, "unit": "GB/s",
           "hw_queues": os.environ.get("GPU_MAX_HW_QUEUES", "runtime default")}
    # both directions at once with plain copies: the peak the mixed stream is
    # measured against
    GiB = 1 << 30
    pin_a = torch.empty(GiB, dtype=torch.uint8, pin_memory=True)
    pin_b = torch.empty(GiB, dtype=torch.uint8, pin_memory=True)
    dev_a = torch.empty(GiB, dtype=torch.uint8, device="cuda")
    dev_b = torch.empty(GiB, dtype=torch.uint8, device="cuda")
    bid = []
    for _ in range(4):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(streams[0]):
            pin_a.copy_(dev_a, non_blocking=True)
        with torch.cuda.stream(streams[1]):
            dev_b.copy_(pin_b, non_blocking=True)
        torch.cuda.synchronize()
        bid.append(2 * GiB / (time.perf_counter() - t0) / GB)
    del pin_a, pin_b, dev_a, dev_b
    res["memcpy_both_directions_gbs"] = round(statistics.median(bid[1:]), 2)
    # backup k and restore k + 1 of the schedule as one kvx_exchange, the
    # pairs round-robin on two streams (four requests in flight)
    def run_exchange():
        nb = nr = 0
        pairs = [(sched[k], sched[k + 1]) for k in range(0, len(sched), 2)]
        for i, ((kb, ib), (kr, ir)) in enumerate(pairs):
            assert kb == "backup" and kr == "restore"
            K.kvx_exchange(pool, ib, slots[4 + nb % 4].ptr, P, (0, w.num_layers), slots[nr % 4].ptr,
                           P, ir, (0, w.num_layers), None, 0, streams[i % 2], K.KVX_PATH_ZEROCOPY)
            nb += 1
            nr += 1
        torch.cuda.synchronize()
    run_exchange()
    t0 = time.perf_counter()
    run_exchange()
    res["zerocopy_exchange"] = round(128 * P / (time.perf_counter() - t0) / GB, 2)
    res["zerocopy_exchange_frac_of_memcpy_both_directions"] = round(
        res["zerocopy_exchange"] / res["memcpy_both_directions_gbs"], 4)
    log(f"mixed zerocopy_exchange: {res['zerocopy_exchange']} GB/s")
    # the same schedule as descriptors through a submission ring, served on
    # one stream by the library's executor; with pairing on it runs each
    # backup and the restore after it as one exchange by itself
    rname = f"/kvx-bench-mixed-{os.getpid()}"
    ring = K.kvx_ring_create(rname, 256, 1)
    srv = K.kvx_ring_open(rname)
    rbufs, rsizes = [h.ptr for h in slots], [P] * len(slots)

    def run_ring():
        nb = nr = 0
        for k, (kind, ids) in enumerate(sched):
            if kind == "backup":
                q = K.make_sqe(K.KVX_OP_BACKUP, k, 1, 0, 4 + nb % 4, ids, 0, w.num_layers,
                               K.KVX_PATH_ZEROCOPY)
                nb += 1
            else:
                q = K.make_sqe(K.KVX_OP_RESTORE, k, 1, 0, nr % 4, ids, 0, w.num_layers,
                               K.KVX_PATH_ZEROCOPY)
                nr += 1
            K.kvx_ring_submit(ring, q)
        done = []
        while len(done) < len(sched):
            K.kvx_ring_serve(srv, [pool], rbufs, rsizes, None, streams[0], 256)
            done += K.kvx_ring_reap(ring, 256)
            time.sleep(0.0002)
        assert all(c[2] == 0 for c in done), [c for c in done if c[2] != 0][:3]

    for pairing in (1, 0):
        K.kvx_set_option(K.KVX_OPT_RING_PAIRING, pairing)
        run_ring()
        t0 = time.perf_counter()
        run_ring()
        key = "ring_zerocopy_paired" if pairing else "ring_zerocopy_one_by_one"
        res[key] = round(128 * P / (time.perf_counter() - t0) / GB, 2)
        log(f"mixed {key}: {res[key]} GB/s")
    K.kvx_set_option(K.KVX_OPT_RING_PAIRING, 1)
    K.kvx_ring_close(srv)
    K.kvx_ring_close(ring)
    for name, bpath, rpath in (("zerocopy", K.KVX_PATH_ZEROCOPY, K.KVX_PATH_ZEROCOPY),
                               ("staged", K.KVX_PATH_STAGED, K.KVX_PATH_STAGED),
                               ("zerocopy_backup_staged_restore", K.KVX_PATH_ZEROCOPY,
                                K.KVX_PATH_STAGED)):
        def run():
            nb = nr = 0
            for k, (kind, ids) in enumerate(sched):
                s = streams[k % 4]
                if kind == "backup":
                    K.kvx_backup(pool, ids, slots[4 + nb % 4].ptr, P, 0, w.num_layers, s, bpath)
                    nb += 1
                else:
                    K.kvx_restore(pool, slots[nr % 4].ptr, P, ids, 0, w.num_layers, None, 0, s,
                                  rpath)
                    nr += 1
            torch.cuda.synchronize()
        run()
        t0 = time.perf_counter()
        run()
        res[name] = round(128 * P / (time.perf_counter() - t0) / GB, 2)
        res[name + "_frac_of_memcpy_both_directions"] = round(
            res[name] / res["memcpy_both_directions_gbs"], 4)
        log(f"mixed {name}: {res[name]} GB/s")
    print(json.dumps({"mixed": res}), flush=True)
    for h in slots:
        h.free()
    K.kvx_unregister_pool(pool)


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
    L = oracle.Layout(outer=tuple({"page": oracle.PAGE, "layer": oracle.LAYER,
                                   "kv": oracle.KV}[a] for a in sample.outer),
                      inner=oracle.NHD if sample.inner == "NHD" else oracle.HND,
                      num_pages=sample.num_pages, num_layers=nl, num_kv=sample.num_kv,
                      page_size=sample.page_size, num_heads=sample.num_heads,
                      head_dim=sample.head_dim, dtype_bytes=sample.dtype_bytes)
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


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_all_cores(w, budget_s: float = 8.0, max_threads: int = 16):
    """The same oracle calls from one host thread per core (the process's
    affinity set, at most max_threads): each thread owns a one-layer host
    pool and packed buffer of the workload's piece shape and runs
    backup + restore passes for about budget_s seconds. The oracle's C
    functions run without the interpreter lock, so the threads run in
    parallel; the oracle itself is unchanged."""
    import threading

    import numpy as np

    import oracle
    import synth

    threads = max(1, min(max_threads, len(os.sched_getaffinity(0))))
    n = w.pages_per_request
    sample = w.scaled(num_pages=2 * n, num_layers=1)
    L = oracle.Layout(outer=tuple({"page": oracle.PAGE, "layer": oracle.LAYER,
                                   "kv": oracle.KV}[a] for a in sample.outer),
                      inner=oracle.NHD if sample.inner == "NHD" else oracle.HND,
                      num_pages=sample.num_pages, num_layers=1, num_kv=sample.num_kv,
                      page_size=sample.page_size, num_heads=sample.num_heads,
                      head_dim=sample.head_dim, dtype_bytes=sample.dtype_bytes)
    perm = synth.page_perm(w.seed, 2 * n)
    src, dst = perm[:n].copy(), perm[n:].copy()
    per_pass = 2 * sample.num_kv * n * sample.piece_bytes
    passes = [0] * threads
    start = threading.Barrier(threads + 1)
    stop = threading.Event()

    def worker(k):
        alloc = np.full(sample.pool_bytes, 0x5A, dtype=np.uint8)
        host = np.zeros(sample.host_bytes(n), dtype=np.uint8)
        start.wait()
        while not stop.is_set():
            oracle.backup(L, alloc, src, 0, 1, host=host)
            oracle.restore(L, alloc, host, dst, 0, 1, out=alloc)
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
    moved = sum(passes) * per_pass
    return {"value": round(moved / t / GB, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{sum(passes)} single-layer backup+restore passes of {n} fragmented pages x "
                      f"{sample.num_kv} x {sample.piece_bytes} B pieces, one {2 * n}-page host pool "
                      f"per thread ({moved / GB:.2f} GB moved in {t:.1f} s)",
            "cpu_model": cpu_model()}


if __name__ == "__main__":
    main()
