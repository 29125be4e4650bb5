"""Benchmark: KV bytes moved per second by kvx backup (GPU pool -> pinned host)
and restore (pinned host -> other GPU pages, per-layer publish) on one MI355X.

One step = the whole hot path over one request of the Llama-3-8B-shaped bf16
pool (32 layers, K+V, 8 KV heads, head_dim 128, page size 64, 2048 pages):
  backup of 256 fragmented pages (16,384 tokens, 2 GiB) to pinned host,
  restore of that buffer into 256 other pages with per-layer publish,
  and the ready-prefix query.
value = 2 x 2 GiB / step time (GB = 1e9 B). Inputs are resident in HBM when
the timed region starts; the host transfer is part of the method (the host
tier is where BACKUP writes and RESTORE reads).

Also reported: the device pack kernel alone (HBM roofline), the pinned
hipMemcpyAsync peaks (host-link roofline), the zero-copy path, and the CPU
oracle on a bounded sample (a baseline only).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--path staged|zerocopy]
       [--no-cpu-baseline] [--kernel-only]
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


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def median(xs):
    return statistics.median(xs) if xs else float("nan")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--path", choices=["staged", "zerocopy"], default="staged")
    ap.add_argument("--workload", default="llama8b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-only", action="store_true",
                    help="time only the device pack/unpack kernels (for profiling runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "kvx moves KV between one GPU and its host; this build "
                                   "measures one GPU only (--gpus 1)"}))
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from paged_kv_offload_amd import kvx as K
    from synth.workloads import WORKLOADS

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    K.lib()
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
    host = K.HostBuffer(P)
    ready = K.kvx_ready_create(w.num_layers, 1)
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

    # ---- device pack / unpack kernels alone (HBM roofline) ----
    def pack():
        K.kvx_backup(pool, src, dev_packed, P, 0, w.num_layers, stream, K.KVX_PATH_DEVICE)

    def unpack():
        K.kvx_restore(pool, dev_packed, P, dst, 0, w.num_layers, None, 0, stream,
                      K.KVX_PATH_DEVICE)

    kreps = max(args.steps, 5)
    timed(pack, 2)
    t_pack = timed(pack, kreps)
    timed(unpack, 2)
    t_unpack = timed(unpack, kreps)
    pack_gbs = 2 * P / median(t_pack) / GB
    unpack_gbs = 2 * P / median(t_unpack) / GB
    log(f"device pack {median(t_pack) * 1e3:.3f} ms = {pack_gbs:.0f} GB/s (read+write); "
        f"unpack {median(t_unpack) * 1e3:.3f} ms = {unpack_gbs:.0f} GB/s")

    # D2D copy of the same byte count (the in-run achievable line)
    d2d_a = torch.empty(P, dtype=torch.uint8, device="cuda")
    with torch.cuda.stream(stream):
        t_d2d = timed(lambda: d2d_a.copy_(dev_packed), 5)
    d2d_gbs = 2 * P / median(t_d2d) / GB
    del d2d_a
    log(f"D2D copy {d2d_gbs:.0f} GB/s (read+write)")

    if args.kernel_only:
        print(json.dumps({"pack_gbs": pack_gbs, "unpack_gbs": unpack_gbs, "d2d_gbs": d2d_gbs}))
        return

    # ---- pinned host-link peaks: 1 GiB hipMemcpyAsync, median of 10 ----
    peak_bytes = 1 << 30
    pin = torch.empty(peak_bytes, dtype=torch.uint8, pin_memory=True)
    dev1 = torch.empty(peak_bytes, dtype=torch.uint8, device="cuda")
    with torch.cuda.stream(stream):
        t_d2h = timed(lambda: pin.copy_(dev1, non_blocking=True), 10)
        t_h2d = timed(lambda: dev1.copy_(pin, non_blocking=True), 10)
    d2h_peak = peak_bytes / median(t_d2h) / GB
    h2d_peak = peak_bytes / median(t_h2d) / GB
    del pin, dev1
    log(f"pinned memcpy peak: D2H {d2h_peak:.1f} GB/s, H2D {h2d_peak:.1f} GB/s")

    # ---- the step ----
    path = {"staged": K.KVX_PATH_STAGED, "zerocopy": K.KVX_PATH_ZEROCOPY}[args.path]

    def step(path=path):
        K.kvx_ready_reset(ready)
        K.kvx_backup(pool, src, host.ptr, P, 0, w.num_layers, stream, path)
        K.kvx_restore(pool, host.ptr, P, dst, 0, w.num_layers, ready, 0, stream, path)

    def backup_only(path=path):
        K.kvx_backup(pool, src, host.ptr, P, 0, w.num_layers, stream, path)

    def restore_only(path=path):
        K.kvx_restore(pool, host.ptr, P, dst, 0, w.num_layers, None, 0, stream, path)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    a, b = ev(), ev()
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(args.steps):
        step()
    b.record(stream)
    b.synchronize()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_total = a.elapsed_time(b) / 1e3
    prefix = K.kvx_ready_prefix(ready)
    assert prefix == n, f"ready prefix {prefix} != {n} after the timed steps"
    ms_per_step = t_total / args.steps * 1e3
    value = 2 * P * args.steps / t_total / GB
    log(f"step ({args.path}): {ms_per_step:.2f} ms -> {value:.2f} GB/s (wall {wall:.2f} s)")

    # per-direction end-to-end rates on both paths
    e2e = {}
    for name, pth in (("staged", K.KVX_PATH_STAGED), ("zerocopy", K.KVX_PATH_ZEROCOPY)):
        tb = timed(lambda: backup_only(pth), 3)
        tr = timed(lambda: restore_only(pth), 3)
        e2e[name] = {"backup_d2h_gbs": P / median(tb) / GB, "restore_h2d_gbs": P / median(tr) / GB}
        log(f"{name}: backup {e2e[name]['backup_d2h_gbs']:.1f} GB/s, "
            f"restore {e2e[name]['restore_h2d_gbs']:.1f} GB/s")

    # layer-0-ready latency of a restore: CPU polls the first layer's count
    K.kvx_ready_reset(ready)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    K.kvx_restore(pool, host.ptr, P, dst, 0, w.num_layers, ready, 0, stream, path)
    while K.kvx_layer_ready(ready, 0) < n:
        pass
    t_l0 = time.perf_counter() - t0
    while K.kvx_ready_prefix(ready) < n:
        pass
    t_all = time.perf_counter() - t0
    stream.synchronize()
    log(f"restore: layer 0 ready after {t_l0 * 1e3:.2f} ms, all layers after {t_all * 1e3:.2f} ms")

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
                   "payload_bytes_per_op": P, "path": args.path},
        "roofline": {"bound": "hbm", "kernel": "kvx_move_kernel (pack, device path)",
                     "achieved": round(pack_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(pack_gbs / HBM_PEAK_GBS, 4), "traffic": None},
        "unpack_roofline": {"achieved": round(unpack_gbs, 1), "peak": HBM_PEAK_GBS,
                            "frac": round(unpack_gbs / HBM_PEAK_GBS, 4)},
        "d2d_copy_gbs": round(d2d_gbs, 1),
        "link": {"d2h_peak_gbs": round(d2h_peak, 2), "h2d_peak_gbs": round(h2d_peak, 2),
                 "e2e": {k: {kk: round(vv, 2) for kk, vv in v.items()} for k, v in e2e.items()},
                 # the step moves P one way then P the other way: its link bound is the
                 # serial combination of the two measured peaks
                 "step_frac_of_serial_peak": round(value / (2 / (1 / d2h_peak + 1 / h2d_peak)), 4)},
        "restore_layer0_ready_ms": round(t_l0 * 1e3, 3),
        "restore_all_ready_ms": round(t_all * 1e3, 3),
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)

    K.kvx_ready_destroy(ready)
    K.kvx_unregister_pool(pool)
    host.free()


def cpu_baseline(w, budget_s: float = 12.0):
    """The oracle's backup + restore byte loops, single-threaded, on a host
    pool with the workload's piece shape and request size but fewer pages
    and layers; runs layer by layer until about budget_s seconds."""
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
    # only the shape matters for the timing; the bytes are a cheap pattern
    alloc = np.full(sample.pool_bytes, 0x5A, dtype=np.uint8)
    src = synth.page_perm(w.seed, 2 * n)[:n].copy()
    dst = synth.page_perm(w.seed, 2 * n)[n:].copy()
    host = np.zeros(sample.host_bytes(n), dtype=np.uint8)
    moved, t, layers = 0, 0.0, 0
    while t < budget_s:
        l = layers % nl
        t0 = time.perf_counter()
        oracle.backup(L, alloc, src, l, l + 1, host=host)
        oracle.restore(L, alloc, host, dst, l, l + 1, out=alloc)
        t += time.perf_counter() - t0
        moved += 2 * sample.num_kv * n * sample.piece_bytes
        layers += 1
    gbs = moved / t / GB
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{layers} single-layer backup+restore passes of {n} fragmented pages x "
                      f"{sample.num_kv} x {sample.piece_bytes} B pieces on a {2 * n}-page, "
                      f"{nl}-layer host pool ({moved / GB:.2f} GB moved in {t:.1f} s)"}


if __name__ == "__main__":
    main()
