#!/usr/bin/env python3
"""Benchmark: restore losslessly coded BF16 weights on one MI355X.

Default workload (`model`): the whole synthetic Qwen3-14B-shaped model, 40
decoder layers plus the embedding, the untied output head and the final norm
(42 units, 14.77G BF16 values, 29.5 GB restored), compressed in pinned host
memory. One step is one pass of the restore over every unit with the
compressed model resident in HBM: one afx_decode_layer_async call (one
kernel launch) per unit, back to back on one stream, each unit into its own
output region. The streamed pass (unit i+1 copied over the host link while
unit i is restored, "Why Weight Offloading Slows Inference", section
"Loading during computation"), the restore of one decoder layer and of the
embedding inside the pass, and the CPU oracle on a bounded sample of the
units are reported beside it.

Other workloads: layer (one decoder layer, 11 tensors in one launch),
tensor-1024 (1024x1024), q_proj (5120x5120), embedding (151936x5120), disk
(the whole model stored compressed in a file, read cold, copied and
restored), tiers (the model spread over residency tiers under memory
budgets), gemv and gemm (the restore fused into the products of one layer's
matrices) and token (one token's products over the whole model).

Prints one JSON line with the throughput of restored BF16, the HBM roofline
fraction of the decode kernel (hipEvent timing on the launch stream), and the
CPU oracle's decode rate on this host as a baseline.

The single-workload steps rotate over enough copies of the workload's blobs
and outputs that a copy is touched again only after about 4 GB of other
traffic, as in a pass over a model whose layers each pass once. Re-running
one resident copy is faster (part of it is still cached) and is not what a
model pass sees; --copies 1 measures that case.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
COLD_BYTES = 4.0e9  # traffic between two touches of the same copy
sys.path.insert(0, ROOT)

METRIC = "decoded BF16 GB/s on 1 MI355X + % of HBM roofline; bit-exact vs CPU oracle"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
CSRC = os.path.join(ROOT, "lossless_bf16_weight_afx_amd", "csrc")
KERNEL_NAME = "afx_decode_kernel"
# the source each kernel is compiled from (a profile taken on other code is stale)
KERNEL_SRCS = {"afx_decode_kernel": "afx_decode.hip", "afx_gemv_kernel": "afx_gemv.hip",
               "afx_gemm_kernel": "afx_gemm.hip"}
GEMV_METRIC = ("BF16 weight GB/s consumed by the fused restore+GEMV on 1 MI355X + % of HBM roofline; "
               "within the FP32 summation bound of the CPU oracle")
GEMM_METRIC = ("BF16 weight GB/s consumed by the fused restore+GEMM (MFMA) on 1 MI355X + % of HBM roofline; "
               "within the FP32 summation bound of the CPU oracle")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_share() -> int:
    """Host threads this process may use: OMP_NUM_THREADS where the host sets
    it (the share of the host's cores that goes with one GPU), else every
    core in the affinity mask."""
    try:
        v = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        v = 0
    return max(1, min(v, host_threads())) if v > 0 else host_threads()


def host_cpu_facts() -> dict:
    return {"affinity_cores": host_threads(), "os_cpu_count": os.cpu_count(),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"), "threads_used": cpu_share()}


def workload_specs(name: str):
    from lossless_bf16_weight_afx_amd import synth

    if name == "layer":
        return "qwen3-14b-decoder-layer", synth.decoder_layer(0)
    if name == "tensor-1024":
        return "bf16-1024x1024", synth.single_tensor(1024, 1024, 1)
    if name == "q_proj":
        return "qwen3-14b-q_proj-5120x5120", synth.single_tensor(5120, 5120, 2)
    if name == "embedding":
        return "qwen3-14b-embedding-151936x5120", synth.embedding()
    raise SystemExit(f"unknown workload {name}")


def kernel_sha(kernel: str = KERNEL_NAME) -> str:
    """Hash of the kernel's generated gfx950 code (build.device_code_sha)."""
    from lossless_bf16_weight_afx_amd import build

    return build.device_code_sha(KERNEL_SRCS[kernel])


def profile_traffic(workload: str, kernel: str = KERNEL_NAME):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = (t.strip() for t in line.split("=", 1))
            kv[k] = v
    if kv.get("kernel_sha") != kernel_sha(kernel):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="model",
                    choices=["layer", "tensor-1024", "q_proj", "embedding", "model", "disk", "tiers", "gemv", "gemm",
                             "token"])
    ap.add_argument("--m", type=int, default=None,
                    help="tokens (activation rows) of the fused products: 1, 2 or 4 for --workload gemv "
                         "(default 1), any for --workload gemm (default 64)")
    ap.add_argument("--layers", type=int, default=40,
                    help="decoder layers of the whole model (--workload model or disk)")
    ap.add_argument("--store-dir", default=os.environ.get("TMPDIR") or "/tmp",
                    help="directory for the model store file (--workload disk)")
    ap.add_argument("--keep-store", action="store_true", help="keep the store file afterwards (--workload disk)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--max-workgroups", type=int, default=0,
                    help="restore on at most this many workgroups (CUs) per launch, through "
                         "afx_decode_layer_grid_async (--workload layer, tensor-1024, q_proj or embedding)")
    ap.add_argument("--copies", type=int, default=0,
                    help="rotate over this many blob/output copies (default: enough for about 4 GB between "
                         "two touches of one copy)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the restore is per-tensor work with no collective (on "
              "several GPUs each restores the tensors of its own shard); run it with --gpus 1.", file=sys.stderr)
        return 2

    import torch

    from lossless_bf16_weight_afx_amd import afx, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    afx.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    threads = cpu_share()
    if args.max_workgroups and args.workload not in ("layer", "tensor-1024", "q_proj", "embedding"):
        print("--max-workgroups applies to --workload layer, tensor-1024, q_proj or embedding", file=sys.stderr)
        return 2
    if args.workload == "model":
        return bench_model(args, threads)
    if args.workload == "disk":
        return bench_disk(args, threads)
    if args.workload == "tiers":
        return bench_tiers(args, threads)
    if args.workload in ("gemv", "gemm"):
        return bench_gemv(args, threads)
    if args.workload == "token":
        return bench_token(args, threads)
    workload, specs = workload_specs(args.workload)
    if args.max_workgroups < 0:
        print("--max-workgroups must be positive", file=sys.stderr)
        return 2
    if args.max_workgroups:
        def enqueue(jobs, s):
            afx.afx_decode_layer_grid_async(jobs, args.max_workgroups, s)
    else:
        enqueue = afx.afx_decode_layer_async

    # ---- inputs: generate, encode with the library's encoder, move to HBM
    t0 = time.time()
    xs, blobs, infos = [], [], []
    for sp in specs:
        x = synth.generate(sp, threads=threads)
        blob = afx.afx_encode(x, sp.shape, threads=threads)
        xs.append(x)
        blobs.append(blob)
        infos.append(afx.afx_query(blob))
    n_total = sum(int(i.n_elems) for i in infos)
    blob_total = sum(int(i.blob_bytes) for i in infos)
    restored = 2 * n_total
    log(f"[bench] {workload}: {len(specs)} tensors, {n_total} values, blob {blob_total} B "
        f"(ratio {blob_total / restored:.4f}); inputs ready in {time.time() - t0:.1f}s")

    traffic_pass = blob_total + restored
    # (the timed steps continue the warm-up's rotation, so with more copies
    # than steps every timed step still finds its copy untouched for ~4 GB)
    copies = args.copies or max(1, int(np.ceil(COLD_BYTES / traffic_pass)))
    dblobs = [[torch.from_numpy(b).to(dev) for b in blobs] for _ in range(copies)]
    douts = [[torch.empty(int(i.n_elems), dtype=torch.int16, device=dev) for i in infos] for _ in range(copies)]
    jobsets = [afx.make_jobs([(i, b.data_ptr(), o.data_ptr(), 2 * int(i.n_elems))
                              for i, b, o in zip(infos, dblobs[c], douts[c])]) for c in range(copies)]
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    # ---- correctness pass (separate from timing): every copy, bit-exact
    for c in range(copies):
        enqueue(jobsets[c], sp)
    torch.cuda.synchronize()
    exact = True
    for t, x in enumerate(xs):
        ref = torch.from_numpy(x.view(np.int16)).to(dev)
        for c in range(copies):
            exact &= bool(torch.equal(ref, douts[c][t]))
        del ref
    if not exact:
        log("[bench] restored bits differ from the originals")

    # ---- timing: hipEvents on the launch stream around the timed region;
    # every step is one launch, back to back
    t_warm, w = time.time(), 0
    while True:  # warm-up: at least W steps and about half a second of work
        for _ in range(max(1, args.warmup)):
            enqueue(jobsets[w % copies], sp)
            w += 1
        torch.cuda.synchronize()
        if time.time() - t_warm > 0.5:
            break
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_all0.record(stream)
    for k in range(args.steps):
        enqueue(jobsets[(w + k) % copies], sp)
    t_all1.record(stream)
    torch.cuda.synchronize()
    total_ms = t_all0.elapsed_time(t_all1)
    ms_per_step = total_ms / args.steps
    launch_ms = ms_per_step  # one kernel launch per step
    value = restored / (ms_per_step * 1e-3) / 1e9

    # the same launch repeated on one copy ("hot": a copy restored again while
    # its code words still sit in the memory-side cache), timed apart from
    # the cold rotation above and reported beside it, labelled
    for _ in range(max(1, args.warmup)):
        enqueue(jobsets[0], sp)
    h0, h1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    h0.record(stream)
    for _ in range(args.steps):
        enqueue(jobsets[0], sp)
    h1.record(stream)
    torch.cuda.synchronize()
    hot_ms = h0.elapsed_time(h1) / args.steps
    hot = {"ms_per_step": round(hot_ms, 5),
           "frac": round(traffic_pass / (hot_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
           "note": "one copy restored again and again; not the result (value and roofline are the cold rotation)"}

    copy_gbps, copy_each_way = copy_ceiling(stream, traffic_pass, copies)

    achieved = traffic_pass / (launch_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": None if args.max_workgroups else profile_traffic(workload),
                "algorithmic_bytes_per_launch": traffic_pass, "kernel": KERNEL_NAME,
                "kernel_ms": round(launch_ms, 5), "copy_ceiling_GBps": round(copy_gbps, 1),
                "calib_copy_bytes_each_way": copy_each_way}

    # ---- CPU oracle baseline on this host, and bit-exactness against it:
    # whole passes over the workload's blobs until ~10 CPU-seconds are spent
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        dec = [oracle.decode(b, threads=threads) for b in blobs]  # also the bit-exact check
        for i, d in enumerate(dec):
            exact &= bool(np.array_equal(d, douts[0][i].cpu().numpy().view(np.uint16)))
        del dec
        passes, t_cpu, cpu0 = 0, 0.0, time.process_time()
        while passes == 0 or (time.process_time() - cpu0 < 10.0 and passes < 50):
            t0 = time.perf_counter()
            for b in blobs:
                oracle.decode(b, threads=threads)
            t_cpu += time.perf_counter() - t0
            passes += 1
        cpu_s = time.process_time() - cpu0
        n_cpu = passes * n_total
        # the same decoder on one thread, over the workload's tensors in turn
        # until about 3 seconds are spent
        n1, t1 = 0, 0.0
        for b, i in zip(blobs * 8, infos * 8):
            t0 = time.perf_counter()
            oracle.decode(b, threads=1)
            t1 += time.perf_counter() - t0
            n1 += int(i.n_elems)
            if t1 > 3.0:
                break
        cpu = {"value": round(2 * n_cpu / t_cpu / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
               "sample": f"{passes} whole passes over the {workload} blobs ({n_total} values each), bit-serial "
                         f"canonical decode, chunk-parallel over {threads} threads; {cpu_s:.1f} CPU-s",
               "seconds": round(t_cpu, 2), "host": host_cpu_facts(),
               "one_thread": {"value": round(2 * n1 / t1 / 1e9, 3), "unit": "GB/s",
                              "sample": f"{n1} values of the workload's tensors in turn, one thread"}}

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "u32", "data": "synthetic",
        "config": {"workload": workload, "tensors": len(specs), "values": n_total, "restored_bytes": restored,
                   "blob_bytes": blob_total, "ratio": round(blob_total / restored, 4), "copies": copies,
                   "encoder": "libafx afx_encode",
                   **({"max_workgroups": args.max_workgroups} if args.max_workgroups else {})},
        "bit_exact": bool(exact), "roofline": roofline, "hot_one_copy": hot, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0 if exact else 1


def copy_ceiling(stream, traffic: int, copies: int):
    """A plain elementwise copy kernel (torch's bitwise_not over int16: read
    N, write N bytes) moving `traffic` bytes per launch over `copies`
    rotated regions: the GPU's practical ceiling for that traffic, and the
    known-size kernel that calibrates rocprofv3's HBM byte counters.
    Returns (GB/s, N)."""
    import torch

    half = traffic // 4  # int16 elements: 2 bytes read + 2 written each
    src = torch.empty(half * copies, dtype=torch.int16, device=stream.device)
    dst = torch.empty_like(src)
    torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_copy = max(10, copies)
    c0.record(stream)
    for k in range(n_copy):
        sl = slice((k % copies) * half, (k % copies + 1) * half)
        torch.bitwise_not(src[sl], out=dst[sl])
    c1.record(stream)
    torch.cuda.synchronize()
    return 4 * half * n_copy / (c0.elapsed_time(c1) * 1e-3) / 1e9, 2 * half


def _time_steps(stream, fn, steps: int, warmup: int) -> float:
    """Milliseconds per step of fn(k) over `steps` back-to-back steps, timed
    with events on the launch stream after at least `warmup` steps and about
    half a second of untimed work."""
    import torch

    t_warm, w = time.time(), 0
    while True:
        for _ in range(max(1, warmup)):
            fn(w)
            w += 1
        torch.cuda.synchronize()
        if time.time() - t_warm > 0.5:
            break
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for k in range(steps):
        fn(w + k)  # continuing the warm-up's rotation
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def bench_gemv(args, threads: int) -> int:
    """The restore fused into its consumer: y += x W^T for the seven matrices
    of one decoder layer, straight from their coded form (one launch per
    step): the matrix-vector kernel (--workload gemv, m = 1, 2 or 4 tokens)
    or the MFMA kernel (--workload gemm, any m). Compared with the same
    products on the BF16 weights already restored (torch.mm, and torch.mv
    at m = 1) and with the restore followed by those products."""
    import torch

    from lossless_bf16_weight_afx_amd import afx, synth

    dev = torch.device("cuda:0")
    gemm = args.workload == "gemm"
    m = args.m if args.m is not None else (64 if gemm else 1)
    if not gemm and m not in (1, 2, 4):
        raise SystemExit("--workload gemv takes --m 1, 2 or 4")
    if m < 1:
        raise SystemExit("--m must be at least 1")
    # (the MFMA entry point runs the matrix-vector kernel for 1, 2 or 4 tokens)
    kernel = "afx_gemm_kernel" if gemm and m not in (1, 2, 4) else "afx_gemv_kernel"
    launch = afx.afx_restore_gemm_batch_async if gemm else afx.afx_restore_gemv_batch_async
    tol = 1.0  # the summation bound (for the matrix instruction, as measured by test_one_matrix_instruction_rounding)
    specs = [sp for sp in synth.decoder_layer(0) if len(sp.shape) == 2]
    workload = f"qwen3-14b-decoder-layer-{args.workload}-m{m}"
    t0 = time.time()
    ws, blobs, infos = [], [], []
    for sp in specs:
        w = synth.generate(sp, threads=threads)
        blobs.append(afx.afx_encode(w, sp.shape, threads=threads))
        infos.append(afx.afx_query(blobs[-1]))
        ws.append(w)
    n_total = sum(int(i.n_elems) for i in infos)
    blob_total = sum(int(i.blob_bytes) for i in infos)
    x_bytes = sum(m * sp.shape[1] * 2 for sp in specs)
    y_bytes = sum(m * sp.shape[0] * 4 for sp in specs)
    alg = blob_total + x_bytes + 2 * y_bytes  # blobs and x read, y read and written
    log(f"[bench] {workload}: {len(specs)} matrices, {n_total} weights, blob {blob_total} B; "
        f"inputs ready in {time.time() - t0:.1f}s")

    copies = args.copies or max(1, int(np.ceil(COLD_BYTES / blob_total)))
    dblobs = [[torch.from_numpy(b).to(dev) for b in blobs] for _ in range(copies)]
    gen = torch.Generator(device="cpu").manual_seed(7)
    xs = [torch.randn((m, sp.shape[1]), generator=gen).to(torch.bfloat16).to(dev) for sp in specs]
    ys = [torch.zeros((m, sp.shape[0]), dtype=torch.float32, device=dev) for sp in specs]
    jobsets = [afx.make_gemv_jobs([(i, b.data_ptr(), sp.shape[0], sp.shape[1], x.data_ptr(), y.data_ptr())
                                   for i, b, sp, x, y in zip(infos, dblobs[c], specs, xs, ys)])
               for c in range(copies)]
    stream = torch.cuda.current_stream(dev)
    sp_ = stream.cuda_stream

    # ---- check (outside the timing): one launch from zero against FP32
    # products of the bit-exact restored weights, within twice the bound
    for y in ys:
        y.zero_()
    launch(jobsets[0], m, sp_)
    torch.cuda.synchronize()
    within = True
    for w, sp, x, y in zip(ws, specs, xs, ys):
        wf = torch.from_numpy(w.view(np.int16)).to(dev).view(torch.bfloat16).view(*sp.shape).float()
        xf = x.float()
        ref = xf @ wf.t()
        j = (sp.shape[1] - 1) * 2.0 ** -24
        bound = j / (1 - j) * (xf.abs() @ wf.abs().t())  # each of the two FP32 sums errs by at most this
        within &= bool(((y - ref).abs() <= 2 * tol * bound + 1e-30).all())
        del wf
    y_fused = [y.cpu().numpy().astype(np.float64) for y in ys]
    if not within:
        log("[bench] fused products fall outside the FP32 summation bound")

    # ---- timing of the fused launch
    def fused(k):
        launch(jobsets[k % copies], m, sp_)

    ms_fused = _time_steps(stream, fused, args.steps, args.warmup)
    hot_ms = _time_steps(stream, lambda k: fused(0), args.steps, args.warmup)

    # ---- the same products on restored BF16 weights, and restore + products
    wbf = [[torch.empty(sp.shape, dtype=torch.bfloat16, device=dev) for sp in specs] for _ in range(copies)]
    djobs = [afx.make_jobs([(i, b.data_ptr(), o.data_ptr(), 2 * int(i.n_elems))
                            for i, b, o in zip(infos, dblobs[c], wbf[c])]) for c in range(copies)]
    for c in range(copies):
        afx.afx_decode_layer_async(djobs[c], sp_)

    def mm(k):
        for x, w in zip(xs, wbf[k % copies]):
            torch.mm(x, w.t())

    def restore_mm(k):
        afx.afx_decode_layer_async(djobs[k % copies], sp_)
        mm(k)

    def mv(k):  # torch's matrix-vector path, for one token
        for x, w in zip(xs, wbf[k % copies]):
            torch.mv(w, x[0])

    ms_mm = _time_steps(stream, mm, args.steps, args.warmup)
    ms_rmm = _time_steps(stream, restore_mm, args.steps, args.warmup)
    ms_mv = _time_steps(stream, mv, args.steps, args.warmup) if m == 1 else None
    del wbf, djobs
    copy_gbps, copy_each_way = copy_ceiling(stream, 2 * blob_total, copies)  # read and write a layer's blobs

    achieved = alg / (ms_fused * 1e-3) / 1e9
    value = 2 * n_total / (ms_fused * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": profile_traffic(workload, kernel),
                "algorithmic_bytes_per_launch": alg, "kernel": kernel, "kernel_ms": round(ms_fused, 5),
                "tflops": round(2 * m * n_total / (ms_fused * 1e-3) / 1e12, 2),
                "copy_ceiling_GBps": round(copy_gbps, 1), "calib_copy_bytes_each_way": copy_each_way}
    compare = {"unit": "us per layer", "fused": round(ms_fused * 1e3, 1), "fused_hot_one_copy": round(hot_ms * 1e3, 1),
               "bf16_torch_mm_on_restored": round(ms_mm * 1e3, 1),
               "restore_then_bf16_torch_mm": round(ms_rmm * 1e3, 1)}
    if ms_mv is not None:
        compare["bf16_torch_mv_on_restored"] = round(ms_mv * 1e3, 1)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        for blob, sp, x, yf in zip(blobs, specs, xs, y_fused):  # also the check against the oracle
            xb = x.cpu().view(torch.int16).numpy().view(np.uint16)
            ref, bound = oracle.restore_gemv(blob, sp.shape[0], sp.shape[1], xb, threads=threads)
            within &= bool((np.abs(yf - ref) <= tol * bound).all())
        passes, t_cpu, cpu0 = 0, 0.0, time.process_time()
        while passes == 0 or (time.process_time() - cpu0 < 10.0 and passes < 20):
            t1 = time.perf_counter()
            for blob, sp, x in zip(blobs, specs, xs):
                oracle.restore_gemv(blob, sp.shape[0], sp.shape[1], x.cpu().view(torch.int16).numpy().view(np.uint16),
                                    threads=threads)
            t_cpu += time.perf_counter() - t1
            passes += 1
        cpu = {"value": round(2 * passes * n_total / t_cpu / 1e9, 3), "unit": "GB/s", "cores": threads,
               "kind": "oracle",
               "sample": f"{passes} whole passes over the layer's {len(specs)} matrices ({n_total} weights): "
                         f"bit-serial decode on {threads} threads, float64 conversion and numpy product; "
                         f"{time.process_time() - cpu0:.1f} CPU-s", "seconds": round(t_cpu, 2)}

    line = {
        "metric": GEMM_METRIC if gemm else GEMV_METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_fused, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 products, f32 sums", "data": "synthetic",
        "config": {"workload": workload, "matrices": len(specs), "weights": n_total, "m": m,
                   "blob_bytes": blob_total, "copies": copies},
        "within_bound": bool(within), "roofline": roofline, "compare": compare, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0 if within else 1


def bench_token(args, threads: int) -> int:
    """The weights of one generated token, end to end: every matrix of the
    whole model (40 layers' seven, and the output head) multiplied by the
    token's activations (m = 1, 2 or 4 rows), straight from the compressed
    model resident in HBM with the fused matrix-vector kernel, one batch call
    per unit. Compared with the same products on the BF16 model resident in
    HBM (torch.mm, and torch.mv at m = 1) and with restoring each unit into one scratch buffer
    before its products. The embedding lookup reads one row and is left out.
    The activations are synthetic; nothing between the products (attention,
    norms) is computed: this times the weight pass the pages' per-token
    figures are made of."""
    import torch

    from lossless_bf16_weight_afx_amd import afx, stream, synth

    dev = torch.device("cuda:0")
    m = args.m if args.m is not None else 1
    if m not in (1, 2, 4):
        raise SystemExit("--workload token takes --m 1, 2 or 4")
    t0 = time.time()
    units = stream.build_model(synth.model_units(args.layers)[1:], threads=threads, progress=log)  # no embedding
    log(f"[bench] model store ready in {time.time() - t0:.0f}s")
    gen = torch.Generator(device="cpu").manual_seed(11)
    xs = {}  # one activation block per input width, shared by the matrices that read it

    def x_for(cols):
        if cols not in xs:
            xs[cols] = torch.randn((m, cols), generator=gen).to(torch.bfloat16).to(dev)
        return xs[cols]

    blobs, per_unit, unit_mats, mats = [], [], [], []  # mats: (spec, info, device blob address, y)
    for u in units:
        db = u.host.to(dev)
        blobs.append(db)
        um = []
        for sp, info, off in zip(u.specs, u.infos, u.offsets):
            if len(sp.shape) == 2:
                um.append((sp, info, db.data_ptr() + off, torch.zeros((m, sp.shape[0]), dtype=torch.float32,
                                                                     device=dev)))
        per_unit.append(afx.make_gemv_jobs([(info, ptr, sp.shape[0], sp.shape[1], x_for(sp.shape[1]).data_ptr(),
                                             y.data_ptr()) for sp, info, ptr, y in um]))
        unit_mats.append(um)
        mats += um
    n_weights = sum(int(mt[1].n_elems) for mt in mats)
    blob_total = sum(int(mt[1].blob_bytes) for mt in mats)
    stream_ = torch.cuda.current_stream(dev)
    sp_ = stream_.cuda_stream
    log(f"[bench] token pass: {len(mats)} matrices, {n_weights} weights, {blob_total} B compressed in HBM")

    def fused(k):
        for jobs in per_unit:
            afx.afx_restore_gemv_batch_async(jobs, m, sp_)

    # BF16 copies of every matrix, restored by the library (bit-exact), for
    # the comparisons and the check
    wbf = []
    for sp, info, ptr, _ in mats:
        w = torch.empty(sp.shape, dtype=torch.bfloat16, device=dev)
        afx.afx_decode_layer_async(afx.make_jobs([(info, ptr, w.data_ptr(), 2 * int(info.n_elems))]), sp_)
        wbf.append(w)
    torch.cuda.synchronize()

    # check (outside the timing): one pass from zero against FP32 products of
    # the restored weights, within twice the summation bound
    for _, _, _, y in mats:
        y.zero_()
    fused(0)
    torch.cuda.synchronize()
    within = True
    for (sp, _, _, y), w in zip(mats, wbf):
        wf, xf = w.float(), x_for(sp.shape[1]).float()
        j = (sp.shape[1] - 1) * 2.0 ** -24
        bound = j / (1 - j) * (xf.abs() @ wf.abs().t())
        within &= bool(((y - xf @ wf.t()).abs() <= 2 * bound + 1e-30).all())
        del wf
    if not within:
        log("[bench] fused products fall outside the FP32 summation bound")

    ms_fused = _time_steps(stream_, fused, args.steps, args.warmup)

    def mm(k):
        for (sp, _, _, _), w in zip(mats, wbf):
            torch.mm(x_for(sp.shape[1]), w.t())

    def mv(k):  # torch's matrix-vector path, for one token
        for (sp, _, _, _), w in zip(mats, wbf):
            torch.mv(w, x_for(sp.shape[1])[0])

    ms_mm = _time_steps(stream_, mm, args.steps, args.warmup)
    ms_mv = _time_steps(stream_, mv, args.steps, args.warmup) if m == 1 else None
    del wbf
    torch.cuda.empty_cache()
    # restore each unit into one scratch buffer (256-byte aligned outputs),
    # then multiply
    slot = lambda n: (n + 127) // 128 * 128
    scratch = torch.empty(max(sum(slot(int(info.n_elems)) for _, info, _, _ in um) for um in unit_mats),
                          dtype=torch.bfloat16, device=dev)
    rjobs, rmats = [], []
    for um in unit_mats:
        js, ws, off = [], [], 0
        for sp, info, ptr, _ in um:
            n = int(info.n_elems)
            w = scratch[off:off + n].view(sp.shape)
            js.append((info, ptr, w.data_ptr(), 2 * n))
            ws.append((sp, w))
            off += slot(n)
        rjobs.append(afx.make_jobs(js))
        rmats.append(ws)

    def restore_mm(k):
        for js, ws in zip(rjobs, rmats):
            afx.afx_decode_layer_async(js, sp_)
            for sp, w in ws:
                torch.mm(x_for(sp.shape[1]), w.t())

    ms_rmm = _time_steps(stream_, restore_mm, args.steps, args.warmup)
    value = 2 * n_weights / (ms_fused * 1e-3) / 1e9
    line = {
        "metric": GEMV_METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_fused, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 products, f32 sums", "data": "synthetic",
        "config": {"workload": f"qwen3-14b-model-{args.layers}-layers-token-pass-m{m}", "matrices": len(mats),
                   "weights": n_weights, "m": m, "blob_bytes": blob_total,
                   "bf16_bytes": 2 * n_weights, "launches": len(per_unit)},
        "within_bound": bool(within),
        "token_pass_ms": {"fused_from_compressed": round(ms_fused, 3), "bf16_resident_torch_mm": round(ms_mm, 3),
                          "restore_each_unit_then_torch_mm": round(ms_rmm, 3),
                          **({"bf16_resident_torch_mv": round(ms_mv, 3)} if ms_mv is not None else {})},
        "hbm_weight_bytes": {"compressed": blob_total, "bf16": 2 * n_weights},
        "roofline": {"bound": "hbm", "achieved": round(blob_total / (ms_fused * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(blob_total / (ms_fused * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "afx_gemv_kernel"},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)
    return 0 if within else 1


def bench_model(args, threads: int) -> int:
    """The default workload: the whole synthetic model, 40 Qwen3-14B-shaped
    layers, the embedding, the untied output head and the final norm (42
    units, ~29.5 GB BF16), compressed in pinned host memory.

    `value` is one pass of the restore over the whole model with its
    compressed bytes resident in HBM (one call and one launch per unit, each
    unit into its own output region). Beside it: the streamed pass (unit i+1
    copied over the host link while unit i is restored), the restore of the
    embedding (unit 0) and of layer 0 (unit 1) timed inside a resident pass,
    and the CPU oracle on a bounded sample of the units.

    Checks, off the clock: a streamed pass that runs free copies every
    unit's restored output aside on the compute stream, and each copy is
    compared with the unit's original bits generated again from its seeds;
    the resident pass is compared with those copies; the oracle's decode of
    the sampled units is compared with them too."""
    import torch

    from lossless_bf16_weight_afx_amd import ready, stream, synth

    dev = torch.device("cuda:0")
    t0 = time.time()
    units = stream.build_model(synth.model_units(args.layers), threads=threads, progress=log)
    restored = 2 * sum(u.n_values for u in units)
    blob_total = sum(u.blob_bytes for u in units)
    workload = f"qwen3-14b-model-{args.layers}-layers"
    log(f"[bench] model store ready in {time.time() - t0:.0f}s: {restored} B restored, {blob_total} B compressed")

    # ---- checked streamed pass, running free: every unit's output copied
    # aside after its restore, then compared with its original bits
    st = stream.Streamer(units)
    snaps = [torch.empty(stream.unit_slots(u), dtype=torch.int16, device=dev) for u in units]
    st.run(snapshot=snaps)
    torch.cuda.synchronize()
    t1 = time.time()
    ok = [stream.check_unit_regen(u, sn, threads) for u, sn in zip(units, snaps)]
    exact = all(ok)
    log(f"[bench] checked streamed pass, {len(units)} units against their original bits "
        f"({time.time() - t1:.0f}s): bit_exact={exact}" + ("" if exact else f" (bad units {[i for i, o in enumerate(ok) if not o]})"))

    # ---- streamed passes, timed
    for _ in range(max(1, args.warmup)):
        st.run()
    runs = [st.run() for _ in range(max(1, args.steps))]
    e2e_ms = float(np.median([r["e2e_ms"] for r in runs]))
    dec_ms = float(np.median([sum(r["decode_ms"]) for r in runs]))
    link_ms = float(np.median([st.link_copy_ms() for _ in range(3)]))
    t_dec_layer = float(np.median([r["decode_ms"][1] for r in runs])) * 1e-3
    del st
    torch.cuda.empty_cache()

    # ---- the resident pass: `value`; checked against the streamed pass's
    # copies, then timed (the whole pass between two events on the launch
    # stream), then one more pass with an event between every two units
    res = stream.resident_decode(units, steps=max(1, args.steps), check=True, reference=snaps,
                                 warmup=max(1, args.warmup), per_unit=True)
    exact &= bool(res["bit_exact"])
    log(f"[bench] checked resident pass against the streamed one: bit_exact={res['bit_exact']}")
    resident_ms = res["ms"]
    launches = res["launches"]
    value = restored / (resident_ms * 1e-3) / 1e9
    alg = blob_total + restored
    achieved = alg / (resident_ms * 1e-3) / 1e9

    def unit_figures(k: int, name: str) -> dict:
        u = units[k]
        ms = res["unit_ms"][k]
        a = u.blob_bytes + 2 * u.n_values
        return {"unit": k, "name": name, "tensors": len(u.specs), "values": u.n_values,
                "restored_bytes": 2 * u.n_values, "blob_bytes": u.blob_bytes, "us": round(ms * 1e3, 1),
                "restored_GBps": round(2 * u.n_values / (ms * 1e-3) / 1e9, 1),
                "roofline_frac": round(a / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}

    per_config = {"decoder_layer_0": unit_figures(1, "qwen3-14b-decoder-layer (layers.0, one launch)"),
                  "embedding": unit_figures(0, "qwen3-14b-embedding-151936x5120 (one launch)")}

    layer_alg = units[1].blob_bytes + 2 * units[1].n_values
    copy_gbps, copy_each_way = copy_ceiling(torch.cuda.current_stream(dev), layer_alg, 4)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": profile_traffic(workload),
                "algorithmic_bytes_per_launch": round(alg / launches), "launches_per_step": launches,
                "kernel": KERNEL_NAME, "kernel_ms": round(resident_ms / launches, 5),
                "copy_ceiling_GBps": round(copy_gbps, 1), "calib_copy_bytes_each_way": copy_each_way}

    link_gbps = blob_total / (link_ms * 1e-3) / 1e9
    layer = units[1]
    eq2 = {"saved_link_s_per_layer": round((2 * layer.n_values - layer.blob_bytes) / (link_gbps * 1e9), 6),
           "decode_s_per_layer": round(t_dec_layer, 6),
           "compression_pays": bool(ready.compression_pays(2 * layer.n_values, layer.blob_bytes,
                                                          link_gbps * 1e9, t_dec_layer))}
    streamed = {"ready_weight_GBps_e2e": round(restored / (e2e_ms * 1e-3) / 1e9, 1),
                "decode_only_GBps": round(restored / (dec_ms * 1e-3) / 1e9, 1),
                "e2e_ms": round(e2e_ms, 2), "decode_ms": round(dec_ms, 2),
                "link_GBps_compressed_copy": round(link_gbps, 1),
                "uncompressed_copy_equiv_ms": round(restored / (link_gbps * 1e9) * 1e3, 2),
                "eq2_per_layer": eq2}

    cpu = None
    if not args.no_cpu_baseline:
        cpu, ok_cpu = model_cpu_baseline(units, snaps, threads)
        exact &= ok_cpu
    del snaps
    torch.cuda.empty_cache()

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(resident_ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "u32", "data": "synthetic",
        "config": {"workload": workload, "units": len(units), "values": restored // 2,
                   "restored_bytes": restored, "blob_bytes": blob_total, "ratio": round(blob_total / restored, 4),
                   "launches_per_pass": launches, "encoder": "libafx afx_encode"},
        "bit_exact": bool(exact), "roofline": roofline, "per_config": per_config, "streamed": streamed,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0 if exact else 1


def model_cpu_baseline(units, snaps, threads: int):
    """The CPU oracle's chunk-parallel decoder on a bounded sample of the
    model's units (layer 0, the embedding, the head, then layers spread over
    the model) until about 15 CPU-seconds are spent, on `threads` threads;
    and the same decoder on one thread for about 3 seconds. Each sampled
    unit's decode is compared with the GPU's restored copy."""
    import oracle

    order = [1, 0, len(units) - 1] + [k for k in range(2, len(units) - 1, 7)]
    n_dec, t_dec, exact, sampled = 0, 0.0, True, []
    cpu0 = time.process_time()
    for k in order:
        u = units[k]
        gpu = snaps[k].cpu().numpy().view(np.uint16)
        off = 0
        for info, boff in zip(u.infos, u.offsets):
            blob = u.host[boff:boff + int(info.blob_bytes)].numpy()
            t0 = time.perf_counter()
            d = oracle.decode(blob, threads=threads)
            t_dec += time.perf_counter() - t0
            n = int(info.n_elems)
            exact &= bool(np.array_equal(d, gpu[off:off + n]))
            off += (n + 127) // 128 * 128
            n_dec += n
        sampled.append(u.name)
        if time.process_time() - cpu0 > 15.0:
            break
    cpu_s = time.process_time() - cpu0
    n1, t1 = 0, 0.0
    for info, boff in zip(units[1].infos, units[1].offsets):
        blob = units[1].host[boff:boff + int(info.blob_bytes)].numpy()
        t0 = time.perf_counter()
        oracle.decode(blob, threads=1)
        t1 += time.perf_counter() - t0
        n1 += int(info.n_elems)
        if t1 > 3.0:
            break
    cpu = {"value": round(2 * n_dec / t_dec / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"units {', '.join(sampled)} of the model ({n_dec} values, {2 * n_dec} B restored): bit-serial "
                     f"canonical decode, chunk-parallel over {threads} threads; {cpu_s:.1f} CPU-s",
           "seconds": round(t_dec, 2), "host": host_cpu_facts(),
           "one_thread": {"value": round(2 * n1 / t1 / 1e9, 3), "unit": "GB/s",
                          "sample": f"{n1} values of layers.0's tensors in turn, one thread"}}
    return cpu, exact


def bench_disk(args, threads: int) -> int:
    """The whole synthetic model stored compressed in a file and made ready
    in HBM: read from disk (O_DIRECT, so the page cache never serves it) into
    pinned memory, copied to the GPU, restored; the three steps of
    consecutive units overlap. `value` is restored BF16 bytes per second of
    the whole pass (time to ready weights); the read, copy and restore rates
    measured alone are reported beside it, with the pages' Eq. (1) and
    Eq. (2) evaluated on them, and the same pass with the pages' placement
    of the unpack (on the host, before the copy)."""
    import torch

    from lossless_bf16_weight_afx_amd import store, synth

    specs = synth.model_units(args.layers)
    path = os.path.join(args.store_dir, f"afx_model_{args.layers}l_{os.getpid()}.afxs")
    t0 = time.time()
    st = store.write_store(path, specs, threads=threads, progress=log)
    write_s = time.time() - t0
    try:
        try:
            fd = os.open(path, os.O_RDONLY | os.O_DIRECT)
            os.close(fd)
            direct = True
        except OSError:
            direct = False
        log(f"[bench] store {path}: {st.file_bytes} B written in {write_s:.0f}s; O_DIRECT={direct}")
        ds = store.DiskStreamer(st, threads=threads, direct=direct)
        stored = sum(u.bytes for u in st.units)
        restored = st.restored_bytes
        # bit-exact pass: the embedding, the first and last layers, the head
        check_idx = {0, 1, len(st.units) - 2, len(st.units) - 1}
        ok = []
        ds.run(on_unit=lambda i, u, out: ok.append(store.check_unit(out, specs[i])) if i in check_idx else None)
        exact = len(ok) == len(check_idx) and all(ok)
        log(f"[bench] checked pass over {sorted(check_idx)}: bit_exact={exact}")
        read_s = float(np.median([ds.read_only_s() for _ in range(max(1, min(args.steps, 3)))]))
        copy_s = float(np.median([ds.copy_only_s() for _ in range(3)]))
        runs = []
        for k in range(max(1, args.steps)):  # each pass takes seconds: report each
            runs.append(ds.run())
            log(f"[bench] pass {k + 1}/{max(1, args.steps)}: {runs[-1]['e2e_s']:.2f} s")
        e2e_s = float(np.median([r["e2e_s"] for r in runs]))
        dec_ms = float(np.median([sum(r["decode_ms"]) for r in runs]))
        b_disk = stored / read_s
        b_link = stored / copy_s
        layer = st.units[1]
        s_disk, s_full = layer.bytes, 2 * layer.n_values
        t_unpack = float(np.median([r["decode_ms"][1] for r in runs])) * 1e-3
        eq1 = {"read_s": round(s_disk / b_disk, 5), "copy_s": round(s_disk / b_link, 5), "unpack_s": round(t_unpack, 6),
               "t_prep_serial_s": round(s_disk / b_disk + s_disk / b_link + t_unpack, 5),
               "uncompressed_read_s": round(s_full / b_disk, 5)}
        eq2 = {"saved_read_s": round((s_full - s_disk) / b_disk, 5), "unpack_s": round(t_unpack, 6),
               "compression_pays": bool((s_full - s_disk) / b_disk > t_unpack)}
        line = {
            "metric": "ready BF16 weights GB/s from disk on 1 MI355X (read + copy + restore, overlapped)",
            "value": round(restored / e2e_s / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": 0, "ms_per_step": round(e2e_s * 1e3, 1), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "u32", "data": "synthetic",
            "config": {"workload": f"qwen3-14b-model-{args.layers}-layers-from-disk", "units": len(st.units),
                       "restored_bytes": restored, "stored_bytes": stored, "o_direct": direct,
                       "reader_threads": threads},
            "bit_exact": bool(exact),
            "disk_read_GBps": round(b_disk / 1e9, 3), "link_GBps": round(b_link / 1e9, 2),
            "decode_only_GBps": round(restored / (dec_ms * 1e-3) / 1e9, 1),
            "uncompressed_read_equiv_s": round(restored / b_disk, 2), "pass_s": round(e2e_s, 2),
            "read_bound_s": round(stored / b_disk, 2),
            "eq1_per_layer": eq1, "eq2_per_layer": eq2, "store_write_s": round(write_s, 1),
            "roofline": None, "cpu_baseline": None,
        }
        del ds
        torch.cuda.empty_cache()
        # the pages' placement: unpack on the host, copy the restored bytes
        hs = store.HostUnpackStreamer(st, read_threads=threads, unpack_threads=threads, direct=direct)
        ok = []
        hs.run(on_unit=lambda i, u, out: ok.append(store.check_unit(out, specs[i])) if i in check_idx else None)
        exact_h = len(ok) == len(check_idx) and all(ok)
        log(f"[bench] checked host-unpack pass over {sorted(check_idx)}: bit_exact={exact_h}")
        t_unpack_host = float(np.median([hs.unpack_only_s(1) for _ in range(3)]))
        hruns = []
        for k in range(max(1, args.steps)):
            hruns.append(hs.run())
            log(f"[bench] host-unpack pass {k + 1}/{max(1, args.steps)}: {hruns[-1]['e2e_s']:.2f} s")
        h_e2e = float(np.median([r["e2e_s"] for r in hruns]))
        line["host_unpack"] = {
            "pass_s": round(h_e2e, 2), "ready_weight_GBps": round(restored / h_e2e / 1e9, 2),
            "unpack_threads": threads, "unpack_GBps_per_layer_alone": round(s_full / t_unpack_host / 1e9, 2),
            "eq2_per_layer": {"saved_read_s": eq2["saved_read_s"], "unpack_s": round(t_unpack_host, 5),
                              "compression_pays": bool((s_full - s_disk) / b_disk > t_unpack_host)},
            "bit_exact": bool(exact_h)}
        line["bit_exact"] = bool(exact and exact_h)
        print(json.dumps(line), flush=True)
        del hs
        torch.cuda.empty_cache()
        return 0 if line["bit_exact"] else 1
    finally:
        if not args.keep_store:
            os.unlink(path)


def bench_tiers(args, threads: int) -> int:
    """Residency tiers: the whole model stored compressed on disk, a plan
    under a GPU-memory budget (and a pinned-RAM budget) keeps some units
    restored or compressed in HBM or compressed in RAM, and one pass over the
    model restores every unit in order. Reports the pass time per budget, the
    trade-off of "Keeping some weights close" (Table 1 of "Why Weight
    Offloading Slows Inference") on this machine."""
    import torch

    from lossless_bf16_weight_afx_amd import store, synth, tiers

    specs = synth.model_units(args.layers)
    path = os.path.join(args.store_dir, f"afx_tiers_{args.layers}l_{os.getpid()}.afxs")
    st = store.write_store(path, specs, threads=threads, progress=log)
    try:
        try:
            fd = os.open(path, os.O_RDONLY | os.O_DIRECT)
            os.close(fd)
            direct = True
        except OSError:
            direct = False
        ds = store.DiskStreamer(st, threads=threads, direct=direct)
        read_s = ds.read_only_s()
        copy_s = ds.copy_only_s()
        dec_ms = ds.run()["decode_ms"]
        del ds
        torch.cuda.empty_cache()
        stored = sum(u.bytes for u in st.units)
        rates = tiers.Rates(read_Bps=stored / read_s, copy_Bps=stored / copy_s, restore_s=[d * 1e-3 for d in dec_ms])
        log(f"[bench] rates: read {rates.read_Bps / 1e9:.2f} GB/s, copy {rates.copy_Bps / 1e9:.1f} GB/s, "
            f"restore {sum(dec_ms):.1f} ms per pass")
        GB = 10 ** 9
        budgets = [(0, 0), (4 * GB, 0), (8 * GB, 0), (16 * GB, 0), (24 * GB, 0), (32 * GB, 0), (0, 24 * GB),
                   (4 * GB, 24 * GB)]
        rows, exact = [], True
        check_idx = {1, len(st.units) - 2}  # the first and the last layer
        for gpu_b, host_b in budgets:
            tier = tiers.plan(st, gpu_b, host_b, rates)
            tp = tiers.TieredPass(st, tier, threads=threads, direct=direct)
            ok = []
            tp.run(on_unit=lambda i, out: ok.append(store.check_unit(out, specs[i])) if i in check_idx else None)
            exact &= len(ok) == len(check_idx) and all(ok)
            passes = []
            for k in range(max(1, args.steps)):  # a pass can take seconds: report each
                passes.append(tp.run())
                log(f"[bench]   pass {k + 1}/{max(1, args.steps)}: {passes[-1]:.3f} s")
            pass_s = float(np.median(passes))
            counts = {t: tier.count(t) for t in tiers.TIERS}
            rows.append({"gpu_budget_GB": gpu_b / GB, "host_budget_GB": host_b / GB, "tiers": counts,
                         "hbm_held_GB": round(tp.hbm_bytes() / GB, 2), "pass_s": round(pass_s, 4),
                         "ready_weight_GBps": round(st.restored_bytes / pass_s / GB, 2),
                         "model_s": round(sum(tiers.unit_cost_s(t, u.bytes, r, rates)
                                              for t, u, r in zip(tier, st.units, rates.restore_s)), 4)})
            log(f"[bench] budget gpu {gpu_b / GB:.0f} GB host {host_b / GB:.0f} GB: {counts}, pass {pass_s:.3f} s")
            del tp
            torch.cuda.empty_cache()
        line = {
            "metric": "seconds per pass over the model by residency budget on 1 MI355X", "value": rows[0]["pass_s"],
            "unit": "s", "n_gpus": 1, "steps": args.steps, "warmup": 1, "ms_per_step": round(rows[0]["pass_s"] * 1e3, 1),
            "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "u32", "data": "synthetic",
            "config": {"workload": f"qwen3-14b-model-{args.layers}-layers-tiers", "units": len(st.units),
                       "restored_bytes": st.restored_bytes, "stored_bytes": stored, "o_direct": direct},
            "bit_exact": bool(exact), "rates": {"read_GBps": round(rates.read_Bps / GB, 3),
                                                "copy_GBps": round(rates.copy_Bps / GB, 2),
                                                "restore_ms_per_pass": round(sum(dec_ms), 2)},
            "budgets": rows, "roofline": None, "cpu_baseline": None,
        }
        print(json.dumps(line), flush=True)
        return 0 if exact else 1
    finally:
        if not args.keep_store:
            os.unlink(path)


if __name__ == "__main__":
    sys.exit(main())
