"""Benchmark of the online-rotation hot path on one MI355X.

One step is one pass over every hot-path call, each on its full workload:
  * kv_rotate_quant   -- R3 on post-RoPE Q and K, bf16 [16, 32, 2048, 128] each;
  * hadamard_quant_int4 -- R4 on the down-projection input, bf16 [8192, 16384], n = 16384;
  * w4a4_gemm         -- A [4096, 4096] x W [11008, 4096] packed INT4, bf16 output.
Inputs are seeded synthetic tensors (workloads.py) already resident in HBM; four input and
output sets per call (more than the 256 MB last-level cache between two uses of a set) are
rotated so the timed reads come from HBM.

Timing:
  * pre-warm: steps run untimed until at least --prewarm-ms of wall time has passed (the
    device runs slower for its first tens of milliseconds of sustained load), then the
    --warmup steps;
  * the timed region: exactly --steps steps, bracketed by synchronisation and one pair of
    HIP events on the stream the library launches on (ms_per_step);
  * per-kernel time: right after, each kernel alone, --steps launches back to back over
    the rotated sets, bracketed by one event pair (no event between two launches, so no
    marker packet separates them); this is the kernel's average launch duration that the
    roofline figures use.

The headline value is the fused Hadamard + INT4 quantizer's throughput at n = 16384 in
algorithmic GB/s (bf16 input read once, packed codes and fp16 scales written once); the
GEMM's TOPS and the per-call times are reported beside it, with the fp64 oracle timed on
a bounded sample on the host cores as a baseline.

usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--only r4|kv|gemm|kron|copy|stream]
"""

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, published
INT8_PEAK_TOPS = 5000.0   # MI355X dense int8 MFMA, published (no sparsity)
NSETS = 4

R4_TOKENS, R4_N = 8192, 16384
KV_SHAPE = (16, 32, 2048, 128)
GEMM_M, GEMM_N, GEMM_K = 4096, 11008, 4096
KRON_N = 14336
KRON_BYTES = 8192 * KRON_N * 2 + 8192 * KRON_N // 2 + 8192 * 2

R4_BYTES = R4_TOKENS * R4_N * 2 + R4_TOKENS * R4_N // 2 + R4_TOKENS * 2
KV_ROWS = KV_SHAPE[0] * KV_SHAPE[1] * KV_SHAPE[2]
KV_BYTES = 2 * (KV_ROWS * KV_SHAPE[3] * 2 + KV_ROWS * KV_SHAPE[3] // 2 + KV_ROWS * 2)
GEMM_OPS = 2 * GEMM_M * GEMM_N * GEMM_K
GEMM_BYTES = GEMM_M * GEMM_K // 2 + GEMM_N * GEMM_K // 2 + GEMM_M * 2 + GEMM_N * 2 + GEMM_M * GEMM_N * 2


def kernel_source_hash(files):
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "rotation_bit_quantization_fwht_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


FWHT_SOURCES = ("common.h", "plan.h", "fwht_engine.h", "devctx.h", "fwht_kernels.hip")
GEMM_SOURCES = ("common.h", "w4a4_gemm.hip")
KRON_SOURCES = ("common.h", "fwht_engine.h", "devctx.h", "kron_engine.h", "kron_factor.h", "kron_quant.hip")


def load_counters(name, src_hash):
    """The committed rocprofv3 counter summary of one kernel (profiles/counters.json), if it
    was taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except ValueError:
        return None
    e = d.get(name)
    if not e or e.get("source_hash") != src_hash:
        return None
    return e


def load_traffic(name, src_hash):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE passes (or None)."""
    e = load_counters(name, src_hash)
    return None if e is None else e.get("hbm_bytes_per_launch")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline():
    """The oracle as it stands, on a bounded sample of the n=16384 workload."""
    import oracle
    import workloads

    try:
        from threadpoolctl import threadpool_info

        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing or no BLAS info
        cores = os.cpu_count() or 1
    rows = 16
    xb, _ = workloads.gen_ffn(seed=7, tokens=rows, n=R4_N)
    x64 = workloads.to_float64(xb, "bfloat16")
    t0 = time.perf_counter()
    reps = 0
    while True:
        oracle.hadamard_quant_int4(x64, "float16", packed=True)
        reps += 1
        if time.perf_counter() - t0 > 12.0 or reps >= 200:
            break
    dt = (time.perf_counter() - t0) / reps
    sample_bytes = rows * (R4_N * 2 + R4_N // 2 + 2)
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    return {
        "value": round(sample_bytes / dt / 1e9, 6),
        "unit": "GB/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"{rows} rows of the bf16 [8192, 16384] R4 workload, explicit fp64 Sylvester "
                  f"multiply + quantizer, {reps} repetitions, {dt:.2f} s each",
        "cpu_model": cpu_model(),
        "host_cpus": os.cpu_count(),
        "host_cpus_usable": affinity,
        "blas_threads": int(cores),
    }


def time_back_to_back(torch, fns, reps):
    """Average device time per launch: ``reps`` launches cycling over ``fns`` (one callable
    per rotated input set), issued back to back and bracketed by one event pair on the
    current stream (the one the binding hands to the library)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(reps):
        fns[i % len(fns)]()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def time_calls(torch, fn, reps):
    """Average device time per call (events on the current stream) and host time per call
    (wall clock from the first launch to the end of the last, synchronised)."""
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    host = (time.perf_counter() - t0) / reps
    return e0.elapsed_time(e1) * 1e3 / reps, host * 1e6


def time_graph(torch, fn, calls=20, replays=10):
    """Device time per call with the launches captured in a HIP graph (no host overhead
    between kernels); returns us per call."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (calls * replays)


def hbm_probe_rates(torch, rbq, dev, reps=20):
    """The streaming probe (rbq_hbm_probe) on 2 GiB of reads and/or writes: reads alone,
    writes alone, and R4's row shape (each workgroup reads 32 KiB then writes 8 KiB, the
    bytes of one bf16 row of 16384 and its packed codes). GB/s of moved bytes."""
    big = 1 << 31
    src = torch.empty(big // 4, dtype=torch.int32, device=dev)
    src.fill_(0x01234567)
    dst = torch.empty(big // 4, dtype=torch.int32, device=dev)
    out = {}
    shapes = (("read_only", 65536, 0, big // 65536),
              ("write_only", 0, 65536, big // 65536),
              ("r4_row_mix", 32768, 8192, big // 32768))
    for name, rd, wr, blocks in shapes:
        fn = lambda rd=rd, wr=wr, blocks=blocks: rbq.hbm_probe(src, rd, dst, wr, blocks)  # noqa: E731
        for _ in range(5):
            fn()
        us = time_back_to_back(torch, [fn], reps)
        moved = blocks * (rd + wr)
        out[name] = {"read_bytes": blocks * rd, "write_bytes": blocks * wr, "avg_us": round(us, 3),
                     "GB_s": round(moved / (us * 1e-6) / 1e9, 1)}
    del src, dst
    return out


def report_small_workloads(torch, rbq, workloads, dev):
    """The latency-bound workloads: the 64 x 4096 fp32 worked example (int8 codes, fp32
    scales; MSE of the dequantized values with and without rotation, computed from the
    GPU outputs) and the decode sweep (per call: device and host microseconds of eager
    launches through the binding, and device microseconds with the launches replayed from
    a HIP graph; next to the same figures for a one-element torch kernel)."""
    out = {}
    x = workloads.gen_worked_example(seed=0)
    xd = torch.from_numpy(x).to(dev)
    codes = torch.empty((64, 4096), dtype=torch.int8, device=dev)
    scales = torch.empty((64,), dtype=torch.float32, device=dev)
    dev_us, host_us = time_calls(
        torch, lambda: rbq.hadamard_quant_int4(xd, scale_dtype=torch.float32, packed=False, codes=codes, scales=scales), 200)
    c, sc, rot = rbq.hadamard_quant_int4(xd, scale_dtype=torch.float32, packed=False, return_rotated=True)
    dc, ds = rbq.hadamard_quant_int4(xd, scale_dtype=torch.float32, packed=False, rotate=False)
    y = rot.cpu().numpy().astype(np.float64)
    q = c.cpu().numpy().astype(np.float64) * sc.cpu().numpy().astype(np.float64)[:, None]
    qd = dc.cpu().numpy().astype(np.float64) * ds.cpu().numpy().astype(np.float64)[:, None]
    # rotation is orthogonal, so the error measured in the rotated basis equals the error of
    # rotate -> quantize -> rotate back in the original basis
    mse_rot = float(np.mean((y - q) ** 2))
    mse_direct = float(np.mean((x.astype(np.float64) - qd) ** 2))
    out["worked_example"] = {
        "workload": "fp32 [64, 4096], channel 142 = 60; int8 codes, fp32 scales",
        "device_us": round(dev_us, 3), "host_us": round(host_us, 3),
        "mse_rotated": mse_rot, "mse_direct": mse_direct, "mse_ratio": mse_rot / mse_direct,
    }
    one = torch.zeros((1,), dtype=torch.float32, device=dev)
    floor_dev, floor_host = time_calls(torch, lambda: one.add_(0.0), 500)
    floor_graph = time_graph(torch, lambda: one.add_(0.0))
    pts = []
    for n in workloads.DECODE_N:
        for t in workloads.DECODE_TOKENS:
            xb, _ = workloads.gen_decode(seed=0, tokens=t, n=n)
            xd16 = torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).view(torch.bfloat16).to(dev)
            cb = torch.empty((t, n // 2), dtype=torch.uint8, device=dev)
            sb = torch.empty((t,), dtype=torch.float16, device=dev)
            call = lambda: rbq.hadamard_quant_int4(xd16, codes=cb, scales=sb)  # noqa: E731
            d_us, h_us = time_calls(torch, call, 200)
            ref_codes = cb.clone()
            g_us = time_graph(torch, call)
            same = bool(torch.equal(cb, ref_codes))
            nbytes = t * n * 2 + t * n // 2 + 2 * t
            pts.append({"tokens": t, "n": n, "device_us": round(d_us, 3), "host_us": round(h_us, 3),
                        "graph_us": round(g_us, 3), "graph_matches_eager": same,
                        "GB_s_graph": round(nbytes / (g_us * 1e-6) / 1e9, 2)})
    out["decode_sweep"] = {"floor_device_us": round(floor_dev, 3), "floor_host_us": round(floor_host, 3),
                           "floor_graph_us": round(floor_graph, 3),
                           "floor_kernel": "one-element torch add", "points": pts}
    return out


def copy_calibration(torch, args):
    """Plain 1 GiB device copy: calibrates the HBM byte counters, and its rate is what a
    simple read+write stream (torch's own copy kernel) reaches on this device."""
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    src.fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    nbytes = src.numel() * 4
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes,
                      "launches": args.warmup + args.steps,
                      "copy_GB_s": round(2 * nbytes * args.steps / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)}))


GEMM_SHAPES = ((4096, 4096, 4096), (4096, 4096, 16384), (4096, 8192, 4096), (4096, 11008, 4096),
               (4096, 11008, 8192), (8192, 11008, 4096))


def gemm_shapes(torch, rbq, dev, reps):
    """W4A4 GEMM over tile grids of one, two and 2.69 waves and over K: where the time goes.
    Seeded random packed codes (the values do not change the timing), four operand sets per
    shape cycled back to back after a 300 ms pre-warm of their own; best of three runs."""
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    out = []
    for (M, N, K) in GEMM_SHAPES:
        sets = []
        for _ in range(NSETS):
            qa = torch.randint(0, 256, (M, K // 2), dtype=torch.uint8, device=dev, generator=g)
            qw = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device=dev, generator=g)
            sa = (torch.rand(M, device=dev, generator=g) * 0.01 + 0.001).half()
            sw = (torch.rand(N, device=dev, generator=g) * 0.01 + 0.001).half()
            sets.append((qa, sa, qw, sw, torch.empty((M, N), dtype=torch.bfloat16, device=dev)))
        fns = [lambda s=s: rbq.w4a4_gemm(s[0], s[1], s[2], s[3], out=s[4]) for s in sets]
        t0 = time.time()
        while time.time() - t0 < 0.3:
            for f in fns:
                f()
            torch.cuda.synchronize()
        us = min(time_back_to_back(torch, fns, reps) for _ in range(3))
        ops = 2 * M * N * K
        out.append({"M": M, "N": N, "K": K, "tiles": -(-M // 256) * -(-N // 256), "avg_us": round(us, 2),
                    "TOPS": round(ops / us / 1e6, 1), "frac_int8_mfma_peak": round(ops / us / 1e6 / INT8_PEAK_TOPS, 4)})
        del sets, fns
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--prewarm-ms", type=float, default=200.0,
                    help="untimed steps run for at least this much wall time before --warmup")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the reports beside the step (worked example, decode sweep, variants)")
    ap.add_argument("--only", choices=["all", "r4", "kv", "gemm", "kron", "copy", "stream", "gemm_shapes"], default="all",
                    help="restrict the step (for profiling one kernel); 'copy' runs a plain 1 GiB "
                         "device copy used to calibrate the HBM byte counters; 'gemm_shapes' times the W4A4 GEMM over several tile grids and K; 'stream' runs the "
                         "HBM streaming probe")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1); "
              "the design notes describe how the path would shard", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.only == "copy":
        copy_calibration(torch, args)
        return

    import rotation_bit_quantization_fwht_amd as rbq
    import workloads

    if not os.path.exists(rbq.library_path()):
        from rotation_bit_quantization_fwht_amd.build import build

        build()
    rbq.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.only == "gemm_shapes":
        print(json.dumps({"w4a4_gemm_shapes": gemm_shapes(torch, rbq, dev, max(args.steps, 20))}), flush=True)
        return

    if args.only == "stream":
        print(json.dumps({"hbm_probe": hbm_probe_rates(torch, rbq, dev, reps=args.steps),
                          "peak_GB_s": HBM_PEAK_GBS}), flush=True)
        return

    def to_dev16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    run_r4 = args.only in ("all", "r4")
    run_kv = args.only in ("all", "kv")
    run_gemm = args.only in ("all", "gemm")

    # ---- inputs: one seeded set from workloads.py, further sets are row rotations of it
    sets = {}
    if run_r4:
        xb, _ = workloads.gen_ffn(seed=0)
        x0 = to_dev16(xb)
        del xb
        sets["r4_x"] = [x0] + [torch.roll(x0, shifts=97 * i, dims=0).contiguous() for i in range(1, NSETS)]
        sets["r4_codes"] = [torch.empty((R4_TOKENS, R4_N // 2), dtype=torch.uint8, device=dev) for _ in range(NSETS)]
        sets["r4_scales"] = [torch.empty((R4_TOKENS,), dtype=torch.float16, device=dev) for _ in range(NSETS)]
    if run_kv:
        qb, kb, _ = workloads.gen_kv(seed=0)
        q0, k0 = to_dev16(qb), to_dev16(kb)
        del qb, kb
        sets["kv_q"] = [q0] + [torch.roll(q0, shifts=31 * i, dims=2).contiguous() for i in range(1, NSETS)]
        sets["kv_k"] = [k0] + [torch.roll(k0, shifts=31 * i, dims=2).contiguous() for i in range(1, NSETS)]
        B, H, S, D = KV_SHAPE
        sets["kv_out"] = [
            {
                "q_codes": torch.empty((B, H, S, D // 2), dtype=torch.uint8, device=dev),
                "q_scales": torch.empty((B, H, S), dtype=torch.float16, device=dev),
                "k_codes": torch.empty((B, H, S, D // 2), dtype=torch.uint8, device=dev),
                "k_scales": torch.empty((B, H, S), dtype=torch.float16, device=dev),
            }
            for _ in range(NSETS)
        ]
    gemm_ok = False
    if run_gemm:
        ab, w, _ = workloads.gen_gemm_inputs(seed=0)
        a0 = to_dev16(ab)
        w0 = torch.from_numpy(w).to(dev)
        del ab, w
        qa, sa = rbq.hadamard_quant_int4(a0)                     # activations, online rotation
        qw, sw = rbq.hadamard_quant_int4(w0)                     # weights, offline rotation
        qa8, sa8 = rbq.hadamard_quant_int8(a0)                   # W4A8: INT8 activation codes
        # operand sets: row rotations of the codes and scales (a set's 121 MB of operands and
        # output is not reused before three other sets have passed through the cache)
        sets["gemm"] = [(qa, sa, qw, sw, torch.empty((GEMM_M, GEMM_N), dtype=torch.bfloat16, device=dev))]
        for i in range(1, NSETS):
            sets["gemm"].append((torch.roll(qa, 61 * i, 0).contiguous(), torch.roll(sa, 61 * i, 0).contiguous(),
                                 torch.roll(qw, 173 * i, 0).contiguous(), torch.roll(sw, 173 * i, 0).contiguous(),
                                 torch.empty((GEMM_M, GEMM_N), dtype=torch.bfloat16, device=dev)))
        out = sets["gemm"][0][4]
        try:
            rbq.w4a4_gemm(qa, sa, qw, sw, out=out)
            gemm_ok = True
        except rbq.RBQError as e:
            if e.status != rbq.RBQ_ENOTSUP:
                raise
        del a0, w0
    torch.cuda.synchronize()

    def call_kv(s):
        rbq.kv_rotate_quant(sets["kv_q"][s], sets["kv_k"][s], **sets["kv_out"][s])

    def call_r4(s):
        rbq.hadamard_quant_int4(sets["r4_x"][s], codes=sets["r4_codes"][s], scales=sets["r4_scales"][s])

    def call_gemm(s):
        a, sa_, w_, sw_, o = sets["gemm"][s]
        rbq.w4a4_gemm(a, sa_, w_, sw_, out=o)

    kernels_in_step = []
    if run_kv:
        kernels_in_step.append(("kv_rotate_quant", call_kv))
    if run_r4:
        kernels_in_step.append(("hadamard_quant_int4", call_r4))
    if run_gemm and gemm_ok:
        kernels_in_step.append(("w4a4_gemm", call_gemm))

    def step(i):
        s = i % NSETS
        for _, fn in kernels_in_step:
            fn(s)

    # ---- pre-warm (time-based, untimed), then the --warmup steps
    t0 = time.perf_counter()
    pre = 0
    while True:
        step(pre)
        pre += 1
        if pre % 4 == 0:
            torch.cuda.synchronize()
            if (time.perf_counter() - t0) * 1e3 >= args.prewarm_ms:
                break
    prewarm_ms = (time.perf_counter() - t0) * 1e3
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- the timed region: exactly --steps steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = e0.elapsed_time(e1) / args.steps

    # ---- per-kernel durations: each kernel alone, back to back over the rotated sets
    avg = {}
    for name, fn in kernels_in_step:
        avg[name] = time_back_to_back(torch, [lambda s=s, fn=fn: fn(s) for s in range(NSETS)], args.steps)

    kernels = {}
    fwht_hash = kernel_source_hash(FWHT_SOURCES)
    gemm_hash = kernel_source_hash(GEMM_SOURCES)
    if "hadamard_quant_int4" in avg:
        t = avg["hadamard_quant_int4"] * 1e-6
        kernels["hadamard_quant_int4"] = {
            "workload": "R4 bf16 [8192, 16384], n=16384, packed INT4 + fp16 scales",
            "avg_us": round(t * 1e6, 3), "algorithmic_bytes": R4_BYTES, "GB_s": round(R4_BYTES / t / 1e9, 2),
            "frac_hbm_peak": round(R4_BYTES / t / 1e9 / HBM_PEAK_GBS, 4),
        }
    if "kv_rotate_quant" in avg:
        t = avg["kv_rotate_quant"] * 1e-6
        kernels["kv_rotate_quant"] = {
            "workload": "R3 bf16 Q and K [16, 32, 2048, 128], packed INT4 + fp16 scales",
            "avg_us": round(t * 1e6, 3), "algorithmic_bytes": KV_BYTES, "GB_s": round(KV_BYTES / t / 1e9, 2),
            "frac_hbm_peak": round(KV_BYTES / t / 1e9 / HBM_PEAK_GBS, 4),
        }
    if "w4a4_gemm" in avg:
        t = avg["w4a4_gemm"] * 1e-6
        kernels["w4a4_gemm"] = {
            "workload": "A [4096, 4096] x W [11008, 4096] packed INT4, bf16 out",
            "avg_us": round(t * 1e6, 3), "algorithmic_ops": GEMM_OPS, "algorithmic_bytes": GEMM_BYTES,
            "TOPS": round(GEMM_OPS / t / 1e12, 2),
            "frac_int8_mfma_peak": round(GEMM_OPS / t / 1e12 / INT8_PEAK_TOPS, 4),
        }

    headline = kernels.get("hadamard_quant_int4")
    value = headline["GB_s"] if headline else None
    roofline = None
    if headline:
        roofline = {
            "kernel": "hadamard_quant_int4 (fwht_quant_kernel<14, bf16>)",
            "bound": "hbm", "achieved": headline["GB_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": headline["frac_hbm_peak"],
            "traffic": load_traffic("hadamard_quant_int4", fwht_hash),
        }
        c = load_counters("hadamard_quant_int4", fwht_hash)
        if c and "valu" in c:
            # from the committed rocprofv3 pass: VALU instructions per element, and VALU
            # issue cycles (4 per wave instruction) over the GPU's active cycles
            roofline["valu_counters"] = c["valu"]
    extra_roofline = {}
    if "kv_rotate_quant" in kernels:
        k = kernels["kv_rotate_quant"]
        extra_roofline["kv_rotate_quant"] = {
            "bound": "hbm", "achieved": k["GB_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": k["frac_hbm_peak"], "traffic": load_traffic("kv_rotate_quant", fwht_hash)}
        c = load_counters("kv_rotate_quant", fwht_hash)
        if c and "valu" in c:
            extra_roofline["kv_rotate_quant"]["valu_counters"] = c["valu"]
    if "w4a4_gemm" in kernels:
        k = kernels["w4a4_gemm"]
        entry = {"bound": "mfma", "achieved": k["TOPS"], "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                 "frac": k["frac_int8_mfma_peak"], "traffic": load_traffic("w4a4_gemm", gemm_hash)}
        c = load_counters("w4a4_gemm", gemm_hash)
        if c and "mfma" in c:
            # from the committed rocprofv3 pass: MFMA busy cycles over the GPU's active
            # cycles, and int8 MFMA operations per dispatch against the algorithmic count
            entry["mfma_counters"] = c["mfma"]
        extra_roofline["w4a4_gemm"] = entry

    extras = {}
    if not args.no_extras and args.only == "all":
        extras["hbm_probe"] = hbm_probe_rates(torch, rbq, dev)
        extras.update(report_small_workloads(torch, rbq, workloads, dev))
    if run_gemm and gemm_ok and not args.no_extras:
        # the W4A8 variant on the same workload (INT8 activation codes, INT4 weights)
        out8 = torch.empty_like(out)
        sets8 = [(torch.roll(qa8, 61 * i, 0).contiguous(), torch.roll(sa8, 61 * i, 0).contiguous()) for i in range(NSETS)]
        fns = [lambda i=i: rbq.w4a8_gemm(sets8[i][0], sets8[i][1], sets["gemm"][i][2], sets["gemm"][i][3], out=out8)
               for i in range(NSETS)]
        for f in fns:
            f()
        t = time_back_to_back(torch, fns, 20) * 1e-6
        extras["w4a8_gemm"] = {
            "workload": "A INT8 [4096, 4096] x W packed INT4 [11008, 4096], bf16 out",
            "avg_us": round(t * 1e6, 3), "TOPS": round(GEMM_OPS / t / 1e12, 2),
            "frac_int8_mfma_peak": round(GEMM_OPS / t / 1e12 / INT8_PEAK_TOPS, 4)}
        # decode: 16 tokens against the same weights (the four rotated weight sets, so the
        # 22.5 MB of codes come from HBM), the few-token kernel; bound by the weight bytes
        dec = {}
        for name, call, a16, s16 in (("w4a4", rbq.w4a4_gemm, qa[:16].contiguous(), sa[:16].contiguous()),
                                     ("w4a8", rbq.w4a8_gemm, qa8[:16].contiguous(), sa8[:16].contiguous())):
            o16 = torch.empty((16, GEMM_N), dtype=torch.bfloat16, device=dev)
            fns = [lambda i=i, call=call, a16=a16, s16=s16, o16=o16: call(a16, s16, sets["gemm"][i][2], sets["gemm"][i][3],
                                                                        out=o16) for i in range(NSETS)]
            fns[0]()
            td = time_back_to_back(torch, fns, 40) * 1e-6
            wbytes = GEMM_N * GEMM_K // 2 + 2 * GEMM_N + 16 * (GEMM_K // (2 if name == "w4a4" else 1)) + 16 * GEMM_N * 2
            dec[name] = {"avg_us": round(td * 1e6, 3), "GB_s": round(wbytes / td / 1e9, 2),
                         "frac_hbm_peak": round(wbytes / td / 1e9 / HBM_PEAK_GBS, 4)}
        extras["gemm_decode_16_tokens"] = {
            "workload": "16 tokens x W packed INT4 [11008, 4096] (A INT4 or INT8), bf16 out, one launch",
            **dec}
        del sets8
        # group-wise weight scales (groups of 256 codes along K) on the same shape: the
        # rotated weights quantized per group, the INT8 activation codes as above
        wr = torch.empty((GEMM_N, GEMM_K), dtype=torch.float32, device=dev)
        wgt = torch.from_numpy(workloads.gen_gemm_inputs(seed=0)[1]).to(dev)
        rbq.hadamard_quant_int4(wgt, rotated=wr)
        del wgt
        qwg, swg = rbq.quantize_groups_int4(wr, 256)
        qwg32, swg32 = rbq.quantize_groups_int4(wr, 32)  # the other group size of the ExecuTorch export
        outg = torch.empty_like(out)
        a16, s16 = qa8[:16].contiguous(), sa8[:16].contiguous()
        outg16 = torch.empty((16, GEMM_N), dtype=torch.bfloat16, device=dev)
        for name, fn in (("quantize_groups_int4", lambda: rbq.quantize_groups_int4(wr, 256, codes=qwg, scales=swg)),
                         ("w4a8_gemm_grouped", lambda: rbq.w4a8_gemm_grouped(qa8, sa8, qwg, swg, 256, out=outg)),
                         ("w4a8_gemm_grouped_32", lambda: rbq.w4a8_gemm_grouped(qa8, sa8, qwg32, swg32, 32, out=outg)),
                         ("w4a8_gemm_grouped_16_tokens",
                          lambda: rbq.w4a8_gemm_grouped(a16, s16, qwg, swg, 256, out=outg16))):
            fn()
            t = time_back_to_back(torch, [fn], 20) * 1e-6
            if name == "w4a8_gemm_grouped_16_tokens":
                wbytes = GEMM_N * GEMM_K // 2 + GEMM_N * (GEMM_K // 256) * 2 + 16 * GEMM_K + 16 * GEMM_N * 2
                extras[name] = {"workload": "16 tokens INT8 x W packed INT4 [11008, 4096], weight scales per 256 "
                                            "codes, bf16 out (one weight set), the few-token kernel",
                                "avg_us": round(t * 1e6, 3), "GB_s": round(wbytes / t / 1e9, 2)}
            elif name.startswith("w4a8_gemm_grouped"):
                gsz = 32 if name.endswith("_32") else 256
                extras[name] = {"workload": "A INT8 [4096, 4096] x W packed INT4 [11008, 4096], weight scales per "
                                            f"{gsz} codes, bf16 out (one operand set)",
                                "avg_us": round(t * 1e6, 3), "TOPS": round(GEMM_OPS / t / 1e12, 2),
                                "frac_int8_mfma_peak": round(GEMM_OPS / t / 1e12 / INT8_PEAK_TOPS, 4)}
            else:
                nbytes = GEMM_N * GEMM_K * 4 + GEMM_N * GEMM_K // 2 + GEMM_N * (GEMM_K // 256) * 2
                extras[name] = {"workload": "rotated fp32 weights [11008, 4096] -> packed INT4, fp16 scales per 256",
                                "avg_us": round(t * 1e6, 3), "GB_s": round(nbytes / t / 1e9, 2)}
        del wr, qwg, swg, qwg32, swg32, outg, a16, s16, outg16
        # context only: the vendor library's int8 GEMM (torch._int_mm, hipBLASLt) on the same
        # shape with the codes already unpacked to int8 and a plain int32 result (no scales)
        try:
            a8 = torch.randint(-8, 8, (GEMM_M, GEMM_K), dtype=torch.int8, device=dev)
            w8 = torch.randint(-8, 8, (GEMM_N, GEMM_K), dtype=torch.int8, device=dev)
            c32 = torch._int_mm(a8, w8.t())
            t = time_back_to_back(torch, [lambda: torch._int_mm(a8, w8.t())], 20) * 1e-6
            extras["library_int8_gemm"] = {
                "workload": "torch._int_mm int8 [4096, 4096] x int8 [4096, 11008]^T -> int32 (unpacked codes, "
                            "no epilogue, one operand set)",
                "avg_us": round(t * 1e6, 3), "TOPS": round(GEMM_OPS / t / 1e12, 2),
                "frac_int8_mfma_peak": round(GEMM_OPS / t / 1e12 / INT8_PEAK_TOPS, 4)}
            del a8, w8, c32
        except Exception as e:  # the library call is context, not part of the step
            extras["library_int8_gemm"] = {"error": f"{type(e).__name__}: {e}"[:200]}
    if run_kv and not args.no_extras:
        # RoPE fused ahead of R3 on the same Q/K (read as pre-RoPE values), and the unfused
        # sequence it replaces: the same RoPE in torch (fp32 arithmetic, bf16 result) writing
        # Q and K back to HBM, then kv_rotate_quant
        B, H, S, D = KV_SHAPE
        inv = 10000.0 ** (-torch.arange(D // 2, dtype=torch.float64, device=dev) * 2.0 / D)
        th = torch.outer(torch.arange(S, dtype=torch.float64, device=dev), inv)
        cs, sn = torch.cos(th).float(), torch.sin(th).float()

        def rope_torch(x):
            xf = x.float()
            a, b = xf[..., : D // 2], xf[..., D // 2:]
            return torch.cat([a * cs - b * sn, b * cs + a * sn], dim=-1).to(x.dtype)

        fused = [lambda i=i: rbq.kv_rotate_quant(sets["kv_q"][i], sets["kv_k"][i], rope_cos=cs, rope_sin=sn,
                                                 **sets["kv_out"][i]) for i in range(NSETS)]
        unfused = [lambda i=i: rbq.kv_rotate_quant(rope_torch(sets["kv_q"][i]), rope_torch(sets["kv_k"][i]),
                                                   **sets["kv_out"][i]) for i in range(NSETS)]
        for name, fns in (("rope_r3_fused", fused), ("rope_r3_unfused_torch", unfused)):
            fns[0]()
            t = time_back_to_back(torch, fns, 8) * 1e-6
            extras[name] = {"workload": "pre-RoPE bf16 Q and K [16, 32, 2048, 128] -> RoPE -> R3 -> packed INT4",
                            "avg_us": round(t * 1e6, 3), "GB_s": round(KV_BYTES / t / 1e9, 2)}
    if run_r4 and not args.no_extras:
        # the randomized transform H diag(s) / sqrt(n) on the same workload and buffers
        sg = torch.from_numpy(workloads.gen_signs(0, R4_N)).to(dev).to(torch.bfloat16)
        fns = [lambda i=i: rbq.hadamard_quant_int4(sets["r4_x"][i], codes=sets["r4_codes"][i],
                                                   scales=sets["r4_scales"][i], signs=sg) for i in range(NSETS)]
        for f in fns:
            f()
        t = time_back_to_back(torch, fns, 20) * 1e-6
        extras["randomized_r4"] = {
            "workload": "R4 bf16 [8192, 16384] with a seeded +-1 diagonal (H diag(s) / sqrt(n))",
            "avg_us": round(t * 1e6, 3), "GB_s": round(R4_BYTES / t / 1e9, 2),
            "frac_hbm_peak": round(R4_BYTES / t / 1e9 / HBM_PEAK_GBS, 4)}

    if run_kv and not args.no_extras:
        # decode attention of one query per (batch, head) over the R3 workload's INT4 key
        # cache (the codes kv_rotate_quant just wrote) and an INT4 value cache of the same shape
        B, H, S, D = KV_SHAPE
        o = sets["kv_out"][0]
        kc, ks = o["k_codes"], o["k_scales"]
        vcodes = torch.from_numpy(workloads.gen_packed_codes(31, B * H * S, D)).to(dev).reshape(B, H, S, D // 2)
        vscales = torch.from_numpy(workloads.gen_scales(32, B * H * S, "float16")).to(dev).reshape(B, H, S)
        qdec = sets["kv_q"][0][:, :, -1, :].contiguous()
        aout = torch.empty_like(qdec)
        fn = lambda: rbq.attention_decode_int4kv(qdec, kc, ks, vcodes, vscales, 1.0 / math.sqrt(D), out=aout)  # noqa
        fn()
        t = time_back_to_back(torch, [fn], 20) * 1e-6
        nbytes = 2 * B * H * S * (D // 2 + 2) + 2 * B * H * D * 2
        extras["attention_decode_int4kv"] = {
            "workload": "one query per (batch, head) over INT4 K and V caches [16, 32, 2048, 128], fp16 scales",
            "avg_us": round(t * 1e6, 3), "GB_s": round(nbytes / t / 1e9, 2),
            "frac_hbm_peak": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": load_traffic("attention_decode_int4kv", kernel_source_hash(("common.h", "attention.hip")))}
        # the same attention with each head's 2048 tokens cut into ranges taken by separate
        # workgroups (512 (batch, head) pairs fill only two workgroups per CU); both kernels,
        # split and merge, inside the timed launches
        split_rates = {}
        ws = torch.empty((rbq.attention_split_workspace_bytes(B, H, 16),), dtype=torch.uint8, device=dev)
        for splits in (2, 4, 8, 16):
            fn = lambda sp=splits: rbq.attention_decode_int4kv_split(  # noqa
                qdec, kc, ks, vcodes, vscales, 1.0 / math.sqrt(D), sp, out=aout, workspace=ws)
            fn()
            ts = time_back_to_back(torch, [fn], 20) * 1e-6
            split_rates[splits] = ts
        best = min(split_rates, key=split_rates.get)
        ts = split_rates[best]
        extras["attention_decode_int4kv_split"] = {
            "workload": "as attention_decode_int4kv, each head's tokens in `splits` ranges + a merge kernel",
            "splits": best, "avg_us": round(ts * 1e6, 3), "GB_s": round(nbytes / ts / 1e9, 2),
            "frac_hbm_peak": round(nbytes / ts / 1e9 / HBM_PEAK_GBS, 4),
            "avg_us_by_splits": {str(k): round(v * 1e6, 3) for k, v in split_rates.items()}}
        del vcodes, vscales, aout, ws
        # grouped key/value heads (32 query heads over 8 key/value heads, LLaMA-3 8B's
        # decode shape): each key/value head's cache is read by 4 query heads' workgroups
        GB_, GH, GHkv, GS = 16, 32, 8, 2048
        gk = torch.from_numpy(workloads.gen_packed_codes(37, GB_ * GHkv * GS, D)).to(dev).reshape(GB_, GHkv, GS, D // 2)
        gv = torch.from_numpy(workloads.gen_packed_codes(38, GB_ * GHkv * GS, D)).to(dev).reshape(GB_, GHkv, GS, D // 2)
        gks = torch.from_numpy(workloads.gen_scales(39, GB_ * GHkv * GS, "float16")).to(dev).reshape(GB_, GHkv, GS)
        gvs = torch.from_numpy(workloads.gen_scales(40, GB_ * GHkv * GS, "float16")).to(dev).reshape(GB_, GHkv, GS)
        gq = qdec[:GB_, :GH].contiguous()
        gout = torch.empty_like(gq)
        gbytes = 2 * GB_ * GHkv * GS * (D // 2 + 2) + 2 * GB_ * GH * D * 2
        fn = lambda: rbq.attention_decode_int4kv(gq, gk, gks, gv, gvs, 1.0 / math.sqrt(D), out=gout)  # noqa
        fn()
        tg = time_back_to_back(torch, [fn], 20) * 1e-6
        extras["attention_decode_gqa"] = {
            "workload": "one query per head, 32 query heads over INT4 K and V caches [16, 8, 2048, 128], fp16 scales",
            "avg_us": round(tg * 1e6, 3), "unique_bytes": gbytes, "GB_s": round(gbytes / tg / 1e9, 2),
            "frac_hbm_peak": round(gbytes / tg / 1e9 / HBM_PEAK_GBS, 4)}
        # the same in token ranges: with at least 256 (batch, key/value head, range) triples
        # the library takes the shared-load kernel (one workgroup loads each cached token once
        # for the four query heads of its key/value head); split and merge kernels both timed
        gws = torch.empty((rbq.attention_split_workspace_bytes(GB_, GH, 8),), dtype=torch.uint8, device=dev)
        gq_rates = {}
        for splits in (2, 4, 8):
            fn = lambda sp=splits: rbq.attention_decode_int4kv_split(  # noqa
                gq, gk, gks, gv, gvs, 1.0 / math.sqrt(D), sp, out=gout, workspace=gws)
            fn()
            gq_rates[splits] = time_back_to_back(torch, [fn], 20) * 1e-6
        best = min(gq_rates, key=gq_rates.get)
        tgs = gq_rates[best]
        extras["attention_decode_gqa_split"] = {
            "workload": "as attention_decode_gqa, each key/value head's tokens in `splits` ranges + a merge kernel",
            "splits": best, "avg_us": round(tgs * 1e6, 3), "unique_bytes": gbytes,
            "GB_s": round(gbytes / tgs / 1e9, 2), "frac_hbm_peak": round(gbytes / tgs / 1e9 / HBM_PEAK_GBS, 4),
            "avg_us_by_splits": {str(k): round(v * 1e6, 3) for k, v in gq_rates.items()}}
        del gk, gv, gks, gvs, gq, gout, gws
        # a decode step's cache write: one token per sequence, RoPE -> R3 -> INT4 keys and
        # INT4 values appended at position 2047 of a 4096-row cache (LLaMA-3 8B heads), the
        # query returned RoPE'd and rotated
        DB, DH, DHkv, DCAP, DPOS = 16, 32, 8, 4096, 2047
        dk = torch.randn((DB, DHkv, 1, D), device=dev).to(torch.bfloat16)
        dv = torch.randn((DB, DHkv, 1, D), device=dev).to(torch.bfloat16)
        dq = torch.randn((DB, DH, 1, D), device=dev).to(torch.bfloat16)
        dkc = torch.zeros((DB, DHkv, DCAP, D // 2), dtype=torch.uint8, device=dev)
        dvc = torch.zeros_like(dkc)
        dks = torch.zeros((DB, DHkv, DCAP), dtype=torch.float16, device=dev)
        dvs = torch.zeros_like(dks)
        dqr = torch.empty_like(dq)
        tth = torch.outer(torch.arange(DCAP, dtype=torch.float64, device=dev), inv)
        tcos, tsin = torch.cos(tth).float(), torch.sin(tth).float()
        fn = lambda: rbq.kv_cache_append_int4(dk, dv, dkc, dks, dvc, dvs, DPOS, q=dq, q_rotated=dqr,  # noqa
                                              rope_cos=tcos, rope_sin=tsin)
        fn()
        dev_us, host_us = time_calls(torch, fn, 200)
        ref_kc, ref_q = dkc.clone(), dqr.clone()
        g_us = time_graph(torch, fn)
        extras["kv_cache_append_decode"] = {
            "workload": "decode step: Q [16, 32, 1, 128], K and V [16, 8, 1, 128] bf16 -> RoPE, R3, INT4 into a "
                        "[16, 8, 4096, 64] cache at position 2047",
            "device_us": round(dev_us, 3), "host_us": round(host_us, 3), "graph_us": round(g_us, 3),
            "graph_matches_eager": bool(torch.equal(dkc, ref_kc) and torch.equal(dqr, ref_q))}
        del ref_kc, ref_q
        del dk, dv, dq, dkc, dvc, dks, dvs, dqr, tth, tcos, tsin
        # long-context decode: one sequence of 32768 tokens, 32 heads (the same cache bytes
        # in 32 (batch, head) pairs): unsplit, 32 workgroups for 256 CUs
        LB, LH, LS = 1, 32, 32768
        lk = torch.from_numpy(workloads.gen_packed_codes(33, LB * LH * LS, D)).to(dev).reshape(LB, LH, LS, D // 2)
        lv = torch.from_numpy(workloads.gen_packed_codes(34, LB * LH * LS, D)).to(dev).reshape(LB, LH, LS, D // 2)
        lks = torch.from_numpy(workloads.gen_scales(35, LB * LH * LS, "float16")).to(dev).reshape(LB, LH, LS)
        lvs = torch.from_numpy(workloads.gen_scales(36, LB * LH * LS, "float16")).to(dev).reshape(LB, LH, LS)
        lq = qdec[:LB].contiguous()
        lout = torch.empty_like(lq)
        lbytes = 2 * LB * LH * LS * (D // 2 + 2) + 2 * LB * LH * D * 2
        fn = lambda: rbq.attention_decode_int4kv(lq, lk, lks, lv, lvs, 1.0 / math.sqrt(D), out=lout)  # noqa
        fn()
        t_one = time_back_to_back(torch, [fn], 20) * 1e-6
        ws = torch.empty((rbq.attention_split_workspace_bytes(LB, LH, 256),), dtype=torch.uint8, device=dev)
        long_rates = {}
        for splits in (16, 32, 64, 128, 256):
            fn = lambda sp=splits: rbq.attention_decode_int4kv_split(  # noqa
                lq, lk, lks, lv, lvs, 1.0 / math.sqrt(D), sp, out=lout, workspace=ws)
            fn()
            long_rates[splits] = time_back_to_back(torch, [fn], 20) * 1e-6
        best = min(long_rates, key=long_rates.get)
        extras["attention_decode_long_context"] = {
            "workload": "one query per head over INT4 K and V caches [1, 32, 32768, 128], fp16 scales",
            "unsplit_avg_us": round(t_one * 1e6, 3), "unsplit_GB_s": round(lbytes / t_one / 1e9, 2),
            "split_splits": best, "split_avg_us": round(long_rates[best] * 1e6, 3),
            "split_GB_s": round(lbytes / long_rates[best] / 1e9, 2),
            "split_frac_hbm_peak": round(lbytes / long_rates[best] / 1e9 / HBM_PEAK_GBS, 4),
            "split_avg_us_by_splits": {str(k): round(v * 1e6, 3) for k, v in long_rates.items()}}
        del lk, lv, lks, lvs, lq, lout, ws
    if args.only == "kron" or (args.only == "all" and not args.no_extras):
        # a row length that is not a power of two: the down-projection input of width
        # 14336 = 28 * 512 (Paley factor of the second kind, q = 13), R4's recipe
        kb, _ = workloads.gen_ffn(seed=0, n=KRON_N)
        k0 = to_dev16(kb)
        del kb
        kx = [k0] + [torch.roll(k0, shifts=97 * i, dims=0).contiguous() for i in range(1, NSETS)]
        kc = [torch.empty((R4_TOKENS, KRON_N // 2), dtype=torch.uint8, device=dev) for _ in range(NSETS)]
        ks = [torch.empty((R4_TOKENS,), dtype=torch.float16, device=dev) for _ in range(NSETS)]
        fns = [lambda i=i: rbq.hadamard_kron_quant_int4(kx[i], codes=kc[i], scales=ks[i]) for i in range(NSETS)]
        for f in fns:
            f()
        t = time_back_to_back(torch, fns, max(args.steps, 8)) * 1e-6
        extras["kron_r4_14336"] = {
            "workload": "R4 bf16 [8192, 14336] = (H_28 (x) H_512) / sqrt(n), packed INT4 + fp16 scales",
            "avg_us": round(t * 1e6, 3), "GB_s": round(KRON_BYTES / t / 1e9, 2),
            "frac_hbm_peak": round(KRON_BYTES / t / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": load_traffic("hadamard_kron_quant_int4", kernel_source_hash(KRON_SOURCES))}
        del kx, kc, ks, k0
        # the GEMM workload's FFN width 11008 = 172 * 64 (the Goethals-Seidel factor)
        n2 = 11008
        kb, _ = workloads.gen_ffn(seed=0, n=n2)
        k0 = to_dev16(kb)
        del kb
        kx = [k0] + [torch.roll(k0, shifts=97 * i, dims=0).contiguous() for i in range(1, NSETS)]
        kc = [torch.empty((R4_TOKENS, n2 // 2), dtype=torch.uint8, device=dev) for _ in range(NSETS)]
        ks = [torch.empty((R4_TOKENS,), dtype=torch.float16, device=dev) for _ in range(NSETS)]
        fns = [lambda i=i: rbq.hadamard_kron_quant_int4(kx[i], codes=kc[i], scales=ks[i]) for i in range(NSETS)]
        for f in fns:
            f()
        t = time_back_to_back(torch, fns, max(args.steps, 8)) * 1e-6
        nbytes = 8192 * n2 * 2 + 8192 * n2 // 2 + 8192 * 2
        extras["kron_r4_11008"] = {
            "workload": "bf16 [8192, 11008] = (H_172 (x) H_64) / sqrt(n), Goethals-Seidel H_172, packed INT4 + fp16 scales",
            "avg_us": round(t * 1e6, 3), "GB_s": round(nbytes / t / 1e9, 2),
            "frac_hbm_peak": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": load_traffic("hadamard_kron_quant_int4_11008", kernel_source_hash(KRON_SOURCES))}
        del kx, kc, ks, k0

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline()

    line = {
        "metric": "Hadamard+INT4 quant GB/s & %HBM peak at n=16384; W4A4 GEMM TOPS & %MFMA",
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm_ms": round(prewarm_ms, 1),
        "prewarm_steps": pre,
        "ms_per_step": round(step_ms, 4),
        "wall_ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in / fp32 transform / int4 codes; int8 MFMA int32 accumulate",
        "data": "synthetic (seeded, workloads.py)",
        "config": {
            "workload": "R4 down_proj input bf16 [8192, 16384] (n=16384) fused Hadamard + INT4 quant; "
                        "step also runs R3 Q/K [16,32,2048,128] and the W4A4 GEMM 4096x11008x4096",
            "tokens": R4_TOKENS, "n": R4_N, "input_sets_rotated": NSETS,
        },
        "timing": "ms_per_step: events around the timed steps; kernels: events around --steps "
                  "back-to-back launches of one kernel over the rotated sets",
        "gemm": kernels.get("w4a4_gemm"),
        "kernels": kernels,
        "roofline": roofline,
        "roofline_other": extra_roofline,
        "cpu_baseline": cpu,
    }
    line.update(extras)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
