"""Benchmark of the online-rotation hot path on one MI355X.

One step is one pass over every hot-path call, each on its full workload:
  * kv_rotate_quant   -- R3 on post-RoPE Q and K, bf16 [16, 32, 2048, 128] each;
  * hadamard_quant_int4 -- R4 on the down-projection input, bf16 [8192, 16384], n = 16384;
  * w4a4_gemm         -- A [4096, 4096] x W [11008, 4096] packed INT4, bf16 output.
Inputs are seeded synthetic tensors (workloads.py) already resident in HBM; four input
sets (more than the 256 MB last-level cache per call) are rotated so the timed reads come
from HBM. Each launch is bracketed by HIP events on the stream it runs on.

The headline value is the fused Hadamard + INT4 quantizer's throughput at n = 16384 in
algorithmic GB/s (bf16 input read once, packed codes and fp16 scales written once); the
GEMM's TOPS and the per-call times are reported beside it, with the fp64 oracle timed on
a bounded sample on the host cores as a baseline.

usage: python bench.py [--gpus 1] [--steps 50] [--warmup 5]
"""

import argparse
import hashlib
import json
import math
import os
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


def load_traffic(name, src_hash):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they were
    taken on the current kernel source (else None)."""
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
    return e.get("hbm_bytes_per_launch")


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
    return {
        "value": round(sample_bytes / dt / 1e9, 6),
        "unit": "GB/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"{rows} rows of the bf16 [8192, 16384] R4 workload, explicit fp64 Sylvester "
                  f"multiply + quantizer, {reps} repetitions, {dt:.2f} s each",
    }


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
    between kernels); returns (us per call, graph output equals an eager call's)."""
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the worked-example and decode-sweep reports")
    ap.add_argument("--only", choices=["all", "r4", "kv", "gemm", "kron", "copy"], default="all",
                    help="restrict the step (for profiling one kernel); 'copy' runs a plain 1 GiB "
                         "device copy used to calibrate the HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.only == "copy":
        # plain 1 GiB device copy: calibrates the HBM byte counters, and its rate is what a
        # simple read+write stream (torch's own copy kernel) reaches on this device
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
        return

    import rotation_bit_quantization_fwht_amd as rbq
    import workloads

    if not os.path.exists(rbq.library_path()):
        from rotation_bit_quantization_fwht_amd.build import build

        build()
    rbq.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

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
        out = torch.empty((GEMM_M, GEMM_N), dtype=torch.bfloat16, device=dev)
        try:
            rbq.w4a4_gemm(qa, sa, qw, sw, out=out)
            gemm_ok = True
        except rbq.RBQError as e:
            if e.status != rbq.RBQ_ENOTSUP:
                raise
        del a0, w0
    torch.cuda.synchronize()

    def step(i, ev):
        s = i % NSETS
        j = 0
        if run_kv:
            ev[j].record()
            o = sets["kv_out"][s]
            rbq.kv_rotate_quant(sets["kv_q"][s], sets["kv_k"][s], **o)
            j += 1
        if run_r4:
            ev[j].record()
            rbq.hadamard_quant_int4(sets["r4_x"][s], codes=sets["r4_codes"][s], scales=sets["r4_scales"][s])
            j += 1
        if run_gemm and gemm_ok:
            ev[j].record()
            rbq.w4a4_gemm(qa, sa, qw, sw, out=out)
            j += 1
        ev[j].record()

    nk = int(run_kv) + int(run_r4) + int(run_gemm and gemm_ok)
    for i in range(args.warmup):
        step(i, [torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)])
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    names = []
    if run_kv:
        names.append("kv_rotate_quant")
    if run_r4:
        names.append("hadamard_quant_int4")
    if run_gemm and gemm_ok:
        names.append("w4a4_gemm")
    per = {n: [] for n in names}
    for ev in events:
        for j, n in enumerate(names):
            per[n].append(ev[j].elapsed_time(ev[j + 1]))
    step_ms = [ev[0].elapsed_time(ev[-1]) for ev in events]
    avg = {n: float(np.mean(v)) for n, v in per.items()}
    med = {n: float(np.median(v)) for n, v in per.items()}

    kernels = {}
    fwht_hash = kernel_source_hash(FWHT_SOURCES)
    if "hadamard_quant_int4" in avg:
        t = avg["hadamard_quant_int4"] * 1e-3
        kernels["hadamard_quant_int4"] = {
            "workload": "R4 bf16 [8192, 16384], n=16384, packed INT4 + fp16 scales",
            "avg_us": round(t * 1e6, 3), "median_us": round(med["hadamard_quant_int4"] * 1e3, 3),
            "algorithmic_bytes": R4_BYTES, "GB_s": round(R4_BYTES / t / 1e9, 2),
            "frac_hbm_peak": round(R4_BYTES / t / 1e9 / HBM_PEAK_GBS, 4),
        }
    if "kv_rotate_quant" in avg:
        t = avg["kv_rotate_quant"] * 1e-3
        kernels["kv_rotate_quant"] = {
            "workload": "R3 bf16 Q and K [16, 32, 2048, 128], packed INT4 + fp16 scales",
            "avg_us": round(t * 1e6, 3), "median_us": round(med["kv_rotate_quant"] * 1e3, 3),
            "algorithmic_bytes": KV_BYTES, "GB_s": round(KV_BYTES / t / 1e9, 2),
            "frac_hbm_peak": round(KV_BYTES / t / 1e9 / HBM_PEAK_GBS, 4),
        }
    if "w4a4_gemm" in avg:
        t = avg["w4a4_gemm"] * 1e-3
        kernels["w4a4_gemm"] = {
            "workload": "A [4096, 4096] x W [11008, 4096] packed INT4, bf16 out",
            "avg_us": round(t * 1e6, 3), "median_us": round(med["w4a4_gemm"] * 1e3, 3),
            "algorithmic_ops": GEMM_OPS, "TOPS": round(GEMM_OPS / t / 1e12, 2),
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
    extra_roofline = {}
    if "kv_rotate_quant" in kernels:
        k = kernels["kv_rotate_quant"]
        extra_roofline["kv_rotate_quant"] = {
            "bound": "hbm", "achieved": k["GB_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": k["frac_hbm_peak"], "traffic": load_traffic("kv_rotate_quant", fwht_hash)}
    if "w4a4_gemm" in kernels:
        k = kernels["w4a4_gemm"]
        extra_roofline["w4a4_gemm"] = {
            "bound": "mfma", "achieved": k["TOPS"], "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
            "frac": k["frac_int8_mfma_peak"],
            "traffic": load_traffic("w4a4_gemm", kernel_source_hash(GEMM_SOURCES))}

    extras = {}
    if args.only == "all" and not args.no_extras:
        extras = report_small_workloads(torch, rbq, workloads, dev)
    if run_gemm and gemm_ok and not args.no_extras:
        # the W4A8 variant on the same workload (INT8 activation codes, INT4 weights)
        out8 = torch.empty_like(out)
        rbq.w4a8_gemm(qa8, sa8, qw, sw, out=out8)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(20):
            rbq.w4a8_gemm(qa8, sa8, qw, sw, out=out8)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / 20
        extras["w4a8_gemm"] = {
            "workload": "A INT8 [4096, 4096] x W packed INT4 [11008, 4096], bf16 out",
            "avg_us": round(t * 1e6, 3), "TOPS": round(GEMM_OPS / t / 1e12, 2),
            "frac_int8_mfma_peak": round(GEMM_OPS / t / 1e12 / INT8_PEAK_TOPS, 4)}
    if run_gemm and gemm_ok and not args.no_extras:
        # group-wise weight scales (groups of 256 codes along K) on the same shape: the
        # rotated weights quantized per group, the INT8 activation codes as above
        wr = torch.empty((GEMM_N, GEMM_K), dtype=torch.float32, device=dev)
        wgt = torch.from_numpy(workloads.gen_gemm_inputs(seed=0)[1]).to(dev)
        rbq.hadamard_quant_int4(wgt, rotated=wr)
        del wgt
        qwg, swg = rbq.quantize_groups_int4(wr, 256)
        qwg32, swg32 = rbq.quantize_groups_int4(wr, 32)  # the other group size of the ExecuTorch export
        outg = torch.empty_like(out)
        for name, fn in (("quantize_groups_int4", lambda: rbq.quantize_groups_int4(wr, 256, codes=qwg, scales=swg)),
                         ("w4a8_gemm_grouped", lambda: rbq.w4a8_gemm_grouped(qa8, sa8, qwg, swg, 256, out=outg)),
                         ("w4a8_gemm_grouped_32", lambda: rbq.w4a8_gemm_grouped(qa8, sa8, qwg32, swg32, 32, out=outg))):
            fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(20):
                fn()
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3 / 20
            if name.startswith("w4a8_gemm_grouped"):
                gsz = 32 if name.endswith("_32") else 256
                extras[name] = {"workload": "A INT8 [4096, 4096] x W packed INT4 [11008, 4096], weight scales per "
                                            f"{gsz} codes, bf16 out",
                                "avg_us": round(t * 1e6, 3), "TOPS": round(GEMM_OPS / t / 1e12, 2),
                                "frac_int8_mfma_peak": round(GEMM_OPS / t / 1e12 / INT8_PEAK_TOPS, 4)}
            else:
                nbytes = GEMM_N * GEMM_K * 4 + GEMM_N * GEMM_K // 2 + GEMM_N * (GEMM_K // 256) * 2
                extras[name] = {"workload": "rotated fp32 weights [11008, 4096] -> packed INT4, fp16 scales per 256",
                                "avg_us": round(t * 1e6, 3), "GB_s": round(nbytes / t / 1e9, 2)}
        del wr, qwg, swg, qwg32, swg32, outg
        # context only: the vendor library's int8 GEMM (torch._int_mm, hipBLASLt) on the same
        # shape with the codes already unpacked to int8 and a plain int32 result (no scales)
        try:
            a8 = torch.randint(-8, 8, (GEMM_M, GEMM_K), dtype=torch.int8, device=dev)
            w8 = torch.randint(-8, 8, (GEMM_N, GEMM_K), dtype=torch.int8, device=dev)
            c32 = torch._int_mm(a8, w8.t())
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(20):
                c32 = torch._int_mm(a8, w8.t())
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3 / 20
            extras["library_int8_gemm"] = {
                "workload": "torch._int_mm int8 [4096, 4096] x int8 [4096, 11008]^T -> int32 (unpacked codes, no epilogue)",
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
        o = sets["kv_out"][0]

        def rope_torch(x):
            xf = x.float()
            a, b = xf[..., : D // 2], xf[..., D // 2:]
            return torch.cat([a * cs - b * sn, b * cs + a * sn], dim=-1).to(x.dtype)

        def fused(i):
            rbq.kv_rotate_quant(sets["kv_q"][i], sets["kv_k"][i], rope_cos=cs, rope_sin=sn, **o)

        def unfused(i):
            rbq.kv_rotate_quant(rope_torch(sets["kv_q"][i]), rope_torch(sets["kv_k"][i]), **o)

        for name, fn in (("rope_r3_fused", fused), ("rope_r3_unfused_torch", unfused)):
            fn(0)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for r in range(8):
                fn(r % NSETS)
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3 / 8
            extras[name] = {"workload": "pre-RoPE bf16 Q and K [16, 32, 2048, 128] -> RoPE -> R3 -> packed INT4",
                            "avg_us": round(t * 1e6, 3), "GB_s": round(KV_BYTES / t / 1e9, 2)}
    if run_r4 and not args.no_extras:
        # the randomized transform H diag(s) / sqrt(n) on the same workload and buffers
        sg = torch.from_numpy(workloads.gen_signs(0, R4_N)).to(dev).to(torch.bfloat16)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * NSETS + 1)]
        for i in range(NSETS):
            rbq.hadamard_quant_int4(sets["r4_x"][i], codes=sets["r4_codes"][i], scales=sets["r4_scales"][i], signs=sg)
        ts = []
        for rep in range(5):
            for i in range(NSETS):
                ev[2 * i].record()
                rbq.hadamard_quant_int4(sets["r4_x"][i], codes=sets["r4_codes"][i], scales=sets["r4_scales"][i],
                                        signs=sg)
                ev[2 * i + 1].record()
            torch.cuda.synchronize()
            ts += [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(NSETS)]
        t = float(np.mean(ts)) * 1e-3
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
        fn = lambda: rbq.attention_decode_int4kv(qdec, kc, ks, vcodes, vscales, 1.0 / math.sqrt(D), out=aout)
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            fn()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / 20
        nbytes = 2 * B * H * S * (D // 2 + 2) + 2 * B * H * D * 2
        extras["attention_decode_int4kv"] = {
            "workload": "one query per (batch, head) over INT4 K and V caches [16, 32, 2048, 128], fp16 scales",
            "avg_us": round(t * 1e6, 3), "GB_s": round(nbytes / t / 1e9, 2),
            "frac_hbm_peak": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": load_traffic("attention_decode_int4kv", kernel_source_hash(("common.h", "attention.hip")))}
        del vcodes, vscales, aout
    if args.only == "kron" or (args.only == "all" and not args.no_extras):
        # a row length that is not a power of two: the down-projection input of width
        # 14336 = 28 * 512 (Paley factor of the second kind, q = 13), R4's recipe
        kb, _ = workloads.gen_ffn(seed=0, n=KRON_N)
        k0 = to_dev16(kb)
        del kb
        kx = [k0] + [torch.roll(k0, shifts=97 * i, dims=0).contiguous() for i in range(1, NSETS)]
        kc = [torch.empty((R4_TOKENS, KRON_N // 2), dtype=torch.uint8, device=dev) for _ in range(NSETS)]
        ks = [torch.empty((R4_TOKENS,), dtype=torch.float16, device=dev) for _ in range(NSETS)]
        for i in range(NSETS):
            rbq.hadamard_kron_quant_int4(kx[i], codes=kc[i], scales=ks[i])
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * NSETS)]
        ts = []
        for rep in range(max(1, args.steps // NSETS)):
            for i in range(NSETS):
                ev[2 * i].record()
                rbq.hadamard_kron_quant_int4(kx[i], codes=kc[i], scales=ks[i])
                ev[2 * i + 1].record()
            torch.cuda.synchronize()
            ts += [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(NSETS)]
        t = float(np.mean(ts)) * 1e-3
        extras["kron_r4_14336"] = {
            "workload": "R4 bf16 [8192, 14336] = (H_28 (x) H_512) / sqrt(n), packed INT4 + fp16 scales",
            "avg_us": round(t * 1e6, 3), "GB_s": round(KRON_BYTES / t / 1e9, 2),
            "frac_hbm_peak": round(KRON_BYTES / t / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": load_traffic("hadamard_kron_quant_int4", kernel_source_hash(KRON_SOURCES))}
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
        "ms_per_step": round(float(np.mean(step_ms)), 4),
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
