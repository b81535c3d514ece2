"""Build librbq.so (the C-ABI HIP library) in-tree for gfx950 with hipcc.

Every kernel translation unit is compiled in parallel; the fused Hadamard + INT4
quantizer is compiled once per row length n = 2^k (k = 1..15) so each unit stays small.
Usage: ``python -m rotation_bit_quantization_fwht_amd.build`` or ``build()``.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "librbq.so")
ARCH = "gfx950"
KMIN, KMAX = 1, 15

HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 VALU instructions are kept out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build librbq.so")


def _units():
    units = []
    for k in range(KMIN, KMAX + 1):
        # the 32-point factor's MFMA results go straight to VGPRs (no AGPR copies)
        units.append((os.path.join(CSRC, "fwht_kernels.hip"), f"fwht_k{k}.o",
                      [f"-DRBQ_K={k}", "-mllvm", "-amdgpu-mfma-vgpr-form"]))
    units.append((os.path.join(CSRC, "fwht_quant.hip"), "fwht_quant.o", []))
    units.append((os.path.join(CSRC, "kron_quant.hip"), "kron_quant.o", ["-mllvm", "-amdgpu-mfma-vgpr-form"]))
    units.append((os.path.join(CSRC, "w4a4_gemm.hip"), "w4a4_gemm.o", []))
    units.append((os.path.join(CSRC, "group_quant.hip"), "group_quant.o", []))
    units.append((os.path.join(CSRC, "attention.hip"), "attention.o", []))
    units.append((os.path.join(CSRC, "probe.hip"), "probe.o", []))
    units.append((os.path.join(CSRC, "status.cpp"), "status.o", ["-x", "hip"]))
    return units


def _compile(hipcc, src, obj, extra, build_dir):
    cmd = [hipcc] + HIP_FLAGS + extra + ["-c", src, "-o", os.path.join(build_dir, obj)]
    t0 = time.time()
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    noise = "is not a recognized feature for this target"
    log = "\n".join(l for l in p.stdout.splitlines() if noise not in l)
    return p.returncode, obj, time.time() - t0, log, cmd


def build(verbose=False, jobs=None, defines=(), lib_path=None, build_dir=None):
    """Compile every translation unit for gfx950 and link librbq.so. Returns its path.

    defines/lib_path/build_dir build a variant library (tuning experiments) elsewhere.
    """
    hipcc = _hipcc()
    build_dir = build_dir or BUILD
    lib_path = lib_path or LIB
    os.makedirs(build_dir, exist_ok=True)
    jobs = jobs or max(1, min(16, os.cpu_count() or 1))
    units = [(s, o, e + [f"-D{d}" for d in defines]) for (s, o, e) in _units()]
    t0 = time.time()
    failed = []
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_compile, hipcc, s, o, e, build_dir) for (s, o, e) in units]
        for f in concurrent.futures.as_completed(futs):
            rc, obj, dt, log, cmd = f.result()
            if verbose:
                print(f"[build] {obj} {dt:.1f}s", flush=True)
            if log.strip() and (verbose or rc != 0):
                print(log, file=sys.stderr)
            if rc != 0:
                failed.append((obj, " ".join(cmd)))
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(o for o, _ in failed))
    objs = [os.path.join(build_dir, o) for (_, o, _) in units]
    tmp = lib_path + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if p.returncode != 0:
        raise RuntimeError("link failed:\n" + p.stdout)
    os.replace(tmp, lib_path)
    if verbose:
        print(f"[build] {lib_path} in {time.time() - t0:.1f}s", flush=True)
    return lib_path


if __name__ == "__main__":
    build(verbose=True)
