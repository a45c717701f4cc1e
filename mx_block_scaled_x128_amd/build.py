"""Build libmxfp8.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

The sources compile to objects in parallel (the GEMM once per pair of operand
formats, plus its host dispatch), which hipcc then links into the library.

Usage: python -m mx_block_scaled_x128_amd.build   (always recompiles)
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmxfp8.so")
ARCH = "gfx950"
# (source, extra flags, object name)
UNITS = [("api.cpp", [], "api"), ("quant.hip", [], "quant"), ("gaussws.hip", [], "gaussws"),
         ("gemm.hip", ["-DMXFP8_GEMM_FMT=-1"], "gemm_dispatch")] + \
        [("gemm.hip", ["-DMXFP8_GEMM_FMT=%d" % k], "gemm_fmt%d" % k) for k in range(4)]

FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-command-line-argument",
    # keep packed-fp32 instructions out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the GPU feature flag; that warning is harmless
    err = "\n".join(l for l in proc.stderr.splitlines() if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed: %s\n%s" % (" ".join(cmd), err))
    return err


def build(verbose=False, jobs=None):
    cc = hipcc()
    tmpdir = tempfile.mkdtemp(prefix="mxfp8_build_")
    try:
        cmds = [[cc] + FLAGS + extra + ["-c", os.path.join(CSRC, src), "-o", os.path.join(tmpdir, name + ".o")]
                for src, extra, name in UNITS]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        jobs = jobs or min(len(cmds), max(1, os.cpu_count() or 1))
        with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as pool:
            errs = list(pool.map(_run, cmds))
        tmp = LIB + ".tmp"
        link = [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + \
               [os.path.join(tmpdir, name + ".o") for _, _, name in UNITS] + ["-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        errs.append(_run(link))
        if verbose:
            for e in errs:
                if e.strip():
                    print(e, file=sys.stderr)
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
