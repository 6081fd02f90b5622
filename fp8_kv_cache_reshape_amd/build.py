"""Build libfp8kv.so (HIP for gfx950) in-tree with hipcc."""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libfp8kv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops keeps the compiler from emitting packed f32 VALU forms.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function"]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


PROBE_LIB = os.path.join(HERE, "libfp8kv_probe.so")


def _run(cmd, verbose, what):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building " + what)


def _compile(srcs, out, includes, verbose):
    """Compile each source to an object in parallel (they are independent translation
    units), then link the shared library; the result replaces `out` atomically."""
    inc = [a for d in includes for a in ("-I", d)]
    tmpdir = tempfile.mkdtemp(prefix="fp8kv_build_")
    try:
        objs = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in srcs]
        flags = [f for f in HIP_FLAGS if f != "-shared"]
        jobs = [([HIPCC, *flags, *inc, "-c", src, "-o", obj], os.path.basename(src))
                for src, obj in zip(srcs, objs)]
        workers = max(1, min(len(jobs), os.cpu_count() or 1, 8))
        with concurrent.futures.ThreadPoolExecutor(workers) as pool:
            for f in [pool.submit(_run, cmd, verbose, what) for cmd, what in jobs]:
                f.result()
        tmp = out + ".tmp%d" % os.getpid()
        _run([HIPCC, *HIP_FLAGS, *objs, "-o", tmp], verbose, os.path.basename(out))
        os.replace(tmp, out)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libfp8kv.so, and the benchmark's read-ceiling probe into
    libfp8kv_probe.so.  Always recompiles."""
    _compile(sources(), LIB, [os.path.join(ROOT, "include"), os.path.join(HERE, "csrc")], verbose)
    _compile([os.path.join(HERE, "probe", "read_ceiling.hip")], PROBE_LIB, [], verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
