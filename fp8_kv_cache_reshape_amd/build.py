"""Build libfp8kv.so (HIP for gfx950) in-tree with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

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


def _compile(srcs, out, includes, verbose):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *HIP_FLAGS, *[a for inc in includes for a in ("-I", inc)], *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building " + os.path.basename(out))
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libfp8kv.so, and the benchmark's read-ceiling probe into
    libfp8kv_probe.so.  Always recompiles."""
    _compile(sources(), LIB, [os.path.join(ROOT, "include"), os.path.join(HERE, "csrc")], verbose)
    _compile([os.path.join(HERE, "probe", "read_ceiling.hip")], PROBE_LIB, [], verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
