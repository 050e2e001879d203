"""Builds the HIP libraries for gfx950: libmdlm.so (include/mdlm.h, the loss
path) and libmdlm_probe.so (include/mdlm_probe.h, the achievable-peak
measurement kernels).

Run as ``python -m uniform_noise_diffusion_amd.build``.  The libraries are
built in-tree next to this file.  Always recompiles.
"""

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libmdlm.so")
SOURCES = ["api.hip", "corrupt.hip", "compact.hip", "head_ce.hip", "check.hip", "scale.hip", "corrupt_compact.hip"]
PROBE_LIB_PATH = os.path.join(PKG_DIR, "libmdlm_probe.so")
PROBE_SOURCES = ["probe.hip"]
ARCH = os.environ.get("MDLM_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    f"--offload-arch={ARCH}",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def _compile(sources, out, verbose):
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(line for line in res.stderr.splitlines()
                    if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


def build(verbose=False):
    """Compiles both libraries; returns the loss-path library's path."""
    _compile(PROBE_SOURCES, PROBE_LIB_PATH, verbose)
    return _compile(SOURCES, LIB_PATH, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
