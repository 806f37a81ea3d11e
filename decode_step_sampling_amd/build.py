"""Build libdss.so in-tree with hipcc for gfx950.

    python -m decode_step_sampling_amd.build

Every HIP source under ``csrc/`` is compiled for ``--offload-arch=gfx950``
and linked into ``decode_step_sampling_amd/libdss.so``.  hipcc cross-compiles
without a GPU, so this runs on any machine with ROCm installed.
"""

import glob
import os
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libdss.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    f"--offload-arch={ARCH}",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Werror", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd[:3])} ...")
    return res


STAMPS_LIB_PATH = os.path.join(PKG_DIR, "libdss_stamps.so")


def build(verbose=False, jobs=8, stamps=False):
    """Compile every source and link libdss.so (always rebuilds).

    stamps=True builds the measurement variant libdss_stamps.so instead: the
    same sources with DSS_PHASE_STAMPS defined, whose split-row sampling
    kernel writes phase clock stamps (read by ``bench.py --phase-stamps``)."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    tmp = tempfile.mkdtemp(prefix="dss_build_")
    try:
        procs, objs = [], []
        for src in sources():
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            objs.append(obj)
            cmd = [HIPCC, *COMMON_FLAGS, *(["-DDSS_PHASE_STAMPS"] if stamps else []), "-c", src,
                   "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.PIPE, text=True)))
            if len(procs) >= jobs:
                _wait(procs.pop(0))
        while procs:
            _wait(procs.pop(0))
        target = STAMPS_LIB_PATH if stamps else LIB_PATH
        out_tmp = target + ".tmp"
        _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", out_tmp],
             verbose)
        os.replace(out_tmp, target)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return target


def _wait(item):
    cmd, proc = item
    out, err = proc.communicate()
    if proc.returncode != 0:
        sys.stderr.write(out + err)
        raise RuntimeError(f"hipcc failed ({proc.returncode}) on {cmd[-3]}")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, stamps="--stamps" in sys.argv))
