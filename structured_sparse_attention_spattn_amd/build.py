"""Build the HIP library libspattn.so in-tree for gfx950.

Each .hip source under csrc/ is compiled to an object in parallel, then the
objects are linked into one shared library next to this file.  Packed-fp32
instruction selection is switched off for device code.
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libspattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-Wno-unused-command-line-argument",
    "-I", os.path.join(HERE, "..", "include"),
]


def build(verbose=False, extra_flags=(), build_dir=None, lib_path=None):
    """Compile every csrc/*.hip to an object and link libspattn.so (or
    ``lib_path``), objects under ``build_dir``."""
    BUILD_DIR = build_dir or globals()["BUILD_DIR"]
    LIB = lib_path or globals()["LIB"]
    os.makedirs(BUILD_DIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    procs = []
    objs = []
    for src in sources:
        obj = os.path.join(BUILD_DIR, os.path.basename(src).replace(".hip", ".o"))
        objs.append(obj)
        cmd = [HIPCC, *COMMON_FLAGS, *extra_flags, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, pr in procs:
        out, _ = pr.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the device-only feature flag
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
        if pr.returncode != 0:
            failed.append(src)
            print("\n".join(lines), file=sys.stderr)
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError(f"hipcc failed for: {', '.join(os.path.basename(f) for f in failed)}")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        print(r.stdout.decode(errors="replace"), file=sys.stderr)
        raise RuntimeError("link of libspattn.so failed")
    os.replace(tmp, LIB)
    return LIB


PROBE_SRC = os.path.join(HERE, "probe", "probe.hip")
PROBE_LIB = os.path.join(HERE, "libspattn_probe.so")


def build_probe(verbose=False):
    """The microbenchmark library libspattn_probe.so (measured MFMA and HBM
    denominators for the benchmark), one source, one hipcc call."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, *COMMON_FLAGS, "-shared", PROBE_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        print(r.stdout.decode(errors="replace"), file=sys.stderr)
        raise RuntimeError("build of libspattn_probe.so failed")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_probe(verbose="-v" in sys.argv))
