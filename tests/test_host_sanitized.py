"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only,
no GPU needed).

The library is rebuilt with the sanitizers on its host code only (hipcc's
-Xarch_host, one flag each; device code is unchanged) and two host programs
run against it:
* tests/c/abi_host.c, the plain C user of the ABI: band and pattern tables
  over a sweep of sizes, workspace sizing, status strings and the argument
  checks of every entry point (each fails before any launch);
* tests/c/seq_view_host.cpp: the packed-sequence view every kernel indexes
  with stays inside the tensors for malformed offset arrays;
* tests/c/schedule_host.cpp: the workgroup -> work item mapping of the band
  kernels covers every tile exactly once.
A sanitizer report makes the program exit non-zero.
"""
import os
import shlex
import shutil
import subprocess

import pytest

from structured_sparse_attention_spattn_amd import _lib, build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = "/opt/rocm"
# host-side only: each sanitizer flag directly after -Xarch_host
SAN_HOST = shlex.split("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                       "-Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer")

pytestmark = pytest.mark.skipif(not os.path.exists(os.path.join(ROCM, "bin", "hipcc")), reason="no hipcc")


@pytest.fixture(scope="module")
def san_lib(tmp_path_factory):
    d = tmp_path_factory.mktemp("san")
    lib = str(d / "libspattn_san.so")
    build.build(extra_flags=SAN_HOST + ["-g", "-O1"], build_dir=str(d / "obj"), lib_path=lib)
    return lib


def _env():
    return dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
                UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=24")


def test_c_abi_program_under_sanitizers(san_lib, tmp_path):
    from test_c_abi import check_output_lines
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    exe = str(tmp_path / "abi_host_san")
    libdir = os.path.dirname(san_lib)
    cmd = [clang, "-std=c11", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_host.c"), "-o", exe, "-L", libdir, "-l:libspattn_san.so",
           f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{ROCM}/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=_env())
    assert out.returncode == 0, out.stderr[-4000:]
    assert "Sanitizer" not in out.stderr, out.stderr[-4000:]
    check_output_lines(out.stdout, _lib.load())


def test_packed_sequence_view_under_sanitizers(tmp_path):
    exe = str(tmp_path / "seq_view_san")
    cmd = [os.path.join(ROCM, "bin", "hipcc"), "--offload-arch=gfx950", "-std=c++17", "-g", "-O1", *SAN_HOST,
           "-I", os.path.join(ROOT, "structured_sparse_attention_spattn_amd", "csrc"),
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "seq_view_host.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    out = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=_env())
    assert out.returncode == 0 and out.stdout.strip() == "violations 0", (out.stdout, out.stderr[-4000:])


def test_dispatch_order_under_sanitizers(tmp_path):
    """Every (sequence, head, tile) is run by exactly one workgroup under the
    kernels' workgroup -> work item mapping (tests/c/schedule_host.cpp)."""
    exe = str(tmp_path / "schedule_san")
    cmd = [os.path.join(ROCM, "bin", "hipcc"), "--offload-arch=gfx950", "-std=c++17", "-g", "-O1", *SAN_HOST,
           "-I", os.path.join(ROOT, "structured_sparse_attention_spattn_amd", "csrc"),
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "schedule_host.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    out = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=_env())
    assert out.returncode == 0 and out.stdout.strip().endswith("violations 0"), (out.stdout[-2000:], out.stderr[-4000:])
