"""Host code under the address and undefined-behaviour sanitizers (CPU only).

* The oracle (oracle/oracle.c) with a driver that calls every function on small
  inputs in exactly-sized heap buffers (oracle/sanitize_check.c), built by gcc.
* The library's host side: every source compiled with the sanitizers on the host
  pass (the device code as usual), loaded into a child Python with the sanitizer
  runtime preloaded, and run through the host-side contract: the workspace sizes of
  every path (the planners) and every rejection of the ABI tests.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"]


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_oracle_under_sanitizers(tmp_path):
    exe = tmp_path / "sanitize_check"
    src = [os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "oracle", "sanitize_check.c")]
    subprocess.run(["gcc", "-O1", "-g", "-std=c99", "-fopenmp", "-fno-omit-frame-pointer", "-ffp-contract=off"] + SAN
                   + src + ["-lm", "-o", str(exe)], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle sanitize check ok" in r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr


CHILD = r'''
import ctypes, sys
sys.path.insert(0, sys.argv[2])
import int4_weight_only_02_amd as w4
w4.LIB_PATH = sys.argv[1]
lib = w4.lib()
from tests import test_abi as t
for name in dir(t):
    if name.startswith("test_") and name.endswith("_rejections"):
        getattr(t, name)(lib)
t.test_workspace_bytes_host_only(lib)
t.test_linear_empty_is_a_noop(lib)
for op in range(4):
    for M in (1, 2, 5, 16, 17, 64, 65, 300, 8192):
        for N, K in ((8, 128), (136, 384), (1024, 2560), (2560, 9728), (9728, 2560), (151936, 2560), (16, 36864)):
            w4.w4a16_workspace_bytes(op, M, N, K)
print("host sanitize check ok")
'''


def test_host_side_under_sanitizers(tmp_path):
    rt = _asan_runtime()
    if not os.path.exists(HIPCC) or rt is None:
        pytest.skip("hipcc or the clang sanitizer runtime not available")
    csrc = os.path.join(ROOT, "int4_weight_only_02_amd", "csrc")
    lib = tmp_path / "libw4a16_hostsan.so"
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", csrc]
    for f in SAN:
        flags += ["-Xarch_host", f]
    srcs = sorted(glob.glob(os.path.join(csrc, "*.hip")))
    procs = [(s, subprocess.Popen([HIPCC] + flags + ["-c", s, "-o", str(tmp_path / (os.path.basename(s) + ".o"))],
                                  stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)) for s in srcs]
    for s, pr in procs:
        out, _ = pr.communicate()
        assert pr.returncode == 0, s + "\n" + out[-3000:]
    objs = [str(tmp_path / (os.path.basename(s) + ".o")) for s in srcs]
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
            "-Xarch_host", "-fsanitize=undefined"] + objs + ["-o", str(lib)]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, "-c", CHILD, str(lib), ROOT], capture_output=True, text=True, env=env,
                       timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "host sanitize check ok" in r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
