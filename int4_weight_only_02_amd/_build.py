"""Build libw4a16.so (the C-ABI library) from csrc/*.hip with hipcc for gfx950, in-tree."""
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libw4a16.so")
SOURCES = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))
HEADERS = sorted(glob.glob(os.path.join(PKG, "csrc", "*.h"))) + [os.path.join(ROOT, "include", "w4a16.h")]
# measurement aid for bench.py (a plain read of a launch's bytes), a library of its own
BENCH_LIB = os.path.join(PKG, "libw4a16_bench.so")
BENCH_SOURCES = sorted(glob.glob(os.path.join(PKG, "bench", "*.hip")))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-fp32 VALU forms are kept out of the generated code on purpose.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function",
         "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]


def stale():
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(s) > t for s in SOURCES + HEADERS)


def build(force=True, verbose=False):
    """Compile every HIP source into one shared library (always, unless force=False and
    fresh).  The sources compile to objects in parallel under _build/, then link."""
    if not force and not stale():
        return LIB
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in FLAGS if f != "-shared"]
    procs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [HIPCC] + compile_flags + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, obj, pr in procs:
        out, _ = pr.communicate()
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if pr.returncode != 0:
            failed.append(out)
        elif verbose and out.strip():
            print(out, flush=True)
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(failed))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + [o for _, o, _ in procs] + ["-o", tmp]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout)
    os.replace(tmp, LIB)
    tmpb = BENCH_LIB + ".tmp%d" % os.getpid()
    res = subprocess.run([HIPCC] + FLAGS + BENCH_SOURCES + ["-o", tmpb], stdout=subprocess.PIPE,
                         stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (bench aid):\n" + res.stdout)
    os.replace(tmpb, BENCH_LIB)
    return LIB


if __name__ == "__main__":
    build(force=True, verbose=True)
    print("built", LIB)
    sys.exit(0)
