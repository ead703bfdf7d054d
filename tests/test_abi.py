"""C-ABI contract tests that need no GPU.

The library loads on a host without a GPU, exports every function include/w4a16.h
declares, and rejects every invalid argument on the host, before any HIP call,
with the documented status.  Pointers below are fake (never dereferenced): each
case is rejected before anything is launched.
"""
import ctypes
import os
import re
import subprocess

import pytest

import int4_weight_only_02_amd as w4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(7)

A = ctypes.c_void_p(0x10000)       # aligned, never dereferenced
A2 = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10008)     # 8-byte aligned only
NUL = None


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(w4.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return w4.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a16_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("w4a16_pack", "w4a16_linear", "w4a16_lmhead_verify", "w4a16_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", w4.LIB_PATH], stdout=subprocess.PIPE,
                         text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)
    assert set(w4.EXPORTED) == set(declared_functions())


def test_version_and_status_strings(lib):
    assert lib.w4a16_abi_version() == 100
    for st in range(7):
        assert w4.status_string(st) and w4.status_string(st) != "unknown status"
    assert w4.status_string(99) == "unknown status"


def test_workspace_bytes_host_only(lib):
    assert w4.w4a16_workspace_bytes(0, 1, 9728, 2560) == 0  # small M owns whole columns: no scratch
    assert w4.w4a16_workspace_bytes(1, 16, 151936, 2560) > 0
    assert w4.w4a16_workspace_bytes(0, 8192, 2560, 9728) >= 8192 * 76 * 4  # group sums
    assert w4.w4a16_workspace_bytes(0, 1, 512, 512, group=64) == 0
    assert w4.w4a16_workspace_bytes(0, 1, 12, 512) == 0      # N % 8
    assert w4.w4a16_workspace_bytes(1, 65, 512, 512) == 0    # lm_head M > 64
    assert w4.w4a16_workspace_bytes(0, 0, 512, 512) == 0     # empty
    assert w4.w4a16_workspace_bytes(7, 1, 512, 512) == 0     # unknown op


def linear(lib, X=A, qw=A, s=A, qz=A, M=1, N=512, K=512, group=128, Y=A2, ydt=0, ws=A, wsb=1 << 30):
    return lib.w4a16_linear(X, qw, s, qz, M, N, K, group, Y, ydt, ws, wsb, None)


def lmhead(lib, X=A, qw=A, s=A, qz=A, M=16, N=512, K=512, group=128, d=A, Y=A2, ydt=0,
           am=A, acc=A, ws=A, wsb=1 << 30):
    return lib.w4a16_lmhead_verify(X, qw, s, qz, M, N, K, group, d, Y, ydt, am, acc, ws, wsb, None)


def test_linear_rejections(lib):
    assert linear(lib, group=64) == ERR_UNSUPPORTED
    assert linear(lib, ydt=2) == ERR_UNSUPPORTED
    assert linear(lib, K=0) == ERR_SHAPE
    assert linear(lib, K=100) == ERR_SHAPE
    assert linear(lib, K=640 + 64) == ERR_SHAPE
    assert linear(lib, N=12) == ERR_SHAPE
    assert linear(lib, M=-1) == ERR_SHAPE
    assert linear(lib, M=1 << 20, N=1 << 12) == ERR_SHAPE     # M*N >= 2^31
    assert linear(lib, X=NUL) == ERR_NULL
    assert linear(lib, qw=NUL) == ERR_NULL
    assert linear(lib, s=NUL) == ERR_NULL
    assert linear(lib, qz=NUL) == ERR_NULL
    assert linear(lib, Y=NUL) == ERR_NULL
    assert linear(lib, X=MIS) == ERR_ALIGN
    assert linear(lib, Y=MIS) == ERR_ALIGN
    assert linear(lib, qz=MIS) == ERR_ALIGN
    # (only shapes that need scratch: a call that passes validation would launch)
    need = w4.w4a16_workspace_bytes(0, 300, 512, 512)
    assert need > 0
    assert linear(lib, M=300, ws=NUL) == ERR_WORKSPACE
    assert linear(lib, M=300, wsb=16) == ERR_WORKSPACE
    assert linear(lib, M=300, wsb=need - 1) == ERR_WORKSPACE


def gated(lib, X=A, qg=A, sg=A, zg=A, qu=A, su=A, zu=A, M=1, N=512, K=512, group=128, Y=A2, ydt=0, ws=A,
          wsb=1 << 30):
    return lib.w4a16_linear_gated(X, qg, sg, zg, qu, su, zu, M, N, K, group, Y, ydt, ws, wsb, None)


def test_static_ws_rejections(lib):
    def call(X=A, qw=A, s=A, qz=A, M=16, N=2560, K=9728, group=128, Y=A2, ydt=0):
        return lib.w4a16_linear_static_ws(X, qw, s, qz, M, N, K, group, Y, ydt, None)
    assert call(group=64) == ERR_UNSUPPORTED
    assert call(ydt=5) == ERR_UNSUPPORTED
    assert call(N=12) == ERR_SHAPE
    assert call(K=100) == ERR_SHAPE
    assert call(M=-1) == ERR_SHAPE
    assert call(M=0) == OK and call(N=0) == OK
    assert call(X=NUL) == ERR_NULL
    assert call(Y=NUL) == ERR_NULL
    assert call(qz=MIS) == ERR_ALIGN
    # more scratch than the library's array (8 MiB) holds: refused on the host
    assert call(M=8192) == ERR_WORKSPACE
    assert call(M=4096, N=9728, K=2560) == ERR_WORKSPACE


def test_gated_rejections(lib):
    assert gated(lib, group=64) == ERR_UNSUPPORTED
    assert gated(lib, ydt=3) == ERR_UNSUPPORTED
    assert gated(lib, N=520) == ERR_SHAPE           # N % 16
    assert gated(lib, K=100) == ERR_SHAPE
    assert gated(lib, M=1 << 18, N=1 << 12) == ERR_SHAPE  # 2 M N >= 2^31
    assert gated(lib, qu=NUL) == ERR_NULL
    assert gated(lib, zg=NUL) == ERR_NULL
    assert gated(lib, su=MIS) == ERR_ALIGN
    need = w4.w4a16_workspace_bytes(w4.OP_LINEAR_GATED, 300, 512, 512)
    assert need >= 2 * 300 * 512 * 4  # both projections' fp32 outputs
    assert gated(lib, M=300, ws=NUL) == ERR_WORKSPACE
    assert gated(lib, M=300, wsb=need - 1) == ERR_WORKSPACE
    assert gated(lib, M=0) == 0 and gated(lib, N=0) == 0
    assert w4.w4a16_workspace_bytes(w4.OP_LINEAR_GATED, 4, 520, 512) == 0  # N % 16


def test_linear_empty_is_a_noop(lib):
    assert linear(lib, M=0, X=NUL, Y=NUL, ws=NUL, wsb=0) == OK
    assert linear(lib, N=0, qw=NUL, s=NUL, qz=NUL, Y=NUL, ws=NUL, wsb=0) == OK


def test_lmhead_rejections(lib):
    assert lmhead(lib, group=256) == ERR_UNSUPPORTED
    assert lmhead(lib, ydt=-1) == ERR_UNSUPPORTED
    assert lmhead(lib, M=0) == ERR_SHAPE
    assert lmhead(lib, M=65) == ERR_SHAPE
    assert lmhead(lib, N=0) == ERR_SHAPE
    assert lmhead(lib, K=64) == ERR_SHAPE
    assert lmhead(lib, d=NUL) == ERR_NULL
    assert lmhead(lib, am=NUL) == ERR_NULL
    assert lmhead(lib, acc=NUL) == ERR_NULL
    assert lmhead(lib, ws=NUL) == ERR_NULL
    assert lmhead(lib, d=MIS) == ERR_ALIGN
    assert lmhead(lib, Y=MIS) == ERR_ALIGN
    assert lmhead(lib, wsb=8) == ERR_WORKSPACE


def batch(lib, probs, count=None, M=4, group=128, ydt=0, ws=None, wsb=0):
    arr = (w4.Problem * max(1, len(probs)))(*probs)
    n = len(probs) if count is None else count
    return lib.w4a16_linear_batch(ctypes.cast(arr, ctypes.c_void_p), n, M, group, ydt, ws, wsb, None)


def test_batch_rejections(lib):
    good = w4.Problem(A.value, A.value, A.value, A.value, A2.value, 512, 512)
    assert batch(lib, [good], group=64) == ERR_UNSUPPORTED
    assert batch(lib, [good], ydt=3) == ERR_UNSUPPORTED
    assert batch(lib, [good], count=-1) == ERR_SHAPE
    assert batch(lib, [good] * 9) == ERR_SHAPE
    assert batch(lib, [good], M=-1) == ERR_SHAPE
    assert lib.w4a16_linear_batch(None, 2, 4, 128, 0, None, 0, None) == ERR_NULL
    assert batch(lib, [good, w4.Problem(A.value, A.value, A.value, A.value, A2.value, 12, 512)]) == ERR_SHAPE
    assert batch(lib, [good, w4.Problem(A.value, A.value, A.value, A.value, A2.value, 512, 500)]) == ERR_SHAPE
    assert batch(lib, [good, w4.Problem(A.value, None, A.value, A.value, A2.value, 512, 512)]) == ERR_NULL
    assert batch(lib, [good, w4.Problem(A.value, A.value, A.value, A.value, MIS.value, 512, 512)]) == ERR_ALIGN
    # large M needs the prefill workspace of the largest entry
    assert batch(lib, [good], M=300) == ERR_WORKSPACE
    # nothing to do: no launch
    assert batch(lib, [], count=0) == OK
    assert batch(lib, [good], M=0) == OK
    assert batch(lib, [w4.Problem(A.value, None, None, None, None, 0, 512)]) == OK


def test_pack_rejections(lib):
    f = lib.w4a16_pack
    assert f(A, A, 512, 512, 64, A, A, None) == ERR_UNSUPPORTED
    assert f(A, A, 12, 512, 128, A, A, None) == ERR_SHAPE
    assert f(A, A, 512, 500, 128, A, A, None) == ERR_SHAPE
    assert f(A, A, 0, 512, 128, NUL, NUL, None) == OK
    assert f(NUL, A, 512, 512, 128, A, A, None) == ERR_NULL
    assert f(A, A, 512, 512, 128, A, NUL, None) == ERR_NULL
    assert f(MIS, A, 512, 512, 128, A, A, None) == ERR_ALIGN


def test_product_path_has_no_oracle_or_fallback():
    pkg = os.path.dirname(w4.__file__)
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "import oracle" not in text and "from oracle" not in text, fn
                assert "oracle.h" not in text, fn
