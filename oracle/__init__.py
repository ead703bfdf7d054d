"""fp64 CPU oracle for the W4A16 group-quantized linear and its verify epilogue.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py``, never by the product library.  The C
source (``oracle.c``) shares nothing with the HIP path; this module only marshals
numpy arrays into it.  See ``oracle.c`` for the definitions and the passages of
the source pages (arXiv 2607.04244 and its reviews) they follow.

Functions (numpy in, numpy out):
  pack(codes u8[N,K], zeros u8[N,G])            -> (qweight u32[N,K/8], qzeros u32[N/8,G])
  unpack(qweight, qzeros, N, K)                 -> (codes, zeros)
  linear(X bf16-bits u16[M,K], qweight, scales f16-bits u16[N,G], qzeros) -> Y f64[M,N]
  linear_at(..., rows, cols)                    -> Y[rows[i], cols[i]] f64
  linear_matmul(X, qweight, scales, qzeros)     -> Y f64[M,N] (dequantize in fp64, then a library matmul)
  argmax_accept(Y f64[M,N], draft i32[M])       -> (argmax i32[M], gap f64[M], L int)
  quantize(W bf16-bits u16[N,K], scales f16-bits u16[N,G], zeros u8[N,G]) -> codes u8[N,K]
  linear_gidx(X, qweight, scales, qzeros, g_idx i32[K]) -> Y f64[M,N] (GPTQ act-order groups)
  swa(Q u16[M,Hq,D], K u16[T,Hkv,D], Vt u16[Hkv,D,T], window) -> O f64[M,Hq,D] (sliding-window attention)
  silu_mul(G f64, U f64)                        -> silu(G) * U elementwise (oracle_silu_mul)
  gated(X, gate, up)                            -> silu(X Wg^T) * (X Wu^T) f64[M,N]; gate/up = (qweight, scales, qzeros)
  bf16_to_f64 / f16_to_f64 (bit patterns -> exact values)
"""
import ctypes
import os
import subprocess

import numpy as np

GROUP = 128
_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force=False):
    """Compile oracle.c with gcc (fp64, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-ffp-contract=off", "-fno-fast-math",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path):
    """Open a compiled oracle library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.oracle_pack.argtypes = [P, P, I, I, I, P, P]
    lib.oracle_unpack.argtypes = [P, P, I, I, I, P, P]
    lib.oracle_linear_f64.argtypes = [P, P, P, P, I, I, I, I, P]
    lib.oracle_linear_at.argtypes = [P, P, P, P, I, I, I, I, P, P, I, P]
    lib.oracle_argmax_accept.argtypes = [P, I, I, P, P, P, P]
    lib.oracle_quantize.argtypes = [P, P, P, I, I, I, P]
    lib.oracle_linear_gidx.argtypes = [P, P, P, P, P, I, I, I, I, P]
    lib.oracle_swa.argtypes = [P, P, P, I, I, I, I, I, I, P]
    lib.oracle_swa_block.argtypes = [P, P, P, I, I, I, I, I, I, P]
    lib.oracle_silu_mul.argtypes = [P, P, ctypes.c_longlong, P]
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = ctypes.c_double
    lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f64.restype = ctypes.c_double
    lib.oracle_num_threads.restype = I
    return lib


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = _bind(_LIB)
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def num_threads():
    return int(_load().oracle_num_threads())


def bf16_to_f64(bits):
    return float(_load().oracle_bf16_to_f64(int(bits)))


def f16_to_f64(bits):
    return float(_load().oracle_f16_to_f64(int(bits)))


def pack(codes, zeros, group=GROUP):
    codes, pc = _c(codes, np.uint8)
    zeros, pz = _c(zeros, np.uint8)
    N, K = codes.shape
    G = K // group
    assert zeros.shape == (N, G) and N % 8 == 0 and K % group == 0
    qweight = np.zeros((N, K // 8), np.uint32)
    qzeros = np.zeros((N // 8, G), np.uint32)
    _load().oracle_pack(pc, pz, N, K, group, qweight.ctypes.data_as(ctypes.c_void_p),
                        qzeros.ctypes.data_as(ctypes.c_void_p))
    return qweight, qzeros


def unpack(qweight, qzeros, N, K, group=GROUP):
    qweight, pw = _c(qweight, np.uint32)
    qzeros, pz = _c(qzeros, np.uint32)
    codes = np.zeros((N, K), np.uint8)
    zeros = np.zeros((N, K // group), np.uint8)
    _load().oracle_unpack(pw, pz, N, K, group, codes.ctypes.data_as(ctypes.c_void_p),
                          zeros.ctypes.data_as(ctypes.c_void_p))
    return codes, zeros


def linear(X, qweight, scales, qzeros, group=GROUP):
    X, px = _c(X, np.uint16)
    qweight, pw = _c(qweight, np.uint32)
    scales, ps = _c(scales, np.uint16)
    qzeros, pz = _c(qzeros, np.uint32)
    M, K = X.shape
    N = qweight.shape[0]
    assert qweight.shape == (N, K // 8) and scales.shape == (N, K // group)
    assert qzeros.shape == (N // 8, K // group)
    Y = np.zeros((M, N), np.float64)
    _load().oracle_linear_f64(px, pw, ps, pz, M, N, K, group, Y.ctypes.data_as(ctypes.c_void_p))
    return Y


def dequantize(qweight, qzeros, scales, N, K, group=GROUP):
    """W f64[N,K] = (q - z) * s per group, from the oracle's own unpack and fp16 decode."""
    codes, zeros = unpack(qweight, qzeros, N, K, group)
    s = np.asarray(scales, np.uint16).view(np.float16).astype(np.float64)  # exact widening
    W = codes.astype(np.float64)
    W -= np.repeat(zeros.astype(np.float64), group, axis=1)
    W *= np.repeat(s, group, axis=1)
    return W


def linear_matmul(X, qweight, scales, qzeros, group=GROUP):
    """The same definition as linear(), with the contraction done by a library fp64 matmul.

    Dequantization is exact in fp64; only the summation order differs from the
    naive loop (fp64 rounding, ~1e-13 relative).  Used for the full-size workloads."""
    X = np.ascontiguousarray(X, np.uint16)
    M, K = X.shape
    N = qweight.shape[0]
    W = dequantize(qweight, qzeros, scales, N, K, group)
    x = (X.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x @ W.T


def linear_at(X, qweight, scales, qzeros, rows, cols, group=GROUP):
    X, px = _c(X, np.uint16)
    qweight, pw = _c(qweight, np.uint32)
    scales, ps = _c(scales, np.uint16)
    qzeros, pz = _c(qzeros, np.uint32)
    rows, pr = _c(rows, np.int32)
    cols, pcl = _c(cols, np.int32)
    M, K = X.shape
    N = qweight.shape[0]
    assert rows.shape == cols.shape and rows.ndim == 1
    assert (rows >= 0).all() and (rows < M).all() and (cols >= 0).all() and (cols < N).all()
    out = np.zeros(rows.shape[0], np.float64)
    _load().oracle_linear_at(px, pw, ps, pz, M, N, K, group, pr, pcl, rows.shape[0],
                             out.ctypes.data_as(ctypes.c_void_p))
    return out


def argmax_accept(Y, draft):
    Y, py = _c(Y, np.float64)
    draft, pd = _c(draft, np.int32)
    M, N = Y.shape
    assert draft.shape == (M,)
    am = np.zeros(M, np.int32)
    gap = np.zeros(M, np.float64)
    L = ctypes.c_int32(0)
    _load().oracle_argmax_accept(py, M, N, pd, am.ctypes.data_as(ctypes.c_void_p),
                                 gap.ctypes.data_as(ctypes.c_void_p), ctypes.byref(L))
    return am, gap, int(L.value)


def quantize(W, scales, zeros, group=GROUP):
    """Round W back onto the grid with frozen scales and zeros (oracle_quantize)."""
    W, pw = _c(W, np.uint16)
    scales, ps = _c(scales, np.uint16)
    zeros, pz = _c(zeros, np.uint8)
    N, K = W.shape
    assert K % group == 0 and scales.shape == (N, K // group) and zeros.shape == (N, K // group)
    codes = np.zeros((N, K), np.uint8)
    _load().oracle_quantize(pw, ps, pz, N, K, group, codes.ctypes.data_as(ctypes.c_void_p))
    return codes


def linear_gidx(X, qweight, scales, qzeros, g_idx, group=GROUP):
    """Y = X W^T with column k of W in group g_idx[k] (oracle_linear_gidx)."""
    X, px = _c(X, np.uint16)
    qweight, pw = _c(qweight, np.uint32)
    scales, ps = _c(scales, np.uint16)
    qzeros, pz = _c(qzeros, np.uint32)
    g_idx, pg = _c(g_idx, np.int32)
    M, K = X.shape
    N = qweight.shape[0]
    G = K // group
    assert qweight.shape == (N, K // 8) and scales.shape == (N, G) and qzeros.shape == (N // 8, G)
    assert g_idx.shape == (K,) and (g_idx >= 0).all() and (g_idx < G).all()
    Y = np.zeros((M, N), np.float64)
    _load().oracle_linear_gidx(px, pw, ps, pz, pg, M, N, K, group, Y.ctypes.data_as(ctypes.c_void_p))
    return Y


def swa(Q, K, Vt, window):
    """Causal sliding-window attention of the last M tokens (oracle_swa)."""
    Q, pq = _c(Q, np.uint16)
    K, pk = _c(K, np.uint16)
    Vt, pv = _c(Vt, np.uint16)
    M, Hq, D = Q.shape
    T, Hkv, D2 = K.shape
    assert D2 == D and Vt.shape == (Hkv, D, T) and Hq % Hkv == 0 and M <= T and window >= 1
    O = np.zeros((M, Hq, D), np.float64)
    _load().oracle_swa(pq, pk, pv, M, T, Hq, Hkv, D, window, O.ctypes.data_as(ctypes.c_void_p))
    return O


def swa_block(Q, K, Vt, window):
    """Attention of the last M tokens, bidirectional within that block, the window over
    the context (oracle_swa_block)."""
    Q, pq = _c(Q, np.uint16)
    K, pk = _c(K, np.uint16)
    Vt, pv = _c(Vt, np.uint16)
    M, Hq, D = Q.shape
    T, Hkv, D2 = K.shape
    assert D2 == D and Vt.shape == (Hkv, D, T) and Hq % Hkv == 0 and M <= T and window >= 1
    O = np.zeros((M, Hq, D), np.float64)
    _load().oracle_swa_block(pq, pk, pv, M, T, Hq, Hkv, D, window, O.ctypes.data_as(ctypes.c_void_p))
    return O


def silu_mul(G, U):
    """Y = silu(G) * U elementwise, silu(g) = g / (1 + exp(-g)) (oracle_silu_mul)."""
    G, pg = _c(G, np.float64)
    U, pu = _c(U, np.float64)
    assert G.shape == U.shape
    Y = np.zeros(G.shape, np.float64)
    _load().oracle_silu_mul(pg, pu, G.size, Y.ctypes.data_as(ctypes.c_void_p))
    return Y


def gated(X, gate, up, group=GROUP):
    """The gated MLP activation of two projections of X: silu(X Wg^T) * (X Wu^T)."""
    return silu_mul(linear(X, *gate, group=group), linear(X, *up, group=group))
