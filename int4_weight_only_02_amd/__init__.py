"""MI355X (gfx950) INT4 group-quantized weight-only linear (W4A16) -- Python binding.

A thin ctypes layer over ``libw4a16.so`` (the C ABI in ``include/w4a16.h``).  It
only marshals torch tensors into pointers, sizes and the current HIP stream:
every step of the computation runs in the library's HIP kernels.  PyTorch
supplies device memory and streams.  There is no CPU fallback: if the library is
not built, every call raises.

Calls (same names as the C ABI):
  w4a16_pack(codes u8[N,K], zeros u8[N,G])          -> (qweight i32[N,K/8], qzeros i32[N/8,G])
  w4a16_linear(X bf16[M,K], qweight, scales f16[N,G], qzeros, out_dtype) -> Y[M,N]
  w4a16_lmhead_verify(X, qweight, scales, qzeros, draft i32[M], return_logits) ->
        (argmax i32[M], accept_len i32[1], logits or None)
  w4a16_linear_static_ws(X, qweight, scales, qzeros, out_dtype) -> Y[M,N]
        (w4a16_linear with the library's own scratch array: no workspace argument)
  w4a16_linear_batch([(X, qweight, scales, qzeros), ...], out_dtype) -> [Y, ...]
        (up to 8 projections with the same M in one launch)
  w4a16_workspace_bytes(op, M, N, K)
Packed words travel as int32 tensors (same bits as uint32).
"""
import ctypes
import os

GROUP = 128
OUT_BF16, OUT_F32 = 0, 1
OP_LINEAR, OP_LMHEAD, OP_LINEAR_ACTORDER, OP_LINEAR_GATED = 0, 1, 2, 3

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libw4a16.so")
_lib = None

EXPORTED = ("w4a16_pack", "w4a16_quantize", "w4a16_linear", "w4a16_linear_static_ws", "w4a16_linear_gated",
            "w4a16_linear_batch",
            "w4a16_lmhead_verify",
            "w4a16_actorder_perm", "w4a16_pack_actorder", "w4a16_linear_actorder",
            "w4a16_swa_attention", "w4a16_swa_attention_block", "w4a16_swa_workspace_bytes",
            "w4a16_workspace_bytes", "w4a16_status_string", "w4a16_abi_version")
MAX_BATCH = 8


class Problem(ctypes.Structure):
    """w4a16_problem: the device tensors of one projection of a batch call."""
    _fields_ = [("X", ctypes.c_void_p), ("qweight", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("qzeros", ctypes.c_void_p), ("Y", ctypes.c_void_p), ("N", ctypes.c_int), ("K", ctypes.c_int)]


class W4A16Error(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, status_string(status), status))


def lib():
    """Load libw4a16.so (built in-tree by __graft_entry__.build()); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libw4a16.so is not built (run __graft_entry__.build()); "
                           "there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.w4a16_pack.argtypes = [P, P, I, I, I, P, P, P]
    L.w4a16_pack.restype = I
    L.w4a16_quantize.argtypes = [P, P, P, I, I, I, P, P]
    L.w4a16_quantize.restype = I
    L.w4a16_swa_attention.argtypes = [P, P, P, I, I, I, I, I, I, I, P, I, P, S, P]
    L.w4a16_swa_attention.restype = I
    L.w4a16_swa_attention_block.argtypes = [P, P, P, I, I, I, I, I, I, I, P, I, P, S, P]
    L.w4a16_swa_attention_block.restype = I
    L.w4a16_swa_workspace_bytes.argtypes = [I, I, I, I, I]
    L.w4a16_swa_workspace_bytes.restype = S
    L.w4a16_actorder_perm.argtypes = [P, I, I, P]
    L.w4a16_actorder_perm.restype = I
    L.w4a16_pack_actorder.argtypes = [P, P, P, I, I, I, P, P, P]
    L.w4a16_pack_actorder.restype = I
    L.w4a16_linear_actorder.argtypes = [P, P, P, P, P, I, I, I, I, P, I, P, S, P]
    L.w4a16_linear_actorder.restype = I
    L.w4a16_linear.argtypes = [P, P, P, P, I, I, I, I, P, I, P, S, P]
    L.w4a16_linear.restype = I
    L.w4a16_linear_static_ws.argtypes = [P, P, P, P, I, I, I, I, P, I, P]
    L.w4a16_linear_static_ws.restype = I
    L.w4a16_linear_gated.argtypes = [P, P, P, P, P, P, P, I, I, I, I, P, I, P, S, P]
    L.w4a16_linear_gated.restype = I
    L.w4a16_linear_batch.argtypes = [P, I, I, I, I, P, S, P]
    L.w4a16_linear_batch.restype = I
    L.w4a16_lmhead_verify.argtypes = [P, P, P, P, I, I, I, I, P, P, I, P, P, P, S, P]
    L.w4a16_lmhead_verify.restype = I
    L.w4a16_workspace_bytes.argtypes = [I, I, I, I, I]
    L.w4a16_workspace_bytes.restype = S
    L.w4a16_status_string.argtypes = [I]
    L.w4a16_status_string.restype = ctypes.c_char_p
    L.w4a16_abi_version.restype = I
    _lib = L
    return L


def status_string(status):
    return lib().w4a16_status_string(int(status)).decode()


def w4a16_workspace_bytes(op, M, N, K, group=GROUP):
    return int(lib().w4a16_workspace_bytes(int(op), int(M), int(N), int(K), int(group)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status, where):
    if status != 0:
        raise W4A16Error(status, where)


class Workspace:
    """A zero-filled device scratch buffer reused across calls (grown on demand).

    The library leaves the counters it uses at zero after every call, so the
    buffer only has to be zero when first allocated.  Calls that share a workspace
    must be ordered: use one Workspace per stream (the default workspaces are kept
    per device and stream), or synchronize the streams between calls."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = None

    def get(self, nbytes, stream=None):
        """The buffer, at least nbytes long.  A new buffer is allocated and zero-filled
        on `stream` (default: the current stream), the stream the call runs on, so the
        call is ordered after the fill and the old buffer is released in that
        stream's order."""
        import torch
        if nbytes == 0:
            return None
        if self.buf is None or self.buf.numel() < nbytes:
            if stream is None:
                self.buf = torch.zeros(nbytes, dtype=torch.uint8, device=self.device)
            else:
                with torch.cuda.stream(stream):
                    self.buf = torch.zeros(nbytes, dtype=torch.uint8, device=self.device)
        return self.buf


_default_ws = {}


def _workspace(ws, device, stream=None):
    """The caller's workspace, or the default one of (device, stream)."""
    import torch
    if ws is not None:
        return ws
    s = torch.cuda.current_stream(device) if stream is None else stream
    key = (str(device), int(s.cuda_stream))
    if key not in _default_ws:
        _default_ws[key] = Workspace(device)
    return _default_ws[key]


def _scratch(ws, device, nbytes, stream):
    return _workspace(ws, device, stream).get(nbytes, stream)


def w4a16_pack(codes, zeros, group=GROUP, stream=None):
    import torch
    N, K = codes.shape
    G = K // group
    qweight = torch.empty((N, K // 8), dtype=torch.int32, device=codes.device)
    qzeros = torch.empty((N // 8, G), dtype=torch.int32, device=codes.device)
    assert codes.dtype == torch.uint8 and zeros.dtype == torch.uint8 and zeros.shape == (N, G)
    st = lib().w4a16_pack(_ptr(codes.contiguous()), _ptr(zeros.contiguous()), N, K, group,
                          _ptr(qweight), _ptr(qzeros), _stream(stream))
    _check(st, "w4a16_pack")
    return qweight, qzeros


def w4a16_actorder_perm(g_idx, group=GROUP):
    """Host: the column permutation that makes every act-order group consecutive."""
    import numpy as np
    g = np.ascontiguousarray(g_idx, dtype=np.int32)
    perm = np.zeros(g.shape[0], np.int32)
    st = lib().w4a16_actorder_perm(g.ctypes.data_as(ctypes.c_void_p), g.shape[0], group,
                                   perm.ctypes.data_as(ctypes.c_void_p))
    _check(st, "w4a16_actorder_perm")
    return perm


def w4a16_pack_actorder(codes, zeros, perm, group=GROUP, stream=None):
    """Pack u8 codes [N,K] (natural column order) in perm order; zeros as w4a16_pack."""
    import torch
    N, K = codes.shape
    G = K // group
    assert codes.dtype == torch.uint8 and zeros.dtype == torch.uint8 and zeros.shape == (N, G)
    assert perm.dtype == torch.int32 and perm.shape == (K,)
    qweight = torch.empty((N, K // 8), dtype=torch.int32, device=codes.device)
    qzeros = torch.empty((N // 8, G), dtype=torch.int32, device=codes.device)
    st = lib().w4a16_pack_actorder(_ptr(codes.contiguous()), _ptr(zeros.contiguous()), _ptr(perm.contiguous()),
                                   N, K, group, _ptr(qweight), _ptr(qzeros), _stream(stream))
    _check(st, "w4a16_pack_actorder")
    return qweight, qzeros


def w4a16_linear_actorder(X, perm, qweight, scales, qzeros, out_dtype=None, group=GROUP, out=None,
                          workspace=None, stream=None):
    """Y = X W^T for an act-order grid packed by w4a16_pack_actorder; X in natural order."""
    import torch
    M, K = X.shape
    N = qweight.shape[0]
    if out_dtype is None:
        out_dtype = torch.bfloat16 if out is None else out.dtype
    ydt = OUT_F32 if out_dtype == torch.float32 else OUT_BF16
    assert X.dtype == torch.bfloat16 and X.is_contiguous() and perm.dtype == torch.int32
    Y = out if out is not None else torch.empty((M, N), dtype=out_dtype, device=X.device)
    nbytes = w4a16_workspace_bytes(OP_LINEAR_ACTORDER, M, N, K, group)
    ws = _scratch(workspace, X.device, nbytes, stream)
    st = lib().w4a16_linear_actorder(_ptr(X), _ptr(perm), _ptr(qweight), _ptr(scales), _ptr(qzeros), M, N, K,
                                     group, _ptr(Y), ydt, _ptr(ws), nbytes, _stream(stream))
    _check(st, "w4a16_linear_actorder")
    return Y


def w4a16_swa_attention(Q, K, Vt, T, window, out_dtype=None, out=None, workspace=None, stream=None, block=False):
    """Causal sliding-window attention of Q [M,Hq,128] over K [T_alloc,Hkv,128] and the
    transposed values Vt [Hkv,128,t_stride] (the first T tokens are the context).
    block=True: bidirectional within the block of the last M tokens
    (w4a16_swa_attention_block)."""
    import torch
    M, Hq, D = Q.shape
    Hkv = K.shape[1]
    t_stride = Vt.shape[2]
    assert Q.dtype == K.dtype == Vt.dtype == torch.bfloat16
    assert Q.is_contiguous() and K.is_contiguous() and Vt.is_contiguous() and K.shape[0] >= T
    if out_dtype is None:
        out_dtype = torch.bfloat16 if out is None else out.dtype
    odt = OUT_F32 if out_dtype == torch.float32 else OUT_BF16
    O = out if out is not None else torch.empty((M, Hq, D), dtype=out_dtype, device=Q.device)
    nbytes = lib().w4a16_swa_workspace_bytes(M, T, Hq, Hkv, window)
    ws = _scratch(workspace, Q.device, nbytes, stream)
    fn = lib().w4a16_swa_attention_block if block else lib().w4a16_swa_attention
    st = fn(_ptr(Q), _ptr(K), _ptr(Vt), M, T, Hq, Hkv, D, window, t_stride, _ptr(O), odt, _ptr(ws), nbytes,
            _stream(stream))
    _check(st, "w4a16_swa_attention_block" if block else "w4a16_swa_attention")
    return O


def w4a16_quantize(W, scales, qzeros, group=GROUP, out=None, stream=None):
    """Round bf16 W [N,K] onto the grid with frozen fp16 scales [N,G] and packed qzeros
    [N/8,G]; returns the packed qweight [N,K/8] (int32 view of the uint32 words)."""
    import torch
    N, K = W.shape
    assert W.dtype == torch.bfloat16 and scales.dtype == torch.float16
    assert W.is_contiguous() and scales.is_contiguous() and qzeros.is_contiguous()
    qweight = out if out is not None else torch.empty((N, K // 8), dtype=torch.int32, device=W.device)
    assert qweight.shape == (N, K // 8) and qweight.dtype == torch.int32 and qweight.is_contiguous()
    st = lib().w4a16_quantize(_ptr(W), _ptr(scales), _ptr(qzeros), N, K, group, _ptr(qweight), _stream(stream))
    _check(st, "w4a16_quantize")
    return qweight


def w4a16_linear(X, qweight, scales, qzeros, out_dtype=None, group=GROUP, out=None,
                 workspace=None, stream=None):
    import torch
    M, K = X.shape
    N = qweight.shape[0]
    assert X.dtype == torch.bfloat16 and scales.dtype == torch.float16
    assert X.is_contiguous() and qweight.is_contiguous() and scales.is_contiguous() and qzeros.is_contiguous()
    if out_dtype is None:
        out_dtype = torch.bfloat16 if out is None else out.dtype
    ydt = OUT_F32 if out_dtype == torch.float32 else OUT_BF16
    Y = out if out is not None else torch.empty((M, N), dtype=out_dtype, device=X.device)
    assert Y.shape == (M, N) and Y.dtype == out_dtype and Y.is_contiguous()
    nbytes = w4a16_workspace_bytes(OP_LINEAR, M, N, K, group)
    ws = _scratch(workspace, X.device, nbytes, stream)
    st = lib().w4a16_linear(_ptr(X), _ptr(qweight), _ptr(scales), _ptr(qzeros), M, N, K, group,
                            _ptr(Y), ydt, _ptr(ws), nbytes, _stream(stream))
    _check(st, "w4a16_linear")
    return Y


def w4a16_linear_static_ws(X, qweight, scales, qzeros, out_dtype=None, group=GROUP, out=None, stream=None):
    """w4a16_linear with the library's own per-device scratch array (no workspace
    argument); pass `out` to make the call allocate nothing at all."""
    import torch
    M, K = X.shape
    N = qweight.shape[0]
    assert X.dtype == torch.bfloat16 and scales.dtype == torch.float16
    assert X.is_contiguous() and qweight.is_contiguous() and scales.is_contiguous() and qzeros.is_contiguous()
    if out_dtype is None:
        out_dtype = torch.bfloat16 if out is None else out.dtype
    ydt = OUT_F32 if out_dtype == torch.float32 else OUT_BF16
    Y = out if out is not None else torch.empty((M, N), dtype=out_dtype, device=X.device)
    assert Y.shape == (M, N) and Y.dtype == out_dtype and Y.is_contiguous()
    st = lib().w4a16_linear_static_ws(_ptr(X), _ptr(qweight), _ptr(scales), _ptr(qzeros), M, N, K, group,
                                      _ptr(Y), ydt, _stream(stream))
    _check(st, "w4a16_linear_static_ws")
    return Y


def w4a16_linear_gated(X, gate, up, out_dtype=None, group=GROUP, out=None, workspace=None, stream=None):
    """Y = silu(X Wg^T) * (X Wu^T); gate and up are (qweight, scales, qzeros) over the same N."""
    import torch
    M, K = X.shape
    (qg, sg, zg), (qu, su, zu) = gate, up
    N = qg.shape[0]
    assert X.dtype == torch.bfloat16 and sg.dtype == torch.float16 and su.dtype == torch.float16
    assert qu.shape == qg.shape and su.shape == sg.shape and zu.shape == zg.shape
    for t in (X, qg, sg, zg, qu, su, zu):
        assert t.is_contiguous()
    if out_dtype is None:
        out_dtype = torch.bfloat16 if out is None else out.dtype
    ydt = OUT_F32 if out_dtype == torch.float32 else OUT_BF16
    Y = out if out is not None else torch.empty((M, N), dtype=out_dtype, device=X.device)
    assert Y.shape == (M, N) and Y.dtype == out_dtype and Y.is_contiguous()
    nbytes = w4a16_workspace_bytes(OP_LINEAR_GATED, M, N, K, group)
    ws = _scratch(workspace, X.device, nbytes, stream)
    st = lib().w4a16_linear_gated(_ptr(X), _ptr(qg), _ptr(sg), _ptr(zg), _ptr(qu), _ptr(su), _ptr(zu), M, N, K,
                                  group, _ptr(Y), ydt, _ptr(ws), nbytes, _stream(stream))
    _check(st, "w4a16_linear_gated")
    return Y


def w4a16_linear_batch(problems, out_dtype=None, group=GROUP, outs=None, workspace=None, stream=None):
    """problems: list of (X, qweight, scales, qzeros) sharing M; returns the list of Y."""
    import torch
    if len(problems) == 0:
        return []
    M = problems[0][0].shape[0]
    if out_dtype is None:
        out_dtype = torch.bfloat16 if outs is None else outs[0].dtype
    ydt = OUT_F32 if out_dtype == torch.float32 else OUT_BF16
    arr = (Problem * len(problems))()
    ys = []
    need = 0
    for q, (X, qweight, scales, qzeros) in enumerate(problems):
        assert X.dtype == torch.bfloat16 and scales.dtype == torch.float16 and X.shape[0] == M
        assert X.is_contiguous() and qweight.is_contiguous() and scales.is_contiguous() and qzeros.is_contiguous()
        K = X.shape[1]
        N = qweight.shape[0]
        Y = outs[q] if outs is not None else torch.empty((M, N), dtype=out_dtype, device=X.device)
        assert Y.shape == (M, N) and Y.dtype == out_dtype and Y.is_contiguous()
        arr[q] = Problem(X.data_ptr(), qweight.data_ptr(), scales.data_ptr(), qzeros.data_ptr(), Y.data_ptr(), N, K)
        need += w4a16_workspace_bytes(OP_LINEAR, M, N, K, group)
        ys.append(Y)
    ws = _scratch(workspace, problems[0][0].device, need, stream)
    st = lib().w4a16_linear_batch(ctypes.cast(arr, ctypes.c_void_p), len(problems), M, group, ydt, _ptr(ws), need,
                                  _stream(stream))
    _check(st, "w4a16_linear_batch")
    return ys


def w4a16_lmhead_verify(X, qweight, scales, qzeros, draft_ids, return_logits=False,
                        logits_dtype=None, group=GROUP, workspace=None, stream=None,
                        argmax_out=None, accept_out=None, logits_out=None):
    import torch
    M, K = X.shape
    N = qweight.shape[0]
    assert X.dtype == torch.bfloat16 and scales.dtype == torch.float16 and draft_ids.dtype == torch.int32
    assert X.is_contiguous() and draft_ids.is_contiguous()
    argmax = argmax_out if argmax_out is not None else torch.empty((M,), dtype=torch.int32, device=X.device)
    accept = accept_out if accept_out is not None else torch.empty((1,), dtype=torch.int32, device=X.device)
    Y = logits_out
    ydt = OUT_BF16
    if Y is not None:
        ydt = OUT_F32 if Y.dtype == torch.float32 else OUT_BF16
        assert Y.shape == (M, N) and Y.is_contiguous()
    elif return_logits:
        ldt = torch.float32 if logits_dtype is None else logits_dtype
        ydt = OUT_F32 if ldt == torch.float32 else OUT_BF16
        Y = torch.empty((M, N), dtype=ldt, device=X.device)
    nbytes = w4a16_workspace_bytes(OP_LMHEAD, M, N, K, group)
    ws = _scratch(workspace, X.device, nbytes, stream)
    st = lib().w4a16_lmhead_verify(_ptr(X), _ptr(qweight), _ptr(scales), _ptr(qzeros), M, N, K, group,
                                   _ptr(draft_ids), _ptr(Y), ydt, _ptr(argmax), _ptr(accept),
                                   _ptr(ws), nbytes, _stream(stream))
    _check(st, "w4a16_lmhead_verify")
    return argmax, accept, Y
