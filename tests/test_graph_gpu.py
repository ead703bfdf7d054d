"""Every entry point captured in a HIP graph (as the benchmark replays them) and
replayed several times, with other eager calls through the same workspace and
device synchronizations between the replays: each replay must reproduce the eager
result bit for bit.  The kernels take no memset and keep their cross-workgroup
counters (arrival tickets, argmax keys) at zero after every call, so nothing in the
workspace carries over from one call, eager or replayed, to the next.
"""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
w4 = pytest.importorskip("int4_weight_only_02_amd")

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    w4.lib()
    return torch.device("cuda:0")


def _packed(seed, M, N, K, dev):
    d = synth.linear_inputs(seed, M, N, K)
    X = torch.from_numpy(d["X"].view(np.int16)).to(dev).view(torch.bfloat16)
    S = torch.from_numpy(d["scales"].view(np.int16)).to(dev).view(torch.float16)
    qw, qz = w4.w4a16_pack(torch.from_numpy(d["codes"]).to(dev), torch.from_numpy(d["zeros"]).to(dev))
    return X, qw, S, qz


def _workspace(dev, nbytes):
    # grown once, before any capture: a graph keeps the buffer it was captured with
    ws = w4.Workspace(dev)
    ws.get(nbytes)
    return ws


_disturb_ref = {}


def _disturb_calls(dev, ws):
    # eager calls of other shapes and paths through one workspace: attention (its
    # per-chunk scratch), a chunked projection (arrival tickets, partial sums) and a
    # small lm_head (argmax keys, ticket)
    rng = np.random.default_rng(7)
    b = lambda shape: torch.from_numpy(synth.f32_to_bf16_bits(rng.normal(0, 1, shape).astype(np.float32))
                                       .view(np.int16)).to(dev).view(torch.bfloat16)
    Q, Kc, Vt = b((16, 8, 128)), b((3000, 2, 128)), b((2, 128, 3000))
    O = w4.w4a16_swa_attention(Q, Kc, Vt, 3000, 2048, out_dtype=torch.float32, workspace=ws)
    X, qw, S, qz = _packed(5, 16, 1024, 9728, dev)
    Y = w4.w4a16_linear(X, qw, S, qz, out_dtype=torch.float32, workspace=ws)
    X, qw, S, qz = _packed(6, 3, 520, 640, dev)
    draft = torch.tensor([1, 2, 3], dtype=torch.int32, device=dev)
    am, acc, _ = w4.w4a16_lmhead_verify(X, qw, S, qz, draft, workspace=ws)
    torch.cuda.synchronize()
    return [O, Y, am, acc]


def _disturb(dev, ws):
    """The eager calls between replays; each result must equal the same call on a
    fresh zero-filled workspace (nothing any call leaves behind may change another)."""
    if "ref" not in _disturb_ref:
        fresh = w4.Workspace(dev)
        fresh.get(1 << 24)
        _disturb_ref["ref"] = [t.clone() for t in _disturb_calls(dev, fresh)]
    for got, want in zip(_disturb_calls(dev, ws), _disturb_ref["ref"]):
        assert torch.equal(got, want), "a call through the shared workspace differs from a fresh one"


def _check_replays(dev, ws, run, outs):
    """run() enqueues the call writing into outs; compare graph replays with eager."""
    run()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()  # on the capture stream once before capturing
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, ref):
            assert torch.equal(o, e), "replay %d differs from the eager result" % r
        _disturb(dev, ws)


@pytest.mark.parametrize("M,N,K,f32", [(16, 2560, 9728, True), (1, 9728, 2560, False), (5, 2560, 9728, True),
                                       (300, 520, 1280, True),
                                       # the prefill stream plan: tiles split at segment boundaries
                                       # meet through arrival counters that each call returns to zero
                                       (4300, 4104, 384, True)])
def test_linear_graph_replays(dev, M, N, K, f32):
    print("graph linear", M, N, K, flush=True)
    X, qw, S, qz = _packed(11 + M, M, N, K, dev)
    ws = _workspace(dev, max(w4.w4a16_workspace_bytes(w4.OP_LINEAR, M, N, K), 1 << 24))
    Y = torch.empty((M, N), dtype=torch.float32 if f32 else torch.bfloat16, device=dev)
    _check_replays(dev, ws, lambda: w4.w4a16_linear(X, qw, S, qz, out=Y, workspace=ws), [Y])


def test_lmhead_graph_replays(dev):
    M, N, K = 16, 65536, 512  # enough columns for the persistent (streaming) plan
    print("graph lm_head", M, N, K, flush=True)
    X, qw, S, qz = _packed(21, M, N, K, dev)
    draft = torch.from_numpy(np.random.default_rng(3).integers(0, N, M).astype(np.int32)).to(dev)
    ws = _workspace(dev, max(w4.w4a16_workspace_bytes(w4.OP_LMHEAD, M, N, K), 1 << 24))
    am = torch.empty((M,), dtype=torch.int32, device=dev)
    acc = torch.empty((1,), dtype=torch.int32, device=dev)
    Y = torch.empty((M, N), dtype=torch.float32, device=dev)

    def run():
        w4.w4a16_lmhead_verify(X, qw, S, qz, draft, workspace=ws, argmax_out=am, accept_out=acc, logits_out=Y)

    _check_replays(dev, ws, run, [am, acc, Y])


def test_batch_graph_replays(dev):
    M = 16
    print("graph batch", M, flush=True)
    shapes = [(2560, 4096), (9728, 2560), (2560, 1024)]  # (K, N): one of them chunked
    probs = [_packed(31 + q, M, N, K, dev) for q, (K, N) in enumerate(shapes)]
    need = sum(w4.w4a16_workspace_bytes(w4.OP_LINEAR, M, N, K) for K, N in shapes)
    ws = _workspace(dev, max(need, 1 << 24))
    ys = [torch.empty((M, N), dtype=torch.float32, device=dev) for K, N in shapes]
    _check_replays(dev, ws, lambda: w4.w4a16_linear_batch(probs, outs=ys, workspace=ws), ys)


def test_batch_one_x_graph_replays(dev):
    # M = 1, three projections reading one X (q, k, v): one launch of the decode kernel
    print("graph batch one X M=1", flush=True)
    shapes = [(2560, 4096), (2560, 1024), (2560, 1024)]  # (K, N)
    probs = [_packed(71 + q, 1, N, K, dev) for q, (K, N) in enumerate(shapes)]
    probs = [(probs[0][0],) + p[1:] for p in probs]
    ws = _workspace(dev, 1 << 24)
    ys = [torch.empty((1, N), dtype=torch.bfloat16, device=dev) for K, N in shapes]
    _check_replays(dev, ws, lambda: w4.w4a16_linear_batch(probs, outs=ys, workspace=ws), ys)


def test_actorder_graph_replays(dev):
    M, N, K = 16, 2560, 9728
    print("graph act-order", M, N, K, flush=True)
    rng = np.random.default_rng(41)
    g_idx = rng.permutation(np.repeat(np.arange(K // 128, dtype=np.int32), 128))
    perm = torch.from_numpy(w4.w4a16_actorder_perm(g_idx)).to(dev)
    d = synth.linear_inputs(42, M, N, K)
    X = torch.from_numpy(d["X"].view(np.int16)).to(dev).view(torch.bfloat16)
    S = torch.from_numpy(d["scales"].view(np.int16)).to(dev).view(torch.float16)
    qw, qz = w4.w4a16_pack_actorder(torch.from_numpy(d["codes"]).to(dev), torch.from_numpy(d["zeros"]).to(dev), perm)
    ws = _workspace(dev, max(w4.w4a16_workspace_bytes(w4.OP_LINEAR_ACTORDER, M, N, K), 1 << 24))
    Y = torch.empty((M, N), dtype=torch.float32, device=dev)
    _check_replays(dev, ws, lambda: w4.w4a16_linear_actorder(X, perm, qw, S, qz, out=Y, workspace=ws), [Y])


def test_swa_graph_replays(dev):
    M, T, Hq, Hkv, W = 16, 8192, 32, 8, 2048
    print("graph swa", M, T, Hq, Hkv, W, flush=True)
    rng = np.random.default_rng(51)
    b = lambda shape: torch.from_numpy(synth.f32_to_bf16_bits(rng.normal(0, 1, shape).astype(np.float32))
                                       .view(np.int16)).to(dev).view(torch.bfloat16)
    Q, K, Vt = b((M, Hq, 128)), b((T, Hkv, 128)), b((Hkv, 128, T))
    ws = _workspace(dev, max(w4.lib().w4a16_swa_workspace_bytes(M, T, Hq, Hkv, W), 1 << 24))
    O = torch.empty((M, Hq, 128), dtype=torch.float32, device=dev)
    _check_replays(dev, ws, lambda: w4.w4a16_swa_attention(Q, K, Vt, T, W, out=O, workspace=ws), [O])


def test_quantize_graph_replays(dev):
    N, K = 1024, 2560
    print("graph quantize", N, K, flush=True)
    d = synth.requant_inputs(61, N, K)
    Wt = torch.from_numpy(d["W"].view(np.int16)).to(dev).view(torch.bfloat16)
    S = torch.from_numpy(d["scales"].view(np.int16)).to(dev).view(torch.float16)
    _, qz = w4.w4a16_pack(torch.zeros((N, K), dtype=torch.uint8, device=dev), torch.from_numpy(d["zeros"]).to(dev))
    ws = _workspace(dev, 1 << 24)
    out = torch.empty((N, K // 8), dtype=torch.int32, device=dev)
    _check_replays(dev, ws, lambda: w4.w4a16_quantize(Wt, S, qz, out=out), [out])


@pytest.mark.parametrize("M,K", [(16, 2560), (16, 9728), (130, 640), (3100, 256)])
def test_gated_graph_replays(dev, M, K):
    # M = 3100: the gated tile kernel (13 x 20 tiles of 256 rows x 128 columns)
    N = 2560
    print("graph gated", M, N, K, flush=True)
    X, qg, sg, zg = _packed(71 + K, M, N, K, dev)
    _, qu, su, zu = _packed(72 + K, M, N, K, dev)
    ws = _workspace(dev, max(w4.w4a16_workspace_bytes(w4.OP_LINEAR_GATED, M, N, K), 1 << 24))
    Y = torch.empty((M, N), dtype=torch.float32, device=dev)
    _check_replays(dev, ws, lambda: w4.w4a16_linear_gated(X, (qg, sg, zg), (qu, su, zu), out=Y, workspace=ws), [Y])


def test_workspace_shared_across_paths(dev):
    """Attention, then lm_head verify, then a K-chunked M = 16 projection through one
    workspace: argmax, accept_len and Y equal the same calls on fresh workspaces."""
    print("shared workspace", flush=True)
    M, N, K = 16, 4096, 2560
    X, qw, S, qz = _packed(81, M, N, K, dev)
    draft = torch.from_numpy(np.random.default_rng(8).integers(0, N, M).astype(np.int32)).to(dev)
    Xc, qwc, Sc, qzc = _packed(82, 16, 2560, 9728, dev)

    def lm(ws):
        am, acc, _ = w4.w4a16_lmhead_verify(X, qw, S, qz, draft, workspace=ws)
        return am, acc

    def lin(ws):
        return w4.w4a16_linear(Xc, qwc, Sc, qzc, out_dtype=torch.float32, workspace=ws)

    def fresh():
        ws = w4.Workspace(dev)
        ws.get(1 << 24)
        return ws

    am0, acc0 = lm(fresh())
    y0 = lin(fresh())
    torch.cuda.synchronize()
    shared = fresh()
    rng = np.random.default_rng(9)
    b = lambda shape: torch.from_numpy(synth.f32_to_bf16_bits(rng.normal(0, 1, shape).astype(np.float32))
                                       .view(np.int16)).to(dev).view(torch.bfloat16)
    Q, Kc, Vt = b((16, 32, 128)), b((8192, 8, 128)), b((8, 128, 8192))
    w4.w4a16_swa_attention(Q, Kc, Vt, 8192, 2048, workspace=shared)
    am1, acc1 = lm(shared)
    y1 = lin(shared)
    torch.cuda.synchronize()
    assert torch.equal(am1, am0) and torch.equal(acc1, acc0)
    assert torch.equal(y1, y0)
