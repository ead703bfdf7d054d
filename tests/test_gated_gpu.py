"""GPU parity of w4a16_linear_gated (Y = silu(X Wg^T) * (X Wu^T)) with the fp64 oracle.

Tolerance: the linear's contract on each projection (|dG| <= 1e-2 rms(G), likewise U)
carried through y = silu(g) u (tests/gpu_util.py, gated_bound), + half a bf16 ulp of y
on bf16 output.  The small-M path keeps the codes exact (errors of about 1e-5 of the
bound); the tile kernels round each weight to fp16 once (about 3e-4 rms per
projection), which the product amplifies where |g| and |u| are large.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check_gated, dev_inputs, gated_bound

torch = pytest.importorskip("torch")
w4 = pytest.importorskip("int4_weight_only_02_amd")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    w4.lib()
    return torch.device("cuda:0")


def _grid(d, dev):
    t = dev_inputs(d, dev)
    qw, qz = w4.w4a16_pack(t["codes"], t["zeros"])
    oqw, oqz = oracle.pack(d["codes"], d["zeros"])
    return t, (qw, t["scales"], qz), (oqw, d["scales"], oqz)


def _pair(seed, M, N, K, dev):
    dg = synth.linear_inputs(seed, M, N, K)
    du = synth.linear_inputs(seed + 1, M, N, K)
    tg, gate, ogate = _grid(dg, dev)
    _, up, oup = _grid(du, dev)
    return dg["X"], tg["X"], gate, up, ogate, oup


@pytest.mark.parametrize("ydt", ["f32", "bf16"])
@pytest.mark.parametrize("workload,jg,ju", [("verify_block_m16", 4, 5), ("decode_gemv_m1", 0, 0)])
def test_gated_full_size(dev, workload, jg, ju, ydt):
    # the draft block's gate and up projections (M = 16, K 2560 -> N 9728) sharing the
    # gate's activations; at M = 1 the decode gate/up shape with two seeded grids
    label, M, K, N = synth.WORKLOADS[workload][jg]
    print("gated full", workload, M, N, K, ydt, flush=True)
    dg = synth.workload_inputs(workload, jg)
    du = synth.workload_inputs(workload, ju) if ju != jg else synth.linear_inputs(synth.seed_for(workload, jg) + 5,
                                                                                   M, N, K)
    tg, gate, ogate = _grid(dg, dev)
    _, up, oup = _grid(du, dev)
    Y = w4.w4a16_linear_gated(tg["X"], gate, up, out_dtype=torch.float32 if ydt == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    G, U = oracle.linear(dg["X"], *ogate), oracle.linear(dg["X"], *oup)
    r = check_gated(Y, G, U, oracle.silu_mul(G, U), "gated %s %s" % (workload, ydt))
    print("  max|dY|/tol %.2e" % r)


# M = 1 up to 40 groups runs the decode kernel (one group, 40 groups with a ragged last
# wave; 41 groups fall back to the small-M pair plan); 2 <= M <= 16 with K whole runs
# the draft-block kernel (one to three column tiles per workgroup, one or two groups per
# wave, ragged tile groups); K split into parts or more than three tiles per CU fall
# back to the small-M pair plan
SHAPES = [(1, 16, 128), (1, 1040, 5120), (1, 528, 5248), (2, 48, 640), (3, 528, 1280), (4, 2064, 2560), (5, 1040, 384), (6, 1040, 128),
          (3, 4112, 128), (5, 8208, 128),
          (8, 336, 9728), (12, 12304, 1280), (16, 4112, 2560), (16, 2560, 9728), (17, 528, 1280), (40, 1040, 640),
          (64, 272, 4096), (65, 528, 1280), (130, 1040, 640), (2000, 4112, 256)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gated_small(dev, M, N, K):
    # ragged tile counts, every small-M plan (private, DMA, shared, chunked, direct), the
    # mid-M path (two tiled projections and the activation kernel) and the gated tile
    # kernel (2000 x 4112: 8 x 33 tiles, the last row tile and column tile ragged)
    print("gated", M, N, K, flush=True)
    Xh, X, gate, up, ogate, oup = _pair(300 + M + N + K, M, N, K, dev)
    Y = w4.w4a16_linear_gated(X, gate, up, out_dtype=torch.float32)
    torch.cuda.synchronize()
    G, U = oracle.linear(Xh, *ogate), oracle.linear(Xh, *oup)
    check_gated(Y, G, U, oracle.silu_mul(G, U), "gated %d %d %d" % (M, N, K))


@pytest.mark.parametrize("ydt", ["f32", "bf16"])
def test_gated_prefill_sampled(dev, ydt):
    # prefill of the MLP's first half (M = 8192, K 2560 -> N 9728: the gated tile
    # kernel), sampled outputs against the oracle evaluated one by one
    M, N, K = 8192, 9728, 2560
    print("gated prefill", M, N, K, flush=True)
    Xh, X, gate, up, ogate, oup = _pair(77, M, N, K, dev)
    Y = w4.w4a16_linear_gated(X, gate, up, out_dtype=torch.float32 if ydt == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.concatenate([rng.integers(0, M, 600), [0, M - 1, M - 1]]).astype(np.int32)
    cols = np.concatenate([rng.integers(0, N, 600), [0, N - 1, 0]]).astype(np.int32)
    g = oracle.linear_at(Xh, *ogate, rows, cols)
    u = oracle.linear_at(Xh, *oup, rows, cols)
    yo = oracle.silu_mul(g, u)
    y = Y.float().cpu().numpy()[rows, cols].astype(np.float64)
    # the bound of each sampled output (the sample's rms of g and u stand in for the
    # whole projections'); bf16 output adds half a bf16 ulp of each value
    tol = gated_bound(g, u)
    if ydt == "bf16":
        tol = tol + np.abs(yo) * 2.0 ** -8
    assert (np.abs(y - yo) <= tol).all(), float(np.abs(y - yo).max())


def test_gated_matches_the_linear_calls_and_is_deterministic(dev):
    # the fused call against silu(gate) * up formed from w4a16_linear's own fp32 outputs
    # (the two plans sum K in different orders: agreement to fp32 rounding, not bits),
    # and bit-exact repeats
    for M, N, K in [(16, 2560, 9728), (1, 9728, 2560), (3, 528, 1280), (130, 1040, 640), (1100, 9728, 256)]:
        Xh, X, gate, up, _, _ = _pair(93 + M, M, N, K, dev)
        Y1 = w4.w4a16_linear_gated(X, gate, up, out_dtype=torch.float32)
        Y2 = w4.w4a16_linear_gated(X, gate, up, out_dtype=torch.float32)
        G = w4.w4a16_linear(X, *gate, out_dtype=torch.float32)
        U = w4.w4a16_linear(X, *up, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(Y1, Y2), (M, N, K)
        g, u = G.double().cpu().numpy(), U.double().cpu().numpy()
        ref = g / (1.0 + np.exp(-g)) * u
        err = np.abs(Y1.double().cpu().numpy() - ref).max()
        assert err <= 1e-4 * float(np.sqrt(np.mean(ref * ref))), (M, N, K, float(err))


def test_gated_errors(dev):
    Xh, X, gate, up, _, _ = _pair(95, 4, 48, 256, dev)
    with pytest.raises(w4.W4A16Error) as e:  # N % 16 != 0
        qg, sg, zg = gate
        qu, su, zu = up
        w4.w4a16_linear_gated(X, (qg[:40], sg[:40], zg[:5]), (qu[:40], su[:40], zu[:5]))
    assert e.value.status == 2
    Xh, X, gate, up, _, _ = _pair(96, 65, 48, 256, dev)
    Y = torch.empty((65, 48), dtype=torch.float32, device=dev)
    st = w4.lib().w4a16_linear_gated(w4._ptr(X), w4._ptr(gate[0]), w4._ptr(gate[1]), w4._ptr(gate[2]),
                                     w4._ptr(up[0]), w4._ptr(up[1]), w4._ptr(up[2]), 65, 48, 256, 128,
                                     w4._ptr(Y), 1, None, 0, w4._stream(None))
    assert st == 5  # M > 64 needs the workspace for both projections' outputs
