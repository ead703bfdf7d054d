"""GPU parity of w4a16_linear_batch (several projections of the same rows in one
launch) against the fp64 CPU oracle, through the C ABI.

Covers one decoder layer's seven projections on a 16-row draft block and the decode
pair at full size, mixed ragged shapes at several row counts (including the
one-after-another path above 64 rows and empty entries), bit-exact dyadic inputs,
and agreement with single calls.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check, dev_inputs

torch = pytest.importorskip("torch")
w4 = pytest.importorskip("int4_weight_only_02_amd")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    w4.lib()
    return torch.device("cuda:0")


def _prep(d, dev):
    t = dev_inputs(d, dev)
    qw, qz = w4.w4a16_pack(t["codes"], t["zeros"])
    oqw, oqz = oracle.pack(d["codes"], d["zeros"])
    return (t["X"], qw, t["scales"], qz), (oqw, oqz)


@pytest.mark.parametrize("workload", ["verify_block_m16", "decode_gemv_m1"])
@pytest.mark.parametrize("ydt", ["f32", "bf16"])
def test_batch_workload_full_size(dev, workload, ydt):
    print("batch", workload, ydt, flush=True)
    shapes = synth.WORKLOADS[workload]
    datas = [synth.workload_inputs(workload, j) for j in range(len(shapes))]
    probs, oras = zip(*[_prep(d, dev) for d in datas])
    ys = w4.w4a16_linear_batch(list(probs), out_dtype=torch.float32 if ydt == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    for (label, M, K, N), d, (oqw, oqz), Y in zip(shapes, datas, oras, ys):
        Yo = oracle.linear_matmul(d["X"], oqw, d["scales"], oqz)
        r = check(Y, Yo, "%s %s" % (label, ydt))
        print("  %s max|dY|/tol %.2e" % (label, r))


MIXED = [(128, 264), (640, 520), (2560, 8), (1280, 1032), (384, 136)]  # (K, N) per projection


@pytest.mark.parametrize("M", [1, 2, 3, 5, 16, 17, 40, 64, 65, 130])
def test_batch_mixed_shapes(dev, M):
    print("batch mixed M", M, flush=True)
    datas = [synth.linear_inputs(1000 + 31 * M + q, M, N, K) for q, (K, N) in enumerate(MIXED)]
    probs, oras = zip(*[_prep(d, dev) for d in datas])
    ys = w4.w4a16_linear_batch(list(probs), out_dtype=torch.float32)
    torch.cuda.synchronize()
    for (K, N), d, (oqw, oqz), Y in zip(MIXED, datas, oras, ys):
        check(Y, oracle.linear(d["X"], oqw, d["scales"], oqz), "M=%d K=%d N=%d" % (M, K, N))


# two projections per launch through the draft-block kernel's multi-projection
# instances: one group per wave with 1, 2 and 3 tiles per workgroup (K = 128), three
# groups per wave (41 groups) with 1 and 2 tiles; ragged tile groups throughout
MULTI = [[(128, 264), (128, 136)], [(128, 2560), (128, 2568)], [(128, 9728), (128, 1032)],
         [(5248, 264), (640, 136)], [(5248, 2568), (640, 2056)]]


@pytest.mark.parametrize("M", [3, 16])
@pytest.mark.parametrize("j", range(len(MULTI)))
def test_batch_block_instances(dev, M, j):
    shapes = MULTI[j]
    print("batch block instances M", M, shapes, flush=True)
    datas = [synth.linear_inputs(2000 + 17 * M + 5 * j + q, M, N, K) for q, (K, N) in enumerate(shapes)]
    probs, oras = zip(*[_prep(d, dev) for d in datas])
    ys = w4.w4a16_linear_batch(list(probs), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for (K, N), d, (oqw, oqz), Y in zip(shapes, datas, oras, ys):
        check(Y, oracle.linear(d["X"], oqw, d["scales"], oqz), "M=%d K=%d N=%d" % (M, K, N))


def _dyadic(seed, M, N, K):
    rng = np.random.default_rng(seed)
    G = K // 128
    return {"codes": rng.integers(0, 16, size=(N, K), dtype=np.uint8),
            "zeros": rng.integers(0, 16, size=(N, G), dtype=np.uint8),
            "scales": synth.f32_to_f16_bits((2.0 ** -rng.integers(6, 10, size=(N, G))).astype(np.float32)),
            "X": synth.f32_to_bf16_bits(rng.integers(-8, 9, size=(M, K)).astype(np.float32))}


@pytest.mark.parametrize("M", [1, 16])
def test_batch_dyadic_bit_exact(dev, M):
    # integer X in [-8, 8], s = 2^-e: every partial sum is exact in fp32, in any order
    print("batch dyadic M", M, flush=True)
    shapes = [(2560, 4096), (2560, 1024), (4096, 2560), (9728, 2560), (2560, 9728)]
    datas = [_dyadic(77 + q, M, N, K) for q, (K, N) in enumerate(shapes)]
    probs, oras = zip(*[_prep(d, dev) for d in datas])
    ys = w4.w4a16_linear_batch(list(probs), out_dtype=torch.float32)
    torch.cuda.synchronize()
    for d, (oqw, oqz), Y in zip(datas, oras, ys):
        Yo = oracle.linear(d["X"], oqw, d["scales"], oqz)
        assert (Y.cpu().numpy().astype(np.float64) == Yo).all()


def test_batch_matches_single_calls_and_is_deterministic(dev):
    print("batch vs single", flush=True)
    shapes = [(2560, 4096), (2560, 1024), (4096, 2560)]
    datas = [synth.linear_inputs(500 + q, 16, N, K) for q, (K, N) in enumerate(shapes)]
    probs = [_prep(d, dev)[0] for d in datas]
    ys1 = w4.w4a16_linear_batch(probs, out_dtype=torch.float32)
    ys2 = w4.w4a16_linear_batch(probs, out_dtype=torch.float32)
    singles = [w4.w4a16_linear(*p, out_dtype=torch.float32) for p in probs]
    torch.cuda.synchronize()
    for d, a, b, s in zip(datas, ys1, ys2, singles):
        assert torch.equal(a, b)  # same launch shape: bit-identical
        ref = s.double()
        tol = 1e-2 * float(ref.pow(2).mean().sqrt())
        assert float((a.double() - ref).abs().max()) <= tol


def test_batch_empty_entries_and_errors(dev):
    print("batch edges", flush=True)
    d = synth.linear_inputs(9, 4, 264, 640)
    p, (oqw, oqz) = _prep(d, dev)
    X, qw, s, qz = p
    empty_qw = torch.empty((0, 80), dtype=torch.int32, device=dev)
    empty_s = torch.empty((0, 5), dtype=torch.float16, device=dev)
    empty_qz = torch.empty((0, 5), dtype=torch.int32, device=dev)
    ys = w4.w4a16_linear_batch([(X, empty_qw, empty_s, empty_qz), p], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert ys[0].shape == (4, 0)
    check(ys[1], oracle.linear(d["X"], oqw, d["scales"], oqz), "after an empty entry")
    assert w4.w4a16_linear_batch([]) == []
    with pytest.raises(w4.W4A16Error):
        w4.w4a16_linear_batch([p] * 9)


@pytest.mark.parametrize("K,N", [(2560, 9728), (5120, 1040), (128, 16), (5248, 528)])
@pytest.mark.parametrize("ydt", ["f32", "bf16"])
def test_batch_pair_one_row(dev, K, N, ydt):
    # two projections of one shape reading the same X at M = 1 (gate and up): one launch
    # of the decode kernel with both grids in each wave up to 40 groups (41 groups: one
    # launch of it with a run of workgroups per projection); each output against the
    # oracle, and bit-identical to the single call (the same per-projection sums in the
    # same order)
    print("batch pair M=1", K, N, ydt, flush=True)
    dt = torch.float32 if ydt == "f32" else torch.bfloat16
    d0 = synth.linear_inputs(300 + K + N, 1, N, K)
    d1 = synth.linear_inputs(301 + K + N, 1, N, K)
    d1 = dict(d1, X=d0["X"])
    p0, (oqw0, oqz0) = _prep(d0, dev)
    p1, (oqw1, oqz1) = _prep(d1, dev)
    p1 = (p0[0],) + tuple(p1[1:])  # the same X tensor
    y0, y1 = w4.w4a16_linear_batch([p0, p1], out_dtype=dt)
    s0 = w4.w4a16_linear(*p0, out_dtype=dt)
    s1 = w4.w4a16_linear(*p1, out_dtype=dt)
    torch.cuda.synchronize()
    for d, (oqw, oqz), Y in ((d0, (oqw0, oqz0), y0), (d1, (oqw1, oqz1), y1)):
        check(Y, oracle.linear(d["X"], oqw, d["scales"], oqz), "pair K=%d N=%d %s" % (K, N, ydt))
    assert torch.equal(y0, s0) and torch.equal(y1, s1)


# projections that read the same X at M = 1 (q, k and v of a decode step): one launch of
# the decode kernel, a run of workgroups per projection.  (K, [N, ...]): 20 groups (8
# columns per workgroup); 76 groups with every N a multiple of 1280 (5 columns) and with
# N a multiple of 4 only (4 columns); eight projections of one group, the last ragged;
# a single projection between empty entries
MULTI_ONE_X = [(2560, [4096, 1024, 1024]), (9728, [2560, 1280, 5120]), (9728, [2568, 1032]),
               (128, [8, 16, 24, 32, 40, 48, 56, 1000]), (640, [0, 520, 0])]


@pytest.mark.parametrize("j", range(len(MULTI_ONE_X)))
@pytest.mark.parametrize("ydt", ["f32", "bf16"])
def test_batch_multi_one_row(dev, j, ydt):
    K, Ns = MULTI_ONE_X[j]
    print("batch one X M=1", K, Ns, ydt, flush=True)
    dt = torch.float32 if ydt == "f32" else torch.bfloat16
    X = None
    probs, cases = [], []
    Xt = None
    for q, N in enumerate(Ns):
        d = synth.linear_inputs(700 + 13 * j + q, 1, max(N, 8), K)
        if X is None:
            X = d["X"]
            Xt = dev_inputs(d, dev)["X"]
        d = dict(d, X=X)
        if N == 0:
            pq = (Xt, torch.empty((0, K // 8), dtype=torch.int32, device=dev),
                  torch.empty((0, K // 128), dtype=torch.float16, device=dev),
                  torch.empty((0, K // 128), dtype=torch.int32, device=dev))
            oq = (None, None)
        else:
            pq, oq = _prep(d, dev)
            pq = (Xt,) + tuple(pq[1:])  # the same X tensor
        probs.append(pq)
        cases.append((N, d, oq))
    ys = w4.w4a16_linear_batch(probs, out_dtype=dt)
    singles = [w4.w4a16_linear(*pq, out_dtype=dt) if pq[1].shape[0] else None for pq in probs]
    torch.cuda.synchronize()
    for (N, d, (oqw, oqz)), Y, S in zip(cases, ys, singles):
        if N == 0:
            assert Y.shape == (1, 0)
            continue
        check(Y, oracle.linear(d["X"], oqw, d["scales"], oqz), "one X K=%d N=%d %s" % (K, N, ydt))
        assert torch.equal(Y, S)
