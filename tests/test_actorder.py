"""GPTQ act-order: the host permutation (CPU) and the packed/gathered path on the GPU
against the oracle's act-order definition (oracle_linear_gidx)."""
import numpy as np
import pytest

import int4_weight_only_02_amd as w4
import oracle
import synth


def _gidx(rng, K, group=128):
    order = rng.permutation(K)
    g = np.empty(K, np.int32)
    g[order] = np.arange(K) // group
    return g


def test_perm_is_the_stable_group_order():
    rng = np.random.default_rng(0)
    for K in (128, 384, 2560):
        g = _gidx(rng, K)
        perm = w4.w4a16_actorder_perm(g)
        assert (perm == np.argsort(g, kind="stable")).all()
        assert (g[perm] == np.arange(K) // 128).all()
    # sequential groups: the identity
    assert (w4.w4a16_actorder_perm(np.arange(512) // 128) == np.arange(512)).all()


def test_perm_rejects_bad_groups():
    with pytest.raises(w4.W4A16Error) as e:
        w4.w4a16_actorder_perm(np.zeros(256, np.int32))  # one group of 256
    assert e.value.status == 2
    g = np.arange(256) // 128
    g[5] = 2  # out of range
    with pytest.raises(w4.W4A16Error) as e:
        w4.w4a16_actorder_perm(g)
    assert e.value.status == 2
    with pytest.raises(w4.W4A16Error):
        w4.w4a16_actorder_perm(np.arange(200) // 128)  # K not a multiple of the group


def _prep(dev, seed, M, N, K, symmetric=False):
    import torch
    rng = np.random.default_rng(seed)
    d = synth.linear_inputs(seed, M, N, K)
    if symmetric:
        d["zeros"][:] = 8
    g = _gidx(rng, K)
    perm = w4.w4a16_actorder_perm(g)
    pdev = torch.from_numpy(perm).to(dev)
    qw, qz = w4.w4a16_pack_actorder(torch.from_numpy(d["codes"]).to(dev), torch.from_numpy(d["zeros"]).to(dev),
                                    pdev)
    X = torch.from_numpy(d["X"].view(np.int16)).to(dev).view(torch.bfloat16)
    S = torch.from_numpy(d["scales"].view(np.int16)).to(dev).view(torch.float16)
    return d, g, perm, pdev, qw, qz, X, S


@pytest.mark.gpu
def test_pack_actorder_is_pack_of_permuted_codes():
    import torch
    dev = torch.device("cuda:0")
    d, g, perm, pdev, qw, qz, X, S = _prep(dev, 5, 1, 136, 1280)
    want_w, want_z = oracle.pack(np.ascontiguousarray(d["codes"][:, perm]), d["zeros"])
    assert (qw.cpu().numpy().view(np.uint32) == want_w).all()
    assert (qz.cpu().numpy().view(np.uint32) == want_z).all()


@pytest.mark.gpu
# M = 1 (gathered inside the M = 1 kernel up to 40 groups, else by a separate launch),
# 2 <= M <= 16 and M > 16 (a gather launch, then the plain kernels: odd group counts,
# row counts below 16, K split across workgroups at K = 9728)
@pytest.mark.parametrize("M,N,K,sym", [(1, 520, 1280, False), (1, 136, 128, True), (1, 9728, 2560, False),
                                       (1, 2560, 9728, True), (1, 264, 6272, False), (2, 264, 384, True),
                                       (5, 264, 2560, True), (7, 520, 1408, False), (16, 1032, 2560, False),
                                       (16, 9728, 2560, False), (16, 2560, 4096, True), (12, 136, 6016, False),
                                       (16, 264, 9728, False), (70, 264, 1280, True)])
def test_linear_actorder_matches_oracle(M, N, K, sym):
    import torch
    dev = torch.device("cuda:0")
    print("actorder", M, N, K, sym, flush=True)
    d, g, perm, pdev, qw, qz, X, S = _prep(dev, 7 + M + N, M, N, K, sym)
    Y = w4.w4a16_linear_actorder(X, pdev, qw, S, qz, out_dtype=torch.float32)
    torch.cuda.synchronize()
    oqw, oqz = oracle.pack(d["codes"], d["zeros"])
    Yo = oracle.linear_gidx(d["X"], oqw, d["scales"], oqz, g)
    tol = 1e-2 * float(np.sqrt((Yo ** 2).mean()))
    err = float(np.abs(Y.cpu().numpy().astype(np.float64) - Yo).max())
    assert err <= tol, (err, tol)
    # the same layer without act-order would be a different function (with one group,
    # the order of k inside it does not matter)
    if K // 128 > 1:
        Yplain = oracle.linear(d["X"], oqw, d["scales"], oqz)
        assert float(np.abs(Yplain - Yo).max()) > 10 * tol


@pytest.mark.gpu
@pytest.mark.parametrize("M,N,K", [(16, 264, 2560), (3, 136, 4096), (1, 264, 2560), (1, 136, 9728)])
def test_linear_actorder_dyadic_exact(M, N, K):
    # integer X and power-of-two scales: exact on both sides, whatever the order of k
    import torch
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(9 + M + K)
    G = K // 128
    codes = rng.integers(0, 16, (N, K)).astype(np.uint8)
    zeros = rng.integers(0, 16, (N, G)).astype(np.uint8)
    scales = (2.0 ** -rng.integers(3, 9, (N, G))).astype(np.float16).view(np.uint16)
    Xf = rng.integers(-8, 9, (M, K)).astype(np.float32)
    Xb = (Xf.view(np.uint32) >> 16).astype(np.uint16)
    g = _gidx(rng, K)
    perm = w4.w4a16_actorder_perm(g)
    pdev = torch.from_numpy(perm).to(dev)
    qw, qz = w4.w4a16_pack_actorder(torch.from_numpy(codes).to(dev), torch.from_numpy(zeros).to(dev), pdev)
    X = torch.from_numpy(Xb.view(np.int16)).to(dev).view(torch.bfloat16)
    S = torch.from_numpy(scales.view(np.int16)).to(dev).view(torch.float16)
    Y = w4.w4a16_linear_actorder(X, pdev, qw, S, qz, out_dtype=torch.float32)
    torch.cuda.synchronize()
    oqw, oqz = oracle.pack(codes, zeros)
    Yo = oracle.linear_gidx(Xb, oqw, scales, oqz, g)
    assert (Y.cpu().numpy().astype(np.float64) == Yo).all()


@pytest.mark.gpu
def test_actorder_leaves_the_zero_region_alone():
    # the gathered X goes after the linear call's scratch and never over the counters:
    # a chunked call (K split across workgroups) on the same workspace afterwards must
    # give what it gives on a fresh one
    import torch
    dev = torch.device("cuda:0")
    ws = w4.Workspace(dev)
    for M in (1, 3, 16):
        d, g, perm, pdev, qw, qz, X, S = _prep(dev, 40 + M, M, 136, 2560)
        w4.w4a16_linear_actorder(X, pdev, qw, S, qz, workspace=ws)
    d = synth.linear_inputs(77, 16, 264, 9728)
    qw, qz = w4.w4a16_pack(torch.from_numpy(d["codes"]).to(dev), torch.from_numpy(d["zeros"]).to(dev))
    X = torch.from_numpy(d["X"].view(np.int16)).to(dev).view(torch.bfloat16)
    S = torch.from_numpy(d["scales"].view(np.int16)).to(dev).view(torch.float16)
    Y1 = w4.w4a16_linear(X, qw, S, qz, out_dtype=torch.float32, workspace=ws)
    Y2 = w4.w4a16_linear(X, qw, S, qz, out_dtype=torch.float32, workspace=w4.Workspace(dev))
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)
