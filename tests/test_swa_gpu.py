"""GPU parity of w4a16_swa_attention (causal sliding-window attention of a query block)
and w4a16_swa_attention_block (bidirectional within the block) with the fp64 oracle.
Bound: |dO| <= 1e-2 * rms(O_oracle) on fp32 output (bf16 output adds half an ulp);
the softmax weights enter the value product as a bf16 pair (about 2^-17 relative), so
the kernel is held to a fifth of that bound, also for peaked softmax rows."""
import numpy as np
import pytest
import torch

import int4_weight_only_02_amd as w4
import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _bits(a):
    return synth.f32_to_bf16_bits(np.asarray(a, np.float32))


def _inputs(seed, M, T, Hq, Hkv, pad_nan=True):
    rng = np.random.default_rng(seed)
    D = 128
    Q = _bits(rng.normal(0, 1, (M, Hq, D)))
    K = _bits(rng.normal(0, 1, (T, Hkv, D)))
    Vt = _bits(rng.normal(0, 1, (Hkv, D, T)))
    ts = (T + 7) // 8 * 8 + 8  # padded rows: the padding must never be read into O
    Vp = np.full((Hkv, D, ts), 0x7FC0 if pad_nan else 0, np.uint16)  # bf16 NaN
    Vp[:, :, :T] = Vt
    return Q, K, Vt, Vp


def _run(dev, Q, K, Vp, T, window, dtype=torch.float32, block=False):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    O = w4.w4a16_swa_attention(t(Q), t(K), t(Vp), T, window, out_dtype=dtype, block=block)
    torch.cuda.synchronize()
    return O


@pytest.mark.parametrize("M,T,Hq,Hkv,W", [(16, 8192, 32, 8, 1024), (16, 8192, 32, 8, 2048), (1, 300, 4, 1, 64),
                                          (5, 77, 8, 2, 1000), (16, 16, 2, 2, 4), (3, 2049, 16, 1, 2048),
                                          (16, 1000, 8, 8, 1), (2, 5000, 4, 2, 3500), (4, 8192, 2, 1, 6000)])
def test_swa_matches_oracle(dev, M, T, Hq, Hkv, W):
    print("swa", M, T, Hq, Hkv, W, flush=True)
    Q, K, Vt, Vp = _inputs(M * 7 + T + W, M, T, Hq, Hkv)
    Oo = oracle.swa(Q, K, Vt, W)
    O = _run(dev, Q, K, Vp, T, W).cpu().numpy().astype(np.float64)
    tol = 1e-2 * float(np.sqrt((Oo ** 2).mean()))
    err = np.abs(O - Oo)
    assert np.isfinite(O).all()
    assert err.max() <= 0.2 * tol, (float(err.max()), tol)


def test_swa_bf16_output(dev):
    M, T, Hq, Hkv, W = 16, 4096, 16, 4, 1024
    Q, K, Vt, Vp = _inputs(5, M, T, Hq, Hkv)
    Oo = oracle.swa(Q, K, Vt, W)
    O = _run(dev, Q, K, Vp, T, W, torch.bfloat16).float().cpu().numpy().astype(np.float64)
    tol = 1e-2 * float(np.sqrt((Oo ** 2).mean()))
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(Oo), 1e-30))) - 7)
    assert (np.abs(O - Oo) <= tol + 0.5 * ulp).all()


def test_swa_window_of_one_is_own_value(dev):
    # one key per query: weight exactly 1, O = V of the query's own position (exact)
    M, T, Hq, Hkv = 16, 200, 4, 2
    Q, K, Vt, Vp = _inputs(9, M, T, Hq, Hkv)
    O = _run(dev, Q, K, Vp, T, 1).cpu().numpy()
    V = (Vt.astype(np.uint32) << 16).view(np.float32)
    for i in range(M):
        for h in range(Hq):
            assert (O[i, h] == V[h // 2, :, T - M + i]).all()


def test_swa_deterministic_and_errors(dev):
    M, T, Hq, Hkv, W = 16, 3000, 8, 2, 2048
    Q, K, Vt, Vp = _inputs(11, M, T, Hq, Hkv)
    O1 = _run(dev, Q, K, Vp, T, W)
    O2 = _run(dev, Q, K, Vp, T, W)
    assert torch.equal(O1, O2)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    with pytest.raises(w4.W4A16Error) as e:  # more than 16 queries
        w4.w4a16_swa_attention(t(np.zeros((17, 8, 128), np.uint16)), t(K), t(Vp), T, W)
    assert e.value.status == 2
    with pytest.raises(w4.W4A16Error) as e:  # head dim 64
        w4.w4a16_swa_attention(t(np.zeros((16, 8, 64), np.uint16)), t(K[:, :, :64]), t(Vp[:, :64]), T, W)
    assert e.value.status == 4


SHAPES_BLOCK = [(16, 8192, 32, 8, 1024), (16, 8192, 32, 8, 2048), (1, 300, 4, 1, 64), (5, 77, 8, 2, 1000),
                (16, 16, 2, 2, 4), (3, 2049, 16, 1, 2048), (16, 1000, 8, 8, 1), (4, 8192, 2, 1, 6000)]


@pytest.mark.parametrize("M,T,Hq,Hkv,W", SHAPES_BLOCK)
def test_swa_block_matches_oracle(dev, M, T, Hq, Hkv, W):
    print("swa block", M, T, Hq, Hkv, W, flush=True)
    Q, K, Vt, Vp = _inputs(M * 11 + T + W, M, T, Hq, Hkv)
    Oo = oracle.swa_block(Q, K, Vt, W)
    O = _run(dev, Q, K, Vp, T, W, block=True).cpu().numpy().astype(np.float64)
    tol = 1e-2 * float(np.sqrt((Oo ** 2).mean()))
    assert np.isfinite(O).all()
    assert np.abs(O - Oo).max() <= 0.2 * tol, (float(np.abs(O - Oo).max()), tol)


@pytest.mark.parametrize("block", [False, True])
def test_swa_peaked_softmax(dev, block):
    # queries scaled by 8: scores of tens of units, each row's weights concentrated on
    # a few keys (the softmax weights' own rounding dominates the error there)
    M, T, Hq, Hkv, W = 16, 4096, 8, 2, 1024
    rng = np.random.default_rng(99)
    Q = _bits(8.0 * rng.normal(0, 1, (M, Hq, 128)))
    K = _bits(rng.normal(0, 1, (T, Hkv, 128)))
    Vt = _bits(rng.normal(0, 1, (Hkv, 128, T)))
    Oo = (oracle.swa_block if block else oracle.swa)(Q, K, Vt, W)
    O = _run(dev, Q, K, Vt, T, W, block=block).cpu().numpy().astype(np.float64)
    tol = 1e-2 * float(np.sqrt((Oo ** 2).mean()))
    assert np.abs(O - Oo).max() <= 0.2 * tol, (float(np.abs(O - Oo).max()), tol)


def test_swa_block_bf16_output(dev):
    M, T, Hq, Hkv, W = 16, 4096, 16, 4, 1024
    Q, K, Vt, Vp = _inputs(6, M, T, Hq, Hkv)
    Oo = oracle.swa_block(Q, K, Vt, W)
    O = _run(dev, Q, K, Vp, T, W, torch.bfloat16, block=True).float().cpu().numpy().astype(np.float64)
    tol = 1e-2 * float(np.sqrt((Oo ** 2).mean()))
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(Oo), 1e-30))) - 7)
    assert (np.abs(O - Oo) <= tol + 0.5 * ulp).all()
