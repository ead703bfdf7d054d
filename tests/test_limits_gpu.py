"""GPU parity at the size limits of the boundary: M*K (the large-M path, X of almost
4 GiB) and N*K (the small-M path, a packed grid of 1 GiB) at 2^31 - 256 elements or
just below, where every byte offset of the kernels' 32-bit buffer addressing is in
use.  Inputs follow the dyadic closed forms of synth (integer activations, power-of-
two scales), so the sampled outputs must equal the oracle's bit for bit, whatever the
summation order."""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
w4 = pytest.importorskip("int4_weight_only_02_amd")

pytestmark = pytest.mark.gpu

LIMIT = 2 ** 31 - 256


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    w4.lib()
    return torch.device("cuda:0")


def _grid(cols, K):
    G = K // 128
    return synth.cf_codes(cols, K), synth.cf_zeros(cols, G), synth.cf_scales(cols, G)


def test_large_m_at_the_mk_limit(dev):
    M, N, K = 1048575, 256, 2048  # M*K = 2^31 - 2048: 4096 tiles of the prefill stream plan
    assert M * K <= LIMIT
    print("limit M*K", M, N, K, flush=True)
    cols = np.arange(N)
    codes, zeros, scales = _grid(cols, K)
    qw, qz = w4.w4a16_pack(torch.from_numpy(codes).to(dev), torch.from_numpy(zeros).to(dev))
    S = torch.from_numpy(scales.view(np.int16)).to(dev).view(torch.float16)
    X = synth.cf_x_torch(M, K, dev)
    Y = w4.w4a16_linear(X, qw, S, qz, out_dtype=torch.float32)
    torch.cuda.synchronize()
    del X
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, M - 256, M - 2, M - 1], rng.integers(0, M, 250)]))
    oqw, oqz = oracle.pack(codes, zeros)
    Yo = oracle.linear(synth.cf_x(rows, K), oqw, scales, oqz)  # [len(rows), N]
    got = Y[torch.from_numpy(rows).to(dev)].cpu().numpy().astype(np.float64)
    assert (got == Yo).all(), "max |dY| %g" % np.abs(got - Yo).max()


@pytest.mark.parametrize("M", [16, 1])
def test_small_m_at_the_nk_limit(dev, M):
    # 838856 columns: a 1 GiB packed grid; M = 16 runs the small-M kernel's stream plan
    # (persistent workgroups over 52429 tiles), M = 1 the decode kernel (104857
    # workgroups of 8 columns); the lm_head call below runs the stream plan too
    K = 2560
    N = (LIMIT // K) // 8 * 8
    print("limit N*K", M, N, K, flush=True)
    codes = synth.cf_codes_torch(N, K, dev)
    zeros = torch.from_numpy(synth.cf_zeros(np.arange(N), K // 128)).to(dev)
    qw, qz = w4.w4a16_pack(codes, zeros)
    del codes
    scales = synth.cf_scales(np.arange(N), K // 128)
    S = torch.from_numpy(scales.view(np.int16)).to(dev).view(torch.float16)
    xh = synth.cf_x(np.arange(M), K)
    X = torch.from_numpy(xh.view(np.int16)).to(dev).view(torch.bfloat16)
    Y = w4.w4a16_linear(X, qw, S, qz, out_dtype=torch.float32)
    torch.cuda.synchronize()
    # whole blocks of 8 columns (one packed zero word each), the first and the last included
    rng = np.random.default_rng(6)
    blocks = np.unique(np.concatenate([[0, N // 8 - 1], rng.integers(0, N // 8, 30)]))
    cols = (blocks[:, None] * 8 + np.arange(8)[None, :]).ravel()
    c, z, s = _grid(cols, K)
    oqw, oqz = oracle.pack(c, z)
    Yo = oracle.linear(xh, oqw, s, oqz)  # [M, len(cols)]
    got = Y[:, torch.from_numpy(cols).to(dev)].cpu().numpy().astype(np.float64)
    assert (got == Yo).all(), "max |dY| %g" % np.abs(got - Yo).max()
    # the same grid through the fused lm_head: its fp32 logits are exact too, so they
    # equal the linear's bit for bit; its argmax is the lowest column holding the
    # row's maximum, and the accepted prefix follows from it
    draft = torch.zeros(M, dtype=torch.int32, device=dev)
    am, acc, L = w4.w4a16_lmhead_verify(X, qw, S, qz, draft, return_logits=True, logits_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(L, Y)
    assert torch.equal(am, torch.argmax(Y, dim=1).to(torch.int32))
    a = am.cpu().numpy()
    assert int(acc.cpu()[0]) == next((i for i in range(M) if a[i] != 0), M)
