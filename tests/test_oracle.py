"""Pins for the fp64 CPU oracle, against facts that do not come from the oracle.

Each pin is chosen so that a plausible mistake in the oracle fails it:
  decode pins      bf16/fp16 bit patterns with textbook values and the library casts
  layout goldens   hand-worked packed words (nibble order along K, zeros along N)
  one-hot X        Y picks one weight: catches a transposed operand, a wrong group
                   index, a wrong zero/scale lookup, a sign error
  equal codes      closed form s*(c - z)*rowsum(X) per group: catches a dropped zero
                   term or scale
  dyadic exact     integer X and power-of-two scales: Y is exact, checked with
                   Python integers
  plain matmul     z = 0, s = 1 reduces to X @ codes^T (numpy)
  brute force      exact rationals on tiny shapes
  by hand          a one-group example worked out on paper
  permutation      permuting weight rows permutes Y columns bit-exactly
  verify goldens   hand-worked argmax / accepted-prefix cases, ties to the lowest id
  statistics       rms(Y) of the synthetic workloads against its closed form
  act-order        GPTQ column groups (g_idx): sequential g_idx is the plain oracle bit
                   for bit; one-hot X picks (q - z[g_idx[k]]) * s[g_idx[k]]; permuting
                   the columns (X, codes and g_idx together) leaves dyadic Y unchanged
  attention        a window of one gives V of the query's own position exactly; equal
                   keys give the window mean of V; an independent numpy formulation
                   (masked score matrix, library softmax) agrees on small shapes
  re-quantization  hand-worked round-to-grid cases (ties to even, clamping, overflow);
                   on-grid weights come back as their own codes; agreement with exact
                   rational rounding everywhere, ties and their neighbours included
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _f16(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def _bf16(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- decoders

def test_bf16_decode_textbook_values():
    cases = {0x3F80: 1.0, 0xC000: -2.0, 0x4049: 3.140625, 0x0000: 0.0, 0x8000: -0.0,
             0x0001: 2.0 ** -133, 0x0080: 2.0 ** -126, 0x7F7F: (2 - 2 ** -7) * 2.0 ** 127,
             0x4300: 128.0, 0x430F: 143.0}
    for bits, v in cases.items():
        assert oracle.bf16_to_f64(bits) == v, hex(bits)


def test_f16_decode_textbook_values():
    cases = {0x3C00: 1.0, 0xC000: -2.0, 0x0001: 2.0 ** -24, 0x03FF: 1023 * 2.0 ** -24,
             0x0400: 2.0 ** -14, 0x7BFF: 65504.0, 0x3555: 0.333251953125, 0x1C00: 2.0 ** -8}
    for bits, v in cases.items():
        assert oracle.f16_to_f64(bits) == v, hex(bits)
    assert math.isinf(oracle.f16_to_f64(0x7C00)) and math.isnan(oracle.f16_to_f64(0x7E00))


def test_decoders_match_library_casts_on_all_patterns():
    # fp16 through numpy's binary16, bf16 through numpy's binary32 view
    rng = np.random.default_rng(5)
    for bits in list(rng.integers(0, 65536, 3000)) + [0, 1, 0x3FF, 0x400, 0x7BFF, 0x8001]:
        f = _f16(bits)
        if not np.isnan(f):
            assert oracle.f16_to_f64(bits) == f
        b = _bf16(bits)
        if not np.isnan(b):
            assert oracle.bf16_to_f64(bits) == b


# ---------------------------------------------------------------- packing

def _read_pack_golden():
    qw, qz = {}, {}
    with open(os.path.join(GOLDEN, "pack_layout.txt")) as f:
        for line in f:
            line = line.split("#")[0].split()
            if not line:
                continue
            kind, a, b, v = line[0], int(line[1]), int(line[2]), int(line[3], 16)
            (qw if kind == "qweight" else qz)[(a, b)] = v
    return qw, qz


def test_pack_layout_golden():
    N, K = 8, 128
    n = np.arange(N)[:, None]
    k = np.arange(K)[None, :]
    codes = ((n + k) % 16).astype(np.uint8)
    zeros = ((np.arange(N) + 1) % 16).astype(np.uint8)[:, None]
    qweight, qzeros = oracle.pack(codes, zeros)
    gw, gz = _read_pack_golden()
    assert gw and gz
    for (r, w), v in gw.items():
        assert int(qweight[r, w]) == v, (r, w, hex(int(qweight[r, w])), hex(v))
    for (r, g), v in gz.items():
        assert int(qzeros[r, g]) == v


@pytest.mark.parametrize("N,K", [(8, 128), (24, 384), (64, 1024)])
def test_pack_roundtrip_and_masking(N, K):
    rng = np.random.default_rng(N + K)
    codes = rng.integers(0, 256, size=(N, K), dtype=np.uint8)  # high bits must be ignored
    zeros = rng.integers(0, 256, size=(N, K // 128), dtype=np.uint8)
    qw, qz = oracle.pack(codes, zeros)
    c2, z2 = oracle.unpack(qw, qz, N, K)
    assert (c2 == (codes & 15)).all() and (z2 == (zeros & 15)).all()
    qw2, qz2 = oracle.pack(codes & 15, zeros & 15)
    assert (qw2 == qw).all() and (qz2 == qz).all()


# ---------------------------------------------------------------- the linear

def _rand_grid(rng, N, K):
    G = K // 128
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    zeros = rng.integers(0, 16, size=(N, G), dtype=np.uint8)
    scales = synth.f32_to_f16_bits(rng.uniform(0.002, 0.02, size=(N, G)).astype(np.float32))
    return codes, zeros, scales


def test_linear_worked_by_hand():
    N, K = 8, 128
    n = np.arange(N)[:, None]
    k = np.arange(K)[None, :]
    codes = ((n + k) % 16).astype(np.uint8)
    zeros = np.arange(N, dtype=np.uint8)[:, None]
    scales = synth.f32_to_f16_bits((2.0 ** -np.arange(N, dtype=np.float32))[:, None])
    X = np.zeros((1, K), np.float32)
    X[0, 0], X[0, 1], X[0, 127] = 1.0, 2.0, -1.0
    qw, qz = oracle.pack(codes, zeros)
    Y = oracle.linear(synth.f32_to_bf16_bits(X), qw, scales, qz)
    expect = {}
    with open(os.path.join(GOLDEN, "linear_by_hand.txt")) as f:
        for line in f:
            line = line.split("#")[0].split()
            if line:
                expect[int(line[0])] = float(line[1])
    assert len(expect) == N
    for col, v in expect.items():
        assert Y[0, col] == v


def test_onehot_picks_one_weight():
    rng = np.random.default_rng(11)
    N, K = 40, 512
    codes, zeros, scales = _rand_grid(rng, N, K)
    ks = np.array([0, 1, 7, 8, 127, 128, 200, 255, 256, 383, 384, 511])
    X = np.zeros((len(ks), K), np.float32)
    X[np.arange(len(ks)), ks] = 1.0
    qw, qz = oracle.pack(codes, zeros)
    Y = oracle.linear(synth.f32_to_bf16_bits(X), qw, scales, qz)
    s = _f16(scales)
    for m, kk in enumerate(ks):
        g = kk // 128
        expect = (codes[:, kk].astype(np.float64) - zeros[:, g]) * s[:, g]
        assert (Y[m] == expect).all(), (m, kk)


def test_equal_codes_closed_form():
    # codes all equal c: Y[m,n] = sum_g s[n,g] * (c - z[n,g]) * sum_{k in g} X[m,k]
    rng = np.random.default_rng(12)
    N, K, M = 16, 640, 3
    G = K // 128
    for c in (0, 9, 15):
        codes = np.full((N, K), c, np.uint8)
        zeros = rng.integers(0, 16, size=(N, G), dtype=np.uint8)
        scales = synth.f32_to_f16_bits(rng.uniform(0.002, 0.02, size=(N, G)).astype(np.float32))
        Xb = synth.f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
        qw, qz = oracle.pack(codes, zeros)
        Y = oracle.linear(Xb, qw, scales, qz)
        x = _bf16(Xb)
        s = _f16(scales)
        for m in range(M):
            S = [math.fsum(x[m, 128 * g:128 * (g + 1)]) for g in range(G)]
            for n in range(N):
                ex = math.fsum(s[n, g] * (c - int(zeros[n, g])) * S[g] for g in range(G))
                assert abs(Y[m, n] - ex) <= 1e-12 * (1 + abs(ex))
        # c == z everywhere: exactly zero
        qw, qz = oracle.pack(codes, np.full((N, G), c, np.uint8))
        assert (oracle.linear(Xb, qw, scales, qz) == 0).all()


def test_dyadic_inputs_exact():
    # X integers in [-8, 8], s = 2^-e: every product is a multiple of 2^-9 and fp64 is exact.
    rng = np.random.default_rng(13)
    M, N, K = 3, 24, 384
    G = K // 128
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    zeros = rng.integers(0, 16, size=(N, G), dtype=np.uint8)
    e = rng.integers(6, 10, size=(N, G))
    scales = synth.f32_to_f16_bits((2.0 ** -e).astype(np.float32))
    Xi = rng.integers(-8, 9, size=(M, K))
    qw, qz = oracle.pack(codes, zeros)
    Y = oracle.linear(synth.f32_to_bf16_bits(Xi.astype(np.float32)), qw, scales, qz)
    for m in range(M):
        for n in range(N):
            tot = 0  # in units of 2^-9
            for kk in range(K):
                g = kk // 128
                tot += int(Xi[m, kk]) * (int(codes[n, kk]) - int(zeros[n, g])) * (1 << (9 - int(e[n, g])))
            assert Y[m, n] == tot / 512.0


def test_reduces_to_plain_matmul():
    # zero-points 0 and scales 1.0: Y = X @ codes^T
    rng = np.random.default_rng(14)
    M, N, K = 4, 32, 768
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    zeros = np.zeros((N, K // 128), np.uint8)
    scales = np.full((N, K // 128), 0x3C00, np.uint16)
    Xb = synth.f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    qw, qz = oracle.pack(codes, zeros)
    Y = oracle.linear(Xb, qw, scales, qz)
    ref = _bf16(Xb) @ codes.T.astype(np.float64)
    assert np.allclose(Y, ref, rtol=1e-13, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_exact_rationals(seed):
    rng = np.random.default_rng(100 + seed)
    M, N, K = 2, 16, 256
    G = K // 128
    codes, zeros, scales = _rand_grid(rng, N, K)
    Xb = synth.f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    qw, qz = oracle.pack(codes, zeros)
    Y = oracle.linear(Xb, qw, scales, qz)
    x = _bf16(Xb)
    s = _f16(scales)
    for m in range(M):
        for n in range(N):
            exact = Fraction(0)
            mag = 0.0
            for kk in range(K):
                g = kk // 128
                t = Fraction(float(x[m, kk])) * (int(codes[n, kk]) - int(zeros[n, g])) * Fraction(float(s[n, g]))
                exact += t
                mag += abs(float(t))
            assert abs(Fraction(float(Y[m, n])) - exact) <= Fraction(1e-12) * Fraction(mag)


def test_weight_row_permutation_permutes_columns():
    rng = np.random.default_rng(15)
    M, N, K = 5, 48, 384
    codes, zeros, scales = _rand_grid(rng, N, K)
    Xb = synth.f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    perm = rng.permutation(N)
    qw, qz = oracle.pack(codes, zeros)
    qwp, qzp = oracle.pack(codes[perm], zeros[perm])
    Y = oracle.linear(Xb, qw, scales, qz)
    Yp = oracle.linear(Xb, qwp, scales[perm], qzp)
    assert (Yp == Y[:, perm]).all()
    rp = rng.permutation(M)
    assert (oracle.linear(Xb[rp], qw, scales, qz) == Y[rp]).all()


def test_linear_at_is_the_same_definition():
    d = synth.linear_inputs(21, 3, 64, 512)
    qw, qz = oracle.pack(d["codes"], d["zeros"])
    Y = oracle.linear(d["X"], qw, d["scales"], qz)
    rng = np.random.default_rng(0)
    rows = rng.integers(0, 3, 50)
    cols = rng.integers(0, 64, 50)
    assert (oracle.linear_at(d["X"], qw, d["scales"], qz, rows, cols) == Y[rows, cols]).all()


# ---------------------------------------------------------------- verification

def _read_verify_cases():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "verify_cases.txt")) as f:
        for line in f:
            t = line.split("#")[0].split()
            if not t:
                continue
            if t[0] == "case":
                cur = {"name": t[1], "rows": []}
                cases.append(cur)
            elif t[0] == "row":
                cur["rows"].append([float(v) for v in t[1:]])
            elif t[0] == "draft":
                cur["draft"] = [int(v) for v in t[1:]]
            elif t[0] == "expect_argmax":
                cur["argmax"] = [int(v) for v in t[1:]]
            elif t[0] == "expect_accept":
                cur["accept"] = int(t[1])
    return cases


def test_verify_golden_cases():
    cases = _read_verify_cases()
    assert len(cases) == 4
    for c in cases:
        am, gap, L = oracle.argmax_accept(np.array(c["rows"]), np.array(c["draft"]))
        assert list(am) == c["argmax"], c["name"]
        assert L == c["accept"], c["name"]
        for r, row in enumerate(c["rows"]):
            srt = sorted(row, reverse=True)
            assert gap[r] == srt[0] - srt[1]


def test_forced_prefix_gives_exact_accept_length():
    rng = np.random.default_rng(3)
    M, N = 16, 1000
    Y = rng.standard_normal((M, N))
    am, _, _ = oracle.argmax_accept(Y, np.zeros(M, np.int32))
    for L0 in (0, 1, 7, 15, 16):
        draft, _, r2 = synth.draft_block(L0, M, N)
        d = synth.force_prefix(draft, L0, am, r2, N)
        assert oracle.argmax_accept(Y, d)[2] == L0


# ---------------------------------------------------------------- generator

@pytest.mark.parametrize("K", [512, 2560])
def test_generator_rms_matches_closed_form(K):
    # E[s^2] for s ~ U[0.002, 0.02) and E[(q-z)^2] = 2 * Var(U{0..15}) = 42.5
    es2 = (0.02 ** 3 - 0.002 ** 3) / (3 * 0.018)
    expect = math.sqrt(K * es2 * 42.5)
    d = synth.linear_inputs(31, 8, 512, K)
    qw, qz = oracle.pack(d["codes"], d["zeros"])
    Y = oracle.linear(d["X"], qw, d["scales"], qz)
    rms = float(np.sqrt((Y ** 2).mean()))
    assert abs(rms / expect - 1) < 0.06, (rms, expect)
    assert (d["codes"] < 16).all() and (d["zeros"] < 16).all()
    s = _f16(d["scales"])
    assert s.min() >= 0.002 - 1e-6 and s.max() <= 0.02 + 1e-5


def test_matmul_variant_matches_naive_oracle():
    d = synth.linear_inputs(41, 5, 96, 1280)
    qw, qz = oracle.pack(d["codes"], d["zeros"])
    Y = oracle.linear(d["X"], qw, d["scales"], qz)
    Ym = oracle.linear_matmul(d["X"], qw, d["scales"], qz)
    assert np.allclose(Ym, Y, rtol=1e-12, atol=1e-12 * float(np.abs(Y).max()))
    # dyadic inputs: both are exact
    rng = np.random.default_rng(42)
    Xi = rng.integers(-8, 9, size=(4, 1280)).astype(np.float32)
    sc = synth.f32_to_f16_bits((2.0 ** -rng.integers(6, 10, size=(96, 10))).astype(np.float32))
    Xb = synth.f32_to_bf16_bits(Xi)
    assert (oracle.linear_matmul(Xb, qw, sc, qz) == oracle.linear(Xb, qw, sc, qz)).all()


def test_dequantize_matches_onehot_linear():
    d = synth.linear_inputs(43, 1, 64, 384)
    qw, qz = oracle.pack(d["codes"], d["zeros"])
    W = oracle.dequantize(qw, qz, d["scales"], 64, 384)
    eye = synth.f32_to_bf16_bits(np.eye(384, dtype=np.float32))
    assert (oracle.linear(eye, qw, d["scales"], qz) == W.T).all()


# ------------------------------------------------------------------ re-quantization


def _read_quantize_cases():
    rows = []
    with open(os.path.join(GOLDEN, "quantize_cases.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                w, sc, z, q = line.split()
                rows.append((int(w, 16), int(sc, 16), int(z), int(q)))
    return rows


def test_quantize_worked_by_hand():
    cases = _read_quantize_cases()
    assert len(cases) >= 12
    # one group of 128 per case (the case's weight repeated), so the group index matters
    W = np.array([[w] * 128 for w, _, _, _ in cases], np.uint16)
    S = np.array([[sc] for _, sc, _, _ in cases], np.uint16)
    Z = np.array([[z] for _, _, z, _ in cases], np.uint8)
    codes = oracle.quantize(W, S, Z)
    for i, (_, _, _, q) in enumerate(cases):
        assert (codes[i] == q).all(), (i, cases[i], codes[i, 0])


def _bf16_rne(x):
    """fp64 -> bfloat16 bits, round to nearest even (via fp32; the values here are
    far from fp32 rounding boundaries)."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("seed", [0, 1])
def test_quantize_returns_on_grid_weights_to_their_codes(seed):
    # W = (q - z) * s rounded to bfloat16 is within 2^-9 |W| <= 0.03 s of the grid
    # point, so rounding W / s back gives q - z exactly: every code must come back
    rng = np.random.default_rng(seed)
    N, K, G = 16, 512, 4
    q = rng.integers(0, 16, (N, K)).astype(np.uint8)
    z = rng.integers(0, 16, (N, G)).astype(np.uint8)
    s = rng.uniform(0.002, 0.02, (N, G)).astype(np.float16)
    Wf = (q.astype(np.float64) - np.repeat(z, 128, axis=1)) * np.repeat(s.astype(np.float64), 128, axis=1)
    codes = oracle.quantize(_bf16_rne(Wf), s.view(np.uint16), z)
    assert (codes == q).all()


def test_quantize_matches_exact_rational_rounding():
    # exact W / s (Fractions), round half to even (Python's round on a Fraction), + z,
    # clamp: the oracle must agree on every weight, near-ties included
    rng = np.random.default_rng(7)
    N, K, G = 8, 256, 2
    s = rng.uniform(0.002, 0.02, (N, G)).astype(np.float16)
    z = rng.integers(0, 16, (N, G)).astype(np.uint8)
    Wf = rng.normal(0.0, 1.0, (N, K)) * np.repeat(s.astype(np.float64), 128, axis=1) * 6.0
    Wb = _bf16_rne(Wf)
    # plus exact ties and values one bfloat16 step either side of them
    for i in range(64):
        n, g = i % N, (i // N) % G
        t = Fraction(int(rng.integers(-12, 12)) * 2 + 1, 2) * Fraction(float(s[n, g]))
        tb = _bf16_rne(np.array([float(t)]))[0]
        Wb[n, g * 128 + i] = (int(tb) + int(rng.integers(-1, 2))) & 0xFFFF
    codes = oracle.quantize(Wb, s.view(np.uint16), z)
    w_exact = (Wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for n in range(N):
        for k in range(K):
            g = k // 128
            x = Fraction(float(w_exact[n, k])) / Fraction(float(s[n, g]))
            want = min(15, max(0, round(x) + int(z[n, g])))
            assert codes[n, k] == want, (n, k, float(x), codes[n, k], want)


# ------------------------------------------------------------------ GPTQ act-order


def _actorder_gidx(rng, K, group=128):
    """GPTQ act-order groups: columns in a random order, consecutive blocks of `group`
    of that order share a group."""
    order = rng.permutation(K)
    g_idx = np.empty(K, np.int32)
    g_idx[order] = np.arange(K) // group
    return g_idx


def test_gidx_sequential_is_the_plain_oracle():
    d = synth.linear_inputs(21, 5, 24, 384)
    qw, qz = oracle.pack(d["codes"], d["zeros"])
    g_idx = (np.arange(384) // 128).astype(np.int32)
    Y1 = oracle.linear(d["X"], qw, d["scales"], qz)
    Y2 = oracle.linear_gidx(d["X"], qw, d["scales"], qz, g_idx)
    assert (Y1 == Y2).all()


def test_gidx_onehot_picks_its_group():
    rng = np.random.default_rng(3)
    N, K = 16, 512
    d = synth.linear_inputs(22, 1, N, K)
    g_idx = _actorder_gidx(rng, K)
    qw, qz = oracle.pack(d["codes"], d["zeros"])
    ks = [0, 1, 127, 128, 300, 511]
    X = np.zeros((len(ks), K), np.uint16)
    for m, k in enumerate(ks):
        X[m, k] = 0x3F80  # bf16 1.0
    Y = oracle.linear_gidx(X, qw, d["scales"], qz, g_idx)
    s = d["scales"].view(np.float16).astype(np.float64)
    for m, k in enumerate(ks):
        g = g_idx[k]
        want = (d["codes"][:, k].astype(np.float64) - d["zeros"][:, g]) * s[:, g]
        assert (Y[m] == want).all(), (m, k, g)


def test_gidx_column_permutation_invariance():
    # dyadic X and power-of-two scales: Y is exact, so permuting the columns of X, the
    # codes and g_idx together must give the same Y bit for bit
    rng = np.random.default_rng(4)
    M, N, K = 3, 8, 256
    codes = rng.integers(0, 16, (N, K)).astype(np.uint8)
    zeros = rng.integers(0, 16, (N, 2)).astype(np.uint8)
    scales = (2.0 ** -rng.integers(3, 8, (N, 2))).astype(np.float16).view(np.uint16)
    Xf = rng.integers(-8, 9, (M, K)).astype(np.float32)
    X = (Xf.view(np.uint32) >> 16).astype(np.uint16)
    g_idx = _actorder_gidx(rng, K)
    p = rng.permutation(K)
    qw, qz = oracle.pack(codes, zeros)
    qwp, _ = oracle.pack(codes[:, p], zeros)
    Y1 = oracle.linear_gidx(X, qw, scales, qz, g_idx)
    Y2 = oracle.linear_gidx(np.ascontiguousarray(X[:, p]), qwp, scales, qz, np.ascontiguousarray(g_idx[p]))
    assert (Y1 == Y2).all()
    # and a grouping other than the sequential one changes the result
    Y3 = oracle.linear(X, qw, scales, qz)
    assert not (Y1 == Y3).all()


# ------------------------------------------------------------------ sliding-window attention


def _bf16_bits(a):
    return _bf16_rne(np.asarray(a, np.float64))


def _bits_to_f64(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _swa_inputs(rng, M, T, Hq, Hkv, D):
    Q = _bf16_bits(rng.normal(0, 1, (M, Hq, D)))
    K = _bf16_bits(rng.normal(0, 1, (T, Hkv, D)))
    Vt = _bf16_bits(rng.normal(0, 1, (Hkv, D, T)))
    return Q, K, Vt


def test_swa_window_of_one_returns_own_value():
    rng = np.random.default_rng(0)
    M, T, Hq, Hkv, D = 4, 40, 4, 2, 16
    Q, K, Vt = _swa_inputs(rng, M, T, Hq, Hkv, D)
    O = oracle.swa(Q, K, Vt, 1)
    V = _bits_to_f64(Vt)
    for i in range(M):
        for h in range(Hq):
            assert (O[i, h] == V[h // 2, :, T - M + i]).all()


def test_swa_equal_keys_give_the_window_mean():
    rng = np.random.default_rng(1)
    M, T, Hq, Hkv, D, W = 3, 50, 2, 1, 8, 7
    Q, K, Vt = _swa_inputs(rng, M, T, Hq, Hkv, D)
    K[:] = K[0]  # every key the same: uniform weights over the window
    O = oracle.swa(Q, K, Vt, W)
    V = _bits_to_f64(Vt)
    for i in range(M):
        p = T - M + i
        want = V[0, :, p - W + 1:p + 1].mean(axis=1)
        assert np.abs(O[i, 0] - want).max() < 1e-12


@pytest.mark.parametrize("W", [1, 5, 64, 1000])
def test_swa_matches_masked_softmax_formulation(W):
    rng = np.random.default_rng(2 + W)
    M, T, Hq, Hkv, D = 5, 70, 6, 2, 32
    Q, K, Vt = _swa_inputs(rng, M, T, Hq, Hkv, D)
    O = oracle.swa(Q, K, Vt, W)
    q, k, v = _bits_to_f64(Q), _bits_to_f64(K), _bits_to_f64(Vt)
    pos = np.arange(T - M, T)
    j = np.arange(T)
    mask = (j[None, :] <= pos[:, None]) & (j[None, :] > pos[:, None] - W)  # [M, T]
    for h in range(Hq):
        kv = h // (Hq // Hkv)
        s = q[:, h, :] @ k[:, kv, :].T / np.sqrt(D)  # [M, T]
        s = np.where(mask, s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        want = p @ v[kv].T  # [M, D]
        assert np.abs(O[:, h, :] - want).max() < 1e-12


# ---- attention bidirectional within the block (oracle_swa_block) -----------------

def test_swa_block_single_query_is_causal():
    # a block of one token has no later key: the bidirectional mode is the causal one
    rng = np.random.default_rng(11)
    M, T, Hq, Hkv, D = 1, 60, 4, 2, 16
    Q, K, Vt = _swa_inputs(rng, M, T, Hq, Hkv, D)
    for W in (1, 7, 100):
        assert np.array_equal(oracle.swa_block(Q, K, Vt, W), oracle.swa(Q, K, Vt, W))


def test_swa_block_equal_keys_give_the_mean_over_context_window_and_block():
    # every key the same: uniform weights over the context keys in the window and all
    # M keys of the block
    rng = np.random.default_rng(12)
    M, T, Hq, Hkv, D, W = 4, 50, 2, 1, 8, 7
    Q, K, Vt = _swa_inputs(rng, M, T, Hq, Hkv, D)
    K[:] = K[0]
    O = oracle.swa_block(Q, K, Vt, W)
    V = _bits_to_f64(Vt)
    for i in range(M):
        p = T - M + i
        lo = max(0, p - W + 1)
        want = V[0, :, lo:T].mean(axis=1)
        assert np.abs(O[i, 0] - want).max() < 1e-12


def test_swa_block_is_invariant_to_permuting_the_block():
    # every query sees every key of the block, so reordering the block's keys and values
    # together changes no output (the causal mode would)
    rng = np.random.default_rng(13)
    M, T, Hq, Hkv, D, W = 6, 40, 4, 2, 16, 9
    Q, K, Vt = _swa_inputs(rng, M, T, Hq, Hkv, D)
    perm = np.arange(T)
    perm[T - M:] = T - M + rng.permutation(M)
    O1 = oracle.swa_block(Q, K, Vt, W)
    O2 = oracle.swa_block(Q, K[perm], Vt[:, :, perm], W)
    assert np.abs(O1 - O2).max() < 1e-12
    assert np.abs(oracle.swa(Q, K, Vt, W) - oracle.swa(Q, K[perm], Vt[:, :, perm], W)).max() > 1e-6


@pytest.mark.parametrize("W", [1, 3, 64, 1000])
def test_swa_block_matches_masked_softmax_formulation(W):
    rng = np.random.default_rng(20 + W)
    M, T, Hq, Hkv, D = 5, 70, 6, 2, 32
    Q, K, Vt = _swa_inputs(rng, M, T, Hq, Hkv, D)
    O = oracle.swa_block(Q, K, Vt, W)
    q, k, v = _bits_to_f64(Q), _bits_to_f64(K), _bits_to_f64(Vt)
    pos = np.arange(T - M, T)
    j = np.arange(T)
    in_block = j[None, :] >= T - M
    mask = in_block | (j[None, :] > pos[:, None] - W)  # [M, T]
    for h in range(Hq):
        kv = h // (Hq // Hkv)
        s = q[:, h, :] @ k[:, kv, :].T / np.sqrt(D)
        s = np.where(mask, s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        assert np.abs(O[:, h, :] - p @ v[kv].T).max() < 1e-12


# ---- gated MLP activation (oracle_silu_mul, gated) ----------------------------

def test_silu_closed_forms():
    # sigmoid(ln 3) = 3/4 and sigmoid(-ln 3) = 1/4; silu(0) = 0; silu(g) -> g for large g
    ln3 = np.log(3.0)
    Y = oracle.silu_mul(np.array([0.0, ln3, -ln3, 40.0, -40.0]), np.ones(5))
    assert Y[0] == 0.0
    assert abs(Y[1] - 0.75 * ln3) <= 1e-15
    assert abs(Y[2] + 0.25 * ln3) <= 1e-15
    assert abs(Y[3] - 40.0) <= 1e-12
    assert abs(Y[4] - (-40.0 * np.exp(-40.0))) <= 1e-25


def test_silu_odd_part_identity():
    # silu(g) - silu(-g) = g (sigmoid(g) + sigmoid(-g) = 1), and the product is linear in U
    rng = np.random.default_rng(71)
    g = rng.normal(0, 3, 1000)
    u = rng.normal(0, 1, 1000)
    d = oracle.silu_mul(g, np.ones_like(g)) - oracle.silu_mul(-g, np.ones_like(g))
    assert np.abs(d - g).max() <= 1e-12
    assert np.abs(oracle.silu_mul(g, u) - oracle.silu_mul(g, np.ones_like(g)) * u).max() <= 1e-12


def test_gated_applies_silu_to_the_gate_and_scales_by_up():
    # one-hot X on k = 0 with s = 1: gate column n gives q - z = 2, up gives -3, so
    # Y = silu(2) * (-3) = -6 / (1 + e^-2) (swapping gate and up would give 2 silu(-3))
    N, K = 16, 128
    X = np.zeros((1, K), np.float32)
    X[0, 0] = 1.0
    Xb = synth.f32_to_bf16_bits(X)
    s = synth.f32_to_f16_bits(np.ones((N, 1), np.float32))
    z = np.full((N, 1), 8, np.uint8)
    cg = np.full((N, K), 8, np.uint8)
    cg[:, 0] = 10
    cu = np.full((N, K), 8, np.uint8)
    cu[:, 0] = 5
    qg, zg = oracle.pack(cg, z)
    qu, zu = oracle.pack(cu, z)
    Y = oracle.gated(Xb, (qg, s, zg), (qu, s, zu))
    assert np.abs(Y - (-6.0 / (1.0 + np.exp(-2.0)))).max() <= 1e-15
