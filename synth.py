"""Seeded synthetic inputs for the W4A16 linear: shared by the tests and the bench.

This module holds none of the method's arithmetic: it only draws random codes,
zero-points, scales, activations and draft ids, and rounds the drawn float32
values to the storage formats (bf16 / fp16 bit patterns).  Packing, dequantizing
and contracting live in the oracle and in the HIP library, separately.

Recipe (one numpy PCG64 stream per tensor set, drawn in this order):
  codes  u8[N,K]    uniform integers in [0, 15]
  zeros  u8[N,K/G]  uniform integers in [0, 15]
  scales           uniform in [0.002, 0.02) as float32, stored as fp16 (round to nearest even)
  X                standard normal float32, stored as bf16 (round to nearest even), row-major [M,K]
The workloads follow the 4B-class shapes used in the pages' system (a Qwen3.5-4B
target; draft blocks of 16 tokens, from the Pith review's free parameters).
"""
import numpy as np

GROUP = 128

# name -> list of (label, M, K, N); seeds are 1000 + index, sub-seed + 10*j
WORKLOADS = {
    "single_512": [("linear", 1, 512, 512)],
    "decode_gemv_m1": [("gate_up", 1, 2560, 9728), ("down", 1, 9728, 2560)],
    "verify_block_m16": [("q", 16, 2560, 4096), ("k", 16, 2560, 1024), ("v", 16, 2560, 1024),
                         ("o", 16, 4096, 2560), ("gate", 16, 2560, 9728), ("up", 16, 2560, 9728),
                         ("down", 16, 9728, 2560)],
    "lmhead_verify_m16": [("lm_head", 16, 2560, 151936)],
    "prefill_m8192": [("gate_up", 8192, 2560, 9728), ("down", 8192, 9728, 2560)],
}
WORKLOAD_INDEX = {name: i for i, name in enumerate(WORKLOADS)}


def seed_for(workload, j=0):
    return 1000 + WORKLOAD_INDEX[workload] + 10 * j


def f32_to_bf16_bits(a):
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def f32_to_f16_bits(a):
    """Round float32 values to IEEE binary16 (numpy's cast: nearest, ties to even)."""
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def linear_inputs(seed, M, N, K, group=GROUP):
    """Random grid + activations for one linear of shape X[M,K] -> Y[M,N]."""
    rng = np.random.default_rng(seed)
    G = K // group
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    zeros = rng.integers(0, 16, size=(N, G), dtype=np.uint8)
    scales = f32_to_f16_bits(rng.uniform(0.002, 0.02, size=(N, G)).astype(np.float32))
    X = f32_to_bf16_bits(rng.standard_normal(size=(M, K), dtype=np.float32))
    return {"codes": codes, "zeros": zeros, "scales": scales, "X": X}


def requant_inputs(seed, N, K, group=GROUP):
    """Weights near a frozen grid, as after distillation: W = (q - z + e) * s with
    e ~ N(0, 0.5) (most weights land near their old code, some cross to a neighbour,
    the extremes fall off the 4-bit range), rounded to bfloat16; scales and zeros as
    in linear_inputs.  Returns W (bf16 bits), scales (fp16 bits), zeros u8."""
    rng = np.random.default_rng(seed)
    G = K // group
    codes = rng.integers(0, 16, size=(N, K)).astype(np.float32)
    zeros = rng.integers(0, 16, size=(N, G), dtype=np.uint8)
    scales = f32_to_f16_bits(rng.uniform(0.002, 0.02, size=(N, G)).astype(np.float32))
    s = np.repeat(scales.view(np.float16).astype(np.float32), group, axis=1)
    e = rng.normal(0.0, 0.5, size=(N, K)).astype(np.float32)
    W = (codes - np.repeat(zeros.astype(np.float32), group, axis=1) + e) * s
    return {"W": f32_to_bf16_bits(W), "scales": scales, "zeros": zeros}


def workload_inputs(workload, j, group=GROUP):
    label, M, K, N = WORKLOADS[workload][j]
    return linear_inputs(seed_for(workload, j), M, N, K, group)


def draft_block(seed, M, N):
    """Random draft ids uint in [0, N) and a forced-prefix length L0 in [0, M]."""
    rng = np.random.default_rng(seed + 7)
    draft = rng.integers(0, N, size=M).astype(np.int32)
    L0 = int(rng.integers(0, M + 1))
    return draft, L0, rng


def force_prefix(draft, L0, target_ids, rng, N):
    """Make the first L0 draft ids equal target_ids and the next one differ.

    target_ids is the greedy choice the expected output holds (computed by the
    caller); the result accepts exactly L0 tokens against it.  Redraws stay in
    [0, N); N must be at least 2 when L0 < len(draft)."""
    d = np.array(draft, dtype=np.int32, copy=True)
    M = d.shape[0]
    d[:L0] = target_ids[:L0]
    if L0 < M:
        while d[L0] == target_ids[L0]:
            d[L0] = int(rng.integers(0, N))
    return d


# ---------------------------------------------------------------- closed forms
# Inputs at the size limits (about 2^31 elements) are too large to draw on the host.
# They follow closed forms of their indices instead, evaluated on the device for the
# whole tensor and on the host for the rows or columns a test samples; every value
# is dyadic (integer activations, power-of-two scales), so any summation order of
# the layer gives the exact result.

def cf_x(rows, K):
    """bf16 bits of X[m, k] = ((7m + 13k + (m k mod 11)) mod 17) - 8 for m in rows."""
    m = np.asarray(rows, np.int64)[:, None]
    k = np.arange(K, dtype=np.int64)[None, :]
    v = (m * 7 + k * 13 + (m * k) % 11) % 17 - 8
    return f32_to_bf16_bits(v.astype(np.float32))


def cf_codes(cols, K):
    """codes[n, k] = (5n + 3k + (n k mod 7)) mod 16 for n in cols (uint8)."""
    n = np.asarray(cols, np.int64)[:, None]
    k = np.arange(K, dtype=np.int64)[None, :]
    return ((n * 5 + k * 3 + (n * k) % 7) % 16).astype(np.uint8)


def cf_zeros(cols, G):
    """zeros[n, g] = (3n + 5g) mod 16 (uint8)."""
    n = np.asarray(cols, np.int64)[:, None]
    g = np.arange(G, dtype=np.int64)[None, :]
    return ((n * 3 + g * 5) % 16).astype(np.uint8)


def cf_scales(cols, G):
    """fp16 bits of scales[n, g] = 2^-(6 + (n + g) mod 4)."""
    n = np.asarray(cols, np.int64)[:, None]
    g = np.arange(G, dtype=np.int64)[None, :]
    return f32_to_f16_bits(np.ldexp(1.0, -(6 + (n + g) % 4)).astype(np.float32))


def cf_x_torch(M, K, device, chunk=1 << 16):
    """cf_x for rows 0..M-1 on a torch device, as a bf16 tensor [M, K]."""
    import torch
    out = torch.empty((M, K), dtype=torch.bfloat16, device=device)
    k = torch.arange(K, dtype=torch.int64, device=device)[None, :]
    for r0 in range(0, M, chunk):
        m = torch.arange(r0, min(M, r0 + chunk), dtype=torch.int64, device=device)[:, None]
        out[r0:r0 + m.shape[0]] = ((m * 7 + k * 13 + (m * k) % 11) % 17 - 8).to(torch.bfloat16)
    return out


def cf_codes_torch(N, K, device, chunk=1 << 16):
    """cf_codes for columns 0..N-1 on a torch device, as uint8 [N, K]."""
    import torch
    out = torch.empty((N, K), dtype=torch.uint8, device=device)
    k = torch.arange(K, dtype=torch.int64, device=device)[None, :]
    for r0 in range(0, N, chunk):
        n = torch.arange(r0, min(N, r0 + chunk), dtype=torch.int64, device=device)[:, None]
        out[r0:r0 + n.shape[0]] = ((n * 5 + k * 3 + (n * k) % 7) % 16).to(torch.uint8)
    return out
