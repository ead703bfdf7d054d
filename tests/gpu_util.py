"""Helpers for the GPU parity tests: move synthetic inputs to the device, compare
device results with the oracle under the accuracy contract.

Contract (from the layer's accuracy requirement, fp32 accumulation):
  fp32 output:  max |Y - Y_oracle| <= 1e-2 * rms(Y_oracle)
  bf16 output:  |Y - Y_oracle| <= 1e-2 * rms(Y_oracle) + half a bf16 ulp of Y_oracle,
                elementwise (a bf16 result cannot be closer than its own rounding)
  argmax:       equal to the oracle's wherever the oracle's top-2 gap exceeds
                1e-2 * rms(Y_oracle); elsewhere the chosen logit is within that
                tolerance of the maximum.
  gated pair:   y = silu(g) * u of two projections, each held to the contract above
                (|dg| <= eg = 1e-2 rms(G), |du| <= eu = 1e-2 rms(U)), carried through
                to first order with |silu'| <= 1.1, plus the product term:
                |dy| <= 1.1 |u| eg + |silu(g)| eu + 1.1 eg eu (+ half a bf16 ulp of y
                on bf16 output).
"""
import numpy as np

import synth

TOL_REL = 1e-2


def dev_inputs(d, device):
    import torch
    out = {
        "codes": torch.from_numpy(d["codes"]).to(device),
        "zeros": torch.from_numpy(d["zeros"]).to(device),
        "X": torch.from_numpy(d["X"].view(np.int16)).to(device).view(torch.bfloat16),
        "scales": torch.from_numpy(d["scales"].view(np.int16)).to(device).view(torch.float16),
    }
    return out


def bf16_bits_to_f64(bits):
    return (np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def y_to_f64(Y):
    import torch
    if Y.dtype == torch.float32:
        return Y.cpu().numpy().astype(np.float64)
    return bf16_bits_to_f64(Y.view(torch.int16).cpu().numpy().view(np.uint16))


def tol_of(Yo):
    return TOL_REL * float(np.sqrt(np.mean(Yo * Yo))) if Yo.size else 0.0


def half_ulp_bf16(Yo):
    a = np.abs(Yo)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126)
    return np.where(a > 0, np.ldexp(1.0, (e - 8).astype(np.int64)), 2.0 ** -134)


def check(Y, Yo, what=""):
    """Assert the accuracy contract; return max |dY| / tol."""
    import torch
    y = y_to_f64(Y)
    tol = tol_of(Yo)
    err = np.abs(y - Yo)
    if Y.dtype == torch.float32:
        bound = tol
    else:
        bound = tol + half_ulp_bf16(Yo)
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d outputs outside the bound, e.g. %s: got %s want %s (tol %g)" % (
            what, int(bad.sum()), idx.tolist(), y[tuple(idx[0])], Yo[tuple(idx[0])], tol))
    return float(err.max() / tol) if tol > 0 else 0.0


def gated_bound(G, U):
    """Elementwise bound of silu(G) * U given the contract on each projection."""
    G = np.asarray(G, np.float64)
    U = np.asarray(U, np.float64)
    eg = TOL_REL * float(np.sqrt(np.mean(G * G))) if G.size else 0.0
    eu = TOL_REL * float(np.sqrt(np.mean(U * U))) if U.size else 0.0
    sg = G / (1.0 + np.exp(-G))
    return 1.1 * np.abs(U) * eg + np.abs(sg) * eu + 1.1 * eg * eu


def check_gated(Y, G, U, Yo, what=""):
    """Assert the gated bound (Yo = silu(G) * U from the oracle); return max |dY| / bound."""
    import torch
    y = y_to_f64(Y)
    bound = gated_bound(G, U)
    if Y.dtype != torch.float32:
        bound = bound + half_ulp_bf16(Yo)
    err = np.abs(y - Yo)
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d outputs outside the bound, e.g. %s: got %s want %s (bound %g)" % (
            what, int(bad.sum()), idx.tolist(), y[tuple(idx[0])], Yo[tuple(idx[0])], bound[tuple(idx[0])]))
    return float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0


def expected_bf16_bits(Yo_exact):
    """bf16 bits of an fp64 result that is exactly representable in fp32."""
    f = Yo_exact.astype(np.float32)
    assert (f.astype(np.float64) == Yo_exact).all()
    return synth.f32_to_bf16_bits(f)
