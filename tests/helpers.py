"""Comparison helpers for the GPU-vs-oracle parity tests.

The pass bars are the stated tolerances: max |error| <= 1e-5 for fp32
inputs, <= 2e-2 for bf16 inputs, and <= 1e-3 for the LSE, always against the
fp64 oracle evaluated on the same (already rounded) inputs.  A second,
relative bar max|err| / max|ref| <= 2^-6 keeps the check meaningful for
outputs whose magnitude is far below 2e-2.
"""

import numpy as np
import torch

BAR = {torch.float32: 1e-5, torch.bfloat16: 2e-2}
LSE_BAR = 1e-3
REL_BAR = 2.0 ** -6


def report(name, got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    mx = float(err.max()) if err.size else 0.0
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    return mx, (mx / scale if scale > 0 else mx)


def assert_bar(name, got, ref, dtype, rel=True):
    """Element-wise comparison of a GPU output with the oracle at the stated bar."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    mx, rl = report(name, got, ref)
    bar = BAR[dtype]
    assert mx <= bar, f"{name}: max abs err {mx:.3e} > {bar:.1e} (rel {rl:.3e})"
    if rel and dtype == torch.bfloat16:
        assert rl <= REL_BAR, f"{name}: max rel err {rl:.3e} > {REL_BAR:.3e}"
    return mx, rl


def assert_lse(name, got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{name}: finiteness differs"
    mx = float(np.abs(got[fin] - ref[fin]).max()) if fin.any() else 0.0
    assert mx <= LSE_BAR, f"{name}: LSE max abs err {mx:.3e} > {LSE_BAR:.1e}"
    return mx
