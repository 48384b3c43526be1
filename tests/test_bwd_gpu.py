"""GPU parity of attn_bwd against the fp64 oracle's backward.

The oracle recomputes P from Q and K on its own; the GPU uses the forward's
saved O and LSE (both produced by attn_fwd on the same inputs).
"""

import math
import sys

import numpy as np
import pytest
import torch

from exact_attention_05_amd import attn_bwd, attn_fwd
from exact_attention_05_amd.inputs import make_head, make_tensor, widen
from oracle import ref_bwd

from helpers import assert_bar

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inputs(seed, B, H, N, d, device="cpu"):
    return [make_tensor(seed, n, B, H, N, d, torch.bfloat16, device=device) for n in ("q", "k", "v", "do")]


def _gpu_bwd(q, k, v, dO, scale, causal, want_lse=False):
    q, k, v, dO = (t.to(DEV) for t in (q, k, v, dO))
    o, lse = attn_fwd(q, k, v, scale=scale, causal=causal)
    dq, dk, dv, ws = attn_bwd(q, k, v, o, dO, lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    if want_lse:
        return dq, dk, dv, ws, o, lse
    return dq, dk, dv, ws, o


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 64, 100, 129, 200, 300, 555, 1100])
def test_bwd_ragged(N, d, causal):
    """Every gradient against the oracle; the longer lengths span 2-5 key
    and query workgroups of both passes with a ragged last one."""
    _say(f"bwd N={N} d={d} causal={causal}")
    q, k, v, dO = _inputs(N + d, 1, 2, N, d)
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv, ws, o, lse = _gpu_bwd(q, k, v, dO, scale, causal, want_lse=True)
    Q, K, V, DO = (widen(t) for t in (q, k, v, dO))
    dQ, dK, dV = ref_bwd(Q, K, V, DO, scale, causal)
    assert_bar("dV", widen(dv), dV, torch.bfloat16)
    assert_bar("dK", widen(dk), dK, torch.bfloat16)
    assert_bar("dQ", widen(dq), dQ, torch.bfloat16)
    # workspace: D = rowsum(dO o O) from the saved O, then -LSE*log2(e), then
    # -D and -LSE*log2(e)/(scale*log2(e)) as three bf16 parts (and a zero)
    # whose sums are the values to ~fp32 precision
    D = (DO * widen(o)).sum(-1)
    rows = D.size
    w = ws.cpu()
    np.testing.assert_allclose(widen(w[:rows]).reshape(D.shape), D, rtol=1e-4, atol=1e-4)
    np.testing.assert_allclose(widen(w[rows:2 * rows]).reshape(D.shape), -widen(lse.cpu()) * math.log2(math.e),
                               rtol=1e-6, atol=1e-6)
    parts = widen(w[2 * rows:4 * rows].contiguous().view(torch.bfloat16).reshape(rows, 4))
    Dk = widen(w[:rows])
    np.testing.assert_allclose(parts[:, :3].sum(-1), -Dk, rtol=1e-6, atol=1e-30)
    assert np.all(parts[:, 3] == 0)
    lparts = widen(w[4 * rows:6 * rows].contiguous().view(torch.bfloat16).reshape(rows, 4))
    nl2 = widen(w[rows:2 * rows])
    np.testing.assert_allclose(lparts[:, :3].sum(-1), nl2 / (scale * math.log2(math.e)), rtol=1e-6, atol=1e-30)
    assert np.all(lparts[:, 3] == 0)


@pytest.mark.parametrize("d,scale", [(64, 0.3), (64, 0.02), (128, 0.05), (128, 0.3)])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_other_scales(d, scale, causal):
    """Softmax scales other than 1/sqrt(d) (the scale enters the exponent, the
    -LSE split and the final scaling of dK and dQ): every gradient against
    the oracle at N = 300 (two key workgroups, ragged).  Q and K are drawn
    with standard deviation (scale sqrt(d))^(-1/2), so the scaled scores
    spread as at the default scale and the gradients keep the magnitudes at
    which the absolute bf16 bar applies (P and dS enter the gradient products
    in bf16, so the error grows with the gradients)."""
    N = 300
    _say(f"bwd d={d} scale={scale} causal={causal}")
    seed = N + d + 7
    sd = (scale * math.sqrt(d)) ** -0.5
    q, k = (make_tensor(seed, n, 1, 2, N, d, torch.bfloat16, sd) for n in ("q", "k"))
    v, dO = (make_tensor(seed, n, 1, 2, N, d, torch.bfloat16) for n in ("v", "do"))
    dq, dk, dv, _, _ = _gpu_bwd(q, k, v, dO, scale, causal)
    Q, K, V, DO = (widen(t) for t in (q, k, v, dO))
    dQ, dK, dV = ref_bwd(Q, K, V, DO, scale, causal)
    assert_bar("dV", widen(dv), dV, torch.bfloat16)
    assert_bar("dK", widen(dk), dK, torch.bfloat16)
    assert_bar("dQ", widen(dq), dQ, torch.bfloat16)


def test_bwd_invariants():
    """sum_j dK_j = 0 (rows of dS sum to zero); Q = 0 gives dK = 0."""
    _say("bwd invariants")
    N, d = 300, 64
    q, k, v, dO = _inputs(77, 1, 2, N, d)
    for causal in (False, True):
        dq, dk, dv, _, _ = _gpu_bwd(q, k, v, dO, 0.125, causal)
        s = widen(dk).sum(axis=2)
        assert np.max(np.abs(s)) <= 0.05, np.max(np.abs(s))
        dq, dk, dv, _, _ = _gpu_bwd(torch.zeros_like(q), k, v, dO, 0.125, causal)
        assert torch.count_nonzero(dk) == 0


def test_bwd_deterministic():
    _say("bwd determinism")
    q, k, v, dO = _inputs(5, 1, 3, 777, 64)
    a = _gpu_bwd(q, k, v, dO, 0.125, True)
    b = _gpu_bwd(q, k, v, dO, 0.125, True)
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)


def test_bwd_causal_workload_sampled():
    """bf16 Q, K, V, dO [B=2, H=16, N=4096, d=64] ~ N(0, 1), causal, scale
    1/8: every gradient of sampled heads against the oracle."""
    B, H, N, d = 2, 16, 4096, 64
    _say(f"bwd workload [{B},{H},{N},{d}] causal")
    seed = 0
    q, k, v, dO = _inputs(seed, B, H, N, d, device=DEV)
    scale = 1.0 / math.sqrt(d)
    o, lse = attn_fwd(q, k, v, scale=scale, causal=True)
    dq, dk, dv, _ = attn_bwd(q, k, v, o, dO, lse, scale=scale, causal=True)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    for b, h in ((0, 0), (1, 15)):
        Q, K, V, DO = (widen(make_head(seed, n, b, h, N, d, torch.bfloat16)) for n in ("q", "k", "v", "do"))
        dQ, dK, dV = ref_bwd(Q, K, V, DO, scale, True)
        assert_bar(f"dV[{b},{h}]", widen(dv[b, h]), dV, torch.bfloat16)
        assert_bar(f"dK[{b},{h}]", widen(dk[b, h]), dK, torch.bfloat16)
        assert_bar(f"dQ[{b},{h}]", widen(dq[b, h]), dQ, torch.bfloat16)


def test_bwd_offsets_beyond_2gib():
    """Q, K, V, dO [1, H, 256, 64] bf16 spanning more than 2^31 bytes each:
    the first and last heads hold seeded data and are checked against the
    oracle (causal), the others are zero and get zero gradients."""
    N, d = 256, 64
    H = (1 << 31) // (N * d * 2) + 16
    _say(f"bwd offsets beyond 2 GiB: [1,{H},{N},{d}]")
    seed = 8
    q, k, v, dO = (torch.zeros((1, H, N, d), dtype=torch.bfloat16, device=DEV) for _ in range(4))
    for h in (0, H - 1):
        for t, n in ((q, "q"), (k, "k"), (v, "v"), (dO, "do")):
            t[0, h].copy_(make_head(seed, n, 0, h, N, d, torch.bfloat16))
    scale = 0.125
    o, lse = attn_fwd(q, k, v, scale=scale, causal=True)
    dq, dk, dv, _ = attn_bwd(q, k, v, o, dO, lse, scale=scale, causal=True)
    torch.cuda.synchronize()
    for h in (0, H - 1):
        Q, K, V, DO = (widen(make_head(seed, n, 0, h, N, d, torch.bfloat16)) for n in ("q", "k", "v", "do"))
        dQ, dK, dV = ref_bwd(Q[None, None], K[None, None], V[None, None], DO[None, None], scale, True)
        assert_bar(f"dQ[{h}]", widen(dq[0, h]), dQ[0, 0], torch.bfloat16)
        assert_bar(f"dK[{h}]", widen(dk[0, h]), dK[0, 0], torch.bfloat16)
        assert_bar(f"dV[{h}]", widen(dv[0, h]), dV[0, 0], torch.bfloat16)
    mid = H // 2
    for t in (dq, dk, dv):
        assert torch.count_nonzero(t[0, mid]) == 0
