"""GPU parity of attn_bwd_atomic_dq (dQ accumulated by fp32 atomic adds in
the dK/dV pass) against the fp64 oracle's backward, and against attn_bwd.

The atomic adds make the order of dQ's fp32 sums depend on timing, so dq is
compared to the bar only; dK and dV do not go through atomics and repeat
bit for bit.
"""

import math
import sys

import pytest
import torch

from exact_attention_05_amd import attn_bwd, attn_bwd_atomic_dq, attn_fwd
from exact_attention_05_amd.inputs import make_head, make_tensor, widen
from oracle import ref_bwd

from helpers import assert_bar

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inputs(seed, B, H, N, d, device=DEV):
    return [make_tensor(seed, n, B, H, N, d, torch.bfloat16, device=device) for n in ("q", "k", "v", "do")]


def _both(q, k, v, dO, scale, causal):
    o, lse = attn_fwd(q, k, v, scale=scale, causal=causal)
    at = attn_bwd_atomic_dq(q, k, v, o, dO, lse, scale=scale, causal=causal)
    ref = attn_bwd(q, k, v, o, dO, lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return at, ref


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N", [(1, 2, 1), (1, 2, 17), (1, 2, 64), (2, 3, 100), (1, 2, 129), (1, 2, 300)])
def test_bwd_atomic_ragged(B, H, N, d, causal):
    """Ragged lengths: a single row, a partial key block of the workgroup
    (keys past N must add nothing to dQ), exact tiles, several workgroups."""
    _say(f"bwd atomic B={B} H={H} N={N} d={d} causal={causal}")
    seed = 500 + N + d
    q, k, v, dO = _inputs(seed, B, H, N, d)
    scale = 1.0 / math.sqrt(d)
    (dq, dk, dv, ws), (dq2, dk2, dv2, _) = _both(q, k, v, dO, scale, causal)
    dQ, dK, dV = ref_bwd(*(widen(t.cpu()) for t in (q, k, v, dO)), scale, causal)
    assert_bar("dQ", widen(dq), dQ, torch.bfloat16)
    assert_bar("dK", widen(dk), dK, torch.bfloat16)
    assert_bar("dV", widen(dv), dV, torch.bfloat16)
    # the two backwards agree to the same bar
    assert_bar("dQ vs attn_bwd", widen(dq), widen(dq2), torch.bfloat16)
    if d == 128:
        # same dK/dV kernel and summation order as attn_bwd at d = 128
        assert torch.equal(dk, dk2) and torch.equal(dv, dv2)


@pytest.mark.parametrize("d,scale", [(64, 0.3), (128, 0.05)])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_atomic_other_scales(d, scale, causal):
    """A softmax scale other than 1/sqrt(d) (it enters the exponent, the -LSE
    split and the final scaling of dK and of the accumulated dQ), with Q and
    K drawn so that the scaled scores spread as at the default scale."""
    N = 300
    _say(f"bwd atomic d={d} scale={scale} causal={causal}")
    seed = 700 + d
    sd = (scale * math.sqrt(d)) ** -0.5
    q, k = (make_tensor(seed, n, 1, 2, N, d, torch.bfloat16, sd, device=DEV) for n in ("q", "k"))
    v, dO = (make_tensor(seed, n, 1, 2, N, d, torch.bfloat16, device=DEV) for n in ("v", "do"))
    (dq, dk, dv, _), _ = _both(q, k, v, dO, scale, causal)
    dQ, dK, dV = ref_bwd(*(widen(t.cpu()) for t in (q, k, v, dO)), scale, causal)
    assert_bar("dQ", widen(dq), dQ, torch.bfloat16)
    assert_bar("dK", widen(dk), dK, torch.bfloat16)
    assert_bar("dV", widen(dv), dV, torch.bfloat16)


def test_bwd_atomic_repeats():
    """dK and dV repeat bit for bit; dQ to the bar."""
    _say("bwd atomic repeat")
    q, k, v, dO = _inputs(6, 1, 3, 777, 64)
    o, lse = attn_fwd(q, k, v, scale=0.125, causal=True)
    a = attn_bwd_atomic_dq(q, k, v, o, dO, lse, scale=0.125, causal=True)
    a = tuple(t.clone() for t in a[:3])
    b = attn_bwd_atomic_dq(q, k, v, o, dO, lse, scale=0.125, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    assert_bar("dQ repeat", widen(a[0]), widen(b[0]), torch.bfloat16)


def test_bwd_atomic_zero_queries():
    """Q = 0: dK = scale dS^T Q is exactly 0, and the atomic dQ (nonzero:
    dS = P o (dP - D) with uniform P) still matches the oracle."""
    _say("bwd atomic Q = 0")
    q, k, v, dO = _inputs(12, 1, 2, 200, 64)
    q.zero_()
    (dq, dk, dv, _), _ = _both(q, k, v, dO, 0.125, False)
    assert torch.count_nonzero(dk) == 0
    dQ, _, _ = ref_bwd(*(widen(t.cpu()) for t in (q, k, v, dO)), 0.125, False)
    assert_bar("dQ", widen(dq), dQ, torch.bfloat16)


def test_bwd_atomic_causal_workload_sampled():
    """bf16 Q, K, V, dO [B=2, H=16, N=4096, d=64] ~ N(0, 1), causal, scale
    1/8: every gradient of sampled heads against the oracle."""
    B, H, N, d = 2, 16, 4096, 64
    _say(f"bwd atomic workload [{B},{H},{N},{d}] causal")
    seed = 0
    q, k, v, dO = _inputs(seed, B, H, N, d)
    scale = 1.0 / math.sqrt(d)
    o, lse = attn_fwd(q, k, v, scale=scale, causal=True)
    dq, dk, dv, _ = attn_bwd_atomic_dq(q, k, v, o, dO, lse, scale=scale, causal=True)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    for b, h in ((0, 3), (1, 12)):
        Q, K, V, DO = (widen(make_head(seed, n, b, h, N, d, torch.bfloat16)) for n in ("q", "k", "v", "do"))
        dQ, dK, dV = ref_bwd(Q, K, V, DO, scale, True)
        assert_bar(f"dQ[{b},{h}]", widen(dq[b, h]), dQ, torch.bfloat16)
        assert_bar(f"dK[{b},{h}]", widen(dk[b, h]), dK, torch.bfloat16)
        assert_bar(f"dV[{b},{h}]", widen(dv[b, h]), dV, torch.bfloat16)


def test_bwd_atomic_offsets_beyond_2gib():
    """Q, K, V, dO [1, H, 256, 64] bf16 spanning more than 2^31 bytes each
    (the fp32 dQ accumulator more than 2^32): the first and last heads hold
    seeded data and are checked against the oracle (causal), the others are
    zero and get zero gradients."""
    N, d = 256, 64
    H = (1 << 31) // (N * d * 2) + 16
    _say(f"bwd atomic offsets beyond 2 GiB: [1,{H},{N},{d}]")
    seed = 9
    q, k, v, dO = (torch.zeros((1, H, N, d), dtype=torch.bfloat16, device=DEV) for _ in range(4))
    for h in (0, H - 1):
        for t, n in ((q, "q"), (k, "k"), (v, "v"), (dO, "do")):
            t[0, h].copy_(make_head(seed, n, 0, h, N, d, torch.bfloat16))
    scale = 0.125
    o, lse = attn_fwd(q, k, v, scale=scale, causal=True)
    dq, dk, dv, _ = attn_bwd_atomic_dq(q, k, v, o, dO, lse, scale=scale, causal=True)
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
