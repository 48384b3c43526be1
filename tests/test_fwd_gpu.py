"""GPU parity of attn_fwd against the fp64 oracle (called through the C ABI).

Small cases compare every element; the full-size workloads compare sampled
heads and rows that the oracle evaluates on their own, plus properties that
hold at any size.
"""

import math
import sys

import numpy as np
import pytest
import torch

from exact_attention_05_amd import attn_fwd
from exact_attention_05_amd.inputs import make_head, make_tensor, widen, worked_example_qkv
from oracle import ref_fwd

from helpers import assert_bar, assert_lse

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inputs(seed, B, H, N, d, dtype, input_scale=1.0):
    return [make_tensor(seed, n, B, H, N, d, dtype, input_scale) for n in ("q", "k", "v")]


def _run(q, k, v, scale, causal):
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    o, lse = attn_fwd(qd, kd, vd, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return widen(o), widen(lse)


@pytest.mark.parametrize("scale,qmul", [(1.0, 1.0), (0.125, 8.0)])
def test_worked_example(scale, qmul):
    """The 4-token example of the cnblogs tiling article (section 2): scores
    S_11 = [[10, 20], [10, 10]], S_12 = [[30, 5], [5, 5]]; V = I, so O rows are
    the probability rows."""
    _say(f"worked example scale={scale}")
    q, k, v = worked_example_qkv(64, torch.bfloat16)
    q = (q.float() * qmul).to(torch.bfloat16)
    o, lse = _run(q, k, v, scale, False)
    O, LSE = ref_fwd(widen(q), widen(k), widen(v), scale, False)
    assert_bar("O", o, O, torch.bfloat16)
    assert_lse("LSE", lse, LSE)
    # row 0 puts almost all weight on key 2 (score 30); row 1 splits between keys 0 and 1
    assert o[0, 0, 0, 2] > 0.99 and abs(o[0, 0, 1, 0] - 0.4966535745378575) < 4e-3


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 4, 17, 64, 100, 129, 300, 555, 1100])
def test_bf16_ragged(N, d, causal):
    _say(f"bf16 N={N} d={d} causal={causal}")
    q, k, v = _inputs(N * 7 + d, 2, 3, N, d, torch.bfloat16)
    scale = 1.0 / math.sqrt(d)
    o, lse = _run(q, k, v, scale, causal)
    O, LSE = ref_fwd(widen(q), widen(k), widen(v), scale, causal)
    assert_bar("O", o, O, torch.bfloat16)
    assert_lse("LSE", lse, LSE)


@pytest.mark.parametrize("d,scale", [(64, 0.3), (64, 0.02), (128, 0.05), (128, 0.4)])
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_other_scales(d, scale, causal):
    """Softmax scales other than 1/sqrt(d) (folded into the exponent's base-2
    factor): O and LSE against the oracle at N = 300."""
    N = 300
    _say(f"bf16 d={d} scale={scale} causal={causal}")
    q, k, v = _inputs(N + 3 * d, 2, 3, N, d, torch.bfloat16)
    o, lse = _run(q, k, v, scale, causal)
    O, LSE = ref_fwd(widen(q), widen(k), widen(v), scale, causal)
    assert_bar("O", o, O, torch.bfloat16)
    assert_lse("LSE", lse, LSE)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 31, 256, 300])
def test_f32(N, causal):
    _say(f"f32 N={N} causal={causal}")
    q, k, v = _inputs(11 + N, 1, 2, N, 64, torch.float32)
    o, lse = _run(q, k, v, 0.125, causal)
    O, LSE = ref_fwd(widen(q), widen(k), widen(v), 0.125, causal)
    assert_bar("O", o, O, torch.float32)
    assert_lse("LSE", lse, LSE)


def test_single_head_fp32_workload():
    """fp32 Q, K, V [256, 64] ~ N(0, 1), scale 1/sqrt(64), non-causal."""
    _say("fp32 [1,1,256,64]")
    for seed in (0, 1, 2):
        q, k, v = _inputs(seed, 1, 1, 256, 64, torch.float32)
        o, lse = _run(q, k, v, 0.125, False)
        O, LSE = ref_fwd(widen(q), widen(k), widen(v), 0.125, False)
        assert_bar("O", o, O, torch.float32)
        assert_lse("LSE", lse, LSE)


@pytest.mark.parametrize("causal", [False, True])
def test_rows_sum_to_one_and_uniform(causal):
    """V = ones gives O = 1; Q = 0 gives the (causal) mean of V and LSE = ln(count)."""
    _say(f"properties causal={causal}")
    N, d = 200, 64
    q, k, v = _inputs(5, 1, 2, N, d, torch.bfloat16)
    o, _ = _run(q, k, torch.ones_like(v), 0.125, causal)
    assert np.max(np.abs(o - 1.0)) <= 2e-2
    o, lse = _run(torch.zeros_like(q), k, v, 0.125, causal)
    vv = widen(v)
    if causal:
        mean = np.cumsum(vv, axis=2) / np.arange(1, N + 1)[None, None, :, None]
        want_lse = np.log(np.arange(1, N + 1))[None, None, :].repeat(2, axis=1)
    else:
        mean = np.broadcast_to(vv.mean(axis=2, keepdims=True), vv.shape)
        want_lse = np.full((1, 2, N), math.log(N))
    assert_bar("O", o, mean, torch.bfloat16, rel=False)
    assert_lse("LSE", lse, want_lse)


def test_large_scores_no_overflow():
    """Scores around +-100: the running max keeps every exponential finite."""
    _say("large scores")
    q, k, v = _inputs(9, 1, 2, 150, 64, torch.bfloat16)
    q = (q.float() * 12.0).to(torch.bfloat16)
    for causal in (False, True):
        o, lse = _run(q, k, v, 0.125, causal)
        O, LSE = ref_fwd(widen(q), widen(k), widen(v), 0.125, causal)
        assert_bar("O", o, O, torch.bfloat16)
        assert_lse("LSE", lse, LSE)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_scores_rising_along_keys_move_the_reference(d, causal):
    """Scores that grow by far more than 64 (log2 units) within every K/V tile.

    The kernels keep the reference m of the exponentials at the first tile's
    row max and move it to the exact running max only when a tile's partial
    sums would exceed 2^64; here that happens on every tile for the even query
    rows (q[0] = 8, k_j[0] = 2j, scale 1/8: score_j = 2j natural units, about
    185 log2 units per 64-key tile), while the odd rows (q[0] = 0) never move
    it, so both branches run inside the same wavefronts.
    """
    _say(f"rising scores d={d} causal={causal}")
    N = 300
    q, k, v = _inputs(21, 1, 2, N, d, torch.bfloat16, 0.125)
    q = q.float()
    k = k.float()
    q[..., 0::2, 0] = 8.0
    q[..., 1::2, 0] = 0.0
    k[..., :, 0] = 2.0 * torch.arange(N, dtype=torch.float32)
    q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    o, lse = _run(q, k, v, 0.125, causal)
    O, LSE = ref_fwd(widen(q), widen(k), widen(v), 0.125, causal)
    assert_bar("O", o, O, torch.bfloat16)
    assert_lse("LSE", lse, LSE)


def test_deterministic_and_launch_on_side_stream():
    _say("determinism")
    q, k, v = (t.to(DEV) for t in _inputs(3, 2, 4, 333, 128, torch.bfloat16))
    o1, l1 = attn_fwd(q, k, v, causal=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o2, l2 = attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_batched_noncausal_workload_sampled():
    """bf16 [B=4, H=16, N=2048, d=64], iid N(0, 1), scale 1/sqrt(d): every
    output of 4 sampled heads against the oracle, and properties on all."""
    B, H, N, d = 4, 16, 2048, 64
    _say(f"workload [{B},{H},{N},{d}]")
    seed = 0
    q, k, v = (make_tensor(seed, n, B, H, N, d, torch.bfloat16, device=DEV) for n in ("q", "k", "v"))
    o, lse = attn_fwd(q, k, v, scale=1.0 / math.sqrt(d), causal=False)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    # LSE >= max score and <= max score + ln N for every row
    for b, h in ((0, 0), (1, 7), (2, 11), (3, 15)):
        qh, kh, vh = (widen(make_head(seed, n, b, h, N, d, torch.bfloat16)) for n in ("q", "k", "v"))
        O, LSE = ref_fwd(qh, kh, vh, 1.0 / math.sqrt(d), False)
        assert_bar(f"O[{b},{h}]", widen(o[b, h]), O, torch.bfloat16)
        assert_lse(f"LSE[{b},{h}]", widen(lse[b, h]), LSE)


@pytest.mark.parametrize("B,H,N,heads", [(4, 16, 2048, ((0, 0), (1, 9), (2, 4), (3, 15))),
                                          (2, 16, 4096, ((0, 0), (1, 15)))])
def test_batched_causal_workload_full_heads(B, H, N, heads):
    """bf16 [B, H, N, d=64], iid N(0, 1), causal, 512 workgroups (8 or 16
    query tiles per head): the launch fills the chip at once, so long and
    short query tiles are paired per CU and every wavefront stops after its
    last visible key tile; every row of the sampled heads against the oracle."""
    d = 64
    _say(f"workload [{B},{H},{N},{d}] causal")
    seed = 3
    q, k, v = (make_tensor(seed, n, B, H, N, d, torch.bfloat16, device=DEV) for n in ("q", "k", "v"))
    o, lse = attn_fwd(q, k, v, scale=1.0 / math.sqrt(d), causal=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    for b, h in heads:
        qh, kh, vh = (widen(make_head(seed, n, b, h, N, d, torch.bfloat16)) for n in ("q", "k", "v"))
        O, LSE = ref_fwd(qh, kh, vh, 1.0 / math.sqrt(d), True)
        assert_bar(f"O[{b},{h}]", widen(o[b, h]), O, torch.bfloat16)
        assert_lse(f"LSE[{b},{h}]", widen(lse[b, h]), LSE)


def test_long_causal_workload_sampled():
    """bf16 [B=2, H=32, N=8192, d=128], inputs N(0, 1) x 0.5, causal: sampled
    rows of sampled heads (first rows, last rows, tile edges, random rows)."""
    B, H, N, d = 2, 32, 8192, 128
    _say(f"workload [{B},{H},{N},{d}] causal")
    seed = 0
    q, k, v = (make_tensor(seed, n, B, H, N, d, torch.bfloat16, 0.5, device=DEV) for n in ("q", "k", "v"))
    scale = 1.0 / math.sqrt(d)
    o, lse = attn_fwd(q, k, v, scale=scale, causal=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    rng = np.random.default_rng(123)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, 4095, 8190, 8191], rng.integers(0, N, 48)]))
    for b, h in ((0, 0), (0, 31), (1, 13)):
        qh, kh, vh = (widen(make_head(seed, n, b, h, N, d, torch.bfloat16, 0.5)) for n in ("q", "k", "v"))
        O, LSE = ref_fwd(qh[rows], kh, vh, scale, True, q_pos=rows)
        assert_bar(f"O[{b},{h}]", widen(o[b, h, rows]), O, torch.bfloat16)
        assert_lse(f"LSE[{b},{h}]", widen(lse[b, h, rows]), LSE)


def test_long_causal_workload_full_head():
    """One whole head of the long causal workload (bf16 [2, 32, 8192, 128],
    inputs N(0, 1) x 0.5): every one of its 8192 rows against the oracle,
    from a launch over all 64 heads."""
    B, H, N, d = 2, 32, 8192, 128
    seed = 0
    b, h = 1, 20
    _say(f"workload [{B},{H},{N},{d}] causal, full head ({b},{h})")
    q, k, v = (make_tensor(seed, n, B, H, N, d, torch.bfloat16, 0.5, device=DEV) for n in ("q", "k", "v"))
    scale = 1.0 / math.sqrt(d)
    o, lse = attn_fwd(q, k, v, scale=scale, causal=True)
    torch.cuda.synchronize()
    qh, kh, vh = (widen(make_head(seed, n, b, h, N, d, torch.bfloat16, 0.5)) for n in ("q", "k", "v"))
    O, LSE = ref_fwd(qh, kh, vh, scale, True)
    assert_bar(f"O[{b},{h}]", widen(o[b, h]), O, torch.bfloat16)
    assert_lse(f"LSE[{b},{h}]", widen(lse[b, h]), LSE)


@pytest.mark.parametrize("d", [64, 128])
def test_offsets_beyond_2gib(d):
    """Each tensor spans more than 2^31 bytes ([1, H, 256, d] bf16 with
    H = 2^31 / (256 d 2) + 16): the first and last heads hold seeded N(0, 1)
    data and are checked against the oracle, the others are zero (so their
    output is zero and their LSE is ln 256)."""
    N = 256
    H = (1 << 31) // (N * d * 2) + 16
    _say(f"fwd offsets beyond 2 GiB: [1,{H},{N},{d}]")
    seed = 7
    q, k, v = (torch.zeros((1, H, N, d), dtype=torch.bfloat16, device=DEV) for _ in range(3))
    for h in (0, H - 1):
        for t, n in ((q, "q"), (k, "k"), (v, "v")):
            t[0, h].copy_(make_head(seed, n, 0, h, N, d, torch.bfloat16))
    scale = 1.0 / math.sqrt(d)
    o, lse = attn_fwd(q, k, v, scale=scale, causal=True)
    torch.cuda.synchronize()
    for h in (0, H - 1):
        Q, K, V = (widen(make_head(seed, n, 0, h, N, d, torch.bfloat16)) for n in ("q", "k", "v"))
        O, LSE = ref_fwd(Q[None, None], K[None, None], V[None, None], scale, True)
        assert_bar(f"O[{h}]", widen(o[0, h]), O[0, 0], torch.bfloat16)
        assert_lse(f"LSE[{h}]", widen(lse[0, h]), LSE[0, 0])
    mid = H // 2
    assert torch.count_nonzero(o[0, mid]) == 0
    assert_lse("LSE[mid]", widen(lse[0, mid]), np.log(np.arange(1, N + 1, dtype=np.float64)))
