"""GPU parity of attn_merge and attn_fwd_merge: results over disjoint key
sets merged into the result over their union, checked against the oracle's
plain attention over the union (and against the oracle's merge for
hand-made states)."""

import math
import sys

import numpy as np
import pytest
import torch

from exact_attention_05_amd import attn_fwd, attn_fwd_merge, attn_merge
from exact_attention_05_amd.inputs import make_head, make_tensor, widen
from oracle import ref_fwd, ref_merge_lse

from helpers import assert_bar, assert_lse

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("d,dtype", [(64, torch.bfloat16), (128, torch.bfloat16), (64, torch.float32)])
@pytest.mark.parametrize("n", [1, 37, 200])
def test_merge_two_key_halves(n, d, dtype):
    """Queries [2, 3, n, d] against keys [2, 3, 2n, d]: the forward over each
    half of the keys, merged, equals attention over all of them."""
    _say(f"merge halves n={n} d={d} {dtype}")
    seed = n + d
    q = make_tensor(seed, "q", 2, 3, n, d, dtype)
    k = make_tensor(seed, "k", 2, 3, 2 * n, d, dtype)
    v = make_tensor(seed, "v", 2, 3, 2 * n, d, dtype)
    scale = 1.0 / math.sqrt(d)
    parts = []
    for h in range(2):
        rows = slice(h * n, (h + 1) * n)
        parts.append(attn_fwd(q.to(DEV), k[:, :, rows].contiguous().to(DEV), v[:, :, rows].contiguous().to(DEV),
                              scale=scale))
    o, lse = attn_merge(parts[0][0], parts[0][1], parts[1][0], parts[1][1])
    torch.cuda.synchronize()
    O, LSE = ref_fwd(widen(q), widen(k), widen(v), scale)
    assert_bar("O", widen(o), O, dtype)
    assert_lse("LSE", widen(lse), LSE)


@pytest.mark.parametrize("d", [64, 128])
def test_ring_of_causal_shards(d):
    """Causal [1, 4, 512, d] cut into G = 4 shards of 128 rows: each query
    shard runs the causal forward on its own shard and the non-causal forward
    on every earlier one, merging in place as the shards arrive (one GPU's
    work in a ring of four); the result is causal attention over the whole
    sequence."""
    G, S, H = 4, 128, 4
    N = G * S
    _say(f"ring of {G} causal shards d={d}")
    seed = 40 + d
    q, k, v = (make_tensor(seed, n, 1, H, N, d, torch.bfloat16, device=DEV) for n in ("q", "k", "v"))
    shard = lambda t, j: t[:, :, j * S:(j + 1) * S].contiguous()
    scale = 1.0 / math.sqrt(d)
    outs = []
    for i in range(G):
        qi = shard(q, i)
        o, lse = attn_fwd(qi, shard(k, i), shard(v, i), scale=scale, causal=True)
        for j in range(i - 1, -1, -1):
            oj, lj = attn_fwd(qi, shard(k, j), shard(v, j), scale=scale, causal=False)
            attn_merge(o, lse, oj, lj, out=o, lse=lse)
        outs.append((o, lse))
    torch.cuda.synchronize()
    for h in (0, H - 1):
        Q, K, V = (widen(make_head(seed, n, 0, h, N, d, torch.bfloat16)) for n in ("q", "k", "v"))
        O, LSE = ref_fwd(Q, K, V, scale, causal=True)
        for i, (o, lse) in enumerate(outs):
            rows = slice(i * S, (i + 1) * S)
            assert_bar(f"O[h{h},shard{i}]", widen(o[0, h]), O[rows], torch.bfloat16)
            assert_lse(f"LSE[h{h},shard{i}]", widen(lse[0, h]), LSE[rows])


def test_merge_in_place_and_empty_sides():
    """In-place merges equal out-of-place ones; a side with LSE = -inf is not
    read (its O may hold anything) and both empty give O = 0, LSE = -inf."""
    _say("merge in place / empty sides")
    B, H, N, d = 1, 2, 96, 64
    g = torch.Generator().manual_seed(5)
    oa = torch.randn((B, H, N, d), generator=g).to(torch.bfloat16)
    ob = torch.randn((B, H, N, d), generator=g).to(torch.bfloat16)
    la = torch.randn((B, H, N), generator=g) * 3
    lb = torch.randn((B, H, N), generator=g) * 3
    lb[:, :, :20] = -math.inf
    ob[:, :, :20] = math.nan
    la[:, :, 10:20] = -math.inf
    oa[:, :, 10:20] = math.nan
    dev = [t.to(DEV) for t in (oa, la, ob, lb)]
    o1, l1 = attn_merge(*dev)
    a_o, a_l = dev[0].clone(), dev[1].clone()
    attn_merge(a_o, a_l, dev[2], dev[3], out=a_o, lse=a_l)
    torch.cuda.synchronize()
    assert torch.equal(a_o, o1) and torch.equal(a_l, l1)
    O, L = ref_merge_lse(widen(oa), widen(la), widen(ob), widen(lb))
    np.testing.assert_allclose(widen(l1), L, rtol=1e-6, atol=1e-6)
    assert_bar("O", widen(o1), O, torch.bfloat16, rel=False)
    assert torch.count_nonzero(o1[:, :, 10:20]) == 0 and torch.isinf(l1[:, :, 10:20]).all()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", [1, 37, 200, 600])
def test_fwd_merge_two_key_halves(n, d):
    """attn_fwd over the first half of the keys, then attn_fwd_merge over the
    second (in place): attention over all of them."""
    _say(f"fused merge halves n={n} d={d}")
    seed = 3 * n + d
    q = make_tensor(seed, "q", 2, 3, n, d, torch.bfloat16, device=DEV)
    k = make_tensor(seed, "k", 2, 3, 2 * n, d, torch.bfloat16, device=DEV)
    v = make_tensor(seed, "v", 2, 3, 2 * n, d, torch.bfloat16, device=DEV)
    scale = 1.0 / math.sqrt(d)
    half = lambda t, h: t[:, :, h * n:(h + 1) * n].contiguous()
    o, lse = attn_fwd(q, half(k, 0), half(v, 0), scale=scale)
    attn_fwd_merge(q, half(k, 1), half(v, 1), o, lse, scale=scale)
    torch.cuda.synchronize()
    O, LSE = ref_fwd(widen(q), widen(k), widen(v), scale)
    assert_bar("O", widen(o), O, torch.bfloat16)
    assert_lse("LSE", widen(lse), LSE)


@pytest.mark.parametrize("d", [64, 128])
def test_fwd_merge_ring_of_causal_shards(d):
    """The ring of test_ring_of_causal_shards with the merge fused into the
    forward: causal attention over the whole sequence, and the same result
    (to the bar) as the forward followed by attn_merge."""
    G, S, H = 4, 160, 4
    N = G * S
    _say(f"fused ring of {G} causal shards d={d}")
    seed = 60 + d
    q, k, v = (make_tensor(seed, n, 1, H, N, d, torch.bfloat16, device=DEV) for n in ("q", "k", "v"))
    shard = lambda t, j: t[:, :, j * S:(j + 1) * S].contiguous()
    scale = 1.0 / math.sqrt(d)
    fused, plain = [], []
    for i in range(G):
        qi = shard(q, i)
        o, lse = attn_fwd(qi, shard(k, i), shard(v, i), scale=scale, causal=True)
        o2, lse2 = o.clone(), lse.clone()
        for j in range(i - 1, -1, -1):
            attn_fwd_merge(qi, shard(k, j), shard(v, j), o, lse, scale=scale)
            oj, lj = attn_fwd(qi, shard(k, j), shard(v, j), scale=scale)
            attn_merge(o2, lse2, oj, lj, out=o2, lse=lse2)
        fused.append((o, lse))
        plain.append((o2, lse2))
    torch.cuda.synchronize()
    for h in (0, H - 1):
        Q, K, V = (widen(make_head(seed, n, 0, h, N, d, torch.bfloat16)) for n in ("q", "k", "v"))
        O, LSE = ref_fwd(Q, K, V, scale, causal=True)
        for i, ((o, lse), (o2, lse2)) in enumerate(zip(fused, plain)):
            rows = slice(i * S, (i + 1) * S)
            assert_bar(f"O[h{h},shard{i}]", widen(o[0, h]), O[rows], torch.bfloat16)
            assert_lse(f"LSE[h{h},shard{i}]", widen(lse[0, h]), LSE[rows])
            assert_bar(f"fused vs plain O[h{h},shard{i}]", widen(o[0, h]), widen(o2[0, h]), torch.bfloat16)


@pytest.mark.parametrize("d", [64, 128])
def test_fwd_merge_into_empty_state(d):
    """A running state with LSE = -inf (and NaN in O, never read) gives
    attn_fwd's result bit for bit; rows whose running LSE is finite mix."""
    _say(f"fused merge into empty state d={d}")
    B, H, N = 1, 2, 300
    q, k, v = (make_tensor(8 + d, n, B, H, N, d, torch.bfloat16, device=DEV) for n in ("q", "k", "v"))
    o_ref, lse_ref = attn_fwd(q, k, v, causal=True)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), -math.inf, dtype=torch.float32, device=DEV)
    attn_fwd_merge(q, k, v, o, lse, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    # merging the same keys twice: the weights are 1/2 each, O unchanged to
    # rounding, LSE up by ln 2
    attn_fwd_merge(q, k, v, o, lse, causal=True)
    torch.cuda.synchronize()
    assert_bar("O twice", widen(o), widen(o_ref), torch.bfloat16)
    np.testing.assert_allclose(widen(lse), widen(lse_ref) + math.log(2.0), rtol=0, atol=1e-5)


def test_fwd_merge_offsets_beyond_2gib():
    """attn_fwd_merge over tensors [1, H, 256, 64] bf16 of more than 2^31
    bytes: the first and last heads hold seeded data (the running result from
    the first half of the keys, merged with the second half), the others are
    zero."""
    N, d = 256, 64
    H = (1 << 31) // (N * d * 2) + 16
    _say(f"fused merge offsets beyond 2 GiB: [1,{H},{N},{d}]")
    seed = 10
    q, k, v = (torch.zeros((1, H, N, d), dtype=torch.bfloat16, device=DEV) for _ in range(3))
    k2, v2 = torch.zeros_like(k), torch.zeros_like(v)
    for h in (0, H - 1):
        q[0, h].copy_(make_head(seed, "q", 0, h, N, d, torch.bfloat16))
        kk = make_head(seed, "k", 0, h, 2 * N, d, torch.bfloat16)
        vv = make_head(seed, "v", 0, h, 2 * N, d, torch.bfloat16)
        k[0, h].copy_(kk[:N])
        v[0, h].copy_(vv[:N])
        k2[0, h].copy_(kk[N:])
        v2[0, h].copy_(vv[N:])
    o, lse = attn_fwd(q, k, v, scale=0.125)
    attn_fwd_merge(q, k2, v2, o, lse, scale=0.125)
    torch.cuda.synchronize()
    for h in (0, H - 1):
        Q = widen(make_head(seed, "q", 0, h, N, d, torch.bfloat16))
        K = widen(make_head(seed, "k", 0, h, 2 * N, d, torch.bfloat16))
        V = widen(make_head(seed, "v", 0, h, 2 * N, d, torch.bfloat16))
        O, LSE = ref_fwd(Q[None, None], K[None, None], V[None, None], 0.125)
        assert_bar(f"O[{h}]", widen(o[0, h]), O[0, 0], torch.bfloat16)
        assert_lse(f"LSE[{h}]", widen(lse[0, h]), LSE[0, 0])
    mid = H // 2
    assert torch.count_nonzero(o[0, mid]) == 0
    np.testing.assert_allclose(widen(lse[0, mid]), np.log(2 * N), rtol=0, atol=1e-5)
