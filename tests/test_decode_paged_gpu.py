"""GPU parity of attn_fwd_splitk_decode_paged against the fp64 oracle.

(O, LSE) are compared with the oracle's paged decode (keys and values
gathered through the block table, then the plain definition); the per-chunk
partials in the workspace are compared with the oracle's map step on each
sequence's gathered cache, so the per-sequence chunk bounds are checked too.
"""

import math
import sys

import numpy as np
import pytest
import torch

from exact_attention_05_amd import attn_fwd_splitk_decode, attn_fwd_splitk_decode_paged, split_decode_workspace
from exact_attention_05_amd.inputs import (make_block_table, make_head, make_pool, make_seq_lens, make_tensor,
                                          pool_head, widen)
from oracle import gather_paged_rows, ref_decode_partials, ref_paged_decode

from helpers import assert_bar, assert_lse

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inputs(seed, B, H, d, bs, max_blocks, spare=3):
    nb = B * max_blocks + spare
    q = make_tensor(seed, "q", B, H, 1, d, torch.bfloat16)
    kp = make_pool(seed, "k", nb, H, bs, d, torch.bfloat16)
    vp = make_pool(seed, "v", nb, H, bs, d, torch.bfloat16)
    tab = make_block_table(seed, B, max_blocks, nb)
    return q, kp, vp, tab


def _run(q, kp, vp, tab, lens, S, scale):
    dev = [t.to(DEV) for t in (q, kp, vp, tab, lens)]
    o, lse, ws = attn_fwd_splitk_decode_paged(*dev, S, scale=scale)
    torch.cuda.synchronize()
    return o, lse, ws


def _check_partials(ws, q, kp, vp, tab, lens, S, scale):
    B, H, _, d = q.shape
    U, m, l = (widen(t) for t in split_decode_workspace(ws, B, H, d, S))
    for b in range(B):
        for h in range(H):
            n = int(lens[b])
            kh = gather_paged_rows(kp, tab[b], n, h)[None, None]
            vh = gather_paged_rows(vp, tab[b], n, h)[None, None]
            Ur, mr, lr = (x[0, 0] for x in ref_decode_partials(q[b:b + 1, h:h + 1], kh, vh, scale, S))
            empty = ~np.isfinite(mr)
            assert np.array_equal(~np.isfinite(m[b, h]), empty), f"empty chunks differ at ({b},{h})"
            assert np.all(U[b, h][empty] == 0) and np.all(l[b, h][empty] == 0)
            full = ~empty
            if not full.any():
                continue
            assert np.max(np.abs(m[b, h][full] - mr[full])) <= 1e-3
            np.testing.assert_allclose(l[b, h][full], lr[full], rtol=1e-3)
            assert_bar("U/l", U[b, h][full] / l[b, h][full][:, None], Ur[full] / lr[full][:, None],
                       torch.bfloat16, rel=False)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bs,S", [(1, 3), (16, 1), (16, 7), (32, 64), (64, 5), (256, 16)])
def test_paged_decode_ragged(bs, S, d):
    """Ragged lengths (an empty sequence, a single token, a partial last block,
    a full table) with blocks scattered over the pool."""
    _say(f"paged decode bs={bs} S={S} d={d}")
    B, H = 4, 3
    max_blocks = max(1, 700 // bs)
    q, kp, vp, tab = _inputs(bs + S + d, B, H, d, bs, max_blocks)
    full = max_blocks * bs
    lens = torch.tensor([0, 1, min(full, bs + 5), full], dtype=torch.int32)
    # table entries past each sequence's last block are never read
    for b in range(B):
        tab[b, (int(lens[b]) + bs - 1) // bs:] = -1
    scale = 1.0 / math.sqrt(d)
    o, lse, ws = _run(q, kp, vp, tab, lens, S, scale)
    Q, KP, VP = widen(q), widen(kp), widen(vp)
    O, LSE = ref_paged_decode(Q, KP, VP, tab.numpy(), lens.numpy(), scale)
    assert_bar("O", widen(o), O, torch.bfloat16)
    assert_lse("LSE", widen(lse), LSE[..., 0])
    _check_partials(ws, Q, KP, VP, tab.numpy(), lens.numpy(), S, scale)


def test_paged_decode_large_grid():
    """8192 chunks over 128 heads, ragged lengths (an empty sequence, a single
    token) and a scattered table."""
    B, H, d, bs, S = 4, 32, 64, 16, 64
    _say(f"paged decode large grid B={B} H={H} S={S}")
    max_blocks = 40
    q, kp, vp, tab = _inputs(77, B, H, d, bs, max_blocks)
    full = max_blocks * bs
    lens = torch.tensor([0, 1, 2 * bs + 5, full], dtype=torch.int32)
    for b in range(B):
        tab[b, (int(lens[b]) + bs - 1) // bs:] = -1
    scale = 1.0 / math.sqrt(d)
    o, lse, ws = _run(q, kp, vp, tab, lens, S, scale)
    Q, KP, VP = widen(q), widen(kp), widen(vp)
    O, LSE = ref_paged_decode(Q, KP, VP, tab.numpy(), lens.numpy(), scale)
    assert_bar("O", widen(o), O, torch.bfloat16)
    assert_lse("LSE", widen(lse), LSE[..., 0])
    _check_partials(ws, Q, KP, VP, tab.numpy(), lens.numpy(), S, scale)


@pytest.mark.parametrize("d", [64, 128])
def test_paged_identity_table_equals_dense_bitwise(d):
    """With the dense cache cut into blocks in order (an identity table) and
    full lengths, the paged call reads the same keys in the same order as the
    dense call, so both outputs and all partials agree bit for bit."""
    _say(f"paged identity table d={d}")
    B, H, L, bs, S = 2, 4, 4096, 16, 37
    k = make_tensor(9, "k", B, H, L, d, torch.bfloat16, device=DEV)
    v = make_tensor(9, "v", B, H, L, d, torch.bfloat16, device=DEV)
    q = make_tensor(9, "q", B, H, 1, d, torch.bfloat16, device=DEV)
    mb = L // bs

    def to_pool(x):
        return x.reshape(B, H, mb, bs, d).permute(0, 2, 1, 3, 4).contiguous().reshape(B * mb, H, bs, d)

    tab = torch.arange(B * mb, dtype=torch.int32, device=DEV).reshape(B, mb)
    lens = torch.full((B,), L, dtype=torch.int32, device=DEV)
    o1, l1, w1 = attn_fwd_splitk_decode(q, k, v, S)
    o2, l2, w2 = attn_fwd_splitk_decode_paged(q, to_pool(k), to_pool(v), tab, lens, S)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(w1, w2)


def test_paged_decode_clamps_device_values():
    """A length beyond the table and block ids outside the pool are clamped
    into range on the device: the result is that of the clamped values."""
    _say("paged decode clamping")
    B, H, d, bs, mb = 2, 2, 64, 16, 4
    q, kp, vp, tab = _inputs(21, B, H, d, bs, mb)
    nb = kp.shape[0]
    tab[0, 1] = -7
    tab[1, 2] = nb + 1000
    lens = torch.tensor([mb * bs + 1000, -5], dtype=torch.int32)
    o, lse, _ = _run(q, kp, vp, tab, lens, 5, 0.125)
    tab_c = tab.clamp(0, nb - 1).numpy()
    lens_c = lens.clamp(0, mb * bs).numpy()
    O, LSE = ref_paged_decode(widen(q), widen(kp), widen(vp), tab_c, lens_c, 0.125)
    assert_bar("O", widen(o), O, torch.bfloat16)
    assert_lse("LSE", widen(lse), LSE[..., 0])
    assert torch.count_nonzero(o[1]) == 0 and torch.isinf(lse[1]).all()


def test_paged_decode_deterministic():
    _say("paged decode determinism")
    q, kp, vp, tab = _inputs(4, 3, 2, 128, 16, 100)
    lens = torch.tensor([1600, 333, 1], dtype=torch.int32)
    a = _run(q, kp, vp, tab, lens, 19, 0.1)
    b = _run(q, kp, vp, tab, lens, 19, 0.1)
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_paged_decode_workload_sampled():
    """q [16, 32, 1, 128] against a paged cache of 16-token blocks holding up
    to 32768 tokens per sequence (2048 table entries each, blocks scattered
    over a pool of 32768 + 64 blocks), ragged lengths in [16384, 32768] with
    sequence 0 at the full 32768, 256 splits: sampled heads against the
    oracle (O, LSE and every partial)."""
    B, H, d, bs, mb, S = 16, 32, 128, 16, 2048, 256
    nb = B * mb + 64
    seed = 3
    _say(f"paged decode workload B={B} H={H} blocks={nb}x{bs} S={S}")
    q = make_tensor(seed, "q", B, H, 1, d, torch.bfloat16, device=DEV)
    kp = make_pool(seed, "k", nb, H, bs, d, torch.bfloat16, device=DEV)
    vp = make_pool(seed, "v", nb, H, bs, d, torch.bfloat16, device=DEV)
    tab = make_block_table(seed, B, mb, nb)
    lens = make_seq_lens(seed, B, mb * bs // 2, mb * bs)
    lens[0] = mb * bs
    _say("inputs ready")
    scale = 1.0 / math.sqrt(d)
    o, lse, ws = attn_fwd_splitk_decode_paged(q, kp, vp, tab.to(DEV), lens.to(DEV), S, scale=scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    U, m, l = split_decode_workspace(ws, B, H, d, S)
    for b, h in ((0, 0), (7, 19), (15, 31)):
        n = int(lens[b])
        # head h of the pools, as a one-head pool [num_blocks, 1, bs, d]
        kpool = widen(pool_head(seed, "k", h, nb, bs, d, torch.bfloat16))[:, None]
        vpool = widen(pool_head(seed, "v", h, nb, bs, d, torch.bfloat16))[:, None]
        qh = widen(make_head(seed, "q", b, h, 1, d, torch.bfloat16))[None, None]
        table = tab[b:b + 1].numpy()
        O, LSE = ref_paged_decode(qh, kpool, vpool, table, np.array([n]), scale)
        assert_bar(f"O[{b},{h}]", widen(o[b, h]), O[0, 0], torch.bfloat16)
        assert_lse(f"LSE[{b},{h}]", widen(lse[b, h]).reshape(1), LSE[0, 0])
        kh = gather_paged_rows(kpool, table[0], n, 0)[None, None]
        vh = gather_paged_rows(vpool, table[0], n, 0)[None, None]
        Ur, mr, lr = ref_decode_partials(qh, kh, vh, scale, S)
        assert np.max(np.abs(widen(m[b, h]) - mr[0, 0])) <= 1e-3
        np.testing.assert_allclose(widen(l[b, h]), lr[0, 0], rtol=1e-3)
        assert_bar("U/l", widen(U[b, h]) / widen(l[b, h])[:, None], Ur[0, 0] / lr[0, 0][:, None],
                   torch.bfloat16, rel=False)
