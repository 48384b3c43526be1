"""Properties of the full-size launches that hold at any size, checked on
every element (no oracle needed):

* heads are independent: permuting the (b, h) slabs of the inputs permutes
  the outputs bitwise (each workgroup's arithmetic depends on its own slab
  only, whatever its place in the grid);
* attention is a weighted mean over the key SET ("FlashAttention",
  xuesongtap.github.io, section 1): without a mask, permuting the keys and
  values together leaves O and the LSE unchanged up to rounding;
* the softmax weights of a row sum to one: V = 1 gives O = 1.

The launches are the bench configurations: the forward [4,16,2048,64] in
both mask settings (bf16 and FP8) and [2,32,8192,128] causal, the split-K
decode [16,32,32768,128] over 256 chunks and the backward [2,16,4096,64]
(causal, and non-causal for the key permutation).
"""

import sys

import numpy as np
import pytest
import torch

from exact_attention_05_amd import attn_bwd, attn_fwd, attn_fwd_fp8, attn_fwd_splitk_decode, attn_quantize_fp8
from exact_attention_05_amd.inputs import make_tensor, widen

from helpers import assert_bar, assert_lse

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _qkv(seed, B, H, N, d, input_scale=1.0):
    return [make_tensor(seed, n, B, H, N, d, torch.bfloat16, input_scale, device=DEV) for n in ("q", "k", "v")]


def _permute_heads(t, B, H):
    """The (b, h) slabs of t in a fixed shuffled order (the same for every call)."""
    perm = torch.from_numpy(np.random.default_rng(17).permutation(B * H)).to(t.device)
    return t.reshape(B * H, *t.shape[2:])[perm].reshape(t.shape), perm


@pytest.mark.parametrize("B,H,N,d,causal,input_scale",
                         [(4, 16, 2048, 64, False, 1.0), (4, 16, 2048, 64, True, 1.0),
                          (2, 32, 8192, 128, True, 0.5)])
def test_fwd_heads_independent(B, H, N, d, causal, input_scale):
    _say(f"fwd head permutation [{B},{H},{N},{d}] causal={causal}")
    q, k, v = _qkv(31, B, H, N, d, input_scale)
    o, lse = attn_fwd(q, k, v, causal=causal)
    qp, perm = _permute_heads(q, B, H)
    kp, _ = _permute_heads(k, B, H)
    vp, _ = _permute_heads(v, B, H)
    op, lsep = attn_fwd(qp, kp, vp, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(op.reshape(B * H, N, d), o.reshape(B * H, N, d)[perm])
    assert torch.equal(lsep.reshape(B * H, N), lse.reshape(B * H, N)[perm])


def test_fwd_key_permutation_full_size():
    """Non-causal [4,16,2048,64]: keys and values reversed within every head,
    and shuffled, give the same O and LSE up to rounding."""
    B, H, N, d = 4, 16, 2048, 64
    _say(f"fwd key permutation [{B},{H},{N},{d}]")
    q, k, v = _qkv(32, B, H, N, d)
    o, lse = attn_fwd(q, k, v, causal=False)
    o, lse = widen(o), widen(lse)
    for name, idx in (("reversed", torch.arange(N - 1, -1, -1)),
                      ("shuffled", torch.from_numpy(np.random.default_rng(5).permutation(N)))):
        idx = idx.to(DEV)
        op, lsep = attn_fwd(q, k[:, :, idx].contiguous(), v[:, :, idx].contiguous(), causal=False)
        torch.cuda.synchronize()
        assert_bar(f"O {name}", widen(op), o, torch.bfloat16)
        assert_lse(f"LSE {name}", widen(lsep), lse)


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_rows_sum_to_one_full_size(causal):
    B, H, N, d = 4, 16, 2048, 64
    _say(f"fwd V = 1 [{B},{H},{N},{d}] causal={causal}")
    q, k, _ = _qkv(33, B, H, N, d)
    o, _ = attn_fwd(q, k, torch.ones_like(q), causal=causal)
    torch.cuda.synchronize()
    err = (o.float() - 1.0).abs().max().item()
    assert err <= 2e-2, err


def test_decode_heads_independent_and_key_order():
    """Split-K decode [16,32,32768,128] over 256 chunks: heads permuted give
    the permuted outputs bitwise; the cache positions shuffled give the same
    result up to rounding."""
    B, H, L, d, S = 16, 32, 32768, 128, 256
    _say(f"decode properties [{B},{H},{L},{d}] S={S}")
    q = make_tensor(41, "q", B, H, 1, d, torch.bfloat16, device=DEV)
    kc = make_tensor(41, "k", B, H, L, d, torch.bfloat16, device=DEV)
    vc = make_tensor(41, "v", B, H, L, d, torch.bfloat16, device=DEV)
    o, lse, ws = attn_fwd_splitk_decode(q, kc, vc, S)
    qp, perm = _permute_heads(q, B, H)
    kp, _ = _permute_heads(kc, B, H)
    vp, _ = _permute_heads(vc, B, H)
    op, lsep, _ = attn_fwd_splitk_decode(qp, kp, vp, S, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(op.reshape(B * H, d), o.reshape(B * H, d)[perm])
    assert torch.equal(lsep.reshape(B * H), lse.reshape(B * H)[perm])
    del qp, kp, vp
    idx = torch.from_numpy(np.random.default_rng(6).permutation(L)).to(DEV)
    os_, lses, _ = attn_fwd_splitk_decode(q, kc[:, :, idx].contiguous(), vc[:, :, idx].contiguous(), S,
                                          workspace=ws)
    torch.cuda.synchronize()
    assert_bar("O shuffled", widen(os_), widen(o), torch.bfloat16)
    assert_lse("LSE shuffled", widen(lses), widen(lse))


def test_bwd_heads_independent():
    """Causal backward [2,16,4096,64]: permuting the heads of every input
    permutes dQ, dK and dV bitwise."""
    B, H, N, d = 2, 16, 4096, 64
    _say(f"bwd head permutation [{B},{H},{N},{d}]")
    q, k, v = _qkv(51, B, H, N, d)
    do = make_tensor(51, "do", B, H, N, d, torch.bfloat16, device=DEV)
    o, lse = attn_fwd(q, k, v, causal=True)
    dq, dk, dv, ws = attn_bwd(q, k, v, o, do, lse, causal=True)
    ins = []
    for t in (q, k, v, o, do):
        tp, perm = _permute_heads(t, B, H)
        ins.append(tp)
    lsep = lse.reshape(B * H, N)[perm].reshape(B, H, N)
    dqp, dkp, dvp, _ = attn_bwd(*ins, lsep, causal=True, workspace=ws)
    torch.cuda.synchronize()
    for name, a, b in (("dQ", dqp, dq), ("dK", dkp, dk), ("dV", dvp, dv)):
        assert torch.equal(a.reshape(B * H, N, d), b.reshape(B * H, N, d)[perm]), name


def test_bwd_key_permutation_noncausal():
    """Non-causal backward [2,16,4096,64]: with the keys and values reversed
    within every head, dK and dV come out reversed and dQ unchanged, up to
    rounding (the gradients of a weighted mean over the key set)."""
    B, H, N, d = 2, 16, 4096, 64
    _say(f"bwd key permutation [{B},{H},{N},{d}]")
    q, k, v = _qkv(52, B, H, N, d)
    do = make_tensor(52, "do", B, H, N, d, torch.bfloat16, device=DEV)
    o, lse = attn_fwd(q, k, v, causal=False)
    dq, dk, dv, ws = attn_bwd(q, k, v, o, do, lse, causal=False)
    idx = torch.arange(N - 1, -1, -1, device=DEV)
    kr, vr = k[:, :, idx].contiguous(), v[:, :, idx].contiguous()
    orv, lser = attn_fwd(q, kr, vr, causal=False)
    dqr, dkr, dvr, _ = attn_bwd(q, kr, vr, orv, do, lser, causal=False, workspace=ws)
    torch.cuda.synchronize()
    assert_bar("dQ", widen(dqr), widen(dq), torch.bfloat16)
    assert_bar("dK", widen(dkr[:, :, idx]), widen(dk), torch.bfloat16)
    assert_bar("dV", widen(dvr[:, :, idx]), widen(dv), torch.bfloat16)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_heads_independent(causal):
    """FP8 [4,16,2048,64]: quantising and running the permuted heads gives
    the permuted codes, scales and outputs bitwise."""
    B, H, N, d = 4, 16, 2048, 64
    _say(f"fp8 head permutation [{B},{H},{N},{d}] causal={causal}")
    q, k, v = _qkv(53, B, H, N, d)

    def run(q, k, v):
        q8, sq = attn_quantize_fp8(q, 32)
        k8, sk = attn_quantize_fp8(k, 64)
        v8, sv = attn_quantize_fp8(v, 64)
        o, lse = attn_fwd_fp8(q8, k8, v8, sq, sk, sv, causal=causal)
        return q8, sq, o, lse

    q8, sq, o, lse = run(q, k, v)
    qp, perm = _permute_heads(q, B, H)
    kp, _ = _permute_heads(k, B, H)
    vp, _ = _permute_heads(v, B, H)
    q8p, sqp, op, lsep = run(qp, kp, vp)
    torch.cuda.synchronize()
    assert torch.equal(q8p.reshape(B * H, -1), q8.reshape(B * H, -1)[perm])
    assert torch.equal(sqp.reshape(B * H, -1), sq.reshape(B * H, -1)[perm])
    assert torch.equal(op.reshape(B * H, N, d), o.reshape(B * H, N, d)[perm])
    assert torch.equal(lsep.reshape(B * H, N), lse.reshape(B * H, N)[perm])
