"""GPU parity of the FP8 path against the fp64 oracle.

* attn_quantize_fp8: codes and scales bit for bit against the oracle's block
  quantisation of the same bf16 input (the integer decisions -- the scale's
  exponent and each E4M3 code -- are taken in fp32 on both sides).  With the
  Hadamard rotation the fp32 rotation can differ from the oracle's
  fp64-then-fp32 value in the last bit; codes are then compared where that
  cannot change them (away from a rounding boundary), and bit for bit on
  inputs whose rotation is exact in fp32.
* attn_fwd_fp8: O and LSE against the oracle's FP8 forward on the same E4M3
  inputs and scales, at the bf16 bar (the kernel's P~ reference differs from
  the oracle's by an integer, which leaves E4M3 rounding unchanged), beyond
  the oracle's rounding slack: a P~ within fp32 error of an E4M3 tie may be
  rounded either way, and on a dominant key that moves O by one E4M3 step.
"""

import math
import sys

import numpy as np
import pytest
import torch

from exact_attention_05_amd import attn_fwd_fp8, attn_quantize_fp8
from exact_attention_05_amd.inputs import fp8_values, make_fp8, make_tensor, widen
from oracle import e4m3_round, hadamard_rotate, quantize_fp8_blocks, ref_fwd_fp8

from helpers import assert_bar, assert_lse

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _quant_input(seed, B, H, N, d):
    """bf16 rows of very different sizes: N(0, 1) times 2^(row % 11 - 5), one
    block of zeros and one of tiny values (to reach the clamped exponent)."""
    x = make_tensor(seed, "q", B, H, N, d, torch.bfloat16).float()
    x *= torch.exp2(torch.arange(N, dtype=torch.float32) % 11 - 5)[:, None]
    if N > 40:
        x[:, :, 20:30] = 0.0
        x[:, :, 30:40] *= 2.0 ** -125
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N,block", [(1, 1), (200, 1), (200, 17), (200, 64), (129, 128), (300, 512)])
def test_quantize_bitexact(N, block, d):
    _say(f"quantize N={N} block={block} d={d}")
    x = _quant_input(N + block, 2, 2, N, d)
    x8, sc = attn_quantize_fp8(x.to(DEV), block)
    torch.cuda.synchronize()
    vals, scales = quantize_fp8_blocks(widen(x), block)
    assert np.array_equal(sc.cpu().double().numpy(), scales)
    assert np.array_equal(fp8_values(x8), vals)


def test_quantize_rotation_exact_grid():
    """Inputs k/32 with |k| <= 255 (exact in bf16): every butterfly sum is
    exact in fp32, so the rotated codes match bit for bit."""
    _say("quantize rotation, exact grid")
    B, H, N, d = 2, 3, 130, 64
    rng = np.random.default_rng(80)
    x = torch.from_numpy((rng.integers(-255, 256, size=(B, H, N, d)) / 32.0).astype(np.float32)).to(torch.bfloat16)
    signs = torch.from_numpy(rng.choice([-1.0, 1.0], d).astype(np.float32))
    x8, sc = attn_quantize_fp8(x.to(DEV), 64, signs=signs.to(DEV))
    torch.cuda.synchronize()
    vals, scales = quantize_fp8_blocks(widen(x), 64, signs.numpy())
    assert np.array_equal(sc.cpu().double().numpy(), scales)
    assert np.array_equal(fp8_values(x8), vals)


def test_quantize_rotation_general():
    _say("quantize rotation, N(0,1)")
    B, H, N, d = 2, 2, 256, 64
    x = make_tensor(81, "k", B, H, N, d, torch.bfloat16)
    signs = torch.from_numpy(np.random.default_rng(81).choice([-1.0, 1.0], d).astype(np.float32))
    x8, sc = attn_quantize_fp8(x.to(DEV), 64, signs=signs.to(DEV))
    torch.cuda.synchronize()
    vals, scales = quantize_fp8_blocks(widen(x), 64, signs.numpy())
    assert np.array_equal(sc.cpu().double().numpy(), scales)
    got = fp8_values(x8)
    # the value being rounded, in fp64: rotated input over its block scale
    y = hadamard_rotate(widen(x), signs.numpy()) / np.repeat(scales, 64, axis=-1)[..., None]
    lo, hi = e4m3_round(y * (1 - 2.0 ** -20)), e4m3_round(y * (1 + 2.0 ** -20))
    firm = lo == hi  # no rounding boundary within 2^-20 (far beyond fp32 rounding of y)
    assert firm.mean() > 0.999
    assert np.array_equal(got[firm], vals[firm])
    assert np.all((got == lo) | (got == hi))


def _fp8_inputs(seed, B, H, N, bm, bn):
    q8, sq = make_fp8(seed, "q", B, H, N, 64, bm)
    k8, sk = make_fp8(seed, "k", B, H, N, 64, bn)
    v8, sv = make_fp8(seed, "v", B, H, N, 64, bn)
    return q8, k8, v8, sq, sk, sv


def _run_fp8(q8, k8, v8, sq, sk, sv, bm, bn, scale, causal):
    dev = [t.to(DEV) for t in (q8, k8, v8, sq, sk, sv)]
    o, lse = attn_fwd_fp8(*dev, bm, bn, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o, lse


# Where the kernel's a_j = 2^(u_j - M + 3) can differ from the exact value:
# the FP8 MFMA does not accumulate its 64 products in full fp32 -- measured
# on gfx950 over 512 random 32x32x64 products of all finite E4M3 codes, the
# error stays below 2^-10.8 of the largest product (SCORE_REL takes 2^-9) --
# and exp2 and the fp32 arithmetic add well under 2^-14.  E4M3 decisions
# within those bounds of a tie may go either way, and so may those in the
# subnormal range; the oracle's slack R covers both.
TIE_REL = 2.0 ** -14
SCORE_REL = 2.0 ** -9


def _oracle(q8, k8, v8, sq, sk, sv, bm, bn, scale, causal):
    return ref_fwd_fp8(fp8_values(q8), fp8_values(k8), fp8_values(v8), widen(sq), widen(sk), widen(sv), scale,
                       causal, block_m=bm, block_n=bn, tie_rel=TIE_REL, score_rel=SCORE_REL)


def _assert_fp8_lse(name, got, ref, slack):
    """The LSE bar (1e-3) beyond the slack of the FP8 scores' accumulation."""
    got = np.asarray(got, dtype=np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{name}: finiteness differs"
    excess = np.maximum(np.abs(got[fin] - ref[fin]) - slack[fin], 0.0)
    assert excess.max() <= 1e-3, f"{name}: LSE error beyond the slack {excess.max():.3e} > 1e-3"


def _assert_fp8_bar(name, got, ref, slack):
    """The bf16 bar (2e-2 absolute, 2^-6 of max|ref|) on the part of the
    error that the rounding slack does not explain."""
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape and np.all(np.isfinite(got)), name
    excess = np.maximum(np.abs(got - ref) - slack, 0.0)
    mx = float(excess.max())
    assert mx <= 2e-2, f"{name}: error beyond the rounding slack {mx:.3e} > 2e-2"
    assert mx <= 2.0 ** -6 * float(np.abs(ref).max()), f"{name}: relative error beyond the slack {mx:.3e}"
    return mx


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 64, 100, 129, 200, 600])
@pytest.mark.parametrize("bm,bn", [(32, 64), (128, 128)])
def test_fp8_fwd_ragged(N, causal, bm, bn):
    _say(f"fp8 fwd N={N} causal={causal} bm={bm} bn={bn}")
    ins = _fp8_inputs(N + bm, 1, 2, N, bm, bn)
    o, lse = _run_fp8(*ins, bm, bn, 0.125, causal)
    O, LSE, R, RL = _oracle(*ins, bm, bn, 0.125, causal)
    _assert_fp8_bar("O", widen(o), O, R)
    _assert_fp8_lse("LSE", widen(lse), LSE, RL)


def test_fp8_fwd_uniform_scores():
    """Q = 0: every P~ is exactly 8, so O is the mean of the dequantised V."""
    _say("fp8 fwd uniform scores")
    N = 300
    q8, k8, v8, sq, sk, sv = _fp8_inputs(82, 1, 2, N, 32, 64)
    o, lse = _run_fp8(torch.zeros_like(q8), k8, v8, sq, sk, sv, 32, 64, 0.125, False)
    vd = fp8_values(v8) * np.repeat(widen(sv), 64, axis=-1)[..., :N, None]
    assert_bar("O", widen(o), np.broadcast_to(vd.mean(axis=2, keepdims=True), vd.shape), torch.bfloat16, rel=False)
    assert_lse("LSE", widen(lse), np.full((1, 2, N), math.log(N)))


def test_fp8_fwd_rescue_path():
    """A K block scaled far above the first tile's makes P~ leave the E4M3
    range under the first reference: the kernel must move its reference."""
    _say("fp8 fwd rescue")
    N = 640
    q8, k8, v8, sq, sk, sv = _fp8_inputs(83, 1, 2, N, 32, 64)
    sk[:, :, 6] = 2.0 ** 2  # keys 384..447: scores about 2^7 larger
    o, lse = _run_fp8(q8, k8, v8, sq, sk, sv, 32, 64, 0.125, False)
    O, LSE, R, RL = _oracle(q8, k8, v8, sq, sk, sv, 32, 64, 0.125, False)
    _assert_fp8_bar("O", widen(o), O, R)
    _assert_fp8_lse("LSE", widen(lse), LSE, RL)


def test_fp8_fwd_deterministic():
    _say("fp8 fwd determinism")
    ins = _fp8_inputs(84, 2, 2, 777, 32, 64)
    a = _run_fp8(*ins, 32, 64, 0.125, True)
    b = _run_fp8(*ins, 32, 64, 0.125, True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_fp8_pipeline_from_bf16():
    """bf16 Q, K, V -> attn_quantize_fp8 (Q, K rotated with the same signs)
    -> attn_fwd_fp8, against the oracle's quantisation and FP8 forward of the
    same bf16 inputs (grid inputs, so the rotated codes are exact)."""
    _say("fp8 pipeline")
    B, H, N, d = 1, 2, 256, 64
    rng = np.random.default_rng(85)
    qkv = [torch.from_numpy((rng.integers(-255, 256, size=(B, H, N, d)) / 64.0).astype(np.float32)).to(torch.bfloat16)
           for _ in range(3)]
    signs = torch.from_numpy(rng.choice([-1.0, 1.0], d).astype(np.float32))
    sd = signs.to(DEV)
    q8, sq = attn_quantize_fp8(qkv[0].to(DEV), 32, signs=sd)
    k8, sk = attn_quantize_fp8(qkv[1].to(DEV), 64, signs=sd)
    v8, sv = attn_quantize_fp8(qkv[2].to(DEV), 64)
    o, lse = attn_fwd_fp8(q8, k8, v8, sq, sk, sv, 32, 64, scale=0.125, causal=True)
    torch.cuda.synchronize()
    Q, K, V = (widen(t) for t in qkv)
    qv, qs = quantize_fp8_blocks(Q, 32, signs.numpy())
    kv, ks = quantize_fp8_blocks(K, 64, signs.numpy())
    vv, vs = quantize_fp8_blocks(V, 64)
    O, LSE, R, RL = ref_fwd_fp8(qv, kv, vv, qs, ks, vs, 0.125, True, block_m=32, block_n=64, tie_rel=TIE_REL,
                                score_rel=SCORE_REL)
    _assert_fp8_bar("O", widen(o), O, R)
    _assert_fp8_lse("LSE", widen(lse), LSE, RL)


def test_fp8_fwd_workload_sampled():
    """E4M3 Q, K, V [4, 16, 2048, 64] with block scales (Q per 128 rows, K
    and V per 64), non-causal, scale 1/8: sampled heads against the oracle."""
    B, H, N, bm, bn = 4, 16, 2048, 128, 64
    _say(f"fp8 fwd workload [{B},{H},{N},64]")
    ins = _fp8_inputs(0, B, H, N, bm, bn)
    o, lse = _run_fp8(*ins, bm, bn, 0.125, False)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    for b, h in ((0, 0), (3, 15)):
        sub = [t[b:b + 1, h:h + 1] for t in ins]
        O, LSE, R, RL = _oracle(*sub, bm, bn, 0.125, False)
        _assert_fp8_bar(f"O[{b},{h}]", widen(o[b:b + 1, h:h + 1]), O, R)
        _assert_fp8_lse(f"LSE[{b},{h}]", widen(lse[b:b + 1, h:h + 1]), LSE, RL)


def test_fp8_fwd_offsets_beyond_2gib():
    """E4M3 Q, K, V [1, H, 256, 64] spanning more than 2^31 bytes each (and
    O more than 2^32): the first and last heads hold seeded data, the others
    zeros with unit scales."""
    N, d, bm, bn = 256, 64, 32, 64
    H = (1 << 31) // (N * d) + 16
    _say(f"fp8 fwd offsets beyond 2 GiB: [1,{H},{N},{d}]")
    seed = 9
    q8, k8, v8 = (torch.zeros((1, H, N, d), dtype=torch.uint8, device=DEV) for _ in range(3))
    sq = torch.ones((1, H, N // bm), dtype=torch.float32, device=DEV)
    sk = torch.ones((1, H, N // bn), dtype=torch.float32, device=DEV)
    sv = torch.ones((1, H, N // bn), dtype=torch.float32, device=DEV)
    ends = {}
    for h in (0, H - 1):
        one = _fp8_inputs(seed + h % 7, 1, 1, N, bm, bn)
        ends[h] = one
        for dst, src in ((q8, one[0]), (k8, one[1]), (v8, one[2]), (sq, one[3]), (sk, one[4]), (sv, one[5])):
            dst[0, h].copy_(src[0, 0])
    o, lse = attn_fwd_fp8(q8, k8, v8, sq, sk, sv, bm, bn, scale=0.125, causal=True)
    torch.cuda.synchronize()
    for h, one in ends.items():
        O, LSE, R, RL = _oracle(*one, bm, bn, 0.125, True)
        _assert_fp8_bar(f"O[{h}]", widen(o[0:1, h:h + 1]), O, R)
        _assert_fp8_lse(f"LSE[{h}]", widen(lse[0:1, h:h + 1]), LSE, RL)
    assert torch.count_nonzero(o[0, H // 2]) == 0
