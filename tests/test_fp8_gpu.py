"""GPU parity of the FP8 path against the fp64 oracle.

* attn_quantize_fp8: codes and scales bit for bit against the oracle's block
  quantisation of the same bf16 input (the scale max|x| / 448 and every
  x / scale are fp32 divisions on both sides, and each E4M3 code the same
  decision).  With the Hadamard rotation the fp32 rotation can differ from
  the oracle's fp64-then-fp32 value in the last bit; codes are then compared
  where that cannot change them (away from a rounding boundary), and bit for
  bit on inputs whose rotation is exact in fp32.
* attn_fwd_fp8: O and LSE against the oracle's FP8 forward (the page's
  method) on the same E4M3 inputs and scales, at the bf16 bar plus a
  rounding allowance derived below for the requantised probabilities.
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
    lo, hi = (e4m3_round(np.clip(y * (1 + t), -448.0, 448.0)) for t in (-2.0 ** -20, 2.0 ** -20))
    lo, hi = np.minimum(lo, hi), np.maximum(lo, hi)
    firm = lo == hi  # no rounding boundary within 2^-20 (far beyond fp32 rounding of y)
    assert firm.mean() > 0.999
    assert np.array_equal(got[firm], vals[firm])
    assert np.all((got == lo) | (got == hi))


def _fp8_inputs(seed, B, H, N, grid=True):
    """E4M3 Q, K, V and their block scales (Q per 32 rows, K and V per 64).
    Grid codes keep q8 . k8 exact (see inputs.make_fp8); their scales are
    chosen so that the scores spread over a few units."""
    lo, hi = (-3.0, -1.0) if grid else (-6.0, -4.0)
    q8, sq = make_fp8(seed, "q", B, H, N, 64, 32, lo, hi, grid)
    k8, sk = make_fp8(seed, "k", B, H, N, 64, 64, lo, hi, grid)
    v8, sv = make_fp8(seed, "v", B, H, N, 64, 64, -6.0, -4.0, grid)
    return q8, k8, v8, sq, sk, sv


def _run_fp8(q8, k8, v8, sq, sk, sv, scale, causal):
    dev = [t.to(DEV) for t in (q8, k8, v8, sq, sk, sv)]
    o, lse = attn_fwd_fp8(*dev, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o, lse


# The kernel evaluates each p / scale_p = 2^(u - m_new - e + log2 448) in
# fp32: u = S (scale log2(e) sq) sk with the product of the scales rounded
# three times, the exponent's offset m_new + e - log2(448) twice, one fused
# multiply-add, and the hardware exp2, whose error is about 1 ulp.  With the
# scores S exact (grid codes), the argument's absolute error stays below
# 2^-21 (|u| + |m_new| + 16) and the result's relative error below
# Y_REL(row) = 2^-21 (max|u| + |m| + 16) ln 2 + 2^-21.  A value closer than
# that to a midpoint of two E4M3 neighbours may be rounded to either, and
# then moves O by one spacing times its weight; that is the tie allowance.
# For codes whose products are not exact in the matrix unit's accumulation
# the scores themselves are off, so any value may land one spacing away: the
# general allowance is one spacing on every value (valid while the scores'
# error moves p by less than a spacing, 2^-4 relative).
def _tie_allowance(Y, W, v8, rel):
    """sum_j |e4m3(y (1 + rel)) - e4m3(y (1 - rel))| W_j |v8_j| per output."""
    y = np.nan_to_num(Y, nan=0.0)
    hi = e4m3_round(np.minimum(y * (1 + rel), 448.0))
    lo = e4m3_round(y * (1 - rel))
    return ((hi - lo) * W) @ np.abs(v8)


def _spacing_allowance(Y, W, v8):
    """sum_j spacing(y_j) W_j |v8_j|: one E4M3 step on every value."""
    y = np.nan_to_num(Y, nan=0.0)
    e = np.maximum(np.floor(np.log2(np.maximum(y, 2.0 ** -30))), -6)
    return ((np.ldexp(1.0, (e - 3).astype(int)) * (y > 0)) * W) @ np.abs(v8)


def _oracle(q8, k8, v8, sq, sk, sv, scale, causal, grid=True):
    """(O, LSE, allowance) for every head of the given tensors."""
    q, k, v = fp8_values(q8), fp8_values(k8), fp8_values(v8)
    O, LSE, Y, W = ref_fwd_fp8(q, k, v, widen(sq), widen(sk), widen(sv), scale, causal, 32, 64, trace=True)
    A = np.zeros(O.shape)
    for h in np.ndindex(*O.shape[:-2]):
        if grid:
            u = np.abs(q[h] @ k[h].T) * (np.repeat(widen(sq)[h], 32)[:q.shape[-2], None]
                                         * np.repeat(widen(sk)[h], 64)[None, :k.shape[-2]]) * scale * math.log2(math.e)
            rel = 2.0 ** -21 * (u.max(axis=1, keepdims=True) + np.abs(LSE[h])[:, None] * math.log2(math.e) + 16.0) \
                * math.log(2.0) + 2.0 ** -21
            A[h] = _tie_allowance(Y[h], W[h], v[h], rel)
        else:
            A[h] = _spacing_allowance(Y[h], W[h], v[h])
    return O, LSE, A


def _assert_fp8(name, o, lse, O, LSE, A):
    """The bf16 bar (2e-2 absolute, 2^-6 of max|ref|) on the part of O's
    error beyond the allowance; the LSE bar (1e-3) on the LSE."""
    got = widen(o)
    assert got.shape == O.shape and np.all(np.isfinite(got)), name
    excess = np.maximum(np.abs(got - O) - A, 0.0)
    mx = float(excess.max())
    assert mx <= 2e-2, f"{name}: O error beyond the allowance {mx:.3e} > 2e-2"
    assert mx <= 2.0 ** -6 * float(np.abs(O).max()), f"{name}: relative O error beyond the allowance {mx:.3e}"
    lse_err = assert_lse(name, widen(lse), LSE)
    _say(f"{name}: max |O err| {float(np.abs(got - O).max()):.3e}, beyond the allowance {mx:.3e}, "
         f"allowance max {float(A.max()):.3e}, LSE err {lse_err:.3e}")
    return mx


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 64, 100, 129, 200, 600])
def test_fp8_fwd_ragged(N, causal):
    _say(f"fp8 fwd N={N} causal={causal}")
    ins = _fp8_inputs(N + 32, 1, 2, N)
    o, lse = _run_fp8(*ins, 0.125, causal)
    _assert_fp8("fp8", o, lse, *_oracle(*ins, 0.125, causal))


@pytest.mark.parametrize("scale", [0.3, 0.05])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_fwd_other_scales(scale, causal):
    """Softmax scales other than 1/8 (the scale multiplies the block scales'
    product in every score): against the oracle at N = 300."""
    N = 300
    _say(f"fp8 fwd scale={scale} causal={causal}")
    ins = _fp8_inputs(N + 64, 1, 2, N)
    o, lse = _run_fp8(*ins, scale, causal)
    _assert_fp8("fp8", o, lse, *_oracle(*ins, scale, causal))


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_fwd_general_codes(causal):
    """Codes over the whole E4M3 range (scores not exact in the matrix
    unit), against the oracle with one E4M3 step allowed on every value."""
    _say(f"fp8 fwd general codes causal={causal}")
    ins = _fp8_inputs(86, 2, 2, 333, grid=False)
    o, lse = _run_fp8(*ins, 0.125, causal)
    _assert_fp8("fp8 general", o, lse, *_oracle(*ins, 0.125, causal, grid=False))


def test_fp8_fwd_uniform_scores():
    """Q = 0: every p is 1 and every p / scale_p exactly 448, so O is the
    mean of the dequantised V and LSE = ln N."""
    _say("fp8 fwd uniform scores")
    N = 300
    q8, k8, v8, sq, sk, sv = _fp8_inputs(82, 1, 2, N)
    o, lse = _run_fp8(torch.zeros_like(q8), k8, v8, sq, sk, sv, 0.125, False)
    vd = fp8_values(v8) * np.repeat(widen(sv), 64, axis=-1)[..., :N, None]
    assert_bar("O", widen(o), np.broadcast_to(vd.mean(axis=2, keepdims=True), vd.shape), torch.bfloat16, rel=False)
    assert_lse("LSE", widen(lse), np.full((1, 2, N), math.log(N)))


def test_fp8_fwd_rising_scores():
    """K block scales that double from block to block: the running max moves
    up on every tile, so every tile rescales l and U (alpha < 1), and the
    block's largest p sits in different rows."""
    _say("fp8 fwd rising scores")
    N = 640
    q8, k8, v8, sq, sk, sv = _fp8_inputs(83, 1, 2, N)
    sk = (sk * torch.exp2(torch.arange(sk.shape[-1], dtype=torch.float32) * 0.5)).contiguous()
    o, lse = _run_fp8(q8, k8, v8, sq, sk, sv, 0.125, False)
    _assert_fp8("fp8 rising", o, lse, *_oracle(q8, k8, v8, sq, sk, sv, 0.125, False))


def test_fp8_fwd_deterministic():
    _say("fp8 fwd determinism")
    ins = _fp8_inputs(84, 2, 2, 777)
    a = _run_fp8(*ins, 0.125, True)
    b = _run_fp8(*ins, 0.125, True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_fp8_pipeline_from_bf16():
    """bf16 Q, K, V -> attn_quantize_fp8 (Q, K rotated with the same signs)
    -> attn_fwd_fp8, against the oracle's quantisation and FP8 forward of the
    same bf16 inputs (grid inputs, so the rotated codes are exact; the codes
    then span the E4M3 range, so the general allowance applies)."""
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
    o, lse = attn_fwd_fp8(q8, k8, v8, sq, sk, sv, scale=0.125, causal=True)
    torch.cuda.synchronize()
    Q, K, V = (widen(t) for t in qkv)
    qv, qs = quantize_fp8_blocks(Q, 32, signs.numpy())
    kv, ks = quantize_fp8_blocks(K, 64, signs.numpy())
    vv, vs = quantize_fp8_blocks(V, 64)
    assert np.array_equal(fp8_values(q8), qv) and np.array_equal(widen(sq), qs)
    O, LSE, Y, W = ref_fwd_fp8(qv, kv, vv, qs, ks, vs, 0.125, True, 32, 64, trace=True)
    A = np.stack([_spacing_allowance(Y[0, h], W[0, h], vv[0, h]) for h in range(H)])[None]
    _assert_fp8("fp8 pipeline", o, lse, O, LSE, A)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_fwd_workload_sampled(causal):
    """E4M3 Q, K, V [4, 16, 2048, 64] (grid codes) with block scales, scale
    1/8: sampled heads against the oracle (causal: the launch fills the chip
    at once, so the long/short pairing and the per-wavefront stop run)."""
    B, H, N = 4, 16, 2048
    _say(f"fp8 fwd workload [{B},{H},{N},64] causal={causal}")
    ins = _fp8_inputs(0, B, H, N)
    o, lse = _run_fp8(*ins, 0.125, causal)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    for b, h in ((0, 0), (3, 15)):
        sub = [t[b:b + 1, h:h + 1] for t in ins]
        _assert_fp8(f"fp8[{b},{h}]", o[b:b + 1, h:h + 1], lse[b:b + 1, h:h + 1], *_oracle(*sub, 0.125, causal))


def test_fp8_fwd_offsets_beyond_2gib():
    """E4M3 Q, K, V [1, H, 256, 64] spanning more than 2^31 bytes each (and
    O more than 2^32): the first and last heads hold seeded data, the others
    zeros with unit scales."""
    N, d = 256, 64
    H = (1 << 31) // (N * d) + 16
    _say(f"fp8 fwd offsets beyond 2 GiB: [1,{H},{N},{d}]")
    seed = 9
    q8, k8, v8 = (torch.zeros((1, H, N, d), dtype=torch.uint8, device=DEV) for _ in range(3))
    sq = torch.ones((1, H, N // 32), dtype=torch.float32, device=DEV)
    sk = torch.ones((1, H, N // 64), dtype=torch.float32, device=DEV)
    sv = torch.ones((1, H, N // 64), dtype=torch.float32, device=DEV)
    ends = {}
    for h in (0, H - 1):
        one = _fp8_inputs(seed + h % 7, 1, 1, N)
        ends[h] = one
        for dst, src in ((q8, one[0]), (k8, one[1]), (v8, one[2]), (sq, one[3]), (sk, one[4]), (sv, one[5])):
            dst[0, h].copy_(src[0, 0])
    o, lse = attn_fwd_fp8(q8, k8, v8, sq, sk, sv, scale=0.125, causal=True)
    torch.cuda.synchronize()
    for h, one in ends.items():
        _assert_fp8(f"fp8[{h}]", o[0:1, h:h + 1], lse[0:1, h:h + 1], *_oracle(*one, 0.125, True))
    assert torch.count_nonzero(o[0, H // 2]) == 0
