"""attn_fwd_splitk_decode_noalloc through the C ABI: the same result as
attn_fwd_splitk_decode (the same kernels, with the partials in the library's
fixed scratch instead of a caller workspace), bit for bit, on two calls in a
row -- the second with a smaller input, so stale partials of the first call
would show -- and the host-side rejection of a call whose partials exceed the
scratch."""

import math
import sys

import pytest
import torch

from exact_attention_05_amd import AttnError, attn_fwd_splitk_decode, attn_fwd_splitk_decode_noalloc
from exact_attention_05_amd.inputs import make_tensor, widen
from oracle import ref_fwd

from helpers import assert_bar, assert_lse

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SCRATCH_FLOATS = (32 << 20) // 4


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inputs(seed, B, H, L, d):
    q = make_tensor(seed, "q", B, H, 1, d, torch.bfloat16)
    k = make_tensor(seed, "k", B, H, L, d, torch.bfloat16)
    v = make_tensor(seed, "v", B, H, L, d, torch.bfloat16)
    return q, k, v


def _run_both(seed, B, H, L, d, S):
    assert B * H * S * (d + 2) <= SCRATCH_FLOATS
    q, k, v = _inputs(seed, B, H, L, d)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    scale = 1.0 / math.sqrt(d)
    o_ref, lse_ref, _ = attn_fwd_splitk_decode(qd, kd, vd, S, scale=scale)
    o = torch.empty_like(qd)
    lse = torch.empty((B, H), dtype=torch.float32, device=DEV)
    attn_fwd_splitk_decode_noalloc(qd, kd, vd, S, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), "O differs from the workspace entry point"
    assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32)), "LSE differs from the workspace entry point"
    return q, k, v, o, lse, scale


def test_noalloc_matches_workspace_decode_twice():
    # first call: 2*8 heads x 128 splits x 130 floats (1 MiB of partials)
    _say("noalloc decode call 1: B=2 H=8 L=5000 d=128 S=128")
    _run_both(11, 2, 8, 5000, 128, 128)
    # second, smaller call (fewer heads, splits and keys, other d): every
    # partial it reads must be its own
    _say("noalloc decode call 2: B=1 H=3 L=333 d=64 S=7")
    q, k, v, o, lse, scale = _run_both(12, 1, 3, 333, 64, 7)
    O, LSE = ref_fwd(widen(q), widen(k), widen(v), scale, False)
    assert_bar("O", widen(o), O, torch.bfloat16)
    assert_lse("LSE", widen(lse), LSE[..., 0])


def test_noalloc_largest_call_that_fits():
    # B*H = 512, d = 128: 126 splits is the most the scratch holds
    B, H, L, d, S = 16, 32, 2048, 128, 126
    _say(f"noalloc decode at the scratch limit: B={B} H={H} L={L} d={d} S={S}")
    _run_both(13, B, H, L, d, S)


def test_noalloc_rejects_partials_beyond_the_scratch():
    q, k, v = (t.to(DEV) for t in _inputs(14, 16, 32, 64, 128))
    with pytest.raises(AttnError) as e:
        attn_fwd_splitk_decode_noalloc(q, k, v, 127)
    assert e.value.name == "ATTN_ERR_SCRATCH"
