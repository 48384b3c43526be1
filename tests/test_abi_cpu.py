"""The C ABI without a GPU: the library loads, exports every entry point that
include/attn.h declares, and rejects bad arguments on the host before any HIP
call (every case below fails validation, so nothing is launched)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def _lib():
    from exact_attention_05_amd import binding

    if not os.path.exists(binding.library_path()):
        pytest.skip("libattn.so not built")
    return binding.raw_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ("attn_fwd", "attn_fwd_merge", "attn_fwd_splitk_decode", "attn_fwd_splitk_decode_paged",
              "attn_fwd_splitk_decode_noalloc", "attn_bwd",
              "attn_quantize_fp8", "attn_fwd_fp8", "attn_merge",
              "attn_decode_workspace_bytes",
              "attn_bwd_workspace_bytes", "attn_bwd_atomic_dq", "attn_bwd_atomic_workspace_bytes",
              "attn_status_string", "attn_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for n in _declared_functions():
        assert hasattr(lib, n), f"missing export {n}"


OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR, SCRATCH = 0, 1, 2, 3, 4, 5
F32, BF16 = 0, 1
P = ctypes.c_void_p(0x10000)          # fake, 16-byte aligned; never dereferenced
MIS = ctypes.c_void_p(0x10008)        # 8-byte aligned only
NULL = None


def test_status_strings_and_version():
    lib = _lib()
    for code in range(6):
        s = lib.attn_status_string(code).decode()
        assert s.startswith("ATTN_")
    assert lib.attn_status_string(99).decode().startswith("unknown")
    assert lib.attn_abi_version() == 1


def test_workspace_sizes():
    lib = _lib()
    assert lib.attn_decode_workspace_bytes(16, 32, 128, 256) == 16 * 32 * 256 * 130 * 4
    assert lib.attn_decode_workspace_bytes(0, 1, 64, 1) == 0
    assert lib.attn_decode_workspace_bytes(1, 1, 64, 0) == 0
    assert lib.attn_bwd_workspace_bytes(2, 16, 4096) == 2 * 16 * 4096 * 24
    assert lib.attn_bwd_workspace_bytes(1, 1, 0) == 0
    # the per-row terms rounded up to 256 bytes, then the fp32 dQ accumulator
    assert lib.attn_bwd_atomic_workspace_bytes(2, 16, 4096, 64) == 2 * 16 * 4096 * (24 + 64 * 4)
    assert lib.attn_bwd_atomic_workspace_bytes(1, 1, 3, 64) == 256 + 3 * 64 * 4
    assert lib.attn_bwd_atomic_workspace_bytes(1, 1, 0, 64) == 0


@pytest.mark.parametrize(
    "args,expect",
    [
        ((NULL, P, P, P, NULL, 1, 1, 8, 64, BF16, 0.125, 0), INVALID),
        ((P, P, P, MIS, NULL, 1, 1, 8, 64, BF16, 0.125, 0), INVALID),
        ((P, P, P, P, MIS, 1, 1, 8, 64, BF16, 0.125, 0), INVALID),  # lse misaligned (replaced below)
        ((P, P, P, P, NULL, 0, 1, 8, 64, BF16, 0.125, 0), INVALID),
        ((P, P, P, P, NULL, 1, 1, 0, 64, BF16, 0.125, 0), INVALID),
        ((P, P, P, P, NULL, 1, 1, (1 << 24) + 1, 64, BF16, 0.125, 0), INVALID),
        ((P, P, P, P, NULL, 1, 1, 8, 64, BF16, 0.0, 0), INVALID),
        ((P, P, P, P, NULL, 1, 1, 8, 64, BF16, float("nan"), 0), INVALID),
        ((P, P, P, P, NULL, 1, 1, 8, 64, BF16, float("inf"), 0), INVALID),
        ((P, P, P, P, NULL, 1, 1, 8, 64, 7, 0.125, 0), INVALID),
        ((P, P, P, P, NULL, 1, 1, 8, 96, BF16, 0.125, 0), UNSUPPORTED),
        ((P, P, P, P, NULL, 1, 1, 8, 128, F32, 0.125, 0), UNSUPPORTED),
        ((P, P, P, P, NULL, 1, 1, 8, 32, F32, 0.125, 0), UNSUPPORTED),
    ],
)
def test_fwd_validation(args, expect):
    lib = _lib()
    if args[4] is MIS:
        # an 8-byte-aligned lse is acceptable (fp32 needs 4), so use a 2-byte offset instead
        args = args[:4] + (ctypes.c_void_p(0x10002),) + args[5:]
        expect = INVALID
    st = lib.attn_fwd(*args, None)
    assert st == expect


def test_fwd_merge_validation():
    lib = _lib()
    base = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=2, N=64, d=64, dt=BF16, sc=0.125, causal=0)

    def call(**kw):
        a = dict(base, **kw)
        return lib.attn_fwd_merge(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                                  a["dt"], a["sc"], a["causal"], None)

    assert call(lse=NULL) == INVALID          # the running LSE is read
    assert call(lse=ctypes.c_void_p(0x10002)) == INVALID
    assert call(o=MIS) == INVALID
    assert call(N=0) == INVALID
    assert call(sc=float("nan")) == INVALID
    assert call(dt=F32) == UNSUPPORTED        # bf16 only
    assert call(d=128, dt=F32) == UNSUPPORTED
    assert call(d=32) == UNSUPPORTED


def test_decode_validation():
    lib = _lib()
    f = lib.attn_fwd_splitk_decode
    ws_need = lib.attn_decode_workspace_bytes(2, 2, 128, 4)
    base = dict(q=P, k=P, v=P, o=P, lse=NULL, ws=P, wsb=ws_need, B=2, H=2, L=100, d=128, S=4, dt=BF16, sc=0.1)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["q"], a["k"], a["v"], a["o"], a["lse"], a["ws"], a["wsb"], a["B"], a["H"], a["L"], a["d"],
                 a["S"], a["dt"], a["sc"], None)

    assert call(q=NULL) == INVALID
    assert call(k=MIS) == INVALID
    assert call(L=0) == INVALID
    assert call(L=(1 << 30) + 1) == INVALID
    assert call(S=0) == INVALID
    assert call(S=65536) == INVALID
    assert call(sc=-1.0) == INVALID
    assert call(d=96) == UNSUPPORTED
    assert call(dt=F32) == UNSUPPORTED
    assert call(ws=NULL) == WORKSPACE
    assert call(ws=MIS) == WORKSPACE
    assert call(wsb=ws_need - 1) == WORKSPACE


def test_decode_noalloc_validation():
    lib = _lib()
    f = lib.attn_fwd_splitk_decode_noalloc
    base = dict(q=P, k=P, v=P, o=P, lse=NULL, B=16, H=32, L=100, d=128, S=126, dt=BF16, sc=0.1)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["L"], a["d"], a["S"], a["dt"], a["sc"],
                 None)

    assert call(q=NULL) == INVALID
    assert call(o=MIS) == INVALID
    assert call(lse=ctypes.c_void_p(0x10002)) == INVALID
    assert call(L=0) == INVALID
    assert call(S=0) == INVALID
    assert call(sc=float("inf")) == INVALID
    assert call(d=96) == UNSUPPORTED
    assert call(dt=F32) == UNSUPPORTED
    # the partials B*H*S*(d+2) fp32 values must fit in the fixed 32 MiB scratch:
    # 512 heads at d = 128 fit 126 splits, not 127
    assert lib.attn_decode_workspace_bytes(16, 32, 128, 126) <= 32 << 20
    assert lib.attn_decode_workspace_bytes(16, 32, 128, 127) > 32 << 20
    assert call(S=127) == SCRATCH
    assert call(S=256) == SCRATCH
    assert call(B=2, H=1, d=128, S=65535) == SCRATCH
    assert lib.attn_status_string(SCRATCH).decode().startswith("ATTN_ERR_SCRATCH")


def test_paged_decode_validation():
    lib = _lib()
    f = lib.attn_fwd_splitk_decode_paged
    ws_need = lib.attn_decode_workspace_bytes(2, 2, 128, 4)
    I4 = ctypes.c_void_p(0x10004)  # 4-byte aligned: enough for the int32 table and lengths
    base = dict(q=P, k=P, v=P, tab=I4, lens=I4, o=P, lse=NULL, ws=P, wsb=ws_need, B=2, H=2, d=128, nb=10, bs=16,
                mb=8, S=4, dt=BF16, sc=0.1)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["q"], a["k"], a["v"], a["tab"], a["lens"], a["o"], a["lse"], a["ws"], a["wsb"], a["B"], a["H"],
                 a["d"], a["nb"], a["bs"], a["mb"], a["S"], a["dt"], a["sc"], None)

    assert call(q=NULL) == INVALID
    assert call(v=MIS) == INVALID
    assert call(tab=NULL) == INVALID
    assert call(lens=NULL) == INVALID
    assert call(tab=ctypes.c_void_p(0x10002)) == INVALID
    assert call(lens=ctypes.c_void_p(0x10001)) == INVALID
    assert call(B=0) == INVALID
    assert call(nb=0) == INVALID
    assert call(mb=0) == INVALID
    for bs in (0, -16, 3, 24, 48):
        assert call(bs=bs) == INVALID, bs
    assert call(bs=1 << 20, mb=(1 << 10) + 1) == INVALID
    assert call(S=0) == INVALID
    assert call(S=65536) == INVALID
    assert call(sc=float("nan")) == INVALID
    assert call(d=96) == UNSUPPORTED
    assert call(d=64, dt=F32) == UNSUPPORTED
    assert call(ws=NULL) == WORKSPACE
    assert call(wsb=ws_need - 1) == WORKSPACE


def test_quantize_fp8_validation():
    lib = _lib()
    f = lib.attn_quantize_fp8
    S4 = ctypes.c_void_p(0x10004)
    base = dict(x=P, signs=NULL, x8=P, sc=S4, B=1, H=2, N=100, d=64, br=32)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["x"], a["signs"], a["x8"], a["sc"], a["B"], a["H"], a["N"], a["d"], a["br"], None)

    assert call(x=NULL) == INVALID
    assert call(x8=MIS) == INVALID
    assert call(sc=NULL) == INVALID
    assert call(sc=ctypes.c_void_p(0x10002)) == INVALID
    assert call(signs=ctypes.c_void_p(0x10001)) == INVALID
    assert call(N=0) == INVALID
    assert call(br=0) == INVALID
    assert call(d=96) == UNSUPPORTED
    assert call(d=128, signs=S4) == UNSUPPORTED


def test_fwd_fp8_validation():
    lib = _lib()
    f = lib.attn_fwd_fp8
    S4 = ctypes.c_void_p(0x10004)
    base = dict(q=P, k=P, v=P, qs=S4, ks=S4, vs=S4, o=P, lse=NULL, B=1, H=2, N=100, d=64, bm=32, bn=64,
                sc=0.125, causal=0)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["q"], a["k"], a["v"], a["qs"], a["ks"], a["vs"], a["o"], a["lse"], a["B"], a["H"], a["N"],
                 a["d"], a["bm"], a["bn"], a["sc"], a["causal"], None)

    assert call(q=NULL) == INVALID
    assert call(v=MIS) == INVALID
    assert call(ks=NULL) == INVALID
    assert call(vs=ctypes.c_void_p(0x10002)) == INVALID
    assert call(lse=ctypes.c_void_p(0x10002)) == INVALID
    for bm, bn in ((0, 64), (32, 0), (-32, 64)):
        assert call(bm=bm, bn=bn) == INVALID, (bm, bn)
    for bm, bn in ((16, 64), (64, 64), (128, 128), (32, 32), (32, 128)):
        assert call(bm=bm, bn=bn) == UNSUPPORTED, (bm, bn)
    assert call(N=0) == INVALID
    assert call(sc=0.0) == INVALID
    assert call(d=128) == UNSUPPORTED


def test_merge_validation():
    lib = _lib()
    f = lib.attn_merge
    S4 = ctypes.c_void_p(0x10004)
    base = dict(oa=P, la=S4, ob=P, lb=S4, o=P, lse=S4, B=1, H=2, N=100, d=64, dt=BF16)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["oa"], a["la"], a["ob"], a["lb"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"], a["dt"], None)

    assert call(oa=NULL) == INVALID
    assert call(ob=MIS) == INVALID
    assert call(lse=NULL) == INVALID
    assert call(lb=ctypes.c_void_p(0x10002)) == INVALID
    assert call(N=0) == INVALID
    assert call(N=(1 << 24) + 1) == INVALID
    assert call(dt=5) == INVALID
    assert call(d=96) == UNSUPPORTED
    assert call(d=32, dt=F32) == UNSUPPORTED


@pytest.mark.parametrize("entry", ["attn_bwd", "attn_bwd_atomic_dq"])
def test_bwd_validation(entry):
    lib = _lib()
    f = getattr(lib, entry)
    need = (lib.attn_bwd_workspace_bytes(1, 2, 64) if entry == "attn_bwd"
            else lib.attn_bwd_atomic_workspace_bytes(1, 2, 64, 64))
    base = dict(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, ws=P, wsb=need, B=1, H=2, N=64, d=64,
                dt=BF16, sc=0.125, causal=1)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"], a["ws"], a["wsb"],
                 a["B"], a["H"], a["N"], a["d"], a["dt"], a["sc"], a["causal"], None)

    assert call(do=NULL) == INVALID
    assert call(lse=NULL) == INVALID
    assert call(dk=MIS) == INVALID
    assert call(N=0) == INVALID
    assert call(sc=0.0) == INVALID
    assert call(d=32) == UNSUPPORTED
    assert call(dt=F32) == UNSUPPORTED
    assert call(ws=NULL) == WORKSPACE
    assert call(wsb=need - 4) == WORKSPACE


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from exact_attention_05_amd import binding

    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        binding.raw_library()
