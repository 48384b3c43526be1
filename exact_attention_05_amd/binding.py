"""ctypes binding of libattn.so; names mirror the C ABI in include/attn.h.

Argument marshalling only: every arithmetic step runs in the HIP kernels.
Torch provides device memory and the current stream.  The shared library is
loaded on first use; when it is missing, every call raises.
"""

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libattn.so")
_lib = None

ATTN_OK = 0
_STATUS_NAMES = {
    0: "ATTN_OK",
    1: "ATTN_ERR_INVALID_ARG",
    2: "ATTN_ERR_UNSUPPORTED",
    3: "ATTN_ERR_WORKSPACE",
    4: "ATTN_ERR_HIP",
    5: "ATTN_ERR_SCRATCH",
}
ATTN_F32 = 0
ATTN_BF16 = 1
_DTYPES = {torch.float32: ATTN_F32, torch.bfloat16: ATTN_BF16}


class AttnError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(msg)
        self.status = status
        self.name = _STATUS_NAMES.get(status, str(status))


def library_path():
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with `python -m exact_attention_05_amd.build` "
            "(there is no fallback implementation)"
        )
    lib = ctypes.CDLL(_LIB_PATH)
    vp, ci, cf, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_status_string.argtypes = [ci]
    lib.attn_abi_version.restype = ci
    lib.attn_abi_version.argtypes = []
    lib.attn_fwd.restype = ci
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, ci, vp]
    lib.attn_fwd_merge.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, ci, vp]
    lib.attn_fwd_merge.restype = ci
    lib.attn_decode_workspace_bytes.restype = sz
    lib.attn_decode_workspace_bytes.argtypes = [ci, ci, ci, ci]
    lib.attn_fwd_splitk_decode.restype = ci
    lib.attn_fwd_splitk_decode.argtypes = [vp, vp, vp, vp, vp, vp, sz, ci, ci, ci, ci, ci, ci, cf, vp]
    lib.attn_fwd_splitk_decode_noalloc.restype = ci
    lib.attn_fwd_splitk_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, vp]
    lib.attn_fwd_splitk_decode_paged.restype = ci
    lib.attn_fwd_splitk_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, sz, ci, ci, ci, ci, ci, ci, ci,
                                                 ci, cf, vp]
    lib.attn_quantize_fp8.restype = ci
    lib.attn_quantize_fp8.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, ci, vp]
    lib.attn_fwd_fp8.restype = ci
    lib.attn_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, ci, vp]
    lib.attn_merge.restype = ci
    lib.attn_merge.argtypes = [vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, vp]
    lib.attn_bwd_workspace_bytes.restype = sz
    lib.attn_bwd_workspace_bytes.argtypes = [ci, ci, ci]
    lib.attn_bwd.restype = ci
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, ci, ci, ci, ci, ci, cf, ci, vp]
    lib.attn_bwd_atomic_workspace_bytes.restype = sz
    lib.attn_bwd_atomic_workspace_bytes.argtypes = [ci, ci, ci, ci]
    lib.attn_bwd_atomic_dq.restype = ci
    lib.attn_bwd_atomic_dq.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, ci, ci, ci, ci, ci, cf, ci, vp]
    _lib = lib
    return lib


def raw_library():
    """The loaded ctypes.CDLL (for ABI-level tests)."""
    return _load()


def attn_status_string(status):
    return _load().attn_status_string(int(status)).decode()


def _check(status, what):
    if status != ATTN_OK:
        raise AttnError(status, f"{what}: {attn_status_string(status)}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t):
    if t.dtype not in _DTYPES:
        raise AttnError(2, f"unsupported dtype {t.dtype}")
    return _DTYPES[t.dtype]


def _require(cond, msg):
    if not cond:
        raise AttnError(1, msg)


def _check_bhnd(name, t, shape, dtype, device):
    _require(t.is_cuda and t.device == device, f"{name} must be on {device}")
    _require(t.dtype == dtype, f"{name} must have dtype {dtype}")
    _require(tuple(t.shape) == tuple(shape), f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    _require(t.is_contiguous(), f"{name} must be contiguous")


def attn_fwd(q, k, v, scale=None, causal=False, out=None, lse=None):
    """O, LSE = softmax(scale Q K^T) V for [B, H, N, d] tensors on one GPU.

    ``scale`` defaults to 1/sqrt(d).  Returns (o, lse) with lse [B, H, N] fp32.
    """
    B, H, N, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_bhnd(name, t, (B, H, N, d), q.dtype, dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_bhnd("out", out, (B, H, N, d), q.dtype, dev)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    else:
        _check_bhnd("lse", lse, (B, H, N), torch.float32, dev)
    st = _load().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, _dtype_code(q),
                          scale, int(bool(causal)), _stream(dev))
    _check(st, "attn_fwd")
    return out, lse


def attn_fwd_merge(q, k, v, o, lse, scale=None, causal=False):
    """Attention of q over the keys k, v combined in place with the running
    result (o, lse) over other keys (rows with lse = -inf have seen none).

    Returns (o, lse), the same tensors, now over both key sets.
    """
    B, H, N, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check_bhnd(name, t, (B, H, N, d), q.dtype, dev)
    _check_bhnd("lse", lse, (B, H, N), torch.float32, dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = _load().attn_fwd_merge(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, _dtype_code(q),
                                scale, int(bool(causal)), _stream(dev))
    _check(st, "attn_fwd_merge")
    return o, lse


def attn_decode_workspace_bytes(B, H, d, num_splits):
    return int(_load().attn_decode_workspace_bytes(B, H, d, num_splits))


def attn_fwd_splitk_decode(q, k_cache, v_cache, num_splits, scale=None, out=None, lse=None, workspace=None):
    """Split-K decode: q [B, H, 1, d] against k_cache, v_cache [B, H, L, d].

    Returns (o [B, H, 1, d], lse [B, H], workspace); the workspace holds the
    fp32 partials U [B, H, S, d], m [B, H, S], l [B, H, S] back to back.
    """
    B, H, one, d = q.shape
    _require(one == 1, "q must be [B, H, 1, d]")
    L = k_cache.shape[2]
    dev = q.device
    _check_bhnd("q", q, (B, H, 1, d), q.dtype, dev)
    _check_bhnd("k_cache", k_cache, (B, H, L, d), q.dtype, dev)
    _check_bhnd("v_cache", v_cache, (B, H, L, d), q.dtype, dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    need = attn_decode_workspace_bytes(B, H, d, num_splits)
    if workspace is None:
        workspace = torch.empty((max(need, 4) + 3) // 4, dtype=torch.float32, device=dev)
    else:
        _require(workspace.is_cuda and workspace.device == dev, f"workspace must be on {dev}")
        _require(workspace.is_contiguous(), "workspace must be contiguous")
    out, lse = _decode_outputs(q, out, lse)
    st = _load().attn_fwd_splitk_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse),
                                        _ptr(workspace), workspace.numel() * workspace.element_size(),
                                        B, H, L, d, int(num_splits), _dtype_code(q), scale, _stream(dev))
    _check(st, "attn_fwd_splitk_decode")
    return out, lse, workspace


def _decode_outputs(q, out, lse):
    """The decode's (o [B, H, 1, d], lse [B, H] fp32): checked when given, else new."""
    B, H, _, d = q.shape
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_bhnd("out", out, (B, H, 1, d), q.dtype, dev)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    else:
        _check_bhnd("lse", lse, (B, H), torch.float32, dev)
    return out, lse


def attn_fwd_splitk_decode_noalloc(q, k_cache, v_cache, num_splits, scale=None, out=None, lse=None):
    """attn_fwd_splitk_decode without a workspace: the library keeps the
    partials in its fixed per-device scratch (ATTN_DECODE_SCRATCH_BYTES) and
    allocates nothing.  With ``out`` and ``lse`` given, this call allocates
    no device memory at all.  Calls that may overlap on one GPU race.

    Returns (o [B, H, 1, d], lse [B, H]).
    """
    B, H, one, d = q.shape
    _require(one == 1, "q must be [B, H, 1, d]")
    L = k_cache.shape[2]
    dev = q.device
    _check_bhnd("q", q, (B, H, 1, d), q.dtype, dev)
    _check_bhnd("k_cache", k_cache, (B, H, L, d), q.dtype, dev)
    _check_bhnd("v_cache", v_cache, (B, H, L, d), q.dtype, dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out, lse = _decode_outputs(q, out, lse)
    with torch.cuda.device(dev):
        st = _load().attn_fwd_splitk_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse),
                                                    B, H, L, d, int(num_splits), _dtype_code(q), scale,
                                                    _stream(dev))
    _check(st, "attn_fwd_splitk_decode_noalloc")
    return out, lse


def attn_fwd_splitk_decode_paged(q, k_pool, v_pool, block_table, seq_lens, num_splits, scale=None, out=None,
                                 lse=None, workspace=None):
    """Split-K decode over a paged cache.

    q [B, H, 1, d]; k_pool, v_pool [num_blocks, H, block_size, d];
    block_table [B, max_blocks] int32 and seq_lens [B] int32 on the same GPU:
    token t of sequence b is row t % block_size of pool block
    block_table[b, t // block_size].  Returns (o [B, H, 1, d], lse [B, H],
    workspace) with the workspace laid out as for attn_fwd_splitk_decode.
    """
    B, H, one, d = q.shape
    _require(one == 1, "q must be [B, H, 1, d]")
    _require(k_pool.dim() == 4, "k_pool must be [num_blocks, H, block_size, d]")
    num_blocks, _, block_size, _ = k_pool.shape
    dev = q.device
    _check_bhnd("q", q, (B, H, 1, d), q.dtype, dev)
    _check_bhnd("k_pool", k_pool, (num_blocks, H, block_size, d), q.dtype, dev)
    _check_bhnd("v_pool", v_pool, (num_blocks, H, block_size, d), q.dtype, dev)
    _require(block_table.dim() == 2 and block_table.shape[0] == B, "block_table must be [B, max_blocks]")
    max_blocks = block_table.shape[1]
    _check_bhnd("block_table", block_table, (B, max_blocks), torch.int32, dev)
    _check_bhnd("seq_lens", seq_lens, (B,), torch.int32, dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    need = attn_decode_workspace_bytes(B, H, d, num_splits)
    if workspace is None:
        workspace = torch.empty((max(need, 4) + 3) // 4, dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_bhnd("out", out, (B, H, 1, d), q.dtype, dev)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    else:
        _check_bhnd("lse", lse, (B, H), torch.float32, dev)
    st = _load().attn_fwd_splitk_decode_paged(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens), _ptr(out), _ptr(lse),
        _ptr(workspace), workspace.numel() * workspace.element_size(), B, H, d, num_blocks, block_size,
        max_blocks, int(num_splits), _dtype_code(q), scale, _stream(dev))
    _check(st, "attn_fwd_splitk_decode_paged")
    return out, lse, workspace


def _check_fp8(name, t, shape, device):
    _require(t.is_cuda and t.device == device, f"{name} must be on {device}")
    _require(t.element_size() == 1, f"{name} must hold one byte per element (E4M3 bit patterns)")
    _require(tuple(t.shape) == tuple(shape), f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    _require(t.is_contiguous(), f"{name} must be contiguous")


def attn_quantize_fp8(x, block_rows, signs=None, out=None, scales=None):
    """Block quantisation of bf16 x [B, H, N, d] to E4M3 bytes plus one fp32
    scale (max|x| / 448) per block of ``block_rows`` rows, optionally after
    the Hadamard rotation with ``signs`` (d floats of +-1).

    Returns (x8 uint8 [B, H, N, d], scales fp32 [B, H, ceil(N / block_rows)]).
    """
    B, H, N, d = x.shape
    dev = x.device
    _check_bhnd("x", x, (B, H, N, d), torch.bfloat16, dev)
    nblk = -(-N // int(block_rows))
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.uint8, device=dev)
    else:
        _check_fp8("out", out, (B, H, N, d), dev)
    if scales is None:
        scales = torch.empty((B, H, nblk), dtype=torch.float32, device=dev)
    else:
        _check_bhnd("scales", scales, (B, H, nblk), torch.float32, dev)
    if signs is not None:
        _check_bhnd("signs", signs, (d,), torch.float32, dev)
    st = _load().attn_quantize_fp8(_ptr(x), _ptr(signs), _ptr(out), _ptr(scales), B, H, N, d, int(block_rows),
                                   _stream(dev))
    _check(st, "attn_quantize_fp8")
    return out, scales


def attn_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, block_m=32, block_n=64, scale=None, causal=False, out=None,
                 lse=None):
    """Attention forward on E4M3 inputs [B, H, N, d] (uint8 bit patterns)
    with positive fp32 per-block scales (q_scale [B, H, ceil(N / block_m)],
    k_scale and v_scale [B, H, ceil(N / block_n)]); the library supports
    block_m = 32 and block_n = 64.

    Returns (o bf16 [B, H, N, d], lse fp32 [B, H, N]).
    """
    B, H, N, d = q8.shape
    dev = q8.device
    for name, t in (("q8", q8), ("k8", k8), ("v8", v8)):
        _check_fp8(name, t, (B, H, N, d), dev)
    _check_bhnd("q_scale", q_scale, (B, H, -(-N // int(block_m))), torch.float32, dev)
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        _check_bhnd(name, t, (B, H, -(-N // int(block_n))), torch.float32, dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev)
    else:
        _check_bhnd("out", out, (B, H, N, d), torch.bfloat16, dev)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    else:
        _check_bhnd("lse", lse, (B, H, N), torch.float32, dev)
    st = _load().attn_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale), _ptr(out),
                              _ptr(lse), B, H, N, d, int(block_m), int(block_n), scale, int(bool(causal)),
                              _stream(dev))
    _check(st, "attn_fwd_fp8")
    return out, lse


def attn_merge(o_a, lse_a, o_b, lse_b, out=None, lse=None):
    """(O, LSE) over the union of two disjoint key sets from the results over
    each: O = e^(LSE_a - L) O_a + e^(LSE_b - L) O_b, L = log(e^LSE_a + e^LSE_b).

    o_* [B, H, N, d], lse_* [B, H, N] fp32; ``out``/``lse`` may be o_a/lse_a
    (or o_b/lse_b) to merge in place.  Returns (out, lse).
    """
    B, H, N, d = o_a.shape
    dev = o_a.device
    _check_bhnd("o_a", o_a, (B, H, N, d), o_a.dtype, dev)
    _check_bhnd("o_b", o_b, (B, H, N, d), o_a.dtype, dev)
    for name, t in (("lse_a", lse_a), ("lse_b", lse_b)):
        _check_bhnd(name, t, (B, H, N), torch.float32, dev)
    if out is None:
        out = torch.empty_like(o_a)
    else:
        _check_bhnd("out", out, (B, H, N, d), o_a.dtype, dev)
    if lse is None:
        lse = torch.empty_like(lse_a)
    else:
        _check_bhnd("lse", lse, (B, H, N), torch.float32, dev)
    st = _load().attn_merge(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(out), _ptr(lse), B, H, N, d,
                            _dtype_code(o_a), _stream(dev))
    _check(st, "attn_merge")
    return out, lse


def split_decode_workspace(workspace, B, H, d, num_splits):
    """Views (U [B, H, S, d], m [B, H, S], l [B, H, S]) of a decode workspace."""
    S = num_splits
    n_u = B * H * S * d
    n_m = B * H * S
    flat = workspace.view(-1)
    return (flat[:n_u].view(B, H, S, d), flat[n_u:n_u + n_m].view(B, H, S),
            flat[n_u + n_m:n_u + 2 * n_m].view(B, H, S))


def attn_bwd_workspace_bytes(B, H, N):
    return int(_load().attn_bwd_workspace_bytes(B, H, N))


def attn_bwd_atomic_workspace_bytes(B, H, N, d):
    return int(_load().attn_bwd_atomic_workspace_bytes(B, H, N, d))


def attn_bwd(q, k, v, o, dO, lse, scale=None, causal=False, dq=None, dk=None, dv=None, workspace=None):
    """dQ, dK, dV of attention from the forward's saved O and LSE.

    Returns (dq, dk, dv, workspace); the workspace starts with D = rowsum(dO o O)
    (B*H*N fp32 values).
    """
    return _bwd_call("attn_bwd", q, k, v, o, dO, lse, scale, causal, dq, dk, dv, workspace)


def attn_bwd_atomic_dq(q, k, v, o, dO, lse, scale=None, causal=False, dq=None, dk=None, dv=None, workspace=None):
    """As attn_bwd, with dQ accumulated by fp32 atomic adds in the dK/dV pass
    (dq is not bitwise reproducible).  Returns (dq, dk, dv, workspace)."""
    return _bwd_call("attn_bwd_atomic_dq", q, k, v, o, dO, lse, scale, causal, dq, dk, dv, workspace)


def _bwd_call(entry, q, k, v, o, dO, lse, scale, causal, dq, dk, dv, workspace):
    B, H, N, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dO", dO)):
        _check_bhnd(name, t, (B, H, N, d), q.dtype, dev)
    _check_bhnd("lse", lse, (B, H, N), torch.float32, dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_bhnd(name, t, (B, H, N, d), q.dtype, dev)
    if entry == "attn_bwd":
        need = attn_bwd_workspace_bytes(B, H, N)
    else:
        need = attn_bwd_atomic_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty((need + 3) // 4, dtype=torch.float32, device=dev)
    else:
        _require(workspace.is_cuda and workspace.device == dev, f"workspace must be on {dev}")
        _require(workspace.is_contiguous(), "workspace must be contiguous")
    st = getattr(_load(), entry)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse), _ptr(dq), _ptr(dk),
                                 _ptr(dv), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 B, H, N, d, _dtype_code(q), scale, int(bool(causal)), _stream(dev))
    _check(st, entry)
    return dq, dk, dv, workspace
