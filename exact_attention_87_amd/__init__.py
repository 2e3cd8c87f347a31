"""Exact attention for AMD Instinct MI355X (gfx950): Python binding.

A thin ctypes layer over ``libattn.so`` (the C ABI in ``include/attn.h``).
Every step of the computation runs in the library's HIP kernels; this module
only marshals arguments.  PyTorch provides device memory and the stream.

Raw entry points with the C names (``attn_fwd``, ``attn_bwd`` and its
stages, ``attn_fwd_splitkv``, ``attn_fwd_blocksparse``, ``attn_fwd_varlen``, the
workspace-size queries,
``attn_status_str``, ``attn_abi_version``) take integer device addresses;
``fwd``, ``fwd_splitkv``, ``fwd_blocksparse``, ``fwd_varlen`` and ``bwd`` are
conveniences over torch tensors.  Importing this package never falls back to another implementation:
if the library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

ATTN_OK = 0
ATTN_ERR_INVALID_ARG = 1
ATTN_ERR_UNSUPPORTED = 2
ATTN_ERR_UNSUPPORTED_DEVICE = 3
ATTN_ERR_HIP = 4
ATTN_F32 = 0
ATTN_BF16 = 1
ATTN_F16 = 2

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {attn_status_str(status)}")


def lib():
    """The loaded libattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m exact_attention_87_amd._build`; "
                "there is no fallback implementation")
        L = ctypes.CDLL(LIB_PATH)
        vp, ci, cf, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.attn_abi_version.argtypes = []
        L.attn_abi_version.restype = ci
        L.attn_status_str.argtypes = [ci]
        L.attn_status_str.restype = ctypes.c_char_p
        L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, ci, vp]
        L.attn_fwd.restype = ci
        L.attn_bwd_workspace_bytes.argtypes = [ci, ci, ci, ci, ci, ci]
        L.attn_bwd_workspace_bytes.restype = sz
        L.attn_bwd.argtypes = [vp] * 10 + [ci, ci, ci, ci, ci, ci, cf, ci, vp]
        L.attn_bwd.restype = ci
        L.attn_bwd_noalloc.argtypes = [vp] * 9 + [ci, ci, ci, ci, ci, ci, cf, ci, vp]
        L.attn_bwd_noalloc.restype = ci
        L.attn_probe_clock.argtypes = [vp, ci, ctypes.c_uint, vp]
        L.attn_probe_clock.restype = ci
        L.attn_bwd_preprocess.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, ci, vp]
        L.attn_bwd_preprocess.restype = ci
        L.attn_bwd_dkdv.argtypes = [vp] * 7 + [ci, ci, ci, ci, ci, ci, cf, ci, vp]
        L.attn_bwd_dkdv.restype = ci
        L.attn_bwd_dq.argtypes = [vp] * 6 + [ci, ci, ci, ci, ci, ci, cf, ci, vp]
        L.attn_bwd_dq.restype = ci
        L.attn_bwd_dq_stats.argtypes = [vp] * 8 + [ci, ci, ci, ci, ci, ci, cf, ci, vp]
        L.attn_bwd_dq_stats.restype = ci
        L.attn_fwd_varlen_strided.argtypes = [vp] * 7 + [ci] * 7 + [cf, ci, vp]
        L.attn_fwd_varlen_strided.restype = ci
        L.attn_bwd_varlen_strided.argtypes = [vp] * 12 + [ci] * 7 + [cf, ci, vp]
        L.attn_bwd_varlen_strided.restype = ci
        L.attn_fwd_splitkv_strided.argtypes = [vp] * 7 + [ci] * 7 + [cf, ci, ci, vp]
        L.attn_fwd_splitkv_strided.restype = ci
        L.attn_fwd_splitkv.argtypes = [vp] * 6 + [ci] * 7 + [cf, ci, ci, vp]
        L.attn_fwd_splitkv.restype = ci
        L.attn_fwd_splitkv_num_splits.argtypes = [ci] * 7
        L.attn_fwd_splitkv_num_splits.restype = ci
        L.attn_fwd_splitkv_workspace_bytes.argtypes = [ci] * 7
        L.attn_fwd_splitkv_workspace_bytes.restype = sz
        L.attn_fwd_blocksparse.argtypes = [vp] * 6 + [ci, vp] + [ci] * 6 + [cf, ci, vp]
        L.attn_fwd_blocksparse_strided.argtypes = [vp] * 6 + [ci, vp, vp] + [ci] * 6 + [cf, ci, vp]
        L.attn_fwd_blocksparse_strided.restype = ci
        L.attn_fwd_blocksparse.restype = ci
        L.attn_fwd_blocksparse_workspace_bytes.argtypes = [ci, ci, ci]
        L.attn_fwd_blocksparse_workspace_bytes.restype = sz
        L.attn_fwd_varlen.argtypes = [vp] * 6 + [ci] * 7 + [cf, ci, vp]
        L.attn_fwd_varlen.restype = ci
        L.attn_fwd_strided.argtypes = [vp] * 6 + [ci] * 6 + [cf, ci, vp]
        L.attn_fwd_strided.restype = ci
        L.attn_bwd_strided.argtypes = [vp] * 11 + [ci] * 6 + [cf, ci, vp]
        L.attn_bwd_strided.restype = ci
        L.attn_bwd_varlen.argtypes = [vp] * 11 + [ci] * 7 + [cf, ci, vp]
        L.attn_bwd_varlen.restype = ci
        _lib = L
    return _lib


# ------------------------------------------------------------ raw C entry points
def attn_abi_version() -> int:
    return int(lib().attn_abi_version())


def attn_status_str(status: int) -> str:
    return lib().attn_status_str(int(status)).decode()


def attn_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, dtype, stream) -> int:
    return int(lib().attn_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, int(causal), float(scale),
                              int(dtype), stream))


def attn_bwd_workspace_bytes(B, Hq, Hkv, N, d, dtype) -> int:
    n = int(lib().attn_bwd_workspace_bytes(B, Hq, Hkv, N, d, int(dtype)))
    return -1 if n == (1 << 64) - 1 else n


def attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, Hq, Hkv, N, d, causal, scale,
             dtype, stream) -> int:
    return int(lib().attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, Hq, Hkv, N, d,
                              int(causal), float(scale), int(dtype), stream))


def attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, causal, scale, dtype,
                     stream) -> int:
    return int(lib().attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d,
                                      int(causal), float(scale), int(dtype), stream))


def attn_probe_clock(out, nwg, ticks, stream) -> int:
    return int(lib().attn_probe_clock(out, int(nwg), int(ticks), stream))


# Bytes of the static device scratch attn_bwd_noalloc uses (ATTN_NOALLOC_SCRATCH_BYTES).
ATTN_NOALLOC_SCRATCH_BYTES = 32 << 20


def attn_bwd_preprocess(o, dout, lse, stats, B, Hq, N, d, dtype, stream) -> int:
    return int(lib().attn_bwd_preprocess(o, dout, lse, stats, B, Hq, N, d, int(dtype), stream))


def attn_bwd_dkdv(q, k, v, dout, stats, dk, dv, B, Hq, Hkv, N, d, causal, scale, dtype,
                  stream) -> int:
    return int(lib().attn_bwd_dkdv(q, k, v, dout, stats, dk, dv, B, Hq, Hkv, N, d,
                                   int(causal), float(scale), int(dtype), stream))


def attn_bwd_dq(q, k, v, dout, stats, dq, B, Hq, Hkv, N, d, causal, scale, dtype,
                stream) -> int:
    return int(lib().attn_bwd_dq(q, k, v, dout, stats, dq, B, Hq, Hkv, N, d, int(causal),
                                 float(scale), int(dtype), stream))


def attn_bwd_dq_stats(q, k, v, o, lse, dout, stats, dq, B, Hq, Hkv, N, d, causal, scale, dtype,
                      stream) -> int:
    return int(lib().attn_bwd_dq_stats(q, k, v, o, lse, dout, stats, dq, B, Hq, Hkv, N, d,
                                       int(causal), float(scale), int(dtype), stream))


def attn_fwd_splitkv(q, k, v, o, lse, workspace, B, Hq, Hkv, Nq, Nk, d, causal, scale,
                     num_splits, dtype, stream) -> int:
    return int(lib().attn_fwd_splitkv(q, k, v, o, lse, workspace, B, Hq, Hkv, Nq, Nk, d,
                                      int(causal), float(scale), int(num_splits), int(dtype),
                                      stream))


def attn_fwd_splitkv_strided(q, k, v, o, lse, workspace, strides, B, Hq, Hkv, Nq, Nk, d, causal,
                             scale, num_splits, dtype, stream) -> int:
    """strides: 9 element strides (q_b, q_h, q_row, kv_b, kv_h, kv_row, o_b, o_h, o_row)."""
    arr = (ctypes.c_longlong * 9)(*[int(x) for x in strides])
    return int(lib().attn_fwd_splitkv_strided(q, k, v, o, lse, workspace, arr, B, Hq, Hkv, Nq, Nk,
                                              d, int(causal), float(scale), int(num_splits),
                                              int(dtype), stream))


def attn_fwd_splitkv_num_splits(B, Hq, Hkv, Nq, Nk, d, num_splits) -> int:
    return int(lib().attn_fwd_splitkv_num_splits(B, Hq, Hkv, Nq, Nk, d, int(num_splits)))


def attn_fwd_splitkv_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, num_splits) -> int:
    n = int(lib().attn_fwd_splitkv_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, int(num_splits)))
    return -1 if n == (1 << 64) - 1 else n


SPARSE_BLOCK_Q = 128  # ATTN_SPARSE_BLOCK_Q
SPARSE_BLOCK_K = 64   # ATTN_SPARSE_BLOCK_K


def attn_fwd_blocksparse(q, k, v, o, lse, block_mask, mask_heads, workspace, B, Hq, Hkv, N, d,
                         causal, scale, dtype, stream) -> int:
    return int(lib().attn_fwd_blocksparse(q, k, v, o, lse, block_mask, int(mask_heads), workspace,
                                          B, Hq, Hkv, N, d, int(causal), float(scale), int(dtype),
                                          stream))


def attn_fwd_blocksparse_strided(q, k, v, o, lse, block_mask, mask_heads, workspace, strides, B, Hq,
                                 Hkv, N, d, causal, scale, dtype, stream) -> int:
    """strides: 9 element strides (q_b, q_h, q_row, kv_b, kv_h, kv_row, o_b, o_h, o_row)."""
    arr = (ctypes.c_longlong * 9)(*[int(x) for x in strides])
    return int(lib().attn_fwd_blocksparse_strided(q, k, v, o, lse, block_mask, mask_heads,
                                                  workspace, arr, B, Hq, Hkv, N, d, int(causal),
                                                  float(scale), int(dtype), stream))


def attn_fwd_blocksparse_workspace_bytes(Hq, N, mask_heads) -> int:
    n = int(lib().attn_fwd_blocksparse_workspace_bytes(Hq, N, int(mask_heads)))
    return -1 if n == (1 << 64) - 1 else n


def attn_fwd_varlen(q, k, v, o, lse, cu_seqlens, nseq, max_seqlen, Hq, Hkv, T, d, causal, scale,
                    dtype, stream) -> int:
    return int(lib().attn_fwd_varlen(q, k, v, o, lse, cu_seqlens, nseq, max_seqlen, Hq, Hkv, T, d,
                                     int(causal), float(scale), int(dtype), stream))


def attn_fwd_strided(q, k, v, o, lse, strides, B, Hq, Hkv, N, d, causal, scale, dtype,
                     stream) -> int:
    """strides: 9 element strides (q_b, q_h, q_row, kv_b, kv_h, kv_row, o_b, o_h, o_row)."""
    arr = (ctypes.c_longlong * 9)(*[int(x) for x in strides])
    return int(lib().attn_fwd_strided(q, k, v, o, lse, arr, B, Hq, Hkv, N, d, int(causal),
                                      float(scale), int(dtype), stream))


def attn_bwd_strided(q, k, v, o, lse, dout, dq, dk, dv, workspace, strides, B, Hq, Hkv, N, d,
                     causal, scale, dtype, stream) -> int:
    """strides: 9 element strides (q/dq, k/v/dk/dv, o/dout; batch, head, row each)."""
    arr = (ctypes.c_longlong * 9)(*[int(x) for x in strides])
    return int(lib().attn_bwd_strided(q, k, v, o, lse, dout, dq, dk, dv, workspace, arr, B, Hq,
                                      Hkv, N, d, int(causal), float(scale), int(dtype), stream))


def attn_bwd_varlen(q, k, v, o, lse, dout, dq, dk, dv, workspace, cu_seqlens, nseq, max_seqlen,
                    Hq, Hkv, T, d, causal, scale, dtype, stream) -> int:
    return int(lib().attn_bwd_varlen(q, k, v, o, lse, dout, dq, dk, dv, workspace, cu_seqlens,
                                     nseq, max_seqlen, Hq, Hkv, T, d, int(causal), float(scale),
                                     int(dtype), stream))


def attn_fwd_varlen_strided(q, k, v, o, lse, cu_seqlens, strides, nseq, max_seqlen, Hq, Hkv, T, d,
                            causal, scale, dtype, stream) -> int:
    """strides: 6 element strides (q_h, q_t, kv_h, kv_t, o_h, o_t)."""
    arr = (ctypes.c_longlong * 6)(*[int(x) for x in strides])
    return int(lib().attn_fwd_varlen_strided(q, k, v, o, lse, cu_seqlens, arr, nseq, max_seqlen,
                                             Hq, Hkv, T, d, int(causal), float(scale), int(dtype),
                                             stream))


def attn_bwd_varlen_strided(q, k, v, o, lse, dout, dq, dk, dv, workspace, cu_seqlens, strides, nseq,
                            max_seqlen, Hq, Hkv, T, d, causal, scale, dtype, stream) -> int:
    """strides: 6 element strides (q/dq, k/v/dk/dv, o/dout; head, token each)."""
    arr = (ctypes.c_longlong * 6)(*[int(x) for x in strides])
    return int(lib().attn_bwd_varlen_strided(q, k, v, o, lse, dout, dq, dk, dv, workspace,
                                             cu_seqlens, arr, nseq, max_seqlen, Hq, Hkv, T, d,
                                             int(causal), float(scale), int(dtype), stream))


# ------------------------------------------------------------ torch conveniences
def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float16:
        return ATTN_F16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.bfloat16, torch.float16 or "
                    "torch.float32")


def _check_qkv(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, N, d]")
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    B, Hq, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError("k and v must be [B, Hkv, N, d] matching q")
    return B, Hq, k.shape[1], N, d


def _stream_ptr(t) -> int:
    import torch

    return torch.cuda.current_stream(t.device).cuda_stream


def fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None):
    """O, LSE = attention forward of device tensors q [B,Hq,N,d], k/v [B,Hkv,N,d]."""
    import torch

    B, Hq, Hkv, N, d = _check_qkv(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, N), device=q.device, dtype=torch.float32)
    st = attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                  B, Hq, Hkv, N, d, causal, scale, _dtype_code(q), _stream_ptr(q))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd")
    return out, lse


def fwd_splitkv(q, k, v, causal: bool = False, scale: float | None = None,
                num_splits: int = 0, out=None, lse=None, workspace=None):
    """O, LSE for q [B,Hq,Nq,d] against a key/value cache k/v [B,Hkv,Nk,d] (16-bit),
    with the keys cut into num_splits ranges (0: chosen from the shape) and the
    causal mask aligned to the last query.  q, k, v (and out) may be
    [B, H, N, d] views of any (batch, head, row) strides, e.g. a token-major
    [B, Nk, Hkv, d] cache transposed; out defaults to q's layout when q is
    contiguous, else to a [B, Nq, Hq, d] tensor viewed as [B, Hq, Nq, d]."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, N, d]")
        if not t.is_cuda or t.stride(3) != 1:
            raise ValueError(f"{name} must be a device tensor with contiguous d")
    if not _same_strides(k, v):
        raise ValueError("k and v must share strides")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k and v must be [B, Hkv, Nk, d] matching q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    code = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q) if q.is_contiguous() else \
            torch.empty((B, Nq, Hq, d), device=q.device, dtype=q.dtype).transpose(1, 2)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), device=q.device, dtype=torch.float32)
    nbytes = attn_fwd_splitkv_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, num_splits)
    if nbytes < 0:
        raise AttnError(ATTN_ERR_UNSUPPORTED, "attn_fwd_splitkv_workspace_bytes")
    if workspace is None or workspace.numel() * workspace.element_size() < nbytes:
        workspace = torch.empty(max(nbytes, 256), device=q.device, dtype=torch.uint8)
    if all(t.is_contiguous() for t in (q, k, v, out)):
        st = attn_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              lse.data_ptr(), workspace.data_ptr(), B, Hq, Hkv, Nq, Nk, d, causal,
                              scale, num_splits, code, _stream_ptr(q))
        what = "attn_fwd_splitkv"
    else:
        strides = _bhnd_strides(q) + _bhnd_strides(k) + _bhnd_strides(out)
        st = attn_fwd_splitkv_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                      lse.data_ptr(), workspace.data_ptr(), strides, B, Hq, Hkv,
                                      Nq, Nk, d, causal, scale, num_splits, code, _stream_ptr(q))
        what = "attn_fwd_splitkv_strided"
    if st != ATTN_OK:
        raise AttnError(st, what)
    return out, lse


def fwd_blocksparse(q, k, v, block_mask, causal: bool = False, scale: float | None = None,
                    out=None, lse=None, workspace=None):
    """O, LSE of the block-sparse forward: block_mask is a device uint8 tensor
    [1 or Hq, ceil(N/128), ceil(N/64)] over tiles of 128 queries x 64 keys.
    q, k, v (and out) may be [B, H, N, d] views of any strides, as for
    fwd_strided (out then defaults to a [B, N, Hq, d] tensor)."""
    import torch

    dense = all(t.is_contiguous() for t in (q, k, v)) and (out is None or out.is_contiguous())
    if dense:
        B, Hq, Hkv, N, d = _check_qkv(q, k, v)
    else:
        for name, t in (("q", q), ("k", k), ("v", v)):
            if t.dim() != 4 or not t.is_cuda:
                raise ValueError(f"{name} must be a 4-D device tensor [B, H, N, d]")
        if not _same_strides(k, v):
            raise ValueError("k and v must share shape and strides")
        B, Hq, N, d = q.shape
        Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nqb, nkt = -(-N // SPARSE_BLOCK_Q), -(-N // SPARSE_BLOCK_K)
    if (block_mask.dtype != torch.uint8 or not block_mask.is_cuda or block_mask.dim() != 3
            or block_mask.shape[1:] != (nqb, nkt) or not block_mask.is_contiguous()):
        raise ValueError(f"block_mask must be a contiguous device uint8 [1 or Hq, {nqb}, {nkt}]")
    mh = block_mask.shape[0]
    if out is None:
        out = torch.empty_like(q) if dense else \
            torch.empty((B, N, Hq, d), device=q.device, dtype=q.dtype).transpose(1, 2)
    if lse is None:
        lse = torch.empty((B, Hq, N), device=q.device, dtype=torch.float32)
    nbytes = attn_fwd_blocksparse_workspace_bytes(Hq, N, mh)
    if nbytes < 0:
        raise AttnError(ATTN_ERR_INVALID_ARG, "attn_fwd_blocksparse_workspace_bytes")
    if workspace is None or workspace.numel() * workspace.element_size() < nbytes:
        workspace = torch.empty(max(nbytes, 256), device=q.device, dtype=torch.uint8)
    if dense:
        st = attn_fwd_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                  lse.data_ptr(), block_mask.data_ptr(), mh, workspace.data_ptr(),
                                  B, Hq, Hkv, N, d, causal, scale, _dtype_code(q), _stream_ptr(q))
        what = "attn_fwd_blocksparse"
    else:
        strides = _bhnd_strides(q) + _bhnd_strides(k) + _bhnd_strides(out)
        st = attn_fwd_blocksparse_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                          out.data_ptr(), lse.data_ptr(), block_mask.data_ptr(),
                                          mh, workspace.data_ptr(), strides, B, Hq, Hkv, N, d,
                                          causal, scale, _dtype_code(q), _stream_ptr(q))
        what = "attn_fwd_blocksparse_strided"
    if st != ATTN_OK:
        raise AttnError(st, what)
    return out, lse


def _ht_strides(t):
    """(head, token) element strides of an [H, T, d] view with a unit stride in d."""
    if t.dim() != 3 or t.stride(2) != 1:
        raise ValueError("tensors must be 3-D [H, T, d] views with contiguous d")
    return [t.stride(0), t.stride(1)]


def _check_cu(cu_seqlens):
    import torch

    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be a device int32 vector")


def fwd_varlen(q, k, v, cu_seqlens, max_seqlen: int, causal: bool = False,
               scale: float | None = None, out=None, lse=None):
    """O [Hq,T,d], LSE [Hq,T] of packed sequences: q [Hq,T,d], k/v [Hkv,T,d] (16-bit),
    cu_seqlens a device int32 tensor of nseq+1 token offsets.  q, k, v (and out)
    may be [H, T, d] views of any (head, token) strides, e.g. [T, H, d] tensors
    transposed; then out defaults to a [T, Hq, d] tensor viewed as [Hq, T, d]."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 3 or not t.is_cuda or t.stride(2) != 1:
            raise ValueError(f"{name} must be a device tensor [H, T, d] with contiguous d")
    Hq, T, d = q.shape
    Hkv = k.shape[0]
    if k.shape != v.shape or k.shape[1:] != (T, d):
        raise ValueError("k and v must be [Hkv, T, d] matching q")
    if not _same_strides(k, v):
        raise ValueError("k and v must share strides")
    _check_cu(cu_seqlens)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dense = all(t.is_contiguous() for t in (q, k, v)) and (out is None or out.is_contiguous())
    if out is None:
        out = torch.empty_like(q) if dense else \
            torch.empty((T, Hq, d), device=q.device, dtype=q.dtype).transpose(0, 1)
    if lse is None:
        lse = torch.empty((Hq, T), device=q.device, dtype=torch.float32)
    nseq = cu_seqlens.numel() - 1
    if dense:
        st = attn_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             lse.data_ptr(), cu_seqlens.data_ptr(), nseq, int(max_seqlen), Hq, Hkv,
                             T, d, causal, scale, _dtype_code(q), _stream_ptr(q))
        what = "attn_fwd_varlen"
    else:
        strides = _ht_strides(q) + _ht_strides(k) + _ht_strides(out)
        st = attn_fwd_varlen_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                     lse.data_ptr(), cu_seqlens.data_ptr(), strides, nseq,
                                     int(max_seqlen), Hq, Hkv, T, d, causal, scale,
                                     _dtype_code(q), _stream_ptr(q))
        what = "attn_fwd_varlen_strided"
    if st != ATTN_OK:
        raise AttnError(st, what)
    return out, lse


def _same_strides(a, b) -> bool:
    """Whether two tensors of one shape lay out their elements alike.  The
    stride of a dimension of size 1 never multiplies a nonzero index, so it is
    not compared (torch gives such dimensions different strides depending on
    how a tensor was made, e.g. a token-major [B, N, 1, d] tensor viewed as
    [B, 1, N, d])."""
    return tuple(a.shape) == tuple(b.shape) and all(
        sa == sb for sa, sb, n in zip(a.stride(), b.stride(), a.shape) if n > 1)


def _bhnd_strides(t):
    """(batch, head, row) element strides of a [B, H, N, d] view with a unit
    stride in d (any permutation of the first three axes in memory)."""
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("tensors must be 4-D [B, H, N, d] views with contiguous d")
    return [t.stride(0), t.stride(1), t.stride(2)]


def fwd_strided(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None):
    """Forward on [B, H, N, d] views of any (batch, head, row) strides, such as
    [B, N, H, d] tensors transposed to [B, H, N, d] or slices of a packed QKV
    projection.  k and v must share strides; out defaults to a [B, N, Hq, d]
    tensor viewed as [B, Hq, N, d]."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 4 or not t.is_cuda:
            raise ValueError(f"{name} must be a 4-D device tensor [B, H, N, d]")
    if not _same_strides(k, v):
        raise ValueError("k and v must share shape and strides")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, N, Hq, d), device=q.device, dtype=q.dtype).transpose(1, 2)
    if lse is None:
        lse = torch.empty((B, Hq, N), device=q.device, dtype=torch.float32)
    strides = _bhnd_strides(q) + _bhnd_strides(k) + _bhnd_strides(out)
    st = attn_fwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                          strides, B, Hq, Hkv, N, d, causal, scale, _dtype_code(q), _stream_ptr(q))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_strided")
    return out, lse


def bwd_strided(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None,
                dq=None, dk=None, dv=None, workspace=None):
    """dQ, dK, dV for [B, H, N, d] views of any strides (q and dq share strides,
    k, v, dk, dv share strides, o and dout share strides).  Gradients default
    to new tensors with their input's strides (for slices of a packed buffer,
    pass slices of a packed gradient buffer instead)."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        if t.dim() != 4 or not t.is_cuda:
            raise ValueError(f"{name} must be a 4-D device tensor [B, H, N, d]")
    if not (_same_strides(k, v) and _same_strides(o, dout)):
        raise ValueError("k/v and o/dout must share strides")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)

    def like(t, grad):
        if grad is not None:
            if not _same_strides(grad, t):
                raise ValueError("gradients must have their input's shape and strides")
            return grad
        return torch.empty_strided(t.shape, t.stride(), device=t.device, dtype=t.dtype)

    dq, dk, dv = like(q, dq), like(k, dk), like(v, dv)
    code = _dtype_code(q)
    nbytes = attn_bwd_workspace_bytes(B, Hq, Hkv, N, d, code)
    if nbytes < 0:
        raise AttnError(ATTN_ERR_UNSUPPORTED, "attn_bwd_workspace_bytes")
    if workspace is None or workspace.numel() * workspace.element_size() < nbytes:
        workspace = torch.empty(max(nbytes, 256), device=q.device, dtype=torch.uint8)
    strides = _bhnd_strides(q) + _bhnd_strides(k) + _bhnd_strides(o)
    st = attn_bwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                          dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                          workspace.data_ptr(), strides, B, Hq, Hkv, N, d, causal, scale, code,
                          _stream_ptr(q))
    if st != ATTN_OK:
        raise AttnError(st, "attn_bwd_strided")
    return dq, dk, dv


def bwd_varlen(q, k, v, o, lse, dout, cu_seqlens, max_seqlen: int, causal: bool = False,
               scale: float | None = None, workspace=None, dq=None, dk=None, dv=None):
    """dQ [Hq,T,d], dK, dV [Hkv,T,d] of packed sequences (the forward's fwd_varlen
    tensors and offsets, upstream dO [Hq,T,d]).  Any (head, token) strides as in
    fwd_varlen (q/dq, k/v/dk/dv and o/dout each share strides); gradients
    default to new tensors with their input's strides."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        if t.dim() != 3 or not t.is_cuda or t.stride(2) != 1:
            raise ValueError(f"{name} must be a device tensor [H, T, d] with contiguous d")
    if not (_same_strides(k, v) and _same_strides(o, dout)):
        raise ValueError("k/v and o/dout must share strides")
    _check_cu(cu_seqlens)
    Hq, T, d = q.shape
    Hkv = k.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    code = _dtype_code(q)

    def like(t, grad):
        if grad is not None:
            if not _same_strides(grad, t):
                raise ValueError("gradients must have their input's shape and strides")
            return grad
        return torch.empty_strided(t.shape, t.stride(), device=t.device, dtype=t.dtype)

    dq, dk, dv = like(q, dq), like(k, dk), like(v, dv)
    nbytes = attn_bwd_workspace_bytes(1, Hq, Hkv, T, d, code)
    if nbytes < 0:
        raise AttnError(ATTN_ERR_UNSUPPORTED, "attn_bwd_workspace_bytes")
    if workspace is None or workspace.numel() * workspace.element_size() < nbytes:
        workspace = torch.empty(max(nbytes, 256), device=q.device, dtype=torch.uint8)
    nseq = cu_seqlens.numel() - 1
    ptrs = [t.data_ptr() for t in (q, k, v, o)] + [lse.data_ptr(), dout.data_ptr()] + \
        [t.data_ptr() for t in (dq, dk, dv, workspace)]
    if all(t.is_contiguous() for t in (q, k, v, o, dout)):
        st = attn_bwd_varlen(*ptrs, cu_seqlens.data_ptr(), nseq, int(max_seqlen), Hq, Hkv, T, d,
                             causal, scale, code, _stream_ptr(q))
        what = "attn_bwd_varlen"
    else:
        strides = _ht_strides(q) + _ht_strides(k) + _ht_strides(o)
        st = attn_bwd_varlen_strided(*ptrs, cu_seqlens.data_ptr(), strides, nseq, int(max_seqlen),
                                     Hq, Hkv, T, d, causal, scale, code, _stream_ptr(q))
        what = "attn_bwd_varlen_strided"
    if st != ATTN_OK:
        raise AttnError(st, what)
    return dq, dk, dv


def bwd(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None,
        workspace=None):
    """dQ, dK, dV of attention given the forward's O and LSE and upstream dO."""
    import torch

    B, Hq, Hkv, N, d = _check_qkv(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    code = _dtype_code(q)
    for name, t in (("o", o), ("dout", dout)):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError(f"{name} must match q")
    if lse.shape != (B, Hq, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be contiguous fp32 [B, Hq, N]")
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    nbytes = attn_bwd_workspace_bytes(B, Hq, Hkv, N, d, code)
    if nbytes < 0:
        raise AttnError(ATTN_ERR_UNSUPPORTED, "attn_bwd_workspace_bytes")
    if workspace is None or workspace.numel() * workspace.element_size() < nbytes:
        workspace = torch.empty(max(nbytes, 256), device=q.device, dtype=torch.uint8)
    st = attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                  dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                  workspace.data_ptr(), B, Hq, Hkv, N, d, causal, scale, code, _stream_ptr(q))
    if st != ATTN_OK:
        raise AttnError(st, "attn_bwd")
    return dq, dk, dv
