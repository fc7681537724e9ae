"""Python binding of the MI355X fused softmax-attention library (libattn_mi355x.so).

Argument marshalling only: tensors are checked and allocated with PyTorch (ROCm)
for device memory, and every step of the computation runs in the library's HIP
kernels on the current PyTorch stream.  There is no CPU path: if the library is
not built, or a tensor is not on the GPU, these functions raise.

    attn_fwd(q, k, v, causal, scale)                  -> (o, lse)
    attn_fwd_varlen(q, k, v, cu_q, cu_k, max_q, ...)  -> (o, lse)
    attn_decode_splitkv(q, k, v, scale, num_splits=0) -> (o, lse)
    attn_decode_splitkv_fused(q, k, v, scale, num_splits=0)  -> (o, lse)
    attn_decode_splitkv_fp8(q, k8, v8, k_scale, v_scale, ...) -> (o, lse)
    attn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, max_seq_len) -> (o, lse)
    attn_fwd_varlen_paged(q, k_cache, v_cache, block_table, cu_q, seq_lens_k, max_q, max_k, ...) -> (o, lse)
    attn_bwd(q, k, v, o, dout, lse, causal, scale)    -> (dq, dk, dv)

Layouts are [B, H, N, d] contiguous (q/o/dout/dq with Hq heads, k/v/dk/dv with
Hkv heads); lse is [B, Hq, Nq] fp32; gradients are fp32.  The variable-length
forward takes packed [H, total, d] tensors and int32 sequence offsets.  See
include/attn.h.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn_mi355x.so")

ATTN_OK, ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE, ATTN_ERR_HIP, ATTN_ERR_SCRATCH = range(6)
DECODE_SCRATCH_BYTES = 8 << 20  # ATTN_DECODE_SCRATCH_BYTES
ATTN_F32, ATTN_BF16 = 0, 1

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {strerror(status)} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m attention_online_softmax_attn_amd.build`"
        )
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, f32, ci, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_size_t
    L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, f32, ci, ci, vp]
    L.attn_fwd.restype = ci
    L.attn_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, f32, ci, ci, vp]
    L.attn_fwd_varlen.restype = ci
    L.attn_decode_num_splits.argtypes = [i64, i64, i64, i64, i64]
    L.attn_decode_num_splits.restype = ci
    L.attn_decode_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, ci]
    L.attn_decode_workspace_bytes.restype = sz
    L.attn_decode_splitkv.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, f32, ci, ci, vp, sz, ci, vp]
    L.attn_decode_splitkv.restype = ci
    L.attn_decode_fused_num_splits.argtypes = [i64, i64, i64, i64, i64]
    L.attn_decode_fused_num_splits.restype = ci
    L.attn_decode_fused_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, ci]
    L.attn_decode_fused_workspace_bytes.restype = sz
    L.attn_decode_splitkv_fused.argtypes = L.attn_decode_splitkv.argtypes
    L.attn_decode_splitkv_fused.restype = ci
    L.attn_decode_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, f32, ci, ci, ci, vp]
    L.attn_decode_splitkv_noalloc.restype = ci
    L.attn_decode_noalloc_scratch_bytes.argtypes = [i64, i64, i64, i64, i64, ci]
    L.attn_decode_noalloc_scratch_bytes.restype = sz
    L.attn_fwd_varlen_paged.argtypes = [vp] * 8 + [i64] * 10 + [f32, ci, vp]
    L.attn_fwd_varlen_paged.restype = ci
    L.attn_decode_paged.argtypes = [vp] * 7 + [i64] * 8 + [f32, ci, vp, sz, vp]
    L.attn_decode_paged.restype = ci
    L.attn_decode_paged_fused.argtypes = L.attn_decode_paged.argtypes
    L.attn_decode_paged_fused.restype = ci
    L.attn_decode_paged_fused_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, ci]
    L.attn_decode_paged_fused_workspace_bytes.restype = sz
    L.attn_decode_splitkv_fp8.argtypes = [vp] * 7 + [i64] * 6 + [f32, ci, vp, sz, vp]
    L.attn_decode_splitkv_fp8.restype = ci
    L.attn_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64]
    L.attn_bwd_workspace_bytes.restype = sz
    L.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, f32, ci, vp, sz, ci, vp]
    L.attn_bwd.restype = ci
    L.attn_bwd_bf16_grads.argtypes = L.attn_bwd.argtypes
    L.attn_bwd_bf16_grads.restype = ci
    L.attn_strerror.argtypes = [ci]
    L.attn_strerror.restype = ctypes.c_char_p
    _lib = L
    return L


def strerror(status: int) -> str:
    return lib().attn_strerror(int(status)).decode()


def _ptr(t):
    # a plain int: the argtypes declare c_void_p, which converts it
    return None if t is None else t.data_ptr()


# torch's current stream of the current device as a raw handle: the
# C-level getter returns the same handle as current_stream().cuda_stream
# without building a Stream object (2.8 of the 9.6 us a tiny forward call
# spent on the host); the public form serves where the getter is absent
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream():
    if _raw_stream is not None:
        return _raw_stream(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use bfloat16 or float32")


def _check_dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU; there is no CPU path")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, H, N, d]")


def _dims(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, N, d]")
    B, Hq, Nq, d = q.shape
    if k.shape[0] != B or k.shape[3] != d or v.shape != k.shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise TypeError("q, k, v must share one dtype")
    return B, Hq, k.shape[1], Nq, k.shape[2], d


def _want(t, shape, dtype, name: str):
    """A caller-supplied buffer must have exactly the shape and dtype the call
    writes or reads: the kernels take its address and trust the sizes."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, not {t.dtype}")


def _scale(scale, d):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def attn_fwd(q, k, v, causal: bool = False, scale=None, out=None, lse=None, want_lse: bool = True):
    """Fused forward.  Returns (o, lse); lse is None when want_lse is False."""
    _check_dev(q, k, v, out, lse)
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v)
    _want(out, q.shape, q.dtype, "out")
    _want(lse, (B, Hq, Nq), torch.float32, "lse")
    o = torch.empty_like(q) if out is None else out
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    st = lib().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse) if want_lse else None, B, Hq, Hkv, Nq, Nk,
                        d, _scale(scale, d), int(bool(causal)), _dtype_code(q), _stream())
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd")
    return o, (lse if want_lse else None)


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, causal: bool = False, scale=None,
                    out=None, lse=None, want_lse: bool = True):
    """Forward over a packed batch of variable-length sequences.

    q [Hq, total_q, d], k/v [Hkv, total_k, d] (bf16); cu_seqlens_q/_k int32
    [n_seqs + 1] device offsets of each sequence's rows; max_seqlen_q at least
    the longest query length.  Returns (o [Hq, total_q, d], lse [Hq, total_q])."""
    _check_dev(q, k, v, cu_seqlens_q, cu_seqlens_k, out, lse)
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be 3-D [H, total, d]")
    Hq, total_q, d = q.shape
    Hkv, total_k = k.shape[0], k.shape[1]
    if k.shape[2] != d or v.shape != k.shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise TypeError("q, k, v must share one dtype")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if cu_seqlens_q.dim() != 1 or cu_seqlens_k.shape != cu_seqlens_q.shape:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must be 1-D of the same length n_seqs + 1")
    n_seqs = cu_seqlens_q.shape[0] - 1
    _want(out, q.shape, q.dtype, "out")
    _want(lse, (Hq, total_q), torch.float32, "lse")
    o = torch.empty_like(q) if out is None else out
    if want_lse and lse is None:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    st = lib().attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse) if want_lse else None,
                               _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), n_seqs, total_q, total_k, int(max_seqlen_q),
                               Hq, Hkv, d, _scale(scale, d), int(bool(causal)), _dtype_code(q), _stream())
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_varlen")
    return o, (lse if want_lse else None)


def decode_num_splits(B: int, Hq: int, Hkv: int, Nk: int, d: int) -> int:
    return int(lib().attn_decode_num_splits(B, Hq, Hkv, Nk, d))


def decode_workspace_bytes(B: int, Hq: int, Hkv: int, Nk: int, d: int, num_splits: int = 0) -> int:
    return int(lib().attn_decode_workspace_bytes(B, Hq, Hkv, Nk, d, num_splits))


def attn_decode_splitkv(q, k, v, scale=None, num_splits: int = 0, workspace=None, out=None, lse=None,
                        want_lse: bool = True):
    """Split-KV decode (q has Nq = 1).  Returns (o, lse)."""
    _check_dev(q, k, v, out, lse, workspace)
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v)
    _want(out, q.shape, q.dtype, "out")
    _want(lse, (B, Hq, Nq), torch.float32, "lse")
    o = torch.empty_like(q) if out is None else out
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    if workspace is None:
        need = decode_workspace_bytes(B, Hq, Hkv, Nk, d, num_splits)
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().attn_decode_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse) if want_lse else None, B, Hq, Hkv,
                                   Nq, Nk, d, _scale(scale, d), 0, int(num_splits), _ptr(workspace), ws_bytes,
                                   _dtype_code(q), _stream())
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode_splitkv")
    return o, (lse if want_lse else None)


def decode_noalloc_scratch_bytes(B: int, Hq: int, Hkv: int, Nk: int, d: int, num_splits: int = 0) -> int:
    return int(lib().attn_decode_noalloc_scratch_bytes(B, Hq, Hkv, Nk, d, num_splits))


def attn_decode_splitkv_noalloc(q, k, v, out, lse=None, scale=None, num_splits: int = 0):
    """attn_decode_splitkv with the partial states in the library's fixed
    device scratch: no workspace, and the C call allocates nothing.  The
    caller passes the outputs (out like q; lse fp32 [B, Hq, 1] or None).
    Calls that overlap on one GPU race on the scratch."""
    _check_dev(q, k, v, out, lse)
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v)
    if out is None:
        raise ValueError("attn_decode_splitkv_noalloc: the caller passes out")
    _want(out, q.shape, q.dtype, "out")
    _want(lse, (B, Hq, Nq), torch.float32, "lse")
    st = lib().attn_decode_splitkv_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Nq, Nk, d,
                                           _scale(scale, d), 0, int(num_splits), _dtype_code(q), _stream())
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode_splitkv_noalloc")
    return out, lse


def decode_fused_num_splits(B: int, Hq: int, Hkv: int, Nk: int, d: int) -> int:
    return int(lib().attn_decode_fused_num_splits(B, Hq, Hkv, Nk, d))


def decode_fused_workspace_bytes(B: int, Hq: int, Hkv: int, Nk: int, d: int, num_splits: int = 0) -> int:
    return int(lib().attn_decode_fused_workspace_bytes(B, Hq, Hkv, Nk, d, num_splits))


def attn_decode_splitkv_fused(q, k, v, scale=None, num_splits: int = 0, workspace=None, out=None, lse=None,
                              want_lse: bool = True):
    """Split-KV decode in one launch (the last split to finish merges).  A
    workspace passed in must have been zeroed before its first use (its
    arrival counts are left zero by every call); without one a zeroed one is
    allocated.  Returns (o, lse)."""
    _check_dev(q, k, v, out, lse, workspace)
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v)
    _want(out, q.shape, q.dtype, "out")
    _want(lse, (B, Hq, Nq), torch.float32, "lse")
    o = torch.empty_like(q) if out is None else out
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    if workspace is None:
        need = decode_fused_workspace_bytes(B, Hq, Hkv, Nk, d, num_splits)
        if need > 0:
            workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().attn_decode_splitkv_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse) if want_lse else None, B, Hq,
                                         Hkv, Nq, Nk, d, _scale(scale, d), 0, int(num_splits), _ptr(workspace),
                                         ws_bytes, _dtype_code(q), _stream())
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode_splitkv_fused")
    return o, (lse if want_lse else None)


def attn_decode_splitkv_fp8(q, k8, v8, k_scale, v_scale, scale=None, num_splits: int = 0, workspace=None, out=None,
                            lse=None, want_lse: bool = True):
    """Split-KV decode over an FP8 KV cache.  q bf16 [B, Hq, 1, d]; k8, v8 uint8
    OCP E4M3 codes [B, Hkv, Nk, d]; k_scale, v_scale fp32 [Hkv] (value = scale *
    code).  Returns (o bf16 [B, Hq, 1, d], lse)."""
    _check_dev(q, k8, v8, k_scale, v_scale, out, lse, workspace)
    if q.dim() != 4 or k8.dim() != 4 or v8.shape != k8.shape:
        raise ValueError("q must be [B, Hq, 1, d] and k8, v8 [B, Hkv, Nk, d]")
    if k8.dtype != torch.uint8 or v8.dtype != torch.uint8:
        raise TypeError("k8 and v8 must hold uint8 E4M3 codes")
    if q.dtype != torch.bfloat16:
        raise TypeError("q must be bfloat16")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k8.shape[1], k8.shape[2]
    if k8.shape[0] != B or k8.shape[3] != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k8 {tuple(k8.shape)}")
    if k_scale.dtype != torch.float32 or v_scale.dtype != torch.float32 or k_scale.numel() != Hkv or v_scale.numel() != Hkv:
        raise ValueError("k_scale and v_scale must be fp32 with one value per kv head")
    _want(out, q.shape, q.dtype, "out")
    _want(lse, (B, Hq, Nq), torch.float32, "lse")
    o = torch.empty_like(q) if out is None else out
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    if workspace is None:
        need = decode_workspace_bytes(B, Hq, Hkv, Nk, d, num_splits)
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().attn_decode_splitkv_fp8(_ptr(q), _ptr(k8), _ptr(v8), _ptr(k_scale), _ptr(v_scale), _ptr(o),
                                       _ptr(lse) if want_lse else None, B, Hq, Hkv, Nq, Nk, d, _scale(scale, d),
                                       int(num_splits), _ptr(workspace), ws_bytes, _stream())
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode_splitkv_fp8")
    return o, (lse if want_lse else None)


def attn_fwd_varlen_paged(q, k_cache, v_cache, block_table, cu_seqlens_q, seq_lens_k, max_seqlen_q: int,
                          max_seqlen_k: int, causal: bool = True, scale=None, out=None, lse=None,
                          want_lse: bool = True):
    """Packed variable-length forward over a paged bf16 K/V cache.  q [Hq,
    total_q, d] packed; k_cache, v_cache [num_pages, Hkv, page_size, d];
    block_table int32 [n_seqs, max_pages]; cu_seqlens_q int32 [n_seqs + 1];
    seq_lens_k int32 [n_seqs].  Returns (o [Hq, total_q, d], lse [Hq, total_q])."""
    _check_dev(q, k_cache, v_cache, block_table, cu_seqlens_q, seq_lens_k, out, lse)
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape or block_table.dim() != 2:
        raise ValueError("q must be [Hq, total_q, d], the caches [num_pages, Hkv, page_size, d], "
                         "block_table [n_seqs, max_pages]")
    if q.dtype != torch.bfloat16 or k_cache.dtype != torch.bfloat16 or v_cache.dtype != torch.bfloat16:
        raise TypeError("q, k_cache and v_cache must be bfloat16")
    for t in (block_table, cu_seqlens_q, seq_lens_k):
        if t.dtype != torch.int32:
            raise TypeError("block_table, cu_seqlens_q and seq_lens_k must be int32")
    Hq, total_q, d = q.shape
    num_pages, Hkv, page, _ = k_cache.shape
    n = seq_lens_k.numel()
    if cu_seqlens_q.numel() != n + 1 or block_table.shape[0] != n or k_cache.shape[3] != d:
        raise ValueError("n_seqs + 1 query offsets, n_seqs key lengths and block-table rows expected")
    for t in (q, k_cache, v_cache, block_table, cu_seqlens_q, seq_lens_k):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    _want(out, q.shape, q.dtype, "out")
    _want(lse, (Hq, total_q), torch.float32, "lse")
    o = torch.empty_like(q) if out is None else out
    if want_lse and lse is None:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    st = lib().attn_fwd_varlen_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(o),
                                     _ptr(lse) if want_lse else None, _ptr(cu_seqlens_q), _ptr(seq_lens_k), n,
                                     total_q, int(max_seqlen_q), int(max_seqlen_k), Hq, Hkv, d, num_pages, page,
                                     block_table.shape[1], _scale(scale, d), int(bool(causal)), _stream())
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_varlen_paged")
    return o, (lse if want_lse else None)


def _paged_args(q, k_cache, v_cache, block_table, seq_lens, out, lse, workspace, want_lse):
    _check_dev(q, k_cache, v_cache, block_table, seq_lens, out, lse, workspace)
    if q.dim() != 4 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [B, Hq, 1, d] and k_cache, v_cache [num_pages, Hkv, page_size, d]")
    if q.dtype != torch.bfloat16 or k_cache.dtype != torch.bfloat16 or v_cache.dtype != torch.bfloat16:
        raise TypeError("q, k_cache and v_cache must be bfloat16")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32 or block_table.dim() != 2:
        raise TypeError("block_table must be int32 [B, max_pages] and seq_lens int32 [B]")
    B, Hq, Nq, d = q.shape
    num_pages, Hkv, page, _ = k_cache.shape
    if k_cache.shape[3] != d or block_table.shape[0] != B or seq_lens.numel() != B:
        raise ValueError("shape mismatch between q, the cache, block_table and seq_lens")
    for t in (q, k_cache, v_cache, block_table, seq_lens):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    _want(out, q.shape, q.dtype, "out")
    _want(lse, (B, Hq, Nq), torch.float32, "lse")
    o = torch.empty_like(q) if out is None else out
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    return B, Hq, Hkv, d, num_pages, page, o, lse


def attn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, max_seq_len: int, scale=None, num_splits: int = 0,
                      workspace=None, out=None, lse=None, want_lse: bool = True):
    """Split-KV decode over a paged bf16 KV cache.  q [B, Hq, 1, d]; k_cache,
    v_cache [num_pages, Hkv, page_size, d]; block_table int32 [B, max_pages];
    seq_lens int32 [B]; max_seq_len >= every seq_lens entry.  Returns
    (o [B, Hq, 1, d], lse [B, Hq, 1])."""
    B, Hq, Hkv, d, num_pages, page, o, lse = _paged_args(q, k_cache, v_cache, block_table, seq_lens, out, lse,
                                                        workspace, want_lse)
    if workspace is None:
        need = decode_workspace_bytes(B, Hq, Hkv, int(max_seq_len), d, num_splits)
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().attn_decode_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens), _ptr(o),
                                 _ptr(lse) if want_lse else None, B, Hq, Hkv, d, num_pages, page,
                                 block_table.shape[1], int(max_seq_len), _scale(scale, d), int(num_splits),
                                 _ptr(workspace), ws_bytes, _stream())
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode_paged")
    return o, (lse if want_lse else None)


def decode_paged_fused_workspace_bytes(B: int, Hq: int, Hkv: int, max_seq_len: int, d: int, num_splits: int = 0) -> int:
    return int(lib().attn_decode_paged_fused_workspace_bytes(B, Hq, Hkv, max_seq_len, d, num_splits))


def attn_decode_paged_fused(q, k_cache, v_cache, block_table, seq_lens, max_seq_len: int, scale=None,
                            num_splits: int = 0, workspace=None, out=None, lse=None, want_lse: bool = True):
    """attn_decode_paged in one launch (the last chunk of each stream and kv
    head to finish merges).  A workspace passed in must have been zeroed
    before its first use (every call leaves its arrival counts zero); without
    one a zeroed one is allocated.  Returns (o, lse)."""
    B, Hq, Hkv, d, num_pages, page, o, lse = _paged_args(q, k_cache, v_cache, block_table, seq_lens, out, lse,
                                                        workspace, want_lse)
    if workspace is None:
        need = decode_paged_fused_workspace_bytes(B, Hq, Hkv, int(max_seq_len), d, num_splits)
        if need > 0:
            workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().attn_decode_paged_fused(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
                                       _ptr(o), _ptr(lse) if want_lse else None, B, Hq, Hkv, d, num_pages, page,
                                       block_table.shape[1], int(max_seq_len), _scale(scale, d), int(num_splits),
                                       _ptr(workspace), ws_bytes, _stream())
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode_paged_fused")
    return o, (lse if want_lse else None)


def bwd_workspace_bytes(B: int, Hq: int, Nq: int, d: int) -> int:
    return int(lib().attn_bwd_workspace_bytes(B, Hq, Nq, d))


def attn_bwd(q, k, v, o, dout, lse, causal: bool = False, scale=None, workspace=None, dq=None, dk=None, dv=None,
             grad_dtype=None):
    """Backward from the saved LSE.  Returns (dq, dk, dv) in grad_dtype:
    torch.float32 (the default) or torch.bfloat16 (attn_bwd_bf16_grads: the
    fp32 results rounded to nearest even)."""
    gdt = torch.float32 if grad_dtype is None else grad_dtype
    if gdt not in (torch.float32, torch.bfloat16):
        raise ValueError(f"attn_bwd: grad_dtype must be float32 or bfloat16, not {gdt}")
    _check_dev(q, k, v, o, dout, lse, workspace, dq, dk, dv)
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v)
    _want(o, q.shape, q.dtype, "o")
    _want(dout, q.shape, q.dtype, "dout")
    _want(lse, (B, Hq, Nq), torch.float32, "lse")
    _want(dq, q.shape, gdt, "dq")
    _want(dk, k.shape, gdt, "dk")
    _want(dv, v.shape, gdt, "dv")
    gd = dict(dtype=gdt, device=q.device)
    dq = torch.empty(q.shape, **gd) if dq is None else dq
    dk = torch.empty(k.shape, **gd) if dk is None else dk
    dv = torch.empty(v.shape, **gd) if dv is None else dv
    if workspace is None:
        need = bwd_workspace_bytes(B, Hq, Nq, d)
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    fn = lib().attn_bwd if gdt == torch.float32 else lib().attn_bwd_bf16_grads
    st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), B,
            Hq, Hkv, Nq, Nk, d, _scale(scale, d), int(bool(causal)), _ptr(workspace), ws_bytes,
            _dtype_code(q), _stream())
    if st != ATTN_OK:
        raise AttnError(st, "attn_bwd" if gdt == torch.float32 else "attn_bwd_bf16_grads")
    return dq, dk, dv
