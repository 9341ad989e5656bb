"""Thin ctypes binding over the C ABI in include/fa.h.

Argument marshalling only: torch tensors supply device pointers, strides and
the current HIP stream; every step of the computation runs in the HIP kernels
of libfa72.so.  There is no fallback: if the library is missing or a call
fails, these functions raise.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa72.so")

FA_OK = 0
FA_ERR_INVALID_ARG = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_HIP = -3

EXPORTS = ("fa_fwd", "fa_fwd_relpos_bias", "fa_fwd_prefix_lm", "fa_fwd_varlen", "fa_fwd_kvcache_paged", "fa_fwd_kvcache_paged_noalloc",
           "fa_fwd_varlen_paged", "fa_varlen_paged_num_splits", "fa_varlen_paged_workspace_size",
           "fa_kvcache_num_splits",
           "fa_kvcache_workspace_size", "fa_kvcache_append", "fa_rotary", "fa_bwd", "fa_bwd_workspace_size",
           "fa_fp8_quantize", "fa_fp8_quantize_v", "fa_fp8_vt_len", "fa_fwd_fp8",
           "fa_fwd_kvcache_paged_fp8", "fa_kvcache_append_fp8", "fa_fp8_quantize_rotated", "fa_bwd_varlen",
           "fa_combine", "fa_merge_attn_states", "fa_tile_class", "fa_last_error", "fa_version")

FA_FP8_Q_BLOCK = 128
FA_FP8_K_BLOCK = 64


class FaError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{msg} (code {code})")
        self.code = code


class fa_attn_opts(ctypes.Structure):
    _fields_ = [("softmax_scale", ctypes.c_float), ("causal", ctypes.c_int),
                ("window_left", ctypes.c_int), ("window_right", ctypes.c_int),
                ("softcap", ctypes.c_float), ("pack_gqa", ctypes.c_int),
                ("alibi_slopes", ctypes.c_void_p), ("alibi_batch_stride", ctypes.c_int64)]


_lib = None


def lib():
    """Load libfa72.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with exact_attention_72_amd._build.build()")
    L = ctypes.CDLL(LIB_PATH)
    P, I, I64, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    S3 = ctypes.POINTER(ctypes.c_int64)
    OPT = ctypes.POINTER(fa_attn_opts)
    L.fa_fwd.argtypes = [OPT, P, P, P, P, P, I, I, I, I, I, I, S3, S3, S3, S3, P]
    L.fa_fwd_varlen.argtypes = [OPT, P, P, P, P, P, P, P, I, I, I, I, I, I, I, S3, S3, S3, S3, P]
    L.fa_fwd_relpos_bias.argtypes = [OPT, P, P, P, P, P, I, I, I, I, I, I, P, I, S3, S3, S3, S3, P]
    L.fa_fwd_prefix_lm.argtypes = [OPT, P, P, P, P, P, I, I, I, I, I, I, P, S3, S3, S3, S3, P]
    L.fa_fwd_kvcache_paged.argtypes = [OPT, P, P, P, P, P, P, P, I, I, I, I, I, I64, I, I, I, P, SZ,
                                       S3, S3, S3, S3, P]
    L.fa_fwd_kvcache_paged_noalloc.argtypes = [OPT, P, P, P, P, P, P, P, I, I, I, I, I, I64, I, I, I,
                                               S3, S3, S3, S3, P]
    L.fa_fwd_kvcache_paged_fp8.argtypes = [OPT, P, P, P, F, F, P, P, P, P, I, I, I, I, I, I64, I, I, I, P, SZ,
                                           S3, S3, S3, S3, P]
    L.fa_kvcache_append_fp8.argtypes = [P, P, P, P, F, F, P, P, I, I, I, I, I64, I, I, S3, S3, S3, S3, P]
    L.fa_kvcache_workspace_size.argtypes = [I, I, I, I, I]
    L.fa_kvcache_workspace_size.restype = SZ
    L.fa_kvcache_num_splits.argtypes = [I, I, I, I, I, I]
    L.fa_kvcache_num_splits.restype = I
    L.fa_combine.argtypes = [P, P, I, I64, I, I64, P, I64, P, P]
    L.fa_merge_attn_states.argtypes = [P, P, P, P, I, P, P, I, I, I, I, S3, S3, S3, P]
    L.fa_kvcache_append.argtypes = [P, P, P, P, P, P, I, I, I, I, I64, I, I, S3, S3, S3, S3, P, P, I, I, P]
    L.fa_rotary.argtypes = [P, I, I, I, I, S3, P, P, P, I, I, P]
    L.fa_bwd.argtypes = [OPT, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, S3, S3, S3, S3, S3, S3, S3, S3, P, SZ, P]
    L.fa_bwd_varlen.argtypes = [OPT, P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I,
                                S3, S3, S3, S3, S3, S3, S3, S3, P, SZ, P]
    L.fa_bwd_workspace_size.argtypes = [I, I, I]
    L.fa_bwd_workspace_size.restype = SZ
    L.fa_fwd_varlen_paged.argtypes = [OPT, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I64, I, I, I, P, SZ,
                                      S3, S3, S3, S3, P]
    L.fa_varlen_paged_num_splits.argtypes = [I, I, I, I]
    L.fa_varlen_paged_num_splits.restype = I
    L.fa_varlen_paged_workspace_size.argtypes = [I, I, I, I]
    L.fa_varlen_paged_workspace_size.restype = SZ
    L.fa_fp8_quantize.argtypes = [P, I, I, I, I, S3, I, P, S3, P, P]
    L.fa_fp8_quantize_v.argtypes = [P, I, I, I, I, S3, P, P, P]
    L.fa_fp8_quantize_rotated.argtypes = [P, I, I, I, I, S3, I, P, P, S3, P, P]
    L.fa_fp8_vt_len.argtypes = [I]
    L.fa_fwd_fp8.argtypes = [OPT, P, P, P, P, P, P, P, P, I, I, I, I, I, I, S3, S3, S3, P]
    L.fa_tile_class.argtypes = [I, I, I, I, I, I, I, I, I]
    L.fa_last_error.restype = ctypes.c_char_p
    L.fa_version.restype = I
    for name in ("fa_fwd", "fa_fwd_relpos_bias", "fa_fwd_prefix_lm", "fa_fwd_varlen", "fa_fwd_kvcache_paged", "fa_fwd_kvcache_paged_noalloc",
                 "fa_combine", "fa_merge_attn_states", "fa_tile_class",
                 "fa_kvcache_append", "fa_fwd_varlen_paged", "fa_rotary", "fa_bwd", "fa_fp8_quantize",
                 "fa_fwd_kvcache_paged_fp8", "fa_kvcache_append_fp8", "fa_fp8_quantize_rotated", "fa_bwd_varlen",
                 "fa_fp8_quantize_v", "fa_fp8_vt_len", "fa_fwd_fp8"):
        getattr(L, name).restype = I
    _lib = L
    return L


def _check(rc):
    if rc != FA_OK:
        raise FaError(rc, lib().fa_last_error().decode())


def _strides(t, dims):
    arr = (ctypes.c_int64 * len(dims))(*[t.stride(i) for i in dims])
    return arr


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _opts(softmax_scale, causal, window, softcap, pack_gqa, alibi_slopes=None):
    wl, wr = (-1, -1) if window is None else window
    ptr, bs = None, 0
    if alibi_slopes is not None:
        if alibi_slopes.dtype != torch.float32 or not alibi_slopes.is_cuda or alibi_slopes.stride(-1) != 1:
            raise TypeError("alibi_slopes must be a float32 tensor on a HIP device, heads contiguous")
        ptr = alibi_slopes.data_ptr()
        bs = alibi_slopes.stride(0) if alibi_slopes.dim() == 2 else 0
    return fa_attn_opts(float(softmax_scale) if softmax_scale else 0.0, int(bool(causal)), int(wl),
                        int(wr), float(softcap), int(pack_gqa), ptr, bs)


def _bf16_cuda(*ts):
    for t in ts:
        if t.dtype != torch.bfloat16 or not t.is_cuda:
            raise TypeError("q, k, v, out must be bfloat16 tensors on a HIP device")
        if t.stride(-1) != 1:
            raise ValueError("the head_dim dimension must be contiguous")


def fa_fwd(q, k, v, *, softmax_scale=None, causal=False, window=None, softcap=0.0, pack_gqa=-1,
           alibi_slopes=None, out=None, lse=None, return_lse=True, stream=None):
    """Dense forward.  q [B, Nq, Hq, d], k/v [B, Nk, Hkv, d] bf16 -> (out, lse [B, Hq, Nq]).
    alibi_slopes: None, or float32 [Hq] / [B, Hq] on the device."""
    _bf16_cuda(q, k, v)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    _bf16_cuda(out)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    o = _opts(softmax_scale, causal, window, softcap, pack_gqa, alibi_slopes)
    _check(lib().fa_fwd(ctypes.byref(o), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Nq, Nk,
                        Hq, Hkv, d, _strides(q, (0, 1, 2)), _strides(k, (0, 1, 2)),
                        _strides(v, (0, 1, 2)), _strides(out, (0, 1, 2)), _stream(stream)))
    return out, lse


def _dense_out(q, out, lse, return_lse):
    B, Nq, Hq, d = q.shape
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    _bf16_cuda(out)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    return out, lse


def fa_fwd_relpos_bias(q, k, v, bias, *, softmax_scale=None, causal=False, window=None, pack_gqa=-1,
                       out=None, lse=None, return_lse=True, stream=None):
    """Dense forward with a relative-position bias table: bias float32 [Hq, 2R + 1] on the device;
    the logit of query position p and key j gets bias[h, clamp(j - p, -R, R) + R]."""
    _bf16_cuda(q, k, v)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if bias.dtype != torch.float32 or not bias.is_cuda or not bias.is_contiguous() or bias.dim() != 2 \
            or bias.shape[0] != Hq or bias.shape[1] % 2 != 1:
        raise TypeError("bias must be a contiguous float32 [heads_q, 2R + 1] device tensor")
    out, lse = _dense_out(q, out, lse, return_lse)
    o = _opts(softmax_scale, causal, window, 0.0, pack_gqa)
    _check(lib().fa_fwd_relpos_bias(ctypes.byref(o), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Nq, Nk,
                                    Hq, Hkv, d, _ptr(bias), (bias.shape[1] - 1) // 2, _strides(q, (0, 1, 2)),
                                    _strides(k, (0, 1, 2)), _strides(v, (0, 1, 2)), _strides(out, (0, 1, 2)),
                                    _stream(stream)))
    return out, lse


def fa_fwd_prefix_lm(q, k, v, prefix_lens, *, softmax_scale=None, window=None, pack_gqa=-1, out=None,
                     lse=None, return_lse=True, stream=None):
    """Dense forward with a prefix-LM mask: prefix_lens int32 [B] on the device; key j is visible
    to the query at position p iff j < prefix_lens[b] or j <= p."""
    _bf16_cuda(q, k, v)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if prefix_lens.dtype != torch.int32 or not prefix_lens.is_cuda or prefix_lens.numel() != B:
        raise TypeError("prefix_lens must be an int32 [batch] device tensor")
    out, lse = _dense_out(q, out, lse, return_lse)
    o = _opts(softmax_scale, False, window, 0.0, pack_gqa)
    _check(lib().fa_fwd_prefix_lm(ctypes.byref(o), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Nq, Nk, Hq,
                                  Hkv, d, _ptr(prefix_lens), _strides(q, (0, 1, 2)), _strides(k, (0, 1, 2)),
                                  _strides(v, (0, 1, 2)), _strides(out, (0, 1, 2)), _stream(stream)))
    return out, lse


def fa_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, *, softmax_scale=None,
                  causal=False, window=None, softcap=0.0, pack_gqa=-1, alibi_slopes=None, out=None, lse=None,
                  return_lse=True, stream=None):
    """Varlen forward.  q [Tq, Hq, d], k/v [Tk, Hkv, d], cu_seqlens int32 on device
    -> (out [Tq, Hq, d], lse [Hq, Tq])."""
    _bf16_cuda(q, k, v)
    Tq, Hq, d = q.shape
    Tk, Hkv = k.shape[0], k.shape[1]
    for c in (cu_seqlens_q, cu_seqlens_k):
        if c.dtype != torch.int32 or not c.is_cuda or not c.is_contiguous():
            raise TypeError("cu_seqlens must be contiguous int32 device tensors")
    B = cu_seqlens_q.numel() - 1
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    _bf16_cuda(out)
    if lse is None and return_lse:
        lse = torch.empty((Hq, Tq), dtype=torch.float32, device=q.device)
    o = _opts(softmax_scale, causal, window, softcap, pack_gqa, alibi_slopes)
    _check(lib().fa_fwd_varlen(ctypes.byref(o), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                               _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B, int(max_seqlen_q), Tq, Tk,
                               Hq, Hkv, d, _strides(q, (0, 1)), _strides(k, (0, 1)),
                               _strides(v, (0, 1)), _strides(out, (0, 1)), _stream(stream)))
    return out, lse


def fa_kvcache_workspace_size(batch, seqlen_q, heads_q, head_dim, num_splits):
    return int(lib().fa_kvcache_workspace_size(batch, seqlen_q, heads_q, head_dim, num_splits))


def fa_kvcache_num_splits(batch, seqlen_q, heads_q, heads_kv, page_size, max_blocks_per_seq):
    """The split count fa_fwd_kvcache_paged uses for num_splits=0."""
    return int(lib().fa_kvcache_num_splits(batch, seqlen_q, heads_q, heads_kv, page_size,
                                           max_blocks_per_seq))


def fa_fwd_kvcache_paged(q, k_cache, v_cache, block_table, cache_seqlens, *, num_splits=1,
                         softmax_scale=None, causal=True, window=None, softcap=0.0, pack_gqa=-1,
                         alibi_slopes=None, out=None, lse=None, workspace=None, return_lse=True, stream=None):
    """Paged-KV forward.  q [B, Nq, Hq, d]; caches [num_pages, page, Hkv, d];
    block_table int32 [B, max_blocks]; cache_seqlens int32 [B] -> (out, lse [B, Hq, Nq]).
    num_splits=0 picks the split count (fa_kvcache_num_splits); more than 32 packed
    query rows per sequence (Nq * Hq / Hkv) run the prefill kernel over the cache."""
    _bf16_cuda(q, k_cache, v_cache)
    B, Nq, Hq, d = q.shape
    num_pages, page, Hkv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    for c in (block_table, cache_seqlens):
        if c.dtype != torch.int32 or not c.is_cuda:
            raise TypeError("block_table and cache_seqlens must be int32 device tensors")
    if block_table.stride(-1) != 1 or block_table.stride(0) != block_table.shape[1]:
        raise ValueError("block_table must be a contiguous [batch, max_blocks] tensor")
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    _bf16_cuda(out)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    if num_splits == 0:
        num_splits = fa_kvcache_num_splits(B, Nq, Hq, Hkv, page, block_table.shape[1])
    need = fa_kvcache_workspace_size(B, Nq, Hq, d, num_splits)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    o = _opts(softmax_scale, causal, window, softcap, pack_gqa, alibi_slopes)
    _check(lib().fa_fwd_kvcache_paged(ctypes.byref(o), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                      _ptr(block_table), _ptr(cache_seqlens), _ptr(out), _ptr(lse),
                                      B, Nq, Hq, Hkv, d, num_pages, page, block_table.shape[1],
                                      int(num_splits), _ptr(workspace), ws_bytes,
                                      _strides(q, (0, 1, 2)), _strides(k_cache, (0, 1, 2)),
                                      _strides(v_cache, (0, 1, 2)), _strides(out, (0, 1, 2)),
                                      _stream(stream)))
    return out, lse


def fa_fwd_kvcache_paged_fp8(q, k_cache, v_cache, k_scale, v_scale, block_table, cache_seqlens, *, num_splits=1,
                             softmax_scale=None, causal=True, window=None, softcap=0.0, alibi_slopes=None, out=None,
                             lse=None, workspace=None, return_lse=True, stream=None):
    """Paged-KV decode over an FP8 (e4m3) cache.  q [B, Nq, Hq, d] bf16 with Nq * Hq / Hkv <= 32;
    caches uint8 [num_pages, page, Hkv, d] of codes whose values are code * k_scale and
    code * v_scale (floats); block_table int32 [B, max_blocks]; cache_seqlens int32 [B]
    -> (out, lse [B, Hq, Nq]).  num_splits=0 picks the split count (fa_kvcache_num_splits)."""
    _bf16_cuda(q)
    _u8_cuda(k_cache, v_cache)
    B, Nq, Hq, d = q.shape
    num_pages, page, Hkv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    for c in (block_table, cache_seqlens):
        if c.dtype != torch.int32 or not c.is_cuda:
            raise TypeError("block_table and cache_seqlens must be int32 device tensors")
    if block_table.stride(-1) != 1 or block_table.stride(0) != block_table.shape[1]:
        raise ValueError("block_table must be a contiguous [batch, max_blocks] tensor")
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    _bf16_cuda(out)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    if num_splits == 0:
        num_splits = fa_kvcache_num_splits(B, Nq, Hq, Hkv, page, block_table.shape[1])
    need = fa_kvcache_workspace_size(B, Nq, Hq, d, num_splits)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    o = _opts(softmax_scale, causal, window, softcap, -1, alibi_slopes)
    _check(lib().fa_fwd_kvcache_paged_fp8(ctypes.byref(o), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                          float(k_scale), float(v_scale), _ptr(block_table), _ptr(cache_seqlens),
                                          _ptr(out), _ptr(lse), B, Nq, Hq, Hkv, d, num_pages, page,
                                          block_table.shape[1], int(num_splits), _ptr(workspace), ws_bytes,
                                          _strides(q, (0, 1, 2)), _strides(k_cache, (0, 1, 2)),
                                          _strides(v_cache, (0, 1, 2)), _strides(out, (0, 1, 2)),
                                          _stream(stream)))
    return out, lse


FA_NOALLOC_SCRATCH_BYTES = 32 << 20


def fa_fwd_kvcache_paged_noalloc(q, k_cache, v_cache, block_table, cache_seqlens, *, num_splits=1,
                                 softmax_scale=None, causal=True, window=None, softcap=0.0, pack_gqa=-1,
                                 alibi_slopes=None, out, lse=None, stream=None):
    """fa_fwd_kvcache_paged without a workspace: the split partials go to the library's static
    device scratch (FA_NOALLOC_SCRATCH_BYTES per device).  The caller passes out (and lse, or
    None); nothing is allocated here or in the library."""
    _bf16_cuda(q, k_cache, v_cache, out)
    B, Nq, Hq, d = q.shape
    num_pages, page, Hkv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    for c in (block_table, cache_seqlens):
        if c.dtype != torch.int32 or not c.is_cuda:
            raise TypeError("block_table and cache_seqlens must be int32 device tensors")
    if block_table.stride(-1) != 1 or block_table.stride(0) != block_table.shape[1]:
        raise ValueError("block_table must be a contiguous [batch, max_blocks] tensor")
    o = _opts(softmax_scale, causal, window, softcap, pack_gqa, alibi_slopes)
    _check(lib().fa_fwd_kvcache_paged_noalloc(ctypes.byref(o), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                              _ptr(block_table), _ptr(cache_seqlens), _ptr(out), _ptr(lse),
                                              B, Nq, Hq, Hkv, d, num_pages, page, block_table.shape[1],
                                              int(num_splits), _strides(q, (0, 1, 2)),
                                              _strides(k_cache, (0, 1, 2)), _strides(v_cache, (0, 1, 2)),
                                              _strides(out, (0, 1, 2)), _stream(stream)))
    return out, lse


def fa_fwd_varlen_paged(q, k_cache, v_cache, cu_seqlens_q, max_seqlen_q, block_table, cache_seqlens, *,
                        num_splits=0, softmax_scale=None, causal=True, window=None, softcap=0.0, pack_gqa=-1,
                        out=None, lse=None, workspace=None, return_lse=True, stream=None):
    """Unified prefill + decode over a paged cache.  q [total_q, Hq, d] packed by cu_seqlens_q;
    caches [num_pages, page, Hkv, d]; block_table int32 [B, max_blocks]; cache_seqlens int32 [B]
    (keys per sequence, new tokens included) -> (out [total_q, Hq, d], lse [Hq, total_q]).
    num_splits: split-KV count of the decode requests (0: fa_varlen_paged_num_splits)."""
    _bf16_cuda(q, k_cache, v_cache)
    total_q, Hq, d = q.shape
    num_pages, page, Hkv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    for c in (cu_seqlens_q, block_table, cache_seqlens):
        if c.dtype != torch.int32 or not c.is_cuda:
            raise TypeError("cu_seqlens_q, block_table and cache_seqlens must be int32 device tensors")
    if block_table.stride(-1) != 1 or block_table.stride(0) != block_table.shape[1]:
        raise ValueError("block_table must be a contiguous [batch, max_blocks] tensor")
    B = cu_seqlens_q.numel() - 1
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    _bf16_cuda(out)
    if lse is None and return_lse:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    if num_splits == 0:
        num_splits = int(lib().fa_varlen_paged_num_splits(B, Hq, Hkv, block_table.shape[1]))
    need = int(lib().fa_varlen_paged_workspace_size(B, Hkv, d, int(num_splits)))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    o = _opts(softmax_scale, causal, window, softcap, pack_gqa)
    _check(lib().fa_fwd_varlen_paged(ctypes.byref(o), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out),
                                     _ptr(lse), _ptr(cu_seqlens_q), _ptr(block_table), _ptr(cache_seqlens),
                                     B, int(max_seqlen_q), total_q, Hq, Hkv, d, num_pages, page,
                                     block_table.shape[1], int(num_splits), _ptr(workspace), ws_bytes,
                                     _strides(q, (0, 1)), _strides(k_cache, (0, 1, 2)),
                                     _strides(v_cache, (0, 1, 2)), _strides(out, (0, 1)), _stream(stream)))
    return out, lse


def _rotary_tables(cos, sin):
    if cos is None and sin is None:
        return None, None, 0
    if cos is None or sin is None:
        raise ValueError("rotary cos and sin go together")
    for c in (cos, sin):
        if c.dtype != torch.float32 or not c.is_cuda or not c.is_contiguous() or c.dim() != 2:
            raise TypeError("rotary tables must be contiguous float32 [positions, rotary_dim / 2] device tensors")
    if cos.shape != sin.shape:
        raise ValueError("rotary cos and sin shapes differ")
    return cos, sin, 2 * cos.shape[1]


def fa_rotary(x, cos, sin, *, position_base=None, interleaved=False, stream=None):
    """In place: rotate x [B, L, H, d] (bf16) at positions position_base[b] + t (0 + t
    without a base) with the fp32 tables cos/sin [positions, rotary_dim / 2]."""
    _bf16_cuda(x)
    B, L, H, d = x.shape
    cos, sin, rdim = _rotary_tables(cos, sin)
    if cos is None:
        raise ValueError("fa_rotary needs cos and sin tables")
    if position_base is not None and (position_base.dtype != torch.int32 or not position_base.is_cuda):
        raise TypeError("position_base must be an int32 device tensor")
    _check(lib().fa_rotary(_ptr(x), B, L, H, d, _strides(x, (0, 1, 2)), _ptr(position_base), _ptr(cos),
                           _ptr(sin), rdim, int(bool(interleaved)), _stream(stream)))
    return x


def fa_kvcache_append(k_new, v_new, k_cache, v_cache, block_table, cache_seqlens, *, rotary_cos=None,
                      rotary_sin=None, rotary_interleaved=False, stream=None):
    """Write k_new/v_new [B, L, Hkv, d] into the paged caches [num_pages, page, Hkv, d]
    at logical positions cache_seqlens[b] + t (in place; cache_seqlens is not updated).
    With rotary tables the keys are rotated at those positions on the way in."""
    _bf16_cuda(k_new, v_new, k_cache, v_cache)
    B, L, Hkv, d = k_new.shape
    if tuple(v_new.shape) != (B, L, Hkv, d) or k_cache.shape != v_cache.shape or k_cache.shape[2:] != (Hkv, d):
        raise ValueError("k_new/v_new [B, L, Hkv, d] and caches [num_pages, page, Hkv, d] disagree")
    for c in (block_table, cache_seqlens):
        if c.dtype != torch.int32 or not c.is_cuda:
            raise TypeError("block_table and cache_seqlens must be int32 device tensors")
    if block_table.stride(-1) != 1 or block_table.stride(0) != block_table.shape[1]:
        raise ValueError("block_table must be a contiguous [batch, max_blocks] tensor")
    cos, sin, rdim = _rotary_tables(rotary_cos, rotary_sin)
    _check(lib().fa_kvcache_append(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                   _ptr(block_table), _ptr(cache_seqlens), B, L, Hkv, d,
                                   k_cache.shape[0], k_cache.shape[1], block_table.shape[1],
                                   _strides(k_new, (0, 1, 2)), _strides(v_new, (0, 1, 2)),
                                   _strides(k_cache, (0, 1, 2)), _strides(v_cache, (0, 1, 2)),
                                   _ptr(cos), _ptr(sin), rdim, int(bool(rotary_interleaved)),
                                   _stream(stream)))


def fa_kvcache_append_fp8(k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_table, cache_seqlens, *,
                          stream=None):
    """Quantize k_new/v_new [B, L, Hkv, d] (bf16) to e4m3 codes of x / k_scale and x / v_scale
    and write them into the uint8 caches [num_pages, page, Hkv, d] at logical positions
    cache_seqlens[b] + t (in place; cache_seqlens is not updated)."""
    _bf16_cuda(k_new, v_new)
    _u8_cuda(k_cache, v_cache)
    B, L, Hkv, d = k_new.shape
    if tuple(v_new.shape) != (B, L, Hkv, d) or k_cache.shape != v_cache.shape or k_cache.shape[2:] != (Hkv, d):
        raise ValueError("k_new/v_new [B, L, Hkv, d] and caches [num_pages, page, Hkv, d] disagree")
    for c in (block_table, cache_seqlens):
        if c.dtype != torch.int32 or not c.is_cuda:
            raise TypeError("block_table and cache_seqlens must be int32 device tensors")
    if block_table.stride(-1) != 1 or block_table.stride(0) != block_table.shape[1]:
        raise ValueError("block_table must be a contiguous [batch, max_blocks] tensor")
    _check(lib().fa_kvcache_append_fp8(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), float(k_scale),
                                       float(v_scale), _ptr(block_table), _ptr(cache_seqlens), B, L, Hkv, d,
                                       k_cache.shape[0], k_cache.shape[1], block_table.shape[1],
                                       _strides(k_new, (0, 1, 2)), _strides(v_new, (0, 1, 2)),
                                       _strides(k_cache, (0, 1, 2)), _strides(v_cache, (0, 1, 2)),
                                       _stream(stream)))


def fa_bwd(q, k, v, out, lse, dout, *, softmax_scale=None, causal=False, window=None, softcap=0.0, dq=None,
           dk=None, dv=None, workspace=None, stream=None):
    """Gradients of fa_fwd: q/out/dout [B, Nq, Hq, d], k/v [B, Nk, Hkv, d] bf16, lse fp32
    [B, Hq, Nq] from the forward -> (dq, dk, dv) bf16 in the shapes of q, k, v."""
    _bf16_cuda(q, k, v, out, dout)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if lse.dtype != torch.float32 or not lse.is_cuda or not lse.is_contiguous() or tuple(lse.shape) != (B, Hq, Nq):
        raise ValueError("lse must be a contiguous float32 [B, Hq, Nq] device tensor")
    dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
    dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
    dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
    _bf16_cuda(dq, dk, dv)
    need = int(lib().fa_bwd_workspace_size(B, Nq, Hq))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    o = _opts(softmax_scale, causal, window, softcap, 0)
    S = lambda t: _strides(t, (0, 1, 2))  # noqa: E731
    _check(lib().fa_bwd(ctypes.byref(o), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq),
                        _ptr(dk), _ptr(dv), B, Nq, Nk, Hq, Hkv, d, S(q), S(k), S(v), S(out), S(dout), S(dq), S(dk),
                        S(dv), _ptr(workspace), ws_bytes, _stream(stream)))
    return dq, dk, dv


def fa_bwd_varlen(q, k, v, out, lse, dout, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, *,
                  softmax_scale=None, causal=False, window=None, softcap=0.0, dq=None, dk=None, dv=None,
                  workspace=None, stream=None):
    """Gradients of fa_fwd_varlen: q/out/dout [total_q, Hq, d], k/v [total_k, Hkv, d] bf16, lse fp32
    [Hq, total_q] from the forward, cu_seqlens int32 [B + 1] -> (dq, dk, dv) in the shapes of q, k, v."""
    _bf16_cuda(q, k, v, out, dout)
    Tq, Hq, d = q.shape
    Tk, Hkv = k.shape[0], k.shape[1]
    B = cu_seqlens_q.numel() - 1
    for c in (cu_seqlens_q, cu_seqlens_k):
        if c.dtype != torch.int32 or not c.is_cuda or not c.is_contiguous() or c.numel() != B + 1:
            raise TypeError("cu_seqlens must be contiguous int32 device tensors of batch + 1 entries")
    if lse.dtype != torch.float32 or not lse.is_cuda or not lse.is_contiguous() or tuple(lse.shape) != (Hq, Tq):
        raise ValueError("lse must be a contiguous float32 [Hq, total_q] device tensor")
    dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
    dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
    dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
    _bf16_cuda(dq, dk, dv)
    need = int(lib().fa_bwd_workspace_size(1, Tq, Hq))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    o = _opts(softmax_scale, causal, window, softcap, 0)
    S = lambda t: _strides(t, (0, 1))  # noqa: E731
    _check(lib().fa_bwd_varlen(ctypes.byref(o), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout),
                               _ptr(dq), _ptr(dk), _ptr(dv), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B,
                               int(max_seqlen_q), int(max_seqlen_k), Tq, Tk, Hq, Hkv, d, S(q), S(k), S(v), S(out),
                               S(dout), S(dq), S(dk), S(dv), _ptr(workspace), ws_bytes, _stream(stream)))
    return dq, dk, dv


def fa_combine(o_part, lse_part, *, out=None, lse=None, stream=None):
    """Merge partial states.  o_part fp32 [S, rows, d] (or a view whose splits are
    part_stride_rows rows apart: split stride = o_part.stride(0) / d), lse_part fp32
    [S, rows] with the same split stride in rows -> (out bf16 [rows, d], lse fp32 [rows])."""
    S, rows, d = o_part.shape
    if o_part.dtype != torch.float32 or lse_part.dtype != torch.float32:
        raise TypeError("partials are float32")
    if o_part.stride(2) != 1 or o_part.stride(1) != d or lse_part.stride(1) != 1:
        raise ValueError("partial rows must be contiguous")
    stride_rows = o_part.stride(0) // d if S > 1 else rows
    if (S > 1 and (o_part.stride(0) % d or lse_part.stride(0) != stride_rows)):
        raise ValueError("o_part and lse_part must share one split stride in rows")
    if out is None:
        out = torch.empty((rows, d), dtype=torch.bfloat16, device=o_part.device)
    if lse is None:
        lse = torch.empty((rows,), dtype=torch.float32, device=o_part.device)
    _check(lib().fa_combine(_ptr(o_part), _ptr(lse_part), S, rows, d, stride_rows, _ptr(out), out.stride(0),
                            _ptr(lse), _stream(stream)))
    return out, lse


FA_DTYPE_FP32 = 0
FA_DTYPE_BF16 = 1


def fa_merge_attn_states(prefix_out, prefix_lse, suffix_out, suffix_lse, *, out=None, lse=None, stream=None):
    """Merge two attention states from separate buffers.  prefix_out / suffix_out
    [B, N, H, d] (bf16 or fp32, same strides), prefix_lse / suffix_lse fp32 [B, H, N]
    (same strides) -> (out bf16 [B, N, H, d], lse fp32 [B, H, N])."""
    if prefix_out.shape != suffix_out.shape or prefix_out.stride() != suffix_out.stride():
        raise ValueError("prefix_out and suffix_out must have the same shape and strides")
    if prefix_lse.stride() != suffix_lse.stride() or prefix_lse.dtype != torch.float32 or \
            suffix_lse.dtype != torch.float32:
        raise ValueError("the LSEs must be float32 with the same strides")
    if prefix_out.dtype != suffix_out.dtype or prefix_out.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("states are float32 or bfloat16")
    dt = FA_DTYPE_FP32 if prefix_out.dtype == torch.float32 else FA_DTYPE_BF16
    B, N, H, d = prefix_out.shape
    if prefix_out.stride(3) != 1:
        raise ValueError("head_dim must be contiguous")
    if out is None:
        out = torch.empty((B, N, H, d), dtype=torch.bfloat16, device=prefix_out.device)
    if lse is None:
        lse = torch.empty_strided(prefix_lse.shape, prefix_lse.stride(), dtype=torch.float32,
                                  device=prefix_out.device)
    _check(lib().fa_merge_attn_states(_ptr(prefix_out), _ptr(prefix_lse), _ptr(suffix_out), _ptr(suffix_lse), dt,
                                      _ptr(out), _ptr(lse), B, N, H, d, _strides(prefix_out, (0, 1, 2)),
                                      _strides(out, (0, 1, 2)), _strides(prefix_lse, (0, 1, 2)),
                                      _stream(stream)))
    return out, lse


def fa_tile_class(tok_lo, tok_hi, seqlen_q, seqlen_k, causal, window_left, window_right, block_n, n):
    return int(lib().fa_tile_class(tok_lo, tok_hi, seqlen_q, seqlen_k, int(bool(causal)),
                                   window_left, window_right, block_n, n))


def fa_last_error():
    return lib().fa_last_error().decode()


def fa_version():
    return int(lib().fa_version())


def default_scale(d):
    return 1.0 / math.sqrt(d)


def _u8_cuda(*ts):
    for t in ts:
        if t.dtype != torch.uint8 or not t.is_cuda:
            raise TypeError("FP8 codes must be uint8 tensors on a HIP device")
        if t.stride(-1) != 1:
            raise ValueError("the head_dim dimension must be contiguous")


def _f32_cuda(*ts):
    for t in ts:
        if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise TypeError("scales must be contiguous float32 tensors on a HIP device")


def fa_fp8_quantize(x, block_rows, *, codes=None, scales=None, stream=None):
    """Per-block e4m3 quantizer.  x [B, N, H, d] bf16 -> (codes uint8 [B, N, H, d],
    scales float32 [B, H, ceil(N / block_rows)])."""
    _bf16_cuda(x)
    B, N, H, d = x.shape
    nblk = -(-N // block_rows)
    if codes is None:
        codes = torch.empty((B, N, H, d), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((B, H, nblk), dtype=torch.float32, device=x.device)
    _u8_cuda(codes)
    _f32_cuda(scales)
    if tuple(scales.shape) != (B, H, nblk):
        raise ValueError(f"scales must be [{B}, {H}, {nblk}]")
    _check(lib().fa_fp8_quantize(_ptr(x), B, N, H, d, _strides(x, (0, 1, 2)), int(block_rows), _ptr(codes),
                                 _strides(codes, (0, 1, 2)), _ptr(scales), _stream(stream)))
    return codes, scales


def fa_fp8_quantize_rotated(x, block_rows, signs, *, codes=None, scales=None, stream=None):
    """fa_fp8_quantize of the rows of x rotated by diag(signs) H / sqrt(d) (randomized Hadamard
    transform; signs float32 [d] of +-1 on the device, the same for Q and K)."""
    _bf16_cuda(x)
    B, N, H, d = x.shape
    nblk = -(-N // block_rows)
    if signs.dtype != torch.float32 or not signs.is_cuda or not signs.is_contiguous() or signs.numel() != d:
        raise TypeError(f"signs must be a contiguous float32 device tensor of {d} values")
    if codes is None:
        codes = torch.empty((B, N, H, d), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((B, H, nblk), dtype=torch.float32, device=x.device)
    _u8_cuda(codes)
    _f32_cuda(scales)
    if tuple(scales.shape) != (B, H, nblk):
        raise ValueError(f"scales must be [{B}, {H}, {nblk}]")
    _check(lib().fa_fp8_quantize_rotated(_ptr(x), B, N, H, d, _strides(x, (0, 1, 2)), int(block_rows), _ptr(signs),
                                         _ptr(codes), _strides(codes, (0, 1, 2)), _ptr(scales), _stream(stream)))
    return codes, scales


def fa_fp8_quantize_v(v, *, vt=None, scales=None, stream=None):
    """V quantizer: v [B, N, Hkv, d] bf16 -> (vt uint8 [B, Hkv, d, fa_fp8_vt_len(N)] in the
    transposed, product-ordered layout, scales float32 [B, Hkv])."""
    _bf16_cuda(v)
    B, N, H, d = v.shape
    L = lib().fa_fp8_vt_len(N)
    if vt is None:
        vt = torch.empty((B, H, d, L), dtype=torch.uint8, device=v.device)
    if scales is None:
        scales = torch.empty((B, H), dtype=torch.float32, device=v.device)
    _u8_cuda(vt)
    _f32_cuda(scales)
    if not vt.is_contiguous() or tuple(vt.shape) != (B, H, d, L) or tuple(scales.shape) != (B, H):
        raise ValueError(f"vt must be a dense [{B}, {H}, {d}, {L}] tensor and scales [{B}, {H}]")
    _check(lib().fa_fp8_quantize_v(_ptr(v), B, N, H, d, _strides(v, (0, 1, 2)), _ptr(vt), _ptr(scales),
                                   _stream(stream)))
    return vt, scales


def fa_fwd_fp8(q, q_scales, k, k_scales, vt, v_scales, *, softmax_scale=None, causal=False, window=None,
               out=None, lse=None, return_lse=True, stream=None):
    """FP8 forward.  q uint8 [B, Nq, Hq, d] with q_scales [B, Hq, ceil(Nq / 128)], k uint8
    [B, Nk, Hkv, d] with k_scales [B, Hkv, ceil(Nk / 64)], vt / v_scales from fa_fp8_quantize_v
    -> (out bf16 [B, Nq, Hq, d], lse [B, Hq, Nq])."""
    _u8_cuda(q, k, vt)
    _f32_cuda(q_scales, k_scales, v_scales)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    L = lib().fa_fp8_vt_len(Nk)
    if (tuple(vt.shape) != (B, Hkv, d, L) or not vt.is_contiguous()
            or tuple(q_scales.shape) != (B, Hq, -(-Nq // FA_FP8_Q_BLOCK))
            or tuple(k_scales.shape) != (B, Hkv, -(-Nk // FA_FP8_K_BLOCK))
            or tuple(v_scales.shape) != (B, Hkv)):
        raise ValueError("FP8 operand or scale shapes do not match q and k")
    if out is None:
        out = torch.empty((B, Nq, Hq, d), dtype=torch.bfloat16, device=q.device)
    _bf16_cuda(out)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    o = _opts(softmax_scale, causal, window, 0.0, -1)
    _check(lib().fa_fwd_fp8(ctypes.byref(o), _ptr(q), _ptr(q_scales), _ptr(k), _ptr(k_scales), _ptr(vt),
                            _ptr(v_scales), _ptr(out), _ptr(lse), B, Nq, Nk, Hq, Hkv, d,
                            _strides(q, (0, 1, 2)), _strides(k, (0, 1, 2)), _strides(out, (0, 1, 2)),
                            _stream(stream)))
    return out, lse
