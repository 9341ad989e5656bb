"""Seeded synthetic inputs for the attention forward workloads.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  The same tensors feed both the HIP path and the fp64
oracle, so both see identical bytes.

Recipe (every draw from a torch generator seeded with the workload's seed):
  * Q, K, V: fp32 standard normal, multiplied by ``mult`` (2 for the softcap
    workload), rounded to bfloat16 (round-to-nearest-even).
  * varlen lengths: integers uniform on [lo, hi] inclusive; cu_seqlens is
    their int32 prefix sum starting at 0.
  * paged KV: cache_seqlens uniform on [lo, hi] inclusive; the page pool has
    B * max_blocks pages and block_table is a random permutation of the pool
    viewed as [B, max_blocks] (only the first ceil(L_b / page) entries of a
    row are live).

The shapes follow the pages' statement of the problem: BSHD tensors for
dense attention, [total_tokens, heads, d] plus cu_seqlens for varlen
("FA4 (CuTeDSL) and engineering interfaces", section 4) and a
[num_pages, page, kv_heads, d] pool addressed through block_table for paged
KV ("Attention kernels: FlashAttention and PagedAttention", sections 6.1 and
8.4).
"""
from __future__ import annotations

import itertools
import math

import numpy as np

import torch

# The five workloads, by name.  Sizes are those of the problem statement.
WORKLOADS = {
    "single_head_256_d64": dict(kind="dense", B=1, N=256, Hq=1, Hkv=1, d=64, causal=False,
                                window=(-1, -1), softcap=0.0, mult=1.0, seed=1),
    "prefill_b4_h16_n4096_d128_causal": dict(kind="dense", B=4, N=4096, Hq=16, Hkv=16, d=128,
                                             causal=True, window=(-1, -1), softcap=0.0,
                                             mult=1.0, seed=2),
    "varlen_gqa_32seq_64to8192_h32kv4_d128_causal": dict(kind="varlen", nseq=32, lo=64, hi=8192,
                                                         Hq=32, Hkv=4, d=128, causal=True,
                                                         window=(-1, -1), softcap=0.0,
                                                         mult=1.0, seed=3),
    "paged_decode_b64_h32kv8_d128_page256": dict(kind="paged", B=64, Hq=32, Hkv=8, d=128,
                                                 page=256, lo=1024, hi=32768, max_blocks=128,
                                                 causal=True, window=(-1, -1), softcap=0.0,
                                                 mult=1.0, seed=4),
    "local_softcap_n32768_h32_d128_w4096_cap30": dict(kind="dense", B=1, N=32768, Hq=32, Hkv=32,
                                                      d=128, causal=True, window=(4096, 0),
                                                      softcap=30.0, mult=2.0, seed=5),
    # chunked prefill: a 4096-token chunk of each of 4 prompts against its paged cache, which
    # holds a 12288-token prefix plus the chunk itself (16384 keys, bottom-right causal)
    "paged_prefill_b4_h32kv8_d128_chunk4096_prefix12288_page256": dict(
        kind="paged_prefill", B=4, Hq=32, Hkv=8, d=128, page=256, Nq=4096, prefix=12288,
        max_blocks=64, causal=True, window=(-1, -1), softcap=0.0, mult=1.0, seed=6),
    # one launch for a mixed batch: 64 decode requests (1 new token, 1024..8192 cached keys)
    # and 4 prefill chunks (2048 new tokens on a 0..8192-token prefix), 32/8 heads
    "unified_decode64_chunk4x2048_h32kv8_d128_page256": dict(
        kind="varlen_paged", n_decode=64, dec_lo=1024, dec_hi=8192, n_chunk=4, chunk=2048,
        pre_lo=0, pre_hi=8192, Hq=32, Hkv=8, d=128, page=256, causal=True, window=(-1, -1),
        softcap=0.0, mult=1.0, seed=7),
}


def generator(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def randn_bf16(gen: torch.Generator, shape, mult: float = 1.0, device="cpu") -> torch.Tensor:
    """fp32 N(0,1) draws times ``mult``, rounded to bfloat16."""
    x = torch.randn(tuple(shape), generator=gen, dtype=torch.float32, device=device)
    if mult != 1.0:
        x.mul_(mult)
    return x.to(torch.bfloat16)


def dense(seed, B, N, Hq, Hkv, d, *, Nk=None, mult=1.0, device="cpu"):
    """q [B, N, Hq, d], k/v [B, Nk, Hkv, d] bf16."""
    Nk = N if Nk is None else Nk
    g = generator(seed, device)
    q = randn_bf16(g, (B, N, Hq, d), mult, device)
    k = randn_bf16(g, (B, Nk, Hkv, d), mult, device)
    v = randn_bf16(g, (B, Nk, Hkv, d), mult, device)
    return dict(q=q, k=k, v=v)


def rising_logits(seed, B, Nq, Nk, H, d, *, top=22.0, device="cpu"):
    """q, k, v [B, N, H, d] bf16 whose logits rise along the key axis: q rows are
    20 e plus noise and k row j is a_j e plus noise, e the unit vector of equal
    entries and a_j running linearly from -top to top, so q . k_j is about 20 a_j."""
    g = generator(seed, device)
    e = torch.full((d,), 1.0 / math.sqrt(d), device=device)
    a = torch.linspace(-top, top, Nk, device=device)
    q = 20.0 * e + 0.05 * torch.randn((B, Nq, H, d), generator=g, device=device)
    k = a[None, :, None, None] * e + 0.05 * torch.randn((B, Nk, H, d), generator=g, device=device)
    v = torch.randn((B, Nk, H, d), generator=g, device=device)
    return dict(q=q.to(torch.bfloat16), k=k.to(torch.bfloat16), v=v.to(torch.bfloat16))


def lengths_uniform(seed, n, lo, hi) -> torch.Tensor:
    """n integers uniform on [lo, hi] inclusive (int32)."""
    g = generator(seed)
    return torch.randint(int(lo), int(hi) + 1, (int(n),), generator=g, dtype=torch.int64).to(torch.int32)


def prefix_sum(lengths) -> torch.Tensor:
    """int32 [len + 1] prefix sum starting at 0 (the cu_seqlens layout)."""
    lengths = torch.as_tensor(lengths, dtype=torch.int64)
    cu = torch.zeros(lengths.numel() + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(lengths, 0)
    return cu.to(torch.int32)


def varlen(seed, nseq, lo, hi, Hq, Hkv, d, *, lengths=None, mult=1.0, device="cpu"):
    """Packed q [T, Hq, d], k/v [T, Hkv, d], cu_seqlens [nseq + 1], max_seqlen."""
    if lengths is None:
        lengths = lengths_uniform(seed, nseq, lo, hi)
    lengths = torch.as_tensor(lengths, dtype=torch.int32)
    cu = prefix_sum(lengths)
    T = int(cu[-1])
    g = generator(seed + 1_000_003, device)
    q = randn_bf16(g, (T, Hq, d), mult, device)
    k = randn_bf16(g, (T, Hkv, d), mult, device)
    v = randn_bf16(g, (T, Hkv, d), mult, device)
    return dict(q=q, k=k, v=v, cu_seqlens=cu, max_seqlen=int(lengths.max()) if T else 0,
                lengths=lengths)


def paged(seed, B, Hq, Hkv, d, page, lo, hi, *, max_blocks=None, Nq=1, cache_seqlens=None,
          mult=1.0, device="cpu"):
    """q [B, Nq, Hq, d]; k_cache/v_cache [B*max_blocks, page, Hkv, d];
    block_table int32 [B, max_blocks] (a random permutation of the pool);
    cache_seqlens int32 [B]."""
    if cache_seqlens is None:
        cache_seqlens = lengths_uniform(seed, B, lo, hi)
    cache_seqlens = torch.as_tensor(cache_seqlens, dtype=torch.int32)
    if max_blocks is None:
        max_blocks = int((int(cache_seqlens.max()) + page - 1) // page) if B else 1
        max_blocks = max(max_blocks, 1)
    num_pages = B * max_blocks
    gt = generator(seed + 2_000_003)
    block_table = torch.randperm(num_pages, generator=gt, dtype=torch.int64).to(torch.int32)
    block_table = block_table.view(B, max_blocks).contiguous()
    g = generator(seed + 1_000_003, device)
    q = randn_bf16(g, (B, Nq, Hq, d), mult, device)
    k_cache = randn_bf16(g, (num_pages, page, Hkv, d), mult, device)
    v_cache = randn_bf16(g, (num_pages, page, Hkv, d), mult, device)
    return dict(q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
                cache_seqlens=cache_seqlens, page=page, max_blocks=max_blocks)


def paged_fp8(seed, B, Hq, Hkv, d, page, lo, hi, *, max_blocks=None, Nq=1, cache_seqlens=None,
              amax=4.0, device="cpu"):
    """An FP8 (e4m3) paged cache: paged() of the same seed, its K and V divided by
    scale = amax / 448 and cast to e4m3 codes by torch's float8_e4m3fn conversion
    (values beyond +-448 clamped first).  Returns paged()'s dict with k_codes,
    v_codes (uint8, the caches' shape) and k_scale = v_scale = amax / 448 added."""
    t = paged(seed, B, Hq, Hkv, d, page, lo, hi, max_blocks=max_blocks, Nq=Nq, cache_seqlens=cache_seqlens,
              device=device)
    scale = float(np.float32(amax / 448.0))
    for n in ("k", "v"):
        x = t[n + "_cache"].float().div_(scale).clamp_(-448.0, 448.0)
        t[n + "_codes"] = x.to(torch.float8_e4m3fn).view(torch.uint8)
        del x
    t["k_scale"] = t["v_scale"] = scale
    return t


def to_bits(t: torch.Tensor) -> np.ndarray:
    """bfloat16 tensor -> numpy uint16 bit patterns (a reinterpretation, no rounding)."""
    if t.dtype != torch.bfloat16:
        raise TypeError("expected a bfloat16 tensor")
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def from_float(x, device="cpu") -> torch.Tensor:
    """A float array -> bfloat16 tensor (round-to-nearest-even)."""
    return torch.as_tensor(np.asarray(x, dtype=np.float32), device=device).to(torch.bfloat16)


def varlen_paged(seed, n_decode, dec_lo, dec_hi, n_chunk, chunk, pre_lo, pre_hi, Hq, Hkv, d, page, *,
                 mult=1.0, device="cpu"):
    """A mixed batch over a paged cache: n_decode sequences with one query token and
    uniform [dec_lo, dec_hi] cached keys (the token's own key included), then n_chunk
    sequences with `chunk` query tokens on a uniform [pre_lo, pre_hi] prefix.
    q [total_q, Hq, d] packed by cu_seqlens_q; caches, block_table, cache_seqlens as paged()."""
    g = generator(seed)
    dec = torch.randint(dec_lo, dec_hi + 1, (n_decode,), generator=g)
    pre = torch.randint(pre_lo, pre_hi + 1, (n_chunk,), generator=g)
    qlens = [1] * n_decode + [chunk] * n_chunk
    lens = dec.tolist() + (pre + chunk).tolist()
    t = paged(seed + 11, len(lens), Hq, Hkv, d, page, 0, 0, cache_seqlens=lens, mult=mult, device=device)
    gq = generator(seed + 13, device)
    t["q"] = randn_bf16(gq, (sum(qlens), Hq, d), mult, device)
    t["cu_seqlens_q"] = torch.tensor([0] + list(itertools.accumulate(qlens)), dtype=torch.int32)
    t["qlens"] = qlens
    return t
