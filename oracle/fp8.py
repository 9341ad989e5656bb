"""FP8 (e4m3) part of the oracle: exact decoding and encoding of the 8-bit
format, the per-block quantizer, and fp64 attention over dequantized inputs.

TEST INFRASTRUCTURE ONLY (like the rest of this package): the tests, the smoke
check and the CPU-baseline leg of the benchmark may use it; the library never
does.  Plain numpy, no code shared with the HIP path.

"Attention kernels: FlashAttention and PagedAttention", section 4.2 (the FP8
item) and "01 FlashAttention project overview & architecture", section 2.2 (the
FP8 E4M3 forward): Q, K and V enter the products as FP8 e4m3, with per-block
scales to keep the precision.
The format is the OCP 8-bit float E4M3 (the one gfx950's matrix units and
conversions use): 1 sign, 4 exponent (bias 7) and 3 mantissa bits; exponent
field 0 holds the subnormals m * 2^-9; S.1111.111 is NaN; there is no infinity;
the largest finite magnitude is 1.75 * 2^8 = 448.

Readings (the pages name the scheme, not its details):
- a block's scale is amax / 448 in fp32 (1 for an all-zero block), and a code is
  the e4m3 rounding (to nearest, ties to even, saturating at 448) of the fp32
  quotient x / scale: the same fp32 operations the GPU quantizer performs, so
  both sides take every rounding decision on the same fp32 number;
- Q is scaled per (batch, head, block of query rows), K per (batch, KV head,
  block of keys), V per (batch, KV head): the P V product accumulates across
  key blocks into one accumulator, so one V scale per head multiplies the
  result once.

Parity pins: tests/test_oracle_pins.py (the "fp8" section).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Exact value of each e4m3 code (uint8) as float64; NaN codes give NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    out = sign * mag
    return np.where((e == 15) & ((c & 0x7) == 7), np.nan, out)


# the 127 finite non-negative codes 0x00..0x7E in increasing order of value
_GRID = e4m3_decode(np.arange(127, dtype=np.uint8))


def e4m3_encode(x) -> np.ndarray:
    """Round each value to the nearest e4m3 code, ties to the even code, with
    magnitudes beyond 448 saturating to 448 and NaN giving 0x7F.  The sign of the
    input (also of -0.0 and of values that round to zero) is kept."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    hi = np.clip(np.searchsorted(_GRID, a, side="left"), 1, 126)   # _GRID[hi-1] < a <= _GRID[hi]
    lo = hi - 1
    dlo, dhi = a - _GRID[lo], _GRID[hi] - a
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(a >= E4M3_MAX, 126, pick)
    pick = np.where(a == 0, 0, pick)
    code = pick.astype(np.uint8) | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def _bf16_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _quantize_block(xb: np.ndarray):
    """xb: fp32 values of one block -> (codes, fp32 scale)."""
    amax = np.float32(np.abs(xb).max()) if xb.size else np.float32(0)
    scale = np.float32(amax / np.float32(E4M3_MAX)) if amax > 0 else np.float32(1.0)
    y = (xb / scale).astype(np.float32)          # one fp32 division per element, rounded to nearest
    return e4m3_encode(y), scale


def quantize_rows(x, block: int):
    """Per-block quantizer of a [B, N, H, d] bf16 tensor (bit patterns): one scale
    per (batch, head, block of `block` rows).  Returns (codes uint8 [B, N, H, d],
    scales float32 [B, H, ceil(N / block)])."""
    xf = _bf16_to_f32(x)
    B, N, H, d = xf.shape
    nb = -(-N // block)
    codes = np.zeros(xf.shape, dtype=np.uint8)
    scales = np.ones((B, H, nb), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                sl = slice(i * block, min(N, (i + 1) * block))
                codes[b, sl, h], scales[b, h, i] = _quantize_block(xf[b, sl, h])
    return codes, scales


def quantize_heads(x):
    """Per-head quantizer of a [B, N, H, d] bf16 tensor: one scale per (batch,
    head).  Returns (codes uint8 [B, N, H, d], scales float32 [B, H])."""
    xf = _bf16_to_f32(x)
    B, N, H, d = xf.shape
    codes = np.zeros(xf.shape, dtype=np.uint8)
    scales = np.ones((B, H), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            codes[b, :, h], scales[b, h] = _quantize_block(xf[b, :, h])
    return codes, scales


def dequantize(codes, scales, block=None) -> np.ndarray:
    """fp64 values of quantized [B, N, H, d] codes: scales [B, H, nblk] with rows in
    blocks of `block`, or [B, H] when block is None."""
    v = e4m3_decode(codes)
    s = np.asarray(scales, dtype=np.float64)
    if block is None:
        return v * s[:, None, :, None]
    N = v.shape[1]
    idx = np.arange(N) // block
    return v * np.transpose(s[:, :, idx], (0, 2, 1))[..., None]


def _visible(Lq, Lk, causal, window):
    """Key j is visible to query i (bottom-right: query i sits at key position
    i + Lk - Lq) inside the causal limit and the window [p - left, p + right]."""
    p = np.arange(Lq)[:, None] + (Lk - Lq)
    j = np.arange(Lk)[None, :]
    vis = np.ones((Lq, Lk), dtype=bool)
    if causal:
        vis &= j <= p
    if window is not None:
        left, right = window
        if left >= 0:
            vis &= j >= p - left
        if right >= 0:
            vis &= j <= p + right
    return vis


def fwd(q, q_scales, q_block, k, k_scales, k_block, v, v_scales, *, scale=None, causal=False,
        window=None, rows=None, with_abs=False):
    """Attention over the dequantized FP8 inputs, in fp64 with S and P materialised.

    q: codes [B, Nq, Hq, d] with q_scales [B, Hq, ceil(Nq / q_block)]; k: codes
    [B, Nk, Hkv, d] with k_scales [B, Hkv, ceil(Nk / k_block)]; v: codes
    [B, Nk, Hkv, d] with v_scales [B, Hkv].  Query head h uses KV head h // (Hq / Hkv).
    rows: None for all query rows, or a list of row indices (then O and LSE hold
    those rows only, in that order).  Returns (O float64 [B, rows, Hq, d],
    LSE float64 [B, Hq, rows]); a row that sees no key gets O = 0, LSE = -inf.
    with_abs: also return A = P |V| (the weights applied to the magnitudes of V),
    the scale of the error a relative rounding of each weight can cause.
    """
    qd = dequantize(q, q_scales, q_block)
    kd = dequantize(k, k_scales, k_block)
    vd = dequantize(v, v_scales)
    B, Nq, Hq, d = qd.shape
    Nk, Hkv = kd.shape[1], kd.shape[2]
    g = Hq // Hkv
    s = d ** -0.5 if scale is None else scale
    sel = np.arange(Nq) if rows is None else np.asarray(rows)
    vis = _visible(Nq, Nk, causal, window)[sel]
    O = np.zeros((B, len(sel), Hq, d))
    A = np.zeros((B, len(sel), Hq, d))
    L = np.full((B, Hq, len(sel)), -np.inf)
    for b in range(B):
        for h in range(Hq):
            S = s * (qd[b, sel, h] @ kd[b, :, h // g].T)
            S = np.where(vis, S, -np.inf)
            m = S.max(axis=1, keepdims=True)
            ok = np.isfinite(m[:, 0])
            E = np.exp(S - np.where(np.isfinite(m), m, 0.0))
            l = E.sum(axis=1)
            O[b, ok, h] = (E[ok] / l[ok, None]) @ vd[b, :, h // g]
            if with_abs:
                A[b, ok, h] = (E[ok] / l[ok, None]) @ np.abs(vd[b, :, h // g])
            L[b, h, ok] = m[ok, 0] + np.log(l[ok])
    return (O, L, A) if with_abs else (O, L)


# ---------------------------------------------------------------- FP8 KV cache
# "Attention kernels: FlashAttention and PagedAttention", section 5.2: a KV cache
# stored in FP8 halves the bytes a decode step reads.  Readings (the pages name the
# storage, not its scaling): one fp32 scale per cache tensor (k_scale, v_scale), an
# element's value is decode(code) * scale, and a new bf16 element x is stored as the
# e4m3 rounding of the fp32 quotient x / scale (the quantizer's rule above).  Pages
# follow section 6.1 of the same page: logical key t of sequence b is slot
# t % page of page block_table[b][t // page].


def encode_scaled(x_bits, scale) -> np.ndarray:
    """e4m3 codes of bf16 values (bit patterns) divided by a fp32 scale: one fp32
    division per element, then round to nearest even, saturating at 448."""
    y = (_bf16_to_f32(x_bits) / np.float32(scale)).astype(np.float32)
    return e4m3_encode(y)


def kvcache_append_fp8(k_new, v_new, k_codes, v_codes, k_scale, v_scale, block_table, cache_seqlens):
    """Append new bf16 tokens k_new, v_new [B, L, Hkv, d] (bit patterns) to the FP8
    caches [num_pages, page, Hkv, d] (uint8 codes): token t of sequence b lands at
    logical position cache_seqlens[b] + t.  Returns new (k_codes, v_codes); the
    inputs are not modified."""
    kn = np.asarray(k_new, dtype=np.uint16)
    vn = np.asarray(v_new, dtype=np.uint16)
    kc = np.array(k_codes, dtype=np.uint8, copy=True)
    vc = np.array(v_codes, dtype=np.uint8, copy=True)
    bt = np.asarray(block_table, dtype=np.int64)
    sl = np.asarray(cache_seqlens, dtype=np.int64)
    page = kc.shape[1]
    for b in range(kn.shape[0]):
        for t in range(kn.shape[1]):
            pos = int(sl[b]) + t
            phys = int(bt[b, pos // page])
            kc[phys, pos % page] = encode_scaled(kn[b, t], k_scale)
            vc[phys, pos % page] = encode_scaled(vn[b, t], v_scale)
    return kc, vc


def _gather(codes, bt_row, Lk, kvh):
    """Decoded [Lk, d] rows of KV head kvh of one sequence (logical key order)."""
    page = codes.shape[1]
    t = np.arange(Lk)
    return e4m3_decode(codes[bt_row[t // page], t % page, kvh])


def fwd_paged_fp8(q, k_codes, v_codes, k_scale, v_scale, block_table, cache_seqlens, *, scale=None,
                  causal=True, window=None, softcap=0.0, batches=None):
    """Attention of bf16 queries q [B, Nq, Hq, d] (bit patterns) over the paged FP8
    cache, in fp64 with S and P materialised: key j of sequence b is
    decode(k_codes[page, slot, h // g]) * k_scale (value likewise with v_scale),
    Lk = cache_seqlens[b] keys, query i at key position i + Lk - Nq (bottom-right).
    softcap c > 0 replaces each scaled logit s by c tanh(s / c).  batches: None for
    every sequence, or a list of sequence indices (O and LSE then hold those, in
    that order).  Returns (O float64 [nb, Nq, Hq, d], LSE float64 [nb, Hq, Nq]); a
    row that sees no key gets O = 0 and LSE = -inf."""
    qf = _bf16_to_f32(q).astype(np.float64)
    B, Nq, Hq, d = qf.shape
    Hkv = k_codes.shape[2]
    g = Hq // Hkv
    s = d ** -0.5 if scale is None else scale
    bt = np.asarray(block_table, dtype=np.int64)
    sl = np.asarray(cache_seqlens, dtype=np.int64)
    sel = list(range(B)) if batches is None else list(batches)
    O = np.zeros((len(sel), Nq, Hq, d))
    L = np.full((len(sel), Hq, Nq), -np.inf)
    for n, b in enumerate(sel):
        Lk = int(sl[b])
        vis = _visible(Nq, Lk, causal, window)
        for kvh in range(Hkv):
            kd = _gather(k_codes, bt[b], Lk, kvh) * np.float64(k_scale)
            vd = _gather(v_codes, bt[b], Lk, kvh) * np.float64(v_scale)
            for h in range(kvh * g, (kvh + 1) * g):
                S = s * (qf[b, :, h] @ kd.T)
                if softcap > 0:
                    S = softcap * np.tanh(S / softcap)
                S = np.where(vis, S, -np.inf)
                m = S.max(axis=1, keepdims=True) if Lk > 0 else np.full((Nq, 1), -np.inf)
                ok = np.isfinite(m[:, 0])
                E = np.exp(S - np.where(np.isfinite(m), m, 0.0))
                l = E.sum(axis=1)
                O[n, ok, h] = (E[ok] / l[ok, None]) @ vd
                L[n, h, ok] = m[ok, 0] + np.log(l[ok])
    return O, L


# ---------------------------------------------------------------- incoherent processing
# "Attention kernels: FlashAttention and PagedAttention", section 4.2 (the FP8
# item): Q and K are multiplied by a random orthogonal matrix before they are
# quantized, which spreads an outlier channel over every channel while leaving
# Q K^T unchanged ((Q R)(K R)^T = Q K^T for orthogonal R).  Reading (the pages
# name the idea, not the matrix): R = diag(s) H / sqrt(d), H the Sylvester
# Hadamard matrix of order d and s a caller-drawn vector of signs (+1 / -1), the
# randomized Hadamard transform, applied to every row of Q and of K with the same
# s.  The rotated values are formed in fp32 by the radix-2 Walsh-Hadamard
# butterfly (pairs i, i + h for h = 1, 2, 4, ..., d / 2 in that order, each giving
# a + b and a - b) and one multiply by fp32(1 / sqrt(d)); the quantizer's codes
# are decided on those fp32 values, as on the GPU.


def hadamard_rotate_f32(x, signs) -> np.ndarray:
    """Rows of x (float32 [..., d], d a power of two) times diag(signs) H / sqrt(d),
    computed in fp32 by the butterfly stages h = 1, 2, ..., d / 2."""
    y = np.asarray(x, dtype=np.float32) * np.asarray(signs, dtype=np.float32)
    d = y.shape[-1]
    lead = y.shape[:-1]
    h = 1
    while h < d:
        z = y.reshape(lead + (d // (2 * h), 2, h))
        a, b = z[..., 0, :], z[..., 1, :]
        y = np.stack([a + b, a - b], axis=-2).reshape(lead + (d,))
        h *= 2
    return (y * np.float32(1.0 / np.sqrt(d))).astype(np.float32)


def quantize_rows_rotated(x, block: int, signs):
    """quantize_rows of the rotated rows: every row of the [B, N, H, d] bf16 tensor
    (bit patterns) goes through hadamard_rotate_f32 with the given signs, then one
    scale per (batch, head, block of `block` rows) over the rotated values.
    Returns (codes uint8 [B, N, H, d], scales float32 [B, H, ceil(N / block)])."""
    yf = hadamard_rotate_f32(_bf16_to_f32(x), signs)
    B, N, H, d = yf.shape
    nb = -(-N // block)
    codes = np.zeros(yf.shape, dtype=np.uint8)
    scales = np.ones((B, H, nb), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                sl = slice(i * block, min(N, (i + 1) * block))
                codes[b, sl, h], scales[b, h, i] = _quantize_block(yf[b, sl, h])
    return codes, scales
