"""fp64 CPU oracle for the exact-attention forward pass (ctypes front end).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark may import this package; the library's compute path never
does.  It shares no code with the HIP path.

The arithmetic lives in ``oracle.c`` (plain C, fp64, S and P materialised,
three-pass softmax); this module only marshals numpy arrays.  Inputs are raw
bfloat16 bit patterns as ``numpy.uint16`` arrays.  Outputs are float64.

Parity-pin status of each function is listed in the header of ``oracle.c``
and in the tests under ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build() -> str:
    """Compile oracle.c into liboracle.so next to it (always recompiles)."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-fPIC", "-shared", "-o", tmp, _SRC,
           "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    L = ctypes.c_long
    D = ctypes.c_double
    I64 = ctypes.c_int64
    lib.oracle_version.restype = I
    lib.oracle_fwd_dense.argtypes = [P, P, P, I, L, L, I, I, I, D, I, L, L, D, P, I64, P, P, I]
    lib.oracle_fwd_dense.restype = I
    lib.oracle_fwd_varlen.argtypes = [P, P, P, P, P, I, I, I, I, D, I, L, L, D, P, I64, P, P, I]
    lib.oracle_fwd_varlen.restype = I
    lib.oracle_fwd_paged.argtypes = [P, P, P, P, P, I, L, I, I, I, L, L, D, I, L, L, D, I, I,
                                     P, I64, P, P, I]
    lib.oracle_fwd_paged.restype = I
    lib.oracle_combine.argtypes = [P, P, I, I64, I, P, P]
    lib.oracle_combine.restype = None
    lib.oracle_online_dense.argtypes = [P, P, P, I, L, L, I, I, I, D, I, L, L, D, L, P, I64, P, P]
    lib.oracle_online_dense.restype = I
    lib.oracle_probs_dense.argtypes = [P, P, P, I, L, L, I, I, I, D, I, L, L, D, L, P]
    lib.oracle_probs_dense.restype = I
    _lib = lib
    return lib


def default_threads() -> int:
    """Host threads for the oracle: OMP_NUM_THREADS if set, at most 16 and the CPU count."""
    try:
        n = int(os.environ.get("OMP_NUM_THREADS", "16") or 16)
    except ValueError:
        n = 16
    return max(1, min(n, 16, os.cpu_count() or 1))


def _threads(n):
    return default_threads() if not n or n <= 0 else int(n)


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("oracle inputs are bfloat16 bit patterns (numpy.uint16)")
    return a


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a) -> int | None:
    return None if a is None else a.ctypes.data


def _rows(rows):
    if rows is None:
        return None, 0
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    return r, int(r.size)


def _scale(scale, d):
    # default softmax scale d^-0.5 ("FA4 (CuTeDSL) and engineering interfaces", section 3)
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def _window(window):
    wl, wr = (-1, -1) if window is None else window
    return int(wl), int(wr)


def fwd_dense(q, k, v, *, scale=None, causal=False, window=None, softcap=0.0,
              rows=None, nthreads=0):
    """Dense BSHD forward.  q [B, Nq, Hq, d], k/v [B, Nk, Hkv, d] (uint16 bf16 bits).

    Returns (O, LSE).  With rows=None: O [B, Nq, Hq, d], LSE [B, Hq, Nq].
    With rows (flat indices r = (b*Hq + h)*Nq + i): O [n, d], LSE [n].
    """
    lib = _load()
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    rr, n = _rows(rows)
    total = B * Hq * Nq if rr is None else n
    o = np.empty((total, d), np.float64)
    lse = np.empty((total,), np.float64)
    wl, wr = _window(window)
    rc = lib.oracle_fwd_dense(_ptr(q), _ptr(k), _ptr(v), B, Nq, Nk, Hq, Hkv, d,
                              _scale(scale, d), int(bool(causal)), wl, wr, float(softcap),
                              _ptr(rr), n, _ptr(o), _ptr(lse), _threads(nthreads))
    if rc < 0:
        raise ValueError("oracle_fwd_dense rejected its arguments")
    if rr is None:
        o = o.reshape(B, Hq, Nq, d).transpose(0, 2, 1, 3).copy()
        lse = lse.reshape(B, Hq, Nq)
    return o, lse


def fwd_varlen(q, k, v, cu_q, cu_k, *, scale=None, causal=False, window=None,
               softcap=0.0, rows=None, nthreads=0):
    """Varlen forward.  q [Tq, Hq, d], k/v [Tk, Hkv, d], cu_q/cu_k [B+1].

    Returns (O, LSE).  With rows=None: O [Tq, Hq, d], LSE [Hq, Tq].
    With rows (flat indices r = h*Tq + t): O [n, d], LSE [n].
    """
    lib = _load()
    q, k, v = _u16(q), _u16(k), _u16(v)
    cu_q, cu_k = _i32(cu_q), _i32(cu_k)
    Tq, Hq, d = q.shape
    Hkv = k.shape[1]
    B = cu_q.size - 1
    rr, n = _rows(rows)
    total = Hq * Tq if rr is None else n
    o = np.empty((total, d), np.float64)
    lse = np.empty((total,), np.float64)
    wl, wr = _window(window)
    rc = lib.oracle_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_q), _ptr(cu_k), B, Hq, Hkv, d,
                               _scale(scale, d), int(bool(causal)), wl, wr, float(softcap),
                               _ptr(rr), n, _ptr(o), _ptr(lse), _threads(nthreads))
    if rc < 0:
        raise ValueError("oracle_fwd_varlen rejected its arguments")
    if rr is None:
        o = o.reshape(Hq, Tq, d).transpose(1, 0, 2).copy()
        lse = lse.reshape(Hq, Tq)
    return o, lse


def fwd_paged(q, k_cache, v_cache, block_table, cache_seqlens, *, scale=None,
              causal=True, window=None, softcap=0.0, num_splits=0, split=0,
              rows=None, nthreads=0):
    """Paged-KV forward.  q [B, Nq, Hq, d]; caches [num_pages, page, Hkv, d];
    block_table [B, max_blocks]; cache_seqlens [B].

    num_splits == 0 attends over the whole cache; num_splits > 0 returns the
    normalised partial (O_s, LSE_s) of split `split` only.
    Returns (O, LSE) shaped like fwd_dense.
    """
    lib = _load()
    q, kc, vc = _u16(q), _u16(k_cache), _u16(v_cache)
    bt, sl = _i32(block_table), _i32(cache_seqlens)
    B, Nq, Hq, d = q.shape
    page, Hkv = kc.shape[1], kc.shape[2]
    max_blocks = bt.shape[1]
    rr, n = _rows(rows)
    total = B * Hq * Nq if rr is None else n
    o = np.empty((total, d), np.float64)
    lse = np.empty((total,), np.float64)
    wl, wr = _window(window)
    rc = lib.oracle_fwd_paged(_ptr(q), _ptr(kc), _ptr(vc), _ptr(bt), _ptr(sl), B, Nq, Hq, Hkv, d,
                              page, max_blocks, _scale(scale, d), int(bool(causal)), wl, wr,
                              float(softcap), int(num_splits), int(split), _ptr(rr), n,
                              _ptr(o), _ptr(lse), _threads(nthreads))
    if rc < 0:
        raise ValueError("oracle_fwd_paged rejected its arguments")
    if rr is None:
        o = o.reshape(B, Hq, Nq, d).transpose(0, 2, 1, 3).copy()
        lse = lse.reshape(B, Hq, Nq)
    return o, lse


def combine(o_part, lse_part):
    """Merge partial states.  o_part [S, rows, d], lse_part [S, rows] (float64).
    Returns (O [rows, d], LSE [rows])."""
    lib = _load()
    o_part = np.ascontiguousarray(o_part, dtype=np.float64)
    lse_part = np.ascontiguousarray(lse_part, dtype=np.float64)
    S, rows, d = o_part.shape
    o = np.empty((rows, d), np.float64)
    lse = np.empty((rows,), np.float64)
    lib.oracle_combine(_ptr(o_part), _ptr(lse_part), S, rows, d, _ptr(o), _ptr(lse))
    return o, lse


def online_dense(q, k, v, *, block_n, scale=None, causal=False, window=None, softcap=0.0,
                 rows=None):
    """The (m, l, O) recurrence over key blocks of block_n keys; outputs as fwd_dense."""
    lib = _load()
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    rr, n = _rows(rows)
    total = B * Hq * Nq if rr is None else n
    o = np.empty((total, d), np.float64)
    lse = np.empty((total,), np.float64)
    wl, wr = _window(window)
    rc = lib.oracle_online_dense(_ptr(q), _ptr(k), _ptr(v), B, Nq, Nk, Hq, Hkv, d,
                                 _scale(scale, d), int(bool(causal)), wl, wr, float(softcap),
                                 int(block_n), _ptr(rr), n, _ptr(o), _ptr(lse))
    if rc < 0:
        raise ValueError("oracle_online_dense rejected its arguments")
    if rr is None:
        o = o.reshape(B, Hq, Nq, d).transpose(0, 2, 1, 3).copy()
        lse = lse.reshape(B, Hq, Nq)
    return o, lse


def probs_dense(q, k, v, row, *, scale=None, causal=False, window=None, softcap=0.0):
    """The materialised probability row P[row, :] (length Nk) of a dense problem."""
    lib = _load()
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    p = np.empty((Nk,), np.float64)
    wl, wr = _window(window)
    rc = lib.oracle_probs_dense(_ptr(q), _ptr(k), _ptr(v), B, Nq, Nk, Hq, Hkv, d,
                                _scale(scale, d), int(bool(causal)), wl, wr, float(softcap),
                                int(row), _ptr(p))
    if rc < 0:
        raise ValueError("oracle_probs_dense rejected its arguments")
    return p


def kvcache_append(k_new, v_new, k_cache, v_cache, block_table, cache_seqlens):
    """In-place append of new tokens to a paged cache, written out from its
    definition ("FA4 (CuTeDSL) and engineering interfaces", section 6.2: the new
    k, v go into the cache; "Attention kernels: FlashAttention and
    PagedAttention", section 6.1: logical key t of sequence b is slot t % page of
    page block_table[b][t // page]).  Token t of sequence b lands at logical
    position cache_seqlens[b] + t.  Pure indexing (no arithmetic), so it lives
    here rather than in oracle.c.

    k_new, v_new: uint16 [B, L, Hkv, d]; caches: uint16 [num_pages, page, Hkv, d].
    Returns new (k_cache, v_cache); the inputs are not modified.
    """
    k_new, v_new = _u16(k_new), _u16(v_new)
    kc, vc = _u16(k_cache).copy(), _u16(v_cache).copy()
    bt, sl = _i32(block_table), _i32(cache_seqlens)
    B, L = k_new.shape[0], k_new.shape[1]
    page = kc.shape[1]
    for b in range(B):
        for t in range(L):
            pos = int(sl[b]) + t
            phys = int(bt[b, pos // page])
            kc[phys, pos % page] = k_new[b, t]
            vc[phys, pos % page] = v_new[b, t]
    return kc, vc


def rotary(x, cos, sin, positions, *, interleaved=False):
    """Rotary position embedding in fp64, from its definition (RoFormer, Su et al.
    2021: a position rotates each pair of dims by its angle; the pages only say the
    kvcache call can apply it, "FA4 (CuTeDSL) and engineering interfaces", section 6.2).

    x: uint16 bf16 bits [..., L, H, d]; cos, sin: float [positions, r/2]; positions:
    int [..., L] (the position of each token).  Frequency i of position p rotates the
    pair of dims (i, i + r/2) (or (2i, 2i + 1) when interleaved) by the angle with
    cosine cos[p, i] and sine sin[p, i]: (a, b) -> (a cos - b sin, a sin + b cos).
    Dims from r on are unchanged.  Returns float64 of x's shape.
    """
    xd = _u16(x).astype(np.uint32) << 16
    xd = xd.view(np.float32).astype(np.float64)
    cos = np.asarray(cos, dtype=np.float64)
    sin = np.asarray(sin, dtype=np.float64)
    pos = np.asarray(positions, dtype=np.int64)
    half = cos.shape[1]
    out = xd.copy()
    c = cos[pos][..., None, :]          # [..., L, 1, r/2]
    s = sin[pos][..., None, :]
    if interleaved:
        a, b = xd[..., 0:2 * half:2], xd[..., 1:2 * half:2]
        out[..., 0:2 * half:2] = a * c - b * s
        out[..., 1:2 * half:2] = a * s + b * c
    else:
        a, b = xd[..., :half], xd[..., half:2 * half]
        out[..., :half] = a * c - b * s
        out[..., half:2 * half] = a * s + b * c
    return out


def _f64(a):
    """bf16 bit patterns (uint16) -> float64."""
    return (_u16(a).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def visible_mask(Lq, Lk, causal, window):
    """visible[i, j] for query i of Lq and key j of Lk, bottom-right aligned (query i at
    key position i + Lk - Lq): the same predicate the forward oracle evaluates."""
    wl, wr = _window(window)
    pos = np.arange(Lq)[:, None] + (Lk - Lq)
    j = np.arange(Lk)[None, :]
    vis = np.ones((Lq, Lk), bool)
    if causal:
        vis &= j <= pos
    if wl >= 0:
        vis &= j >= pos - wl
    if wr >= 0:
        vis &= j <= pos + wr
    return vis


def _masked_softmax_rows(S, vis, V):
    """Three-pass softmax of each row of S over its visible keys, then P V.
    Returns (O [rows, d], LSE [rows]); a row with no visible key gives 0 and -inf."""
    S = np.where(vis, S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    ok = np.isfinite(m[:, 0])
    E = np.exp(S - np.where(np.isfinite(m), m, 0.0))
    l = E.sum(axis=1)
    O = np.zeros((S.shape[0], V.shape[1]))
    L = np.full(S.shape[0], -np.inf)
    O[ok] = (E[ok] / l[ok, None]) @ V
    L[ok] = m[ok, 0] + np.log(l[ok])
    return O, L


def fwd_dense_relpos(q, k, v, bias, *, scale=None, causal=False, window=None, rows=None):
    """Attention with a learned relative-position bias, a score_mod ("FA4 (CuTeDSL) and
    engineering interfaces", sections 1 and 7: a function that rewrites each logit after
    Q K^T and before the softmax): the logit of the query at position p_i = i + Lk - Lq
    and key j is scale q_i . k_j + bias[h, clamp(j - p_i, -R, R) + R] for a table of
    2R + 1 entries per query head; then the usual masked softmax.  fp64 with S and P
    materialised, in numpy.

    q: bf16 bits [B, Nq, Hq, d]; k, v: [B, Nk, Hkv, d]; bias: float [Hq, 2R + 1].
    rows: None, or a list of query rows (O and LSE hold those rows only).
    Returns (O float64 [B, rows, Hq, d], LSE float64 [B, Hq, rows])."""
    qd, kd, vd = _f64(q), _f64(k), _f64(v)
    B, Nq, Hq, d = qd.shape
    Nk, Hkv = kd.shape[1], kd.shape[2]
    g = Hq // Hkv
    s = _scale(scale, d)
    tb = np.asarray(bias, dtype=np.float64)
    R = (tb.shape[1] - 1) // 2
    sel = np.arange(Nq) if rows is None else np.asarray(rows)
    vis = visible_mask(Nq, Nk, causal, window)[sel]
    rel = np.clip(np.arange(Nk)[None, :] - (sel[:, None] + (Nk - Nq)), -R, R) + R
    O = np.zeros((B, len(sel), Hq, d))
    L = np.full((B, Hq, len(sel)), -np.inf)
    for b in range(B):
        for h in range(Hq):
            S = s * (qd[b, sel, h] @ kd[b, :, h // g].T) + tb[h][rel]
            O[b, :, h], L[b, h] = _masked_softmax_rows(S, vis, vd[b, :, h // g])
    return O, L


def prefix_lm_visible(Lq, Lk, prefix, window=None):
    """visible[i, j] of the prefix-LM mask, a mask_mod ("FA4 (CuTeDSL) and engineering
    interfaces", sections 1 and 7): the first `prefix` keys are visible to every query,
    later keys causally (j <= p_i, p_i = i + Lk - Lq), intersected with the window and
    with 0 <= j < Lk."""
    pos = np.arange(Lq)[:, None] + (Lk - Lq)
    j = np.arange(Lk)[None, :]
    vis = (j < prefix) | (j <= pos)
    return vis & visible_mask(Lq, Lk, False, window)


def fwd_dense_prefix_lm(q, k, v, prefix_lens, *, scale=None, window=None, rows=None):
    """Attention under the prefix-LM mask (prefix_lm_visible, prefix_lens [B]); otherwise
    as fwd_dense_relpos without a bias.  fp64, S and P materialised, in numpy."""
    qd, kd, vd = _f64(q), _f64(k), _f64(v)
    B, Nq, Hq, d = qd.shape
    Nk, Hkv = kd.shape[1], kd.shape[2]
    g = Hq // Hkv
    s = _scale(scale, d)
    sel = np.arange(Nq) if rows is None else np.asarray(rows)
    O = np.zeros((B, len(sel), Hq, d))
    L = np.full((B, Hq, len(sel)), -np.inf)
    for b in range(B):
        vis = prefix_lm_visible(Nq, Nk, int(prefix_lens[b]), window)[sel]
        for h in range(Hq):
            S = s * (qd[b, sel, h] @ kd[b, :, h // g].T)
            O[b, :, h], L[b, h] = _masked_softmax_rows(S, vis, vd[b, :, h // g])
    return O, L


def bwd_dense(q, k, v, dout, *, scale=None, causal=False, window=None, softcap=0.0, heads=None):
    """Gradients of the attention forward, in fp64 with S and P materialised.

    "Attention kernels: FlashAttention and PagedAttention", section 4.3: the
    backward recomputes S = Q K^T, takes P from the saved log-sum-exp and forms
    dV = P^T dO and dS.  The rest is the derivative of softmax attention written
    out: dP = dO V^T, D = rowsum(dO * O) (the preprocess the overview page lists),
    dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q.  Query head h uses KV
    head h // (Hq / Hkv), so dK and dV sum over the query heads of a group.
    Rows that see no key have P = 0 and contribute nothing.
    softcap c > 0: the logit is c tanh(scale q.k / c) (the forward's transform,
    "FA4 (CuTeDSL) and engineering interfaces", section 7), so by the chain rule dS
    is multiplied by its derivative 1 - tanh^2(scale q.k / c) before dQ and dK.

    q, dout: uint16 bf16 bits [B, Nq, Hq, d]; k, v: [B, Nk, Hkv, d].  heads: None for
    all query heads, or a list of query heads (then dK, dV hold only their share).
    Returns float64 (dq [B, Nq, Hq, d], dk [B, Nk, Hkv, d], dv [B, Nk, Hkv, d]).
    """
    qd, kd, vd, od = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Nq, Hq, d = qd.shape
    Nk, Hkv = kd.shape[1], kd.shape[2]
    g = Hq // Hkv
    s = _scale(scale, d)
    vis = visible_mask(Nq, Nk, causal, window)
    dq = np.zeros_like(qd)
    dk = np.zeros_like(kd)
    dv = np.zeros_like(vd)
    for b in range(B):
        for h in (range(Hq) if heads is None else heads):
            hk = h // g
            S = s * (qd[b, :, h] @ kd[b, :, hk].T)
            dcap = 1.0
            if softcap > 0:
                th = np.tanh(S / softcap)
                S = softcap * th
                dcap = 1.0 - th * th
            S = np.where(vis, S, -np.inf)
            m = S.max(axis=1, keepdims=True)
            empty = ~np.isfinite(m)
            E = np.exp(S - np.where(empty, 0.0, m))
            P = E / np.where(empty, 1.0, E.sum(axis=1, keepdims=True))
            O = P @ vd[b, :, hk]
            dO = od[b, :, h]
            Dr = np.sum(dO * O, axis=1, keepdims=True)
            dP = dO @ vd[b, :, hk].T
            dS = P * (dP - Dr) * dcap
            dv[b, :, hk] += P.T @ dO
            dq[b, :, h] = s * (dS @ kd[b, :, hk])
            dk[b, :, hk] += s * (dS.T @ qd[b, :, h])
    return dq, dk, dv


def fwd_dense_alibi(q, k, v, slopes, *, scale=None, causal=False, window=None, rows=None):
    """Attention with ALiBi ("FA4 (CuTeDSL) and engineering interfaces", section 7:
    a linear positional bias on the logits, alibi_slopes per head): the logit of
    query i and key j is scale q_i . k_j - slope_h |p_i - j| with p_i = i + Lk - Lq
    (the bottom-right position, as for the causal mask), then the usual masked
    softmax.  fp64 with S and P materialised, in numpy.

    q: bf16 bits [B, Nq, Hq, d]; k, v: [B, Nk, Hkv, d]; slopes: [Hq] or [B, Hq].
    rows: None, or a list of query rows (O and LSE hold those rows only).
    Returns (O float64 [B, rows, Hq, d], LSE float64 [B, Hq, rows])."""
    qd, kd, vd = _f64(q), _f64(k), _f64(v)
    B, Nq, Hq, d = qd.shape
    Nk, Hkv = kd.shape[1], kd.shape[2]
    g = Hq // Hkv
    s = _scale(scale, d)
    sl = np.asarray(slopes, dtype=np.float64)
    sl = np.broadcast_to(sl, (B, Hq)) if sl.ndim == 1 else sl
    sel = np.arange(Nq) if rows is None else np.asarray(rows)
    vis = visible_mask(Nq, Nk, causal, window)[sel]
    dist = np.abs((sel[:, None] + (Nk - Nq)) - np.arange(Nk)[None, :]).astype(np.float64)
    O = np.zeros((B, len(sel), Hq, d))
    L = np.full((B, Hq, len(sel)), -np.inf)
    for b in range(B):
        for h in range(Hq):
            S = s * (qd[b, sel, h] @ kd[b, :, h // g].T) - sl[b, h] * dist
            S = np.where(vis, S, -np.inf)
            m = S.max(axis=1, keepdims=True)
            ok = np.isfinite(m[:, 0])
            E = np.exp(S - np.where(np.isfinite(m), m, 0.0))
            l = E.sum(axis=1)
            O[b, ok, h] = (E[ok] / l[ok, None]) @ vd[b, :, h // g]
            L[b, h, ok] = m[ok, 0] + np.log(l[ok])
    return O, L
