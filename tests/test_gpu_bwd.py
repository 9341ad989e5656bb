"""GPU parity for the backward pass (fa_bwd) against the fp64 oracle (oracle.bwd_dense).

Tolerance: the gradients are rounded to bf16 on output (half an ulp, 2^-9 relative)
and P and dS are rounded to bf16 before their products (about as much again), so
an element carries up to about 2^-8 of relative error; with a factor of two of
margin the largest error must stay within 1 % of the tensor's largest magnitude
and the mean error within 0.4 % of its mean magnitude.  Gradients that vanish
exactly (one visible key: dS = dP - D = 0) keep what fp32 accumulation of two
d-term dot products in different orders leaves, about 2^-24 d of the unit-scale
inputs, hence an absolute floor of 1e-4 (max) and 1e-5 (mean).
"""
import numpy as np
import pytest
import torch

import oracle
from exact_attention_72_amd import api, workloads as W
from gpu_util import DEV, bits

pytestmark = pytest.mark.gpu

MAX_REL, MEAN_REL = 1e-2, 4e-3
MAX_ABS, MEAN_ABS = 1e-4, 1e-5


def check_grads(got, ref, what):
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        x = g.float().cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(x)), f"{what} {name}: non-finite"
        e = np.abs(x - r)
        scale_max, scale_mean = np.abs(r).max(), np.abs(r).mean()
        msg = (f"{what} {name}: max err {e.max():.3e} (tensor max {scale_max:.3e}), "
               f"mean err {e.mean():.3e} (tensor mean {scale_mean:.3e})")
        print(msg)
        assert e.max() <= MAX_REL * scale_max + MAX_ABS and e.mean() <= MEAN_REL * scale_mean + MEAN_ABS, msg


def run_case(B, Nq, Nk, Hq, Hkv, d, causal, window, seed):
    t = W.dense(seed, B, Nq, Hq, Hkv, d, Nk=Nk)
    do = W.randn_bf16(W.generator(seed + 1), (B, Nq, Hq, d))
    q, k, v = (t[n].to(DEV) for n in "qkv")
    out, lse = api.fa_fwd(q, k, v, causal=causal, window=window)
    grads = api.fa_bwd(q, k, v, out, lse, do.to(DEV), causal=causal, window=window)
    torch.cuda.synchronize()
    return t, do, grads


CASES = [
    # B, Nq, Nk, Hq, Hkv, d, causal, window
    (2, 200, 200, 4, 4, 128, True, None),
    (1, 333, 333, 4, 2, 128, False, None),   # GQA, dK/dV summed over 2 query heads
    (2, 130, 190, 4, 1, 64, True, None),     # bottom-right, Nk > Nq, MQA
    (1, 190, 120, 2, 2, 128, True, None),    # first rows see no key
    (1, 300, 300, 2, 2, 128, True, (70, 0)), # sliding window
    (1, 257, 257, 2, 2, 64, False, (40, 20)),
    (1, 1, 1, 1, 1, 128, False, None),
]


@pytest.mark.parametrize("B,Nq,Nk,Hq,Hkv,d,causal,window", CASES)
def test_bwd_small(B, Nq, Nk, Hq, Hkv, d, causal, window):
    t, do, got = run_case(B, Nq, Nk, Hq, Hkv, d, causal, window, 401 + Nq + Nk)
    ref = oracle.bwd_dense(bits(t["q"]), bits(t["k"]), bits(t["v"]), bits(do), causal=causal, window=window)
    check_grads(got, ref, f"bwd {B}x{Nq}x{Nk} h{Hq}/{Hkv} d{d}")


def test_bwd_empty_rows_and_determinism():
    """Rows that see no key give exactly zero dQ; repeated runs are bitwise identical,
    also with other kernels run in between (they change what a kernel's waves
    find in registers and LDS, and how long its exits take)."""
    B, Nq, Nk, H, d = 1, 190, 120, 2, 128
    t, do, a = run_case(B, Nq, Nk, H, H, d, True, None, 77)
    other = W.dense(5, 1, 2048, 8, 8, 128, device=DEV)
    for _ in range(8):
        api.fa_fwd(other["q"], other["k"], other["v"], causal=True)
        _, _, b = run_case(B, Nq, Nk, H, H, d, True, None, 77)
        for x, y in zip(a, b):
            assert torch.equal(x, y)
    assert torch.count_nonzero(a[0][:, : Nq - Nk].float()) == 0


def test_bwd_custom_scale_and_strided_grads():
    B, N, Hq, Hkv, d = 1, 150, 4, 2, 128
    t = W.dense(88, B, N, Hq, Hkv, d)
    do = W.randn_bf16(W.generator(89), (B, N, Hq, d))
    q, k, v = (t[n].to(DEV) for n in "qkv")
    out, lse = api.fa_fwd(q, k, v, causal=True, softmax_scale=0.05)
    wide = torch.zeros(B, N, 2 * Hkv, d, dtype=torch.bfloat16, device=DEV)
    dk = wide[:, :, ::2]                   # gradients written into a strided view
    got = api.fa_bwd(q, k, v, out, lse, do.to(DEV), causal=True, softmax_scale=0.05, dk=dk)
    torch.cuda.synchronize()
    assert torch.count_nonzero(wide[:, :, 1::2]) == 0
    ref = oracle.bwd_dense(bits(t["q"]), bits(t["k"]), bits(t["v"]), bits(do), causal=True, scale=0.05)
    check_grads(got, ref, "bwd scale 0.05, strided dk")


def test_bwd_full_size_heads():
    """The benchmark's shape (batch 4, 16 heads, N = 4096, d = 128, causal), every row
    of three heads of the first sequence against the oracle."""
    c = W.WORKLOADS["prefill_b4_h16_n4096_d128_causal"]
    B, N, H, d = c["B"], c["N"], c["Hq"], c["d"]
    t = W.dense(c["seed"], B, N, H, H, d, device=DEV)
    do = W.randn_bf16(W.generator(c["seed"] + 100, DEV), (B, N, H, d), 1.0, DEV)
    out, lse = api.fa_fwd(t["q"], t["k"], t["v"], causal=True)
    dq, dk, dv = api.fa_bwd(t["q"], t["k"], t["v"], out, lse, do, causal=True)
    torch.cuda.synchronize()
    heads = [0, 7, 15]
    ref = oracle.bwd_dense(bits(t["q"][:1]), bits(t["k"][:1]), bits(t["v"][:1]), bits(do[:1]), causal=True,
                           heads=heads)
    got = [x[:1, :, heads] for x in (dq, dk, dv)]
    check_grads(got, [r[:, :, heads] for r in ref], "bwd full size, batch 0, heads 0/7/15")


# ---------------------------------------------------------------- varlen (fa_bwd_varlen)
VARLEN_CASES = [
    # query lengths, key lengths, Hq, Hkv, d, causal, window
    ([1, 64, 130, 257, 3], None, 8, 2, 128, True, None),
    ([5, 200, 0, 77, 40], [300, 200, 10, 77, 0], 4, 4, 128, True, None),   # Lk > Lq, an empty query set, no keys
    ([100, 333, 17], None, 4, 1, 64, False, (40, 20)),
    ([129, 31], [150, 31], 2, 2, 128, True, (64, 0)),
]


@pytest.mark.parametrize("lq,lk,Hq,Hkv,d,causal,window", VARLEN_CASES)
def test_bwd_varlen(lq, lk, Hq, Hkv, d, causal, window):
    """Packed sequences (the varlen forward's layout) against the oracle's dense backward of
    each sequence on its own (bottom-right per sequence; GQA sums over the group)."""
    lk = lq if lk is None else lk
    print(f"bwd varlen lq={lq} lk={lk} h{Hq}/{Hkv} d{d}", flush=True)
    g = W.generator(501 + sum(lq) + d)
    cq, ck = W.prefix_sum(torch.tensor(lq)), W.prefix_sum(torch.tensor(lk))
    Tq, Tk = int(cq[-1]), int(ck[-1])
    q = W.randn_bf16(g, (Tq, Hq, d))
    k = W.randn_bf16(g, (Tk, Hkv, d))
    v = W.randn_bf16(g, (Tk, Hkv, d))
    do = W.randn_bf16(g, (Tq, Hq, d))
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    cqd, ckd = cq.to(DEV), ck.to(DEV)
    out, lse = api.fa_fwd_varlen(qd, kd, vd, cqd, ckd, max(lq), causal=causal, window=window)
    dq, dk, dv = api.fa_bwd_varlen(qd, kd, vd, out, lse, do.to(DEV), cqd, ckd, max(lq), max(lk), causal=causal,
                                   window=window)
    torch.cuda.synchronize()
    cqh, ckh = cq.tolist(), ck.tolist()
    for s in range(len(lq)):
        a, b = cqh[s], cqh[s + 1]
        c, e = ckh[s], ckh[s + 1]
        got = (dq[a:b], dk[c:e], dv[c:e])
        if b == a or e == c:
            # no queries or no keys: nothing flows, every gradient element is zero
            for x in got:
                assert torch.count_nonzero(x.float()) == 0, f"sequence {s}"
            continue
        ref = oracle.bwd_dense(bits(q[a:b][None]), bits(k[c:e][None]), bits(v[c:e][None]), bits(do[a:b][None]),
                               causal=causal, window=window)
        check_grads(got, tuple(r[0] for r in ref), f"bwd varlen sequence {s} ({b - a} x {e - c})")


def test_bwd_varlen_equals_dense_on_equal_lengths():
    """Four sequences of one length packed: bitwise the dense backward of the same tensors."""
    B, N, Hq, Hkv, d = 4, 300, 4, 2, 128
    t = W.dense(511, B, N, Hq, Hkv, d, device=DEV)
    do = W.randn_bf16(W.generator(512), (B, N, Hq, d)).to(DEV)
    out, lse = api.fa_fwd(t["q"], t["k"], t["v"], causal=True)
    dense = api.fa_bwd(t["q"], t["k"], t["v"], out, lse, do, causal=True)
    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32, device=DEV)
    flat = lambda x: x.reshape(B * x.shape[1], x.shape[2], x.shape[3])  # noqa: E731
    lse_v = lse.permute(1, 0, 2).reshape(Hq, B * N).contiguous()
    packed = api.fa_bwd_varlen(flat(t["q"]), flat(t["k"]), flat(t["v"]), flat(out), lse_v, flat(do), cu, cu, N, N,
                               causal=True)
    torch.cuda.synchronize()
    for x, y in zip(dense, packed):
        assert torch.equal(x.reshape(y.shape), y)


# ---------------------------------------------------------------- softcap
SOFTCAP_CASES = [
    # B, Nq, Nk, Hq, Hkv, d, causal, window, softcap, input scale
    (2, 200, 200, 4, 4, 128, True, None, 30.0, 2.0),     # the long-context workload's cap on its inputs
    (1, 333, 333, 4, 2, 128, False, None, 3.0, 2.0),     # a small cap that bends most scores
    (1, 190, 120, 2, 2, 64, True, None, 5.0, 1.0),       # rows that see no key
    (1, 300, 300, 2, 2, 128, True, (70, 0), 4.0, 2.0),   # window
]


@pytest.mark.parametrize("B,Nq,Nk,Hq,Hkv,d,causal,window,cap,mult", SOFTCAP_CASES)
def test_bwd_softcap(B, Nq, Nk, Hq, Hkv, d, causal, window, cap, mult):
    t = W.dense(451 + Nq + Nk, B, Nq, Hq, Hkv, d, Nk=Nk, mult=mult)
    do = W.randn_bf16(W.generator(452 + Nq), (B, Nq, Hq, d))
    q, k, v = (t[n].to(DEV) for n in "qkv")
    out, lse = api.fa_fwd(q, k, v, causal=causal, window=window, softcap=cap)
    got = api.fa_bwd(q, k, v, out, lse, do.to(DEV), causal=causal, window=window, softcap=cap)
    torch.cuda.synchronize()
    ref = oracle.bwd_dense(bits(t["q"]), bits(t["k"]), bits(t["v"]), bits(do), causal=causal, window=window,
                           softcap=cap)
    check_grads(got, ref, f"bwd softcap {cap} {B}x{Nq}x{Nk} h{Hq}/{Hkv} d{d}")
    if causal and Nq > Nk:
        assert torch.count_nonzero(got[0][:, : Nq - Nk].float()) == 0


def test_bwd_varlen_softcap():
    lq = [1, 64, 130, 257]
    g = W.generator(461)
    cu = W.prefix_sum(torch.tensor(lq))
    T, Hq, Hkv, d, cap = int(cu[-1]), 8, 2, 128, 4.0
    q, k, v = W.randn_bf16(g, (T, Hq, d), 2.0), W.randn_bf16(g, (T, Hkv, d), 2.0), W.randn_bf16(g, (T, Hkv, d), 2.0)
    do = W.randn_bf16(g, (T, Hq, d))
    cud = cu.to(DEV)
    out, lse = api.fa_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cud, cud, max(lq), causal=True, softcap=cap)
    dq, dk, dv = api.fa_bwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), out, lse, do.to(DEV), cud, cud, max(lq), max(lq),
                                   causal=True, softcap=cap)
    torch.cuda.synchronize()
    c = cu.tolist()
    for s in range(len(lq)):
        a, b = c[s], c[s + 1]
        ref = oracle.bwd_dense(bits(q[a:b][None]), bits(k[a:b][None]), bits(v[a:b][None]), bits(do[a:b][None]),
                               causal=True, softcap=cap)
        check_grads((dq[a:b], dk[a:b], dv[a:b]), tuple(r[0] for r in ref), f"bwd varlen softcap sequence {s}")
