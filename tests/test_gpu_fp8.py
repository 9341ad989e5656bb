"""GPU parity of the FP8 (e4m3) forward: the quantizers bit-exact against the
oracle's, the attention against the fp64 oracle over the oracle's own
quantization of the same inputs.

Attention tolerance, per element (row i, dim d).  The scores are exact products
of e4m3 codes summed in fp32 and the row sum is fp32, so what remains is the
e4m3 rounding of each weight in the P V product: a weight w_j enters as
w_j (1 + e_j) with |e_j| <= 2^-4 (round to nearest in a format with 3 mantissa
bits; weights below e4m3's normal range are 2^-14 of the row maximum or less),
and the bf16 rounding of O (2^-9 relative).  Hence
    |O_gpu - O| <= 2^-4 A + 2^-9 |O|,   A = sum_j w_j |V_jd|  (from the oracle),
checked for every element with 5 % slack and 1e-5 absolute, and on average
against half of it (the e_j have both signs).  LSE: fp32 sums, max-abs 1e-3.
"""
import numpy as np
import pytest
import torch

from oracle import fp8 as F8
from exact_attention_72_amd import api, workloads as W
from gpu_util import DEV, bits

pytestmark = pytest.mark.gpu


def key_of_position(p):
    """Position p of a 64-key group of the transposed V layout -> key in the group
    (include/fa.h, fa_fp8_quantize_v)."""
    return 32 * ((p >> 4) & 1) + 8 * ((p >> 2) & 3) + 4 * (p >> 5) + (p & 3)


def vt_to_rows(vt, N):
    """[B, H, d, L] transposed codes -> [B, N, H, d] codes, and the padding positions."""
    vt = vt.cpu().numpy()
    B, H, d, L = vt.shape
    keys = np.array([64 * (p // 64) + key_of_position(p % 64) for p in range(L)])
    out = np.zeros((B, L, H, d), dtype=np.uint8)
    out[:, keys] = np.transpose(vt, (0, 3, 1, 2))
    return out[:, :N], out[:, N:]


@pytest.mark.parametrize("d,block,N,strided", [(128, 128, 300, False), (128, 64, 200, True), (64, 64, 77, False),
                                                 (128, 128, 1, False)])
def test_quantize_rows_bit_exact(d, block, N, strided):
    x = W.randn_bf16(W.generator(61 + N), (2, N, 3, d), 2.0)
    xd = x.to(DEV)
    if strided:
        wide = torch.zeros(2, N, 6, d, dtype=torch.bfloat16, device=DEV)
        wide[:, :, ::2] = xd
        xd = wide[:, :, ::2]
    codes, scales = api.fa_fp8_quantize(xd, block)
    torch.cuda.synchronize()
    rc, rs = F8.quantize_rows(bits(x), block)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


@pytest.mark.parametrize("d,N", [(128, 150), (128, 64), (64, 100), (128, 1)])
def test_quantize_v_layout_bit_exact(d, N):
    v = W.randn_bf16(W.generator(71 + N), (2, N, 2, d))
    vt, scales = api.fa_fp8_quantize_v(v.to(DEV))
    torch.cuda.synchronize()
    assert vt.shape[-1] == -(-N // 64) * 64
    rc, rs = F8.quantize_heads(bits(v))
    assert np.array_equal(scales.cpu().numpy(), rs)
    rows, pad = vt_to_rows(vt, N)
    assert np.array_equal(rows, rc)
    assert not pad.any()


def quantized(t):
    """GPU side: quantize q, k, v with the library; oracle side: with the oracle."""
    q8, qs = api.fa_fp8_quantize(t["q"].to(DEV), api.FA_FP8_Q_BLOCK)
    k8, ks = api.fa_fp8_quantize(t["k"].to(DEV), api.FA_FP8_K_BLOCK)
    vt, vs = api.fa_fp8_quantize_v(t["v"].to(DEV))
    rq = F8.quantize_rows(bits(t["q"]), 128)
    rk = F8.quantize_rows(bits(t["k"]), 64)
    rv = F8.quantize_heads(bits(t["v"]))
    return (q8, qs, k8, ks, vt, vs), (rq, rk, rv)


def check_fp8(out, lse, O, L, A, what):
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o)), what
    bound = 2.0 ** -4 * A + 2.0 ** -9 * np.abs(O)
    e = np.abs(o - O)
    worst = (e - 1.05 * bound).max()
    fin = np.isfinite(L)
    assert np.array_equal(np.isfinite(l), fin), f"{what}: LSE finiteness"
    el = np.abs(l[fin] - L[fin]).max() if fin.any() else 0.0
    msg = (f"{what}: O max err {e.max():.3e} (bound there {bound.flat[e.argmax()]:.3e}), mean err {e.mean():.3e} "
           f"(mean bound {bound.mean():.3e}), LSE max {el:.3e}")
    print(msg)
    assert worst <= 1e-5, msg
    assert e.mean() <= 0.5 * bound.mean() + 1e-6, msg
    assert el <= 1e-3, msg


CASES = [
    # B, Nq, Nk, Hq, Hkv, causal, window
    (2, 200, 200, 4, 4, True, None),
    (1, 333, 333, 4, 2, False, None),
    (2, 130, 190, 4, 1, True, None),
    (1, 190, 120, 2, 2, True, None),      # the first 70 rows see no key
    (1, 300, 300, 2, 2, True, (70, 0)),
    (1, 257, 257, 2, 2, False, (40, 20)),
    (1, 1, 1, 1, 1, False, None),
    (1, 64, 64, 1, 1, True, None),
]


@pytest.mark.parametrize("B,Nq,Nk,Hq,Hkv,causal,window", CASES)
def test_fp8_fwd_parity(B, Nq, Nk, Hq, Hkv, causal, window):
    t = W.dense(81 + Nq + Nk, B, Nq, Hq, Hkv, 128, Nk=Nk)
    gpu, ref = quantized(t)
    out, lse = api.fa_fwd_fp8(*gpu, causal=causal, window=window)
    torch.cuda.synchronize()
    (rq, qs), (rk, ks), (rv, vs) = ref
    O, L, A = F8.fwd(rq, qs, 128, rk, ks, 64, rv, vs, causal=causal, window=window, with_abs=True)
    check_fp8(out, lse, O, L, A, f"fp8 {B}x{Nq}x{Nk} h{Hq}/{Hkv} causal={causal} window={window}")
    if causal and Nq > Nk:
        assert torch.count_nonzero(out[:, : Nq - Nk].float()) == 0
        assert torch.all(lse[:, :, : Nq - Nk] == float("-inf"))


def test_fp8_fwd_custom_scale_and_determinism():
    t = W.dense(91, 1, 256, 2, 2, 128)
    gpu, ref = quantized(t)
    a = api.fa_fwd_fp8(*gpu, causal=True, softmax_scale=0.2)
    b = api.fa_fwd_fp8(*gpu, causal=True, softmax_scale=0.2)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    (rq, qs), (rk, ks), (rv, vs) = ref
    O, L, A = F8.fwd(rq, qs, 128, rk, ks, 64, rv, vs, causal=True, scale=0.2, with_abs=True)
    check_fp8(a[0], a[1], O, L, A, "fp8 scale 0.2")


def test_fp8_fwd_full_size_sampled_rows():
    """The benchmark's launch: batch 4 x 16 heads x 4096, causal; sampled rows of every head."""
    B, N, H, d = 4, 4096, 16, 128
    t = W.dense(5, B, N, H, H, d, device=DEV)
    q8, qs = api.fa_fp8_quantize(t["q"], 128)
    k8, ks = api.fa_fp8_quantize(t["k"], 64)
    vt, vs = api.fa_fp8_quantize_v(t["v"])
    out, lse = api.fa_fwd_fp8(q8, qs, k8, ks, vt, vs, causal=True)
    torch.cuda.synchronize()
    cpu = {n: t[n].cpu() for n in "qkv"}
    rq = F8.quantize_rows(bits(cpu["q"]), 128)
    rk = F8.quantize_rows(bits(cpu["k"]), 64)
    rv = F8.quantize_heads(bits(cpu["v"]))
    assert np.array_equal(qs.cpu().numpy(), rq[1]) and np.array_equal(ks.cpu().numpy(), rk[1])
    rows = [0, 1, 63, 64, 127, 128, 1000, 2047, 2048, 4094, 4095]
    O, L, A = F8.fwd(rq[0], rq[1], 128, rk[0], rk[1], 64, rv[0], rv[1], causal=True, rows=rows, with_abs=True)
    check_fp8(out[:, rows], lse[:, :, rows], O, L, A, "fp8 4x16x4096 causal, sampled rows")


# ---------------------------------------------------------------- incoherent processing
def _signs(d, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randint(0, 2, (d,), generator=g) * 2 - 1).to(torch.float32)


@pytest.mark.parametrize("d,block,N,strided", [(128, 128, 300, False), (128, 64, 200, True), (64, 64, 77, False),
                                                 (128, 128, 1, False)])
def test_quantize_rows_rotated_bit_exact(d, block, N, strided):
    x = W.randn_bf16(W.generator(161 + N), (2, N, 3, d), 2.0)
    s = _signs(d, N)
    xd = x.to(DEV)
    if strided:
        wide = torch.zeros(2, N, 6, d, dtype=torch.bfloat16, device=DEV)
        wide[:, :, ::2] = xd
        xd = wide[:, :, ::2]
    codes, scales = api.fa_fp8_quantize_rotated(xd, block, s.to(DEV))
    torch.cuda.synchronize()
    rc, rs = F8.quantize_rows_rotated(bits(x), block, s.numpy())
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


@pytest.mark.parametrize("B,Nq,Nk,Hq,Hkv,causal", [(2, 200, 200, 4, 2, True), (1, 190, 300, 2, 2, False)])
def test_fp8_fwd_rotated_parity(B, Nq, Nk, Hq, Hkv, causal):
    """Q and K rotated by the same signs, V plain: the attention over those codes against the
    oracle over the oracle's rotated codes."""
    t = W.dense(171 + Nq, B, Nq, Hq, Hkv, 128, Nk=Nk)
    s = _signs(128, 7)
    q8, qs = api.fa_fp8_quantize_rotated(t["q"].to(DEV), 128, s.to(DEV))
    k8, ks = api.fa_fp8_quantize_rotated(t["k"].to(DEV), 64, s.to(DEV))
    vt, vs = api.fa_fp8_quantize_v(t["v"].to(DEV))
    out, lse = api.fa_fwd_fp8(q8, qs, k8, ks, vt, vs, causal=causal)
    torch.cuda.synchronize()
    rq = F8.quantize_rows_rotated(bits(t["q"]), 128, s.numpy())
    rk = F8.quantize_rows_rotated(bits(t["k"]), 64, s.numpy())
    rv = F8.quantize_heads(bits(t["v"]))
    O, L, A = F8.fwd(rq[0], rq[1], 128, rk[0], rk[1], 64, rv[0], rv[1], causal=causal, with_abs=True)
    check_fp8(out, lse, O, L, A, f"fp8 rotated {B}x{Nq}x{Nk} causal={causal}")


def test_fp8_rotation_reduces_the_error_of_outlier_channels():
    """Q and K with a few outlier channels (x 30): the FP8 attention with the rotation is closer
    to the exact bf16 attention (fp64 oracle) than without it."""
    import oracle
    B, N, H, d = 1, 256, 2, 128
    t = W.dense(181, B, N, H, H, d)
    for n in "qk":
        x = t[n].float()
        x[..., [3, 40, 77]] *= 30.0
        t[n] = x.to(torch.bfloat16)
    exact_o, exact_l = oracle.fwd_dense(bits(t["q"]), bits(t["k"]), bits(t["v"]), causal=True)
    vt, vs = api.fa_fp8_quantize_v(t["v"].to(DEV))
    errs = {}
    for rot in (False, True):
        s = _signs(d, 3).to(DEV)
        qz = api.fa_fp8_quantize_rotated(t["q"].to(DEV), 128, s) if rot else api.fa_fp8_quantize(t["q"].to(DEV), 128)
        kz = api.fa_fp8_quantize_rotated(t["k"].to(DEV), 64, s) if rot else api.fa_fp8_quantize(t["k"].to(DEV), 64)
        out, lse = api.fa_fwd_fp8(*qz, *kz, vt, vs, causal=True)
        torch.cuda.synchronize()
        errs[rot] = (np.abs(out.float().cpu().numpy() - exact_o).mean(),
                     np.abs(lse.cpu().numpy() - exact_l).mean())
    print("fp8 outlier channels, mean |error| (O, LSE): plain", errs[False], "rotated", errs[True])
    assert errs[True][0] < 0.7 * errs[False][0] and errs[True][1] < 0.7 * errs[False][1]
