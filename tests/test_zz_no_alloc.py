"""The no-allocation paged entry point (fa_fwd_kvcache_paged_noalloc) against the
workspace entry point (fa_fwd_kvcache_paged) it mirrors: the same kernels on the same
inputs, so results must agree bitwise, on two calls in a row (the second smaller, so it
runs on what the first left in the shared scratch), and both within the fp64 oracle's
tolerance.  Also the size limit, checked on the host before anything is launched."""
import ctypes

import pytest
import torch

import oracle
from exact_attention_72_amd import api, workloads as W
from gpu_util import DEV, bits, check_close


def _poison(t):
    kc, vc = t["k_cache"].clone(), t["v_cache"].clone()
    page = kc.shape[1]
    live = torch.zeros(kc.shape[0], page, dtype=torch.bool)
    for b, L in enumerate(t["cache_seqlens"].tolist()):
        for tok in range(0, L, page):
            live[int(t["block_table"][b, tok // page]), : min(page, L - tok)] = True
    kc[~live] = float("nan")
    vc[~live] = float("nan")
    return kc, vc


def _case(seed, lens, Hq, Hkv, d, page, Nq=1):
    t = W.paged(seed, len(lens), Hq, Hkv, d, page, 0, 0, cache_seqlens=lens, Nq=Nq)
    kc, vc = _poison(t)
    dev = {n: t[n].to(DEV) for n in ("q", "block_table", "cache_seqlens")}
    dev["k_cache"], dev["v_cache"] = kc.to(DEV), vc.to(DEV)
    return t, dev


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point_twice():
    cases = [
        # first call: 24 sequences up to 9000 keys, 32/8 heads, 256-token pages, 8 splits
        (_case(301, [int(x) for x in torch.randint(1, 9001, (24,), generator=torch.Generator().manual_seed(3))],
               32, 8, 128, 256), 8),
        # second call, smaller: 5 sequences, 8/2 heads, d = 64, 16-token pages, 3 splits, 2 new tokens
        (_case(302, [1, 17, 300, 64, 999], 8, 2, 64, 16, Nq=2), 3),
    ]
    for (t, dv), S in cases:
        print(f"noalloc case B={len(t['cache_seqlens'])} S={S}", flush=True)
        out_ws, lse_ws = api.fa_fwd_kvcache_paged(dv["q"], dv["k_cache"], dv["v_cache"], dv["block_table"],
                                                  dv["cache_seqlens"], num_splits=S, causal=True)
        out_na = torch.empty_like(dv["q"])
        lse_na = torch.empty_like(lse_ws)
        api.fa_fwd_kvcache_paged_noalloc(dv["q"], dv["k_cache"], dv["v_cache"], dv["block_table"],
                                         dv["cache_seqlens"], num_splits=S, causal=True, out=out_na, lse=lse_na)
        torch.cuda.synchronize()
        assert torch.equal(out_na.view(torch.int16), out_ws.view(torch.int16))
        assert torch.equal(lse_na.view(torch.int32), lse_ws.view(torch.int32))
        o_ref, l_ref = oracle.fwd_paged(bits(t["q"]), bits(t["k_cache"]), bits(t["v_cache"]),
                                        t["block_table"].numpy(), t["cache_seqlens"].numpy(), causal=True)
        check_close(out_na, lse_na, o_ref, l_ref, f"noalloc S={S}")


def test_noalloc_rejects_partials_beyond_the_scratch():
    """64 sequences x 32 heads x d 128 at 64 splits need 64 * 2048 * 129 * 4 B > 32 MiB: an
    error before any device work (fake, never dereferenced pointers)."""
    L = api.lib()
    FAKE = ctypes.c_void_p(0x1000)
    o = api.fa_attn_opts(0.0, 1, -1, -1, 0.0, -1, None, 0)
    s3 = (ctypes.c_int64 * 3)
    qs, ks = s3(32 * 128, 32 * 128, 128), s3(256 * 8 * 128, 8 * 128, 128)
    need = L.fa_kvcache_workspace_size(64, 1, 32, 128, 64)
    assert need > api.FA_NOALLOC_SCRATCH_BYTES
    rc = L.fa_fwd_kvcache_paged_noalloc(ctypes.byref(o), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 64, 1, 32, 8,
                                        128, 8192, 256, 128, 64, qs, ks, ks, qs, None)
    assert rc == api.FA_ERR_INVALID_ARG
    assert "scratch" in api.fa_last_error()
