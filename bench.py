"""Benchmark of the attention forward on one MI355X.

A step is one forward pass of the dense causal prefill workload
(batch 4, 16 heads, N = 4096, d = 128, bf16) through the C ABI.  The line also
carries, as secondary figures, the paged split-KV decode measurement (64
sequences, 32/8 heads, d = 128, 256-token pages, num_splits in {1, 4, 16}) and
the same decode over an FP8 (e4m3) cache, the varlen GQA prefill (32 sequences of 64..8192 tokens, 32/4 heads, packed),
the long-context local attention with softcap (N = 32768, 32 heads,
window 4096, softcap 30), and the chunked prefill over a paged cache (4 x 4096
new tokens against 16384 cached keys, 32/8 heads) with the in-place K/V append
of that chunk, a unified batch of 64 decode requests and 4 prefill chunks
in one launch, the backward pass of the prefill workload, the FP8 (e4m3) forward of the
prefill workload, the prefill workload with ALiBi, and the prefill workload through the
two score_mod / mask_mod hooks (relative-position bias, prefix-LM).

Prints one JSON line:
  value        prefill TFLOP/s, FLOPs counted as 4 * B * H * N^2 * d * 1/2 (the
               pages' causal convention, "Attention kernels: FlashAttention and
               PagedAttention", section 8.3)
  roofline     achieved bf16 MFMA rate of the prefill kernel (FLOPs per launch /
               mean launch time from HIP events recorded on the launch stream around the
               timed back-to-back launches) against
               the 2.5 PFLOP/s dense bf16 peak; traffic from the committed
               rocprofv3 counter summary when it matches the current kernel source
  cpu_baseline the fp64 oracle timed on host threads on a bounded row sample of
               the same workload
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
KERNEL_SRC = os.path.join(ROOT, "exact_attention_72_amd", "csrc", "fa_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for f in ("fa_kernels.hip", "fa_blockinfo.h", "fa_internal.h"):
        with open(os.path.join(ROOT, "exact_attention_72_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel: str):
    """HBM bytes per launch from the committed counter summary, if it was taken on
    the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    e = d.get(kernel)
    if not e or e.get("source_sha") != kernel_source_sha():
        return None
    return e.get("bytes_per_launch")


def settle(fn, min_s=1.0, max_s=6.0, window=20, tol=0.01):
    """Launch fn back to back until the GPU clock has settled under this load: at least
    min_s seconds have passed and two successive windows of `window` launches agree in mean
    time within tol (at most max_s seconds).  The kernels' clock ramps up over the first
    hundreds of milliseconds of sustained matrix work, so a few untimed launches alone leave
    the timed ones on a cold clock.  Returns the seconds spent."""
    import torch
    t0 = time.perf_counter()
    prev = None
    while True:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(window):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / window
        el = time.perf_counter() - t0
        if el >= max_s or (el >= min_s and prev is not None and abs(ms - prev) <= tol * prev):
            return el
        prev = ms


def time_launches(fn, steps, warmup, settle_s=0.5):
    """Settle the clock (settle(), at least settle_s seconds), run `warmup` untimed calls, then
    time `steps` back-to-back calls between two HIP events recorded on the current stream
    (the stream the library launches on).  Returns the wall time of the timed region (s), the
    mean time per call from the events (ms) and the settle time (s)."""
    import torch
    st = settle(fn, min_s=settle_s) if settle_s > 0 else 0.0
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, e0.elapsed_time(e1) / steps, st


def prefill_flops(B, H, N, d, causal):
    return 4.0 * B * H * N * N * d * (0.5 if causal else 1.0)


def cpu_baseline(W, t, c, target_s=15.0):
    """The fp64 oracle on a row sample of the same workload; TFLOP/s on the same
    FLOP convention (each sampled row counted with its visible keys)."""
    import numpy as np
    import oracle
    host_cores = os.cpu_count() or 1
    try:
        share = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        share = host_cores
    # every core this process may run on, up to the per-GPU CPU share the box grants (16)
    threads = max(1, min(share, int(os.environ.get("OMP_NUM_THREADS", "16") or 16), 16))
    B, N, H, d = c["B"], c["N"], c["Hq"], c["d"]
    qb, kb, vb = (W.to_bits(t[n]) for n in "qkv")
    rng = np.random.default_rng(0)

    def run(n):
        rows = np.sort(rng.integers(0, B * H * N, n))
        i = rows % N
        keys = float(np.sum(i + 1)) if c["causal"] else float(n) * N
        t0 = time.perf_counter()
        used = oracle.fwd_dense(qb, kb, vb, causal=c["causal"], window=c["window"],
                                softcap=c["softcap"], rows=rows, nthreads=threads)
        dt = time.perf_counter() - t0
        return dt, keys * 4 * d, n
    # the first runs are dominated by fixed costs, so extrapolate twice towards target_s
    dt, fl, n = run(threads * 8)
    for _ in range(2):
        if dt >= 0.66 * target_s:
            break
        n = int(max(threads * 8, min(4000000, n * target_s / max(dt, 1e-3))))
        dt, fl, n = run(n)
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "host_cores": host_cores,
            "affinity_cores": share, "kind": "oracle",
            "sample": f"{n} random query rows of the batch-4 x 16-head N=4096 d=128 causal "
                      f"workload, fp64, {dt:.1f} s"}


def bench_varlen(api, W, steps, warmup):
    """Varlen GQA prefill: 32 sequences, lengths uniform [64, 8192], 32 Q / 4 KV heads packed,
    causal.  FLOPs: 4 d Hq sum_b L_b (L_b + 1) / 2 (visible pairs only)."""
    import torch
    name = "varlen_gqa_32seq_64to8192_h32kv4_d128_causal"
    c = W.WORKLOADS[name]
    t = W.varlen(c["seed"], c["nseq"], c["lo"], c["hi"], c["Hq"], c["Hkv"], c["d"], device="cuda")
    cu = t["cu_seqlens"].cuda()
    L = t["lengths"].to(torch.float64)
    flops = float(4 * c["d"] * c["Hq"] * (L * (L + 1) / 2).sum())
    out = torch.empty_like(t["q"])
    lse = torch.empty((c["Hq"], t["q"].shape[0]), dtype=torch.float32, device="cuda")
    fn = lambda: api.fa_fwd_varlen(t["q"], t["k"], t["v"], cu, cu, t["max_seqlen"], causal=True,  # noqa
                                   pack_gqa=1, out=out, lse=lse)
    wall, ms, _ = time_launches(fn, steps, warmup)
    tf = flops / (ms * 1e-3) / 1e12
    return {"metric": "varlen prefill TFLOP/s", "unit": "TFLOP/s", "value": round(tf, 2),
            "kernel_ms": round(ms, 4), "flops": flops,
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4)},
            "config": {"workload": name, "sequences": c["nseq"], "total_tokens": int(t["q"].shape[0]),
                       "heads_q": c["Hq"], "heads_kv": c["Hkv"], "head_dim": c["d"], "pack_gqa": True,
                       "causal": True, "flop_convention": "4*d*Hq*sum L(L+1)/2"}}


def bench_local(api, W, steps, warmup):
    """Long-context local attention with softcap: N = 32768, 32 heads, window (4096, 0),
    softcap 30, inputs N(0,1) x 2.  FLOPs: 4 d H sum_i (min(i, 4096) + 1)."""
    import torch
    name = "local_softcap_n32768_h32_d128_w4096_cap30"
    c = W.WORKLOADS[name]
    B, N, H, d = c["B"], c["N"], c["Hq"], c["d"]
    t = W.dense(c["seed"], B, N, H, c["Hkv"], d, mult=c["mult"], device="cuda")
    wl = c["window"][0]
    pairs = sum(min(i, wl) + 1 for i in range(N))
    flops = 4.0 * d * B * H * pairs
    out = torch.empty_like(t["q"])
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fn = lambda: api.fa_fwd(t["q"], t["k"], t["v"], causal=True, window=c["window"],  # noqa
                            softcap=c["softcap"], out=out, lse=lse)
    wall, ms, _ = time_launches(fn, steps, warmup)
    tf = flops / (ms * 1e-3) / 1e12
    return {"metric": "local softcap prefill TFLOP/s", "unit": "TFLOP/s", "value": round(tf, 2),
            "kernel_ms": round(ms, 4), "flops": flops,
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4)},
            "config": {"workload": name, "batch": B, "heads": H, "seq_len": N, "head_dim": d,
                       "causal": True, "window": list(c["window"]), "softcap": c["softcap"],
                       "flop_convention": "4*d*H*sum_i(min(i,4096)+1)"}}


def paged_prefill_inputs(W, device="cuda"):
    c = W.WORKLOADS["paged_prefill_b4_h32kv8_d128_chunk4096_prefix12288_page256"]
    Lk = c["prefix"] + c["Nq"]
    t = W.paged(c["seed"], c["B"], c["Hq"], c["Hkv"], c["d"], c["page"], 0, 0,
                max_blocks=c["max_blocks"], Nq=c["Nq"], cache_seqlens=[Lk] * c["B"], device=device)
    return c, t


def bench_paged_prefill(api, W, steps, warmup):
    """Chunked prefill over a paged cache: 4 sequences, a 4096-token chunk against 16384 cached
    keys (12288-token prefix + the chunk), 32 Q / 8 KV heads packed, 256-token pages.  FLOPs:
    4 d Hq B sum_i (prefix + i + 1) (visible pairs only).  Also times the in-place append of the
    chunk's K/V into the cache (bytes read + written per call)."""
    import torch
    c, t = paged_prefill_inputs(W)
    name = "paged_prefill_b4_h32kv8_d128_chunk4096_prefix12288_page256"
    B, Nq, P = c["B"], c["Nq"], c["prefix"]
    flops = 4.0 * c["d"] * c["Hq"] * B * (Nq * P + Nq * (Nq + 1) / 2)
    bt, sl = t["block_table"].cuda(), t["cache_seqlens"].cuda()
    out = torch.empty_like(t["q"])
    lse = torch.empty((B, c["Hq"], Nq), dtype=torch.float32, device="cuda")
    fn = lambda: api.fa_fwd_kvcache_paged(t["q"], t["k_cache"], t["v_cache"], bt, sl, num_splits=0,  # noqa
                                          causal=True, out=out, lse=lse)
    wall, ms, _ = time_launches(fn, steps, warmup)
    tf = flops / (ms * 1e-3) / 1e12
    # append: the chunk's K/V (new tensors of the chunk's shape) at positions prefix .. prefix + Nq - 1
    g = W.generator(c["seed"] + 7, "cuda")
    kn = W.randn_bf16(g, (B, Nq, c["Hkv"], c["d"]), 1.0, "cuda")
    vn = W.randn_bf16(g, (B, Nq, c["Hkv"], c["d"]), 1.0, "cuda")
    start = torch.full((B,), P, dtype=torch.int32, device="cuda")
    fa = lambda: api.fa_kvcache_append(kn, vn, t["k_cache"], t["v_cache"], bt, start)  # noqa
    _, ms_a, _ = time_launches(fa, steps, min(warmup, 50))
    moved = 2.0 * 2 * kn.numel() * 2          # K and V, read once and written once, bf16
    gbs = moved / (ms_a * 1e-3) / 1e9
    # the same append with the keys rotated on the way (full head_dim, 10000^(-2i/d) frequencies)
    r = c["d"]
    theta = 10000.0 ** (-2.0 * torch.arange(r // 2, dtype=torch.float64, device="cuda") / r)
    ang = torch.arange(P + Nq, dtype=torch.float64, device="cuda")[:, None] * theta[None, :]
    cos, sin = torch.cos(ang).float(), torch.sin(ang).float()
    fr = lambda: api.fa_kvcache_append(kn, vn, t["k_cache"], t["v_cache"], bt, start,  # noqa
                                       rotary_cos=cos, rotary_sin=sin)
    _, ms_r, _ = time_launches(fr, steps, min(warmup, 50))
    return {"metric": "chunked prefill over a paged cache TFLOP/s", "unit": "TFLOP/s", "value": round(tf, 2),
            "kernel_ms": round(ms, 4), "flops": flops,
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4)},
            "config": {"workload": name, "batch": B, "chunk": Nq, "prefix": P, "heads_q": c["Hq"],
                       "heads_kv": c["Hkv"], "head_dim": c["d"], "page_size": c["page"],
                       "num_splits": 0, "flop_convention": "4*d*Hq*B*sum_i(prefix+i+1)"},
            "append": {"metric": "K/V append GB/s (read + write)", "unit": "GB/s", "value": round(gbs, 1),
                       "kernel_ms": round(ms_a, 4), "bytes": moved,
                       "rotary_kernel_ms": round(ms_r, 4),
                       "rotary_GBps": round(moved / (ms_r * 1e-3) / 1e9, 1),
                       "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                    "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)},
                       "config": {"tokens": B * Nq, "heads_kv": c["Hkv"], "head_dim": c["d"],
                                  "page_size": c["page"]}}}


def bench_unified(api, W, steps, warmup):
    """One launch over a mixed batch (fa_fwd_varlen_paged): 64 decode requests with one new
    token and 4 prefill chunks of 2048 tokens, 32/8 heads, 256-token pages.  FLOPs on visible
    pairs, 4 d Hq sum over queries of the keys each sees."""
    import torch
    name = "unified_decode64_chunk4x2048_h32kv8_d128_page256"
    c = W.WORKLOADS[name]
    t = W.varlen_paged(c["seed"], c["n_decode"], c["dec_lo"], c["dec_hi"], c["n_chunk"], c["chunk"],
                       c["pre_lo"], c["pre_hi"], c["Hq"], c["Hkv"], c["d"], c["page"], device="cuda")
    pairs = 0
    for Lq, Lk in zip(t["qlens"], t["cache_seqlens"].tolist()):
        pairs += sum(min(Lk, i + Lk - Lq + 1) for i in range(Lq))
    flops = 4.0 * c["d"] * c["Hq"] * pairs
    cu, bt, sl = t["cu_seqlens_q"].cuda(), t["block_table"].cuda(), t["cache_seqlens"].cuda()
    out = torch.empty_like(t["q"])
    lse = torch.empty((c["Hq"], t["q"].shape[0]), dtype=torch.float32, device="cuda")
    S = int(api.lib().fa_varlen_paged_num_splits(len(t["qlens"]), c["Hq"], c["Hkv"], t["block_table"].shape[1]))
    ws = torch.empty(max(1, int(api.lib().fa_varlen_paged_workspace_size(len(t["qlens"]), c["Hkv"], c["d"], S))),
                     dtype=torch.uint8, device="cuda")
    fn = lambda: api.fa_fwd_varlen_paged(t["q"], t["k_cache"], t["v_cache"], cu, c["chunk"], bt, sl,  # noqa
                                         causal=True, num_splits=S, out=out, lse=lse, workspace=ws)
    wall, ms, _ = time_launches(fn, steps, warmup)
    tf = flops / (ms * 1e-3) / 1e12
    return {"metric": "unified prefill+decode batch TFLOP/s", "unit": "TFLOP/s", "value": round(tf, 2),
            "kernel_ms": round(ms, 4), "flops": flops,
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4)},
            "config": {"workload": name, "decode_requests": c["n_decode"], "chunks": c["n_chunk"],
                       "chunk": c["chunk"], "heads_q": c["Hq"], "heads_kv": c["Hkv"], "head_dim": c["d"],
                       "page_size": c["page"], "decode_num_splits": S,
                       "flop_convention": "4*d*Hq*sum visible pairs"}}


def bench_bwd(api, W, steps, warmup):
    """Backward of the dense causal prefill workload (batch 4, 16 heads, N = 4096, d = 128):
    fa_bwd per call (D preprocess, dQ kernel, dK/dV kernel).  FLOPs: 2.5 x the forward's
    4 B H N^2 d / 2 (five products against the forward's two, "Attention kernels...",
    section 4.3); the recomputation the kernels add is not counted."""
    import torch
    c = W.WORKLOADS["prefill_b4_h16_n4096_d128_causal"]
    B, N, H, d = c["B"], c["N"], c["Hq"], c["d"]
    t = W.dense(c["seed"], B, N, H, c["Hkv"], d, device="cuda")
    do = W.randn_bf16(W.generator(c["seed"] + 100, "cuda"), (B, N, H, d), 1.0, "cuda")
    out, lse = api.fa_fwd(t["q"], t["k"], t["v"], causal=True)
    dq, dk, dv = (torch.empty_like(t[n]) for n in "qkv")
    ws = torch.empty(api.lib().fa_bwd_workspace_size(B, N, H), dtype=torch.uint8, device="cuda")
    fn = lambda: api.fa_bwd(t["q"], t["k"], t["v"], out, lse, do, causal=True, dq=dq, dk=dk, dv=dv,  # noqa
                            workspace=ws)
    wall, ms, _ = time_launches(fn, steps, warmup)
    flops = 2.5 * prefill_flops(B, H, N, d, True)
    tf = flops / (ms * 1e-3) / 1e12
    return {"metric": "attn bwd TFLOP/s (bf16 N=4k d=128 causal)", "unit": "TFLOP/s", "value": round(tf, 2),
            "ms": round(ms, 4), "flops": flops,
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4)},
            "config": {"workload": "prefill_b4_h16_n4096_d128_causal backward", "batch": B, "heads": H,
                       "seq_len": N, "head_dim": d, "causal": True,
                       "flop_convention": "2.5 * 4*B*H*N^2*d/2"}}


def bench_alibi(api, W, steps, warmup):
    """The dense causal prefill workload with ALiBi (slopes 2^(-8 (h + 1) / H)): fa_fwd per
    launch, TFLOP/s on the same convention (the bias is not counted)."""
    import torch
    c = W.WORKLOADS["prefill_b4_h16_n4096_d128_causal"]
    B, N, H, d = c["B"], c["N"], c["Hq"], c["d"]
    t = W.dense(c["seed"], B, N, H, c["Hkv"], d, device="cuda")
    slopes = torch.exp2(-8.0 * (torch.arange(H, dtype=torch.float32, device="cuda") + 1) / H)
    out = torch.empty_like(t["q"])
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fn = lambda: api.fa_fwd(t["q"], t["k"], t["v"], causal=True, alibi_slopes=slopes, out=out, lse=lse)  # noqa
    _, ms, _ = time_launches(fn, steps, warmup)
    tf = prefill_flops(B, H, N, d, True) / (ms * 1e-3) / 1e12
    return {"metric": "attn fwd with ALiBi TFLOP/s (bf16 N=4k d=128 causal)", "unit": "TFLOP/s",
            "value": round(tf, 2), "ms": round(ms, 4),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4)},
            "config": {"workload": "prefill_b4_h16_n4096_d128_causal alibi", "batch": B, "heads": H,
                       "seq_len": N, "head_dim": d, "causal": True, "slopes": "2^(-8(h+1)/H)"}}


def bench_mods(api, W, steps, warmup):
    """The dense causal prefill workload through the two score_mod / mask_mod hooks: a
    relative-position bias table (R = 256) with causal masking, and a prefix-LM mask with
    prefixes 0, 1024, 2048, 4096 (the four sequences).  TFLOP/s on visible pairs (the bias
    is not counted)."""
    import torch
    c = W.WORKLOADS["prefill_b4_h16_n4096_d128_causal"]
    B, N, H, d = c["B"], c["N"], c["Hq"], c["d"]
    t = W.dense(c["seed"], B, N, H, c["Hkv"], d, device="cuda")
    out = torch.empty_like(t["q"])
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    R = 256
    table = torch.randn(H, 2 * R + 1, device="cuda")
    fr = lambda: api.fa_fwd_relpos_bias(t["q"], t["k"], t["v"], table, causal=True, out=out, lse=lse)  # noqa
    _, ms_r, _ = time_launches(fr, steps, warmup)
    prefixes = [0, 1024, 2048, 4096]
    pl = torch.tensor(prefixes, dtype=torch.int32, device="cuda")
    fp = lambda: api.fa_fwd_prefix_lm(t["q"], t["k"], t["v"], pl, out=out, lse=lse)  # noqa
    _, ms_p, _ = time_launches(fp, steps, warmup)
    fl_r = prefill_flops(B, H, N, d, True)
    pairs = sum(sum(min(N, max(P, i + 1)) for i in range(N)) for P in prefixes)
    fl_p = 4.0 * d * H * pairs
    tr, tp = fl_r / (ms_r * 1e-3) / 1e12, fl_p / (ms_p * 1e-3) / 1e12
    return {"metric": "attn fwd with score_mod / mask_mod TFLOP/s", "unit": "TFLOP/s",
            "relpos_bias": {"value": round(tr, 2), "ms": round(ms_r, 4), "max_distance": R,
                            "frac": round(tr / PEAK_BF16_TFLOPS, 4)},
            "prefix_lm": {"value": round(tp, 2), "ms": round(ms_p, 4), "prefix_lens": prefixes,
                          "frac": round(tp / PEAK_BF16_TFLOPS, 4)},
            "config": {"workload": "prefill_b4_h16_n4096_d128 mods", "batch": B, "heads": H, "seq_len": N,
                       "head_dim": d, "flop_convention": "4*d*H*sum visible pairs"}}


def bench_fp8(api, W, steps, warmup):
    """FP8 (e4m3) forward of the dense causal prefill workload (batch 4, 16 heads, N = 4096,
    d = 128): fa_fwd_fp8 per launch on inputs quantized beforehand, TFLOP/s on the same
    4 B H N^2 d / 2 convention against the dense FP8 matrix peak; the quantizers (Q and K
    per block, V per head into the transposed layout) timed separately."""
    import torch
    c = W.WORKLOADS["prefill_b4_h16_n4096_d128_causal"]
    B, N, H, d = c["B"], c["N"], c["Hq"], c["d"]
    t = W.dense(c["seed"], B, N, H, c["Hkv"], d, device="cuda")
    q8, qs = api.fa_fp8_quantize(t["q"], api.FA_FP8_Q_BLOCK)
    k8, ks = api.fa_fp8_quantize(t["k"], api.FA_FP8_K_BLOCK)
    vt, vs = api.fa_fp8_quantize_v(t["v"])
    out = torch.empty((B, N, H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fn = lambda: api.fa_fwd_fp8(q8, qs, k8, ks, vt, vs, causal=True, out=out, lse=lse)  # noqa: E731
    _, ms, _ = time_launches(fn, steps, warmup)
    flops = prefill_flops(B, H, N, d, True)
    tf = flops / (ms * 1e-3) / 1e12

    def quant():
        api.fa_fp8_quantize(t["q"], api.FA_FP8_Q_BLOCK, codes=q8, scales=qs)
        api.fa_fp8_quantize(t["k"], api.FA_FP8_K_BLOCK, codes=k8, scales=ks)
        api.fa_fp8_quantize_v(t["v"], vt=vt, scales=vs)
    _, qms, _ = time_launches(quant, max(3, steps // 10), 2, settle_s=0)
    return {"metric": "attn fwd fp8 TFLOP/s (e4m3 N=4k d=128 causal)", "unit": "TFLOP/s", "value": round(tf, 2),
            "ms": round(ms, 4),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_FP8_TFLOPS, 4)},
            "quantize_ms": round(qms, 4),
            "config": {"workload": "prefill_b4_h16_n4096_d128_causal fp8", "batch": B, "heads": H, "seq_len": N,
                       "head_dim": d, "causal": True, "flop_convention": "4*B*H*N^2*d/2",
                       "scales": "Q per 128 rows, K per 64 keys, V per head"}}


def bench_decode(api, W, steps, warmup):
    import torch
    c = W.WORKLOADS["paged_decode_b64_h32kv8_d128_page256"]
    t = W.paged(c["seed"], c["B"], c["Hq"], c["Hkv"], c["d"], c["page"], c["lo"], c["hi"],
                max_blocks=c["max_blocks"], device="cuda")
    bt, sl = t["block_table"].cuda(), t["cache_seqlens"].cuda()
    kv_bytes = 4096.0 * float(t["cache_seqlens"].sum())   # K and V of live tokens, bf16
    out = torch.empty_like(t["q"])
    lse = torch.empty((c["B"], c["Hq"], 1), dtype=torch.float32, device="cuda")
    res = {}
    auto = api.fa_kvcache_num_splits(c["B"], 1, c["Hq"], c["Hkv"], c["page"], c["max_blocks"])
    # the configured split counts, then the library's own choice (num_splits = 0)
    for S in (1, 4, 16, 0):
        need = api.fa_kvcache_workspace_size(c["B"], 1, c["Hq"], c["d"], S or auto)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        fn = lambda: api.fa_fwd_kvcache_paged(t["q"], t["k_cache"], t["v_cache"], bt, sl,  # noqa
                                              num_splits=S, causal=True, out=out, lse=lse,
                                              workspace=ws)
        wall, ms, _ = time_launches(fn, steps, warmup)
        res[S] = {"ms": ms, "kv_GBps": kv_bytes / (ms * 1e-3) / 1e9}
    # the best of the configured counts and the library's own choice (what a caller
    # gets with num_splits = 0)
    best = max((1, 4, 16, 0), key=lambda s: res[s]["kv_GBps"])
    return {"metric": "paged decode KV GB/s", "unit": "GB/s",
            "value": res[best]["kv_GBps"], "ms": round(res[best]["ms"], 4), "num_splits": best or auto,
            "num_splits_auto": auto,
            "kv_bytes": kv_bytes,
            "per_split": {(str(s) if s else "auto"): {"ms": round(r["ms"], 4), "kv_GBps": round(r["kv_GBps"], 1)}
                          for s, r in res.items()},
            "roofline": {"bound": "hbm", "achieved": res[best]["kv_GBps"], "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": res[best]["kv_GBps"] / PEAK_HBM_GBS,
                         "traffic": stored_traffic("fa_paged_kernel")},
            "config": {"workload": "paged_decode_b64_h32kv8_d128_page256", "batch": c["B"],
                       "heads_q": c["Hq"], "heads_kv": c["Hkv"], "head_dim": c["d"],
                       "page_size": c["page"], "cache_seqlens": "uniform [1024, 32768]"}}


def bench_decode_fp8(api, W, steps, warmup, bf16_ms=None):
    """The decode workload over an FP8 (e4m3) cache (fa_fwd_kvcache_paged_fp8): the same
    sequences, heads and pages, one byte per cached element."""
    import torch
    c = W.WORKLOADS["paged_decode_b64_h32kv8_d128_page256"]
    t = W.paged_fp8(c["seed"], c["B"], c["Hq"], c["Hkv"], c["d"], c["page"], c["lo"], c["hi"],
                    max_blocks=c["max_blocks"], device="cuda")
    del t["k_cache"], t["v_cache"]
    torch.cuda.empty_cache()
    bt, sl = t["block_table"].cuda(), t["cache_seqlens"].cuda()
    kv_bytes = 2048.0 * float(t["cache_seqlens"].sum())   # K and V of live tokens, one byte each
    out = torch.empty_like(t["q"])
    lse = torch.empty((c["B"], c["Hq"], 1), dtype=torch.float32, device="cuda")
    res = {}
    auto = api.fa_kvcache_num_splits(c["B"], 1, c["Hq"], c["Hkv"], c["page"], c["max_blocks"])
    for S in (1, 4, 16, 0):
        need = api.fa_kvcache_workspace_size(c["B"], 1, c["Hq"], c["d"], S or auto)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        fn = lambda: api.fa_fwd_kvcache_paged_fp8(t["q"], t["k_codes"], t["v_codes"], t["k_scale"],  # noqa
                                                  t["v_scale"], bt, sl, num_splits=S, out=out, lse=lse,
                                                  workspace=ws)
        wall, ms, _ = time_launches(fn, steps, warmup)
        res[S] = {"ms": ms, "kv_GBps": kv_bytes / (ms * 1e-3) / 1e9}
    best = max((1, 4, 16, 0), key=lambda s: res[s]["kv_GBps"])
    r = {"metric": "paged decode over an FP8 KV cache, KV GB/s", "unit": "GB/s",
         "value": res[best]["kv_GBps"], "ms": round(res[best]["ms"], 4), "num_splits": best or auto,
         "kv_bytes": kv_bytes,
         "per_split": {(str(s) if s else "auto"): {"ms": round(q["ms"], 4), "kv_GBps": round(q["kv_GBps"], 1)}
                       for s, q in res.items()},
         "roofline": {"bound": "hbm", "achieved": res[best]["kv_GBps"], "peak": PEAK_HBM_GBS,
                      "unit": "GB/s", "frac": res[best]["kv_GBps"] / PEAK_HBM_GBS,
                      "traffic": stored_traffic("fa_paged_kernel_fp8")},
         "config": {"workload": "paged_decode_b64_h32kv8_d128_page256 (e4m3 cache)", "batch": c["B"],
                    "heads_q": c["Hq"], "heads_kv": c["Hkv"], "head_dim": c["d"],
                    "page_size": c["page"], "cache_seqlens": "uniform [1024, 32768]"}}
    if bf16_ms:
        r["speedup_vs_bf16_cache"] = round(bf16_ms / res[best]["ms"], 3)
    return r


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle", type=float, default=1.0,
                    help="seconds (at least) of untimed launches before the warm-up, until the clock "
                         "has settled (two successive 20-launch windows within 1 %%)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-decode-fp8", action="store_true")
    ap.add_argument("--no-varlen", action="store_true")
    ap.add_argument("--no-local", action="store_true")
    ap.add_argument("--no-paged-prefill", action="store_true")
    ap.add_argument("--no-unified", action="store_true")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--no-alibi", action="store_true")
    ap.add_argument("--no-mods", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 1 GiB device-to-device copy (reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the attention forward here has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from exact_attention_72_amd import api, workloads as W

    if args.calibrate_copy:
        src = torch.empty(1 << 29, dtype=torch.bfloat16, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()

    name = "prefill_b4_h16_n4096_d128_causal"
    c = W.WORKLOADS[name]
    B, N, H, d = c["B"], c["N"], c["Hq"], c["d"]
    t = W.dense(c["seed"], B, N, H, c["Hkv"], d, device="cuda")
    out = torch.empty_like(t["q"])
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fn = lambda: api.fa_fwd(t["q"], t["k"], t["v"], causal=True, out=out, lse=lse)  # noqa
    torch.cuda.synchronize()
    wall, kern_ms, settle_s = time_launches(fn, args.steps, args.warmup, settle_s=args.settle)
    flops = prefill_flops(B, H, N, d, True)
    ms_step = wall / args.steps * 1e3
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (kern_ms * 1e-3) / 1e12
    line = {
        "metric": "attn fwd TFLOPS (bf16 N=4k d=128 causal) + paged decode KV GB/s, 1 GPU",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle_s": round(settle_s, 3), "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": name, "batch": B, "heads": H, "seq_len": N, "head_dim": d,
                   "causal": True, "flop_convention": "4*B*H*N^2*d/2"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": stored_traffic("fa_prefill_kernel"),
                     "kernel_ms": round(kern_ms, 4)},
    }
    del t, out, lse
    torch.cuda.empty_cache()
    if not args.no_decode:
        line["decode"] = bench_decode(api, W, args.steps, args.warmup)
        torch.cuda.empty_cache()
    if not args.no_decode_fp8:
        line["decode_fp8"] = bench_decode_fp8(api, W, args.steps, args.warmup,
                                              line.get("decode", {}).get("ms"))
        torch.cuda.empty_cache()
    if not args.no_varlen:
        line["varlen"] = bench_varlen(api, W, args.steps, args.warmup)
        torch.cuda.empty_cache()
    if not args.no_local:
        line["local_softcap"] = bench_local(api, W, max(5, args.steps // 5), max(3, args.warmup // 5))
        torch.cuda.empty_cache()
    if not args.no_paged_prefill:
        line["paged_prefill"] = bench_paged_prefill(api, W, max(10, args.steps // 5), max(5, args.warmup // 5))
        torch.cuda.empty_cache()
    if not args.no_unified:
        line["unified"] = bench_unified(api, W, max(10, args.steps // 5), max(5, args.warmup // 5))
        torch.cuda.empty_cache()
    if not args.no_bwd:
        line["bwd"] = bench_bwd(api, W, max(10, args.steps // 5), max(5, args.warmup // 5))
        torch.cuda.empty_cache()
    if not args.no_fp8:
        line["fp8"] = bench_fp8(api, W, max(20, args.steps // 2), max(20, args.warmup // 2))
        torch.cuda.empty_cache()
    if not args.no_alibi:
        line["alibi"] = bench_alibi(api, W, max(20, args.steps // 2), max(20, args.warmup // 2))
        torch.cuda.empty_cache()
    if not args.no_mods:
        line["mods"] = bench_mods(api, W, max(20, args.steps // 2), max(20, args.warmup // 2))
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        tc = W.dense(c["seed"], B, N, H, c["Hkv"], d)
        line["cpu_baseline"] = cpu_baseline(W, tc, c)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
