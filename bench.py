#!/usr/bin/env python3
"""Benchmark of the Gated MLA hot path on one MI355X.

One step = one whole mla_prefill of the K3 Gated MLA layer over B=1, T=4096 causal tokens
(hidden 7168, 96 heads, q/k 192 = 128 nope + 64 shared, v 128, kv_lora 512, q_lora 1536,
sigmoid output gate), inputs resident in HBM. `value` is the layer's algorithmic TFLOP/s.

Also reported on the same JSON line:
* roofline: the dominant kernel of the step, timed live with HIP events on the stream it runs
  on, against the bf16 MFMA peak (2.5 PFLOP/s) or HBM (8 TB/s);
* decode: latent-absorbed decode attention for B=32 sequences with a T=8192 cache (8,193
  visible positions: the new token is appended first), as KV GB/s against HBM, Infinity
  Cache flushed between iterations; the whole mla_decode step; the expanded-cache path at the
  same shape; long-context decode (B=4, T=131072); Gated DSA decode (B=8, T=65536, top-2048);
  and the attainable HBM bandwidth of a plain device copy;
* dsa_prefill: the Gated DSA prefill (every token's own top-2048 selection) at B=1, T=4096;
* cpu_baseline: the oracle (float64 NumPy) timed on the host on a bounded sample of the same
  prefill workload.
All inputs are seeded synthetic data (workloads module); no trained weights are involved.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Gated-MLA prefill TFLOP/s + decode KV GB/s (% of MI355X roofline)"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def prefill_flops(d, T):
    """Algorithmic flops of one prefill of T tokens (B=1): the six projections + attention."""
    H = d.n_heads
    proj = 2 * T * (d.hidden * (d.q_lora + d.kv_lora + d.d_shared + H * d.d_v)   # x -> q_a, kv_a, gate
                    + d.q_lora * H * d.d_qk                                       # q_b
                    + d.kv_lora * H * (d.d_nope + d.d_v)                          # kv_b
                    + H * d.d_v * d.hidden)                                       # o_proj
    attn = 2 * H * (d.d_qk + d.d_v) * (T * (T + 1) // 2)                          # causal pairs
    return proj, attn


def time_events(fn, iters, flush=None):
    """Per-call durations (ms) with events on torch's current stream (the library's stream)."""
    import torch
    out = []
    for _ in range(iters):
        if flush is not None:
            flush()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        e.synchronize()
        out.append(s.elapsed_time(e))
    return out


def time_batched(fn, iters):
    """Average duration (ms) of back-to-back calls, events around the whole batch (launch gaps
    amortised, so it compares with a kernel trace's per-dispatch average)."""
    import torch
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(iters):
        fn()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / iters


def median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def traffic_for(key):
    """HBM bytes per launch of a kernel (or kernel group) from the committed counter runs
    (profiles/traffic.json: rocprofv3 FETCH_SIZE and WRITE_SIZE per dispatch, scaled by what the
    same counters read for a 256 MiB device copy), or None when the kernel's sources changed
    since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            e = json.load(f)["entries"][key]
        h = hashlib.sha256()
        for fn in e["sources"]:
            with open(os.path.join(ROOT, "gated_mla_kv_amd", "csrc", fn), "rb") as f:
                h.update(f.read())
        return e["hbm_bytes_per_launch"] if h.hexdigest()[:16] == e["sources_sha256_16"] else None
    except (OSError, KeyError, ValueError):
        return None


def hbm_copy_gbs(torch, log):
    """Attainable HBM bandwidth: a 2 GiB device-to-device copy (read + write bytes / time)."""
    src = torch.empty(1 << 31, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    dst.copy_(src)
    torch.cuda.synchronize()
    t = median(time_events(lambda: dst.copy_(src), 10))
    del src, dst
    gbs = 2 * (1 << 31) / (t * 1e-3) / 1e9
    log(f"[bench] attainable HBM (2 GiB copy): {gbs:.0f} GB/s")
    return gbs


def roof_hbm(kernel, nbytes, us, traffic_key=None):
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"kernel": kernel, "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic_for(traffic_key) if traffic_key else None}


def decode_benches(args, d, lw, log):
    """Decode-side configurations: batched decode (absorbed and expanded caches, and the whole
    mla_decode step), long-context absorbed decode with split-K and merge, and Gated DSA decode
    (index scores + top-k, then sparse latent attention)."""
    import numpy as np
    import torch

    import gated_mla_kv_amd as gm
    from gated_mla_kv_amd.layer import LayerBuffers, bf16_tensor
    from workloads import K3, make_index_prefix, make_latent_prefix, make_tokens, normal_bf16

    dev = "cuda"
    H = d.n_heads
    it = args.decode_iters
    # Infinity Cache flush between timed calls: read a 1 GiB buffer, which leaves clean lines (a
    # 1 GiB write would leave 256 MB of dirty lines whose write-back halves the next kernel's
    # read bandwidth: 2.8 vs 5.8 TB/s measured for a plain 302 MB stream)
    flush_buf = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    flush = lambda: flush_buf.max()  # noqa: E731
    out = {"hbm_copy_gbs": round(hbm_copy_gbs(torch, log), 1)}
    L = LayerBuffers(d, {k: v for k, v in lw.w.items() if not k.startswith(("w_idx", "g_idx", "b_idx"))}, dev)

    # -- batched decode: B=32, cache T=8192 (8,193 visible) --
    B, Tc = 32, 8192
    nvis = Tc + 1
    log("[bench] batched decode workload (B=32, T=8192)")
    lat = bf16_tensor(make_latent_prefix(d, B, nvis, seed=0), dev)
    dcache = gm.MlaCache(lat.data_ptr(), None, None, None, B, nvis)
    qt = bf16_tensor(normal_bf16((B, H, d.d_latent), 0.05, 0, 22), dev)
    n_vis = torch.full((B,), nvis, dtype=torch.int32, device=dev)
    o = torch.empty((B, H, d.kv_lora), dtype=torch.float32, device=dev)
    dws = torch.empty(gm.workspace_bytes(L.dims, B, 1, nvis, gm.PATH_ABSORBED), dtype=torch.uint8, device=dev)

    def dec():
        gm.mla_decode_attention(L.dims, qt, dcache, n_vis, nvis, B, o, None, 0, dws)

    dec()
    torch.cuda.synchronize()
    t_cold = median(time_events(dec, it, flush=flush))
    t_hot = median(time_events(dec, it))
    kv_bytes = B * nvis * d.d_latent * 2
    r = roof_hbm("decode_attn_k3_kernel<false, false>+decode_merge_kernel", kv_bytes, t_cold * 1e3, "decode:B32_T8192")
    log(f"[bench] absorbed decode attention: {t_cold * 1e3:.1f} us cold, {t_hot * 1e3:.1f} us hot, "
        f"{r['achieved']:.0f} GB/s")
    out.update({"workload": "K3 absorbed decode attention, B=32, cache T=8192 (8193 visible), bf16 latent",
                "kv_bytes": kv_bytes, "us": round(t_cold * 1e3, 2), "us_hot_cache": round(t_hot * 1e3, 2),
                "value": r["achieved"], "unit": "GB/s", "roofline": r})
    # whole decode step (projections, append, attention, gate, o_proj) at the same shape
    dc2 = L.new_cache(B, nvis, expanded=False)
    dc2.latent.copy_(lat)
    xd = bf16_tensor(make_tokens(d, B, 1, seed=0, step=0)[:, 0], dev)
    seq = torch.full((B,), Tc, dtype=torch.int32, device=dev)
    wsd = L.workspace(B, 1, nvis, gm.PATH_ABSORBED)
    yd = torch.empty((B, d.hidden), dtype=torch.bfloat16, device=dev)
    step = lambda: gm.mla_decode(L.dims, L.cw, dc2.c, seq, nvis, xd, B, gm.PATH_ABSORBED, yd,  # noqa: E731
                                 gm.OUT_BF16, None, None, 0, wsd)
    step()
    torch.cuda.synchronize()
    out["mla_decode_step_us"] = round(median(time_events(step, it, flush=flush)) * 1e3, 2)
    # the step's algorithmic bytes: every weight matrix read once (x-projection W_qa | W_kva | W_g,
    # q_b, kv_b for the absorb and the value-up, o_proj), the latent cache read once, the new
    # latent rows written, x read and y written
    H = d.n_heads
    w_bytes = 2 * (d.hidden * (d.q_lora + d.kv_lora + d.d_shared + H * d.d_v) + d.q_lora * H * d.d_qk
                   + d.kv_lora * H * (d.d_nope + d.d_v) + H * d.d_v * d.hidden)
    step_bytes = w_bytes + kv_bytes + B * d.d_latent * 2 + 2 * B * d.hidden * 2
    out["mla_decode_step_roofline"] = roof_hbm("mla_decode (all kernels of the step)", step_bytes,
                                               out["mla_decode_step_us"])
    out["mla_decode_step_roofline"]["weight_bytes"] = w_bytes
    log(f"[bench] whole mla_decode step (absorbed): {out['mla_decode_step_us']:.1f} us, "
        f"{step_bytes / 1e6:.1f} MB ({w_bytes / 1e6:.1f} MB weights), "
        f"{out['mla_decode_step_roofline']['achieved']:.0f} GB/s")
    # the same step captured once in a HIP graph and replayed (no launch gaps between its kernels)
    gs = torch.cuda.Stream()
    gs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(gs):
        step()
    torch.cuda.current_stream().wait_stream(gs)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    graph.replay()
    torch.cuda.synchronize()
    out["mla_decode_step_graph_us"] = round(median(time_events(graph.replay, it, flush=flush)) * 1e3, 2)
    log(f"[bench] whole mla_decode step (absorbed), HIP graph replay: {out['mla_decode_step_graph_us']:.1f} us")
    del graph
    del dc2, wsd

    # the same sequences in the FP8 main cache (656 B per position), quantized by kv_append (setup)
    fcache = L.new_cache(B, nvis, expanded=False, fp8_latent=True)
    zpos = torch.zeros(B, dtype=torch.int32, device=dev)
    gm.kv_append(L.dims, fcache.c, zpos, nvis, B, nvis, lat[..., :d.kv_lora].contiguous(),
                 lat[..., d.kv_lora:].contiguous())
    dec8 = lambda: gm.mla_decode_attention(L.dims, qt, fcache.c, n_vis, nvis, B, o, None, 0, dws)  # noqa: E731
    dec8()
    torch.cuda.synchronize()
    t8 = median(time_events(dec8, it, flush=flush))
    b8 = B * nvis * gm.FP8_LATENT_ROW_BYTES
    r8 = roof_hbm("decode_attn_k3_kernel<false, true>+decode_merge_kernel", b8, t8 * 1e3, "decode_fp8:B32_T8192")
    log(f"[bench] FP8-cache absorbed decode attention: {t8 * 1e3:.1f} us, {r8['achieved']:.0f} GB/s "
        f"({kv_bytes / (t8 * 1e-3) / 1e9:.0f} GB/s of bf16-cache bytes)")
    out["fp8_cache"] = {"workload": "K3 absorbed decode attention, B=32, cache T=8192 (8193 visible), FP8 latent "
                                    "cache (656 B per position)", "kv_bytes": b8, "us": round(t8 * 1e3, 2),
                        "value": r8["achieved"], "unit": "GB/s", "roofline": r8}
    del fcache
    # the same sequences in a paged cache: 64-position pages, each sequence's pages shuffled over the pool
    page = 64
    nbk = -(-nvis // page)
    table = torch.randperm(B * nbk, generator=torch.Generator().manual_seed(0)).view(B, nbk).to(torch.int32)
    pcache = L.new_cache(B, nbk * page, expanded=False, page_size=page, n_pages=B * nbk, block_table=table)
    gm.kv_append(L.dims, pcache.c, zpos, nvis, B, nvis, lat[..., :d.kv_lora].contiguous(),
                 lat[..., d.kv_lora:].contiguous())
    decp = lambda: gm.mla_decode_attention(L.dims, qt, pcache.c, n_vis, nvis, B, o, None, 0, dws)  # noqa: E731
    decp()
    torch.cuda.synchronize()
    tp = median(time_events(decp, it, flush=flush))
    rp = roof_hbm("decode_attn_k3_kernel+decode_merge_kernel (paged)", kv_bytes, tp * 1e3)
    log(f"[bench] paged-cache absorbed decode attention (64-position pages): {tp * 1e3:.1f} us, {rp['achieved']:.0f} GB/s")
    out["paged_cache"] = {"workload": "K3 absorbed decode attention, B=32, cache T=8192 (8193 visible), bf16 latent "
                                      "in 64-position pages, shuffled", "kv_bytes": kv_bytes, "us": round(tp * 1e3, 2),
                          "value": rp["achieved"], "unit": "GB/s", "roofline": rp}
    del pcache

    # expanded cache for the same sequences, built from the latents by the kv_b projection (setup)
    log("[bench] expanded decode workload: building K/V [32, 96, 8193, 192|128] from the latents")
    ecache = L.new_cache(B, nvis, expanded=True)
    ecache.latent.copy_(lat)
    pos0 = torch.zeros(1, dtype=torch.int32, device=dev)
    kvb = torch.empty((nvis, H * (d.d_nope + d.d_v)), dtype=torch.bfloat16, device=dev)
    for b in range(B):
        cb = lat[b, :, :d.kv_lora].contiguous()
        rb = lat[b, :, d.kv_lora:].contiguous()
        gm.mla_gemm(cb, d.kv_lora, L.w["w_kv_b"], nvis, kvb.shape[1], d.kv_lora, kvb, kvb.shape[1])
        kv4 = kvb.view(nvis, H, d.d_nope + d.d_v)
        kn, vv = kv4[..., :d.d_nope].contiguous(), kv4[..., d.d_nope:].contiguous()
        view = gm.MlaCache(ecache.latent[b].data_ptr(), ecache.k[b].data_ptr(), ecache.v[b].data_ptr(), None, 1,
                           nvis)
        gm.kv_append(L.dims, view, pos0, nvis, 1, nvis, cb, rb, kn, vv)
    torch.cuda.synchronize()
    del kvb, kn, vv, cb, rb
    qe = bf16_tensor(normal_bf16((B, H, d.d_qk), 0.8, 0, 23), dev)
    z = torch.empty((B, H, d.d_v), dtype=torch.float32, device=dev)
    exp_fn = lambda: gm.mla_expanded_attention(L.dims, qe, ecache.c, n_vis, nvis, B, z)  # noqa: E731
    exp_fn()
    torch.cuda.synchronize()
    t_exp = median(time_events(exp_fn, max(3, it // 4), flush=flush))
    e_bytes = B * H * nvis * (d.d_qk + d.d_v) * 2
    re = roof_hbm("expanded_attn_kernel", e_bytes, t_exp * 1e3)
    log(f"[bench] expanded decode attention: {t_exp * 1e3:.1f} us, {re['achieved']:.0f} GB/s")
    out["expanded"] = {"workload": "K3 expanded-cache decode attention, B=32, T=8192 (8193 visible)",
                       "kv_bytes": e_bytes, "us": round(t_exp * 1e3, 2), "value": re["achieved"], "unit": "GB/s",
                       "roofline": re}
    del ecache, lat, dcache, o, dws, qe, z
    torch.cuda.empty_cache()

    # -- long-context decode: B=4, cache T=131072 --
    B4, T4 = 4, 131072
    nv4 = T4 + 1
    log("[bench] long-context decode workload (B=4, T=131072)")
    lat4 = bf16_tensor(make_latent_prefix(d, B4, nv4, seed=0), dev)
    c4 = gm.MlaCache(lat4.data_ptr(), None, None, None, B4, nv4)
    qt4 = bf16_tensor(normal_bf16((B4, H, d.d_latent), 0.05, 0, 24), dev)
    n4 = torch.full((B4,), nv4, dtype=torch.int32, device=dev)
    o4 = torch.empty((B4, H, d.kv_lora), dtype=torch.float32, device=dev)
    ws4 = torch.empty(gm.workspace_bytes(L.dims, B4, 1, nv4, gm.PATH_ABSORBED), dtype=torch.uint8, device=dev)
    f4 = lambda: gm.mla_decode_attention(L.dims, qt4, c4, n4, nv4, B4, o4, None, 0, ws4)  # noqa: E731
    f4()
    torch.cuda.synchronize()
    t4 = median(time_events(f4, it, flush=flush))
    b4 = B4 * nv4 * d.d_latent * 2
    r4 = roof_hbm("decode_attn_k3_kernel+decode_merge_kernel", b4, t4 * 1e3, "decode:B4_T131072")
    log(f"[bench] long-context absorbed decode: {t4 * 1e3:.1f} us, {r4['achieved']:.0f} GB/s")
    out["long_context"] = {"workload": "K3 absorbed decode attention, B=4, cache T=131072 (131073 visible), "
                                       "split-K + softmax merge", "kv_bytes": b4, "us": round(t4 * 1e3, 2),
                           "value": r4["achieved"], "unit": "GB/s", "roofline": r4}
    del lat4, c4, o4, ws4
    torch.cuda.empty_cache()

    # -- Gated DSA decode: B=8, cache T=65536 (65,537 visible), top-2048 --
    dd = K3
    B5, T5 = 8, 65536
    nv5 = T5 + 1
    log("[bench] DSA decode workload (B=8, T=65536)")
    L5 = LayerBuffers(dd, lw.w, dev)
    lat5 = bf16_tensor(make_latent_prefix(dd, B5, nv5, seed=0), dev)
    idx5 = bf16_tensor(make_index_prefix(dd, B5, nv5, seed=0), dev)
    c5 = gm.MlaCache(lat5.data_ptr(), None, None, idx5.data_ptr(), B5, nv5)
    f32 = lambda bits: torch.from_numpy((bits.astype("uint32") << 16).view("float32")).to(dev)  # noqa: E731
    # the index query in fp32, as the indexer produces it (the library takes it unrounded)
    qi = torch.from_numpy(np.random.default_rng(25).standard_normal((B5, dd.n_idx_heads, dd.d_idx))
                          .astype(np.float32) * np.float32(0.5)).to(dev)
    wi = f32(normal_bf16((B5, dd.n_idx_heads), 1.0, 0, 26))
    n5 = torch.full((B5,), nv5, dtype=torch.int32, device=dev)
    sel = torch.empty((B5, dd.topk), dtype=torch.int32, device=dev)
    cnt = torch.empty((B5,), dtype=torch.int32, device=dev)
    ws5 = torch.empty(gm.workspace_bytes(L5.dims, B5, 1, nv5, gm.PATH_SPARSE), dtype=torch.uint8, device=dev)
    qt5 = bf16_tensor(normal_bf16((B5, H, dd.d_latent), 0.05, 0, 27), dev)
    o5 = torch.empty((B5, H, dd.kv_lora), dtype=torch.float32, device=dev)
    topk_fn = lambda: gm.dsa_index_topk(L5.dims, qi, wi, idx5, nv5, n5, nv5, B5, sel, cnt, None, ws5)  # noqa: E731
    sparse_fn = lambda: gm.mla_sparse_attention(L5.dims, qt5, c5, sel, cnt, B5, o5, None, 0, ws5)  # noqa: E731

    def dsa_fn():
        topk_fn()
        sparse_fn()

    dsa_fn()
    torch.cuda.synchronize()
    t_topk = median(time_events(topk_fn, it, flush=flush))
    t_sparse = median(time_events(sparse_fn, it, flush=flush))
    t_dsa = median(time_events(dsa_fn, it, flush=flush))
    b_idx = B5 * nv5 * dd.d_idx * 2
    b_sel = B5 * dd.topk * dd.d_latent * 2
    r5 = roof_hbm("index_scores_kernel+topk_count_kernel+topk_select_kernel+topk_compact_kernel+decode_attn_k3_kernel<true, false>+decode_merge_kernel",
                  b_idx + b_sel, t_dsa * 1e3, "dsa:B8_T65536")
    log(f"[bench] DSA decode: index+top-k {t_topk * 1e3:.1f} us, sparse {t_sparse * 1e3:.1f} us, "
        f"together {t_dsa * 1e3:.1f} us, {r5['achieved']:.0f} GB/s")
    out["dsa"] = {"workload": "K3.1 Gated DSA decode, B=8, cache T=65536 (65537 visible), top-2048",
                  "bytes": b_idx + b_sel, "us": round(t_dsa * 1e3, 2), "value": r5["achieved"], "unit": "GB/s",
                  "roofline": r5,
                  "index_topk": {"us": round(t_topk * 1e3, 2), "bytes": b_idx,
                                 "gbs": round(b_idx / (t_topk * 1e-6 * 1e3) / 1e9, 1)},
                  "sparse_attention": {"us": round(t_sparse * 1e3, 2), "bytes": b_sel,
                                       "gbs": round(b_sel / (t_sparse * 1e-6 * 1e3) / 1e9, 1)}}
    # the same DSA step over FP8 caches (656 B latent rows, 132 B index keys), quantized by kv_append
    f5 = L5.new_cache(B5, nv5, expanded=False, index=True, fp8_latent=True, fp8_index=True)
    gm.kv_append(L5.dims, f5.c, torch.zeros(B5, dtype=torch.int32, device=dev), nv5, B5, nv5,
                 lat5[..., :dd.kv_lora].contiguous(), lat5[..., dd.kv_lora:].contiguous(), None, None, idx5)
    topk8 = lambda: gm.dsa_index_topk_fp8(L5.dims, qi, wi, f5.idx_codes, f5.idx_scales, nv5, n5, nv5, B5,  # noqa: E731
                                          sel, cnt, None, ws5)
    sparse8 = lambda: gm.mla_sparse_attention(L5.dims, qt5, f5.c, sel, cnt, B5, o5, None, 0, ws5)  # noqa: E731

    def dsa8_fn():
        topk8()
        sparse8()

    dsa8_fn()
    torch.cuda.synchronize()
    t8 = median(time_events(dsa8_fn, it, flush=flush))
    t8_topk = median(time_events(topk8, it, flush=flush))
    b8 = B5 * nv5 * (dd.d_idx + 4) + B5 * dd.topk * gm.FP8_LATENT_ROW_BYTES
    r8 = roof_hbm("index_scores_kernel (FP8 keys)+topk_count_kernel+topk_select_kernel+topk_compact_kernel+decode_attn_k3_kernel<true, true>+decode_merge_kernel",
                  b8, t8 * 1e3, "dsa_fp8:B8_T65536")
    log(f"[bench] FP8-cache DSA decode: index+top-k {t8_topk * 1e3:.1f} us, together {t8 * 1e3:.1f} us, "
        f"{r8['achieved']:.0f} GB/s")
    out["dsa"]["fp8_cache"] = {"workload": "K3.1 Gated DSA decode, B=8, T=65536, FP8 caches (132 B index keys, "
                                           "656 B latent rows)", "bytes": b8, "us": round(t8 * 1e3, 2),
                               "index_topk_us": round(t8_topk * 1e3, 2), "value": r8["achieved"], "unit": "GB/s",
                               "roofline": r8}
    del flush_buf
    return out


def dsa_prefill_bench(args, lw, log):
    """Gated DSA prefill (mla_prefill_sparse) of B=1, T tokens with the K3.1 indexer (top-2048):
    the whole call timed with events; its algorithmic flops counted per token (projections
    without kv_b, index projections, index scores over t positions, the sparse core over
    min(k, t) positions, query absorption and value up-projection)."""
    import torch

    import gated_mla_kv_amd as gm
    from gated_mla_kv_amd.layer import LayerBuffers, bf16_tensor
    from workloads import K3, make_tokens

    d, T, H = K3, args.T, K3.n_heads
    L = LayerBuffers(d, lw.w, "cuda")
    x = bf16_tensor(make_tokens(d, 1, T, seed=0), "cuda")
    cache = L.new_cache(1, T, expanded=False, index=True)
    start = torch.zeros(1, dtype=torch.int32, device="cuda")
    y = torch.empty((1, T, d.hidden), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(gm.workspace_bytes_prefill_sparse(L.dims, 1, T, T), dtype=torch.uint8, device="cuda")

    def run():
        gm.mla_prefill_sparse(L.dims, L.cw, cache.c, start, T, x, 1, T, y, gm.OUT_BF16, None, None, ws)

    run()
    torch.cuda.synchronize()
    ms = median(time_events(run, max(3, args.steps // 4)))
    tok = 2 * T * (d.hidden * (d.q_lora + d.kv_lora + d.d_shared + H * d.d_v + d.d_idx + d.n_idx_heads)
                   + d.q_lora * (H * d.d_qk + d.n_idx_heads * d.d_idx)
                   + H * d.d_v * d.hidden
                   + 2 * H * d.d_nope * d.kv_lora)                       # absorb + value up
    pos = sum(range(1, T + 1))
    sel = sum(min(d.topk, t) for t in range(1, T + 1))
    fl = tok + 2 * d.n_idx_heads * d.d_idx * pos + 2 * H * (d.d_latent + d.kv_lora) * sel
    tf = fl / (ms * 1e-3) / 1e12
    log(f"[bench] DSA prefill (B=1, T={T}, top-{d.topk}): {ms:.3f} ms, {tf:.1f} TFLOP/s algorithmic")
    return {"workload": f"K3.1 Gated DSA prefill, B=1, T={T} causal, top-{d.topk}, bf16", "ms": round(ms, 4),
            "flops": fl, "tflops": round(tf, 1)}


def counter_pass(log):
    """--counters: each measured kernel launched twice at the bench's shapes (the four prefill GEMMs
    in the order x_proj, q_b, kv_b, o_proj, then the prefill attention and the decode kernels), and a plain device
    copy of 256 MiB (reads 256 MiB, writes 256 MiB) that calibrates rocprofv3's FETCH_SIZE and
    WRITE_SIZE, for counter runs (rocprofv3 --pmc ... -- python3 bench.py --counters)."""
    import torch

    import gated_mla_kv_amd as gm
    from workloads import K3, device_normal_bf16, device_normal_f32

    dev = "cuda"
    d, dd = K3.replace(n_idx_heads=0), K3
    H, T = d.n_heads, 4096
    dims, dims5 = gm.make_dims(d), gm.make_dims(dd)
    src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    log("[counters] copy 256 MiB x2 done")
    # prefill stages (same calls as the timed stages)
    x = device_normal_bf16((T, d.hidden), 1.0, 9, 1)
    w_x = device_normal_bf16((d.q_lora + d.kv_lora + d.d_shared + H * d.d_v, d.hidden), 0.02, 9, 2)
    out_x = torch.empty((T, w_x.shape[0]), dtype=torch.float32, device=dev)
    for _ in range(2):
        gm.mla_gemm(x, d.hidden, w_x, T, w_x.shape[0], d.hidden, out_x, w_x.shape[0], gm.OUT_F32)
    del out_x, w_x
    cq = device_normal_bf16((T, d.q_lora), 1.0, 9, 16)
    w_qb = device_normal_bf16((H * d.d_qk, d.q_lora), 0.02, 9, 17)
    qb = torch.empty((T, H * d.d_qk), dtype=torch.bfloat16, device=dev)
    for _ in range(2):
        gm.mla_gemm(cq, d.q_lora, w_qb, T, H * d.d_qk, d.q_lora, qb, H * d.d_qk)
    del cq, w_qb, qb
    c = device_normal_bf16((T, d.kv_lora), 1.0, 9, 18)
    w_kvb = device_normal_bf16((H * (d.d_nope + d.d_v), d.kv_lora), 0.02, 9, 19)
    kvb = torch.empty((T, H * (d.d_nope + d.d_v)), dtype=torch.bfloat16, device=dev)
    for _ in range(2):
        gm.mla_gemm(c, d.kv_lora, w_kvb, T, H * (d.d_nope + d.d_v), d.kv_lora, kvb, H * (d.d_nope + d.d_v))
    del c, w_kvb, kvb
    u = device_normal_bf16((T, H * d.d_v), 1.0, 9, 3)
    w_o = device_normal_bf16((d.hidden, H * d.d_v), 0.02, 9, 4)
    y = torch.empty((T, d.hidden), dtype=torch.bfloat16, device=dev)
    for _ in range(2):
        gm.mla_gemm(u, H * d.d_v, w_o, T, d.hidden, H * d.d_v, y, d.hidden)
    del u, w_o, y
    q = device_normal_bf16((1, T, H, d.d_qk), 0.8, 9, 5)
    K = device_normal_bf16((1, H, T, d.d_qk), 0.8, 9, 6)
    V = device_normal_bf16((1, H, T, d.d_v), 1.0, 9, 7)
    g = torch.zeros((1, T, H * d.d_v), device=dev)
    ua = torch.empty((1, T, H * d.d_v), dtype=torch.bfloat16, device=dev)
    cache = gm.MlaCache(None, K.data_ptr(), V.data_ptr(), None, 1, T)
    start = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(2):
        gm.mla_prefill_attention(dims, q, cache, start, T, 1, T, g, ua, gm.OUT_BF16, None)
    torch.cuda.synchronize()
    del q, K, V, g, ua
    log("[counters] prefill stages done")
    # absorbed decode: B=32 x 8193 and B=4 x 131073
    for B, nv in ((32, 8193), (4, 131073)):
        lat = device_normal_bf16((B, nv, d.d_latent), 1.0, 9, 8)
        qt = device_normal_bf16((B, H, d.d_latent), 0.05, 9, 9)
        c = gm.MlaCache(lat.data_ptr(), None, None, None, B, nv)
        n = torch.full((B,), nv, dtype=torch.int32, device=dev)
        o = torch.empty((B, H, d.kv_lora), dtype=torch.float32, device=dev)
        ws = torch.empty(gm.workspace_bytes(dims, B, 1, nv, gm.PATH_ABSORBED), dtype=torch.uint8, device=dev)
        for _ in range(2):
            gm.mla_decode_attention(dims, qt, c, n, nv, B, o, None, 0, ws)
        torch.cuda.synchronize()
        del lat, qt, o, ws
    log("[counters] absorbed decode done")
    # DSA decode: B=8 x 65537
    B, nv = 8, 65537
    lat = device_normal_bf16((B, nv, dd.d_latent), 1.0, 9, 10)
    idx = device_normal_bf16((B, nv, dd.d_idx), 1.0, 9, 11)
    qi = device_normal_f32((B, dd.n_idx_heads, dd.d_idx), 0.5, 9, 12)
    wi = torch.ones((B, dd.n_idx_heads), device=dev)
    qt = device_normal_bf16((B, H, dd.d_latent), 0.05, 9, 13)
    c = gm.MlaCache(lat.data_ptr(), None, None, idx.data_ptr(), B, nv)
    n = torch.full((B,), nv, dtype=torch.int32, device=dev)
    sel = torch.empty((B, dd.topk), dtype=torch.int32, device=dev)
    cnt = torch.empty((B,), dtype=torch.int32, device=dev)
    o = torch.empty((B, H, dd.kv_lora), dtype=torch.float32, device=dev)
    ws = torch.empty(gm.workspace_bytes(dims5, B, 1, nv, gm.PATH_SPARSE), dtype=torch.uint8, device=dev)
    for _ in range(2):
        gm.dsa_index_topk(dims5, qi, wi, idx, nv, n, nv, B, sel, cnt, None, ws)
        gm.mla_sparse_attention(dims5, qt, c, sel, cnt, B, o, None, 0, ws)
    torch.cuda.synchronize()
    log("[counters] DSA decode done")
    # FP8 caches (quantized by kv_append first): the DSA step B=8 x 65537, then absorbed decode B=32 x 8193
    from gated_mla_kv_amd.layer import CacheBuffers
    f8 = CacheBuffers(dd, B, nv, expanded=False, index=True, fp8_latent=True, fp8_index=True)
    gm.kv_append(dims5, f8.c, torch.zeros(B, dtype=torch.int32, device=dev), nv, B, nv,
                 lat[..., :dd.kv_lora].contiguous(), lat[..., dd.kv_lora:].contiguous(), None, None, idx)
    for _ in range(2):
        gm.dsa_index_topk_fp8(dims5, qi, wi, f8.idx_codes, f8.idx_scales, nv, n, nv, B, sel, cnt, None, ws)
        gm.mla_sparse_attention(dims5, qt, f8.c, sel, cnt, B, o, None, 0, ws)
    torch.cuda.synchronize()
    del lat, idx, f8, c, o, ws
    B, nv = 32, 8193
    lat = device_normal_bf16((B, nv, d.d_latent), 1.0, 9, 14)
    qt = device_normal_bf16((B, H, d.d_latent), 0.05, 9, 15)
    f8 = CacheBuffers(d, B, nv, expanded=False, fp8_latent=True)
    gm.kv_append(dims, f8.c, torch.zeros(B, dtype=torch.int32, device=dev), nv, B, nv,
                 lat[..., :d.kv_lora].contiguous(), lat[..., d.kv_lora:].contiguous())
    n = torch.full((B,), nv, dtype=torch.int32, device=dev)
    o = torch.empty((B, H, d.kv_lora), dtype=torch.float32, device=dev)
    ws = torch.empty(gm.workspace_bytes(dims, B, 1, nv, gm.PATH_ABSORBED), dtype=torch.uint8, device=dev)
    for _ in range(2):
        gm.mla_decode_attention(dims, qt, f8.c, n, nv, B, o, None, 0, ws)
    torch.cuda.synchronize()
    log("[counters] FP8 caches done")


def cpu_decode_baselines(log):
    """The oracle on sampled sequences of the decode workloads, in the GPU lines' unit (GB/s of
    algorithmic bytes: 1,152 B per visible latent position; DSA: 256 B per index key plus 1,152 B
    per selected position). Each sample is the first sequences of the GPU workload's own inputs
    (the generators draw sequences in order)."""
    import numpy as np

    import oracle as O
    from workloads import K3, bf16_bits_to_f32, make_index_prefix, make_latent_prefix, normal_bf16

    d = K3
    out = {}
    for key, B, n_s, T, q_id in (("B32_T8192", 32, 4, 8192, 22), ("B4_T131072", 4, 1, 131072, 24)):
        nv = T + 1
        lat = bf16_bits_to_f32(make_latent_prefix(d, n_s, nv, seed=0)).astype(np.float64)
        qt = bf16_bits_to_f32(normal_bf16((B, d.n_heads, d.d_latent), 0.05, 0, q_id)).astype(np.float64)[:n_s]
        t0 = time.perf_counter()
        for b in range(n_s):
            O.attention_absorbed(qt[b][None, None], lat[b][None], O.softmax_scale(d), nv - 1, d)
        dt = time.perf_counter() - t0
        nbytes = n_s * nv * d.d_latent * 2
        out[key] = {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "kind": "oracle",
                    "sample": f"absorbed decode attention (oracle.attention_absorbed) of {n_s} of the {B} sequences, "
                              f"{nv} visible positions each, {dt:.1f} s"}
        log(f"[bench] CPU oracle decode {key}: {dt:.1f} s, {out[key]['value']} GB/s")
        del lat
    B, nv = 8, 65537
    lat = bf16_bits_to_f32(make_latent_prefix(d, B, nv, seed=0)).astype(np.float64)
    idx = bf16_bits_to_f32(make_index_prefix(d, B, nv, seed=0)).astype(np.float64)
    rng = np.random.default_rng(25)
    qi = rng.standard_normal((B, d.n_idx_heads, d.d_idx)).astype(np.float32) * np.float32(0.5)
    wi = bf16_bits_to_f32(normal_bf16((B, d.n_idx_heads), 1.0, 0, 26)).astype(np.float64)
    qt = bf16_bits_to_f32(normal_bf16((B, d.n_heads, d.d_latent), 0.05, 0, 27)).astype(np.float64)
    t0 = time.perf_counter()
    for b in range(B):
        I = O.index_scores(qi[b].astype(np.float64), wi[b], idx[b], nv)
        S = O.select_topk(I, d.topk)
        O.attention_absorbed_subset(qt[b], lat[b], S, O.softmax_scale(d), d)
    dt = time.perf_counter() - t0
    nbytes = B * (nv * d.d_idx * 2 + d.topk * d.d_latent * 2)
    out["dsa_B8_T65536"] = {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "kind": "oracle",
                            "sample": f"index scores, top-{d.topk} and sparse attention (oracle.index_scores, "
                                      f"select_topk, attention_absorbed_subset) of all {B} sequences, {nv} visible "
                                      f"positions each, {dt:.1f} s"}
    log(f"[bench] CPU oracle DSA decode: {dt:.1f} s, {out['dsa_B8_T65536']['value']} GB/s")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--T", type=int, default=4096)
    ap.add_argument("--cpu-sample-tokens", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--decode-iters", type=int, default=20)
    ap.add_argument("--counters", action="store_true",
                    help="launch each measured kernel twice (for rocprofv3 --pmc runs) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (sharding is described in "
              "DESIGN.md but not built); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.counters:
        counter_pass(lambda *a: print(*a, file=sys.stderr, flush=True))
        return

    import numpy as np
    import torch

    import gated_mla_kv_amd as gm
    from gated_mla_kv_amd.layer import LayerBuffers, bf16_tensor
    from workloads import K3, make_latent_prefix, make_layer_weights, make_tokens, normal_bf16

    dev = "cuda"
    d = K3.replace(n_idx_heads=0)  # the dense Gated MLA layer
    T = args.T
    log = lambda *a: print(*a, file=sys.stderr, flush=True)  # noqa: E731
    log(f"[bench] building K3 weights and inputs (T={T})")
    lw = make_layer_weights(K3, seed=0)  # dense layer weights plus the DSA indexer's
    L = LayerBuffers(d, lw.w, dev)
    x_bits = make_tokens(d, 1, T, seed=0)
    x = bf16_tensor(x_bits, dev)
    cache = L.new_cache(1, T, expanded=True)
    start = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = L.workspace(1, T, T)
    y = torch.empty((1, T, d.hidden), dtype=torch.bfloat16, device=dev)

    def step():
        gm.mla_prefill(L.dims, L.cw, cache.c, start, T, x, 1, T, y, gm.OUT_BF16, None, ws)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} prefill steps")
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    proj_fl, attn_fl = prefill_flops(d, T)
    total_fl = proj_fl + attn_fl
    tflops = total_fl / (ms_step * 1e-3) / 1e12
    log(f"[bench] prefill {ms_step:.3f} ms/step, {tflops:.1f} TFLOP/s")

    # ---- per-stage kernels of the step, each timed alone with the same launch shapes ----
    H = d.n_heads
    M = T
    iters = max(5, args.steps)
    stages = {}
    xa = x.view(M, d.hidden)
    w_x = torch.cat([L.w["w_q_a"], L.w["w_kv_a"], L.w["w_g"]], 0).contiguous()
    out_x = torch.empty((M, w_x.shape[0]), dtype=torch.float32, device=dev)
    stages["x_proj_gemm"] = (lambda: gm.mla_gemm(xa, d.hidden, w_x, M, w_x.shape[0], d.hidden, out_x,
                                                 w_x.shape[0], gm.OUT_F32),
                             2 * M * d.hidden * w_x.shape[0], "gemm_nt_dma")
    cq = torch.randn((M, d.q_lora), device=dev).to(torch.bfloat16)
    qb = torch.empty((M, H * d.d_qk), dtype=torch.bfloat16, device=dev)
    stages["q_b_gemm"] = (lambda: gm.mla_gemm(cq, d.q_lora, L.w["w_q_b"], M, H * d.d_qk, d.q_lora, qb, H * d.d_qk),
                          2 * M * d.q_lora * H * d.d_qk, "gemm_nt_dma")
    c = torch.randn((M, d.kv_lora), device=dev).to(torch.bfloat16)
    kvb = torch.empty((M, H * (d.d_nope + d.d_v)), dtype=torch.bfloat16, device=dev)
    stages["kv_b_gemm"] = (lambda: gm.mla_gemm(c, d.kv_lora, L.w["w_kv_b"], M, H * 256, d.kv_lora, kvb, H * 256),
                           2 * M * d.kv_lora * H * 256, "gemm_nt_dma")
    u = torch.randn((M, H * d.d_v), device=dev).to(torch.bfloat16)
    yo = torch.empty((M, d.hidden), dtype=torch.bfloat16, device=dev)
    stages["o_proj_gemm"] = (lambda: gm.mla_gemm(u, H * d.d_v, L.w["w_o"], M, d.hidden, H * d.d_v, yo, d.hidden),
                             2 * M * H * d.d_v * d.hidden, "gemm_nt_dma")
    qa = (torch.randn((1, T, H, d.d_qk), device=dev) * 0.8).to(torch.bfloat16)
    gpre = torch.randn((1, T, H * d.d_v), device=dev)
    ua = torch.empty((1, T, H * d.d_v), dtype=torch.bfloat16, device=dev)
    stages["prefill_attention"] = (lambda: gm.mla_prefill_attention(L.dims, qa, cache.c, start, T, 1, T, gpre, ua,
                                                                    gm.OUT_BF16, None),
                                   attn_fl, "prefill_attn_k3_kernel")
    stage_ms = {}
    for name, (fn, fl, kern) in stages.items():
        fn()
        torch.cuda.synchronize()
        stage_ms[name] = time_batched(fn, iters)
        log(f"[bench] {name}: {stage_ms[name]:.3f} ms, {fl / (stage_ms[name] * 1e-3) / 1e12:.1f} TFLOP/s")
    dom = max(stage_ms, key=stage_ms.get)
    dom_fl = stages[dom][1]
    ach = dom_fl / (stage_ms[dom] * 1e-3) / 1e12
    tkey = {"x_proj_gemm": "prefill:x_proj_gemm", "o_proj_gemm": "prefill:o_proj_gemm",
            "prefill_attention": "prefill:attention"}.get(dom)
    roofline = {"kernel": stages[dom][2], "stage": dom, "bound": "mfma", "achieved": round(ach, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_for(tkey) if tkey else None, "flops_per_launch": dom_fl,
                "ms_per_launch": round(stage_ms[dom], 4)}
    kernels = {k: {"ms": round(v, 4), "tflops": round(stages[k][1] / (v * 1e-3) / 1e12, 1)}
               for k, v in stage_ms.items()}
    del out_x, w_x, cq, qb, c, kvb, u, yo, qa, gpre, ua

    # ---- decode configurations (each kernel timed alone; Infinity Cache flushed between calls) ----
    decode = None
    if not args.no_decode:
        del cache
        torch.cuda.empty_cache()
        decode = decode_benches(args, d, lw, log)
    dsa_prefill = None
    if not args.no_decode:
        torch.cuda.empty_cache()
        dsa_prefill = dsa_prefill_bench(args, lw, log)
    # ---- CPU baseline: the oracle on a bounded sample of the prefill workload ----
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O
        from workloads import bf16_bits_to_f32
        Ts = min(args.cpu_sample_tokens, T)
        log(f"[bench] CPU baseline: oracle prefill of the first {Ts} tokens")
        w64 = {k: bf16_bits_to_f32(v).astype(np.float64) for k, v in lw.w.items()}
        xs = bf16_bits_to_f32(x_bits[:, :Ts]).astype(np.float64)
        cores = len(os.sched_getaffinity(0))
        try:
            from threadpoolctl import threadpool_info
            blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            blas_threads = None
        t_a = time.perf_counter()
        O.layer_forward(xs, w64, O.Cache(d, 1), d)
        dt = time.perf_counter() - t_a
        pf, af = prefill_flops(d, Ts)
        cpu = {"value": round((pf + af) / dt / 1e12, 5), "unit": "TFLOP/s", "cores": cores,
               "blas_threads": blas_threads, "kind": "oracle",
               "sample": f"float64 NumPy oracle, full K3 layer prefill of the first {Ts} of the 4096 tokens "
                         f"(B=1, same weights), {dt:.1f} s; a sample, not the whole step"}
        log(f"[bench] CPU oracle: {dt:.1f} s, {cpu['value']} TFLOP/s ({cores} cores, {blas_threads} BLAS threads)")
        if not args.no_decode:
            cpu["decode"] = cpu_decode_baselines(log)

    line = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,0.02^2) weights, N(0,1) inputs)",
        "config": {"workload": f"K3 Gated MLA prefill, B=1, T={T} causal, bf16", "B": 1, "T": T,
                   "hidden": d.hidden, "heads": H, "d_qk": d.d_qk, "d_v": d.d_v, "kv_lora": d.kv_lora,
                   "q_lora": d.q_lora, "flops_per_step": total_fl, "attention_flops": attn_fl},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "decode": decode,
        "dsa_prefill": dsa_prefill,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
