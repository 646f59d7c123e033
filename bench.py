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
  Cache flushed between iterations; and the whole mla_decode step;
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


def median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


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
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (sharding is described in "
              "DESIGN.md but not built); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

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
    lw = make_layer_weights(d, seed=0)
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
        stage_ms[name] = median(time_events(fn, iters))
        log(f"[bench] {name}: {stage_ms[name]:.3f} ms, {fl / (stage_ms[name] * 1e-3) / 1e12:.1f} TFLOP/s")
    dom = max(stage_ms, key=stage_ms.get)
    dom_fl = stages[dom][1]
    ach = dom_fl / (stage_ms[dom] * 1e-3) / 1e12
    roofline = {"kernel": stages[dom][2], "stage": dom, "bound": "mfma", "achieved": round(ach, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": None, "flops_per_launch": dom_fl, "ms_per_launch": round(stage_ms[dom], 4)}
    kernels = {k: {"ms": round(v, 4), "tflops": round(stages[k][1] / (v * 1e-3) / 1e12, 1)}
               for k, v in stage_ms.items()}
    del out_x, w_x, cq, qb, c, kvb, u, yo, qa, gpre, ua

    # ---- decode: latent-absorbed attention over B=32 x 8,193 positions ----
    decode = None
    if not args.no_decode:
        B, Tc = 32, 8192
        nvis = Tc + 1
        log("[bench] building the decode workload (B=32, T=8192)")
        lat = bf16_tensor(make_latent_prefix(d, B, nvis, seed=0), dev)
        dcache = gm.MlaCache(lat.data_ptr(), None, None, None, B, nvis)
        qt = bf16_tensor(normal_bf16((B, H, d.d_latent), 0.05, 0, 22), dev)
        n_vis = torch.full((B,), nvis, dtype=torch.int32, device=dev)
        o = torch.empty((B, H, d.kv_lora), dtype=torch.float32, device=dev)
        dws = torch.empty(gm.workspace_bytes(L.dims, B, 1, nvis, gm.PATH_ABSORBED), dtype=torch.uint8, device=dev)
        flush_buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)

        def dec():
            gm.mla_decode_attention(L.dims, qt, dcache, n_vis, nvis, B, o, None, 0, dws)

        dec()
        torch.cuda.synchronize()
        cold = time_events(dec, args.decode_iters, flush=lambda: flush_buf.zero_())
        hot = time_events(dec, args.decode_iters)
        kv_bytes = B * nvis * d.d_latent * 2
        t_cold = median(cold)
        gbs = kv_bytes / (t_cold * 1e-3) / 1e9
        log(f"[bench] absorbed decode attention: {t_cold * 1e3:.1f} us cold, {median(hot) * 1e3:.1f} us hot, "
            f"{gbs:.0f} GB/s")
        # whole decode step (projections, append, attention, gate, o_proj) at the same shape
        dcache2 = L.new_cache(B, nvis, expanded=False)
        dcache2.latent.copy_(lat)
        del lat
        xd = bf16_tensor(make_tokens(d, B, 1, seed=0, step=0)[:, 0], dev)
        seq = torch.full((B,), Tc, dtype=torch.int32, device=dev)
        wsd = L.workspace(B, 1, nvis, gm.PATH_ABSORBED)
        yd = torch.empty((B, d.hidden), dtype=torch.bfloat16, device=dev)

        def dstep():
            gm.mla_decode(L.dims, L.cw, dcache2.c, seq, nvis, xd, B, gm.PATH_ABSORBED, yd, gm.OUT_BF16, None, None,
                          0, wsd)

        dstep()
        torch.cuda.synchronize()
        t_step = median(time_events(dstep, args.decode_iters, flush=lambda: flush_buf.zero_()))
        decode = {"workload": "K3 absorbed decode attention, B=32, cache T=8192 (8193 visible), bf16 latent",
                  "kv_bytes": kv_bytes, "us": round(t_cold * 1e3, 2), "us_hot_cache": round(median(hot) * 1e3, 2),
                  "value": round(gbs, 1), "unit": "GB/s",
                  "roofline": {"kernel": "decode_attn_k3_kernel+decode_merge_kernel", "bound": "hbm",
                               "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                               "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None},
                  "mla_decode_step_us": round(t_step * 1e3, 2)}
        del flush_buf

    # ---- CPU baseline: the oracle on a bounded sample of the prefill workload ----
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O
        from workloads import bf16_bits_to_f32
        Ts = min(args.cpu_sample_tokens, T)
        log(f"[bench] CPU baseline: oracle prefill of the first {Ts} tokens")
        w64 = {k: bf16_bits_to_f32(v).astype(np.float64) for k, v in lw.w.items()}
        xs = bf16_bits_to_f32(x_bits[:, :Ts]).astype(np.float64)
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            threads = len(os.sched_getaffinity(0))
        t_a = time.perf_counter()
        O.layer_forward(xs, w64, O.Cache(d, 1), d)
        dt = time.perf_counter() - t_a
        pf, af = prefill_flops(d, Ts)
        cpu = {"value": round((pf + af) / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
               "sample": f"float64 NumPy oracle, full K3 layer prefill of the first {Ts} of the 4096 tokens "
                         f"(B=1, same weights), {dt:.1f} s"}
        log(f"[bench] CPU oracle: {dt:.1f} s, {cpu['value']} TFLOP/s on {threads} threads")

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
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
