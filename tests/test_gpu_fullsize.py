"""Parity at the full workload sizes, in the launch configurations bench.py times, on outputs
the oracle computes one by one (sampled rows, heads and sequences):

* K3 prefill, B=1, T=4096: the attention kernel at sampled (head, row) pairs, and the whole
  mla_prefill on the rows t <= 300 (causality: row t depends on tokens 0..t only);
* batched decode, B=32, cache T=8192 (8,193 visible): absorbed attention per sampled sequence,
  expanded-cache attention per sampled (sequence, head), and whole mla_decode steps;
* long-context decode, B=4, cache T=131072: absorbed attention (split-K + merge) per sequence;
* Gated DSA decode, B=8, cache T=65536: index scores, top-2048 (boundary rule), sparse attention,
  and the whole sparse mla_decode step for sampled sequences;
* Gated DSA prefill, B=1, T=4096, top-2048: sampled rows past 2048 (where the selection drops
  positions) against the oracle's DSA steps over the first 2,100 tokens;
* FP8 caches (656-byte latent rows, 132-byte index keys) written by kv_append: absorbed decode
  at B=32, T=8192, and the DSA index scores, top-2048 and sparse attention at B=8, T=65536.
Large inputs are drawn on the device (workloads.device_normal_bf16); the oracle gets the rows
copied back."""
import numpy as np
import pytest
import torch

import gated_mla_kv_amd as gm
import oracle as O
from gated_mla_kv_amd.layer import LayerBuffers, bf16_bits, bf16_tensor
from gpu_helpers import check_rows, check_scores, check_selection, dev_bf16, oracle_row_for_selection, to_np
from workloads import (K3, bf16_bits_to_f32, device_normal_bf16, device_normal_f32, make_layer_weights, make_tokens,
                       normal_bf16)

pytestmark = pytest.mark.gpu

D = K3                      # the K3.1 layer (dense Gated MLA plus the DSA indexer)
DD = K3.replace(n_idx_heads=0)
H = D.n_heads


def f64t(t):
    """bf16 tensor (device) -> float64 numpy."""
    return bf16_bits_to_f32(bf16_bits(t)).astype(np.float64)


@pytest.fixture(scope="module")
def k3_weights():
    lw = make_layer_weights(D, seed=5)
    w64 = {k: bf16_bits_to_f32(v).astype(np.float64) for k, v in lw.w.items()}
    return lw, w64


def test_prefill_attention_T4096_sampled():
    T = 4096
    print("prefill attention B=1 T=4096", flush=True)
    q = device_normal_bf16((1, T, H, D.d_qk), 0.8, 1, 1)
    K = device_normal_bf16((1, H, T, D.d_qk), 0.8, 1, 2)
    V = device_normal_bf16((1, H, T, D.d_v), 1.0, 1, 3)
    g = torch.randn((1, T, H * D.d_v), generator=torch.Generator(device="cuda").manual_seed(4), device="cuda")
    u = torch.empty((1, T, H * D.d_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, H, T), dtype=torch.float32, device="cuda")
    cache = gm.MlaCache(None, K.data_ptr(), V.data_ptr(), None, 1, T)
    start = torch.zeros(1, dtype=torch.int32, device="cuda")
    gm.mla_prefill_attention(gm.make_dims(DD), q, cache, start, T, 1, T, g, u, gm.OUT_BF16, lse)
    torch.cuda.synchronize()
    scale = O.softmax_scale(DD)
    gn = g.cpu().numpy().astype(np.float64)
    for h in (0, 47, 95):
        Kh, Vh = f64t(K[0, h]), f64t(V[0, h])
        for t in (0, 1, 255, 256, 1000, 2047, 4095):
            qv = f64t(q[0, t, h])
            z, l_ref = O.attention_expanded(qv[None, None, None], Kh[None, None, :t + 1], Vh[None, None, :t + 1],
                                            scale, t)
            u_ref = z[0, 0, 0] * O.sigmoid(gn[0, t, h * D.d_v:(h + 1) * D.d_v])
            check_rows(to_np(u[0, t, h * D.d_v:(h + 1) * D.d_v]), u_ref, f"u h={h} t={t}", bf16_out=True)
            check_scores(np.array([to_np(lse[0, h, t:t + 1])[0]]), l_ref[0, 0], f"lse h={h} t={t}")


def test_prefill_layer_T4096_first_rows(k3_weights):
    lw, w64 = k3_weights
    T, R = 4096, 301
    print("mla_prefill B=1 T=4096 (rows < 301 checked)", flush=True)
    L = LayerBuffers(DD, lw.w)
    x_bits = make_tokens(DD, 1, T, seed=6)
    cache = L.new_cache(1, T, expanded=True)
    y = L.prefill(cache, dev_bf16(x_bits), torch.zeros(1, dtype=torch.int32, device="cuda"), T)
    torch.cuda.synchronize()
    y_ref, _ = O.layer_forward(bf16_bits_to_f32(x_bits[:, :R]).astype(np.float64), w64, O.Cache(DD, 1), DD)
    rows = [0, 3, 255, 256, 300]
    check_rows(to_np(y[0, rows]), y_ref[0, rows], "prefill y rows", bf16_out=True)


def test_dsa_prefill_T4096_selecting_rows(k3_weights):
    """mla_prefill_sparse at B=1, T=4096, top-2048: rows 2048.. are the first whose visible
    length exceeds k, so their selection drops positions. Sampled rows there are compared with
    the oracle's DSA steps (eqs. (5)-(6), (9) over S_t) computed from the first 2,100 tokens:
    the row-blocked scorer's index scores, the selection (the oracle's own except swaps across
    its k-th score within 1e-4), the output rows, and the appended index keys bit for bit."""
    lw, w64 = k3_weights
    T, R = 4096, 2100
    rows = [2047, 2048, 2060, 2099]
    print("mla_prefill_sparse B=1 T=4096 (sampled rows >= 2047)", flush=True)
    L = LayerBuffers(D, lw.w)
    x_bits = make_tokens(D, 1, T, seed=7)
    cache = L.new_cache(1, T, expanded=False, index=True)
    sel = torch.empty((1, T, D.topk), dtype=torch.int32, device="cuda")
    cnt = torch.empty((1, T), dtype=torch.int32, device="cuda")
    scores = torch.empty((1, T, T), dtype=torch.float32, device="cuda")
    y = L.prefill_sparse(cache, dev_bf16(x_bits), torch.zeros(1, dtype=torch.int32, device="cuda"), T,
                         out_dtype=gm.OUT_F32, sel_idx=sel, sel_cnt=cnt, scores=scores)
    torch.cuda.synchronize()
    sel_h, cnt_h, y_h = sel.cpu().numpy()[0], cnt.cpu().numpy()[0], to_np(y[0])
    sc_h = scores[0, rows].cpu().numpy().astype(np.float64)
    # the oracle's caches and per-token quantities for the first R tokens (the same steps as
    # O.dsa_prefill, evaluated only at the sampled rows)
    x = bf16_bits_to_f32(x_bits[:, :R]).astype(np.float64)
    cq, q_nope, q_shared = O.query_path(x, w64, D)
    c, r = O.kv_down_path(x, w64, D)
    qi, ki, a = O.index_projections(x, cq, w64, D)
    oc = O.Cache(D, 1, expanded=False)
    oc.append(c, r, idx_k=ki)
    np.testing.assert_array_equal(f64t(cache.idx[0, :R]), oc.idx[0])
    qt = O.absorbed_query(q_nope, q_shared, w64, D)
    for n, i in enumerate(rows):
        t = i + 1
        I = O.index_scores(qi[0, i], a[0, i], oc.idx[0], t)
        check_scores(sc_h[n, :t], I, f"dsa prefill scores row {i}")
        k = min(D.topk, t)
        assert cnt_h[i] == k
        got = sel_h[i, :k]
        np.testing.assert_array_equal(got, O.select_topk(sc_h[n, :t], k))  # exact on the GPU's scores
        S = O.select_topk(I, k)
        if not check_selection(got, I, k, f"dsa prefill row {i}"):
            S = got
        y_ref = oracle_row_for_selection(D, w64, x[0, i], qt[0, i], oc.latent[0], S)
        check_rows(y_h[i], y_ref, f"dsa prefill y row {i}")


def test_absorbed_decode_B32_T8192():
    B, nvis = 32, 8193
    print("absorbed decode B=32 n_vis=8193", flush=True)
    lat = device_normal_bf16((B, nvis, D.d_latent), 1.0, 2, 1)
    qt = device_normal_bf16((B, H, D.d_latent), 0.05, 2, 2)
    dims = gm.make_dims(DD)
    cache = gm.MlaCache(lat.data_ptr(), None, None, None, B, nvis)
    n = torch.full((B,), nvis, dtype=torch.int32, device="cuda")
    o = torch.empty((B, H, D.kv_lora), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(gm.workspace_bytes(dims, B, 1, nvis, gm.PATH_ABSORBED), dtype=torch.uint8, device="cuda")
    gm.mla_decode_attention(dims, qt, cache, n, nvis, B, o, lse, 0, ws)
    torch.cuda.synchronize()
    for b in (0, 13, 31):
        o_ref, l_ref = O.attention_absorbed(f64t(qt[b])[None, None], f64t(lat[b])[None], O.softmax_scale(DD),
                                            nvis - 1, DD)
        check_rows(to_np(o[b]), o_ref[0, 0], f"absorbed o b={b}")
        check_scores(to_np(lse[b]), l_ref[0, :, 0], f"absorbed lse b={b}")


def test_expanded_decode_B32_T8192():
    B, nvis = 32, 8193
    print("expanded decode B=32 n_vis=8193 (16 GB cache)", flush=True)
    K = device_normal_bf16((B, H, nvis, D.d_qk), 0.8, 3, 1)
    V = device_normal_bf16((B, H, nvis, D.d_v), 1.0, 3, 2)
    q = device_normal_bf16((B, H, D.d_qk), 0.8, 3, 3)
    cache = gm.MlaCache(None, K.data_ptr(), V.data_ptr(), None, B, nvis)
    n = torch.full((B,), nvis, dtype=torch.int32, device="cuda")
    z = torch.empty((B, H, D.d_v), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    gm.mla_expanded_attention(gm.make_dims(DD), q, cache, n, nvis, B, z, lse)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (17, 42), (31, 95)):
        z_ref, l_ref = O.attention_expanded(f64t(q[b, h])[None, None, None], f64t(K[b, h])[None, None],
                                            f64t(V[b, h])[None, None], O.softmax_scale(DD), nvis - 1)
        check_rows(to_np(z[b, h]), z_ref[0, 0, 0], f"expanded z b={b} h={h}")
        check_scores(np.array([to_np(lse[b, h:h + 1])[0]]), l_ref[0, 0], f"expanded lse b={b} h={h}")
    del K, V
    torch.cuda.empty_cache()


def test_long_context_decode_B4_T131072():
    B, nvis = 4, 131073
    print("absorbed decode B=4 n_vis=131073", flush=True)
    lat = device_normal_bf16((B, nvis, D.d_latent), 1.0, 4, 1)
    qt = device_normal_bf16((B, H, D.d_latent), 0.05, 4, 2)
    dims = gm.make_dims(DD)
    cache = gm.MlaCache(lat.data_ptr(), None, None, None, B, nvis)
    n = torch.full((B,), nvis, dtype=torch.int32, device="cuda")
    o = torch.empty((B, H, D.kv_lora), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(gm.workspace_bytes(dims, B, 1, nvis, gm.PATH_ABSORBED), dtype=torch.uint8, device="cuda")
    gm.mla_decode_attention(dims, qt, cache, n, nvis, B, o, lse, 0, ws)
    torch.cuda.synchronize()
    for b in (0, 3):
        o_ref, l_ref = O.attention_absorbed(f64t(qt[b])[None, None], f64t(lat[b])[None], O.softmax_scale(DD),
                                            nvis - 1, DD)
        check_rows(to_np(o[b]), o_ref[0, 0], f"long-context o b={b}")
        check_scores(to_np(lse[b]), l_ref[0, :, 0], f"long-context lse b={b}")


def test_dsa_index_topk_sparse_B8_T65536():
    B, nvis = 8, 65537
    print("DSA index + top-2048 + sparse attention B=8 n_vis=65537", flush=True)
    dims = gm.make_dims(D)
    lat = device_normal_bf16((B, nvis, D.d_latent), 1.0, 5, 1)
    idx = device_normal_bf16((B, nvis, D.d_idx), 1.0, 5, 2)
    qi = device_normal_f32((B, D.n_idx_heads, D.d_idx), 0.5, 5, 3)
    wi = normal_bf16((B, D.n_idx_heads), 1.0, 5, 4)
    wi_d = torch.tensor(bf16_bits_to_f32(wi), device="cuda")
    qt = device_normal_bf16((B, H, D.d_latent), 0.05, 5, 5)
    n = torch.full((B,), nvis, dtype=torch.int32, device="cuda")
    sel = torch.empty((B, D.topk), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B,), dtype=torch.int32, device="cuda")
    scores = torch.empty((B, nvis), dtype=torch.float32, device="cuda")
    ws = torch.empty(gm.workspace_bytes(dims, B, 1, nvis, gm.PATH_SPARSE), dtype=torch.uint8, device="cuda")
    gm.dsa_index_topk(dims, qi, wi_d, idx, nvis, n, nvis, B, sel, cnt, scores, ws)
    cache = gm.MlaCache(lat.data_ptr(), None, None, idx.data_ptr(), B, nvis)
    o = torch.empty((B, H, D.kv_lora), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    gm.mla_sparse_attention(dims, qt, cache, sel, cnt, B, o, lse, 0, ws)
    torch.cuda.synchronize()
    sel_h, cnt_h, sc_h = sel.cpu().numpy(), cnt.cpu().numpy(), scores.cpu().numpy().astype(np.float64)
    for b in (0, 7):
        ref = O.index_scores(to_np(qi[b]), bf16_bits_to_f32(wi[b]).astype(np.float64), f64t(idx[b]), nvis)
        check_scores(sc_h[b], ref, f"index scores b={b}")
        assert cnt_h[b] == D.topk
        got = sel_h[b]
        np.testing.assert_array_equal(got, O.select_topk(sc_h[b], D.topk))  # exact on the GPU's scores
        check_selection(got, ref, D.topk, f"b={b}")
        o_ref, l_ref = O.attention_absorbed_subset(f64t(qt[b]), f64t(lat[b]), got, O.softmax_scale(D), D)
        check_rows(to_np(o[b]), o_ref, f"sparse o b={b}")
        check_scores(to_np(lse[b]), l_ref, f"sparse lse b={b}")


@pytest.mark.parametrize("path", [gm.PATH_ABSORBED, gm.PATH_SPARSE])
def test_decode_step_full_size(k3_weights, path):
    lw, w64 = k3_weights
    sparse = path == gm.PATH_SPARSE
    d = D if sparse else DD
    B, Tc = (8, 65536) if sparse else (32, 8192)
    print(f"mla_decode path={path} B={B} T={Tc}", flush=True)
    L = LayerBuffers(d, lw.w)
    cache = L.new_cache(B, Tc + 1, expanded=False, index=sparse)
    cache.latent[:, :Tc] = device_normal_bf16((B, Tc, d.d_latent), 1.0, 6, 1)
    if sparse:
        cache.idx[:, :Tc] = device_normal_bf16((B, Tc, d.d_idx), 1.0, 6, 2)
    x_bits = make_tokens(d, B, 1, seed=6, step=0)[:, 0]
    seq = torch.full((B,), Tc, dtype=torch.int32, device="cuda")
    sel = torch.empty((B, d.topk), dtype=torch.int32, device="cuda") if sparse else None
    cnt = torch.empty((B,), dtype=torch.int32, device="cuda") if sparse else None
    y = L.decode(cache, dev_bf16(x_bits), seq, Tc + 1, path=path, out_dtype=gm.OUT_F32, sel_idx=sel, sel_cnt=cnt)
    torch.cuda.synchronize()
    for b in (0, B - 1):
        oc = O.Cache(d, 1, expanded=False)
        oc.set_prefix(f64t(cache.latent[b:b + 1, :Tc]), f64t(cache.idx[b:b + 1, :Tc]) if sparse else None)
        xb = bf16_bits_to_f32(x_bits[b:b + 1]).astype(np.float64)
        if sparse:
            y_ref, ex = O.dsa_decode_step(xb, w64, oc, d)
            got = sel.cpu().numpy()[b]
            assert cnt.cpu().numpy()[b] == d.topk
            y_row = y_ref[0]
            if not check_selection(got, ex["scores"][0], d.topk, f"sparse decode b={b}"):
                # a legal boundary swap: the oracle's layer output over the set the GPU selected
                y_row = oracle_row_for_selection(d, w64, xb[0], ex["q_tilde"][0], oc.latent[0], got)
            check_rows(to_np(y[b]), y_row, f"sparse decode y b={b}")
            np.testing.assert_array_equal(f64t(cache.idx[b, Tc]), oc.idx[0, Tc])
        else:
            y_ref, _ = O.layer_forward(xb[:, None], w64, oc, d, form="absorbed")
            check_rows(to_np(y[b]), y_ref[0, 0], f"absorbed decode y b={b}")


def _fp8_cache_from(lat, idx=None):
    """FP8 caches quantized by kv_append from device bf16 rows (all positions of every sequence)."""
    from gated_mla_kv_amd.layer import CacheBuffers
    B, nvis = lat.shape[:2]
    cache = CacheBuffers(D, B, nvis, expanded=False, index=idx is not None, fp8_latent=True,
                         fp8_index=idx is not None)
    gm.kv_append(gm.make_dims(D), cache.c, torch.zeros(B, dtype=torch.int32, device="cuda"), nvis, B, nvis,
                 lat[..., :D.kv_lora].contiguous(), lat[..., D.kv_lora:].contiguous(), None, None, idx)
    return cache


def test_absorbed_decode_fp8_B32_T8192():
    B, nvis = 32, 8193
    print("FP8-cache absorbed decode B=32 n_vis=8193", flush=True)
    lat = device_normal_bf16((B, nvis, D.d_latent), 1.0, 8, 1)
    qt = device_normal_bf16((B, H, D.d_latent), 0.05, 8, 2)
    dims = gm.make_dims(DD)
    cache = _fp8_cache_from(lat)
    n = torch.full((B,), nvis, dtype=torch.int32, device="cuda")
    o = torch.empty((B, H, D.kv_lora), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(gm.workspace_bytes(dims, B, 1, nvis, gm.PATH_ABSORBED), dtype=torch.uint8, device="cuda")
    gm.mla_decode_attention(dims, qt, cache.c, n, nvis, B, o, lse, 0, ws)
    torch.cuda.synchronize()
    for b in (0, 13, 31):
        oc = O.Cache(DD, 1, expanded=False, fp8_latent=True)
        oc.set_prefix(f64t(lat[b])[None])
        o_ref, l_ref = O.attention_absorbed(f64t(qt[b])[None, None], oc.latent, O.softmax_scale(DD), nvis - 1, DD)
        check_rows(to_np(o[b]), o_ref[0, 0], f"fp8 absorbed o b={b}")
        check_scores(to_np(lse[b]), l_ref[0, :, 0], f"fp8 absorbed lse b={b}")


def test_dsa_fp8_B8_T65536():
    B, nvis = 8, 65537
    print("FP8-cache DSA index + top-2048 + sparse attention B=8 n_vis=65537", flush=True)
    dims = gm.make_dims(D)
    lat = device_normal_bf16((B, nvis, D.d_latent), 1.0, 9, 1)
    idx = device_normal_bf16((B, nvis, D.d_idx), 1.0, 9, 2)
    qi = device_normal_f32((B, D.n_idx_heads, D.d_idx), 0.5, 9, 3)
    wi = normal_bf16((B, D.n_idx_heads), 1.0, 9, 4)
    wi_d = torch.tensor(bf16_bits_to_f32(wi), device="cuda")
    qt = device_normal_bf16((B, H, D.d_latent), 0.05, 9, 5)
    cache = _fp8_cache_from(lat, idx)
    n = torch.full((B,), nvis, dtype=torch.int32, device="cuda")
    sel = torch.empty((B, D.topk), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B,), dtype=torch.int32, device="cuda")
    scores = torch.empty((B, nvis), dtype=torch.float32, device="cuda")
    ws = torch.empty(gm.workspace_bytes(dims, B, 1, nvis, gm.PATH_SPARSE), dtype=torch.uint8, device="cuda")
    gm.dsa_index_topk_fp8(dims, qi, wi_d, cache.idx_codes, cache.idx_scales, nvis, n, nvis, B, sel, cnt, scores, ws)
    o = torch.empty((B, H, D.kv_lora), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    gm.mla_sparse_attention(dims, qt, cache.c, sel, cnt, B, o, lse, 0, ws)
    torch.cuda.synchronize()
    sel_h, cnt_h, sc_h = sel.cpu().numpy(), cnt.cpu().numpy(), scores.cpu().numpy().astype(np.float64)
    for b in (0, 7):
        oc = O.Cache(D, 1, expanded=False, fp8_latent=True, fp8_index=True)
        oc.set_prefix(f64t(lat[b])[None], f64t(idx[b])[None])
        ref = O.index_scores(to_np(qi[b]), bf16_bits_to_f32(wi[b]).astype(np.float64), oc.idx[0], nvis)
        check_scores(sc_h[b], ref, f"fp8 index scores b={b}")
        assert cnt_h[b] == D.topk
        got = sel_h[b]
        np.testing.assert_array_equal(got, O.select_topk(sc_h[b], D.topk))
        check_selection(got, ref, D.topk, f"fp8 b={b}")
        o_ref, l_ref = O.attention_absorbed_subset(f64t(qt[b]), oc.latent[0], got, O.softmax_scale(D), D)
        check_rows(to_np(o[b]), o_ref, f"fp8 sparse o b={b}")
        check_scores(to_np(lse[b]), l_ref, f"fp8 sparse lse b={b}")


def test_paged_decode_B32_T8192_equals_contiguous():
    """The bench's paged layout (64-position pages shuffled over the pool) at full size: the
    absorbed decode over it equals the contiguous cache's bit for bit, and the contiguous
    result is the one checked against the oracle above."""
    from gated_mla_kv_amd.layer import CacheBuffers
    B, nvis, page = 32, 8193, 64
    print("paged decode B=32 n_vis=8193", flush=True)
    lat = device_normal_bf16((B, nvis, D.d_latent), 1.0, 10, 1)
    qt = device_normal_bf16((B, H, D.d_latent), 0.05, 10, 2)
    dims = gm.make_dims(DD)
    nb = -(-nvis // page)
    table = torch.randperm(B * nb, generator=torch.Generator().manual_seed(10)).view(B, nb).to(torch.int32)
    paged = CacheBuffers(DD, B, nb * page, expanded=False, page_size=page, n_pages=B * nb, block_table=table)
    gm.kv_append(dims, paged.c, torch.zeros(B, dtype=torch.int32, device="cuda"), nvis, B, nvis,
                 lat[..., :D.kv_lora].contiguous(), lat[..., D.kv_lora:].contiguous())
    flat = gm.MlaCache(lat.data_ptr(), None, None, None, B, nvis)
    n = torch.full((B,), nvis, dtype=torch.int32, device="cuda")
    ws = torch.empty(gm.workspace_bytes(dims, B, 1, nvis, gm.PATH_ABSORBED), dtype=torch.uint8, device="cuda")
    outs = []
    for c in (paged.c, flat):
        o = torch.empty((B, H, D.kv_lora), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
        gm.mla_decode_attention(dims, qt, c, n, nvis, B, o, lse, 0, ws)
        torch.cuda.synchronize()
        outs.append((o, lse))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
