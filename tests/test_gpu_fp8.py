"""FP8 caches on the GPU against the oracle (oracle/fp8.py, the K3.1 Gated DSA blog's cache
section): kv_append's codes, scales and shared keys bit-exact; attention, index scores and whole
decode / DSA steps over FP8 caches within the bf16 paths' tolerances. Both sides read a latent
value back as bf16(fp32(decode(code) * scale)), and an index key as decode(code) * scale."""
import numpy as np
import pytest
import torch

import oracle as O
from oracle import fp8 as F
from gpu_helpers import (check_rows, check_scores, check_selection, dev_bf16, dev_f32, f64, i32,
                         oracle_row_for_selection, rand_bf16, rand_f32, to_np)
from workloads import (K3, K3_SMALL_TOPK, bf16_bits, make_index_prefix, make_latent_prefix, make_layer_weights,
                       make_tokens)

pytestmark = pytest.mark.gpu
gm = pytest.importorskip("gated_mla_kv_amd")


def _sync():
    torch.cuda.synchronize()


def _fp8_cache(d, lat_bits, idx_bits=None, T_cap=None, fill=None):
    """An FP8 cache written by the library's kv_append from bf16 rows c ‖ r (and index keys);
    positions past the rows keep the fill byte."""
    from gated_mla_kv_amd.layer import CacheBuffers
    B, T = lat_bits.shape[:2]
    T_cap = T_cap or T
    cache = CacheBuffers(d, B, T_cap, expanded=False, index=idx_bits is not None, fp8_latent=True,
                         fp8_index=idx_bits is not None)
    if fill is not None:
        cache.latent.fill_(fill)
        if cache.idx is not None:
            cache.idx.fill_(fill)
    if T:
        gm.kv_append(gm.make_dims(d), cache.c, i32([0] * B), T, B, T, dev_bf16(lat_bits[..., :d.kv_lora]),
                     dev_bf16(lat_bits[..., d.kv_lora:]), None, None,
                     dev_bf16(idx_bits) if idx_bits is not None else None)
    return cache


def test_kv_append_fp8_bit_exact():
    d = K3
    B, T, T_cap = 3, 6, 20
    pos = np.array([0, 9, 14], np.int32)             # the last sequence ends exactly at T_cap
    c = rand_bf16((B, T, d.kv_lora), 100)
    r = rand_bf16((B, T, d.d_shared), 101)
    ik = rand_bf16((B, T, d.d_idx), 102)
    # special blocks: all zeros (scale 0, signed zero codes), tiny values (subnormal codes),
    # scale exactly 1 (max 448) with E4M3 midpoints (ties to even)
    c[0, 0, 0:128] = bf16_bits(np.zeros(128, np.float32))
    c[0, 0, 5] = bf16_bits(np.array([-0.0], np.float32))[0]
    c[0, 1, 128:256] = bf16_bits((np.random.default_rng(103).standard_normal(128) * 1e-5).astype(np.float32))
    c[0, 1, 130] = bf16_bits(np.array([0.5], np.float32))[0]  # large next to tiny: tiny ones code as subnormals
    mids = np.array([1.0625, 1.1875, 2.125, 17.0, 19.0, 0.0146484375, -1.0625, 448.0], np.float32)
    c[1, 2, 256:384] = bf16_bits(np.resize(mids, 128))
    ik[2, 3] = bf16_bits(np.zeros(128, np.float32))
    from gated_mla_kv_amd.layer import CacheBuffers
    cache = CacheBuffers(d, B, T_cap, expanded=False, index=True, fp8_latent=True, fp8_index=True)
    cache.latent.fill_(0xA5)
    cache.idx.fill_(0xA5)
    gm.kv_append(gm.make_dims(d), cache.c, i32(pos), T_cap, B, T, dev_bf16(c), dev_bf16(r), None, None, dev_bf16(ik))
    _sync()
    lat = cache.latent.cpu().numpy()
    codes = cache.idx_codes.cpu().numpy()
    scales = cache.idx_scales.cpu().numpy()
    for b in range(B):
        sl = slice(pos[b], pos[b] + T)
        lc, ls = F.quantize_latent(f64(c[b]), d)
        np.testing.assert_array_equal(lat[b, sl, :512], lc)
        np.testing.assert_array_equal(lat[b, sl, 512:528].copy().view(np.float32), ls)
        np.testing.assert_array_equal(lat[b, sl, 528:].copy().view(np.uint16), r[b])
        kc, ks = F.quantize_index_keys(f64(ik[b]))
        np.testing.assert_array_equal(codes[b, sl], kc)
        np.testing.assert_array_equal(scales[b, sl], ks[:, 0])
        # positions outside the appended range are untouched
        outside = np.ones(T_cap, bool)
        outside[sl] = False
        assert (lat[b, outside] == 0xA5).all() and (codes[b, outside] == 0xA5).all()
    assert (lat[0, 0, 0:128] == np.where(np.arange(128) == 5, 0x80, 0)).all()


@pytest.mark.parametrize("n_vis,splits", [([1, 33, 300, 777], 0), ([1, 33, 300, 777], 5), ([4097, 64], 0)])
def test_decode_attention_fp8(n_vis, splits):
    d = K3
    print(f"decode_attention fp8 n_vis={n_vis} splits={splits}", flush=True)
    B, H = len(n_vis), d.n_heads
    T_cap = max(n_vis) + 5
    qt = rand_bf16((B, H, d.d_latent), 110, std=0.05)
    lat = rand_bf16((B, T_cap, d.d_latent), 111)
    cache = _fp8_cache(d, lat)
    dims_c = gm.make_dims(d)
    o = torch.empty((B, H, d.kv_lora), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(gm.workspace_bytes(dims_c, B, 1, max(n_vis), gm.PATH_ABSORBED, splits), dtype=torch.uint8,
                     device="cuda")
    gm.mla_decode_attention(dims_c, dev_bf16(qt), cache.c, i32(n_vis), max(n_vis), B, o, lse, splits, ws)
    _sync()
    oc = O.Cache(d, B, expanded=False, fp8_latent=True)
    oc.set_prefix(f64(lat))
    for b in range(B):
        n = n_vis[b]
        o_ref, lse_ref = O.attention_absorbed(f64(qt[b:b + 1])[:, None], oc.latent[b:b + 1, :n],
                                              O.softmax_scale(d), n - 1, d)
        check_rows(to_np(o[b]), o_ref[0, 0], f"fp8 absorbed o b={b}")
        check_scores(to_np(lse[b]), lse_ref[0, :, 0], f"fp8 absorbed lse b={b}")


@pytest.mark.parametrize("with_lse", [True, False])
def test_sparse_attention_fp8(with_lse):
    """Gathered rows; without lse and with one split the kernel writes the output itself."""
    d = K3_SMALL_TOPK
    B, H, T_cap = 3, d.n_heads, 500
    rng = np.random.default_rng(120)
    cnts = [1, 40, 64]
    sel = np.full((B, d.topk), -1, np.int32)
    for b, c in enumerate(cnts):
        sel[b, :c] = np.sort(rng.choice(T_cap, size=c, replace=False))
    qt = rand_bf16((B, H, d.d_latent), 121, std=0.05)
    lat = rand_bf16((B, T_cap, d.d_latent), 122)
    cache = _fp8_cache(d, lat)
    dims_c = gm.make_dims(d)
    o = torch.empty((B, H, d.kv_lora), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda") if with_lse else None
    ws = torch.empty(gm.workspace_bytes(dims_c, B, 1, d.topk, gm.PATH_SPARSE), dtype=torch.uint8, device="cuda")
    gm.mla_sparse_attention(dims_c, dev_bf16(qt), cache.c, i32(sel), i32(cnts), B, o, lse, 0 if with_lse else 1, ws)
    _sync()
    oc = O.Cache(d, B, expanded=False, fp8_latent=True)
    oc.set_prefix(f64(lat))
    for b in range(B):
        o_ref, lse_ref = O.attention_absorbed_subset(f64(qt[b]), oc.latent[b], sel[b, :cnts[b]], O.softmax_scale(d), d)
        check_rows(to_np(o[b]), o_ref, f"fp8 sparse o b={b}")
        if with_lse:
            check_scores(to_np(lse[b]), lse_ref, f"fp8 sparse lse b={b}")


@pytest.mark.parametrize("topk,t_vis", [(64, [10, 64, 65, 1500]), (2048, [5000, 2049])])
def test_index_scores_fp8(topk, t_vis):
    d = K3.replace(topk=topk)
    B = len(t_vis)
    T_cap = max(t_vis) + 7
    rng = np.random.default_rng(130)
    qi = rand_f32((B, d.n_idx_heads, d.d_idx), 131, std=0.1)
    a = rng.standard_normal((B, d.n_idx_heads)).astype(np.float32)
    codes = rng.integers(0, 256, (B, T_cap, d.d_idx)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] ^= 1                  # no NaN codes
    scales = (np.abs(rng.standard_normal((B, T_cap))) / 448).astype(np.float32)
    scales[0, 3] = 0.0
    dims_c = gm.make_dims(d)
    out_idx = torch.empty((B, topk), dtype=torch.int32, device="cuda")
    out_cnt = torch.empty((B,), dtype=torch.int32, device="cuda")
    sc = torch.full((B, T_cap), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(gm.workspace_bytes(dims_c, B, 1, T_cap, gm.PATH_SPARSE), dtype=torch.uint8, device="cuda")
    gm.dsa_index_topk_fp8(dims_c, dev_f32(qi), dev_f32(a), torch.from_numpy(codes).cuda(),
                          torch.from_numpy(scales).cuda(), T_cap, i32(t_vis), max(t_vis), B, out_idx, out_cnt, sc, ws)
    _sync()
    sel, cnt, sc_gpu = out_idx.cpu().numpy(), out_cnt.cpu().numpy(), sc.cpu().numpy()
    keys = F.dequantize_index_keys(codes, scales[..., None])
    for b in range(B):
        t = t_vis[b]
        ref = O.index_scores(qi[b].astype(np.float64), a[b].astype(np.float64), keys[b], t)
        check_scores(sc_gpu[b, :t], ref, f"fp8 index scores b={b}")
        k = min(topk, t)
        assert cnt[b] == k and (sel[b, k:] == -1).all()
        np.testing.assert_array_equal(sel[b, :k], O.select_topk(sc_gpu[b, :t].astype(np.float64), topk))
        check_selection(sel[b, :k], ref, k, f"fp8 b={b}")


def _layer(d, seed):
    from gated_mla_kv_amd.layer import LayerBuffers
    lw = make_layer_weights(d, seed=seed, dist="k3", perturb_norms=True)
    return {k: f64(v) for k, v in lw.w.items()}, LayerBuffers(d, lw.w)


def test_absorbed_decode_step_fp8():
    """mla_decode (absorbed) over an FP8 latent cache: the new token is quantized by kv_append."""
    d = K3
    w, L = _layer(d, 140)
    B, T = 2, 300
    lat = make_latent_prefix(d, B, T, seed=140)
    cache = _fp8_cache(d, lat, T_cap=T + 2)
    x = make_tokens(d, B, 1, seed=140, step=0)[:, 0]
    y = L.decode(cache, dev_bf16(x), i32([T] * B), T + 1, path=gm.PATH_ABSORBED, out_dtype=gm.OUT_F32)
    _sync()
    oc = O.Cache(d, B, expanded=False, fp8_latent=True)
    oc.set_prefix(f64(lat))
    y_ref, _ = O.layer_forward(f64(x)[:, None], w, oc, d, form="absorbed")
    check_rows(to_np(y), y_ref[:, 0], "fp8 absorbed decode y")


@pytest.mark.parametrize("fp8_index", [True, False])
def test_dsa_decode_step_fp8(fp8_index):
    d = K3_SMALL_TOPK
    w, L = _layer(d, 150)
    B, T = 2, 300
    lat = make_latent_prefix(d, B, T, seed=150)
    idx = make_index_prefix(d, B, T, seed=150)
    from gated_mla_kv_amd.layer import CacheBuffers
    cache = CacheBuffers(d, B, T + 4, expanded=False, index=True, fp8_latent=True, fp8_index=fp8_index)
    gm.kv_append(gm.make_dims(d), cache.c, i32([0] * B), T, B, T, dev_bf16(lat[..., :d.kv_lora]),
                 dev_bf16(lat[..., d.kv_lora:]), None, None, dev_bf16(idx))
    x = make_tokens(d, B, 1, seed=150, step=0)[:, 0]
    sel = torch.empty((B, d.topk), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B,), dtype=torch.int32, device="cuda")
    y = L.decode(cache, dev_bf16(x), i32([T] * B), T + 1, path=gm.PATH_SPARSE, out_dtype=gm.OUT_F32,
                 sel_idx=sel, sel_cnt=cnt)
    _sync()
    oc = O.Cache(d, B, expanded=False, fp8_latent=True, fp8_index=fp8_index)
    oc.set_prefix(f64(lat), f64(idx))
    y_ref, ex = O.dsa_decode_step(f64(x), w, oc, d)
    sel_np = sel.cpu().numpy()
    y_cmp = y_ref.copy()
    for b in range(B):
        got = sel_np[b]
        if not check_selection(got, ex["scores"][b], d.topk, f"fp8 dsa decode b={b}"):
            # a legal boundary swap: the oracle's output for the GPU's set
            y_cmp[b] = oracle_row_for_selection(d, w, f64(x[b]), ex["q_tilde"][b], oc.latent[b], got)
    check_rows(to_np(y), y_cmp, "fp8 dsa decode y")
    # the appended index key: the fp64 LayerNorm output rounded to bf16, then quantized to the
    # cache format, equal to the oracle's (codes and scale) bit for bit
    if fp8_index:
        np.testing.assert_array_equal(cache.idx_codes[:, T].cpu().numpy(), oc.idx_codes[:, T])
        np.testing.assert_array_equal(cache.idx_scales[:, T].cpu().numpy(), oc.idx_scales[:, T, 0])


def test_dsa_sparse_prefill_fp8():
    """mla_prefill_sparse over FP8 caches: the new rows are quantized first, then every token
    scores and attends over the read-back values."""
    d = K3_SMALL_TOPK
    w, L = _layer(d, 160)
    B, P, T = 1, 70, 60
    lat = make_latent_prefix(d, B, P, seed=160)
    idx = make_index_prefix(d, B, P, seed=160)
    from gated_mla_kv_amd.layer import CacheBuffers
    cache = CacheBuffers(d, B, P + T + 2, expanded=False, index=True, fp8_latent=True, fp8_index=True)
    gm.kv_append(gm.make_dims(d), cache.c, i32([0] * B), P, B, P, dev_bf16(lat[..., :d.kv_lora]),
                 dev_bf16(lat[..., d.kv_lora:]), None, None, dev_bf16(idx))
    x = make_tokens(d, B, T, seed=160)
    sel = torch.empty((B, T, d.topk), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, T), dtype=torch.int32, device="cuda")
    y = L.prefill_sparse(cache, dev_bf16(x), i32([P]), P + T, out_dtype=gm.OUT_F32, sel_idx=sel, sel_cnt=cnt)
    _sync()
    oc = O.Cache(d, B, expanded=False, fp8_latent=True, fp8_index=True)
    oc.set_prefix(f64(lat), f64(idx))
    y_ref, ex = O.dsa_prefill(f64(x), w, oc, d)
    sel_np, y_np = sel.cpu().numpy(), to_np(y)
    y_cmp = y_ref[0].copy()
    n_selecting = 0
    for i in range(T):
        t = P + i + 1
        k = min(d.topk, t)
        got = sel_np[0, i, :k]
        if k < t:
            n_selecting += 1
            I = O.index_scores(ex["q_idx"][0, i], ex["a"][0, i], oc.idx[0], t)
            if not check_selection(got, I, k, f"fp8 dsa prefill row {i}"):
                y_cmp[i] = oracle_row_for_selection(d, w, f64(x[0, i]), ex["q_tilde"][0, i], oc.latent[0], got)
        else:
            np.testing.assert_array_equal(got, np.arange(t))
    check_rows(y_np[0], y_cmp, "fp8 dsa prefill y")
    assert n_selecting > 0
    # the appended index keys equal the oracle's codes and scales bit for bit
    np.testing.assert_array_equal(cache.idx_codes[0, P:P + T].cpu().numpy(), oc.idx_codes[0, P:P + T])
    np.testing.assert_array_equal(cache.idx_scales[0, P:P + T].cpu().numpy(), oc.idx_scales[0, P:P + T, 0])
