"""Kernel-boundary parity on the GPU: each stage entry point of the C ABI against the oracle,
with identical bf16 inputs on both sides (tolerances in gpu_helpers)."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_helpers import check_rows, check_scores, check_selection, dev_bf16, dev_f32, f64, i32, rand_bf16, rand_f32, to_np
from workloads import K3, K3_SMALL_TOPK, TINY, bf16_bits_to_f32

pytestmark = pytest.mark.gpu

gm = pytest.importorskip("gated_mla_kv_amd")


def _sync():
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------------------------
# Projections and norms
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(1, 14400, 7168), (7, 300, 1536), (32, 7168, 12288), (33, 200, 256),
                                   (64, 2112, 512), (300, 1000, 64), (513, 2112, 7168), (256, 24576, 32),
                                   (1000, 2120, 1536), (768, 520, 128),
                                   # decode kernel (operand tiles copied into a three-slot LDS ring): two,
                                   # six and ten 128-wide k chunks (fewer chunks than slots, and ring wraps)
                                   (5, 640, 256), (17, 1000, 768), (32, 2056, 1280)])
def test_gemm(M, N, K):
    print(f"gemm M={M} N={N} K={K}", flush=True)
    a = rand_bf16((M, K), 1)
    w = rand_bf16((N, K), 2, std=K ** -0.5)
    ref = O.linear(f64(a), f64(w))
    out32 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    out16 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    da, dw = dev_bf16(a), dev_bf16(w)
    gm.mla_gemm(da, K, dw, M, N, K, out32, N, gm.OUT_F32)
    gm.mla_gemm(da, K, dw, M, N, K, out16, N, gm.OUT_BF16)
    _sync()
    check_rows(to_np(out32), ref, "gemm f32", tol=1e-4)
    check_rows(to_np(out16), ref, "gemm bf16", bf16_out=True)


@pytest.mark.parametrize("N", [1536, 512, 128, 64, 32])
def test_rmsnorm_and_layernorm(N):
    M = 37
    rng = np.random.default_rng(N)
    x = (rng.standard_normal((M, N)) * 2.5 + 0.3).astype(np.float32)
    g = rand_bf16((N,), 3, std=0.1)
    g = (bf16_bits_to_f32(g) + 1.0).astype(np.float32)
    from workloads import bf16_bits
    gb = bf16_bits(g)
    bb = rand_bf16((N,), 4, std=0.1)
    dx = torch.tensor(x, device="cuda")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    gm.mla_rmsnorm(dx, N, dev_bf16(gb), M, N, 1e-6, out, N)
    _sync()
    check_rows(to_np(out), O.rms_norm(x.astype(np.float64), f64(gb), 1e-6), "rmsnorm", bf16_out=True)
    gm.mla_layernorm(dx, N, dev_bf16(gb), dev_bf16(bb), M, N, 1e-6, out, N)
    _sync()
    check_rows(to_np(out), O.layer_norm(x.astype(np.float64), f64(gb), f64(bb), 1e-6), "layernorm", bf16_out=True)


# ---------------------------------------------------------------------------------------------
# Cache append (bit-exact)
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dims,with_idx", [(TINY, False), (K3, True)])
def test_kv_append_bit_exact(dims, with_idx):
    d = dims
    B, T, T_cap = 3, 5, 24
    pos = np.array([0, 7, 19], np.int32)     # the last sequence ends exactly at T_cap
    H = d.n_heads
    c = rand_bf16((B, T, d.kv_lora), 10)
    r = rand_bf16((B, T, d.d_shared), 11)
    kn = rand_bf16((B, T, H, d.d_nope), 12)
    v = rand_bf16((B, T, H, d.d_v), 13)
    ik = rand_bf16((B, T, d.d_idx), 14) if with_idx else None
    dims_c = gm.make_dims(d)
    sentinel = np.uint16(0x7F7F)
    lat = torch.full((B, T_cap, d.d_latent), 0, dtype=torch.int16, device="cuda").fill_(int(sentinel))
    K = torch.zeros((B, H, T_cap, d.d_qk), dtype=torch.int16, device="cuda").fill_(int(sentinel))
    V = torch.zeros((B, H, T_cap, d.d_v), dtype=torch.int16, device="cuda").fill_(int(sentinel))
    I = torch.zeros((B, T_cap, max(d.d_idx, 8)), dtype=torch.int16, device="cuda").fill_(int(sentinel))
    cache = gm.MlaCache(lat.data_ptr(), K.data_ptr(), V.data_ptr(), I.data_ptr() if with_idx else None, B, T_cap)
    gm.kv_append(dims_c, cache, i32(pos), T_cap, B, T, dev_bf16(c), dev_bf16(r), dev_bf16(kn), dev_bf16(v),
                 dev_bf16(ik) if with_idx else None)
    _sync()
    # expected cache from the oracle's append of the same rows (stored values are already bf16)
    exp_lat = np.full((B, T_cap, d.d_latent), sentinel, np.uint16)
    exp_K = np.full((B, H, T_cap, d.d_qk), sentinel, np.uint16)
    exp_V = np.full((B, H, T_cap, d.d_v), sentinel, np.uint16)
    from workloads import bf16_bits
    for b in range(B):
        oc = O.Cache(d, 1)
        kk = O.expand_keys(f64(kn[b:b + 1]), f64(r[b:b + 1]))
        oc.append(f64(c[b:b + 1]), f64(r[b:b + 1]), kk, f64(v[b:b + 1]).transpose(0, 2, 1, 3))
        sl = slice(pos[b], pos[b] + T)
        exp_lat[b, sl] = bf16_bits(oc.latent[0].astype(np.float32))
        exp_K[b, :, sl] = bf16_bits(oc.k[0].astype(np.float32))
        exp_V[b, :, sl] = bf16_bits(oc.v[0].astype(np.float32))
    np.testing.assert_array_equal(lat.cpu().numpy().view(np.uint16), exp_lat)
    np.testing.assert_array_equal(K.cpu().numpy().view(np.uint16), exp_K)
    np.testing.assert_array_equal(V.cpu().numpy().view(np.uint16), exp_V)
    # the shared key slice is identical across heads and equals r (shared-key-split page)
    Kn = K.cpu().numpy().view(np.uint16)
    for b in range(B):
        for h in range(H):
            np.testing.assert_array_equal(Kn[b, h, pos[b]:pos[b] + T, d.d_nope:], r[b])
    if with_idx:
        got = I.cpu().numpy().view(np.uint16)
        for b in range(B):
            np.testing.assert_array_equal(got[b, pos[b]:pos[b] + T], ik[b])
            assert (got[b, :pos[b]] == sentinel).all() and (got[b, pos[b] + T:] == sentinel).all()


# ---------------------------------------------------------------------------------------------
# Prefill attention with the gate epilogue
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dims,B,T,starts", [(K3, 1, 64, [0]), (K3, 2, 200, [0, 37]), (K3, 1, 300, [129]),
                                             (K3, 1, 1000, [300]), (K3, 2, 520, [0, 700]),
                                             (TINY, 1, 64, [0]), (TINY, 2, 70, [5, 0])])
def test_prefill_attention(dims, B, T, starts):
    d = dims
    print(f"prefill_attention H={d.n_heads} B={B} T={T} starts={starts}", flush=True)
    H = d.n_heads
    T_cap = max(starts) + T + 3
    q = rand_bf16((B, T, H, d.d_qk), 20, std=0.8)
    kc = rand_bf16((B, H, T_cap, d.d_qk), 21, std=0.8)
    vc = rand_bf16((B, H, T_cap, d.d_v), 22)
    g = np.random.default_rng(23).standard_normal((B, T, H * d.d_v)).astype(np.float32)
    gd = torch.tensor(g, device="cuda")
    K, V = dev_bf16(kc), dev_bf16(vc)
    cache = gm.MlaCache(None, K.data_ptr(), V.data_ptr(), None, B, T_cap)
    u = torch.empty((B, T, H * d.d_v), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    dims_c = gm.make_dims(d)
    gm.mla_prefill_attention(dims_c, dev_bf16(q), cache, i32(starts), max(starts) + T, B, T, gd, u,
                             gm.OUT_F32, lse)
    u16 = torch.empty((B, T, H * d.d_v), dtype=torch.bfloat16, device="cuda")
    gm.mla_prefill_attention(dims_c, dev_bf16(q), cache, i32(starts), max(starts) + T, B, T, gd, u16,
                             gm.OUT_BF16, None)
    _sync()
    scale = O.softmax_scale(d)
    for b in range(B):
        P = starts[b]
        z, lse_ref = O.attention_expanded(f64(q[b:b + 1]), f64(kc[b:b + 1, :, :P + T]), f64(vc[b:b + 1, :, :P + T]),
                                          scale, P)
        u_ref = z.reshape(1, T, H * d.d_v) * O.sigmoid(g[b:b + 1].astype(np.float64))
        check_rows(to_np(u[b:b + 1]), u_ref, f"prefill u b={b}")
        check_rows(to_np(u16[b:b + 1]), u_ref, f"prefill u bf16 b={b}", bf16_out=True)
        check_scores(to_np(lse[b]), lse_ref[0], f"prefill lse b={b}")


# ---------------------------------------------------------------------------------------------
# Decode attention: absorbed, sparse, expanded; absorption and value up-projection
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dims,n_vis,splits", [(K3, [1, 33, 300, 777], 0), (K3, [1, 33, 300, 777], 5),
                                               (K3, [4097, 64], 0), (TINY, [1, 70], 0), (TINY, [40, 9], 3)])
def test_decode_attention_absorbed(dims, n_vis, splits):
    d = dims
    print(f"decode_attention H={d.n_heads} n_vis={n_vis} splits={splits}", flush=True)
    B, H = len(n_vis), d.n_heads
    T_cap = max(n_vis) + 5
    qt = rand_bf16((B, H, d.d_latent), 30, std=0.05)
    lat = rand_bf16((B, T_cap, d.d_latent), 31)
    dims_c = gm.make_dims(d)
    L = dev_bf16(lat)
    cache = gm.MlaCache(L.data_ptr(), None, None, None, B, T_cap)
    o = torch.empty((B, H, d.kv_lora), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(gm.workspace_bytes(dims_c, B, 1, max(n_vis), gm.PATH_ABSORBED, splits), dtype=torch.uint8,
                     device="cuda")
    gm.mla_decode_attention(dims_c, dev_bf16(qt), cache, i32(n_vis), max(n_vis), B, o, lse, splits, ws)
    _sync()
    scale = O.softmax_scale(d)
    for b in range(B):
        n = n_vis[b]
        o_ref, lse_ref = O.attention_absorbed(f64(qt[b:b + 1])[:, None], f64(lat[b:b + 1, :n]), scale, n - 1, d)
        check_rows(to_np(o[b]), o_ref[0, 0], f"absorbed o b={b}")
        check_scores(to_np(lse[b]), lse_ref[0, :, 0], f"absorbed lse b={b}")


def test_sparse_attention():
    d = K3_SMALL_TOPK
    print("sparse_attention", flush=True)
    B, H, T_cap = 3, d.n_heads, 500
    rng = np.random.default_rng(40)
    cnts = [1, 40, 64]
    sel = np.full((B, d.topk), -1, np.int32)
    for b, c in enumerate(cnts):
        sel[b, :c] = np.sort(rng.choice(T_cap, size=c, replace=False))
    qt = rand_bf16((B, H, d.d_latent), 41, std=0.05)
    lat = rand_bf16((B, T_cap, d.d_latent), 42)
    dims_c = gm.make_dims(d)
    L = dev_bf16(lat)
    cache = gm.MlaCache(L.data_ptr(), None, None, None, B, T_cap)
    o = torch.empty((B, H, d.kv_lora), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(gm.workspace_bytes(dims_c, B, 1, d.topk, gm.PATH_SPARSE), dtype=torch.uint8, device="cuda")
    gm.mla_sparse_attention(dims_c, dev_bf16(qt), cache, i32(sel), i32(cnts), B, o, lse, 0, ws)
    _sync()
    for b in range(B):
        o_ref, lse_ref = O.attention_absorbed_subset(f64(qt[b]), f64(lat[b]), sel[b, :cnts[b]], O.softmax_scale(d), d)
        check_rows(to_np(o[b]), o_ref, f"sparse o b={b}")
        check_scores(to_np(lse[b]), lse_ref, f"sparse lse b={b}")


@pytest.mark.parametrize("splits", [0, 2])
def test_sparse_attention_leaves_out_positions_outside_the_cache(splits):
    """Selected entries outside [0, T_cap) (-1, T_cap, larger) among the first sel_cnt get
    probability 0: the result is the oracle's attention over the valid entries alone. A row with no
    valid entry gives o = 0 and lse = -inf; with two splits, one split of a row can be all invalid."""
    d = K3_SMALL_TOPK
    B, H, T_cap = 4, d.n_heads, 300
    rng = np.random.default_rng(43)
    sel = np.full((B, d.topk), -1, np.int32)
    cnts = [40, 64, 10, 64]
    valid = []
    for b, c in enumerate(cnts):
        v = np.sort(rng.choice(T_cap, size=c, replace=False)).astype(np.int32)
        bad = rng.random(c) < 0.3
        v[bad] = rng.choice([-1, T_cap, T_cap + 7, -1000], size=int(bad.sum()))
        if b == 2:
            v[:] = -1                       # nothing valid
        if b == 3:
            v[:32] = T_cap                  # the first split (32 entries) all invalid
        sel[b, :c] = v
        valid.append(v[(v >= 0) & (v < T_cap)])
    qt = rand_bf16((B, H, d.d_latent), 44, std=0.05)
    lat = rand_bf16((B, T_cap, d.d_latent), 45)
    dims_c = gm.make_dims(d)
    Ld = dev_bf16(lat)
    cache = gm.MlaCache(Ld.data_ptr(), None, None, None, B, T_cap)
    o = torch.full((B, H, d.kv_lora), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(gm.workspace_bytes(dims_c, B, 1, d.topk, gm.PATH_SPARSE, splits), dtype=torch.uint8,
                     device="cuda")
    gm.mla_sparse_attention(dims_c, dev_bf16(qt), cache, i32(sel), i32(cnts), B, o, lse, splits, ws)
    _sync()
    for b in range(B):
        if len(valid[b]) == 0:
            assert torch.count_nonzero(o[b]) == 0 and bool(torch.isinf(lse[b]).all()) and bool((lse[b] < 0).all())
            continue
        o_ref, lse_ref = O.attention_absorbed_subset(f64(qt[b]), f64(lat[b]), valid[b], O.softmax_scale(d), d)
        check_rows(to_np(o[b]), o_ref, f"sparse o b={b} (valid entries only)")
        check_scores(to_np(lse[b]), lse_ref, f"sparse lse b={b}")


@pytest.mark.parametrize("dims,n_vis", [(K3, [1, 300, 65]), (TINY, [1, 70])])
def test_expanded_attention(dims, n_vis):
    d = dims
    B, H = len(n_vis), d.n_heads
    T_cap = max(n_vis) + 2
    q = rand_bf16((B, H, d.d_qk), 50, std=0.8)
    kc = rand_bf16((B, H, T_cap, d.d_qk), 51, std=0.8)
    vc = rand_bf16((B, H, T_cap, d.d_v), 52)
    K, V = dev_bf16(kc), dev_bf16(vc)
    cache = gm.MlaCache(None, K.data_ptr(), V.data_ptr(), None, B, T_cap)
    z = torch.empty((B, H, d.d_v), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    gm.mla_expanded_attention(gm.make_dims(d), dev_bf16(q), cache, i32(n_vis), max(n_vis), B, z, lse)
    _sync()
    for b in range(B):
        n = n_vis[b]
        z_ref, lse_ref = O.attention_expanded(f64(q[b:b + 1])[:, None], f64(kc[b:b + 1, :, :n]), f64(vc[b:b + 1, :, :n]),
                                              O.softmax_scale(d), n - 1)
        check_rows(to_np(z[b]), z_ref[0, 0], f"expanded z b={b}")
        check_scores(to_np(lse[b]), lse_ref[0, :, 0], f"expanded lse b={b}")


@pytest.mark.parametrize("dims,B", [(K3, 5), (K3, 33), (K3, 300), (TINY, 3)])
def test_absorb_query_and_value_up(dims, B):
    d = dims
    H = d.n_heads
    from workloads import make_layer_weights
    lw = make_layer_weights(d, seed=60, dist="fan_in" if d is TINY else "k3")
    wkvb = lw.w["w_kv_b"]
    w64 = {"w_kv_b": f64(wkvb)}
    q = rand_bf16((B, H * d.d_qk), 61, std=0.8)
    qt = torch.empty((B, H, d.d_latent), dtype=torch.bfloat16, device="cuda")
    dims_c = gm.make_dims(d)
    Wd = dev_bf16(wkvb)
    gm.mla_absorb_query(dims_c, dev_bf16(q), H * d.d_qk, Wd, B, qt)
    qv = f64(q).reshape(B, H, d.d_qk)
    qt_ref = O.absorbed_query(qv[..., :d.d_nope], qv[..., d.d_nope:], w64, d)
    o = rand_bf16((B, H, d.kv_lora), 62)
    g = np.random.default_rng(63).standard_normal((B, H * d.d_v)).astype(np.float32)
    u = torch.empty((B, H * d.d_v), dtype=torch.float32, device="cuda")
    gm.mla_value_up_gate(dims_c, torch.tensor(bf16_bits_to_f32(o), device="cuda"), Wd, torch.tensor(g, device="cuda"),
                         B, u, gm.OUT_F32)
    ub = torch.empty((B, H * d.d_v), dtype=torch.bfloat16, device="cuda")  # the bf16 output's store path
    gm.mla_value_up_gate(dims_c, torch.tensor(bf16_bits_to_f32(o), device="cuda"), Wd, torch.tensor(g, device="cuda"),
                         B, ub, gm.OUT_BF16)
    _sync()
    check_rows(to_np(qt), qt_ref, "absorbed query", bf16_out=True)
    u_ref = O.value_up(f64(o), w64, d).reshape(B, H * d.d_v) * O.sigmoid(g.astype(np.float64))
    check_rows(to_np(u), u_ref, "value up + gate")
    check_rows(to_np(ub), u_ref, "value up + gate (bf16 out)", bf16_out=True)


# ---------------------------------------------------------------------------------------------
# DSA index scores and top-k
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("topk,t_vis", [(64, [10, 64, 65, 1500]), (2048, [5000, 2048, 2049]), (2048, [65537])])
def test_index_scores_and_topk(topk, t_vis):
    d = K3.replace(topk=topk)
    print(f"index_topk k={topk} t={t_vis}", flush=True)
    B = len(t_vis)
    T_cap = max(t_vis) + 7
    qi = rand_f32((B, d.n_idx_heads, d.d_idx), 70, std=0.1)    # fp32, not bf16-representable
    a = np.random.default_rng(71).standard_normal((B, d.n_idx_heads)).astype(np.float32)
    keys = rand_bf16((B, T_cap, d.d_idx), 72)
    dims_c = gm.make_dims(d)
    out_idx = torch.empty((B, topk), dtype=torch.int32, device="cuda")
    out_cnt = torch.empty((B,), dtype=torch.int32, device="cuda")
    scores = torch.full((B, T_cap), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(gm.workspace_bytes(dims_c, B, 1, T_cap, gm.PATH_SPARSE), dtype=torch.uint8, device="cuda")
    gm.dsa_index_topk(dims_c, dev_f32(qi), dev_f32(a), dev_bf16(keys), T_cap, i32(t_vis),
                      max(t_vis), B, out_idx, out_cnt, scores, ws)
    _sync()
    sel = out_idx.cpu().numpy()
    cnt = out_cnt.cpu().numpy()
    sc_gpu = scores.cpu().numpy()
    for b in range(B):
        t = t_vis[b]
        ref = O.index_scores(qi[b].astype(np.float64), a[b].astype(np.float64), f64(keys[b]), t)
        check_scores(sc_gpu[b, :t], ref, f"index scores b={b}")
        # the hi + lo query keeps the scores far inside the selection rule's 1e-4
        assert np.max(np.abs(sc_gpu[b, :t] - ref)) < 2e-5, np.max(np.abs(sc_gpu[b, :t] - ref))
        k = min(topk, t)
        assert cnt[b] == k
        assert (sel[b, k:] == -1).all()
        got = sel[b, :k]
        # exact: the oracle's selection rule applied to the GPU's own fp32 scores
        np.testing.assert_array_equal(got, O.select_topk(sc_gpu[b, :t].astype(np.float64), topk))
        # against the oracle's float64 scores: equal except swaps across the k-th score within 1e-4
        check_selection(got, ref, k, f"b={b}")


def test_topk_ties_take_lowest_positions():
    d = K3.replace(topk=16)
    B, T_cap, t = 2, 100, 90
    qi = np.zeros((B, d.n_idx_heads, d.d_idx), np.float32)     # all scores exactly zero (+0 or -0)
    a = np.random.default_rng(80).standard_normal((B, d.n_idx_heads)).astype(np.float32)
    keys = rand_bf16((B, T_cap, d.d_idx), 81)
    out_idx = torch.empty((B, 16), dtype=torch.int32, device="cuda")
    out_cnt = torch.empty((B,), dtype=torch.int32, device="cuda")
    ws = torch.empty(gm.workspace_bytes(gm.make_dims(d), B, 1, t, gm.PATH_SPARSE), dtype=torch.uint8, device="cuda")
    gm.dsa_index_topk(gm.make_dims(d), dev_f32(qi), dev_f32(a), dev_bf16(keys), T_cap,
                      i32([t, t]), t, B, out_idx, out_cnt, None, ws)
    _sync()
    np.testing.assert_array_equal(out_idx.cpu().numpy(), np.tile(np.arange(16, dtype=np.int32), (B, 1)))


@pytest.mark.parametrize("t,n_pos", [(20000, 0), (9000, 1000), (70000, 600)])
def test_topk_many_equal_scores(t, n_pos):
    """Rows where the k-th score is shared by thousands of positions: the zero score of every
    position whose index key is zero, with n_pos scattered positions scoring above it. The kept
    copies of the tie are the lowest positions (some rows straddle several 2048-position chunks;
    (20000, 0) has more tied positions than the selection keeps in LDS, which takes the one-row
    path)."""
    d = K3.replace(topk=2048)
    print(f"topk ties t={t} n_pos={n_pos}", flush=True)
    B, T_cap = 2, t + 5
    rng = np.random.default_rng(90 + n_pos)
    qi = rand_f32((B, d.n_idx_heads, d.d_idx), 91, std=0.1)
    a = np.abs(rng.standard_normal((B, d.n_idx_heads))).astype(np.float32) + 0.1  # positive weights
    keys = rand_bf16((B, T_cap, d.d_idx), 92)
    keys_z = keys.copy()
    for b in range(B):
        live = rng.choice(t, n_pos, replace=False) if n_pos else np.zeros(0, np.int64)
        mask = np.ones(T_cap, bool)
        mask[live] = False
        keys_z[b, mask] = 0  # q . 0 = 0 for every head: the score is exactly 0
    dims_c = gm.make_dims(d)
    out_idx = torch.empty((B, 2048), dtype=torch.int32, device="cuda")
    out_cnt = torch.empty((B,), dtype=torch.int32, device="cuda")
    scores = torch.full((B, T_cap), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(gm.workspace_bytes(dims_c, B, 1, T_cap, gm.PATH_SPARSE), dtype=torch.uint8, device="cuda")
    gm.dsa_index_topk(dims_c, dev_f32(qi), dev_f32(a), dev_bf16(keys_z), T_cap,
                      i32([t, t]), t, B, out_idx, out_cnt, scores, ws)
    _sync()
    sel = out_idx.cpu().numpy()
    sc_gpu = scores.cpu().numpy()
    for b in range(B):
        assert out_cnt[b].item() == 2048
        np.testing.assert_array_equal(sel[b], O.select_topk(sc_gpu[b, :t].astype(np.float64), 2048))
        n_zero_kept = int((sc_gpu[b, sel[b]] == 0).sum())
        assert n_zero_kept >= 2048 - n_pos


@pytest.mark.parametrize("B,t", [(64, 9000), (128, 20000), (1, 300000)])
def test_topk_row_counts(B, t):
    """The chunked top-k in both launch forms: few rows per call spread each row's select over
    several workgroups that each compact a few chunks (64 rows of 9,000: two chunks per
    workgroup; one row of 300,000: one chunk each), many long rows take one select workgroup per
    row and one compaction workgroup per chunk (128 rows of 20,000: ten chunks per row over two
    workgroups would be five each). Selection exact against the oracle's rule on the GPU's own
    scores; ragged lengths (every row shorter than the longest by a different amount)."""
    d = K3.replace(topk=2048)
    print(f"topk rows B={B} t={t}", flush=True)
    rng = np.random.default_rng(100 + B)
    t_vis = [t - (37 * b) % 1500 for b in range(B)]
    T_cap = t + 3
    qi = rand_f32((B, d.n_idx_heads, d.d_idx), 101, std=0.1)
    a = rng.standard_normal((B, d.n_idx_heads)).astype(np.float32)
    keys = rand_bf16((B, T_cap, d.d_idx), 102)
    dims_c = gm.make_dims(d)
    out_idx = torch.empty((B, 2048), dtype=torch.int32, device="cuda")
    out_cnt = torch.empty((B,), dtype=torch.int32, device="cuda")
    scores = torch.full((B, T_cap), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(gm.workspace_bytes(dims_c, B, 1, T_cap, gm.PATH_SPARSE), dtype=torch.uint8, device="cuda")
    gm.dsa_index_topk(dims_c, dev_f32(qi), dev_f32(a), dev_bf16(keys), T_cap, i32(t_vis),
                      max(t_vis), B, out_idx, out_cnt, scores, ws)
    _sync()
    sel = out_idx.cpu().numpy()
    cnt = out_cnt.cpu().numpy()
    sc_gpu = scores.cpu().numpy()
    for b in range(B):
        tb = t_vis[b]
        assert cnt[b] == 2048
        np.testing.assert_array_equal(sel[b], O.select_topk(sc_gpu[b, :tb].astype(np.float64), 2048),
                                      err_msg=f"row {b}")
    # the scores themselves against the oracle on a few rows
    for b in (0, B - 1):
        ref = O.index_scores(qi[b].astype(np.float64), a[b].astype(np.float64), f64(keys[b]), t_vis[b])
        assert np.max(np.abs(sc_gpu[b, :t_vis[b]] - ref)) < 2e-5


# ---------------------------------------------------------------------------------------------
# Raw logits (stage entry point)
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("form,B,Tq,Tk", [("expanded", 2, 37, 70), ("absorbed", 2, 33, 65), ("expanded", 1, 1, 1),
                                          ("absorbed", 1, 64, 32)])
def test_debug_scores_against_oracle(form, B, Tq, Tk):
    """mla_debug_scores against the oracle's logits: per-head keys (D = 192) and the shared latent
    rows of the absorbed form (D = 576), ragged tiles and a single (query, key) pair. The kernel
    multiplies bf16 values exactly and accumulates D products in fp32: each logit is within
    D * 2^-24 of the sum of the products' magnitudes (times the scale), plus the fp32 scale's rounding."""
    d = K3
    print(f"debug_scores {form} B={B} Tq={Tq} Tk={Tk}", flush=True)
    H = d.n_heads
    D = d.d_qk if form == "expanded" else d.d_latent
    Hk = H if form == "expanded" else 1
    q = rand_bf16((B, Tq, H, D), 120)
    k = rand_bf16((B, Hk, Tk, D), 121)
    logits = torch.full((B, H, Tq, Tk), float("nan"), dtype=torch.float32, device="cuda")
    gm.mla_debug_scores(gm.make_dims(d), dev_bf16(q), dev_bf16(k), Hk, B, Tq, Tk, D, logits)
    _sync()
    scale = O.softmax_scale(d)
    ref = O.attention_logits(f64(q), f64(k), scale)
    mag = O.attention_logits(np.abs(f64(q)), np.abs(f64(k)), scale)
    got = logits.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    bound = D * 2.0 ** -24 * mag + 2.0 ** -23 * np.abs(ref)
    err = np.abs(got - ref)
    assert (err <= bound).all(), float(np.max(err - bound))

