"""Paged latent and index caches on the GPU: the kernels read and write pool rows through a
page table. Filled by the library's kv_append from the same rows, a paged cache holds, read
back through its table, exactly the bytes of the contiguous cache; attention, DSA decode and
DSA prefill over it give results equal bit for bit to the contiguous cache's (same arithmetic,
other addresses), and the paged results are checked against the oracle here as well: attention
outputs within the row tolerance, DSA selections equal to the oracle's except swaps across its
k-th index score within 1e-4, and the layer outputs of the DSA steps."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_helpers import (check_rows, check_scores, check_selection, dev_bf16, f64, i32, oracle_row_for_selection,
                         rand_bf16, to_np)
from workloads import K3, K3_SMALL_TOPK, make_index_prefix, make_latent_prefix, make_layer_weights, make_tokens

pytestmark = pytest.mark.gpu
gm = pytest.importorskip("gated_mla_kv_amd")


def _table(B, max_blocks, n_pages, seed):
    """Distinct pool pages for every (sequence, block), in shuffled order."""
    rng = np.random.default_rng(seed)
    return rng.permutation(n_pages)[:B * max_blocks].reshape(B, max_blocks).astype(np.int32)


def _caches(d, B, T_cap, page, spare, seed, **kw):
    from gated_mla_kv_amd.layer import CacheBuffers
    nb = T_cap // page
    table = _table(B, nb, B * nb + spare, seed)
    paged = CacheBuffers(d, B, T_cap, expanded=False, page_size=page, n_pages=B * nb + spare, block_table=table, **kw)
    flat = CacheBuffers(d, B, T_cap, expanded=False, **kw)
    return paged, flat, table


def _append(d, caches, lat, idx=None):
    B, T = lat.shape[:2]
    for c in caches:
        gm.kv_append(gm.make_dims(d), c.c, i32([0] * B), T, B, T, dev_bf16(lat[..., :d.kv_lora]),
                     dev_bf16(lat[..., d.kv_lora:]), None, None, dev_bf16(idx) if idx is not None else None)


def _through_table(pool, table, page):
    """[n_pages, page, ...] pool rows read in each sequence's logical order -> [B, T_cap, ...]."""
    B, nb = table.shape
    t = torch.as_tensor(table, device=pool.device, dtype=torch.long)
    return pool[t.reshape(-1)].reshape(B, nb * page, *pool.shape[2:])


@pytest.mark.parametrize("fp8", [False, True])
def test_paged_append_and_decode_attention(fp8):
    d = K3
    B, T_cap, page = 3, 384, 64
    n_vis = [1, 200, 333]
    print(f"paged decode fp8={fp8}", flush=True)
    paged, flat, table = _caches(d, B, T_cap, page, 5, 170, fp8_latent=fp8)
    lat = rand_bf16((B, max(n_vis), d.d_latent), 171)
    _append(d, (paged, flat), lat)
    torch.cuda.synchronize()
    # the pool read through the table holds the contiguous cache's bytes
    got = _through_table(paged.latent, table, page)
    assert torch.equal(got[:, :max(n_vis)], flat.latent[:, :max(n_vis)])
    qt = rand_bf16((B, d.n_heads, d.d_latent), 172, std=0.05)
    dims = gm.make_dims(d)
    outs = []
    for c in (paged, flat):
        o = torch.empty((B, d.n_heads, d.kv_lora), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, d.n_heads), dtype=torch.float32, device="cuda")
        ws = torch.empty(gm.workspace_bytes(dims, B, 1, max(n_vis), gm.PATH_ABSORBED, 5), dtype=torch.uint8,
                         device="cuda")
        gm.mla_decode_attention(dims, dev_bf16(qt), c.c, i32(n_vis), max(n_vis), B, o, lse, 5, ws)
        outs.append((o, lse))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    if not fp8:  # and against the oracle
        for b in range(B):
            n = n_vis[b]
            o_ref, l_ref = O.attention_absorbed(f64(qt[b:b + 1])[:, None], f64(lat[b:b + 1, :n]), O.softmax_scale(d),
                                                n - 1, d)
            check_rows(to_np(outs[0][0][b]), o_ref[0, 0], f"paged o b={b}")
            check_scores(to_np(outs[0][1][b]), l_ref[0, :, 0], f"paged lse b={b}")


@pytest.mark.parametrize("fp8", [False, True])
def test_paged_dsa_decode_step(fp8):
    """mla_decode on the sparse path: append of the new token, index scores, top-k and gathered
    attention all go through the page table."""
    from gated_mla_kv_amd.layer import LayerBuffers
    d = K3_SMALL_TOPK
    lw = make_layer_weights(d, seed=180, dist="k3", perturb_norms=True)
    L = LayerBuffers(d, lw.w)
    B, T, T_cap, page = 2, 300, 320, 32
    paged, flat, table = _caches(d, B, T_cap, page, 3, 181, index=True, fp8_latent=fp8, fp8_index=fp8)
    lat, idx = make_latent_prefix(d, B, T, seed=181), make_index_prefix(d, B, T, seed=181)
    _append(d, (paged, flat), lat, idx)
    x_bits = make_tokens(d, B, 1, seed=181, step=0)[:, 0]
    x = dev_bf16(x_bits)
    res = []
    for c in (paged, flat):
        sel = torch.empty((B, d.topk), dtype=torch.int32, device="cuda")
        cnt = torch.empty((B,), dtype=torch.int32, device="cuda")
        y = L.decode(c, x, i32([T] * B), T + 1, path=gm.PATH_SPARSE, out_dtype=gm.OUT_F32, sel_idx=sel, sel_cnt=cnt)
        res.append((y, sel, cnt))
    torch.cuda.synchronize()
    for a, b in zip(res[0], res[1]):
        assert torch.equal(a, b)
    # the new token's rows went to the right pool row
    got = _through_table(paged.latent, table, page)
    assert torch.equal(got[:, :T + 1], flat.latent[:, :T + 1])
    # the paged step against the oracle's DSA decode step over the same caches
    w = {k: f64(v) for k, v in lw.w.items()}
    oc = O.Cache(d, B, expanded=False, fp8_latent=fp8, fp8_index=fp8)
    oc.set_prefix(f64(lat), f64(idx))
    y_ref, ex = O.dsa_decode_step(f64(x_bits), w, oc, d)
    y, sel, cnt = res[0]
    sel_np = sel.cpu().numpy()
    assert (cnt.cpu().numpy() == d.topk).all()
    for b in range(B):
        y_row = y_ref[b]
        if not check_selection(sel_np[b], ex["scores"][b], d.topk, f"paged dsa decode b={b}"):
            y_row = oracle_row_for_selection(d, w, f64(x_bits[b]), ex["q_tilde"][b], oc.latent[b], sel_np[b])
        check_rows(to_np(y[b]), y_row, f"paged dsa decode y b={b}")


@pytest.mark.parametrize("B", [1, 2])
def test_paged_dsa_prefill(B):
    """B = 1 takes the row-blocked index-score kernel (rows of one sequence), B = 2 the per-row one."""
    from gated_mla_kv_amd.layer import LayerBuffers
    d = K3_SMALL_TOPK
    lw = make_layer_weights(d, seed=190, dist="k3", perturb_norms=True)
    L = LayerBuffers(d, lw.w)
    P, T, T_cap, page = 40, 300, 352, 32
    paged, flat, table = _caches(d, B, T_cap, page, 4, 191, index=True)
    lat, idx = make_latent_prefix(d, B, P, seed=191), make_index_prefix(d, B, P, seed=191)
    _append(d, (paged, flat), lat, idx)
    x_bits = make_tokens(d, B, T, seed=191)
    x = dev_bf16(x_bits)
    res = []
    for c in (paged, flat):
        sel = torch.empty((B, T, d.topk), dtype=torch.int32, device="cuda")
        cnt = torch.empty((B, T), dtype=torch.int32, device="cuda")
        y = L.prefill_sparse(c, x, i32([P] * B), P + T, out_dtype=gm.OUT_F32, sel_idx=sel, sel_cnt=cnt)
        res.append((y, sel, cnt))
    torch.cuda.synchronize()
    for a, b in zip(res[0], res[1]):
        assert torch.equal(a, b)
    # the paged prefill against the oracle's DSA prefill
    w = {k: f64(v) for k, v in lw.w.items()}
    y, sel, cnt = (t.cpu().numpy() if t.dtype != torch.float32 else to_np(t) for t in res[0])
    for b in range(B):
        oc = O.Cache(d, 1, expanded=False)
        oc.set_prefix(f64(lat[b:b + 1]), f64(idx[b:b + 1]))
        y_ref, ex = O.dsa_prefill(f64(x_bits[b:b + 1]), w, oc, d)
        y_cmp = y_ref[0].copy()
        for i in range(T):
            t = P + i + 1
            k = min(d.topk, t)
            assert cnt[b, i] == k
            I = O.index_scores(ex["q_idx"][0, i], ex["a"][0, i], oc.idx[0], t)
            if not check_selection(sel[b, i, :k], I, k, f"paged dsa prefill b={b} row {i}"):
                y_cmp[i] = oracle_row_for_selection(d, w, f64(x_bits[b, i]), ex["q_tilde"][0, i], oc.latent[0],
                                                    sel[b, i, :k])
        check_rows(y[b], y_cmp, f"paged dsa prefill y b={b}")
