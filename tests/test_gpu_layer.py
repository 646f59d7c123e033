"""Whole-layer parity on the GPU: mla_prefill then mla_decode against the oracle's layer on the
same seeded bf16 inputs (tolerances in gpu_helpers)."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_helpers import (check_rows, check_scores, check_selection, dev_bf16, f64, i32, oracle_row_for_selection,
                         to_np)
from gated_mla_kv_amd.layer import bf16_bits
from workloads import (K3, K3_SMALL_TOPK, TINY, make_index_prefix, make_latent_prefix, make_layer_weights,
                       make_tokens)

pytestmark = pytest.mark.gpu
gm = pytest.importorskip("gated_mla_kv_amd")


def _layer(d, seed, dist):
    from gated_mla_kv_amd.layer import LayerBuffers
    lw = make_layer_weights(d, seed=seed, dist=dist, perturb_norms=True)
    return lw, LayerBuffers(d, lw.w)


def _w64(lw):
    return {k: f64(v) for k, v in lw.w.items()}


@pytest.mark.parametrize("dims,dist,B,T,steps,path", [
    (TINY, "fan_in", 1, 64, 8, gm.PATH_ABSORBED),     # the tiny oracle-scale layer
    (TINY, "fan_in", 1, 64, 8, gm.PATH_EXPANDED),
    (K3, "k3", 2, 40, 3, gm.PATH_ABSORBED),
    (K3, "k3", 1, 150, 2, gm.PATH_EXPANDED),
])
def test_prefill_then_decode(dims, dist, B, T, steps, path):
    d = dims
    print(f"layer H={d.n_heads} B={B} T={T} steps={steps} path={path}", flush=True)
    lw, L = _layer(d, 90, dist)
    w = _w64(lw)
    T_cap = T + steps + 3
    cache = L.new_cache(B, T_cap, expanded=True)
    x = make_tokens(d, B, T, seed=90)
    y = L.prefill(cache, dev_bf16(x), i32([0] * B), T, out_dtype=gm.OUT_F32)
    oc = O.Cache(d, B)
    y_ref, _ = O.layer_forward(f64(x), w, oc, d)
    torch.cuda.synchronize()
    check_rows(to_np(y), y_ref, "prefill y")
    for s in range(steps):
        xs = make_tokens(d, B, 1, seed=90, step=s)[:, 0]
        yd = L.decode(cache, dev_bf16(xs), i32([T + s] * B), T + s + 1, path=path, out_dtype=gm.OUT_F32)
        yd_ref, _ = O.layer_forward(f64(xs)[:, None], w, oc, d, form="absorbed" if path == gm.PATH_ABSORBED
                                    else "expanded")
        torch.cuda.synchronize()
        check_rows(to_np(yd), yd_ref[:, 0], f"decode step {s} y")
    # the caches the GPU kept equal the oracle's bf16 caches
    from gated_mla_kv_amd.layer import bf16_bits
    n = T + steps
    np.testing.assert_array_equal(f64(bf16_bits(cache.latent))[:, :n].shape, oc.latent.shape)
    lat_err = np.abs(f64(bf16_bits(cache.latent))[:, :n] - oc.latent)
    # equal up to an occasional one-ulp difference where fp32 and fp64 round differently
    assert np.mean(lat_err > 0) < 0.02


def test_prefill_expanded_cache_rows():
    """At more than 128 token rows the kv up-projection writes k_nope and v straight into the
    expanded cache; every written row equals, bit for bit, the same GEMM's output for the cached
    latents (run through the stage entry point), and the shared-key part of each head's k row is the
    cached r. Rows of positions that were not written stay untouched."""
    d = K3
    lw, L = _layer(d, 92, "k3")
    B, T, T_cap = 2, 150, 200
    starts = [0, 37]
    cache = L.new_cache(B, T_cap, expanded=True)
    cache.k.fill_(7)
    cache.v.fill_(7)
    x = make_tokens(d, B, T, seed=92)
    L.prefill(cache, dev_bf16(x), i32(starts), max(starts) + T)
    torch.cuda.synchronize()
    H, dn, dv = d.n_heads, d.d_nope, d.d_v
    lat = torch.stack([cache.latent[b, starts[b]:starts[b] + T] for b in range(B)]).reshape(B * T, -1)
    c = lat[:, :d.kv_lora].contiguous()
    kvb = torch.empty((B * T, H * (dn + dv)), dtype=torch.bfloat16, device="cuda")
    gm.mla_gemm(c, d.kv_lora, L.w["w_kv_b"], B * T, H * (dn + dv), d.kv_lora, kvb, H * (dn + dv))
    torch.cuda.synchronize()
    kvb = kvb.reshape(B, T, H, dn + dv)
    for b in range(B):
        p0 = starts[b]
        k = cache.k[b, :, p0:p0 + T]  # [H, T, dn + d_shared]
        v = cache.v[b, :, p0:p0 + T]
        assert torch.equal(k[..., :dn], kvb[b, :, :, :dn].transpose(0, 1)), f"k_nope b={b}"
        assert torch.equal(v, kvb[b, :, :, dn:].transpose(0, 1)), f"v b={b}"
        r = cache.latent[b, p0:p0 + T, d.kv_lora:]
        assert torch.equal(k[..., dn:], r.unsqueeze(0).expand(H, -1, -1)), f"shared key b={b}"
        # positions before this sequence's start were not written
        assert bool((cache.k[b, :, :p0] == 7).all()) and bool((cache.v[b, :, :p0] == 7).all())


def test_prefill_bf16_output_and_chunked_start():
    """Two prefill calls (P = 0 then P = 24) equal one 40-token prefill."""
    d = K3
    lw, L = _layer(d, 91, "k3")
    w = _w64(lw)
    B, T1, T2 = 1, 24, 16
    cache = L.new_cache(B, T1 + T2)
    x = make_tokens(d, B, T1 + T2, seed=91)
    L.prefill(cache, dev_bf16(x[:, :T1]), i32([0]), T1)
    y2 = L.prefill(cache, dev_bf16(x[:, T1:]), i32([T1]), T1 + T2)
    y_ref, _ = O.layer_forward(f64(x), w, O.Cache(d, B), d)
    torch.cuda.synchronize()
    check_rows(to_np(y2), y_ref[:, T1:], "chunked prefill y (bf16)", bf16_out=True)


def test_decode_ragged_lengths():
    d = K3
    lw, L = _layer(d, 92, "k3")
    w = _w64(lw)
    lens = [3, 130, 57]
    B = len(lens)
    T_cap = max(lens) + 2
    cache = L.new_cache(B, T_cap, expanded=True)
    lat = make_latent_prefix(d, B, max(lens), seed=92)
    cache.latent[:, :max(lens)] = dev_bf16(lat)
    x = make_tokens(d, B, 1, seed=92, step=0)[:, 0]
    y = L.decode(cache, dev_bf16(x), i32(lens), max(lens) + 1, path=gm.PATH_ABSORBED, out_dtype=gm.OUT_F32)
    torch.cuda.synchronize()
    for b in range(B):
        oc = O.Cache(d, 1, expanded=False)
        oc.set_prefix(f64(lat[b:b + 1, :lens[b]]))
        yr, _ = O.layer_forward(f64(x[b:b + 1])[:, None], w, oc, d, form="absorbed")
        check_rows(to_np(y[b]), yr[0, 0], f"ragged decode b={b}")


def test_dsa_sparse_decode_step():
    d = K3_SMALL_TOPK
    lw, L = _layer(d, 93, "k3")
    w = _w64(lw)
    B, T = 2, 300
    T_cap = T + 4
    cache = L.new_cache(B, T_cap, expanded=False, index=True)
    lat = make_latent_prefix(d, B, T, seed=93)
    idx = make_index_prefix(d, B, T, seed=93)
    cache.latent[:, :T] = dev_bf16(lat)
    cache.idx[:, :T] = dev_bf16(idx)
    x = make_tokens(d, B, 1, seed=93, step=0)[:, 0]
    sel = torch.empty((B, d.topk), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B,), dtype=torch.int32, device="cuda")
    y = L.decode(cache, dev_bf16(x), i32([T] * B), T + 1, path=gm.PATH_SPARSE, out_dtype=gm.OUT_F32,
                 sel_idx=sel, sel_cnt=cnt)
    torch.cuda.synchronize()
    oc = O.Cache(d, B, expanded=False)
    oc.set_prefix(f64(lat), f64(idx))
    y_ref, ex = O.dsa_decode_step(f64(x), w, oc, d)
    sel_np = sel.cpu().numpy()
    assert (cnt.cpu().numpy() == d.topk).all()
    y_cmp = y_ref.copy()
    for b in range(B):
        got = sel_np[b]
        # the oracle's own selection on its own scores, except swaps across its k-th score
        # within 1e-4 (then the oracle's output for the GPU's set is the reference)
        if not check_selection(got, ex["scores"][b], d.topk, f"dsa decode b={b}"):
            y_cmp[b] = oracle_row_for_selection(d, w, f64(x[b]), ex["q_tilde"][b], oc.latent[b], got)
    check_rows(to_np(y), y_cmp, "dsa decode y")
    # the current token's index key was appended at position T, equal to the oracle's bf16 key
    # (its LayerNorm is computed in fp64 and rounded once) bit for bit
    np.testing.assert_array_equal(f64(bf16_bits(cache.idx[:, T])), oc.idx[:, T])


def test_dsa_sparse_prefill_equal_prefix_keys():
    """A prefix of 400 identical index keys: every row scores them equally, so each 128-position
    key block puts all its positions in one histogram bin (the largest count the row-blocked
    kernel's 8-bit counters hold), and the top-k must take the tied prefix positions lowest
    first (the tie rule the selection uses throughout): the selected prefix positions are
    exactly 0 .. m-1."""
    d = K3_SMALL_TOPK
    lw, L = _layer(d, 95, "k3")
    B, P, T = 1, 400, 8
    cache = L.new_cache(B, P + T + 3, expanded=False, index=True)
    cache.latent[0, :P] = dev_bf16(make_latent_prefix(d, B, P, seed=95)[0])
    key = make_index_prefix(d, 1, 1, seed=95)[0, 0]
    cache.idx[0, :P] = dev_bf16(np.ascontiguousarray(np.broadcast_to(key, (P, d.d_idx))))
    x = make_tokens(d, B, T, seed=95)
    sel = torch.empty((B, T, d.topk), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, T), dtype=torch.int32, device="cuda")
    y = L.prefill_sparse(cache, dev_bf16(x), i32([P]), P + T, out_dtype=gm.OUT_F32, sel_idx=sel, sel_cnt=cnt)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all())
    sel_np, cnt_np = sel.cpu().numpy(), cnt.cpu().numpy()
    for i in range(T):
        t = P + i + 1
        k = min(d.topk, t)
        assert cnt_np[0, i] == k
        got = sel_np[0, i, :k]
        assert np.all(np.diff(got) > 0) and got[-1] < t
        pre = got[got < P]
        assert np.array_equal(pre, np.arange(len(pre))), f"row {i}: tied prefix keys not taken lowest first"


@pytest.mark.parametrize("starts,T", [([100, 37], 150), ([0], 90), ([210], 160), ([5000], 16), ([5000, 4400], 12)])
def test_dsa_sparse_prefill(starts, T):
    """mla_prefill_sparse against the oracle's dsa_prefill, per sequence (ragged starts, P > 0,
    rows seeing up to three 128-position key blocks, or more than 4096 positions so that the
    top-k takes its chunked path): every row's index scores (the row-blocked scorer for a
    one-sequence call, the per-row scorer otherwise) against eq. (5) within the score rule, the
    selections equal to the oracle's except swaps across its k-th score within 1e-4 (rows with a
    swap are compared with the oracle's output for the GPU's set), the output rows within the
    tolerance, and the appended index keys equal to the oracle's bit for bit."""
    d = K3_SMALL_TOPK
    print(f"dsa prefill starts={starts} T={T} k={d.topk}", flush=True)
    lw, L = _layer(d, 94, "k3")
    w = _w64(lw)
    B, P = len(starts), max(starts)
    T_cap = P + T + 3
    cache = L.new_cache(B, T_cap, expanded=False, index=True)
    lat = make_latent_prefix(d, B, max(P, 1), seed=94)
    idx = make_index_prefix(d, B, max(P, 1), seed=94)
    for b, s in enumerate(starts):
        if s:
            cache.latent[b, :s] = dev_bf16(lat[b, :s])
            cache.idx[b, :s] = dev_bf16(idx[b, :s])
    x = make_tokens(d, B, T, seed=94)
    sel = torch.empty((B, T, d.topk), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, T), dtype=torch.int32, device="cuda")
    scores = torch.full((B, T, P + T), float("nan"), dtype=torch.float32, device="cuda")
    y = L.prefill_sparse(cache, dev_bf16(x), i32(starts), P + T, out_dtype=gm.OUT_F32, sel_idx=sel, sel_cnt=cnt,
                         scores=scores)
    torch.cuda.synchronize()
    y_np, sel_np, cnt_np, sc_np = to_np(y), sel.cpu().numpy(), cnt.cpu().numpy(), scores.cpu().numpy()
    n_selecting = n_swapped = 0
    for b, s in enumerate(starts):
        oc = O.Cache(d, 1, expanded=False)
        oc.set_prefix(f64(lat[b:b + 1, :s]), f64(idx[b:b + 1, :s]))
        y_ref, ex = O.dsa_prefill(f64(x[b:b + 1]), w, oc, d)
        y_cmp = y_ref[0].copy()
        for i in range(T):
            t = s + i + 1
            k = min(d.topk, t)
            assert cnt_np[b, i] == k
            got = sel_np[b, i, :k]
            assert (sel_np[b, i, k:] == -1).all() and np.all(np.diff(got) > 0) and got[-1] < t
            I = O.index_scores(ex["q_idx"][0, i], ex["a"][0, i], oc.idx[0], t)
            check_scores(sc_np[b, i, :t], I, f"dsa prefill scores b={b} row {i}")
            # exact on the GPU's own scores
            np.testing.assert_array_equal(got, O.select_topk(sc_np[b, i, :t].astype(np.float64), k))
            if k < t:
                n_selecting += 1
                if not check_selection(got, I, k, f"dsa prefill b={b} row {i}"):
                    n_swapped += 1
                    y_cmp[i] = oracle_row_for_selection(d, w, f64(x[b, i]), ex["q_tilde"][0, i], oc.latent[0], got)
            else:
                np.testing.assert_array_equal(got, np.arange(t))
        check_rows(y_np[b], y_cmp, f"dsa prefill y b={b}")
        # the appended index keys equal the oracle's bf16 keys bit for bit
        np.testing.assert_array_equal(f64(bf16_bits(cache.idx[b, s:s + T])), oc.idx[0, s:s + T])
    assert n_selecting > 0
    print(f"selecting rows {n_selecting}, legal boundary swaps {n_swapped}")
