"""Determinism: every whole-path call run twice on the same inputs (with other GPU work in
between) gives bitwise identical outputs. The kernels reduce in a fixed order (split-K
partials and GEMM partials are summed in slot order, histograms count integers), so any
difference would point at a race, e.g. in LDS."""
import pytest
import torch

from gpu_helpers import dev_bf16, i32
from workloads import (K3, K3_SMALL_TOPK, make_index_prefix, make_latent_prefix, make_layer_weights,
                       make_tokens)

pytestmark = pytest.mark.gpu
gm = pytest.importorskip("gated_mla_kv_amd")


def _layer(d, seed):
    from gated_mla_kv_amd.layer import LayerBuffers
    return LayerBuffers(d, make_layer_weights(d, seed=seed, dist="k3").w)


def _twice(fn):
    a = fn()
    torch.cuda.synchronize()
    torch.randn(1 << 20, device="cuda").sum().item()  # unrelated work in between
    b = fn()
    torch.cuda.synchronize()
    return a, b


def _same(a, b, what):
    for x, y in zip(a, b):
        assert torch.equal(x, y), what


def test_prefill_is_deterministic():
    d = K3.replace(n_idx_heads=0)
    L = _layer(d, 210)
    B, T = 1, 1024
    x = dev_bf16(make_tokens(d, B, T, seed=210))

    def run():
        cache = L.new_cache(B, T)
        lse = torch.empty((B, d.n_heads, T), dtype=torch.float32, device="cuda")
        y = L.prefill(cache, x, i32([0]), T, out_dtype=gm.OUT_F32, lse=lse)
        return y, lse, cache.latent, cache.k, cache.v

    _same(*_twice(run), "prefill")


@pytest.mark.parametrize("fp8", [False, True])
def test_decode_is_deterministic(fp8):
    d = K3
    L = _layer(d, 211)
    B, T = 8, 3000
    lat = make_latent_prefix(d, B, T, seed=211)
    x = dev_bf16(make_tokens(d, B, 1, seed=211, step=0)[:, 0])

    def run():
        cache = L.new_cache(B, T + 1, expanded=False, fp8_latent=fp8)
        gm.kv_append(L.dims, cache.c, i32([0] * B), T, B, T, dev_bf16(lat[..., :d.kv_lora]),
                     dev_bf16(lat[..., d.kv_lora:]))
        y = L.decode(cache, x, i32([T] * B), T + 1, path=gm.PATH_ABSORBED, out_dtype=gm.OUT_F32)
        return y, cache.latent

    _same(*_twice(run), "decode")


def test_dsa_decode_and_prefill_are_deterministic():
    d = K3_SMALL_TOPK.replace(topk=256)
    L = _layer(d, 212)
    B, T = 4, 5000
    lat = dev_bf16(make_latent_prefix(d, B, T, seed=212))
    idx = dev_bf16(make_index_prefix(d, B, T, seed=212))
    x1 = dev_bf16(make_tokens(d, B, 1, seed=212, step=0)[:, 0])
    xs = dev_bf16(make_tokens(d, B, 300, seed=212))

    def run():
        cache = L.new_cache(B, T + 301, expanded=False, index=True)
        cache.latent[:, :T] = lat
        cache.idx[:, :T] = idx
        sel = torch.empty((B, d.topk), dtype=torch.int32, device="cuda")
        cnt = torch.empty((B,), dtype=torch.int32, device="cuda")
        y = L.decode(cache, x1, i32([T] * B), T + 1, path=gm.PATH_SPARSE, out_dtype=gm.OUT_F32, sel_idx=sel,
                     sel_cnt=cnt)
        sp = torch.empty((B, 300, d.topk), dtype=torch.int32, device="cuda")
        cp = torch.empty((B, 300), dtype=torch.int32, device="cuda")
        yp = L.prefill_sparse(cache, xs, i32([T + 1] * B), T + 301, out_dtype=gm.OUT_F32, sel_idx=sp, sel_cnt=cp)
        return y, sel, cnt, yp, sp, cp, cache.latent, cache.idx

    _same(*_twice(run), "dsa")
