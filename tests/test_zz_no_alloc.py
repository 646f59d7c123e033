"""mla_decode_noalloc, the decode step whose workspace is the library's static device buffer,
against mla_decode with a caller-owned workspace: two calls in a row on one GPU, the second with
a smaller input. Each runs the same kernels with the same workspace layout at another address, so
the outputs, selections and cache appends equal the existing entry point's bit for bit (within
the parity tolerance a fortiori); the buffer keeps the first call's contents when the second runs.
A request larger than the buffer is refused before anything runs."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_helpers import dev_bf16, i32
from workloads import K3, K3_SMALL_TOPK, make_index_prefix, make_latent_prefix, make_layer_weights, make_tokens

gm = pytest.importorskip("gated_mla_kv_amd")


def _pair(d, seed, B, T, path):
    """The same decode step on two identical caches: mla_decode, then mla_decode_noalloc."""
    from gated_mla_kv_amd.layer import LayerBuffers
    print(f"noalloc decode path={path} B={B} T={T}", flush=True)
    lw = make_layer_weights(d, seed=seed, dist="k3", perturb_norms=True)
    L = LayerBuffers(d, lw.w)
    sparse = path == gm.PATH_SPARSE
    lat = dev_bf16(make_latent_prefix(d, B, T, seed=seed))
    idx = dev_bf16(make_index_prefix(d, B, T, seed=seed)) if sparse else None
    x = dev_bf16(make_tokens(d, B, 1, seed=seed, step=0)[:, 0])
    seq = i32([T] * B)
    res = []
    for noalloc in (False, True):
        c = L.new_cache(B, T + 1, expanded=False, index=sparse)
        c.latent[:, :T] = lat
        if sparse:
            c.idx[:, :T] = idx
        y = torch.empty((B, d.hidden), dtype=torch.float32, device="cuda")
        sel = torch.full((B, d.topk), -7, dtype=torch.int32, device="cuda") if sparse else None
        cnt = torch.full((B,), -7, dtype=torch.int32, device="cuda") if sparse else None
        if noalloc:
            gm.mla_decode_noalloc(L.dims, L.cw, c.c, seq, T + 1, x, B, path, y, gm.OUT_F32, sel, cnt)
        else:
            ws = L.workspace(B, 1, T + 1, path)
            gm.mla_decode(L.dims, L.cw, c.c, seq, T + 1, x, B, path, y, gm.OUT_F32, sel, cnt, 0, ws)
        torch.cuda.synchronize()
        res.append((y, sel, cnt, c))
    (y0, s0, n0, c0), (y1, s1, n1, c1) = res
    assert torch.isfinite(y1).all()
    assert torch.equal(y0, y1), f"y differs: max {float((y0 - y1).abs().max()):.3e}"
    assert torch.equal(c0.latent, c1.latent)
    if sparse:
        assert torch.equal(s0, s1) and torch.equal(n0, n1)
        assert torch.equal(c0.idx, c1.idx)


@pytest.mark.gpu
def test_noalloc_decode_matches_decode_twice():
    # largest first (DSA path with rows past 4096 positions: index scores, the chunked top-k with
    # its histograms, candidate lists and chunk counts, sparse attention), then smaller calls over
    # the same buffer (DSA with one-workgroup top-k rows, then the absorbed path)
    _pair(K3, 212, 2, 9000, gm.PATH_SPARSE)
    _pair(K3_SMALL_TOPK, 210, 6, 700, gm.PATH_SPARSE)
    _pair(K3.replace(n_idx_heads=0), 211, 2, 300, gm.PATH_ABSORBED)


def test_noalloc_refuses_more_than_its_buffer():
    """B = 128 sequences at 4,097 visible positions need about 89 MiB, more than the 64 MiB
    buffer: refused with MLA_ERR_WORKSPACE before any device call (runs without a GPU)."""
    d = gm.make_dims(K3.replace(n_idx_heads=0))
    B, n = 128, 4097
    assert gm.workspace_bytes(d, B, 1, n, gm.PATH_ABSORBED) > gm.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x1000)
    w = gm.MlaWeights(*([0x1000] * 13))
    c = gm.MlaCache(0x1000, None, None, None, B, n)
    rc = gm.lib().mla_decode_noalloc(ctypes.byref(d), ctypes.byref(w), ctypes.byref(c), fake, n, fake,
                                     B, gm.PATH_ABSORBED, 0, None, None, fake, gm.OUT_BF16, None)
    assert rc == -5  # MLA_ERR_WORKSPACE
