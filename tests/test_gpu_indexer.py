"""The Gated DSA indexer's projections on the GPU (K3.1 Gated DSA blog, eqs. (2)-(4) and the
LayerNorm paragraph after eq. (3)) against the oracle, through mla_index_projections, which runs
the launches of a decode / prefill step:
* q^I = reshape(c^Q W_q^I^T) in fp32 (c^Q the normalised query latent, fed as a bf16 hi + lo pair)
  and a = x W_a^I^T within the score rule, and well inside the top-k rule's 1e-4;
* k^I = LayerNorm(x W_k^I^T) * gain + bias computed in fp64, rounded once to bf16: bit-exact.
The token counts cover the decode GEMM (M <= 32), the mid-size GEMM (M <= 128) and the large-M DMA
GEMM with its ragged last tile, and the fp64 key kernel's split-K at each."""
import numpy as np
import pytest
import torch

import oracle as O
from gated_mla_kv_amd.layer import LayerBuffers, bf16_bits
from gpu_helpers import check_scores, dev_bf16, f64, i32, to_np
from workloads import K3_SMALL_TOPK, make_index_prefix, make_latent_prefix, make_layer_weights, make_tokens

pytestmark = pytest.mark.gpu
gm = pytest.importorskip("gated_mla_kv_amd")


def _layer(d, seed):
    lw = make_layer_weights(d, seed=seed, dist="k3", perturb_norms=True)
    return {k: f64(v) for k, v in lw.w.items()}, LayerBuffers(d, lw.w)


def _projections(L, d, x_bits):
    M = x_bits.shape[0]
    qi = torch.empty((M, d.n_idx_heads, d.d_idx), dtype=torch.float32, device="cuda")
    a = torch.empty((M, d.n_idx_heads), dtype=torch.float32, device="cuda")
    ki = torch.empty((M, d.d_idx), dtype=torch.bfloat16, device="cuda")
    ws = L.workspace(M, 1, 1, gm.PATH_SPARSE)
    gm.mla_index_projections(L.dims, L.cw, dev_bf16(x_bits), M, qi, a, ki, ws)
    torch.cuda.synchronize()
    return qi, a, ki


@pytest.mark.parametrize("M", [4, 64, 300])
def test_index_projections_against_oracle(M):
    d = K3_SMALL_TOPK
    print(f"index projections M={M}", flush=True)
    w, L = _layer(d, 96)
    x = make_tokens(d, 1, M, seed=96)[0]
    qi, a, ki = _projections(L, d, x)
    cq, _, _ = O.query_path(f64(x), w, d)
    q_ref, k_ref, a_ref = O.index_projections(f64(x), cq, w, d)
    check_scores(to_np(qi), q_ref, "q^I")
    check_scores(to_np(a), a_ref, "a")
    q_err = np.max(np.abs(to_np(qi) - q_ref)) / np.sqrt(np.mean(q_ref ** 2))
    a_err = np.max(np.abs(to_np(a) - a_ref)) / np.sqrt(np.mean(a_ref ** 2))
    print(f"max |dq^I| = {q_err:.2e} x rms, max |da| = {a_err:.2e} x rms")
    assert q_err < 1e-4 and a_err < 1e-4
    # the index cache type's one rounding of the fp64 LayerNorm output: equal bit for bit
    np.testing.assert_array_equal(f64(bf16_bits(ki)), O.round_to_bf16(k_ref))


def test_index_projections_are_what_the_decode_step_uses():
    """A sparse decode step appends exactly the stage's k^I, and its selection equals
    dsa_index_topk run on the stage's q^I and a over the same cache."""
    d = K3_SMALL_TOPK
    _, L = _layer(d, 97)
    B, T = 3, 200
    cache = L.new_cache(B, T + 1, expanded=False, index=True)
    cache.latent[:, :T] = dev_bf16(make_latent_prefix(d, B, T, seed=97))
    cache.idx[:, :T] = dev_bf16(make_index_prefix(d, B, T, seed=97))
    x = make_tokens(d, B, 1, seed=97, step=0)[:, 0]
    qi, a, ki = _projections(L, d, x)
    sel = torch.empty((B, d.topk), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B,), dtype=torch.int32, device="cuda")
    L.decode(cache, dev_bf16(x), i32([T] * B), T + 1, path=gm.PATH_SPARSE, sel_idx=sel, sel_cnt=cnt)
    torch.cuda.synchronize()
    assert torch.equal(cache.idx[:, T], ki)
    sel2 = torch.empty_like(sel)
    cnt2 = torch.empty_like(cnt)
    ws = L.workspace(B, 1, T + 1, gm.PATH_SPARSE)
    gm.dsa_index_topk(L.dims, qi, a, cache.idx, T + 1, i32([T + 1] * B), T + 1, B, sel2, cnt2, None, ws)
    torch.cuda.synchronize()
    assert torch.equal(sel, sel2) and torch.equal(cnt, cnt2)
