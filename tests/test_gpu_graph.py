"""Whole decode steps captured in a HIP graph (torch.cuda.CUDAGraph over the library's stream
calls): the library allocates nothing and clears its counters with kernels, so a captured step
replays correctly. Every replay, with eager work and synchronizations between replays, equals
the eager step bit for bit."""
import pytest
import torch

from gpu_helpers import dev_bf16, i32
from workloads import K3_SMALL_TOPK, make_index_prefix, make_latent_prefix, make_layer_weights, make_tokens

pytestmark = pytest.mark.gpu
gm = pytest.importorskip("gated_mla_kv_amd")


@pytest.mark.parametrize("path", ["absorbed", "sparse"])
def test_decode_step_graph_replays_equal_eager(path):
    from gated_mla_kv_amd.layer import LayerBuffers
    d = K3_SMALL_TOPK
    lw = make_layer_weights(d, seed=200, dist="k3")
    L = LayerBuffers(d, lw.w)
    B, T = 4, 700
    sparse = path == "sparse"
    cache = L.new_cache(B, T + 2, expanded=False, index=True)
    cache.latent[:, :T] = dev_bf16(make_latent_prefix(d, B, T, seed=200))
    cache.idx[:, :T] = dev_bf16(make_index_prefix(d, B, T, seed=200))
    x = dev_bf16(make_tokens(d, B, 1, seed=200, step=0)[:, 0])
    seq = i32([T] * B)
    p = gm.PATH_SPARSE if sparse else gm.PATH_ABSORBED
    ws = L.workspace(B, 1, T + 1, p)
    y = torch.empty((B, d.hidden), dtype=torch.float32, device="cuda")
    sel = torch.empty((B, d.topk), dtype=torch.int32, device="cuda") if sparse else None
    cnt = torch.empty((B,), dtype=torch.int32, device="cuda") if sparse else None

    def step():
        gm.mla_decode(L.dims, L.cw, cache.c, seq, T + 1, x, B, p, y, gm.OUT_F32, sel, cnt, 0, ws)

    step()  # eager; appends the token at position T (the replays rewrite the same rows)
    torch.cuda.synchronize()
    y_eager = y.clone()
    sel_eager = sel.clone() if sparse else None
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm the capture stream
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(3):
        y.fill_(float("nan"))
        if sparse:
            sel.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {i}"
        if sparse:
            assert torch.equal(sel, sel_eager), f"replay {i} selection"
        torch.randn(1000, device="cuda").sum().item()  # eager work between replays
