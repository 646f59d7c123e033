"""Pins of the oracle against what the pages and the mathematics fix (CPU only).

Each test ties an oracle function to something other than itself: a figure printed on the
pages (tests/golden/page_figures.json), an explicit-loop brute force written separately
(tests/brute_force.py), a library routine (torch CPU float64), a closed form, or an identity
of the method (absorbed == expanded, causality, prefill == prefill + decode, gate at W_g = 0,
sort-based top-k, dense == sparse when k >= t).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle as O
from workloads import (K2_SHAPE, K3, TINY, TINY_DSA, bf16_bits, bf16_bits_to_f32, make_layer_weights,
                       make_tokens)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def _figures():
    with open(GOLDEN) as f:
        return {e["name"]: e["value"] for e in json.load(f)["figures"]}


def _weights_f64(lw):
    return {k: bf16_bits_to_f32(v).astype(np.float64) for k, v in lw.w.items()}


def _x(dims, B, T, seed=0, step=None):
    return bf16_bits_to_f32(make_tokens(dims, B, T, seed, step)).astype(np.float64)


# ---------------------------------------------------------------------------------------------
# Cache accounting printed on the pages
# ---------------------------------------------------------------------------------------------

def test_cache_sizes_match_page_figures():
    fig = _figures()
    k3 = O.cache_values_per_position(K3)
    k2 = O.cache_values_per_position(K2_SHAPE)
    assert k3["expanded"] == fig["k3_expanded_values_per_position"]
    assert k3["latent"] == fig["k3_latent_values_per_position"]
    assert k3["index"] == fig["k31_index_key_values_per_position"]
    assert k2["expanded"] == fig["k2_expanded_values_per_position"]
    assert k2["latent"] == fig["k2_latent_values_per_position"]
    # first length at which the expanded MLA cache holds more values than a KDA layer's state
    n = next(n for n in range(1, 10_000) if n * k3["expanded"] > fig["kda_state_values"])
    assert n == fig["k3_mla_exceeds_kda_from_positions"]
    gib = 2 ** 30
    layers, positions, bf16_bytes = 24, fig["max_positions"], 2
    assert layers * k3["latent"] * bf16_bytes * positions == fig["k3_mla_cache_24_layers_1M_gib"] * gib
    assert (layers * (k3["latent"] + k3["index"]) * bf16_bytes * positions
            == fig["k31_mla_plus_index_cache_24_layers_1M_gib"] * gib)
    # indexer dot products per query per visible position: 2 * heads * dims
    assert 2 * K3.n_idx_heads * K3.d_idx == fig["indexer_flops_per_query_per_position"]
    assert K3.topk == fig["dsa_topk"]
    assert round(100 * K3.topk / fig["max_positions"], 3) == fig["selected_share_at_1M_percent"]


def test_shared_key_identical_across_heads():
    """The last d_shared key features are the same r for every head (shared-key-split page)."""
    lw = make_layer_weights(TINY, seed=3, dist="fan_in")
    w = _weights_f64(lw)
    cache = O.Cache(TINY, 2)
    _, ex = O.layer_forward(_x(TINY, 2, 7, seed=3), w, cache, TINY)
    shared = cache.k[:, :, :, TINY.d_nope:]
    for h in range(TINY.n_heads):
        np.testing.assert_array_equal(shared[:, h], shared[:, 0])
    np.testing.assert_array_equal(shared[:, 0], O.round_to_bf16(ex["r"]))
    np.testing.assert_array_equal(cache.latent[..., TINY.kv_lora:], O.round_to_bf16(ex["r"]))


# ---------------------------------------------------------------------------------------------
# Elementary operations
# ---------------------------------------------------------------------------------------------

def test_round_to_bf16_agrees_with_bit_rounding():
    rng = np.random.default_rng(0)
    a = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    # exact ties: 1 + 2^-8 rounds down to 1 (even), 1 + 3*2^-8 rounds up to 1 + 2^-6
    a = np.concatenate([a, np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.0], np.float32)])
    ref = bf16_bits_to_f32(bf16_bits(a)).astype(np.float64)
    np.testing.assert_array_equal(O.round_to_bf16(a.astype(np.float64)), ref)
    assert O.round_to_bf16(1 + 2 ** -8) == 1.0
    assert O.round_to_bf16(1 + 3 * 2 ** -8) == 1 + 2 ** -6


def test_rms_norm_closed_form_and_library():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    v = rng.standard_normal((5, 64)) * 3.0
    g = 1 + 0.1 * rng.standard_normal(64)
    out = O.rms_norm(v, np.ones(64), 1e-6)
    ms = np.mean(v * v, axis=-1)
    np.testing.assert_allclose(np.mean(out * out, axis=-1), ms / (ms + 1e-6), rtol=1e-13)
    lib = torch.nn.functional.rms_norm(torch.from_numpy(v), (64,), torch.from_numpy(g), eps=1e-6)
    np.testing.assert_allclose(O.rms_norm(v, g, 1e-6), lib.numpy(), rtol=1e-13, atol=1e-14)


def test_layer_norm_closed_form_and_library():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(2)
    v = rng.standard_normal((6, 128)) * 1.7 + 0.3
    g = 1 + 0.1 * rng.standard_normal(128)
    b = 0.1 * rng.standard_normal(128)
    plain = O.layer_norm(v, np.ones(128), np.zeros(128), 1e-6)
    np.testing.assert_allclose(np.mean(plain, -1), 0.0, atol=1e-13)
    var = np.var(v, -1)
    np.testing.assert_allclose(np.var(plain, -1), var / (var + 1e-6), rtol=1e-12)
    lib = torch.nn.functional.layer_norm(torch.from_numpy(v), (128,), torch.from_numpy(g),
                                         torch.from_numpy(b), eps=1e-6)
    np.testing.assert_allclose(O.layer_norm(v, g, b, 1e-6), lib.numpy(), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------------------------

def _brute_attention(q, k, v, scale, offset):
    """exp without max subtraction, explicit sum; q [T,dqk], k [N,dqk], v [N,dv]."""
    out = np.zeros((q.shape[0], v.shape[1]))
    for i in range(q.shape[0]):
        w = [math.exp(scale * float(np.dot(q[i], k[j]))) for j in range(offset + i + 1)]
        den = sum(w)
        for j in range(len(w)):
            out[i] += (w[j] / den) * v[j]
    return out


def test_attention_matches_brute_force_and_library():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(4)
    B, H, T, P, dqk, dv = 2, 3, 6, 5, 24, 16
    q = rng.standard_normal((B, T, H, dqk))
    k = rng.standard_normal((B, H, P + T, dqk))
    v = rng.standard_normal((B, H, P + T, dv))
    scale = dqk ** -0.5
    z, lse = O.attention_expanded(q, k, v, scale, P)
    for b in range(B):
        for h in range(H):
            ref = _brute_attention(q[b, :, h], k[b, h], v[b, h], scale, P)
            np.testing.assert_allclose(z[b, :, h], ref, rtol=1e-12, atol=1e-13)
            for i in range(T):
                s = [scale * float(np.dot(q[b, i, h], k[b, h, j])) for j in range(P + i + 1)]
                assert abs(lse[b, h, i] - math.log(sum(math.exp(x) for x in s))) < 1e-12
    # offset 0: the library's top-left-aligned causal mask is the same mask
    z0, _ = O.attention_expanded(q, k[:, :, :T], v[:, :, :T], scale, 0)
    lib = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.transpose(0, 2, 1, 3).copy()), torch.from_numpy(k[:, :, :T].copy()),
        torch.from_numpy(v[:, :, :T].copy()), is_causal=True, scale=scale)
    np.testing.assert_allclose(z0, lib.numpy().transpose(0, 2, 1, 3), rtol=1e-12, atol=1e-13)


def test_attention_logits_brute_force_one_hot_and_lse():
    """The raw logits: scalar loops with per-head and shared keys (non-square B, T, H, N so that a
    transposed operand or a wrong head index shows), one-hot features, and the expanded
    attention's softmax denominators as the logsumexp of the masked logits."""
    from brute_force import brute_attention_logits
    rng = np.random.default_rng(41)
    B, T, H, N, D = 2, 3, 4, 5, 24
    q = rng.standard_normal((B, T, H, D))
    k = rng.standard_normal((B, H, N, D))
    kl = rng.standard_normal((B, 1, N, D))
    scale = D ** -0.5
    for kk in (k, kl):
        s = O.attention_logits(q, kk, scale)
        assert s.shape == (B, H, T, N)
        np.testing.assert_allclose(s, np.array(brute_attention_logits(q.tolist(), kk.tolist(), scale)),
                                   rtol=1e-12, atol=1e-13)
    qo = np.zeros((1, 1, 1, D))
    qo[0, 0, 0, 5] = 1.0
    ko = np.zeros((1, 1, 2, D))
    ko[0, 0, 0, 5] = 1.0
    ko[0, 0, 1, 6] = 1.0
    np.testing.assert_array_equal(O.attention_logits(qo, ko, 0.25)[0, 0, 0], [0.25, 0.0])
    P = 2
    v = rng.standard_normal((B, H, N, 16))
    _, lse = O.attention_expanded(q, k, v, scale, P)
    s = O.attention_logits(q, k, scale)
    for i in range(T):
        np.testing.assert_allclose(lse[:, :, i], np.log(np.exp(s[:, :, i, :P + i + 1]).sum(-1)), rtol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(5)
    k = rng.standard_normal((1, 2, 9, 24))
    v = rng.standard_normal((1, 2, 9, 16))
    # one visible position: the output is v_0 exactly
    z, _ = O.attention_expanded(rng.standard_normal((1, 1, 2, 24)), k[:, :, :1], v[:, :, :1], 0.2, 0)
    np.testing.assert_array_equal(z[0, 0], v[0, :, 0])
    # q = 0: uniform weights, the mean of the visible values
    z, _ = O.attention_expanded(np.zeros((1, 3, 2, 24)), k, v, 0.2, 6)
    for i in range(3):
        np.testing.assert_allclose(z[0, i], v[0, :, :7 + i].mean(axis=1), rtol=1e-13)


def test_causality_future_positions_do_not_matter():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 8, 2, 24))
    k = rng.standard_normal((1, 2, 8, 24))
    v = rng.standard_normal((1, 2, 8, 16))
    z, _ = O.attention_expanded(q, k, v, 0.2, 0)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 5:] += 10.0
    v2[:, :, 5:] -= 7.0
    z2, _ = O.attention_expanded(q, k2, v2, 0.2, 0)
    np.testing.assert_array_equal(z[:, :5], z2[:, :5])
    assert not np.allclose(z[:, 5:], z2[:, 5:])


# ---------------------------------------------------------------------------------------------
# The whole layer
# ---------------------------------------------------------------------------------------------

def test_layer_matches_explicit_loop_brute_force():
    from brute_force import brute_layer
    d = TINY
    lw = make_layer_weights(d, seed=7, dist="fan_in", perturb_norms=True)
    w = _weights_f64(lw)
    x = _x(d, 1, 5, seed=7)
    y, _ = O.layer_forward(x, w, O.Cache(d, 1, store_bf16=False), d)
    ref = brute_layer(x[0].tolist(), {k: v.tolist() for k, v in w.items()}, d)
    np.testing.assert_allclose(y[0], np.array(ref), rtol=1e-10, atol=1e-12)


def test_absorbed_equals_expanded():
    """Latent absorption computes exactly eq. (9) (K3.1 blog, the note after eq. (10))."""
    d = TINY
    w = _weights_f64(make_layer_weights(d, seed=8, dist="fan_in", perturb_norms=True))
    x = _x(d, 2, 9, seed=8)
    y_e, ex_e = O.layer_forward(x, w, O.Cache(d, 2, store_bf16=False), d, form="expanded")
    y_a, ex_a = O.layer_forward(x, w, O.Cache(d, 2, store_bf16=False), d, form="absorbed")
    np.testing.assert_allclose(y_a, y_e, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(ex_a["lse"], ex_e["lse"], rtol=1e-12)
    # at K3 dims too (a short prefill)
    d = K3
    w = _weights_f64(make_layer_weights(d, seed=8))
    x = _x(d, 1, 3, seed=8)
    y_e, _ = O.layer_forward(x, w, O.Cache(d, 1, store_bf16=False), d, form="expanded")
    y_a, _ = O.layer_forward(x, w, O.Cache(d, 1, store_bf16=False), d, form="absorbed")
    np.testing.assert_allclose(y_a, y_e, rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("store_bf16", [False, True])
def test_prefill_equals_prefill_then_decode(store_bf16):
    d = TINY
    w = _weights_f64(make_layer_weights(d, seed=9, dist="fan_in"))
    x = _x(d, 2, 12, seed=9)
    y_full, _ = O.layer_forward(x, w, O.Cache(d, 2, store_bf16), d)
    cache = O.Cache(d, 2, store_bf16)
    y_pre, _ = O.layer_forward(x[:, :4], w, cache, d)
    steps = [O.layer_forward(x[:, t:t + 1], w, cache, d)[0] for t in range(4, 12)]
    np.testing.assert_allclose(y_pre, y_full[:, :4], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(np.concatenate(steps, 1), y_full[:, 4:], rtol=1e-11, atol=1e-13)


def test_gate_at_zero_weights_halves_output():
    d = TINY
    w = _weights_f64(make_layer_weights(d, seed=10, dist="fan_in"))
    w["w_g"] = np.zeros_like(w["w_g"])
    x = _x(d, 1, 6, seed=10)
    y_g, ex = O.layer_forward(x, w, O.Cache(d, 1), d)
    y_u, ex_u = O.layer_forward(x, w, O.Cache(d, 1), d.replace(use_gate=False))
    np.testing.assert_array_equal(ex["u"], 0.5 * ex_u["u"])
    np.testing.assert_allclose(y_g, 0.5 * y_u, rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------------------------------------
# Gated DSA
# ---------------------------------------------------------------------------------------------

def test_index_scores_brute_force_relu_identity_and_scale_folding():
    from brute_force import brute_index_scores
    rng = np.random.default_rng(11)
    nh, di, t = 4, 16, 23
    qi = rng.standard_normal((nh, di))
    a = rng.standard_normal(nh)           # head weights may be negative (eq. (4))
    keys = rng.standard_normal((t + 5, di))
    got = O.index_scores(qi, a, keys, t)
    np.testing.assert_allclose(got, brute_index_scores(qi.tolist(), a.tolist(), keys.tolist(), t),
                               rtol=1e-12, atol=1e-14)
    assert got.shape == (t,) and (got < 0).any()
    # at K3's 32 x 128 the scale is 1/64: folding it into a is exact
    qi = rng.standard_normal((32, 128))
    a = rng.standard_normal(32)
    keys = rng.standard_normal((40, 128))
    folded = np.sum((a / 64.0)[:, None] * np.maximum(qi @ keys.T, 0.0), axis=0)
    np.testing.assert_array_equal(O.index_scores(qi, a, keys, 40), folded)


def test_index_projections_match_explicit_loops():
    """Eqs. (2)-(4) of the Gated DSA blog against scalar loops (tests/brute_force.py): q^I from
    the normalised query latent c^Q read head-major, k^I = LayerNorm(W_k^I x) * gamma + beta,
    a = W_a^I x raw; on the oracle's function and on what its decode step and prefill use.
    Gains and the bias are perturbed, and each plausible slip (q^I from the un-normalised
    latent, a transposed head reshape, RMSNorm for the LayerNorm, a dropped bias, a sigmoid on
    a) is shown to move the result, so the pin would catch it."""
    from brute_force import brute_index_projections
    d = TINY_DSA
    lw = make_layer_weights(d, seed=18, dist="fan_in", perturb_norms=True)
    w = _weights_f64(lw)
    Wl = {k: v.tolist() for k, v in w.items()}
    B, T = 2, 3
    x = _x(d, B, T, seed=18)
    cq, _, _ = O.query_path(x, w, d)
    qi, ki, a = O.index_projections(x, cq, w, d)
    assert qi.shape == (B, T, d.n_idx_heads, d.d_idx) and ki.shape == (B, T, d.d_idx)
    assert a.shape == (B, T, d.n_idx_heads)
    ref = [[brute_index_projections(x[b, t].tolist(), Wl, d) for t in range(T)] for b in range(B)]
    q_ref = np.array([[r[0] for r in row] for row in ref])
    k_ref = np.array([[r[1] for r in row] for row in ref])
    a_ref = np.array([[r[2] for r in row] for row in ref])
    np.testing.assert_allclose(qi, q_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ki, k_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(a, a_ref, rtol=1e-12, atol=1e-13)
    # what the decode step and the prefill feed the score (no rounding of the query side)
    y, ex = O.dsa_decode_step(x[:, 0], w, O.Cache(d, B, expanded=False), d)
    np.testing.assert_allclose(ex["q_idx"], q_ref[:, 0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ex["k_idx"], k_ref[:, 0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ex["a"], a_ref[:, 0], rtol=1e-12, atol=1e-13)
    _, exp_ = O.dsa_prefill(x, w, O.Cache(d, B, expanded=False), d)
    np.testing.assert_allclose(exp_["q_idx"], q_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(exp_["k_idx"], k_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(exp_["a"], a_ref, rtol=1e-12, atol=1e-13)
    # the slips the pin must catch all change the numbers
    raw = x @ w["w_q_a"].T
    slips = {
        "q from the un-normalised latent": ((raw @ w["w_idx_q"].T).reshape(qi.shape), q_ref),
        "q from x-side RMSNorm without the gain": (
            ((raw / np.sqrt(np.mean(raw ** 2, -1, keepdims=True) + d.rms_eps)) @ w["w_idx_q"].T).reshape(qi.shape),
            q_ref),
        "q reshaped feature-major": (
            (cq @ w["w_idx_q"].T).reshape(B, T, d.d_idx, d.n_idx_heads).swapaxes(-1, -2), q_ref),
        "k with RMSNorm": (O.rms_norm(x @ w["w_idx_k"].T, w["g_idx_k"], d.ln_eps) + w["b_idx_k"], k_ref),
        "k without the bias": (ki - w["b_idx_k"], k_ref),
        "a through a sigmoid": (O.sigmoid(a), a_ref),
    }
    for what, (slip, good) in slips.items():
        assert np.max(np.abs(slip - good)) > 1e-3 * np.max(np.abs(good)), what


def test_select_topk_matches_stable_sort():
    rng = np.random.default_rng(12)
    for trial in range(200):
        t = int(rng.integers(1, 40))
        k = int(rng.integers(1, 12))
        s = rng.integers(-3, 4, size=t).astype(np.float64) * 0.5   # many exact ties
        s[rng.random(t) < 0.2] = -0.0
        got = O.select_topk(s, k)
        order = sorted(range(t), key=lambda i: (-s[i], i))
        assert got.tolist() == sorted(order[:min(k, t)])
    # k >= t keeps every position (short history)
    np.testing.assert_array_equal(O.select_topk(rng.standard_normal(9), 2048), np.arange(9))


def test_sparse_with_all_positions_equals_dense():
    d = K3
    rng = np.random.default_rng(13)
    qt = rng.standard_normal((d.n_heads, d.d_latent)) * 0.05
    lat = O.round_to_bf16(rng.standard_normal((37, d.d_latent)))
    o_s, lse_s = O.attention_absorbed_subset(qt, lat, np.arange(37), O.softmax_scale(d), d)
    o_d, lse_d = O.attention_absorbed(qt[None, None], lat[None], O.softmax_scale(d), 36, d)
    np.testing.assert_allclose(o_s, o_d[0, 0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse_s, lse_d[0, :, 0], rtol=1e-13)


def test_dsa_step_with_k_at_least_t_equals_dense_decode():
    """t <= k keeps every position, so the DSA step is the dense layer's decode step."""
    d = TINY_DSA.replace(topk=64)
    w = _weights_f64(make_layer_weights(d, seed=14, dist="fan_in", perturb_norms=True))
    x = _x(d, 2, 10, seed=14)
    dense = O.Cache(d, 2)
    O.layer_forward(x[:, :9], w, dense, d)
    y_dense, _ = O.layer_forward(x[:, 9:], w, dense, d, form="absorbed")
    sparse = O.Cache(d, 2, expanded=False)
    _, ex = O.layer_forward(x[:, :9], w, O.Cache(d, 2), d)
    sparse.set_prefix(O.round_to_bf16(np.concatenate([ex["c"], ex["r"]], -1)),
                      np.zeros((2, 9, d.d_idx)))
    y_sparse, ex_s = O.dsa_decode_step(x[:, 9], w, sparse, d)
    for S in ex_s["selected"]:
        np.testing.assert_array_equal(S, np.arange(10))     # current token included (t = 10)
    np.testing.assert_allclose(y_sparse, y_dense[:, 0], rtol=1e-11, atol=1e-13)


def test_dsa_prefill_equals_successive_decode_steps():
    """DSA prefill of T tokens = T DSA decode steps, each appending its token first: token i's
    scores, selection and output only involve positions up to its own (eq. (6) at every t).
    k = 6 is below the visible length for most tokens, so the selections are real."""
    d = TINY_DSA.replace(topk=6)
    w = _weights_f64(make_layer_weights(d, seed=16, dist="fan_in", perturb_norms=True))
    x = _x(d, 2, 12, seed=16)
    a_cache = O.Cache(d, 2, expanded=False)
    O.dsa_prefill(x[:, :5], w, a_cache, d)
    b_cache = O.Cache(d, 2, expanded=False)
    b_cache.latent, b_cache.idx = a_cache.latent.copy(), a_cache.idx.copy()
    y_pre, ex = O.dsa_prefill(x[:, 5:], w, a_cache, d)
    for i in range(7):
        y_dec, ex_d = O.dsa_decode_step(x[:, 5 + i], w, b_cache, d)
        np.testing.assert_allclose(y_pre[:, i], y_dec, rtol=1e-11, atol=1e-13)
        for b in range(2):
            np.testing.assert_array_equal(ex["selected"][b][i], ex_d["selected"][b])
    assert any(len(S) == 6 and S[-1] > 6 for S in ex["selected"][0])  # some rows do select
    np.testing.assert_array_equal(a_cache.latent, b_cache.latent)
    np.testing.assert_array_equal(a_cache.idx, b_cache.idx)


def test_dsa_prefill_with_k_at_least_t_equals_dense_prefill():
    """k >= every visible length keeps every position, so DSA prefill is the dense layer."""
    d = TINY_DSA.replace(topk=64)
    w = _weights_f64(make_layer_weights(d, seed=17, dist="fan_in", perturb_norms=True))
    x = _x(d, 2, 11, seed=17)
    y_dense, _ = O.layer_forward(x, w, O.Cache(d, 2), d, form="absorbed")
    y_sparse, ex = O.dsa_prefill(x, w, O.Cache(d, 2, expanded=False), d)
    for i in range(11):
        np.testing.assert_array_equal(ex["selected"][1][i], np.arange(i + 1))
    np.testing.assert_allclose(y_sparse, y_dense, rtol=1e-11, atol=1e-13)


def test_dsa_step_selects_by_index_score():
    d = TINY_DSA
    w = _weights_f64(make_layer_weights(d, seed=15, dist="fan_in", perturb_norms=True))
    rng = np.random.default_rng(15)
    T = 30
    cache = O.Cache(d, 1, expanded=False)
    cache.set_prefix(O.round_to_bf16(rng.standard_normal((1, T, d.d_latent))),
                     O.round_to_bf16(rng.standard_normal((1, T, d.d_idx))))
    x = _x(d, 1, 1, seed=15)[:, 0]
    y, ex = O.dsa_decode_step(x, w, cache, d)
    I = ex["scores"][0]
    assert I.shape == (T + 1,)
    S = ex["selected"][0]
    assert len(S) == d.topk and np.all(np.diff(S) > 0)
    # every selected score is >= every unselected one
    mask = np.zeros(T + 1, bool)
    mask[S] = True
    assert I[mask].min() >= I[~mask].max()
    # the index key of the current token was appended before scoring
    np.testing.assert_array_equal(cache.idx[0, T], O.round_to_bf16(ex["k_idx"][0]))
    # selection decides the output: restricting to a different set changes y
    o_all, _ = O.attention_absorbed_subset(ex["q_tilde"][0], cache.latent[0], np.arange(T + 1),
                                           O.softmax_scale(d), d)
    o_sel, _ = O.attention_absorbed_subset(ex["q_tilde"][0], cache.latent[0], S, O.softmax_scale(d), d)
    np.testing.assert_allclose(O.value_up(o_sel, w, d), ex["z"][0], rtol=1e-12)
    assert not np.allclose(o_all, o_sel)
