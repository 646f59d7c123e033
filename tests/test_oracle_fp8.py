"""Pins of the FP8 cache oracle (oracle/fp8.py) to facts outside it: the page's byte counts
(tests/golden/page_figures.json), torch's CPU float8_e4m3fn conversions (a library routine
for the OCP E4M3 format), closed forms of the format, and error bounds of the quantizer."""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O
from oracle import fp8 as F
from workloads import K3, bf16_bits_to_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def _fig(name):
    with open(GOLDEN) as f:
        return {e["name"]: e["value"] for e in json.load(f)["figures"]}[name]


def test_byte_counts_match_page_figures():
    assert F.latent_row_bytes(K3) == _fig("fp8_main_cache_bytes_per_position")
    assert F.index_key_bytes(K3) == _fig("fp8_index_key_bytes_per_position")
    per_pos = F.latent_row_bytes(K3) + F.index_key_bytes(K3)
    assert per_pos == _fig("fp8_caches_bytes_per_position")
    assert round(24 * per_pos * 2 ** 20 / 2 ** 30, 2) == _fig("fp8_caches_24_layers_1M_gib")


def test_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.isnan(got).sum() == 2                      # S.1111.111 only
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    # closed forms of the format
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0
    assert got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9 and got[0x07] == 7 * 2.0 ** -9
    assert got[0x38] == 1.0 and got[0x39] == 1.125


def test_encode_matches_torch():
    rng = np.random.default_rng(5)
    vals = [rng.standard_normal(20000) * s for s in (1e-4, 1e-3, 1e-2, 0.1, 1, 10, 100)]
    x = np.concatenate(vals + [rng.uniform(-463.9, 463.9, 20000)]).astype(np.float32)
    # every finite code value and every midpoint between neighbours (ties to even)
    pos = F.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    edge = np.concatenate([pos, -pos, mids, -mids, [464.0, -464.0, 0.0, -0.0]]).astype(np.float32)
    x = np.concatenate([x, edge])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode(x)
    assert np.array_equal(got, ref)


def test_encode_decode_round_trip_and_saturation():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    assert np.array_equal(F.e4m3_encode(F.e4m3_decode(codes)), codes)
    # just above 448 by an fp32 rounding of the scale: saturates to 448, never NaN
    assert F.e4m3_encode(np.float32(448.00003)) == 0x7E
    assert F.e4m3_encode(np.float32(-448.00003)) == 0xFE


def test_block_quantizer_scale_and_error_bound():
    rng = np.random.default_rng(6)
    v = bf16_bits_to_f32(torch.from_numpy(rng.standard_normal((64, 512)).astype(np.float32))
                         .to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)).astype(np.float64)
    codes, scales = F.quantize_latent(v, K3)
    assert codes.shape == (64, 512) and scales.shape == (64, 4) and scales.dtype == np.float32
    vb = v.reshape(64, 4, 128)
    # the scale is the smallest power of two with max|v| <= 448 * scale
    amax = np.abs(vb).max(-1)
    m, e = np.frexp(scales.astype(np.float64))
    assert np.all(m == 0.5) and np.all(amax <= 448 * scales) and np.all(amax > 224 * scales)
    # so the block's largest element codes into [224, 448] (just above 224 rounds to 224)
    cb = codes.reshape(64, 4, 128)
    top = np.abs(vb).argmax(-1)
    top_vals = np.abs(F.e4m3_decode(np.take_along_axis(cb, top[..., None], -1)[..., 0]))
    assert np.all((top_vals >= 224) & (top_vals <= 448))
    # read-back error: half an E4M3 step (2^-4 relative; 2^-10 * scale below the normal range)
    back = F.dequantize_latent(codes, scales)
    s = np.repeat(scales.astype(np.float64), 128, -1)
    assert np.all(np.abs(back - v) <= 2.0 ** -4 * np.abs(v) + 2.0 ** -10 * s)
    # exactly representable values come back exactly
    assert np.array_equal(F.dequantize_latent(*F.quantize_latent(back, K3)), back)


def test_zero_block():
    v = np.zeros((2, 512))
    v[1, 200] = -3.0
    codes, scales = F.quantize_latent(v, K3)
    assert scales[0].tolist() == [0, 0, 0, 0] and scales[1, 1] == 2.0 ** -7   # 3 <= 448 / 128
    assert np.all(F.dequantize_latent(codes, scales)[0] == 0)
    assert F.dequantize_latent(codes, scales)[1, 200] == -3.0                  # 384 * 2^-7, exact


def test_cache_reads_back_dequantized_values():
    """The FP8 caches hold what the format reads back; the bf16 shared key is kept as it is."""
    from workloads import TINY_DSA
    d = TINY_DSA
    rng = np.random.default_rng(7)
    B, T = 2, 5
    c = rng.standard_normal((B, T, d.kv_lora))
    r = rng.standard_normal((B, T, d.d_shared))
    ik = rng.standard_normal((B, T, d.d_idx))
    oc = O.Cache(d, B, expanded=False, fp8_latent=True, fp8_index=True)
    oc.append(c, r, idx_k=ik)
    cb = O.round_to_bf16(c)
    assert np.array_equal(oc.latent[..., d.kv_lora:], O.round_to_bf16(r))
    assert np.array_equal(oc.latent[..., :d.kv_lora], F.latent_read_back(*F.quantize_latent(cb, d)))
    assert np.array_equal(oc.idx, F.dequantize_index_keys(*F.quantize_index_keys(O.round_to_bf16(ik))))
    assert oc.idx_scales.shape == (B, T, 1) and oc.latent_scales.shape == (B, T, d.kv_lora // F.latent_block(d))


@pytest.mark.parametrize("fp8_index", [False, True])
def test_fp8_decode_step_equals_bf16_step_on_read_back_values(fp8_index):
    """A DSA decode step over FP8 caches equals the same step over bf16 caches preset to the
    values the FP8 caches read back (the layer is unchanged; only the stored values are)."""
    from workloads import TINY_DSA, make_layer_weights, make_tokens
    d = TINY_DSA
    lw = make_layer_weights(d, seed=8, dist="fan_in", perturb_norms=True)
    w = {k: bf16_bits_to_f32(v).astype(np.float64) for k, v in lw.w.items()}
    B, T = 2, 20
    rng = np.random.default_rng(8)
    lat = O.round_to_bf16(rng.standard_normal((B, T, d.kv_lora + d.d_shared)))
    idx = O.round_to_bf16(rng.standard_normal((B, T, d.d_idx)))
    x = bf16_bits_to_f32(make_tokens(d, B, 1, seed=8)).astype(np.float64)[:, 0]
    q8 = O.Cache(d, B, expanded=False, fp8_latent=True, fp8_index=fp8_index)
    q8.set_prefix(lat, idx)
    ref = O.Cache(d, B, expanded=False)
    ref.set_prefix(q8.latent.copy(), q8.idx.copy())
    y8, ex8 = O.dsa_decode_step(x, w, q8, d)
    # the new token's rows: the bf16 cache gets what the FP8 cache read back
    y, ex = O.dsa_decode_step(x, w, _Preset(ref, q8), d)
    assert np.array_equal(y8, y)


class _Preset:
    """A bf16 cache whose appends store the values another (FP8) cache read back for them."""

    def __init__(self, ref, q8):
        self.ref, self.q8 = ref, q8

    def __getattr__(self, name):
        return getattr(self.ref, name)

    def append(self, c, r, k=None, v=None, idx_k=None):
        n = self.ref.length
        self.ref.latent = np.concatenate([self.ref.latent, self.q8.latent[:, n:n + 1]], 1)
        self.ref.idx = np.concatenate([self.ref.idx, self.q8.idx[:, n:n + 1]], 1)


def test_latent_read_back_matches_torch():
    """A latent value reads back as decode(code) * scale in fp32, rounded once to bf16: torch's
    float8_e4m3fn -> float32 product -> bfloat16 casts give the same values."""
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 256, (50, 512)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] ^= 1
    scales = (np.abs(rng.standard_normal((50, 4))) / 448).astype(np.float32)
    got = F.latent_read_back(codes, scales)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().reshape(50, 4, 128)
    ref = (vals * torch.from_numpy(scales)[..., None]).to(torch.bfloat16).double().reshape(50, 512).numpy()
    assert np.array_equal(got, ref)
    # within one bf16 rounding (2^-8 relative) of the exact read-back value, and equal to it for
    # power-of-two scales (the quantizer's): E4M3 values are bf16 values
    exact = F.dequantize_latent(codes, scales)
    assert np.all(np.abs(got - exact) <= 2.0 ** -8 * np.abs(exact) * (1 + 2.0 ** -20))
    pow2 = np.ldexp(1.0, rng.integers(-30, 5, (50, 4))).astype(np.float32)
    assert np.array_equal(F.latent_read_back(codes, pow2), F.dequantize_latent(codes, pow2))


def test_power_of_two_scale_at_the_boundary():
    """max|v| exactly 448 * 2^k takes scale 2^k (the element codes to 448); just above takes 2^(k+1)."""
    v = np.zeros((3, 128))
    v[0, 0] = 448.0 * 2.0 ** -5
    v[1, 0] = 450.0 * 2.0 ** -5      # the next bf16 value above 448 * 2^-5
    v[2, 0] = 224.0 * 2.0 ** -5
    codes, scales = F.quantize_blocks(v, 128)
    assert scales[0, 0] == 2.0 ** -5 and F.e4m3_decode(codes[0, 0]) == 448
    assert scales[1, 0] == 2.0 ** -4
    assert scales[2, 0] == 2.0 ** -6 and F.e4m3_decode(codes[2, 0]) == 448
