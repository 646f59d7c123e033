"""Seeded synthetic inputs for the Gated MLA layer and the Gated DSA decode path.

This module is shared by the oracle's tests, the GPU parity tests, the smoke check and the
bench. It holds the layer shapes and counter-seeded generators, and nothing of the method's
arithmetic: no projection, normalisation, attention or selection happens here.

Every tensor is drawn from its own ``numpy.random.Generator(PCG64([seed, tensor_id]))``
stream, so a tensor does not depend on which other tensors were drawn before it. Values are
drawn in float32, scaled, and rounded to bfloat16 with round-to-nearest-even. Both sides of a
parity check receive the same bf16 bit patterns; the oracle widens them to float64.

Shapes follow the pages:
* Kimi K3 Gated MLA (atlas.klimoza.dev, "Kimi K3 > Gated MLA > KV cache" card and the
  released config excerpt): 96 heads, q latent 1536, KV latent 512, 128 nope + 64 shared key
  features, 128 value features, hidden width 7168.
* Kimi K3.1 Gated DSA (blog.javazero.top, "Kimi K3 model structure (11)", eqs. (2)-(6)):
  32 index heads of 128 features, top-2048.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

__all__ = [
    "MLADims", "K3", "K2_SHAPE", "TINY", "TINY_DSA", "K3_SMALL_TOPK",
    "bf16_bits", "bf16_bits_to_f32", "normal_bf16", "LayerInputs", "make_layer_weights",
    "make_tokens", "make_latent_prefix", "make_index_prefix", "TensorId", "device_normal_bf16",
    "device_normal_f32",
]


@dataclass(frozen=True)
class MLADims:
    """Dimensions of one Gated MLA layer (field names follow the released config.json)."""

    hidden: int
    n_heads: int
    q_lora: int
    kv_lora: int
    d_nope: int
    d_shared: int  # "qk_rope_head_dim" in the config; in K3 nothing rotates it
    d_v: int
    rms_eps: float = 1e-6
    use_gate: bool = True
    n_idx_heads: int = 0  # 0 disables the Gated DSA indexer
    d_idx: int = 0
    topk: int = 0
    ln_eps: float = 1e-6

    @property
    def d_qk(self) -> int:
        return self.d_nope + self.d_shared

    @property
    def d_latent(self) -> int:
        return self.kv_lora + self.d_shared

    def replace(self, **kw) -> "MLADims":
        return dataclasses.replace(self, **kw)


# Kimi K3 Gated MLA with the K3.1 Gated DSA indexer dimensions.
K3 = MLADims(hidden=7168, n_heads=96, q_lora=1536, kv_lora=512, d_nope=128, d_shared=64,
             d_v=128, n_idx_heads=32, d_idx=128, topk=2048)
# K3 dims with a small top-k, so that selection (t > k) is exercised at oracle-friendly sizes.
K3_SMALL_TOPK = K3.replace(topk=64)
# Kimi K2's MLA attention shape (64 heads); only its cache accounting is used.
K2_SHAPE = MLADims(hidden=7168, n_heads=64, q_lora=1536, kv_lora=512, d_nope=128, d_shared=64,
                   d_v=128)
# The tiny oracle-scale layer: hidden 256, 4 heads, q_lora 64, kv_lora 32, nope 16, shared 8,
# value 16, sigmoid output gate.
TINY = MLADims(hidden=256, n_heads=4, q_lora=64, kv_lora=32, d_nope=16, d_shared=8, d_v=16)
# The tiny layer with a small indexer, for oracle-only selection checks.
TINY_DSA = TINY.replace(n_idx_heads=4, d_idx=16, topk=8)


class TensorId:
    """Fixed stream ids, one per tensor (the second word of the PCG64 seed)."""

    X = 1
    W_Q_A = 2
    W_Q_B = 3
    W_KV_A = 4
    W_KV_B = 5
    W_G = 6
    W_O = 7
    G_Q_A = 8
    G_KV_A = 9
    W_IDX_Q = 10
    W_IDX_K = 11
    G_IDX_K = 12
    B_IDX_K = 13
    W_IDX_W = 14
    LATENT_PREFIX = 20
    INDEX_PREFIX = 21
    Q_LATENT = 22
    DECODE_X = 100  # + step


# ---------------------------------------------------------------------------------------------
# bfloat16 storage format (input quantisation only)
# ---------------------------------------------------------------------------------------------

def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32)
    # finite inputs: u <= 0xFF7FFFFF, so the rounding add cannot overflow 32 bits
    t = u >> np.uint32(16)
    t &= np.uint32(1)
    t += np.uint32(0x7FFF)
    t += u
    t >>= np.uint32(16)
    return t.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _gen(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([int(seed), int(tensor_id)]))


def normal_bf16(shape, std: float, seed: int, tensor_id: int, mean: float = 0.0) -> np.ndarray:
    """Draw N(mean, std^2) in float32 from the tensor's own stream and round to bf16 bits."""
    g = _gen(seed, tensor_id)
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if mean != 0.0:
        a += np.float32(mean)
    return bf16_bits(a)


# ---------------------------------------------------------------------------------------------
# Layer weights and activations
# ---------------------------------------------------------------------------------------------

@dataclass
class LayerInputs:
    """bf16 bit patterns (uint16 arrays) of one layer's parameters, nn.Linear [out, in] layout."""

    dims: MLADims
    w: dict

    def f32(self, name: str) -> np.ndarray:
        return bf16_bits_to_f32(self.w[name])


def make_layer_weights(dims: MLADims, seed: int = 0, dist: str = "k3",
                       perturb_norms: bool = False) -> LayerInputs:
    """Weights of one layer.

    dist="k3": every weight N(0, 0.02^2) (the K3 workloads).
    dist="fan_in": weight N(0, 1/fan_in) (the tiny oracle-scale layer).
    Norm gains are 1 and the index-key LayerNorm bias 0 (module initialisation); with
    perturb_norms they are 1 + 0.1 N(0,1) and 0.1 N(0,1) so that the multiplies are exercised.
    """
    d = dims
    H = d.n_heads
    shapes = {
        "w_q_a": ((d.q_lora, d.hidden), TensorId.W_Q_A),
        "w_q_b": ((H * d.d_qk, d.q_lora), TensorId.W_Q_B),
        "w_kv_a": ((d.kv_lora + d.d_shared, d.hidden), TensorId.W_KV_A),
        "w_kv_b": ((H * (d.d_nope + d.d_v), d.kv_lora), TensorId.W_KV_B),
        "w_g": ((H * d.d_v, d.hidden), TensorId.W_G),
        "w_o": ((d.hidden, H * d.d_v), TensorId.W_O),
    }
    if d.n_idx_heads:
        shapes.update({
            "w_idx_q": ((d.n_idx_heads * d.d_idx, d.q_lora), TensorId.W_IDX_Q),
            "w_idx_k": ((d.d_idx, d.hidden), TensorId.W_IDX_K),
            "w_idx_w": ((d.n_idx_heads, d.hidden), TensorId.W_IDX_W),
        })
    w = {}
    for name, (shape, tid) in shapes.items():
        if dist == "k3":
            std = 0.02
        elif dist == "fan_in":
            std = float(1.0 / np.sqrt(shape[1]))
        else:
            raise ValueError(f"unknown weight distribution {dist!r}")
        w[name] = normal_bf16(shape, std, seed, tid)
    gains = {"g_q_a": (d.q_lora, TensorId.G_Q_A), "g_kv_a": (d.kv_lora, TensorId.G_KV_A)}
    if d.n_idx_heads:
        gains["g_idx_k"] = (d.d_idx, TensorId.G_IDX_K)
    for name, (n, tid) in gains.items():
        if perturb_norms:
            w[name] = normal_bf16((n,), 0.1, seed, tid, mean=1.0)
        else:
            w[name] = bf16_bits(np.ones(n, np.float32))
    if d.n_idx_heads:
        if perturb_norms:
            w["b_idx_k"] = normal_bf16((d.d_idx,), 0.1, seed, TensorId.B_IDX_K)
        else:
            w["b_idx_k"] = bf16_bits(np.zeros(d.d_idx, np.float32))
    return LayerInputs(dims=d, w=w)


def make_tokens(dims: MLADims, B: int, T: int, seed: int = 0, step: int | None = None) -> np.ndarray:
    """Layer inputs x [B, T, hidden] ~ N(0, 1), bf16 bits. step selects a decode token stream."""
    tid = TensorId.X if step is None else TensorId.DECODE_X + int(step)
    return normal_bf16((B, T, dims.hidden), 1.0, seed, tid)


def make_latent_prefix(dims: MLADims, B: int, T: int, seed: int = 0) -> np.ndarray:
    """Cached latent rows [B, T, kv_lora + d_shared] ~ N(0, 1), bf16 bits."""
    return normal_bf16((B, T, dims.d_latent), 1.0, seed, TensorId.LATENT_PREFIX)


def make_index_prefix(dims: MLADims, B: int, T: int, seed: int = 0) -> np.ndarray:
    """Cached index keys [B, T, d_idx] ~ N(0, 1), bf16 bits."""
    return normal_bf16((B, T, dims.d_idx), 1.0, seed, TensorId.INDEX_PREFIX)


def device_normal_f32(shape, std: float, seed: int, tensor_id: int, device="cuda"):
    """N(0, std^2) float32 tensor drawn on the device by torch's seeded generator (fp32 inputs such
    as the DSA index query, which the library takes unrounded)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + int(tensor_id))
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def device_normal_bf16(shape, std: float, seed: int, tensor_id: int, device="cuda"):
    """N(0, std^2) bf16 tensor drawn on the device by torch's seeded generator (Philox), for the
    full-size inputs (the expanded cache alone holds 8 G values). The same bits go to both sides:
    the GPU path reads the tensor, the oracle the rows copied back from it."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + int(tensor_id))
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.bfloat16)
    if std != 1.0:
        t.mul_(std)
    return t
