"""Float64 oracle of the FP8 latent and index-key caches (Kimi K3.1 Gated DSA).

TEST INFRASTRUCTURE: see the package docstring. Nothing on the product path may import this.

Source: "Kimi K3 model structure (11): K3.1 Pro's Gated DSA from the inference code"
(blog.javazero.top), the cache section: a deployed main cache holds, per position and layer,
512 bytes of FP8 latent, four FP32 scales and the 64 shared-key values in BF16 (656 B); a
default FP8 index key holds 128 bytes of data and one 4-byte scale (132 B).

Readings where the page is silent (listed with their support in the design notes):
* FP8 is the OCP E4M3 format (4 exponent bits, bias 7, 3 mantissa bits, no infinities, largest
  finite value 448, S.1111.111 the only NaN).
* The four latent scales belong to four blocks of 128 consecutive latent features (a latent
  narrower than 128, as in the small test layer, is one block); the index key has one scale
  for its 128 features.
* A block's scale is the smallest power of two 2^k (k >= -126, an FP32 value) with
  max|v| <= 448 * 2^k, so the block's largest element codes into [224, 448]; the code of a value
  v is v / 2^k (exact) rounded to the nearest E4M3 value, ties to even, with the sign copied (a
  block of zeros has scale 0 and codes +-0). The page gives the scales' type, not their rule; a
  power of two keeps E4M3's full relative precision, makes the division exact, and makes
  decode(code) * scale an exponent shift that gfx950's scaled FP8 conversions perform in one
  instruction.
* A cached index key reads back as decode(code) * scale, exact in float64. A cached latent
  value reads back in the layer's compute type: decode(code) * scale formed in FP32 and rounded
  once to BF16 (the page's deployed path feeds the main cache to BF16 attention kernels; the
  shared key is BF16 already). The layer then runs on those values exactly as on a BF16 cache.
"""
from __future__ import annotations

import numpy as np

__all__ = ["E4M3_MAX", "e4m3_decode", "e4m3_encode", "quantize_blocks", "dequantize_blocks",
           "latent_block", "latent_row_bytes", "index_key_bytes", "quantize_latent", "quantize_index_keys",
           "dequantize_latent", "latent_read_back", "dequantize_index_keys"]

F64 = np.float64
E4M3_MAX = 448.0
LATENT_BLOCK = 128


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 byte as float64 (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(F64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(F64) - 7.0))
    mag = np.where((e == 15) & (c & 7 == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 byte (ties to even) of each finite value, sign copied, saturating at 448."""
    x = np.asarray(x, dtype=F64)
    neg = np.signbit(x)
    a = np.abs(x)
    # subnormal range (a < 2^-6): steps of 2^-9; a count of 8 steps is the smallest normal, code 8
    sub = np.rint(a / 2.0 ** -9)
    # normal range: a = f * 2^E with 0.5 <= f < 1, i.e. a = (1 + m/8) * 2^e with e = E - 1
    f, E = np.frexp(np.where(a > 0, a, 1.0))
    e = E - 1
    q = np.rint((2.0 * f - 1.0) * 8.0)           # 0..8; rint rounds half to even
    e = np.where(q == 8, e + 1, e)
    q = np.where(q == 8, 0, q)
    normal = ((e + 7) << 3) + q.astype(np.int64)
    mag = np.where(a < 2.0 ** -6, sub.astype(np.int64), normal)
    mag = np.minimum(mag, 0x7E)                   # 448
    return ((neg.astype(np.int64) << 7) | mag).astype(np.uint8)


def quantize_blocks(v, block: int):
    """v [..., n] (values of the cache type) -> codes [..., n] uint8, scales [..., n/block] fp32.

    scale = the smallest 2^k (k >= -126) with max|v| <= 448 * 2^k per block, 0 for a zero block;
    code = e4m3(v / scale).
    """
    v = np.asarray(v, dtype=F64)
    n = v.shape[-1]
    vb = v.reshape(v.shape[:-1] + (n // block, block))
    absmax = np.abs(vb).max(-1)
    # absmax = f * 2^E with 0.5 <= f < 1, and 448 = 0.875 * 2^9: the bound holds for k = E - 9
    # when f <= 0.875, else for k = E - 8
    f, E = np.frexp(np.where(absmax > 0, absmax, 1.0))
    k = np.maximum(np.where(f <= 0.875, E - 9, E - 8), -126)
    scale = np.where(absmax > 0, np.ldexp(1.0, k), 0.0)
    safe = np.where(scale > 0, scale, 1.0)
    codes = np.where(scale[..., None] > 0, e4m3_encode(vb / safe[..., None]), e4m3_encode(vb * 0.0))
    return codes.reshape(v.shape).astype(np.uint8), scale.astype(np.float32)


def dequantize_blocks(codes, scales, block: int) -> np.ndarray:
    """decode(code) * scale, exact in float64."""
    codes = np.asarray(codes, dtype=np.uint8)
    n = codes.shape[-1]
    vals = e4m3_decode(codes).reshape(codes.shape[:-1] + (n // block, block))
    return (vals * np.asarray(scales, dtype=F64)[..., None]).reshape(codes.shape)


def latent_block(dims) -> int:
    return min(LATENT_BLOCK, dims.kv_lora)


def latent_row_bytes(dims) -> int:
    """Bytes per position of the FP8 main cache: latent codes, one FP32 scale per block of 128,
    the shared key in BF16."""
    return dims.kv_lora + 4 * (dims.kv_lora // latent_block(dims)) + 2 * dims.d_shared


def index_key_bytes(dims) -> int:
    """Bytes per position of the FP8 index-key cache: codes plus one FP32 scale."""
    return dims.d_idx + 4


def quantize_latent(c, dims):
    """The latent part of a main-cache row: codes [.., kv_lora], scales [.., kv_lora/128]."""
    return quantize_blocks(c, latent_block(dims))


def dequantize_latent(codes, scales) -> np.ndarray:
    codes = np.asarray(codes)
    return dequantize_blocks(codes, scales, codes.shape[-1] // np.shape(scales)[-1])


def latent_read_back(codes, scales) -> np.ndarray:
    """What an FP8 latent value reads back as: bf16(fp32(decode(code) * scale)), as float64."""
    from .mla import round_to_bf16
    codes = np.asarray(codes, dtype=np.uint8)
    n = codes.shape[-1]
    block = n // np.shape(scales)[-1]
    vals = e4m3_decode(codes).astype(np.float32).reshape(codes.shape[:-1] + (n // block, block))
    prod = (vals * np.asarray(scales, dtype=np.float32)[..., None]).astype(np.float32)   # fp32 product
    return round_to_bf16(prod.astype(F64)).reshape(codes.shape)


def quantize_index_keys(k):
    """Index keys [.., d_idx] -> codes [.., d_idx], one scale [.., 1] per key."""
    k = np.asarray(k, dtype=F64)
    return quantize_blocks(k, k.shape[-1])


def dequantize_index_keys(codes, scales) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    return dequantize_blocks(codes, scales, codes.shape[-1])
