"""Device buffers for one Gated MLA layer: weights, caches and workspace as torch tensors, with
the ctypes views the C ABI takes. Marshalling only; every computation is a library call."""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import (CACHE_BF16, CACHE_FP8, FP8_LATENT_ROW_BYTES, MlaCache, MlaWeights, OUT_BF16, PATH_ABSORBED,
               make_dims, mla_decode, mla_prefill, workspace_bytes, mla_prefill_sparse,
               workspace_bytes_prefill_sparse)

_WEIGHT_NAMES = ("w_q_a", "g_q_a", "w_q_b", "w_kv_a", "g_kv_a", "w_kv_b", "w_g", "w_o",
                 "w_idx_q", "w_idx_k", "g_idx_k", "b_idx_k", "w_idx_w")


def bf16_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """Upload bf16 bit patterns (uint16 numpy array) as a torch.bfloat16 tensor."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Download a bf16 tensor as uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class LayerBuffers:
    """Weights of one layer on the device and the C structs that point at them."""

    def __init__(self, dims_obj, weight_bits: dict, device="cuda"):
        self.shape = dims_obj
        self.dims = make_dims(dims_obj)
        self.device = device
        self.w = {k: bf16_tensor(v, device) for k, v in weight_bits.items()}
        self.cw = MlaWeights(*[self.w[n].data_ptr() if n in self.w else None for n in _WEIGHT_NAMES])

    def new_cache(self, B: int, T_cap: int, expanded: bool = True, index: bool = False, fp8_latent: bool = False,
                  fp8_index: bool = False, page_size: int = 0, n_pages: int = 0, block_table=None):
        return CacheBuffers(self.shape, B, T_cap, expanded, index, self.device, fp8_latent, fp8_index, page_size,
                            n_pages, block_table)

    def workspace(self, B, T_new, max_len, path=PATH_ABSORBED, num_splits=0):
        n = workspace_bytes(self.dims, B, T_new, max_len, path, num_splits)
        return torch.empty(max(n, 1), dtype=torch.uint8, device=self.device)

    def prefill(self, cache: "CacheBuffers", x: torch.Tensor, start_pos: torch.Tensor, max_end: int,
                out_dtype=OUT_BF16, lse=None, ws=None):
        B, T, _ = x.shape
        y = torch.empty((B, T, self.shape.hidden), device=self.device,
                        dtype=torch.bfloat16 if out_dtype == OUT_BF16 else torch.float32)
        ws = ws if ws is not None else self.workspace(B, T, max_end)
        mla_prefill(self.dims, self.cw, cache.c, start_pos, max_end, x, B, T, y, out_dtype, lse, ws)
        return y

    def prefill_sparse(self, cache: "CacheBuffers", x: torch.Tensor, start_pos: torch.Tensor, max_end: int,
                       out_dtype=OUT_BF16, sel_idx=None, sel_cnt=None, ws=None, scores=None):
        B, T, _ = x.shape
        y = torch.empty((B, T, self.shape.hidden), device=self.device,
                        dtype=torch.bfloat16 if out_dtype == OUT_BF16 else torch.float32)
        if ws is None:
            ws = torch.empty(workspace_bytes_prefill_sparse(self.dims, B, T, max_end), dtype=torch.uint8,
                             device=self.device)
        mla_prefill_sparse(self.dims, self.cw, cache.c, start_pos, max_end, x, B, T, y, out_dtype, sel_idx, sel_cnt,
                           ws, scores=scores)
        return y

    def decode(self, cache: "CacheBuffers", x: torch.Tensor, seq_len: torch.Tensor, max_len: int,
               path=PATH_ABSORBED, out_dtype=OUT_BF16, sel_idx=None, sel_cnt=None, num_splits=0, ws=None):
        B = x.shape[0]
        y = torch.empty((B, self.shape.hidden), device=self.device,
                        dtype=torch.bfloat16 if out_dtype == OUT_BF16 else torch.float32)
        ws = ws if ws is not None else self.workspace(B, 1, max_len, path, num_splits)
        mla_decode(self.dims, self.cw, cache.c, seq_len, max_len, x, B, path, y, out_dtype, sel_idx, sel_cnt,
                   num_splits, ws)
        return y


class CacheBuffers:
    """Caller-owned caches of one layer: latent, optional expanded K/V and index keys.

    FP8 formats: ``latent`` is [B, T_cap, 656] uint8 rows (512 E4M3 codes, four fp32 scales,
    64 bf16 shared-key values); ``idx`` is one uint8 buffer holding the [B, T_cap, 128] codes and
    then the [B, T_cap] fp32 scales, viewed as ``idx_codes`` and ``idx_scales``.

    Paged (``page_size`` > 0): latent and idx are pools of ``n_pages`` pages of ``page_size``
    rows ([n_pages, page_size, ...] in place of [B, T_cap, ...]) and ``block_table`` [B, T_cap /
    page_size] int32 maps each sequence's blocks to pages; the expanded cache is not kept."""

    def __init__(self, d, B, T_cap, expanded=True, index=False, device="cuda", fp8_latent=False, fp8_index=False,
                 page_size=0, n_pages=0, block_table=None):
        bf = torch.bfloat16
        paged = page_size > 0
        R0, R1 = (n_pages, page_size) if paged else (B, T_cap)   # rows of the latent / index arrays
        if fp8_latent:
            self.latent = torch.zeros((R0, R1, FP8_LATENT_ROW_BYTES), dtype=torch.uint8, device=device)
        else:
            self.latent = torch.zeros((R0, R1, d.kv_lora + d.d_shared), dtype=bf, device=device)
        expanded = expanded and not paged
        self.k = torch.zeros((B, d.n_heads, T_cap, d.d_nope + d.d_shared), dtype=bf, device=device) if expanded else None
        self.v = torch.zeros((B, d.n_heads, T_cap, d.d_v), dtype=bf, device=device) if expanded else None
        self.idx = self.idx_codes = self.idx_scales = None
        if index and fp8_index:
            self.idx = torch.zeros(R0 * R1 * (d.d_idx + 4), dtype=torch.uint8, device=device)
            self.idx_codes = self.idx[:R0 * R1 * d.d_idx].view(R0, R1, d.d_idx)
            self.idx_scales = self.idx[R0 * R1 * d.d_idx:].view(torch.float32).view(R0, R1)
        elif index:
            self.idx = torch.zeros((R0, R1, d.d_idx), dtype=bf, device=device)
        self.block_table = None
        if paged:
            self.block_table = torch.as_tensor(block_table, dtype=torch.int32).to(device).contiguous()
            assert self.block_table.shape == (B, T_cap // page_size)
        self.B, self.T_cap = B, T_cap
        p = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
        self.c = MlaCache(p(self.latent), p(self.k), p(self.v), p(self.idx), B, T_cap,
                          CACHE_FP8 if fp8_latent else CACHE_BF16, CACHE_FP8 if fp8_index else CACHE_BF16,
                          p(self.block_table), page_size, T_cap // page_size if paged else 0, n_pages)

    def struct(self) -> MlaCache:
        return self.c

    def ref(self):
        return ctypes.byref(self.c)
