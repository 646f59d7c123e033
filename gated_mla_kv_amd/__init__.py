"""Python binding of libgmla.so, the Gated MLA / Gated DSA attention library for MI355X.

Argument marshalling only: each function takes torch tensors (device memory) and passes their
data pointers, sizes and the current HIP stream to the C ABI declared in include/gmla.h. All
computation runs in the library's HIP kernels. The library is built in-tree by
``gated_mla_kv_amd.build.build()``; if it is missing, loading raises instead of falling back.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "GmlaError", "lib", "MlaDims", "MlaWeights", "MlaCache", "make_dims", "OUT_BF16", "OUT_F32",
    "PATH_ABSORBED", "PATH_EXPANDED", "PATH_SPARSE", "status_string", "dims_supported",
    "workspace_bytes", "workspace_bytes_prefill_sparse", "mla_prefill", "mla_prefill_sparse", "mla_decode",
    "mla_decode_noalloc", "NOALLOC_SCRATCH_BYTES", "kv_append", "dsa_index_topk", "dsa_index_topk_fp8", "mla_index_projections", "mla_gemm",
    "mla_rmsnorm", "mla_layernorm", "mla_prefill_attention", "mla_absorb_query",
    "mla_decode_attention", "mla_sparse_attention", "mla_expanded_attention", "mla_value_up_gate",
    "mla_debug_scores", "DEBUG_SCORES_MAX", "mla_debug_flags", "LIB_PATH", "DEBUG_LIB_PATH",
]

# GMLA_LIB selects another build of the library (the debug-checks or the host-ASan variant)
LIB_PATH = os.environ.get("GMLA_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgmla.so")
DEBUG_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgmla_debug.so")

OUT_BF16, OUT_F32 = 0, 1
PATH_ABSORBED, PATH_EXPANDED, PATH_SPARSE = 0, 1, 2
CACHE_BF16, CACHE_FP8 = 0, 1
FP8_LATENT_ROW_BYTES = 656  # 512 E4M3 codes, four fp32 scales, 64 bf16 shared-key values
DEBUG_SCORES_MAX = 1 << 26  # MLA_DEBUG_SCORES_MAX: most logits one mla_debug_scores call writes


class GmlaError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn} returned {status} ({status_string(status)})")


class MlaDims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("q_lora", ctypes.c_int32),
                ("kv_lora", ctypes.c_int32), ("d_nope", ctypes.c_int32), ("d_shared", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("rms_eps", ctypes.c_float), ("softmax_scale", ctypes.c_float),
                ("use_gate", ctypes.c_int32), ("n_idx_heads", ctypes.c_int32), ("d_idx", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("ln_eps", ctypes.c_float)]


class MlaWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w_q_a", "g_q_a", "w_q_b", "w_kv_a", "g_kv_a", "w_kv_b", "w_g", "w_o",
        "w_idx_q", "w_idx_k", "g_idx_k", "b_idx_k", "w_idx_w")]


class MlaCache(ctypes.Structure):
    _fields_ = [("latent", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("idx_k", ctypes.c_void_p), ("batch", ctypes.c_int32), ("T_cap", ctypes.c_int32),
                ("latent_format", ctypes.c_int32), ("idx_format", ctypes.c_int32),
                ("block_table", ctypes.c_void_p), ("page_size", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
                ("n_pages", ctypes.c_int32)]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float
_SZ = ctypes.c_size_t
_SIGS = {
    "mla_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "mla_dims_supported": (ctypes.c_int, [_P]),
    "mla_workspace_bytes": (_SZ, [_P, _I, _I, _I, _I]),
    "mla_workspace_bytes_ex": (_SZ, [_P, _I, _I, _I, _I, _I]),
    "mla_prefill": (ctypes.c_int, [_P, _P, _P, _P, _I, _P, _I, _I, _P, _I, _P, _P, _SZ, _P]),
    "mla_workspace_bytes_prefill_sparse": (_SZ, [_P, _I, _I, _I]),
    "mla_prefill_sparse": (ctypes.c_int, [_P, _P, _P, _P, _I, _P, _I, _I, _P, _I, _P, _P, _P, _P, _SZ, _P]),
    "mla_index_projections": (ctypes.c_int, [_P, _P, _P, _I, _P, _P, _P, _P, _SZ, _P]),
    "mla_decode": (ctypes.c_int, [_P, _P, _P, _P, _I, _P, _I, _I, _I, _P, _P, _P, _I, _P, _SZ, _P]),
    "mla_decode_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _I, _P, _I, _I, _I, _P, _P, _P, _I, _P]),
    "kv_append": (ctypes.c_int, [_P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P]),
    "dsa_index_topk": (ctypes.c_int, [_P, _P, _P, _P, _I, _P, _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "dsa_index_topk_fp8": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _P, _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "mla_gemm": (ctypes.c_int, [_P, _I, _P, _I, _I, _I, _P, _I, _I, _P]),
    "mla_rmsnorm": (ctypes.c_int, [_P, _I, _P, _I, _I, _F, _P, _I, _P]),
    "mla_layernorm": (ctypes.c_int, [_P, _I, _P, _P, _I, _I, _F, _P, _I, _P]),
    "mla_prefill_attention": (ctypes.c_int, [_P, _P, _P, _P, _I, _I, _I, _P, _P, _I, _P, _P]),
    "mla_absorb_query": (ctypes.c_int, [_P, _P, _I, _P, _I, _P, _P]),
    "mla_decode_attention": (ctypes.c_int, [_P, _P, _P, _P, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "mla_sparse_attention": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _P, _P, _P, _SZ, _P]),
    "mla_expanded_attention": (ctypes.c_int, [_P, _P, _P, _P, _I, _I, _P, _P, _P]),
    "mla_value_up_gate": (ctypes.c_int, [_P, _P, _P, _P, _I, _P, _I, _P]),
    "mla_debug_scores": (ctypes.c_int, [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P]),
    "mla_debug_flags": (ctypes.c_int, [_P, _P, _P]),
}


def lib() -> ctypes.CDLL:
    """Load libgmla.so (once). Raises if the library has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with gated_mla_kv_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().mla_status_string(int(status)).decode()


def _check(status: int, fn: str) -> None:
    if status != 0:
        raise GmlaError(status, fn)


def make_dims(d, use_gate: bool | None = None) -> MlaDims:
    """C dims from any object with the config attributes (hidden, n_heads, q_lora, ...)."""
    dq = d.d_nope + d.d_shared
    g = getattr(d, "use_gate", True) if use_gate is None else use_gate
    return MlaDims(d.hidden, d.n_heads, d.q_lora, d.kv_lora, d.d_nope, d.d_shared, d.d_v,
                   getattr(d, "rms_eps", 1e-6), dq ** -0.5, 1 if g else 0,
                   getattr(d, "n_idx_heads", 0), getattr(d, "d_idx", 0), getattr(d, "topk", 0),
                   getattr(d, "ln_eps", 1e-6))


def _p(t):
    """Device pointer of a tensor (or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ref(x):
    return ctypes.byref(x) if x is not None else None


def dims_supported(dims: MlaDims) -> bool:
    return lib().mla_dims_supported(ctypes.byref(dims)) == 0


def workspace_bytes(dims: MlaDims, B: int, T_new: int, max_len: int, path: int = 0,
                    num_splits: int = 0) -> int:
    return int(lib().mla_workspace_bytes_ex(ctypes.byref(dims), B, T_new, max_len, path, num_splits))


def _ws(ws):
    if ws is None:
        return None, 0
    return ws.data_ptr(), ws.numel() * ws.element_size()


def mla_prefill(dims, weights: MlaWeights, cache: MlaCache, start_pos, max_end, x, B, T, y,
                out_dtype=OUT_BF16, lse=None, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check(lib().mla_prefill(ctypes.byref(dims), ctypes.byref(weights), ctypes.byref(cache), _p(start_pos),
                             max_end, _p(x), B, T, _p(y), out_dtype, _p(lse), wp, wn, _stream(stream)),
           "mla_prefill")


def workspace_bytes_prefill_sparse(dims: MlaDims, B: int, T: int, max_end: int) -> int:
    return int(lib().mla_workspace_bytes_prefill_sparse(ctypes.byref(dims), B, T, max_end))


def mla_prefill_sparse(dims, weights: MlaWeights, cache: MlaCache, start_pos, max_end, x, B, T, y,
                       out_dtype=OUT_BF16, sel_idx=None, sel_cnt=None, ws=None, stream=None, scores=None):
    wp, wn = _ws(ws)
    _check(lib().mla_prefill_sparse(ctypes.byref(dims), ctypes.byref(weights), ctypes.byref(cache),
                                    _p(start_pos), max_end, _p(x), B, T, _p(y), out_dtype, _p(sel_idx),
                                    _p(sel_cnt), _p(scores), wp, wn, _stream(stream)),
           "mla_prefill_sparse")


def mla_index_projections(dims, weights: MlaWeights, x, M, q_idx, w_idx, k_idx, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check(lib().mla_index_projections(ctypes.byref(dims), ctypes.byref(weights), _p(x), M, _p(q_idx), _p(w_idx),
                                       _p(k_idx), wp, wn, _stream(stream)), "mla_index_projections")


def mla_decode(dims, weights: MlaWeights, cache: MlaCache, seq_len, max_len, x, B, path, y,
               out_dtype=OUT_BF16, sel_idx=None, sel_cnt=None, num_splits=0, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check(lib().mla_decode(ctypes.byref(dims), ctypes.byref(weights), ctypes.byref(cache), _p(seq_len),
                            max_len, _p(x), B, path, num_splits, _p(sel_idx), _p(sel_cnt), _p(y),
                            out_dtype, wp, wn, _stream(stream)),
           "mla_decode")


NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024


def mla_decode_noalloc(dims, weights: MlaWeights, cache: MlaCache, seq_len, max_len, x, B, path, y,
                       out_dtype=OUT_BF16, sel_idx=None, sel_cnt=None, num_splits=0, stream=None):
    _check(lib().mla_decode_noalloc(ctypes.byref(dims), ctypes.byref(weights), ctypes.byref(cache), _p(seq_len),
                                    max_len, _p(x), B, path, num_splits, _p(sel_idx), _p(sel_cnt), _p(y),
                                    out_dtype, _stream(stream)),
           "mla_decode_noalloc")


def kv_append(dims, cache: MlaCache, pos, max_end, B, T, c, r, k_nope=None, v=None, idx_k=None, stream=None):
    _check(lib().kv_append(ctypes.byref(dims), ctypes.byref(cache), _p(pos), max_end, B, T, _p(c), _p(r),
                           _p(k_nope), _p(v), _p(idx_k), _stream(stream)), "kv_append")


def dsa_index_topk(dims, q_idx, w_idx, idx_k_cache, T_cap, n_visible, max_visible, B, out_idx, out_cnt,
                   out_scores=None, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check(lib().dsa_index_topk(ctypes.byref(dims), _p(q_idx), _p(w_idx), _p(idx_k_cache), T_cap,
                                _p(n_visible), max_visible, B, _p(out_idx), _p(out_cnt), _p(out_scores),
                                wp, wn, _stream(stream)), "dsa_index_topk")


def dsa_index_topk_fp8(dims, q_idx, w_idx, idx_codes, idx_scales, T_cap, n_visible, max_visible, B, out_idx,
                       out_cnt, out_scores=None, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check(lib().dsa_index_topk_fp8(ctypes.byref(dims), _p(q_idx), _p(w_idx), _p(idx_codes), _p(idx_scales),
                                    T_cap, _p(n_visible), max_visible, B, _p(out_idx), _p(out_cnt),
                                    _p(out_scores), wp, wn, _stream(stream)), "dsa_index_topk_fp8")


def mla_gemm(a, lda, w, M, N, K, out, ldo, out_dtype=OUT_BF16, stream=None):
    _check(lib().mla_gemm(_p(a), lda, _p(w), M, N, K, _p(out), ldo, out_dtype, _stream(stream)), "mla_gemm")


def mla_rmsnorm(x, ldx, gain, M, N, eps, out, ldo, stream=None):
    _check(lib().mla_rmsnorm(_p(x), ldx, _p(gain), M, N, eps, _p(out), ldo, _stream(stream)), "mla_rmsnorm")


def mla_layernorm(x, ldx, gain, bias, M, N, eps, out, ldo, stream=None):
    _check(lib().mla_layernorm(_p(x), ldx, _p(gain), _p(bias), M, N, eps, _p(out), ldo, _stream(stream)),
           "mla_layernorm")


def mla_prefill_attention(dims, q, cache: MlaCache, start_pos, max_end, B, T, g_pre, u,
                          out_dtype=OUT_BF16, lse=None, stream=None):
    _check(lib().mla_prefill_attention(ctypes.byref(dims), _p(q), ctypes.byref(cache), _p(start_pos), max_end,
                                       B, T, _p(g_pre), _p(u), out_dtype, _p(lse), _stream(stream)),
           "mla_prefill_attention")


def mla_absorb_query(dims, q, ldq, w_kv_b, B, q_tilde, stream=None):
    _check(lib().mla_absorb_query(ctypes.byref(dims), _p(q), ldq, _p(w_kv_b), B, _p(q_tilde), _stream(stream)),
           "mla_absorb_query")


def mla_decode_attention(dims, q_tilde, cache: MlaCache, n_visible, max_visible, B, o_latent, lse=None,
                         num_splits=0, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check(lib().mla_decode_attention(ctypes.byref(dims), _p(q_tilde), ctypes.byref(cache), _p(n_visible),
                                      max_visible, B, num_splits, _p(o_latent), _p(lse), wp, wn,
                                      _stream(stream)), "mla_decode_attention")


def mla_sparse_attention(dims, q_tilde, cache: MlaCache, sel_idx, sel_cnt, B, o_latent, lse=None,
                         num_splits=0, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check(lib().mla_sparse_attention(ctypes.byref(dims), _p(q_tilde), ctypes.byref(cache), _p(sel_idx),
                                      _p(sel_cnt), B, num_splits, _p(o_latent), _p(lse), wp, wn,
                                      _stream(stream)), "mla_sparse_attention")


def mla_expanded_attention(dims, q, cache: MlaCache, n_visible, max_visible, B, z, lse=None, stream=None):
    _check(lib().mla_expanded_attention(ctypes.byref(dims), _p(q), ctypes.byref(cache), _p(n_visible),
                                        max_visible, B, _p(z), _p(lse), _stream(stream)),
           "mla_expanded_attention")


def mla_value_up_gate(dims, o_latent, w_kv_b, g_pre, B, u, out_dtype=OUT_BF16, stream=None):
    _check(lib().mla_value_up_gate(ctypes.byref(dims), _p(o_latent), _p(w_kv_b), _p(g_pre), B, _p(u),
                                   out_dtype, _stream(stream)), "mla_value_up_gate")


def mla_debug_scores(dims, q, k, k_heads, B, Tq, Tk, D, logits, stream=None):
    _check(lib().mla_debug_scores(ctypes.byref(dims), _p(q), _p(k), k_heads, B, Tq, Tk, D, _p(logits),
                                  _stream(stream)), "mla_debug_scores")


def mla_debug_flags(stream=None):
    """(flags, checks_built): the device-side bound-check bits recorded since the last call
    (cleared by this call), and whether this build of the library has the checks."""
    flags, built = ctypes.c_uint32(0), ctypes.c_int32(0)
    _check(lib().mla_debug_flags(ctypes.byref(flags), ctypes.byref(built), _stream(stream)), "mla_debug_flags")
    return int(flags.value), bool(built.value)
