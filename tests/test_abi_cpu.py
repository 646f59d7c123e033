"""C ABI contract on the host (no GPU needed): the library loads, exports every function that
include/gmla.h declares, and its host-side validation returns the documented error codes
before anything is launched."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gmla.h")

gm = pytest.importorskip("gated_mla_kv_amd")
from workloads import K3, TINY  # noqa: E402

if not os.path.exists(gm.LIB_PATH):
    pytest.skip("libgmla.so not built", allow_module_level=True)

OK, ERR_NULL, ERR_SHAPE, ERR_CAPACITY, ERR_UNSUPPORTED, ERR_WORKSPACE = 0, -1, -2, -3, -4, -5
FAKE = 0x1000  # a non-null pointer value; never dereferenced by the validation paths tested


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(mla_\w+|kv_append|dsa_index_topk\w*)\s*\(",
                                 text, flags=re.M)))


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert len(names) >= 17, names
    L = gm.lib()
    for n in names:
        assert hasattr(L, n), f"{n} declared in gmla.h but not exported"
    # and nothing the binding calls is undeclared
    for n in gm._SIGS:
        assert n in names, n


def test_status_strings():
    assert gm.status_string(0) == "MLA_OK"
    assert gm.status_string(-4) == "MLA_ERR_UNSUPPORTED"
    assert gm.status_string(123) == "MLA_ERR_UNKNOWN"


def test_dims_supported():
    assert gm.dims_supported(gm.make_dims(K3))
    assert gm.dims_supported(gm.make_dims(TINY))
    assert not gm.dims_supported(gm.make_dims(K3.replace(n_heads=64)))
    assert not gm.dims_supported(gm.make_dims(TINY.replace(n_idx_heads=4, d_idx=16, topk=8)))
    assert not gm.dims_supported(gm.make_dims(K3.replace(topk=4096)))


def test_workspace_bytes():
    d = gm.make_dims(K3)
    pre = gm.workspace_bytes(d, 1, 4096, 4096)
    assert pre > 4096 * 12288 * 2  # at least the gated head outputs
    dec = gm.workspace_bytes(d, 32, 1, 8193, gm.PATH_ABSORBED)
    assert dec > 32 * 8 * 96 * 512 * 2  # split partials (fp16)
    assert gm.workspace_bytes(d, 32, 1, 8193, gm.PATH_ABSORBED, 16) > dec
    assert gm.workspace_bytes(gm.make_dims(K3.replace(n_heads=8)), 1, 1, 10) == 0


def _cache(latent=FAKE, k=FAKE, v=FAKE, idx=None, B=2, T_cap=100):
    return gm.MlaCache(latent, k, v, idx, B, T_cap)


def _weights():
    return gm.MlaWeights(*([FAKE] * 8 + [None] * 5))


def _call_prefill(dims, cache, max_end=50, B=2, T=10, ws_bytes=1 << 40, weights=None, x=FAKE):
    L = gm.lib()
    return L.mla_prefill(ctypes.byref(dims), ctypes.byref(weights or _weights()), ctypes.byref(cache), FAKE,
                         max_end, x, B, T, FAKE, 0, None, FAKE, ws_bytes, None)


def test_prefill_validation():
    d = gm.make_dims(K3)
    assert _call_prefill(gm.make_dims(K3.replace(hidden=1000)), _cache()) == ERR_UNSUPPORTED
    assert _call_prefill(d, _cache(), x=None) == ERR_NULL
    assert _call_prefill(d, _cache(k=None)) == ERR_NULL
    assert _call_prefill(d, _cache(T_cap=100), max_end=101) == ERR_CAPACITY
    assert _call_prefill(d, _cache(B=1), B=2) == ERR_SHAPE
    assert _call_prefill(d, _cache(), B=-1) == ERR_SHAPE
    assert _call_prefill(d, _cache(), ws_bytes=10) == ERR_WORKSPACE
    w = _weights()
    w.w_g = None
    assert _call_prefill(d, _cache(), weights=w) == ERR_NULL
    # empty work is valid and launches nothing
    assert _call_prefill(d, _cache(), B=0) == OK
    assert _call_prefill(d, _cache(), T=0) == OK


def _call_decode(dims, cache, path=0, max_len=50, B=2, ws_bytes=1 << 40, weights=None, splits=0):
    L = gm.lib()
    return L.mla_decode(ctypes.byref(dims), ctypes.byref(weights or _weights()), ctypes.byref(cache), FAKE,
                        max_len, FAKE, B, path, splits, None, None, FAKE, 0, FAKE, ws_bytes, None)


def test_decode_validation():
    d = gm.make_dims(K3)
    assert _call_decode(d, _cache(), path=7) == ERR_UNSUPPORTED
    assert _call_decode(d, _cache(T_cap=64), max_len=65) == ERR_CAPACITY
    assert _call_decode(d, _cache(k=None, v=None), path=gm.PATH_EXPANDED) == ERR_NULL
    assert _call_decode(d, _cache(), ws_bytes=1000) == ERR_WORKSPACE
    # sparse needs the indexer
    assert _call_decode(gm.make_dims(K3.replace(n_idx_heads=0)), _cache(), path=gm.PATH_SPARSE) == ERR_UNSUPPORTED
    assert _call_decode(d, _cache(idx=None), path=gm.PATH_SPARSE) == ERR_NULL
    assert _call_decode(d, _cache(), B=0) == OK
    assert _call_decode(d, _cache(), splits=-1) == ERR_SHAPE


def test_kv_append_validation():
    L = gm.lib()
    d = gm.make_dims(TINY)
    c = _cache(T_cap=16)
    call = lambda max_end, B=2, T=4, idx=None, cc=c, dd=d, cp=FAKE: L.kv_append(  # noqa: E731
        ctypes.byref(dd), ctypes.byref(cc), FAKE, max_end, B, T, cp, FAKE, FAKE, FAKE, idx, None)
    assert call(17) == ERR_CAPACITY
    assert call(3) == ERR_SHAPE           # max_end below T
    assert call(8, cp=None) == ERR_NULL
    assert call(8, idx=FAKE) == ERR_UNSUPPORTED   # index keys without the indexer
    assert call(8, B=0) == OK


def test_dsa_and_stage_validation():
    L = gm.lib()
    d = gm.make_dims(K3)
    assert L.dsa_index_topk(ctypes.byref(gm.make_dims(TINY)), FAKE, FAKE, FAKE, 10, FAKE, 5, 1, FAKE, FAKE,
                            None, FAKE, 1 << 20, None) == ERR_UNSUPPORTED
    assert L.dsa_index_topk(ctypes.byref(d), FAKE, FAKE, FAKE, 10, FAKE, 11, 1, FAKE, FAKE, None, FAKE,
                            1 << 20, None) == ERR_CAPACITY
    assert L.dsa_index_topk(ctypes.byref(d), FAKE, FAKE, FAKE, 100, FAKE, 90, 2, FAKE, FAKE, None, FAKE,
                            100, None) == ERR_WORKSPACE
    assert L.mla_gemm(FAKE, 30, FAKE, 4, 4, 30, FAKE, 4, 0, None) == ERR_SHAPE   # K not a multiple of 8
    assert L.mla_gemm(FAKE, 32, FAKE, 4, 4, 32, FAKE, 4, 5, None) == ERR_UNSUPPORTED
    assert L.mla_rmsnorm(None, 64, FAKE, 4, 64, 1e-6, FAKE, 64, None) == ERR_NULL
    c = _cache()
    assert L.mla_decode_attention(ctypes.byref(d), FAKE, ctypes.byref(c), FAKE, 101, 2, 0, FAKE, None, FAKE,
                                  1 << 40, None) == ERR_CAPACITY
    assert L.mla_decode_attention(ctypes.byref(d), FAKE, ctypes.byref(c), FAKE, 50, 2, 0, FAKE, None, FAKE,
                                  16, None) == ERR_WORKSPACE
    assert L.mla_expanded_attention(ctypes.byref(d), FAKE, ctypes.byref(_cache(v=None)), FAKE, 10, 2, FAKE,
                                    None, None) == ERR_NULL


def test_prefill_sparse_validation():
    L = gm.lib()
    d = gm.make_dims(K3)
    w = gm.MlaWeights(*([FAKE] * 13))
    call = lambda dims=d, c=None, ws_bytes=1 << 40, B=2, T=10, max_end=50, ww=w: L.mla_prefill_sparse(  # noqa: E731
        ctypes.byref(dims), ctypes.byref(ww), ctypes.byref(c or _cache(idx=FAKE)), FAKE, max_end, FAKE, B, T, FAKE,
        0, None, None, None, FAKE, ws_bytes, None)
    assert call(dims=gm.make_dims(K3.replace(n_idx_heads=0))) == ERR_UNSUPPORTED   # needs the indexer
    assert call(c=_cache(idx=None)) == ERR_NULL
    assert call(ww=_weights()) == ERR_NULL                                            # no index weights
    assert call(c=_cache(idx=FAKE, T_cap=40)) == ERR_CAPACITY
    assert call(ws_bytes=100) == ERR_WORKSPACE
    assert call(B=0) == OK
    assert gm.workspace_bytes_prefill_sparse(d, 2, 10, 50) > gm.workspace_bytes(d, 2, 10, 50)
    assert gm.workspace_bytes_prefill_sparse(gm.make_dims(K3.replace(n_idx_heads=0)), 2, 10, 50) == 0


def test_cache_format_validation():
    """FP8 caches exist for the K3 shape only; unknown formats are rejected before any launch."""
    L = gm.lib()
    call = lambda dims, cc: L.kv_append(ctypes.byref(gm.make_dims(dims)), ctypes.byref(cc), FAKE, 8, 2, 4,  # noqa: E731
                                        FAKE, FAKE, None, None, None, None)
    c = _cache(T_cap=16)
    c.latent_format = gm.CACHE_FP8
    assert call(TINY, c) == ERR_UNSUPPORTED
    c.latent_format = 7
    assert call(K3, c) == ERR_UNSUPPORTED
    c.latent_format, c.idx_format = gm.CACHE_BF16, 2
    assert call(K3, c) == ERR_UNSUPPORTED
    # and the decode entry points see the same check
    c2 = _cache()
    c2.latent_format = gm.CACHE_FP8
    assert _call_decode(gm.make_dims(TINY), c2) == ERR_UNSUPPORTED
    assert L.dsa_index_topk_fp8(ctypes.byref(gm.make_dims(K3)), FAKE, FAKE, FAKE, None, 10, FAKE, 5, 1, FAKE,
                                FAKE, None, FAKE, 1 << 30, None) == ERR_NULL


def test_paged_cache_validation():
    """Page tables: page_size a multiple of 32, T_cap = page_size * max_blocks, no expanded
    cache, K3 shape; dense prefill (expanded attention) refuses them."""
    L = gm.lib()
    d = gm.make_dims(K3)

    def paged(page=64, blocks=4, pages=10, k=None, v=None):
        c = _cache(k=k, v=v, T_cap=page * blocks)
        c.block_table, c.page_size, c.max_blocks, c.n_pages = FAKE, page, blocks, pages
        return c

    call = lambda cc, dims=d: L.kv_append(ctypes.byref(dims), ctypes.byref(cc), FAKE, 8, 2, 4,  # noqa: E731
                                          FAKE, FAKE, None, None, None, None)
    assert call(paged(page=48, blocks=5)) == ERR_SHAPE
    c = paged()
    c.T_cap = 300
    assert call(c) == ERR_SHAPE
    assert call(paged(pages=0)) == ERR_SHAPE
    assert call(paged(k=FAKE, v=FAKE)) == ERR_UNSUPPORTED
    assert call(paged(), gm.make_dims(TINY)) == ERR_UNSUPPORTED
    assert _call_prefill(d, paged(k=None, v=None), max_end=50) == ERR_UNSUPPORTED


def test_index_projections_validation():
    L = gm.lib()
    d = gm.make_dims(K3)
    w = gm.MlaWeights(*([FAKE] * 13))
    call = lambda dims=d, ww=w, M=4, q=FAKE, ws_bytes=1 << 40: L.mla_index_projections(  # noqa: E731
        ctypes.byref(dims), ctypes.byref(ww), FAKE, M, q, FAKE, FAKE, FAKE, ws_bytes, None)
    assert call(dims=gm.make_dims(K3.replace(n_idx_heads=0))) == ERR_UNSUPPORTED   # needs the indexer
    assert call(dims=gm.make_dims(TINY)) == ERR_UNSUPPORTED
    assert call(ww=_weights()) == ERR_NULL                                            # no index weights
    assert call(q=None) == ERR_NULL
    assert call(M=-1) == ERR_SHAPE
    assert call(M=0) == OK
    assert call(ws_bytes=100) == ERR_WORKSPACE
    assert call(ws_bytes=gm.workspace_bytes(d, 4, 1, 1, gm.PATH_SPARSE) - 1) == ERR_WORKSPACE


def test_debug_scores_validation():
    L = gm.lib()
    d = gm.make_dims(K3)

    def call(q, k, hk, B, Tq, Tk, D, out):
        return L.mla_debug_scores(ctypes.byref(d), q, k, hk, B, Tq, Tk, D, out, None)
    assert call(FAKE, FAKE, 96, 1, 4, 4, 100, FAKE) == ERR_SHAPE        # D neither d_qk nor d_latent
    assert call(FAKE, FAKE, 2, 1, 4, 4, 192, FAKE) == ERR_SHAPE         # key heads neither 1 nor H
    assert call(FAKE, FAKE, 96, 1, 1024, 1024, 192, FAKE) == ERR_SHAPE  # more logits than the stage writes
    assert call(FAKE, FAKE, 96, 1, 4, 4, 192, None) == ERR_NULL
    assert call(FAKE + 2, FAKE, 1, 1, 4, 4, 576, FAKE) == ERR_SHAPE     # q not 16-byte aligned
    assert call(None, None, 96, 0, 4, 4, 192, None) == 0                # empty: nothing launched


def test_debug_flags_entry():
    """mla_debug_flags: NULL outputs are refused; the build under test reports whether it has the
    device-side checks (the normal build: no, and no bits; it touches no device to say so)."""
    L = gm.lib()
    flags, built = ctypes.c_uint32(7), ctypes.c_int32(7)
    assert L.mla_debug_flags(None, ctypes.byref(built), None) == ERR_NULL
    assert L.mla_debug_flags(ctypes.byref(flags), None, None) == ERR_NULL
    if os.path.basename(gm.LIB_PATH) == "libgmla_debug.so":
        pytest.skip("the debug build reads its flags from the device")
    assert L.mla_debug_flags(ctypes.byref(flags), ctypes.byref(built), None) == OK
    assert (flags.value, built.value) == (0, 0)


def test_launch_logging():
    """GMLA_LOG=1: an entry point writes one line naming itself, its sizes and the stream to
    stderr on entry, before validation (so a refused call is logged too); unset, nothing."""
    import subprocess
    import sys
    code = ("import ctypes, gated_mla_kv_amd as gm; L = gm.lib(); "
            "print(L.mla_gemm(None, 8, None, -1, 16, 8, None, 16, 0, None)); "
            "print(L.kv_append(None, None, None, 5, 2, 3, None, None, None, None, None, None))")
    env = dict(os.environ, PYTHONPATH=ROOT)
    for on in (True, False):
        env["GMLA_LOG"] = "1" if on else "0"
        r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stderr
        assert r.stdout.split() == [str(ERR_SHAPE), str(ERR_NULL)]
        lines = [ln for ln in r.stderr.splitlines() if ln.startswith("[gmla]")]
        if on:
            assert len(lines) == 2, r.stderr
            assert lines[0].startswith("[gmla] mla_gemm M=-1 N=16 K=8 lda=8 ldo=16 out_dtype=0 stream=")
            assert lines[1].startswith("[gmla] kv_append B=2 T=3 max_end=5 stream=")
        else:
            assert lines == [], r.stderr
