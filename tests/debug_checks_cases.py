"""Cases for the device-side bound checks (run by test_gpu_debug_checks.py in-process on the
normal library and, with GMLA_LIB set, in a child process on the debug-checks build).

Each case runs kv_append or dsa_index_topk on seeded inputs and returns its outputs as numpy
arrays, with the flags mla_debug_flags reports right after it. The out-of-range cases are ones
the host cannot see (token positions and page-table entries live in device memory); every kernel
skips or clamps such writes, so each case reads and writes only memory it owns.

Run as a script (the child): python debug_checks_cases.py OUT.npz; it prints one JSON line with
each case's flags and whether the build has the checks."""
import json
import os
import sys

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
if os.path.dirname(HERE) not in sys.path:
    sys.path.insert(0, os.path.dirname(HERE))
if HERE not in sys.path:
    sys.path.insert(0, HERE)

import gated_mla_kv_amd as gm  # noqa: E402
from gated_mla_kv_amd.layer import CacheBuffers, bf16_tensor  # noqa: E402
from workloads import K3, bf16_bits  # noqa: E402


def _bf16(shape, seed):
    return bf16_tensor(bf16_bits(np.random.default_rng(seed).standard_normal(shape).astype(np.float32)), "cuda")


def _flags():
    torch.cuda.synchronize()
    return gm.mla_debug_flags()


def _append(pos, T_cap, T=4, page_size=0, n_pages=0, table=None):
    d = K3
    B = len(pos)
    cb = CacheBuffers(d, B, T_cap, expanded=page_size == 0, index=True, page_size=page_size, n_pages=n_pages,
                      block_table=table)
    c = _bf16((B, T, d.kv_lora), 1)
    r = _bf16((B, T, d.d_shared), 2)
    ik = _bf16((B, T, d.d_idx), 3)
    kn = _bf16((B, T, d.n_heads, d.d_nope), 4) if page_size == 0 else None
    v = _bf16((B, T, d.n_heads, d.d_v), 5) if page_size == 0 else None
    p = torch.tensor(pos, dtype=torch.int32, device="cuda")
    gm.kv_append(gm.make_dims(d), cb.c, p, T_cap, B, T, c, r, kn, v, ik)
    flags = _flags()
    out = {"latent": cb.latent.view(torch.int16).cpu().numpy(), "idx": cb.idx.view(torch.int16).cpu().numpy()}
    if cb.k is not None:
        out["k"] = cb.k.view(torch.int16).cpu().numpy()
        out["v"] = cb.v.view(torch.int16).cpu().numpy()
    return out, flags


def _topk(t_vis, topk=2048):
    d = K3.replace(topk=topk)
    B = len(t_vis)
    T_cap = max(t_vis) + 5
    rng = np.random.default_rng(7)
    qi = torch.from_numpy(rng.standard_normal((B, d.n_idx_heads, d.d_idx)).astype(np.float32) * 0.1).cuda()
    a = torch.from_numpy(rng.standard_normal((B, d.n_idx_heads)).astype(np.float32)).cuda()
    keys = _bf16((B, T_cap, d.d_idx), 8)
    dims = gm.make_dims(d)
    sel = torch.empty((B, topk), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B,), dtype=torch.int32, device="cuda")
    ws = torch.empty(gm.workspace_bytes(dims, B, 1, T_cap, gm.PATH_SPARSE), dtype=torch.uint8, device="cuda")
    nv = torch.tensor(t_vis, dtype=torch.int32, device="cuda")
    gm.dsa_index_topk(dims, qi, a, keys, T_cap, nv, max(t_vis), B, sel, cnt, None, ws)
    flags = _flags()
    return {"sel": sel.cpu().numpy(), "cnt": cnt.cpu().numpy()}, flags


# name -> (runner, the bits the debug build must report)
CASES = {
    # sequence 1's last two tokens fall past T_cap = 64
    "append_past_capacity": (lambda: _append([0, 62], 64), 1),
    # sequence 1's second block maps to page 9 of a 4-page pool (clamped to page 3)
    "append_bad_page": (lambda: _append([0, 38], 64, page_size=32, n_pages=4, table=[[0, 1], [2, 9]]), 2),
    "append_in_range": (lambda: _append([3, 10], 64), 0),
    "append_paged_in_range": (lambda: _append([0, 38], 64, page_size=32, n_pages=4, table=[[0, 1], [2, 3]]), 0),
    "topk_chunked": (lambda: _topk([6000, 5000]), 0),    # the count / select / compact kernels
    "topk_one_row": (lambda: _topk([3000, 2500]), 0),    # the one-workgroup row kernel
}


def run_all():
    flags, arrays, built = {}, {}, None
    gm.mla_debug_flags()  # start from a clear word
    for name, (fn, _) in CASES.items():
        out, (f, b) = fn()
        flags[name] = f
        built = b
        for k, v in out.items():
            arrays[f"{name}.{k}"] = v
    return flags, arrays, built


if __name__ == "__main__":
    flags, arrays, built = run_all()
    np.savez(sys.argv[1], **arrays)
    print(json.dumps({"lib": os.path.basename(gm.LIB_PATH), "built": built, "flags": flags}), flush=True)
