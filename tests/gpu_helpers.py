"""Helpers shared by the GPU parity tests: device uploads of seeded bf16 data and the tolerance
checks.

Tolerances (written out here, used by every parity test):
* floating-point outputs: max |got - ref| <= 2e-2 * rms(ref row) per output row (one token's
  feature vector or one (b, h) row), plus half a bf16 ulp of ref when the output is bf16;
* scores and log-sum-exps: |got - ref| <= 1e-3 * (|ref| + rms(ref row));
* cache appends and selected indices: bit-exact (selection boundary rule in the DSA tests).
"""
import numpy as np
import torch

from workloads import bf16_bits, bf16_bits_to_f32

ROW_TOL = 2e-2
SCORE_TOL = 1e-3


def dev_bf16(bits):
    from gated_mla_kv_amd.layer import bf16_tensor
    return bf16_tensor(bits, "cuda")


def f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def rand_bf16(shape, seed, std=1.0):
    rng = np.random.default_rng(seed)
    return bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def half_ulp_bf16(ref):
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 8), 0.0)


def check_rows(got, ref, what, tol=ROW_TOL, bf16_out=False):
    """Max per-row error relative to the row rms of ref (rows = all but the last axis)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    g2 = got.reshape(-1, ref.shape[-1])
    r2 = ref.reshape(-1, ref.shape[-1])
    rms = np.sqrt(np.mean(r2 * r2, axis=1, keepdims=True))
    rms = np.where(rms > 0, rms, 1e-30)
    allow = tol * rms + (half_ulp_bf16(r2) if bf16_out else 0.0)
    err = np.abs(g2 - r2)
    bad = err > allow
    worst = float(np.max(err / rms))
    assert not bad.any(), f"{what}: {bad.sum()} elements over tolerance, worst {worst:.3e} x rms_row"
    return worst


def check_scores(got, ref, what, tol=SCORE_TOL):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite"
    r2 = ref.reshape(-1, ref.shape[-1]) if ref.ndim > 1 else ref.reshape(1, -1)
    g2 = got.reshape(r2.shape)
    rms = np.sqrt(np.mean(r2 * r2, axis=1, keepdims=True))
    err = np.abs(g2 - r2)
    allow = tol * (np.abs(r2) + rms)
    bad = err > allow
    assert not bad.any(), f"{what}: {bad.sum()} over tolerance, worst {float(np.max(err / (np.abs(r2) + rms))):.3e}"


def i32(a):
    return torch.tensor(np.asarray(a, np.int32), device="cuda")


def index_score_ulp_bound(qi, a, keys):
    """Per position s, how far the index score I_s (eq. (5)) can move when every element of the
    bf16 index query sits one bf16 ulp (<= 2^-7 |q|) from the oracle's: scale * sum_h |a_h|
    sum_d 2^-7 |q_hd| |k_sd| (ReLU is 1-Lipschitz). End to end, the GPU rounds q^I to bf16 from
    its own fp32 c^Q and the oracle from its float64 one, so single elements may round apart."""
    q = np.abs(np.asarray(qi, np.float64))
    k = np.abs(np.asarray(keys, np.float64))
    scale = 1.0 / np.sqrt(q.shape[0] * q.shape[1])
    return scale * 2.0 ** -7 * (np.abs(np.asarray(a, np.float64)) @ (q @ k.T))


def check_selection_end_to_end(got, I, k, bound):
    """The GPU's top-k set against the oracle's scores I: equal to select_topk(I, k) except for
    swapped positions whose scores lie within 1e-4 plus their ulp bounds of the k-th largest.
    Kernel-boundary tests (identical index inputs) use the plain 1e-4 rule instead."""
    import oracle as O
    exp = O.select_topk(I, k)
    order = np.argsort(-I, kind="stable")
    tau_pos = order[k - 1]
    tau = I[tau_pos]
    extra, missing = np.setdiff1d(got, exp), np.setdiff1d(exp, got)
    assert len(extra) == len(missing), (extra, missing)
    for s_ in np.concatenate([extra, missing]):
        assert abs(I[s_] - tau) < 1e-4 + bound[s_] + bound[tau_pos], (s_, I[s_], tau, bound[s_], bound[tau_pos])
    return exp
