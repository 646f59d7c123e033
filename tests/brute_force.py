"""Explicit-loop float64 brute force of the Gated MLA layer and the DSA index score.

Used only to pin the oracle on tiny inputs. It is written independently of ``oracle`` in a
different style (scalar Python loops over the pages' equations, softmax as exp over an explicit
sum without subtracting the maximum, ReLU written as (z + |z|) / 2) so that a dropped term, a
wrong index or a transposed operand in either one shows up as a disagreement.

Equations: "Kimi K3" attention code page (KimiRMSNorm, KimiMLAAttention.forward) and the K3.1
Gated DSA blog, eqs. (2)-(10).
"""
import math


def _matvec(W, x):
    """y[o] = sum_i W[o][i] x[i]  (nn.Linear, W in [out, in])."""
    return [sum(W[o][i] * x[i] for i in range(len(x))) for o in range(len(W))]


def _rms(v, g, eps):
    ms = sum(a * a for a in v) / len(v)
    return [g[i] * v[i] / math.sqrt(ms + eps) for i in range(len(v))]


def brute_layer(x, W, dims):
    """Prefill of T tokens of ONE sequence from an empty cache. x: list of T lists.

    Returns y as a list of T lists. Every weight is a list of lists in [out, in] layout.
    """
    H, dn, ds, dv, L = dims.n_heads, dims.d_nope, dims.d_shared, dims.d_v, dims.kv_lora
    dqk = dn + ds
    T = len(x)
    q, k, v = [], [], []
    for t in range(T):
        cq = _rms(_matvec(W["w_q_a"], x[t]), W["g_q_a"], dims.rms_eps)
        qf = _matvec(W["w_q_b"], cq)                          # H * dqk
        q.append([[qf[h * dqk + e] for e in range(dqk)] for h in range(H)])
        ckv = _matvec(W["w_kv_a"], x[t])                      # L + ds
        c = _rms(ckv[:L], W["g_kv_a"], dims.rms_eps)
        r = ckv[L:]
        kv = _matvec(W["w_kv_b"], c)                          # H * (dn + dv)
        k.append([[kv[h * (dn + dv) + e] for e in range(dn)] + list(r) for h in range(H)])
        v.append([[kv[h * (dn + dv) + dn + e] for e in range(dv)] for h in range(H)])
    scale = 1.0 / math.sqrt(dqk)
    ys = []
    for t in range(T):
        g = _matvec(W["w_g"], x[t])
        u = [0.0] * (H * dv)
        for h in range(H):
            w = [math.exp(scale * sum(q[t][h][e] * k[j][h][e] for e in range(dqk)))
                 for j in range(t + 1)]
            den = sum(w)
            for d in range(dv):
                z = sum(w[j] * v[j][h][d] for j in range(t + 1)) / den
                gate = 1.0 / (1.0 + math.exp(-g[h * dv + d])) if dims.use_gate else 1.0
                u[h * dv + d] = z * gate
        ys.append(_matvec(W["w_o"], u))
    return ys


def brute_index_scores(qi, a, keys, t):
    """Eq. (5) with ReLU(z) = (z + |z|)/2: I_s = sum_h a_h relu(q_h . k_s) / (sqrt(nh) sqrt(d))."""
    nh, d = len(qi), len(qi[0])
    out = []
    for s in range(t):
        acc = 0.0
        for h in range(nh):
            z = sum(qi[h][e] * keys[s][e] for e in range(d))
            acc += a[h] * (z + abs(z)) / 2.0
        out.append(acc / (math.sqrt(nh) * math.sqrt(d)))
    return out


def brute_index_projections(x, W, dims):
    """The indexer's projections of ONE token x (a list of hidden values), eqs. (2)-(4) of the
    K3.1 Gated DSA blog, as scalar loops:
      q^I: the normalised query latent c^Q (the main query path's RMSNorm with its gain) times
           W_q^I, read head-major: q[h][e] = (W_q^I c^Q)[h * d_idx + e]          (eq. (2))
      k^I: LayerNorm of W_k^I x with the population variance, then gain and bias    (eq. (3))
      a:   W_a^I x, used raw (no sigmoid, no softmax)                               (eq. (4))
    Returns (q [n_idx][d_idx], k [d_idx], a [n_idx])."""
    nh, d = dims.n_idx_heads, dims.d_idx
    cq = _rms(_matvec(W["w_q_a"], x), W["g_q_a"], dims.rms_eps)
    qf = _matvec(W["w_idx_q"], cq)
    q = [[qf[h * d + e] for e in range(d)] for h in range(nh)]
    v = _matvec(W["w_idx_k"], x)
    mean = sum(v) / d
    var = sum((e - mean) * (e - mean) for e in v) / d
    k = [(v[e] - mean) / math.sqrt(var + dims.ln_eps) * W["g_idx_k"][e] + W["b_idx_k"][e] for e in range(d)]
    a = _matvec(W["w_idx_w"], x)
    return q, k, a


def brute_attention_logits(q, k, scale):
    """s[b][h][i][j] = scale * sum_d q[b][i][h][d] * k[b][hk][j][d], where hk = h, or 0 when k
    holds one key row per position for every head. q: nested lists [B][T][H][D]; k: [B][Hk][N][D]."""
    out = []
    for b in range(len(q)):
        per_head = []
        for h in range(len(q[b][0])):
            hk = 0 if len(k[b]) == 1 else h
            rows = []
            for i in range(len(q[b])):
                row = []
                for j in range(len(k[b][hk])):
                    acc = 0.0
                    for e in range(len(q[b][i][h])):
                        acc += q[b][i][h][e] * k[b][hk][j][e]
                    row.append(scale * acc)
                rows.append(row)
            per_head.append(rows)
        out.append(per_head)
    return out
