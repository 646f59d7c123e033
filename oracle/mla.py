"""Float64 oracle of the Gated MLA layer (Kimi K3) and the Gated DSA decode step (Kimi K3.1).

TEST INFRASTRUCTURE: see the package docstring. Nothing on the product path may import this.

Sources (the pages):
* [KV]  "Kimi K3 > Gated MLA > KV cache" (atlas.klimoza.dev, kimi-k3 attention/kv-cache):
        cache shapes k [B, 96, T, 192], v [B, 96, T, 128], bfloat16, grown by concatenation
        along the position axis in ``update``.
* [ATT] "Kimi K3" attention code page (atlas.klimoza.dev, kimi-k3 attention/key-value/x):
        ``KimiRMSNorm``, ``KimiMLAAttention.__init__`` and ``forward`` with the output gate.
* [SK]  "Kimi K3 - Take the shared key part" (atlas.klimoza.dev, shared-key-split): the last
        64 features of the joint down-projection are a key part every head shares, unrotated.
* [K2]  "Kimi K2 > Latent attention > KV cache" (atlas.klimoza.dev, kimi-k2 kv-cache): the
        eager form ``softmax(q k^T * scale) v`` and the 20,480-vs-576 figure.
* [DSA] "Kimi K3 model structure (11): K3.1 Pro's Gated DSA from the inference code"
        (blog.javazero.top): indexer eqs. (2)-(6), MLA eqs. (7)-(10), the note on latent
        absorption, the per-query pseudocode and the cache table.

Readings where the pages are silent or garbled (each is listed with its support in the
design notes of the repository):
* The attention call is missing from ``forward``; it is read as eager causal softmax
  attention with scale = q_head_dim^-1/2 and no dropout ([ATT] ``self.scaling``,
  ``is_causal``; [DSA] eq. (9); [K2] eager form).
* Query i of a call sits at absolute position P + i (P cached positions) and sees 0..P+i.
* The output gate is on (K3 keeps the sigmoid output gate, [DSA] comparison table and
  eq. (10)); its input is the attention input x.
* RMSNorm and LayerNorm are computed exactly; the gain multiplies the normalised value.
* The index-key LayerNorm has a gain and a bias ([DSA] eq. (3) and the text after it); its
  eps is not printed and is taken as 1e-6.
* Top-k ties go to the lower position; -0.0 and +0.0 are equal; the selected set is returned
  in ascending position order.
"""
from __future__ import annotations

import numpy as np

from . import fp8

__all__ = [
    "round_to_bf16", "rms_norm", "layer_norm", "linear", "sigmoid", "softmax_scale",
    "Cache", "query_path", "kv_down_path", "kv_up", "expand_keys", "attention_expanded", "attention_logits",
    "absorbed_query", "attention_absorbed", "value_up", "gate_output", "layer_forward",
    "index_projections", "index_scores", "select_topk", "attention_absorbed_subset",
    "dsa_decode_step", "dsa_prefill", "cache_values_per_position",
]

F64 = np.float64


# ---------------------------------------------------------------------------------------------
# Elementary operations
# ---------------------------------------------------------------------------------------------

def round_to_bf16(a) -> np.ndarray:
    """Round to the nearest bfloat16 value (8 significant bits, ties to even), as float64.

    Storage format of the caches: [KV] says the cache is held in bfloat16, the checkpoint's
    type; [DSA]'s cache table counts the index keys in the same 2-byte type.
    """
    a = np.asarray(a, dtype=F64)
    m, e = np.frexp(a)                     # a = m * 2**e with 0.5 <= |m| < 1
    m = np.rint(m * 256.0) / 256.0         # 8 significant bits; rint rounds half to even
    return np.ldexp(m, e)


def rms_norm(v, gain, eps: float) -> np.ndarray:
    """KimiRMSNorm ([ATT]): v * rsqrt(mean(v^2) + eps), then times the gain (last axis)."""
    v = np.asarray(v, dtype=F64)
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return (v / np.sqrt(ms + eps)) * np.asarray(gain, dtype=F64)


def layer_norm(v, gain, bias, eps: float) -> np.ndarray:
    """LayerNorm with gain and bias over the last axis ([DSA] eq. (3) and the text after it).

    Normalises by the population variance, the textbook LayerNorm.
    """
    v = np.asarray(v, dtype=F64)
    mu = np.mean(v, axis=-1, keepdims=True)
    var = np.mean((v - mu) ** 2, axis=-1, keepdims=True)
    return (v - mu) / np.sqrt(var + eps) * np.asarray(gain, dtype=F64) + np.asarray(bias, dtype=F64)


def linear(x, w) -> np.ndarray:
    """nn.Linear without bias: x W^T, with W in the [out, in] layout ([ATT] __init__)."""
    return np.asarray(x, dtype=F64) @ np.asarray(w, dtype=F64).T


def sigmoid(z) -> np.ndarray:
    z = np.asarray(z, dtype=F64)
    return 1.0 / (1.0 + np.exp(-z))


def softmax_scale(dims) -> float:
    """scale = q_head_dim ** -0.5 with q_head_dim = nope + shared ([ATT] ``self.scaling``)."""
    return float((dims.d_nope + dims.d_shared) ** -0.5)


def _w(weights, name) -> np.ndarray:
    return np.asarray(weights[name], dtype=F64)


# ---------------------------------------------------------------------------------------------
# Caches
# ---------------------------------------------------------------------------------------------

class Cache:
    """The caches of one layer for B sequences advancing together.

    * k [B, H, T, d_nope + d_shared] and v [B, H, T, d_v]: the expanded KV cache ([KV]).
    * latent [B, T, kv_lora + d_shared]: the normalised latent c_s and the shared key r_s,
      576 values per position at K3 ([DSA] eq. (7) and the cache table).
    * idx [B, T, d_idx]: the index keys of the Gated DSA indexer ([DSA] eq. (3), cache table).

    ``append`` concatenates along the position axis, as the page's ``update`` does. With
    ``store_bf16`` the stored values are rounded to bfloat16, the cache type the pages give.
    With ``expanded=False`` only the latent and index caches are kept (the absorbed and the
    sparse paths read nothing else).

    With ``fp8_latent`` / ``fp8_index`` the latent c_s / the index keys are held in the FP8
    formats of the [DSA] cache section (``oracle.fp8``): the bf16 value is quantized, and
    ``latent`` / ``idx`` hold what the cache reads back (``fp8.latent_read_back``,
    ``fp8.dequantize_index_keys``); the codes and
    scales are kept in ``latent_codes``, ``latent_scales``, ``idx_codes``, ``idx_scales``.
    """

    def __init__(self, dims, B: int, store_bf16: bool = True, expanded: bool = True,
                 fp8_latent: bool = False, fp8_index: bool = False):
        H = dims.n_heads
        self.dims = dims
        self.store_bf16 = store_bf16
        self.expanded = expanded
        self.fp8_latent = fp8_latent
        self.fp8_index = fp8_index
        self.latent_codes = np.zeros((B, 0, dims.kv_lora), np.uint8)
        self.latent_scales = np.zeros((B, 0, dims.kv_lora // fp8.latent_block(dims)), np.float32)
        self.idx_codes = np.zeros((B, 0, max(dims.d_idx, 0)), np.uint8)
        self.idx_scales = np.zeros((B, 0, 1), np.float32)
        self.k = np.zeros((B, H, 0, dims.d_nope + dims.d_shared), F64)
        self.v = np.zeros((B, H, 0, dims.d_v), F64)
        self.latent = np.zeros((B, 0, dims.kv_lora + dims.d_shared), F64)
        self.idx = np.zeros((B, 0, max(dims.d_idx, 0)), F64)

    @property
    def length(self) -> int:
        return self.latent.shape[1]

    def _store(self, a):
        a = np.asarray(a, dtype=F64)
        return round_to_bf16(a) if self.store_bf16 else a

    def append(self, c, r, k=None, v=None, idx_k=None):
        """Append T new positions: c [B,T,kv_lora], r [B,T,d_shared], k [B,H,T,d_qk],
        v [B,H,T,d_v] (ignored without the expanded cache), idx_k [B,T,d_idx] or None."""
        c = self._store(c)
        if self.fp8_latent:
            codes, scales = fp8.quantize_latent(c, self.dims)
            self.latent_codes = np.concatenate([self.latent_codes, codes], 1)
            self.latent_scales = np.concatenate([self.latent_scales, scales], 1)
            c = fp8.latent_read_back(codes, scales)
        self.latent = np.concatenate([self.latent, np.concatenate([c, self._store(r)], -1)], 1)
        if self.expanded:
            self.k = np.concatenate([self.k, self._store(k)], 2)
            self.v = np.concatenate([self.v, self._store(v)], 2)
        if idx_k is not None:
            ik = self._store(idx_k)
            if self.fp8_index:
                codes, scales = fp8.quantize_index_keys(ik)
                self.idx_codes = np.concatenate([self.idx_codes, codes], 1)
                self.idx_scales = np.concatenate([self.idx_scales, scales], 1)
                ik = fp8.dequantize_index_keys(codes, scales)
            self.idx = np.concatenate([self.idx, ik], 1)

    def set_prefix(self, latent, idx=None):
        """Start from given latent rows (already in the cache type) with no expanded rows.
        With the FP8 formats the rows are given as bf16 values and quantized here."""
        latent = np.asarray(latent, dtype=F64)
        if self.fp8_latent:
            L = self.dims.kv_lora
            self.latent_codes, self.latent_scales = fp8.quantize_latent(latent[..., :L], self.dims)
            latent = np.concatenate([fp8.latent_read_back(self.latent_codes, self.latent_scales),
                                     latent[..., L:]], -1)
        self.latent = latent
        if idx is not None:
            idx = np.asarray(idx, dtype=F64)
            if self.fp8_index:
                self.idx_codes, self.idx_scales = fp8.quantize_index_keys(idx)
                idx = fp8.dequantize_index_keys(self.idx_codes, self.idx_scales)
            self.idx = idx


def cache_values_per_position(dims) -> dict:
    """Values one position adds to each cache, counted on arrays built by ``Cache.append``."""
    d = dims
    c = Cache(d, 1, store_bf16=False)
    H = d.n_heads
    c.append(np.zeros((1, 1, d.kv_lora)), np.zeros((1, 1, d.d_shared)),
             np.zeros((1, H, 1, d.d_nope + d.d_shared)), np.zeros((1, H, 1, d.d_v)),
             np.zeros((1, 1, d.d_idx)) if d.d_idx else None)
    return {"expanded": c.k.size + c.v.size, "latent": c.latent.size, "index": c.idx.size}


# ---------------------------------------------------------------------------------------------
# Projections ([ATT] forward; [DSA] eqs. (2), (7), (8))
# ---------------------------------------------------------------------------------------------

def query_path(x, w, dims):
    """Query through the low-rank latent: c^Q = RMSNorm(x W_qa^T) * g_qa; q = c^Q W_qb^T.

    q is viewed per head as [.., H, nope + shared] and split into the nope part and the shared
    part; nothing rotates it ([ATT] forward; [DSA] eq. (2)). Returns (cQ, q_nope, q_shared).
    """
    cq = rms_norm(linear(x, _w(w, "w_q_a")), _w(w, "g_q_a"), dims.rms_eps)
    q = linear(cq, _w(w, "w_q_b"))
    q = q.reshape(*q.shape[:-1], dims.n_heads, dims.d_nope + dims.d_shared)
    return cq, q[..., :dims.d_nope], q[..., dims.d_nope:]


def kv_down_path(x, w, dims):
    """Joint down-projection split into the KV latent and the shared key part.

    [c_bar ; r] = x W_kva^T; c = RMSNorm(c_bar) * g_kva; r is neither normalised nor rotated
    ([ATT] forward; [SK]; [DSA] eq. (7)). Returns (c, r).
    """
    ckv = linear(x, _w(w, "w_kv_a"))
    c_bar, r = ckv[..., :dims.kv_lora], ckv[..., dims.kv_lora:]
    return rms_norm(c_bar, _w(w, "g_kv_a"), dims.rms_eps), r


def kv_up(c, w, dims):
    """Per-head keys and values from the latent: c W_kvb^T viewed [.., H, nope + v], split
    into k_nope and v ([ATT] forward; [DSA] eq. (8)). Returns (k_nope, v)."""
    kv = linear(c, _w(w, "w_kv_b"))
    kv = kv.reshape(*kv.shape[:-1], dims.n_heads, dims.d_nope + dims.d_v)
    return kv[..., :dims.d_nope], kv[..., dims.d_nope:]


def expand_keys(k_nope, r):
    """k_h = [k_nope_h ; r]: the shared key r is given unchanged to every head ([SK]).

    k_nope [B,T,H,nope], r [B,T,shared] -> k [B,H,T,nope+shared] (the cache layout of [KV]).
    """
    B, T, H, _ = k_nope.shape
    r_all = np.broadcast_to(r[:, :, None, :], (B, T, H, r.shape[-1]))
    return np.concatenate([k_nope, r_all], -1).transpose(0, 2, 1, 3)


# ---------------------------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------------------------

def attention_expanded(q, k, v, scale: float, offset: int):
    """Causal softmax attention over the expanded cache ([DSA] eq. (9) over all s <= t).

    q [B,T,H,dqk] (query i at absolute position offset + i), k [B,H,N,dqk], v [B,H,N,dv].
    Returns z [B,T,H,dv] and lse [B,H,T] (natural log of the softmax denominator, with the
    scaled logits).
    """
    B, T, H, _ = q.shape
    N = k.shape[2]
    qh = q.transpose(0, 2, 1, 3)                       # [B,H,T,dqk]
    s = np.einsum("bhtd,bhnd->bhtn", qh, k) * scale      # [B,H,T,N]
    pos = offset + np.arange(T)
    mask = np.arange(N)[None, :] > pos[:, None]          # key after the query: not visible
    s = np.where(mask[None, None], -np.inf, s)
    m = np.max(s, axis=-1, keepdims=True)
    p = np.exp(s - m)
    l = np.sum(p, axis=-1, keepdims=True)
    z = np.einsum("bhtn,bhnd->bhtd", p / l, v)
    lse = (m + np.log(l))[..., 0]
    return z.transpose(0, 2, 1, 3), lse


def attention_logits(q, k, scale: float):
    """The attention logits before the mask and the softmax: s[b,h,i,j] = (q_{b,i,h} . k_{b,h,j})
    * scale, the argument of the softmax in [DSA] eq. (9) ([K2] eager form q k^T * scale).

    q [B,T,H,D]; k [B,H,N,D] (per-head keys, the expanded form) or [B,1,N,D] (one row per
    position shared by every head: the latent [c ; r] of the absorbed form). Returns s [B,H,T,N]
    for every (i, j), with no mask.
    """
    B, T, H, D = q.shape
    kk = np.broadcast_to(k, (B, H) + k.shape[2:])
    return np.einsum("bthd,bhnd->bhtn", q, kk) * scale


def absorbed_query(q_nope, q_shared, w, dims):
    """Latent absorption ([DSA], the note after eq. (10)): W^K_h moves to the query side.

    W_kvb viewed [H, nope + v, kv_lora]: W^K_h = rows [0, nope), W^V_h = rows [nope, nope+v).
    q~_h = [ (W^K_h)^T q_nope_h ; q_shared_h ] in R^(kv_lora + shared).
    """
    W = _w(w, "w_kv_b").reshape(dims.n_heads, dims.d_nope + dims.d_v, dims.kv_lora)
    WK = W[:, :dims.d_nope, :]
    qc = np.einsum("...hi,hic->...hc", q_nope, WK)
    return np.concatenate([qc, q_shared], -1)


def attention_absorbed(q_tilde, latent, scale: float, offset: int, dims):
    """Scores in the latent space: s_j = q~_h . [c_j ; r_j] * scale over j <= position;
    o_h = sum_j p_j c_j (kv_lora features). Equal to eq. (9) with k_h = [W^K_h c ; r].

    q_tilde [B,T,H,L+S], latent [B,N,L+S]. Returns o [B,T,H,L] and lse [B,H,T].
    """
    B, T, H, _ = q_tilde.shape
    N = latent.shape[1]
    s = np.einsum("bthc,bnc->bhtn", q_tilde, latent) * scale
    pos = offset + np.arange(T)
    mask = np.arange(N)[None, :] > pos[:, None]
    s = np.where(mask[None, None], -np.inf, s)
    m = np.max(s, axis=-1, keepdims=True)
    p = np.exp(s - m)
    l = np.sum(p, axis=-1, keepdims=True)
    o = np.einsum("bhtn,bnc->bthc", p / l, latent[..., :dims.kv_lora])
    return o, (m + np.log(l))[..., 0]


def value_up(o, w, dims):
    """z_h = W^V_h o_h: the value of each head recovered from the latent-space output."""
    W = _w(w, "w_kv_b").reshape(dims.n_heads, dims.d_nope + dims.d_v, dims.kv_lora)
    WV = W[:, dims.d_nope:, :]
    return np.einsum("...hc,hdc->...hd", o, WV)


def gate_output(z, x, w, dims):
    """Output gate and projection ([ATT] forward; [DSA] eq. (10)).

    u[.., h*dv + d] = z_h[d] * sigmoid(x W_g^T)[.., h*dv + d]; y = u W_o^T.
    Returns (u, y). Without the gate, u is the concatenated head outputs.
    """
    zc = z.reshape(*z.shape[:-2], dims.n_heads * dims.d_v)
    if dims.use_gate:
        u = zc * sigmoid(linear(x, _w(w, "w_g")))
    else:
        u = zc
    return u, linear(u, _w(w, "w_o"))


def layer_forward(x, w, cache: Cache, dims, form: str = "expanded"):
    """One call of the Gated MLA layer on new tokens x [B,T,hidden] ([ATT] forward).

    Projects queries, keys and values, appends the new positions to ``cache``, attends
    causally over all cached positions and applies the output gate and o_proj.
    form="expanded" attends over the expanded cache; form="absorbed" in the latent space.
    Returns (y [B,T,hidden], extras dict of intermediates).
    """
    x = np.asarray(x, dtype=F64)
    P = cache.length
    cq, q_nope, q_shared = query_path(x, w, dims)
    c, r = kv_down_path(x, w, dims)
    # Each head's key and value are W^K_h c_s and W^V_h c_s of the latent as the cache holds it
    # ([DSA] eqs. (7)-(8): the cache keeps the normalised c_s and r_s; [KV]: in bfloat16).
    c_s = cache._store(c)
    k_nope, v = kv_up(c_s, w, dims)
    k = expand_keys(k_nope, cache._store(r))
    cache.append(c, r, k, v.transpose(0, 2, 1, 3))
    scale = softmax_scale(dims)
    if form == "expanded":
        q = np.concatenate([q_nope, q_shared], -1)
        z, lse = attention_expanded(q, cache.k, cache.v, scale, P)
        extras = {}
    elif form == "absorbed":
        qt = absorbed_query(q_nope, q_shared, w, dims)
        o, lse = attention_absorbed(qt, cache.latent, scale, P, dims)
        z = value_up(o, w, dims)
        extras = {"q_tilde": qt, "o_latent": o}
    else:
        raise ValueError(form)
    u, y = gate_output(z, x, w, dims)
    extras.update(cq=cq, q_nope=q_nope, q_shared=q_shared, c=c, r=r, k_nope=k_nope, v=v,
                  z=z, u=u, lse=lse)
    return y, extras


# ---------------------------------------------------------------------------------------------
# Gated DSA ([DSA] eqs. (2)-(6) and the per-query pseudocode)
# ---------------------------------------------------------------------------------------------

def index_projections(x, cq, w, dims):
    """The indexer's three projections for the current tokens.

    q^I = reshape_{n_idx x d_idx}(W_q^I c^Q)    eq. (2), c^Q the normalised query latent
    k^I = LayerNorm(W_k^I x) * gamma + beta     eq. (3)
    a   = W_a^I x                                eq. (4), no sigmoid or softmax
    """
    qi = linear(cq, _w(w, "w_idx_q"))
    qi = qi.reshape(*qi.shape[:-1], dims.n_idx_heads, dims.d_idx)
    ki = layer_norm(linear(x, _w(w, "w_idx_k")), _w(w, "g_idx_k"), _w(w, "b_idx_k"), dims.ln_eps)
    a = linear(x, _w(w, "w_idx_w"))
    return qi, ki, a


def index_scores(qi, a, idx_keys, t: int):
    """I_s = 1/(sqrt(n_idx) sqrt(d_idx)) * sum_h a_h ReLU(q^I_h . k^I_s) for s < t (eq. (5)).

    qi [n_idx, d_idx], a [n_idx], idx_keys [>= t, d_idx]; t counts the visible positions,
    the current one included. Returns I [t].
    """
    qi = np.asarray(qi, dtype=F64)
    a = np.asarray(a, dtype=F64)
    keys = np.asarray(idx_keys, dtype=F64)[:t]
    dots = qi @ keys.T                                   # [n_idx, t]
    # 1/(sqrt(n_idx) sqrt(d_idx)) written as 1/sqrt(n_idx d_idx): the same number, and exact
    # (1/64 at 32 x 128) instead of rounding each root separately
    scale = 1.0 / np.sqrt(qi.shape[0] * qi.shape[1])
    return scale * np.sum(a[:, None] * np.maximum(dots, 0.0), axis=0)


def select_topk(scores, k: int) -> np.ndarray:
    """S = TopK(I, min(k, t)) (eq. (6)): the min(k, t) largest scores, ties to the lower
    position, -0.0 equal to +0.0; returned as ascending positions (int64)."""
    s = np.asarray(scores, dtype=F64)
    t = s.shape[0]
    n = min(int(k), t)
    order = np.lexsort((np.arange(t), -s))           # by score descending, then position
    return np.sort(order[:n]).astype(np.int64)


def attention_absorbed_subset(q_tilde, latent, positions, scale: float, dims):
    """Eq. (9) restricted to the selected set S_t, in the absorbed form: softmax over the
    positions of S only. q_tilde [H, L+S], latent [N, L+S]. Returns o [H, L] and lse [H]."""
    rows = np.asarray(latent, dtype=F64)[np.asarray(positions)]
    s = (q_tilde @ rows.T) * scale                     # [H, |S|]
    m = np.max(s, axis=-1, keepdims=True)
    p = np.exp(s - m)
    l = np.sum(p, axis=-1, keepdims=True)
    o = (p / l) @ rows[:, :dims.kv_lora]
    return o, (m + np.log(l))[:, 0]


def dsa_decode_step(x, w, cache: Cache, dims):
    """One decode token per sequence through the Gated DSA layer (the per-query pseudocode).

    x [B, hidden]. The main latent and the index key of the current token are appended
    first, so t includes it; scores, top-k, then sparse MLA with the main q and latent
    cache, then the gate and o_proj. Returns (y [B, hidden], extras).

    The index score is eq. (5) as written, with no quantisation or intermediate rounding of
    its query side: q^I comes from the float64 c^Q and a from x. The only rounding on the
    indexer path is the index cache's storage type (bf16, or FP8 when the cache is FP8).
    """
    x = np.asarray(x, dtype=F64)
    B = x.shape[0]
    cq, q_nope, q_shared = query_path(x, w, dims)
    c, r = kv_down_path(x, w, dims)
    qi, ki, a = index_projections(x, cq, w, dims)
    H = dims.n_heads
    if cache.expanded:
        k_nope, v = kv_up(cache._store(c), w, dims)
        cache.append(c[:, None], r[:, None], expand_keys(k_nope[:, None], cache._store(r)[:, None]),
                     v[:, None].transpose(0, 2, 1, 3), ki[:, None])
    else:
        cache.append(c[:, None], r[:, None], idx_k=ki[:, None])
    t = cache.length
    qt = absorbed_query(q_nope, q_shared, w, dims)        # [B, H, L+S]
    scale = softmax_scale(dims)
    z = np.zeros((B, H, dims.d_v))
    sel, scores, lse = [], [], []
    for b in range(B):
        I = index_scores(qi[b], a[b], cache.idx[b], t)
        S = select_topk(I, dims.topk)
        o, l_b = attention_absorbed_subset(qt[b], cache.latent[b], S, scale, dims)
        z[b] = value_up(o, w, dims)
        sel.append(S)
        scores.append(I)
        lse.append(l_b)
    u, y = gate_output(z, x, w, dims)
    return y, {"cq": cq, "q_idx": qi, "k_idx": ki, "a": a, "scores": scores, "selected": sel,
               "q_tilde": qt, "z": z, "u": u, "lse": np.stack(lse)}


def dsa_prefill(x, w, cache: Cache, dims):
    """T new tokens per sequence through the Gated DSA layer (eq. (6) applied at every t).

    x [B, T, hidden]. The main latent, the index keys (and the expanded K/V when the cache
    keeps them) of all T tokens are appended first; token i then sits at absolute position
    P + i (P = positions cached before the call) and, with t = P + i + 1 visible positions,
    scores the index keys 0..P+i (eq. (5)), keeps S = TopK(I, min(k, t)) (eq. (6)) and
    attends over S only in the absorbed form (eq. (9) over S), followed by the gate and
    o_proj. Appending all T keys before scoring is the per-query pseudocode's order for every
    token, since token i only reads positions up to its own. The index score is unrounded
    eq. (5), as in ``dsa_decode_step``. Returns (y [B, T, hidden], extras).
    """
    x = np.asarray(x, dtype=F64)
    B, T = x.shape[:2]
    P = cache.length
    cq, q_nope, q_shared = query_path(x, w, dims)
    c, r = kv_down_path(x, w, dims)
    qi, ki, a = index_projections(x, cq, w, dims)
    if cache.expanded:
        k_nope, v = kv_up(cache._store(c), w, dims)
        cache.append(c, r, expand_keys(k_nope, cache._store(r)), v.transpose(0, 2, 1, 3), ki)
    else:
        cache.append(c, r, idx_k=ki)
    qt = absorbed_query(q_nope, q_shared, w, dims)        # [B, T, H, L+S]
    scale = softmax_scale(dims)
    z = np.zeros((B, T, dims.n_heads, dims.d_v))
    sel = [[None] * T for _ in range(B)]
    for b in range(B):
        for i in range(T):
            t = P + i + 1
            I = index_scores(qi[b, i], a[b, i], cache.idx[b], t)
            S = select_topk(I, dims.topk)
            o, _ = attention_absorbed_subset(qt[b, i], cache.latent[b], S, scale, dims)
            z[b, i] = value_up(o, w, dims)
            sel[b][i] = S
    u, y = gate_output(z, x, w, dims)
    return y, {"q_idx": qi, "k_idx": ki, "a": a, "selected": sel, "q_tilde": qt, "z": z, "u": u}
