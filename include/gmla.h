/*
 * gmla.h - C ABI of the Gated MLA / Gated DSA attention library for AMD MI355X (gfx950).
 *
 * The library computes one Kimi K3 Gated MLA attention layer and the Kimi K3.1 Gated DSA
 * decode step on one GPU. Sources:
 *   [KV]  "Kimi K3 > Gated MLA > KV cache" card (atlas.klimoza.dev, kimi-k3 attention/kv-cache)
 *   [ATT] "Kimi K3" attention code page (atlas.klimoza.dev, kimi-k3 attention/key-value/x):
 *         KimiRMSNorm, KimiMLAAttention.__init__ and forward with the output gate
 *   [SK]  "Kimi K3 - Take the shared key part" (atlas.klimoza.dev, shared-key-split)
 *   [DSA] "Kimi K3 model structure (11): K3.1 Pro's Gated DSA from the inference code"
 *         (blog.javazero.top): eqs. (2)-(10), latent absorption, per-query pseudocode, caches
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers unless marked [host].
 *   - Tensors are bfloat16 (passed as void*, 2-byte bit patterns) unless marked f32 / i32.
 *     Layouts are dense row-major in the order written, e.g. [B,T,H,D] has D contiguous.
 *     Weights use the nn.Linear [out, in] layout ([ATT] __init__).
 *   - Every call validates on the host, then enqueues its kernels on `stream` and returns;
 *     it never synchronises. Device faults surface at the caller's next synchronisation.
 *   - Ownership: the caller owns all memory (weights, caches, outputs, workspace). The
 *     library allocates no device memory in these calls and keeps no pointer after it
 *     returns, beyond the kernels already enqueued. It has no mutable global state; calls on
 *     different streams with disjoint buffers may run concurrently.
 *   - Errors: the return value is MLA_OK (0) or a negative MLA_ERR_* code. Validation happens
 *     before any launch, so a failing call has no effect. MLA_ERR_HIP reports a failed launch.
 *     mla_status_string() names a code.
 *   - Empty work (B == 0 or T == 0) is valid and launches nothing.
 *   - Supported shapes: the Kimi K3 layer (hidden 7168, 96 heads, q_lora 1536, kv_lora 512,
 *     128 nope + 64 shared key features, 128 value features; DSA indexer 32 x 128) and the
 *     tiny oracle-scale layer (hidden 256, 4 heads, q_lora 64, kv_lora 32, 16 + 8 key, 16
 *     value; no DSA). Other dims return MLA_ERR_UNSUPPORTED.
 */
#ifndef GMLA_H
#define GMLA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MLA_OK = 0,
  MLA_ERR_NULL = -1,        /* a required pointer is NULL */
  MLA_ERR_SHAPE = -2,       /* a size is negative, inconsistent or out of range */
  MLA_ERR_CAPACITY = -3,    /* positions would exceed the cache capacity T_cap */
  MLA_ERR_UNSUPPORTED = -4, /* dims, dtype or path not compiled into this library */
  MLA_ERR_WORKSPACE = -5,   /* ws_bytes below what mla_workspace_bytes() asks for */
  MLA_ERR_HIP = -6          /* a kernel launch failed */
};

enum { MLA_OUT_BF16 = 0, MLA_OUT_F32 = 1 };
enum { MLA_PATH_ABSORBED = 0, MLA_PATH_EXPANDED = 1, MLA_PATH_SPARSE = 2 };

/* [host] Layer dimensions; field meanings follow the released config ([ATT] __init__). */
typedef struct mla_dims {
  int32_t hidden;        /* hidden_size: 7168 */
  int32_t n_heads;       /* num_attention_heads: 96 */
  int32_t q_lora;        /* q_lora_rank: 1536 */
  int32_t kv_lora;       /* kv_lora_rank: 512 */
  int32_t d_nope;        /* qk_nope_head_dim: 128 */
  int32_t d_shared;      /* qk_rope_head_dim: 64, the shared key part; never rotated ([SK]) */
  int32_t d_v;           /* v_head_dim: 128 */
  float rms_eps;         /* KimiRMSNorm eps: 1e-6 ([ATT] KimiRMSNorm) */
  float softmax_scale;   /* (d_nope + d_shared)^-1/2 ([ATT] self.scaling) */
  int32_t use_gate;      /* 1: sigmoid output gate before o_proj ([ATT] forward; [DSA] eq. (10)) */
  int32_t n_idx_heads;   /* DSA index heads: 32, or 0 without the indexer ([DSA] eq. (2)) */
  int32_t d_idx;         /* DSA index head dim: 128 ([DSA] eq. (2)-(3)) */
  int32_t topk;          /* DSA selection size, 1..2048 ([DSA] eq. (6)) */
  float ln_eps;          /* index-key LayerNorm eps; the pages print none, 1e-6 is used */
} mla_dims;

/* Device pointers to one layer's parameters (bf16, [out, in]; gains and bias [n]). */
typedef struct mla_weights {
  const void* w_q_a;     /* [q_lora, hidden]                 q_a_proj */
  const void* g_q_a;     /* [q_lora]                         q_a_layernorm gain */
  const void* w_q_b;     /* [H*(d_nope+d_shared), q_lora]    q_b_proj; head h rows [h*192, h*192+192) = nope ‖ shared */
  const void* w_kv_a;    /* [kv_lora+d_shared, hidden]       kv_a_proj_with_mqa */
  const void* g_kv_a;    /* [kv_lora]                        kv_a_layernorm gain */
  const void* w_kv_b;    /* [H*(d_nope+d_v), kv_lora]        kv_b_proj; head h rows = k_nope (128) ‖ v (128) */
  const void* w_g;       /* [H*d_v, hidden]                  g_proj (output gate) */
  const void* w_o;       /* [hidden, H*d_v]                  o_proj */
  const void* w_idx_q;   /* [n_idx*d_idx, q_lora]            DSA W_q^I  ([DSA] eq. (2)), or NULL */
  const void* w_idx_k;   /* [d_idx, hidden]                  DSA W_k^I  ([DSA] eq. (3)), or NULL */
  const void* g_idx_k;   /* [d_idx]                          index-key LayerNorm gain, or NULL */
  const void* b_idx_k;   /* [d_idx]                          index-key LayerNorm bias, or NULL */
  const void* w_idx_w;   /* [n_idx, hidden]                  DSA W_a^I  ([DSA] eq. (4)), or NULL */
} mla_weights;

/* Caller-owned caches with a fixed capacity of T_cap positions per sequence ([KV]; [DSA]
 * cache table). Unlike the pages' concatenating update, capacity is enforced.
 *
 * Formats ([DSA] cache section, deployed caches): with latent_format = MLA_CACHE_FP8 a latent
 * row is 656 bytes: the 512 OCP E4M3 codes of c_s, four fp32 scales (one per block of 128
 * features: the smallest power of two 2^k, k >= -126, with max|c| <= 448 * 2^k; code =
 * e4m3(c / 2^k) rounded to nearest even), then r_s as 64 bf16. With idx_format =
 * MLA_CACHE_FP8, idx_k holds [batch, T_cap, 128] E4M3 codes followed by [batch, T_cap] fp32
 * scales of the same rule (132 bytes per position). A value reads back as decode(code) * scale.
 * kv_append writes these formats; FP8 formats need the K3 shape, others return
 * MLA_ERR_UNSUPPORTED. Expanded k / v are always bf16. */
enum { MLA_CACHE_BF16 = 0, MLA_CACHE_FP8 = 1 };
typedef struct mla_cache {
  void* latent;          /* [batch, T_cap, kv_lora + d_shared] bf16: c_s (normalised) ‖ r_s;
                            FP8: [batch, T_cap, 656] bytes */
  void* k;               /* [batch, H, T_cap, d_nope + d_shared]: expanded keys, or NULL */
  void* v;               /* [batch, H, T_cap, d_v]: expanded values, or NULL */
  void* idx_k;           /* [batch, T_cap, d_idx] bf16: DSA index keys, or NULL; FP8: see above */
  int32_t batch;
  int32_t T_cap;
  int32_t latent_format; /* MLA_CACHE_BF16 or MLA_CACHE_FP8 */
  int32_t idx_format;    /* MLA_CACHE_BF16 or MLA_CACHE_FP8 */
  /* Paged latent and index caches ([DSA] pseudocode note: the deployed path maps positions to
   * pages), or block_table = NULL for the [batch, T_cap] layout above. With a table, latent and
   * idx_k are pools of n_pages pages of page_size rows each (FP8 index scales: one per pool row,
   * after the codes), and position p of sequence s is pool row
   *   block_table[s * max_blocks + p / page_size] * page_size + p % page_size.
   * page_size must be a multiple of 32 and T_cap = page_size * max_blocks; page indices are
   * clamped into [0, n_pages) on the device. The expanded k / v are not paged (must be NULL),
   * and mla_prefill (which attends over them) returns MLA_ERR_UNSUPPORTED. Pages may be shared
   * between sequences for reading; two sequences appending into one page race. */
  const int32_t* block_table; /* [batch, max_blocks] device, or NULL */
  int32_t page_size;
  int32_t max_blocks;
  int32_t n_pages;
} mla_cache;

/* Status name ("MLA_OK", "MLA_ERR_SHAPE", ...). Never NULL. */
const char* mla_status_string(int status);

/* MLA_OK when these dims are compiled into the library, else MLA_ERR_UNSUPPORTED. */
int mla_dims_supported(const mla_dims* dims);

/* [host] Workspace bytes that mla_prefill (T_new > 1, path ignored) or mla_decode (T_new == 1,
 * with `path` and `max_len` = largest visible length) needs for B sequences. 0 on bad input. */
size_t mla_workspace_bytes(const mla_dims* dims, int32_t B, int32_t T_new, int32_t max_len,
                           int32_t path);

/* [host] As mla_workspace_bytes, for a decode call (T_new == 1) made with an explicit
 * num_splits (0 = automatic, the same as mla_workspace_bytes). This size also covers the
 * stage entry points mla_decode_attention / mla_sparse_attention / dsa_index_topk called with
 * the same B, max_len (max_visible; topk for the sparse path) and num_splits. */
size_t mla_workspace_bytes_ex(const mla_dims* dims, int32_t B, int32_t T_new, int32_t max_len,
                              int32_t path, int32_t num_splits);

/* ---------------------------------------------------------------------------------------
 * Whole-layer entry points
 * ------------------------------------------------------------------------------------- */

/* Prefill: T new tokens for each of B sequences ([ATT] forward).
 *   x [B,T,hidden] -> y [B,T,hidden] (bf16 or f32 per out_dtype).
 *   start_pos [B] i32: positions already cached per sequence; token i of sequence b is
 *   written at position start_pos[b]+i and attends causally to positions 0..start_pos[b]+i.
 *   max_end [host]: an upper bound of start_pos[b]+T over b; must be <= cache->T_cap.
 *   Appends the latent rows and the expanded K/V (cache->k, cache->v required) and, when the
 *   indexer is enabled and cache->idx_k is set, the index keys.
 *   lse [B,H,T] f32 or NULL: natural-log softmax denominators of the scaled logits.
 *   ws: device workspace of at least mla_workspace_bytes(dims, B, T, max_end, 0) bytes. */
int mla_prefill(const mla_dims* dims, const mla_weights* w, const mla_cache* cache,
                const int32_t* start_pos, int32_t max_end, const void* x, int32_t B, int32_t T,
                void* y, int32_t out_dtype, float* lse, void* ws, size_t ws_bytes,
                hipStream_t stream);

/* Gated DSA prefill ([DSA] eq. (6) at every position, eq. (9) over S_t): T new tokens of each
 * of B sequences with the indexer's selection applied to every token.
 *   Arguments as mla_prefill. Requires the indexer (dims->n_idx_heads > 0, every w_idx_* weight)
 *   and cache->idx_k; cache->k / cache->v are appended to when set (not read).
 *   The latent rows and index keys of all T tokens are appended first. Token i of sequence b
 *   (position p = start_pos[b]+i, t = p+1 visible positions) then scores index keys 0..p
 *   (eq. (5)), keeps S = the min(topk, t) largest (eq. (6), ties to the lower position),
 *   attends over S only in the absorbed form, and goes through the gate and o_proj.
 *   sel_idx [B,T,topk] i32 (ascending, -1 padded) and sel_cnt [B,T] i32, or NULL, receive S.
 *   scores [B,T,max_end] f32 or NULL receives each token's index scores I_s for s < t (eq. (5));
 *   entries at s >= t are left unwritten.
 *   ws: device workspace of at least mla_workspace_bytes_prefill_sparse(dims, B, T, max_end)
 *   bytes. Errors as mla_prefill; MLA_ERR_UNSUPPORTED without the indexer. */
int mla_prefill_sparse(const mla_dims* dims, const mla_weights* w, const mla_cache* cache,
                       const int32_t* start_pos, int32_t max_end, const void* x, int32_t B,
                       int32_t T, void* y, int32_t out_dtype, int32_t* sel_idx, int32_t* sel_cnt,
                       float* scores, void* ws, size_t ws_bytes, hipStream_t stream);

/* [host] Workspace bytes of mla_prefill_sparse; 0 on bad input or without the indexer. */
size_t mla_workspace_bytes_prefill_sparse(const mla_dims* dims, int32_t B, int32_t T, int32_t max_end);

/* Decode: one new token per sequence ([ATT] forward with one position; [DSA] pseudocode).
 *   seq_len [B] i32: positions cached before this token; the token is written at position
 *   seq_len[b] and sees seq_len[b]+1 positions. max_len [host]: >= max_b seq_len[b]+1, and
 *   <= cache->T_cap.
 *   path MLA_PATH_ABSORBED: scores in the latent space over cache->latent (576 values read per
 *        position; [DSA] latent absorption).
 *   path MLA_PATH_EXPANDED: attention over cache->k / cache->v (30,720 values per position).
 *   path MLA_PATH_SPARSE: the DSA indexer appends the index key, scores, selects the top-k
 *        (written to sel_idx [B,topk] i32 ascending, -1 padded, and sel_cnt [B] i32), then
 *        absorbed attention over the selected positions only ([DSA] eqs. (2)-(9)).
 *   num_splits: split-K factor over the cache (0 = automatic).
 *   x [B,hidden] -> y [B,hidden]. ws: at least mla_workspace_bytes(dims, B, 1, max_len, path). */
int mla_decode(const mla_dims* dims, const mla_weights* w, const mla_cache* cache,
               const int32_t* seq_len, int32_t max_len, const void* x, int32_t B, int32_t path,
               int32_t num_splits, int32_t* sel_idx, int32_t* sel_cnt, void* y,
               int32_t out_dtype, void* ws, size_t ws_bytes, hipStream_t stream);

/* The DSA indexer's projections of M tokens, with the launches a decode or prefill step runs
 * ([DSA] eqs. (2)-(4) and the LayerNorm paragraph after eq. (3)):
 *   q_idx [M,n_idx,d_idx] f32 = reshape(c^Q W_q^I^T), c^Q the normalised query latent (fp32,
 *         entering the GEMM as a bf16 hi + lo pair);
 *   w_idx [M,n_idx] f32 = x W_a^I^T, raw (no sigmoid);
 *   k_idx [M,d_idx] bf16 = LayerNorm(x W_k^I^T) * gain + bias, computed in fp64 and rounded once
 *         (the value mla_decode / mla_prefill_sparse append to the index cache).
 *   x [M,hidden] bf16. ws: at least mla_workspace_bytes(dims, M, 1, 1, MLA_PATH_SPARSE) bytes.
 *   Requires the indexer (MLA_ERR_UNSUPPORTED without it) and every w_idx_* weight. */
int mla_index_projections(const mla_dims* dims, const mla_weights* w, const void* x, int32_t M,
                          float* q_idx, float* w_idx, void* k_idx, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, serving loops
 * and harnesses that forbid hipMalloc): mla_decode with the same arguments minus the
 * workspace, which comes from a static device buffer of the library instead,
 * MLA_NOALLOC_SCRATCH_BYTES (64 MiB) on each GPU the library runs on, held until the process
 * ends. The call allocates nothing. Its first call on a device looks the buffer's address up
 * (hipGetSymbolAddress, with that device current); MLA_ERR_HIP if that fails.
 *   Returns MLA_ERR_WORKSPACE, before touching the device, when the call would need more than
 *   that (mla_workspace_bytes_ex(dims, B, 1, max_len, path, num_splits) > the buffer): e.g.
 *   B = 32 at max_len 8193 needs 44 MiB, B = 4 at 131073 27 MiB, the DSA path at B = 8,
 *   65537 24 MiB. Other errors as mla_decode.
 *   Every call on one GPU shares the buffer: calls that overlap in time on one GPU (other
 *   streams, other threads) race and must be serialised by the caller. Nothing in the buffer
 *   needs to start at zero; the kernels clear what they count into. */
#define MLA_NOALLOC_SCRATCH_BYTES (64 * 1024 * 1024)
int mla_decode_noalloc(const mla_dims* dims, const mla_weights* w, const mla_cache* cache,
                       const int32_t* seq_len, int32_t max_len, const void* x, int32_t B, int32_t path,
                       int32_t num_splits, int32_t* sel_idx, int32_t* sel_cnt, void* y,
                       int32_t out_dtype, hipStream_t stream);

/* Cache append ([KV] update; [SK]; [DSA] eq. (7) and pseudocode).
 *   For b < B and i < T, at position p = pos[b] + i:
 *     latent[b,p] = c[b,i] ‖ r[b,i]
 *     k[b,h,p]    = k_nope[b,i,h] ‖ r[b,i]   for every head h (if k_nope and cache->k set)
 *     v[b,h,p]    = v[b,i,h]                 (if v and cache->v set)
 *     idx_k[b,p]  = idx_k[b,i]               (if idx_k and cache->idx_k set)
 *   c [B,T,kv_lora], r [B,T,d_shared], k_nope [B,T,H,d_nope], v [B,T,H,d_v], idx_k [B,T,d_idx].
 *   Bit-exact copies. max_end [host]: upper bound of pos[b]+T, <= cache->T_cap. */
int kv_append(const mla_dims* dims, const mla_cache* cache, const int32_t* pos, int32_t max_end,
              int32_t B, int32_t T, const void* c, const void* r, const void* k_nope,
              const void* v, const void* idx_k, hipStream_t stream);

/* DSA index scores and top-k for one query per sequence ([DSA] eqs. (5)-(6)).
 *   q_idx [B,n_idx,d_idx] f32 index query (eq. (2)), unrounded as eq. (5) takes it: each value
 *   enters the bf16 MFMA as a hi + lo pair, so the scores carry it to about 17 bits;
 *   w_idx [B,n_idx] f32 raw head weights a_t (eq. (4));
 *   idx_k_cache [B,T_cap,d_idx] bf16; n_visible [B] i32 = t (current token included);
 *   max_visible [host] >= max t, <= T_cap.
 *   I_s = (1/sqrt(n_idx*d_idx)) sum_h a_h ReLU(q_h . k_s) for s < t; the min(topk, t) largest
 *   (ties to the lower position) are written ascending to out_idx [B,topk] i32, -1 padded,
 *   with out_cnt [B] i32. out_scores [B,T_cap] f32 or NULL receives I for s < t.
 *   ws: at least mla_workspace_bytes(dims, B, 1, max_visible, MLA_PATH_SPARSE). */
int dsa_index_topk(const mla_dims* dims, const float* q_idx, const float* w_idx,
                   const void* idx_k_cache, int32_t T_cap, const int32_t* n_visible,
                   int32_t max_visible, int32_t B, int32_t* out_idx, int32_t* out_cnt,
                   float* out_scores, void* ws, size_t ws_bytes, hipStream_t stream);

/* As dsa_index_topk over FP8 index keys ([DSA] cache section): idx_k_codes [B, T_cap, 128] OCP
 * E4M3 codes, idx_k_scales [B, T_cap] fp32 (>= 0); key s reads back as decode(code) * scale,
 * so its score is scale times the score of the decoded codes. d_idx must be 128. */
int dsa_index_topk_fp8(const mla_dims* dims, const float* q_idx, const float* w_idx,
                       const void* idx_k_codes, const float* idx_k_scales, int32_t T_cap,
                       const int32_t* n_visible, int32_t max_visible, int32_t B, int32_t* out_idx,
                       int32_t* out_cnt, float* out_scores, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * Stage entry points: the kernels of the whole-layer calls, each callable alone so that every
 * step can be checked against the oracle with identical inputs.
 * ------------------------------------------------------------------------------------- */

/* out[m, n] = sum_k a[m, k] * w[n, k]  (nn.Linear, fp32 accumulation).
 * a [M, lda] bf16 (first K columns used), w [N, K] bf16, out [M, ldo] bf16 or f32. */
int mla_gemm(const void* a, int32_t lda, const void* w, int32_t M, int32_t N, int32_t K,
             void* out, int32_t ldo, int32_t out_dtype, hipStream_t stream);

/* KimiRMSNorm ([ATT]): out[m,:] = bf16( x[m,:] * rsqrt(mean(x[m,:]^2) + eps) * gain ).
 * x [M, ldx] f32, gain [N] bf16, out [M, ldo] bf16. */
int mla_rmsnorm(const float* x, int32_t ldx, const void* gain, int32_t M, int32_t N, float eps,
                void* out, int32_t ldo, hipStream_t stream);

/* Index-key LayerNorm ([DSA] eq. (3)): out = bf16( (x - mean) * rsqrt(var + eps) * gain + bias ).
 * x [M, ldx] f32, gain/bias [N] bf16, out [M, ldo] bf16. */
int mla_layernorm(const float* x, int32_t ldx, const void* gain, const void* bias, int32_t M,
                  int32_t N, float eps, void* out, int32_t ldo, hipStream_t stream);

/* Prefill attention with the gate epilogue ([DSA] eqs. (9)-(10) before W_o):
 *   u[b,i,h*d_v+d] = z[b,i,h,d] * sigmoid(g_pre[b,i,h*d_v+d])  (times 1 when g_pre is NULL)
 *   z = softmax_j(q[b,i,h].k[b,h,j] * scale) v[b,h,j] over j <= start_pos[b]+i.
 * q [B,T,H,d_nope+d_shared] bf16, K/V from cache->k / cache->v, g_pre [B,T,H*d_v] f32 or NULL,
 * u [B,T,H*d_v] (bf16 or f32), lse [B,H,T] f32 or NULL. */
int mla_prefill_attention(const mla_dims* dims, const void* q, const mla_cache* cache,
                          const int32_t* start_pos, int32_t max_end, int32_t B, int32_t T,
                          const float* g_pre, void* u, int32_t out_dtype, float* lse,
                          hipStream_t stream);

/* Query absorption ([DSA] latent absorption): q_tilde[b,h] = [ W^K_h^T q_nope[b,h] ‖ q_shared[b,h] ]
 * with W^K_h = w_kv_b rows [h*(d_nope+d_v), h*(d_nope+d_v)+d_nope).
 * q [B,H,d_nope+d_shared] bf16 (row stride ldq elements per token), q_tilde [B,H,kv_lora+d_shared] bf16. */
int mla_absorb_query(const mla_dims* dims, const void* q, int32_t ldq, const void* w_kv_b,
                     int32_t B, void* q_tilde, hipStream_t stream);

/* Absorbed decode attention over the latent cache, split over positions and merged:
 *   s_j = q_tilde[b,h] . latent[b,j] * scale for j < n_visible[b]
 *   o_latent[b,h,:] = sum_j softmax(s)_j latent[b,j,:kv_lora]   (f32), lse[b,h] (f32, or NULL).
 * n_visible[b] >= 1. ws: mla_workspace_bytes_ex(dims, B, 1, max_visible, MLA_PATH_ABSORBED,
 * num_splits) bytes. */
int mla_decode_attention(const mla_dims* dims, const void* q_tilde, const mla_cache* cache,
                         const int32_t* n_visible, int32_t max_visible, int32_t B,
                         int32_t num_splits, float* o_latent, float* lse, void* ws,
                         size_t ws_bytes, hipStream_t stream);

/* Sparse absorbed decode attention ([DSA] eq. (9) over S_t): as mla_decode_attention but over
 * the positions sel_idx[b, 0..sel_cnt[b]) only (sel_idx [B,topk] i32). An entry outside
 * [0, T_cap) is left out of the softmax (probability 0); a row with no valid entry gives
 * o_latent = 0 and lse = -inf. ws: mla_workspace_bytes_ex(dims, B, 1, topk, MLA_PATH_SPARSE,
 * num_splits). */
int mla_sparse_attention(const mla_dims* dims, const void* q_tilde, const mla_cache* cache,
                         const int32_t* sel_idx, const int32_t* sel_cnt, int32_t B,
                         int32_t num_splits, float* o_latent, float* lse, void* ws,
                         size_t ws_bytes, hipStream_t stream);

/* Expanded decode attention over cache->k / cache->v ([KV]): z[b,h,:] f32 and lse[b,h]
 * (or NULL) for one query q [B,H,d_nope+d_shared] bf16 per sequence over j < n_visible[b]. */
int mla_expanded_attention(const mla_dims* dims, const void* q, const mla_cache* cache,
                           const int32_t* n_visible, int32_t max_visible, int32_t B, float* z,
                           float* lse, hipStream_t stream);

/* Value up-projection and gate: u[b,h*d_v+d] = (W^V_h o_latent[b,h])[d] * sigmoid(g_pre[b,h*d_v+d])
 * with W^V_h = w_kv_b rows [h*(d_nope+d_v)+d_nope, (h+1)*(d_nope+d_v)).
 * o_latent [B,H,kv_lora] f32, g_pre [B,H*d_v] f32 or NULL, u [B,H*d_v] bf16 or f32. */
int mla_value_up_gate(const mla_dims* dims, const float* o_latent, const void* w_kv_b,
                      const float* g_pre, int32_t B, void* u, int32_t out_dtype,
                      hipStream_t stream);

/* Raw attention logits, for checking the score computation on small shapes: the argument of the
 * softmax in [DSA] eq. (9) (the eager softmax(q k^T * scale) of the Kimi K2 KV-cache card), with
 * no causal mask:
 *   logits[b,h,i,j] = dims->softmax_scale * sum_d q[b,i,h,d] * k[b,hk,j,d],  hk = (k_heads == 1 ? 0 : h)
 *   q [B,Tq,H,D] bf16; k [B,k_heads,Tk,D] bf16; logits [B,H,Tq,Tk] f32 (every (i, j) written).
 *   D = d_nope + d_shared with per-head keys (k_heads = H: the expanded form [KV]), or
 *   D = kv_lora + d_shared with k_heads = 1 (the absorbed form: q~ against the latent rows
 *   [c ; r] every head shares, [DSA] note after eq. (10)). q and k 16-byte aligned.
 *   Products as in the attention kernels: bf16 operands, fp32 accumulation.
 *   B * H * Tq * Tk may not exceed MLA_DEBUG_SCORES_MAX (MLA_ERR_SHAPE): a debugging aid, not a
 *   fast path. */
#define MLA_DEBUG_SCORES_MAX ((size_t)1 << 26)
int mla_debug_scores(const mla_dims* dims, const void* q, const void* k, int32_t k_heads, int32_t B,
                     int32_t Tq, int32_t Tk, int32_t D, float* logits, hipStream_t stream);

/* Device-side bound checks (for debugging callers' indices and the library itself; not a
 * passage of the pages). In the debug build of the library (libgmla_debug.so, compiled with
 * GMLA_DEBUG_CHECKS), kv_append checks every token position against [0, T_cap) and every
 * page-table entry it uses against [0, n_pages), and the top-k compactions check every output
 * offset against the kept count. A failed check sets a bit in *flags:
 *   MLA_DBG_APPEND_POS, MLA_DBG_APPEND_PAGE, MLA_DBG_TOPK_OFFSET.
 * Every build skips such writes (a position outside the cache is not written, a bad page entry
 * is clamped to a valid page), so the checks change no result; the normal build only does not
 * record them. This call synchronises `stream`, returns the bits set since the last call and
 * clears them (for the current device). *checks_built = 1 in the debug build, 0 otherwise (then
 * *flags is always 0). MLA_ERR_NULL if flags or checks_built is NULL; MLA_ERR_HIP on a HIP error. */
#define MLA_DBG_APPEND_POS 1u
#define MLA_DBG_APPEND_PAGE 2u
#define MLA_DBG_TOPK_OFFSET 4u
int mla_debug_flags(uint32_t* flags, int32_t* checks_built, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* GMLA_H */
