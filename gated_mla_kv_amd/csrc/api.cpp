// C ABI of the Gated MLA / Gated DSA library: host-side validation, workspace layout and the
// whole-layer pipelines. Every public function validates all of its arguments before it
// enqueues anything, so a call that returns an error has had no effect.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "../../include/gmla.h"
#include "gemm.h"
#include "kernels.h"

using namespace gmla;

namespace {

constexpr int kMaxTopk = 2048;

// GMLA_LOG set to anything but "" or "0": every entry point that can launch work writes one line
// to stderr on entry ("[gmla] <function> <sizes> stream=<stream>"), before it validates anything.
bool log_enabled() {
  static const bool on = [] {
    const char* e = getenv("GMLA_LOG");
    return e && *e && strcmp(e, "0") != 0;
  }();
  return on;
}
__attribute__((format(printf, 3, 4))) void trace(const char* fn, hipStream_t st, const char* fmt, ...) {
  if (!log_enabled()) return;
  char buf[320];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  fprintf(stderr, "[gmla] %s %s stream=%p\n", fn, buf, (void*)st);
  fflush(stderr);
}

bool shape_of(const mla_dims* d, Shape* s) {
  if (!d) return false;
  const bool k3 = d->hidden == 7168 && d->n_heads == 96 && d->q_lora == 1536 && d->kv_lora == 512 &&
                  d->d_nope == 128 && d->d_shared == 64 && d->d_v == 128;
  const bool tiny = d->hidden == 256 && d->n_heads == 4 && d->q_lora == 64 && d->kv_lora == 32 &&
                    d->d_nope == 16 && d->d_shared == 8 && d->d_v == 16;
  if (!k3 && !tiny) return false;
  if (d->n_idx_heads != 0) {
    if (!k3 || d->n_idx_heads != 32 || d->d_idx != 128) return false;
    if (d->topk < 1 || d->topk > kMaxTopk) return false;
  }
  if (!(d->softmax_scale > 0.f) || !isfinite(d->softmax_scale)) return false;
  if (!(d->rms_eps >= 0.f) || !(d->ln_eps >= 0.f)) return false;
  *s = k3 ? Shape::K3 : Shape::Tiny;
  return true;
}

bool has_dsa(const mla_dims* d) { return d->n_idx_heads > 0; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Bump allocator over the caller's workspace.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* p) : base((char*)p) {}
  template <class T>
  T* take(size_t count) {
    T* p = base ? (T*)(base + off) : nullptr;
    off += align256(count * sizeof(T));
    return p;
  }
};

int auto_splits(int B, int max_len, int requested) {
  if (requested > 0) return requested;
  int s = (256 + B - 1) / B;                     // one workgroup per CU
  const int cap = (max_len + 127) / 128;         // at least four 32-position tiles per split
  if (s > cap) s = cap;
  return s < 1 ? 1 : s;
}

int split_chunk(int max_len, int splits) {
  int c = (max_len + splits - 1) / splits;
  return (c + 31) / 32 * 32;
}

// Workspace regions of one layer call with M token rows.
struct Ws {
  float* xq;       // [M, q_lora]   q_a_proj output (pre-norm)
  float* xc;       // [M, kv_lora]  latent before its norm
  uint16_t* r;     // [M, d_shared] shared key
  float* gpre;     // [M, H*d_v]    gate pre-activation (fp32)
  double* kpart;   // [splits, M, d_idx]  index-key split-K partial sums (fp64)
  float* aw;       // [M, n_idx]    index head weights
  uint16_t* cq;    // [M, ldcq]     normalised query latent: bf16 hi, then (DSA) bf16 lo
  int ldcq;        // q_lora, or 2 q_lora with the indexer (the split operand of the q^I GEMM)
  uint16_t* c;     // [M, kv_lora]
  uint16_t* kidx;  // [M, d_idx]
  uint16_t* q;     // [M, H*(d_nope+d_shared)]
  float* qidx;     // [M, n_idx*d_idx]  index query (fp32)
  uint16_t* kv;    // [M, H*(d_nope+d_v)]
  uint16_t* u;     // [M, H*d_v]
  uint16_t* qt;    // [M, H, kv_lora+d_shared]   (decode)
  uint16_t* part_o;  // [M, S, H, kv_lora] fp16  (decode)
  float* part_ml;  // [M, S, H, 2]
  float* olat;     // [M, H, kv_lora]
  float* z;        // [M, H, d_v]
  float* scores;   // [M, max_len]
  int32_t* sel;    // [M, topk]
  int32_t* cnt;    // [M]
  int32_t* topk_scratch;  // index_topk_scratch_words(M, max_len)
  void* gemm_ws;
  size_t gemm_ws_bytes;
  size_t total;
};

Ws carve(const mla_dims* d, int M, bool decode, int max_len, int path, int splits, void* ws) {
  Carver cv(ws);
  Ws w{};
  const int H = d->n_heads, dqk = d->d_nope + d->d_shared;
  const bool dsa = has_dsa(d);
  w.xq = cv.take<float>((size_t)M * d->q_lora);
  w.xc = cv.take<float>((size_t)M * d->kv_lora);
  w.r = cv.take<uint16_t>((size_t)M * d->d_shared);
  w.gpre = cv.take<float>((size_t)M * H * d->d_v);
  w.kpart = cv.take<double>(dsa ? (size_t)index_key_splits(M, d->hidden) * M * d->d_idx : 0);
  w.aw = cv.take<float>(dsa ? (size_t)M * d->n_idx_heads : 0);
  w.ldcq = dsa ? 2 * d->q_lora : d->q_lora;
  w.cq = cv.take<uint16_t>((size_t)M * w.ldcq);
  w.c = cv.take<uint16_t>((size_t)M * d->kv_lora);
  w.kidx = cv.take<uint16_t>(dsa ? (size_t)M * d->d_idx : 0);
  w.q = cv.take<uint16_t>((size_t)M * H * dqk);
  w.qidx = cv.take<float>(dsa ? (size_t)M * d->n_idx_heads * d->d_idx : 0);
  w.kv = cv.take<uint16_t>((size_t)M * H * (d->d_nope + d->d_v));
  w.u = cv.take<uint16_t>((size_t)M * H * d->d_v);
  if (decode) {
    const int S = splits;
    w.qt = cv.take<uint16_t>((size_t)M * H * (d->kv_lora + d->d_shared));
    w.part_o = cv.take<uint16_t>((size_t)M * S * H * d->kv_lora);
    w.part_ml = cv.take<float>((size_t)M * S * H * 2);
    w.olat = cv.take<float>((size_t)M * H * d->kv_lora);
    w.z = cv.take<float>((size_t)M * H * d->d_v);
    if (path == MLA_PATH_SPARSE) {
      w.scores = cv.take<float>((size_t)M * max_len);
      w.sel = cv.take<int32_t>((size_t)M * d->topk);
      w.cnt = cv.take<int32_t>((size_t)M);
      w.topk_scratch = cv.take<int32_t>(index_topk_scratch_words(M, max_len));
    }
  }
  // split-K partials of the small-M GEMMs (the largest of the layer's GEMMs)
  size_t g = 0;
  const int Nx = d->q_lora + d->kv_lora + d->d_shared + H * d->d_v + (dsa ? d->n_idx_heads : 0);
  const size_t cand[5] = {gemm_ws_bytes(M, Nx, d->hidden), gemm_ws_bytes(M, H * dqk, d->q_lora),
                          gemm_ws_bytes(M, H * (d->d_nope + d->d_v), d->kv_lora),
                          gemm_ws_bytes(M, d->hidden, H * d->d_v),
                          dsa ? gemm_ws_bytes(M, d->n_idx_heads * d->d_idx, d->q_lora) : 0};
  for (size_t c : cand) g = c > g ? c : g;
  w.gemm_ws_bytes = g;
  w.gemm_ws = g ? cv.take<char>(g) : nullptr;
  w.total = cv.off;
  return w;
}

#define CHECK_HIP(expr)                          \
  do {                                           \
    if ((expr) != hipSuccess) return MLA_ERR_HIP; \
  } while (0)

GemmSeg seg(const void* w, int rows, void* out, int ldo, bool f32, int& n) {
  GemmSeg s;
  s.w = (const uint16_t*)w;
  s.out = out;
  s.n0 = n;
  s.n1 = n + rows;
  s.ldo = ldo;
  s.out_f32 = f32 ? 1 : 0;
  n += rows;
  return s;
}

GemmArgs gemm_args(const void* a, int lda, int M, int K) {
  GemmArgs g{};
  g.a = (const uint16_t*)a;
  g.lda = lda;
  g.M = M;
  g.K = K;
  return g;
}

void push(GemmArgs& g, GemmSeg s) {
  g.seg[g.nseg++] = s;
  g.N = s.n1;
}

// x -> [q_a | latent | shared key | gate | index head weights] in one GEMM (x read once).
int run_x_gemm(const mla_dims* d, const mla_weights* w, const void* x, int M, const Ws& ws,
               bool with_idx, hipStream_t st) {
  GemmArgs g = gemm_args(x, d->hidden, M, d->hidden);
  int n = 0;
  push(g, seg(w->w_q_a, d->q_lora, ws.xq, d->q_lora, true, n));
  push(g, seg(w->w_kv_a, d->kv_lora, ws.xc, d->kv_lora, true, n));
  push(g, seg((const uint16_t*)w->w_kv_a + (size_t)d->kv_lora * d->hidden, d->d_shared, ws.r,
              d->d_shared, false, n));
  if (d->use_gate) push(g, seg(w->w_g, d->n_heads * d->d_v, ws.gpre, d->n_heads * d->d_v, true, n));
  if (with_idx) push(g, seg(w->w_idx_w, d->n_idx_heads, ws.aw, d->n_idx_heads, true, n));
  CHECK_HIP(launch_gemm(g, ws.gemm_ws, ws.gemm_ws_bytes, st));
  return MLA_OK;
}

// The projections of M new tokens (everything the attention and the indexer read, before any
// cache append): the x-GEMM, the two RMSNorms, q = c^Q W_qb^T and, with the indexer,
//   q^I = c^Q W_q^I^T in fp32 ([DSA] eq. (2)): c^Q (fp32 after its RMSNorm) enters the GEMM as a
//         bf16 hi + lo pair (GemmArgs::a_split), when idx_query;
//   a   = x W_a^I^T in fp32 ([DSA] eq. (4)), a segment of the x-GEMM;
//   k^I = bf16(LayerNorm(x W_k^I^T) * gain + bias) computed in fp64 ([DSA] eq. (3)).
int run_projections(const mla_dims* d, const mla_weights* w, const void* x, int M, const Ws& wsp,
                    bool with_idx, bool idx_query, hipStream_t st) {
  const int H = d->n_heads, dqk = d->d_nope + d->d_shared;
  int rc = run_x_gemm(d, w, x, M, wsp, with_idx, st);
  if (rc) return rc;
  // the two RMSNorms (c^Q, and the latent c) in one launch
  CHECK_HIP(launch_rmsnorm2(
      RmsNormJob{wsp.xq, d->q_lora, (const uint16_t*)w->g_q_a, M, d->q_lora, wsp.cq, wsp.ldcq,
                 idx_query ? wsp.cq + d->q_lora : nullptr},
      RmsNormJob{wsp.xc, d->kv_lora, (const uint16_t*)w->g_kv_a, M, d->kv_lora, wsp.c, d->kv_lora, nullptr},
      d->rms_eps, st));
  {
    GemmArgs g = gemm_args(wsp.cq, wsp.ldcq, M, d->q_lora);
    int n = 0;
    push(g, seg(w->w_q_b, H * dqk, wsp.q, H * dqk, false, n));
    CHECK_HIP(launch_gemm(g, wsp.gemm_ws, wsp.gemm_ws_bytes, st));
  }
  if (idx_query) {
    GemmArgs g = gemm_args(wsp.cq, wsp.ldcq, M, d->q_lora);
    g.a_split = 1;
    int n = 0;
    push(g, seg(w->w_idx_q, d->n_idx_heads * d->d_idx, wsp.qidx, d->n_idx_heads * d->d_idx, true, n));
    CHECK_HIP(launch_gemm(g, wsp.gemm_ws, wsp.gemm_ws_bytes, st));
  }
  if (with_idx)
    CHECK_HIP(launch_index_key_f64((const uint16_t*)x, d->hidden, (const uint16_t*)w->w_idx_k,
                                   (const uint16_t*)w->g_idx_k, (const uint16_t*)w->b_idx_k, M, d->hidden,
                                   (double)d->ln_eps, wsp.kpart, wsp.kidx, d->d_idx, st));
  return MLA_OK;
}

bool null_any(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!p) return true;
  return false;
}

// FP8 caches ([DSA] cache section) exist for the K3 layer shape: 656-byte latent rows
// (kv_lora 512 in four scale blocks, d_shared 64) and 128-feature index keys.
bool fp8_latent(const mla_cache* c) { return c->latent_format == MLA_CACHE_FP8; }
bool fp8_index(const mla_cache* c) { return c->idx_format == MLA_CACHE_FP8; }

int check_cache(const mla_dims* d, const mla_cache* c, int B, int max_end) {
  if (!c) return MLA_ERR_NULL;
  if (!c->latent) return MLA_ERR_NULL;
  if (c->batch < B || c->T_cap <= 0) return MLA_ERR_SHAPE;
  if (max_end > c->T_cap) return MLA_ERR_CAPACITY;
  if ((c->latent_format != MLA_CACHE_BF16 && c->latent_format != MLA_CACHE_FP8) ||
      (c->idx_format != MLA_CACHE_BF16 && c->idx_format != MLA_CACHE_FP8))
    return MLA_ERR_UNSUPPORTED;
  const bool k3 = d->kv_lora == 512 && d->d_shared == 64 && d->n_heads == 96;
  if (fp8_latent(c) && !k3) return MLA_ERR_UNSUPPORTED;
  if (fp8_index(c) && (!k3 || d->d_idx != 128)) return MLA_ERR_UNSUPPORTED;
  if (c->block_table) {  // paged latent / index caches ([DSA] pseudocode note on page mapping)
    if (!k3 || c->k || c->v) return MLA_ERR_UNSUPPORTED;  // the expanded cache is not paged
    if (c->page_size <= 0 || c->page_size % 32 != 0 || c->max_blocks <= 0 || c->n_pages <= 0)
      return MLA_ERR_SHAPE;
    if ((int64_t)c->page_size * c->max_blocks != c->T_cap) return MLA_ERR_SHAPE;
    if ((int64_t)c->n_pages * c->page_size >= ((int64_t)1 << 31)) return MLA_ERR_SHAPE;
  }
  return MLA_OK;
}

PageTable page_table(const mla_cache* c) {
  PageTable p{};
  if (c->block_table) p = PageTable{c->block_table, c->page_size, c->max_blocks, c->n_pages};
  return p;
}

// FP8 index keys: the scales follow the codes, one per cache row ([batch, T_cap] rows, or
// [n_pages, page_size] when paged)
float* idx_scales(const mla_dims* d, const mla_cache* c) {
  if (!fp8_index(c) || !c->idx_k) return nullptr;
  const size_t rows = c->block_table ? (size_t)c->n_pages * c->page_size : (size_t)c->batch * c->T_cap;
  return (float*)((uint8_t*)c->idx_k + rows * d->d_idx);
}

int check_weights(const mla_dims* d, const mla_weights* w) {
  if (!w) return MLA_ERR_NULL;
  if (null_any({w->w_q_a, w->g_q_a, w->w_q_b, w->w_kv_a, w->g_kv_a, w->w_kv_b, w->w_o})) return MLA_ERR_NULL;
  if (d->use_gate && !w->w_g) return MLA_ERR_NULL;
  return MLA_OK;
}

bool idx_weights(const mla_weights* w) {
  return w->w_idx_q && w->w_idx_k && w->g_idx_k && w->b_idx_k && w->w_idx_w;
}

KvAppendArgs append_args(const mla_dims* d, const mla_cache* c, const int32_t* pos, int B, int T) {
  KvAppendArgs a{};
  a.pos = pos;
  a.B = B;
  a.T = T;
  a.T_cap = c->T_cap;
  a.H = d->n_heads;
  a.L = d->kv_lora;
  a.DS = d->d_shared;
  a.DN = d->d_nope;
  a.DV = d->d_v;
  a.DI = d->d_idx;
  a.latent_fp8 = fp8_latent(c);
  a.idx_fp8 = fp8_index(c);
  a.idx_scale = idx_scales(d, c);
  a.pages = page_table(c);
  return a;
}

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL: return "MLA_ERR_NULL";
    case MLA_ERR_SHAPE: return "MLA_ERR_SHAPE";
    case MLA_ERR_CAPACITY: return "MLA_ERR_CAPACITY";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
    default: return "MLA_ERR_UNKNOWN";
  }
}

int mla_dims_supported(const mla_dims* dims) {
  Shape s;
  return shape_of(dims, &s) ? MLA_OK : MLA_ERR_UNSUPPORTED;
}

size_t mla_workspace_bytes_ex(const mla_dims* d, int32_t B, int32_t T_new, int32_t max_len, int32_t path,
                              int32_t num_splits) {
  Shape s;
  if (!shape_of(d, &s) || B < 0 || T_new < 0 || max_len < 0 || num_splits < 0) return 0;
  if (path < MLA_PATH_ABSORBED || path > MLA_PATH_SPARSE) return 0;
  const bool decode = T_new == 1;
  const int splits = decode ? auto_splits(B, path == MLA_PATH_SPARSE ? d->topk : max_len, num_splits) : 1;
  return carve(d, B * T_new, decode, max_len, path, splits, nullptr).total;
}

size_t mla_workspace_bytes(const mla_dims* d, int32_t B, int32_t T_new, int32_t max_len, int32_t path) {
  return mla_workspace_bytes_ex(d, B, T_new, max_len, path, 0);
}

// ------------------------------------------------------------------------------------------
// Stage entry points
// ------------------------------------------------------------------------------------------
int mla_gemm(const void* a, int32_t lda, const void* w, int32_t M, int32_t N, int32_t K, void* out,
             int32_t ldo, int32_t out_dtype, hipStream_t stream) {
  trace(__func__, stream, "M=%d N=%d K=%d lda=%d ldo=%d out_dtype=%d", M, N, K, lda, ldo, out_dtype);
  if (M < 0 || N < 0 || K < 0) return MLA_ERR_SHAPE;
  if (M == 0 || N == 0) return MLA_OK;
  if (!a || !w || !out) return MLA_ERR_NULL;
  if (K % 8 != 0 || lda < K || lda % 8 != 0 || ldo < N) return MLA_ERR_SHAPE;
  if (out_dtype != MLA_OUT_BF16 && out_dtype != MLA_OUT_F32) return MLA_ERR_UNSUPPORTED;
  GemmArgs g = gemm_args(a, lda, M, K);
  int n = 0;
  push(g, seg(w, N, out, ldo, out_dtype == MLA_OUT_F32, n));
  CHECK_HIP(launch_gemm(g, nullptr, 0, stream));
  return MLA_OK;
}

int mla_rmsnorm(const float* x, int32_t ldx, const void* gain, int32_t M, int32_t N, float eps,
                void* out, int32_t ldo, hipStream_t stream) {
  trace(__func__, stream, "M=%d N=%d ldx=%d ldo=%d", M, N, ldx, ldo);
  if (M < 0 || N < 0) return MLA_ERR_SHAPE;
  if (M == 0 || N == 0) return MLA_OK;
  if (!x || !gain || !out) return MLA_ERR_NULL;
  if (N % 4 != 0 || ldx < N || ldx % 4 != 0 || ldo < N || ldo % 4 != 0) return MLA_ERR_SHAPE;
  CHECK_HIP(launch_rmsnorm(x, ldx, (const uint16_t*)gain, M, N, eps, (uint16_t*)out, ldo, nullptr, stream));
  return MLA_OK;
}

int mla_layernorm(const float* x, int32_t ldx, const void* gain, const void* bias, int32_t M,
                  int32_t N, float eps, void* out, int32_t ldo, hipStream_t stream) {
  trace(__func__, stream, "M=%d N=%d ldx=%d ldo=%d", M, N, ldx, ldo);
  if (M < 0 || N < 0) return MLA_ERR_SHAPE;
  if (M == 0 || N == 0) return MLA_OK;
  if (!x || !gain || !bias || !out) return MLA_ERR_NULL;
  if (N % 4 != 0 || ldx < N || ldx % 4 != 0 || ldo < N || ldo % 4 != 0) return MLA_ERR_SHAPE;
  CHECK_HIP(launch_layernorm(x, ldx, (const uint16_t*)gain, (const uint16_t*)bias, M, N, eps,
                             (uint16_t*)out, ldo, stream));
  return MLA_OK;
}

int mla_prefill_attention(const mla_dims* d, const void* q, const mla_cache* cache,
                          const int32_t* start_pos, int32_t max_end, int32_t B, int32_t T,
                          const float* g_pre, void* u, int32_t out_dtype, float* lse,
                          hipStream_t stream) {
  trace(__func__, stream, "B=%d T=%d max_end=%d out_dtype=%d", B, T, max_end, out_dtype);
  Shape s;
  if (!d) return MLA_ERR_NULL;
  if (!shape_of(d, &s)) return MLA_ERR_UNSUPPORTED;
  if (B < 0 || T < 0) return MLA_ERR_SHAPE;
  if (B == 0 || T == 0) return MLA_OK;
  if (!q || !start_pos || !u || !cache) return MLA_ERR_NULL;
  if (!cache->k || !cache->v) return MLA_ERR_NULL;
  if (cache->batch < B || cache->T_cap <= 0 || max_end < T) return MLA_ERR_SHAPE;
  if (max_end > cache->T_cap) return MLA_ERR_CAPACITY;
  if (out_dtype != MLA_OUT_BF16 && out_dtype != MLA_OUT_F32) return MLA_ERR_UNSUPPORTED;
  PrefillAttnArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)cache->k;
  a.v = (const uint16_t*)cache->v;
  a.start = start_pos;
  a.g_pre = g_pre;
  a.u = u;
  a.u_f32 = out_dtype == MLA_OUT_F32;
  a.lse = lse;
  a.B = B;
  a.T = T;
  a.T_cap = cache->T_cap;
  a.scale = d->softmax_scale;
  CHECK_HIP(launch_prefill_attention(s, a, stream));
  return MLA_OK;
}

int mla_absorb_query(const mla_dims* d, const void* q, int32_t ldq, const void* w_kv_b, int32_t B,
                     void* q_tilde, hipStream_t stream) {
  trace(__func__, stream, "B=%d ldq=%d", B, ldq);
  Shape s;
  if (!d) return MLA_ERR_NULL;
  if (!shape_of(d, &s)) return MLA_ERR_UNSUPPORTED;
  if (B < 0) return MLA_ERR_SHAPE;
  if (B == 0) return MLA_OK;
  if (!q || !w_kv_b || !q_tilde) return MLA_ERR_NULL;
  if (ldq < d->n_heads * (d->d_nope + d->d_shared)) return MLA_ERR_SHAPE;
  CHECK_HIP(launch_absorb_q(s, (const uint16_t*)q, ldq, (const uint16_t*)w_kv_b, B, (uint16_t*)q_tilde, stream));
  return MLA_OK;
}

static int decode_attention_common(const mla_dims* d, const void* q_tilde, const mla_cache* cache,
                                   const int32_t* n_visible, int32_t max_visible,
                                   const int32_t* sel_idx, const int32_t* sel_cnt, int32_t B,
                                   int32_t num_splits, float* o_latent, float* lse, void* ws,
                                   size_t ws_bytes, hipStream_t stream, bool gather) {
  Shape s;
  if (!d) return MLA_ERR_NULL;
  if (!shape_of(d, &s)) return MLA_ERR_UNSUPPORTED;
  if (B < 0 || num_splits < 0) return MLA_ERR_SHAPE;
  if (B == 0) return MLA_OK;
  if (!q_tilde || !cache || !o_latent || !ws) return MLA_ERR_NULL;
  if (gather ? (!sel_idx || !sel_cnt || !has_dsa(d)) : !n_visible) return gather && !has_dsa(d) ? MLA_ERR_UNSUPPORTED : MLA_ERR_NULL;
  const int span = gather ? d->topk : max_visible;
  int rc = check_cache(d, cache, B, gather ? 0 : max_visible);
  if (rc) return rc;
  if (span < 1) return MLA_ERR_SHAPE;
  const int splits = auto_splits(B, span, num_splits);
  Carver cv(ws);
  uint16_t* part_o = cv.take<uint16_t>((size_t)B * splits * d->n_heads * d->kv_lora);
  float* part_ml = cv.take<float>((size_t)B * splits * d->n_heads * 2);
  if (cv.off > ws_bytes) return MLA_ERR_WORKSPACE;
  DecodeAttnArgs a{};
  a.q_tilde = (const uint16_t*)q_tilde;
  a.latent = (const uint16_t*)cache->latent;
  a.fp8 = fp8_latent(cache);
  a.pages = page_table(cache);
  a.n_vis = n_visible;
  a.vis_offset = 0;
  a.sel_idx = sel_idx;
  a.sel_cnt = sel_cnt;
  a.sel_stride = d->topk;
  a.B = B;
  a.T_cap = cache->T_cap;
  a.n_splits = splits;
  a.chunk = split_chunk(span, splits);
  a.scale = d->softmax_scale;
  a.part_o = part_o;
  a.part_ml = part_ml;
  a.o_latent = o_latent;
  a.lse = lse;
  CHECK_HIP(launch_decode_attention(s, a, gather, stream));
  return MLA_OK;
}

int mla_decode_attention(const mla_dims* d, const void* q_tilde, const mla_cache* cache,
                         const int32_t* n_visible, int32_t max_visible, int32_t B, int32_t num_splits,
                         float* o_latent, float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  trace(__func__, stream, "B=%d max_visible=%d num_splits=%d ws_bytes=%zu", B, max_visible, num_splits, ws_bytes);
  return decode_attention_common(d, q_tilde, cache, n_visible, max_visible, nullptr, nullptr, B,
                                 num_splits, o_latent, lse, ws, ws_bytes, stream, false);
}

int mla_sparse_attention(const mla_dims* d, const void* q_tilde, const mla_cache* cache,
                         const int32_t* sel_idx, const int32_t* sel_cnt, int32_t B, int32_t num_splits,
                         float* o_latent, float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  trace(__func__, stream, "B=%d num_splits=%d ws_bytes=%zu", B, num_splits, ws_bytes);
  return decode_attention_common(d, q_tilde, cache, nullptr, 0, sel_idx, sel_cnt, B, num_splits,
                                 o_latent, lse, ws, ws_bytes, stream, true);
}

int mla_expanded_attention(const mla_dims* d, const void* q, const mla_cache* cache,
                           const int32_t* n_visible, int32_t max_visible, int32_t B, float* z,
                           float* lse, hipStream_t stream) {
  trace(__func__, stream, "B=%d max_visible=%d", B, max_visible);
  Shape s;
  if (!d) return MLA_ERR_NULL;
  if (!shape_of(d, &s)) return MLA_ERR_UNSUPPORTED;
  if (B < 0) return MLA_ERR_SHAPE;
  if (B == 0) return MLA_OK;
  if (!q || !cache || !n_visible || !z) return MLA_ERR_NULL;
  if (!cache->k || !cache->v) return MLA_ERR_NULL;
  if (cache->batch < B || cache->T_cap <= 0) return MLA_ERR_SHAPE;
  if (max_visible > cache->T_cap) return MLA_ERR_CAPACITY;
  ExpandedAttnArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)cache->k;
  a.v = (const uint16_t*)cache->v;
  a.n_vis = n_visible;
  a.B = B;
  a.T_cap = cache->T_cap;
  a.scale = d->softmax_scale;
  a.z = z;
  a.lse = lse;
  CHECK_HIP(launch_expanded_attention(s, a, stream));
  return MLA_OK;
}

int mla_debug_scores(const mla_dims* d, const void* q, const void* k, int32_t k_heads, int32_t B, int32_t Tq,
                     int32_t Tk, int32_t D, float* logits, hipStream_t stream) {
  trace(__func__, stream, "B=%d Tq=%d Tk=%d D=%d k_heads=%d", B, Tq, Tk, D, k_heads);
  Shape s;
  if (!d) return MLA_ERR_NULL;
  if (!shape_of(d, &s)) return MLA_ERR_UNSUPPORTED;
  if (B < 0 || Tq < 0 || Tk < 0) return MLA_ERR_SHAPE;
  if (D != d->d_nope + d->d_shared && D != d->kv_lora + d->d_shared) return MLA_ERR_SHAPE;
  if (k_heads != 1 && k_heads != d->n_heads) return MLA_ERR_SHAPE;
  if ((size_t)B * d->n_heads * Tq * Tk > MLA_DEBUG_SCORES_MAX) return MLA_ERR_SHAPE;
  if (B == 0 || Tq == 0 || Tk == 0) return MLA_OK;
  if (!q || !k || !logits) return MLA_ERR_NULL;
  if (((uintptr_t)q & 15) != 0 || ((uintptr_t)k & 15) != 0) return MLA_ERR_SHAPE;
  ScoresArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.B = B;
  a.H = d->n_heads;
  a.Hk = k_heads;
  a.Tq = Tq;
  a.Tk = Tk;
  a.D = D;
  a.scale = d->softmax_scale;
  a.logits = logits;
  CHECK_HIP(launch_debug_scores(a, stream));
  return MLA_OK;
}

int mla_value_up_gate(const mla_dims* d, const float* o_latent, const void* w_kv_b, const float* g_pre,
                      int32_t B, void* u, int32_t out_dtype, hipStream_t stream) {
  trace(__func__, stream, "B=%d out_dtype=%d", B, out_dtype);
  Shape s;
  if (!d) return MLA_ERR_NULL;
  if (!shape_of(d, &s)) return MLA_ERR_UNSUPPORTED;
  if (B < 0) return MLA_ERR_SHAPE;
  if (B == 0) return MLA_OK;
  if (!o_latent || !w_kv_b || !u) return MLA_ERR_NULL;
  if (out_dtype != MLA_OUT_BF16 && out_dtype != MLA_OUT_F32) return MLA_ERR_UNSUPPORTED;
  CHECK_HIP(launch_vup_gate(s, o_latent, (const uint16_t*)w_kv_b, g_pre, B, u,
                            out_dtype == MLA_OUT_F32, stream));
  return MLA_OK;
}

int mla_index_projections(const mla_dims* d, const mla_weights* w, const void* x, int32_t M, float* q_idx,
                          float* w_idx, void* k_idx, void* ws, size_t ws_bytes, hipStream_t stream) {
  trace(__func__, stream, "M=%d ws_bytes=%zu", M, ws_bytes);
  Shape s;
  if (!d) return MLA_ERR_NULL;
  if (!shape_of(d, &s)) return MLA_ERR_UNSUPPORTED;
  if (!has_dsa(d)) return MLA_ERR_UNSUPPORTED;
  if (M < 0) return MLA_ERR_SHAPE;
  if (M == 0) return MLA_OK;
  int rc = check_weights(d, w);
  if (rc) return rc;
  if (!idx_weights(w) || !w->w_idx_q) return MLA_ERR_NULL;
  if (!x || !q_idx || !w_idx || !k_idx || !ws) return MLA_ERR_NULL;
  // the workspace of a sparse decode step of M sequences, which runs these same launches
  Ws wsp = carve(d, M, true, 1, MLA_PATH_SPARSE, auto_splits(M, d->topk, 0), ws);
  if (wsp.total > ws_bytes) return MLA_ERR_WORKSPACE;
  wsp.qidx = q_idx;
  wsp.aw = w_idx;
  wsp.kidx = (uint16_t*)k_idx;
  return run_projections(d, w, x, M, wsp, true, true, stream);
}

int kv_append(const mla_dims* d, const mla_cache* cache, const int32_t* pos, int32_t max_end,
              int32_t B, int32_t T, const void* c, const void* r, const void* k_nope, const void* v,
              const void* idx_k, hipStream_t stream) {
  trace(__func__, stream, "B=%d T=%d max_end=%d", B, T, max_end);
  Shape s;
  if (!d) return MLA_ERR_NULL;
  if (!shape_of(d, &s)) return MLA_ERR_UNSUPPORTED;
  if (B < 0 || T < 0) return MLA_ERR_SHAPE;
  if (B == 0 || T == 0) return MLA_OK;
  if (!pos || !c || !r) return MLA_ERR_NULL;
  int rc = check_cache(d, cache, B, max_end);
  if (rc) return rc;
  if (max_end < T) return MLA_ERR_SHAPE;
  if (idx_k && !has_dsa(d)) return MLA_ERR_UNSUPPORTED;
  KvAppendArgs a = append_args(d, cache, pos, B, T);
  const int H = d->n_heads;
  a.c = (const uint16_t*)c;
  a.ld_c = d->kv_lora;
  a.r = (const uint16_t*)r;
  a.ld_r = d->d_shared;
  a.latent = (uint16_t*)cache->latent;
  if (k_nope && cache->k) {
    a.k_nope = (const uint16_t*)k_nope;
    a.ld_k_tok = H * d->d_nope;
    a.ld_k_head = d->d_nope;
    a.k = (uint16_t*)cache->k;
  }
  if (v && cache->v) {
    a.v_new = (const uint16_t*)v;
    a.ld_v_tok = H * d->d_v;
    a.ld_v_head = d->d_v;
    a.v = (uint16_t*)cache->v;
  }
  if (idx_k && cache->idx_k) {
    a.idx_new = (const uint16_t*)idx_k;
    a.ld_idx = d->d_idx;
    a.idx = (uint16_t*)cache->idx_k;
  }
  CHECK_HIP(launch_kv_append(a, stream));
  return MLA_OK;
}

static int index_topk_common(const mla_dims* d, const float* q_idx, const float* w_idx,
                             const void* idx_k_cache, const float* idx_k_scales, int32_t T_cap,
                             const int32_t* n_visible, int32_t max_visible, int32_t B, int32_t* out_idx,
                             int32_t* out_cnt, float* out_scores, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  Shape s;
  if (!d) return MLA_ERR_NULL;
  if (!shape_of(d, &s)) return MLA_ERR_UNSUPPORTED;
  if (!has_dsa(d)) return MLA_ERR_UNSUPPORTED;
  if (B < 0 || T_cap <= 0 || max_visible < 0) return MLA_ERR_SHAPE;
  if (B == 0) return MLA_OK;
  if (!q_idx || !w_idx || !idx_k_cache || !n_visible || !out_idx || !out_cnt) return MLA_ERR_NULL;
  if (max_visible > T_cap) return MLA_ERR_CAPACITY;
  if (!ws) return MLA_ERR_NULL;
  Carver cv(ws);
  float* scores = out_scores;
  int stride = T_cap;
  if (!scores) {
    stride = max_visible > 0 ? max_visible : 1;
    scores = cv.take<float>((size_t)B * stride);
  }
  int32_t* scratch = cv.take<int32_t>(index_topk_scratch_words(B, stride));
  if (cv.off > ws_bytes) return MLA_ERR_WORKSPACE;
  IndexScoreArgs sa{};
  sa.q_idx = q_idx;
  sa.w_idx = w_idx;
  sa.idx_k = (const uint16_t*)idx_k_cache;
  sa.idx_scale = idx_k_scales;
  sa.n_vis = n_visible;
  sa.B = B;
  sa.T_cap = T_cap;
  sa.scale = 1.0f / sqrtf((float)(d->n_idx_heads * d->d_idx));
  sa.scores = scores;
  sa.score_stride = stride;
  TopkArgs ta{};
  ta.scores = scores;
  ta.score_stride = stride;
  ta.n_vis = n_visible;
  ta.B = B;
  ta.k = d->topk;
  ta.out_idx = out_idx;
  ta.out_stride = d->topk;
  ta.out_cnt = out_cnt;
  CHECK_HIP(launch_index_topk(sa, max_visible, ta, scratch, stream));
  return MLA_OK;
}

int dsa_index_topk(const mla_dims* d, const float* q_idx, const float* w_idx, const void* idx_k_cache,
                   int32_t T_cap, const int32_t* n_visible, int32_t max_visible, int32_t B,
                   int32_t* out_idx, int32_t* out_cnt, float* out_scores, void* ws, size_t ws_bytes,
                   hipStream_t stream) {
  trace(__func__, stream, "B=%d T_cap=%d max_visible=%d ws_bytes=%zu", B, T_cap, max_visible, ws_bytes);
  return index_topk_common(d, q_idx, w_idx, idx_k_cache, nullptr, T_cap, n_visible, max_visible, B,
                           out_idx, out_cnt, out_scores, ws, ws_bytes, stream);
}

int dsa_index_topk_fp8(const mla_dims* d, const float* q_idx, const float* w_idx, const void* idx_k_codes,
                       const float* idx_k_scales, int32_t T_cap, const int32_t* n_visible,
                       int32_t max_visible, int32_t B, int32_t* out_idx, int32_t* out_cnt,
                       float* out_scores, void* ws, size_t ws_bytes, hipStream_t stream) {
  trace(__func__, stream, "B=%d T_cap=%d max_visible=%d ws_bytes=%zu", B, T_cap, max_visible, ws_bytes);
  if (!idx_k_scales) return MLA_ERR_NULL;
  if (d && d->d_idx != 128) return MLA_ERR_UNSUPPORTED;
  return index_topk_common(d, q_idx, w_idx, idx_k_codes, idx_k_scales, T_cap, n_visible, max_visible, B,
                           out_idx, out_cnt, out_scores, ws, ws_bytes, stream);
}

// ------------------------------------------------------------------------------------------
// Whole-layer calls
// ------------------------------------------------------------------------------------------
// The projections of T new tokens per sequence and their append to every cache present
// (everything before attention): x-GEMM, the two RMSNorms, q_b (with the index query segment
// when idx_query), kv_b when the expanded cache is kept, the index-key LayerNorm, kv_append.
static int prefill_front(const mla_dims* d, const mla_weights* w, const mla_cache* cache,
                         const int32_t* start_pos, const void* x, int B, int T, const Ws& wsp, bool with_idx,
                         bool idx_query, hipStream_t stream) {
  const int M = B * T, H = d->n_heads;
  const bool expanded_cache = cache->k && cache->v;
  int rc = run_projections(d, w, x, M, wsp, with_idx, idx_query, stream);
  if (rc) return rc;
  // the kv up-projection writes k_nope and v straight into the expanded cache when its large-M
  // kernel runs (kv_append then adds the shared-key part of each head's k row); otherwise it
  // writes them to the workspace for kv_append to copy
  bool kv_scattered = false;
  if (expanded_cache) {
    GemmArgs g = gemm_args(wsp.c, d->kv_lora, M, d->kv_lora);
    int n = 0;
    push(g, seg(w->w_kv_b, H * (d->d_nope + d->d_v), wsp.kv, H * (d->d_nope + d->d_v), false, n));
    if (!cache->block_table) {
      g.cs = CacheScatter{(uint16_t*)cache->k, (uint16_t*)cache->v, start_pos, T, cache->T_cap, H, d->d_nope, d->d_v,
                          d->d_nope + d->d_shared};
      kv_scattered = gemm_scatter_ok(g);
      if (!kv_scattered) g.cs = CacheScatter{};
    }
    CHECK_HIP(launch_gemm(g, wsp.gemm_ws, wsp.gemm_ws_bytes, stream));
  }
  KvAppendArgs a = append_args(d, cache, start_pos, B, T);
  a.c = wsp.c;
  a.ld_c = d->kv_lora;
  a.r = wsp.r;
  a.ld_r = d->d_shared;
  a.latent = (uint16_t*)cache->latent;
  if (expanded_cache && kv_scattered) {
    a.k = (uint16_t*)cache->k;  // shared-key part only (k_nope null)
  } else if (expanded_cache) {
    a.k_nope = wsp.kv;
    a.ld_k_tok = H * (d->d_nope + d->d_v);
    a.ld_k_head = d->d_nope + d->d_v;
    a.v_new = wsp.kv + d->d_nope;
    a.ld_v_tok = H * (d->d_nope + d->d_v);
    a.ld_v_head = d->d_nope + d->d_v;
    a.k = (uint16_t*)cache->k;
    a.v = (uint16_t*)cache->v;
  }
  if (with_idx) {
    a.idx_new = wsp.kidx;
    a.ld_idx = d->d_idx;
    a.idx = (uint16_t*)cache->idx_k;
  }
  CHECK_HIP(launch_kv_append(a, stream));
  return MLA_OK;
}

int mla_prefill(const mla_dims* d, const mla_weights* w, const mla_cache* cache, const int32_t* start_pos,
                int32_t max_end, const void* x, int32_t B, int32_t T, void* y, int32_t out_dtype,
                float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  trace(__func__, stream, "B=%d T=%d max_end=%d out_dtype=%d ws_bytes=%zu", B, T, max_end, out_dtype, ws_bytes);
  Shape s;
  if (!d) return MLA_ERR_NULL;
  if (!shape_of(d, &s)) return MLA_ERR_UNSUPPORTED;
  if (B < 0 || T < 0) return MLA_ERR_SHAPE;
  if (B == 0 || T == 0) return MLA_OK;
  int rc = check_weights(d, w);
  if (rc) return rc;
  if (!start_pos || !x || !y || !ws) return MLA_ERR_NULL;
  rc = check_cache(d, cache, B, max_end);
  if (rc) return rc;
  if (cache->block_table) return MLA_ERR_UNSUPPORTED;  // dense prefill attends over the expanded cache
  if (!cache->k || !cache->v) return MLA_ERR_NULL;
  if (max_end < T) return MLA_ERR_SHAPE;
  if (out_dtype != MLA_OUT_BF16 && out_dtype != MLA_OUT_F32) return MLA_ERR_UNSUPPORTED;
  const bool with_idx = has_dsa(d) && cache->idx_k && w->w_idx_k && w->g_idx_k && w->b_idx_k && w->w_idx_w;
  const int M = B * T, H = d->n_heads, dqk = d->d_nope + d->d_shared;
  const Ws wsp = carve(d, M, false, max_end, 0, 1, ws);
  if (wsp.total > ws_bytes) return MLA_ERR_WORKSPACE;

  rc = prefill_front(d, w, cache, start_pos, x, B, T, wsp, with_idx, false, stream);
  if (rc) return rc;
  {
    PrefillAttnArgs a{};
    a.q = wsp.q;
    a.k = (const uint16_t*)cache->k;
    a.v = (const uint16_t*)cache->v;
    a.start = start_pos;
    a.g_pre = d->use_gate ? wsp.gpre : nullptr;
    a.u = wsp.u;
    a.u_f32 = 0;
    a.lse = lse;
    a.B = B;
    a.T = T;
    a.T_cap = cache->T_cap;
    a.scale = d->softmax_scale;
    CHECK_HIP(launch_prefill_attention(s, a, stream));
  }
  {
    GemmArgs g = gemm_args(wsp.u, H * d->d_v, M, H * d->d_v);
    int n = 0;
    push(g, seg(w->w_o, d->hidden, y, d->hidden, out_dtype == MLA_OUT_F32, n));
    CHECK_HIP(launch_gemm(g, wsp.gemm_ws, wsp.gemm_ws_bytes, stream));
  }
  return MLA_OK;
}

// ---- Gated DSA prefill ----
// Rows (tokens) are processed in chunks of sparse_rows(): absorbed queries, index scores + top-k,
// gathered latent attention (one split per row), value up-projection and gate; then one o_proj
// GEMM over all rows.

struct SparseWs {
  uint16_t* qt;      // [R, H, kv_lora + d_shared]
  float* scores;     // [R, max_end]
  int32_t* sel;      // [R, topk]
  int32_t* cnt;      // [R]
  int32_t* scratch;  // index_topk_scratch_words(R, max_end)
  uint16_t* part_o;  // [R, H, kv_lora] fp16
  float* part_ml;    // [R, H, 2]
  float* olat;       // [R, H, kv_lora]
  size_t total;
};

static SparseWs carve_sparse(const mla_dims* d, int R, int max_end, char* base) {
  Carver cv(base);
  SparseWs w{};
  const int H = d->n_heads;
  w.qt = cv.take<uint16_t>((size_t)R * H * (d->kv_lora + d->d_shared));
  w.scores = cv.take<float>((size_t)R * max_end);
  w.sel = cv.take<int32_t>((size_t)R * d->topk);
  w.cnt = cv.take<int32_t>((size_t)R);
  w.scratch = cv.take<int32_t>(index_topk_scratch_words(R, max_end));
  w.part_o = cv.take<uint16_t>((size_t)R * H * d->kv_lora);
  w.part_ml = cv.take<float>((size_t)R * H * 2);
  w.olat = cv.take<float>((size_t)R * H * d->kv_lora);
  w.total = cv.off;
  return w;
}

// Rows per chunk: the largest of 2048, 1024, 512, 256 whose per-chunk buffers fit in 1 GiB (256
// at least), and never more than the call's rows.
static int sparse_rows(const mla_dims* d, int M, int max_end) {
  int R = 4096;
  while (R > 256 && carve_sparse(d, R, max_end, nullptr).total > (size_t(1) << 31)) R /= 2;
  return M < R ? M : R;
}

size_t mla_workspace_bytes_prefill_sparse(const mla_dims* d, int32_t B, int32_t T, int32_t max_end) {
  Shape s;
  if (!d || !shape_of(d, &s) || !has_dsa(d) || B <= 0 || T <= 0 || max_end < T) return 0;
  const int M = B * T, R = sparse_rows(d, M, max_end);
  return carve(d, M, false, max_end, 0, 1, nullptr).total + carve_sparse(d, R, max_end, nullptr).total;
}

int mla_prefill_sparse(const mla_dims* d, const mla_weights* w, const mla_cache* cache, const int32_t* start_pos,
                       int32_t max_end, const void* x, int32_t B, int32_t T, void* y, int32_t out_dtype,
                       int32_t* sel_idx, int32_t* sel_cnt, float* scores, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  trace(__func__, stream, "B=%d T=%d max_end=%d out_dtype=%d ws_bytes=%zu", B, T, max_end, out_dtype, ws_bytes);
  Shape s;
  if (!d) return MLA_ERR_NULL;
  if (!shape_of(d, &s)) return MLA_ERR_UNSUPPORTED;
  if (!has_dsa(d)) return MLA_ERR_UNSUPPORTED;
  if (B < 0 || T < 0) return MLA_ERR_SHAPE;
  if (B == 0 || T == 0) return MLA_OK;
  int rc = check_weights(d, w);
  if (rc) return rc;
  if (!idx_weights(w) || !w->w_idx_q) return MLA_ERR_NULL;
  if (!start_pos || !x || !y || !ws) return MLA_ERR_NULL;
  rc = check_cache(d, cache, B, max_end);
  if (rc) return rc;
  if (!cache->idx_k) return MLA_ERR_NULL;
  if (max_end < T) return MLA_ERR_SHAPE;
  if (out_dtype != MLA_OUT_BF16 && out_dtype != MLA_OUT_F32) return MLA_ERR_UNSUPPORTED;
  const int M = B * T, H = d->n_heads, dqk = d->d_nope + d->d_shared, R = sparse_rows(d, M, max_end);
  const Ws wsp = carve(d, M, false, max_end, 0, 1, ws);
  const SparseWs sw = carve_sparse(d, R, max_end, (char*)ws + wsp.total);
  if (wsp.total + sw.total > ws_bytes) return MLA_ERR_WORKSPACE;

  rc = prefill_front(d, w, cache, start_pos, x, B, T, wsp, true, true, stream);
  if (rc) return rc;
  for (int r0 = 0; r0 < M; r0 += R) {
    const int n = M - r0 < R ? M - r0 : R;  // rows r0 .. r0 + n - 1; row r is token r % T of sequence r / T
    int32_t* sel = sel_idx ? sel_idx + (size_t)r0 * d->topk : sw.sel;
    int32_t* cnt = sel_cnt ? sel_cnt + r0 : sw.cnt;
    CHECK_HIP(launch_absorb_q(s, wsp.q + (size_t)r0 * H * dqk, H * dqk, (const uint16_t*)w->w_kv_b, n, sw.qt, stream));
    IndexScoreArgs sa{};
    sa.q_idx = wsp.qidx + (size_t)r0 * d->n_idx_heads * d->d_idx;
    sa.w_idx = wsp.aw + (size_t)r0 * d->n_idx_heads;
    sa.idx_k = (const uint16_t*)cache->idx_k;
    sa.idx_scale = idx_scales(d, cache);
    sa.pages = page_table(cache);
    sa.n_vis = start_pos;
    sa.vis_offset = 1;
    sa.B = n;
    sa.T_cap = cache->T_cap;
    sa.scale = 1.0f / sqrtf((float)(d->n_idx_heads * d->d_idx));
    float* row_scores = scores ? scores + (size_t)r0 * max_end : sw.scores;
    sa.scores = row_scores;
    sa.score_stride = max_end;
    sa.row0 = r0;
    sa.rows_per_seq = T;
    TopkArgs ta{};
    ta.scores = row_scores;
    ta.score_stride = max_end;
    ta.n_vis = start_pos;
    ta.vis_offset = 1;
    ta.B = n;
    ta.k = d->topk;
    ta.out_idx = sel;
    ta.out_stride = d->topk;
    ta.out_cnt = cnt;
    ta.row0 = r0;
    ta.rows_per_seq = T;
    CHECK_HIP(launch_index_topk(sa, max_end, ta, sw.scratch, stream));
    DecodeAttnArgs a{};
    a.q_tilde = sw.qt;
    a.latent = (const uint16_t*)cache->latent;
    a.fp8 = fp8_latent(cache);
    a.pages = page_table(cache);
    a.sel_idx = sel;
    a.sel_cnt = cnt;
    a.sel_stride = d->topk;
    a.B = n;
    a.T_cap = cache->T_cap;
    a.n_splits = 1;
    a.chunk = split_chunk(d->topk, 1);
    a.scale = d->softmax_scale;
    a.part_o = sw.part_o;
    a.part_ml = sw.part_ml;
    a.o_latent = sw.olat;
    a.lse = nullptr;
    a.row0 = r0;
    a.rows_per_seq = T;
    CHECK_HIP(launch_decode_attention(s, a, true, stream));
    CHECK_HIP(launch_vup_gate(s, sw.olat, (const uint16_t*)w->w_kv_b,
                              d->use_gate ? wsp.gpre + (size_t)r0 * H * d->d_v : nullptr, n,
                              wsp.u + (size_t)r0 * H * d->d_v, 0, stream));
  }
  {
    GemmArgs g = gemm_args(wsp.u, H * d->d_v, M, H * d->d_v);
    int n = 0;
    push(g, seg(w->w_o, d->hidden, y, d->hidden, out_dtype == MLA_OUT_F32, n));
    CHECK_HIP(launch_gemm(g, wsp.gemm_ws, wsp.gemm_ws_bytes, stream));
  }
  return MLA_OK;
}

int mla_decode(const mla_dims* d, const mla_weights* w, const mla_cache* cache, const int32_t* seq_len,
               int32_t max_len, const void* x, int32_t B, int32_t path, int32_t num_splits,
               int32_t* sel_idx, int32_t* sel_cnt, void* y, int32_t out_dtype, void* ws, size_t ws_bytes,
               hipStream_t stream) {
  trace(__func__, stream, "B=%d max_len=%d path=%d num_splits=%d out_dtype=%d ws_bytes=%zu", B, max_len, path, num_splits, out_dtype, ws_bytes);
  Shape s;
  if (!d) return MLA_ERR_NULL;
  if (!shape_of(d, &s)) return MLA_ERR_UNSUPPORTED;
  if (path < MLA_PATH_ABSORBED || path > MLA_PATH_SPARSE) return MLA_ERR_UNSUPPORTED;
  if (B < 0 || num_splits < 0 || max_len < 0) return MLA_ERR_SHAPE;
  if (B == 0) return MLA_OK;
  int rc = check_weights(d, w);
  if (rc) return rc;
  if (!seq_len || !x || !y || !ws) return MLA_ERR_NULL;
  rc = check_cache(d, cache, B, max_len);
  if (rc) return rc;
  if (max_len < 1) return MLA_ERR_SHAPE;
  if (out_dtype != MLA_OUT_BF16 && out_dtype != MLA_OUT_F32) return MLA_ERR_UNSUPPORTED;
  const bool sparse = path == MLA_PATH_SPARSE;
  if (sparse && (!has_dsa(d) || !idx_weights(w) || !cache->idx_k)) return has_dsa(d) ? MLA_ERR_NULL : MLA_ERR_UNSUPPORTED;
  if (path == MLA_PATH_EXPANDED && (!cache->k || !cache->v)) return MLA_ERR_NULL;
  const bool with_idx = has_dsa(d) && cache->idx_k && idx_weights(w);
  const bool expanded_cache = cache->k && cache->v;
  const int H = d->n_heads, dqk = d->d_nope + d->d_shared;
  const int span = sparse ? d->topk : max_len;
  const int splits = auto_splits(B, span, num_splits);
  const Ws wsp = carve(d, B, true, max_len, path, splits, ws);
  if (wsp.total > ws_bytes) return MLA_ERR_WORKSPACE;

  // projections of the new token
  rc = run_projections(d, w, x, B, wsp, with_idx, sparse, stream);
  if (rc) return rc;
  if (expanded_cache) {
    GemmArgs g = gemm_args(wsp.c, d->kv_lora, B, d->kv_lora);
    int n = 0;
    push(g, seg(w->w_kv_b, H * (d->d_nope + d->d_v), wsp.kv, H * (d->d_nope + d->d_v), false, n));
    CHECK_HIP(launch_gemm(g, wsp.gemm_ws, wsp.gemm_ws_bytes, stream));
  }
  // append the new token to every cache present, before attending (it sees itself)
  {
    KvAppendArgs a = append_args(d, cache, seq_len, B, 1);
    a.c = wsp.c;
    a.ld_c = d->kv_lora;
    a.r = wsp.r;
    a.ld_r = d->d_shared;
    a.latent = (uint16_t*)cache->latent;
    if (expanded_cache) {
      a.k_nope = wsp.kv;
      a.ld_k_tok = H * (d->d_nope + d->d_v);
      a.ld_k_head = d->d_nope + d->d_v;
      a.v_new = wsp.kv + d->d_nope;
      a.ld_v_tok = H * (d->d_nope + d->d_v);
      a.ld_v_head = d->d_nope + d->d_v;
      a.k = (uint16_t*)cache->k;
      a.v = (uint16_t*)cache->v;
    }
    if (with_idx) {
      a.idx_new = wsp.kidx;
      a.ld_idx = d->d_idx;
      a.idx = (uint16_t*)cache->idx_k;
    }
    CHECK_HIP(launch_kv_append(a, stream));
  }
  const float* gate = d->use_gate ? wsp.gpre : nullptr;
  if (path == MLA_PATH_EXPANDED) {
    ExpandedAttnArgs a{};
    a.q = wsp.q;
    a.k = (const uint16_t*)cache->k;
    a.v = (const uint16_t*)cache->v;
    a.n_vis = seq_len;
    a.vis_offset = 1;
    a.B = B;
    a.T_cap = cache->T_cap;
    a.scale = d->softmax_scale;
    a.z = wsp.z;
    a.lse = nullptr;
    CHECK_HIP(launch_expanded_attention(s, a, stream));
    CHECK_HIP(launch_gate_mul(wsp.z, gate, B * H * d->d_v, wsp.u, 0, stream));
  } else {
    int32_t* sel = sel_idx ? sel_idx : wsp.sel;
    int32_t* cnt = sel_cnt ? sel_cnt : wsp.cnt;
    if (sparse) {
      IndexScoreArgs sa{};
      sa.q_idx = wsp.qidx;
      sa.w_idx = wsp.aw;
      sa.idx_k = (const uint16_t*)cache->idx_k;
      sa.idx_scale = idx_scales(d, cache);
      sa.pages = page_table(cache);
      sa.n_vis = seq_len;
      sa.vis_offset = 1;
      sa.B = B;
      sa.T_cap = cache->T_cap;
      sa.scale = 1.0f / sqrtf((float)(d->n_idx_heads * d->d_idx));
      sa.scores = wsp.scores;
      sa.score_stride = max_len;
      TopkArgs ta{};
      ta.scores = wsp.scores;
      ta.score_stride = max_len;
      ta.n_vis = seq_len;
      ta.vis_offset = 1;
      ta.B = B;
      ta.k = d->topk;
      ta.out_idx = sel;
      ta.out_stride = d->topk;
      ta.out_cnt = cnt;
      CHECK_HIP(launch_index_topk(sa, max_len, ta, wsp.topk_scratch, stream));
    }
    CHECK_HIP(launch_absorb_q(s, wsp.q, H * dqk, (const uint16_t*)w->w_kv_b, B, wsp.qt, stream));
    DecodeAttnArgs a{};
    a.q_tilde = wsp.qt;
    a.latent = (const uint16_t*)cache->latent;
    a.fp8 = fp8_latent(cache);
    a.pages = page_table(cache);
    a.n_vis = seq_len;
    a.vis_offset = 1;
    a.sel_idx = sel;
    a.sel_cnt = cnt;
    a.sel_stride = d->topk;
    a.B = B;
    a.T_cap = cache->T_cap;
    a.n_splits = splits;
    a.chunk = split_chunk(span, splits);
    a.scale = d->softmax_scale;
    a.part_o = wsp.part_o;
    a.part_ml = wsp.part_ml;
    a.o_latent = wsp.olat;
    a.lse = nullptr;
    CHECK_HIP(launch_decode_attention(s, a, sparse, stream));
    CHECK_HIP(launch_vup_gate(s, wsp.olat, (const uint16_t*)w->w_kv_b, gate, B, wsp.u, 0, stream));
  }
  {
    GemmArgs g = gemm_args(wsp.u, H * d->d_v, B, H * d->d_v);
    int n = 0;
    push(g, seg(w->w_o, d->hidden, y, d->hidden, out_dtype == MLA_OUT_F32, n));
    CHECK_HIP(launch_gemm(g, wsp.gemm_ws, wsp.gemm_ws_bytes, stream));
  }
  return MLA_OK;
}

}  // extern "C"

// ------------------------------------------------------------------------------------------
// Decode without allocation: mla_decode's workspace in a static device array of the library
// (one copy per GPU, kept until the process ends). In host code `scratch` only names the symbol;
// its device address on each GPU comes from hipGetSymbolAddress, looked up once per device with
// that device current, and only that address is ever passed to a kernel.
// ------------------------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// this device's address of `scratch`, or null (err set) if the lookup failed
void* scratch_on_current_device(hipError_t* err) {
  int dev = -1;
  if ((*err = hipGetDevice(&dev)) != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  ScratchSlot& s = g_scratch[dev];
  std::call_once(s.once, [&s]() {
    void* p = nullptr;
    s.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    s.ptr = s.err == hipSuccess ? p : nullptr;
  });
  *err = s.err;
  return s.ptr;
}
}  // namespace

extern "C" int mla_decode_noalloc(const mla_dims* d, const mla_weights* w, const mla_cache* cache,
                                  const int32_t* seq_len, int32_t max_len, const void* x, int32_t B, int32_t path,
                                  int32_t num_splits, int32_t* sel_idx, int32_t* sel_cnt, void* y,
                                  int32_t out_dtype, hipStream_t stream) {
  trace(__func__, stream, "B=%d max_len=%d path=%d num_splits=%d out_dtype=%d", B, max_len, path, num_splits, out_dtype);
  // the size check comes first and touches no device
  if (d && B > 0) {
    const size_t need = mla_workspace_bytes_ex(d, B, 1, max_len, path, num_splits);
    if (need > (size_t)MLA_NOALLOC_SCRATCH_BYTES) return MLA_ERR_WORKSPACE;
  }
  hipError_t err;
  void* ws = scratch_on_current_device(&err);
  if (!ws) return MLA_ERR_HIP;
  return mla_decode(d, w, cache, seq_len, max_len, x, B, path, num_splits, sel_idx, sel_cnt, y, out_dtype, ws,
                    (size_t)MLA_NOALLOC_SCRATCH_BYTES, stream);
}

extern "C" int mla_debug_flags(uint32_t* flags, int32_t* checks_built, hipStream_t stream) {
  if (!flags || !checks_built) return MLA_ERR_NULL;
  static_assert(kDbgAppendPos == MLA_DBG_APPEND_POS && kDbgAppendPage == MLA_DBG_APPEND_PAGE &&
                    kDbgTopkOffset == MLA_DBG_TOPK_OFFSET,
                "debug flag bits");
  *flags = 0;
  *checks_built = kDebugChecks ? 1 : 0;
  uint32_t fa = 0, ft = 0;
  if (read_debug_flags_append(&fa, stream) != hipSuccess || read_debug_flags_topk(&ft, stream) != hipSuccess)
    return MLA_ERR_HIP;
  *flags = fa | ft;
  return MLA_OK;
}
