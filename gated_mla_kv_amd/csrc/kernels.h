// Internal launchers of the gfx950 kernels (host side). The C ABI in api.cpp validates its
// arguments and calls these.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gmla {

enum class Shape { K3, Tiny };

// out_lo (or null): the bf16 residual f - hi of every output, at the same ldo
// RMSNorm of M rows of N fp32 values (N % 4 == 0): out = bf16(x * rsqrt(mean(x^2) + eps) * gain),
// and out_lo (if set) the remainder x*... - out in bf16.
struct RmsNormJob {
  const float* x;
  int ldx;
  const uint16_t* gain;
  int M, N;
  uint16_t* out;
  int ldo;
  uint16_t* out_lo;
};
// both jobs in one launch (b.M = 0: job a only)
hipError_t launch_rmsnorm2(const RmsNormJob& a, const RmsNormJob& b, float eps, hipStream_t s);
hipError_t launch_rmsnorm(const float* x, int ldx, const uint16_t* gain, int M, int N, float eps,
                          uint16_t* out, int ldo, uint16_t* out_lo, hipStream_t s);
hipError_t launch_layernorm(const float* x, int ldx, const uint16_t* gain, const uint16_t* bias,
                            int M, int N, float eps, uint16_t* out, int ldo, hipStream_t s);
// The DSA index key of M tokens in fp64: out[m] = bf16(LayerNorm(w . x[m]) * gain + bias) with a
// 128-row w [128, K] (K a multiple of 32). partial: index_key_splits(M, K) * M * 128 doubles.
int index_key_splits(int M, int K);
hipError_t launch_index_key_f64(const uint16_t* x, int ldx, const uint16_t* w, const uint16_t* gain,
                                const uint16_t* bias, int M, int K, double eps, double* partial, uint16_t* out,
                                int ldo, hipStream_t s);

// Paged latent and index caches: position p of sequence s lives in cache row
//   table[s * max_blocks + p / page_size] * page_size + p % page_size
// of a pool of n_pages pages (page indices clamped into the pool); without a table, in row
// s * T_cap + p. page_size is a multiple of 32, so a 32-position tile never crosses a page.
struct PageTable {
  const int32_t* table;  // [batch, max_blocks] or null
  int page_size, max_blocks, n_pages;
};
__device__ __forceinline__ size_t cache_row(const PageTable& pt, int T_cap, int seq, int pos) {
  if (!pt.table) return (size_t)seq * T_cap + pos;
  const int pg = min(max(pt.table[(size_t)seq * pt.max_blocks + pos / pt.page_size], 0), pt.n_pages - 1);
  return (size_t)pg * pt.page_size + pos % pt.page_size;
}
// As cache_row for a wave-uniform (seq, pos), with the table entry read through the scalar
// cache: its wait (lgkmcnt) leaves the wave's outstanding vector loads in flight, where a vector
// load of the entry would wait for all of them.
__device__ __forceinline__ size_t cache_row_uniform(const PageTable& pt, int T_cap, int seq, int pos) {
  if (!pt.table) return (size_t)seq * T_cap + pos;
  const int32_t* e = pt.table + (size_t)__builtin_amdgcn_readfirstlane(seq) * pt.max_blocks +
                     __builtin_amdgcn_readfirstlane(pos) / pt.page_size;
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(e) : "memory");
  const int pg = min(max(v, 0), pt.n_pages - 1);
  return (size_t)pg * pt.page_size + pos % pt.page_size;
}

struct KvAppendArgs {
  const int32_t* pos;  // [B] first position of each sequence's new tokens
  int B, T, T_cap, H, L, DS, DN, DV, DI;
  const uint16_t* c; int ld_c;            // [B*T, ld_c]
  const uint16_t* r; int ld_r;            // [B*T, ld_r]
  const uint16_t* k_nope; int ld_k_tok, ld_k_head;
  const uint16_t* v_new; int ld_v_tok, ld_v_head;
  const uint16_t* idx_new; int ld_idx;
  uint16_t* latent;  // [B, T_cap, L+DS] or null (FP8: [B, T_cap, kFp8RowBytes] bytes)
  uint16_t* k;       // [B, H, T_cap, DN+DS] or null
  uint16_t* v;       // [B, H, T_cap, DV] or null
  uint16_t* idx;     // [B, T_cap, DI] or null (FP8: [B, T_cap, DI] codes)
  int latent_fp8, idx_fp8;
  float* idx_scale;  // FP8 index keys: [B, T_cap] scales
  PageTable pages;   // rows of latent / idx / idx_scale (k and v are never paged)
};
// FP8 main-cache row (K3): 512 E4M3 codes of c, four fp32 scales (blocks of 128), r in bf16
constexpr int kFp8Codes = 512, kFp8ScaleOff = 512, kFp8ROff = 528, kFp8RowBytes = 656;
hipError_t launch_kv_append(const KvAppendArgs& a, hipStream_t s);

struct PrefillAttnArgs {
  const uint16_t* q;       // [B, T, H, DQK]
  const uint16_t* k;       // [B, H, T_cap, DQK]
  const uint16_t* v;       // [B, H, T_cap, DV]
  const int32_t* start;    // [B]
  const float* g_pre;      // [B, T, H*DV] f32 or null
  void* u;                 // [B, T, H*DV]
  int u_f32;
  float* lse;              // [B, H, T] or null
  int B, T, T_cap;
  float scale;             // softmax scale
};
hipError_t launch_prefill_attention(Shape s, const PrefillAttnArgs& a, hipStream_t st);
hipError_t launch_prefill_attention_k3(const PrefillAttnArgs& a, hipStream_t st);

struct DecodeAttnArgs {
  const uint16_t* q_tilde;  // [B, H, L+DS]
  const uint16_t* latent;   // [B, T_cap, L+DS]
  const int32_t* n_vis;     // [B] visible positions (contiguous mode), plus vis_offset
  int vis_offset;
  const int32_t* sel_idx;   // [B, sel_stride] selected positions (gather mode)
  const int32_t* sel_cnt;   // [B]
  int sel_stride;
  int B, T_cap, n_splits, chunk;
  float scale;
  uint16_t* part_o; // [B, n_splits, H, L] fp16: each split's output divided by its own sum l
  float* part_ml;   // [B, n_splits, H, 2]
  float* o_latent;  // [B, H, L]
  float* lse;       // [B, H] or null
  int row0, rows_per_seq;  // see row_map (latent rows of sequence row_map(..).seq)
  int fp8;          // latent rows are FP8 main-cache rows (kFp8RowBytes each)
  PageTable pages;  // latent rows of (sequence, position)
};
hipError_t launch_decode_attention(Shape s, const DecodeAttnArgs& a, bool gather, hipStream_t st);
hipError_t launch_absorb_q(Shape s, const uint16_t* q, int ldq, const uint16_t* wkvb, int B,
                           uint16_t* qt, hipStream_t st);
hipError_t launch_vup_gate(Shape s, const float* o, const uint16_t* wkvb, const float* g_pre,
                           int B, void* u, int u_f32, hipStream_t st);

// Row b of a launch over B rows is row row0 + b of the call. rows_per_seq consecutive rows of the
// call (1 when 0) belong to one sequence: the new tokens of a prefill, each seeing one more
// position than the one before it. The sequence indexes the caches and n_vis; the visible length
// of the row is n_vis[seq] + vis_offset + (its rank in the sequence).
struct RowMap {
  int seq, extra;
};
__device__ __forceinline__ RowMap row_map(int row0, int rows_per_seq, int b) {
  const int g = row0 + b, r = rows_per_seq > 0 ? rows_per_seq : 1;
  return RowMap{g / r, g % r};
}

struct IndexScoreArgs {
  const float* q_idx;     // [B, 32, 128] fp32 (fed to the MFMA as bf16 hi + lo)
  const float* w_idx;     // [B, 32]
  const uint16_t* idx_k;  // [B, T_cap, 128] bf16, or E4M3 codes when idx_scale is set
  const float* idx_scale; // [B, T_cap] FP8 key scales, or null
  PageTable pages;        // rows of idx_k / idx_scale
  const int32_t* n_vis;   // [B], plus vis_offset
  int vis_offset;
  int B, T_cap;
  float scale;            // 1/sqrt(n_idx * d_idx)
  float* scores;          // [B, score_stride]
  int score_stride;
  int32_t* hist;          // [B, 4096] counts of the scores' top-12-bit order-key digit (zeroed first)
  int row0, rows_per_seq; // see row_map
  int n_chunks, row_tiles; // index_scores_kernel: workgroups per row; 32-position tiles of the longest row
};

struct TopkArgs {
  const float* scores;  // [B, score_stride]
  int score_stride;
  const int32_t* n_vis;  // [B], plus vis_offset
  int vis_offset;
  int B, k;
  int32_t* out_idx;  // [B, out_stride]
  int out_stride;
  int32_t* out_cnt;  // [B]
  int32_t* hist;     // [B, 4096] from the score kernel
  int32_t* info;     // [B, 4]: boundary bin, keys above it, keys in it
  int32_t* sel;      // [B, 4]: path, threshold key, last kept tie position, chunk count
  int32_t* off;      // [B, off_stride]: output offset of each 2048-position chunk
  int32_t* above;    // [B, off_stride]: per chunk, keys above the boundary bin
  int32_t* ncand;    // [B, off_stride]: per chunk, keys inside the boundary bin
  uint32_t* cand;    // [B, off_stride, 2, 2048]: per chunk, those keys, then their positions
  int off_stride;    // chunk slots per row
  int cpw;           // chunks per workgroup of the fused select + compaction
  int row0, rows_per_seq;  // see row_map
};
// int32 scratch words of the index-score + top-k launches for B rows of score_stride scores
size_t index_topk_scratch_words(int B, int score_stride);
// index scores, then the top-k selection; scratch: index_topk_scratch_words(a.B, score_stride)
hipError_t launch_index_topk(IndexScoreArgs sa, int max_visible, TopkArgs ta, int32_t* scratch,
                             hipStream_t st);

struct ExpandedAttnArgs {
  const uint16_t* q;  // [B, H, DQK]
  const uint16_t* k;  // [B, H, T_cap, DQK]
  const uint16_t* v;  // [B, H, T_cap, DV]
  const int32_t* n_vis;
  int vis_offset;
  int B, T_cap;
  float scale;
  float* z;    // [B, H, DV]
  float* lse;  // [B, H] or null
};
// Raw attention logits s[b,h,i,j] = scale * q[b,i,h,:] . k[b, Hk == 1 ? 0 : h, j, :] (unmasked)
struct ScoresArgs {
  const uint16_t* q;  // [B, Tq, H, D] bf16
  const uint16_t* k;  // [B, Hk, Tk, D] bf16, Hk = H or 1
  int B, H, Hk, Tq, Tk, D;  // D a multiple of 8
  float scale;
  float* logits;      // [B, H, Tq, Tk]
};
hipError_t launch_debug_scores(const ScoresArgs& a, hipStream_t st);
hipError_t launch_expanded_attention(Shape s, const ExpandedAttnArgs& a, hipStream_t st);
hipError_t launch_gate_mul(const float* z, const float* g_pre, int n, void* u, int u_f32,
                           hipStream_t st);

// Debug builds (GMLA_DEBUG_CHECKS): device-side bound checks in kv_append and the top-k
// compaction. A failed check sets its bit in a device word of the kernel's source file; the
// offending write is skipped in every build, so the checks change no result. read_debug_flags_*
// return that word and clear it (0 and no device access in a normal build).
enum : uint32_t {
  kDbgAppendPos = 1u,   // kv_append: a token position outside [0, T_cap)
  kDbgAppendPage = 2u,  // kv_append: a page-table entry outside [0, n_pages)
  kDbgTopkOffset = 4u,  // top-k compaction: an output offset at or past the kept count
};
#ifdef GMLA_DEBUG_CHECKS
constexpr bool kDebugChecks = true;
#else
constexpr bool kDebugChecks = false;
#endif
hipError_t read_debug_flags_append(uint32_t* flags, hipStream_t st);
hipError_t read_debug_flags_topk(uint32_t* flags, hipStream_t st);

}  // namespace gmla
