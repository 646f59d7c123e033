// Gated DSA index scores and top-k selection, and decode attention over the expanded cache.
//
// index_scores_kernel (K3.1 Gated DSA blog, eq. (5)):
//   I[b, s] = (1/sqrt(n_idx d_idx)) sum_h a[b,h] ReLU(q^I[b,h] . k^I[b,s]),  s < t
// The dot products are a [32 heads x 128] . [128 x 32 positions] bf16 MFMA per wave, with the
// index keys loaded from HBM straight into the B operand (one 16-byte load per lane and k-step,
// 256 bytes per position, each read once). Lane l ends with position l%32 and 16 heads, so the
// head-weighted ReLU sum is in-lane plus one xor-32 shuffle. 1/sqrt(32*128) = 1/64 is folded
// into a exactly.
//
// Top-k (eq. (6)): S = the min(k, t) largest I, ties to the lower position, -0 == +0, written
// in ascending position order, over order-preserving 32-bit keys of the fp32 scores.
// * index_scores_kernel also counts the top 12-bit digit of every key into the row's histogram.
// * topk_select_kernel (one workgroup per row) takes the bin where the count from the top reaches
//   k, sorts that bin's keys (with their positions) in LDS, and fixes the threshold key and the
//   last kept position among its copies; it scans the per-2048-position-chunk kept counts into
//   output offsets.
// * topk_compact_kernel (one workgroup per chunk) writes each chunk's kept positions in order.
// * A row whose boundary bin exceeds the LDS candidate buffer (e.g. thousands of equal scores)
//   runs the whole selection in its select workgroup instead: a radix select over 12-, 12- and
//   8-bit digits with the row's keys in registers, and an ordered compaction in which every
//   wave owns a contiguous run of positions.
//
// expanded_attn_kernel: one query per (b, h) against the expanded cache k [B,H,T_cap,192],
// v [B,H,T_cap,128] (KV cache card): 61,440 bytes per position, HBM bound at ~1 flop per byte,
// so plain fp32 VALU dot products; 4 lanes per key, 16 keys per wave per step, per-wave online
// softmax, waves merged through LDS.
#include "common.h"
#include "kernels.h"

namespace gmla {

// ------------------------------------------------------------------------------------------
// Index scores (K3 indexer: 32 heads x 128)
// ------------------------------------------------------------------------------------------
constexpr int kScorePosPerWG = 256;

__device__ __forceinline__ uint32_t order_key(float f);
constexpr int kHistBins = 4096;  // first radix digit: the top 12 bits of the order key

__global__ __launch_bounds__(256) void index_scores_kernel(IndexScoreArgs a) {
  constexpr int NIH = 32, DI = 128, KS = DI / 16;
  __shared__ int lhist[kHistBins];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g2 = lane >> 5, l32 = lane & 31;
  const int b = blockIdx.y;
  const int t = min(min(a.n_vis[b] + a.vis_offset, a.T_cap), a.score_stride);
  const int base = blockIdx.x * kScorePosPerWG;
  if (base >= t) return;
  for (int i = threadIdx.x; i < kHistBins; i += 256) lhist[i] = 0;
  const int end = min(base + kScorePosPerWG, t);
  const uint16_t* kb = a.idx_k + (size_t)b * a.T_cap * DI;
  // keys of this wave's positions p0 + l32 (two 32-position steps per wave), both loads in flight
  auto load_keys = [&](int p0, u32x4* kf) __attribute__((always_inline)) {
    const int pos = min(p0 + l32, end - 1);  // rows past the end re-read a valid row (not stored)
#pragma unroll
    for (int s = 0; s < KS; ++s) kf[s] = ld16(kb + (size_t)pos * DI + s * 16 + g2 * 8);
  };
  const int p0a = base + wave * 32, p0b = p0a + 4 * 32;
  u32x4 kfa[KS], kfb[KS];
  load_keys(p0a, kfa);
  if (p0b < end) load_keys(p0b, kfb);
  // A operand: q^I rows (heads) for this lane's head l32
  u32x4 qa[KS];
  const uint16_t* qrow = a.q_idx + ((size_t)b * NIH + l32) * DI;
#pragma unroll
  for (int s = 0; s < KS; ++s) qa[s] = ld16(qrow + s * 16 + g2 * 8);
  // head weights of the 16 heads this lane's accumulators hold: (r/4)*8 + g2*4 + r%4
  float wgt[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) wgt[r] = a.w_idx[(size_t)b * NIH + (r >> 2) * 8 + g2 * 4 + (r & 3)] * a.scale;
  auto score = [&](int p0, const u32x4* kf) __attribute__((always_inline)) {
    f32x16 acc = f32x16{};
#pragma unroll
    for (int s = 0; s < KS; ++s) acc = mfma32(qa[s], kf[s], acc);
    float sc = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc += wgt[r] * fmaxf(acc[r], 0.f);
    sc += __shfl_xor(sc, 32, 64);
    const int pos = p0 + l32;
    if (pos < end && g2 == 0) {
      a.scores[(size_t)b * a.score_stride + pos] = sc;
      atomicAdd(&lhist[order_key(sc) >> 20], 1);
    }
  };
  __syncthreads();  // histogram cleared
  if (p0a < end) score(p0a, kfa);
  if (p0b < end) score(p0b, kfb);
  __syncthreads();
  // the row's histogram gathers the workgroup's nonzero bins
  int* gh = a.hist + (size_t)b * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += 256) {
    const int c = lhist[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

__global__ void zero_words_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// ------------------------------------------------------------------------------------------
// Top-k
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0) u = 0;  // -0.0 and +0.0 are the same score
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int NT>
__device__ int block_exclusive_scan(int v, int* tmp /* NT/64 + 1 ints */, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < NT / 64; ++w) {
      const int c = tmp[w];
      tmp[w] = run;
      run += c;
    }
    tmp[NT / 64] = run;
  }
  __syncthreads();
  const int r = tmp[wave] + x - v;
  total = tmp[NT / 64];
  __syncthreads();
  return r;
}

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;

// number of lanes below this one with `pred` set, and the wave's total
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

constexpr int kTopkR = 65;                        // keys held per thread (one segment)
constexpr int kTopkSeg = kTopkR * kTopkThreads;    // 66,560 positions per segment

constexpr int kHistRep = 8;        // histogram replicas (lane % 8): at most 8 lanes per address
constexpr int kHistPitch = 4097;   // replica stride in words (not a multiple of the bank count)

// Positions past the row hold key 0. A real score never maps to a key below 2^20 (those are NaN
// bit patterns), so key 0 sits in digit-0 bin 0, under any threshold, and no pass needs a
// bounds test.
// The whole selection of row b inside one workgroup: the general path, for rows whose boundary
// bin holds more candidates than the chunked path keeps in LDS, or longer than it covers.
// hist: kHistRep * kHistPitch ints of LDS; scan_tmp: kTopkWaves + 1; shv: 3; wcnt: 2 * kTopkWaves.
__device__ __forceinline__ void topk_full_row(const TopkArgs& a, const int b, int* hist, int* scan_tmp,
                                           int* shv, int* wcnt_flat) {
  int& sh_bin = shv[0];
  int& sh_above = shv[1];
  int& sh_cnt = shv[2];
  int(*wcnt)[kTopkWaves] = (int(*)[kTopkWaves])wcnt_flat;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = min(a.n_vis[b] + a.vis_offset, a.score_stride);
  const int k = min(a.k, t);
  int32_t* out = a.out_idx + (size_t)b * a.out_stride;
  const float* sc = a.scores + (size_t)b * a.score_stride;
  if (t <= a.k) {  // short history: every visible position is kept
    for (int i = tid; i < a.k; i += kTopkThreads) out[i] = (i < t) ? i : -1;
    if (tid == 0) a.out_cnt[b] = t;
    return;
  }

  // Keys of segment sg: wave w owns positions sg*kTopkSeg + w*65*64 .. +65*64-1, its key u being
  // position ... + u*64 + lane (coalesced), all loads in flight at once. A row of one segment
  // (t <= 66,560) stays in registers for every pass.
  const int n_segs = cdiv(t, kTopkSeg);
  uint32_t keys[kTopkR];
  auto seg_base = [&](int sg) __attribute__((always_inline)) { return sg * kTopkSeg + wave * (kTopkR * 64); };
  auto load_seg = [&](int sg) __attribute__((always_inline)) {
    const int base = seg_base(sg);
    const float* p = sc + base + lane;
    const int lim = t - 1 - base - lane;  // u*64 <= lim <=> the position is visible
#pragma unroll
    for (int u = 0; u < kTopkR; ++u) keys[u] = __float_as_uint(p[min(u * 64, max(lim, 0))]);
#pragma unroll
    for (int u = 0; u < kTopkR; ++u) keys[u] = u * 64 <= lim ? order_key(__uint_as_float(keys[u])) : 0u;
  };
  load_seg(0);

  // ---- radix select over the keys: digits of 12, 12 and 8 bits from the top ----
  uint32_t prefix = 0, pmask = 0;
  int krem = k;
  bool whole_bin = false;  // the last decided bin is taken entirely
  int* my_hist = hist + (lane & (kHistRep - 1)) * kHistPitch;
#pragma unroll 1
  for (int level = 0; level < 3; ++level) {
    const int shift = level == 0 ? 20 : (level == 1 ? 8 : 0);
    const int nbins = level == 2 ? 256 : 4096;
    for (int i = tid; i < kHistRep * kHistPitch; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
#pragma unroll 1
    for (int sg = 0; sg < n_segs; ++sg) {
      if (n_segs > 1) load_seg(sg);
#pragma unroll
      for (int u = 0; u < kTopkR; ++u)
        if ((keys[u] & pmask) == prefix) atomicAdd(&my_hist[(keys[u] >> shift) & (uint32_t)(nbins - 1)], 1);
    }
    __syncthreads();
    // the bin where the count from the top reaches krem: thread j owns bins nbins-1-4j .. -3
    constexpr int PER = 4096 / kTopkThreads;
    int cntb[PER];
    int local = 0;
    const int top = nbins - 1 - PER * tid;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      cntb[q] = 0;
      if (top - q >= 0)
#pragma unroll
        for (int r = 0; r < kHistRep; ++r) cntb[q] += hist[r * kHistPitch + top - q];
      local += cntb[q];
    }
    int total;
    const int before = block_exclusive_scan<kTopkThreads>(local, scan_tmp, total);
    if (before < krem && before + local >= krem) {
      int cum = before;
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        if (cum < krem && cum + cntb[q] >= krem) {
          sh_bin = top - q;
          sh_above = cum;
          sh_cnt = cntb[q];
        }
        cum += cntb[q];
      }
    }
    __syncthreads();
    prefix |= (uint32_t)sh_bin << shift;
    pmask |= (uint32_t)(nbins - 1) << shift;
    krem -= sh_above;
    const int cnt = sh_cnt;
    __syncthreads();
    if (cnt == krem) {
      whole_bin = true;
      break;
    }
  }
  // kept: key > thr, plus (all 32 bits decided, tau = prefix) the krem lowest-position copies
  // of tau. A whole bin taken is key >= prefix (its undecided low bits are zero): thr = prefix-1.
  const uint32_t tau = prefix;
  const uint32_t thr = whole_bin ? prefix - 1u : tau;
  if (whole_bin) krem = 0;
  auto kept_gt = [&](uint32_t key) __attribute__((always_inline)) { return key > thr; };

  // ---- ordered compaction: wave w owns a contiguous run of each segment ----
  int out_base = 0, eq_base = 0;
#pragma unroll 1
  for (int sg = 0; sg < n_segs; ++sg) {
    if (n_segs > 1) load_seg(sg);
    int nk = 0, ne = 0;
#pragma unroll
    for (int u = 0; u < kTopkR; ++u) {
      nk += (int)__popcll(__ballot(kept_gt(keys[u])));
      ne += (int)__popcll(__ballot(!whole_bin && keys[u] == tau));
    }
    if (lane == 0) {
      wcnt[0][wave] = nk;
      wcnt[1][wave] = ne;
    }
    // recompute the predicates in the writing pass rather than keep 2 x 65 of them live
#pragma unroll
    for (int u = 0; u < kTopkR; ++u) asm volatile("" : "+v"(keys[u]));
    __syncthreads();
    int eq_before = eq_base, out_before = out_base, seg_keep = 0, seg_eq = 0;
    for (int w = 0; w < kTopkWaves; ++w) {
      const int take = max(0, min(krem - (eq_base + seg_eq), wcnt[1][w]));
      if (w < wave) {
        eq_before += wcnt[1][w];
        out_before += wcnt[0][w] + take;
      }
      seg_keep += wcnt[0][w] + take;
      seg_eq += wcnt[1][w];
    }
    const int take_w = max(0, min(krem - eq_before, ne));  // copies of tau this wave keeps
    int wpos = out_before, eq_seen = 0;
    const int base = seg_base(sg);
#pragma unroll
    for (int u = 0; u < kTopkR; ++u) {
      const bool eq = !whole_bin && keys[u] == tau;
      const uint64_t em = __ballot(eq);
      const bool keep = kept_gt(keys[u]) || (eq && eq_seen + lanes_below(em) < take_w);
      const uint64_t km = __ballot(keep);
      const int w = wpos + lanes_below(km);
      if (keep && w < a.k) out[w] = base + u * 64 + lane;
      wpos += (int)__popcll(km);
      eq_seen += (int)__popcll(em);
    }
    out_base += seg_keep;
    eq_base += seg_eq;
    __syncthreads();
  }
  for (int i = k + tid; i < a.k; i += kTopkThreads) out[i] = -1;
  if (tid == 0) a.out_cnt[b] = k;
}


// ---- chunked path ----
// The score kernel leaves each row's histogram of the 12-bit top digit. topk_select_kernel (one
// workgroup per row) finds the bin b0 where the count from the top reaches k, collects the keys
// of that bin (with their positions) in LDS, and radix-selects among them the threshold key thr
// (the krem-th largest, krem = k minus the count above b0) and, when only some of its copies
// are kept, the last kept position p_lim (the copies' positions radix-selected in turn).
// A position is kept iff key > thr, or key == thr and position <= p_lim.
// It also counts the kept positions of every 2048-position chunk and writes their exclusive scan.
// topk_compact_kernel (one workgroup per chunk) then writes its chunk's kept positions in order
// at that offset, so the output is ascending.
constexpr int kChunk = 2048;        // positions per compaction workgroup
constexpr int kMaxChunks = 1024;    // the chunked path covers rows of up to 2,097,152 positions
constexpr int kCandCap = 8192;      // boundary-bin keys held in LDS
enum { kSelDone = 0, kSelChunked = 1 };
constexpr int kSelLds = kHistRep * kHistPitch * 4 > kCandCap * 12 + kHistBins * 4
                            ? kHistRep * kHistPitch * 4 : kCandCap * 12 + kHistBins * 4;

// The r-th largest (1 <= r <= n) of the 32-bit values vals[0, n) in LDS, for the whole
// workgroup: three radix levels (12, 12 and 8 bits from the top) over an LDS histogram of 4096
// ints. *n_gt receives the count of values above it, *n_eq the count equal to it.
__device__ __forceinline__ uint32_t block_select_desc(const uint32_t* vals, int n, int r, int* hist,
                                                      int* scan_tmp, int* shv, int* n_gt, int* n_eq) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
  int gt = 0, eq = 0;
#pragma unroll 1
  for (int level = 0; level < 3; ++level) {
    const int shift = level == 0 ? 20 : (level == 1 ? 8 : 0);
    const int nbins = level == 2 ? 256 : 4096;
    for (int i = tid; i < kHistBins; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kTopkThreads) {
      const uint32_t v = vals[i];
      if ((v & pmask) == prefix) atomicAdd(&hist[(v >> shift) & (uint32_t)(nbins - 1)], 1);
    }
    __syncthreads();
    constexpr int PER = kHistBins / kTopkThreads;
    const int top = nbins - 1 - PER * tid;
    int cntb[PER];
    int local = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      cntb[q] = top - q >= 0 ? hist[top - q] : 0;
      local += cntb[q];
    }
    int total;
    const int before = block_exclusive_scan<kTopkThreads>(local, scan_tmp, total);
    const int rr = r - gt;
    if (before < rr && before + local >= rr) {
      int cum = before;
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        if (cum < rr && cum + cntb[q] >= rr) {
          shv[0] = top - q;
          shv[1] = cum;
          shv[2] = cntb[q];
        }
        cum += cntb[q];
      }
    }
    __syncthreads();
    prefix |= (uint32_t)shv[0] << shift;
    pmask |= (uint32_t)(nbins - 1) << shift;
    gt += shv[1];
    eq = shv[2];
    __syncthreads();
  }
  *n_gt = gt;
  *n_eq = eq;
  return prefix;
}

__global__ __launch_bounds__(kTopkThreads) void topk_select_kernel(TopkArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t big[kSelLds];  // full-row histograms | candidates
  __shared__ int scan_tmp[kTopkWaves + 1];
  __shared__ int shv[4];
  __shared__ int wcnt[2 * kTopkWaves];
  __shared__ int ccnt[kMaxChunks];
  const int tid = threadIdx.x, lane = tid & 63;
  const int b = blockIdx.x;
  const int t = min(a.n_vis[b] + a.vis_offset, a.score_stride);
  const int k = min(a.k, t);
  int32_t* sel = a.sel + (size_t)b * 4;
  int32_t* out = a.out_idx + (size_t)b * a.out_stride;
  const float* sc = a.scores + (size_t)b * a.score_stride;
  if (t <= a.k) {  // short history: every visible position is kept
    for (int i = tid; i < a.k; i += kTopkThreads) out[i] = (i < t) ? i : -1;
    if (tid == 0) {
      a.out_cnt[b] = t;
      sel[0] = kSelDone;
    }
    return;
  }
  const int nch = cdiv(t, kChunk);
  // ---- the bin where the count from the top reaches k: thread j owns bins 4095-4j .. -3 ----
  const int* gh = a.hist + (size_t)b * kHistBins;
  constexpr int PER = kHistBins / kTopkThreads;
  const int top = kHistBins - 1 - PER * tid;
  int cntb[PER];
  int local = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    cntb[q] = gh[top - q];
    local += cntb[q];
  }
  int total;
  const int before = block_exclusive_scan<kTopkThreads>(local, scan_tmp, total);
  if (before < k && before + local >= k) {
    int cum = before;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      if (cum < k && cum + cntb[q] >= k) {
        shv[0] = top - q;
        shv[1] = cum;
        shv[2] = cntb[q];
      }
      cum += cntb[q];
    }
  }
  if (tid == 0) shv[3] = 0;
  __syncthreads();
  const uint32_t b0 = (uint32_t)shv[0];
  const int krem = k - shv[1];
  const int c0 = shv[2];
  if (c0 > kCandCap || nch > kMaxChunks) {
    __syncthreads();
    topk_full_row(a, b, (int*)big, scan_tmp, shv, wcnt);
    if (tid == 0) sel[0] = kSelDone;
    return;
  }
  // ---- one pass over the row: chunk counts above b0, and the keys of bin b0 with their
  // positions. Wave w owns the chunks w, w + 16, ...: it counts each alone, then reserves room
  // for its candidates with one LDS atomic ----
  uint32_t* ckey = (uint32_t*)big;         // [kCandCap]
  int* cpos = (int*)(ckey + kCandCap);     // [kCandCap]
  int* lh = cpos + kCandCap;               // [kHistBins] histogram of the candidate selections
  uint32_t* tv = (uint32_t*)(lh + kHistBins);  // [kCandCap] ~position of each copy of thr
  const int wave = tid >> 6;
  constexpr int R = kChunk / 64;  // 32 loads per lane per chunk, all in flight
  for (int c = wave; c < nch; c += kTopkWaves) {
    const int p0 = c * kChunk;
    uint32_t kv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int p = p0 + r * 64 + lane;
      kv[r] = __float_as_uint(sc[min(p, t - 1)]);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) kv[r] = p0 + r * 64 + lane < t ? order_key(__uint_as_float(kv[r])) : 0u;
    int above = 0, nc = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      above += (int)__popcll(__ballot((kv[r] >> 20) > b0));
      nc += (int)__popcll(__ballot((kv[r] >> 20) == b0));
    }
    if (lane == 0) ccnt[c] = above;
    if (nc) {
      int cb = 0;
      if (lane == 0) cb = atomicAdd(&shv[3], nc);
      cb = __shfl(cb, 0, 64);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const bool is_c = (kv[r] >> 20) == b0;
        const uint64_t cm = __ballot(is_c);
        const int ci = cb + lanes_below(cm);
        if (is_c && ci < kCandCap) {
          ckey[ci] = kv[r];
          cpos[ci] = p0 + r * 64 + lane;
        }
        cb += (int)__popcll(cm);
      }
    }
  }
  __syncthreads();
  const int n = min(shv[3], kCandCap);
  // ---- thr = the krem-th largest candidate key; of its e copies the keep lowest positions stay ----
  int n_gt, e;
  const uint32_t thr = block_select_desc(ckey, n, krem, lh, scan_tmp, shv, &n_gt, &e);
  const int keep = krem - n_gt;  // 1 <= keep <= e
  int p_lim = 0x7FFFFFFF;
  if (keep < e) {
    if (tid == 0) shv[3] = 0;
    __syncthreads();
    for (int i0 = 0; i0 < n; i0 += kTopkThreads) {
      const int i = i0 + tid;
      const bool is_t = i < n && ckey[i] == thr;
      const uint64_t m = __ballot(is_t);
      if (m) {
        int cb = 0;
        if (lane == 0) cb = atomicAdd(&shv[3], (int)__popcll(m));
        cb = __shfl(cb, 0, 64);
        if (is_t) tv[cb + lanes_below(m)] = ~(uint32_t)cpos[i];
      }
    }
    __syncthreads();
    int g2, e2;
    p_lim = (int)~block_select_desc(tv, min(shv[3], kCandCap), keep, lh, scan_tmp, shv, &g2, &e2);
  }
  // ---- kept candidates per chunk, then the chunks' output offsets ----
  for (int i = tid; i < n; i += kTopkThreads) {
    const uint32_t key = ckey[i];
    if (key > thr || (key == thr && cpos[i] <= p_lim)) atomicAdd(&ccnt[cpos[i] / kChunk], 1);
  }
  __syncthreads();
  int tot;
  const int ex = block_exclusive_scan<kTopkThreads>(tid < nch ? ccnt[tid] : 0, scan_tmp, tot);
  if (tid < nch) a.off[(size_t)b * a.off_stride + tid] = ex;
  for (int i = k + tid; i < a.k; i += kTopkThreads) out[i] = -1;
  if (tid == 0) {
    a.out_cnt[b] = k;
    sel[1] = (int32_t)thr;
    sel[2] = p_lim;
    sel[3] = nch;
    sel[0] = kSelChunked;
  }
}

// grid (chunks, B), 256 threads: wave w writes the kept positions of chunk positions
// [512 w, 512 w + 512) in order, after those of the waves before it
__global__ __launch_bounds__(256) void topk_compact_kernel(TopkArgs a) {
  __shared__ int wc[4];
  const int b = blockIdx.y, c = blockIdx.x;
  const int32_t* sel = a.sel + (size_t)b * 4;
  if (sel[0] != kSelChunked || c >= sel[3]) return;
  const uint32_t thr = (uint32_t)sel[1];
  const int p_lim = sel[2];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = min(a.n_vis[b] + a.vis_offset, a.score_stride);
  const float* sc = a.scores + (size_t)b * a.score_stride;
  const int base = c * kChunk + wave * (kChunk / 4);
  constexpr int R = kChunk / 4 / 64;
  uint64_t km[R];
  int n = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int p = base + r * 64 + lane;
    const uint32_t key = p < t ? order_key(sc[p]) : 0u;
    km[r] = __ballot(key > thr || (key == thr && p <= p_lim));
    n += (int)__popcll(km[r]);
  }
  if (lane == 0) wc[wave] = n;
  __syncthreads();
  int w = a.off[(size_t)b * a.off_stride + c];
  for (int i = 0; i < wave; ++i) w += wc[i];
  int32_t* out = a.out_idx + (size_t)b * a.out_stride;
  const int kk = min(a.k, t);  // the kept total (guards the writes should the counts disagree)
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int o = w + lanes_below(km[r]);
    if (((km[r] >> lane) & 1) && o < kk) out[o] = base + r * 64 + lane;
    w += (int)__popcll(km[r]);
  }
}

// ------------------------------------------------------------------------------------------
// Expanded-cache decode attention
// ------------------------------------------------------------------------------------------
template <class S>
__global__ __launch_bounds__(256) void expanded_attn_kernel(ExpandedAttnArgs a) {
  constexpr int H = S::H, DQK = S::DN + S::DS, DV = S::DV, DQ4 = DQK / 4;
  static_assert(DQK % 4 == 0, "quarters");
  __shared__ float ms[4], lsum[4];
  __shared__ float os[4][DV];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kq = lane & 3, kk = lane >> 2;
  const int bh = blockIdx.x, b = bh / H, h = bh % H;
  const int n = min(a.n_vis[b] + a.vis_offset, a.T_cap);
  float qv[DQ4];
  const uint16_t* qrow = a.q + ((size_t)b * H + h) * DQK + kq * DQ4;
#pragma unroll
  for (int i = 0; i < DQ4; ++i) qv[i] = bf16_bits_to_f32(qrow[i]);
  const uint16_t* kb = a.k + (size_t)bh * a.T_cap * DQK;
  const uint16_t* vb = a.v + (size_t)bh * a.T_cap * DV;
  const float sl2 = a.scale * 1.4426950408889634f;
  constexpr int NV = cdiv(DV, 128);  // value pairs per lane
  float m_run = -INFINITY, l_run = 0.f, o[NV][2];
#pragma unroll
  for (int i = 0; i < NV; ++i) o[i][0] = o[i][1] = 0.f;
  for (int base = wave * 16; base < n; base += 64) {
    const int j = base + kk;
    float s = 0.f;
    if (j < n) {
      const uint16_t* kr = kb + (size_t)j * DQK + kq * DQ4;
      if constexpr (DQ4 % 8 == 0) {
#pragma unroll
        for (int c = 0; c < DQ4; c += 8) {
          const u32x4 w = ld16(kr + c);
          s += qv[c + 0] * lo_bf16(w.x) + qv[c + 1] * hi_bf16(w.x) + qv[c + 2] * lo_bf16(w.y) +
               qv[c + 3] * hi_bf16(w.y) + qv[c + 4] * lo_bf16(w.z) + qv[c + 5] * hi_bf16(w.z) +
               qv[c + 6] * lo_bf16(w.w) + qv[c + 7] * hi_bf16(w.w);
        }
      } else {
#pragma unroll
        for (int c = 0; c < DQ4; ++c) s += qv[c] * bf16_bits_to_f32(kr[c]);
      }
    }
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    s = (j < n) ? s * sl2 : -INFINITY;
    float mt = s;
#pragma unroll
    for (int off = 4; off < 64; off <<= 1) mt = fmaxf(mt, __shfl_xor(mt, off, 64));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = fast_exp2(m_run - m_new);
    const float p = fast_exp2(s - m_new);
    float ps = (kq == 0) ? p : 0.f;
    ps = wave_sum(ps);
    l_run = l_run * alpha + ps;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      o[i][0] *= alpha;
      o[i][1] *= alpha;
    }
#pragma unroll 4
    for (int k2 = 0; k2 < 16; ++k2) {
      const float pj = __shfl(p, k2 * 4, 64);
      const int j2 = base + k2;
      if (j2 < n) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          const int dv = 2 * lane + 128 * i;
          if (dv < DV) {
            const uint32_t w = *(const uint32_t*)(vb + (size_t)j2 * DV + dv);
            o[i][0] += pj * lo_bf16(w);
            o[i][1] += pj * hi_bf16(w);
          }
        }
      }
    }
  }
  if (lane == 0) {
    ms[wave] = m_run;
    lsum[wave] = l_run;
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int dv = 2 * lane + 128 * i;
    if (dv < DV) {
      os[wave][dv] = o[i][0];
      os[wave][dv + 1] = o[i][1];
    }
  }
  __syncthreads();
  float M = -INFINITY;
  for (int w = 0; w < 4; ++w) M = fmaxf(M, ms[w]);
  float den = 0.f, f[4];
  for (int w = 0; w < 4; ++w) {
    f[w] = (ms[w] == -INFINITY) ? 0.f : fast_exp2(ms[w] - M);
    den += f[w] * lsum[w];
  }
  for (int d = threadIdx.x; d < DV; d += 256) {
    float acc = 0.f;
    for (int w = 0; w < 4; ++w) acc += f[w] * os[w][d];
    a.z[(size_t)bh * DV + d] = den > 0.f ? acc / den : 0.f;
  }
  if (threadIdx.x == 0 && a.lse) a.lse[bh] = (M + __log2f(den)) * 0.6931471805599453f;
}

// u[i] = z[i] * sigmoid(g_pre[i]) over B*H*DV elements (z and g_pre f32; g_pre may be null).
__global__ void gate_mul_kernel(const float* z, const float* g_pre, int n, void* u, int u_f32) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float v = z[i];
  if (g_pre) v *= sigmoidf_(g_pre[i]);
  if (u_f32)
    ((float*)u)[i] = v;
  else
    ((uint16_t*)u)[i] = f32_to_bf16_bits(v);
}

size_t index_topk_scratch_words(int B, int score_stride) {
  return (size_t)B * (kHistBins + 4 + cdiv(score_stride, kChunk));
}

hipError_t launch_index_topk(IndexScoreArgs sa, int max_visible, TopkArgs ta, int32_t* scratch,
                             hipStream_t st) {
  if (sa.B <= 0) return hipSuccess;
  const int B = sa.B;
  sa.hist = ta.hist = scratch;
  ta.sel = scratch + (size_t)B * kHistBins;
  ta.off = ta.sel + (size_t)B * 4;
  ta.off_stride = cdiv(ta.score_stride, kChunk);
  zero_words_kernel<<<cdiv(B * kHistBins, 256), 256, 0, st>>>(sa.hist, B * kHistBins);
  if (max_visible > 0)
    index_scores_kernel<<<dim3(cdiv(max_visible, kScorePosPerWG), B), 256, 0, st>>>(sa);
  topk_select_kernel<<<B, kTopkThreads, 0, st>>>(ta);
  topk_compact_kernel<<<dim3(ta.off_stride, B), 256, 0, st>>>(ta);
  return hipGetLastError();
}

hipError_t launch_expanded_attention(Shape s, const ExpandedAttnArgs& a, hipStream_t st) {
  if (a.B <= 0) return hipSuccess;
  if (s == Shape::K3)
    expanded_attn_kernel<ShapeK3><<<a.B * ShapeK3::H, 256, 0, st>>>(a);
  else
    expanded_attn_kernel<ShapeTiny><<<a.B * ShapeTiny::H, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_gate_mul(const float* z, const float* g_pre, int n, void* u, int u_f32,
                           hipStream_t st) {
  if (n <= 0) return hipSuccess;
  gate_mul_kernel<<<cdiv(n, 256), 256, 0, st>>>(z, g_pre, n, u, u_f32);
  return hipGetLastError();
}

}  // namespace gmla
