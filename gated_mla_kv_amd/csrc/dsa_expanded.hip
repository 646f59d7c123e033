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
// topk_kernel (eq. (6)): S = the min(k, t) largest I, ties to the lower position, -0 == +0,
// written in ascending position order. One workgroup per query row. A radix select over
// order-preserving 32-bit keys with 12-, 12- and 8-bit digits (the row's keys held in registers,
// LDS histograms) narrows the
// k-th largest key down until a whole bin is taken or the key tau is exact. The compaction gives
// each wave a contiguous run of positions: a counting pass, a scan of the 16 wave counts, and a
// writing pass with ballot prefix counts, so the output is ascending by construction and the
// copies of tau kept are the lowest-position ones.
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

__global__ __launch_bounds__(256) void index_scores_kernel(IndexScoreArgs a) {
  constexpr int NIH = 32, DI = 128, KS = DI / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g2 = lane >> 5, l32 = lane & 31;
  const int b = blockIdx.y;
  const int t = min(min(a.n_vis[b] + a.vis_offset, a.T_cap), a.score_stride);
  const int base = blockIdx.x * kScorePosPerWG;
  if (base >= t) return;
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
    if (pos < end && g2 == 0) a.scores[(size_t)b * a.score_stride + pos] = sc;
  };
  if (p0a < end) score(p0a, kfa);
  if (p0b < end) score(p0b, kfb);
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
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
  __shared__ int hist[kHistRep * kHistPitch];
  __shared__ int scan_tmp[kTopkThreads / 64 + 1];
  __shared__ int sh_bin, sh_above, sh_cnt;
  __shared__ int wcnt[2][kTopkWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x;
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

hipError_t launch_index_scores(const IndexScoreArgs& a, int max_visible, hipStream_t st) {
  if (a.B <= 0 || max_visible <= 0) return hipSuccess;
  index_scores_kernel<<<dim3(cdiv(max_visible, kScorePosPerWG), a.B), 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  if (a.B <= 0) return hipSuccess;
  topk_kernel<<<a.B, kTopkThreads, 0, st>>>(a);
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
