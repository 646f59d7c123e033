// Decode attention in the latent space (absorbed MLA) and its sparse (Gated DSA) variant.
//
// With latent absorption (K3.1 Gated DSA blog, the note after eq. (10)) the score of head h
// against cached position j is q~_h . [c_j ; r_j] * scale, where q~_h = [W^K_h^T q_nope_h ;
// q_shared_h], and the head output is recovered as z_h = W^V_h sum_j p_j c_j. Each cached
// position is read once, as one 576-value latent row, for all 96 heads at once: 1,152 bytes
// instead of the expanded cache's 61,440 (KV cache card: 30,720 values per position).
//
// decode_attn_kernel: the generic form, used for the tiny oracle-scale shape (the K3 shape has
// its own kernel in decode_attn_k3.hip). One workgroup per (sequence, split), 4 waves.
// * The latent rows of a 32-position tile are staged in LDS (double-buffered, via registers,
//   16-byte loads, each HBM byte read once).
// * Waves 0..HP/32-1 each own 32 heads: their q~ rows sit in VGPRs as the B operand of
//   S^T = Lat Q~^T (v_mfma_f32_32x32x16_bf16, k over the 576 latent features), so lane l holds
//   head l%32; max/sum need one xor-32 shuffle. P^T (bf16) and the rescale factors go to LDS.
// * All four waves then accumulate O^T = Lat^T P^T for a quarter of the 512 latent output
//   features, taking Lat^T straight from the row-major tile with ds_read_b64_tr_b16.
// * Each split writes (max, sum) per head and its output divided by the sum, in fp16 (a convex
//   combination of latent rows, so bounded by the largest entry); decode_merge combines splits.
// GATHER (sparse DSA): positions come from the selected list instead of a contiguous range.
#include "common.h"
#include "kernels.h"

namespace gmla {

template <class S>
struct DecodeCfg {
  static constexpr int H = S::H, L = S::L, DS = S::DS, DL = S::L + S::DS;
  static constexpr int HP = round_up(H, 32);     // heads padded to 32-wide MFMA blocks
  static constexpr int DLP = round_up(DL, 32);   // score k dimension, padded
  static constexpr int LP = round_up(L, 32);     // output features, padded
  static constexpr int NSW = HP / 32;            // waves that compute scores
  static constexpr int KSD = DLP / 16;           // score k-steps
  static constexpr int NDT = LP / 32;            // 32-wide output feature tiles
  static constexpr int DTW = cdiv(NDT, 4);       // feature tiles per wave
  static constexpr int BT = 32;                  // positions per tile
  static constexpr int LROW = DLP + 8;           // LDS row stride of the latent tile (bf16)
  static constexpr int PROW = BT + 8;            // LDS row stride of P^T [head][pos]
  static constexpr int CH = DLP / 8;             // 16-byte chunks per padded row
  static constexpr int NCH = cdiv(BT * CH, 256); // chunks per thread per tile
  static_assert(NSW <= 4, "at most four score waves");
};

__device__ __forceinline__ int perm_row_d(int m) {
  const int a = m >> 3, g = (m >> 2) & 1, b = m & 3;
  return 16 * (a >> 1) + 8 * g + 4 * (a & 1) + b;
}

template <class S, bool GATHER>
__global__ __launch_bounds__(256) void decode_attn_kernel(DecodeAttnArgs a) {
  using C = DecodeCfg<S>;
  __shared__ __attribute__((aligned(16))) uint16_t Ls[2][C::BT * C::LROW];
  __shared__ __attribute__((aligned(16))) uint16_t Ps[C::HP * C::PROW];
  __shared__ float alpha_s[C::HP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g2 = lane >> 5, l32 = lane & 31;
  const int b = blockIdx.x / a.n_splits, split = blockIdx.x % a.n_splits;
  const int n_vis = GATHER ? min(a.sel_cnt[b], a.sel_stride) : min(a.n_vis[b] + a.vis_offset, a.T_cap);
  const int p0 = split * a.chunk;
  const int p1 = min(p0 + a.chunk, n_vis);
  const int n_pos = max(p1 - p0, 0);
  const int n_tiles = cdiv(n_pos, C::BT);
  const uint16_t* lat = a.latent + (size_t)row_map(a.row0, a.rows_per_seq, b).seq * a.T_cap * C::DL;
  const int32_t* sel = GATHER ? a.sel_idx + (size_t)b * a.sel_stride : nullptr;

  // ---- score waves: q~ for heads wave*32 + l32 ----
  const bool is_sw = wave < C::NSW;
  const int head = wave * 32 + l32;
  u32x4 qf[C::KSD];
  if (is_sw) {
    const uint16_t* qrow = a.q_tilde + ((size_t)b * C::H + head) * C::DL;
#pragma unroll
    for (int s = 0; s < C::KSD; ++s) {
      const int d = s * 16 + g2 * 8;
      qf[s] = (head < C::H && d < C::DL) ? ld16(qrow + d) : zero16();
    }
  }

  u32x4 rl[C::NCH];
  auto load_tile = [&](int t) {
    const int j0 = p0 + t * C::BT;
#pragma unroll
    for (int i = 0; i < C::NCH; ++i) {
      const int c = tid + 256 * i;
      const int row = c / C::CH, col = (c % C::CH) * 8;
      const int j = j0 + row;
      bool ok = c < C::BT * C::CH && j < p1 && col < C::DL;
      int pos = j;
      if (GATHER && ok) {
        pos = sel[j];
        ok = pos >= 0 && pos < a.T_cap;
      }
      rl[i] = ok ? ld16(lat + (size_t)pos * C::DL + col) : zero16();
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::NCH; ++i) {
      const int c = tid + 256 * i;
      if (c < C::BT * C::CH) st16(&Ls[buf][(c / C::CH) * C::LROW + (c % C::CH) * 8], rl[i]);
    }
  };

  const float sl2 = a.scale * 1.4426950408889634f;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[C::DTW][C::NSW];
#pragma unroll
  for (int i = 0; i < C::DTW; ++i)
#pragma unroll
    for (int j = 0; j < C::NSW; ++j) o[i][j] = f32x16{};

  const int krow_a = perm_row_d(l32);
  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    const int cur = t & 1;
    const int j0 = p0 + t * C::BT;
    if (t + 1 < n_tiles) load_tile(t + 1);
    if (is_sw) {
      // S^T [32 positions x 32 heads]
      f32x16 sacc = f32x16{};
      const uint16_t* lr = &Ls[cur][krow_a * C::LROW + g2 * 8];
#pragma unroll
      for (int s = 0; s < C::KSD; ++s) sacc = mfma32(ld16(lr + s * 16), qf[s], sacc);
      float mt = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = j0 + 16 * (r >> 3) + 8 * g2 + (r & 7);
        // a gathered position outside the cache gets probability 0
        const bool live = j < p1 && (!GATHER || (sel[j] >= 0 && sel[j] < a.T_cap));
        const float x = live ? sacc[r] * sl2 : -INFINITY;
        sacc[r] = x;
        mt = fmaxf(mt, x);
      }
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float m_new = fmaxf(m_run, mt);
      // while no position has been live, every p is 0 (not exp2(-inf + inf))
      const float m_ref = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_ref);
      m_run = m_new;
      float ls = 0.f;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          p[i] = fast_exp2(sacc[hh * 8 + i] - m_ref);
          ls += p[i];
        }
        st16(&Ps[head * C::PROW + hh * 16 + g2 * 8],
             u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                   pack_bf16x2(p[6], p[7])});
      }
      l_run = l_run * alpha + ls;
      if (g2 == 0) alpha_s[head] = alpha;
    }
    __syncthreads();
    // ---- O^T [features x heads] += Lat^T P^T for this wave's feature tiles ----
    {
      const int G = lane >> 4, jj = lane & 15;
      float al[C::NSW];
#pragma unroll
      for (int hs = 0; hs < C::NSW; ++hs) al[hs] = alpha_s[hs * 32 + l32];
      u32x4 pb[C::NSW][2];
#pragma unroll
      for (int hs = 0; hs < C::NSW; ++hs)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) pb[hs][ks] = ld16(&Ps[(hs * 32 + l32) * C::PROW + ks * 16 + g2 * 8]);
#pragma unroll
      for (int dt = 0; dt < C::DTW; ++dt) {
        const int ft = wave + 4 * dt;  // feature tile
        if (ft >= C::NDT) break;
#pragma unroll
        for (int hs = 0; hs < C::NSW; ++hs)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dt][hs][r] *= al[hs];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const uint16_t* lp =
              &Ls[cur][(ks * 16 + 8 * (G >> 1) + (jj >> 2)) * C::LROW + ft * 32 + 16 * (G & 1) + 4 * (jj & 3)];
          const u32x2 lo = lds_read_tr16(lp);
          const u32x2 hi = lds_read_tr16(lp + 4 * C::LROW);
          const u32x4 af = u32x4{lo.x, lo.y, hi.x, hi.y};
#pragma unroll
          for (int hs = 0; hs < C::NSW; ++hs) o[dt][hs] = mfma32(af, pb[hs][ks], o[dt][hs]);
        }
      }
    }
    if (t + 1 < n_tiles) store_tile(cur ^ 1);
    __syncthreads();
  }

  // ---- write this split's partial results: (max, sum) and O / sum in fp16 ----
  const size_t part = (size_t)b * a.n_splits + split;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (is_sw && g2 == 0) {
    if (head < C::H) {
      a.part_ml[(part * C::H + head) * 2 + 0] = m_run;  // base-2 scaled logits
      a.part_ml[(part * C::H + head) * 2 + 1] = l_tot;
    }
    alpha_s[head] = l_tot > 0.f ? 1.0f / l_tot : 0.f;  // the loop's last barrier has passed
  }
  __syncthreads();
#pragma unroll
  for (int dt = 0; dt < C::DTW; ++dt) {
    const int ft = wave + 4 * dt;
    if (ft >= C::NDT) break;
#pragma unroll
    for (int hs = 0; hs < C::NSW; ++hs) {
      const int hd = hs * 32 + l32;
      if (hd >= C::H) continue;
      const float inv = alpha_s[hd];
      uint16_t* dst = a.part_o + (part * C::H + hd) * C::L;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const int f = ft * 32 + rb * 8 + g2 * 4;
        if (f < C::L)
          *(u32x2*)(dst + f) = u32x2{pack_f16x2(o[dt][hs][rb * 4 + 0] * inv, o[dt][hs][rb * 4 + 1] * inv),
                                     pack_f16x2(o[dt][hs][rb * 4 + 2] * inv, o[dt][hs][rb * 4 + 3] * inv)};
      }
    }
  }
}

// Combine the splits of one (sequence, head): with w_s = 2^(m_s - M) l_s over the splits s,
// o = sum_s w_s O~_s / sum_s w_s, where O~_s is split s's output divided by its own sum l_s.
// One workgroup of 256 threads per (b, h), b fastest (the XCD of the decode splits of b); wave w
// takes splits w, w+4, ...; lane l owns latent features 8l .. 8l+7 (16 bytes of fp16 partial).
template <class S>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeAttnArgs a) {
  constexpr int L = S::L, H = S::H;
  static_assert(L % 8 == 0 && L <= 512, "eight features per lane, one wave per split");
  __shared__ float red_m[4], red_d[4];
  __shared__ f32x4 red_o[4][L / 4];
  const int b = blockIdx.x % a.B, h = blockIdx.x / a.B;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ns = a.n_splits;
  const float* ml = a.part_ml + ((size_t)b * ns * H + h) * 2;  // split s at ml[s * H * 2]
  float mx = -INFINITY;
  for (int s = tid; s < ns; s += 256) mx = fmaxf(mx, ml[(size_t)s * H * 2]);
  mx = wave_max(mx);
  if (lane == 0) red_m[wave] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
  const int f = lane * 8;
  const bool own = f < L;
  const uint16_t* po = a.part_o + ((size_t)b * ns * H + h) * L + f;  // split s at po[s * H * L]
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  constexpr int U = 4;  // splits in flight per wave
  for (int s0 = wave; s0 < ns; s0 += 4 * U) {
    u32x4 v[U];
    float wgt[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + 4 * u;
      const bool ok = s < ns;
      const float m = ok ? ml[(size_t)s * H * 2] : -INFINITY;
      const float l = ok ? ml[(size_t)s * H * 2 + 1] : 0.f;
      wgt[u] = m == -INFINITY ? 0.f : fast_exp2(m - M) * l;
      v[u] = (ok && own) ? ld16(po + (size_t)s * H * L) : zero16();
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      den += wgt[u];
      const uint32_t w4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += wgt[u] * lo_f16(w4[e]);
        acc[2 * e + 1] += wgt[u] * hi_f16(w4[e]);
      }
    }
  }
  if (own) {
    red_o[wave][lane * 2] = f32x4{acc[0], acc[1], acc[2], acc[3]};
    red_o[wave][lane * 2 + 1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
  }
  if (lane == 0) red_d[wave] = den;
  __syncthreads();
  const float dtot = red_d[0] + red_d[1] + red_d[2] + red_d[3];
  const float inv = dtot > 0.f ? 1.0f / dtot : 0.f;  // no visible position: zeros
  if (tid < L / 4) {
    const f32x4 o = (red_o[0][tid] + red_o[1][tid] + red_o[2][tid] + red_o[3][tid]) * inv;
    *(f32x4*)(a.o_latent + ((size_t)b * H + h) * L + tid * 4) = o;
  }
  if (tid == 0 && a.lse) a.lse[(size_t)b * H + h] = (M + __log2f(dtot)) * 0.6931471805599453f;
}

// q~[b,h,:L] = W^K_h^T q_nope[b,h], q~[b,h,L:] = q_shared[b,h]  (fp32 accumulate, bf16 out).
// One workgroup per head; thread t owns latent features t, t+256, ...; tokens in chunks of 8.
template <class S>
__global__ __launch_bounds__(256) void absorb_q_kernel(const uint16_t* __restrict__ q, int ldq,
                                                       const uint16_t* __restrict__ wkvb, int B,
                                                       uint16_t* __restrict__ qt) {
  constexpr int H = S::H, DN = S::DN, DS = S::DS, DV = S::DV, L = S::L, DQK = DN + DS;
  constexpr int BC = 8;
  __shared__ float qn[BC][DN];
  const int h = blockIdx.x;
  const uint16_t* wk = wkvb + (size_t)h * (DN + DV) * L;
  for (int b0 = 0; b0 < B; b0 += BC) {
    __syncthreads();
    for (int i = threadIdx.x; i < BC * DN; i += blockDim.x) {
      const int bb = i / DN, e = i % DN;
      qn[bb][e] = (b0 + bb < B) ? bf16_bits_to_f32(q[(size_t)(b0 + bb) * ldq + h * DQK + e]) : 0.f;
    }
    __syncthreads();
    for (int c = threadIdx.x; c < L; c += blockDim.x) {
      float acc[BC];
#pragma unroll
      for (int bb = 0; bb < BC; ++bb) acc[bb] = 0.f;
      for (int i = 0; i < DN; ++i) {
        const float w = bf16_bits_to_f32(wk[(size_t)i * L + c]);
#pragma unroll
        for (int bb = 0; bb < BC; ++bb) acc[bb] += qn[bb][i] * w;
      }
#pragma unroll
      for (int bb = 0; bb < BC; ++bb)
        if (b0 + bb < B) qt[((size_t)(b0 + bb) * H + h) * (L + DS) + c] = f32_to_bf16_bits(acc[bb]);
    }
    for (int i = threadIdx.x; i < BC * DS; i += blockDim.x) {
      const int bb = i / DS, e = i % DS;
      if (b0 + bb < B)
        qt[((size_t)(b0 + bb) * H + h) * (L + DS) + L + e] = q[(size_t)(b0 + bb) * ldq + h * DQK + DN + e];
    }
  }
}

// u[b, h*DV + d] = (W^V_h o[b,h])[d] * sigmoid(g_pre[b, h*DV + d])  (fp32 throughout).
// One workgroup per head; thread t takes value row d = t % DV and the latent slice t / DV.
template <class S>
__global__ __launch_bounds__(256) void vup_gate_kernel(const float* __restrict__ o,
                                                       const uint16_t* __restrict__ wkvb,
                                                       const float* __restrict__ g_pre, int B,
                                                       void* __restrict__ u, int u_f32) {
  constexpr int H = S::H, DN = S::DN, DV = S::DV, L = S::L;
  constexpr int PARTS = (256 / DV) < (L / 8) ? (256 / DV) : (L / 8);  // latent slices of >= 8
  constexpr int SL = L / PARTS;
  constexpr int BC = 8;
  static_assert(L % PARTS == 0, "slice");
  __shared__ float os[BC][L];
  __shared__ float red[PARTS][BC][DV];
  const int h = blockIdx.x;
  const int d = threadIdx.x % DV, part = threadIdx.x / DV;
  const uint16_t* wrow = wkvb + ((size_t)h * (DN + DV) + DN + d) * L + part * SL;
  for (int b0 = 0; b0 < B; b0 += BC) {
    __syncthreads();
    for (int i = threadIdx.x; i < BC * L; i += blockDim.x) {
      const int bb = i / L, c = i % L;
      os[bb][c] = (b0 + bb < B) ? o[((size_t)(b0 + bb) * H + h) * L + c] : 0.f;
    }
    __syncthreads();
    float acc[BC];
#pragma unroll
    for (int bb = 0; bb < BC; ++bb) acc[bb] = 0.f;
    for (int c = 0; c < (part < PARTS ? SL : 0); c += 8) {
      const u32x4 w = ld16(wrow + c);
      const float wf[8] = {lo_bf16(w.x), hi_bf16(w.x), lo_bf16(w.y), hi_bf16(w.y),
                           lo_bf16(w.z), hi_bf16(w.z), lo_bf16(w.w), hi_bf16(w.w)};
#pragma unroll
      for (int bb = 0; bb < BC; ++bb)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[bb] += wf[e] * os[bb][part * SL + c + e];
    }
    if (part < PARTS) {
#pragma unroll
      for (int bb = 0; bb < BC; ++bb) red[part][bb][d] = acc[bb];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < BC * DV; i += blockDim.x) {
      const int bb = i / DV, dd = i % DV;
      if (b0 + bb >= B) continue;
      float z = 0.f;
      for (int p = 0; p < PARTS; ++p) z += red[p][bb][dd];
      const size_t ui = (size_t)(b0 + bb) * H * DV + h * DV + dd;
      if (g_pre) z *= sigmoidf_(g_pre[ui]);
      if (u_f32)
        ((float*)u)[ui] = z;
      else
        ((uint16_t*)u)[ui] = f32_to_bf16_bits(z);
    }
  }
}

hipError_t launch_decode_attention_k3(const DecodeAttnArgs& a, bool gather, hipStream_t st);

template <class S>
static hipError_t launch_decode_t(const DecodeAttnArgs& a, bool gather, hipStream_t st) {
  const int grid = a.B * a.n_splits;
  if constexpr (S::H == ShapeK3::H) {
    const hipError_t e = launch_decode_attention_k3(a, gather, st);
    if (e != hipSuccess || (a.n_splits == 1 && !a.lse)) return e;  // wrote o_latent itself
  } else if (gather) {
    decode_attn_kernel<S, true><<<grid, 256, 0, st>>>(a);
  } else {
    decode_attn_kernel<S, false><<<grid, 256, 0, st>>>(a);
  }
  decode_merge_kernel<S><<<a.B * S::H, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_decode_attention(Shape s, const DecodeAttnArgs& a, bool gather, hipStream_t st) {
  if (a.B <= 0) return hipSuccess;
  if (s == Shape::K3) return launch_decode_t<ShapeK3>(a, gather, st);
  return launch_decode_t<ShapeTiny>(a, gather, st);
}

// ---- K3 shape: the same two products on the matrix cores ----
// Rows of 512 bf16 (1,024 bytes: one wave-wide LDS DMA each) from `src` (row stride 512) into LDS
// at row pitch `pitch` elements; wave w of four takes rows w, w + 4, ...; returns after the
// workgroup's barrier, with every row in LDS.
__device__ __forceinline__ void stage_rows_512(uint16_t* dst, int pitch, const uint16_t* __restrict__ src,
                                               int rows, int wave, int lane) {
  const uint32_t base = lds_addr(dst);
  for (int r = wave; r < rows; r += 4) lds_dma16(src + (size_t)r * 512 + lane * 8, base + r * pitch * 2);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// absorb: Q~^T[n, tok] = (W^K_h)^T[n, k] Q_nope^T[k, tok] per head. W^K_h ([128 k][512 n], n
// contiguous) is staged in LDS once per head (rows padded to 1,056 bytes) and read transposed
// with ds_read_b64_tr_b16 as the A operand; q_nope rows are the B operand (k contiguous).
// Workgroup (h, y) takes head h and the token blocks y, y + gridDim.y, ... of 32 tokens; wave w
// computes latent features [128 w, 128 w + 128) of a block (4 x 8 v_mfma_f32_32x32x16_bf16).
constexpr int kAbsPitch = 528;  // LDS row pitch of W^K_h in bf16 (conflict-free transposed reads)

__global__ __launch_bounds__(256) void absorb_q_k3_kernel(const uint16_t* __restrict__ q, int ldq,
                                                          const uint16_t* __restrict__ wkvb, int B,
                                                          uint16_t* __restrict__ qt) {
  using S = ShapeK3;
  constexpr int H = S::H, DN = S::DN, DS = S::DS, DV = S::DV, L = S::L, DQK = DN + DS;
  __shared__ __attribute__((aligned(16))) uint16_t wk_s[DN * kAbsPitch];
  // per wave, 32 tokens x 64 latent features of output (half the wave's 128), 16-byte chunk c of
  // token t at chunk position c ^ (t & 7), so that the stores are whole 128-byte runs per token
  __shared__ __attribute__((aligned(16))) uint16_t st_s[4][32 * 64];
  const int h = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // token blocks of 32: this workgroup takes blocks blockIdx.y, + gridDim.y, ...
  if ((int)blockIdx.y * 32 >= B) return;
  stage_rows_512(wk_s, kAbsPitch, wkvb + (size_t)h * (DN + DV) * L, DN, wave, lane);  // W^K_h
  const int G = lane >> 4, jj = lane & 15, g2 = lane >> 5, l32 = lane & 31;
  // q_nope of this lane's token in block t0 (tokens past B: the last one, computed, not stored),
  // and the 16-byte chunk tid % 8 of token t0 + tid / 8's q_shared, copied to q~[.., L:]
  const int ctok = tid / (DS / 8), cch = tid % (DS / 8);  // 32 tokens x 8 chunks = 256 threads
  auto load_q = [&](int t0, u32x4* qb, u32x4& sh) __attribute__((always_inline)) {
    const int tok = min(t0 + l32, B - 1);
    const uint16_t* qrow = q + (size_t)tok * ldq + h * DQK + g2 * 8;
#pragma unroll
    for (int ks = 0; ks < DN / 16; ++ks) qb[ks] = ld16(qrow + ks * 16);
    sh = ld16(q + (size_t)min(t0 + ctok, B - 1) * ldq + h * DQK + DN + cch * 8);
  };
  const int tstep = gridDim.y * 32, tlast = (B - 1) / 32 * 32;
  u32x4 qb[DN / 16], qn[DN / 16], sh, shn;
  load_q(blockIdx.y * 32, qb, sh);
  for (int t0 = blockIdx.y * 32; t0 < B; t0 += tstep) {
    // the next block's loads (no branch: they stay in flight under this block's MFMAs)
    load_q(min(t0 + tstep, tlast), qn, shn);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 acc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < DN / 16; ++ks) {
      const int r0 = ks * 16 + 8 * (G >> 1) + (jj >> 2);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int col = wave * 128 + dt * 32 + 16 * (G & 1) + 4 * (jj & 3);
        const u32x2 lo = lds_read_tr16(&wk_s[r0 * kAbsPitch + col]);
        const u32x2 hi = lds_read_tr16(&wk_s[(r0 + 4) * kAbsPitch + col]);
        acc[dt] = mfma32(u32x4{lo.x, lo.y, hi.x, hi.y}, qb[ks], acc[dt]);
      }
    }
    // acc[dt][4 jg + e] is latent feature wave*128 + dt*32 + jg*8 + g2*4 + e of token t0 + l32;
    // each half (dt = 2 hf, 2 hf + 1) goes through the wave's LDS block, then out as 16-byte
    // chunks, eight tokens' 128-byte runs per store
    uint16_t* stg = st_s[wave];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
      for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          const int dt = 2 * hf + d2, c = d2 * 4 + jg;
          *(u32x2*)(stg + l32 * 64 + ((c ^ (l32 & 7)) << 3) + g2 * 4) =
              u32x2{pack_bf16x2(acc[dt][jg * 4], acc[dt][jg * 4 + 1]),
                    pack_bf16x2(acc[dt][jg * 4 + 2], acc[dt][jg * 4 + 3])};
        }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // LDS ops of a wave complete in order
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tk = i * 8 + (lane >> 3), c = lane & 7;
        const u32x4 v = *(const u32x4*)(stg + tk * 64 + ((c ^ (tk & 7)) << 3));
        if (t0 + tk < B) st16(qt + ((size_t)(t0 + tk) * H + h) * (L + DS) + wave * 128 + hf * 64 + c * 8, v);
      }
    }
    if (t0 + ctok < B) st16(qt + ((size_t)(t0 + ctok) * H + h) * (L + DS) + L + cch * 8, sh);
#pragma unroll
    for (int ks = 0; ks < DN / 16; ++ks) qb[ks] = qn[ks];
    sh = shn;
  }
}

// absorb for at most 32 tokens (decode): one wave per (head h, block c of 128 latent features),
// four times the workgroups of absorb_q_k3_kernel, so that the 12.6 MB of W^K reach all CUs (with
// one workgroup per head, 96 CUs staged 128 KB each). The wave copies W^K_h[:, 128 c, +128)
// (128 rows x 256 bytes) into LDS by 32 wave-wide DMA loads (four rows each), 16-byte piece p of
// row r at r*256 + ((p ^ 2 (r & 7)) << 4): the transposed reads of four rows x 32 bytes per 16
// lanes then fall on distinct banks, as with the padded rows of the wide kernel.
__global__ __launch_bounds__(64) void absorb_q_k3_small_kernel(const uint16_t* __restrict__ q, int ldq,
                                                               const uint16_t* __restrict__ wkvb, int B,
                                                               uint16_t* __restrict__ qt) {
  using S = ShapeK3;
  constexpr int H = S::H, DN = S::DN, DS = S::DS, DV = S::DV, L = S::L, DQK = DN + DS;
  __shared__ __attribute__((aligned(1024))) uint8_t wk_s[DN * 256];
  const int h = blockIdx.x, c = blockIdx.y;
  const int lane = threadIdx.x;
  const uint16_t* wsrc = wkvb + (size_t)h * (DN + DV) * L + c * 128;
  {
    const uint32_t base = lds_addr(wk_s);
    const int lr = lane >> 4, pos = lane & 15;
#pragma unroll 8
    for (int i = 0; i < DN / 4; ++i) {
      const int row = 4 * i + lr;
      lds_dma16(wsrc + (size_t)row * L + ((pos ^ (2 * (row & 7))) << 3), base + i * 1024);
    }
  }
  const int G = lane >> 4, jj = lane & 15, g2 = lane >> 5, l32 = lane & 31;
  const int tok = min(l32, B - 1);  // tokens past B repeat the last (computed, not stored)
  u32x4 qb[DN / 16];
  const uint16_t* qrow = q + (size_t)tok * ldq + h * DQK + g2 * 8;
#pragma unroll
  for (int ks = 0; ks < DN / 16; ++ks) qb[ks] = ld16(qrow + ks * 16);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // W^K block and q (loaded after it) are in
  f32x16 acc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  auto rd = [&](int r, int col) __attribute__((always_inline)) {
    return lds_read_tr16(wk_s + r * 256 + (((col >> 3) ^ (2 * (r & 7))) << 4) + (col & 7) * 2);
  };
#pragma unroll
  for (int ks = 0; ks < DN / 16; ++ks) {
    const int r0 = ks * 16 + 8 * (G >> 1) + (jj >> 2);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int col = dt * 32 + 16 * (G & 1) + 4 * (jj & 3);
      const u32x2 lo = rd(r0, col), hi = rd(r0 + 4, col);
      acc[dt] = mfma32(u32x4{lo.x, lo.y, hi.x, hi.y}, qb[ks], acc[dt]);
    }
  }
  if (l32 < B) {
    uint16_t* dst = qt + ((size_t)l32 * H + h) * (L + DS) + c * 128;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int n = dt * 32 + jg * 8 + g2 * 4;
        *(u32x2*)(dst + n) = u32x2{pack_bf16x2(acc[dt][jg * 4], acc[dt][jg * 4 + 1]),
                                   pack_bf16x2(acc[dt][jg * 4 + 2], acc[dt][jg * 4 + 3])};
      }
  }
  if (c == 0) {  // q_shared passes through to q~[.., L:]: 32 tokens x 8 chunks of 16 bytes
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = i * 64 + lane, t = idx >> 3, ch = idx & 7;
      if (t < B) st16(qt + ((size_t)t * H + h) * (L + DS) + L + ch * 8, ld16(q + (size_t)t * ldq + h * DQK + DN + ch * 8));
    }
  }
}

// value up-projection and gate: Z^T[d, tok] = W^V_h[d, c] O~^T[c, tok]. W^V_h rows (c contiguous)
// are the A operand straight from memory; o~ is fp32, split into bf16 hi + lo parts (two MFMAs,
// products exact to ~2^-17 relative) as the B operand. Workgroup (h, y) takes head h and the
// token blocks y, y + gridDim.y, ... of 32 tokens; wave w computes value rows [32 w, 32 w + 32)
// of a block; the epilogue multiplies by sigmoid(g_pre).
__global__ __launch_bounds__(256) void vup_gate_k3_kernel(const float* __restrict__ o,
                                                          const uint16_t* __restrict__ wkvb,
                                                          const float* __restrict__ g_pre, int B,
                                                          void* __restrict__ u, int u_f32) {
  using S = ShapeK3;
  constexpr int H = S::H, DN = S::DN, DV = S::DV, L = S::L;
  // 256 threads: the four row groups of head blockIdx.x; 64 threads: row group blockIdx.x % 4 of
  // head blockIdx.x / 4 (four times the workgroups, for few tokens)
  const bool one_wave = blockDim.x == 64;
  const int h = one_wave ? blockIdx.x >> 2 : blockIdx.x;
  const int lane = threadIdx.x & 63, wave = one_wave ? (blockIdx.x & 3) : (threadIdx.x >> 6);
  const int g2 = lane >> 5, l32 = lane & 31;
  const uint16_t* wrow = wkvb + ((size_t)h * (DN + DV) + DN + wave * 32 + l32) * L + g2 * 8;
  for (int t0 = blockIdx.y * 32; t0 < B; t0 += gridDim.y * 32) {  // token blocks of this workgroup
    const int tok = min(t0 + l32, B - 1);
    const float* orow = o + ((size_t)tok * H + h) * L + g2 * 8;
    f32x16 acc = f32x16{};
    constexpr int U = 8;  // k-steps whose loads are in flight together
#pragma unroll 1
    for (int k0 = 0; k0 < L / 16; k0 += U) {
      u32x4 wa[U];
      f32x4 ov[U][2];
#pragma unroll
      for (int i = 0; i < U; ++i) {
        wa[i] = ld16(wrow + (k0 + i) * 16);
        ov[i][0] = *(const f32x4*)(orow + (k0 + i) * 16);
        ov[i][1] = *(const f32x4*)(orow + (k0 + i) * 16 + 4);
      }
#pragma unroll
      for (int i = 0; i < U; ++i) {
        float x[8] = {ov[i][0][0], ov[i][0][1], ov[i][0][2], ov[i][0][3],
                      ov[i][1][0], ov[i][1][1], ov[i][1][2], ov[i][1][3]};
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hi[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
          lo[e] = pack_bf16x2(x[2 * e] - lo_bf16(hi[e]), x[2 * e + 1] - hi_bf16(hi[e]));
        }
        acc = mfma32(wa[i], u32x4{hi[0], hi[1], hi[2], hi[3]}, acc);
        acc = mfma32(wa[i], u32x4{lo[0], lo[1], lo[2], lo[3]}, acc);
      }
    }
    if (t0 + l32 < B) {
      const size_t ub = (size_t)(t0 + l32) * H * DV + (size_t)h * DV;
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int d = wave * 32 + jg * 8 + g2 * 4;
        float z[4] = {acc[jg * 4], acc[jg * 4 + 1], acc[jg * 4 + 2], acc[jg * 4 + 3]};
        if (g_pre) {
          const f32x4 gv = *(const f32x4*)(g_pre + ub + d);
#pragma unroll
          for (int e = 0; e < 4; ++e) z[e] *= sigmoidf_(gv[e]);
        }
        if (u_f32)
          *(f32x4*)((float*)u + ub + d) = f32x4{z[0], z[1], z[2], z[3]};
        else
          *(u32x2*)((uint16_t*)u + ub + d) = u32x2{pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3])};
      }
    }
  }
}

// The same product for many tokens: W^V_h is staged in LDS (rows padded to 1,040 bytes) and read
// as the A operand; workgroup (h, y) takes head h and the four 32-token blocks 4y .. 4y + 3, one
// per wave, each wave computing all 128 value rows of its block.
constexpr int kVupPitch = 520;  // LDS row pitch of W^V_h in bf16 (16-byte reads conflict-free)

__global__ __launch_bounds__(256) void vup_gate_k3_lds_kernel(const float* __restrict__ o,
                                                              const uint16_t* __restrict__ wkvb,
                                                              const float* __restrict__ g_pre, int B,
                                                              void* __restrict__ u, int u_f32) {
  using S = ShapeK3;
  constexpr int H = S::H, DN = S::DN, DV = S::DV, L = S::L;
  __shared__ __attribute__((aligned(16))) uint16_t wv_s[DV * kVupPitch];
  // bf16 output staging, per wave 32 tokens x 64 value features (16-byte chunk c of token t at
  // chunk position c ^ (t & 7)), so that the stores are whole 128-byte runs per token
  __shared__ __attribute__((aligned(16))) uint16_t st_s[4][32 * 64];
  const int h = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g2 = lane >> 5, l32 = lane & 31;
  stage_rows_512(wv_s, kVupPitch, wkvb + ((size_t)h * (DN + DV) + DN) * L, DV, wave, lane);
  // wave w takes the 32-token blocks 4 blockIdx.y + w, + 4 gridDim.y, ... (W^V_h staged once). The
  // loads run one k-slice ahead, across blocks too: the last slice of a block issues the block's
  // gate pre-activations and the next block's first slice of o~, so neither waits a full memory
  // latency at a block boundary.
  const int tstep = gridDim.y * 128;
  const uint16_t* arow = wv_s + l32 * kVupPitch + g2 * 8;
  auto orow_of = [&](int t0) __attribute__((always_inline)) {  // this lane's o~ row (tokens past B: the last)
    return o + ((size_t)min(t0 + l32, B - 1) * H + h) * L + g2 * 8;
  };
  constexpr int U = 8;  // k-steps of o~ loaded together
  f32x4 ov[U][2];
  int t0 = (blockIdx.y * 4 + wave) * 32;
  if (t0 < B) {
    const float* orow = orow_of(t0);
#pragma unroll
    for (int i = 0; i < U; ++i) {
      ov[i][0] = *(const f32x4*)(orow + i * 16);
      ov[i][1] = *(const f32x4*)(orow + i * 16 + 4);
    }
  }
  for (; t0 < B; t0 += tstep) {
    const float* orow = orow_of(t0);
    const int tn = t0 + tstep;
    const float* nrow = orow_of(min(tn, B - 1));
    const size_t ubl = (size_t)min(t0 + l32, B - 1) * H * DV + (size_t)h * DV;
    f32x16 acc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
    f32x4 gv[4][4];
#pragma unroll 1
    for (int k0 = 0; k0 < L / 16; k0 += U) {
      u32x4 bh[U], bl[U];
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const float x[8] = {ov[i][0][0], ov[i][0][1], ov[i][0][2], ov[i][0][3],
                            ov[i][1][0], ov[i][1][1], ov[i][1][2], ov[i][1][3]};
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hi[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
          lo[e] = pack_bf16x2(x[2 * e] - lo_bf16(hi[e]), x[2 * e + 1] - hi_bf16(hi[e]));
        }
        bh[i] = u32x4{hi[0], hi[1], hi[2], hi[3]};
        bl[i] = u32x4{lo[0], lo[1], lo[2], lo[3]};
      }
      if (k0 + U < L / 16) {  // the next U k-steps of o~ while these run
#pragma unroll
        for (int i = 0; i < U; ++i) {
          ov[i][0] = *(const f32x4*)(orow + (k0 + U + i) * 16);
          ov[i][1] = *(const f32x4*)(orow + (k0 + U + i) * 16 + 4);
        }
      } else {  // last slice: this block's gates, then the next block's first slice
        if (g_pre) {
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int jg = 0; jg < 4; ++jg) gv[dt][jg] = *(const f32x4*)(g_pre + ubl + dt * 32 + jg * 8 + g2 * 4);
        }
        if (tn < B) {
#pragma unroll
          for (int i = 0; i < U; ++i) {
            ov[i][0] = *(const f32x4*)(nrow + i * 16);
            ov[i][1] = *(const f32x4*)(nrow + i * 16 + 4);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < U; ++i)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const u32x4 wa = *(const u32x4*)(arow + dt * 32 * kVupPitch + (k0 + i) * 16);
          acc[dt] = mfma32(wa, bh[i], acc[dt]);
          acc[dt] = mfma32(wa, bl[i], acc[dt]);
        }
    }
    // acc[dt][4 jg + e] is value feature dt*32 + jg*8 + g2*4 + e of token t0 + l32
    auto gated = [&](int dt, int jg, float* z) __attribute__((always_inline)) {
#pragma unroll
      for (int e = 0; e < 4; ++e) z[e] = acc[dt][jg * 4 + e];
      if (g_pre) {
#pragma unroll
        for (int e = 0; e < 4; ++e) z[e] *= sigmoidf_(gv[dt][jg][e]);
      }
    };
    if (u_f32) {
      if (t0 + l32 < B) {
        const size_t ub = (size_t)(t0 + l32) * H * DV + (size_t)h * DV;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int jg = 0; jg < 4; ++jg) {
            float z[4];
            gated(dt, jg, z);
            *(f32x4*)((float*)u + ub + dt * 32 + jg * 8 + g2 * 4) = f32x4{z[0], z[1], z[2], z[3]};
          }
      }
    } else {  // bf16: each half (dt = 2 hf, 2 hf + 1) through the wave's LDS block, then 16-byte chunks
      uint16_t* stg = st_s[wave];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
          for (int jg = 0; jg < 4; ++jg) {
            const int c = d2 * 4 + jg;
            float z[4];
            gated(2 * hf + d2, jg, z);
            *(u32x2*)(stg + l32 * 64 + ((c ^ (l32 & 7)) << 3) + g2 * 4) =
                u32x2{pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3])};
          }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // LDS ops of a wave complete in order
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tk = i * 8 + (lane >> 3), c = lane & 7;
          const u32x4 v = *(const u32x4*)(stg + tk * 64 + ((c ^ (tk & 7)) << 3));
          if (t0 + tk < B) st16((uint16_t*)u + (size_t)(t0 + tk) * H * DV + (size_t)h * DV + hf * 64 + c * 8, v);
        }
      }
    }
  }
}

hipError_t launch_absorb_q(Shape s, const uint16_t* q, int ldq, const uint16_t* wkvb, int B,
                           uint16_t* qt, hipStream_t st) {
  if (B <= 0) return hipSuccess;
  if (s == Shape::K3 && B <= 32)  // one wave per (head, 128-feature block)
    absorb_q_k3_small_kernel<<<dim3(ShapeK3::H, 4), 64, 0, st>>>(q, ldq, wkvb, B, qt);
  else if (s == Shape::K3)  // up to eight token blocks per workgroup (W^K_h is staged once per workgroup)
    absorb_q_k3_kernel<<<dim3(ShapeK3::H, cdiv(B, 256)), 256, 0, st>>>(q, ldq, wkvb, B, qt);
  else
    absorb_q_kernel<ShapeTiny><<<ShapeTiny::H, 256, 0, st>>>(q, ldq, wkvb, B, qt);
  return hipGetLastError();
}

hipError_t launch_vup_gate(Shape s, const float* o, const uint16_t* wkvb, const float* g_pre,
                           int B, void* u, int u_f32, hipStream_t st) {
  if (B <= 0) return hipSuccess;
  if (s == Shape::K3 && B > 32)  // many tokens: W^V_h staged once per up to 256 tokens
    vup_gate_k3_lds_kernel<<<dim3(ShapeK3::H, cdiv(B, 256)), 256, 0, st>>>(o, wkvb, g_pre, B, u, u_f32);
  else if (s == Shape::K3)  // one wave per (head, row group): 384 workgroups stream W^V
    vup_gate_k3_kernel<<<dim3(ShapeK3::H * 4, cdiv(B, 32)), 64, 0, st>>>(o, wkvb, g_pre, B, u, u_f32);
  else
    vup_gate_kernel<ShapeTiny><<<ShapeTiny::H, 256, 0, st>>>(o, wkvb, g_pre, B, u, u_f32);
  return hipGetLastError();
}

}  // namespace gmla
