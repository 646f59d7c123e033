// Causal flash attention for prefill with the sigmoid output-gate epilogue.
//
// Computes, for each sequence b, head h and new token i (absolute position p = start[b] + i),
//   z = softmax_j( q[b,i,h] . k[b,h,j] * scale ) v[b,h,j]   over j <= p
//   u[b,i,h*DV + d] = z[d] * sigmoid(g_pre[b,i,h*DV + d])
// which is eq. (9) over every visible position followed by the gate of eq. (10) (K3.1 Gated DSA
// blog; "Kimi K3" attention code page, forward, where the gate multiplies the concatenated
// head outputs before o_proj). K and V are read from the expanded cache [B, H, T_cap, *].
//
// Design (gfx950, wave64, v_mfma_f32_32x32x16_bf16):
// * A workgroup takes 32*NW query rows of one (b, h); each wave owns 32 rows. Keys stream
//   through LDS in tiles of 64, double-buffered and staged through registers.
// * Scores are formed transposed, S^T = K Q^T, so lane l holds query column l%32 and 16 of the
//   32 keys of each 32x32 block: the row max is an in-lane max plus one xor-32 shuffle, and the
//   row sum stays per lane until the end.
// * K rows enter the MFMA A operand under the permutation pi (below), which makes the score
//   accumulators of a lane exactly the B operand P^T of the next MFMA (8 consecutive keys per
//   k-step): P never leaves registers.
// * O^T = V^T P^T takes V^T straight from the row-major V tile with ds_read_b64_tr_b16.
// * The online softmax works in base 2 with scale*log2(e) folded into the logits.
// * Workgroups are ordered so each XCD walks one head at a time, its longest query tiles
//   first: the head's K/V stays in that XCD's L2 and the causal tail is balanced.
#include "common.h"
#include "kernels.h"

namespace gmla {

template <class S, int NW>
struct PrefillCfg {
  static constexpr int DQK = S::DN + S::DS, DV = S::DV, H = S::H;
  static constexpr int DQKP = round_up(DQK, 32);  // padded to whole 32-wide k blocks
  static constexpr int DVP = round_up(DV, 32);
  static constexpr int KS = DQKP / 16;             // MFMA k-steps for the scores
  static constexpr int DT = DVP / 32;              // value tiles of 32
  static constexpr int KROW = DQKP + 8;            // K tile row stride (bf16): 16 rows conflict-free
  static constexpr int VROW = DVP + 32;            // V tile row stride: 4 rows x 32 B on distinct banks
  static constexpr int BQ = 32 * NW, BKV = 64;
  static constexpr int NT = 64 * NW;
  static constexpr int KCH = DQKP / 8, VCH = DVP / 8;  // 16-byte chunks per padded row
  static constexpr int NCK = cdiv(BKV * KCH, NT), NCV = cdiv(BKV * VCH, NT);
};

// Row of the K tile that lane row m (= lane % 32) feeds into the score MFMA. With this choice
// the accumulator register r of lane group g = lane/32 holds key 16*(r/8) + 8*g + r%8 of the
// 32-key block, i.e. 8 consecutive keys per half, the B-operand order of the P^T V^T MFMA.
__device__ __forceinline__ int perm_row(int m) {
  const int a = m >> 3, g = (m >> 2) & 1, b = m & 3;
  return 16 * (a >> 1) + 8 * g + 4 * (a & 1) + b;
}

template <class S, int NW>
__global__ __launch_bounds__(64 * NW) void prefill_attn_kernel(PrefillAttnArgs a) {
  using C = PrefillCfg<S, NW>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][C::BKV * C::KROW];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][C::BKV * C::VROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g2 = lane >> 5, l32 = lane & 31;

  // ---- workgroup -> (b, h, query tile) ----
  const int nqt = cdiv(a.T, C::BQ);
  const int BH = a.B * C::H;
  int bh, qt;
  if (BH % 8 == 0) {
    // XCD x (= blockIdx % 8) runs heads bh = x (mod 8), one head at a time, longest tile first
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    bh = (local / nqt) * 8 + xcd;
    qt = nqt - 1 - (local % nqt);
  } else {
    bh = blockIdx.x % BH;
    qt = nqt - 1 - blockIdx.x / BH;
  }
  const int b = bh / C::H, h = bh % C::H;
  const int start = a.start[b];
  const int n_keys = min(start + a.T, a.T_cap);         // positions present after the append
  const int row0 = qt * C::BQ;                          // first query row of the tile
  const int kv_end = min(n_keys, start + min(a.T, row0 + C::BQ));
  const int n_tiles = cdiv(kv_end, C::BKV);

  // ---- this lane's query (the B operand of S^T = K Q^T) ----
  const int qi = row0 + wave * 32 + l32;                // query row within the call
  const int qpos = start + qi;                          // its absolute position
  const int lim = min(qpos, n_keys - 1);                // last visible key
  const int wave_first = start + row0 + wave * 32;      // first query position of this wave
  const int wave_last = min(wave_first + 31, n_keys - 1);
  u32x4 qf[C::KS];
  {
    const uint16_t* qrow = a.q + (((size_t)b * a.T + qi) * C::H + h) * C::DQK;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      const int d = s * 16 + g2 * 8;
      qf[s] = (qi < a.T && d < C::DQK) ? ld16(qrow + d) : zero16();
    }
  }

  const uint16_t* kbase = a.k + (size_t)bh * a.T_cap * C::DQK;
  const uint16_t* vbase = a.v + (size_t)bh * a.T_cap * C::DV;
  u32x4 rk[C::NCK], rv[C::NCV];
  auto load_tile = [&](int t) {
    const int j0 = t * C::BKV;
#pragma unroll
    for (int i = 0; i < C::NCK; ++i) {
      const int c = tid + C::NT * i;
      const int row = c / C::KCH, col = (c % C::KCH) * 8;
      const bool ok = c < C::BKV * C::KCH && j0 + row < n_keys && col < C::DQK;
      rk[i] = ok ? ld16(kbase + (size_t)(j0 + row) * C::DQK + col) : zero16();
    }
#pragma unroll
    for (int i = 0; i < C::NCV; ++i) {
      const int c = tid + C::NT * i;
      const int row = c / C::VCH, col = (c % C::VCH) * 8;
      const bool ok = c < C::BKV * C::VCH && j0 + row < n_keys && col < C::DV;
      rv[i] = ok ? ld16(vbase + (size_t)(j0 + row) * C::DV + col) : zero16();
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::NCK; ++i) {
      const int c = tid + C::NT * i;
      if (c < C::BKV * C::KCH) st16(&Ks[buf][(c / C::KCH) * C::KROW + (c % C::KCH) * 8], rk[i]);
    }
#pragma unroll
    for (int i = 0; i < C::NCV; ++i) {
      const int c = tid + C::NT * i;
      if (c < C::BKV * C::VCH) st16(&Vs[buf][(c / C::VCH) * C::VROW + (c % C::VCH) * 8], rv[i]);
    }
  };

  const float sl2 = a.scale * 1.4426950408889634f;  // logits in base 2
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[C::DT];
#pragma unroll
  for (int d = 0; d < C::DT; ++d) o[d] = f32x16{};

  const int krow_a = perm_row(l32);
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    const int cur = t & 1;
    const int j0 = t * C::BKV;
    if (t + 1 < n_tiles) load_tile(t + 1);
    if (j0 <= wave_last) {  // otherwise every key of the tile is in this wave's future
      // ---- S^T for 64 keys x 32 queries ----
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = f32x16{};
        const uint16_t* kr = &Ks[cur][(kb * 32 + krow_a) * C::KROW + g2 * 8];
#pragma unroll
        for (int s = 0; s < C::KS; ++s) sacc[kb] = mfma32(ld16(kr + s * 16), qf[s], sacc[kb]);
      }
      // ---- scale, causal mask, online softmax (per query = per lane pair) ----
      const bool need_mask = j0 + C::BKV - 1 > wave_first;
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = sacc[kb][r] * sl2;
          if (need_mask) {
            const int key = j0 + kb * 32 + 16 * (r >> 3) + 8 * g2 + (r & 7);
            if (key > lim) x = -INFINITY;
          }
          sacc[kb][r] = x;
          mt = fmaxf(mt, x);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float m_new = fmaxf(m_run, mt);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      float ls = 0.f;
      u32x4 pb[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          float p[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            p[i] = fast_exp2(sacc[kb][hh * 8 + i] - m_new);
            ls += p[i];
          }
          pb[kb * 2 + hh] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                  pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
        }
      l_run = l_run * alpha + ls;
      // ---- O^T = alpha O^T + V^T P^T ----
      const int G = lane >> 4, j = lane & 15;
#pragma unroll
      for (int d = 0; d < C::DT; ++d) {
#pragma unroll
        for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const uint16_t* vp =
              &Vs[cur][(ks * 16 + 8 * (G >> 1) + (j >> 2)) * C::VROW + d * 32 + 16 * (G & 1) + 4 * (j & 3)];
          const u32x2 lo = lds_read_tr16(vp);
          const u32x2 hi = lds_read_tr16(vp + 4 * C::VROW);
          o[d] = mfma32(u32x4{lo.x, lo.y, hi.x, hi.y}, pb[ks], o[d]);
        }
      }
    }
    if (t + 1 < n_tiles) store_tile(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise, gate, store ----
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv_l = 1.0f / l_tot;
  if (qi < a.T) {
    if (a.lse && g2 == 0)
      a.lse[((size_t)b * C::H + h) * a.T + qi] = (m_run + __log2f(l_tot)) * 0.6931471805599453f;
    const size_t urow = ((size_t)b * a.T + qi) * (C::H * C::DV) + (size_t)h * C::DV;
#pragma unroll
    for (int d = 0; d < C::DT; ++d)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const int dv = d * 32 + rb * 8 + g2 * 4;
        if (dv >= C::DV) continue;
        float z[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) z[i] = o[d][rb * 4 + i] * inv_l;
        if (a.g_pre) {
          const f32x4 gv = *(const f32x4*)(a.g_pre + urow + dv);
          z[0] *= sigmoidf_(gv[0]);
          z[1] *= sigmoidf_(gv[1]);
          z[2] *= sigmoidf_(gv[2]);
          z[3] *= sigmoidf_(gv[3]);
        }
        if (a.u_f32) {
          *(f32x4*)((float*)a.u + urow + dv) = f32x4{z[0], z[1], z[2], z[3]};
        } else {
          *(u32x2*)((uint16_t*)a.u + urow + dv) = u32x2{pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3])};
        }
      }
  }
}

template <class S, int NW>
static hipError_t launch_prefill_t(const PrefillAttnArgs& a, hipStream_t st) {
  using C = PrefillCfg<S, NW>;
  const int nqt = cdiv(a.T, C::BQ);
  prefill_attn_kernel<S, NW><<<a.B * S::H * nqt, C::NT, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_prefill_attention(Shape s, const PrefillAttnArgs& a, hipStream_t st) {
  if (a.B <= 0 || a.T <= 0) return hipSuccess;
  if (s == Shape::K3) return launch_prefill_attention_k3(a, st);
  return launch_prefill_t<ShapeTiny, 4>(a, st);
}

}  // namespace gmla
