// Causal prefill flash attention with the output-gate epilogue, for the K3 layer shape
// (96 heads, 192-wide query/key rows, 128-wide value rows).
//
// Same computation as prefill_attn_kernel (prefill_attn.hip): for sequence b, head h and new
// token i at absolute position p = start[b] + i,
//   z = softmax_j( q . k_j * scale ) v_j over j <= p,   u = z * sigmoid(g_pre)
// (K3.1 Gated DSA blog, eq. (9) over every visible position, and eq. (10) before W_o).
//
// One workgroup = 256 query rows of one (b, h); each wave owns QB consecutive 32-row MFMA blocks
// (QB = 1: 8 waves, two per SIMD, so one wave's softmax runs under the other's MFMAs).
// * Scores are formed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16 over the 192 features):
//   q is the register-resident B operand (every K fragment read from LDS feeds QB MFMAs) and lane
//   l owns query column l%32 (row max: one permlane32 swap; row sum: per lane until the end).
// * K rows enter the A operand under a row permutation that makes the score accumulators the
//   B operand P^T of O^T = V^T P^T directly; V^T comes from row-major V through
//   ds_read_b64_tr_b16.
// * 64-key K/V tiles (24 KB + 16 KB) are copied HBM/L2 -> LDS by global_load_lds_dwordx4 into a
//   4-slot ring filling the CU's 160 KB (16-byte chunks XOR-swizzled per row), issued four tiles
//   ahead of their P.V (the scores run two sub-tiles ahead of it); one barrier per tile.
// * Software pipeline over 32-key sub-tiles u inside each wave: step u issues the score MFMAs of
//   u+2 and the P.V MFMAs of u, and runs the softmax of u+1 on the VALU between them.
// * The running max moves only when it grows by more than 8 (base 2); otherwise the rescale
//   factor is exactly 1 and the accumulators are not touched.
// * Workgroups are ordered so each XCD walks one head at a time (its K/V stay in that XCD's L2),
//   longest query tiles first.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace gmla {

namespace k3pre {
constexpr int H = 96, DQK = 192, DV = 128;
constexpr int BQ = 256;                       // query rows per workgroup
constexpr int BKV = 64, SUB = 32;             // keys per tile / per pipeline step
constexpr int KCH = DQK / 8, VCH = DV / 8;    // 16-byte chunks per K / V row
constexpr int KROWB = DQK * 2, VROWB = DV * 2;
constexpr int KBYTES = BKV * KROWB, VBYTES = BKV * VROWB;
constexpr int SLOT = KBYTES + VBYTES;         // 40 KB
constexpr int NSLOT = 4;                      // the ring fills the CU's 160 KB of LDS
constexpr int NLOAD_K = KBYTES / 1024;
constexpr int KS = DQK / 16;                  // score k-steps
constexpr float RESCALE_SLACK = 8.0f;
// QB 32-row query blocks per wave: 1 -> 8 waves (two per SIMD), 2 -> 4 waves (one per SIMD)
template <int QB> struct Cfg {
  static constexpr int NW = 8 / QB, NT = NW * 64, WROWS = QB * 32;
  static constexpr int NLOAD_W = SLOT / 1024 / NW;  // wave-wide 1 KB DMA loads per wave per tile
  static constexpr int NKOFS = NLOAD_W < 6 ? NLOAD_W : 6;
  static_assert(NLOAD_W * NW * 1024 == SLOT, "tile must split evenly over the waves");
  static_assert(NW * WROWS == BQ, "rows per workgroup");
};
}  // namespace k3pre

// chunk swizzles: K rows (24 chunks) XOR the low 3 bits, V rows (16 chunks) XOR bits 2..3
__device__ __forceinline__ int k3_kswz(int r) { return ((r ^ (r >> 2)) & 1) | (r & 2) | ((r >> 1) & 4); }
__device__ __forceinline__ int k3_vswz(int r) { return 4 * (r & 3); }
// key row (within 32) placed at A-operand row m, so that C element j of lane l is key
// 16*(j/8) + 8*(l/32) + j%8
__device__ __forceinline__ int k3_perm_row(int m) {
  const int a = m >> 3, g = (m >> 2) & 1, b = m & 3;
  return 16 * (a >> 1) + 8 * g + 4 * (a & 1) + b;
}
// max over lanes l and l^32
__device__ __forceinline__ float k3_max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int V> using ic = std::integral_constant<int, V>;

// Key tiles of the job (bh, qt): tiles [0, n) of keys [0, kv_end), kv_end = min(n_keys, last row's
// position + 1).
__device__ __forceinline__ int k3_job_tiles(const PrefillAttnArgs& a, int bh, int qt, int* n_keys_out) {
  using namespace k3pre;
  const int start = a.start[bh / H];
  const int n_keys = min(start + a.T, a.T_cap);
  *n_keys_out = n_keys;
  return cdiv(min(n_keys, start + min(a.T, qt * BQ + BQ)), BKV);
}

// One (b*H + h, query tile) job of a workgroup; `ring` is the workgroup's K/V ring. Every LDS
// read of a job happens before its last barrier, so jobs can follow each other without one.
// With `ahead` the job's first NSLOT K/V tiles are already in flight (issued by the previous job
// of this workgroup); with next_bh >= 0 this job issues the first tiles of job (next_bh, next_qt)
// into the free ring right after its last barrier, ahead of its own epilogue.
template <int QB>
__device__ __forceinline__ void prefill_k3_job(const PrefillAttnArgs& a, uint8_t* ring, const int bh,
                                               const int qt, const bool ahead, const int next_bh,
                                               const int next_qt) {
  using namespace k3pre;
  using C = Cfg<QB>;
  constexpr int NW = C::NW, WROWS = C::WROWS, NLOAD_W = C::NLOAD_W, NKOFS = C::NKOFS;
  (void)NW;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g2 = lane >> 5, l32 = lane & 31;
  const int b = bh / H, h = bh % H;
  const int start = a.start[b];
  const int n_keys = min(start + a.T, a.T_cap);
  const int row0 = qt * BQ;
  const int kv_end = min(n_keys, start + min(a.T, row0 + BQ));
  const int n_tiles = cdiv(kv_end, BKV);

  // this wave: rows [wrow0, wrow0 + WROWS) of the call, sub-tiles [0, nw) visible to them
  const int wrow0 = row0 + wave * WROWS;
  const int wlast = min(wrow0 + WROWS - 1, a.T - 1);
  const int wpos_first = start + wrow0;
  const int nw = wlast < wrow0 ? 0 : cdiv(min(start + wlast, n_keys - 1) + 1, SUB);
  int lim[QB];  // last visible key of this lane's query in each block
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) lim[qb] = min(start + wrow0 + qb * 32 + l32, n_keys - 1);

  const uint16_t* kbase = a.k + (size_t)bh * a.T_cap * DQK;
  const uint16_t* vbase = a.v + (size_t)bh * a.T_cap * DV;

  // ---- DMA: load i of a tile fills slot bytes [1024 i, 1024 i + 1024); lane L of it writes linear
  // chunk P = 64 i + L. K rows are 24 chunks, so the per-lane source offset repeats every 3 loads
  // (the K swizzle repeats every 16 rows = 384 chunks = 6 loads) up to a wave-uniform 6 KB step;
  // V rows are 16 chunks (4 rows per load).
  auto k_src = [](int P) {
    const int r = P / KCH;
    return r * KROWB + (((P - r * KCH) ^ k3_kswz(r)) << 4);
  };
  auto v_src = [](int P) {
    const int r = P / VCH;
    return r * VROWB + (((P - r * VCH) ^ k3_vswz(r)) << 4);
  };
  uint32_t kofs[NKOFS];  // kofs[m]: per-lane source offset of this wave's loads k with k % 6 == m
#pragma unroll
  for (int m = 0; m < NKOFS; ++m) {
    const int i = wave * NLOAD_W + m;
    kofs[m] = (uint32_t)(k_src((i % 6) * 64 + lane));
  }
  const uint32_t vofs = (uint32_t)v_src(lane);
  const uint32_t ring_lds = lds_addr(ring) + wave * NLOAD_W * 1024;
  // tile t of the job whose K/V rows start at kbase_/vbase_ (n_keys_ keys, n_tiles_ tiles)
  auto issue_for = [&](const uint16_t* kbase_, const uint16_t* vbase_, int n_keys_, int n_tiles_,
                       int t) __attribute__((always_inline)) {
    if (t >= n_tiles_) return;
    const uint32_t sa = ring_lds + (t % NSLOT) * SLOT;
    const int j0 = t * BKV;
    const uint8_t* kb = (const uint8_t*)(kbase_ + (size_t)j0 * DQK);
    const uint8_t* vb = (const uint8_t*)(vbase_ + (size_t)j0 * DV);
    if (j0 + BKV <= n_keys_) {
#pragma unroll
      for (int k = 0; k < NLOAD_W; ++k) {
        const int i = wave * NLOAD_W + k;
        if (i < NLOAD_K)
          lds_dma16_sbase(kofs[k % NKOFS], kb + (i / 6) * 6144, sa + k * 1024);
        else
          lds_dma16_sbase(vofs, vb + (i - NLOAD_K) * 1024, sa + k * 1024);
      }
    } else {  // last tile: rows past the end re-read the last key (masked later)
      const int rmax = n_keys_ - 1 - j0;
#pragma unroll 1
      for (int k = 0; k < NLOAD_W; ++k) {
        const int i = wave * NLOAD_W + k;
        const bool isk = i < NLOAD_K;
        const int P = (isk ? i : i - NLOAD_K) * 64 + lane;
        const int r = P / (isk ? KCH : VCH);
        int off = isk ? k_src(P) : v_src(P);
        if (r > rmax) off -= (r - rmax) * (isk ? KROWB : VROWB);
        lds_dma16_sbase((uint32_t)off, isk ? kb : vb, sa + k * 1024);
      }
    }
  };
  auto issue = [&](int t) __attribute__((always_inline)) { issue_for(kbase, vbase, n_keys, n_tiles, t); };

  // ---- q fragments (B operand): query rows wrow0 + 32 qb + l32, features 16 s + 8 g2 .. +8 ----
  u32x4 qf[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = min(wrow0 + qb * 32 + l32, a.T - 1);  // rows past the end: computed, not stored
    const uint16_t* qrow = a.q + (((size_t)b * a.T + qi) * H + h) * DQK + g2 * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[qb][s] = ld16(qrow + s * 16);
  }
  if (!ahead) {
#pragma unroll
    for (int t = 0; t < NSLOT; ++t) issue(t);
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int s = 0; s < KS; ++s) asm volatile("" ::"v"(qf[qb][s]));

  const float sl2 = a.scale * 1.4426950408889634f;
  const int srow = k3_perm_row(l32);
  const int ksw = k3_kswz(srow);
  const int G = lane >> 4, jj = lane & 15;

  f32x16 o[4][QB];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) o[d][qb] = f32x16{};
  float m_run[QB], l_run[QB], alpha[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
    alpha[qb] = 1.f;
  }
  f32x16 sacc[2][QB];    // [sub-tile parity][query block]
  u32x4 pb[2][2][QB];    // [sub-tile parity][16-key half][query block]

  // LDS read addresses. K fragment s of sub-tile v: row (v%2)*32 + srow of slot (v/2)%3, chunk
  // (2s + g2) ^ ksw = 8*(s/4) + ((2*(s%4) + g2) ^ ksw): four per-lane bases + immediates.
  // V^T fragment (16-key step ks of sub-tile u, value block d): rows 16*(2*(u%2) + ks) + 8*(G/2)
  // + jj/4 (+4 for the upper half), chunk (4d + 2*(G%2) + (jj%4)/2) ^ 4*(jj/4): four per-lane
  // bases (one per d) + immediates.
  const uint32_t ring0 = lds_addr(ring);
  uint32_t kaddr[4], vaddr[4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
    kaddr[m] = ring0 + srow * KROWB + (((2 * m + g2) ^ ksw) << 4);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int q = jj >> 2;
    const int c = (4 * d + 2 * (G & 1) + ((jj & 3) >> 1)) ^ (4 * q);
    vaddr[d] = ring0 + KBYTES + (8 * (G >> 1) + q) * VROWB + (c << 4) + 8 * (jj & 1);
  }

  // score MFMAs of sub-tile v (parity P) into sacc[P]
  auto scores = [&](int v, auto P) __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value;
    const uint32_t so = ((v >> 1) % NSLOT) * SLOT + p * 32 * KROWB;
    uint32_t kb[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) kb[m] = kaddr[m] + so;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) sacc[p][qb] = f32x16{};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const u32x4 kf = *(GMLA_LDS const u32x4*)(kb[s & 3] + 128 * (s >> 2));
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sacc[p][qb] = mfma32(kf, qf[qb][s], sacc[p][qb]);
    }
  };
  // online softmax of sub-tile v (parity P) from sacc[P] into pb[P]; sets alpha
  auto apply_mask = [&](int v, auto P) __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int rel = lim[qb] - v * SUB - 8 * g2;  // key offset 16*(j/8) + j%8 visible iff <= rel
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (16 * (j >> 3) + (j & 7) > rel) sacc[p][qb][j] = -INFINITY;
    }
  };
  auto softmax = [&](int v, auto P) __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float x[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) x[j] = sacc[p][qb][j];
      float mt = x[0];
#pragma unroll
      for (int j = 1; j < 16; ++j) mt = fmaxf(mt, x[j]);
      mt = k3_max_xor32(mt) * sl2;
      const float m_new = (mt > m_run[qb] + RESCALE_SLACK) ? mt : m_run[qb];
      alpha[qb] = fast_exp2(m_run[qb] - m_new);
      m_run[qb] = m_new;
      float ls = 0.f;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          e[i] = fast_exp2(fmaf(x[hh * 8 + i], sl2, -m_new));
          ls += e[i];
        }
        pb[p][hh][qb] = u32x4{pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]),
                              pack_bf16x2(e[4], e[5]), pack_bf16x2(e[6], e[7])};
      }
      l_run[qb] = l_run[qb] * alpha[qb] + ls;
    }
  };
  // O^T *= alpha before the next P.V (the factor is exactly 1 unless the max moved)
  auto rescale = [&]() __attribute__((always_inline)) {
    bool any = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) any |= alpha[qb] != 1.f;
    if (__any(any)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[d][qb][r] *= alpha[qb];
    }
  };
  // sub-tiles [0, mv) lie below every query of this wave (no mask needed)
  const int mv = (min(wpos_first, n_keys - 1) + 1) / SUB;

  // One pipeline step: S(u+2) and P.V(u) on the matrix cores, softmax(u+1) on the VALU. Every
  // wave runs every sub-tile of the workgroup's key range (keys after a row's position get
  // probability 0), so the waves stay in step between barriers.
  // The LDS fragments of both products are read ahead of their MFMAs (K: KPF k-steps, V^T: two
  // fragments).
  auto step = [&](int u, auto P) __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value;
    static_assert(QB == 1, "one query block per wave");
    if (u + 1 >= mv) apply_mask(u + 1, ic<1 - p>{});
    const uint32_t so = (((u + 2) >> 1) % NSLOT) * SLOT + p * 32 * KROWB;
    uint32_t kb[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) kb[m] = kaddr[m] + so;
    auto kread = [&](int s) __attribute__((always_inline)) {
      return *(GMLA_LDS const u32x4*)(kb[s & 3] + 128 * (s >> 2));
    };
    const uint32_t sv = ((u >> 1) % NSLOT) * SLOT;
    uint32_t vb[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) vb[d] = vaddr[d] + sv;
    auto vread = [&](int i) __attribute__((always_inline)) {  // i = 4 ks + d
      const uint32_t ad = vb[i & 3] + (2 * p + (i >> 2)) * 16 * VROWB;
      const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((GMLA_LDS i16x4*)(ad)));
      const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((GMLA_LDS i16x4*)(ad + 4 * VROWB)));
      return u32x4{lo.x, lo.y, hi.x, hi.y};
    };
    constexpr int KPF = 4;
    u32x4 kf[KPF], vf[2];
#pragma unroll
    for (int s = 0; s < KPF; ++s) kf[s] = kread(s);
    sacc[p][0] = f32x16{};
    // (the scheduling barriers keep each read KPF / two MFMAs ahead of its use: left free, the
    // compiler sank the reads next to their MFMAs, and every MFMA waited out an LDS latency)
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const u32x4 cur = kf[s % KPF];
      if (s + KPF < KS) kf[s % KPF] = kread(s + KPF);
      else if (s + KPF - KS < 2) vf[s + KPF - KS] = vread(s + KPF - KS);
      sacc[p][0] = mfma32(cur, qf[0][s], sacc[p][0]);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4 cur = vf[i & 1];
      if (i + 2 < 8) vf[i & 1] = vread(i + 2);
      o[i & 3][0] = mfma32(cur, pb[p][i >> 2][0], o[i & 3][0]);
      __builtin_amdgcn_sched_barrier(0);
    }
    softmax(u + 1, ic<1 - p>{});
    rescale();
  };

  // vmcnt wait leaving at most n of this wave's most recent tiles in flight
  auto wait_tiles = [&](int n) __attribute__((always_inline)) {
    if (n >= 3)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * NLOAD_W) : "memory");
    else if (n == 2)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NLOAD_W) : "memory");
    else if (n == 1)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NLOAD_W) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };
  static_assert(NSLOT == 4, "wait_tiles covers three tiles in flight");
  // ---- prologue: tile 0 -> scores of sub-tiles 0 and 1, softmax of 0 ----
  // (tiles issued ahead precede this job's q loads in the wave's memory queue: wait for all)
  const int issued0 = min(n_tiles, NSLOT);
  if (ahead)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else
    wait_tiles(issued0 - 1);
  __syncthreads();
  scores(0, ic<0>{});
  scores(1, ic<1>{});
  if (mv == 0) apply_mask(0, ic<0>{});
  softmax(0, ic<0>{});  // alpha = 0 here, on accumulators that are still 0
  if (!ahead) wait_tiles(max(issued0 - 2, 0));
  __syncthreads();  // tile 1 is in LDS

  // ---- main loop: tile t holds sub-tiles 2t, 2t+1; tiles t+2 and t+3 are in flight ----
  for (int t = 0; t < n_tiles; ++t) {
    step(2 * t, ic<0>{});
    step(2 * t + 1, ic<1>{});
    // own share of tile t+2 has landed (tiles up to t+3 are issued; t+3 may stay in flight)
    wait_tiles(t + 3 < n_tiles ? 1 : 0);
    __syncthreads();  // ... everyone's; slot of tile t is free
    issue(t + NSLOT);
  }

  // ---- the next job's first tiles: the ring is free once every wave has passed the barrier ----
  if (next_bh >= 0) {
    int nk;
    const int nt = k3_job_tiles(a, next_bh, next_qt, &nk);
    const uint16_t* kb = a.k + (size_t)next_bh * a.T_cap * DQK;
    const uint16_t* vb = a.v + (size_t)next_bh * a.T_cap * DV;
#pragma unroll
    for (int t = 0; t < NSLOT; ++t) issue_for(kb, vb, nk, nt, t);
  }

  // ---- epilogue: normalise, gate, store ----
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32, 64);
    const float inv_l = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    const int qi = wrow0 + qb * 32 + l32;
    if (qi >= a.T) continue;
    if (a.lse && g2 == 0)
      a.lse[((size_t)b * H + h) * a.T + qi] = (m_run[qb] + __log2f(l_tot)) * 0.6931471805599453f;
    const size_t urow = ((size_t)b * a.T + qi) * (H * DV) + (size_t)h * DV;
    // all gate loads first (16 per lane), so their latencies overlap
    f32x4 gv[4][4];
    if (a.g_pre) {
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) gv[d][rb] = *(const f32x4*)(a.g_pre + urow + d * 32 + rb * 8 + g2 * 4);
    }
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const int dv = d * 32 + rb * 8 + g2 * 4;
        float z[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) z[i] = o[d][qb][rb * 4 + i] * inv_l;
        if (a.g_pre) {
#pragma unroll
          for (int i = 0; i < 4; ++i) z[i] *= sigmoidf_(gv[d][rb][i]);
        }
        if (a.u_f32)
          *(f32x4*)((float*)a.u + urow + dv) = f32x4{z[0], z[1], z[2], z[3]};
        else
          *(u32x2*)((uint16_t*)a.u + urow + dv) = u32x2{pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3])};
      }
  }
}

// Work distribution. A query tile qt costs qt + 1 key tiles, so the tiles of one (b, h) pair up
// as (nqt-1-j, j) at nqt + 1 each. With n_wg > 0 the grid is n_wg persistent workgroups (a
// multiple of 8, about one per CU) that take pairs p = blockIdx.x, blockIdx.x + n_wg, ...: every
// workgroup gets the same number of equal pairs. Pair p serves b*H + h = 8*(p/8 / (nqt/2)) + p%8,
// so a workgroup (on XCD blockIdx.x % 8) only meets the heads of its own XCD, four at a time,
// whose K/V rows stay in that XCD's L2. With n_wg == 0 (odd nqt or B*H not a multiple of 8)
// there is one workgroup per query tile, ordered so each XCD walks one head at a time, longest
// query tiles first.
template <int QB>
__global__ __launch_bounds__(k3pre::Cfg<QB>::NT) void prefill_attn_k3_kernel(PrefillAttnArgs a, int n_wg) {
  using namespace k3pre;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NSLOT * SLOT];
  const int nqt = cdiv(a.T, BQ);
  const int BH = a.B * H;
  if (n_wg > 0) {
    const int half = nqt / 2, n_pairs = BH * half;
    for (int p = blockIdx.x; p < n_pairs; p += n_wg) {
      const int xcd = p & 7, local = p >> 3;
      const int bh = (local / half) * 8 + xcd, j = local % half;
      // odd workgroups take the short query tile of each pair first, so that the epilogues (gate
      // loads, output stores) of neighbouring workgroups do not all fall at the same moment
      const bool short_first = blockIdx.x & 8;
#pragma unroll 1
      for (int k = 0; k < 2; ++k) {
        // the job after this one: the pair's second tile, else the first tile of the next pair
        int nbh = bh, nq = (k == 0) != short_first ? j : nqt - 1 - j;
        if (k == 1) {
          const int pn = p + n_wg;
          nbh = -1;
          if (pn < n_pairs) {
            const int ln = pn >> 3;
            nbh = (ln / half) * 8 + (pn & 7);
            nq = short_first ? ln % half : nqt - 1 - ln % half;
          }
        }
        prefill_k3_job<QB>(a, ring, bh, (k == 0) != short_first ? nqt - 1 - j : j, !(p == (int)blockIdx.x && k == 0), nbh, nq);
      }
    }
    return;
  }
  int bh, qt;
  if (BH % 8 == 0) {
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    bh = (local / nqt) * 8 + xcd;
    qt = nqt - 1 - (local % nqt);
  } else {
    bh = blockIdx.x % BH;
    qt = nqt - 1 - blockIdx.x / BH;
  }
  prefill_k3_job<QB>(a, ring, bh, qt, false, -1, 0);
}

hipError_t launch_prefill_attention_k3(const PrefillAttnArgs& a, hipStream_t st) {
  using namespace k3pre;
  const int nqt = cdiv(a.T, BQ);
  const int BH = a.B * H;
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu < 8)
    n_cu = 8;
  // one 32-row block per wave, two waves per SIMD: the second wave's MFMAs cover this wave's
  // softmax (the one-wave-per-SIMD form needs more than 512 registers per lane at 64 rows)
  if (nqt % 2 == 0 && BH % 8 == 0) {
    const int n_pairs = BH * (nqt / 2);
    int n_wg = n_cu / 8 * 8;
    if (n_wg > n_pairs) n_wg = n_pairs;  // n_pairs is a multiple of 8
    prefill_attn_k3_kernel<1><<<n_wg, Cfg<1>::NT, 0, st>>>(a, n_wg);
  } else {
    prefill_attn_k3_kernel<1><<<BH * nqt, Cfg<1>::NT, 0, st>>>(a, 0);
  }
  return hipGetLastError();
}

}  // namespace gmla
