// NT GEMM kernels for the layer's projections: out[m, n] = sum_k a[m, k] w[n, k].
//
// Weights are nn.Linear [out, in] matrices, so both operands are K-contiguous and feed the
// bf16 MFMA directly (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// * gemm_nt_dma: M > 128 with K % 64 == 0 (prefill). 256 x 256 tiles, operands copied straight
//   into LDS by global_load_lds, two waves per SIMD, LDS-staged row-contiguous epilogue.
// * gemm_nt_big: the other M > 32 shapes. 256 threads, a BM x BN tile per workgroup, BK = 64,
//   double-buffered LDS tiles with a 144-byte row stride (conflict-free 16-byte reads over 16
//   consecutive rows), workgroup ids remapped so that each XCD walks a contiguous, M-grouped
//   range of tiles (operands reused from that XCD's L2).
// * gemm_nt_skinny_dma: M <= 32 with K % 256 == 0 (decode at the K3 shape), see below.
// * gemm_nt_skinny: other M <= 32 (decode). Weight-bandwidth bound: each wave computes
//   W[32 rows] . X^T for all tokens, streaming weights straight from HBM into MFMA operands
//   with eight 16-byte loads in flight per lane; four waves split K inside the workgroup and
//   reduce through LDS; a grid-level split-K writes fp32 partials that gemm_reduce sums.
#include "common.h"
#include "gemm.h"

namespace gmla {

// ----------------------------------------------------------------------------------------
// Segment helpers
// ----------------------------------------------------------------------------------------
__device__ __forceinline__ int seg_of(const GemmArgs& g, int n) {
  int s = 0;
#pragma unroll
  for (int i = 1; i < kMaxSegs; ++i)
    if (i < g.nseg && n >= g.seg[i].n0) s = i;
  return s;
}

__device__ __forceinline__ const uint16_t* wrow_ptr(const GemmArgs& g, int n) {
  if (n >= g.N) return nullptr;
  const int s = seg_of(g, n);
  return g.seg[s].w + (size_t)(n - g.seg[s].n0) * g.K;
}

struct OutCol {
  char* base;   // address of element (0, n)
  int ldo_bytes;
  int f32;
};

__device__ __forceinline__ OutCol out_col(const GemmArgs& g, int n) {
  OutCol o{nullptr, 0, 0};
  if (n >= g.N) return o;
  const int s = seg_of(g, n);
  const GemmSeg& sg = g.seg[s];
  const int esz = sg.out_f32 ? 4 : 2;
  o.base = (char*)sg.out + (size_t)(n - sg.n0) * esz;
  o.ldo_bytes = sg.ldo * esz;
  o.f32 = sg.out_f32;
  return o;
}

__device__ __forceinline__ void store_out(const OutCol& o, int m, float v) {
  char* p = o.base + (size_t)m * o.ldo_bytes;
  if (o.f32)
    *(float*)p = v;
  else
    *(uint16_t*)p = f32_to_bf16_bits(v);
}

// Workgroup id -> tile id so that the tiles one XCD runs (ids congruent mod 8, since the
// dispatcher deals workgroups round-robin over the 8 XCDs) are a contiguous tile range.
__device__ __forceinline__ int xcd_contiguous(int pid, int total) {
  const int q = total / 8, r = total % 8;
  const int xcd = pid % 8, local = pid / 8;
  return (xcd < r) ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

// ----------------------------------------------------------------------------------------
// Large-M kernel
// ----------------------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(256) void gemm_nt_big(GemmArgs g) {
  constexpr int BK = 64;
  constexpr int LDR = 72;  // LDS row stride in bf16 elements (144 bytes)
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int CA = BM * 8 / 256, CB = BN * 8 / 256;  // 16-byte chunks per thread per tile
  static_assert(WM * WN == 4, "four waves");
  static_assert(CA >= 1 && CB >= 1, "tile too small");

  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDR];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDR];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tiles_m = cdiv(g.M, BM), tiles_n = cdiv(g.N, BN);
  const int pid = xcd_contiguous(blockIdx.x, tiles_m * tiles_n);
  constexpr int GROUP = 8;
  const int in_group = GROUP * tiles_n;
  const int first_m = (pid / in_group) * GROUP;
  const int gsize = min(tiles_m - first_m, GROUP);
  const int tile_m = first_m + (pid % in_group) % gsize;
  const int tile_n = (pid % in_group) / gsize;
  const int m0 = tile_m * BM, n0 = tile_n * BN;

  // Thread tid loads 16-byte chunk (tid & 7) of rows (tid >> 3) + 32 i of each tile.
  const int kc = (tid & 7) * 8;
  const int lrow = tid >> 3;
  const uint16_t* pa0 = g.a + (size_t)(m0 + lrow) * g.lda + kc;
  const size_t a_step = (size_t)32 * g.lda;
  uint32_t a_ok = 0;
#pragma unroll
  for (int i = 0; i < CA; ++i) a_ok |= (m0 + lrow + 32 * i < g.M) ? (1u << i) : 0u;
  const uint16_t* pb[CB];
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const uint16_t* w = wrow_ptr(g, n0 + lrow + 32 * i);
    pb[i] = w ? w + kc : nullptr;
  }

  u32x4 ra[CA], rb[CB];
  // split operand: A columns K..2K-1 (the lo half) meet the weight columns 0..K-1 again
  const int KA = g.a_split ? 2 * g.K : g.K;
  auto load_tile = [&](int k0) {
    const int kw = k0 >= g.K ? k0 - g.K : k0;
    const bool kin = kw + kc < g.K;
#pragma unroll
    for (int i = 0; i < CA; ++i)
      ra[i] = (kin && ((a_ok >> i) & 1u)) ? ld16(pa0 + i * a_step + k0) : zero16();
#pragma unroll
    for (int i = 0; i < CB; ++i) rb[i] = (kin && pb[i]) ? ld16(pb[i] + kw) : zero16();
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CA; ++i) st16(&As[buf][(lrow + 32 * i) * LDR + kc], ra[i]);
#pragma unroll
    for (int i = 0; i < CB; ++i) st16(&Bs[buf][(lrow + 32 * i) * LDR + kc], rb[i]);
  };

  const int wm0 = (wave / WN) * WTM, wn0 = (wave % WN) * WTN;
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  const int KT = g.a_split ? cdiv(KA, BK) : cdiv(g.K, BK);
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load_tile((kt + 1) * BK);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      u32x4 fa[TM], fb[TN];
      const int kcol = s * 16 + (lane >> 5) * 8;
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[i] = ld16(&As[cur][(wm0 + i * 32 + (lane & 31)) * LDR + kcol]);
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[j] = ld16(&Bs[cur][(wn0 + j * 32 + (lane & 31)) * LDR + kcol]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(fa[i], fb[j], acc[i][j]);
    }
    if (kt + 1 < KT) store_tile(cur ^ 1);
    __syncthreads();
  }

  // epilogue: acc[i][j][r] is (m0 + wm0 + 32i + (r/4)*8 + (lane/32)*4 + r%4, n0 + wn0 + 32j + lane%32)
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int n = n0 + wn0 + j * 32 + (lane & 31);
    const OutCol oc = out_col(g, n);
    if (!oc.base) continue;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm0 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (m < g.M) store_out(oc, m, acc[i][j][r]);
      }
  }
}

// ----------------------------------------------------------------------------------------
// Large-M kernel with LDS-DMA operand staging (M > 128, K % BK == 0)
//
// 256 x 256 output tile per workgroup, NWV waves (8: two per SIMD, 128 x 64 each). BK-wide K slabs
// of x and W are copied HBM/L2 -> LDS by global_load_lds_dwordx4 (no register staging) into an
// NST-stage ring, NST - 1 slabs ahead of the MFMAs, one barrier per slab. Only one wave per SIMD
// issues the copies, so its partner's MFMAs cover the issue time.
// LDS rows are 2*BK bytes; 16-byte chunk c of row r sits at position c ^ f(r), with f chosen so
// that the fragment reads (32 consecutive rows, one chunk each) are free of bank conflicts
// whether the LDS serves 8 or 16 lanes per cycle:
//   BK = 64 (8 chunks): f(r) = (r & 7) ^ ((r >> 3) & 1)
//   BK = 32 (4 chunks): f(r) = ((r >> 1) ^ (r >> 3)) & 3
// The MFMA A operand is the weight tile, so each lane ends with 4 consecutive output columns of
// one row: the epilogue stores 16 bytes (fp32) or 8 bytes (bf16) per lane and register group.
// ----------------------------------------------------------------------------------------
template <int BK_, int NST_, int NWV_>
struct GdCfg {
  static constexpr int BM = 256, BN = 256, BK = BK_, NST = NST_, NWV = NWV_;
  static constexpr int NIW = 4;  // waves that issue the copies (one per SIMD)
  static constexpr int WN = 128, WM = 256 * 256 / NWV / WN;  // per-wave tile (n x m)
  static constexpr int TI = WN / 32, TJ = WM / 32;
  static constexpr int ROWB = BK * 2, CPR = BK / 8, RPL = 1024 / ROWB;  // chunks per row, rows per 1 KB load
  static constexpr int ABYTES = BM * ROWB, STAGE = 2 * ABYTES;
  static constexpr int LOADS_W = ABYTES / 1024 / NIW;  // DMA loads per issuing wave per operand per slab
  static constexpr int LPW = 2 * LOADS_W;             // per issuing wave per slab
  static constexpr int PITCH = 68;                    // epilogue staging row pitch (floats)
  static constexpr int LDS_BYTES = NST * STAGE > NWV * WM * PITCH * 4 ? NST * STAGE : NWV * WM * PITCH * 4;
  static constexpr int KSUB = BK / 16;
  static_assert(NST * STAGE <= 160 * 1024, "LDS");
  static_assert((NST - 1) * LPW <= 63, "vmcnt range");
};

template <int BK>
__device__ __forceinline__ int gd_swz(int r) {
  if constexpr (BK == 64)
    return (r & 7) ^ ((r >> 3) & 1);
  else
    return ((r >> 1) ^ (r >> 3)) & 3;
}

// wait until at most n slabs of this wave's copies (LPW loads each) are still in flight
template <int LPW>
__device__ __forceinline__ void gd_wait_slabs(int n) {
  if (n >= 3) {
    if constexpr (3 * LPW <= 63) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * LPW) : "memory");
  } else if (n == 2) {
    if constexpr (2 * LPW <= 63) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * LPW) : "memory");
  } else if (n == 1) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPW) : "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

template <int BK, int NST, int NWV>
__global__ __launch_bounds__(NWV * 64) void gemm_nt_dma(GemmArgs g) {
  using C = GdCfg<BK, NST, NWV>;
  constexpr int WM = C::WM, TI = C::TI, TJ = C::TJ;
  constexpr int BM = C::BM, BN = C::BN, ROWB = C::ROWB, CPR = C::CPR, RPL = C::RPL;
  constexpr int ABYTES = C::ABYTES, STAGE = C::STAGE, LOADS_W = C::LOADS_W, LPW = C::LPW;
  constexpr int KSUB = C::KSUB, NIW = C::NIW, PITCH = C::PITCH;
  static_assert(NST - 2 <= 3, "gd_wait_slabs covers up to three slabs");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tiles_m = cdiv(g.M, BM), tiles_n = cdiv(g.N, BN);
  const int pid = xcd_contiguous(blockIdx.x, tiles_m * tiles_n);
  constexpr int GROUP = 8;
  const int in_group = GROUP * tiles_n;
  const int first_m = (pid / in_group) * GROUP;
  const int gsize = min(tiles_m - first_m, GROUP);
  const int tile_m = first_m + (pid % in_group) % gsize;
  const int tile_n = (pid % in_group) / gsize;
  const int m0 = tile_m * BM, n0 = tile_n * BN;

  // ---- DMA: load i of an operand fills rows RPL*i .. RPL*i + RPL-1 of its region; lane L writes
  // row RPL*i + L/CPR at position L%CPR, i.e. logical chunk (L%CPR) ^ f(row). f(RPL*i + x)
  // depends on i only through its parity. Waves 0..NIW-1 (one per SIMD) issue the copies, wave w
  // loads w*LOADS_W .. +LOADS_W-1; their partner waves keep the SIMD's matrix core busy meanwhile.
  const int iw = wave < NIW ? wave : 0;  // loads computed for the partner waves go unused
  const int lr = lane / CPR;
  int coff[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) coff[p] = (lane % CPR) ^ gd_swz<BK>(RPL * p + lr);
  uint32_t aoffs[LOADS_W];  // x rows clamped to M - 1 (rows past M are computed, never stored)
#pragma unroll
  for (int k = 0; k < LOADS_W; ++k) {
    const int i = iw * LOADS_W + k;
    const int row = min(RPL * i + lr, g.M - 1 - m0);
    aoffs[k] = (uint32_t)(row * g.lda * 2 + (coff[i & 1] << 4));
  }
  uint32_t woff[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) woff[p] = (uint32_t)(lr * g.K * 2 + (coff[p] << 4));
  const uint8_t* abase = (const uint8_t*)g.a + (size_t)m0 * g.lda * 2;
  const uint8_t* wbase[LOADS_W];  // weight rows n0 + RPL*i (segments start at multiples of RPL)
#pragma unroll
  for (int k = 0; k < LOADS_W; ++k) {
    int nf = n0 + RPL * (iw * LOADS_W + k);
    if (nf >= g.N) nf = g.N - RPL;  // rows past N re-read the last RPL (never stored)
    const int sg = seg_of(g, nf);
    wbase[k] = (const uint8_t*)g.seg[sg].w + (size_t)(nf - g.seg[sg].n0) * g.K * 2;
  }
  const uint32_t smem0 = lds_addr(smem);
  const uint32_t dst0 = smem0 + iw * LOADS_W * 1024;
  const int KTW = g.K / BK;                    // weight slabs
  const int KT = g.a_split ? 2 * KTW : KTW;    // operand slabs: the lo half follows the hi half

  auto issue = [&](int kt) __attribute__((always_inline)) {
    if (wave >= NIW) return;
    const uint32_t sa = dst0 + (kt % NST) * STAGE;
    const int k0b = kt * BK * 2;
    const int kw0b = (kt < KTW ? kt : kt - KTW) * BK * 2;
#pragma unroll
    for (int k = 0; k < LOADS_W; ++k) lds_dma16_sbase(aoffs[k], abase + k0b, sa + k * 1024);
#pragma unroll
    for (int k = 0; k < LOADS_W; ++k)
      lds_dma16_sbase(woff[(iw * LOADS_W + k) & 1], wbase[k] + kw0b, sa + ABYTES + k * 1024);
  };

  // ---- fragment addresses: row 32b + (lane % 32) of a region, chunk (2s + lane/32) ^ f(row)
  const int fr = lane & 31, fg = lane >> 5;
  uint32_t koff[KSUB];
#pragma unroll
  for (int s = 0; s < KSUB; ++s) koff[s] = fr * ROWB + ((((2 * s + fg) ^ gd_swz<BK>(fr))) << 4);

  const int wn0 = (wave & 1) * 128, wm0 = (wave >> 1) * WM;
  f32x16 acc[TI][TJ];  // [n block][m block]
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16{};

  u32x4 fw[2][TI], fx[2][TJ];
  auto load_frags = [&](uint32_t sb, int s, int fb) __attribute__((always_inline)) {
    const uint32_t ba = sb + koff[s];
#pragma unroll
    for (int i = 0; i < TI; ++i) fw[fb][i] = *(GMLA_LDS const u32x4*)(ba + ABYTES + (wn0 + 32 * i) * ROWB);
#pragma unroll
    for (int j = 0; j < TJ; ++j) fx[fb][j] = *(GMLA_LDS const u32x4*)(ba + (wm0 + 32 * j) * ROWB);
  };
  auto mfmas = [&](int fb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] = mfma32(fw[fb][i], fx[fb][j], acc[i][j]);
  };
  // the MFMAs of a step with the fragment reads of the next step spread between them
  auto interleave = [&]() __attribute__((always_inline)) {
    constexpr int NR = TI + TJ, NM = TI * TJ;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, NM / NR, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NM - (NM / NR) * NR, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  // Per slab kt: fragments of step s + 1 load while the MFMAs of step s run. Before the last
  // step's MFMAs (its fragments already in registers) the wave waits for slab kt+1, meets the
  // others at the barrier (slab kt is now drained everywhere), starts the copy of slab kt+NST
  // into slab kt's stage, and loads the first fragments of slab kt+1.
#pragma unroll
  for (int t = 0; t < NST; ++t)
    if (t < KT) issue(t);
  gd_wait_slabs<LPW>(min(NST, KT) - 1);
  __syncthreads();
  load_frags(smem0, 0, 0);
  for (int kt = 0; kt < KT; ++kt) {
    const uint32_t sb = smem0 + (kt % NST) * STAGE;
#pragma unroll
    for (int s = 0; s + 1 < KSUB; ++s) {
      load_frags(sb, s + 1, (s + 1) & 1);
      mfmas(s & 1);
      interleave();
    }
    gd_wait_slabs<LPW>(min(NST - 2, KT - 2 - kt));  // slab kt+1 has landed
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __syncthreads();
    if (kt + NST < KT) issue(kt + NST);
    if (kt + 1 < KT) load_frags(smem0 + ((kt + 1) % NST) * STAGE, 0, 0);
    mfmas((KSUB - 1) & 1);
    interleave();
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue, staged through LDS so that global stores are row-contiguous:
  // acc[i][j][4q + e] = out(m0 + wm0 + 32j + lane%32, n0 + wn0 + 32i + 8q + 4(lane/32) + e).
  // Per pass of 64 columns each wave writes its WM x 64 fp32 block to its own LDS area (row pitch
  // 68 floats: conflict-free), then reads it back as 16-byte row chunks and stores them with the
  // column's segment type (fp32: 16 bytes, bf16: 8 bytes per lane).
  __syncthreads();  // every wave is done with the ring
  GMLA_LDS float* stg = (GMLA_LDS float*)(smem0) + wave * (WM * PITCH);
  // cache scatter: when all of the tile's rows belong to one sequence (the usual case), its start
  // is read once and row m goes to position m + sp0
  int sb = -1, sp0 = 0;
  if (g.cs.k) {
    const int bf = m0 / g.cs.T, bl = min(m0 + BM - 1, g.M - 1) / g.cs.T;
    if (bf == bl) {
      sb = bf;
      sp0 = g.cs.start[bf] - bf * g.cs.T;
    }
  }
  const int nl = 4 * (lane & 15);
#pragma unroll
  for (int pass = 0; pass < TI / 2; ++pass) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x16& a = acc[2 * pass + ii][j];
          *(GMLA_LDS f32x4*)(stg + (32 * j + fr) * PITCH + 32 * ii + 8 * q + 4 * fg) =
              f32x4{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
        }
    const int n = n0 + wn0 + 64 * pass + nl;
    if (g.cs.k && n < g.N) {
      // expanded-cache rows: 4 columns of one head's k or v row (dn, dv multiples of 4)
      const CacheScatter& cs = g.cs;
      const int h = n / (cs.dn + cs.dv), j = n - h * (cs.dn + cs.dv);
      const bool isk = j < cs.dn;
      const int rowlen = isk ? cs.dk : cs.dv;
      uint16_t* base = (isk ? cs.k + j : cs.v + (j - cs.dn)) + (size_t)h * cs.T_cap * rowlen;
#pragma unroll
      for (int k = 0; k < WM / 4; ++k) {
        const int ml = (lane >> 4) + 4 * k;
        const int m = m0 + wm0 + ml;
        const f32x4 v = *(GMLA_LDS const f32x4*)(stg + ml * PITCH + nl);
        if (m < g.M) {
          const int b = sb >= 0 ? sb : m / cs.T;
          const int p = sb >= 0 ? sp0 + m : cs.start[b] + (m - b * cs.T);
          if (p >= 0 && p < cs.T_cap)
            *(u32x2*)(base + ((size_t)b * cs.H * cs.T_cap + p) * rowlen) =
                u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
      }
    } else if (n < g.N) {
      // this lane's segment (a 4-column chunk never straddles one: segments start at multiples of 8)
      const GemmSeg& s0 = g.seg[0];
      char* outp = (char*)s0.out;
      int ldo = s0.ldo, f32 = s0.out_f32, sn0 = s0.n0;
#pragma unroll
      for (int i = 1; i < kMaxSegs; ++i)
        if (i < g.nseg && n >= g.seg[i].n0) {
          outp = (char*)g.seg[i].out;
          ldo = g.seg[i].ldo;
          f32 = g.seg[i].out_f32;
          sn0 = g.seg[i].n0;
        }
      const int col = n - sn0;
#pragma unroll
      for (int k = 0; k < WM / 4; ++k) {
        const int ml = (lane >> 4) + 4 * k;
        const int m = m0 + wm0 + ml;
        const f32x4 v = *(GMLA_LDS const f32x4*)(stg + ml * PITCH + nl);
        if (m < g.M) {
          if (f32)
            *(f32x4*)((float*)outp + (size_t)m * ldo + col) = v;
          else
            *(u32x2*)((uint16_t*)outp + (size_t)m * ldo + col) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
      }
    }
  }
}

// the DMA kernel's layout needs K % BK == 0, 16-byte aligned rows, and weight segments (and N)
// in whole RPL-row loads
static bool dma_gemm_ok(const GemmArgs& g, int BK) {
  const int rpl = 1024 / (2 * BK);
  if (g.M <= 128 || g.K % BK != 0 || g.lda % 8 != 0 || g.N % rpl != 0 || g.N < rpl) return false;
  if (g.lda < (g.a_split ? 2 * g.K : g.K)) return false;
  for (int i = 0; i < g.nseg; ++i) {
    const GemmSeg& s = g.seg[i];
    if (s.n0 % rpl != 0 || s.ldo % 4 != 0) return false;
    if (((uintptr_t)s.out & 15) != 0 || ((uintptr_t)s.w & 15) != 0) return false;
  }
  return ((uintptr_t)g.a & 15) == 0;
}

// ----------------------------------------------------------------------------------------
// Small-M kernel (M <= 32)
// ----------------------------------------------------------------------------------------
constexpr int kSkinnyUnroll = 8;

// grid: (cdiv(N, 32), ksplit). Wave w of split s covers k steps (16 wide) of its quarter.
__global__ __launch_bounds__(256) void gemm_nt_skinny(GemmArgs g, float* partial, int steps_per_wave) {
  __shared__ float red[4][16][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 32;
  const int ks = blockIdx.y;
  const int half = lane >> 5;
  const uint16_t* wrow = wrow_ptr(g, n0 + (lane & 31));
  const int m = lane & 31;
  const uint16_t* xrow = (m < g.M) ? g.a + (size_t)m * g.lda : nullptr;

  const int step0 = (ks * 4 + wave) * steps_per_wave;
  const int nsteps_total = cdiv(g.K, 16);
  const int step1 = min(step0 + steps_per_wave, nsteps_total);

  f32x16 acc = f32x16{};
  for (int s = step0; s < step1; s += kSkinnyUnroll) {
    u32x4 a[kSkinnyUnroll], b[kSkinnyUnroll];
#pragma unroll
    for (int u = 0; u < kSkinnyUnroll; ++u) {
      const int k = (s + u) * 16 + half * 8;
      const bool ok = (s + u < step1) && (k < g.K);
      a[u] = (ok && wrow) ? ld16(wrow + k) : zero16();
      b[u] = (ok && xrow) ? ld16(xrow + k) : zero16();
    }
#pragma unroll
    for (int u = 0; u < kSkinnyUnroll; ++u) acc = mfma32(a[u], b[u], acc);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) red[wave][r][lane] = acc[r];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float v = red[0][r][lane] + red[1][r][lane] + red[2][r][lane] + red[3][r][lane];
      const int n = n0 + (r >> 2) * 8 + half * 4 + (r & 3);
      if (m >= g.M || n >= g.N) continue;
      if (partial) {
        partial[((size_t)ks * g.M + m) * g.N + n] = v;
      } else {
        store_out(out_col(g, n), m, v);
      }
    }
  }
}

// M <= 32 with K % 256 == 0: the decode projections at the K3 shape, bound by the weight stream.
// Wave w of a workgroup computes out[0:32, n0 + 32 w, +32) (n0 = 128 x) over the 128-wide k chunks
// [nch y / ks, nch (y + 1) / ks) of split y (x, y = workgroup ids), with the weight rows as the
// MFMA A operand and the activations as B. Each chunk's operand tiles (32 rows x 256 bytes: a
// wave's weight rows, and the workgroup's activation rows) are copied whole into LDS by
// wave-wide 1 KB DMA loads, four rows per load, into a three-slot ring: two chunks are in flight
// while one is multiplied, with one barrier per chunk (the activation tile is shared). A fourth
// slot, or 256-wide chunks in a two-slot ring (512-byte row segments), measured no faster. Loaded
// straight into the operand registers, each load took 16 bytes from each of 32 weight rows and
// the stream ran at ~4.3 TB/s. Row r of a tile holds its 16-byte chunk c at r*256 + ((c ^ (r & 15)) << 4),
// so the operand reads (one chunk of 16 consecutive rows per 16 lanes) are free of bank conflicts.
// One workgroup per CU (120 KB of LDS; 144 KB with the split operand).
constexpr int kSkChunk = 128;  // k values per chunk

// wait until at most n chunks' copies (VPC loads each) of this wave are still in flight
template <int VPC>
__device__ __forceinline__ void sk_wait_chunks(int n) {
  if (n >= 2)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * VPC) : "memory");
  else if (n == 1)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(VPC) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// SPLIT: the split operand (GemmArgs::a_split): each chunk stages the hi and the lo activations
// and every weight fragment feeds two MFMAs, so the weights are still read once.
template <bool SPLIT>
__global__ __launch_bounds__(256) void gemm_nt_skinny_dma(GemmArgs g, float* partial, int ks) {
  constexpr int NX = SPLIT ? 2 : 1;
  constexpr int RB = kSkChunk * 2;         // bytes of a row per chunk
  constexpr int TB = 32 * RB;              // one 32-row tile, 8 KB
  constexpr int XL = NX * TB / 1024 / 4;   // activation loads per wave per chunk (2 or 4)
  constexpr int VPC = TB / 1024 + XL;      // DMA loads per wave per chunk (10 or 12)
  constexpr int NS = 3;                     // ring slots (four measured no faster)
  __shared__ __attribute__((aligned(1024))) uint8_t wring[4][NS][TB];
  __shared__ __attribute__((aligned(1024))) uint8_t xring[NS][NX][TB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  const int n0 = blockIdx.x * 128 + wave * 32;
  const int nch_all = g.K / kSkChunk;
  const int c0 = (int)((long long)blockIdx.y * nch_all / ks), c1 = (int)((long long)(blockIdx.y + 1) * nch_all / ks);
  const int nch = c1 - c0;
  // load i of a tile fills its rows 4i .. 4i+3: lane L copies row 4i + L/16's source chunk
  // (L % 16) ^ (row & 15) into position L % 16. Weight rows past N re-read row N - 1 and
  // activation rows past M row M - 1 (computed, never stored).
  const int lrow = lane >> 4, lpos = lane & 15;
  const uint16_t* wsrc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 4 * i + lrow;
    wsrc[i] = wrow_ptr(g, min(n0 + row, g.N - 1)) + (size_t)c0 * kSkChunk + ((lpos ^ (row & 15)) << 3);
  }
  const uint16_t* xsrc[XL];
#pragma unroll
  for (int q = 0; q < XL; ++q) {
    const int j = wave * XL + q, row = 4 * (j & 7) + lrow;  // load j: half j / 8, rows 4 (j % 8) ..
    xsrc[q] = g.a + (size_t)min(row, g.M - 1) * g.lda + (j >> 3) * g.K + (size_t)c0 * kSkChunk +
              ((lpos ^ (row & 15)) << 3);
  }
  auto issue = [&](int ch) __attribute__((always_inline)) {
    const int sl = ch % NS;
    const uint32_t wd = lds_addr(wring[wave][sl]);
#pragma unroll
    for (int i = 0; i < 8; ++i) lds_dma16(wsrc[i] + ch * kSkChunk, wd + i * 1024);
#pragma unroll
    for (int q = 0; q < XL; ++q) {
      const int j = wave * XL + q;
      lds_dma16(xsrc[q] + ch * kSkChunk, lds_addr(xring[sl][j >> 3]) + (j & 7) * 1024);
    }
  };
  const int r = lane & 31;
  const uint32_t roff = r * RB, rsw = r & 15;
  f32x16 acc = f32x16{};
  auto compute = [&](int ch) __attribute__((always_inline)) {
    const int sl = ch % NS;
    const uint8_t* wt = wring[wave][sl] + roff;
    u32x4 wf[8], xf[NX][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t co = ((2 * u + half) ^ rsw) << 4;
      wf[u] = *(const u32x4*)(wt + co);
#pragma unroll
      for (int h = 0; h < NX; ++h) xf[h][u] = *(const u32x4*)(xring[sl][h] + roff + co);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int h = 0; h < NX; ++h) acc = mfma32(wf[u], xf[h][u], acc);
  };
  static_assert(NS - 2 <= 2, "sk_wait_chunks covers two chunks");
  // the source addresses (their segment lookups read the kernel arguments with vector loads) are
  // complete before the first copy, so that no wait for them lands between copies
#pragma unroll
  for (int i = 0; i < 8; ++i) asm volatile("" ::"v"(wsrc[i]));
#pragma unroll
  for (int q = 0; q < XL; ++q) asm volatile("" ::"v"(xsrc[q]));
  if (nch > 0) {
    for (int c = 0; c < NS - 1 && c < nch; ++c) issue(c);
    sk_wait_chunks<VPC>(min(NS - 2, nch - 1));  // chunk 0 has landed
    __syncthreads();
    for (int ch = 0; ch < nch; ++ch) {
      // chunk ch + NS - 1 goes to the slot of chunk ch - 1, which every wave finished before the
      // barrier that ended the previous step
      if (ch + NS - 1 < nch) issue(ch + NS - 1);
      compute(ch);
      sk_wait_chunks<VPC>(min(NS - 2, nch - 2 - ch));  // chunk ch + 1 has landed
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __syncthreads();
    }
  }
  // acc[r] = out(m = lane % 32, n = n0 + 8 (r / 4) + 4 half + r % 4)
  const int m = lane & 31;
  if (m >= g.M) return;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int n = n0 + (e >> 2) * 8 + half * 4 + (e & 3);
    if (n >= g.N) continue;
    if (partial)
      partial[((size_t)blockIdx.y * g.M + m) * g.N + n] = acc[e];
    else
      store_out(out_col(g, n), m, acc[e]);
  }
}

__global__ void gemm_reduce(GemmArgs g, const float* partial, int ksplit) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= g.M * g.N) return;
  const int m = idx / g.N, n = idx % g.N;
  float v = 0.f;
  for (int s = 0; s < ksplit; ++s) v += partial[((size_t)s * g.M + m) * g.N + n];
  store_out(out_col(g, n), m, v);
}

// ----------------------------------------------------------------------------------------
// Host launchers
// ----------------------------------------------------------------------------------------
static bool skinny_lds_ok(int M, int K) { return M <= 32 && K % 256 == 0; }

static int skinny_ksplit(int M, int N, int K) {
  if (skinny_lds_ok(M, K)) {
    // one 128-row workgroup per CU: the most k splits (at least two chunks each) that keep the
    // grid within 256 workgroups
    const int groups = cdiv(N, 128), nch = K / kSkChunk;
    int ks = 1;
    while (groups * (ks + 1) <= 256 && 2 * (ks + 1) <= nch) ++ks;
    return ks;
  }
  const int ntiles = cdiv(N, 32);
  int ks = 1;
  // aim for >= 512 workgroups while every wave keeps >= 16 k steps
  while (ntiles * ks < 512 && (cdiv(K, 16) / (ks * 2 * 4)) >= 16) ks *= 2;
  return ks;
}

size_t gemm_ws_bytes(int M, int N, int K) {
  if (M > 32 || M <= 0) return 0;
  const int ks = skinny_ksplit(M, N, K);
  return ks > 1 ? (size_t)ks * M * N * sizeof(float) : 0;
}

bool gemm_scatter_ok(const GemmArgs& g) {
  const CacheScatter& cs = g.cs;
  return g.nseg == 1 && dma_gemm_ok(g, 64) && cs.k && cs.v && cs.start && cs.T > 0 && cs.T_cap > 0 && cs.H > 0 &&
         cs.dn % 4 == 0 && cs.dv % 4 == 0 && cs.dk % 4 == 0 && cs.dn <= cs.dk && g.N == cs.H * (cs.dn + cs.dv) &&
         ((uintptr_t)cs.k & 7) == 0 && ((uintptr_t)cs.v & 7) == 0;
}

hipError_t launch_gemm(const GemmArgs& g, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (g.cs.k && !gemm_scatter_ok(g)) return hipErrorInvalidValue;
  // the split operand runs on the skinny LDS kernel (M <= 32), the DMA kernel or the 64-wide
  // k tiles of the large-M kernel
  if (g.a_split && (g.K % kSkChunk != 0 || g.lda < 2 * g.K || g.cs.k)) return hipErrorInvalidValue;
  if (g.M <= 32) {
    const int ks = ws ? skinny_ksplit(g.M, g.N, g.K) : 1;  // no workspace: one K split
    const int nsteps = cdiv(g.K, 16);
    const int spw = cdiv(nsteps, ks * 4);
    float* partial = nullptr;
    if (ks > 1) {
      if (ws_bytes < (size_t)ks * g.M * g.N * sizeof(float)) return hipErrorInvalidValue;
      partial = (float*)ws;
    }
    if (skinny_lds_ok(g.M, g.K) && g.a_split)
      gemm_nt_skinny_dma<true><<<dim3(cdiv(g.N, 128), ks), 256, 0, stream>>>(g, partial, ks);
    else if (skinny_lds_ok(g.M, g.K))
      gemm_nt_skinny_dma<false><<<dim3(cdiv(g.N, 128), ks), 256, 0, stream>>>(g, partial, ks);
    else
      gemm_nt_skinny<<<dim3(cdiv(g.N, 32), ks), 256, 0, stream>>>(g, partial, spw);
    if (ks > 1) {
      const int total = g.M * g.N;
      gemm_reduce<<<cdiv(total, 256), 256, 0, stream>>>(g, partial, ks);
    }
    return hipGetLastError();
  }
  if (dma_gemm_ok(g, 64)) {
    gemm_nt_dma<64, 2, 8><<<cdiv(g.M, 256) * cdiv(g.N, 256), 512, 0, stream>>>(g);
  } else if (g.M <= 128) {
    const int tiles = cdiv(g.M, 64) * cdiv(g.N, 128);
    gemm_nt_big<64, 128, 2, 2><<<tiles, 256, 0, stream>>>(g);
  } else {
    const int tiles = cdiv(g.M, 256) * cdiv(g.N, 256);
    gemm_nt_big<256, 256, 2, 2><<<tiles, 256, 0, stream>>>(g);
  }
  return hipGetLastError();
}

}  // namespace gmla
