// NT GEMM kernels for the layer's projections: out[m, n] = sum_k a[m, k] w[n, k].
//
// Weights are nn.Linear [out, in] matrices, so both operands are K-contiguous and feed the
// bf16 MFMA directly (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// * gemm_nt_big: M >= 64 (prefill). 256 threads, a BM x BN tile per workgroup, BK = 64,
//   double-buffered LDS tiles with a 144-byte row stride (conflict-free 16-byte reads over 16
//   consecutive rows), workgroup ids remapped so that each XCD walks a contiguous, M-grouped
//   range of tiles (operands reused from that XCD's L2).
// * gemm_nt_skinny: M <= 32 (decode). Weight-bandwidth bound: each wave computes
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
  auto load_tile = [&](int k0) {
    const bool kin = k0 + kc < g.K;
#pragma unroll
    for (int i = 0; i < CA; ++i)
      ra[i] = (kin && ((a_ok >> i) & 1u)) ? ld16(pa0 + i * a_step + k0) : zero16();
#pragma unroll
    for (int i = 0; i < CB; ++i) rb[i] = (kin && pb[i]) ? ld16(pb[i] + k0) : zero16();
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

  const int KT = cdiv(g.K, BK);
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
static int skinny_ksplit(int M, int N, int K) {
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

hipError_t launch_gemm(const GemmArgs& g, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (g.M <= 32) {
    const int ks = ws ? skinny_ksplit(g.M, g.N, g.K) : 1;  // no workspace: one K split
    const int nsteps = cdiv(g.K, 16);
    const int spw = cdiv(nsteps, ks * 4);
    float* partial = nullptr;
    if (ks > 1) {
      if (ws_bytes < (size_t)ks * g.M * g.N * sizeof(float)) return hipErrorInvalidValue;
      partial = (float*)ws;
    }
    gemm_nt_skinny<<<dim3(cdiv(g.N, 32), ks), 256, 0, stream>>>(g, partial, spw);
    if (ks > 1) {
      const int total = g.M * g.N;
      gemm_reduce<<<cdiv(total, 256), 256, 0, stream>>>(g, partial, ks);
    }
    return hipGetLastError();
  }
  if (g.M <= 128) {
    const int tiles = cdiv(g.M, 64) * cdiv(g.N, 128);
    gemm_nt_big<64, 128, 2, 2><<<tiles, 256, 0, stream>>>(g);
  } else {
    const int tiles = cdiv(g.M, 256) * cdiv(g.N, 256);
    gemm_nt_big<256, 256, 2, 2><<<tiles, 256, 0, stream>>>(g);
  }
  return hipGetLastError();
}

}  // namespace gmla
