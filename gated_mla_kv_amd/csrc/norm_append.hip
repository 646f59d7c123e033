// Row normalisations and the cache append.
//
// * rmsnorm_rows: KimiRMSNorm ("Kimi K3" attention code page): x * rsqrt(mean(x^2) + eps) in
//   fp32, times the gain, rounded once to bf16. One wave per row. With out_lo, the fp32 result
//   is also written as the bf16 pair (hi, lo), hi + lo within 2^-17 of it (the split operand of
//   the index-query GEMM).
// * layernorm_rows: the index-key LayerNorm with gain and bias (K3.1 Gated DSA blog, eq. (3)),
//   fp32 statistics (population variance), rounded once to bf16. One wave per row.
// * kv_append_kernel: the cache update of the KV cache card, with preallocated capacity in
//   place of concatenation: the latent row c ‖ r, the expanded keys k_nope_h ‖ r for every
//   head (the shared key part is the same r for all heads, shared-key-split page), the values
//   and the index key. Pure 16-byte copies, bit-exact.
//   FP8 caches (K3.1 Gated DSA blog, cache section): a latent row is the 512 E4M3 codes of c,
//   four fp32 scales (blocks of 128) and r in bf16, 656 bytes; an index key is 128 codes with
//   one fp32 scale kept in a separate array. A block's scale is the smallest power of two 2^k
//   (k >= -126) with max|v| <= 448 * 2^k; a code is e4m3(v * 2^-k), the product exact.
#include "common.h"
#include "kernels.h"

namespace gmla {

// One wave normalises row `row` of job j: out = bf16(x * rsqrt(mean(x^2) + eps) * gain), and with
// out_lo the bf16 rounding remainder of each value (the split operand's lo half).
__device__ __forceinline__ void rmsnorm_row(const RmsNormJob& j, int row, int lane, float eps) {
  const float* xr = j.x + (size_t)row * j.ldx;
  float ss = 0.f;
  for (int i = lane * 4; i < j.N; i += 256) {
    const float4 v = *(const float4*)(xr + i);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = wave_sum(ss);
  const float inv = rsqrtf(ss / (float)j.N + eps);
  uint16_t* orow = j.out + (size_t)row * j.ldo;
  for (int i = lane * 4; i < j.N; i += 256) {
    const float4 v = *(const float4*)(xr + i);
    const uint2 gw = *(const uint2*)(j.gain + i);
    const float f0 = v.x * inv * lo_bf16(gw.x), f1 = v.y * inv * hi_bf16(gw.x);
    const float f2 = v.z * inv * lo_bf16(gw.y), f3 = v.w * inv * hi_bf16(gw.y);
    uint2 o;
    o.x = pack_bf16x2(f0, f1);
    o.y = pack_bf16x2(f2, f3);
    *(uint2*)(orow + i) = o;
    if (j.out_lo) {  // f - hi is exact in fp32; its bf16 rounding leaves at most 2^-17 |f|
      uint2 r;
      r.x = pack_bf16x2(f0 - lo_bf16(o.x), f1 - hi_bf16(o.x));
      r.y = pack_bf16x2(f2 - lo_bf16(o.y), f3 - hi_bf16(o.y));
      *(uint2*)(j.out_lo + (size_t)row * j.ldo + i) = r;
    }
  }
}

// Four rows per workgroup: the first cdiv(a.M, 4) workgroups take job a, the rest job b (two
// normalisations of one step in one launch).
__global__ __launch_bounds__(256) void rmsnorm_rows(RmsNormJob a, RmsNormJob b, float eps) {
  const int lane = threadIdx.x & 63;
  const int na = cdiv(a.M, 4);
  const bool first = (int)blockIdx.x < na;
  const RmsNormJob& j = first ? a : b;
  const int row = ((int)blockIdx.x - (first ? 0 : na)) * 4 + (threadIdx.x >> 6);
  if (row >= j.M) return;
  rmsnorm_row(j, row, lane, eps);
}

__global__ __launch_bounds__(256) void layernorm_rows(const float* __restrict__ x, int ldx,
                                                      const uint16_t* __restrict__ gain,
                                                      const uint16_t* __restrict__ bias, int M,
                                                      int N, float eps, uint16_t* __restrict__ out,
                                                      int ldo) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const float* xr = x + (size_t)row * ldx;
  float s = 0.f;
  for (int i = lane * 4; i < N; i += 256) {
    const float4 v = *(const float4*)(xr + i);
    s += v.x + v.y + v.z + v.w;
  }
  const float mean = wave_sum(s) / (float)N;
  float ss = 0.f;
  for (int i = lane * 4; i < N; i += 256) {
    const float4 v = *(const float4*)(xr + i);
    const float a = v.x - mean, b = v.y - mean, c = v.z - mean, d = v.w - mean;
    ss += a * a + b * b + c * c + d * d;
  }
  const float inv = rsqrtf(wave_sum(ss) / (float)N + eps);
  uint16_t* orow = out + (size_t)row * ldo;
  for (int i = lane * 4; i < N; i += 256) {
    const float4 v = *(const float4*)(xr + i);
    const uint2 gw = *(const uint2*)(gain + i);
    const uint2 bw = *(const uint2*)(bias + i);
    uint2 o;
    o.x = pack_bf16x2((v.x - mean) * inv * lo_bf16(gw.x) + lo_bf16(bw.x),
                      (v.y - mean) * inv * hi_bf16(gw.x) + hi_bf16(bw.x));
    o.y = pack_bf16x2((v.z - mean) * inv * lo_bf16(gw.y) + lo_bf16(bw.y),
                      (v.w - mean) * inv * hi_bf16(gw.y) + hi_bf16(bw.y));
    *(uint2*)(orow + i) = o;
  }
}

// ---------------------------------------------------------------------------------------------
// The index key in fp64 (K3.1 Gated DSA blog, eq. (3) and the LayerNorm paragraph after it):
// k^I = LayerNorm(W_k^I x) * gain + bias, computed in fp64 and rounded once to bf16, the index
// cache type. The key's only rounding is then the storage rounding of an fp64 value, so the
// cached key is the bf16 rounding of the exact LayerNorm output (an fp32 computation lands a
// few keys per thousand features one bf16 step away from it).
//
// index_key_partial_f64: partial[ks][m][j] = sum of x[m][k] w[j][k] over split ks's k range, on
//   the fp64 MFMA (v_mfma_f64_16x16x4_f64): bf16 inputs and their products are exact in fp64.
//   A workgroup takes 32 token rows and all 128 features, wave w the features [32w, 32w + 32)
//   as 2 x 2 tiles of 16 x 16. Per 32-wide k chunk every lane loads 8 consecutive k (16 bytes)
//   of its two x rows and its two weight rows; the chunk's 8 MFMA steps give MFMA k slot g
//   (lane group g = lane / 16) the chunk index 8 g + step.
// index_key_finalize: one wave per row: the splits summed in order, the mean and the population
//   variance in fp64, then the gain, the bias and one rounding to bf16 (nearest, ties to even).
// ---------------------------------------------------------------------------------------------
typedef double f64x4 __attribute__((ext_vector_type(4)));
constexpr int kIkRows = 32, kIkChunk = 32;

__device__ __forceinline__ double bf16_to_f64(uint32_t bits16) {
  return (double)__uint_as_float(bits16 << 16);
}

// bf16 bits of an fp64 value: 8 significant bits, round to nearest, ties to even (normal range)
__device__ __forceinline__ uint16_t f64_to_bf16_bits(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t sign = (uint32_t)(u >> 63) << 15;
  uint64_t mag = u & 0x7FFFFFFFFFFFFFFFull;
  if (mag == 0) return (uint16_t)sign;
  mag += ((mag >> 45) & 1ull) + ((1ull << 44) - 1ull);  // a carry into the exponent is right
  mag >>= 45;                                            // 11 exponent bits, 7 mantissa bits
  const int e = (int)(mag >> 7) - 1023 + 127;
  if (e >= 255) return (uint16_t)(sign | 0x7F80u);
  if (e <= 0) return (uint16_t)sign;                     // below bf16's normal range
  return (uint16_t)(sign | ((uint32_t)e << 7) | (uint32_t)(mag & 0x7Fu));
}

__global__ __launch_bounds__(256) void index_key_partial_f64(const uint16_t* __restrict__ x, int ldx,
                                                             const uint16_t* __restrict__ w, int M, int K,
                                                             int chunks_per_split, double* __restrict__ partial) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m0 = blockIdx.x * kIkRows, ks = blockIdx.y;
  const int c0 = ks * chunks_per_split, c1 = min(c0 + chunks_per_split, K / kIkChunk);
  const int r = lane & 15, g = lane >> 4;
  // rows past M re-read row M - 1 (computed, never stored)
  const uint16_t* xr0 = x + (size_t)min(m0 + r, M - 1) * ldx + 8 * g;
  const uint16_t* xr1 = x + (size_t)min(m0 + 16 + r, M - 1) * ldx + 8 * g;
  const uint16_t* wr0 = w + (size_t)(32 * wave + r) * K + 8 * g;
  const uint16_t* wr1 = w + (size_t)(32 * wave + 16 + r) * K + 8 * g;
  f64x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
  u32x4 cur[4], nxt[4];
  auto load = [&](int c, u32x4* v) __attribute__((always_inline)) {
    const int k = c * kIkChunk;
    v[0] = ld16(xr0 + k);
    v[1] = ld16(xr1 + k);
    v[2] = ld16(wr0 + k);
    v[3] = ld16(wr1 + k);
  };
  if (c0 < c1) load(c0, cur);
  for (int c = c0; c < c1; ++c) {
    load(min(c + 1, c1 - 1), nxt);  // the last chunk again after the last: unused
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const int word = st >> 1;
      const bool hi = st & 1;
      double a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t wa = cur[i][word], wb = cur[2 + i][word];
        a[i] = bf16_to_f64(hi ? (wa >> 16) : (wa & 0xFFFFu));
        b[i] = bf16_to_f64(hi ? (wb >> 16) : (wb & 0xFFFFu));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) cur[i] = nxt[i];
  }
  // D lane l, item v: row l / 16 + 4 v, column l % 16 of the 16 x 16 tile (the fp64 MFMA's
  // output layout, measured: unlike the fp32 16x16x4 one, the item steps over rows by 4)
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = m0 + 16 * i + g + 4 * v;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        partial[((size_t)ks * M + m) * 128 + 32 * wave + 16 * j + r] = acc[i][j][v];
    }
}

__global__ __launch_bounds__(256) void index_key_finalize(const double* __restrict__ partial, int ksplit, int M,
                                                          const uint16_t* __restrict__ gain,
                                                          const uint16_t* __restrict__ bias, double eps,
                                                          uint16_t* __restrict__ out, int ldo) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  double v0 = 0.0, v1 = 0.0;
  for (int s = 0; s < ksplit; ++s) {
    const double* p = partial + ((size_t)s * M + m) * 128 + 2 * lane;
    v0 += p[0];
    v1 += p[1];
  }
  double sum = v0 + v1;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
  const double mean = sum / 128.0;
  const double d0 = v0 - mean, d1 = v1 - mean;
  double ss = d0 * d0 + d1 * d1;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  const double inv = 1.0 / sqrt(ss / 128.0 + eps);
  const uint32_t gw = *(const uint32_t*)(gain + 2 * lane), bw = *(const uint32_t*)(bias + 2 * lane);
  const uint16_t o0 = f64_to_bf16_bits(d0 * inv * bf16_to_f64(gw & 0xFFFFu) + bf16_to_f64(bw & 0xFFFFu));
  const uint16_t o1 = f64_to_bf16_bits(d1 * inv * bf16_to_f64(gw >> 16) + bf16_to_f64(bw >> 16));
  *(uint32_t*)(out + (size_t)m * ldo + 2 * lane) = (uint32_t)o0 | ((uint32_t)o1 << 16);
}

static int index_key_chunks_per_split(int M, int K) {
  const int chunks = K / kIkChunk, blocks = cdiv(M, kIkRows);
  const int ks = max(1, min(cdiv(256, blocks), 56));  // about one workgroup per CU
  return cdiv(chunks, ks);
}

int index_key_splits(int M, int K) {
  if (M <= 0 || K <= 0) return 0;
  return cdiv(K / kIkChunk, index_key_chunks_per_split(M, K));
}

hipError_t launch_index_key_f64(const uint16_t* x, int ldx, const uint16_t* w, const uint16_t* gain,
                                const uint16_t* bias, int M, int K, double eps, double* partial, uint16_t* out,
                                int ldo, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (K % kIkChunk != 0 || ldx % 8 != 0 || ldo % 2 != 0) return hipErrorInvalidValue;
  const int cps = index_key_chunks_per_split(M, K), ks = index_key_splits(M, K);
  index_key_partial_f64<<<dim3(cdiv(M, kIkRows), ks), 256, 0, s>>>(x, ldx, w, M, K, cps, partial);
  index_key_finalize<<<cdiv(M, 4), 256, 0, s>>>(partial, ks, M, gain, bias, eps, out, ldo);
  return hipGetLastError();
}

// E4M3 codes of n = 8 * lanes values v (8 per lane, lanes in groups of `group` sharing a scale):
// returns the 8 codes as two words and the group's scale.
template <int GROUP>
__device__ __forceinline__ u32x2 fp8_group(const u32x4 v, float& scale) {
  float x[8] = {lo_bf16(v.x), hi_bf16(v.x), lo_bf16(v.y), hi_bf16(v.y),
                lo_bf16(v.z), hi_bf16(v.z), lo_bf16(v.w), hi_bf16(v.w)};
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x[i]));
#pragma unroll
  for (int o = 1; o < GROUP; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  // m = 1.f * 2^(e - 127): 448 * 2^k >= m for k = e - 135 when 1.f <= 1.75, else for k = e - 134
  const uint32_t mb = __float_as_uint(m);
  const int e = (int)(mb >> 23);
  const int k = max((mb & 0x7FFFFFu) <= 0x600000u ? e - 135 : e - 134, -126);
  scale = m > 0.f ? __uint_as_float((uint32_t)(k + 127) << 23) : 0.f;
  const float inv = __uint_as_float((uint32_t)(127 - k) << 23);  // 2^-k, exact
  uint32_t c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    c[i] = m > 0.f ? e4m3_encode(x[i] * inv) : (__float_as_uint(x[i]) >> 24) & 0x80u;
  return u32x2{c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24), c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24)};
}

// One workgroup per new token (b, t). Work items are 16-byte chunks:
//   latent row: L/8 chunks of c then DS/8 of r; per head: DN/8 chunks of k_nope then DS/8 of r
//   for K, DV/8 chunks for V; the index key: DI/8 chunks.
#ifdef GMLA_DEBUG_CHECKS
__device__ uint32_t g_debug_flags_append;
#endif

__global__ __launch_bounds__(256) void kv_append_kernel(KvAppendArgs a) {
  const int tok = blockIdx.x;
  const int b = tok / a.T, t = tok % a.T;
  const int p = a.pos[b] + t;
  if (p < 0 || p >= a.T_cap) {  // outside the cache: nothing is written
#ifdef GMLA_DEBUG_CHECKS
    if (threadIdx.x == 0) atomicOr(&g_debug_flags_append, kDbgAppendPos);
#endif
    return;
  }
#ifdef GMLA_DEBUG_CHECKS
  if (a.pages.table && threadIdx.x == 0) {  // cache_row clamps a bad entry to a valid page
    const int e = a.pages.table[(size_t)b * a.pages.max_blocks + p / a.pages.page_size];
    if (e < 0 || e >= a.pages.n_pages) atomicOr(&g_debug_flags_append, kDbgAppendPage);
  }
#endif
  const size_t bt = (size_t)b * a.T + t;
  const size_t crow = cache_row(a.pages, a.T_cap, b, p);  // latent / index-key row
  const int cL = a.L / 8, cS = a.DS / 8, cN = a.DN / 8, cV = a.DV / 8, cI = a.DI / 8;
  // latent
  if (a.latent && a.latent_fp8) {  // K3 only (L = 512, DS = 64): wave 0, lane l codes c[8l .. 8l+7]
    if (threadIdx.x < 64) {
      const int l = threadIdx.x;
      uint8_t* row = (uint8_t*)a.latent + crow * kFp8RowBytes;
      float scale;
      const u32x2 codes = fp8_group<16>(ld16(a.c + bt * a.ld_c + l * 8), scale);
      *(u32x2*)(row + l * 8) = codes;
      if ((l & 15) == 0) *(float*)(row + kFp8ScaleOff + (l >> 4) * 4) = scale;
      if (l < 8) st16(row + kFp8ROff + l * 16, ld16(a.r + bt * a.ld_r + l * 8));
    }
  } else if (a.latent) {
    uint16_t* dst = a.latent + crow * (a.L + a.DS);
    for (int i = threadIdx.x; i < cL + cS; i += blockDim.x) {
      const uint16_t* src = (i < cL) ? a.c + bt * a.ld_c + i * 8 : a.r + bt * a.ld_r + (i - cL) * 8;
      st16(dst + i * 8, ld16(src));
    }
  }
  if (a.k && !a.k_nope) {  // k_nope and v already in the cache (written by the kv up-projection)
    for (int i = threadIdx.x; i < a.H * cS; i += blockDim.x) {
      const int h = i / cS, j = i % cS;
      uint16_t* dst = a.k + (((size_t)b * a.H + h) * a.T_cap + p) * (a.DN + a.DS) + (cN + j) * 8;
      st16(dst, ld16(a.r + bt * a.ld_r + j * 8));
    }
  } else if (a.k) {
    const int per_head = cN + cS;
    for (int i = threadIdx.x; i < a.H * per_head; i += blockDim.x) {
      const int h = i / per_head, j = i % per_head;
      const uint16_t* src = (j < cN) ? a.k_nope + bt * a.ld_k_tok + (size_t)h * a.ld_k_head + j * 8
                                     : a.r + bt * a.ld_r + (j - cN) * 8;
      uint16_t* dst = a.k + (((size_t)b * a.H + h) * a.T_cap + p) * (a.DN + a.DS) + j * 8;
      st16(dst, ld16(src));
    }
  }
  if (a.v) {
    for (int i = threadIdx.x; i < a.H * cV; i += blockDim.x) {
      const int h = i / cV, j = i % cV;
      const uint16_t* src = a.v_new + bt * a.ld_v_tok + (size_t)h * a.ld_v_head + j * 8;
      uint16_t* dst = a.v + (((size_t)b * a.H + h) * a.T_cap + p) * a.DV + j * 8;
      st16(dst, ld16(src));
    }
  }
  if (a.idx && a.idx_fp8) {  // DI = 128: lanes 0..15 of wave 1, one scale per key
    if (threadIdx.x >= 64 && threadIdx.x < 80) {
      const int l = threadIdx.x - 64;
      float scale;
      const u32x2 codes = fp8_group<16>(ld16(a.idx_new + bt * a.ld_idx + l * 8), scale);
      *(u32x2*)((uint8_t*)a.idx + crow * a.DI + l * 8) = codes;
      if (l == 0) a.idx_scale[crow] = scale;
    }
  } else if (a.idx) {
    for (int i = threadIdx.x; i < cI; i += blockDim.x)
      st16(a.idx + crow * a.DI + i * 8, ld16(a.idx_new + bt * a.ld_idx + i * 8));
  }
}

hipError_t launch_rmsnorm(const float* x, int ldx, const uint16_t* gain, int M, int N, float eps,
                          uint16_t* out, int ldo, uint16_t* out_lo, hipStream_t s) {
  return launch_rmsnorm2(RmsNormJob{x, ldx, gain, M, N, out, ldo, out_lo}, RmsNormJob{}, eps, s);
}

hipError_t launch_rmsnorm2(const RmsNormJob& a, const RmsNormJob& b, float eps, hipStream_t s) {
  const int blocks = cdiv(max(a.M, 0), 4) + cdiv(max(b.M, 0), 4);
  if (blocks == 0) return hipSuccess;
  rmsnorm_rows<<<blocks, 256, 0, s>>>(a, b, eps);
  return hipGetLastError();
}

hipError_t launch_layernorm(const float* x, int ldx, const uint16_t* gain, const uint16_t* bias,
                            int M, int N, float eps, uint16_t* out, int ldo, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  layernorm_rows<<<cdiv(M, 4), 256, 0, s>>>(x, ldx, gain, bias, M, N, eps, out, ldo);
  return hipGetLastError();
}

hipError_t launch_kv_append(const KvAppendArgs& a, hipStream_t s) {
  if (a.B <= 0 || a.T <= 0) return hipSuccess;
  kv_append_kernel<<<a.B * a.T, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t read_debug_flags_append(uint32_t* flags, hipStream_t st) {
  *flags = 0;
#ifdef GMLA_DEBUG_CHECKS
  hipError_t e = hipMemcpyFromSymbolAsync(flags, HIP_SYMBOL(g_debug_flags_append), sizeof(uint32_t), 0,
                                          hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  const uint32_t zero = 0;
  if (e == hipSuccess)
    e = hipMemcpyToSymbolAsync(HIP_SYMBOL(g_debug_flags_append), &zero, sizeof(uint32_t), 0, hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  return e;
#else
  (void)st;
  return hipSuccess;
#endif
}

}  // namespace gmla
