// Row normalisations and the cache append.
//
// * rmsnorm_rows: KimiRMSNorm ("Kimi K3" attention code page): x * rsqrt(mean(x^2) + eps) in
//   fp32, times the gain, rounded once to bf16. One wave per row.
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

__global__ __launch_bounds__(256) void rmsnorm_rows(const float* __restrict__ x, int ldx,
                                                    const uint16_t* __restrict__ gain, int M, int N,
                                                    float eps, uint16_t* __restrict__ out, int ldo) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const float* xr = x + (size_t)row * ldx;
  float ss = 0.f;
  for (int i = lane * 4; i < N; i += 256) {
    const float4 v = *(const float4*)(xr + i);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = wave_sum(ss);
  const float inv = rsqrtf(ss / (float)N + eps);
  uint16_t* orow = out + (size_t)row * ldo;
  for (int i = lane * 4; i < N; i += 256) {
    const float4 v = *(const float4*)(xr + i);
    const uint2 gw = *(const uint2*)(gain + i);
    uint2 o;
    o.x = pack_bf16x2(v.x * inv * lo_bf16(gw.x), v.y * inv * hi_bf16(gw.x));
    o.y = pack_bf16x2(v.z * inv * lo_bf16(gw.y), v.w * inv * hi_bf16(gw.y));
    *(uint2*)(orow + i) = o;
  }
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
__global__ __launch_bounds__(256) void kv_append_kernel(KvAppendArgs a) {
  const int tok = blockIdx.x;
  const int b = tok / a.T, t = tok % a.T;
  const int p = a.pos[b] + t;
  if (p < 0 || p >= a.T_cap) return;  // outside the cache: nothing is written
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
                          uint16_t* out, int ldo, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  rmsnorm_rows<<<cdiv(M, 4), 256, 0, s>>>(x, ldx, gain, M, N, eps, out, ldo);
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

}  // namespace gmla
