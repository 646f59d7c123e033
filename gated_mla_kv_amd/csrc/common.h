// Device helpers shared by the gfx950 kernels: vector types, bf16 conversion, MFMA wrappers,
// the LDS transpose read, wave reductions, and the compile-time layer shapes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gmla {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define GMLA_LDS __attribute__((address_space(3)))

// ---------------------------------------------------------------------------------------
// bf16 <-> f32. Rounding is to nearest, ties to even (no NaN inputs on this path).
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
typedef float f32x2_ __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_ __attribute__((ext_vector_type(2)));
// two floats -> packed bf16 pair (lo in bits 0..15): one v_cvt_pk_bf16_f32 on gfx950
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_{lo, hi}, bf16x2_));
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return (uint16_t)(pack_bf16x2(f, 0.f) & 0xFFFFu);
}
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
// Eight fp32 values as two bf16 MFMA operands: hi = bf16(f) (nearest even) and lo = bf16(f - hi).
// f - hi is exact in fp32 and lo rounds it with error <= 2^-9 |f - hi| <= 2^-18 |f|, so an MFMA
// pair hi.b + lo.b carries f to about 17 bits, with every product exact.
__device__ __forceinline__ void split_bf16x8(const float* f, uint32_t* hi, uint32_t* lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hi[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    lo[i] = pack_bf16x2(f[2 * i] - lo_bf16(hi[i]), f[2 * i + 1] - hi_bf16(hi[i]));
  }
}
typedef _Float16 f16x2_ __attribute__((ext_vector_type(2)));
// two floats -> packed fp16 pair, round to nearest even (lo in bits 0..15)
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_{lo, hi}, f16x2_));
}
__device__ __forceinline__ float lo_f16(uint32_t w) { return (float)__builtin_bit_cast(f16x2_, w).x; }
__device__ __forceinline__ float hi_f16(uint32_t w) { return (float)__builtin_bit_cast(f16x2_, w).y; }

// ---------------------------------------------------------------------------------------
// MFMA (CDNA4 bf16, fp32 accumulate). Lane layouts (checked on the hardware):
//   32x32x16: A lane l holds row l%32, k = 8*(l/32)+i; B lane l holds col l%32, same k;
//             C lane l holds col l%32, rows (j/4)*8 + (l/32)*4 + j%4, j = 0..15.
//   16x16x32: A lane l holds row l%16, k = 8*(l/16)+i; B col l%16, same k;
//             C lane l holds col l%16, rows 4*(l/16) + j, j = 0..3.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------------------
// LDS transpose read (ds_read_b64_tr_b16). Within each group of 16 lanes, with chunk_j the
// four 16-bit values at lane j's address, lane i receives
//   out[r] = chunk_{(i>>2) + 4r}[i & 3],  r = 0..3.
// To read an MFMA operand whose k index runs down the rows of a row-major [k][n] LDS tile
// (lane needs column n, four consecutive k), lane j of the group points at
//   &tile[k0 + (j>>2)][n0 + 4*(j&3)]
// and lane i then holds tile[k0 + r][n0 + i] for r = 0..3.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ u32x2 lds_read_tr16(const void* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GMLA_LDS i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// LDS transpose read of bytes (ds_read_b64_tr_b8). Within each group of 16 lanes, lane j points
// at &tile[k0 + (j>>1)][n0 + 8*(j&1)] of a row-major byte tile; lane i then holds
// tile[k0 + r][n0 + i] in byte r, r = 0..7 (eight rows of one column).
// Takes the LDS byte address (as from lds_addr).
__device__ __forceinline__ u32x2 lds_read_tr8(uint32_t lds_byte_addr) {
  typedef int i32x2_t __attribute__((ext_vector_type(2)));
  i32x2_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((GMLA_LDS i32x2_t*)(uintptr_t)lds_byte_addr);
  return __builtin_bit_cast(u32x2, v);
}

// One wave-wide global_load_lds_dwordx4: lane L's 16 bytes from `gsrc` land in LDS at
// lds_byte_addr + 16*L (which must be the same in every lane). Issued from inline asm so that the compiler does not place a blanket
// vmcnt(0) wait in front of every later LDS read (it cannot tell LDS-DMA destinations apart);
// callers wait on vmcnt themselves before the data is read.
__device__ __forceinline__ void lds_dma16(const void* gsrc, uint32_t lds_byte_addr) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds_byte_addr)), "v"(gsrc)
      : "memory", "m0");
}
// As lds_dma16, with the source at sbase (wave-uniform, kept in SGPRs) + voff bytes (per lane).
__device__ __forceinline__ void lds_dma16_sbase(uint32_t voff, const void* sbase, uint32_t lds_byte_addr) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds_byte_addr)), "v"(voff), "s"(sbase)
      : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(GMLA_LDS const void*)p;
}

// ---------------------------------------------------------------------------------------
// Loads / stores
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *(const u32x2*)p; }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *(u32x4*)p = v; }
__device__ __forceinline__ u32x4 zero16() { return u32x4{0u, 0u, 0u, 0u}; }

// ---------------------------------------------------------------------------------------
// Wave reductions (wave64)
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// ---------------------------------------------------------------------------------------
// OCP E4M3 (FP8 caches). Decoding uses the hardware conversion (exact); encoding is written
// out: round to nearest, ties to even, sign copied, magnitudes from 448 up saturate to 448.
// ---------------------------------------------------------------------------------------
// four E4M3 bytes -> four bf16 (exact: every E4M3 value is a bf16 value), as two packed words,
// one v_cvt_scalef32_pk_bf16_fp8 per pair (scale 1: the exponent adjustment is zero)
__device__ __forceinline__ u32x2 e4m3x4_to_bf16(uint32_t w) {
  return u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true))};
}
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  uint32_t mag;
  if (a >= 448.f) {
    mag = 0x7Eu;
  } else if (a < 0.015625f) {  // below 2^-6: steps of 2^-9 (8 steps is the smallest normal)
    mag = (uint32_t)rintf(a * 512.f);
  } else {
    const uint32_t ua = __float_as_uint(a);
    const uint32_t e = (ua >> 23) - 120u;  // biased E4M3 exponent, 1..8
    uint32_t q = (ua >> 20) & 7u;
    const uint32_t rem = ua & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ++q;  // a carry into the exponent is right
    mag = min((e << 3) + q, 0x7Eu);
  }
  return sign | mag;
}

// logistic function; the reciprocal is v_rcp_f32 (within 1 ulp) rather than an IEEE division,
// whose scale/fixup sequence was ten instructions per call in the gate epilogues
__device__ __forceinline__ float sigmoidf_(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// ---------------------------------------------------------------------------------------
// Compile-time layer shapes (the dims a kernel is instantiated for)
// ---------------------------------------------------------------------------------------
struct ShapeK3 {
  static constexpr int H = 96, DN = 128, DS = 64, DV = 128, L = 512, QL = 1536, HID = 7168;
  static constexpr int NIH = 32, DI = 128;
};
struct ShapeTiny {
  static constexpr int H = 4, DN = 16, DS = 8, DV = 16, L = 32, QL = 64, HID = 256;
  static constexpr int NIH = 0, DI = 0;
};

__host__ __device__ constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ constexpr int round_up(int a, int b) { return cdiv(a, b) * b; }

}  // namespace gmla
