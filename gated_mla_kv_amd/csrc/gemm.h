// Host-side interface of the NT GEMM kernels (out = a . w^T, bf16 operands, fp32 accumulate).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gmla {

// One weight segment: rows [n0, n1) of the virtual N axis come from `w` (row n at
// w + (n - n0) * K) and their outputs go to `out` (element (m, n) at out + m * ldo + (n - n0)),
// as fp32 (out_f32) or bf16.
struct GemmSeg {
  const uint16_t* w;
  void* out;
  int n0, n1;
  int ldo;
  int out_f32;
};

constexpr int kMaxSegs = 6;

// Optional epilogue that writes a single bf16 segment straight into the expanded KV cache (the
// kv up-projection of a prefill): output column n is head h = n / (dn + dv), j = n % (dn + dv);
// j < dn goes to k[b][h][p][j] (rows of dk values), else v[b][h][p][j - dn] (rows of dv); output row
// m is token m % T of sequence b = m / T at position p = start[b] + m % T (positions outside
// [0, T_cap) are skipped). k == nullptr: off.
struct CacheScatter {
  uint16_t* k;
  uint16_t* v;
  const int32_t* start;
  int T, T_cap, H, dn, dv, dk;
};

struct GemmArgs {
  const uint16_t* a;  // [M, lda], first K columns used (2K with a_split)
  int lda;
  int M, N, K;        // N = n1 of the last segment; K = weight row length
  int nseg;
  GemmSeg seg[kMaxSegs];
  CacheScatter cs;
  // Split operand: row m of a holds K bf16 values a_hi then K values a_lo (an fp32 activation
  // written as hi + lo), and out = (a_hi + a_lo) . w^T, both products accumulated in fp32. The
  // weight is read once per k step and used by two MFMAs. Needs K % 256 == 0 and lda >= 2K.
  int a_split;
};

// Workspace bytes the launcher may use (split-K partial sums for small M).
size_t gemm_ws_bytes(int M, int N, int K);
// Whether launch_gemm can run `args` with its cache-scatter epilogue (the large-M kernel, one
// segment, head rows in whole 4-column groups).
bool gemm_scatter_ok(const GemmArgs& args);
// Enqueue out = a . w^T over all segments. Returns hipSuccess or the launch error
// (hipErrorInvalidValue for a scatter that gemm_scatter_ok rejects).
hipError_t launch_gemm(const GemmArgs& args, void* ws, size_t ws_bytes, hipStream_t stream);

}  // namespace gmla
