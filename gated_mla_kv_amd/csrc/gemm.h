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

struct GemmArgs {
  const uint16_t* a;  // [M, lda], first K columns used
  int lda;
  int M, N, K;        // N = n1 of the last segment
  int nseg;
  GemmSeg seg[kMaxSegs];
};

// Workspace bytes the launcher may use (split-K partial sums for small M).
size_t gemm_ws_bytes(int M, int N, int K);
// Enqueue out = a . w^T over all segments. Returns hipSuccess or the launch error.
hipError_t launch_gemm(const GemmArgs& args, void* ws, size_t ws_bytes, hipStream_t stream);

}  // namespace gmla
