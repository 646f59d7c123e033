// Raw attention logits, for checking the score computation at the kernel boundary on small
// shapes: s[b,h,i,j] = scale * (q_{b,i,h} . k_{b,h,j}), the argument of the softmax in the
// attention ([DSA] eq. (9); the eager form softmax(q k^T * scale) on the Kimi K2 KV-cache card),
// unmasked. Keys are either per head (the expanded form, [B,H,Tk,D]) or one row per position
// shared by every head (the absorbed form's latent [c ; r], [B,1,Tk,D]).
//
// The products use the same arithmetic as the attention kernels: bf16 operands into
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation over 16-wide steps of D. One wave computes
// a 32 (queries) x 32 (keys) tile of one (b, h) with its operands read straight from memory
// (lane l: query or key row l % 32, features 8 (l / 32) .. +8 of each step); features past D
// (D a multiple of 8) enter as zeros, rows past Tq or Tk repeat the last row and are not stored.
#include "common.h"
#include "kernels.h"

namespace gmla {

__global__ __launch_bounds__(64) void debug_scores_kernel(ScoresArgs a) {
  const int lane = threadIdx.x, g2 = lane >> 5, l32 = lane & 31;
  const int j0 = blockIdx.x * 32, i0 = blockIdx.y * 32;
  const int b = blockIdx.z / a.H, h = blockIdx.z % a.H;
  const int qi = min(i0 + l32, a.Tq - 1), kj = min(j0 + l32, a.Tk - 1);
  const uint16_t* qrow = a.q + (((size_t)b * a.Tq + qi) * a.H + h) * a.D;
  const uint16_t* krow = a.k + (((size_t)b * a.Hk + (a.Hk == 1 ? 0 : h)) * a.Tk + kj) * a.D;
  f32x16 acc = f32x16{};
  for (int s = 0; s * 16 < a.D; ++s) {
    const int f = s * 16 + g2 * 8;  // this lane's 8 features of the step
    const u32x4 qa = f < a.D ? ld16(qrow + f) : u32x4{0u, 0u, 0u, 0u};
    const u32x4 kb = f < a.D ? ld16(krow + f) : u32x4{0u, 0u, 0u, 0u};
    acc = mfma32(qa, kb, acc);  // D[i][j] += q_i . k_j over the step
  }
  // lane l holds column j = l % 32 and rows 8 (r / 4) + 4 (l / 32) + r % 4
  const int j = j0 + l32;
  if (j >= a.Tk) return;
  float* out = a.logits + ((size_t)b * a.H + h) * a.Tq * a.Tk;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = i0 + 8 * (r >> 2) + 4 * g2 + (r & 3);
    if (i < a.Tq) out[(size_t)i * a.Tk + j] = acc[r] * a.scale;
  }
}

hipError_t launch_debug_scores(const ScoresArgs& a, hipStream_t st) {
  if (a.B <= 0 || a.H <= 0 || a.Tq <= 0 || a.Tk <= 0) return hipSuccess;
  const dim3 grid(cdiv(a.Tk, 32), cdiv(a.Tq, 32), a.B * a.H);
  debug_scores_kernel<<<grid, 64, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace gmla
