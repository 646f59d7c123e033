// Gated DSA index scores and top-k selection, and decode attention over the expanded cache.
//
// index_scores_kernel (K3.1 Gated DSA blog, eq. (5)):
//   I[b, s] = (1/sqrt(n_idx d_idx)) sum_h a[b,h] ReLU(q^I[b,h] . k^I[b,s]),  s < t
// The query q^I is fp32, as eq. (5) leaves it unrounded: each of its values enters the MFMA as a
// bf16 pair hi + lo (split_bf16x8), so a key tile takes two MFMAs per k-step on the same keys and
// the dot products carry the query to about 17 bits (fp32 accumulation, exact products).
// The dot products are a [32 heads x 128] . [128 x 32 positions] bf16 MFMA per wave, with each
// 32-position tile of index keys (256 bytes per position, each read once) copied whole into the
// wave's LDS ring and the B operand read from there; eight waves per workgroup, one workgroup
// per CU. Lane l ends with position l%32 and 16 heads, so the head-weighted ReLU sum is in-lane
// plus one xor-32 shuffle. 1/sqrt(32*128) = 1/64 is folded into a exactly. FP8 index keys (128
// E4M3 codes and one scale s >= 0 per position, the blog's cache section) are copied the same
// way, widened exactly to bf16 when read, and the position's score is multiplied by s
// (ReLU(s z) = s ReLU(z) for s >= 0).
//
// Top-k (eq. (6)): S = the min(k, t) largest I, ties to the lower position, -0 == +0, written
// in ascending position order, over order-preserving 32-bit keys of the fp32 scores.
// * index_scores_kernel also counts the top 12-bit digit of every key into the row's histogram.
// * topk_count_kernel (one workgroup per 2048-position chunk) finds the bin where the count from
//   the top reaches k, counts the chunk's keys above it and lists the keys inside it.
// * topk_select_compact_kernel (a few workgroups per row, each covering a few chunks): every
//   workgroup radix-selects among the listed keys the threshold key and the last kept position
//   among its copies, scans the per-chunk kept counts into output offsets and writes its chunks'
//   kept positions in order. Where a row would need more than four chunks per workgroup (many
//   long rows), topk_select_kernel (one workgroup per row) selects and scans once, and
//   topk_compact_kernel (one workgroup per chunk) writes the chunks.
// * A row whose boundary bin exceeds the LDS candidate buffer (e.g. thousands of equal scores)
//   runs the whole selection in one select workgroup instead: a radix select over 12-, 12- and
//   8-bit digits with the row's keys in registers, and an ordered compaction in which every
//   wave owns a contiguous run of positions.
// * Rows of at most 4096 positions skip the chunk lists: topk_row_kernel runs that one-workgroup
//   selection directly, with the first digit's bin read off the score kernel's histogram.
//
// expanded_attn_kernel: one query per (b, h) against the expanded cache k [B,H,T_cap,192],
// v [B,H,T_cap,128] (KV cache card): 61,440 bytes per position, HBM bound at ~1 flop per byte,
// so plain fp32 VALU dot products; 4 lanes per key, 16 keys per wave per step, per-wave online
// softmax, waves merged through LDS.
#include "common.h"
#include "kernels.h"

namespace gmla {

// As lds_dma16_sbase with 4 bytes per lane (global_load_lds_dword): lane L's word lands at
// lds_byte_addr + 4*L.
#ifdef GMLA_DEBUG_CHECKS
__device__ uint32_t g_debug_flags_topk;  // kDbgTopkOffset, set by the top-k compactions
#endif

__device__ __forceinline__ void lds_dma4_sbase(uint32_t voff, const void* sbase, uint32_t lds_byte_addr) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, %2"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds_byte_addr)), "v"(voff), "s"(sbase)
      : "memory", "m0");
}

// ------------------------------------------------------------------------------------------
// Index scores (K3 indexer: 32 heads x 128)
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(float f);
constexpr int kHistBins = 4096;      // first radix digit: the top 12 bits of the order key
constexpr int kScoreTilesMin = 16;   // fewest 32-position tiles per workgroup
constexpr int kScoreWaves = 8;

// One workgroup per (chunk, row); a row's chunks split the 32-position tiles of the longest row
// as evenly as whole tiles allow, and wave w scores the tiles w, w+8, ... of its chunk. A tile's
// keys are contiguous (32 consecutive cache rows; a tile never crosses a page), so the wave
// copies each tile whole into its own two-slot LDS ring with wave-wide 1 KB DMA loads, the next
// tile in flight while it scores the current one, and reads the MFMA's B operand from there. Loaded straight into the operand registers, each load took
// 16 or 8 bytes from each of 32 rows: 31 against 26 us for 134 MB in a probe of the two forms.
// Every score's top digit goes into an LDS histogram that is added to the row's histogram at
// the end. The launcher picks the chunks per row so that all rows' workgroups fill the CUs once
// (one per CU). A workgroup takes as long as its busiest wave: B = 8 rows of 65,537 positions
// (2,049 tiles) in 32 chunks of 64 or 65 tiles leave one wave per row a ninth tile that holds a
// single position, where chunks of 65 whole tiles gave one wave in every workgroup a ninth full
// tile (and fixed chunks of 64 tiles made 264 workgroups, the 8 past the 256 CUs a second
// round).
// Tile layouts in LDS (conflict-free 16-byte reads of one chunk from 16 rows):
// * bf16: row r (256 B) holds its 16-byte chunk c at r*256 + ((c ^ (r & 15)) << 4);
// * FP8: row r (128 B of codes) holds chunk c at r*128 + ((c ^ ((r >> 1) & 7)) << 4), and the
//   tile's 32 scales follow the codes.
// FP8 and PAGED are template parameters so that the tile loop has no branches; a paged tile's
// table entry is read through the scalar cache, leaving the DMA in flight.
template <bool FP8, bool PAGED>
__global__ __launch_bounds__(kScoreWaves * 64) void index_scores_kernel(IndexScoreArgs a) {
  constexpr int NIH = 32, DI = 128, KS = DI / 16;
  constexpr int RB = FP8 ? DI : 2 * DI;        // bytes per key row
  constexpr int NDMA = 32 * RB / 1024;         // wave-wide 1 KB loads per tile (8 or 4)
  constexpr int SLOT = 32 * RB + (FP8 ? 256 : 0);
  constexpr int VPT = NDMA + (FP8 ? 1 : 0);    // vector memory operations per tile
  static_assert(VPT == 8 || VPT == 5, "vmcnt immediates");
  __shared__ int lhist[kHistBins];
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kScoreWaves][2][SLOT];
  // the row's q^I (32 heads x 128 fp32), head h's 16-byte chunk c at h*512 + ((c ^ h) << 4)
  __shared__ __attribute__((aligned(1024))) uint8_t q_s[NIH * DI * 4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g2 = lane >> 5, l32 = lane & 31;
  const int b = blockIdx.y;
  const RowMap rm = row_map(a.row0, a.rows_per_seq, b);
  const int t = min(min(a.n_vis[rm.seq] + a.vis_offset + rm.extra, a.T_cap), a.score_stride);
  const int tile0 = (int)((long long)blockIdx.x * a.row_tiles / a.n_chunks);
  const int tile1 = (int)((long long)(blockIdx.x + 1) * a.row_tiles / a.n_chunks);
  const int base = tile0 * 32;
  if (base >= t) return;
  const int end = min(tile1 * 32, t);
  for (int i = threadIdx.x; i < kHistBins; i += kScoreWaves * 64) lhist[i] = 0;
  const int n_tiles = cdiv(end - base, 32);
  const int nt_w = wave < n_tiles ? cdiv(n_tiles - wave, kScoreWaves) : 0;  // this wave's tiles
  // The wave's j-th tile into ring slot j & 1. Tiles past the chunk's last re-read it, and rows
  // past the end repeat the last valid one (their scores are not stored), so the loop needs no
  // branches.
  auto issue = [&](int j) __attribute__((always_inline)) {
    const int p0 = __builtin_amdgcn_readfirstlane(base + min(wave + kScoreWaves * j, n_tiles - 1) * 32);
    const int nval = min(32, end - p0);
    const size_t row0 = PAGED ? cache_row_uniform(a.pages, a.T_cap, rm.seq, p0) : (size_t)rm.seq * a.T_cap + p0;
    const uint8_t* src = (const uint8_t*)a.idx_k + row0 * RB;
    const uint32_t dst = lds_addr(ring[wave][j & 1]);
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      const int P = i * 64 + lane;  // 16-byte chunk of the slot this lane fills
      const int r = FP8 ? P >> 3 : P >> 4;
      const int c = FP8 ? ((P & 7) ^ ((r >> 1) & 7)) : ((P & 15) ^ (r & 15));
      lds_dma16_sbase((uint32_t)(min(r, nval - 1) * RB + c * 16), src, dst + i * 1024);
    }
    if constexpr (FP8)  // 32 scales; lanes 32-63 repeat them into the next 128 bytes
      lds_dma4_sbase((uint32_t)(min(l32, nval - 1) * 4), a.idx_scale + row0, dst + 32 * RB);
  };
  // The query is copied once per workgroup (each wave 2 KB of it), ahead of the first two tiles:
  // loaded by every lane straight from memory, it took 16 scattered 16-byte loads per lane, as
  // many bytes of L2 traffic as the keys, and the first tile waited for it.
  {
    const float* qbase = a.q_idx + (size_t)__builtin_amdgcn_readfirstlane(b) * NIH * DI;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int G = wave * 128 + i * 64 + lane, h = G >> 5, c = (G & 31) ^ h;
      lds_dma16_sbase((uint32_t)(h * 512 + c * 16), qbase, lds_addr(q_s) + wave * 2048 + i * 1024);
    }
  }
  issue(0);
  issue(1);
  // head weights of the 16 heads this lane's accumulators hold, (r/4)*8 + g2*4 + r%4, read through
  // the scalar cache (its wait leaves the copies in flight)
  float wgt[16];
  {
    f32x16 w0, w1;
    const float* wrow = a.w_idx + (size_t)__builtin_amdgcn_readfirstlane(b) * NIH;
    asm volatile("s_load_dwordx16 %0, %2, 0x0\n\ts_load_dwordx16 %1, %2, 0x40\n\ts_waitcnt lgkmcnt(0)"
                 : "=s"(w0), "=s"(w1) : "s"(wrow) : "memory");
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = (r >> 2) * 8 + (r & 3);  // head for g2 = 0; g2 = 1 takes i + 4
      const float lo = i < 16 ? w0[i] : w1[i - 16], hi = i + 4 < 16 ? w0[i + 4] : w1[i - 12];
      wgt[r] = (g2 ? hi : lo) * a.scale;
    }
  }
  // this wave's part of the query has landed (its two tiles stay in flight); the barrier then
  // covers every wave's part and the cleared histogram
  if constexpr (VPT == 8)
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
  __syncthreads();
  // A operand: q^I of this lane's head l32 as bf16 hi + lo pairs. k-step s takes, in lane group
  // g2, the features the B operand holds there: bf16 keys 16 s + 8 g2 + (0..7); FP8 keys, whose
  // 16-byte chunk 2 (s / 2) + g2 serves k-steps s and s + 1, 16 (2 (s / 2) + g2) + 8 (s % 2) + (0..7).
  u32x4 qa[KS], ql[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int c0 = (FP8 ? 16 * (2 * (s >> 1) + g2) + 8 * (s & 1) : 16 * s + 8 * g2) >> 2;
    float f[8];
    *(u32x4*)&f[0] = *(const u32x4*)(q_s + l32 * 512 + ((c0 ^ l32) << 4));
    *(u32x4*)&f[4] = *(const u32x4*)(q_s + l32 * 512 + (((c0 + 1) ^ l32) << 4));
    uint32_t h[4], l[4];
    split_bf16x8(f, h, l);
    qa[s] = u32x4{h[0], h[1], h[2], h[3]};
    ql[s] = u32x4{l[0], l[1], l[2], l[3]};
  }
  auto score = [&](int j, int slot) __attribute__((always_inline)) {
    const uint8_t* tile = ring[wave][slot];
    f32x16 acc = f32x16{};
    if constexpr (FP8) {
      const uint8_t* row = tile + l32 * RB;
      const int sw = (l32 >> 1) & 7;
      u32x4 kr[KS / 2];
#pragma unroll
      for (int s2 = 0; s2 < KS / 2; ++s2) kr[s2] = *(const u32x4*)(row + (((2 * s2 + g2) ^ sw) << 4));
#pragma unroll
      for (int s2 = 0; s2 < KS / 2; ++s2) {
        const u32x2 a0 = e4m3x4_to_bf16(kr[s2].x), a1 = e4m3x4_to_bf16(kr[s2].y);
        const u32x2 b0 = e4m3x4_to_bf16(kr[s2].z), b1 = e4m3x4_to_bf16(kr[s2].w);
        const u32x4 k0 = u32x4{a0.x, a0.y, a1.x, a1.y}, k1 = u32x4{b0.x, b0.y, b1.x, b1.y};
        acc = mfma32(qa[2 * s2], k0, acc);
        acc = mfma32(ql[2 * s2], k0, acc);
        acc = mfma32(qa[2 * s2 + 1], k1, acc);
        acc = mfma32(ql[2 * s2 + 1], k1, acc);
      }
    } else {
      const uint8_t* row = tile + l32 * RB;
      u32x4 kf[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) kf[s] = *(const u32x4*)(row + (((2 * s + g2) ^ (l32 & 15)) << 4));
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        acc = mfma32(qa[s], kf[s], acc);
        acc = mfma32(ql[s], kf[s], acc);
      }
    }
    float sc = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc += wgt[r] * fmaxf(acc[r], 0.f);
    sc += __shfl_xor(sc, 32, 64);
    if constexpr (FP8) sc *= *(const float*)(tile + 32 * RB + 4 * l32);
    const int pos = base + (wave + kScoreWaves * j) * 32 + l32;
    if (pos < end && g2 == 0) {
      a.scores[(size_t)b * a.score_stride + pos] = sc;
      atomicAdd(&lhist[order_key(sc) >> 20], 1);
    }
  };
  // steady state: wait for tile j (tile j + 1 stays in flight; a score store issued in between
  // is waited for too), score it, and refill its slot with tile j + 2
  for (int j = 0; j < nt_w; j += 2) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if constexpr (VPT == 8)
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
      score(j + i, i);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the slot's reads are done
      issue(j + i + 2);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no copy into LDS outlives the loop
  __syncthreads();
  // the row's histogram gathers the workgroup's nonzero bins
  int* gh = a.hist + (size_t)b * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += kScoreWaves * 64) {
    const int c = lhist[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

// Prefill rows of one sequence see nested prefixes of one index cache, so a workgroup takes 8
// consecutive rows (one per wave) and, in turn, four consecutive 128-position blocks of keys,
// each staged once in LDS for all of them (256-byte rows, 16-byte chunk c at c ^ (row & 15); FP8
// codes: 128-byte rows, chunk c at c ^ (row & 7), widened when read, and the block's scales);
// the rows' q^I is loaded once for the four blocks. Each wave scores its row's visible positions
// of a block as index_scores_kernel does; the top digits go to per-row LDS histograms of 8-bit
// counters (four bins per word: at most 128 per bin), added to the rows' histograms after each
// block. 66 KB of LDS: two workgroups per CU, so one's key loads and histogram flush overlap the
// other's scoring.
constexpr int kRowsPerWg = 8, kRowBlock = 128;
constexpr int kRowBlocksPerWg = 4;  // key blocks a workgroup takes in turn (its rows' q^I loaded once)

// at most 128 VGPRs, so that two 8-wave workgroups share a CU (four waves per SIMD)
// FP8 is a template parameter so that each form's registers fit the 128 without spills.
template <bool FP8>
__global__ __launch_bounds__(kRowsPerWg * 64) __attribute__((amdgpu_waves_per_eu(4))) void index_scores_rows_kernel(IndexScoreArgs a) {
  constexpr int NIH = 32, DI = 128, KS = DI / 16;
  __shared__ __attribute__((aligned(16))) uint8_t keys_s[kRowBlock * DI * 2];
  // per-row histograms with 8-bit counters, four bins per word (a block puts at most 128 keys in a
  // bin): with the 32 KB key block this leaves room for two workgroups per CU
  __shared__ uint32_t hist4[kRowsPerWg * kHistBins / 4];
  __shared__ float kscale_s[kRowBlock];
  // the rows' head weights times the score scale, read per tile (not held in registers)
  __shared__ __attribute__((aligned(16))) float wgt_s[kRowsPerWg][32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g2 = lane >> 5, l32 = lane & 31;
  auto visible = [&](int row) __attribute__((always_inline)) {
    const RowMap rm = row_map(a.row0, a.rows_per_seq, row);
    return min(min(a.n_vis[rm.seq] + a.vis_offset + rm.extra, a.T_cap), a.score_stride);
  };
  const int b = blockIdx.y * kRowsPerWg + wave;  // this wave's row
  const int b_last = min((int)blockIdx.y * kRowsPerWg + kRowsPerWg, a.B) - 1;
  const int seq = row_map(a.row0, a.rows_per_seq, b_last).seq;
  const int t_last = visible(b_last);  // the block's longest row
  const int base0 = blockIdx.x * kRowBlocksPerWg * kRowBlock;
  if (base0 >= t_last) return;
  const int t = b < a.B ? visible(b) : 0;
  constexpr bool fp8 = FP8;
  constexpr int NT = kRowsPerWg * 64;
  if (b < a.B && lane < 32) wgt_s[wave][lane] = a.w_idx[(size_t)b * NIH + lane] * a.scale;
  u32x4 qa[KS], ql[KS];  // q^I as bf16 hi + lo pairs, as in index_scores_kernel (loaded once)
  if (b < a.B) {
    const float* qrow = a.q_idx + ((size_t)b * NIH + l32) * DI;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      float f[8];
      *(u32x4*)&f[0] = ld16(qrow + s * 16 + g2 * 8);
      *(u32x4*)&f[4] = ld16(qrow + s * 16 + g2 * 8 + 4);
      uint32_t h[4], l[4];
      split_bf16x8(f, h, l);
      qa[s] = u32x4{h[0], h[1], h[2], h[3]};
      ql[s] = u32x4{l[0], l[1], l[2], l[3]};
    }
  }
#pragma unroll 1
  for (int blk = 0; blk < kRowBlocksPerWg; ++blk) {
    const int p0 = base0 + blk * kRowBlock;
    if (p0 >= t_last) break;
    for (int i = tid; i < kRowsPerWg * kHistBins / 4; i += NT) hist4[i] = 0;
    // the block's keys (positions past t_last repeat its last one; never scored)
    if constexpr (!fp8) {
      // copied straight into LDS (no registers next to the query): wave-wide 1 KB load i fills
      // slots 64 i .. 64 i + 63, slot P holding row P / 16's chunk (P % 16) ^ (row & 15)
      constexpr int LPW = kRowBlock * 256 / 1024 / kRowsPerWg;  // loads per wave
      // (lane through an opaque move: the per-lane addresses are formed per block, not hoisted
      // out of the block loop where they would hold registers next to the query)
      int ln;
      asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
#pragma unroll
      for (int k = 0; k < LPW; ++k) {
        const int i = wave * LPW + k, P = i * 64 + ln, r = P >> 4, c = (P & 15) ^ (r & 15);
        lds_dma16(a.idx_k + cache_row(a.pages, a.T_cap, seq, min(p0 + r, t_last - 1)) * DI + c * 8,
                  lds_addr(keys_s) + i * 1024);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's copies have landed
    } else {
      u32x4 v[kRowBlock * 8 / NT];
#pragma unroll
      for (int k = 0; k < kRowBlock * 8 / NT; ++k) {
        const int i = k * NT + tid, r = i >> 3, c = i & 7;
        v[k] = ld16((const uint8_t*)a.idx_k + cache_row(a.pages, a.T_cap, seq, min(p0 + r, t_last - 1)) * DI + c * 16);
      }
#pragma unroll
      for (int k = 0; k < kRowBlock * 8 / NT; ++k) {
        const int i = k * NT + tid, r = i >> 3, c = i & 7;
        st16(keys_s + r * 128 + ((c ^ (r & 7)) << 4), v[k]);
      }
      for (int i = tid; i < kRowBlock; i += NT)
        kscale_s[i] = a.idx_scale[cache_row(a.pages, a.T_cap, seq, min(p0 + i, t_last - 1))];
    }
    __syncthreads();  // keys staged, histograms cleared (and head weights staged)
    int l32o;  // l32 through an opaque move, for the same reason as ln above
    asm volatile("v_mov_b32 %0, %1" : "=v"(l32o) : "v"(l32));
    for (int j = 0; j < kRowBlock / 32 && p0 + 32 * j < t; ++j) {
      const int r = 32 * j + l32o;  // key row of this lane
      f32x16 acc = f32x16{};
      if constexpr (fp8) {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const u32x2 w = ld8(keys_s + r * 128 + ((s ^ (r & 7)) << 4) + g2 * 8);
          const u32x2 lo = e4m3x4_to_bf16(w.x), hi = e4m3x4_to_bf16(w.y);
          const u32x4 kv = u32x4{lo.x, lo.y, hi.x, hi.y};
          acc = mfma32(qa[s], kv, acc);
          acc = mfma32(ql[s], kv, acc);
        }
      } else {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const u32x4 kv = ld16(keys_s + r * 256 + (((2 * s + g2) ^ (r & 15)) << 4));
          acc = mfma32(qa[s], kv, acc);
          acc = mfma32(ql[s], kv, acc);
        }
      }
      // acc[4 qq + e] holds head 8 qq + 4 g2 + e
      float sc = 0.f;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const f32x4 wv = *(const f32x4*)&wgt_s[wave][8 * qq + 4 * g2];
#pragma unroll
        for (int e = 0; e < 4; ++e) sc += wv[e] * fmaxf(acc[4 * qq + e], 0.f);
      }
      sc += __shfl_xor(sc, 32, 64);
      if constexpr (fp8) sc *= kscale_s[r];
      const int pos = p0 + r;
      if (pos < t && g2 == 0) {
        a.scores[(size_t)b * a.score_stride + pos] = sc;
        const uint32_t bin = order_key(sc) >> 20;
        atomicAdd(&hist4[wave * (kHistBins / 4) + (bin >> 2)], 1u << (8 * (bin & 3)));
      }
    }
    __syncthreads();
    for (int i = tid; i < kRowsPerWg * kHistBins / 4; i += NT) {
      const uint32_t w = hist4[i];
      const int row = blockIdx.y * kRowsPerWg + i / (kHistBins / 4), bin = 4 * (i % (kHistBins / 4));
      if (w && row < a.B) {
        int* gh = a.hist + (size_t)row * kHistBins + bin;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if ((w >> (8 * e)) & 0xFFu) atomicAdd(gh + e, (int)((w >> (8 * e)) & 0xFFu));
      }
    }
    __syncthreads();  // the histograms and keys are reused by the next block
  }
}

__global__ void zero_words_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// The same clear in 16-byte stores over a grid-stride loop (p 16-byte aligned, n4 = words / 4):
// a decode's 8 row histograms take 32 workgroups instead of 128, a prefill chunk's 64 MB at most
// 1024 workgroups of whole-line stores.
__global__ void zero_words16_kernel(int4* p, int n4) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += gridDim.x * blockDim.x) p[i] = int4{0, 0, 0, 0};
}

// ------------------------------------------------------------------------------------------
// Top-k
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0) u = 0;  // -0.0 and +0.0 are the same score
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int NT>
__device__ int block_exclusive_scan(int v, int* tmp /* NT/64 + 1 ints */, int& total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  if (wave == 0) {  // the wave totals, scanned by the first NW lanes of wave 0
    const int c = lane < NW ? tmp[lane] : 0;
    int y = c;
#pragma unroll
    for (int o = 1; o < NW; o <<= 1) {
      const int z = __shfl_up(y, o, 64);
      if (lane >= o) y += z;
    }
    if (lane < NW) tmp[lane] = y - c;
    if (lane == NW - 1) tmp[NW] = y;
  }
  __syncthreads();
  const int r = tmp[wave] + x - v;
  total = tmp[NW];
  __syncthreads();
  return r;
}

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;

// number of lanes below this one with `pred` set, and the wave's total
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

constexpr int kTopkR = 65;                        // keys held per thread (one segment)
constexpr int kTopkSeg = kTopkR * kTopkThreads;    // 66,560 positions per segment

constexpr int kHistRep = 8;        // histogram replicas (lane % 8): at most 8 lanes per address
constexpr int kHistPitch = 4097;   // replica stride in words (not a multiple of the bank count)

// Positions past the row hold key 0. A real score never maps to a key below 2^20 (those are NaN
// bit patterns), so key 0 sits in digit-0 bin 0, under any threshold, and no pass needs a
// bounds test.
// The whole selection of row b inside one workgroup: the general path, for rows whose boundary
// bin holds more candidates than the chunked path keeps in LDS, or longer than it covers.
// hist: kHistRep * kHistPitch ints of LDS; scan_tmp: kTopkWaves + 1; shv: 3; wcnt: 2 * kTopkWaves.
// With from_hist the first digit's bin is read off the row histogram the score kernel left (it
// counts exactly the row's keys) instead of being counted again over the keys.
template <int NT>
__device__ __forceinline__ void boundary_bin(const int32_t* gh, int k, int* scan_tmp, int* shv);
template <int R = kTopkR>
__device__ __forceinline__ void topk_full_row(const TopkArgs& a, const int b, int* hist, int* scan_tmp,
                                           int* shv, int* wcnt_flat, bool from_hist = false) {
  constexpr int SEG = R * kTopkThreads;
  int& sh_bin = shv[0];
  int& sh_above = shv[1];
  int& sh_cnt = shv[2];
  int(*wcnt)[kTopkWaves] = (int(*)[kTopkWaves])wcnt_flat;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const RowMap rm = row_map(a.row0, a.rows_per_seq, b);
  const int t = min(a.n_vis[rm.seq] + a.vis_offset + rm.extra, a.score_stride);
  const int k = min(a.k, t);
  int32_t* out = a.out_idx + (size_t)b * a.out_stride;
  const float* sc = a.scores + (size_t)b * a.score_stride;
  if (t <= a.k) {  // short history: every visible position is kept
    for (int i = tid; i < a.k; i += kTopkThreads) out[i] = (i < t) ? i : -1;
    if (tid == 0) a.out_cnt[b] = t;
    return;
  }

  // Keys of segment sg: wave w owns positions sg*SEG + w*R*64 .. +R*64-1, its key u being
  // position ... + u*64 + lane (coalesced), all loads in flight at once. A row of one segment
  // (t <= SEG, 66,560 positions with R = 65) stays in registers for every pass.
  const int n_segs = cdiv(t, SEG);
  uint32_t keys[R];
  auto seg_base = [&](int sg) __attribute__((always_inline)) { return sg * SEG + wave * (R * 64); };
  auto load_seg = [&](int sg) __attribute__((always_inline)) {
    const int base = seg_base(sg);
    const float* p = sc + base + lane;
    const int lim = t - 1 - base - lane;  // u*64 <= lim <=> the position is visible
#pragma unroll
    for (int u = 0; u < R; ++u) keys[u] = __float_as_uint(p[min(u * 64, max(lim, 0))]);
#pragma unroll
    for (int u = 0; u < R; ++u) keys[u] = u * 64 <= lim ? order_key(__uint_as_float(keys[u])) : 0u;
  };
  load_seg(0);

  // ---- radix select over the keys: digits of 12, 12 and 8 bits from the top ----
  uint32_t prefix = 0, pmask = 0;
  int krem = k;
  bool whole_bin = false;  // the last decided bin is taken entirely
  int* my_hist = hist + (lane & (kHistRep - 1)) * kHistPitch;
  int level0 = 0;
  if (from_hist) {
    boundary_bin<kTopkThreads>(a.hist + (size_t)b * kHistBins, k, scan_tmp, shv);
    prefix = (uint32_t)sh_bin << 20;
    pmask = 0xFFF00000u;
    krem -= sh_above;
    whole_bin = sh_cnt == krem;
    level0 = 1;
    __syncthreads();
  }
#pragma unroll 1
  for (int level = level0; level < 3 && !whole_bin; ++level) {
    const int shift = level == 0 ? 20 : (level == 1 ? 8 : 0);
    const int nbins = level == 2 ? 256 : 4096;
    for (int i = tid; i < kHistRep * kHistPitch; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
#pragma unroll 1
    for (int sg = 0; sg < n_segs; ++sg) {
      if (n_segs > 1) load_seg(sg);
#pragma unroll
      for (int u = 0; u < R; ++u)
        if ((keys[u] & pmask) == prefix) atomicAdd(&my_hist[(keys[u] >> shift) & (uint32_t)(nbins - 1)], 1);
    }
    __syncthreads();
    // the bin where the count from the top reaches krem: thread j owns bins nbins-1-4j .. -3
    constexpr int PER = 4096 / kTopkThreads;
    int cntb[PER];
    int local = 0;
    const int top = nbins - 1 - PER * tid;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      cntb[q] = 0;
      if (top - q >= 0)
#pragma unroll
        for (int r = 0; r < kHistRep; ++r) cntb[q] += hist[r * kHistPitch + top - q];
      local += cntb[q];
    }
    int total;
    const int before = block_exclusive_scan<kTopkThreads>(local, scan_tmp, total);
    if (before < krem && before + local >= krem) {
      int cum = before;
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        if (cum < krem && cum + cntb[q] >= krem) {
          sh_bin = top - q;
          sh_above = cum;
          sh_cnt = cntb[q];
        }
        cum += cntb[q];
      }
    }
    __syncthreads();
    prefix |= (uint32_t)sh_bin << shift;
    pmask |= (uint32_t)(nbins - 1) << shift;
    krem -= sh_above;
    const int cnt = sh_cnt;
    __syncthreads();
    if (cnt == krem) {
      whole_bin = true;
      break;
    }
  }
  // kept: key > thr, plus (all 32 bits decided, tau = prefix) the krem lowest-position copies
  // of tau. A whole bin taken is key >= prefix (its undecided low bits are zero): thr = prefix-1.
  const uint32_t tau = prefix;
  const uint32_t thr = whole_bin ? prefix - 1u : tau;
  if (whole_bin) krem = 0;
  auto kept_gt = [&](uint32_t key) __attribute__((always_inline)) { return key > thr; };

  // ---- ordered compaction: wave w owns a contiguous run of each segment ----
  int out_base = 0, eq_base = 0;
#pragma unroll 1
  for (int sg = 0; sg < n_segs; ++sg) {
    if (n_segs > 1) load_seg(sg);
    int nk = 0, ne = 0;
#pragma unroll
    for (int u = 0; u < R; ++u) {
      nk += (int)__popcll(__ballot(kept_gt(keys[u])));
      ne += (int)__popcll(__ballot(!whole_bin && keys[u] == tau));
    }
    if (lane == 0) {
      wcnt[0][wave] = nk;
      wcnt[1][wave] = ne;
    }
    // recompute the predicates in the writing pass rather than keep 2 x 65 of them live
#pragma unroll
    for (int u = 0; u < R; ++u) asm volatile("" : "+v"(keys[u]));
    __syncthreads();
    int eq_before = eq_base, out_before = out_base, seg_keep = 0, seg_eq = 0;
    for (int w = 0; w < kTopkWaves; ++w) {
      const int take = max(0, min(krem - (eq_base + seg_eq), wcnt[1][w]));
      if (w < wave) {
        eq_before += wcnt[1][w];
        out_before += wcnt[0][w] + take;
      }
      seg_keep += wcnt[0][w] + take;
      seg_eq += wcnt[1][w];
    }
    const int take_w = max(0, min(krem - eq_before, ne));  // copies of tau this wave keeps
    int wpos = out_before, eq_seen = 0;
    const int base = seg_base(sg);
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const bool eq = !whole_bin && keys[u] == tau;
      const uint64_t em = __ballot(eq);
      const bool keep = kept_gt(keys[u]) || (eq && eq_seen + lanes_below(em) < take_w);
      const uint64_t km = __ballot(keep);
      const int w = wpos + lanes_below(km);
      if (keep && w < a.k) out[w] = base + u * 64 + lane;
#ifdef GMLA_DEBUG_CHECKS
      if (keep && w >= k) atomicOr(&g_debug_flags_topk, kDbgTopkOffset);
#endif
      wpos += (int)__popcll(km);
      eq_seen += (int)__popcll(em);
    }
    out_base += seg_keep;
    eq_base += seg_eq;
    __syncthreads();
  }
  for (int i = k + tid; i < a.k; i += kTopkThreads) out[i] = -1;
  if (tid == 0) a.out_cnt[b] = k;
}


// ---- chunked path ----
// The score kernel leaves each row's histogram of the 12-bit top digit. Every 2048-position
// chunk (topk_count_kernel) finds the bin b0 where the count from the top reaches k, counts its
// keys above b0 and appends the keys of b0 (with their positions) to the row's candidate list.
// The select (row_threshold) radix-selects among the candidates in LDS the threshold key thr
// (the krem-th largest, krem = k minus the count above b0) and, when only some of its copies
// are kept, the last kept position p_lim (the copies' positions radix-selected in turn).
// A position is kept iff key > thr, or key == thr and position <= p_lim.
// It also counts the kept positions of every 2048-position chunk; their exclusive scan is each
// chunk's output offset, and each chunk's kept positions are written in order at that offset,
// so the output is ascending.
constexpr int kChunk = 2048;        // positions per compaction workgroup
constexpr int kMaxChunks = 1024;    // the chunked path covers rows of up to 2,097,152 positions
constexpr int kCandCap = 8192;      // boundary-bin keys held in LDS
enum { kSelDone = 0, kSelChunked = 1 };
constexpr int kSelLds = kHistRep * kHistPitch * 4 > kCandCap * 12 + kHistBins * 4
                            ? kHistRep * kHistPitch * 4 : kCandCap * 12 + kHistBins * 4;

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}
// sum over the workgroup (kTopkThreads); tmp: kTopkWaves ints of LDS, free on entry
__device__ __forceinline__ int block_sum_int(int v, int* tmp) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = v;
  __syncthreads();
  int s = 0;
  for (int w = 0; w < kTopkWaves; ++w) s += tmp[w];
  __syncthreads();
  return s;
}

// The r-th largest (1 <= r <= n) of the 32-bit values vals[0, n) in LDS, for the whole
// workgroup: radix levels of 12, 12 and 8 bits from the top over an LDS histogram of 4096 ints,
// ending early when the r-th lands on a bin that is taken whole (then the answer is that bin's
// smallest value). *n_gt receives the count of values above it, *n_eq the count equal to it.
// With first_level = 1 every value is known to have the top 12 bits top12, and level 0 is
// skipped.
__device__ __forceinline__ uint32_t block_select_desc(const uint32_t* vals, int n, int r, int* hist,
                                                      int* scan_tmp, int* shv, int* n_gt, int* n_eq,
                                                      int first_level = 0, uint32_t top12 = 0) {
  const int tid = threadIdx.x;
  uint32_t prefix = first_level ? top12 << 20 : 0u, pmask = first_level ? 0xFFF00000u : 0u;
  int gt = 0, eq = n;
#pragma unroll 1
  for (int level = first_level; level < 3; ++level) {
    const int shift = level == 0 ? 20 : (level == 1 ? 8 : 0);
    const int nbins = level == 2 ? 256 : 4096;
    for (int i = tid; i < kHistBins; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kTopkThreads) {
      const uint32_t v = vals[i];
      if ((v & pmask) == prefix) atomicAdd(&hist[(v >> shift) & (uint32_t)(nbins - 1)], 1);
    }
    __syncthreads();
    constexpr int PER = kHistBins / kTopkThreads;
    const int top = nbins - 1 - PER * tid;
    int cntb[PER];
    int local = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      cntb[q] = top - q >= 0 ? hist[top - q] : 0;
      local += cntb[q];
    }
    int total;
    const int before = block_exclusive_scan<kTopkThreads>(local, scan_tmp, total);
    const int rr = r - gt;
    if (before < rr && before + local >= rr) {
      int cum = before;
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        if (cum < rr && cum + cntb[q] >= rr) {
          shv[0] = top - q;
          shv[1] = cum;
          shv[2] = cntb[q];
        }
        cum += cntb[q];
      }
    }
    __syncthreads();
    prefix |= (uint32_t)shv[0] << shift;
    pmask |= (uint32_t)(nbins - 1) << shift;
    gt += shv[1];
    eq = shv[2];
    const bool whole = rr - shv[1] == shv[2] && level < 2;  // the bin's values are all taken
    __syncthreads();
    if (whole) {  // every value of the bin is taken: its smallest one is the answer
      uint32_t lo = 0xFFFFFFFFu;
      for (int i = tid; i < n; i += kTopkThreads) {
        const uint32_t v = vals[i];
        if ((v & pmask) == prefix) lo = min(lo, v);
      }
      lo = wave_min_u32(lo);
      if ((tid & 63) == 0) scan_tmp[tid >> 6] = (int)lo;
      __syncthreads();
      lo = 0xFFFFFFFFu;
      for (int w = 0; w < kTopkWaves; ++w) lo = min(lo, (uint32_t)scan_tmp[w]);
      int c_lo = 0;  // copies of the bin's smallest value: it is taken entirely, so e == keep
      for (int i = tid; i < n; i += kTopkThreads) c_lo += vals[i] == lo;
      __syncthreads();
      c_lo = block_sum_int(c_lo, scan_tmp);
      *n_gt = gt + eq - c_lo;
      *n_eq = c_lo;
      return lo;
    }
  }
  *n_gt = gt;
  *n_eq = eq;
  return prefix;
}

// The bin of the row histogram gh where the count from the top reaches k (k <= the row's
// count): shv[0] = bin, shv[1] = count above it, shv[2] = its count. Thread j of NT owns bins
// 4095 - PER j .. -PER+1. Ends with a barrier.
template <int NT>
__device__ __forceinline__ void boundary_bin(const int32_t* gh, int k, int* scan_tmp, int* shv) {
  constexpr int PER = kHistBins / NT;
  const int top = kHistBins - 1 - PER * (int)threadIdx.x;
  int cntb[PER];
  int local = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    cntb[q] = gh[top - q];
    local += cntb[q];
  }
  int total;
  const int before = block_exclusive_scan<NT>(local, scan_tmp, total);
  if (before < k && before + local >= k) {
    int cum = before;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      if (cum < k && cum + cntb[q] >= k) {
        shv[0] = top - q;
        shv[1] = cum;
        shv[2] = cntb[q];
      }
      cum += cntb[q];
    }
  }
  __syncthreads();
}

// grid (chunks, B), 256 threads: per chunk, the count of keys above the boundary bin, and the
// boundary bin's keys and positions (in position order) in the chunk's own candidate slot. The
// first chunk's workgroup also records the boundary bin for the select.
__global__ __launch_bounds__(256) void topk_count_kernel(TopkArgs a) {
  __shared__ int scan_tmp[256 / 64 + 1];
  __shared__ int shv[4];
  __shared__ int wa[4], wn[4];
  const int b = blockIdx.y, c = blockIdx.x;
  const RowMap rm = row_map(a.row0, a.rows_per_seq, b);
  const int t = min(a.n_vis[rm.seq] + a.vis_offset + rm.extra, a.score_stride);
  if (t <= a.k || c * kChunk >= t) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* sc = a.scores + (size_t)b * a.score_stride;
  const int base = c * kChunk + wave * (kChunk / 4);
  constexpr int R = kChunk / 4 / 64;
  uint32_t kv[R];  // the chunk's scores, loaded while the boundary bin is found
#pragma unroll
  for (int r = 0; r < R; ++r) kv[r] = __float_as_uint(sc[min(base + r * 64 + lane, t - 1)]);
  boundary_bin<256>(a.hist + (size_t)b * kHistBins, a.k, scan_tmp, shv);
  int32_t* info = a.info + (size_t)b * 4;
  if (c == 0 && threadIdx.x == 0) {
    info[0] = shv[0];
    info[1] = shv[1];
    info[2] = shv[2];
  }
  if (shv[2] > kCandCap) return;  // the select takes the whole row
  const uint32_t b0 = (uint32_t)shv[0];
#pragma unroll
  for (int r = 0; r < R; ++r) kv[r] = base + r * 64 + lane < t ? order_key(__uint_as_float(kv[r])) : 0u;
  int above = 0, nc = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    above += (int)__popcll(__ballot((kv[r] >> 20) > b0));
    nc += (int)__popcll(__ballot((kv[r] >> 20) == b0));
  }
  if (lane == 0) {
    wa[wave] = above;
    wn[wave] = nc;
  }
  __syncthreads();
  if (nc) {
    int cb = 0;
    for (int i = 0; i < wave; ++i) cb += wn[i];
    uint32_t* ck = a.cand + ((size_t)b * a.off_stride + c) * 2 * kChunk;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const bool is_c = (kv[r] >> 20) == b0;
      const uint64_t cm = __ballot(is_c);
      const int ci = cb + lanes_below(cm);
      if (is_c) {
        ck[ci] = kv[r];
        ck[kChunk + ci] = (uint32_t)(base + r * 64 + lane);
      }
      cb += (int)__popcll(cm);
    }
  }
  if (threadIdx.x == 0) {
    a.above[(size_t)b * a.off_stride + c] = wa[0] + wa[1] + wa[2] + wa[3];
    a.ncand[(size_t)b * a.off_stride + c] = wn[0] + wn[1] + wn[2] + wn[3];
  }
}

// LDS of the select: the whole-row selection's histograms, or the candidates and their
// selection histograms; per-chunk counts.
struct SelLds {
  __attribute__((aligned(16))) uint8_t big[kSelLds];
  int scan_tmp[kTopkWaves + 1];
  int shv[4];
  int wcnt[2 * kTopkWaves];
  int ccnt[kMaxChunks];
};

// The threshold of row b (t > k visible positions, nch chunks, boundary bin holding at most
// kCandCap keys): thr, the krem-th largest candidate key (krem = k minus the keys above the
// boundary bin), and p_lim, the last kept position among thr's copies when only some are kept.
// Leaves in L.ccnt[c] the kept positions of every chunk c < nch. Ends with a barrier.
__device__ __forceinline__ void row_threshold(const TopkArgs& a, int b, int k, int nch, SelLds& L,
                                              uint32_t& thr_out, int& p_lim_out) {
  static_assert(kMaxChunks == kTopkThreads, "one chunk per thread");
  const int tid = threadIdx.x, lane = tid & 63;
  const int32_t* info = a.info + (size_t)b * 4;
  const uint32_t b0 = (uint32_t)info[0];
  const int krem = k - info[1];
  const size_t slot0 = (size_t)b * a.off_stride;
  const int my_nc = tid < nch ? a.ncand[slot0 + tid] : 0;
  const int my_above = tid < nch ? a.above[slot0 + tid] : 0;
  uint32_t* ckey = (uint32_t*)L.big;          // [kCandCap]
  int* cpos = (int*)(ckey + kCandCap);        // [kCandCap]
  int* lh = cpos + kCandCap;                  // [kHistBins] histogram of the candidate selections
  uint32_t* tv = (uint32_t*)(lh + kHistBins); // [kCandCap] ~position of each copy of thr
  // the chunks' candidate lists, concatenated in LDS: candidate i belongs to the last chunk whose
  // offset is at most i (found by bisection), so every load is in flight at once
  int ntot;
  const int cpre = block_exclusive_scan<kTopkThreads>(my_nc, L.scan_tmp, ntot);
  L.ccnt[tid] = cpre;
  __syncthreads();
  const int n = min(ntot, kCandCap);
  const int top_step = nch > 1 ? 1 << (31 - __builtin_clz(nch - 1)) : 0;  // bisection over nch
#pragma unroll 1
  for (int i0 = 0; i0 < n; i0 += 2 * kTopkThreads) {  // two candidates per thread in flight
    uint32_t kv[2], pv[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = i0 + tid + u * kTopkThreads;
      if (i < n) {
        int lo = 0;  // L.ccnt[lo] <= i
        for (int step = top_step; step >= 1; step >>= 1)
          if (lo + step < nch && L.ccnt[lo + step] <= i) lo += step;
        const uint32_t* gk = a.cand + (slot0 + lo) * 2 * kChunk + (i - L.ccnt[lo]);
        kv[u] = gk[0];
        pv[u] = gk[kChunk];
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = i0 + tid + u * kTopkThreads;
      if (i < n) {
        ckey[i] = kv[u];
        cpos[i] = (int)pv[u];
      }
    }
  }
  __syncthreads();
  L.ccnt[tid] = my_above;
  __syncthreads();
  // ---- thr = the krem-th largest candidate key; of its e copies the keep lowest positions stay ----
  int n_gt, e;
  const uint32_t thr = block_select_desc(ckey, n, krem, lh, L.scan_tmp, L.shv, &n_gt, &e, 1, b0);
  const int keep = krem - n_gt;  // 1 <= keep <= e
  int p_lim = 0x7FFFFFFF;
  if (keep < e) {
    if (tid == 0) L.shv[3] = 0;
    __syncthreads();
    for (int i0 = 0; i0 < n; i0 += kTopkThreads) {
      const int i = i0 + tid;
      const bool is_t = i < n && ckey[i] == thr;
      const uint64_t m = __ballot(is_t);
      if (m) {
        int cb = 0;
        if (lane == 0) cb = atomicAdd(&L.shv[3], (int)__popcll(m));
        cb = __shfl(cb, 0, 64);
        if (is_t) tv[cb + lanes_below(m)] = ~(uint32_t)cpos[i];
      }
    }
    __syncthreads();
    int g2, e2;
    p_lim = (int)~block_select_desc(tv, min(L.shv[3], kCandCap), keep, lh, L.scan_tmp, L.shv, &g2, &e2);
  }
  // ---- kept candidates per chunk ----
  for (int i = tid; i < n; i += kTopkThreads) {
    const uint32_t key = ckey[i];
    const unsigned ch = (unsigned)cpos[i] / kChunk;  // < nch for every listed candidate
    if ((key > thr || (key == thr && cpos[i] <= p_lim)) && ch < (unsigned)nch) atomicAdd(&L.ccnt[ch], 1);
  }
  __syncthreads();
  thr_out = thr;
  p_lim_out = p_lim;
}

// One workgroup per row: the row's threshold, and the chunks' output offsets for
// topk_compact_kernel (rows whose boundary bin is too large for LDS: the whole selection).
__global__ __launch_bounds__(kTopkThreads) void topk_select_kernel(TopkArgs a) {
  __shared__ SelLds L;
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const RowMap rm = row_map(a.row0, a.rows_per_seq, b);
  const int t = min(a.n_vis[rm.seq] + a.vis_offset + rm.extra, a.score_stride);
  const int k = min(a.k, t);
  int32_t* sel = a.sel + (size_t)b * 4;
  int32_t* out = a.out_idx + (size_t)b * a.out_stride;
  if (t <= a.k) {  // short history: every visible position is kept
    for (int i = tid; i < a.k; i += kTopkThreads) out[i] = (i < t) ? i : -1;
    if (tid == 0) {
      a.out_cnt[b] = t;
      sel[0] = kSelDone;
    }
    return;
  }
  const int nch = cdiv(t, kChunk);
  if (a.info[(size_t)b * 4 + 2] > kCandCap || nch > kMaxChunks) {
    topk_full_row(a, b, (int*)L.big, L.scan_tmp, L.shv, L.wcnt);
    if (tid == 0) sel[0] = kSelDone;
    return;
  }
  uint32_t thr;
  int p_lim;
  row_threshold(a, b, k, nch, L, thr, p_lim);
  int tot;
  const int ex = block_exclusive_scan<kTopkThreads>(tid < nch ? L.ccnt[tid] : 0, L.scan_tmp, tot);
  if (tid < nch) a.off[(size_t)b * a.off_stride + tid] = ex;
  for (int i = k + tid; i < a.k; i += kTopkThreads) out[i] = -1;
  if (tid == 0) {
    a.out_cnt[b] = k;
    sel[1] = (int32_t)thr;
    sel[2] = p_lim;
    sel[3] = nch;
    sel[0] = kSelChunked;
  }
}

// grid (cdiv(chunks, cpw), B), kTopkThreads threads: the select of topk_select_kernel, done by
// every workgroup of the row, followed by the compaction of the workgroup's cpw chunks (wave w
// writes the kept positions of chunk positions [128 w, 128 w + 128) in order, after those of
// the waves before it). One launch instead of two for rows spread over few workgroups; the
// workgroup's scores are loaded before the select, which hides their latency.
constexpr int kFuseMaxCpw = 4;
__global__ __launch_bounds__(kTopkThreads) void topk_select_compact_kernel(TopkArgs a) {
  __shared__ SelLds L;
  __shared__ int wc[kTopkWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.y, g = blockIdx.x;
  const RowMap rm = row_map(a.row0, a.rows_per_seq, b);
  const int t = min(a.n_vis[rm.seq] + a.vis_offset + rm.extra, a.score_stride);
  const int k = min(a.k, t);
  const int nch = cdiv(t, kChunk);
  const int c_lo = g * a.cpw, c_hi = min(nch, c_lo + a.cpw);
  int32_t* out = a.out_idx + (size_t)b * a.out_stride;
  if (t <= a.k) {  // short history: every visible position is kept
    if (g == 0) {
      for (int i = tid; i < a.k; i += kTopkThreads) out[i] = (i < t) ? i : -1;
      if (tid == 0) a.out_cnt[b] = t;
    }
    return;
  }
  if (c_lo >= nch && g != 0) return;
  constexpr int RW = kChunk / kTopkWaves / 64;  // positions per lane per chunk
  const float* sc = a.scores + (size_t)b * a.score_stride;
  float sv[kFuseMaxCpw][RW];
#pragma unroll
  for (int j = 0; j < kFuseMaxCpw; ++j)
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int p = (c_lo + j) * kChunk + wave * (kChunk / kTopkWaves) + r * 64 + lane;
      sv[j][r] = j < a.cpw && p < t ? sc[p] : 0.f;
    }
  if (a.info[(size_t)b * 4 + 2] > kCandCap || nch > kMaxChunks) {
    if (g == 0) topk_full_row(a, b, (int*)L.big, L.scan_tmp, L.shv, L.wcnt);
    return;
  }
  uint32_t thr;
  int p_lim;
  row_threshold(a, b, k, nch, L, thr, p_lim);
  int tot;
  const int ex = block_exclusive_scan<kTopkThreads>(tid < nch ? L.ccnt[tid] : 0, L.scan_tmp, tot);
  if (tid < nch) L.ccnt[tid] = ex;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kFuseMaxCpw; ++j) {
    const int c = c_lo + j;
    if (c >= c_hi) break;
    const int base = c * kChunk + wave * (kChunk / kTopkWaves);
    uint64_t km[RW];
    int n = 0;
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int p = base + r * 64 + lane;
      const uint32_t key = p < t ? order_key(sv[j][r]) : 0u;
      km[r] = __ballot(key > thr || (key == thr && p <= p_lim));
      n += (int)__popcll(km[r]);
    }
    if (lane == 0) wc[wave] = n;
    __syncthreads();
    int w = L.ccnt[c];
    for (int i = 0; i < wave; ++i) w += wc[i];
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int o = w + lanes_below(km[r]);
      if (((km[r] >> lane) & 1) && o < k) out[o] = base + r * 64 + lane;
#ifdef GMLA_DEBUG_CHECKS
      if (((km[r] >> lane) & 1) && o >= k) atomicOr(&g_debug_flags_topk, kDbgTopkOffset);
#endif
      w += (int)__popcll(km[r]);
    }
    __syncthreads();
  }
  if (g == 0) {
    for (int i = k + tid; i < a.k; i += kTopkThreads) out[i] = -1;
    if (tid == 0) a.out_cnt[b] = k;
  }
}

// One workgroup per row, for rows of at most R * kTopkThreads positions: the whole selection with
// the row's keys in registers and the first digit's bin read off the score kernel's histogram, so
// that nothing passes through memory between the score kernel and the output.
template <int R>
__global__ __launch_bounds__(kTopkThreads) void topk_row_kernel(TopkArgs a) {
  __shared__ int hist[kHistRep * kHistPitch];
  __shared__ int scan_tmp[kTopkWaves + 1];
  __shared__ int shv[4];
  __shared__ int wcnt[2 * kTopkWaves];
  topk_full_row<R>(a, blockIdx.x, hist, scan_tmp, shv, wcnt, true);
}

// grid (chunks, B), 256 threads: wave w writes the kept positions of chunk positions
// [512 w, 512 w + 512) in order, after those of the waves before it
__global__ __launch_bounds__(256) void topk_compact_kernel(TopkArgs a) {
  __shared__ int wc[4];
  const int b = blockIdx.y, c = blockIdx.x;
  const int32_t* sel = a.sel + (size_t)b * 4;
  if (sel[0] != kSelChunked || c >= sel[3]) return;
  const uint32_t thr = (uint32_t)sel[1];
  const int p_lim = sel[2];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const RowMap rm = row_map(a.row0, a.rows_per_seq, b);
  const int t = min(a.n_vis[rm.seq] + a.vis_offset + rm.extra, a.score_stride);
  const float* sc = a.scores + (size_t)b * a.score_stride;
  const int base = c * kChunk + wave * (kChunk / 4);
  constexpr int R = kChunk / 4 / 64;
  uint64_t km[R];
  int n = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int p = base + r * 64 + lane;
    const uint32_t key = p < t ? order_key(sc[p]) : 0u;
    km[r] = __ballot(key > thr || (key == thr && p <= p_lim));
    n += (int)__popcll(km[r]);
  }
  if (lane == 0) wc[wave] = n;
  __syncthreads();
  int w = a.off[(size_t)b * a.off_stride + c];
  for (int i = 0; i < wave; ++i) w += wc[i];
  int32_t* out = a.out_idx + (size_t)b * a.out_stride;
  const int kk = min(a.k, t);  // the kept total (guards the writes should the counts disagree)
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int o = w + lanes_below(km[r]);
    if (((km[r] >> lane) & 1) && o < kk) out[o] = base + r * 64 + lane;
#ifdef GMLA_DEBUG_CHECKS
    if (((km[r] >> lane) & 1) && o >= kk) atomicOr(&g_debug_flags_topk, kDbgTopkOffset);
#endif
    w += (int)__popcll(km[r]);
  }
}

// ------------------------------------------------------------------------------------------
// Expanded-cache decode attention
// ------------------------------------------------------------------------------------------
template <class S>
__global__ __launch_bounds__(256) void expanded_attn_kernel(ExpandedAttnArgs a) {
  constexpr int H = S::H, DQK = S::DN + S::DS, DV = S::DV, DQ4 = DQK / 4;
  static_assert(DQK % 4 == 0, "quarters");
  __shared__ float ms[4], lsum[4];
  __shared__ float os[4][DV];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kq = lane & 3, kk = lane >> 2;
  const int bh = blockIdx.x, b = bh / H, h = bh % H;
  const int n = min(a.n_vis[b] + a.vis_offset, a.T_cap);
  float qv[DQ4];
  const uint16_t* qrow = a.q + ((size_t)b * H + h) * DQK + kq * DQ4;
#pragma unroll
  for (int i = 0; i < DQ4; ++i) qv[i] = bf16_bits_to_f32(qrow[i]);
  const uint16_t* kb = a.k + (size_t)bh * a.T_cap * DQK;
  const uint16_t* vb = a.v + (size_t)bh * a.T_cap * DV;
  const float sl2 = a.scale * 1.4426950408889634f;
  constexpr int NV = cdiv(DV, 128);  // value pairs per lane
  float m_run = -INFINITY, l_run = 0.f, o[NV][2];
#pragma unroll
  for (int i = 0; i < NV; ++i) o[i][0] = o[i][1] = 0.f;
  for (int base = wave * 16; base < n; base += 64) {
    const int j = base + kk;
    float s = 0.f;
    if (j < n) {
      const uint16_t* kr = kb + (size_t)j * DQK + kq * DQ4;
      if constexpr (DQ4 % 8 == 0) {
#pragma unroll
        for (int c = 0; c < DQ4; c += 8) {
          const u32x4 w = ld16(kr + c);
          s += qv[c + 0] * lo_bf16(w.x) + qv[c + 1] * hi_bf16(w.x) + qv[c + 2] * lo_bf16(w.y) +
               qv[c + 3] * hi_bf16(w.y) + qv[c + 4] * lo_bf16(w.z) + qv[c + 5] * hi_bf16(w.z) +
               qv[c + 6] * lo_bf16(w.w) + qv[c + 7] * hi_bf16(w.w);
        }
      } else {
#pragma unroll
        for (int c = 0; c < DQ4; ++c) s += qv[c] * bf16_bits_to_f32(kr[c]);
      }
    }
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    s = (j < n) ? s * sl2 : -INFINITY;
    float mt = s;
#pragma unroll
    for (int off = 4; off < 64; off <<= 1) mt = fmaxf(mt, __shfl_xor(mt, off, 64));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = fast_exp2(m_run - m_new);
    const float p = fast_exp2(s - m_new);
    float ps = (kq == 0) ? p : 0.f;
    ps = wave_sum(ps);
    l_run = l_run * alpha + ps;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      o[i][0] *= alpha;
      o[i][1] *= alpha;
    }
#pragma unroll 4
    for (int k2 = 0; k2 < 16; ++k2) {
      const float pj = __shfl(p, k2 * 4, 64);
      const int j2 = base + k2;
      if (j2 < n) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          const int dv = 2 * lane + 128 * i;
          if (dv < DV) {
            const uint32_t w = *(const uint32_t*)(vb + (size_t)j2 * DV + dv);
            o[i][0] += pj * lo_bf16(w);
            o[i][1] += pj * hi_bf16(w);
          }
        }
      }
    }
  }
  if (lane == 0) {
    ms[wave] = m_run;
    lsum[wave] = l_run;
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int dv = 2 * lane + 128 * i;
    if (dv < DV) {
      os[wave][dv] = o[i][0];
      os[wave][dv + 1] = o[i][1];
    }
  }
  __syncthreads();
  float M = -INFINITY;
  for (int w = 0; w < 4; ++w) M = fmaxf(M, ms[w]);
  float den = 0.f, f[4];
  for (int w = 0; w < 4; ++w) {
    f[w] = (ms[w] == -INFINITY) ? 0.f : fast_exp2(ms[w] - M);
    den += f[w] * lsum[w];
  }
  for (int d = threadIdx.x; d < DV; d += 256) {
    float acc = 0.f;
    for (int w = 0; w < 4; ++w) acc += f[w] * os[w][d];
    a.z[(size_t)bh * DV + d] = den > 0.f ? acc / den : 0.f;
  }
  if (threadIdx.x == 0 && a.lse) a.lse[bh] = (M + __log2f(den)) * 0.6931471805599453f;
}

// u[i] = z[i] * sigmoid(g_pre[i]) over B*H*DV elements (z and g_pre f32; g_pre may be null).
// The K3 shape (192-wide keys, 128-wide values) with the next 16-key step's K and V loaded while
// the current one is scored: both loads of a step are issued together, a step ahead, into
// registers (two buffers), so a step waits on neither. Lanes as in expanded_attn_kernel: key
// base + lane/4, feature quarter lane%4 of the key; value features 2 lane, 2 lane + 1. The two
// buffers take the kernel to ~200 VGPRs, two workgroups per CU: the 3072 (b, h) workgroups of
// B = 32 run in six whole rounds.
__global__ __launch_bounds__(256) void expanded_attn_k3_kernel(ExpandedAttnArgs a) {
  constexpr int H = ShapeK3::H, DQK = 192, DV = 128, DQ4 = DQK / 4, KC = DQ4 / 8;
  __shared__ float ms[4], lsum[4];
  __shared__ float os[4][DV];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kq = lane & 3, kk = lane >> 2;
  const int bh = blockIdx.x, b = bh / H, h = bh % H;
  const int n = min(a.n_vis[b] + a.vis_offset, a.T_cap);
  float qv[DQ4];
  {
    const uint16_t* qrow = a.q + ((size_t)b * H + h) * DQK + kq * DQ4;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const u32x4 w = ld16(qrow + 8 * c);
      qv[8 * c + 0] = lo_bf16(w.x); qv[8 * c + 1] = hi_bf16(w.x);
      qv[8 * c + 2] = lo_bf16(w.y); qv[8 * c + 3] = hi_bf16(w.y);
      qv[8 * c + 4] = lo_bf16(w.z); qv[8 * c + 5] = hi_bf16(w.z);
      qv[8 * c + 6] = lo_bf16(w.w); qv[8 * c + 7] = hi_bf16(w.w);
    }
  }
  const uint16_t* kb = a.k + (size_t)bh * a.T_cap * DQK;
  const uint16_t* vb = a.v + (size_t)bh * a.T_cap * DV;
  const float sl2 = a.scale * 1.4426950408889634f;
  float m_run = -INFINITY, l_run = 0.f, o0 = 0.f, o1 = 0.f;
  u32x4 kf[2][KC];
  uint32_t vf[2][16];
  // keys past the last visible one re-read it (their scores are -inf, their values unused)
  auto load = [&](int base, u32x4* k, uint32_t* v) __attribute__((always_inline)) {
    const uint16_t* kr = kb + (size_t)min(base + kk, n - 1) * DQK + kq * DQ4;
#pragma unroll
    for (int c = 0; c < KC; ++c) k[c] = ld16(kr + 8 * c);
#pragma unroll
    for (int k2 = 0; k2 < 16; ++k2) v[k2] = *(const uint32_t*)(vb + (size_t)min(base + k2, n - 1) * DV + 2 * lane);
  };
  auto step = [&](int base, const u32x4* k, const uint32_t* v) __attribute__((always_inline)) {
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < KC; ++c)
      s += qv[8 * c + 0] * lo_bf16(k[c].x) + qv[8 * c + 1] * hi_bf16(k[c].x) + qv[8 * c + 2] * lo_bf16(k[c].y) +
           qv[8 * c + 3] * hi_bf16(k[c].y) + qv[8 * c + 4] * lo_bf16(k[c].z) + qv[8 * c + 5] * hi_bf16(k[c].z) +
           qv[8 * c + 6] * lo_bf16(k[c].w) + qv[8 * c + 7] * hi_bf16(k[c].w);
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    s = (base + kk < n) ? s * sl2 : -INFINITY;
    float mt = s;
#pragma unroll
    for (int off = 4; off < 64; off <<= 1) mt = fmaxf(mt, __shfl_xor(mt, off, 64));
    const float m_new = fmaxf(m_run, mt);  // finite: key base is visible
    const float alpha = fast_exp2(m_run - m_new);
    const float p = fast_exp2(s - m_new);
    const float ps = wave_sum(kq == 0 ? p : 0.f);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    o0 *= alpha;
    o1 *= alpha;
#pragma unroll
    for (int k2 = 0; k2 < 16; ++k2) {
      const float pj = __shfl(p, k2 * 4, 64);
      if (base + k2 < n) {
        o0 += pj * lo_bf16(v[k2]);
        o1 += pj * hi_bf16(v[k2]);
      }
    }
  };
  int base = wave * 16;
  if (base < n) load(base, kf[0], vf[0]);
  for (; base < n; base += 128) {
    if (base + 64 < n) load(base + 64, kf[1], vf[1]);
    step(base, kf[0], vf[0]);
    if (base + 64 >= n) break;
    if (base + 128 < n) load(base + 128, kf[0], vf[0]);
    step(base + 64, kf[1], vf[1]);
  }
  if (lane == 0) {
    ms[wave] = m_run;
    lsum[wave] = l_run;
  }
  os[wave][2 * lane] = o0;
  os[wave][2 * lane + 1] = o1;
  __syncthreads();
  float M = -INFINITY;
  for (int w = 0; w < 4; ++w) M = fmaxf(M, ms[w]);
  float den = 0.f, f[4];
  for (int w = 0; w < 4; ++w) {
    f[w] = (ms[w] == -INFINITY) ? 0.f : fast_exp2(ms[w] - M);
    den += f[w] * lsum[w];
  }
  for (int d = threadIdx.x; d < DV; d += 256) {
    float acc = 0.f;
    for (int w = 0; w < 4; ++w) acc += f[w] * os[w][d];
    a.z[(size_t)bh * DV + d] = den > 0.f ? acc / den : 0.f;
  }
  if (threadIdx.x == 0 && a.lse) a.lse[bh] = (M + __log2f(den)) * 0.6931471805599453f;
}

__global__ void gate_mul_kernel(const float* z, const float* g_pre, int n, void* u, int u_f32) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float v = z[i];
  if (g_pre) v *= sigmoidf_(g_pre[i]);
  if (u_f32)
    ((float*)u)[i] = v;
  else
    ((uint16_t*)u)[i] = f32_to_bf16_bits(v);
}

size_t index_topk_scratch_words(int B, int score_stride) {
  const size_t S = cdiv(score_stride, kChunk);
  return (size_t)B * (kHistBins + 8 + 3 * S + S * 2 * kChunk);
}

hipError_t launch_index_topk(IndexScoreArgs sa, int max_visible, TopkArgs ta, int32_t* scratch,
                             hipStream_t st) {
  if (sa.B <= 0) return hipSuccess;
  const int B = sa.B;
  const int S = cdiv(ta.score_stride, kChunk);
  sa.hist = ta.hist = scratch;  // zeroed before the score kernel adds to it
  ta.info = scratch + (size_t)B * kHistBins;
  ta.sel = ta.info + (size_t)B * 4;
  ta.off = ta.sel + (size_t)B * 4;
  ta.above = ta.off + (size_t)B * S;
  ta.ncand = ta.above + (size_t)B * S;
  ta.cand = (uint32_t*)(ta.ncand + (size_t)B * S);
  ta.off_stride = S;
  const int nz = B * kHistBins;
  if (((uintptr_t)scratch & 15) == 0 && nz % 4 == 0)
    zero_words16_kernel<<<min(cdiv(nz / 4, 256), 1024), 256, 0, st>>>((int4*)scratch, nz / 4);
  else
    zero_words_kernel<<<cdiv(nz, 256), 256, 0, st>>>(scratch, nz);
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu < 1)
    n_cu = 256;
  // rows of one sequence (a prefill's tokens) share each key block among eight rows
  const bool one_seq = sa.rows_per_seq > 1 && sa.row0 / sa.rows_per_seq == (sa.row0 + B - 1) / sa.rows_per_seq;
  if (max_visible > 0 && one_seq) {
    const dim3 grid(cdiv(max_visible, kRowBlock * kRowBlocksPerWg), cdiv(B, kRowsPerWg));
    if (sa.idx_scale)
      index_scores_rows_kernel<true><<<grid, kRowsPerWg * 64, 0, st>>>(sa);
    else
      index_scores_rows_kernel<false><<<grid, kRowsPerWg * 64, 0, st>>>(sa);
  } else if (max_visible > 0) {
    // chunks per row such that the B rows' workgroups fill the CUs a whole number of times
    const int cpr = max(1, n_cu * cdiv(B, n_cu) / B);
    sa.row_tiles = cdiv(max_visible, 32);
    sa.n_chunks = max(1, min(cpr, sa.row_tiles / kScoreTilesMin));
    const dim3 grid(sa.n_chunks, B);
    const bool fp8 = sa.idx_scale != nullptr, paged = sa.pages.table != nullptr;
    if (fp8 && paged)
      index_scores_kernel<true, true><<<grid, kScoreWaves * 64, 0, st>>>(sa);
    else if (fp8)
      index_scores_kernel<true, false><<<grid, kScoreWaves * 64, 0, st>>>(sa);
    else if (paged)
      index_scores_kernel<false, true><<<grid, kScoreWaves * 64, 0, st>>>(sa);
    else
      index_scores_kernel<false, false><<<grid, kScoreWaves * 64, 0, st>>>(sa);
  }
  // Rows of at most 4096 positions (a prefill's) take one kernel: 74 us against 91 us for the
  // three chunked kernels over 4096 rows of up to 4096 positions. Long rows keep the chunked path,
  // whose count and compaction spread a row over many workgroups: for 8 rows of 65,537 positions
  // it takes 20 us, one workgroup per row 33 us. (A row longer than 4096 would still be selected
  // right by the row kernel, its keys loaded segment by segment.)
  const int row_max = min(max_visible, ta.score_stride);
  if (row_max <= 4 * kTopkThreads) {
    topk_row_kernel<4><<<B, kTopkThreads, 0, st>>>(ta);
  } else {
    topk_count_kernel<<<dim3(S, B), 256, 0, st>>>(ta);
    // rows spread over up to n_cu / B workgroups each: the fused select and compaction when each
    // workgroup then holds at most kFuseMaxCpw chunks (8 rows of 65,537: 10.8 us against 14.1 us
    // for the select and compaction kernels, kernel trace), else one
    // select workgroup per row and one compaction workgroup per chunk
    const int cpw = cdiv(S, min(S, max(1, n_cu / B)));
    if (cpw <= kFuseMaxCpw) {
      ta.cpw = cpw;
      topk_select_compact_kernel<<<dim3(cdiv(S, cpw), B), kTopkThreads, 0, st>>>(ta);
    } else {
      topk_select_kernel<<<B, kTopkThreads, 0, st>>>(ta);
      topk_compact_kernel<<<dim3(S, B), 256, 0, st>>>(ta);
    }
  }
  return hipGetLastError();
}

hipError_t read_debug_flags_topk(uint32_t* flags, hipStream_t st) {
  *flags = 0;
#ifdef GMLA_DEBUG_CHECKS
  hipError_t e = hipMemcpyFromSymbolAsync(flags, HIP_SYMBOL(g_debug_flags_topk), sizeof(uint32_t), 0,
                                          hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  const uint32_t zero = 0;
  if (e == hipSuccess)
    e = hipMemcpyToSymbolAsync(HIP_SYMBOL(g_debug_flags_topk), &zero, sizeof(uint32_t), 0, hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  return e;
#else
  (void)st;
  return hipSuccess;
#endif
}

hipError_t launch_expanded_attention(Shape s, const ExpandedAttnArgs& a, hipStream_t st) {
  if (a.B <= 0) return hipSuccess;
  if (s == Shape::K3)
    expanded_attn_k3_kernel<<<a.B * ShapeK3::H, 256, 0, st>>>(a);
  else
    expanded_attn_kernel<ShapeTiny><<<a.B * ShapeTiny::H, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_gate_mul(const float* z, const float* g_pre, int n, void* u, int u_f32,
                           hipStream_t st) {
  if (n <= 0) return hipSuccess;
  gate_mul_kernel<<<cdiv(n, 256), 256, 0, st>>>(z, g_pre, n, u, u_f32);
  return hipGetLastError();
}

}  // namespace gmla
