// Absorbed (latent-space) decode attention for the K3 layer shape, dense and gathered (DSA).
//
// Same computation as decode_attn_kernel (see decode_attn.hip): for every head h of sequence b,
// scores q~_h . [c_j ; r_j] * scale over the positions of one split, an online softmax, and the
// unnormalised latent-space output sum_j p_j c_j, with (max, sum) per head for the merge.
// (K3.1 Gated DSA blog, the note on latent absorption after eq. (10); eq. (9).)
//
// Layout of the work on one CU (448 threads = 7 waves), software-pipelined by tile:
// * 32-position tiles of latent rows (32 x 1,152 B) stream from HBM straight into LDS with
//   global_load_lds_dwordx4 (no staging registers) into a ring of NSLOT slots (4 dense, 3 when
//   gathering); the four P.V waves issue them (9 wave-wide loads each per tile), NSLOT-1 tiles
//   ahead of the tile they consume. 16-byte chunk c of row r sits at chunk r*72 + (c ^ swz(r)),
//   which keeps the score MFMA's row reads free of bank conflicts.
// * In step t the score waves work on tile t+1 while the P.V waves consume tile t, with P^T and
//   the rescale factors double-buffered: one barrier per tile.
// * waves 0-2 hold q~ for 32 heads each in VGPRs (the B operand of S^T = Lat Q~^T, 36 k-steps
//   of v_mfma_f32_32x32x16_bf16 over the 576 features) and run the online softmax: lane l owns
//   head l%32, so max and sum need one xor-32 shuffle. P^T goes to LDS as bf16.
// * waves 3-6 each accumulate O^T = Lat^T P^T for 128 of the 512 latent features and all 96
//   heads (192 fp32 accumulators per lane), reading Lat^T from the row-major tile with
//   ds_read_b64_tr_b16.
// * The running max is only moved when it grows by more than 8 (base 2): otherwise the old
//   max stays and the rescale factor is exactly 1, so the accumulators are rarely rescaled.
//   The result is the same softmax; only the reference point of the exponentials differs.
// * FP8 main cache (K3.1 Gated DSA blog, cache section: 512 E4M3 codes, four fp32 block scales
//   and r in bf16 per 656-byte row): P.V waves 3-5 DMA the raw rows (7 of a tile's 21
//   wave-wide loads each) into a 6-slot ring of raw tiles (rows at a 656-byte pitch), five tiles
//   ahead, and the MFMA operands are formed from the raw tile in registers, one barrier per tile
//   as above. Score waves read 8 codes of their row and decode them with the row's block scale
//   (v_cvt_scalef32_pk_bf16_fp8: the scales are powers of two, so the bf16 value is exactly
//   decode(code) * scale); r is read as bf16. P.V waves read 8 positions of one feature with
//   ds_read_b64_tr_b8, decode them unscaled, and multiply the P^T entries of those positions by
//   the positions' scales for the wave's 128-feature block (a power of two again, so
//   bf16(p) * scale is exact and every product equals the bf16 path's).
// * Each split writes its output divided by its own softmax sum, in fp16: a convex combination
//   of cached rows, so bounded by the largest latent entry, at half the bytes of fp32 partials
//   (11-bit significand; the merge weights them by 2^(m - M) * l in fp32).
#include "common.h"
#include "kernels.h"

namespace gmla {

namespace k3dec {
constexpr int H = 96, L = 512, DL = 576;
constexpr int BT = 32;                        // positions per tile
constexpr int CH = DL / 8;                    // 72 chunks of 16 bytes per latent row
constexpr int TILE_BYTES = BT * DL * 2;       // 36,864
constexpr int NLOAD = TILE_BYTES / 1024;      // 36 wave-wide 1 KB DMA loads per tile
constexpr int NLOAD_W = NLOAD / 4;            // issued by each of the 4 P.V waves
constexpr int NTHREADS = 7 * 64;
constexpr int PROW = BT + 8;                  // P^T [head][position] row stride (bf16)
constexpr int KSD = DL / 16;                  // 36 score k-steps
constexpr int MAX_SEL = 2048;                 // gathered positions per split (<= top-k)
constexpr float RESCALE_SLACK = 8.0f;         // base-2 growth of the max before rescaling
constexpr int F8CH = kFp8RowBytes / 16;       // 41 chunks of 16 bytes per FP8 row
constexpr int F8SLOT = 21 * 1024;             // 32 rows (20,992 bytes) and the 21st load's spill
constexpr int NS8 = 6;                        // raw FP8 tiles in the ring
constexpr int NL8 = 7;                        // 1 KB loads per tile issued by each of waves 3-5
}  // namespace k3dec

__device__ __forceinline__ int swz_row(int r) { return ((r ^ (r >> 2)) & 1) | (r & 2) | ((r >> 1) & 4); }

__device__ __forceinline__ int perm_row_k3(int m) {
  const int a = m >> 3, g = (m >> 2) & 1, b = m & 3;
  return 16 * (a >> 1) + 8 * g + 4 * (a & 1) + b;
}

// two E4M3 codes (bytes 2*HI, 2*HI + 1 of w) -> packed bf16 pair, times 2^exponent(sc)
template <bool HI>
__device__ __forceinline__ uint32_t cvt_fp8x2(uint32_t w, float sc) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, sc, HI));
}
__device__ __forceinline__ u32x4 cvt_fp8x8(u32x2 c, float sc) {
  return u32x4{cvt_fp8x2<false>(c.x, sc), cvt_fp8x2<true>(c.x, sc), cvt_fp8x2<false>(c.y, sc),
               cvt_fp8x2<true>(c.y, sc)};
}
// eight bf16 values (k = 0..7 of an MFMA operand) times per-k powers of two: exact
__device__ __forceinline__ u32x4 scale_bf16x8(u32x4 w, const float* s) {
  uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float lo = __builtin_bit_cast(float, x[q] << 16) * s[2 * q];
    const float hi = __builtin_bit_cast(float, x[q] & 0xFFFF0000u) * s[2 * q + 1];
    x[q] = (__builtin_bit_cast(uint32_t, hi) & 0xFFFF0000u) | (__builtin_bit_cast(uint32_t, lo) >> 16);
  }
  return u32x4{x[0], x[1], x[2], x[3]};
}

// vmcnt wait leaving at most `tiles` of this wave's most recent tile loads (9 each) in flight.
__device__ __forceinline__ void wait_tiles_in_flight(int tiles) {
  if (tiles >= 2)
    asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
  else if (tiles == 1)
    asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <bool GATHER, bool FP8>
__global__ __launch_bounds__(k3dec::NTHREADS) void decode_attn_k3_kernel(DecodeAttnArgs a) {
  using namespace k3dec;
  constexpr int NSLOT = GATHER ? 3 : 4;  // bf16 tiles in the ring
  __shared__ __attribute__((aligned(1024))) uint8_t lat_s[FP8 ? 1 : NSLOT][FP8 ? 16 : TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t f8_s[FP8 ? NS8 : 1][FP8 ? F8SLOT : 16];
  __shared__ __attribute__((aligned(16))) uint16_t Ps[2][H * PROW];
  __shared__ float alpha_s[2][H];
  __shared__ int sel_s[GATHER ? MAX_SEL : 1];
  __shared__ int wcnt_s[GATHER ? 8 : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g2 = lane >> 5, l32 = lane & 31;
  // consecutive workgroups take different sequences, so that (with B a multiple of 8) all splits of
  // a sequence run on one XCD and share its L2 for q~ and, in the merge, for the partials. Rows go
  // out last first: in causal prefill the later rows of a chunk select the most positions, and
  // dispatching them first keeps them out of the launch's tail.
  const int b = a.B - 1 - (int)(blockIdx.x % a.B), split = blockIdx.x / a.B;
  const int n_vis = GATHER ? min(a.sel_cnt[b], a.sel_stride) : min(a.n_vis[b] + a.vis_offset, a.T_cap);
  const int p0 = split * a.chunk;
  const int p1 = min(p0 + a.chunk, n_vis);
  int n_pos = GATHER ? min(max(p1 - p0, 0), MAX_SEL) : max(p1 - p0, 0);
  // cache rows: unpaged, position p of this sequence is row p past lat; paged, the page table
  // gives the row within the pool (lat = the pool)
  const int seq = row_map(a.row0, a.rows_per_seq, b).seq;
  const bool paged = a.pages.table != nullptr;
  const size_t seq_rows = paged ? 0 : (size_t)seq * a.T_cap;
  auto crow = [&](int p) __attribute__((always_inline)) {
    return paged ? (int)cache_row(a.pages, a.T_cap, seq, p) : p;
  };
  auto crow_uniform = [&](int p) __attribute__((always_inline)) {  // p the same in every lane
    return paged ? (int)cache_row_uniform(a.pages, a.T_cap, seq, p) : p;
  };
  const uint16_t* lat = a.latent + seq_rows * DL;

  if (GATHER) {
    // this split's selected positions as cache rows, in order, leaving out any outside [0, T_cap)
    // (they get probability 0): a stable compaction by wave ballots, 448 entries per round
    const int32_t* sel = a.sel_idx + (size_t)b * a.sel_stride;
    int n_ok = 0;
    for (int base = 0; base < n_pos; base += NTHREADS) {
      const int i = base + tid;
      const int p = i < n_pos ? sel[p0 + i] : -1;
      const bool ok = p >= 0 && p < a.T_cap;
      const uint64_t m = __ballot(ok);
      if (lane == 0) wcnt_s[wave] = __popcll(m);
      __syncthreads();
      int before = n_ok;
      for (int w = 0; w < wave; ++w) before += wcnt_s[w];
      if (ok) sel_s[before + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))] = crow(p);
      for (int w = 0; w < NTHREADS / 64; ++w) n_ok += wcnt_s[w];
      __syncthreads();
    }
    n_pos = n_ok;
  }
  const int n_tiles = (n_pos + BT - 1) / BT;

  const float sl2 = a.scale * 1.4426950408889634f;
  const size_t part = (size_t)b * a.n_splits + split;

  // The two roles run separate code with the same barriers, so that the score waves' q~
  // registers and the P.V waves' accumulators are never live at the same point.
  if (wave < 3) {
    // ---------------- score waves: heads wave*32 + l32 ----------------
    const int head = wave * 32 + l32;
    u32x4 qf[KSD];
    const uint16_t* qrow = a.q_tilde + ((size_t)b * H + head) * DL + g2 * 8;
#pragma unroll
    for (int s = 0; s < KSD; ++s) qf[s] = ld16(qrow + s * 16);
    // use q~ here, so that its loads are waited for once, before the loop
#pragma unroll
    for (int s = 0; s < KSD; ++s) asm volatile("" ::"v"(qf[s]));
    const int srow = perm_row_k3(l32);
    const int srow_base = srow * CH * 16;
    const int srow_swz = swz_row(srow);
    float m_run = -INFINITY, l_run = 0.f;

    // scores, online-softmax statistics and P^T of tile t into buffer t%2
    // chunk (2s + g2) ^ swz = 8*(s/4) + ((2*(s%4) + g2) ^ swz): four per-lane LDS offsets plus
    // immediates
    uint32_t aoff[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) aoff[m] = lds_addr(lat_s[0]) + srow_base + (((2 * m + g2) ^ srow_swz) << 4);
    const uint32_t f8_row = lds_addr(f8_s[0]) + srow * kFp8RowBytes + 8 * g2;  // FP8: this lane's codes
    auto score_tile = [&](int t) {
      f32x16 sacc2[2] = {f32x16{}, f32x16{}};
      if constexpr (FP8) {
        // the row's 512 codes decoded with its block scales, 8 per lane and k-step; r as bf16
        // one address register per tile; the k-steps are immediate offsets from it (the empty asm
        // keeps the compiler from hoisting one loop-invariant address per k-step instead)
        uint32_t fr = f8_row + (t % NS8) * F8SLOT;
        asm volatile("" : "+v"(fr));
        const f32x4 sc4 = *(GMLA_LDS const f32x4*)(fr - 8 * g2 + kFp8ScaleOff);
        auto raw = [&](int s) __attribute__((always_inline)) {
          return *(GMLA_LDS const u32x2*)(fr + 16 * s);
        };
        auto rpart = [&](int s) __attribute__((always_inline)) {
          return *(GMLA_LDS const u32x4*)(fr + 8 * g2 + kFp8ROff + 32 * s);
        };
        constexpr int PF8 = 8;  // LDS reads run PF8 k-steps ahead of their MFMA
        u32x2 cr[PF8];
        u32x4 rr[KSD - L / 16];
#pragma unroll
        for (int s = 0; s < PF8; ++s) cr[s] = raw(s);
#pragma unroll
        for (int s = 0; s < KSD; ++s) {
          u32x4 cur;
          if (s < L / 16) {
            cur = cvt_fp8x8(cr[s % PF8], sc4[s >> 3]);
            if (s + PF8 < L / 16)
              cr[s % PF8] = raw(s + PF8);
            else if (s + PF8 < KSD)
              rr[s + PF8 - L / 16] = rpart(s + PF8 - L / 16);
          } else {
            cur = rr[s - L / 16];
          }
          __builtin_amdgcn_sched_barrier(0);
          sacc2[s & 1] = mfma32(cur, qf[s], sacc2[s & 1]);
        }
      } else {
        const uint32_t so = (t % NSLOT) * TILE_BYTES;
        uint32_t ab[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) ab[m] = aoff[m] + so;
        auto lat_row = [&](int s) __attribute__((always_inline)) {
          return *(GMLA_LDS const u32x4*)(ab[s & 3] + 128 * (s >> 2));
        };
        constexpr int PF = GATHER ? 6 : 8;  // LDS reads run PF k-steps ahead of their MFMA
        u32x4 ar[PF];
#pragma unroll
        for (int s = 0; s < PF; ++s) ar[s] = lat_row(s);
        // two accumulator chains (even and odd k-steps) so that consecutive MFMAs are independent
#pragma unroll
        for (int s = 0; s < KSD; ++s) {
          const u32x4 cur = ar[s % PF];
          if (s + PF < KSD) ar[s % PF] = lat_row(s + PF);
          __builtin_amdgcn_sched_barrier(0);
          sacc2[s & 1] = mfma32(cur, qf[s], sacc2[s & 1]);
        }
      }
      f32x16 sacc = sacc2[0] + sacc2[1];
      const int jbase = t * BT;
      if (jbase + BT > n_pos) {  // the split's last, partial tile: positions past it get -inf
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (jbase + 16 * (r >> 3) + 8 * g2 + (r & 7) >= n_pos) sacc[r] = -INFINITY;
      }
      // the raw scores' max, scaled once (sl2 > 0); the exponent arguments below are one FMA each
      float mt = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[r]);
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64)) * sl2;
      float alpha = 1.f;
      if (mt > m_run + RESCALE_SLACK || m_run == -INFINITY) {
        alpha = fast_exp2(m_run - mt);  // 0 on the first tile
        m_run = mt;
      }
      float ls = 0.f;
      uint16_t* prow = Ps[t & 1] + head * PROW + g2 * 8;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          p[i] = fast_exp2(fmaf(sacc[hh * 8 + i], sl2, -m_run));
          ls += p[i];
        }
        st16(prow + hh * 16, u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                                   pack_bf16x2(p[6], p[7])});
      }
      l_run = l_run * alpha + ls;
      if (g2 == 0) alpha_s[t & 1][head] = alpha;
    };

    __syncthreads();  // tile 0 is in LDS
    if (n_tiles > 0) score_tile(0);
    __syncthreads();  // P of tile 0 is ready; tile 1 is in LDS
    for (int t = 0; t < n_tiles; ++t) {
      if (t + 1 < n_tiles) score_tile(t + 1);
      __syncthreads();
    }
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    if (g2 == 0) {
      a.part_ml[(part * H + head) * 2 + 0] = m_run;
      a.part_ml[(part * H + head) * 2 + 1] = l_tot;
      alpha_s[0][head] = l_tot > 0.f ? 1.0f / l_tot : 0.f;  // no longer read as a rescale factor
    }
    __syncthreads();  // 1/l of every head is in LDS
  } else {
    // ---------------- P.V waves: latent features [pw*128, pw*128 + 128) ----------------
    const int pw = wave - 3;
    // ---- FP8 rows: issued by P.V waves 3-5 (7 of a tile's 21 wave-wide loads each) ----
    // Load i of a tile fills tile bytes 1024 i .. 1024 i + 1023 (the last one's upper half repeats
    // the tile's last chunk); d8[k] holds this lane's source row r in the tile (bits 16+) and the
    // byte offset r * 656 + 16 c of its chunk (bits 0-15).
    const uint8_t* lat8 = (const uint8_t*)a.latent + seq_rows * kFp8RowBytes;
    uint32_t d8[NL8];
#pragma unroll
    for (int k = 0; k < NL8; ++k) {
      const int i = (wave - 3) * NL8 + k;
      const int P = min(i * 64 + lane, BT * F8CH - 1);
      const int r = P / F8CH;
      d8[k] = ((uint32_t)r << 16) | (uint32_t)(P * 16);
    }
    int issued8 = 0;
    auto issue8 = [&]() {  // the next tile's raw rows
      if (!FP8 || issued8 >= n_tiles) return;
      const int t = issued8++;
      if (wave < 3 || wave == 6) return;
      const uint32_t fs = lds_addr(f8_s[t % NS8]) + (wave - 3) * NL8 * 1024;
      const int j0 = t * BT;
      if (!GATHER && j0 + BT <= n_pos) {  // whole tile of consecutive rows (one page): offsets only
        const int row0 = __builtin_amdgcn_readfirstlane(crow_uniform(p0 + j0));
        const uint8_t* base = lat8 + (size_t)row0 * kFp8RowBytes;
#pragma unroll
        for (int k = 0; k < NL8; ++k) lds_dma16_sbase(d8[k] & 0xFFFFu, base, fs + k * 1024);
        return;
      }
      // gathered rows, or the partial last tile (rows past the end repeat a valid row, masked)
      const int row0 = GATHER ? 0 : crow_uniform(p0 + j0);
#pragma unroll 1
      for (int k = 0; k < NL8; ++k) {
        const int r = (int)(d8[k] >> 16);
        const uint32_t coff = (d8[k] & 0xFFFFu) - (uint32_t)(r * kFp8RowBytes);
        const int jr = min(j0 + r, n_pos - 1);
        const int row = GATHER ? sel_s[jr] : row0 + (jr - j0);
        lds_dma16(lat8 + (size_t)row * kFp8RowBytes + coff, fs + k * 1024);
      }
    };
    auto wait8 = [&](int need) {  // this wave's loads of tile `need` have landed
      const int after = issued8 - 1 - need;
      static_assert(NL8 == 7, "vmcnt immediates");
      if (after >= 4)
        asm volatile("s_waitcnt vmcnt(28)" ::: "memory");
      else if (after == 3)
        asm volatile("s_waitcnt vmcnt(21)" ::: "memory");
      else if (after == 2)
        asm volatile("s_waitcnt vmcnt(14)" ::: "memory");
      else if (after == 1)
        asm volatile("s_waitcnt vmcnt(7)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };
    // before the first step: tiles 0 .. NS8-2 issued, tile 0 landed (the barrier follows)
    auto prologue8 = [&]() {
#pragma unroll
      for (int i = 0; i + 1 < NS8; ++i) issue8();
      wait8(0);
    };
    // Per-lane source offsets (bytes from the tile's first row) of this wave's 9 loads, with the
    // row in the top bits for the clamped path: chunk P = i*64 + lane of the tile is row P/72,
    // swizzled chunk (P%72) ^ swz(row).
    uint32_t doff[NLOAD_W];
#pragma unroll
    for (int k = 0; k < NLOAD_W; ++k) {
      const int P = (pw * NLOAD_W + k) * 64 + lane;
      const int r = P / CH, c = (P - r * CH) ^ swz_row(r);
      doff[k] = (uint32_t)(r * DL * 2 + c * 16) | ((uint32_t)r << 16);
    }
    auto issue = [&](int t) {  // this wave's 9 of the 36 DMA loads of tile t
      if constexpr (!FP8) {
        if (t >= n_tiles) return;
        const uint32_t slot_addr = lds_addr(lat_s[t % NSLOT]);
        const int j0 = t * BT;
        if (!GATHER && j0 + BT <= n_pos) {  // whole tile of consecutive rows: offsets only
          // a tile lies in one page; its first row is wave-uniform (the DMA takes it in SGPRs)
          const int row0 = __builtin_amdgcn_readfirstlane(crow_uniform(p0 + j0));
          const char* base = (const char*)(lat + (size_t)row0 * DL);
#pragma unroll
          for (int k = 0; k < NLOAD_W; ++k)
            lds_dma16_sbase(doff[k] & 0xFFFFu, base, slot_addr + (pw * NLOAD_W + k) * 1024);
          return;
        }
        // rows past the end repeat a valid row (masked)
        if constexpr (GATHER) {
          // gathered rows, three loads at a time: the lane's chunk geometry is recomputed on every
          // call from an opaque copy of the lane id. Held across the loop, the nine offsets spill
          // next to the accumulators, and reloading a spill waits for every load in flight,
          // the tiles' DMA included.
          int ln = lane;
          asm volatile("" : "+v"(ln));
#pragma unroll
          for (int k0 = 0; k0 < NLOAD_W; k0 += 3) {
            int rows[3];
            uint32_t coff[3];
#pragma unroll
            for (int k = 0; k < 3; ++k) {
              const int P = (pw * NLOAD_W + k0 + k) * 64 + ln;
              const int r = P / CH;
              coff[k] = (uint32_t)(((P - r * CH) ^ swz_row(r)) << 4);
              rows[k] = sel_s[min(j0 + r, n_pos - 1)];
            }
#pragma unroll
            for (int k = 0; k < 3; ++k)
              lds_dma16((const char*)lat + (size_t)rows[k] * (DL * 2) + coff[k], slot_addr + (pw * NLOAD_W + k0 + k) * 1024);
          }
        } else {
          // the partial last tile of a split: consecutive rows (a rolled loop keeps the P.V waves'
          // registers free)
          const int row0 = crow_uniform(p0 + j0);
#pragma unroll 1
          for (int k = 0; k < NLOAD_W; ++k) {
            const int i = pw * NLOAD_W + k;
            const int P = i * 64 + lane;  // destination chunk of this lane
            const int r = P / CH, c = (P - r * CH) ^ swz_row(r);
            const int jr = min(j0 + r, n_pos - 1);
            lds_dma16(lat + (size_t)(row0 + (jr - j0)) * DL + c * 8, slot_addr + i * 1024);
          }
        }
      }
    };
    // tiles issued so far are [0, issued); wait until tile `need` has landed
    auto wait_for = [&](int need, int issued) { wait_tiles_in_flight(max(0, issued - 1 - need)); };
    int issued = FP8 ? 0 : min(n_tiles, NSLOT - 1);
    for (int t = 0; t < issued; ++t) issue(t);
    if (!FP8) wait_for(0, issued);
    const int G = lane >> 4, jj = lane & 15;
    const uint32_t tr8_off = (8 * (G >> 1) + (jj >> 1)) * kFp8RowBytes + 16 * (G & 1) + 8 * (jj & 1);
    const uint32_t f8_slot0 = lds_addr(f8_s[0]);
    f32x16 o[4][3];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 3; ++j) o[i][j] = f32x16{};
    if constexpr (FP8) {
      prologue8();
      __syncthreads();  // tile 0 is in LDS
      wait8(1);
      __syncthreads();  // P of tile 0 is ready; tile 1 is in LDS
    } else {
      __syncthreads();  // tile 0 is in LDS
      if (n_tiles > 1) wait_for(1, issued);
      __syncthreads();  // P of tile 0 is ready; tile 1 is in LDS
    }
    for (int t = 0; t < n_tiles; ++t) {
      if constexpr (FP8)
        issue8();  // tile t + NS8 - 1, into the slot tile t - 1 used
      else if (issued < n_tiles)
        issue(issued++);  // tile t + NSLOT - 1, into the slot tile t-1 used
      const uint8_t* slot = lat_s[t % (FP8 ? 1 : NSLOT)];
      const uint16_t* pbuf = Ps[t & 1];
      float al[3];
#pragma unroll
      for (int hs = 0; hs < 3; ++hs) al[hs] = alpha_s[t & 1][hs * 32 + l32];
#pragma unroll
      for (int hs = 0; hs < 3; ++hs) {
        if (__any(al[hs] != 1.f)) {
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[dt][hs][r] *= al[hs];
        }
      }
      // P^T for both 16-position halves, then Lat^T fragments one (half, block) ahead of their MFMAs
      u32x4 pb[2][3];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int hs = 0; hs < 3; ++hs) pb[ks][hs] = ld16(pbuf + (hs * 32 + l32) * PROW + ks * 16 + g2 * 8);
      if constexpr (FP8) {
        // P^T entries times their positions' scales for this wave's block: the products with the
        // unscaled codes are then those of the decoded values
        uint32_t fsa = f8_slot0 + (t % NS8) * F8SLOT;
        asm volatile("" : "+v"(fsa));  // one address register; the rest are immediate offsets
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          float psc[8];
#pragma unroll
          for (int i = 0; i < 8; ++i)
            psc[i] = *(GMLA_LDS const float*)(fsa + g2 * 8 * kFp8RowBytes + (ks * 16 + i) * kFp8RowBytes + kFp8ScaleOff +
                                              4 * pw);
#pragma unroll
          for (int hs = 0; hs < 3; ++hs) pb[ks][hs] = scale_bf16x8(pb[ks][hs], psc);
        }
        // Lat^T fragments: 8 positions of one feature per lane, one transposed byte read each
        // lane (G, jj) starts at row 8 (G >> 1) + (jj >> 1), byte 16 (G & 1) + 8 (jj & 1) of the block
        const uint32_t fla = fsa + pw * 128 + tr8_off;
        auto raw_frag = [&](int k) __attribute__((always_inline)) {
          const int ks = k >> 2, dt = k & 3;
          return lds_read_tr8(fla + ks * 16 * kFp8RowBytes + dt * 32);
        };
        u32x2 cr = raw_frag(0);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const u32x2 cn = raw_frag(k < 7 ? k + 1 : 7);
          const u32x4 af = cvt_fp8x8(cr, 1.0f);
#pragma unroll
          for (int hs = 0; hs < 3; ++hs) o[k & 3][hs] = mfma32(af, pb[k >> 2][hs], o[k & 3][hs]);
          cr = cn;
        }
      } else {
        auto lat_frag = [&](int k) __attribute__((always_inline)) {
          const int ks = k >> 2, dt = k & 3;
          const int r0 = ks * 16 + 8 * (G >> 1) + (jj >> 2), r1 = r0 + 4;
          const int fcol = (pw * 4 + dt) * 32 + 16 * (G & 1) + 4 * (jj & 3);
          const int c = fcol >> 3, off = (fcol & 7) * 2;
          const u32x2 lo = lds_read_tr16(slot + (r0 * CH + (c ^ swz_row(r0))) * 16 + off);
          const u32x2 hi = lds_read_tr16(slot + (r1 * CH + (c ^ swz_row(r1))) * 16 + off);
          return u32x4{lo.x, lo.y, hi.x, hi.y};
        };
        u32x4 af = lat_frag(0);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const u32x4 an = lat_frag(k < 7 ? k + 1 : 7);
#pragma unroll
          for (int hs = 0; hs < 3; ++hs) o[k & 3][hs] = mfma32(af, pb[k >> 2][hs], o[k & 3][hs]);
          af = an;
        }
      }
      if constexpr (FP8)
        wait8(t + 2);  // the score waves read it in the next step
      else if (t + 2 < n_tiles)
        wait_for(t + 2, issued);  // the score waves read it in the next step
      __syncthreads();
    }
    __syncthreads();  // 1/l of every head is in LDS
    if (a.n_splits == 1 && !a.lse) {  // one split: its normalised output is the result
#pragma unroll
      for (int hs = 0; hs < 3; ++hs) {
        const float inv = alpha_s[0][hs * 32 + l32];
        float* dst = a.o_latent + ((size_t)b * H + hs * 32 + l32) * L;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int rb = 0; rb < 4; ++rb) {
            const int f = (pw * 4 + dt) * 32 + rb * 8 + g2 * 4;
            *(f32x4*)(dst + f) = f32x4{o[dt][hs][rb * 4 + 0], o[dt][hs][rb * 4 + 1], o[dt][hs][rb * 4 + 2],
                                       o[dt][hs][rb * 4 + 3]} * inv;
          }
      }
      return;
    }
    // The wave's 96 x 128 fp16 block is staged in LDS (every tile has landed and been read by
    // now, so the ring is free), so that the stores are whole 256-byte head rows: written from the
    // accumulators, a store covers 16 bytes of each of 32 head rows. Head h's 16-byte chunk c sits
    // at h*256 + (c ^ (h & 15))*16 of the wave's 24 KB region.
    uint8_t* stage = (FP8 ? f8_s[0] : lat_s[0]) + pw * (H * 256);
    static_assert((FP8 ? NS8 * F8SLOT : NSLOT * TILE_BYTES) >= 4 * H * 256, "staging fits the ring");
#pragma unroll
    for (int hs = 0; hs < 3; ++hs) {
      const int h = hs * 32 + l32;
      const float inv = alpha_s[0][h];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const f32x4 v = f32x4{o[dt][hs][rb * 4 + 0], o[dt][hs][rb * 4 + 1], o[dt][hs][rb * 4 + 2],
                                o[dt][hs][rb * 4 + 3]} * inv;
          *(u32x2*)(stage + h * 256 + (((dt * 4 + rb) ^ (h & 15)) << 4) + g2 * 8) =
              u32x2{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3])};
        }
    }
    const int j = lane & 15;
#pragma unroll 4
    for (int i = 0; i < H / 4; ++i) {
      const int h = i * 4 + (lane >> 4);
      const u32x4 v = *(const u32x4*)(stage + h * 256 + ((j ^ (h & 15)) << 4));
      *(u32x4*)(a.part_o + (part * H + h) * L + pw * 128 + j * 8) = v;
    }
  }
}

hipError_t launch_decode_attention_k3(const DecodeAttnArgs& a, bool gather, hipStream_t st) {
  const int grid = a.B * a.n_splits;
  if (gather && a.fp8)
    decode_attn_k3_kernel<true, true><<<grid, k3dec::NTHREADS, 0, st>>>(a);
  else if (gather)
    decode_attn_k3_kernel<true, false><<<grid, k3dec::NTHREADS, 0, st>>>(a);
  else if (a.fp8)
    decode_attn_k3_kernel<false, true><<<grid, k3dec::NTHREADS, 0, st>>>(a);
  else
    decode_attn_k3_kernel<false, false><<<grid, k3dec::NTHREADS, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace gmla
