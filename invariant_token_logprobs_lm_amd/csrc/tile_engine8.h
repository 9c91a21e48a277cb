// Eight-wavefront tile engine (gfx950 / CDNA4): the K loop of the wide bf16
// / fp32 contractions (the logprob forward, and the backward's dlogits, dH
// and dW) with two wavefronts per SIMD.
//
// A 512-thread workgroup multiplies 256-row tiles of an operand A (walked in
// order) with one fixed 256-row block of an operand B, acc = A_tile B^T,
// both row-major and K-contiguous, fp32 accumulate, K ascending in steps of
// 128 bytes, through the five LDS slots, swizzle and direct-to-LDS loads
// of tile_engine.h. Wavefront w = 4 g + r (g = 0, 1,
// r = 0..3) holds A rows 128 (r & 1) .. + 127 of the tile against B rows
// 64 ((r >> 1) + 2 g) .. + 63 of the block, as 4 x 2 blocks of 32 x 32: the
// same per-block MFMA sequence (fragments, sub-step order, fresh
// accumulators at a tile's first step) as run_tiles_narrow, so an output
// element has the same bits in both.
//
// Schedule. Waves w and w + 4 share a SIMD (the workgroup's wavefronts go
// to the four SIMDs in a rotating order, w and w + 4 on the same one, as
// read from the hardware-id register), so each SIMD's matrix core is fed by
// two instruction streams and one wavefront's waits are covered by the
// other's MFMAs. Each wavefront runs a K step as four sub-steps of 8 MFMAs;
// during each sub-step it reads the next sub-step's 6 operand fragments
// from LDS. One workgroup barrier per K step, after sub-step 2 (whose reads
// are the step's last): it publishes step g + 1 (every wavefront has waited
// for its own loads of it) and frees step g's slots; sub-step 3 loads the
// near operand's step g + 2 into them (after its second MFMA), and
// sub-step 0 of step g + 1 the far operand's step g + 3 (after its fourth).
// Every wavefront loads rows 32 w .. 32 w + 31 of both operands, four loads
// of each step back to back under one M0 value. The near operand (two
// slots) is the B block, the far one (three slots) the walked A tiles; with
// kBFar the other way round. A tile's last
// K step leaves the next tile's first fragments unread; they are read after
// the epilogue, which then has those registers.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "itl_config.h"
#include "tile_engine.h"

namespace itl {

constexpr int kDma8PerWave = 4;  // loads per wavefront per K step of each operand (32 rows)

struct Lanes8 {
  int lane, wave, grp, r, wv, tq, half, col;
};

__device__ __forceinline__ Lanes8 lanes8() {
  Lanes8 L;
  L.lane = threadIdx.x & 63;
  L.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  L.grp = L.wave >> 2;
  L.r = L.wave & 3;
  L.wv = L.r & 1;                     // which 128 rows of the A tile
  L.tq = (L.r >> 1) | (L.grp << 1);   // which 64 rows of the B block
  L.half = L.lane >> 5;
  L.col = L.lane & 31;
  return L;
}

// Runs tiles tile_begin .. tile_end - 1 (tile_end > tile_begin): a_rsrc(t)
// is A tile t's buffer resource (its first row at offset 0, its valid rows'
// bytes as the range: rows past it load as zeros), b_rsrc the B block's;
// rows are row_bytes apart; nks K steps of 128 bytes (nks >= 1,
// nks * 128 <= row_bytes). epi(t, acc)
// sees tile t's accumulators acc[bm][bn] (A rows 32 bm, B rows 32 bn of the
// wavefront's 128 x 64); it may read them directly. Every thread of the
// 512-thread workgroup must call this.
template <int kDtype, bool kBFar, class ARsrc, class Epi>
__device__ __forceinline__ void run_tiles8(uint4* smem, const Lanes8& L, int row_bytes, int tile_begin, int tile_end,
                                           int nks, const ARsrc& a_rsrc, int4v b_rsrc, Epi&& epi) {
  constexpr int kAS = kBFar ? kHSlots : kWSlots;  // slots of A
  constexpr int kBS = kBFar ? kWSlots : kHSlots;  // slots of B
  static_assert(kAS + kBS == 5 && (kAS == 2 || kAS == 3), "five slots: two near, three far");
  const int lane = L.lane, wave = L.wave, half = L.half, col = L.col;

  // Loader: wavefront w fills rows 32 w .. 32 w + 31 of both operands' slots
  // with four 16-byte-per-lane loads each, under one M0 value (dma16x4);
  // lane i of load j fetches row 32 w + 8 j + i / 8 at logical chunk
  // (i % 8) ^ swz(row), which lands at its swizzled position
  // (swz(32 w + 8 j + i / 8) = (i / 8) ^ (j & 1)). voff[j] holds that offset
  // less 1024 j, which it never underflows (8 j rows are at least 1024 j
  // bytes: a row holds at least one 128-byte K step).
  static_assert(kDma8PerWave == 4, "dma16x4 issues a wavefront's four loads of a step");
  const int lr = lane >> 3;
  uint32_t voff[kDma8PerWave];
#pragma unroll
  for (int j = 0; j < kDma8PerWave; ++j)
    voff[j] = (uint32_t)(wave * 32 + j * kDmaRows + lr) * (uint32_t)row_bytes + (((lane & 7) ^ lr ^ (j & 1)) * 16) -
              (uint32_t)j * 1024u;
  const uint32_t lds0 = (uint32_t)(size_t)((__attribute__((address_space(3))) uint4*)smem);
  const uint32_t my_rows = (uint32_t)wave * 32 * kStepBytes;
  const int n_steps = (tile_end - tile_begin) * nks;
  // The four loads of step s of A / of B into its slot. A step past the end
  // loads the last step's data instead (a valid address) into slot s, which
  // is free and which nothing reads again.
  auto a_load = [&](int s) {
    const int c = s < n_steps ? s : n_steps - 1;
    const int q = c / nks;
    dma16x4(a_rsrc(tile_begin + q), voff, (uint32_t)(c - q * nks) * kStepBytes,
            lds0 + (uint32_t)(s % kAS) * kSlotBytes + my_rows);
  };
  auto b_load = [&](int s) {
    const int c = s < n_steps ? s : n_steps - 1;
    dma16x4(b_rsrc, voff, (uint32_t)(c % nks) * kStepBytes, lds0 + (uint32_t)(kAS + s % kBS) * kSlotBytes + my_rows);
  };

  // MFMA operand reads of sub-step kk: A rows 128 wv + 32 bm + (l mod 32),
  // B rows 64 tq + 32 bn + (l mod 32), logical chunk 2 kk + l / 32.
  int a_off[4], b_off[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int pc = (2 * kk + half) ^ swz(col);
    a_off[kk] = (L.wv * 128 + col) * kRowChunks + pc;
    b_off[kk] = (L.tq * 64 + col) * kRowChunks + pc;
  }

  // The near operand (two slots) and the far one (three slots).
  auto near_load = [&](int s) {
    if constexpr (kAS == 2) a_load(s);
    else b_load(s);
  };
  auto far_load = [&](int s) {
    if constexpr (kAS == 2) b_load(s);
    else a_load(s);
  };

  // Prologue: near and far steps 0 and 1, in that order; then step 0 is
  // published (step 1 may be in flight).
  near_load(0);
  far_load(0);
  near_load(1);
  far_load(1);
  wait_and_barrier<2 * kDma8PerWave>();
  __builtin_amdgcn_sched_barrier(0);

  // Fragment sets: F[x] holds one sub-step's 4 A and 2 B fragments.
  uint4 FA[2][4], FB[2][2];
  auto read_sub = [&](int x, int s, int kk) {
    const uint4* sa = smem + (s % kAS) * kSlotChunks;
    const uint4* sb = smem + (kAS + s % kBS) * kSlotChunks;
#pragma unroll
    for (int bm = 0; bm < 4; ++bm) FA[x][bm] = sa[a_off[kk] + bm * 32 * kRowChunks];
#pragma unroll
    for (int bn = 0; bn < 2; ++bn) FB[x][bn] = sb[b_off[kk] + bn * 32 * kRowChunks];
  };
  // A tile's accumulators start as +0.0 registers (the same sums as an MFMA
  // whose C operand is the constant 0).
  floatx16 acc[4][2];
  auto zero_acc = [&]() {
#pragma unroll
    for (int bm = 0; bm < 4; ++bm)
#pragma unroll
      for (int bn = 0; bn < 2; ++bn) acc[bm][bn] = floatx16{};
  };
  // One sub-step: 8 MFMAs on set X; with kRead the reads of the next
  // sub-step (step rs, sub-step rkk, into set X ^ 1) go after the first four
  // MFMAs: A blocks 0 and 1, then A block 2, then B block 0, then A block 3
  // and B block 1 (the last two then have four MFMAs to pass). kDma = 1: the
  // far operand's step s + 2, after the fourth MFMA (its slot, that of step
  // s - 1, was released at the previous barrier); kDma = 2: the near
  // operand's step s + 2, after the second MFMA (into the slot step s
  // released at this step's barrier). At each barrier exactly the far
  // operand's latest four loads may then still be in flight.
  auto sub = [&](auto X, auto read, auto dma, int rs, int rkk, int s) {
    constexpr int x = decltype(X)::value;
    constexpr int kDma = decltype(dma)::value;
    const uint4* sa = smem + (rs % kAS) * kSlotChunks;
    const uint4* sb = smem + (kAS + rs % kBS) * kSlotChunks;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int bm = q >> 1, bn = q & 1;
      Mma<kDtype>::step(acc[bm][bn], FA[x][bm], FB[x][bn]);
      if constexpr (decltype(read)::value) {
        if (q == 0) {
          FA[x ^ 1][0] = sa[a_off[rkk]];
          FA[x ^ 1][1] = sa[a_off[rkk] + 32 * kRowChunks];
        } else if (q == 1) {
          FA[x ^ 1][2] = sa[a_off[rkk] + 2 * 32 * kRowChunks];
        } else if (q == 2) {
          FB[x ^ 1][0] = sb[b_off[rkk]];
        } else if (q == 3) {
          FA[x ^ 1][3] = sa[a_off[rkk] + 3 * 32 * kRowChunks];
          FB[x ^ 1][1] = sb[b_off[rkk] + 32 * kRowChunks];
        }
      }
      if constexpr (kDma == 1) {
        if (q == 3) far_load(s + 2);
      } else if constexpr (kDma == 2) {
        if (q == 1) near_load(s + 2);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using T = std::true_type;
  using F = std::false_type;
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  // K step s; kNext: sub-step 3 reads step s + 1's first fragments (not in a
  // tile's last step: they are read after the epilogue).
  using D0 = std::integral_constant<int, 0>;
  using D1 = std::integral_constant<int, 1>;
  using D2 = std::integral_constant<int, 2>;
  auto k_step = [&](int s, auto next) {
    sub(I0{}, T{}, D1{}, s, 1, s);
    sub(I1{}, T{}, D0{}, s, 2, s);
    sub(I0{}, T{}, D0{}, s, 3, s);
    // step s + 1 landed (the far operand's step s + 2, issued in this step's
    // first sub-step, may be in flight); every wavefront is done reading
    // step s
    wait_and_barrier<kDma8PerWave>();
    __builtin_amdgcn_sched_barrier(0);
    sub(I1{}, next, D2{}, s + 1, 0, s);
  };

  zero_acc();
  read_sub(0, 0, 0);
  int s = 0;
  for (int tile = tile_begin; tile < tile_end; ++tile) {
    for (int ks = 0; ks + 1 < nks; ++ks, ++s) k_step(s, T{});
    k_step(s, F{});
    ++s;
    epi(tile, acc);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    zero_acc();
    if (tile + 1 < tile_end) read_sub(0, s, 0);
  }
  // Every wavefront is done with the LDS ring (and its loads) on return.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

}  // namespace itl
