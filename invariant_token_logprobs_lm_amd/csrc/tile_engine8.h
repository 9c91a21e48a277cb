// Eight-wavefront tile engine (gfx950 / CDNA4): the K loop of the wide bf16
// / fp32 / FP8 contractions (the logprob forward, and the backward's
// dlogits, dH and dW) with two wavefronts per SIMD, on 16 x 16 MFMA blocks.
//
// A 512-thread workgroup multiplies 256-row tiles of an operand A (walked in
// order) with one fixed 256-row block of an operand B, acc = A_tile B^T,
// both row-major and K-contiguous, fp32 accumulate, K ascending in steps of
// 128 bytes, through the five LDS slots, swizzle and direct-to-LDS loads
// of tile_engine.h. Wavefront w = 4 g + r (g = 0, 1, r = 0..3) holds A rows
// 128 (r & 1) .. + 127 of the tile against B rows 64 ((r >> 1) + 2 g) .. +
// 63 of the block, as 8 x 4 blocks of 16 x 16 (Mma16: v_mfma_f32_16x16x32_bf16;
// v_mfma_f32_16x16x4f32 for fp32 operands). The 16 x 16 x 32 instruction
// keeps the matrix cores at a higher clock under the part's power limit
// than the 32 x 32 x 16 one for the same flops (a register-only loop: about
// 2.05 against 1.8 GHz), which is why the blocks are 16 x 16.
//
// MFMA layout: in sub-step kk (0, 1) of a K step lane l supplies row
// (l mod 16) of an A block and of a B block with logical 16-byte chunk
// 4 kk + lane_chunk(l / 16) of the row's 128-byte K step (lane quarters 0,
// 1, 2, 3 take chunks 0, 2, 1, 3; bf16: k = 64 s + 8 chunk .. + 7);
// accumulator register i of lane l holds A row
// 4 (l / 16) + i of the block against B row (l mod 16). Every block takes
// its K step as sub-step 0 then sub-step 1, one instruction each (four for
// fp32), with fresh accumulators at a tile's first step: the same sequence
// as run_tiles_narrow, so an output element has the same bits in both.
//
// Schedule. Waves w and w + 4 share a SIMD (the workgroup's wavefronts go
// to the four SIMDs in a rotating order, w and w + 4 on the same one, as
// read from the hardware-id register), so each SIMD's matrix core is fed by
// two instruction streams and one wavefront's waits are covered by the
// other's MFMAs. A K step is eight sub-steps of 8 MFMAs (K half 0 with A
// blocks 0, 1, then 2, 3, ...; then K half 1 likewise, each pair against
// the four B blocks); each reads, into registers no earlier one still uses,
// the next sub-step's A pair and a share of the B blocks of the next K
// half, so two A pairs and two sets of four B blocks (48 registers) serve
// and the LDS reads are spread over the step. One workgroup barrier per K
// step, in sub-step 6 (after the step's last reads): it publishes step
// s + 1 (every wavefront has waited for its own loads of it) and frees step
// s's slots; the near operand's step s + 2 is loaded into its slot right
// after the barrier (2 % faster than after the next sub-step's first
// MFMAs), and the next step's sub-step 0 loads the far operand's step s + 3
// (its slot was freed one barrier earlier). Every
// wavefront loads rows 32 w .. 32 w + 31 of both operands, four loads of
// each step back to back under one M0 value. The near operand (two slots) is the B block, the
// far one (three slots) the walked A tiles; with kBFar the other way round.
// A tile's last K step leaves the next tile's first fragments unread; they
// are read after the epilogue, which then has those registers.
//
// FP8 (kDtype 2: E4M3 operands, v_mfma_scale_f32_16x16x128_f8f6f4 with
// block scales 1): one instruction takes a block's whole 128-value K step,
// lane l supplying the two 16-byte chunks lane_chunk(l / 16) and
// 4 + lane_chunk(l / 16) of its row (A and B alike, so every product pairs
// the same k). A K step is four sub-steps of 8 MFMAs (A blocks 2 p, 2 p + 1
// against the four B blocks); two A fragments (16 registers), each refilled
// right after its last use, and the four B fragments (32) serve the step.
// The barrier is in sub-step 3 after its second MFMA (the step's last
// read); sub-step 3 then reads step s + 1's A block 0 and, each after its
// last use, its four B fragments. The loads keep the bf16 schedule's
// places: the far operand's step s + 2 in sub-step 0, the near operand's
// right after the barrier (after the side load, if any).
//
// side(t, lds, chunk), if given, is called in tile t's last K step right
// after the barrier: the far operand's slot of that step is free from there
// until the next step's sub-step 0, and this wavefront's own rows of it
// (4 KiB at LDS byte address lds, smem chunk index chunk) are written by no
// other wavefront's loads; side may fill them with loads into LDS (the
// epilogue may read them once it has waited for them: the step issues
// kDma8PerWave more loads after side returns).
#pragma once

#include <type_traits>

#include "device_common.h"
#include "itl_config.h"
#include "tile_engine.h"

namespace itl {

constexpr int kDma8PerWave = 4;  // loads per wavefront per K step of each operand (32 rows)

struct Lanes8 {
  int lane, wave, grp, r, wv, tq, quad, c16;
};

__device__ __forceinline__ Lanes8 lanes8() {
  Lanes8 L;
  L.lane = threadIdx.x & 63;
  L.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  L.grp = L.wave >> 2;
  L.r = L.wave & 3;
  L.wv = L.r & 1;                     // which 128 rows of the A tile
  L.tq = (L.r >> 1) | (L.grp << 1);   // which 64 rows of the B block
  L.quad = L.lane >> 4;               // which 4 rows of each 16-row A block the accumulators hold
  L.c16 = L.lane & 15;                // which row of each 16-row B block
  return L;
}

// Runs tiles tile_begin .. tile_end - 1 (tile_end > tile_begin): a_rsrc(t)
// is A tile t's buffer resource (its first row at offset 0, its valid rows'
// bytes as the range: rows past it load as zeros), b_rsrc the B block's;
// rows are row_bytes apart; nks K steps of 128 bytes (nks >= 1,
// nks * 128 <= row_bytes). epi(t, acc) sees tile t's accumulators
// acc[bm][bn] (A rows 16 bm + 4 quad + i, B row 16 bn + c16 of the
// wavefront's 128 x 64); it may read them directly. Every thread of the
// 512-thread workgroup must call this.
template <int kDtype, bool kBFar, class ARsrc, class Epi, class Side>
__device__ __forceinline__ void run_tiles8(uint4* smem, const Lanes8& L, int row_bytes, int tile_begin, int tile_end,
                                           int nks, const ARsrc& a_rsrc, int4v b_rsrc, Epi&& epi, Side&& side) {
  constexpr int kAS = kBFar ? kHSlots : kWSlots;  // slots of A
  constexpr int kBS = kBFar ? kWSlots : kHSlots;  // slots of B
  static_assert(kAS + kBS == 5 && (kAS == 2 || kAS == 3), "five slots: two near, three far");
  const int lane = L.lane, wave = L.wave, quad = L.quad, c16 = L.c16;

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
  // The four loads of step s of A / of B into its slot; each operand's
  // loads come in step order, so the step's (tile, K step) is kept as a
  // running count (no division). A step past the end loads the last step's
  // data instead (a valid address) into slot s, which is free and which
  // nothing reads again.
  int a_tile = tile_begin, a_ks = 0, b_ks = 0, b_left = (tile_end - tile_begin) * nks;
  auto a_load = [&](int s) {
    dma16x4(a_rsrc(a_tile), voff, (uint32_t)a_ks * kStepBytes, lds0 + (uint32_t)(s % kAS) * kSlotBytes + my_rows);
    if (a_ks + 1 < nks) ++a_ks;
    else if (a_tile + 1 < tile_end) a_ks = 0, ++a_tile;
    a_ks = __builtin_amdgcn_readfirstlane(a_ks);  // wave-uniform: kept in SGPRs
    a_tile = __builtin_amdgcn_readfirstlane(a_tile);
  };
  auto b_load = [&](int s) {
    dma16x4(b_rsrc, voff, (uint32_t)b_ks * kStepBytes, lds0 + (uint32_t)(kAS + s % kBS) * kSlotBytes + my_rows);
    if (--b_left > 0) b_ks = b_ks + 1 < nks ? b_ks + 1 : 0;
    b_ks = __builtin_amdgcn_readfirstlane(b_ks);
  };

  // MFMA operand reads of sub-step kk: A rows 128 wv + 16 bm + (l mod 16),
  // B rows 64 tq + 16 bn + (l mod 16), logical chunk 4 kk +
  // lane_chunk(l / 16) (the swizzle of a row depends on its low four bits
  // only).
  int a_off[2], b_off[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int pc = (4 * kk + lane_chunk(quad)) ^ swz(c16);
    a_off[kk] = (L.wv * 128 + c16) * kRowChunks + pc;
    b_off[kk] = (L.tq * 64 + c16) * kRowChunks + pc;
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
  // This wavefront's rows of the far operand's slot of step s: LDS byte
  // address and smem chunk index.
  auto far_rows = [&](int s) {
    const int slot = kAS == 2 ? kAS + s % kBS : s % kAS;
    return slot * kSlotChunks + wave * 32 * kRowChunks;
  };

  // Prologue: near and far steps 0 and 1, in that order; then step 0 is
  // published (step 1 may be in flight).
  near_load(0);
  far_load(0);
  near_load(1);
  far_load(1);
  wait_and_barrier<2 * kDma8PerWave>();
  __builtin_amdgcn_sched_barrier(0);

  // Fragments: FA[x][b] A block 2 p + b of a sub-step's pair p (x = p mod
  // 2), FB[kk][bn] B block bn of K half kk.
  uint4 FA[2][2], FB[2][4];
  auto read_a = [&](int s, int kk, int bm) {
    FA[(bm >> 1) & 1][bm & 1] = smem[(s % kAS) * kSlotChunks + a_off[kk] + bm * 16 * kRowChunks];
  };
  auto read_b = [&](int s, int kk, int bn) {
    FB[kk][bn] = smem[(kAS + s % kBS) * kSlotChunks + b_off[kk] + bn * 16 * kRowChunks];
  };
  // A tile's accumulators start as +0.0 registers (the same sums as an MFMA
  // whose C operand is the constant 0).
  floatx4 acc[8][4];
  auto zero_acc = [&]() {
#pragma unroll
    for (int bm = 0; bm < 8; ++bm)
#pragma unroll
      for (int bn = 0; bn < 4; ++bn) acc[bm][bn] = floatx4{};
  };
  // Sub-step j (0..7) of K step s: K half kk = j / 4, A blocks 2 p and
  // 2 p + 1 (p = j mod 4) against the four B blocks, 8 MFMAs (MFMA q on A
  // block 2 p + q / 4 and B block q mod 4). It reads what later sub-steps
  // need into registers no earlier one still uses: the next sub-step's A
  // pair (after its MFMAs 0 and 1) and, in sub-steps 0-3, B block j of half
  // 1 (after MFMA 2). Sub-step 6's A pair is the step's last read; the
  // barrier that publishes step s + 1 follows after MFMA 5, then B blocks
  // 0, 1 of step s + 1's half 0; sub-step 7 reads step s + 1's first A pair
  // and its B blocks 2, 3. A tile's last step (kNext false) leaves step s + 1's reads to the
  // code after the epilogue. Loads: the far operand's step s + 2 in
  // sub-step 0 (its slot, that of step s - 1, was released at the previous
  // barrier), the near operand's step s + 2 right after this step's barrier
  // (into the slot step s released there). At each barrier exactly the far
  // operand's latest four loads may then still be in flight.
  auto sub = [&](auto J, auto next, int s) {
    constexpr int j = decltype(J)::value;
    constexpr int kk = j >> 2, p = j & 3;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int b = q >> 2, bn = q & 3;
      if constexpr (kDtype != 2) Mma16<kDtype>::step(acc[2 * p + b][bn], FA[p & 1][b], FB[kk][bn]);
      if constexpr (j < 6) {
        // the next sub-step's A pair, then (sub-steps 0-3) B block j of
        // half 1
        if (q < 2) read_a(s, (j + 1) >> 2, 2 * ((j + 1) & 3) + q);
        if (j < 4 && q == 2) read_b(s, 1, j);
      } else if constexpr (j == 6) {
        if (q < 2) read_a(s, 1, 6 + q);  // the step's last reads
        if (q == 5) {
          // step s + 1 landed (the far operand's step s + 2 may be in
          // flight); every wavefront is done reading step s, whose near
          // slot takes the near operand's step s + 2 at once
          wait_and_barrier<kDma8PerWave>();
          near_load(s + 2);
        }
        if (decltype(next)::value && q >= 6) read_b(s + 1, 0, q - 6);
      } else {
        if (decltype(next)::value && q < 2) read_a(s + 1, 0, q);
        if (decltype(next)::value && (q == 2 || q == 3)) read_b(s + 1, 0, q);
      }
      if constexpr (j == 0) {
        if (q == 3) far_load(s + 2);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using T = std::true_type;
  using F = std::false_type;
  // K step s; kNext: its last sub-steps read step s + 1's first fragments
  // (not in a tile's last step: they are read after the epilogue).
  auto k_step = [&](int s, auto next) {
    sub(std::integral_constant<int, 0>{}, next, s);
    sub(std::integral_constant<int, 1>{}, next, s);
    sub(std::integral_constant<int, 2>{}, next, s);
    sub(std::integral_constant<int, 3>{}, next, s);
    sub(std::integral_constant<int, 4>{}, next, s);
    sub(std::integral_constant<int, 5>{}, next, s);
    sub(std::integral_constant<int, 6>{}, next, s);
    sub(std::integral_constant<int, 7>{}, next, s);
  };
  // The fragments of a step's first sub-step: A blocks 0, 1 and the B
  // blocks of half 0.
  auto read_first = [&](int s) {
    read_a(s, 0, 0);
    read_a(s, 0, 1);
#pragma unroll
    for (int bn = 0; bn < 4; ++bn) read_b(s, 0, bn);
  };

  // FP8: 32-byte fragments GA[b] (the A block of MFMAs 4 b .. 4 b + 3 of
  // a sub-step: block 2 p + b) and GB[bn]; half h of a fragment is logical
  // chunk 4 h + lane_chunk(l / 16), read at a_off[h] / b_off[h].
  Frag8 GA[2], GB[4];
  auto read_a8 = [&](int s, int bm, int h) {
    const uint4 v = smem[(s % kAS) * kSlotChunks + a_off[h] + bm * 16 * kRowChunks];
    if (h == 0) GA[bm & 1].lo = v;
    else GA[bm & 1].hi = v;
  };
  auto read_b8 = [&](int s, int bn, int h) {
    const uint4 v = smem[(kAS + s % kBS) * kSlotChunks + b_off[h] + bn * 16 * kRowChunks];
    if (h == 0) GB[bn].lo = v;
    else GB[bn].hi = v;
  };
  // FP8 sub-step p (0..3) of K step s: MFMA q on A block 2 p + q / 4 and B
  // block q mod 4. Each A register is refilled right after the MFMAs that
  // use it: A block 2 p + 1 after MFMAs 0, 1 (its register last held block
  // 2 p - 1), block 2 p + 2 after MFMAs 4, 5 (sub-steps 0-2). Sub-step 3
  // meets the barrier after MFMA 1 (its A block 7, read there, is the step's
  // last read), then, with kNext, reads step s + 1's A block 0 (after MFMAs
  // 4, 5) and B block bn after MFMA 4 + bn, its last use.
  auto sub8 = [&](auto P, auto next, int s, int tile) {
    constexpr int p = decltype(P)::value;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      mma_f8_16(acc[2 * p + (q >> 2)][q & 3], GA[q >> 2], GB[q & 3]);
      if (q < 2) read_a8(s, 2 * p + 1, q);
      if constexpr (p < 3) {
        if (q == 4 || q == 5) read_a8(s, 2 * p + 2, q - 4);
      } else {
        if (q == 1) {
          wait_and_barrier<kDma8PerWave>();
          if constexpr (!decltype(next)::value) {
            const int chunk = far_rows(s);
            side(tile, lds0 + (uint32_t)chunk * 16u, chunk);
          }
          near_load(s + 2);
        }
        if constexpr (decltype(next)::value) {
          if (q == 4 || q == 5) read_a8(s + 1, 0, q - 4);
          if (q >= 4) {
            read_b8(s + 1, q - 4, 0);
            read_b8(s + 1, q - 4, 1);
          }
        }
      }
      if constexpr (p == 0) {
        if (q == 3) far_load(s + 2);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto k_step8 = [&](int s, auto next, int tile) {
    sub8(std::integral_constant<int, 0>{}, next, s, tile);
    sub8(std::integral_constant<int, 1>{}, next, s, tile);
    sub8(std::integral_constant<int, 2>{}, next, s, tile);
    sub8(std::integral_constant<int, 3>{}, next, s, tile);
  };
  // A step's first fragments: A block 0 and the B blocks (block 1 comes in
  // sub-step 0).
  auto read_first8 = [&](int s) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      read_a8(s, 0, h);
#pragma unroll
      for (int bn = 0; bn < 4; ++bn) read_b8(s, bn, h);
    }
  };

  zero_acc();
  if constexpr (kDtype == 2) read_first8(0);
  else read_first(0);
  int s = 0;
  for (int tile = tile_begin; tile < tile_end; ++tile) {
    if constexpr (kDtype == 2) {
      for (int ks = 0; ks + 1 < nks; ++ks, ++s) k_step8(s, T{}, tile);
      k_step8(s, F{}, tile);
    } else {
      for (int ks = 0; ks + 1 < nks; ++ks, ++s) k_step(s, T{});
      k_step(s, F{});
    }
    ++s;
    epi(tile, acc);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    zero_acc();
    if (tile + 1 < tile_end) {
      if constexpr (kDtype == 2) read_first8(s);
      else read_first(s);
    }
  }
  // Every wavefront is done with the LDS ring (and its loads) on return.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// run_tiles8 without a side load (the bf16 / fp32 kernels).
template <int kDtype, bool kBFar, class ARsrc, class Epi>
__device__ __forceinline__ void run_tiles8(uint4* smem, const Lanes8& L, int row_bytes, int tile_begin, int tile_end,
                                           int nks, const ARsrc& a_rsrc, int4v b_rsrc, Epi&& epi) {
  run_tiles8<kDtype, kBFar>(smem, L, row_bytes, tile_begin, tile_end, nks, a_rsrc, b_rsrc, epi,
                            [](int, uint32_t, int) {});
}

}  // namespace itl
