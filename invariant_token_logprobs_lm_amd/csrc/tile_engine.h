// Tile engines (gfx950 / CDNA4): the pieces every contraction of the
// library shares (MFMA steps, LDS slots and swizzle, direct-to-LDS loads,
// waits) and the four-wavefront K loops: the narrow one for decode-shaped
// calls and the MXFP4 ones. The bf16 / fp32 / FP8 wide contractions (the
// forward and the backward) run on the eight-wavefront loop of
// tile_engine8.h, which uses the same slots, swizzle and per-block MFMA
// sequence as the narrow loop.
//
// bf16 / fp32 / FP8 blocks are 16 x 16: in sub-step kk (0, 1) of a 128-byte
// K step (Mma16; FP8: the two halves of one mma_f8_16 instruction) lane l
// supplies row (l mod 16) of an A block and of a B block with logical
// 16-byte chunk 4 kk + lane_chunk(l / 16); accumulator register i of lane l
// holds A row 4 (l / 16) + i against B row (l mod 16).
//
// MXFP4 geometry: a 256-thread workgroup (2 x 2 wavefronts)
// multiplies 256-row tiles of an operand A, walked in order, with one fixed
// 256-row block of an operand B: acc = A_tile B^T (both row-major and
// K-contiguous, fp32 accumulate, K ascending in steps of 128 bytes). After
// each tile an epilogue sees the accumulators. Wavefront (wv, wt) holds rows
// 128 wv .. 128 wv + 127 of the A tile against rows 128 wt .. 128 wt + 127
// of the B block, as 4 x 4 blocks of 32 x 32: lane l supplies row (l mod 32)
// of A and of B with the k range chosen by l / 32, and accumulator register
// i of lane l holds A row 8 (i / 4) + 4 (l / 32) + (i mod 4) against B row
// (l mod 32).
//
// Fixed tile shapes, K order and instruction sequence: an output element's
// bits depend only on its A row, its B row and K, never on the launch shape
// or the element's position in the tile (rows past an operand's end are
// loaded as zeros). There is no split-K.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "itl_config.h"

namespace itl {

// One 16-byte fragment per lane and operand feeds one 16 x 16 block for one
// sub-step (32 bf16 or 16 fp32 values of K).
template <int kDtype>
struct Mma16;

template <>
struct Mma16<0> {  // bf16: 8 elements per lane, k32 per instruction
  __device__ static __forceinline__ void step(floatx4& acc, uint4 a, uint4 b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                  acc, 0, 0, 0);
  }
};

template <>
struct Mma16<1> {  // fp32: 4 elements per lane; instruction j takes element j (k4 each)
  __device__ static __forceinline__ void step(floatx4& acc, uint4 a, uint4 b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
};

// A 32-byte FP8 fragment: two 16-byte chunks of one lane.
struct Frag8 {
  uint4 lo, hi;
};

typedef int intx8 __attribute__((ext_vector_type(8)));

// v_mfma_scale_f32_16x16x128_f8f6f4, both operands E4M3, block scales 1
// (E8M0 127): acc += one 16 x 16 block over a whole 128-value K step, lane l
// supplying 32 values of row (l mod 16) of each operand. The instruction
// sums its 128 products as one dot product whatever K values sit in which
// lane (A and B use the same placement), so the result is
// sum_k A[r, k] B[c, k] in a fixed order.
__device__ __forceinline__ void mma_f8_16(floatx4& acc, const Frag8& a, const Frag8& b) {
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(__builtin_bit_cast(intx8, a), __builtin_bit_cast(intx8, b),
                                                         acc, 0, 0, 0, 127, 0, 127);
}

// LDS slots hold one K step of one operand: 256 rows x 128 bytes (8 chunks
// of 16 bytes), so that every global load moves whole 128-byte lines. Five
// slots fill the LDS: one operand rotates through three of them, loaded two
// K steps ahead, the other through two, one step ahead. By default the
// walked operand (A) is the far one (kWSlots = 3, kHSlots = 2); run_tiles8's
// kBFar swaps the roles. Which pays depends on the K loop's length: the
// workgroups sharing an operand segment through an XCD's L2 drift apart
// over a long loop, and the operand that fewer of them share then misses
// L2 more often and needs the longer lead. Chunk c
// of row r sits at position c ^ swz(r): for the MFMA operand reads (lanes
// 0-31 take rows r0..r0+31 at one chunk, lanes 32-63 the next chunk) any 8
// or 16 consecutive lanes then touch distinct 16-byte bank groups.
constexpr int kRowChunks = kStepBytes / 16;      // 8
constexpr int kSlotChunks = kBV * kRowChunks;    // 2048 chunks = 32 KiB per slot
constexpr int kSlotBytes = kSlotChunks * 16;
constexpr int kDmaRows = 64 * 16 / kStepBytes;   // rows one wavefront-wide 16-byte load fills (8)
constexpr int kDmaPerWave = 64 / kDmaRows;       // loads per operand per wavefront per K step (8)
static_assert(kBV == kBT && kThreads == 256 && kStepBytes == 128 && kWSlots == 3 && kHSlots == 2,
              "the loop below assumes this geometry (5 slots = 160 KiB, all of a CU's LDS)");

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// 16 x 16 blocks: the 16-byte chunk of a sub-step's four that lane quarter
// q = l / 16 supplies (A and B alike, so the instruction still sums the
// sub-step's whole K range). Quarters 0 and 2, and 1 and 3, take chunks
// that differ in bit 0: an LDS read serves lanes 8 g .. 8 g + 7 together
// with lanes 32 + 8 g .. + 7, and with the row swizzle above such pairs hit
// distinct banks (quarters 0 and 2 two chunks apart conflicted: measured).
__device__ __forceinline__ int lane_chunk(int q) { return 2 * (q & 1) + (q >> 1); }

// Raw buffer resource words over [base, base + nbytes) (gfx9-family raw
// buffer: no stride, no swizzle, 32-bit data format). Loads whose row lies
// past nbytes return zeros and touch no memory.
__device__ __forceinline__ int4v rsrc_words(const void* base, uint32_t nbytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return int4v{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), (int)nbytes, 0x00020000};
}

// One wavefront-wide 16-byte-per-lane load from global memory straight into
// LDS: lane i's 16 bytes land at LDS address lds + 16 i. The LDS base goes
// through M0 (saved and restored here, so the compiler's view of M0 holds).
// The load is issued from inline assembly so the compiler does not order
// every later LDS read behind it; the K-step loop waits for it explicitly
// (vmcnt) before the barrier that publishes the K step.
__device__ __forceinline__ void dma16(int4v rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  // The scalar operands are wave-uniform by construction; readfirstlane
  // pins them to SGPRs even where the register allocator parked a copy in
  // a VGPR (a no-op when they already are SGPRs).
  const int4v r = {__builtin_amdgcn_readfirstlane(rsrc[0]), __builtin_amdgcn_readfirstlane(rsrc[1]),
                   __builtin_amdgcn_readfirstlane(rsrc[2]), __builtin_amdgcn_readfirstlane(rsrc[3])};
  const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %4\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(r), "s"(so), "s"(l)
      : "memory");
}

// Four such loads under one M0 value: load j fills LDS lds + 1024 j from
// offset voff_j + 1024 j (the instruction's immediate offset is added to both
// the memory and the LDS address), so the caller passes voff_j - 1024 j.
__device__ __forceinline__ void dma16x4(int4v rsrc, const uint32_t (&voff)[4], uint32_t soff, uint32_t lds) {
  const int4v r = {__builtin_amdgcn_readfirstlane(rsrc[0]), __builtin_amdgcn_readfirstlane(rsrc[1]),
                   __builtin_amdgcn_readfirstlane(rsrc[2]), __builtin_amdgcn_readfirstlane(rsrc[3])};
  const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %7\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %5, %6 offen lds\n\t"
      "buffer_load_dwordx4 %2, %5, %6 offen offset:1024 lds\n\t"
      "buffer_load_dwordx4 %3, %5, %6 offen offset:2048 lds\n\t"
      "buffer_load_dwordx4 %4, %5, %6 offen offset:3072 lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(r), "s"(so), "s"(l)
      : "memory");
}

// Wait until at most kPending of this wavefront's loads are outstanding
// (loads complete in issue order) and its LDS reads are done, then meet the
// other wavefronts.
template <int kPending>
__device__ __forceinline__ void wait_and_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kPending) : "memory");
}

// Copy accumulator register i of a 32x32 MFMA result into a VGPR at this
// point of the program. Issued from inline assembly so that each copy
// happens where it is used; left to the compiler, all 256 copies are made at
// once at the end of the K loop and spill.
__device__ __forceinline__ float acc_read(const floatx16& v, int i) {
  float r;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(v[i]));
  return r;
}

// The accumulator copies above are invisible to the compiler's hazard
// tracking: after the tile's last MFMA (16 passes) a VALU read of its result
// needs wait states. The scheduling barriers keep every MFMA of the tile
// before the wait (the compiler would otherwise sink the last MFMAs below it,
// next to the copies of the registers they write) and every copy after it.
__device__ __forceinline__ void mfma_result_wait() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// z[8 b3 + 4 b2 + 2 b1 + b0] by a tree of selects.
__device__ __forceinline__ float select16(const floatx16& z, bool b0, bool b1, bool b2, bool b3) {
  const float a0 = b0 ? z[1] : z[0], a1 = b0 ? z[3] : z[2], a2 = b0 ? z[5] : z[4], a3 = b0 ? z[7] : z[6];
  const float a4 = b0 ? z[9] : z[8], a5 = b0 ? z[11] : z[10], a6 = b0 ? z[13] : z[12], a7 = b0 ? z[15] : z[14];
  const float c0 = b1 ? a1 : a0, c1 = b1 ? a3 : a2, c2 = b1 ? a5 : a4, c3 = b1 ? a7 : a6;
  const float e0 = b2 ? c1 : c0, e1 = b2 ? c3 : c2;
  return b3 ? e1 : e0;
}

// Lane geometry of the workgroup.
struct Lanes {
  int lane, wave, wv, wt, half, col;
};

__device__ __forceinline__ Lanes lanes() {
  Lanes L;
  L.lane = threadIdx.x & 63;
  L.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  L.wv = L.wave & 1;   // which 128 rows of the A tile
  L.wt = L.wave >> 1;  // which 128 rows of the B block
  L.half = L.lane >> 5;
  L.col = L.lane & 31;
  return L;
}

// LDS the engine needs (uint4 elements): all of a CU's 160 KiB.
constexpr int kEngineSmemChunks = (kWSlots + kHSlots) * kSlotChunks;

// Narrow engine for few B rows (decode-shaped calls): 256-row A tiles
// against a 64-row B block (or 128 rows, below). Wavefront (wv, wt) holds
// rows 128 wv .. 128 wv + 127 of the A tile against B rows 32 wt .. 32 wt +
// 31 as 8 x 2 blocks of 16 x 16. Every MFMA of an accumulator block takes the same operand
// fragments, in the same order, as in the eight-wavefront engine run_tiles8
// (same slot layout and swizzle, same K sub-step order, fresh accumulators
// at a tile's first step), so an output element has the same bits in both.
// The work per A tile is a quarter of the wide engine's: the loop streams A
// from memory, so both operands rotate through four slots and are loaded
// three K steps ahead.
constexpr int kNarrowSlots = 4;
constexpr int kNarrowBSlotChunks = kNarrowBRows * kRowChunks;  // 512 chunks = 8 KiB
constexpr int kNarrowBDmaPerWave = kNarrowBRows / 4 / kDmaRows;  // 2
static_assert(kNarrowSlots * (kSlotChunks + kNarrowBSlotChunks) <= kEngineSmemChunks, "LDS budget");

// kBRows = 64 or 128 token rows per B block: wavefront (wv, wt) holds B rows
// (kBRows / 2) wt .. + kBRows / 2 - 1, as kBRows / 32 blocks per A block.
// The 128-row block (calls of 65 to 128 tokens) has three slots, loaded two
// K steps ahead (four of its slots would not fit the LDS). epi(t, acc) sees
// tile t's accumulators acc[bm][bn] (A rows 16 bm + 4 (l / 16) + i, B row
// 16 bn + (l mod 16) of the wavefront's 128 x kBRows / 2).
template <int kDtype, int kBRows = kNarrowBRows, class ARsrc, class Epi>
__device__ __forceinline__ void run_tiles_narrow(uint4* smem, const Lanes& L, int row_bytes, int tile_begin,
                                                 int tile_end, int nks, const ARsrc& a_rsrc, int4v b_rsrc, Epi&& epi) {
  static_assert(kBRows == 64 || kBRows == 128, "64- or 128-row token blocks");
  constexpr int kBN = kBRows / 32;                      // B blocks per wavefront
  constexpr int kSlots = kBRows == 64 ? kNarrowSlots : 3;
  constexpr int kBSlotChunks = kBRows * kRowChunks;
  constexpr int kBDma = kBRows / 4 / kDmaRows;          // B loads per wavefront per step
  static_assert(kSlots * (kSlotChunks + kBSlotChunks) <= kEngineSmemChunks, "LDS budget");
  const int lane = L.lane, wave = L.wave, wv = L.wv, wt = L.wt;
  const int quad = lane >> 4, c16 = lane & 15;
  // Loader: wavefront w fills A rows 64 w .. 64 w + 63 (8 loads) and B rows
  // (kBRows / 4) w .. + kBRows / 4 - 1 of a slot; lane i fetches row (i / 8)
  // of an 8-row group at logical chunk (i % 8) ^ swz(row), as in every
  // engine here.
  const int lr = lane >> 3;
  uint32_t avoff[kDmaPerWave], bvoff[kBDma];
#pragma unroll
  for (int j = 0; j < kDmaPerWave; ++j)
    avoff[j] = (uint32_t)(wave * 64 + j * kDmaRows + lr) * (uint32_t)row_bytes + (((lane & 7) ^ lr ^ (j & 1)) * 16);
#pragma unroll
  for (int j = 0; j < kBDma; ++j)
    bvoff[j] = (uint32_t)(wave * (kBRows / 4) + j * kDmaRows + lr) * (uint32_t)row_bytes +
               (((lane & 7) ^ lr ^ (j & 1)) * 16);
  const uint32_t lds0 = (uint32_t)(size_t)((__attribute__((address_space(3))) uint4*)smem);
  auto a_lds = [&](int slot) { return lds0 + (uint32_t)slot * kSlotBytes + (uint32_t)wave * 64 * kStepBytes; };
  auto b_lds = [&](int slot) {
    return lds0 + (uint32_t)kSlots * kSlotBytes + (uint32_t)slot * kBSlotChunks * 16 +
           (uint32_t)wave * (kBRows / 4) * kStepBytes;
  };
  // Load K step (tile, ks) of both operands into a slot: B first, then A.
  auto load_step = [&](int tile, int ks, int slot) {
    const int4v ar = a_rsrc(tile);
    const uint32_t so = (uint32_t)ks * kStepBytes;
#pragma unroll
    for (int j = 0; j < kBDma; ++j) dma16(b_rsrc, bvoff[j], so, b_lds(slot) + j * 1024);
#pragma unroll
    for (int j = 0; j < kDmaPerWave; ++j) dma16(ar, avoff[j], so, a_lds(slot) + j * 1024);
  };
  // Loads run over the steps (tile, ks), K fastest, clamped at the last step
  // (a clamped load refills a free slot that nothing reads again).
  int ld_tile = tile_begin, ld_ks = 0;
  auto next_load = [&]() {
    if (++ld_ks == nks) {
      ld_ks = 0;
      if (ld_tile + 1 < tile_end) ++ld_tile;
      else ld_ks = nks - 1;
    }
  };
#pragma unroll
  for (int p = 0; p < kSlots - 1; ++p) {
    load_step(ld_tile, ld_ks, p);
    next_load();
  }
  // MFMA operand reads: row (l mod 16) of each 16-row block at logical chunk
  // 4 kk + lane_chunk(l / 16) of sub-step kk, as in run_tiles8.
  int a_off[2], b_off[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int pc = (4 * kk + lane_chunk(quad)) ^ swz(c16);
    a_off[kk] = (wv * 128 + c16) * kRowChunks + pc;
    b_off[kk] = (wt * (kBRows / 2) + c16) * kRowChunks + pc;
  }
  constexpr int kPending = (kSlots - 2) * (kDmaPerWave + kBDma);
  int slot = 0;
  // One K step.
  auto k_step = [&](floatx4 (&acc)[8][kBN]) {
    // This step's loads landed (the later steps' may be in flight); every
    // wavefront is done reading the previous step's slot.
    wait_and_barrier<kPending>();
    load_step(ld_tile, ld_ks, slot == 0 ? kSlots - 1 : slot - 1);
    next_load();
    const uint4* sa = smem + slot * kSlotChunks;
    const uint4* sb = smem + kSlots * kSlotChunks + slot * kBSlotChunks;
    // All of the step's fragments are read up front (one LDS round trip per
    // step rather than one per sub-step), then its MFMAs.
    uint4 A[2][8], B[2][kBN];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int m = 0; m < 8; ++m) A[kk][m] = sa[a_off[kk] + m * 16 * kRowChunks];
#pragma unroll
      for (int n = 0; n < kBN; ++n) B[kk][n] = sb[b_off[kk] + n * 16 * kRowChunks];
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kDtype == 2) {
      // FP8: one instruction per block and step, on the two halves' chunks
      // (the fragments of run_tiles8's FP8 schedule)
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int n = 0; n < kBN; ++n) mma_f8_16(acc[m][n], Frag8{A[0][m], A[1][m]}, Frag8{B[0][n], B[1][n]});
    } else {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
          for (int n = 0; n < kBN; ++n) Mma16<kDtype>::step(acc[m][n], A[kk][m], B[kk][n]);
    }
    slot = slot == kSlots - 1 ? 0 : slot + 1;
  };
  for (int tile = tile_begin; tile < tile_end; ++tile) {
    // A tile's accumulators start as +0.0 registers, as in run_tiles8.
    floatx4 acc[8][kBN];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int n = 0; n < kBN; ++n) acc[m][n] = floatx4{};
    for (int ks = 0; ks < nks; ++ks) k_step(acc);
    epi(tile, acc);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// MXFP4-weight variant (A = W in OCP MXFP4: E2M1 codes, two per byte, one
// E8M0 scale per 32 values along K; B = H in E4M3), on
// v_mfma_scale_f32_32x32x64_f8f6f4 with A in FP4 format and the A block
// scales applied by the instruction. A K step is 128 values: 64 bytes of W
// and 4 scale bytes per W row, 128 bytes of H per H row; two sub-steps of
// 64. Lane half h of sub-step j carries W values 64 j + 32 h .. + 31 (one
// 16-byte chunk, one MX block, the lane's scale byte) and the H values the
// instruction pairs with them: 16-byte chunks 4 j + h and 4 j + 2 + h of
// the H row segment (the FP4 operand's halves pair with the FP8 operand's
// chunks that way: a measured property of the instruction).
//
// LDS: W slots of 256 rows x 64 bytes (chunk c of row r at c ^ ((r >> 1) & 3)
// so that 8 consecutive rows at one chunk hit distinct 16-byte bank groups)
// followed by the slot's 256 x 4 scale bytes; H slots of 256 rows x 128 bytes as in the
// other engines.
constexpr int kMx4RowChunks = 4;                        // 64-byte W rows
constexpr int kMx4WDataBytes = kBV * 64;                // 16 KiB
constexpr int kMx4WSlotBytes = kMx4WDataBytes + kBV * 4;  // + 1 KiB of scales
constexpr int kMx4HBase = kWSlots * kMx4WSlotBytes;     // H slots after the W slots
constexpr int kMx4WDataLoads = kBV * 64 / 1024 / 4;     // wavefront-wide loads per wavefront per step (4)
constexpr int kMx4WLoads = kMx4WDataLoads + 1;          // + one 4-byte-per-lane load of scales
static_assert(kMx4HBase + kHSlots * kSlotBytes <= kEngineSmemChunks * 16, "LDS budget");
static_assert(kMx4WSlotBytes % 16 == 0, "slot alignment");

__device__ __forceinline__ int swz4(int r) { return (r >> 1) & 3; }

// As dma16, 4 bytes per lane: lane i's dword lands at LDS address lds + 4 i.
__device__ __forceinline__ void dma4(int4v rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  const int4v r = {__builtin_amdgcn_readfirstlane(rsrc[0]), __builtin_amdgcn_readfirstlane(rsrc[1]),
                   __builtin_amdgcn_readfirstlane(rsrc[2]), __builtin_amdgcn_readfirstlane(rsrc[3])};
  const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %4\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, %3 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(r), "s"(so), "s"(l)
      : "memory");
}

__device__ __forceinline__ void mma_mx4(floatx16& acc, const uint4& a, const Frag8& b, int scale_a) {
  const intx8 av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, __builtin_bit_cast(intx8, b), acc, 4, 0, 0, scale_a, 0,
                                                        127);
}
__device__ __forceinline__ void mma_mx4_first(floatx16& acc, const uint4& a, const Frag8& b, int scale_a) {
  const intx8 av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, __builtin_bit_cast(intx8, b), floatx16{}, 4, 0, 0,
                                                        scale_a, 0, 127);
}

// a_rsrc(t) / s_rsrc(t): W codes and W scale bytes of tile t (rows at
// w_row_bytes and s_row_bytes apart); b_rsrc: the H block (rows at
// h_row_bytes). nks K steps of 128 values.
template <class ARsrc, class SRsrc, class Epi>
__device__ __forceinline__ void run_tiles_mx4(uint4* smem, const Lanes& L, int w_row_bytes, int s_row_bytes,
                                              int h_row_bytes, int tile_begin, int tile_end, int nks,
                                              const ARsrc& a_rsrc, const SRsrc& s_rsrc, int4v b_rsrc, Epi&& epi) {
  const int lane = L.lane, wave = L.wave, wv = L.wv, wt = L.wt, half = L.half, col = L.col;
  const int lr = lane >> 3;
  // H loads: rows 64 wave + 8 j + lane / 8, logical chunk (lane % 8) ^ swz(row).
  uint32_t hvoff[kDmaPerWave];
#pragma unroll
  for (int j = 0; j < kDmaPerWave; ++j)
    hvoff[j] = (uint32_t)(wave * 64 + j * kDmaRows + lr) * (uint32_t)h_row_bytes + (((lane & 7) ^ lr ^ (j & 1)) * 16);
  // W code loads: rows 64 wave + 16 j + lane / 4, logical chunk (lane % 4) ^ swz4(row).
  uint32_t wvoff[kMx4WDataLoads];
#pragma unroll
  for (int j = 0; j < kMx4WDataLoads; ++j) {
    const int row = wave * 64 + j * 16 + (lane >> 2);
    wvoff[j] = (uint32_t)row * (uint32_t)w_row_bytes + (uint32_t)(((lane & 3) ^ swz4(row)) * 16);
  }
  // W scale loads: row 64 wave + lane, the step's 4 bytes.
  const uint32_t svoff = (uint32_t)(wave * 64 + lane) * (uint32_t)s_row_bytes;
  const uint32_t lds0 = (uint32_t)(size_t)((__attribute__((address_space(3))) uint4*)smem);
  auto w_slot = [&](int slot) { return lds0 + (uint32_t)slot * kMx4WSlotBytes; };
  auto h_slot = [&](int slot) { return lds0 + (uint32_t)kMx4HBase + (uint32_t)slot * kSlotBytes; };
  const int4v hr = b_rsrc;

  // Fragment offsets (uint4 units from a slot's base): A chunk 2 j + half of
  // row 128 wv + 32 m + col; B chunks 4 j + half and 4 j + 2 + half of row
  // 128 wt + 32 m + col; the scale dword of row 128 wv + 32 m + col.
  int a_off[2], b_off[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int ra = wv * 128 + col;
    a_off[j] = ra * kMx4RowChunks + ((2 * j + half) ^ swz4(ra));
#pragma unroll
    for (int p = 0; p < 2; ++p) b_off[j][p] = (wt * 128 + col) * kRowChunks + ((4 * j + 2 * p + half) ^ swz(col));
  }
  // swz4 of rows 128 wv + 32 m + col equals swz4(col + 32 m + 128 wv) = swz4(col)
  // only when 32 m + 128 wv keeps bits 1-2: it does (multiples of 32).

  int w_tile = tile_begin, w_ks = 0;
  int h_ks = 0;
  int w_slot_next = 0, h_slot_next = 0;
  auto next_w = [&]() {
    if (++w_ks == nks) {
      w_ks = 0;
      w_tile = min(w_tile + 1, tile_end - 1);
    }
    w_slot_next = w_slot_next == kWSlots - 1 ? 0 : w_slot_next + 1;
  };
  auto next_h = [&]() {
    h_ks = h_ks + 1 == nks ? 0 : h_ks + 1;
    h_slot_next ^= 1;
  };
  auto load_w = [&](int slot) {  // W(w_tile, w_ks): codes then scales
    const int4v ar = a_rsrc(w_tile);
    const int4v sr = s_rsrc(w_tile);
    const uint32_t base = w_slot(slot) + (uint32_t)wave * 64 * 64;
#pragma unroll
    for (int j = 0; j < kMx4WDataLoads; ++j) dma16(ar, wvoff[j], (uint32_t)w_ks * 64, base + j * 1024);
    dma4(sr, svoff, (uint32_t)w_ks * 4, w_slot(slot) + kMx4WDataBytes + (uint32_t)wave * 256);
  };
  auto load_h = [&](int slot) {
    const uint32_t base = h_slot(slot) + (uint32_t)wave * 64 * kStepBytes;
#pragma unroll
    for (int j = 0; j < kDmaPerWave; ++j) dma16(hr, hvoff[j], (uint32_t)h_ks * kStepBytes, base + j * 1024);
  };

  // One sub-step: MFMA q (q = 4 bm + bn) with A[bm] (scale byte of sub-step
  // sj from SC[bm]), B[bn]; the 12 reads of the next sub-step (A0 B0 B1 B2
  // B3 A1 A2 A3, B in two halves) from slots (wsl, hsl), sub-step rj, one
  // per MFMA (kFront: in the first 12 MFMAs, the same), plus with kScales the
  // 4 scale dwords of the next step into NSC, and with kDma the loads of
  // H(g + 2) and W(g + 3), one per MFMA.
  auto phase = [&](floatx16 (&acc)[4][4], const uint4 (&A)[4], const Frag8 (&B)[4], const uint32_t (&SC)[4], int sj,
                   auto first, auto scales, auto dma, int wsl, int hsl, int rj, uint4 (&RA)[4], Frag8 (&RB)[4],
                   uint32_t (&NSC)[4]) {
    const uint4* sa = smem + (wsl * kMx4WSlotBytes) / 16;
    const uint32_t* ss = reinterpret_cast<const uint32_t*>(smem) + (wsl * kMx4WSlotBytes + kMx4WDataBytes) / 4;
    const uint4* sb = smem + (kMx4HBase + hsl * kSlotBytes) / 16;
    auto read = [&](int r) {
      if (r == 0) RA[0] = sa[a_off[rj]];
      else if (r <= 8) {
        const int f = (r - 1) >> 1, p = (r - 1) & 1;
        (p ? RB[f].hi : RB[f].lo) = sb[b_off[rj][p] + f * 32 * kRowChunks];
      } else RA[r - 8] = sa[a_off[rj] + (r - 8) * 32 * kMx4RowChunks];
    };
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int sa_byte = (int)((SC[q >> 2] >> (8 * (2 * sj + half))) & 0xffu);
      if constexpr (decltype(first)::value) mma_mx4_first(acc[q >> 2][q & 3], A[q >> 2], B[q & 3], sa_byte);
      else mma_mx4(acc[q >> 2][q & 3], A[q >> 2], B[q & 3], sa_byte);
      if (q < 12) read(q);
      if constexpr (decltype(scales)::value) {
        if (q >= 12) NSC[q - 12] = ss[wv * 128 + (q - 12) * 32 + col];
      }
      if constexpr (decltype(dma)::value) {
        if (q < 8) {
          dma16(hr, hvoff[q], (uint32_t)h_ks * kStepBytes, h_slot(h_slot_next) + (uint32_t)wave * 64 * kStepBytes + q * 1024);
        } else if (q < 8 + kMx4WDataLoads) {
          const int j = q - 8;
          dma16(a_rsrc(w_tile), wvoff[j], (uint32_t)w_ks * 64, w_slot(w_slot_next) + (uint32_t)wave * 64 * 64 + j * 1024);
        } else if (q == 8 + kMx4WDataLoads) {
          dma4(s_rsrc(w_tile), svoff, (uint32_t)w_ks * 4, w_slot(w_slot_next) + kMx4WDataBytes + (uint32_t)wave * 256);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (decltype(dma)::value) {
      next_h();
      next_w();
    }
  };

  using T = std::true_type;
  using F = std::false_type;
  load_w(0);
  load_h(0);
  next_w();
  next_h();
  load_w(1);
  next_w();
  wait_and_barrier<kMx4WLoads>();  // W(0), H(0) landed
  load_h(h_slot_next);
  load_w(w_slot_next);
  next_h();
  next_w();
  uint4 xa[4], ya[4];
  Frag8 xb[4], yb[4];
  uint32_t sc[4], nsc[4];
  {
    const uint4* sa = smem;
    const uint32_t* ss = reinterpret_cast<const uint32_t*>(smem) + kMx4WDataBytes / 4;
    const uint4* sb = smem + kMx4HBase / 16;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      xa[m] = sa[a_off[0] + m * 32 * kMx4RowChunks];
      xb[m].lo = sb[b_off[0][0] + m * 32 * kRowChunks];
      xb[m].hi = sb[b_off[0][1] + m * 32 * kRowChunks];
      sc[m] = ss[wv * 128 + m * 32 + col];
    }
  }
  int wslot = 0, hslot = 0;
  auto k_step = [&](floatx16 (&acc)[4][4], auto first) {
    phase(acc, xa, xb, sc, 0, first, F{}, F{}, wslot, hslot, 1, ya, yb, nsc);
    wait_and_barrier<kMx4WLoads>();  // W(g + 1), H(g + 1) landed; W(g + 2) may still be in flight
    wslot = wslot == kWSlots - 1 ? 0 : wslot + 1;
    hslot ^= 1;
    phase(acc, ya, yb, sc, 1, F{}, T{}, T{}, wslot, hslot, 0, xa, xb, nsc);
#pragma unroll
    for (int m = 0; m < 4; ++m) sc[m] = nsc[m];
  };
  for (int tile = tile_begin; tile < tile_end; ++tile) {
    floatx16 acc[4][4];
    k_step(acc, T{});
    for (int ks = 1; ks < nks; ++ks) k_step(acc, F{});
    epi(tile, acc);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// Narrow variant of run_tiles_mx4 for decode-shaped calls: the same W tiles
// against a block of kBRows (64 or 128) E4M3 token rows, wavefront (wv, wt)
// = 128 W rows x kBRows / 2 token rows (kBRows / 64 column blocks of 32).
// Every MFMA of an accumulator takes the same fragments and scale bytes, in
// the same order, as in the wide engine (same W slot layout and swizzle,
// same H chunk choice, same sub-step order), so each output element has the
// same bits. Both operands rotate through 4 slots, loaded three K steps
// ahead; all of a step's fragments are read up front.
template <int kBRows, class ARsrc, class SRsrc, class Epi>
__device__ __forceinline__ void run_tiles_narrow_mx4(uint4* smem, const Lanes& L, int w_row_bytes, int s_row_bytes,
                                                     int h_row_bytes, int tile_begin, int tile_end, int nks,
                                                     const ARsrc& a_rsrc, const SRsrc& s_rsrc, int4v b_rsrc,
                                                     Epi&& epi) {
  const int lane = L.lane, wave = L.wave, wv = L.wv, wt = L.wt, half = L.half, col = L.col;
  const int lr = lane >> 3;
  static_assert(kBRows == 64 || kBRows == 128, "token block of 64 or 128 rows");
  constexpr int kBN = kBRows / 64;                     // 32-row column blocks per wavefront
  constexpr int kBDma = kBRows / 4 / kDmaRows;         // token-row loads per wavefront per step
  constexpr int kBSlotChunks = kBRows * kRowChunks;
  constexpr int kLoads = kMx4WDataLoads + 1 + kBDma;  // loads per wavefront per step
  constexpr int kHBase = kNarrowSlots * kMx4WSlotBytes;
  static_assert(kHBase + kNarrowSlots * kBSlotChunks * 16 <= kEngineSmemChunks * 16, "LDS budget");
  uint32_t wvoff[kMx4WDataLoads];
#pragma unroll
  for (int j = 0; j < kMx4WDataLoads; ++j) {
    const int row = wave * 64 + j * 16 + (lane >> 2);
    wvoff[j] = (uint32_t)row * (uint32_t)w_row_bytes + (uint32_t)(((lane & 3) ^ swz4(row)) * 16);
  }
  const uint32_t svoff = (uint32_t)(wave * 64 + lane) * (uint32_t)s_row_bytes;
  uint32_t hvoff[kBDma];
#pragma unroll
  for (int j = 0; j < kBDma; ++j)
    hvoff[j] = (uint32_t)(wave * (kBRows / 4) + j * kDmaRows + lr) * (uint32_t)h_row_bytes +
               (((lane & 7) ^ lr ^ (j & 1)) * 16);
  const uint32_t lds0 = (uint32_t)(size_t)((__attribute__((address_space(3))) uint4*)smem);
  auto w_slot = [&](int slot) { return lds0 + (uint32_t)slot * kMx4WSlotBytes; };
  auto h_slot = [&](int slot) { return lds0 + (uint32_t)kHBase + (uint32_t)slot * kBSlotChunks * 16; };
  constexpr uint32_t kWStepBytes = 64;  // W bytes per row per K step
  auto load_step = [&](int tile, int ks, int slot) {
    const int4v ar = a_rsrc(tile);
#pragma unroll
    for (int j = 0; j < kBDma; ++j)
      dma16(b_rsrc, hvoff[j], (uint32_t)ks * kStepBytes,
            h_slot(slot) + (uint32_t)wave * (kBRows / 4) * kStepBytes + j * 1024);
#pragma unroll
    for (int j = 0; j < kMx4WDataLoads; ++j)
      dma16(ar, wvoff[j], (uint32_t)ks * kWStepBytes, w_slot(slot) + (uint32_t)wave * 64 * kWStepBytes + j * 1024);
    dma4(s_rsrc(tile), svoff, (uint32_t)ks * 4, w_slot(slot) + kMx4WDataBytes + (uint32_t)wave * 256);
  };
  int ld_tile = tile_begin, ld_ks = 0;
  auto next_load = [&]() {
    if (++ld_ks == nks) {
      ld_ks = 0;
      if (ld_tile + 1 < tile_end) ++ld_tile;
      else ld_ks = nks - 1;
    }
  };
#pragma unroll
  for (int p = 0; p < kNarrowSlots - 1; ++p) {
    load_step(ld_tile, ld_ks, p);
    next_load();
  }
  // Fragment offsets (uint4 units from a slot's base), as in run_tiles_mx4.
  int a_off[2], b_off[kBN][2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int ra = wv * 128 + col;
    a_off[j] = ra * kMx4RowChunks + ((2 * j + half) ^ swz4(ra));
#pragma unroll
    for (int n = 0; n < kBN; ++n)
#pragma unroll
      for (int p = 0; p < 2; ++p)
        b_off[n][j][p] = (wt * (kBRows / 2) + n * 32 + col) * kRowChunks + ((4 * j + 2 * p + half) ^ swz(col));
  }
  constexpr int kPending = (kNarrowSlots - 2) * kLoads;
  int slot = 0;
  auto k_step = [&](floatx16 (&acc)[4][kBN], auto first) {
    wait_and_barrier<kPending>();
    load_step(ld_tile, ld_ks, slot == 0 ? kNarrowSlots - 1 : slot - 1);
    next_load();
    const uint4* sa = smem + (slot * kMx4WSlotBytes) / 16;
    const uint4* sb = smem + (kHBase + slot * kBSlotChunks * 16) / 16;
    uint4 A[2][4];
    Frag8 B[2][kBN];
    uint32_t SC[4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int m = 0; m < 4; ++m) A[j][m] = sa[a_off[j] + m * 32 * kMx4RowChunks];
#pragma unroll
      for (int n = 0; n < kBN; ++n) {
        B[j][n].lo = sb[b_off[n][j][0]];
        B[j][n].hi = sb[b_off[n][j][1]];
      }
    }
    const uint32_t* ss = reinterpret_cast<const uint32_t*>(smem) + (slot * kMx4WSlotBytes + kMx4WDataBytes) / 4;
#pragma unroll
    for (int m = 0; m < 4; ++m) SC[m] = ss[wv * 128 + m * 32 + col];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int sbyte = (int)((SC[m] >> (8 * (2 * j + half))) & 0xffu);
#pragma unroll
        for (int n = 0; n < kBN; ++n) {
          if (decltype(first)::value && j == 0) mma_mx4_first(acc[m][n], A[j][m], B[j][n], sbyte);
          else mma_mx4(acc[m][n], A[j][m], B[j][n], sbyte);
        }
      }
    slot = slot == kNarrowSlots - 1 ? 0 : slot + 1;
  };
  using T = std::true_type;
  using F = std::false_type;
  for (int tile = tile_begin; tile < tile_end; ++tile) {
    floatx16 acc[4][kBN];
    k_step(acc, T{});
    for (int ks = 1; ks < nks; ++ks) k_step(acc, F{});
    epi(tile, acc);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

}  // namespace itl
