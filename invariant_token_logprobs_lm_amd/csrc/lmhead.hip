// Fused LM-head contraction + online log-sum-exp + sampled-token gather.
//
// What is computed ("vLLM says aligned kernels make asynchronous RL stable at
// lag 64", section "REINFORCE Zero removes the mismatch first": the logprob
// of each sampled token; "vLLM Train-Inference Consistency Release Notes",
// section "Achieving Bitwise Consistency": deterministic, batch-independent
// and phase-consistent):
//
//   z[t, v]    = sum_k H[t, k] W[v, k]         fp32 accumulate, ascending k
//   lse[t]     = log sum_v exp(z[t, v])
//   logprob[t] = z[t, y_t] - lse[t]
//
// Kernel 1 (lmhead_lse_partial) computes z^T tiles on the matrix cores: the
// MFMA A operand is a 256-row tile of W, the B operand a 256-token block of
// H, both read K-contiguous. A workgroup owns one token block and one
// vocabulary slice of kTilesPerSlice tiles and walks the slice's tiles in
// ascending order; after each tile its lanes fold the tile into a running
// (max, sum of exp) per token and pick out z[t, y_t] if y_t falls in the
// tile. The logits never leave registers. At the end of the slice the two
// lane halves and the two wavefronts that share a token are merged in a
// fixed order and one (max, sumexp) pair per (slice, token) is written.
// Kernel 2 (lse_combine) merges a token's slice partials in slice order.
//
// Why the bits do not depend on the batch: the tile shapes, K order, slice
// width and every reduction tree are compile-time constants; a token's
// column is computed by the same instruction sequence whatever its position
// in the block, and rows beyond n_tok are loaded as zeros and never written.
// There is no split-K and no atomic.
//
// MFMA layouts used (v_mfma_f32_32x32x16_bf16, and v_mfma_f32_32x32x2f32 for
// fp32 heads): lane l supplies row (l mod 32) of A and column (l mod 32) of
// B, with the k range chosen by l / 32; accumulator register i of lane l
// holds row 8*(i/4) + 4*(l/32) + (i mod 4), column (l mod 32).

#include <type_traits>

#include "device_common.h"
#include "itl_config.h"
#include "itl_launch.h"

namespace itl {

namespace {

// One 16-byte fragment per lane and operand feeds one K sub-step. first()
// starts a tile's accumulation from zero (the MFMA takes a zero C operand).
template <int kDtype>
struct Mma;

template <>
struct Mma<0> {  // bf16: 8 elements per lane, k16 per instruction
  __device__ static __forceinline__ void step(floatx16& acc, uint4 a, uint4 b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  }
  __device__ static __forceinline__ void first(floatx16& acc, uint4 a, uint4 b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), floatx16{}, 0, 0, 0);
  }
};

template <>
struct Mma<1> {  // fp32: 4 elements per lane; instruction j takes element j (k2 each)
  __device__ static __forceinline__ void step(floatx16& acc, uint4 a, uint4 b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
  __device__ static __forceinline__ void first(floatx16& acc, uint4 a, uint4 b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), floatx16{}, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
};

// LDS slots hold one K step of one operand: 256 rows x 128 bytes (8 chunks
// of 16 bytes), so that every global load moves whole 128-byte lines. W
// tiles rotate through kWSlots slots and are loaded two K steps ahead; H
// blocks rotate through kHSlots slots, one step ahead (an H block is shared
// by more of the workgroups running together on an XCD, so its lines are
// more often in L2). Chunk c of row r sits at position c ^ swz(r): for the
// MFMA operand reads (lanes 0-31 take rows r0..r0+31 at one chunk, lanes
// 32-63 the next chunk) any 8 or 16 consecutive lanes then touch distinct
// 16-byte bank groups.
constexpr int kRowChunks = kStepBytes / 16;      // 8
constexpr int kSlotChunks = kBV * kRowChunks;    // 2048 chunks = 32 KiB per slot
constexpr int kSlotBytes = kSlotChunks * 16;
constexpr int kDmaRows = 64 * 16 / kStepBytes;   // rows one wavefront-wide 16-byte load fills (8)
constexpr int kDmaPerWave = 64 / kDmaRows;       // loads per operand per wavefront per K step (8)
static_assert(kBV == kBT && kThreads == 256 && kStepBytes == 128 && kWSlots == 3 && kHSlots == 2,
              "the loop below assumes this geometry (5 slots = 160 KiB, all of a CU's LDS)");

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

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
// tracking: give the last MFMA (16 passes) the wait states a VALU read of
// its result needs before the first copy.
__device__ __forceinline__ void mfma_result_wait() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// z[8 b3 + 4 b2 + 2 b1 + b0] by a tree of selects.
__device__ __forceinline__ float select16(const floatx16& z, bool b0, bool b1, bool b2, bool b3) {
  const float a0 = b0 ? z[1] : z[0], a1 = b0 ? z[3] : z[2], a2 = b0 ? z[5] : z[4], a3 = b0 ? z[7] : z[6];
  const float a4 = b0 ? z[9] : z[8], a5 = b0 ? z[11] : z[10], a6 = b0 ? z[13] : z[12], a7 = b0 ? z[15] : z[14];
  const float c0 = b1 ? a1 : a0, c1 = b1 ? a3 : a2, c2 = b1 ? a5 : a4, c3 = b1 ? a7 : a6;
  const float e0 = b2 ? c1 : c0, e1 = b2 ? c3 : c2;
  return b3 ? e1 : e0;
}

template <int kDtype>
__global__ __launch_bounds__(kThreads, 1) void lmhead_lse_partial_kernel(
    const char* __restrict__ H, const char* __restrict__ W, const int32_t* __restrict__ tokens, int n_tok,
    int row_bytes, int vocab, int n_tb, int n_slices, float2* __restrict__ part, float* __restrict__ zy_out) {
  __shared__ uint4 smem[(kWSlots + kHSlots) * kSlotChunks];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wv = wave & 1;   // which 128 vocabulary rows of the tile
  const int wt = wave >> 1;  // which 128 tokens of the block
  const int half = lane >> 5;
  const int col = lane & 31;

  // Workgroup order: super-bands of kSuperBand token blocks, walked slice by
  // slice with the token block fastest. Workgroups are dispatched to the 8
  // XCDs round-robin, so the 32 workgroups an XCD runs at once hold 4 token
  // blocks x 8 slices (each H block read by 8 of them, each W tile by 4,
  // through the XCD's L2), and all XCDs walk the same slices at the same
  // time (W shared through the Infinity Cache). The order changes only which
  // workgroup runs when, never any arithmetic.
  const int S = n_slices;
  const int b = blockIdx.x;
  const int band = b / (kSuperBand * S);
  const int tb_first = band * kSuperBand;
  const int nb = min(kSuperBand, n_tb - tb_first);
  const int rem = b - band * kSuperBand * S;
  const int slice = rem / nb;
  const int t0 = (tb_first + rem % nb) * kBT;
  const int n_vt = (vocab + kBV - 1) / kBV;
  const int tile_begin = slice_tile(slice, n_vt, S);
  const int tile_end = slice_tile(slice + 1, n_vt, S);
  const int nks = row_bytes / kStepBytes;

  // Loader: wavefront w fills rows 64 w .. 64 w + 63 of both operands with
  // eight loads each; lane i fetches row (i / 8) of an 8-row group, logical
  // chunk (i % 8) ^ swz(row), so that it lands in its swizzled position.
  // swz(row) = (i / 8) ^ (j & 1) for load j (row = 64 w + 8 j + i / 8).
  const int lr = lane >> 3;
  uint32_t voff[kDmaPerWave];
#pragma unroll
  for (int j = 0; j < kDmaPerWave; ++j)
    voff[j] = (uint32_t)(wave * 64 + j * kDmaRows + lr) * (uint32_t)row_bytes + (((lane & 7) ^ lr ^ (j & 1)) * 16);
  const uint32_t lds_wave =
      (uint32_t)(size_t)((__attribute__((address_space(3))) uint4*)smem) + wave * 64 * kStepBytes;
  const int4v hr = rsrc_words(H + (size_t)t0 * row_bytes, (uint32_t)min(kBT, n_tok - t0) * row_bytes);
  auto w_rsrc = [&](int tile) {
    const int v0 = tile * kBV;
    return rsrc_words(W + (size_t)v0 * row_bytes, (uint32_t)min(kBV, vocab - v0) * row_bytes);
  };
  auto w_slot_lds = [&](int slot) { return lds_wave + (uint32_t)slot * kSlotBytes; };
  auto h_slot_lds = [&](int slot) { return lds_wave + (uint32_t)(kWSlots + slot) * kSlotBytes; };

  // MFMA operand reads: lane l takes row (l mod 32) of each 32-row block at
  // logical chunk 2 kk + l / 32 (kk = K sub-step 0..3); swz(row) = swz(l mod 32).
  int a_off[4], b_off[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int pc = (2 * kk + half) ^ swz(col);
    a_off[kk] = (wv * 128 + col) * kRowChunks + pc;
    b_off[kk] = (wt * 128 + col) * kRowChunks + pc;
  }

  int y[4];
  float mrun[4], srun[4], zy[4];
  bool found[4];
#pragma unroll
  for (int bn = 0; bn < 4; ++bn) {
    const int tok = t0 + wt * 128 + bn * 32 + col;
    y[bn] = tok < n_tok ? tokens[tok] : -1;
    mrun[bn] = -INFINITY;
    srun[bn] = 0.0f;
    zy[bn] = 0.0f;
    found[bn] = false;
  }

  // K-step pipeline over the workgroup's steps g (all tiles of the slice,
  // K fastest): W(g) sits in W slot g % 3, H(g) in H slot g % 2. Right after
  // the barrier that publishes step g, H(g + 1) and W(g + 2) are issued into
  // the slots step g - 1 used. A step is four sub-steps of 16 MFMAs; during
  // one sub-step's MFMAs the wavefront reads the next sub-step's 8 operand
  // fragments from LDS, and each step's last sub-step is multiplied after
  // the next barrier, while the next step's loads are issued and its first
  // operands read: the matrix cores keep busy across the barrier. The
  // order is pinned with scheduling barriers: left alone, the compiler
  // issues each sub-step's LDS reads after its MFMAs and then waits for
  // them.
  auto mma_all = [&](floatx16 (&acc)[4][4], const uint4 (&A)[4], const uint4 (&B)[4]) {
#pragma unroll
    for (int bm = 0; bm < 4; ++bm)
#pragma unroll
      for (int bn = 0; bn < 4; ++bn) Mma<kDtype>::step(acc[bm][bn], A[bm], B[bn]);
  };
  int w_tile = tile_begin, w_ks = 0;  // next W step to load
  int h_ks = 0;                        // next H step to load (H rows do not depend on the tile)
  int w_slot_next = 0, h_slot_next = 0;
  auto next_w = [&]() {  // advance, clamped to a valid step past the end
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
  // One sub-step: MFMA q (q = 4 bm + bn) on (A, B), interleaved with the 8
  // reads of the next operands (RA, RB; order A0 B0 B1 B2 B3 A1 A2 A3, the
  // order the next sub-step needs them) from slots (wsl, hsl), sub-step rkk:
  // one read every second MFMA, or in the first 8 MFMAs when kFront (the
  // last sub-step's reads must land before the barrier). With kDma, the 8
  // loads of H(g + 1) and then the 8 of W(g + 2) go one per MFMA.
  auto phase = [&](floatx16 (&acc)[4][4], const uint4 (&A)[4], const uint4 (&B)[4], auto first, auto do_mma,
                   auto front, auto dma, int wsl, int hsl, int rkk, uint4 (&RA)[4], uint4 (&RB)[4]) {
    const uint4* sa = smem + wsl * kSlotChunks;
    const uint4* sb = smem + (kWSlots + hsl) * kSlotChunks;
    int4v wr;
    uint32_t wsoff = 0, hsoff = 0, wm = 0, hm = 0;
    if constexpr (decltype(dma)::value) {
      wr = w_rsrc(w_tile);
      wsoff = (uint32_t)w_ks * kStepBytes;
      hsoff = (uint32_t)h_ks * kStepBytes;
      wm = w_slot_lds(w_slot_next);
      hm = h_slot_lds(h_slot_next);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if constexpr (decltype(do_mma)::value) {
        if constexpr (decltype(first)::value) Mma<kDtype>::first(acc[q >> 2][q & 3], A[q >> 2], B[q & 3]);
        else Mma<kDtype>::step(acc[q >> 2][q & 3], A[q >> 2], B[q & 3]);
      }
      constexpr bool kFront = decltype(front)::value;
      if (kFront ? q < 8 : (q & 1) == 0) {
        const int r = kFront ? q : q >> 1;
        if (r == 0) RA[0] = sa[a_off[rkk]];
        else if (r <= 4) RB[r - 1] = sb[b_off[rkk] + (r - 1) * 32 * kRowChunks];
        else RA[r - 4] = sa[a_off[rkk] + (r - 4) * 32 * kRowChunks];
      }
      if constexpr (decltype(dma)::value) {
        if (q < 8) dma16(hr, voff[q], hsoff, hm + q * 1024);
        else dma16(wr, voff[q - 8], wsoff, wm + (q - 8) * 1024);
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
  // Prologue: W(0), H(0), W(1).
  {
    const int4v wr0 = w_rsrc(w_tile);
#pragma unroll
    for (int j = 0; j < kDmaPerWave; ++j) dma16(wr0, voff[j], (uint32_t)w_ks * kStepBytes, w_slot_lds(0) + j * 1024);
#pragma unroll
    for (int j = 0; j < kDmaPerWave; ++j) dma16(hr, voff[j], 0, h_slot_lds(0) + j * 1024);
    next_w();
    next_h();
    const int4v wr1 = w_rsrc(w_tile);
#pragma unroll
    for (int j = 0; j < kDmaPerWave; ++j) dma16(wr1, voff[j], (uint32_t)w_ks * kStepBytes, w_slot_lds(1) + j * 1024);
    next_w();
  }
  int wslot = 0, hslot = 0;  // slots of the step being multiplied
  uint4 pa[4], pb[4];        // kk = 3 operands of the previous step, multiplied late
  // One K step; kFirst = the tile's first step (fresh accumulators, no
  // deferred sub-step from the previous tile). The next steps' loads are
  // always issued: past the workgroup's last step they re-read a valid
  // step into a free slot, which nothing reads again.
  auto k_step = [&](floatx16 (&acc)[4][4], auto first) {
    constexpr bool kFirst = decltype(first)::value;
    wait_and_barrier<kDmaPerWave>();  // W(g), H(g) landed; W(g + 1) may still be in flight
    uint4 fa[4], fb[4], ga[4], gb[4];
    if constexpr (kFirst) phase(acc, pa, pb, F{}, F{}, F{}, T{}, wslot, hslot, 0, fa, fb);
    else phase(acc, pa, pb, F{}, T{}, F{}, T{}, wslot, hslot, 0, fa, fb);
    phase(acc, fa, fb, first, T{}, F{}, F{}, wslot, hslot, 1, ga, gb);
    phase(acc, ga, gb, F{}, T{}, F{}, F{}, wslot, hslot, 2, fa, fb);
    phase(acc, fa, fb, F{}, T{}, T{}, F{}, wslot, hslot, 3, pa, pb);
    wslot = wslot == kWSlots - 1 ? 0 : wslot + 1;
    hslot ^= 1;
  };
  for (int tile = tile_begin; tile < tile_end; ++tile) {
    floatx16 acc[4][4];
    k_step(acc, T{});
    for (int ks = 1; ks < nks; ++ks) k_step(acc, F{});
    mma_all(acc, pa, pb);  // the tile's last sub-step

    // Tile epilogue: fold this tile's logits into the running state, one
    // token column (64 logits per lane) at a time. Register q = 16 bm + i of
    // a lane holds vocabulary row vw + 32 bm + 8 (i / 4) + 4 half + (i % 4).
    // Each lane folds its 16 logits of one 32x32 block at a time into the
    // running (max, sum of exp) of that token column. The logits are copied
    // out of the matrix-core registers 16 at a time, where they are used
    // (acc_read), so the epilogue needs few VGPRs next to the 256
    // accumulators. The sampled logit is picked with a select tree keyed on
    // the bits of its row, without a branch.
    const int vw = tile * kBV + wv * 128;
    const bool partial = tile * kBV + kBV > vocab;  // only the vocabulary's last tile
    mfma_result_wait();
#pragma unroll
    for (int bn = 0; bn < 4; ++bn) {
      const int o = y[bn] - vw;  // sampled row relative to this wavefront's 128 rows
      // Register i of a lane holds row 32 bm + 8 (i / 4) + 4 half + (i % 4):
      // bits 0, 1, 3, 4 of the row pick i, bit 2 picks the lane half.
      const bool b0 = (o & 1) != 0, b1 = (o & 2) != 0, b2 = (o & 8) != 0, b3 = (o & 16) != 0;
      const bool mine = (unsigned)o < 128u && ((o >> 2) & 1) == half;
#pragma unroll
      for (int bm = 0; bm < 4; ++bm) {
        floatx16 z;  // a vector, not an array: it must stay in registers
#pragma unroll
        for (int i = 0; i < 16; ++i) z[i] = acc_read(acc[bm][bn], i);
        if (partial) {
          const int lim = vocab - (vw + bm * 32 + 4 * half);  // rows at or past this offset do not exist
#pragma unroll
          for (int i = 0; i < 16; ++i) z[i] = (8 * (i >> 2) + (i & 3) >= lim) ? -INFINITY : z[i];
        }
        const float pick = select16(z, b0, b1, b2, b3);
        const bool here = mine && (o >> 5) == bm;
        zy[bn] = here ? pick : zy[bn];
        found[bn] = found[bn] || here;

        float bmax = z[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) bmax = fmaxf(bmax, z[i]);
        const float mnew = fmaxf(mrun[bn], bmax);
        // A lane whose rows so far are all absent has mnew = -inf; it then
        // scales by exp2(-inf) = 0 around 0 and keeps (m, s) = (-inf, 0).
        const float mref = mnew == -INFINITY ? 0.0f : mnew;
        // (z - m) is exactly 0 for the running maximum, so its term is
        // exactly 1 and stays 1 (later rescales by exp2(0)): the final sum
        // is >= 1 and logprob <= 0 holds in fp32.
        float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          s0 += fast_exp2((z[i] - mref) * kLog2e);
          s1 += fast_exp2((z[i + 1] - mref) * kLog2e);
        }
        srun[bn] = srun[bn] * fast_exp2((mrun[bn] - mref) * kLog2e) + (s0 + s1);
        mrun[bn] = mnew;
      }
    }
  }

  // Slice end. Lanes l and l^32 hold the same tokens (different rows).
#pragma unroll
  for (int bn = 0; bn < 4; ++bn) {
    const float m2 = __shfl_xor(mrun[bn], 32, 64);
    const float s2 = __shfl_xor(srun[bn], 32, 64);
    lse_merge(mrun[bn], srun[bn], m2, s2);
    if (found[bn]) zy_out[t0 + wt * 128 + bn * 32 + col] = zy[bn];
  }
  // Wavefronts wv = 0 and wv = 1 hold the same tokens; merge through LDS
  // once every wavefront is done with the ring.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  float2* xch = reinterpret_cast<float2*>(smem);
  if (wv == 1 && half == 0) {
#pragma unroll
    for (int bn = 0; bn < 4; ++bn) xch[wt * 128 + bn * 32 + col] = make_float2(mrun[bn], srun[bn]);
  }
  __syncthreads();
  if (wv == 0 && half == 0) {
#pragma unroll
    for (int bn = 0; bn < 4; ++bn) {
      const int tok = t0 + wt * 128 + bn * 32 + col;
      const float2 o = xch[wt * 128 + bn * 32 + col];
      float m = mrun[bn], s = srun[bn];
      lse_merge(m, s, o.x, o.y);
      if (tok < n_tok) part[(size_t)slice * n_tok + tok] = make_float2(m, s);
    }
  }
}

// Per token: merge the slice partials in ascending slice order.
__global__ __launch_bounds__(256) void lse_combine_kernel(const float2* __restrict__ part,
                                                          const float* __restrict__ zy, int n_tok,
                                                          int n_slices, float* __restrict__ logprob,
                                                          float* __restrict__ lse) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= n_tok) return;
  float M = -INFINITY;
  for (int s = 0; s < n_slices; ++s) M = fmaxf(M, part[(size_t)s * n_tok + t].x);
  float S = 0.0f;
  for (int s = 0; s < n_slices; ++s) {
    const float2 p = part[(size_t)s * n_tok + t];
    S += p.y * fast_exp2((p.x - M) * kLog2e);
  }
  const float l = M + fast_log2(S) * kLn2;
  logprob[t] = zy[t] - l;
  if (lse) lse[t] = l;
}

}  // namespace

size_t lmhead_workspace_bytes(long long n_tok, long long vocab) {
  if (n_tok <= 0) return 0;
  return align256((size_t)n_slices(vocab) * (size_t)n_tok * sizeof(float2)) + align256((size_t)n_tok * sizeof(float));
}

hipError_t launch_lmhead_logprob(const void* H, const void* W, int dtype, int n_tok, int d, int vocab,
                                 const int32_t* tokens, float* logprob, float* lse, void* workspace,
                                 hipStream_t stream) {
  const int es = dtype == 0 ? 2 : 4;
  const int row_bytes = d * es;
  const int S = n_slices(vocab);
  const int ntb = (int)ceil_div(n_tok, kBT);
  float2* part = static_cast<float2*>(workspace);
  float* zy = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                       align256((size_t)S * (size_t)n_tok * sizeof(float2)));
  const dim3 grid((unsigned)ntb * (unsigned)S);
  if (dtype == 0)
    hipLaunchKernelGGL(lmhead_lse_partial_kernel<0>, grid, dim3(kThreads), 0, stream, static_cast<const char*>(H),
                       static_cast<const char*>(W), tokens, n_tok, row_bytes, vocab, ntb, S, part, zy);
  else
    hipLaunchKernelGGL(lmhead_lse_partial_kernel<1>, grid, dim3(kThreads), 0, stream, static_cast<const char*>(H),
                       static_cast<const char*>(W), tokens, n_tok, row_bytes, vocab, ntb, S, part, zy);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lse_combine_kernel, dim3((unsigned)ceil_div(n_tok, 256)), dim3(256), 0, stream, part, zy, n_tok,
                     S, logprob, lse);
  return hipGetLastError();
}

}  // namespace itl
