// Sampled term of the REINFORCE Zero gradient of the LM head's weights
// ("vLLM says aligned kernels make asynchronous RL stable at lag 64",
// section "REINFORCE Zero removes the mismatch first": plain REINFORCE, so
// the dlogits row of token t is coef[t] (onehot(y_t) - p_t), and its
// one-hot part adds coef[t] H[t] to row y_t of dW):
//
//   dW[v] = sum over tokens t with y_t = v of coef[t] H[t]   (fp32)
//
// written for every vocabulary row (rows no token samples get zeros), before
// the dense part is added chunk by chunk. The order of each sum is fixed by
// the run of tokens with that id alone (sampled_plan.h): the tokens are
// stably sorted by id with a counting sort, so a run lists its tokens in
// ascending order, and a run is summed in segments of kRunSeg tokens, groups
// of kRunGroup segments, then the groups, each in order. Every product and
// sum is rounded to fp32 on its own (no fused multiply-add), so the order is
// the whole definition of the bits.
//
// Counting sort, one pass per 8-bit digit, least significant first:
//   1. each workgroup counts the digits of its kSortTile keys (LDS counters),
//   2. one workgroup turns the digit-major table of counts into start
//      positions (exclusive scan: digit d of block b starts after every
//      smaller digit and after digit d of blocks 0 .. b - 1),
//   3. each workgroup places its keys in rounds of 256, in order: a lane's
//      rank among the earlier lanes of its wavefront with the same digit
//      comes from the digit's bits' ballots, the earlier wavefronts' counts
//      of the round from LDS, the earlier rounds' from a running counter.
// Within a block every key keeps its order among equal digits, so each pass
// is stable and the sort is the unique stable one: the result does not
// depend on the block size or on timing. Integer counting only; no float
// arithmetic and no atomics outside a workgroup's LDS counters.

#include "itl_launch.h"
#include "sampled_plan.h"

namespace itl {

namespace {

// Eight consecutive values of a token's row as floats (lane-contiguous
// 16-byte loads: bf16 rows one load, fp32 rows two).
template <int kDtype>
struct Row8;
template <>
struct Row8<0> {
  __device__ static __forceinline__ void load(const void* base, size_t off, float (&x)[8]) {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <>
struct Row8<1> {
  __device__ static __forceinline__ void load(const void* base, size_t off, float (&x)[8]) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    const float4 a = p[0], b = p[1];
    x[0] = a.x, x[1] = a.y, x[2] = a.z, x[3] = a.w;
    x[4] = b.x, x[5] = b.y, x[6] = b.z, x[7] = b.w;
  }
};

// A wavefront covers a row in chunks of 512 values (8 per lane, lane-major),
// kC chunks per pass; d is a multiple of 64, so a lane's 8 values are all in
// the row or all past it.
constexpr int kChunk = 512;
constexpr int kSegChunks = 4;                   // chunks per pass of a long run's segment
constexpr int kSegSlice = kChunk * kSegChunks;  // the values one segment_sums wavefront covers
constexpr int kRowChunks8 = 8;                  // chunks per pass of a short run's row

__device__ __forceinline__ void store_row8(float* out, int k, const float (&a)[8]) {
  float4* p = reinterpret_cast<float4*>(out + k);
  p[0] = make_float4(a[0], a[1], a[2], a[3]);
  p[1] = make_float4(a[4], a[5], a[6], a[7]);
}

template <int kDtype, int kC>
__device__ __forceinline__ void load_token(const void* __restrict__ H, uint32_t t, int d, int cg, int lane,
                                           float (&x)[kC][8]) {
#pragma unroll
  for (int ch = 0; ch < kC; ++ch) {
    const int k = cg + ch * kChunk + lane * 8;
    if (k < d) Row8<kDtype>::load(H, (size_t)t * (size_t)d + k, x[ch]);
  }
}
template <int kC>
__device__ __forceinline__ void add_token(float (&acc)[kC][8], float c, const float (&x)[kC][8]) {
#pragma unroll
  for (int ch = 0; ch < kC; ++ch)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[ch][e] = acc[ch][e] + c * x[ch][e];
}

// out[k] = sum over j < cnt, in order, of coef[t_j] H[t_j][k], t_j = ts[p0 + j]
// (cnt = 0 writes zeros), for k in [k0, min(k1, d)); cnt <= 64. kC chunks
// per pass. With kPair (long runs' segments: 64 tokens) the tokens' ids are
// loaded once, one per lane, and read back with readlane, and two tokens'
// rows are loaded before their additions (which keep token order); without
// it (runs of a few tokens) each id is a scalar load, one token at a time,
// which keeps the registers, and so the wavefronts per SIMD, of the kernel
// that writes every vocabulary row.
template <int kDtype, int kC, bool kPair>
__device__ __forceinline__ void sum_token_rows(const uint32_t* __restrict__ ts, long long p0, int cnt,
                                               const void* __restrict__ H, const float* __restrict__ coef, int d,
                                               int k0, int k1, int lane, float* __restrict__ out) {
  const uint32_t my_t = kPair && lane < cnt ? ts[p0 + lane] : 0u;
  auto tok = [&](int j) {
    if constexpr (kPair) return (uint32_t)__builtin_amdgcn_readlane((int)my_t, j);
    else return ts[p0 + j];
  };
  auto cof = [&](int j) { return coef[tok(j)]; };
  for (int cg = k0; cg < min(k1, d); cg += kChunk * kC) {
    float acc[kC][8];
#pragma unroll
    for (int ch = 0; ch < kC; ++ch)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[ch][e] = 0.0f;
    int j = 0;
    if constexpr (kPair) {
      for (; j + 2 <= cnt; j += 2) {
        float x0[kC][8], x1[kC][8];
        load_token<kDtype, kC>(H, tok(j), d, cg, lane, x0);
        load_token<kDtype, kC>(H, tok(j + 1), d, cg, lane, x1);
        add_token<kC>(acc, cof(j), x0);
        add_token<kC>(acc, cof(j + 1), x1);
      }
    }
#pragma unroll 1
    for (; j < cnt; ++j) {
      const uint32_t t = tok(j);
      const float c = cof(j);
#pragma unroll
      for (int ch = 0; ch < kC; ++ch) {
        const int k = cg + ch * kChunk + lane * 8;
        if (k < d) {
          float x[8];
          Row8<kDtype>::load(H, (size_t)t * (size_t)d + k, x);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[ch][e] = acc[ch][e] + c * x[e];
        }
      }
    }
#pragma unroll
    for (int ch = 0; ch < kC; ++ch) {
      const int k = cg + ch * kChunk + lane * 8;
      if (k < d) store_row8(out, k, acc[ch]);
    }
  }
}

// out[k] = sum over j < cnt, in order, of P[(slot0 + j) d + k] (cnt >= 1),
// for the 512 values k in [k0, k0 + 512) (k < d). Eight rows' loads are
// issued before their additions.
__device__ __forceinline__ void sum_slot_rows(const float* __restrict__ P, long long slot0, int cnt, int d, int k0,
                                              int lane, float* __restrict__ out) {
  const int k = k0 + lane * 8;
  if (k >= d) return;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  constexpr int kAhead = 8;
  int j = 0;
  for (; j + kAhead <= cnt; j += kAhead) {
    float x[kAhead][8];
#pragma unroll
    for (int a = 0; a < kAhead; ++a) Row8<1>::load(P + (size_t)(slot0 + j + a) * (size_t)d, k, x[a]);
#pragma unroll
    for (int a = 0; a < kAhead; ++a)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = acc[e] + x[a][e];
  }
  for (; j < cnt; ++j) {
    float x[8];
    Row8<1>::load(P + (size_t)(slot0 + j) * (size_t)d, k, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc[e] + x[e];
  }
  store_row8(out, k, acc);
}

// Pass input: the token ids (first pass; positions are the token indices)
// or the previous pass's keys and positions.
struct PassIn {
  const uint32_t* keys;  // null on the first pass
  const uint32_t* vals;
  const int32_t* tokens;
};

__device__ __forceinline__ void pass_load(const PassIn& in, long long i, int vocab, uint32_t& key, uint32_t& val) {
  if (in.keys) {
    key = in.keys[i];
    val = in.vals[i];
  } else {
    key = sort_key(in.tokens[i], vocab);
    val = (uint32_t)i;
  }
}

// 1. Digit counts of block b: hist[digit * n_blocks + b].
__global__ __launch_bounds__(kSortThreads) void sort_count_kernel(PassIn in, int n, int vocab, int shift,
                                                                  uint32_t* __restrict__ hist, int n_blocks) {
  __shared__ uint32_t cnt[kSortBins];
  const int b = blockIdx.x;
  cnt[threadIdx.x] = 0;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kSortPerThread; ++r) {
    const long long i = (long long)b * kSortTile + r * kSortThreads + threadIdx.x;
    if (i < n) {
      uint32_t key, val;
      pass_load(in, i, vocab, key, val);
      atomicAdd(&cnt[(key >> shift) & (kSortBins - 1)], 1u);
    }
  }
  __syncthreads();
  hist[(size_t)threadIdx.x * n_blocks + b] = cnt[threadIdx.x];
}

// 2. Exclusive scan of h[0 .. m) in place, one 1024-thread workgroup:
// wavefront w takes a run of consecutive entries (a multiple of 64), sums it
// (lanes striding by 64: integers, so any order), the runs' totals give each
// run's start, and each wavefront then rewrites its run 64 entries at a
// time (a wavefront scan per step, carried across steps).
constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void sort_scan_kernel(uint32_t* __restrict__ h, int m) {
  constexpr int kWaves = kScanThreads / 64;
  __shared__ uint32_t wave_total[kWaves];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int per = ((m + kWaves - 1) / kWaves + 63) / 64 * 64;
  const int b = min(m, w * per), e = min(m, b + per);
  uint32_t s = 0;
  for (int i = b + lane; i < e; i += 64) s += h[i];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if (lane == 0) wave_total[w] = s;
  __syncthreads();
  uint32_t carry = 0;
  for (int v = 0; v < w; ++v) carry += wave_total[v];
  constexpr int kAhead = 4;  // steps whose loads are issued together
  for (int i0 = b; i0 < e; i0 += 64 * kAhead) {
    uint32_t x[kAhead];
#pragma unroll
    for (int a = 0; a < kAhead; ++a) {
      const int i = i0 + 64 * a + lane;
      x[a] = i < e ? h[i] : 0u;
    }
#pragma unroll
    for (int a = 0; a < kAhead; ++a) {
      uint32_t inc = x[a];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(inc, off, 64);
        if (lane >= off) inc += y;
      }
      const int i = i0 + 64 * a + lane;
      if (i < e) h[i] = carry + inc - x[a];
      carry += __shfl(inc, 63, 64);
    }
  }
}

// 3. Stable placement of block b's keys (and their positions).
static_assert(kSortThreads == kSortBins, "a thread per digit keeps each digit's running position");
__global__ __launch_bounds__(kSortThreads) void sort_place_kernel(PassIn in, int n, int vocab, int shift,
                                                                  const uint32_t* __restrict__ hist, int n_blocks,
                                                                  uint32_t* __restrict__ keys_out,
                                                                  uint32_t* __restrict__ vals_out) {
  constexpr int kWaves = kSortThreads / 64;
  __shared__ uint32_t next[kSortBins];        // next free position of each digit
  __shared__ uint32_t wcnt[kWaves][kSortBins];  // this round's count of each digit per wavefront
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  next[tid] = hist[(size_t)tid * n_blocks + b];
#pragma unroll
  for (int v = 0; v < kWaves; ++v) wcnt[v][tid] = 0;
  uint32_t key[kSortPerThread], val[kSortPerThread];
#pragma unroll
  for (int r = 0; r < kSortPerThread; ++r) {
    const long long i = (long long)b * kSortTile + r * kSortThreads + tid;
    key[r] = 0;
    val[r] = 0;
    if (i < n) pass_load(in, i, vocab, key[r], val[r]);
  }
  __syncthreads();
  const uint64_t lt = (1ull << lane) - 1ull;
#pragma unroll
  for (int r = 0; r < kSortPerThread; ++r) {
    const bool ok = (long long)b * kSortTile + r * kSortThreads + tid < n;
    const uint32_t dg = (key[r] >> shift) & (kSortBins - 1);
    uint64_t same = __ballot(ok);
#pragma unroll
    for (int bit = 0; bit < kSortDigitBits; ++bit) {
      const bool set = (dg >> bit) & 1u;
      const uint64_t m = __ballot(ok && set);
      same &= set ? m : ~m;
    }
    const uint32_t below = (uint32_t)__popcll(same & lt);
    if (ok && below == 0) wcnt[w][dg] = (uint32_t)__popcll(same);
    __syncthreads();
    if (ok) {
      uint32_t pos = next[dg] + below;
      for (int v = 0; v < w; ++v) pos += wcnt[v][dg];
      keys_out[pos] = key[r];
      vals_out[pos] = val[r];
    }
    __syncthreads();
    uint32_t add = 0;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      add += wcnt[v][tid];
      wcnt[v][tid] = 0;
    }
    next[tid] += add;
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t* __restrict__ p, long long n) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Run bounds: rs[v], re[v] = first and one-past-last sorted position of id v
// (both zero for an id no token samples).
__global__ __launch_bounds__(256) void run_bounds_kernel(const uint32_t* __restrict__ ks, int n, int vocab,
                                                         uint32_t* __restrict__ rs, uint32_t* __restrict__ re) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const uint32_t v = ks[i];
  if (v >= (uint32_t)vocab) return;
  if (i == 0 || ks[i - 1] != v) rs[v] = (uint32_t)i;
  if (i == n - 1 || ks[i + 1] != v) re[v] = (uint32_t)i + 1u;
}

// Rows of runs of at most one segment (and of ids no token samples): one
// wavefront per vocabulary row writes its sum (zeros for an empty run).
template <int kDtype>
__global__ __launch_bounds__(256) void short_rows_kernel(const uint32_t* __restrict__ ts,
                                                         const uint32_t* __restrict__ rs,
                                                         const uint32_t* __restrict__ re, int vocab,
                                                         const void* __restrict__ H, const float* __restrict__ coef,
                                                         int d, float* __restrict__ dW) {
  const int v = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  if (v >= vocab) return;
  const uint32_t s = rs[v], L = re[v] - s;
  if (L > (uint32_t)kRunSeg) return;
  sum_token_rows<kDtype, kRowChunks8, false>(ts, s, (int)L, H, coef, d, 0, d, lane, dW + (size_t)v * (size_t)d);
}

// The wavefront's 64 sorted positions w * 64 + lane that start a piece of
// length len of a run longer than more_than tokens (start_only: only the
// run's first position). Lane bits of the result; the run's start, length
// and id in s, L, v.
__device__ __forceinline__ uint64_t piece_starts(const uint32_t* __restrict__ ks, const uint32_t* __restrict__ rs,
                                                 const uint32_t* __restrict__ re, int n, int vocab, long long len,
                                                 long long more_than, bool start_only, long long i, uint32_t& v,
                                                 uint32_t& s, uint32_t& L) {
  bool q = false;
  v = 0, s = 0, L = 0;
  if (i < n) {
    v = ks[i];
    if (v < (uint32_t)vocab) {
      s = rs[v];
      L = re[v] - s;
      const long long off = i - (long long)s;
      q = (long long)L > more_than && (start_only ? off == 0 : off % len == 0);
    }
  }
  return __ballot(q);
}

// Segment sums of runs longer than one segment, into slots of P1.
template <int kDtype>
__global__ __launch_bounds__(256) void segment_sums_kernel(const uint32_t* __restrict__ ks,
                                                           const uint32_t* __restrict__ ts,
                                                           const uint32_t* __restrict__ rs,
                                                           const uint32_t* __restrict__ re, int n, int vocab,
                                                           const void* __restrict__ H, const float* __restrict__ coef,
                                                           int d, float* __restrict__ P1) {
  const long long w = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const long long i = w * 64 + lane;
  uint32_t v, s, L;
  uint64_t mask = piece_starts(ks, rs, re, n, vocab, kRunSeg, kRunSeg, false, i, v, s, L);
  while (mask) {
    const int src = __builtin_ctzll(mask);
    mask &= mask - 1;
    const uint32_t s0 = __builtin_amdgcn_readlane(s, src), L0 = __builtin_amdgcn_readlane(L, src);
    const long long i0 = w * 64 + src;
    const long long j = (i0 - s0) / kRunSeg;
    const int cnt = (int)min((long long)kRunSeg, (long long)L0 - j * kRunSeg);
    const int k0 = blockIdx.y * kSegSlice;
    sum_token_rows<kDtype, kSegChunks, true>(ts, i0, cnt, H, coef, d, k0, k0 + kSegSlice, lane,
                           P1 + (size_t)run_slot(s0, j, kRunSeg) * (size_t)d);
  }
}

// Group sums of runs longer than one segment: the row itself for a run of
// one group, else a slot of P2.
__global__ __launch_bounds__(256) void group_sums_kernel(const uint32_t* __restrict__ ks,
                                                         const uint32_t* __restrict__ rs,
                                                         const uint32_t* __restrict__ re, int n, int vocab, int d,
                                                         const float* __restrict__ P1, float* __restrict__ P2,
                                                         float* __restrict__ dW) {
  const long long w = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const long long i = w * 64 + lane;
  uint32_t v, s, L;
  uint64_t mask = piece_starts(ks, rs, re, n, vocab, kRunGroupTokens, kRunSeg, false, i, v, s, L);
  while (mask) {
    const int src = __builtin_ctzll(mask);
    mask &= mask - 1;
    const uint32_t v0 = __builtin_amdgcn_readlane(v, src), s0 = __builtin_amdgcn_readlane(s, src),
                   L0 = __builtin_amdgcn_readlane(L, src);
    const long long g = (w * 64 + src - s0) / kRunGroupTokens;
    const long long j0 = g * kRunGroup;
    const int cnt = (int)min((long long)kRunGroup, n_pieces(L0, kRunSeg) - j0);
    float* out = (long long)L0 <= kRunGroupTokens ? dW + (size_t)v0 * (size_t)d
                                                 : P2 + (size_t)run_slot(s0, g, kRunGroupTokens) * (size_t)d;
    sum_slot_rows(P1, run_slot(s0, j0, kRunSeg), cnt, d, blockIdx.y * kChunk, lane, out);
  }
}

// Rows of runs longer than one group: their group sums in order.
__global__ __launch_bounds__(256) void group_rows_kernel(const uint32_t* __restrict__ ks,
                                                         const uint32_t* __restrict__ rs,
                                                         const uint32_t* __restrict__ re, int n, int vocab, int d,
                                                         const float* __restrict__ P2, float* __restrict__ dW) {
  const long long w = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const long long i = w * 64 + lane;
  uint32_t v, s, L;
  uint64_t mask = piece_starts(ks, rs, re, n, vocab, 0, kRunGroupTokens, true, i, v, s, L);
  while (mask) {
    const int src = __builtin_ctzll(mask);
    mask &= mask - 1;
    const uint32_t v0 = __builtin_amdgcn_readlane(v, src), s0 = __builtin_amdgcn_readlane(s, src),
                   L0 = __builtin_amdgcn_readlane(L, src);
    sum_slot_rows(P2, run_slot(s0, 0, kRunGroupTokens), (int)n_pieces(L0, kRunGroupTokens), d, blockIdx.y * kChunk,
                  lane, dW + (size_t)v0 * (size_t)d);
  }
}

struct SampledLayout {
  size_t keys[2], vals[2], hist, rs, re, p1, p2, total;
};

SampledLayout sampled_layout(long long n_tok, long long d, long long vocab) {
  SampledLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  for (int k = 0; k < 2; ++k) {
    L.keys[k] = take((size_t)n_tok * 4);
    L.vals[k] = take((size_t)n_tok * 4);
  }
  L.hist = take((size_t)kSortBins * (size_t)sort_blocks(n_tok) * 4);
  L.rs = take((size_t)vocab * 4);
  L.re = take((size_t)vocab * 4);
  L.p1 = take((size_t)n_run_slots(n_tok, kRunSeg) * (size_t)d * 4);
  L.p2 = take((size_t)n_run_slots(n_tok, kRunGroupTokens) * (size_t)d * 4);
  L.total = off;
  return L;
}

template <int kDtype>
hipError_t run_sampled(const void* H, int n_tok, int d, int vocab, const int32_t* tokens, const float* coef,
                       float* dW, void* workspace, hipStream_t stream) {
  const SampledLayout Ly = sampled_layout(n_tok, d, vocab);
  char* ws = static_cast<char*>(workspace);
  uint32_t* keys[2] = {reinterpret_cast<uint32_t*>(ws + Ly.keys[0]), reinterpret_cast<uint32_t*>(ws + Ly.keys[1])};
  uint32_t* vals[2] = {reinterpret_cast<uint32_t*>(ws + Ly.vals[0]), reinterpret_cast<uint32_t*>(ws + Ly.vals[1])};
  uint32_t* hist = reinterpret_cast<uint32_t*>(ws + Ly.hist);
  uint32_t* rs = reinterpret_cast<uint32_t*>(ws + Ly.rs);
  uint32_t* re = reinterpret_cast<uint32_t*>(ws + Ly.re);
  float* P1 = reinterpret_cast<float*>(ws + Ly.p1);
  float* P2 = reinterpret_cast<float*>(ws + Ly.p2);
  hipError_t e;
#define ITL_CHECK_LAUNCH()         \
  do {                             \
    e = hipGetLastError();         \
    if (e != hipSuccess) return e; \
  } while (0)

  // run bounds start at zero (the placement below leaves absent ids so)
  hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)ceil_div(vocab, 256)), dim3(256), 0, stream, rs, (long long)vocab);
  ITL_CHECK_LAUNCH();
  hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)ceil_div(vocab, 256)), dim3(256), 0, stream, re, (long long)vocab);
  ITL_CHECK_LAUNCH();
  const uint32_t* ks = nullptr;
  const uint32_t* ts = nullptr;
  if (n_tok > 0) {
    const int n_blocks = (int)sort_blocks(n_tok);
    const int passes = sort_passes(vocab);
    PassIn in{nullptr, nullptr, tokens};
    for (int p = 0; p < passes; ++p) {
      const int shift = p * kSortDigitBits;
      uint32_t* ko = keys[p & 1];
      uint32_t* vo = vals[p & 1];
      hipLaunchKernelGGL(sort_count_kernel, dim3((unsigned)n_blocks), dim3(kSortThreads), 0, stream, in, n_tok, vocab,
                         shift, hist, n_blocks);
      ITL_CHECK_LAUNCH();
      hipLaunchKernelGGL(sort_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, hist, kSortBins * n_blocks);
      ITL_CHECK_LAUNCH();
      hipLaunchKernelGGL(sort_place_kernel, dim3((unsigned)n_blocks), dim3(kSortThreads), 0, stream, in, n_tok, vocab,
                         shift, hist, n_blocks, ko, vo);
      ITL_CHECK_LAUNCH();
      in = PassIn{ko, vo, nullptr};
    }
    ks = in.keys;
    ts = in.vals;
    hipLaunchKernelGGL(run_bounds_kernel, dim3((unsigned)ceil_div(n_tok, 256)), dim3(256), 0, stream, ks, n_tok, vocab,
                       rs, re);
    ITL_CHECK_LAUNCH();
  }
  hipLaunchKernelGGL(short_rows_kernel<kDtype>, dim3((unsigned)ceil_div(vocab, 4)), dim3(256), 0, stream, ts, rs, re,
                     vocab, H, coef, d, dW);
  ITL_CHECK_LAUNCH();
  if (n_tok > kRunSeg) {
    // a wavefront per 64 sorted positions and slice of the row (several
    // slices, so that a long run's pieces are summed by many wavefronts)
    const unsigned grid = (unsigned)ceil_div(ceil_div(n_tok, 64), 4);
    const unsigned wide = (unsigned)ceil_div(d, kSegSlice), narrow = (unsigned)ceil_div(d, kChunk);
    hipLaunchKernelGGL(segment_sums_kernel<kDtype>, dim3(grid, wide), dim3(256), 0, stream, ks, ts, rs, re, n_tok,
                       vocab, H, coef, d, P1);
    ITL_CHECK_LAUNCH();
    hipLaunchKernelGGL(group_sums_kernel, dim3(grid, narrow), dim3(256), 0, stream, ks, rs, re, n_tok, vocab, d, P1, P2,
                       dW);
    ITL_CHECK_LAUNCH();
    if (n_tok > kRunGroupTokens) {
      hipLaunchKernelGGL(group_rows_kernel, dim3(grid, narrow), dim3(256), 0, stream, ks, rs, re, n_tok, vocab, d, P2,
                         dW);
      ITL_CHECK_LAUNCH();
    }
  }
#undef ITL_CHECK_LAUNCH
  return hipSuccess;
}

}  // namespace

size_t sampled_dw_workspace_bytes(long long n_tok, long long d, long long vocab) {
  return sampled_layout(n_tok, d, vocab).total;
}

hipError_t launch_sampled_dw(const void* H, int dtype, int n_tok, int d, int vocab, const int32_t* tokens,
                             const float* coef, float* dW, void* workspace, hipStream_t stream) {
  if (dtype == 0) return run_sampled<0>(H, n_tok, d, vocab, tokens, coef, dW, workspace, stream);
  return run_sampled<1>(H, n_tok, d, vocab, tokens, coef, dW, workspace, stream);
}

}  // namespace itl
