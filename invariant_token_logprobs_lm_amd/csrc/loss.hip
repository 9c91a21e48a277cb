// Group advantage and REINFORCE Zero loss ("vLLM says aligned kernels make
// asynchronous RL stable at lag 64", section "REINFORCE Zero removes the
// mismatch first"):
//
//   A_i          = r_i - mean of the rewards of i's group
//   ratio_t      = exp(logprob_t - rollout_logprob_t)      (no clipping)
//   resp_loss[i] = -A_i * (sum_{t in i} ratio_t) / T_i       (tokens averaged in a response)
//   loss         = (1/N) sum_i resp_loss[i]                  (then over responses)
//   coef[t]      = -ratio_t * A_i / (N * T_i)                (dloss/dlogprob_t, plain REINFORCE)
//
// Precision. ratio_t and coef[t] are fp32 values; every sum is fp64. The mean
// over responses nearly cancels when the advantages are centred within their
// groups (it can be 1e-5 of the typical |resp_loss|), so it is formed from the
// fp64 per-response losses, not from their fp32 roundings: rounding each
// resp_loss to fp32 first would alone move the mean by a few 1e-4 of itself.
//
// Invariance. A response is cut into segments of kSegTokens tokens counted
// from its first token; a segment is summed by one of three fixed trees
// chosen by its length (one lane in token order; one wavefront, lane j adding
// tokens j, j + 64, ... then an xor butterfly; the workgroup, thread j adding
// tokens j, j + 512, ..., then the wavefront butterflies and the eight wave
// sums in a fixed tree), and a response's segments are added in order. So a
// response's loss is a function of the response alone, wherever it sits in
// the batch. The mean's tree depends on the number of responses only.
//
// Work. Token pass: workgroup b owns the segments that start in tokens
// [b kSeg, (b + 1) kSeg) of the packed batch; it finds the responses holding
// tokens b kSeg and (b + 1) kSeg by a search of the offsets (batches of up to
// kLossThreads responses: one round) or from a window map written by one
// thread per response beforehand (larger batches: the search's dependent
// rounds were most of a workgroup's time). They tile a contiguous span of
// fewer than 2 kSeg tokens, which the workgroup reads once, coalesced, into
// LDS as ratios, sums segment by segment (turning each segment's ratios into
// its coefficients in place) and then writes the coefficients, coalesced.
// A response of one segment is finished there; the segment sums of longer
// ones go to the workspace. Finishing pass: per chunk of kFinishChunk
// responses, the longer responses' segment sums are added in order, and the
// chunk's fp64 losses are summed; a last single-workgroup pass adds the chunk
// sums in order (skipped when there is one chunk).

#include <algorithm>

#include "device_common.h"
#include "itl_config.h"
#include "itl_launch.h"
#include "loss_plan.h"

namespace itl {

namespace {

constexpr int kSpan = 2 * kSegTokens;                  // a token-pass span is shorter than this
constexpr int kLossWaves = kLossThreads / 64;
constexpr int kSpanPerThread = kSpan / kLossThreads;   // ratios staged per thread
constexpr int kMaxWaveSegs = kSpan / (kLaneSeg + 1) + 1;
constexpr int kMaxGroupSegs = kSpan / (kWaveSeg + 1) + 1;
constexpr int kMaxRounds = 64;                         // response rounds of the enumeration (valid input: <= 9)
static_assert(kSpan % kLossThreads == 0 && kLossThreads % 64 == 0, "span geometry");
static_assert(kSpan <= 32767, "span offsets are stored in 16 bits");

// Response i's token range, clamped into [0, n_tok] (bad offsets cannot
// index out of bounds; they give unspecified values).
__device__ __forceinline__ void resp_bounds(const int64_t* __restrict__ off, int i, long long n_tok, long long& s,
                                            long long& e) {
  s = plan_clamp(off[i], 0, n_tok);
  e = plan_clamp(off[i + 1], s, n_tok);
}

__device__ __forceinline__ float ratio_of(float lp, float lpr) { return fast_exp2((lp - lpr) * kLog2e); }

// d loss / d logprob of a response's tokens, per unit ratio.
__device__ __forceinline__ float coef_scale(float A, int n_resp, long long T) {
  return (float)(-(double)A / ((double)n_resp * (double)T));
}

// For two token positions ta <= tb, the largest i in [0, n_resp) with
// off[i] <= t, for both at once: a 512-way search (each round the
// workgroup's threads probe evenly spaced offsets of both ranges). Every
// thread must call it; the results are uniform.
__device__ void find_responses(const int64_t* __restrict__ off, int n_resp, long long ta, long long tb, int& ia,
                               int& ib) {
  int lo_a = 0, hi_a = n_resp, lo_b = 0, hi_b = n_resp;
  while (hi_a - lo_a > 1 || hi_b - lo_b > 1) {
    const int step_a = (hi_a - lo_a + kLossThreads - 1) / kLossThreads;
    const int step_b = (hi_b - lo_b + kLossThreads - 1) / kLossThreads;
    const long long ja = lo_a + (long long)(threadIdx.x + 1) * step_a;
    const long long jb = lo_b + (long long)(threadIdx.x + 1) * step_b;
    const bool la = ja < hi_a && off[ja] <= ta;
    const bool lb = jb < hi_b && off[jb] <= tb;
    // probes past the answer fail and (for increasing offsets) so do all
    // later ones: the count of hits is the answer's bracket
    const int ca = __syncthreads_count(la);
    const int cb = __syncthreads_count(lb);
    lo_a += ca * step_a;
    hi_a = min(hi_a, lo_a + step_a);
    lo_b += cb * step_b;
    hi_b = min(hi_b, lo_b + step_b);
  }
  ia = lo_a;
  ib = lo_b;
}

// Fixed trees over the workgroup (eight wavefronts): butterflies, then the
// eight wave sums as ((w0 + w1) + (w2 + w3)) + ((w4 + w5) + (w6 + w7)).
// Every thread gets the same bits.
__device__ __forceinline__ double group_sum(double x, double* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x = wave_sum_d(x);
  if (lane == 0) red[wave] = x;
  __syncthreads();
  static_assert(kLossWaves == 8, "the tree below is written for eight wavefronts");
  const double r = ((red[0] + red[1]) + (red[2] + red[3])) + ((red[4] + red[5]) + (red[6] + red[7]));
  __syncthreads();
  return r;
}

// Block exclusive prefix of per-thread flags for two classes at once:
// at0 / at1 get this thread's offsets, tot0 / tot1 the sums.
__device__ __forceinline__ void prefix2(bool f0, bool f1, int (*wave_tot)[2], int& at0, int& at1, int& tot0,
                                        int& tot1) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  const uint64_t b0 = __builtin_amdgcn_ballot_w64(f0), b1 = __builtin_amdgcn_ballot_w64(f1);
  at0 = __popcll(b0 & below);
  at1 = __popcll(b1 & below);
  if (lane == 0) {
    wave_tot[wave][0] = __popcll(b0);
    wave_tot[wave][1] = __popcll(b1);
  }
  __syncthreads();
  tot0 = tot1 = 0;
  for (int w = 0; w < kLossWaves; ++w) {
    const int v0 = wave_tot[w][0], v1 = wave_tot[w][1];
    at0 += w < wave ? v0 : 0;
    at1 += w < wave ? v1 : 0;
    tot0 += v0;
    tot1 += v1;
  }
  __syncthreads();
}

// A segment summed by a wavefront or by the workgroup, as listed for the
// second phase of the token pass.
struct SegEntry {
  long long s, e;  // its response's tokens
  float A;         // its response's advantage
  int i;           // its response
  int rel;         // its start - the span's start
};

// A segment's sum is known: finish its response if the segment is all of it,
// else park the sum for the finishing pass (segment_slot: the slots of
// different responses never meet).
__device__ __forceinline__ void emit_segment(int i, long long s, long long e, long long c, double S, float A,
                                             float* __restrict__ resp_loss, double* __restrict__ l64,
                                             double* __restrict__ segp, long long n_segp) {
  const long long T = e - s;
  if (T <= kSegTokens) {
    const double l = -(double)A * (S / (double)T);
    resp_loss[i] = (float)l;
    l64[i] = l;
  } else {
    const long long slot = segment_slot(s, c);
    if (slot < n_segp) segp[slot] = S;
  }
}

// The response holding token w kSeg (w = a window of the token pass), with
// its token range: written by loss_window_kernel, one thread per response,
// for batches of more than kLossThreads responses (smaller ones search the
// offsets inside the token pass in one round).
struct WinHolder {
  long long s, e;
  long long i;
};

__global__ __launch_bounds__(256) void loss_window_kernel(const int64_t* __restrict__ off, int n_resp,
                                                          long long n_tok, long long n_win,
                                                          WinHolder* __restrict__ win) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n_resp) return;
  long long s, e;
  resp_bounds(off, i, n_tok, s, e);
  const long long w1 = end_window(e) < n_win ? end_window(e) : n_win;
  for (long long w = first_window(s); w < w1; ++w) win[w] = WinHolder{s, e, i};
}

__global__ __launch_bounds__(kLossThreads) void loss_tokens_kernel(
    const float* __restrict__ lp, const float* __restrict__ lpr, const float* __restrict__ adv,
    const int64_t* __restrict__ off, int n_resp, long long n_tok, float* __restrict__ resp_loss,
    float* __restrict__ coef, double* __restrict__ l64, double* __restrict__ segp, long long n_segp,
    const WinHolder* __restrict__ win) {
  // the span's ratios; a segment's entries become its coefficients once the
  // segment is summed
  __shared__ float ratio_s[kSpan];
  __shared__ SegEntry wave_list[kMaxWaveSegs];
  __shared__ SegEntry group_list[kMaxGroupSegs];
  __shared__ int wave_tot[kLossWaves][2];
  __shared__ double red[kLossWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // The span [p, q): from the first segment start at or after W0 to the
  // first at or after W1 (the end of the batch if W1 is past it).
  const long long W0 = (long long)blockIdx.x * kSegTokens, W1 = W0 + kSegTokens;
  int ia, ib;
  long long sa, ea, sb, eb;
  if (win != nullptr) {  // the holders from the window map, clamped (bad offsets: unspecified, in bounds)
    const WinHolder ha = win[blockIdx.x];
    const WinHolder hb = W1 < n_tok ? win[blockIdx.x + 1] : ha;
    ia = (int)plan_clamp(ha.i, 0, n_resp - 1);
    ib = (int)plan_clamp(hb.i, 0, n_resp - 1);
    sa = plan_clamp(ha.s, 0, n_tok);
    ea = plan_clamp(ha.e, sa, n_tok);
    sb = plan_clamp(hb.s, 0, n_tok);
    eb = plan_clamp(hb.e, sb, n_tok);
  } else {
    find_responses(off, n_resp, W0, W1 < n_tok ? W1 : W0, ia, ib);
    resp_bounds(off, ia, n_tok, sa, ea);
    resp_bounds(off, ib, n_tok, sb, eb);
  }
  const Span sp = window_span(W0, n_tok, sa, ea, sb, eb);
  const long long p = sp.p, q = sp.q;
  const int span = (int)(q - p);
  const int i0 = (p < ea || ia + 1 >= n_resp) ? ia : ia + 1;

  // One memory round trip for the span's logprobs and the first round of
  // responses (offsets and advantages); then the ratios into LDS.
  float a[kSpanPerThread], b[kSpanPerThread];
#pragma unroll
  for (int k = 0; k < kSpanPerThread; ++k) {
    const int r = tid + k * kLossThreads;
    a[k] = r < span ? lp[p + r] : 0.0f;
    b[k] = r < span ? lpr[p + r] : 0.0f;
  }
  auto load_round = [&](int base, long long& s, long long& e, float& A) {
    const int i = base + tid;
    if (i < n_resp) {
      resp_bounds(off, i, n_tok, s, e);
      A = adv[i];
    } else {
      s = e = n_tok;
      A = 0.0f;
    }
  };
  long long rs, re;
  float rA;
  load_round(i0, rs, re, rA);
#pragma unroll
  for (int k = 0; k < kSpanPerThread; ++k) {
    const int r = tid + k * kLossThreads;
    if (r < span) ratio_s[r] = ratio_of(a[k], b[k]);
  }

  // Rounds of kLossThreads responses from the one holding p. A response's
  // segment in the span (at most one) of up to kLaneSeg tokens is summed at
  // once by its thread, in token order; longer ones are listed by class.
  int n_wave = 0, n_group = 0;  // uniform
  for (int base = i0, round = 0; base < n_resp && round < kMaxRounds; base += kLossThreads, ++round) {
    if (round > 0) load_round(base, rs, re, rA);
    const int i = base + tid;
    long long c = 0;
    int cls = -1;
    if (i < n_resp && segment_in_span(rs, re, p, q, c)) cls = segment_class(segment_len(re, c, q));
    int at0, at1, tot0, tot1;
    prefix2(cls == 1, cls == 2, wave_tot, at0, at1, tot0, tot1);  // (its barrier also publishes the ratios)
    if (cls == 0) {
      const int rel = (int)(c - p), len = (int)segment_len(re, c, q);
      double S = 0.0;
      for (int r = 0; r < len; ++r) S += (double)ratio_s[rel + r];
      const float k = coef_scale(rA, n_resp, re - rs);
      for (int r = 0; r < len; ++r) ratio_s[rel + r] *= k;
      emit_segment(i, rs, re, c, S, rA, resp_loss, l64, segp, n_segp);
    } else if (cls > 0) {
      const int slot = cls == 1 ? n_wave + at0 : n_group + at1;
      const SegEntry ent{rs, re, rA, i, (int)(c - p)};
      if (cls == 1 && slot < kMaxWaveSegs) wave_list[slot] = ent;
      if (cls == 2 && slot < kMaxGroupSegs) group_list[slot] = ent;
    }
    n_wave += tot0;
    n_group += tot1;
    // another round if the response after this round's last one starts
    // before q (that thread has its start as its round's end offset)
    const bool more = tid == kLossThreads - 1 && i + 1 < n_resp && re < q;
    if (!__syncthreads_or(more)) break;
  }
  __syncthreads();
  n_wave = std::min(n_wave, kMaxWaveSegs);
  n_group = std::min(n_group, kMaxGroupSegs);

  // Long segments: the whole workgroup, one at a time.
  for (int g = 0; g < n_group; ++g) {
    const SegEntry ent = group_list[g];
    const long long c = p + ent.rel;
    const int len = (int)segment_len(ent.e, c, q);
    double acc = 0.0;
    for (int r = tid; r < len; r += kLossThreads) acc += (double)ratio_s[ent.rel + r];
    const double S = group_sum(acc, red);  // every ratio of the segment has been read
    const float k = coef_scale(ent.A, n_resp, ent.e - ent.s);
    for (int r = tid; r < len; r += kLossThreads) ratio_s[ent.rel + r] *= k;
    if (tid == 0) emit_segment(ent.i, ent.s, ent.e, c, S, ent.A, resp_loss, l64, segp, n_segp);
  }
  // Middle segments: one wavefront each.
  for (int g = wave; g < n_wave; g += kLossWaves) {
    const SegEntry ent = wave_list[g];
    const long long c = p + ent.rel;
    const int len = (int)segment_len(ent.e, c, q);
    double acc = 0.0;
    for (int r = lane; r < len; r += 64) acc += (double)ratio_s[ent.rel + r];
    const double S = wave_sum_d(acc);  // every lane's reads are in S
    const float k = coef_scale(ent.A, n_resp, ent.e - ent.s);
    for (int r = lane; r < len; r += 64) ratio_s[ent.rel + r] *= k;
    if (lane == 0) emit_segment(ent.i, ent.s, ent.e, c, S, ent.A, resp_loss, l64, segp, n_segp);
  }
  if (coef == nullptr) return;
  __syncthreads();
  for (int r = tid; r < span; r += kLossThreads) coef[p + r] = ratio_s[r];
}

// Finishing pass: chunk c of kFinishChunk responses, four per thread (thread
// j: responses j, j + 256, j + 512, j + 768 of the chunk, added in that
// order), then the chunk's tree (butterflies, then the four wave sums).
constexpr int kFinishThreads = 256;
static_assert(kFinishChunk % kFinishThreads == 0, "finish geometry");

__device__ __forceinline__ double block_sum_d256(double x, double* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x = wave_sum_d(x);
  if (lane == 0) red[wave] = x;
  __syncthreads();
  const double r = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kFinishThreads) void loss_finish_kernel(
    const float* __restrict__ adv, const int64_t* __restrict__ off, int n_resp, long long n_tok,
    float* __restrict__ resp_loss, const double* __restrict__ l64, const double* __restrict__ segp, long long n_segp,
    double* __restrict__ part, float* __restrict__ loss) {
  __shared__ double red[kFinishThreads / 64];
  const int c0 = blockIdx.x * kFinishChunk;
  double sum = 0.0;
#pragma unroll
  for (int r = 0; r < kFinishChunk / kFinishThreads; ++r) {
    const int i = c0 + (int)threadIdx.x + r * kFinishThreads;
    if (i >= n_resp) continue;
    long long s, e;
    resp_bounds(off, i, n_tok, s, e);
    const long long T = e - s;
    double l;
    if (T <= 0) {  // an empty response (invalid input): a zero loss
      l = 0.0;
      resp_loss[i] = 0.0f;
    } else if (T <= kSegTokens) {
      l = l64[i];
    } else {  // the segment sums in order, eight loads in flight at a time
      const long long base = 2 * (s / kSegTokens);
      const long long nseg = (T + kSegTokens - 1) / kSegTokens;
      double S = 0.0;
      for (long long j = 0; j < nseg; j += 8) {
        double v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = (j + u < nseg && base + j + u < n_segp) ? segp[base + j + u] : 0.0;
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (j + u < nseg) S += v[u];
      }
      l = -(double)adv[i] * (S / (double)T);
      resp_loss[i] = (float)l;
    }
    sum += l;
  }
  const double tot = block_sum_d256(sum, red);
  if (threadIdx.x == 0) {
    if (gridDim.x == 1) loss[0] = (float)(tot / (double)n_resp);
    else part[blockIdx.x] = tot;
  }
}

// The chunk sums in order (thread j adds chunks j, j + 256, ...), then the
// tree of the finishing pass.
__global__ __launch_bounds__(kFinishThreads) void loss_final_kernel(const double* __restrict__ part, int n_part,
                                                                    int n_resp, float* __restrict__ loss) {
  __shared__ double red[kFinishThreads / 64];
  double acc = 0.0;
  for (int c = threadIdx.x; c < n_part; c += kFinishThreads) acc += part[c];
  const double tot = block_sum_d256(acc, red);
  if (threadIdx.x == 0) loss[0] = (float)(tot / (double)n_resp);
}

// Group advantage. A wavefront owns eight consecutive groups. Groups of at
// most 8 responses are reduced by eight lanes each (lane j holds response j;
// an xor butterfly 4, 2, 1); larger ones by the whole wavefront, one at a
// time (lane j adds responses j, j + 64, ... in order, then the 64-lane xor
// butterfly). For groups of at most 8 the two trees give the same bits (the
// 64-lane butterfly only adds exact zeros in its first three steps), so the
// choice depends on the group's size alone.
__global__ __launch_bounds__(256) void group_advantage_kernel(const float* __restrict__ rewards,
                                                              const int32_t* __restrict__ goff, int n_groups,
                                                              int n_resp, float* __restrict__ adv) {
  const int lane = threadIdx.x & 63;
  const int wv = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int sub = lane >> 3, j = lane & 7;
  const int g = wv * 8 + sub;
  int s = 0, n = 0;
  if (g < n_groups) {
    s = min(max(goff[g], 0), n_resp);
    n = min(max(goff[g + 1], s), n_resp) - s;
  }
  const bool small = n >= 1 && n <= 8;
  const float r = small && j < n ? rewards[s + j] : 0.0f;
  float x = 0.0f + r;
  x += __shfl_xor(x, 4, 64);
  x += __shfl_xor(x, 2, 64);
  x += __shfl_xor(x, 1, 64);
  if (small && j < n) adv[s + j] = r - x / (float)n;
  uint64_t big = __builtin_amdgcn_ballot_w64(j == 0 && n > 8);
  while (big) {  // ascending group order
    const int k = __builtin_ctzll(big) >> 3;
    big &= big - 1;
    const int gb = wv * 8 + k;
    const int sb = min(max(goff[gb], 0), n_resp);
    const int eb = min(max(goff[gb + 1], sb), n_resp);
    float acc = 0.0f;
    for (int i = sb + lane; i < eb; i += 64) acc += rewards[i];
    const float mean = wave_sum(acc) / (float)(eb - sb);
    for (int i = sb + lane; i < eb; i += 64) adv[i] = rewards[i] - mean;
  }
}

__global__ void check_tokens_kernel(const int32_t* __restrict__ tokens, long long n_tok, int vocab, int* flag) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t < n_tok) {
    const int y = tokens[t];
    if (y < 0 || y >= vocab) flag[0] = 1;
  }
}

__global__ void check_offsets_kernel(const int64_t* __restrict__ off, int n_resp, long long n_tok, int* flag) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i == 0 && (off[0] != 0 || off[n_resp] != n_tok)) flag[0] = 2;
  if (i < n_resp && off[i + 1] <= off[i]) flag[0] = 2;
}

long long n_finish_chunks(long long n_resp) { return ceil_div(n_resp, kFinishChunk); }

}  // namespace

hipError_t launch_group_advantage(const float* rewards, const int32_t* group_offsets, int n_groups, int n_resp,
                                  float* advantages, hipStream_t stream) {
  hipLaunchKernelGGL(group_advantage_kernel, dim3((unsigned)ceil_div(n_groups, 32)), dim3(256), 0, stream, rewards,
                     group_offsets, n_groups, n_resp, advantages);
  return hipGetLastError();
}

long long n_windows(long long n_tok) { return ceil_div(n_tok, kSegTokens); }
bool use_window_map(long long n_resp) { return n_resp > kLossThreads; }

size_t loss_workspace_bytes(long long n_tok, long long n_resp) {
  if (n_resp <= 0) return 0;
  return align256((size_t)n_resp * sizeof(double)) + align256((size_t)n_segment_slots(n_tok) * sizeof(double)) +
         align256((size_t)n_finish_chunks(n_resp) * sizeof(double)) +
         (use_window_map(n_resp) ? align256((size_t)n_windows(n_tok) * sizeof(WinHolder)) : 0);
}

hipError_t launch_reinforce_zero_loss(const float* logprob, const float* rollout_logprob, const float* advantages,
                                      const int64_t* resp_offsets, int n_resp, long long n_tok, float* resp_loss,
                                      float* loss, float* coef, void* workspace, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  double* l64 = reinterpret_cast<double*>(ws);
  double* segp = reinterpret_cast<double*>(ws + align256((size_t)n_resp * sizeof(double)));
  const long long n_segp = n_segment_slots(n_tok);
  double* part = reinterpret_cast<double*>(reinterpret_cast<char*>(segp) + align256((size_t)n_segp * sizeof(double)));
  WinHolder* win = use_window_map(n_resp) ? reinterpret_cast<WinHolder*>(reinterpret_cast<char*>(part) +
                                                                       align256((size_t)n_finish_chunks(n_resp) *
                                                                                sizeof(double)))
                                          : nullptr;
  if (n_tok > 0) {
    if (win != nullptr) {
      hipLaunchKernelGGL(loss_window_kernel, dim3((unsigned)ceil_div(n_resp, 256)), dim3(256), 0, stream,
                         resp_offsets, n_resp, n_tok, n_windows(n_tok), win);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(loss_tokens_kernel, dim3((unsigned)n_windows(n_tok)), dim3(kLossThreads), 0, stream, logprob,
                       rollout_logprob, advantages, resp_offsets, n_resp, n_tok, resp_loss, coef, l64, segp, n_segp,
                       win);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int n_chunks = (int)n_finish_chunks(n_resp);
  hipLaunchKernelGGL(loss_finish_kernel, dim3((unsigned)n_chunks), dim3(kFinishThreads), 0, stream, advantages,
                     resp_offsets, n_resp, n_tok, resp_loss, l64, segp, n_segp, part, loss);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_chunks == 1) return e;
  hipLaunchKernelGGL(loss_final_kernel, dim3(1), dim3(kFinishThreads), 0, stream, part, n_chunks, n_resp, loss);
  return hipGetLastError();
}

hipError_t launch_check_inputs(const int32_t* tokens, long long n_tok, int vocab, const int64_t* resp_offsets,
                               int n_resp, int* flag, hipStream_t stream) {
  if (tokens && n_tok > 0) {
    hipLaunchKernelGGL(check_tokens_kernel, dim3((unsigned)ceil_div(n_tok, 256)), dim3(256), 0, stream, tokens,
                       n_tok, vocab, flag);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (resp_offsets && n_resp > 0) {
    hipLaunchKernelGGL(check_offsets_kernel, dim3((unsigned)ceil_div(n_resp, 256)), dim3(256), 0, stream,
                       resp_offsets, n_resp, n_tok, flag);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace itl
