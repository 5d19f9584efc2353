// Survival top-k draft budget on gfx950: which draft positions of a batch to
// verify this step (page "New approaches to speculative decoding: block
// drafts, load-aware verification and PD disaggregation", section "Deciding
// how much to verify by load"; page "The speculative decoding zoo", section
// "The finer loop: DSpark's confidence budget").
//
// A (request, position) slot's score is the chance that all of the
// request's drafts up to that position are accepted: the fp32 product of its
// confidences so far (each clamped to [0, 1], NaN as 0).  Slots are ranked by score, higher first, ties to the earlier
// position and then to the smaller request index, so each request's admitted
// slots form a prefix.  Admitting the top B slots is worth
// (base + sum of their scores) / cost[B] expected tokens per unit of cost;
// the budget is the first B in 0..min(max_budget, slots) that maximises it.
//
// One workgroup of 1024 threads does the whole plan in LDS (a batch has at
// most SV_PLAN_MAX_SLOTS slots): the slot keys
//   (~bits(score)) << 32 | position << 20 | request
// sort ascending in the required order (scores are >= 0, so their fp32 bit
// patterns order like their values; unused slots are all-ones and sort
// last).  A request's keys are already ascending along its positions, so
// the slots start as bs sorted runs of K and a bottom-up merge sorts them in
// ceil(log2 bs) rounds: each key finds its place in the partner run by a
// binary search (keys of the left run go before equal keys of the right
// one) and moves to the other LDS buffer.  Then fp64 prefix sums of the
// sorted scores by contiguous chunks and one block scan; the first maximum
// of the ratio by a block reduction; the admitted count of each request by
// an atomic max of position + 1.  The work is a few thousand slots:
// latency, not bandwidth, bounds it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specverify.h"

namespace svp {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

struct PlanParams {
  int32_t bs, K, bmax_table;
  const float* conf;
  const int32_t* num_steps;
  const double* cost;
  double base;
  int32_t* budget;
  int32_t* draft_len;
  double* rate;
};

// Better (rate, B): a larger rate, or the same rate at a smaller B.  A NaN
// rate is never better.
__device__ __forceinline__ bool better(double r, int b, double br, int bb) {
  return r > br || (r == br && b < bb);
}

// Number of keys of the sorted range [lo, hi) of k below x (or, with
// `upper`, not above x).
__device__ __forceinline__ int count_before(const uint64_t* k, int lo, int hi, uint64_t x, bool upper) {
  int n = hi - lo;
  int base = lo;
  while (n > 0) {
    const int half = n >> 1;
    const uint64_t v = k[base + half];
    if (v < x || (upper && v == x)) {
      base += half + 1;
      n -= half + 1;
    } else {
      n = half;
    }
  }
  return base - lo;
}

__global__ __launch_bounds__(kThreads) void plan_kernel(PlanParams P) {
  __shared__ uint64_t buf[2][SV_PLAN_MAX_SLOTS];
  __shared__ double scan[kThreads];
  __shared__ double red_r[kWaves];
  __shared__ int red_b[kWaves];
  __shared__ int n_slots;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = P.K, N = P.bs * P.K;
  uint64_t* keys = buf[0];
  if (tid == 0) n_slots = 0;
  for (int i = tid; i < N; i += kThreads) keys[i] = ~0ull;
  __syncthreads();
  // scores: one thread per request walks its positions in order
  int mine = 0;
  for (int b = tid; b < P.bs; b += kThreads) {
    int len = P.num_steps ? P.num_steps[b] : K;
    len = len < 0 ? 0 : (len > K ? K : len);
    float s = 1.0f;
    for (int j = 0; j < len; ++j) {
      float c = P.conf[(int64_t)b * K + j];
      if (!(c > 0.0f)) c = 0.0f;
      if (c > 1.0f) c = 1.0f;
      s = __fmul_rn(s, c);
      keys[b * K + j] = ((uint64_t)(0xFFFFFFFFu - __float_as_uint(s)) << 32) | ((uint64_t)j << 20) | (uint64_t)b;
    }
    mine += len;
  }
  if (mine) atomicAdd(&n_slots, mine);
  // bottom-up merge of the sorted runs
  int cur = 0;
  for (int L = K; L < N; L <<= 1) {
    __syncthreads();
    const uint64_t* src = buf[cur];
    uint64_t* dst = buf[cur ^ 1];
    for (int p = tid; p < N; p += kThreads) {
      const int run = p / L;
      const int a0 = (run & ~1) * L, b0 = a0 + L, b1 = min(b0 + L, N);
      const uint64_t x = src[p];
      int pos;
      if (b0 >= N) pos = p;  // the last run has no partner this round
      else if (run & 1) pos = a0 + (p - b0) + count_before(src, a0, b0, x, true);
      else pos = a0 + (p - a0) + count_before(src, b0, b1, x, false);
      dst[pos] = x;
    }
    cur ^= 1;
  }
  __syncthreads();
  keys = buf[cur];
  const int n = n_slots;
  const int bmax = P.bmax_table < n ? P.bmax_table : n;
  // gain(B) = sum of the first B sorted scores.  Thread t owns positions
  // [t*C, (t+1)*C) of the sorted list (C = ceil(bmax / 1024)): its chunk
  // total, an exclusive block scan of the totals, then its own B values.
  const int C = (bmax + kThreads - 1) / kThreads;
  const int r0 = tid * C, r1 = min(r0 + C, bmax);
  double part = 0.0;
  for (int r = r0; r < r1; ++r) part += (double)__uint_as_float(0xFFFFFFFFu - (uint32_t)(keys[r] >> 32));
  scan[tid] = part;
  __syncthreads();
  for (int o = 1; o < kThreads; o <<= 1) {  // inclusive Hillis-Steele scan, fixed order
    const double v = tid >= o ? scan[tid - o] : 0.0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  double gain = scan[tid] - part;  // exclusive prefix: gain at B = r0
  double best_r = -INFINITY;
  int best_b = INT32_MAX;
  if (tid == 0) {  // B = 0
    best_r = P.base / P.cost[0];
    if (!(best_r > -INFINITY)) best_r = -INFINITY, best_b = INT32_MAX;
    else best_b = 0;
  }
  for (int r = r0; r < r1; ++r) {
    gain += (double)__uint_as_float(0xFFFFFFFFu - (uint32_t)(keys[r] >> 32));
    const int B = r + 1;
    const double rt = (P.base + gain) / P.cost[B];
    if (better(rt, B, best_r, best_b)) {
      best_r = rt;
      best_b = B;
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const double orr = __shfl_xor(best_r, o, 64);
    const int ob = __shfl_xor(best_b, o, 64);
    if (better(orr, ob, best_r, best_b)) {
      best_r = orr;
      best_b = ob;
    }
  }
  if (lane == 0) {
    red_r[wave] = best_r;
    red_b[wave] = best_b;
  }
  __syncthreads();
  best_r = red_r[0];
  best_b = red_b[0];
  for (int w = 1; w < kWaves; ++w)
    if (better(red_r[w], red_b[w], best_r, best_b)) {
      best_r = red_r[w];
      best_b = red_b[w];
    }
  const int bstar = best_b == INT32_MAX ? 0 : best_b;
  for (int b = tid; b < P.bs; b += kThreads) P.draft_len[b] = 0;
  __syncthreads();
  for (int r = tid; r < bstar; r += kThreads) {
    const uint64_t key = keys[r];
    atomicMax(&P.draft_len[(int)(key & 0xFFFFFu)], (int)((key >> 20) & 63u) + 1);
  }
  if (tid == 0) {
    *P.budget = bstar;
    if (P.rate) *P.rate = best_r;
  }
}

}  // namespace svp

extern "C" sv_status sv_plan_budget(const sv_plan_desc* d, void* stream) {
  if (d == nullptr) return SV_ERR_INVALID_ARGUMENT;
  if (d->batch < 1 || d->max_steps < 1 || d->max_steps > 64 || d->max_budget < 0) return SV_ERR_INVALID_ARGUMENT;
  if ((int64_t)d->batch * d->max_steps > SV_PLAN_MAX_SLOTS) return SV_ERR_UNSUPPORTED;
  if (d->confidence == nullptr || d->cost == nullptr || d->budget == nullptr || d->draft_len == nullptr)
    return SV_ERR_INVALID_ARGUMENT;
  svp::PlanParams P;
  P.bs = d->batch;
  P.K = d->max_steps;
  P.bmax_table = d->max_budget;
  P.conf = d->confidence;
  P.num_steps = d->num_steps;
  P.cost = d->cost;
  P.base = d->base_tokens;
  P.budget = d->budget;
  P.draft_len = d->draft_len;
  P.rate = d->rate;
  hipLaunchKernelGGL(svp::plan_kernel, dim3(1), dim3(svp::kThreads), 0, (hipStream_t)stream, P);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}
