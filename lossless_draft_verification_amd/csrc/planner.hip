// Survival top-k draft budget on gfx950: which draft positions of a batch to
// verify this step (page "New approaches to speculative decoding: block
// drafts, load-aware verification and PD disaggregation", section "Deciding
// how much to verify by load"; page "The speculative decoding zoo", section
// "The finer loop: DSpark's confidence budget").
//
// A (request, position) slot's score is the chance that all of the
// request's drafts up to that position are accepted: the fp32 product of its
// confidences so far (each clamped to [0, 1], NaN as 0).  Slots are ranked
// by score, higher first, ties to the earlier position and then to the
// smaller request index, so each request's admitted slots form a prefix.
// Admitting the top B slots is worth (base + sum of their scores) / cost[B]
// expected tokens per unit of cost; the budget is the first B in
// 0..min(max_budget, slots) that maximises it.
//
// The slot keys
//   (~bits(score)) << 32 | position << 20 | request
// order ascending in the required order (scores are >= 0, so their fp32 bit
// patterns order like their values; unused slots are all-ones and come
// last), and they are distinct, so a slot's rank is the number of keys below
// its own.  One launch of a grid of workgroups: each computes every key into
// LDS (position-major, so that the lanes of a wave write consecutive words)
// and ranks its kSlots slots against them -- thread t compares the kReg
// slots of group t / kParts with the keys t % kParts + m kParts, and the
// counts are summed over the parts (a wave holds 64 parts of one group) --
// then stores each slot's key at its rank: the sorted list of keys.  The
// last workgroup to finish takes fp64 prefix sums of the sorted scores (by
// contiguous chunks and one block scan), the first maximum of the ratio,
// and each request's admitted count (one more than the largest position of
// its keys ranked below the budget: a request's admitted slots are a
// prefix), and leaves its counter at zero for the next call.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specverify.h"

namespace svp {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kParts = 128;                  // threads that share one slot's comparisons
constexpr int kReg = 4;                      // slots a thread compares every key it reads with
constexpr int kSlots = kThreads / kParts * kReg;  // slots a workgroup ranks
constexpr int kPer = SV_PLAN_MAX_SLOTS / kThreads;  // entries per thread of the last workgroup, at most

// Workspace: the completion counter, then the keys in rank order (sized for
// SV_PLAN_MAX_SLOTS: one layout for every shape).
constexpr size_t kWsKeys = 256;
constexpr size_t kWsBytes = kWsKeys + 8 * (size_t)SV_PLAN_MAX_SLOTS;

struct PlanParams {
  int32_t bs, K, bmax_table;
  const float* conf;
  const int32_t* num_steps;
  const double* cost;
  double base;
  int32_t* budget;
  int32_t* draft_len;
  double* rate;
  uint32_t* counter;
  uint64_t* skey;
};

// Better (rate, B): a larger rate, or the same rate at a smaller B.  A NaN
// rate is never better.
__device__ __forceinline__ bool better(double r, int b, double br, int bb) {
  return r > br || (r == br && b < bb);
}

__device__ __forceinline__ int steps_of(const PlanParams& P, int b) {
  const int len = P.num_steps ? P.num_steps[b] : P.K;
  return len < 0 ? 0 : (len > P.K ? P.K : len);
}

// Keys of every slot (slot s = b K + j; all-ones past a request's drafted
// positions) into out[j bs + b]: one thread per request, its confidences
// loaded eight at a time ahead of the running product.
__device__ __forceinline__ void slot_keys(const PlanParams& P, uint64_t* out) {
  const int K = P.K, bs = P.bs;
  for (int b = (int)threadIdx.x; b < bs; b += kThreads) {
    const int len = steps_of(P, b);
    float sc = 1.0f;
    for (int j0 = 0; j0 < K; j0 += 8) {
      float c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) c[u] = j0 + u < K ? P.conf[(int64_t)b * K + j0 + u] : 0.0f;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u;
        if (j >= K) break;
        float x = c[u];
        if (!(x > 0.0f)) x = 0.0f;
        if (x > 1.0f) x = 1.0f;
        sc = __fmul_rn(sc, x);
        out[j * bs + b] = j < len ? ((uint64_t)(0xFFFFFFFFu - __float_as_uint(sc)) << 32) | ((uint64_t)j << 20) |
                                        (uint64_t)b
                                  : ~0ull;
      }
    }
  }
}

__device__ __forceinline__ float key_score(uint64_t k) { return __uint_as_float(0xFFFFFFFFu - (uint32_t)(k >> 32)); }

// Stores and loads of data that other workgroups of the launch write or read
// (agent-scope relaxed atomics: they bypass the caches that are not
// coherent across the device), and a wait for this wave's memory operations.
__device__ __forceinline__ void cst32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t cld32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void cst64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t cld64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_mem() { __builtin_amdgcn_s_waitcnt(0); }

// For each of the kReg keys x[r], the keys keys[p], keys[p + kParts], ...
// (below n) below it: the lanes of a wave, taking consecutive parts, read
// consecutive keys.
__device__ __forceinline__ void count_below(const uint64_t* keys, int p, int n, const uint64_t* x, uint32_t* c) {
#pragma unroll
  for (int r = 0; r < kReg; ++r) c[r] = 0;
  int q = p;
  for (; q + 3 * kParts < n; q += 4 * kParts) {
    uint64_t k[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) k[u] = keys[q + u * kParts];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < kReg; ++r) c[r] += k[u] < x[r] ? 1u : 0u;
  }
  for (; q < n; q += kParts) {
    const uint64_t k = keys[q];
#pragma unroll
    for (int r = 0; r < kReg; ++r) c[r] += k < x[r] ? 1u : 0u;
  }
}

// Exclusive prefix over the workgroup of one double per thread, in a fixed
// order (a wave scan, then the waves' totals).
__device__ __forceinline__ double block_exclusive(double v, double* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double in = v;
  for (int o = 1; o < 64; o <<= 1) {
    const double u = __shfl_up(in, o, 64);
    if (lane >= o) in += u;
  }
  if (lane == 63) wsum[wave] = in;
  __syncthreads();
  double before = 0.0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  return before + in - v;
}

__global__ __launch_bounds__(kThreads) void plan_kernel(PlanParams P) {
  __shared__ uint64_t keys[SV_PLAN_MAX_SLOTS];
  __shared__ uint32_t part[kWaves][kReg / 2];
  __shared__ double wsum[kWaves];
  __shared__ double red_r[kWaves];
  __shared__ int red_b[kWaves];
  __shared__ int red_n[kWaves];
  __shared__ int last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = P.bs * P.K;
  // every key; this workgroup's slots [s0, s1)
  slot_keys(P, keys);
  __syncthreads();
  const int s0 = blockIdx.x * kSlots, s1 = min(s0 + kSlots, N);
  const int g = tid / kParts, p = tid % kParts;  // slot group, part of the keys
  uint64_t x[kReg];
#pragma unroll
  for (int r = 0; r < kReg; ++r) {
    const int s = s0 + g * kReg + r;
    x[r] = s < s1 ? keys[(s % P.K) * P.bs + s / P.K] : ~0ull;
  }
  uint32_t c[kReg];
  count_below(keys, p, N, x, c);
  // sum over the parts: within the wave (two counts packed per word, each
  // at most SV_PLAN_MAX_SLOTS < 2^16), then the group's two waves
  uint32_t c2[kReg / 2];
#pragma unroll
  for (int r = 0; r < kReg / 2; ++r) c2[r] = c[2 * r] | (c[2 * r + 1] << 16);
#pragma unroll
  for (int r = 0; r < kReg / 2; ++r)
    for (int o = 32; o > 0; o >>= 1) c2[r] += (uint32_t)__shfl_xor((int)c2[r], o, 64);
  if (lane == 0)
#pragma unroll
    for (int r = 0; r < kReg / 2; ++r) part[wave][r] = c2[r];
  __syncthreads();
  static_assert(kParts == 128, "two waves per slot group");
  if (tid < kSlots) {
    const int gg = tid / kReg, r = tid % kReg;
    const uint32_t w2 = part[2 * gg][r >> 1] + part[2 * gg + 1][r >> 1];
    const uint32_t rk = (w2 >> (16 * (r & 1))) & 0xFFFFu;
    const int s = s0 + tid;
    if (s < s1) {
      const uint64_t xs = keys[(s % P.K) * P.bs + s / P.K];
      if (xs != ~0ull) cst64(&P.skey[rk], xs);
    }
  }
  // the last workgroup to finish does the rest: every wave's stores are
  // complete before the count
  wait_mem();
  __syncthreads();
  if (tid == 0)
    last = __hip_atomic_fetch_add(P.counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1u;
  __syncthreads();
  if (!last) return;
  // drafted positions: the keys in use (the sorted list's length)
  int mine = 0;
  for (int i = tid; i < N; i += kThreads) mine += keys[i] != ~0ull ? 1 : 0;
  for (int o = 32; o > 0; o >>= 1) mine += __shfl_xor(mine, o, 64);
  if (lane == 0) red_n[wave] = mine;
  // every load up front: the sorted keys and the costs that can be needed
  const int bmax0 = min(P.bmax_table, N);
  const int C0 = (bmax0 + kThreads - 1) / kThreads;  // <= kPer
  const int r0 = tid * C0;
  uint64_t sk[kPer];
  double cs[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    sk[u] = (u < C0 && r0 + u < bmax0) ? cld64(&P.skey[r0 + u]) : ~0ull;
    cs[u] = (u < C0 && r0 + u < bmax0) ? P.cost[r0 + u + 1] : 1.0;
  }
  __syncthreads();
  int n = 0;
  for (int w = 0; w < kWaves; ++w) n += red_n[w];
  const int bmax = P.bmax_table < n ? P.bmax_table : n;
  // each request's admitted count, in LDS over the keys (no longer needed)
  int* adm = (int*)keys;
  for (int b = tid; b < P.bs; b += kThreads) adm[b] = 0;
  // gain(B) = sum of the first B sorted scores.  Thread t owns positions
  // [t C0, (t + 1) C0) of the sorted list, below bmax: its chunk total, an
  // exclusive block scan of the totals, then its own B.
  double part_sum = 0.0;
#pragma unroll
  for (int u = 0; u < kPer; ++u)
    if (u < C0 && r0 + u < bmax) part_sum += (double)key_score(sk[u]);
  double gain = block_exclusive(part_sum, wsum);  // gain at B = r0
  double best_r = -INFINITY;
  int best_b = INT32_MAX;
  if (tid == 0) {  // B = 0
    best_r = P.base / P.cost[0];
    if (!(best_r > -INFINITY)) best_r = -INFINITY, best_b = INT32_MAX;
    else best_b = 0;
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    if (u < C0 && r0 + u < bmax) {
      gain += (double)key_score(sk[u]);
      const int B = r0 + u + 1;
      const double rt = (P.base + gain) / cs[u];
      if (better(rt, B, best_r, best_b)) {
        best_r = rt;
        best_b = B;
      }
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
  // a request's admitted count: one more than the largest position among
  // its keys ranked below the budget
#pragma unroll
  for (int u = 0; u < kPer; ++u)
    if (u < C0 && r0 + u < bstar)
      atomicMax(&adm[(int)(sk[u] & 0xFFFFFu)], (int)((sk[u] >> 20) & 0xFFFu) + 1);
  __syncthreads();
  for (int b = tid; b < P.bs; b += kThreads) P.draft_len[b] = adm[b];
  if (tid == 0) {
    *P.budget = bstar;
    if (P.rate) *P.rate = best_r;
    cst32(P.counter, 0u);
  }
}

}  // namespace svp

extern "C" size_t sv_plan_workspace_bytes(int32_t batch, int32_t max_steps) {
  if (batch < 1 || max_steps < 1 || max_steps > 64 || (int64_t)batch * max_steps > SV_PLAN_MAX_SLOTS) return 0;
  return svp::kWsBytes;
}

extern "C" sv_status sv_plan_budget(const sv_plan_desc* d, void* stream) {
  if (d == nullptr) return SV_ERR_INVALID_ARGUMENT;
  if (d->batch < 1 || d->max_steps < 1 || d->max_steps > 64 || d->max_budget < 0) return SV_ERR_INVALID_ARGUMENT;
  if ((int64_t)d->batch * d->max_steps > SV_PLAN_MAX_SLOTS) return SV_ERR_UNSUPPORTED;
  if (d->confidence == nullptr || d->cost == nullptr || d->budget == nullptr || d->draft_len == nullptr)
    return SV_ERR_INVALID_ARGUMENT;
  const int64_t n = (int64_t)d->batch * d->max_steps;
  if (d->workspace == nullptr || ((uintptr_t)d->workspace & 255u) != 0) return SV_ERR_INVALID_ARGUMENT;
  if (d->workspace_bytes < svp::kWsBytes) return SV_ERR_WORKSPACE_TOO_SMALL;
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
  uint8_t* ws = (uint8_t*)d->workspace;
  P.counter = (uint32_t*)ws;
  P.skey = (uint64_t*)(ws + svp::kWsKeys);
  const int grid = (int)((n + svp::kSlots - 1) / svp::kSlots);
  hipLaunchKernelGGL(svp::plan_kernel, dim3((unsigned)grid), dim3(svp::kThreads), 0, (hipStream_t)stream, P);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}
