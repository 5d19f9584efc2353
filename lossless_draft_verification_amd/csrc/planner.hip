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
// its own.  Two launches.  The first is a grid of workgroups, each building
// every key in LDS (position-major, so that the lanes of a wave write
// consecutive words) and ranking its own 16 or 32 slots against them by
// counting; it stores each slot's key at its rank in the workspace: the
// sorted list of keys.  The second, one workgroup, reads the sorted keys and
// takes fp64 prefix sums of their scores (by contiguous chunks and one block
// scan), the first maximum of the ratio, and each request's admitted count
// (one more than the largest position of its keys ranked below the budget:
// a request's admitted slots are a prefix).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "specverify.h"

namespace svp {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kParts = 256;                  // threads that share one slot group's comparisons
constexpr int kGroups = kThreads / kParts;   // slot groups of a workgroup
constexpr int kPer = SV_PLAN_MAX_SLOTS / kThreads;  // entries per thread of the tail workgroup, at most
// staged confidences: request b's row at b Kp, Kp = K rounded up to odd
constexpr int kConfLds = SV_PLAN_MAX_SLOTS + SV_PLAN_MAX_SLOTS / 2;

// Workspace: the keys of the ranks below min(max_budget, slots), each where
// the second launch reads it, passed from the first launch to the second
// (sized for SV_PLAN_MAX_SLOTS: one layout for every shape).
constexpr size_t kWsBytes = 8 * (size_t)SV_PLAN_MAX_SLOTS;

struct PlanParams {
  int32_t bs, K, bmax_table;
  int32_t bmax0;  // min(bmax_table, bs K): sorted positions the second launch reads
  int32_t lg;     // log2 of C0, the power of two >= bmax0 / kThreads: positions per thread
  const float* conf;
  const int32_t* num_steps;
  const double* cost;
  double base;
  int32_t* budget;
  int32_t* draft_len;
  double* rate;
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
// positions) into out[j bs + b], and those of slots s0 .. s0 + R - 1 also
// into own[s - s0] (which the caller has set to all-ones).  The confidences
// are first staged in shared memory by loads in which the lanes of a wave
// read consecutive words, request b's at cs[b Kp] with an odd row stride Kp
// (so the lanes, one request each, then read distinct banks); one thread per
// request takes the running product.
__device__ __forceinline__ void slot_keys(const PlanParams& P, uint64_t* out, float* cs, uint64_t* own, int s0,
                                          int R) {
  const int K = P.K, bs = P.bs, N = bs * K;
  const bool pad = (K & 1) == 0;
  const int Kp = K | 1;
  const int n4 = ((uintptr_t)P.conf & 15u) == 0 ? N / 4 : 0;
  for (int q = (int)threadIdx.x; q < n4; q += kThreads) {
    const float4 v = ((const float4*)P.conf)[q];
    const float e[4] = {v.x, v.y, v.z, v.w};
    int i = 4 * q, b = pad ? i / K : 0, j = i - b * K;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      cs[pad ? b * Kp + j : i + u] = e[u];
      if (++j == K) j = 0, ++b;
    }
  }
  for (int i = 4 * n4 + (int)threadIdx.x; i < N; i += kThreads) cs[pad ? i + i / K : i] = P.conf[i];
  __syncthreads();
  for (int b = (int)threadIdx.x; b < bs; b += kThreads) {
    const int len = steps_of(P, b);
    float sc = 1.0f;
    for (int j = 0; j < K; ++j) {
      float x = cs[b * Kp + j];
      if (!(x > 0.0f)) x = 0.0f;
      if (x > 1.0f) x = 1.0f;
      sc = __fmul_rn(sc, x);
      const uint64_t key =
          j < len ? ((uint64_t)(0xFFFFFFFFu - __float_as_uint(sc)) << 32) | ((uint64_t)j << 20) | (uint64_t)b : ~0ull;
      out[j * bs + b] = key;
      if ((unsigned)(b * K + j - s0) < (unsigned)R) own[b * K + j - s0] = key;
    }
  }
}

__device__ __forceinline__ float key_score(uint64_t k) { return __uint_as_float(0xFFFFFFFFu - (uint32_t)(k >> 32)); }

// Exclusive prefix over the workgroup of one double per thread, in a fixed
// order (a wave scan, then the waves' totals).  A thread's result is formed
// from the values of lower threads only (the inclusive scan shifted by one
// lane, not minus the thread's own value), so a non-finite value reaches
// only the threads above it.
__device__ __forceinline__ double block_exclusive(double v, double* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double in = v;
  for (int o = 1; o < 64; o <<= 1) {
    const double u = __shfl_up(in, o, 64);
    if (lane >= o) in += u;
  }
  if (lane == 63) wsum[wave] = in;
  double ex = __shfl_up(in, 1, 64);
  if (lane == 0) ex = 0.0;
  __syncthreads();
  double before = 0.0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  return before + ex;
}

// For each of the R keys x[r], the keys keys[p], keys[p + kParts], ...
// (below n) below it: the lanes of a wave, taking consecutive parts, read
// consecutive keys.
template <int R>
__device__ __forceinline__ void count_below(const uint64_t* keys, int p, int n, const uint64_t* x, uint32_t* c) {
#pragma unroll
  for (int r = 0; r < R; ++r) c[r] = 0;
  int q = p;
  for (; q + 3 * kParts < n; q += 4 * kParts) {
    uint64_t k[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) k[u] = keys[q + u * kParts];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r) c[r] += k[u] < x[r] ? 1u : 0u;
  }
  for (; q < n; q += kParts) {
    const uint64_t k = keys[q];
#pragma unroll
    for (int r = 0; r < R; ++r) c[r] += k < x[r] ? 1u : 0u;
  }
}

// Ranks of the S slots [S blockIdx.x, S (blockIdx.x + 1)), S = R kGroups:
// thread t compares the R slots of group t / kParts with the keys
// t % kParts + m kParts, and the counts are summed over the parts (a wave
// holds 64 parts of one group).  Each slot's key is then stored at its rank.
template <int R>
__global__ __launch_bounds__(kThreads) void rank_kernel(PlanParams P) {
  static_assert(R % 2 == 0 && kParts == 256, "packed counts; four waves per slot group");
  constexpr int S = R * kGroups;
  __shared__ uint64_t keys[SV_PLAN_MAX_SLOTS];
  __shared__ float confs[kConfLds];
  __shared__ uint32_t part[kWaves][R / 2];
  __shared__ uint64_t own[S];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = P.bs * P.K;
  const int s0 = blockIdx.x * S;
  if (tid < S) own[tid] = ~0ull;
  slot_keys(P, keys, confs, own, s0, S);
  __syncthreads();
  const int g = tid / kParts, p = tid % kParts;  // slot group, part of the keys
  uint64_t x[R];
#pragma unroll
  for (int r = 0; r < R; ++r) x[r] = own[g * R + r];
  uint32_t c[R];
  count_below<R>(keys, p, N, x, c);
  // sum over the parts: within the wave (two counts packed per word, each
  // at most SV_PLAN_MAX_SLOTS < 2^16), then the group's four waves
  uint32_t c2[R / 2];
#pragma unroll
  for (int r = 0; r < R / 2; ++r) c2[r] = c[2 * r] | (c[2 * r + 1] << 16);
#pragma unroll
  for (int r = 0; r < R / 2; ++r)
    for (int o = 32; o > 0; o >>= 1) c2[r] += (uint32_t)__shfl_xor((int)c2[r], o, 64);
  if (lane == 0)
#pragma unroll
    for (int r = 0; r < R / 2; ++r) part[wave][r] = c2[r];
  __syncthreads();
  if (tid < S) {
    const int gg = tid / R, r = tid % R;
    const uint32_t w2 = part[4 * gg][r >> 1] + part[4 * gg + 1][r >> 1] + part[4 * gg + 2][r >> 1] +
                        part[4 * gg + 3][r >> 1];
    const uint32_t rk = (w2 >> (16 * (r & 1))) & 0xFFFFu;
    if (s0 + tid < N) {
      const uint64_t xs = own[tid];
      // rank rk belongs to thread rk / C0 of the second launch, which reads
      // its u-th entry at u kThreads + thread
      if (xs != ~0ull && (int)rk < P.bmax0) P.skey[((int)rk & ((1 << P.lg) - 1)) * kThreads + ((int)rk >> P.lg)] = xs;
    }
  }
}

// The rest, by one workgroup once the ranks are stored (the launch
// boundary makes them visible): fp64 prefix sums of the sorted scores, the
// first maximum of the ratio, each request's admitted count.  Thread t owns
// sorted positions [t C0, (t + 1) C0), stored so that its u-th entry is read
// at u kThreads + t (the lanes of a wave read consecutive words).  Every
// global load is issued first.  Entries at or past the drafted count n are
// stale, but they only reach the sums at positions past n, and no budget
// past n is taken, so the chunk sums need not wait for n: it is reduced
// beside the scan.  With more than four positions per thread the prefix
// sums then pass through LDS (rows of odd stride C0 + 1) to the threads
// holding the costs, which are loaded for position u kThreads + t.
__global__ __launch_bounds__(kThreads) void tail_kernel(PlanParams P) {
  __shared__ double gsum[(kPer + 1) * kThreads];
  __shared__ int adm[SV_PLAN_MAX_SLOTS];
  __shared__ double wsum[kWaves];
  __shared__ double red_r[kWaves];
  __shared__ int red_b[kWaves];
  __shared__ int red_n[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bmax0 = P.bmax0, lg = P.lg, C0 = 1 << lg, S = C0 + 1;
  const int r0 = tid * C0;
  // up to four positions per thread: each thread loads its own positions'
  // costs (a short stride) and takes their ratios where its prefix sums
  // are; more: the costs of positions u kThreads + t, reached through LDS
  const bool own = lg <= 2;
  uint64_t sk[kPer];
  double cc[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = u * kThreads + tid, pos = own ? r0 + u : i;
    sk[u] = (u < C0 && r0 + u < bmax0) ? P.skey[i] : ~0ull;
    cc[u] = (u < C0 && pos < bmax0) ? P.cost[pos + 1] : 1.0;
  }
  const double cost0 = tid == 0 ? P.cost[0] : 1.0;
  int mine = 0;
  for (int b = tid; b < P.bs; b += kThreads) mine += steps_of(P, b);
  for (int b = tid; b < P.bs; b += kThreads) adm[b] = 0;
  // drafted positions (the sorted list's length), reduced beside the scan
  for (int o = 32; o > 0; o >>= 1) mine += __shfl_xor(mine, o, 64);
  if (lane == 0) red_n[wave] = mine;
  // gain(B) = sum of the first B sorted scores: the chunk totals, an
  // exclusive block scan of them, then the thread's own prefix sums
  double part_sum = 0.0;
#pragma unroll
  for (int u = 0; u < kPer; ++u)
    if (u < C0 && r0 + u < bmax0) part_sum += (double)key_score(sk[u]);
  double gain = block_exclusive(part_sum, wsum);  // gain at B = r0
  int n = 0;
  for (int w = 0; w < kWaves; ++w) n += red_n[w];
  const int bmax = P.bmax_table < n ? P.bmax_table : n;
  double best_r = -INFINITY;
  int best_b = INT32_MAX;
  if (tid == 0) {  // B = 0
    best_r = P.base / cost0;
    if (!(best_r > -INFINITY)) best_r = -INFINITY, best_b = INT32_MAX;
    else best_b = 0;
  }
  if (own) {
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (u < C0 && r0 + u < bmax) {
        gain += (double)key_score(sk[u]);  // gain at B = r0 + u + 1
        const double rt = (P.base + gain) / cc[u];
        if (better(rt, r0 + u + 1, best_r, best_b)) {
          best_r = rt;
          best_b = r0 + u + 1;
        }
      }
  } else {
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (u < C0 && r0 + u < bmax) {
        gain += (double)key_score(sk[u]);
        gsum[tid * S + u] = gain;  // gain at B = r0 + u + 1
      }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = u * kThreads + tid;
      if (u < C0 && i < bmax) {
        const double rt = (P.base + gsum[(i >> lg) * S + (i & (C0 - 1))]) / cc[u];
        if (better(rt, i + 1, best_r, best_b)) {
          best_r = rt;
          best_b = i + 1;
        }
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
  }
}

// The current device's compute units, looked up once per device.
static int compute_units() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
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
  P.skey = (uint64_t*)d->workspace;
  P.bmax0 = (int32_t)(d->max_budget < n ? d->max_budget : n);
  P.lg = 0;
  while ((svp::kThreads << P.lg) < P.bmax0) ++P.lg;
  // 16 slots a workgroup where that still needs no more workgroups than the
  // device has compute units, else 32
  const int cus = svp::compute_units();
  if (cus <= 0) return SV_ERR_LAUNCH;
  constexpr int s16 = 4 * svp::kGroups, s32 = 8 * svp::kGroups;
  const hipStream_t st = (hipStream_t)stream;
  if ((n + s16 - 1) / s16 <= cus)
    hipLaunchKernelGGL(svp::rank_kernel<4>, dim3((unsigned)((n + s16 - 1) / s16)), dim3(svp::kThreads), 0, st, P);
  else
    hipLaunchKernelGGL(svp::rank_kernel<8>, dim3((unsigned)((n + s32 - 1) / s32)), dim3(svp::kThreads), 0, st, P);
  hipLaunchKernelGGL(svp::tail_kernel, dim3(1u), dim3(svp::kThreads), 0, st, P);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}
