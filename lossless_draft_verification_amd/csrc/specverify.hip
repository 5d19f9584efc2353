// specverify.hip - libspecverify: batched lossless verification of speculative
// drafts on AMD Instinct MI355X (gfx950, wave64).
//
// The method (page "投机解码" (Speculative decoding), section "接受规则为什么不改变分布"):
// softmax each target row, accept drafts left to right with probability
// min(1, p/q), resample the first rejected position from max(0, p - q), draw a
// bonus token when all drafts pass; one-hot drafts and target-only trees are
// the special cases of the same rule.  The public contract is in
// include/specverify.h.
//
// Work decomposition.  One call is three kinds of work item:
//   K1  a streaming chunk of one logit row: max, first argmax and
//       sum exp((l - m)/T) of CH consecutive entries (16-byte nontemporal
//       loads, wave shuffles, a cross-wave LDS reduction).  Almost all HBM
//       bytes are read here, once.
//   K2  the per-request decision step, run by the workgroup that finishes a
//       request's last K1 chunk: combine the row partials in fp64, gather
//       p (and q) at the draft ids, draw the Philox coins, find the first
//       rejection (chain) or walk the tree, write the outputs, and publish
//       the request's sampling job.
//   K3  a chunk of one sampling race (residual, one-hot residual or bonus)
//       over 4096 vocabulary ids: Philox noise, fp32 keys with rigorous
//       error bounds, and a short list of near-maximal candidates; the
//       workgroup that finishes a request's last K3 chunk re-evaluates the
//       candidates in fp64 and writes the emitted token.
// The fused schedule runs everything in one launch with one work item per
// workgroup.  Item order interleaves the K1 chunks of request g with the K3
// chunks of request g - L, so the ALU-heavy races of early requests overlap
// the HBM stream of later ones, and a launch is paid once.  A K3 item waits
// (bounded, about a second, then SV_REQ_INTERNAL) for its request's K2.
// Workgroups are dispatched in index order, so every K1 item a waiter
// depends on (a smaller index) is already running or finished: the waits
// always end.  There is no global counter: per-request counters and flags
// are reset by their last user, so the workspace is ready for the next call
// without any reset pass.  The split schedule is two stream-ordered
// launches: K1 (each request's last workgroup running its K2, as above),
// then K3 with nothing left to wait for.  The phased schedule runs K1, K2
// and K3 as three launches.  All three give bit-identical results.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "specverify.h"

namespace sv {

constexpr int kWG = 256;
constexpr int kWaves = kWG / 64;
#ifndef SV_K1_VEC
#define SV_K1_VEC 2
#endif
#ifndef SV_K1_SUBS
#define SV_K1_SUBS 8
#endif
constexpr int kVecPerThread = SV_K1_VEC;        // 16-byte loads per thread in a K1 sub-chunk
constexpr int kSubChunks = SV_K1_SUBS;          // sub-chunks per K1 work item (register double buffer)
constexpr int kK3Groups = 4;                    // groups of 4 vocabulary ids per thread in a K3 chunk
constexpr int kK3Chunk = 4 * kWG * kK3Groups;   // 4096 ids per K3 chunk
constexpr int kCandMax = 8;                     // candidates kept per K3 chunk
constexpr int kMergeCandMax = 256;              // candidates re-evaluated per race
constexpr uint32_t kSpinLimit = 1u << 20;       // bounded waits (about a second)

enum { MODE_CHAIN = 0, MODE_TREE = 1, MODE_ROWS = 2 };
enum { JOB_NONE = 0, JOB_P = 1, JOB_RESID = 2, JOB_EXCL = 3 };
enum { SCHED_FUSED = 0, SCHED_PHASED = 1, SCHED_SPLIT = 2 };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- workspace
struct Ctrl {
  uint32_t aborted;   // a bounded wait expired (left set: the workspace must be re-initialised)
  uint32_t pad[63];
};
struct Sync {
  uint32_t k1_count;  // K1 chunks of the request finished in this call (reset by the K2 runner)
  uint32_t k3_count;  // K3 chunks of the request finished in this call (reset by the last one)
  uint32_t ready;     // 1 once the request's job is published (reset by the last K3 chunk)
  uint32_t pad;
};
// Target logit (and draft probability) at a draft token, gathered by the K1
// chunk that holds it: chain slot r = row r's draft, tree slot n = node n's
// token in its parent's row.
struct Gather {
  uint32_t l;         // fp32 bits of the logit
  uint32_t q;         // fp32 bits of q at the draft (chain, draft probabilities)
};
struct Partial {
  uint64_t s;         // bits of the chunk sum of 2^((l - m_c) log2(e)/T) (fp64), or a NaN flag for greedy rows
  uint64_t m_amax;    // bits of the chunk max (fp32, low half) and the smallest index attaining it (high half)
};
struct Job {
  int32_t kind, row, qrow, r, n_excl, out_slot;
  float m, c_hi, c_lo, inv_s;
  double s, t;
  int32_t excl[SV_MAX_NODES];
};
struct K3Rec {
  float lo;           // max over the chunk of the keys' lower bounds
  int32_t count;      // candidates listed
  float ovf_hi;       // if more than kCandMax qualified: the largest upper bound among them, else -inf
  int32_t pad;
  int32_t idx[kCandMax];
  float hi[kCandMax];
};

constexpr size_t kSyncOffset = 256;
constexpr size_t kDataOffset = kSyncOffset + sizeof(Sync) * SV_MAX_BATCH;

__host__ __device__ constexpr size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Params {
  int32_t mode, bs, R, V, k;
  int32_t dtype, draft_kind, aligned, q_aligned;
  int64_t lstride, qstride;
  const void* logits;
  const float* q;
  const int32_t* ids;
  const float* temp;
  const uint64_t* seed;
  const int32_t* node_tokens;
  const int32_t* parent;
  int32_t* accept_len;
  int32_t* tokens;
  int32_t* status;
  double* p_draft;
  int32_t* accept_path;
  float* rs_max;
  int32_t* rs_amax;
  double* rs_sum;
  int32_t* rs_status;
  Ctrl* ctrl;
  Sync* sync;
  Gather* gat;        // [bs][SV_MAX_NODES]
  Job* jobs;
  Partial* part;
  K3Rec* k3;
  int32_t CH, CPR, n1r, C3, lag, n_tickets, sched;
  uint32_t flags;
};

// ------------------------------------------------------------- small helpers
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

template <bool BF16>
__device__ __forceinline__ float load_logit(const Params& P, int64_t row, int64_t y) {
  const int64_t off = row * P.lstride + y;
  if (BF16) return bf16_to_f32(((const uint16_t*)P.logits)[off]);
  return ((const float*)P.logits)[off];
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ int wave_min_i(int v) {
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// log2(e)/T as an unevaluated fp32 sum hi + lo (about 48 significant bits),
// so that (l - m) * log2(e)/T carries no systematic rounding bias.  hi is
// rounded toward zero and lo is kept strictly positive, so that for a masked
// entry (l = -inf) fma(d, hi, d * lo) is -inf rather than inf - inf = NaN.
__device__ __forceinline__ void scale_pair(double T, float& hi, float& lo) {
  const double c = 1.4426950408889634074 / T;
  hi = __double2float_rz(c);
  if ((double)hi == c) hi = __int_as_float(__float_as_int(hi) - 1);
  lo = (float)(c - (double)hi);
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): per round, with
// multipliers A = 0xD2511F53 (on word 0) and B = 0xCD9E8D57 (on word 2),
// (c0,c1,c2,c3) <- (hi(B c2) ^ c1 ^ k0, lo(B c2), hi(A c0) ^ c3 ^ k1, lo(A c0)),
// and the key advances by (0x9E3779B9, 0xBB67AE85) between rounds.
__device__ __forceinline__ u32x4 philox10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const uint64_t pa = (uint64_t)0xD2511F53u * c.x;
    const uint64_t pb = (uint64_t)0xCD9E8D57u * c.z;
    u32x4 n;
    n.x = (uint32_t)(pb >> 32) ^ c.y ^ k0;
    n.y = (uint32_t)pb;
    n.z = (uint32_t)(pa >> 32) ^ c.w ^ k1;
    n.w = (uint32_t)pa;
    c = n;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// Uniform in (0,1): (2*(w>>9)+1) * 2^-24, exact in fp32.
__device__ __forceinline__ float uniform_f32(uint32_t w) {
  return __builtin_fmaf((float)(w >> 9), 0x1p-23f, 0x1p-24f);
}
__device__ __forceinline__ double uniform_f64(uint32_t w) { return (double)uniform_f32(w); }

__device__ __forceinline__ double coin(uint64_t seed, int b, int r) {
  u32x4 c = {0u, (uint32_t)r, (uint32_t)b, 0u};
  return uniform_f64(philox10(c, (uint32_t)seed, (uint32_t)(seed >> 32)).x);
}
__device__ __forceinline__ uint32_t noise_word(uint64_t seed, int b, int r, int y) {
  u32x4 c = {(uint32_t)y >> 2, (uint32_t)r, (uint32_t)b, 1u};
  u32x4 o = philox10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  const int w = y & 3;
  return w == 0 ? o.x : w == 1 ? o.y : w == 2 ? o.z : o.w;
}

// Communication between workgroups.  Every word that another workgroup
// reads is written and read with agent-scope atomic stores and loads, which
// are coherent across the XCDs' separate L2 caches on their own; the writer
// waits for its stores to complete (s_waitcnt) before it bumps the relaxed
// counter or flag that announces them, and the reader loads the data only
// after it has observed that counter or flag.  No release/acquire fence is
// used: on gfx950 those write back and invalidate a whole L2 cache, which
// thousands of workgroups per call cannot afford.
__device__ __forceinline__ void cst32(void* p, uint32_t v) {
  __hip_atomic_store((uint32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void cst64(void* p, uint64_t v) {
  __hip_atomic_store((uint64_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t cld32(const void* p) {
  return __hip_atomic_load((const uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t cld64(const void* p) {
  return __hip_atomic_load((const uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void cst_f32(float* p, float v) { cst32(p, __float_as_uint(v)); }
__device__ __forceinline__ void cst_f64(double* p, double v) { cst64(p, (uint64_t)__double_as_longlong(v)); }
__device__ __forceinline__ float cld_f32(const float* p) { return __uint_as_float(cld32(p)); }
__device__ __forceinline__ double cld_f64(const double* p) { return __longlong_as_double((long long)cld64(p)); }
__device__ __forceinline__ int32_t cld_i32(const int32_t* p) { return (int32_t)cld32(p); }
__device__ __forceinline__ void cst_i32(int32_t* p, int32_t v) { cst32(p, (uint32_t)v); }
// Wait until this wave's memory operations have completed.
__device__ __forceinline__ void wait_mem() { __builtin_amdgcn_s_waitcnt(0); }
__device__ __forceinline__ uint32_t atomic_add_relaxed(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A value that is the same in every lane, made visibly uniform (an SGPR) so
// that branches on it are scalar branches rather than divergent regions.
__device__ __forceinline__ int uniform_i(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint32_t uniform_u(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }

// The scalar part of a published job, read once with coherent loads.
struct JobView {
  int kind, row, qrow, r, n_excl, out_slot;
  float m, c_hi, c_lo, inv_s;
  double s, t;
  const int32_t* excl;  // read with coherent loads
};

// Shared memory of one workgroup (every role reuses it).
struct Smem {
  float red_f[kWaves];
  int red_i[kWaves];
  double red_d[kWaves];
  int flag;
  uint32_t ticket;
  // per-row results of the decision step
  float rm[SV_MAX_NODES];
  int ramax[SV_MAX_NODES];
  double rs[SV_MAX_NODES];
  int rbad[SV_MAX_NODES];
  double px[SV_MAX_NODES];
  double u[SV_MAX_NODES];
  double qx[SV_MAX_NODES];
  int par[SV_MAX_NODES];
  int tok[SV_MAX_NODES];
  int xs[SV_MAX_NODES];
  int path[SV_MAX_NODES];
  int a, kb, status, cur, len, emit;
  // race candidates
  JobView job;
  int ncand;
  int cand_y[kMergeCandMax];
  double cand_key[kMergeCandMax];
  float cand_h[kCandMax];
  int overflow;
};

__device__ __forceinline__ float block_max(float v, Smem& sm) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sm.red_f[wave] = v;
  __syncthreads();
  float r = sm.red_f[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = fmaxf(r, sm.red_f[w]);
  return r;
}
__device__ __forceinline__ int block_min_i(int v, Smem& sm) {
  v = wave_min_i(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sm.red_i[wave] = v;
  __syncthreads();
  int r = sm.red_i[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = min(r, sm.red_i[w]);
  return r;
}
__device__ __forceinline__ double block_sum_d(double v, Smem& sm) {
  v = wave_sum_d(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sm.red_d[wave] = v;
  __syncthreads();
  double r = sm.red_d[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r += sm.red_d[w];
  return r;
}

// Temperature of the request (chain/tree) or of the row (row statistics).
__device__ __forceinline__ float temp_of(const Params& P, int b) { return P.temp[b]; }
__device__ __forceinline__ bool is_stochastic(float T) { return T > 0.f && isfinite(T); }

// Number of chain drafts in use: the index of the first -1, else k.  Every
// wave computes the same value (k <= 63 fits one wave).
__device__ __forceinline__ int chain_kb(const Params& P, int b, int& xi) {
  const int lane = threadIdx.x & 63;
  xi = (lane < P.k) ? P.ids[(int64_t)b * P.k + lane] : -1;
  const uint64_t m = __ballot(lane < P.k && xi == -1);
  return m ? (int)__builtin_ctzll(m) : P.k;
}

// ===================================================================== K1
// Streaming statistics of one work item: kSubChunks consecutive sub-chunks of
// one row, each 256 threads x kVecPerThread nontemporal 16-byte loads
// (consecutive lanes on consecutive 16-byte pieces).  The loads of sub-chunk
// s+1 are in flight while sub-chunk s is reduced (a register double buffer).
// Per sub-chunk a thread first takes the max of its entries.  Stochastic
// rows then add 2^(l c - o) over the entries, with c = log2(e)/T rounded to
// fp32 and o = fl(m c) the fp32 offset of the thread's running max m: one
// fma and one exp2 per entry, the terms summed pairwise in fp32 and the
// running sum kept in fp64, rescaled by 2^(o_old - o_new) when the max
// grows.  At the end the rounding of o is undone exactly (m c is exact in
// fp64) and the threads are combined with the fp64 scale, so a term
// 2^((l - m) log2(e)/T) is evaluated with a relative exponent error of at
// most 2^-24 from c plus the fma's rounding.  Greedy rows (and every row of
// a row-statistics call) keep the first index of the running max and a NaN
// flag.  One block reduction per item gives the item's (max, first argmax,
// sum), in a fixed order (bit-reproducible).
template <bool BF16>
__device__ __forceinline__ void k1_issue(const Params& P, int64_t elem0, int n, u32x4* raw) {
  constexpr int EPV = BF16 ? 8 : 4;
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < kVecPerThread; ++j) {
    const int e0 = (j * kWG + tid) * EPV;
    if (P.aligned && e0 + EPV <= n) {
      raw[j] = __builtin_nontemporal_load((const u32x4*)((const char*)P.logits + (elem0 + e0) * (BF16 ? 2 : 4)));
    } else {
      // partial (or unaligned) group: scalar loads, -inf past the end
      uint32_t w[4];
      if (BF16) {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const int i0 = e0 + 2 * h;
          const uint32_t lo = (i0 < n) ? ((const uint16_t*)P.logits)[elem0 + i0] : 0xFF80u;
          const uint32_t hi = (i0 + 1 < n) ? ((const uint16_t*)P.logits)[elem0 + i0 + 1] : 0xFF80u;
          w[h] = lo | (hi << 16);
        }
      } else {
#pragma unroll
        for (int h = 0; h < 4; ++h)
          w[h] = (e0 + h < n) ? ((const uint32_t*)P.logits)[elem0 + e0 + h] : 0xFF800000u;
      }
      raw[j] = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
}

// Running per-thread statistics of a K1 item.
struct K1Run {
  float m;       // running max
  float off;     // fl(m c): the running sum is relative to 2^off (-inf while m = -inf)
  int idx;       // first index (in the item) of the running max
  double s;      // sum of 2^(l c - off) (stochastic rows)
  bool nan;      // a NaN was seen (greedy rows; stochastic rows see it in s)
};

// The thread's entries of one sub-chunk, widened to fp32 (bf16 widening is
// exact; as a conversion its results need no canonicalisation before max).
template <bool BF16>
__device__ __forceinline__ void k1_unpack(const u32x4* v, float* x) {
#pragma unroll
  for (int j = 0; j < kVecPerThread; ++j) {
    if (BF16) {
      __bf16 h[8];
      __builtin_memcpy(h, &v[j], 16);
#pragma unroll
      for (int i = 0; i < 8; ++i) x[j * 8 + i] = (float)h[i];
    } else {
      x[j * 4 + 0] = __uint_as_float(v[j].x);
      x[j * 4 + 1] = __uint_as_float(v[j].y);
      x[j * 4 + 2] = __uint_as_float(v[j].z);
      x[j * 4 + 3] = __uint_as_float(v[j].w);
    }
  }
}

// Folds the NV entries x of one sub-chunk into the running statistics.
// Entry i sits at item offset base + (i / EPV) * kWG * EPV + i % EPV, so the
// thread's order is the row order and the first hit is the smallest index.
template <int NV, int EPV, bool STOCH, bool NEED_AMAX>
__device__ __forceinline__ void k1_fold_sub(const float* x, int base, float c, K1Run& st) {
#pragma clang fp contract(off)
  float mx = x[0];
#pragma unroll
  for (int i = 1; i < NV; ++i) mx = fmaxf(mx, x[i]);
  if (!STOCH || NEED_AMAX) {
    if (mx > st.m) {  // strict: an earlier sub-chunk keeps a tie
      int pos = 0;
#pragma unroll
      for (int i = NV - 1; i >= 0; --i)
        if (x[i] == mx) pos = (i / EPV) * kWG * EPV + (i % EPV);
      st.idx = base + pos;
    }
  }
  if (!STOCH) {
    bool nan_seen = false;
#pragma unroll
    for (int i = 0; i < NV; ++i) nan_seen |= (x[i] != x[i]);
    st.nan |= nan_seen;
    st.m = fmaxf(st.m, mx);
  } else {
    const float mn = fmaxf(st.m, mx);
    const float off = (mn == -INFINITY) ? 0.f : mn * c;  // keeps l = -inf terms at 2^-inf = 0
    // rescale factor: 0 until the first finite max (st.off = -inf; never
    // inf * 0), exactly 1 while the max is unchanged, else at most 1
    const float f = __builtin_amdgcn_exp2f(st.off - off);
    float e[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) e[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], c, -off));
#pragma unroll
    for (int w = 1; w < NV; w *= 2)
#pragma unroll
      for (int i = 0; i + w < NV; i += 2 * w) e[i] += e[i + w];
    st.s = st.s * (double)f + (double)e[0];
    st.m = mn;
    st.off = (mn == -INFINITY) ? -INFINITY : off;
  }
}

// Streams the item's sub-chunks from raw0 (the first sub-chunk, already in
// flight) and writes the item's partial.
template <bool BF16, bool STOCH, bool NEED_AMAX>
__device__ __forceinline__ void k1_item_stats(const Params& P, int64_t row, int c, float T, u32x4* raw0, Smem& sm) {
  constexpr int EPV = BF16 ? 8 : 4;
  constexpr int NV = kVecPerThread * EPV;  // entries per thread per sub-chunk
  constexpr int SUB = NV * kWG;            // entries per sub-chunk
  const int64_t start = (int64_t)c * P.CH;
  const int n_item = (int)min((int64_t)P.CH, (int64_t)P.V - start);
  const int64_t elem0 = row * P.lstride + start;
  float cf = 0.f;
  double cd = 0.0;
  if (STOCH) {
    cd = 1.4426950408889634074 / (double)T;
    cf = (float)cd;
  }
  K1Run st;
  st.m = -INFINITY;
  st.off = -INFINITY;
  st.idx = INT32_MAX;
  st.s = 0.0;
  st.nan = false;
  u32x4 cur[kVecPerThread], nxt[kVecPerThread];
#pragma unroll
  for (int j = 0; j < kVecPerThread; ++j) cur[j] = raw0[j];
#pragma unroll 1
  for (int sub = 0; sub < kSubChunks; ++sub) {
    if (sub + 1 < kSubChunks && (sub + 1) * SUB < n_item)
      k1_issue<BF16>(P, elem0 + (int64_t)(sub + 1) * SUB, n_item - (sub + 1) * SUB, nxt);
    if (sub * SUB < n_item) {
      float x[NV];
      k1_unpack<BF16>(cur, x);
      k1_fold_sub<NV, EPV, STOCH, NEED_AMAX>(x, sub * SUB + threadIdx.x * EPV, cf, st);
    }
#pragma unroll
    for (int j = 0; j < kVecPerThread; ++j) cur[j] = nxt[j];
  }
  const float mc = block_max(st.m, sm);
  double out_s = 0.0;
  int32_t out_amax = (int32_t)start;
  if (!STOCH || NEED_AMAX) {
    const int amax = block_min_i(st.m == mc ? st.idx : INT32_MAX, sm);
    out_amax = (int32_t)(start + (amax == INT32_MAX ? 0 : amax));
  }
  if (!STOCH) {
    const int any_nan = block_min_i(st.nan ? 0 : 1, sm) == 0;
    out_s = any_nan ? __builtin_nan("") : 0.0;
  } else {
    // this thread's sum relative to 2^((mc) log2(e)/T): undo the offset's
    // rounding (m cf is exact in fp64), then move from m to mc at the exact scale
    double mine = 0.0;
    if (st.m != -INFINITY && mc != -INFINITY)
      mine = st.s * exp2((double)st.off - (double)st.m * (double)cf + ((double)st.m - (double)mc) * cd);
    else if (st.s != st.s)
      mine = st.s;
    out_s = block_sum_d(mine, sm);
  }
  if (threadIdx.x == 0) {
    Partial* dst = &P.part[row * P.CPR + c];
    cst64(&dst->s, (uint64_t)__double_as_longlong(out_s));
    cst64(&dst->m_amax, (uint64_t)__float_as_uint(mc) | ((uint64_t)(uint32_t)out_amax << 32));
  }
}

// ===================================================================== K2
// Combine the chunk partials of one row (one wave): max, first argmax,
// NaN/inf detection, and S = sum_c S_c 2^((m_c - m) log2(e)/T) in fp64.
__device__ void combine_row(const Params& P, int64_t row, float T, float& m_out, int& amax_out, double& s_out,
                            int& bad_out) {
  const int lane = threadIdx.x & 63;
  float m = -INFINITY;
  int nanflag = 0;
  for (int c = lane; c < P.CPR; c += 64) {
    const Partial* pt = &P.part[row * P.CPR + c];
    const float pm = __uint_as_float((uint32_t)cld64(&pt->m_amax));
    const double ps = __longlong_as_double((long long)cld64(&pt->s));
    m = fmaxf(m, pm);
    if (ps != ps) nanflag = 1;
  }
  m = wave_max(m);
  int amax = INT32_MAX;
  double s = 0.0;
  const bool stoch = is_stochastic(T);
  const double cd = stoch ? 1.4426950408889634074 / (double)T : 0.0;
  for (int c = lane; c < P.CPR; c += 64) {
    const Partial* pt = &P.part[row * P.CPR + c];
    const uint64_t ma = cld64(&pt->m_amax);
    const float pm = __uint_as_float((uint32_t)ma);
    const double ps = __longlong_as_double((long long)cld64(&pt->s));
    if (pm == m) amax = min(amax, (int)(int32_t)(uint32_t)(ma >> 32));
    if (stoch && pm != -INFINITY && m != -INFINITY) s += ps * exp2(((double)pm - (double)m) * cd);
  }
  amax = wave_min_i(amax);
  s = wave_sum_d(s);
  const int any_nan = wave_min_i(nanflag ? 0 : 1) == 0;
  m_out = m;
  amax_out = amax;
  s_out = stoch ? s : __builtin_nan("");
  bad_out = any_nan || m == INFINITY || m == -INFINITY || (stoch && !(s > 0.0));
}

// p(y) of a stochastic row in fp64: exp((l - m)/T) / S.
__device__ __forceinline__ double p_at(double l, float m, double T, double S) { return exp((l - (double)m) / T) / S; }

// Called by thread 0 of a stochastic request once its job is written: wait
// for the job's stores, then raise the request's ready flag (the last of
// the request's K3 chunks lowers it again).
__device__ void publish_job(const Params& P, int b) {
  wait_mem();
  cst32(&P.sync[b].ready, 1u);
}

// Writes the sampling job of request b (thread 0 only).
__device__ void write_job(const Params& P, int b, int kind, int row, int qrow, int r, int out_slot, float m,
                          double S, double T) {
  Job* J = &P.jobs[b];
  cst_i32(&J->kind, kind);
  if (kind == JOB_NONE) return;
  cst_i32(&J->row, row);
  cst_i32(&J->qrow, qrow);
  cst_i32(&J->r, r);
  cst_i32(&J->out_slot, out_slot);
  cst_f32(&J->m, m);
  cst_f64(&J->s, S);
  cst_f64(&J->t, T);
  float hi, lo;
  scale_pair(T, hi, lo);
  cst_f32(&J->c_hi, hi);
  cst_f32(&J->c_lo, lo);
  cst_f32(&J->inv_s, (float)(1.0 / S));
}

__device__ __forceinline__ void k2_rows(const Params& P, int b, Smem& sm) {
  // Row-statistics mode: the "request" is one row.
  const int tid = threadIdx.x;
  if (tid < 64) {
    const float T = temp_of(P, b);
    float m;
    int amax, bad;
    double s;
    combine_row(P, b, T, m, amax, s, bad);
    if (tid == 0) {
      if (P.rs_max) P.rs_max[b] = m;
      if (P.rs_amax) P.rs_amax[b] = amax;
      if (P.rs_sum) P.rs_sum[b] = s;
      if (P.rs_status) P.rs_status[b] = bad ? SV_REQ_NONFINITE : SV_REQ_OK;
    }
  }
}

template <bool BF16>
__device__ __forceinline__ void k2_chain(const Params& P, int b, Smem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = P.k, R = P.R, V = P.V;
  const float Tf = temp_of(P, b);
  const double T = (double)Tf;
  const bool greedy = !(Tf > 0.f);
  // the gathered target logit and q at this lane's draft (K1 stored them)
  uint64_t gl = 0;
  if (wave == 0 && lane < k && !greedy) gl = cld64(&P.gat[(int64_t)b * SV_MAX_NODES + lane]);
  int xi;
  const int kb = chain_kb(P, b, xi);
  const bool bad_id = __ballot(lane < kb && (xi < 0 || xi >= V)) != 0;
  int status = !isfinite(Tf) ? SV_REQ_BAD_TEMPERATURE : bad_id ? SV_REQ_BAD_DRAFT_ID : SV_REQ_OK;
  if (status == SV_REQ_OK) {
    for (int r = wave; r <= kb; r += kWaves) {
      float m;
      int amax, bad;
      double s;
      combine_row(P, (int64_t)b * R + r, Tf, m, amax, s, bad);
      if (lane == 0) {
        sm.rm[r] = m;
        sm.ramax[r] = amax;
        sm.rs[r] = s;
        sm.rbad[r] = bad;
      }
    }
  }
  __syncthreads();
  if (status == SV_REQ_OK)
    for (int r = 0; r <= kb; ++r)
      if (sm.rbad[r]) status = SV_REQ_NONFINITE;
  if (status == SV_REQ_OK && wave == 0 && lane < kb) {
    const int64_t row = (int64_t)b * R + lane;
    double p;
    (void)row;
    if (greedy) {
      p = (xi == sm.ramax[lane]) ? 1.0 : 0.0;
    } else {
      p = p_at((double)__uint_as_float((uint32_t)gl), sm.rm[lane], T, sm.rs[lane]);
      sm.u[lane] = coin(P.seed[b], b, lane);
      if (P.draft_kind == SV_DRAFT_PROBS) sm.qx[lane] = (double)__uint_as_float((uint32_t)(gl >> 32));
    }
    sm.px[lane] = p;
    sm.xs[lane] = xi;
  }
  __syncthreads();
  if (tid == 0) {
    int a = 0;
    if (status == SV_REQ_OK) {
      for (int i = 0; i < kb; ++i) {
        bool accept;
        if (greedy) accept = (sm.xs[i] == sm.ramax[i]);
        else if (P.draft_kind == SV_DRAFT_ONEHOT) accept = sm.u[i] < sm.px[i];
        else if (sm.qx[i] <= 0.0) accept = sm.px[i] > 0.0;
        else accept = sm.u[i] * sm.qx[i] < sm.px[i];
        if (!accept) break;
        ++a;
      }
    }
    sm.a = a;
    sm.kb = kb;
    sm.status = status;
    P.accept_len[b] = a;
    if (P.status) P.status[b] = status;
    if (status == SV_REQ_OK && !greedy) {
      const int kind = (a < kb) ? (P.draft_kind == SV_DRAFT_PROBS ? JOB_RESID : JOB_EXCL) : JOB_P;
      write_job(P, b, kind, b * R + a, b * k + a, a, b * R + a, sm.rm[a], sm.rs[a], T);
      cst_i32(&P.jobs[b].n_excl, kind == JOB_EXCL ? 1 : 0);
      if (kind == JOB_EXCL) cst_i32(&P.jobs[b].excl[0], sm.xs[a]);
    } else {
      write_job(P, b, JOB_NONE, 0, 0, 0, 0, 0.f, 1.0, 1.0);
    }
  }
  __syncthreads();
  const int a = sm.a;
  for (int i = tid; i < R; i += kWG) {
    int t = -1;
    if (sm.status == SV_REQ_OK) {
      if (i < a) t = sm.xs[i];
      else if (i == a && greedy) t = sm.ramax[a];
      else if (i == a) continue;  // written by the race merge
    }
    P.tokens[(int64_t)b * R + i] = t;
  }
  if (P.p_draft)
    for (int i = tid; i < k; i += kWG)
      P.p_draft[(int64_t)b * k + i] = (sm.status == SV_REQ_OK && i < kb) ? sm.px[i] : __builtin_nan("");
  __syncthreads();
  if (tid == 0 && is_stochastic(Tf)) publish_job(P, b);
}

template <bool BF16>
__device__ __forceinline__ void k2_tree(const Params& P, int b, Smem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = P.R, V = P.V;
  const float Tf = temp_of(P, b);
  const double T = (double)Tf;
  const bool greedy = !(Tf > 0.f);
  uint32_t gl = 0;  // node lane's token's logit in its parent's row (K1 stored it)
  if (wave == 0 && lane >= 1 && lane < N && !greedy) gl = cld32(&P.gat[(int64_t)b * SV_MAX_NODES + lane].l);
  int par = -2, tok = -1;
  if (lane < N) {
    par = P.parent[(int64_t)b * N + lane];
    tok = P.node_tokens[(int64_t)b * N + lane];
  }
  bool bad = false;
  if (lane < N) {
    if (lane == 0) bad = (par != -1);
    else bad = (par < 0 || par >= lane || tok < 0 || tok >= V);
  }
  for (int j = 1; j < N; ++j) {
    const int pj = __shfl(par, j, 64), tj = __shfl(tok, j, 64);
    if (lane >= 1 && lane < N && j > lane && pj == par && tj == tok) bad = true;
  }
  const bool bad_tree = __ballot(bad) != 0;
  int status = !isfinite(Tf) ? SV_REQ_BAD_TEMPERATURE : bad_tree ? SV_REQ_BAD_TREE : SV_REQ_OK;
  if (wave == 0 && lane < N) {
    sm.par[lane] = par;
    sm.tok[lane] = tok;
  }
  if (status == SV_REQ_OK) {
    for (int r = wave; r < N; r += kWaves) {
      float m;
      int amax, badr;
      double s;
      combine_row(P, (int64_t)b * N + r, Tf, m, amax, s, badr);
      if (lane == 0) {
        sm.rm[r] = m;
        sm.ramax[r] = amax;
        sm.rs[r] = s;
        sm.rbad[r] = badr;
      }
    }
  }
  __syncthreads();
  if (status == SV_REQ_OK)
    for (int r = 0; r < N; ++r)
      if (sm.rbad[r]) status = SV_REQ_NONFINITE;
  // per-node values: p_parent(tok_n) and the coin drawn when node n is current
  if (status == SV_REQ_OK && wave == 0 && lane < N) {
    if (lane >= 1) {
      const int pn = sm.par[lane];
      if (greedy) sm.px[lane] = (tok == sm.ramax[pn]) ? 1.0 : 0.0;
      else sm.px[lane] = p_at((double)__uint_as_float(gl), sm.rm[pn], T, sm.rs[pn]);
    }
    if (!greedy) sm.u[lane] = coin(P.seed[b], b, lane);
  }
  __syncthreads();
  if (tid == 0) {
    int cur = 0, len = 0, emit = -1;
    int kind = JOB_NONE;
    if (status == SV_REQ_OK) {
      for (;;) {
        int next = -1, nchild = 0;
        if (greedy) {
          for (int c = cur + 1; c < N; ++c)
            if (sm.par[c] == cur && sm.tok[c] == sm.ramax[cur]) next = c;
          if (next < 0) {
            emit = sm.ramax[cur];
            break;
          }
        } else {
          const double u = sm.u[cur];
          double acc = 0.0;
          for (int c = cur + 1; c < N; ++c) {
            if (sm.par[c] != cur) continue;
            ++nchild;
            const double pc = sm.px[c];
            acc += pc;
            if (pc > 0.0 && u < acc) {
              next = c;
              break;
            }
          }
          if (next < 0) {
            kind = nchild ? JOB_EXCL : JOB_P;
            break;
          }
        }
        sm.path[len++] = next;
        cur = next;
      }
    }
    sm.cur = cur;
    sm.len = len;
    sm.emit = emit;
    sm.status = status;
    P.accept_len[b] = len;
    if (P.status) P.status[b] = status;
    if (kind != JOB_NONE) {
      write_job(P, b, kind, b * N + cur, 0, cur, b * N + len, sm.rm[cur], sm.rs[cur], T);
      int ne = 0;
      if (kind == JOB_EXCL)
        for (int c = cur + 1; c < N; ++c)
          if (sm.par[c] == cur) cst_i32(&P.jobs[b].excl[ne++], sm.tok[c]);
      cst_i32(&P.jobs[b].n_excl, ne);
    } else {
      write_job(P, b, JOB_NONE, 0, 0, 0, 0, 0.f, 1.0, 1.0);
    }
  }
  __syncthreads();
  const int len = sm.len;
  for (int i = tid; i < N; i += kWG) {
    int node = -1, t = -1;
    bool skip = false;
    if (sm.status == SV_REQ_OK) {
      if (i < len) {
        node = sm.path[i];
        t = sm.tok[node];
      } else if (i == len) {
        if (greedy) t = sm.emit;
        else skip = true;  // written by the race merge
      }
    }
    P.accept_path[(int64_t)b * N + i] = node;
    if (!skip) P.tokens[(int64_t)b * N + i] = t;
  }
  __syncthreads();
  if (tid == 0 && is_stochastic(Tf)) publish_job(P, b);
}

// ===================================================================== K3

// Thread 0 reads the job (coherent loads) into shared memory; the caller
// synchronises before the others read it.
__device__ __forceinline__ void read_job(const Params& P, int b, JobView& v) {
  const Job* src = &P.jobs[b];
  v.kind = cld_i32(&src->kind);
  v.row = cld_i32(&src->row);
  v.qrow = cld_i32(&src->qrow);
  v.r = cld_i32(&src->r);
  v.n_excl = cld_i32(&src->n_excl);
  v.out_slot = cld_i32(&src->out_slot);
  v.m = cld_f32(&src->m);
  v.c_hi = cld_f32(&src->c_hi);
  v.c_lo = cld_f32(&src->c_lo);
  v.inv_s = cld_f32(&src->inv_s);
  v.s = cld_f64(&src->s);
  v.t = cld_f64(&src->t);
  v.excl = src->excl;
}

// Exact fp64 race key of vocabulary id y, the same formula as the
// definition: w(y) / (-ln U_y).  With use_p the weight is p itself (the
// fallback for an all-zero residual).
template <bool BF16>
__device__ double race_weight_f64(const Params& P, const JobView& J, int y, bool use_p) {
  const double p = p_at((double)load_logit<BF16>(P, J.row, y), J.m, J.t, J.s);
  if (use_p) return p;
  if (J.kind == JOB_RESID) {
    const double d = p - (double)P.q[(int64_t)J.qrow * P.qstride + y];
    return d > 0.0 ? d : 0.0;
  }
  if (J.kind == JOB_EXCL)
    for (int i = 0; i < J.n_excl; ++i)
      if (cld_i32(&J.excl[i]) == y) return 0.0;
  return p;
}
template <bool BF16>
__device__ double race_key_f64(const Params& P, const JobView& J, int b, int y, bool use_p) {
  const double w = race_weight_f64<BF16>(P, J, y, use_p);
  const double U = uniform_f64(noise_word(P.seed[b], b, J.r, y));
  return w / -log(U);
}

// Pick the larger key, ties to the smaller id.
__device__ __forceinline__ bool better(double ka, int ya, double kb_, int yb) {
  return ka > kb_ || (ka == kb_ && ya < yb);
}

// Whole-row race in fp64 by one workgroup: used when the fp32 screen
// cannot certify its candidate list, and on request.
template <bool BF16>
__device__ __forceinline__ int race_row_f64(const Params& P, const JobView& J, int b, Smem& sm) {
  // an all-zero weight vector falls back to p
  int any_pos = 0;
  for (int y = threadIdx.x; y < P.V; y += kWG)
    if (race_weight_f64<BF16>(P, J, y, false) > 0.0) any_pos = 1;
  const bool use_p = block_min_i(any_pos ? 0 : 1, sm) == 1;
  double best_k = -1.0;
  int best_y = INT32_MAX;
  for (int y = threadIdx.x; y < P.V; y += kWG) {
    const double key = race_key_f64<BF16>(P, J, b, y, use_p);
    if (better(key, y, best_k, best_y)) {
      best_k = key;
      best_y = y;
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const double ok = __shfl_xor(best_k, o, 64);
    const int oy = __shfl_xor(best_y, o, 64);
    if (better(ok, oy, best_k, best_y)) {
      best_k = ok;
      best_y = oy;
    }
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) {
    sm.red_d[wave] = best_k;
    sm.red_i[wave] = best_y;
  }
  __syncthreads();
  best_k = sm.red_d[0];
  best_y = sm.red_i[0];
  for (int w = 1; w < kWaves; ++w)
    if (better(sm.red_d[w], sm.red_i[w], best_k, best_y)) {
      best_k = sm.red_d[w];
      best_y = sm.red_i[w];
    }
  return best_y;
}

// Merge of one race: L = the largest certified lower bound over all chunks;
// the true winner's upper bound reaches L, so re-evaluating in fp64 every
// listed candidate with upper bound >= L finds it, unless some chunk had to
// drop qualifying entries with an upper bound >= L (then, or when L is too
// small for fp32 to certify, the whole row is raced in fp64).
template <bool BF16>
__device__ __forceinline__ void k3_merge(const Params& P, int b, const JobView& J, Smem& sm) {
  const int tid = threadIdx.x;
  float lo = -INFINITY, ovf = -INFINITY;
  for (int c = tid; c < P.C3; c += kWG) {
    const K3Rec* rec = &P.k3[(int64_t)b * P.C3 + c];
    lo = fmaxf(lo, cld_f32(&rec->lo));
    ovf = fmaxf(ovf, cld_f32(&rec->ovf_hi));
  }
  const float L = block_max(lo, sm);
  const float OVF = block_max(ovf, sm);
  if (tid == 0) {
    sm.ncand = 0;
    sm.overflow = 0;
  }
  __syncthreads();
  bool fallback = (P.flags & SV_FLAG_FP64_RACE) || !(L >= 0x1p-70f) || OVF >= L;
  if (!fallback) {
    for (int c = tid; c < P.C3; c += kWG) {
      const K3Rec* rec = &P.k3[(int64_t)b * P.C3 + c];
      const int cnt = cld_i32(&rec->count);
      for (int i = 0; i < cnt; ++i) {
        if (cld_f32(&rec->hi[i]) >= L) {
          const int slot = atomicAdd(&sm.ncand, 1);
          if (slot < kMergeCandMax) sm.cand_y[slot] = cld_i32(&rec->idx[i]);
          else sm.overflow = 1;
        }
      }
    }
    __syncthreads();
    fallback = sm.overflow != 0;
  }
  int best_y = -1;
  if (!fallback) {
    const int nc = sm.ncand;
    for (int i = tid; i < nc; i += kWG) sm.cand_key[i] = race_key_f64<BF16>(P, J, b, sm.cand_y[i], false);
    __syncthreads();
    if (tid == 0) {
      double bk = -1.0;
      int by = INT32_MAX;
      for (int i = 0; i < nc; ++i)
        if (better(sm.cand_key[i], sm.cand_y[i], bk, by)) {
          bk = sm.cand_key[i];
          by = sm.cand_y[i];
        }
      sm.flag = (bk > 0.0) ? by : -1;  // a zero best key means an all-zero residual
    }
    __syncthreads();
    best_y = sm.flag;
    fallback = best_y < 0;
  }
  if (fallback) best_y = race_row_f64<BF16>(P, J, b, sm);
  if (tid == 0) P.tokens[J.out_slot] = best_y;
}

// Per-element fp32 race keys with certified bounds, for the 4*kK3Groups ids
// this thread owns in chunk c3.  e = 2^t approximates exp((l - m)/T) with
// relative error at most eta = (|t| 2^-21 + 2^-17) (argument rounding plus
// v_exp_f32, far above the measured 2^-23.5); E2 = -log2(U) and its
// reciprocal are each within 2^-22 (v_log_f32 measured at 2^-23 over every
// possible U, v_rcp_f32 at 2^-23.4).  The key w / E2 is a constant multiple
// of w / E.  hi[] gets each key's upper bound (-1 when the id does not
// race); lo_max the largest lower bound.
template <bool BF16, int KIND>
__device__ void k3_chunk_keys(const Params& P, const JobView& J, int b, int c3, float* hi, float& lo_max) {
  const int tid = threadIdx.x;
  const uint64_t seed = P.seed[b];
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  const float m = J.m, chi = J.c_hi, clo = J.c_lo, inv_s = J.inv_s;
  const int jr = J.r;
  const int64_t lrow = (int64_t)J.row * P.lstride;
  const int64_t qrow = (int64_t)J.qrow * P.qstride;
  uint32_t excl_mask = 0;  // bit g*4+i: this thread's id is a removed token
  if (KIND == JOB_EXCL) {
    const int n_excl = J.n_excl;
    for (int i = 0; i < n_excl; ++i) {
      const int z = cld_i32(&J.excl[i]) - c3 * kK3Chunk;
      if (z >= 0 && z < kK3Chunk) {
        const int gi = z >> 2;
        if ((gi % kWG) == tid) excl_mask |= 1u << ((gi / kWG) * 4 + (z & 3));
      }
    }
  }
#pragma unroll
  for (int g = 0; g < kK3Groups; ++g) {
    const int y0 = c3 * kK3Chunk + 4 * (g * kWG + tid);
    float l[4], qv[4] = {0.f, 0.f, 0.f, 0.f};
    const bool full = y0 + 4 <= P.V;
    if (full && P.aligned) {
      if (BF16) {
        const u32x2 w = __builtin_nontemporal_load((const u32x2*)((const uint16_t*)P.logits + lrow + y0));
        l[0] = __uint_as_float(w.x << 16);
        l[1] = __uint_as_float(w.x & 0xffff0000u);
        l[2] = __uint_as_float(w.y << 16);
        l[3] = __uint_as_float(w.y & 0xffff0000u);
      } else {
        const u32x4 w = __builtin_nontemporal_load((const u32x4*)((const float*)P.logits + lrow + y0));
        l[0] = __uint_as_float(w.x);
        l[1] = __uint_as_float(w.y);
        l[2] = __uint_as_float(w.z);
        l[3] = __uint_as_float(w.w);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) l[i] = (y0 + i < P.V) ? load_logit<BF16>(P, J.row, y0 + i) : -INFINITY;
    }
    if (KIND == JOB_RESID) {
      if (full && P.q_aligned) {
        const u32x4 w = __builtin_nontemporal_load((const u32x4*)(P.q + qrow + y0));
        qv[0] = __uint_as_float(w.x);
        qv[1] = __uint_as_float(w.y);
        qv[2] = __uint_as_float(w.z);
        qv[3] = __uint_as_float(w.w);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) qv[i] = (y0 + i < P.V) ? P.q[qrow + y0 + i] : 0.f;
      }
    }
    const u32x4 ctr = {(uint32_t)y0 >> 2, (uint32_t)jr, (uint32_t)b, 1u};
    const u32x4 rnd = philox10(ctr, k0, k1);
    const uint32_t words[4] = {rnd.x, rnd.y, rnd.z, rnd.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float d = l[i] - m;
      const float t = __builtin_fmaf(d, chi, d * clo);
      const float e = __builtin_amdgcn_exp2f(t);
      const float e2 = -__builtin_amdgcn_logf(uniform_f32(words[i]));  // -log2 U > 0
      const float rE = __builtin_amdgcn_rcpf(e2);
      const float eta = __builtin_fmaf(fminf(fabsf(t), 256.f), 0x1p-21f, 0x1p-17f);
      float h, lw;
      if (KIND == JOB_RESID) {
        const float p = e * inv_s;
        const float w = fmaxf(p - qv[i], 0.f);
        const float err = __builtin_fmaf(eta, p, 0x1p-22f * w);
        h = (w + err) * rE * (1.f + 0x1p-20f);
        lw = (w - err) * rE * (1.f - 0x1p-20f);
      } else {
        const float key = e * rE;
        h = __builtin_fmaf(key, eta + 0x1p-20f, key);
        lw = __builtin_fmaf(-key, eta + 0x1p-20f, key);
      }
      const bool out = !(y0 + i < P.V) || (KIND == JOB_EXCL && ((excl_mask >> (g * 4 + i)) & 1u));
      hi[g * 4 + i] = out ? -1.f : h;
      if (!out) lo_max = fmaxf(lo_max, lw);
    }
  }
}

template <bool BF16>
__device__ void k3_chunk(const Params& P, int b, int c3, Smem& sm) {
  const int tid = threadIdx.x;
  if (!is_stochastic(temp_of(P, b))) return;  // greedy requests and bad temperatures race nothing
  if (tid == 0) {
    int ok = 1;
    if (P.sched == SCHED_FUSED) {
      uint32_t spins = 0;
      while (cld32(&P.sync[b].ready) == 0u) {
        __builtin_amdgcn_s_sleep(8);
        if (++spins > kSpinLimit || cld32(&P.ctrl->aborted)) {
          ok = 0;
          break;
        }
      }
      if (!ok) {
        cst32(&P.ctrl->aborted, 1u);
        if (P.status) P.status[b] = SV_REQ_INTERNAL;
      }
    }
    sm.flag = ok;
    if (ok) read_job(P, b, sm.job);
  }
  __syncthreads();
  if (!uniform_i(sm.flag)) return;
  const JobView J = sm.job;
  const int kind = uniform_i(J.kind);
  float L = -INFINITY, ovf_hi = -INFINITY;
  if (kind != JOB_NONE) {
    float hi[kK3Groups * 4];
    float lo_max = -INFINITY;
    if (kind == JOB_RESID) k3_chunk_keys<BF16, JOB_RESID>(P, J, b, c3, hi, lo_max);
    else if (kind == JOB_EXCL) k3_chunk_keys<BF16, JOB_EXCL>(P, J, b, c3, hi, lo_max);
    else k3_chunk_keys<BF16, JOB_P>(P, J, b, c3, hi, lo_max);
    L = block_max(lo_max, sm);
    if (tid == 0) sm.ncand = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kK3Groups * 4; ++i) {
      if (hi[i] >= L && hi[i] > 0.f) {
        const int slot = atomicAdd(&sm.ncand, 1);
        if (slot < kCandMax) {
          sm.cand_y[slot] = c3 * kK3Chunk + 4 * ((i >> 2) * kWG + tid) + (i & 3);
          sm.cand_h[slot] = hi[i];
        }
        ovf_hi = fmaxf(ovf_hi, hi[i]);
      }
    }
    ovf_hi = block_max(ovf_hi, sm);
  }
  // wave 0 publishes the chunk's record, then thread 0 counts the chunk; the
  // last chunk of the request lowers the ready flag and merges
  if (tid < 64) {
    if (kind != JOB_NONE) {
      K3Rec* rec = &P.k3[(int64_t)b * P.C3 + c3];
      const int n = sm.ncand;
      const int cnt = min(n, kCandMax);
      if (tid < cnt) {
        cst_i32(&rec->idx[tid], sm.cand_y[tid]);
        cst_f32(&rec->hi[tid], sm.cand_h[tid]);
      }
      if (tid == 0) {
        cst_f32(&rec->lo, L);
        cst_i32(&rec->count, cnt);
        cst_f32(&rec->ovf_hi, n > kCandMax ? ovf_hi : -INFINITY);
      }
      wait_mem();
    }
    if (tid == 0) {
      const uint32_t old = atomic_add_relaxed(&P.sync[b].k3_count, 1u);
      const int last = (old == (uint32_t)P.C3 - 1u);
      if (last) {
        cst32(&P.sync[b].k3_count, 0u);
        cst32(&P.sync[b].ready, 0u);
      }
      sm.flag = last && kind != JOB_NONE;
    }
  }
  __syncthreads();
  if (uniform_i(sm.flag)) k3_merge<BF16>(P, b, J, sm);
}

// ===================================================================== driver
// K1 work item (request b, row r, chunk c).  Its HBM loads are issued first;
// then the request's temperature and drafts decide whether the row is needed
// (rows after a chain's first -1 are not).  Wave 0 also gathers the target
// logit (and q) at the draft tokens that fall in this chunk, so the decision
// step needs no dependent loads.  The workgroup that completes the
// request's last chunk runs its decision step.
template <int MODE, bool BF16>
__device__ __forceinline__ void run_k1(const Params& P, int b, int r, int c, Smem& sm) {
  const int64_t row = (int64_t)b * P.R + r;
  const int64_t start = (int64_t)c * P.CH;
  u32x4 raw0[kVecPerThread];
  k1_issue<BF16>(P, row * P.lstride + start, (int)min((int64_t)P.CH, (int64_t)P.V - start), raw0);
  const float T = temp_of(P, b);
  bool need = true;
  if (MODE == MODE_CHAIN) {
    int xi;
    const int kb = chain_kb(P, b, xi);
    need = (r <= kb) && isfinite(T);
  } else if (MODE == MODE_TREE) {
    need = isfinite(T);
  }
  const bool stoch = uniform_i(is_stochastic(T));
  if (uniform_i(need)) {
    if (stoch) k1_item_stats<BF16, true, MODE == MODE_ROWS>(P, row, c, T, raw0, sm);
    else k1_item_stats<BF16, false, false>(P, row, c, T, raw0, sm);
    if (MODE != MODE_ROWS && threadIdx.x < 64 && stoch) {
      const int lane = threadIdx.x;
      const int64_t stop = min(start + P.CH, (int64_t)P.V);
      int tok = -1, slot = -1;
      if (MODE == MODE_CHAIN) {
        if (lane == 0 && r < P.k) {
          tok = P.ids[(int64_t)b * P.k + r];
          slot = r;
        }
      } else if (lane >= 1 && lane < P.R && P.parent[(int64_t)b * P.R + lane] == r) {
        tok = P.node_tokens[(int64_t)b * P.R + lane];
        slot = lane;
      }
      if (slot >= 0 && tok >= start && tok < stop) {
        const float l = load_logit<BF16>(P, row, tok);
        float q = 0.f;
        if (MODE == MODE_CHAIN && P.draft_kind == SV_DRAFT_PROBS) q = P.q[((int64_t)b * P.k + r) * P.qstride + tok];
        cst64(&P.gat[(int64_t)b * SV_MAX_NODES + slot], (uint64_t)__float_as_uint(l) | ((uint64_t)__float_as_uint(q) << 32));
      }
    }
  }
  if (P.sched == SCHED_PHASED) return;
  if (threadIdx.x == 0) {
    wait_mem();  // this wave's partial and gathers are complete
    const uint32_t old = atomic_add_relaxed(&P.sync[b].k1_count, 1u);
    sm.flag = (old == (uint32_t)P.n1r - 1u);
  }
  __syncthreads();
  if (uniform_i(sm.flag)) {
    if (threadIdx.x == 0) cst32(&P.sync[b].k1_count, 0u);
    if (MODE == MODE_CHAIN) k2_chain<BF16>(P, b, sm);
    else if (MODE == MODE_TREE) k2_tree<BF16>(P, b, sm);
    else k2_rows(P, b, sm);
  }
}

// Work item t of the fused schedule.  Blocks g = 0 .. bs+L-1: block g holds
// the K1 chunks of request g (if g < bs) followed by the K3 chunks of
// request g - L (if g >= L).
template <int MODE, bool BF16>
__device__ __forceinline__ void run_item(const Params& P, uint32_t t, Smem& sm) {
  const uint32_t n1 = (uint32_t)P.n1r, n3 = (uint32_t)P.C3, L = (uint32_t)P.lag, bs = (uint32_t)P.bs;
  const uint32_t seg1 = L * n1;
  const uint32_t seg2 = (bs - L) * (n1 + n3);
  int b = 0, kind1 = 1;
  uint32_t o = 0;
  if (t < seg1) {
    b = (int)(t / n1);
    o = t % n1;
  } else if (t < seg1 + seg2) {
    const uint32_t u = t - seg1;
    const uint32_t g = L + u / (n1 + n3);
    const uint32_t oo = u % (n1 + n3);
    if (oo < n1) {
      b = (int)g;
      o = oo;
    } else {
      b = (int)(g - L);
      o = oo - n1;
      kind1 = 0;
    }
  } else {
    const uint32_t u = t - seg1 - seg2;
    b = (int)(bs - L + u / n3);
    o = u % n3;
    kind1 = 0;
  }
  if (kind1) {
    run_k1<MODE, BF16>(P, b, (int)(o / (uint32_t)P.CPR), (int)(o % (uint32_t)P.CPR), sm);
  } else if (MODE != MODE_ROWS) {
    k3_chunk<BF16>(P, b, (int)o, sm);
  }
}

template <int MODE, bool BF16>
__global__ __launch_bounds__(kWG) void fused_kernel(Params P) {
  __shared__ Smem sm;
  run_item<MODE, BF16>(P, blockIdx.x, sm);
}

// Phased schedule, K1: one item per workgroup.
template <int MODE, bool BF16>
__global__ __launch_bounds__(kWG) void k1_kernel(Params P) {
  __shared__ Smem sm;
  const uint32_t t = blockIdx.x;
  const int b = (int)(t / (uint32_t)P.n1r);
  const uint32_t o = t % (uint32_t)P.n1r;
  run_k1<MODE, BF16>(P, b, (int)(o / (uint32_t)P.CPR), (int)(o % (uint32_t)P.CPR), sm);
}

template <int MODE, bool BF16>
__global__ __launch_bounds__(kWG) void k2_kernel(Params P) {
  __shared__ Smem sm;
  const int b = blockIdx.x;
  if (MODE == MODE_CHAIN) k2_chain<BF16>(P, b, sm);
  else if (MODE == MODE_TREE) k2_tree<BF16>(P, b, sm);
  else k2_rows(P, b, sm);
}

template <bool BF16>
__global__ __launch_bounds__(kWG) void k3_kernel(Params P) {
  __shared__ Smem sm;
  const int b = (int)(blockIdx.x / (uint32_t)P.C3);
  const int c3 = (int)(blockIdx.x % (uint32_t)P.C3);
  k3_chunk<BF16>(P, b, c3, sm);
}

__global__ void fill_zero_kernel(uint8_t* p, size_t n) {
  const size_t n16 = n / 16;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    ((u32x4*)p)[i] = u32x4{0u, 0u, 0u, 0u};
  for (size_t i = n16 * 16 + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0;
}

// ===================================================================== host
struct Shape {
  int CH, CPR, C3;
  size_t gat_off, jobs_off, part_off, k3_off, total;
};

static Shape shape_of(int64_t bs, int64_t R, int64_t V, int dtype, bool races) {
  Shape s;
  s.CH = (dtype == SV_BF16 ? 8 : 4) * kVecPerThread * kWG * kSubChunks;
  s.CPR = (int)((V + s.CH - 1) / s.CH);
  s.C3 = races ? (int)((V + kK3Chunk - 1) / kK3Chunk) : 0;
  s.gat_off = kDataOffset;
  s.jobs_off = s.gat_off + align256(sizeof(Gather) * SV_MAX_NODES * (size_t)bs);
  s.part_off = s.jobs_off + align256(sizeof(Job) * (size_t)bs);
  s.k3_off = s.part_off + align256(sizeof(Partial) * (size_t)(bs * R * s.CPR));
  s.total = s.k3_off + align256(sizeof(K3Rec) * (size_t)(bs * s.C3));
  return s;
}

// Read-only cache of device properties: compute-unit count and the resident
// workgroups per CU of each fused kernel (slot = mode * 2 + bf16).
struct DeviceInfo {
  std::atomic<int> cu{0};
  std::atomic<int> occ[12];  // fused kernels (slots 0..5), K1 kernels (slots 6..11)
};
static DeviceInfo g_dev[64];

typedef void (*KernelFn)(Params);

template <int MODE, bool BF16>
static void kernels_for(KernelFn& fused, KernelFn& k1, KernelFn& k2, KernelFn& k3) {
  fused = fused_kernel<MODE, BF16>;
  k1 = k1_kernel<MODE, BF16>;
  k2 = k2_kernel<MODE, BF16>;
  k3 = k3_kernel<BF16>;
}

static void select_kernels(int mode, bool bf16, KernelFn& fused, KernelFn& k1, KernelFn& k2, KernelFn& k3) {
  if (mode == MODE_CHAIN) {
    if (bf16) kernels_for<MODE_CHAIN, true>(fused, k1, k2, k3);
    else kernels_for<MODE_CHAIN, false>(fused, k1, k2, k3);
  } else if (mode == MODE_TREE) {
    if (bf16) kernels_for<MODE_TREE, true>(fused, k1, k2, k3);
    else kernels_for<MODE_TREE, false>(fused, k1, k2, k3);
  } else {
    if (bf16) kernels_for<MODE_ROWS, true>(fused, k1, k2, k3);
    else kernels_for<MODE_ROWS, false>(fused, k1, k2, k3);
  }
}

static sv_status device_info(KernelFn kernel, int slot, int& cu, int& occ) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return SV_ERR_LAUNCH;
  cu = g_dev[dev].cu.load();
  occ = g_dev[dev].occ[slot].load();
  if (cu > 0 && occ > 0) return SV_OK;
  int c = 0, o = 0;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return SV_ERR_LAUNCH;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, (const void*)kernel, kWG, 0) != hipSuccess)
    return SV_ERR_LAUNCH;
  if (c <= 0 || o <= 0) return SV_ERR_LAUNCH;
  g_dev[dev].cu.store(c);
  g_dev[dev].occ[slot].store(o);
  cu = c;
  occ = o;
  return SV_OK;
}

static int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  if (!s || !*s) return dflt;
  return atoi(s);
}

static sv_status launch(Params& P, const Shape& S, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (ws == nullptr) return SV_ERR_INVALID_ARGUMENT;
  if (ws_bytes < S.total) return SV_ERR_WORKSPACE_TOO_SMALL;
  if (((uintptr_t)ws & 255u) != 0) return SV_ERR_INVALID_ARGUMENT;
  uint8_t* base = (uint8_t*)ws;
  P.ctrl = (Ctrl*)base;
  P.sync = (Sync*)(base + kSyncOffset);
  P.gat = (Gather*)(base + S.gat_off);
  P.jobs = (Job*)(base + S.jobs_off);
  P.part = (Partial*)(base + S.part_off);
  P.k3 = (K3Rec*)(base + S.k3_off);
  P.CH = S.CH;
  P.CPR = S.CPR;
  P.C3 = S.C3;
  P.n1r = P.R * S.CPR;
  const int64_t n_tickets = (int64_t)P.bs * (P.n1r + P.C3);
  if (n_tickets <= 0 || n_tickets > (int64_t)INT32_MAX) return SV_ERR_UNSUPPORTED;
  P.n_tickets = (int32_t)n_tickets;
  // Schedule: split unless another one is asked for (it measures fastest on
  // the shapes benchmarked so far).
  P.sched = (P.flags & SV_FLAG_FUSED) ? SCHED_FUSED : (P.flags & SV_FLAG_PHASED) ? SCHED_PHASED : SCHED_SPLIT;
  KernelFn fused, k1, k2, k3;
  const bool bf16 = P.dtype == SV_BF16;
  select_kernels(P.mode, bf16, fused, k1, k2, k3);
  if (P.sched != SCHED_FUSED) {
    P.lag = 0;
    hipLaunchKernelGGL(k1, dim3((unsigned)((int64_t)P.bs * P.n1r)), dim3(kWG), 0, stream, P);
    if (P.sched == SCHED_PHASED) hipLaunchKernelGGL(k2, dim3((unsigned)P.bs), dim3(kWG), 0, stream, P);
    if (P.C3 > 0) hipLaunchKernelGGL(k3, dim3((unsigned)(P.bs * P.C3)), dim3(kWG), 0, stream, P);
  } else {
    int cu = 0, occ = 0;
    sv_status st = device_info(fused, P.mode * 2 + (bf16 ? 1 : 0), cu, occ);
    if (st != SV_OK) return st;
    const int64_t resident = (int64_t)cu * occ;
    // Lag between a request's K1 chunks and its K3 chunks, in requests:
    // about the number of requests the resident workgroups stream at once,
    // so that a K3 item rarely has to wait for its request's decision.
    // (SV_LAG overrides it, for tuning.)
    int lag = env_int("SV_LAG", -1);
    if (lag < 0) lag = (int)((resident + P.n1r - 1) / P.n1r) + 1;
    if (P.C3 == 0) lag = 0;
    P.lag = lag > P.bs ? P.bs : lag;
    const int64_t grid = n_tickets;
    hipLaunchKernelGGL(fused, dim3((unsigned)grid), dim3(kWG), 0, stream, P);
  }
  if (hipGetLastError() != hipSuccess) return SV_ERR_LAUNCH;
  return SV_OK;
}

static bool aligned16(const void* p, int64_t stride_bytes) {
  return ((uintptr_t)p & 15u) == 0 && (stride_bytes & 15) == 0;
}

}  // namespace sv

using namespace sv;

extern "C" {

int32_t sv_abi_version(void) { return SV_ABI_VERSION; }

const char* sv_status_string(sv_status s) {
  switch (s) {
    case SV_OK: return "ok";
    case SV_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SV_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case SV_ERR_UNSUPPORTED: return "unsupported";
    case SV_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

static bool dtype_ok(sv_dtype d) { return d == SV_F32 || d == SV_BF16; }

static const uint32_t kKnownFlags = SV_FLAG_PHASED | SV_FLAG_FP64_RACE | SV_FLAG_FUSED | SV_FLAG_SPLIT;
// At most one schedule bit.
static bool one_schedule(uint32_t flags) {
  const uint32_t s = flags & (SV_FLAG_PHASED | SV_FLAG_FUSED | SV_FLAG_SPLIT);
  return (s & (s - 1)) == 0;
}

size_t sv_chain_workspace_bytes(int32_t batch, int32_t max_draft, int32_t vocab, sv_dtype dt) {
  if (batch < 1 || batch > SV_MAX_BATCH || max_draft < 0 || max_draft > SV_MAX_DRAFT || vocab < 1 ||
      vocab > SV_MAX_VOCAB || !dtype_ok(dt))
    return 0;
  return shape_of(batch, max_draft + 1, vocab, dt, true).total;
}

size_t sv_tree_workspace_bytes(int32_t batch, int32_t num_nodes, int32_t vocab, sv_dtype dt) {
  if (batch < 1 || batch > SV_MAX_BATCH || num_nodes < 1 || num_nodes > SV_MAX_NODES || vocab < 1 ||
      vocab > SV_MAX_VOCAB || !dtype_ok(dt))
    return 0;
  return shape_of(batch, num_nodes, vocab, dt, true).total;
}

size_t sv_row_stats_workspace_bytes(int32_t rows, int32_t vocab, sv_dtype dt) {
  if (rows < 1 || rows > SV_MAX_BATCH || vocab < 1 || vocab > SV_MAX_VOCAB || !dtype_ok(dt)) return 0;
  return shape_of(rows, 1, vocab, dt, false).total;
}

sv_status sv_workspace_init(void* ws, size_t bytes, void* stream) {
  if (ws == nullptr || bytes == 0 || ((uintptr_t)ws & 15u) != 0) return SV_ERR_INVALID_ARGUMENT;
  size_t blocks = (bytes / 16 + kWG - 1) / kWG;
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(kWG), 0, (hipStream_t)stream, (uint8_t*)ws,
                     bytes);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

sv_status sv_verify_chain(const sv_chain_desc* d, void* ws, size_t ws_bytes, void* stream) {
  if (d == nullptr) return SV_ERR_INVALID_ARGUMENT;
  if (d->batch < 1 || d->batch > SV_MAX_BATCH || d->max_draft < 0 || d->max_draft > SV_MAX_DRAFT ||
      d->vocab < 1 || d->vocab > SV_MAX_VOCAB)
    return SV_ERR_INVALID_ARGUMENT;
  if (!dtype_ok(d->logits_dtype)) return SV_ERR_UNSUPPORTED;
  if (d->draft_kind != SV_DRAFT_PROBS && d->draft_kind != SV_DRAFT_ONEHOT) return SV_ERR_UNSUPPORTED;
  if (d->flags & ~kKnownFlags) return SV_ERR_UNSUPPORTED;
  if (!one_schedule(d->flags)) return SV_ERR_INVALID_ARGUMENT;
  if (d->logits == nullptr || d->temperature == nullptr || d->seed == nullptr || d->accept_len == nullptr ||
      d->tokens == nullptr)
    return SV_ERR_INVALID_ARGUMENT;
  if (d->max_draft > 0 && d->draft_ids == nullptr) return SV_ERR_INVALID_ARGUMENT;
  if (d->logits_row_stride < d->vocab) return SV_ERR_INVALID_ARGUMENT;
  const bool probs = d->draft_kind == SV_DRAFT_PROBS;
  if (probs && d->max_draft > 0 && (d->draft_probs == nullptr || d->q_row_stride < d->vocab))
    return SV_ERR_INVALID_ARGUMENT;
  const size_t esz = d->logits_dtype == SV_BF16 ? 2 : 4;
  Params P;
  memset(&P, 0, sizeof P);
  P.mode = MODE_CHAIN;
  P.bs = d->batch;
  P.R = d->max_draft + 1;
  P.V = d->vocab;
  P.k = d->max_draft;
  P.dtype = d->logits_dtype;
  P.draft_kind = d->draft_kind;
  P.aligned = aligned16(d->logits, d->logits_row_stride * (int64_t)esz);
  P.lstride = d->logits_row_stride;
  P.qstride = probs ? d->q_row_stride : 0;
  P.q_aligned = probs ? aligned16(d->draft_probs, d->q_row_stride * 4) : 0;
  P.logits = d->logits;
  P.q = probs ? d->draft_probs : nullptr;
  P.ids = d->draft_ids;
  P.temp = d->temperature;
  P.seed = d->seed;
  P.accept_len = d->accept_len;
  P.tokens = d->tokens;
  P.status = d->req_status;
  P.p_draft = d->p_draft;
  P.flags = d->flags;
  const Shape S = shape_of(P.bs, P.R, P.V, P.dtype, true);
  return launch(P, S, ws, ws_bytes, (hipStream_t)stream);
}

sv_status sv_verify_tree(const sv_tree_desc* d, void* ws, size_t ws_bytes, void* stream) {
  if (d == nullptr) return SV_ERR_INVALID_ARGUMENT;
  if (d->batch < 1 || d->batch > SV_MAX_BATCH || d->num_nodes < 1 || d->num_nodes > SV_MAX_NODES ||
      d->vocab < 1 || d->vocab > SV_MAX_VOCAB)
    return SV_ERR_INVALID_ARGUMENT;
  if (!dtype_ok(d->logits_dtype)) return SV_ERR_UNSUPPORTED;
  if (d->flags & ~kKnownFlags) return SV_ERR_UNSUPPORTED;
  if (!one_schedule(d->flags)) return SV_ERR_INVALID_ARGUMENT;
  if (d->logits == nullptr || d->node_tokens == nullptr || d->parent == nullptr || d->temperature == nullptr ||
      d->seed == nullptr || d->accept_len == nullptr || d->accept_path == nullptr || d->tokens == nullptr)
    return SV_ERR_INVALID_ARGUMENT;
  if (d->logits_row_stride < d->vocab) return SV_ERR_INVALID_ARGUMENT;
  const size_t esz = d->logits_dtype == SV_BF16 ? 2 : 4;
  Params P;
  memset(&P, 0, sizeof P);
  P.mode = MODE_TREE;
  P.bs = d->batch;
  P.R = d->num_nodes;
  P.V = d->vocab;
  P.k = d->num_nodes - 1;
  P.dtype = d->logits_dtype;
  P.aligned = aligned16(d->logits, d->logits_row_stride * (int64_t)esz);
  P.lstride = d->logits_row_stride;
  P.logits = d->logits;
  P.temp = d->temperature;
  P.seed = d->seed;
  P.node_tokens = d->node_tokens;
  P.parent = d->parent;
  P.accept_len = d->accept_len;
  P.accept_path = d->accept_path;
  P.tokens = d->tokens;
  P.status = d->req_status;
  P.flags = d->flags;
  const Shape S = shape_of(P.bs, P.R, P.V, P.dtype, true);
  return launch(P, S, ws, ws_bytes, (hipStream_t)stream);
}

sv_status sv_row_stats(int32_t rows, int32_t vocab, sv_dtype dt, const void* logits, int64_t stride,
                       const float* temperature, float* row_max, int32_t* row_argmax, double* row_sumexp,
                       int32_t* row_status, void* ws, size_t ws_bytes, void* stream) {
  if (rows < 1 || rows > SV_MAX_BATCH || vocab < 1 || vocab > SV_MAX_VOCAB) return SV_ERR_INVALID_ARGUMENT;
  if (!dtype_ok(dt)) return SV_ERR_UNSUPPORTED;
  if (logits == nullptr || temperature == nullptr || stride < vocab) return SV_ERR_INVALID_ARGUMENT;
  const size_t esz = dt == SV_BF16 ? 2 : 4;
  Params P;
  memset(&P, 0, sizeof P);
  P.mode = MODE_ROWS;
  P.bs = rows;
  P.R = 1;
  P.V = vocab;
  P.k = 0;
  P.dtype = dt;
  P.aligned = aligned16(logits, stride * (int64_t)esz);
  P.lstride = stride;
  P.logits = logits;
  P.temp = temperature;
  P.rs_max = row_max;
  P.rs_amax = row_argmax;
  P.rs_sum = row_sumexp;
  P.rs_status = row_status;
  const Shape S = shape_of(rows, 1, vocab, dt, false);
  return launch(P, S, ws, ws_bytes, (hipStream_t)stream);
}

}  // extern "C"
