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
// Work decomposition.  One call is two kinds of work item:
//   K1  a streaming segment of one logit row: max, first argmax and
//       sum exp((l - m)/T) over a run of sub-chunks (16-byte nontemporal
//       loads, wave shuffles, a cross-wave LDS reduction).  Almost all HBM
//       bytes are read here, once.  Every row is cut into Q segments, Q
//       chosen from the shape alone so that all the segments' workgroups
//       are resident at once and the stream ends in one round; each
//       segment writes one partial of its row.
//   K23 a run of race chunks (2048 vocabulary ids each) of one request.
//       The workgroup first runs the request's decision step itself (K2):
//       combine the row partials in fp64, take p (and q) at the draft ids
//       that K1 gathered, draw the Philox coins, find the first rejection
//       (chain) or walk the tree.  Every item of the request computes the
//       same decision from the same few hundred bytes, so no workgroup
//       waits for another's result; item 0 writes the request's outputs.
//       Then (K3) the sampling race runs on two levels.  Each item bounds
//       the weight sum W_c of each of its chunks from one fp32 exp per id
//       (certified lower and upper bounds, no Philox) and stores the
//       chunk's key bounds W_c / E_c in a record.  The request's last item
//       waits for every record, keeps the chunks whose upper bound reaches
//       the largest lower bound (several are re-summed exactly in fp64),
//       and races the ids of the winning chunk alone: fp32 key bounds, the
//       near-maximal keys re-evaluated in fp64; it writes the emitted
//       token.
// Two optional passes sit between them in the phased schedule: KR, the
// block rule's residual masses of draft rows 1..k_b-1 (SV_FLAG_BLOCK), and
// KF, the top-k / top-p thresholds and kept sums of every filtered row (the
// descriptors' top_k / top_p): for top-k up to kCandTopK from the
// candidates that K1 publishes for such rows (every thread's two largest
// 16-entry groups), else from passes over the row.  Unfiltered one-hot
// chains and trees run K23C in place of K23: K1 also publishes every race
// chunk's sum, and one workgroup per request decides and races from those.
// The phased schedule is two stream-ordered launches (K1, then K23).  The
// fused schedule is one launch: the K23 items come after every K1 item in
// dispatch order and wait (bounded, about a second, then SV_REQ_INTERNAL)
// until their request's K1 segments are counted; workgroups are dispatched
// in index order, so the K1 items they wait for are running or done.
// Per-request counters are reset by their last user, so the workspace is
// ready for the next call without any reset pass.  Both schedules give
// bit-identical results.
#include <hip/hip_runtime.h>
#include <type_traits>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>

#include "specverify.h"

namespace sv {

constexpr int kWG = 256;
constexpr int kWaves = kWG / 64;
#ifndef SV_K1_VEC
#define SV_K1_VEC 2
#endif
#ifndef SV_K1_SLOTS
#define SV_K1_SLOTS (256 * 4)
#endif
#ifndef SV_K1_ROUNDS
#define SV_K1_ROUNDS 1
#endif
#ifndef SV_K1_OCC
#define SV_K1_OCC 7
#endif
constexpr int kVecPerThread = SV_K1_VEC;        // 16-byte loads per thread in a K1 sub-chunk
#ifndef SV_KR_WORKGROUPS
#define SV_KR_WORKGROUPS (256 * 7)
#endif
#ifndef SV_KR_UNROLL
#define SV_KR_UNROLL 4
#endif
constexpr int kKRWorkgroups = SV_KR_WORKGROUPS;  // block rule's residual-mass pass: workgroups it aims at
// K1 workgroups per call: at least four per CU of an MI355X where the rows
// allow, and no more than it holds at once (seven per CU at K1's 71 VGPRs),
// so the stream is one round.  Longer segments stream as fast as shorter
// ones on large batches, faster on small ones, and leave fewer partials for
// the decision step to fold.
constexpr int kK1Workgroups = SV_K1_SLOTS * SV_K1_ROUNDS;
constexpr int kK1Resident = 256 * SV_K1_OCC * SV_K1_ROUNDS;
// Ids per chunk of the sampling race: part of the sampler's definition (the
// race picks a chunk, then an id inside it), fixed independently of any
// workgroup shape; the kernels' tiles are sized to it.
constexpr int kK3Chunk = 2048;
constexpr int kK3Groups = 2;                    // groups of 4 vocabulary ids per thread in a race chunk
static_assert(kK3Chunk % (4 * kWG) == 0 && kK3Chunk == 4 * kWG * kK3Groups,
              "a race chunk is a whole number of 4-id groups per thread");
// K23 items per call the chunk grouping aims at: 256 CUs x 8 resident
// workgroups.  Up to two rounds of one-chunk items are kept (each item
// decides for itself, which is cheaper than a longer item); past that,
// items take several chunks, so that large batches decide once per item.
constexpr int kK3Slots = 2048;
constexpr int kCandMax = 64;                    // candidates a race level re-keys in fp64 (more: fp64 race)
constexpr int kCandTopK = 128;                  // largest top-k whose thresholds come from candidates
constexpr int kChunkE = 64;                     // chunk noise values an item computes up front
constexpr uint32_t kSpinLimit = 1u << 20;       // bounded waits (about a second)

enum { MODE_CHAIN = 0, MODE_TREE = 1, MODE_ROWS = 2 };
enum { JOB_NONE = 0, JOB_P = 1, JOB_RESID = 2, JOB_EXCL = 3 };
enum { SCHED_FUSED = 0, SCHED_PHASED = 1 };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- workspace
struct Ctrl {
  uint32_t aborted;   // a bounded wait expired (left set: the workspace must be re-initialised)
  uint32_t pad[63];
};
// One per request, each on its own 256 bytes: the fused schedule's waiting
// workgroups poll these counters while K1 workgroups add to them, and
// counters sharing cache lines serialise those accesses.
struct Sync {
  uint32_t k1_count;  // K1 segments of the request (row, in row-statistics calls) done in this call,
                      // reset to 0 by its last user
  uint32_t pad[63];
};
// Target logit (and draft probability) at a draft token, gathered by the K1
// segment that holds it: chain slot r = row r's draft, tree slot n = node n's
// token in its parent's row.
struct Gather {
  uint32_t l;         // fp32 bits of the logit
  uint32_t q;         // fp32 bits of q at the draft (chain, draft probabilities)
};
struct Partial {
  uint64_t s;         // bits of the segment sum of 2^((l - m_c) log2(e)/T) (fp64), or a NaN flag for greedy rows
  uint64_t m_amax;    // bits of the segment max (fp32, low half) and the smallest index attaining it (high half)
};
// A sampling chunk's result: certified bounds on its race key W_c / E_c.
struct K3Rec {
  double klo;         // lower bound (0: no weight of the chunk is certainly positive)
  double khi;         // upper bound
  int32_t count;      // 0 until the record is complete, then 1; reset by the request's first
                      // K1 segment of each call
  int32_t pad[3];
};

// One share of a race chunk's sum in a row-statistics segment (the
// chunk-sum path): the fp32 sum of the terms 2^(l c - off) of one row of 16
// lanes, c = fp32(log2(e)/T), with off the row's running offset (fl(m c) of
// its running max) when the chunk was folded.
struct CSum {
  float s;
  float off;
};
constexpr int kCSumShares = kWG / 16;  // shares per race chunk: one per row of 16 lanes
// Race chunks of one statistics segment whose shares are gathered in shared
// memory and stored in one burst after the segment (stores issued between
// the stream's loads would hold up its waits); longer segments store each
// share as it is made.
constexpr int kCSumLds = 80;

// A filtered row's threshold and kept sum (written by the thresholds pass).
struct FiltRec {
  double s;           // S' = sum over kept ids of exp((l - m)/T)
  float tau;          // ids with a logit below tau are cut (p = 0)
  int32_t pad;
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
  Partial* part;      // [bs*R][CPR]
  K3Rec* k3;          // [bs][C3]
  int32_t SUB;        // entries per K1 sub-chunk
  int32_t nsub;       // sub-chunks per row
  int32_t Q;          // segments (K1 items, partials) per row, <= 64
  int32_t Qp;         // the power of two >= Q
  int32_t G;          // K1 items: rows * Q
  int32_t CPR;        // partial slots per row (= Q)
  int32_t C3;         // sampling chunks per request
  int32_t G3;         // sampling chunks per K23 item
  int32_t CI;         // K23 items per request: ceil(C3 / G3)
  int32_t CHr;        // block rule: residual-mass items per row (rows 1..k-1)
  double* rpart;      // block rule: [bs][k][CHr] residual-mass partials
  const int32_t* top_k;  // per-request top-k (NULL: off)
  const float* top_p;    // per-request top-p (NULL: off)
  FiltRec* filt;         // [bs*R] thresholds and kept sums of filtered rows
  CSum* csum;            // [bs*R][C3][kCSumShares] race-chunk sums of the rows' segments (csum calls)
  int32_t csum_fold;     // stochastic rows fold with offsets shared by rows of 16 lanes (one-hot chains, trees)
  int32_t csum_on;       // ... and publish their race-chunk sums (phased schedule, unfiltered)
  u32x4* cand;           // [bs*R][Q][kWG] top-k candidates: per thread and segment, the keys and sub-chunks
                         // of its two largest groups (key 0: none)
  int32_t lag;        // fused schedule: requests between a request's K1 items and its sampling chunks
  int32_t sched;
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
// Reductions over each row of 16 lanes with DPP butterflies (quad swaps,
// then the half-row and row mirrors): every lane of the row gets the result,
// in a fixed order of operations.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
// The max is v_max_f32 with the DPP operand (one instruction per step; the
// s_nop gives the two wait states a DPP read of a just-written VGPR needs).
// Its inputs are the entries' running maxima (never signalling NaNs), so no
// canonicalisation is needed.
__device__ __forceinline__ float row16_max(float v) {
  asm volatile(
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 row_mirror row_mask:0xf bank_mask:0xf bound_ctrl:1"
      : "+v"(v));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
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
// Loads of data that an earlier launch wrote (COH = false: plain, cached
// loads; a kernel boundary makes the writes visible) or that other
// workgroups of the same launch wrote (COH = true).
template <bool COH>
__device__ __forceinline__ uint64_t ld64(const void* p) {
  return COH ? cld64(p) : *(const uint64_t*)p;
}
template <bool COH>
__device__ __forceinline__ uint32_t ld32(const void* p) {
  return COH ? cld32(p) : *(const uint32_t*)p;
}
__device__ __forceinline__ void cst_i32(int32_t* p, int32_t v) { cst32(p, (uint32_t)v); }
// Wait until this wave's memory operations have completed.
__device__ __forceinline__ void wait_mem() { __builtin_amdgcn_s_waitcnt(0); }
__device__ __forceinline__ uint32_t atomic_add_relaxed(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A value that is the same in every lane, made visibly uniform (an SGPR) so
// that branches on it are scalar branches rather than divergent regions.
__device__ __forceinline__ int uniform_i(int v) { return __builtin_amdgcn_readfirstlane(v); }
// 32-bit keys that order like the logits they stand for (-0 as +0, so equal
// logits share one key; NaNs above +inf), and back.
__device__ __forceinline__ uint32_t kf_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float kf_val(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
// Lanes of mask m below this lane.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}
__device__ __forceinline__ uint32_t uniform_u(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }

// A request's sampling job: the result of its decision step (in LDS).
struct Job {
  int kind, row, qrow, r, out_slot, n_excl;
  float m, c_hi, c_lo, inv_s;  // row max; log2(e)/T as hi + lo; 1/S rounded
  double s, t;                  // S = sum exp((l - m)/T); T
  double wmul;                  // JOB_RESID weight max(wmul p - q, 0): 1, or the block rule's prefix weight
  float tau;                    // ids with a logit below tau have p = 0 (top-k / top-p; -inf: none)
  int excl[SV_MAX_NODES];       // ids removed from p (JOB_EXCL)
};

// Shared memory of one workgroup (every role reuses it).
struct Smem {
  float red_f[kWaves];
  int red_i[kWaves];
  double red_d[kWaves];
  double red_d2[kWaves];
  uint64_t red_u[kWaves];
  int flag;
  float l0;
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
  int a, kb, status, len, emit;
  Job job;
  // noise E_c of the item's first kChunkE chunks, from chunk chunk_e0 on
  int chunk_e0;
  double chunk_e[kChunkE];
  // race candidates (chunks, then ids) re-keyed in fp64
  int ncand;
  int cand_y[kCandMax];
  double cand_key[kCandMax];
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
__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, Smem& sm) {
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t w = __shfl_xor(v, o, 64);
    v = w > v ? w : v;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sm.red_u[wave] = v;
  __syncthreads();
  uint64_t r = sm.red_u[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = sm.red_u[w] > r ? sm.red_u[w] : r;
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

// Two block sums at once (every thread gets both).
__device__ __forceinline__ void block_sum2_d(double& a, double& b, Smem& sm) {
  a = wave_sum_d(a);
  b = wave_sum_d(b);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) {
    sm.red_d[wave] = a;
    sm.red_d2[wave] = b;
  }
  __syncthreads();
  a = sm.red_d[0];
  b = sm.red_d2[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    a += sm.red_d[w];
    b += sm.red_d2[w];
  }
}

// Temperature of the request (chain/tree) or of the row (row statistics).
__device__ __forceinline__ float temp_of(const Params& P, int b) { return P.temp[b]; }
__device__ __forceinline__ bool is_stochastic(float T) { return T > 0.f && isfinite(T); }

// Whether request b's target is top-k / top-p filtered: stochastic, and k
// in (0, V) or p in (0, 1).
__device__ __forceinline__ bool request_filtered(const Params& P, int b, float T) {
  if (!is_stochastic(T)) return false;
  const int tk = P.top_k ? P.top_k[b] : 0;
  const float tp = P.top_p ? P.top_p[b] : 1.f;
  return (tk > 0 && tk < P.V) || (tp > 0.f && tp < 1.f);
}

// Number of chain drafts in use: the index of the first -1, else k.  Every
// wave computes the same value (k <= 63 fits one wave).
__device__ __forceinline__ int chain_kb(const Params& P, int b, int& xi) {
  const int lane = threadIdx.x & 63;
  xi = (lane < P.k) ? P.ids[(int64_t)b * P.k + lane] : -1;
  const uint64_t m = __ballot(lane < P.k && xi == -1);
  return m ? (int)__builtin_ctzll(m) : P.k;
}

// ===================================================================== K1
// Streaming statistics of one segment: consecutive sub-chunks of one row,
// each 256 threads x kVecPerThread nontemporal 16-byte loads (consecutive
// lanes on consecutive 16-byte pieces).  The loads of sub-chunk s+1 are in
// flight while sub-chunk s is reduced (a register double buffer).
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
// flag.  One block reduction per segment gives its (max, first argmax,
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
  float offc;    // the offset the terms are computed with: off, or 0 while m = -inf
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

// ---------------------------------------------------------- top-k candidates
// Statistics segments of a top-k filtered row (page "投机解码", section
// "接受规则为什么不改变分布": the target p is the one after top-k / top-p)
// also publish what the thresholds pass needs to find the kept set without
// reading the row again.  A group is one thread's entries of one sub-chunk
// (its kVecPerThread loads), named by gid = sub-chunk * kWG + thread within
// the row; its key is the key of its largest logit.  Every thread keeps, in
// registers, the keys and sub-chunks of its two largest groups of the
// segment, and publishes them (a "lane" record per thread and segment).
// The thresholds pass then takes g', the k-th largest published key: the
// published keys are keys of distinct groups, so g' is at most the row's
// k-th largest group key, which is at most tau, the row's k-th largest logit
// (k groups with keys above tau would hold k logits above tau).  Every logit
// >= g' lies in a group whose key is >= g'.  Such a group is either one of
// its lane's two published groups, or its lane's second key is >= g' too;
// so the published groups >= g' together with every group of the lanes
// whose second key is >= g' (rare lanes) hold all of the row's logits
// >= g', a set that holds every logit >= tau.
// Whether a stochastic row with top-k tk takes its thresholds from candidates.
__device__ __forceinline__ bool kc_row(const Params& P, int tk) {
  return tk > 0 && tk < P.V && tk <= kCandTopK && !(P.flags & SV_FLAG_KF_ROWS);
}

// Folds the NV entries x of one sub-chunk into the running statistics.
// Entry i sits at item offset base + (i / EPV) * kWG * EPV + i % EPV, so the
// thread's order is the row order and the first hit is the smallest index.
// With CHUNKS (stochastic rows whose race chunks' sums are published) the
// running offset is shared by each row of 16 lanes (their running max), so
// that the lanes' terms add up per race chunk; cs[j] gets the thread's sum
// over load j (bf16: one race chunk per load; fp32: the two loads form one
// chunk, in cs[0]).  Returns the thread's max of the entries.
template <int NV, int EPV, bool STOCH, bool NEED_AMAX, bool CHUNKS = false>
__device__ __forceinline__ float k1_fold_sub(const float* x, int base, float c, K1Run& st, float* cs = nullptr) {
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
    // Only when some lane of the wave sees a new maximum do the offsets move
    // (a wave-uniform branch); otherwise the rescale factor would be exactly
    // 1 and is skipped, with the same result.
    const bool grow = __ballot(mx > st.m) != 0;
    float f = 1.f;
    if (grow) {
      const float mn = CHUNKS ? row16_max(fmaxf(st.m, mx)) : fmaxf(st.m, mx);
      const float off = (mn == -INFINITY) ? 0.f : mn * c;  // keeps l = -inf terms at 2^-inf = 0
      // rescale factor: 0 until the first finite max (st.off = -inf; never
      // inf * 0), exactly 1 while the max is unchanged, else at most 1
      f = __builtin_amdgcn_exp2f(st.off - off);
      st.m = mn;
      st.off = (mn == -INFINITY) ? -INFINITY : off;
      st.offc = off;
    }
    const float off = st.offc;
    float e[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) e[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], c, -off));
#pragma unroll
    for (int w = 1; w < NV; w *= 2) {
      if (CHUNKS && w == NV / 2) {
        // the two halves are the two loads
        if (EPV == 8) {
          cs[0] = e[0];
          cs[1] = e[NV / 2];
        } else {
          cs[0] = e[0] + e[NV / 2];
        }
      }
#pragma unroll
      for (int i = 0; i + w < NV; i += 2 * w) e[i] += e[i + w];
    }
    st.s = grow ? st.s * (double)f + (double)e[0] : st.s + (double)e[0];
  }
  return mx;
}

// Streams sub-chunks [s0, s1) of row `row` (the first already in flight in
// raw0) and writes the segment's partial to slot `slot` of the row.  With
// CHUNKS, each row of 16 lanes also stores, per race chunk of the segment,
// the sum of its lanes' terms and its offset (read by csum_race).  With
// CAND and top-k tk > 0, every thread publishes its two largest groups (the
// top-k candidates; CHUNKS then only sets the fold, nothing of the race
// chunks is published).
template <bool BF16, bool STOCH, bool NEED_AMAX, bool CHUNKS = false, bool CAND = false>
__device__ __forceinline__ void k1_seg_stats(const Params& P, int64_t row, int s0, int s1, int slot, float T,
                                             u32x4* raw0, Smem& sm, CSum* cs_lds = nullptr, int tk = 0) {
  constexpr int EPV = BF16 ? 8 : 4;
  constexpr int NV = kVecPerThread * EPV;  // entries per thread per sub-chunk
  constexpr int SUB = NV * kWG;            // entries per sub-chunk
  constexpr int NCH = BF16 ? 2 : 1;        // race chunks per sub-chunk
  static_assert(SUB == NCH * kK3Chunk, "a sub-chunk is a whole number of race chunks");
  const int64_t start = (int64_t)s0 * SUB;
  const int n_seg = (int)(min((int64_t)s1 * SUB, (int64_t)P.V) - start);
  const int nsub = s1 - s0;
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
  st.offc = 0.f;
  st.idx = INT32_MAX;
  st.s = 0.0;
  st.nan = false;
  // the thread's two largest group maxima (top-k candidates; NaN: none yet,
  // so that groups of -inf count too) and their sub-chunks in the segment
  float c1 = __builtin_nanf(""), c2 = __builtin_nanf("");
  int u1 = -1, u2 = -1;
  // two register buffers: the next sub-chunk is in flight while one is folded
  u32x4 cur[kVecPerThread], nxt[kVecPerThread];
#pragma unroll
  for (int j = 0; j < kVecPerThread; ++j) cur[j] = raw0[j];
#pragma unroll 1
  for (int sub = 0; sub < nsub; ++sub) {
    if (sub + 1 < nsub) k1_issue<BF16>(P, elem0 + (int64_t)(sub + 1) * SUB, n_seg - (sub + 1) * SUB, nxt);
    float x[NV];
    k1_unpack<BF16>(cur, x);
    float mx;
    if constexpr (CHUNKS) {
      float cs[NCH];
      mx = k1_fold_sub<NV, EPV, STOCH, NEED_AMAX, true>(x, sub * SUB + threadIdx.x * EPV, cf, st, cs);
      if constexpr (!CAND) {
        const int c0 = sub * NCH;  // the segment's chunk index of load 0
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
          const float rs = row16_sum(cs[j]);
          if ((threadIdx.x & 15) == 15 && P.csum_on) {
            if (nsub * NCH <= kCSumLds) cs_lds[(c0 + j) * kCSumShares + (threadIdx.x >> 4)] = CSum{rs, st.off};
            else if (start / kK3Chunk + c0 + j < P.C3)
              P.csum[(row * P.C3 + start / kK3Chunk + c0 + j) * kCSumShares + (threadIdx.x >> 4)] =
                  CSum{rs, st.off};
          }
        }
      }
    } else {
      mx = k1_fold_sub<NV, EPV, STOCH, NEED_AMAX>(x, sub * SUB + threadIdx.x * EPV, cf, st);
    }
    if constexpr (CAND) {
      const bool a1 = !(mx <= c1), a2 = !(mx <= c2);  // strict, and true while empty
      c2 = a1 ? c1 : (a2 ? mx : c2);
      u2 = a1 ? u1 : (a2 ? sub : u2);
      c1 = a1 ? mx : c1;
      u1 = a1 ? sub : u1;
    }
#pragma unroll
    for (int j = 0; j < kVecPerThread; ++j) cur[j] = nxt[j];
  }
  if constexpr (CAND) {
    if (tk > 0)
      P.cand[(row * P.Q + slot) * kWG + threadIdx.x] =
          u32x4{u1 >= 0 ? kf_key(c1) : 0u, (uint32_t)(s0 + u1), u2 >= 0 ? kf_key(c2) : 0u, (uint32_t)(s0 + u2)};
  }
  const float mc = block_max(st.m, sm);  // its barriers also order the shared-memory shares
  if constexpr (CHUNKS && !CAND) {
    if (P.csum_on && nsub * NCH <= kCSumLds) {
      // the segment's shares, one burst of whole chunks of kCSumShares
      const int c0 = (int)(start / kK3Chunk);
      const int n = min(nsub * NCH, P.C3 - c0) * kCSumShares;
      uint64_t* dst = (uint64_t*)&P.csum[(row * P.C3 + c0) * kCSumShares];
      const uint64_t* src = (const uint64_t*)cs_lds;
      for (int i = threadIdx.x; i < n; i += kWG) dst[i] = src[i];
    }
  }
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
    // this thread's sum relative to 2^(mc log2(e)/T): undo the offset's
    // rounding (m cf is exact in fp64), then move from m to mc at the exact scale
    double mine = 0.0;
    if (st.m != -INFINITY && mc != -INFINITY)
      mine = st.s * exp2((double)st.off - (double)st.m * (double)cf + ((double)st.m - (double)mc) * cd);
    else if (st.s != st.s)
      mine = st.s;
    out_s = block_sum_d(mine, sm);
  }
  if (threadIdx.x == 0) {
    Partial* dst = &P.part[row * P.CPR + slot];
    cst64(&dst->s, (uint64_t)__double_as_longlong(out_s));
    cst64(&dst->m_amax, (uint64_t)__float_as_uint(mc) | ((uint64_t)(uint32_t)out_amax << 32));
  }
}

// Every row is split into Q segments of (almost) equal length, one K1
// work item each: segment c of a row covers sub-chunks [c nsub / Q,
// (c + 1) nsub / Q) and writes the row's partial c.
__device__ __forceinline__ int k1_segments(const Params& P, int64_t row) { return P.Q; }

// ===================================================================== K2
// p(y) of a stochastic row in fp64: exp((l - m)/T) / S.
__device__ __forceinline__ double p_at(double l, float m, double T, double S) { return exp((l - (double)m) / T) / S; }

// 2^x for x <= 0 (rescale factors of partial sums), within about 2^-22
// relative: 2^frac(x) by v_exp_f32, scaled by 2^floor(x) exactly.
__device__ __forceinline__ double exp2_scale(double x) {
  if (!(x > -1074.0)) return x != x ? x : 0.0;
  const double n = floor(x);
  return ldexp((double)__builtin_amdgcn_exp2f((float)(x - n)), (int)n);
}

// Per-row results from the rows' segment partials, into shared memory
// (rm, ramax, rs, rbad): max, first argmax, a bad flag (NaN or +inf seen,
// the row entirely -inf, or S not positive) and, for stochastic rows,
// S = sum over segments of S_c 2^((m_c - m) log2(e)/T) in fp64.  One thread
// per partial: the Q partials of a row sit in a group of Qp adjacent lanes
// (Qp the power of two >= Q, so the groups never straddle a wave) and are
// reduced with butterflies in a fixed order; all loads of a pass are issued
// together.  Every thread of the workgroup calls it; it ends with a barrier.
template <bool COH>
__device__ __forceinline__ void fold_rows(const Params& P, int64_t row0, int nrows, float T, Smem& sm) {
  const int q = P.Q, qp = P.Qp;
  const bool stoch = is_stochastic(T);
  const double cd = stoch ? 1.4426950408889634074 / (double)T : 0.0;
  for (int e0 = 0; e0 < nrows * qp; e0 += kWG) {
    const int e = e0 + (int)threadIdx.x;
    const int r = e / qp, c = e - r * qp;
    uint64_t ma = 0xFF800000ull, sb = 0ull;  // max -inf, argmax 0, sum 0
    if (r < nrows && c < q) {
      const Partial* pt = &P.part[(row0 + r) * P.CPR + c];
      ma = ld64<COH>(&pt->m_amax);
      sb = ld64<COH>(&pt->s);
    }
    const float pm = __uint_as_float((uint32_t)ma);
    const int pa = (int)(uint32_t)(ma >> 32);
    const double ps = __longlong_as_double((long long)sb);
    int nan = (ps != ps);
    float m = pm;
    for (int o = 1; o < qp; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    int a = (pm == m) ? pa : INT32_MAX;
    double s = 0.0;
    if (stoch) {
      if (pm != -INFINITY && m != -INFINITY) s = ps * exp2_scale(((double)pm - (double)m) * cd);
      else if (ps != ps) s = ps;
    }
    for (int o = 1; o < qp; o <<= 1) {
      a = min(a, __shfl_xor(a, o, 64));
      s += __shfl_xor(s, o, 64);
      nan |= __shfl_xor(nan, o, 64);
    }
    if (r < nrows && c == 0) {
      sm.rm[r] = m;
      sm.ramax[r] = a;
      sm.rs[r] = stoch ? s : __builtin_nan("");
      sm.rbad[r] = nan || m == INFINITY || m == -INFINITY || (stoch && !(s > 0.0));
    }
  }
  __syncthreads();
}

struct RowStats {
  float m;
  int amax;
  double s;
  bool bad;
};
__device__ __forceinline__ RowStats row_stats_of(const Smem& sm, int r) {
  RowStats x;
  x.m = sm.rm[r];
  x.amax = sm.ramax[r];
  x.s = sm.rs[r];
  x.bad = sm.rbad[r] != 0;
  return x;
}

// Row-statistics call: the "request" is one row.
__device__ __forceinline__ void k2_rows(const Params& P, int b, Smem& sm) {
  fold_rows<true>(P, b, 1, temp_of(P, b), sm);
  if (threadIdx.x == 0) {
    if (P.rs_max) P.rs_max[b] = sm.rm[0];
    if (P.rs_amax) P.rs_amax[b] = sm.ramax[0];
    if (P.rs_sum) P.rs_sum[b] = sm.rs[0];
    if (P.rs_status) P.rs_status[b] = sm.rbad[0] ? SV_REQ_NONFINITE : SV_REQ_OK;
  }
}

// Prefix weights of the block rule (page "The speculative decoding zoo",
// vLLM's "block" method, after Sun et al. 2024): w_0 = 1 and
// w_{j+1} = min(w_j p_j / q_j, 1), with p_j, q_j the target and draft
// probabilities of draft j (lane j).  A zero draft probability gives ratio
// +inf (p > 0) or 0, and a zero weight stays zero.  Every lane of the wave
// calls it; lane j gets w_j (j <= n).
__device__ __forceinline__ double prefix_weights(double p, double q, int n) {
  const int lane = threadIdx.x & 63;
  double w = 1.0, mine = 1.0;
  for (int j = 0; j < n; ++j) {
    const double pj = __shfl(p, j, 64), qj = __shfl(q, j, 64);
    const double ratio = qj > 0.0 ? pj / qj : (pj > 0.0 ? INFINITY : 0.0);
    double nw = w * ratio;
    if (w == 0.0 || ratio == 0.0) nw = 0.0;
    w = nw < 1.0 ? nw : 1.0;
    if (lane == j + 1) mine = w;
  }
  return mine;
}

// Accepted length of chain request b under the block rule (wave 0, lane j
// on draft j): prefix length j + 1 passes when its coin u_j is at most
// h = r / (r + 1 - w) (1 when that denominator is 0; h = w for the whole
// chain), with w and r the prefix weight and residual mass of row j + 1 --
// for one-hot drafts r = w (1 - p(x)), otherwise the sum of the residual
// pass's partials.  The longest passing prefix is accepted.  wa gets the
// accepted length's prefix weight.
__device__ __forceinline__ int block_accept(const Params& P, int b, int kb, int lane, int status, double p,
                                            double u, uint64_t gl, double& wa) {
  const bool onehot = P.draft_kind == SV_DRAFT_ONEHOT;
  const double q = onehot ? 1.0 : (double)__uint_as_float((uint32_t)(gl >> 32));
  const double wl = prefix_weights(p, q, kb);
  const double wn = __shfl(wl, (lane + 1) & 63, 64);  // w of row lane + 1
  const double pn = __shfl(p, (lane + 1) & 63, 64);   // p of draft lane + 1
  double h = wn;
  if (lane + 1 < kb) {
    double r = 0.0;
    if (onehot) {
      r = wn * (1.0 - pn);
    } else {
      const double* rp = P.rpart + ((int64_t)b * P.k + lane + 1) * P.CHr;
      for (int c = 0; c < P.CHr; ++c) r += rp[c];
    }
    const double den = r + 1.0 - wn;
    h = den > 0.0 ? r / den : 1.0;
  }
  const uint64_t pass = __ballot(status == SV_REQ_OK && lane < kb && u <= h);
  const int a = (status != SV_REQ_OK || !pass) ? 0 : 64 - __builtin_clzll(pass);
  wa = __shfl(wl, a, 64);
  return a;
}

// Decision step of chain request b, by wave 0 with lane r on row r (and on
// draft r): every workgroup that samples for the request runs it (its
// inputs are a few hundred bytes, in L2 after the first), so none waits for
// another's result; `writer` also writes the request's outputs, except the
// token that the request's race emits.  Leaves the status and the sampling
// job (kind JOB_NONE: nothing to sample) in shared memory, behind a barrier.
template <bool BF16, bool COH>
__device__ void decide_chain(const Params& P, int b, bool writer, Smem& sm) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int k = P.k, R = P.R, V = P.V;
  const float Tf = temp_of(P, b);
  const double T = (double)Tf;
  const bool greedy = !(Tf > 0.f);
  // the loads first, none depending on another: the seed, the drafts and the
  // gathered target logit and q at each draft (wave 0), every row's partials
  // (rows after the chain's end hold stale values, ignored)
  const uint64_t seed = P.seed[b];
  int xi = -1, kb = 0;
  uint64_t gl = 0;
  if (tid < 64) {
    kb = chain_kb(P, b, xi);
    if (lane < k) gl = ld64<COH>(&P.gat[(int64_t)b * SV_MAX_NODES + lane]);
  }
  fold_rows<COH>(P, (int64_t)b * R, R, Tf, sm);
  if (tid < 64) {
    RowStats rs;
    rs.m = -INFINITY;
    rs.amax = 0;
    rs.s = 1.0;
    rs.bad = false;
    if (lane < R) rs = row_stats_of(sm, lane);
    float ftau = -INFINITY;  // top-k / top-p: the row's threshold (and its kept sum replaces S)
    if (request_filtered(P, b, Tf) && lane <= kb) {
      rs.s = P.filt[(int64_t)b * R + lane].s;
      ftau = P.filt[(int64_t)b * R + lane].tau;
    }
    const bool bad_id = __ballot(lane < kb && (xi < 0 || xi >= V)) != 0;
    int status = !isfinite(Tf) ? SV_REQ_BAD_TEMPERATURE : bad_id ? SV_REQ_BAD_DRAFT_ID : SV_REQ_OK;
    double u = 0.0;
    if (status == SV_REQ_OK && !greedy && lane < kb) u = coin(seed, b, lane);
    if (status == SV_REQ_OK && __ballot(lane <= kb && rs.bad)) status = SV_REQ_NONFINITE;
    bool accept = false;
    double p = 0.0;
    if (status == SV_REQ_OK && lane < kb) {
      if (greedy) {
        accept = (xi == rs.amax);
        p = accept ? 1.0 : 0.0;
      } else {
        const float lx = __uint_as_float((uint32_t)gl);
        p = lx < ftau ? 0.0 : p_at((double)lx, rs.m, T, rs.s);
        if (P.draft_kind == SV_DRAFT_ONEHOT) {
          accept = u < p;
        } else {
          const double q = (double)__uint_as_float((uint32_t)(gl >> 32));
          accept = (q <= 0.0) ? p > 0.0 : u * q < p;
        }
      }
    }
    int a;
    double wa = 1.0;  // block rule: prefix weight of the emitted row
    if ((P.flags & SV_FLAG_BLOCK) && !greedy) {
      a = block_accept(P, b, kb, lane, status, p, u, gl, wa);
    } else {
      const uint64_t rejected = __ballot(status == SV_REQ_OK && lane < kb && !accept);
      a = status != SV_REQ_OK ? 0 : rejected ? (int)__builtin_ctzll(rejected) : kb;
    }
    sm.xs[lane] = xi;
    sm.px[lane] = p;
    sm.ramax[lane] = rs.amax;
    // lane a holds the emitted row's statistics and the draft it rejected
    if (lane == a) {
      sm.a = a;
      sm.kb = kb;
      sm.status = status;
      Job& J = sm.job;
      J.kind = JOB_NONE;
      if (status == SV_REQ_OK && !greedy) {
        J.kind = (a < kb) ? (P.draft_kind == SV_DRAFT_PROBS ? JOB_RESID : JOB_EXCL) : JOB_P;
        J.row = b * R + a;
        J.qrow = b * k + a;
        J.r = a;
        J.out_slot = b * R + a;
        J.m = rs.m;
        J.s = rs.s;
        J.t = T;
        scale_pair(T, J.c_hi, J.c_lo);
        J.wmul = (J.kind == JOB_RESID) ? wa : 1.0;
        J.tau = ftau;
        J.inv_s = (float)(J.wmul / rs.s);
        J.n_excl = (J.kind == JOB_EXCL) ? 1 : 0;
        J.excl[0] = xi;
      }
    }
  }
  __syncthreads();
  if (!writer) return;
  const int a = sm.a;
  if (tid == 0) {
    P.accept_len[b] = a;
    // a request with a race gets its status from the race's merge, after
    // its token: a wait that gives up on the way writes REQ_INTERNAL, and no
    // earlier OK may land after it
    if (P.status && sm.job.kind == JOB_NONE) P.status[b] = sm.status;
  }
  for (int i = tid; i < R; i += kWG) {
    int t = -1;
    if (sm.status == SV_REQ_OK) {
      if (i < a) t = sm.xs[i];
      else if (i == a && greedy) t = sm.ramax[a];
      else if (i == a) continue;  // written by the race's merge
    }
    P.tokens[(int64_t)b * R + i] = t;
  }
  if (P.p_draft)
    for (int i = tid; i < k; i += kWG)
      P.p_draft[(int64_t)b * k + i] = (sm.status == SV_REQ_OK && i < sm.kb) ? sm.px[i] : __builtin_nan("");
}

// Decision step of tree request b (same contract as decide_chain): lane n
// on node n's row; p at node n uses its parent's row (by shuffle); thread 0
// walks the tree.
template <bool BF16, bool COH>
__device__ void decide_tree(const Params& P, int b, bool writer, Smem& sm) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int N = P.R, V = P.V;
  const float Tf = temp_of(P, b);
  const double T = (double)Tf;
  const bool greedy = !(Tf > 0.f);
  const uint64_t seed = P.seed[b];  // loaded with the others, used after the fold
  uint32_t gl = 0;  // node lane's token's logit in its parent's row (K1 gathered it)
  int par = -2, tok = -1;
  if (tid < 64) {
    if (lane >= 1 && lane < N) gl = ld32<COH>(&P.gat[(int64_t)b * SV_MAX_NODES + lane].l);
    if (lane < N) {
      par = P.parent[(int64_t)b * N + lane];
      tok = P.node_tokens[(int64_t)b * N + lane];
    }
  }
  fold_rows<COH>(P, (int64_t)b * N, N, Tf, sm);
  if (tid < 64) {
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
    RowStats rs;
    rs.m = -INFINITY;
    rs.amax = 0;
    rs.s = 1.0;
    rs.bad = false;
    if (lane < N) rs = row_stats_of(sm, lane);
    float ftau = -INFINITY;  // top-k / top-p: the row's threshold (and its kept sum replaces S)
    if (request_filtered(P, b, Tf) && lane < N) {
      rs.s = P.filt[(int64_t)b * N + lane].s;
      ftau = P.filt[(int64_t)b * N + lane].tau;
    }
    double u = 0.0;
    if (status == SV_REQ_OK && !greedy && lane < N) u = coin(seed, b, lane);
    if (status == SV_REQ_OK && __ballot(lane < N && rs.bad)) status = SV_REQ_NONFINITE;
    // p_parent(tok_n), from the parent lane's row statistics
    const int src = (lane >= 1 && lane < N && status == SV_REQ_OK) ? par : 0;
    const float pm = __shfl(rs.m, src, 64);
    const double ps = __shfl(rs.s, src, 64);
    const int pa = __shfl(rs.amax, src, 64);
    const float ptau = __shfl(ftau, src, 64);
    if (lane < N) {
      sm.par[lane] = par;
      sm.tok[lane] = tok;
      sm.ramax[lane] = rs.amax;
      sm.rm[lane] = rs.m;
      sm.rs[lane] = rs.s;
      sm.u[lane] = u;
      sm.qx[lane] = (double)ftau;  // the row's threshold, for the sampling job
      const float lx = __uint_as_float(gl);
      if (lane >= 1 && status == SV_REQ_OK)
        sm.px[lane] = greedy ? (tok == pa ? 1.0 : 0.0) : (lx < ptau ? 0.0 : p_at((double)lx, pm, T, ps));
    }
    if (lane == 0) sm.status = status;
  }
  __syncthreads();
  if (tid == 0) {
    const int status = sm.status;
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
          const double uc = sm.u[cur];
          double acc = 0.0;
          for (int c = cur + 1; c < N; ++c) {
            if (sm.par[c] != cur) continue;
            ++nchild;
            const double pc = sm.px[c];
            acc += pc;
            if (pc > 0.0 && uc < acc) {
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
    sm.len = len;
    sm.emit = emit;
    Job& J = sm.job;
    J.kind = kind;
    if (kind != JOB_NONE) {
      J.row = b * N + cur;
      J.qrow = 0;
      J.r = cur;
      J.out_slot = b * N + len;
      J.m = sm.rm[cur];
      J.s = sm.rs[cur];
      J.t = T;
      scale_pair(T, J.c_hi, J.c_lo);
      J.inv_s = (float)(1.0 / J.s);
      J.wmul = 1.0;
      J.tau = (float)sm.qx[cur];
      int ne = 0;
      if (kind == JOB_EXCL)
        for (int c = cur + 1; c < N; ++c)
          if (sm.par[c] == cur) J.excl[ne++] = sm.tok[c];
      J.n_excl = ne;
    }
  }
  __syncthreads();
  if (!writer) return;
  const int len = sm.len;
  if (tid == 0) {
    P.accept_len[b] = len;
    if (P.status && sm.job.kind == JOB_NONE) P.status[b] = sm.status;  // else written by the race's merge
  }
  for (int i = tid; i < N; i += kWG) {
    int node = -1, t = -1;
    bool skip = false;
    if (sm.status == SV_REQ_OK) {
      if (i < len) {
        node = sm.path[i];
        t = sm.tok[node];
      } else if (i == len) {
        if (greedy) t = sm.emit;
        else skip = true;  // written by the race's merge
      }
    }
    P.accept_path[(int64_t)b * N + i] = node;
    if (!skip) P.tokens[(int64_t)b * N + i] = t;
  }
}

// ===================================================================== K3
// Exact fp64 race key of vocabulary id y, the same formula as the
// definition: w(y) / (-ln U_y).  With use_p the weight is p itself (the
// fallback for an all-zero residual).  l and q are the id's target logit
// and draft probability (fp32 values, exact in fp64).
__device__ __forceinline__ bool is_excluded(const Job& J, int y) {
  for (int i = 0; i < J.n_excl; ++i)
    if (J.excl[i] == y) return true;
  return false;
}
__device__ __forceinline__ double race_key_from(const Job& J, uint64_t seed, int b, int y, double l, double q,
                                                bool use_p) {
  const double p = l < (double)J.tau ? 0.0 : p_at(l, J.m, J.t, J.s);
  double w = p;
  if (!use_p) {
    if (J.kind == JOB_RESID) w = (J.wmul * p - q > 0.0) ? J.wmul * p - q : 0.0;
    else if (J.kind == JOB_EXCL && is_excluded(J, y)) w = 0.0;
  }
  const double U = uniform_f64(noise_word(seed, b, J.r, y));
  return w / -log(U);
}
// Pick the larger key, ties to the smaller id.
__device__ __forceinline__ bool better(double ka, int ya, double kb_, int yb) {
  return ka > kb_ || (ka == kb_ && ya < yb);
}

// Block-wide best (key, id) pair.
__device__ __forceinline__ void block_best(double& k, int& y, Smem& sm) {
  for (int o = 32; o > 0; o >>= 1) {
    const double ok = __shfl_xor(k, o, 64);
    const int oy = __shfl_xor(y, o, 64);
    if (better(ok, oy, k, y)) {
      k = ok;
      y = oy;
    }
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) {
    sm.red_d[wave] = k;
    sm.red_i[wave] = y;
  }
  __syncthreads();
  k = sm.red_d[0];
  y = sm.red_i[0];
  for (int w = 1; w < kWaves; ++w)
    if (better(sm.red_d[w], sm.red_i[w], k, y)) {
      k = sm.red_d[w];
      y = sm.red_i[w];
    }
}

// Exact fp64 key of one id, kept out of line for the fp64 loops below:
// inlined into them, its fp64 constants would be held in registers for the
// whole kernel.
__device__ __attribute__((noinline)) double race_key_cold(double l, double q, double m, double T, double S,
                                                          double wmul, int resid, int use_p, uint64_t seed, int b,
                                                          int r, int y, double tau) {
  const double p = l < tau ? 0.0 : exp((l - m) / T) / S;
  double w = p;
  if (!use_p && resid) w = (wmul * p - q > 0.0) ? wmul * p - q : 0.0;
  const double U = uniform_f64(noise_word(seed, b, r, y));
  return w / -log(U);
}
// Exact fp64 weight of one id (p, or the residual max(wmul p - q, 0)).
__device__ __attribute__((noinline)) double weight_cold(double l, double q, double m, double T, double S,
                                                        double wmul, int resid, double tau) {
  const double p = l < tau ? 0.0 : exp((l - m) / T) / S;
  if (resid) return (wmul * p - q > 0.0) ? wmul * p - q : 0.0;
  return p;
}

// Chunk noise of the race: word 0 of counter (c, r, b, 2), and E_c = -ln U_c.
__device__ __forceinline__ double chunk_exp(uint64_t seed, int b, int r, int c) {
  const u32x4 ctr = {(uint32_t)c, (uint32_t)r, (uint32_t)b, 2u};
  return -log(uniform_f64(philox10(ctr, (uint32_t)seed, (uint32_t)(seed >> 32)).x));
}

// fp64 weight sum of chunk c (block-wide; every thread gets it).  use_p:
// the weights are p itself (the fallback for an all-zero residual).
template <bool BF16>
__device__ double chunk_sum_f64(const Params& P, const Job& J, int c, bool use_p, Smem& sm) {
  const float* qrow = J.kind == JOB_RESID ? P.q + (int64_t)J.qrow * P.qstride : nullptr;
  const int resid = !use_p && J.kind == JOB_RESID;
  const int y1 = min(P.V, (c + 1) * kK3Chunk);
  double s = 0.0;
#pragma unroll 1
  for (int y = c * kK3Chunk + (int)threadIdx.x; y < y1; y += kWG) {
    if (!use_p && J.kind == JOB_EXCL && is_excluded(J, y)) continue;
    const double l = (double)load_logit<BF16>(P, J.row, y);
    const double q = qrow ? (double)qrow[y] : 0.0;
    s += weight_cold(l, q, J.m, J.t, J.s, J.wmul, resid, (double)J.tau);
  }
  return block_sum_d(s, sm);
}

// The id race of chunk c in fp64 (block-wide): exact keys for every id.
template <bool BF16>
__device__ int chunk_race_f64(const Params& P, const Job& J, int b, int c, bool use_p, Smem& sm) {
  const float* qrow = J.kind == JOB_RESID ? P.q + (int64_t)J.qrow * P.qstride : nullptr;
  const uint64_t seed = P.seed[b];
  const int y1 = min(P.V, (c + 1) * kK3Chunk);
  double best_k = -1.0;
  int best_y = INT32_MAX;
#pragma unroll 1
  for (int y = c * kK3Chunk + (int)threadIdx.x; y < y1; y += kWG) {
    const double l = (double)load_logit<BF16>(P, J.row, y);
    const double q = qrow ? (double)qrow[y] : 0.0;
    const bool zero = !use_p && J.kind == JOB_EXCL && is_excluded(J, y);
    const double key = zero ? 0.0 : race_key_cold(l, q, J.m, J.t, J.s, J.wmul, J.kind == JOB_RESID, use_p, seed, b,
                                                          J.r, y, (double)J.tau);
    if (better(key, y, best_k, best_y)) {
      best_k = key;
      best_y = y;
    }
  }
  block_best(best_k, best_y, sm);
  return best_y;
}

// The whole two-level race in fp64 by one workgroup: used when the fp32
// screen cannot certify its result, and on request.  If every weight is
// zero the race is run over p instead.
template <bool BF16>
__device__ int race_row_f64(const Params& P, const Job& J, int b, Smem& sm) {
  const uint64_t seed = P.seed[b];
  for (int pass = 0; pass < 2; ++pass) {
    const bool use_p = pass == 1;
    double best_k = -1.0;
    int best_c = INT32_MAX;
#pragma unroll 1
    for (int c = 0; c < P.C3; ++c) {
      const double key = chunk_sum_f64<BF16>(P, J, c, use_p, sm) / chunk_exp(seed, b, J.r, c);
      if (better(key, c, best_k, best_c)) {
        best_k = key;
        best_c = c;
      }
    }
    if (best_k > 0.0) return chunk_race_f64<BF16>(P, J, b, best_c, use_p, sm);
  }
  return 0;  // unreachable: p has a positive entry (the row maximum)
}

// fp32 bounds wlo <= w(y) <= whi of this thread's 8 ids of chunk c, ids
// c*kK3Chunk + 4*(g*kWG + tid) + i (group g, lane i).  e = 2^t approximates exp((l - m)/T) with relative error at most
// eta = (|t| 2^-21 + 2^-17) (argument rounding plus v_exp_f32, far above
// the measured 2^-23.5); t is clamped to [-256, 0], where e is below every
// fp32 weight that matters (and no NaN arises from a -inf logit).  For a
// residual w = max(p - q, 0) with p = e/S; otherwise w = e/S.  Ids past
// the vocabulary, removed ids and ids whose logit is below the job's
// threshold get 0 for both bounds.
template <bool BF16, int KIND>
__device__ __forceinline__ void weight_bounds(const Params& P, const Job& J, int c, float* whi, float* wlo) {
  const int tid = threadIdx.x;
  const float m = J.m, chi = J.c_hi, clo = J.c_lo, inv_s = J.inv_s;
  const float tau = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(J.tau)));
  const int y_base = c * kK3Chunk;
  const int64_t lrow = (int64_t)J.row * P.lstride;
  const int64_t qrow = (int64_t)J.qrow * P.qstride;
  uint32_t excl_mask = 0;  // bit g*4+i: this thread's id is a removed token
  if (KIND == JOB_EXCL) {
    for (int i = 0; i < J.n_excl; ++i) {
      const int z = J.excl[i] - y_base;
      if (z >= 0 && z < kK3Chunk) {
        const int gi = z >> 2;
        if ((gi % kWG) == tid) excl_mask |= 1u << ((gi / kWG) * 4 + (z & 3));
      }
    }
  }
#pragma unroll
  for (int g = 0; g < kK3Groups; ++g) {
    const int y0 = y_base + 4 * (g * kWG + tid);
    const bool full = y0 + 4 <= P.V;
    float l[4], q[4];
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
    if (tau > -INFINITY)  // a scalar branch: top-k / top-p cut ids count as -inf
#pragma unroll
      for (int i = 0; i < 4; ++i) l[i] = l[i] < tau ? -INFINITY : l[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = 0.f;
    if (KIND == JOB_RESID) {
      if (full && P.q_aligned) {
        const u32x4 w = __builtin_nontemporal_load((const u32x4*)(P.q + qrow + y0));
        q[0] = __uint_as_float(w.x);
        q[1] = __uint_as_float(w.y);
        q[2] = __uint_as_float(w.z);
        q[3] = __uint_as_float(w.w);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = (y0 + i < P.V) ? P.q[qrow + y0 + i] : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float d = l[i] - m;
      const float t = fmaxf(__builtin_fmaf(d, chi, d * clo), -256.f);
      const float e = __builtin_amdgcn_exp2f(t);
      const float eta = __builtin_fmaf(t, -0x1p-21f, 0x1p-17f);
      const float p = e * inv_s;
      float h, lw;
      if (KIND == JOB_RESID) {
        h = fmaxf(__builtin_fmaf(p, eta, p) - q[i], 0.f) * (1.f + 0x1p-22f);
        lw = fmaxf(__builtin_fmaf(-p, eta, p) - q[i], 0.f) * (1.f - 0x1p-22f);
      } else {
        h = __builtin_fmaf(p, eta, p) * (1.f + 0x1p-22f);
        lw = __builtin_fmaf(-p, eta, p) * (1.f - 0x1p-22f);
      }
      const bool out = !(y0 + i < P.V) || (KIND == JOB_EXCL && ((excl_mask >> (g * 4 + i)) & 1u));
      whi[g * 4 + i] = out ? 0.f : h;
      wlo[g * 4 + i] = out ? 0.f : lw;
    }
  }
}

// Id-race screen of this thread's 8 ids of chunk c, in fp32: E2 = -log2 U
// and its reciprocal are each within 2^-22 (v_log_f32 measured at 2^-23
// over every possible U, v_rcp_f32 at 2^-23.4), and w / E2 is a constant
// multiple of w / E.  On return whi holds the key upper bounds; the
// largest key lower bound is returned.
__device__ __forceinline__ float race_screen(const Job& J, uint64_t seed, int b, int c, float* whi, const float* wlo) {
  const int tid = threadIdx.x;
  float lo_max = 0.f;
#pragma unroll
  for (int g = 0; g < kK3Groups; ++g) {
    const int y0 = c * kK3Chunk + 4 * (g * kWG + tid);
    const u32x4 ctr = {(uint32_t)y0 >> 2, (uint32_t)J.r, (uint32_t)b, 1u};
    const u32x4 rnd = philox10(ctr, (uint32_t)seed, (uint32_t)(seed >> 32));
    const uint32_t words[4] = {rnd.x, rnd.y, rnd.z, rnd.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float rE = __builtin_amdgcn_rcpf(-__builtin_amdgcn_logf(uniform_f32(words[i])));
      const int j = g * 4 + i;
      lo_max = fmaxf(lo_max, wlo[j] * rE * (1.f - 0x1p-20f));
      whi[j] = whi[j] * rE * (1.f + 0x1p-20f);
    }
  }
  return lo_max;
}

// The id race of chunk c once the screen's bound L (block-wide) is known:
// the ids whose key upper bound reaches L (the candidates) are re-keyed
// exactly in fp64.  Returns the winner, or -1 when the screen cannot
// certify it (L too small for fp32, or more than kCandMax candidates).
template <bool BF16>
__device__ __forceinline__ int race_pick(const Params& P, const Job& J, int b, int c, const float* khi, float L,
                                         Smem& sm) {
  const int tid = threadIdx.x;
  if (!(L >= 0x1p-70f)) return -1;
#pragma unroll
  for (int j = 0; j < 4 * kK3Groups; ++j) {
    if (khi[j] >= L) {
      const int slot = atomicAdd(&sm.ncand, 1);
      if (slot < kCandMax) sm.cand_y[slot] = c * kK3Chunk + 4 * ((j >> 2) * kWG + tid) + (j & 3);
    }
  }
  __syncthreads();
  const int nc = sm.ncand;
  if (nc < 1 || nc > kCandMax) return -1;
  if (nc == 1) return sm.cand_y[0];
  if (tid < nc) {
    const int y = sm.cand_y[tid];
    const double l = (double)load_logit<BF16>(P, J.row, y);
    const double q = J.kind == JOB_RESID ? (double)P.q[(int64_t)J.qrow * P.qstride + y] : 0.0;
    sm.cand_key[tid] = race_key_from(J, P.seed[b], b, y, l, q, false);
  }
  __syncthreads();
  double bk = -1.0;
  int by = INT32_MAX;
  for (int i = 0; i < nc; ++i)
    if (better(sm.cand_key[i], sm.cand_y[i], bk, by)) {
      bk = sm.cand_key[i];
      by = sm.cand_y[i];
    }
  return bk > 0.0 ? by : -1;
}

// Raw loads of this thread's ids of one race chunk (a whole chunk in
// aligned rows): the target logits (4 bf16 or 4 fp32 per group) and, for a
// residual, q.
template <bool BF16>
struct ChunkRaw {
  typename std::conditional<BF16, u32x2, u32x4>::type l[kK3Groups];
  u32x4 q[kK3Groups];
};

// Whether chunk c of the job's rows can be loaded as whole vectors.
__device__ __forceinline__ bool chunk_whole(const Params& P, const Job& J, int c) {
  return (c + 1) * kK3Chunk <= P.V && P.aligned && (J.kind != JOB_RESID || P.q_aligned);
}

template <bool BF16, int KIND>
__device__ __forceinline__ void chunk_load(const Params& P, const Job& J, int c, ChunkRaw<BF16>& r) {
  const int64_t lrow = (int64_t)J.row * P.lstride;
  const int64_t qrow = (int64_t)J.qrow * P.qstride;
#pragma unroll
  for (int g = 0; g < kK3Groups; ++g) {
    const int y0 = c * kK3Chunk + 4 * (g * kWG + (int)threadIdx.x);
    if constexpr (BF16) r.l[g] = __builtin_nontemporal_load((const u32x2*)((const uint16_t*)P.logits + lrow + y0));
    else r.l[g] = __builtin_nontemporal_load((const u32x4*)((const float*)P.logits + lrow + y0));
    if (KIND == JOB_RESID) r.q[g] = __builtin_nontemporal_load((const u32x4*)(P.q + qrow + y0));
  }
}

// Certified bounds dlo <= W_c <= dhi on the weight sum of chunk c, this
// thread's share before the block sum (r: the chunk's whole-vector loads,
// or null to load here, entry by entry where needed).  Per id, with e = 2^t
// as in weight_bounds and p = e/S computed as e * fl(1/S): the fp32 p is
// within (eta + 2^-23) p of the exact one, eta = |t| 2^-21 + 2^-17, and
// since max(., 0) is 1-Lipschitz the fp32 residual max(p - q, 0) is within
// that too (plus its own rounding, 2^-24 of itself).  So the thread sums
// the fp32 weights and, for the error, e and |t| e: no per-id bounds.  Ids
// whose logit is below the job's threshold count as -inf logits.
template <bool BF16, int KIND>
__device__ __forceinline__ void chunk_sum_bounds(const Params& P, const Job& J, int c, double& dhi, double& dlo,
                                                 const ChunkRaw<BF16>* r = nullptr) {
  const int tid = threadIdx.x;
  const float m = J.m, chi = J.c_hi, clo = J.c_lo, inv_s = J.inv_s;
  const float tau = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(J.tau)));
  const int y_base = c * kK3Chunk;
  const int64_t lrow = (int64_t)J.row * P.lstride;
  const int64_t qrow = (int64_t)J.qrow * P.qstride;
  uint32_t excl_mask = 0;  // bit g*4+i: this thread's id is a removed token
  if (KIND == JOB_EXCL) {
    for (int i = 0; i < J.n_excl; ++i) {
      const int z = J.excl[i] - y_base;
      if (z >= 0 && z < kK3Chunk) {
        const int gi = z >> 2;
        if ((gi % kWG) == tid) excl_mask |= 1u << ((gi / kWG) * 4 + (z & 3));
      }
    }
  }
  float sw = 0.f, se = 0.f, ste = 0.f;  // sum of residual weights; of e; of |t| e
#pragma unroll
  for (int g = 0; g < kK3Groups; ++g) {
    const int y0 = y_base + 4 * (g * kWG + tid);
    const bool full = y0 + 4 <= P.V;
    float l[4], q[4];
    if (r != nullptr || (full && P.aligned)) {
      if constexpr (BF16) {
        const u32x2 w = (r != nullptr) ? r->l[g]
                                       : __builtin_nontemporal_load((const u32x2*)((const uint16_t*)P.logits + lrow + y0));
        l[0] = __uint_as_float(w.x << 16);
        l[1] = __uint_as_float(w.x & 0xffff0000u);
        l[2] = __uint_as_float(w.y << 16);
        l[3] = __uint_as_float(w.y & 0xffff0000u);
      } else {
        const u32x4 w = (r != nullptr) ? r->l[g]
                                       : __builtin_nontemporal_load((const u32x4*)((const float*)P.logits + lrow + y0));
        l[0] = __uint_as_float(w.x);
        l[1] = __uint_as_float(w.y);
        l[2] = __uint_as_float(w.z);
        l[3] = __uint_as_float(w.w);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) l[i] = (y0 + i < P.V) ? load_logit<BF16>(P, J.row, y0 + i) : -INFINITY;
    }
    if (tau > -INFINITY)  // a scalar branch: top-k / top-p cut ids count as -inf
#pragma unroll
      for (int i = 0; i < 4; ++i) l[i] = l[i] < tau ? -INFINITY : l[i];
    if (KIND == JOB_RESID) {
      if (r != nullptr || (full && P.q_aligned)) {
        const u32x4 w = (r != nullptr) ? r->q[g] : __builtin_nontemporal_load((const u32x4*)(P.q + qrow + y0));
        q[0] = __uint_as_float(w.x);
        q[1] = __uint_as_float(w.y);
        q[2] = __uint_as_float(w.z);
        q[3] = __uint_as_float(w.w);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = (y0 + i < P.V) ? P.q[qrow + y0 + i] : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float d = l[i] - m;
      const float t = fmaxf(__builtin_fmaf(d, chi, d * clo), -256.f);  // a -inf logit gives e = 0
      float e = __builtin_amdgcn_exp2f(t);
      if (KIND == JOB_EXCL && ((excl_mask >> (g * 4 + i)) & 1u)) e = 0.f;
      se += e;
      ste = __builtin_fmaf(-t, e, ste);
      if (KIND == JOB_RESID) sw += fmaxf(__builtin_fmaf(e, inv_s, -q[i]), 0.f);
    }
  }
  // the fp32 sums of 8 non-negative terms are within 7 * 2^-24 of exact
  // (widened by 2^-20); the error terms are scaled up generously
  const double err = (double)inv_s * ((double)se * (0x1p-17 + 0x1p-22) + (double)ste * 0x1p-21) * (1.0 + 0x1p-10);
  const double w = (KIND == JOB_RESID) ? (double)sw : (double)se * (double)inv_s;
  dhi = w * (1.0 + 0x1p-20) + err;
  dlo = w * (1.0 - 0x1p-20) - err;
}

// Chunk c3 of a race: certified bounds on its weight sum W_c and so on its
// key W_c / E_c, stored in its record for the merge (only the winning
// chunk's ids race, in the merge).  With one chunk per item the record's
// marker follows at once; otherwise the item publishes its markers together
// once all its records are stored, and E_c comes from shared memory.  The
// fp64 block sum is within 2^-40; 2^-100 covers weights lost to underflow;
// the key's division and E_c's log are within 2^-48.
// A chunk's block sums and record, from this thread's share of its bounds.
template <bool BF16>
__device__ __forceinline__ void k3_chunk_record(const Params& P, const Job& J, int b, int c3, double dhi, double dlo,
                                                Smem& sm) {
  block_sum2_d(dhi, dlo, sm);
  if (threadIdx.x == 0) {
    const int e = c3 - sm.chunk_e0;
    const double E = (e >= 0 && e < kChunkE) ? sm.chunk_e[e] : chunk_exp(P.seed[b], b, J.r, c3);
    K3Rec* rec = &P.k3[(int64_t)b * P.C3 + c3];
    const double whi = dhi * (1.0 + 0x1p-40) + 0x1p-100;
    const double wlo = dlo > 0.0 ? dlo * (1.0 - 0x1p-40) : 0.0;
    cst_f64(&rec->khi, whi / E * (1.0 + 0x1p-48));
    cst_f64(&rec->klo, wlo / E * (1.0 - 0x1p-48));
    if (P.G3 == 1) {
      wait_mem();  // the record is stored before its marker
      cst_i32(&rec->count, 1);
    }
  }
}

template <bool BF16, int KIND>
__device__ __forceinline__ void k3_chunk(const Params& P, const Job& J, int b, int c3, Smem& sm) {
  double dhi, dlo;
  chunk_sum_bounds<BF16, KIND>(P, J, c3, dhi, dlo);
  k3_chunk_record<BF16>(P, J, b, c3, dhi, dlo, sm);
}

// The chunks [c_lo, c_hi) of an item, software-pipelined: a chunk's loads
// are issued before the previous chunk's block sums and record, which hide
// their latency.
template <bool BF16, int KIND>
__device__ __forceinline__ void k3_item_chunks(const Params& P, const Job& J, int b, int c_lo, int c_hi, Smem& sm) {
  ChunkRaw<BF16> r;
  bool whole = chunk_whole(P, J, c_lo);
  if (whole) chunk_load<BF16, KIND>(P, J, c_lo, r);
#pragma unroll 1
  for (int c3 = c_lo; c3 < c_hi; ++c3) {
    double dhi, dlo;
    if (whole) chunk_sum_bounds<BF16, KIND>(P, J, c3, dhi, dlo, &r);
    else chunk_sum_bounds<BF16, KIND>(P, J, c3, dhi, dlo);
    whole = c3 + 1 < c_hi && chunk_whole(P, J, c3 + 1);
    if (whole) chunk_load<BF16, KIND>(P, J, c3 + 1, r);
    k3_chunk_record<BF16>(P, J, b, c3, dhi, dlo, sm);
  }
}

template <bool BF16>
__device__ __forceinline__ void sample_chunk(const Params& P, int b, int c3, Smem& sm) {
  const int kind = uniform_i(sm.job.kind);
  if (kind == JOB_RESID) k3_chunk<BF16, JOB_RESID>(P, sm.job, b, c3, sm);
  else if (kind == JOB_EXCL) k3_chunk<BF16, JOB_EXCL>(P, sm.job, b, c3, sm);
  else k3_chunk<BF16, JOB_P>(P, sm.job, b, c3, sm);
}

// The id race of chunk c by one workgroup: the fp32 screen, then fp64 where
// it cannot certify the winner.
template <bool BF16, int KIND>
__device__ __forceinline__ int chunk_race(const Params& P, const Job& J, int b, int c, Smem& sm) {
  constexpr int NI = 4 * kK3Groups;
  float whi[NI], wlo[NI];
  weight_bounds<BF16, KIND>(P, J, c, whi, wlo);
  const float lo = race_screen(J, P.seed[b], b, c, whi, wlo);
  if (threadIdx.x == 0) sm.ncand = 0;
  const float L = block_max(lo, sm);
  const int y = race_pick<BF16>(P, J, b, c, whi, L, sm);
  if (y >= 0) return y;
  return chunk_race_f64<BF16>(P, J, b, c, false, sm);
}

// Merge of one race by the request's last chunk, once every chunk's record
// is complete (lo: the largest key lower bound this thread read, kh0: the
// upper bound of chunk `tid`).  L = the largest certified lower bound over
// the chunks; the winning chunk's upper bound reaches L, so it is among the
// chunks whose upper bound does: a single one is the winner, several are
// keyed exactly in fp64.  Then the ids of the winning chunk race.  L = 0 (no
// chunk certainly positive: an all-zero residual, or weights too small to
// certify) and more than kCandMax candidates go to the fp64 race.
template <bool BF16>
__device__ __forceinline__ void k3_merge(const Params& P, int b, double lo, double kh0, Smem& sm) {
  const Job& J = sm.job;
  const int tid = threadIdx.x;
  if (tid == 0) sm.ncand = 0;
  const double L = __longlong_as_double((long long)block_max_u64((uint64_t)__double_as_longlong(lo), sm));
  bool fallback = (P.flags & SV_FLAG_FP64_RACE) || !(L > 0.0);
  if (!fallback) {
    for (int c = tid; c < P.C3; c += kWG) {
      const double kh = (c == tid) ? kh0 : cld_f64(&P.k3[(int64_t)b * P.C3 + c].khi);
      if (kh >= L) {
        const int slot = atomicAdd(&sm.ncand, 1);
        if (slot < kCandMax) sm.cand_y[slot] = c;
      }
    }
    __syncthreads();
    fallback = sm.ncand < 1 || sm.ncand > kCandMax;
  }
  int by = -1;
  if (!fallback) {
    const int nc = uniform_i(sm.ncand);
    int best_c = sm.cand_y[0];
    if (nc > 1) {
      double bk = -1.0;
      best_c = INT32_MAX;
#pragma unroll 1
      for (int i = 0; i < nc; ++i) {
        const int c = uniform_i(sm.cand_y[i]);
        const double key = chunk_sum_f64<BF16>(P, J, c, false, sm) / chunk_exp(P.seed[b], b, J.r, c);
        if (better(key, c, bk, best_c)) {
          bk = key;
          best_c = c;
        }
      }
      fallback = !(bk > 0.0);
    }
    __syncthreads();  // every thread has read the candidates before LDS is reused
    if (!fallback) {
      const int c = uniform_i(best_c);
      const int kind = uniform_i(J.kind);
      if (kind == JOB_RESID) by = chunk_race<BF16, JOB_RESID>(P, J, b, c, sm);
      else if (kind == JOB_EXCL) by = chunk_race<BF16, JOB_EXCL>(P, J, b, c, sm);
      else by = chunk_race<BF16, JOB_P>(P, J, b, c, sm);
    }
  }
  if (fallback) by = race_row_f64<BF16>(P, J, b, sm);
  if (tid == 0) P.tokens[J.out_slot] = by;
}

// The race of a P or EXCL job (one-hot chains and trees, unfiltered) from
// the race-chunk sums that the statistics pass published, by one
// workgroup: certified bounds on every chunk's weight sum W_c without
// reading the row, then the merge (candidate chunks, the winning chunk's id
// race), which writes the sampled token.
//
// A published share s (fp32 sum of 2^t_i, t_i = fl(l_i c - off), c =
// fp32(log2(e)/T)) stands for the exact sum of 2^(l_i c* - off), c* =
// log2(e)/T, within  2^-23 (n + |off| s) + 2^-20 s + 2^-110  (units of
// 2^off, n <= 128 ids): the argument's rounding and the rounding of c give
// a relative error of each term of at most 2^-24 ln2 (2 |t_i| + |off|)
// since |l_i c*| <= |t_i| + |off| + tiny, and sum_i 2^t_i |t_i| <= 0.531 n
// for t_i <= 0; v_exp_f32 and the fp32 additions add at most 2^-20 s; terms
// below the fp32 range add less than 2^-117.  Scaled by 2^(off - m c*) the
// shares give W_c in units of the row's largest term (1/S is common to all
// chunks and cancels in the race); an EXCL job subtracts the exact terms of
// its removed ids.
template <bool BF16, bool COH>
__device__ __forceinline__ void csum_race(const Params& P, int b, Smem& sm) {
  const Job& J = sm.job;
  const int tid = threadIdx.x;
  const double cd = 1.4426950408889634074 / J.t;
  const double mref = (double)J.m * cd;
  const uint64_t seed = P.seed[b];
  double lo = 0.0, kh0 = -1.0;
  static_assert(kCSumShares % 2 == 0, "shares are loaded two at a time");
  for (int c = tid; c < P.C3; c += kWG) {
    const CSum* cs = &P.csum[((int64_t)J.row * P.C3 + c) * kCSumShares];
    // every share of the chunk in flight at once (128 contiguous bytes)
    uint64_t sb[kCSumShares];
    if constexpr (COH) {
#pragma unroll
      for (int w = 0; w < kCSumShares; ++w) sb[w] = ld64<COH>(&cs[w]);
    } else {
#pragma unroll
      for (int w = 0; w < kCSumShares / 2; ++w) {
        const u32x4 v = *(const u32x4*)&cs[2 * w];
        sb[2 * w] = (uint64_t)v.x | ((uint64_t)v.y << 32);
        sb[2 * w + 1] = (uint64_t)v.z | ((uint64_t)v.w << 32);
      }
    }
    double E = 0.0, err = 0.0;
#pragma unroll
    for (int w = 0; w < kCSumShares; ++w) {
      const uint64_t bits = sb[w];
      const float ws = __uint_as_float((uint32_t)bits), off = __uint_as_float((uint32_t)(bits >> 32));
      if (off == -INFINITY) continue;  // the row of lanes saw only masked ids
      // 2^(off - m c*) by v_exp_f32 (within 2^-22, and the argument's
      // rounding 2^-24 |d|), counted in the bound below
      const double d = (double)off - mref;
      const double sc = (double)__builtin_amdgcn_exp2f((float)d);
      E += (double)ws * sc;
      err += (0x1p-23 * (128.0 + fabs((double)off) * (double)ws) + (0x1p-19 + 0x1p-23 * fabs(d)) * (double)ws +
              0x1p-110) * sc;
    }
    double ex = 0.0;
    if (J.kind == JOB_EXCL)
      for (int i = 0; i < J.n_excl; ++i) {
        const int x = J.excl[i];
        if (x >= c * kK3Chunk && x < (c + 1) * kK3Chunk)
          ex += exp(((double)load_logit<BF16>(P, J.row, x) - (double)J.m) / J.t);
      }
    const double whi = (E + err - ex * (1.0 - 0x1p-50)) * (1.0 + 0x1p-40);
    const double wd = E - err - ex * (1.0 + 0x1p-50);
    const double wlo = wd > 0.0 ? wd * (1.0 - 0x1p-40) : 0.0;
    const double En = chunk_exp(seed, b, J.r, c);
    const double khi = whi / En * (1.0 + 0x1p-48), klo = wlo / En * (1.0 - 0x1p-48);
    if (P.C3 > kWG) {
      // k3_merge reads the upper bounds of the chunks past the block from
      // the records (its own thread's from kh0)
      K3Rec* rec = &P.k3[(int64_t)b * P.C3 + c];
      cst_f64(&rec->khi, khi);
      cst_f64(&rec->klo, klo);
    }
    lo = fmax(lo, klo);
    if (c == tid) kh0 = khi;
  }
  if (P.C3 > kWG) wait_mem();  // those records are stored before k3_merge reads them
  __syncthreads();
  k3_merge<BF16>(P, b, lo, kh0, sm);
}

// ===================================================================== driver
// K1 segment: sub-chunks [s0, s1) of row r of request b, written to the
// row's partial slot `slot`.  Its first HBM loads are issued before
// anything else; then the request's temperature and drafts decide whether
// the row is needed (rows after a chain's first -1 are not).  Wave 0 also
// gathers the target logit (and q) at the draft tokens that fall in the
// segment, so the decision step needs no dependent loads.  Row-statistics
// calls count each row's segments; the workgroup that completes a row
// combines it.  The fused schedule counts each request's segments for its
// sampling chunks to wait on.
template <int MODE, bool BF16, bool CS = false, bool CAND = false>
__device__ __forceinline__ void run_k1_seg(const Params& P, int b, int r, int s0, int s1, int slot, Smem& sm,
                                           CSum* cs_lds = nullptr) {
  const int64_t row = (int64_t)b * P.R + r;
  const int64_t start = (int64_t)s0 * P.SUB;
  const int n_seg = (int)(min((int64_t)s1 * P.SUB, (int64_t)P.V) - start);
  u32x4 raw0[kVecPerThread];
  k1_issue<BF16>(P, row * P.lstride + start, n_seg, raw0);
  // The workspace region of the sampling records depends on the call's
  // shape, so it may hold anything: the segment that starts the request's
  // first row clears the request's completion markers (wave 0, whose
  // stores the count below waits for; a kernel boundary orders them for
  // the phased schedule).
  if (MODE != MODE_ROWS && r == 0 && s0 == 0 && threadIdx.x < 64)
    for (int c = threadIdx.x; c < P.C3; c += 64) cst_i32(&P.k3[(int64_t)b * P.C3 + c].count, 0);
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
    // top-k rows whose thresholds come from candidate groups
    int tk = 0;
    if (CAND && stoch) {
      const int k = P.top_k ? P.top_k[b] : 0;
      if (kc_row(P, k)) tk = k;
    }
    if (CS && stoch && MODE != MODE_ROWS && P.csum_fold)
      k1_seg_stats<BF16, true, false, CS, CAND>(P, row, s0, s1, slot, T, raw0, sm, cs_lds, tk);
    else if (stoch)
      k1_seg_stats<BF16, true, MODE == MODE_ROWS, false, CAND>(P, row, s0, s1, slot, T, raw0, sm, nullptr, tk);
    else k1_seg_stats<BF16, false, false>(P, row, s0, s1, slot, T, raw0, sm);
    if (MODE != MODE_ROWS && threadIdx.x < 64 && stoch) {
      const int lane = threadIdx.x;
      const int64_t stop = start + n_seg;
      int tok = -1, gslot = -1;
      if (MODE == MODE_CHAIN) {
        if (lane == 0 && r < P.k) {
          tok = P.ids[(int64_t)b * P.k + r];
          gslot = r;
        }
      } else if (lane >= 1 && lane < P.R && P.parent[(int64_t)b * P.R + lane] == r) {
        tok = P.node_tokens[(int64_t)b * P.R + lane];
        gslot = lane;
      }
      if (gslot >= 0 && tok >= start && tok < stop) {
        const float l = load_logit<BF16>(P, row, tok);
        float q = 0.f;
        if (MODE == MODE_CHAIN && P.draft_kind == SV_DRAFT_PROBS) q = P.q[((int64_t)b * P.k + r) * P.qstride + tok];
        cst64(&P.gat[(int64_t)b * SV_MAX_NODES + gslot],
              (uint64_t)__float_as_uint(l) | ((uint64_t)__float_as_uint(q) << 32));
      }
    }
  }
  if (MODE != MODE_ROWS && P.sched != SCHED_FUSED) return;
  if (threadIdx.x == 0) {
    wait_mem();  // this wave's partial and gathers are complete
    const uint32_t old = atomic_add_relaxed(&P.sync[b].k1_count, 1u);
    sm.flag = (MODE == MODE_ROWS) && old == (uint32_t)k1_segments(P, row) - 1u;
  }
  if (MODE == MODE_ROWS) {
    __syncthreads();
    if (uniform_i(sm.flag)) {
      if (threadIdx.x == 0) cst32(&P.sync[b].k1_count, 0u);
      k2_rows(P, b, sm);
    }
  }
}

// K1 item o of request b: segment o % Q of row o / Q.
template <int MODE, bool BF16, bool CS = false, bool CAND = false>
__device__ __forceinline__ void run_k1_item(const Params& P, int b, int o, Smem& sm, CSum* cs_lds = nullptr) {
  const int q = P.Q;
  const int r = o / q, c = o - r * q;
  run_k1_seg<MODE, BF16, CS, CAND>(P, b, r, (int)((int64_t)c * P.nsub / q), (int)((int64_t)(c + 1) * P.nsub / q), c,
                                   sm, cs_lds);
}

// Request order of the decision/sampling work: for batches of at most 64
// requests the sampling requests go first (then the others, each group in
// index order), so that their chunks are dispatched first and the launch
// ends with the requests that have no race to run; larger batches keep
// index order.
__device__ __forceinline__ int request_at(const Params& P, int g) {
  if (P.bs > 64) return g;
  const int lane = threadIdx.x & 63;
  const uint64_t st = __ballot(lane < P.bs && is_stochastic(P.temp[lane]));
  const int ns = __popcll(st);
  const uint64_t want = g < ns ? st : (~st & (P.bs == 64 ? ~0ull : ((1ull << P.bs) - 1ull)));
  const int k = g < ns ? g : g - ns;
  // the position of the k-th set bit of `want`
  const uint64_t below = (lane == 0) ? 0ull : (want & ((1ull << lane) - 1ull));
  const uint64_t hit = __ballot(((want >> lane) & 1ull) && __popcll(below) == k);
  return (int)__builtin_ctzll(hit);
}

// K23 item `item` of request b: its own run of the decision step, then the
// sampling chunks [item G3, (item + 1) G3).  Greedy requests (and bad
// temperatures) sample nothing: only their item 0 works, to decide and
// write the outputs.  The request's last item merges the chunks' results
// and resets the request's counters.
template <int MODE, bool BF16, bool COH>
__device__ __forceinline__ void run_k23(const Params& P, int b, int item, Smem& sm) {
  const int tid = threadIdx.x;
  const bool writer = (item == 0);
  const bool stoch = uniform_i(is_stochastic(temp_of(P, b)));
  const bool work = stoch || writer;
  int ok = 1;
  if (P.sched == SCHED_FUSED && work) {
    if (tid == 0) {
      uint32_t expect = 0;
      for (int r = 0; r < P.R; ++r) expect += (uint32_t)k1_segments(P, (int64_t)b * P.R + r);
      uint32_t spins = 0;
      while (cld32(&P.sync[b].k1_count) < expect) {
        __builtin_amdgcn_s_sleep(40);  // about a microsecond between polls
        if (++spins > kSpinLimit || cld32(&P.ctrl->aborted)) {
          ok = 0;
          break;
        }
      }
      if (!ok) {
        cst32(&P.ctrl->aborted, 1u);
        if (P.status) P.status[b] = SV_REQ_INTERNAL;
      }
      sm.flag = ok;
    }
    __syncthreads();
    ok = uniform_i(sm.flag);
  }
  bool sampled = false;
  const int c_lo = item * P.G3, c_hi = min(P.C3, c_lo + P.G3);  // this item's chunks
  if (work && ok) {
    if (MODE == MODE_CHAIN) decide_chain<BF16, COH>(P, b, writer, sm);
    else decide_tree<BF16, COH>(P, b, writer, sm);
    if (uniform_i(sm.job.kind) != JOB_NONE) {
      if (P.G3 == 1) {
        if (tid == 0) sm.chunk_e0 = INT32_MIN / 2;  // no precomputed noise
        sample_chunk<BF16>(P, b, c_lo, sm);
      } else {
        // the item's chunk noise, one thread per chunk
        if (tid == 0) sm.chunk_e0 = c_lo;
        if (tid < min(c_hi - c_lo, kChunkE)) sm.chunk_e[tid] = chunk_exp(P.seed[b], b, sm.job.r, c_lo + tid);
        __syncthreads();
        const int kind = uniform_i(sm.job.kind);
        if (kind == JOB_RESID) k3_item_chunks<BF16, JOB_RESID>(P, sm.job, b, c_lo, c_hi, sm);
        else if (kind == JOB_EXCL) k3_item_chunks<BF16, JOB_EXCL>(P, sm.job, b, c_lo, c_hi, sm);
        else k3_item_chunks<BF16, JOB_P>(P, sm.job, b, c_lo, c_hi, sm);
        // one wait for all the item's records, then their markers
        if (tid == 0) wait_mem();
        __syncthreads();
        for (int c3 = c_lo + tid; c3 < c_hi; c3 += kWG) cst_i32(&P.k3[(int64_t)b * P.C3 + c3].count, 1);
      }
      sampled = true;
    } else if (stoch) {
      for (int c3 = c_lo + tid; c3 < c_hi; c3 += kWG)
        cst_i32(&P.k3[(int64_t)b * P.C3 + c3].count, 1);  // complete, nothing raced
    }
  }
  if (!stoch) {
    // only chunk 0 worked; in the fused schedule it was the counter's last user
    if (P.sched == SCHED_FUSED && work && ok && tid == 0) cst32(&P.sync[b].k1_count, 0u);
    return;
  }
  if (item != P.CI - 1) return;
  // The request's last item (dispatched after all its others, so none of
  // them waits on it) merges once every chunk's record is complete (bounded
  // wait), then resets the request's counter.  A record's contents are
  // read after its marker (they are stored before it).
  int done = ok;
  double lo = 0.0, kh0 = -1.0;
  if (ok) {
    for (int c = tid; c < P.C3; c += kWG) {
      const K3Rec* rec = &P.k3[(int64_t)b * P.C3 + c];
      uint32_t spins = 0;
      while (cld_i32(&rec->count) == 0) {
        __builtin_amdgcn_s_sleep(2);
        if (++spins > kSpinLimit || cld32(&P.ctrl->aborted)) {
          done = 0;
          break;
        }
      }
      if (!done) break;
      if (sampled) {
        lo = fmax(lo, cld_f64(&rec->klo));
        if (c == tid) kh0 = cld_f64(&rec->khi);
      }
    }
  }
  done = block_min_i(done, sm);
  if (!done && ok && tid == 0) {
    cst32(&P.ctrl->aborted, 1u);
    if (P.status) P.status[b] = SV_REQ_INTERNAL;
  }
  if (done && sampled) {
    k3_merge<BF16>(P, b, lo, kh0, sm);
    if (tid == 0 && P.status) P.status[b] = SV_REQ_OK;  // the request's status, after its token
  }
  if (tid == 0 && P.sched == SCHED_FUSED) cst32(&P.sync[b].k1_count, 0u);
}

template <int MODE, bool BF16>
__global__ __launch_bounds__(kWG, SV_K1_OCC) void k1_kernel(Params P) {
  __shared__ Smem sm;
  __shared__ CSum cs_lds[MODE == MODE_ROWS ? 1 : kCSumLds * kCSumShares];  // race-chunk shares of the segment
  const int n1 = P.R * P.Q;
  const int b = (int)(blockIdx.x / (uint32_t)n1);
  run_k1_item<MODE, BF16, MODE != MODE_ROWS>(P, b, (int)(blockIdx.x - (uint32_t)b * (uint32_t)n1), sm, cs_lds);
}

// The statistics pass of a top-k filtered call: K1 that also publishes the
// filtered rows' top-k candidates.
template <int MODE, bool BF16>
__global__ __launch_bounds__(kWG, SV_K1_OCC) void k1f_kernel(Params P) {
  __shared__ Smem sm;
  const int n1 = P.R * P.Q;
  const int b = (int)(blockIdx.x / (uint32_t)n1);
  run_k1_item<MODE, BF16, true, true>(P, b, (int)(blockIdx.x - (uint32_t)b * (uint32_t)n1), sm);
}

// Decisions and sampling of a call whose statistics pass published the race
// chunk sums (phased schedule): one workgroup per request decides and races
// from the sums.  A kernel of its own, so that the fp64 bound arithmetic
// has the registers it needs without taxing the other kernels'.
template <int MODE, bool BF16>
__global__ __launch_bounds__(kWG, 2) void k23c_kernel(Params P) {
  __shared__ Smem sm;
  if constexpr (MODE != MODE_ROWS) {
    const int b = (int)blockIdx.x;
    if (MODE == MODE_CHAIN) decide_chain<BF16, false>(P, b, true, sm);
    else decide_tree<BF16, false>(P, b, true, sm);
    if (uniform_i(sm.job.kind) != JOB_NONE) {
      csum_race<BF16, false>(P, b, sm);
      if (threadIdx.x == 0 && P.status) P.status[b] = SV_REQ_OK;  // the request's status, after its token
    }
  }
}

template <int MODE, bool BF16>
__global__ __launch_bounds__(kWG, 8) void k23_kernel(Params P) {
  __shared__ Smem sm;
  if constexpr (MODE != MODE_ROWS) {
    // item 0 of every request first (it writes the request's outputs),
    // then items 1.. of the requests in request_at order: the sampling
    // requests' items before the greedy requests' idle ones
    const uint32_t t = blockIdx.x, bs = (uint32_t)P.bs;
    int b, item;
    if (t < bs) {
      b = (int)t;
      item = 0;
    } else {
      const uint32_t n = (uint32_t)P.CI - 1u, g = (t - bs) / n;
      b = uniform_i(request_at(P, (int)g));
      item = (int)(t - bs - g * n) + 1;
    }
    run_k23<MODE, BF16, false>(P, b, item, sm);
  }
}

// One launch.  Work item order: for g = 0 .. bs + lag - 1, the K1 items of
// request g (if g < bs), then the sampling chunks of request g - lag (if
// g >= lag), requests in request_at order.  A sampling chunk waits only for
// K1 items of its own request and the merge only for chunks of its own
// request, all earlier in dispatch order.
template <int MODE, bool BF16>
__global__ __launch_bounds__(kWG, 7) void fused_kernel(Params P) {
  __shared__ Smem sm;
  __shared__ CSum cs_lds[MODE == MODE_ROWS ? 1 : kCSumLds * kCSumShares];  // unused: no shares are published
  if constexpr (MODE != MODE_ROWS) {
    const uint32_t n1 = (uint32_t)(P.R * P.Q), n3 = (uint32_t)P.CI, L = (uint32_t)P.lag, bs = (uint32_t)P.bs;
    const uint32_t seg1 = L * n1, seg2 = (bs - L) * (n1 + n3);
    const uint32_t t = blockIdx.x;
    uint32_t g, o;
    bool k1;
    if (t < seg1) {
      g = t / n1;
      o = t - g * n1;
      k1 = true;
    } else if (t < seg1 + seg2) {
      const uint32_t u = t - seg1, blk = u / (n1 + n3), oo = u - blk * (n1 + n3);
      k1 = oo < n1;
      g = k1 ? L + blk : blk;
      o = k1 ? oo : oo - n1;
    } else {
      const uint32_t u = t - seg1 - seg2;
      g = bs - L + u / n3;
      o = u - (g - (bs - L)) * n3;
      k1 = false;
    }
    const int b = uniform_i(request_at(P, (int)g));
    if (k1) run_k1_item<MODE, BF16, true>(P, b, (int)o, sm, cs_lds);
    else run_k23<MODE, BF16, true>(P, b, (int)o, sm);
  } else {
    const int n1 = P.R * P.Q;
    const int b = (int)(blockIdx.x / (uint32_t)n1);
    run_k1_item<MODE, BF16>(P, b, (int)(blockIdx.x - (uint32_t)b * (uint32_t)n1), sm);
  }
}

// ===================================================================== KR
// Residual masses of the block rule: r_i = sum_y max(w_i p_i(y) - q_i(y), 0)
// for rows i = 1..kb-1 of the stochastic requests with draft probabilities
// (one-hot drafts have the closed form w_i (1 - p_i(x_i)), taken by the
// decision step).  One workgroup per (request, row i, item); an item is a
// run of whole 2048-id chunks.  Each workgroup folds the request's row
// statistics of rows 0..i and its gathered draft values to get w_i, then
// streams its ids of target row i and draft row i.  Every term is evaluated
// in fp64 as 2^((l - m) log2(e)/T) (w/S) - q, within about 1e-13 relative
// of the definition's w exp((l - m)/T)/S - q (an fp32 screen that skipped
// the clearly negative terms cost more than it saved: its branch diverges
// within a wave).  The fp64 partial sums are reduced in a fixed
// order: the decision step adds the items' partials in item order.
//
// 2^t for t <= 0 in fp64 without a division or a branch: t = n/64 + f with
// n = rint(64 t) and |f| <= 1/128; 2^f by its Taylor polynomial of degree 4
// (remainder below 4e-14 relative for |f ln 2| <= 0.0055), times 2^((n mod
// 64)/64) from a table of 64 entries (`tab`, in LDS), scaled by 2^(n div 64)
// exactly.  Below 2^-1022 (t = -inf included) it returns 0.
__device__ __forceinline__ double exp2_f64_nonpos(double t, const double* tab) {
  const double tc = fmax(t, -1022.0);
  const double n = __builtin_rint(tc * 64.0);
  const double f = __builtin_fma(n, -0.015625, tc);
  const int ni = (int)n;
  double p = __builtin_fma(0.009618129107628477, f, 0.055504108664821576);  // (ln 2)^4/4!, (ln 2)^3/3!
  p = __builtin_fma(p, f, 0.2402265069591007);                                // (ln 2)^2/2!
  p = __builtin_fma(p, f, 0.6931471805599453);                                // ln 2
  p = __builtin_fma(p, f, 1.0);
  const double r = __builtin_ldexp(tab[ni & 63] * p, ni >> 6);
  return t > -1022.0 ? r : 0.0;
}

template <bool BF16, bool VEC>
__device__ __forceinline__ void kr_load4(const Params& P, int64_t lrow, int64_t qrow, int y0, float* l, float* q) {
  if (VEC || (y0 + 4 <= P.V && P.aligned && P.q_aligned)) {
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
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)(P.q + qrow + y0));
    q[0] = __uint_as_float(v.x);
    q[1] = __uint_as_float(v.y);
    q[2] = __uint_as_float(v.z);
    q[3] = __uint_as_float(v.w);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool in = y0 + i < P.V;
      l[i] = in ? (BF16 ? bf16_to_f32(((const uint16_t*)P.logits)[lrow + y0 + i]) : ((const float*)P.logits)[lrow + y0 + i])
                : -INFINITY;
      q[i] = in ? P.q[qrow + y0 + i] : 0.f;
    }
  }
}

constexpr int kKRUnroll = SV_KR_UNROLL;  // groups of 4 ids whose loads a thread issues together

// The thread's share of sum_y max(2^((l - m) cd) wS - q, 0) over ids
// [y_lo, y_hi): kKRUnroll groups of 4 ids per step, all loads first.  Ids
// past y_hi load the range's first group again and count as l = -inf,
// q = 0 (a zero term), so with VEC every load is unconditional.  With
// FILT, ids whose logit is below tau count as -inf logits.
template <bool BF16, bool VEC, bool FILT>
__device__ __forceinline__ double kr_stream(const Params& P, int64_t lrow, int64_t qrow, int y_lo, int y_hi,
                                            double m, double cd, double wS, const double* tab, float tau) {
  const int tid = threadIdx.x;
  double acc = 0.0;
#pragma unroll 1
  for (int base = y_lo; base < y_hi; base += 4 * kWG * kKRUnroll) {
    float l[kKRUnroll][4], q[kKRUnroll][4];
    bool in[kKRUnroll];
#pragma unroll
    for (int g = 0; g < kKRUnroll; ++g) {
      const int y0 = base + 4 * (g * kWG + tid);
      in[g] = y0 < y_hi;
      kr_load4<BF16, VEC>(P, lrow, qrow, in[g] ? y0 : y_lo, l[g], q[g]);
    }
#pragma unroll
    for (int g = 0; g < kKRUnroll; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float le = (FILT && l[g][e] < tau) ? -INFINITY : l[g][e];
        const double ex = exp2_f64_nonpos(((double)le - m) * cd, tab);
        const double term = __builtin_fma(ex, wS, -(double)q[g][e]);
        acc += in[g] ? fmax(term, 0.0) : 0.0;
      }
  }
  return acc;
}

// Aligned rows: two register stages of kKRPipe groups each, alternating, so
// the next stage's loads are in flight while the current one is folded; the
// first stage is issued before the workgroup's prologue.  Loads past y_hi
// re-read the range's first group (and count as zero), so every load is
// unconditional and no stage is copied.
constexpr int kKRPipe = 2;
struct KRStage {
  float l[kKRPipe][4], q[kKRPipe][4];
};
template <bool BF16>
__device__ __forceinline__ void kr_issue(const Params& P, int64_t lrow, int64_t qrow, int base, int y_lo, int y_hi,
                                         KRStage& st) {
#pragma unroll
  for (int g = 0; g < kKRPipe; ++g) {
    const int y0 = base + 4 * (g * kWG + (int)threadIdx.x);
    kr_load4<BF16, true>(P, lrow, qrow, y0 < y_hi ? y0 : y_lo, st.l[g], st.q[g]);
  }
}
template <bool FILT>
__device__ __forceinline__ double kr_fold(const KRStage& st, int base, int y_hi, double m, double cd, double wS,
                                          const double* tab, float tau) {
  double acc = 0.0;
#pragma unroll
  for (int g = 0; g < kKRPipe; ++g) {
    const bool in = base + 4 * (g * kWG + (int)threadIdx.x) < y_hi;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float le = (FILT && st.l[g][e] < tau) ? -INFINITY : st.l[g][e];
      const double ex = exp2_f64_nonpos(((double)le - m) * cd, tab);
      const double term = __builtin_fma(ex, wS, -(double)st.q[g][e]);
      acc += in ? fmax(term, 0.0) : 0.0;
    }
  }
  return acc;
}
template <bool BF16, bool FILT>
__device__ __forceinline__ double kr_stream_pipe(const Params& P, int64_t lrow, int64_t qrow, int y_lo, int y_hi,
                                                 double m, double cd, double wS, const double* tab, KRStage& a,
                                                 float tau) {
  constexpr int step = 4 * kWG * kKRPipe;
  double acc = 0.0;
  KRStage bst;
#pragma unroll 1
  for (int base = y_lo;;) {
    kr_issue<BF16>(P, lrow, qrow, base + step, y_lo, y_hi, bst);
    acc += kr_fold<FILT>(a, base, y_hi, m, cd, wS, tab, tau);
    base += step;
    if (base >= y_hi) break;
    kr_issue<BF16>(P, lrow, qrow, base + step, y_lo, y_hi, a);
    acc += kr_fold<FILT>(bst, base, y_hi, m, cd, wS, tab, tau);
    base += step;
    if (base >= y_hi) break;
  }
  return acc;
}

template <bool BF16>
__global__ __launch_bounds__(kWG, 4) void kr_kernel(Params P) {
  __shared__ Smem sm;
  __shared__ double tab[64];  // 2^(j/64)
  const int tid = threadIdx.x, lane = tid & 63;
  const uint32_t per_req = (uint32_t)((P.k - 1) * P.CHr);
  const int b = (int)(blockIdx.x / per_req);
  const int rem = (int)(blockIdx.x - (uint32_t)b * per_req);
  const int i = 1 + rem / P.CHr;
  const int c = rem - (i - 1) * P.CHr;
  const float Tf = temp_of(P, b);
  if (!is_stochastic(Tf) || P.draft_kind != SV_DRAFT_PROBS) return;
  int xi;
  const int kb = chain_kb(P, b, xi);
  if (i >= kb) return;
  // this item's ids and the first stage of its stream, issued before the prologue
  const int c_lo = (int)((int64_t)c * P.C3 / P.CHr), c_hi = (int)((int64_t)(c + 1) * P.C3 / P.CHr);
  const int y_lo = c_lo * kK3Chunk, y_hi = min(c_hi * kK3Chunk, P.V);
  const int64_t lrow = ((int64_t)b * P.R + i) * P.lstride;
  const int64_t qrow = ((int64_t)b * P.k + i) * P.qstride;
  const bool vec = P.aligned && P.q_aligned && (P.V & 3) == 0;
  KRStage first;
  if (vec) kr_issue<BF16>(P, lrow, qrow, y_lo, y_lo, y_hi, first);
  uint64_t gl = 0;
  const bool filt = request_filtered(P, b, Tf);
  double fs = 0.0;  // top-k / top-p: kept sum and threshold of row `lane`
  float ftau = -INFINITY;
  if (tid < 64 && lane < i) gl = P.gat[(int64_t)b * SV_MAX_NODES + lane].l | ((uint64_t)P.gat[(int64_t)b * SV_MAX_NODES + lane].q << 32);
  if (tid < 64 && filt && lane <= i) {
    fs = P.filt[(int64_t)b * P.R + lane].s;
    ftau = P.filt[(int64_t)b * P.R + lane].tau;
  }
  if (tid < 64) tab[tid] = exp2((double)tid / 64.0);
  fold_rows<false>(P, (int64_t)b * P.R, i + 1, Tf, sm);  // ends with a barrier
  const double T = (double)Tf;
  if (tid < 64) {
    const bool bad = __ballot(lane <= i && sm.rbad[lane]) != 0;
    double p = 0.0, q = 0.0;
    if (lane < i && !bad) {
      const float lx = __uint_as_float((uint32_t)gl);
      p = lx < ftau ? 0.0 : p_at((double)lx, sm.rm[lane], T, filt ? fs : sm.rs[lane]);
      q = (double)__uint_as_float((uint32_t)(gl >> 32));
    }
    const double w = __shfl(prefix_weights(p, q, i), i, 64);
    if (lane == 0) {
      sm.u[0] = w;
      sm.flag = bad;
    }
    if (lane == i) {
      sm.u[1] = filt ? fs : sm.rs[i];
      sm.l0 = ftau;
    }
  }
  __syncthreads();
  double* out = P.rpart + ((int64_t)b * P.k + i) * P.CHr + c;
  if (uniform_i(sm.flag)) {  // the decision step reports the request as non-finite
    if (tid == 0) *out = 0.0;
    return;
  }
  const double w = sm.u[0], S = sm.u[1];
  const float m = sm.rm[i], tau = sm.l0;
  const double wS = w / S, cd = 1.4426950408889634074 / T;
  double acc;
  if (filt) {
    if (vec) acc = kr_stream_pipe<BF16, true>(P, lrow, qrow, y_lo, y_hi, (double)m, cd, wS, tab, first, tau);
    else acc = kr_stream<BF16, false, true>(P, lrow, qrow, y_lo, y_hi, (double)m, cd, wS, tab, tau);
  } else {
    if (vec) acc = kr_stream_pipe<BF16, false>(P, lrow, qrow, y_lo, y_hi, (double)m, cd, wS, tab, first, tau);
    else acc = kr_stream<BF16, false, false>(P, lrow, qrow, y_lo, y_hi, (double)m, cd, wS, tab, tau);
  }
  acc = block_sum_d(acc, sm);
  if (tid == 0) *out = acc;
}

// ===================================================================== KF
// Top-k / top-p thresholds (page "投机解码", section
// "接受规则为什么不改变分布": the target p is the one after the top-k /
// top-p sampling parameters).  One workgroup of kKF threads per row
// r <= k_b of a chain request that is stochastic and has a filter on; it
// writes the row's threshold tau (the kept ids are those with l >= tau) and
// its kept sum S' = sum over them of exp((l - m)/T), m the row max from the
// statistics pass's partials.
//
// Logits map to 32-bit keys that order like their values (-0 as +0, so
// equal logits share one key).  A threshold is found by a radix descent
// over the keys, most significant digit first (11, 11 and 10 bits), with a
// histogram of the digit in LDS per level:
//  - top-k counts keys; the k-th largest key lies in the first bin, from the
//    top, at which the count of keys at or above it reaches k;
//  - top-p adds the masses e = 2^((l - m) log2(e)/T) of the top-k set's keys
//    in 96-bit fixed point (integer parts of e 2^32 and of its fraction
//    2^32: exact up to 2^-64 per id, and independent of the order of the
//    atomic adds); the cut is the first group of equal logits, from the top,
//    at which the mass at or above it reaches top_p times the set's mass.
// Only the first level reads the row from memory: a second pass copies the
// keys that can still matter into LDS (top-k: every key in or above the
// first level's bin, which holds the whole top-k set; top-p alone: the keys
// of the bin the cut falls in, the mass above it being known), and the
// descent finishes there.  When those keys exceed the LDS list, every level
// reads the row again.  The kept sum is the fixed-point mass at or above the
// cut (exact up to the same truncation, whatever the order).
constexpr int kKF = 512;                 // threads of a thresholds workgroup
constexpr int kKFWaves = kKF / 64;
constexpr int kKFBins = 2048;
constexpr int kKFList = 8192;            // keys the LDS list holds
constexpr int kKFUnroll = 8;             // groups of 4 ids per step on unaligned rows

// Digit levels: shift and width.
__device__ __forceinline__ int kf_shift(int L) { return L == 0 ? 21 : (L == 1 ? 10 : 0); }
__device__ __forceinline__ int kf_width(int L) { return L == 2 ? 10 : 11; }
// Whether a key lies under the prefix of the levels above L.
__device__ __forceinline__ bool kf_under(uint32_t key, int L, uint32_t pre) {
  return L == 0 || (key >> (kf_shift(L) + kf_width(L))) == pre;
}
// Fixed-point values h 2^-32 + l 2^-64 (both parts may exceed 2^32 in a
// sum): comparison and subtraction after carrying l's high part into h.
__device__ __forceinline__ bool kf_ge(uint64_t h, uint64_t l, uint64_t nh, uint64_t nl) {
  h += l >> 32;
  l &= 0xFFFFFFFFull;
  return h > nh || (h == nh && l >= nl);
}
__device__ __forceinline__ void kf_sub(uint64_t& nh, uint64_t& nl, uint64_t ah, uint64_t al) {
  ah += al >> 32;
  al &= 0xFFFFFFFFull;
  if (nl >= al) {
    nl -= al;
    nh -= ah;
  } else {
    nl = nl + 0x100000000ull - al;
    nh -= ah + 1;
  }
}
__device__ __forceinline__ void kf_fix(double x, uint64_t& h, uint64_t& l) {
  x = fmin(fmax(x, 0.0), 4294967296.0) * 4294967296.0;  // a NaN becomes 0
  const double fh = floor(x);
  h = (uint64_t)fh;
  l = (uint64_t)floor((x - fh) * 4294967296.0);
}
__device__ __forceinline__ double kf_float(uint64_t h, uint64_t l) {
  return (double)h * 0x1p-32 + (double)l * 0x1p-64;
}

struct KFShared {
  uint64_t hh[kKFBins];   // per bin: integer parts of e 2^32 (top-p)
  uint64_t hl[kKFBins];   // per bin: counts (top-k) or fraction parts 2^32 (top-p)
  uint32_t list[kKFList];
  int nlist;
  uint64_t wh[kKFWaves], wl[kKFWaves];  // per wave: sums of its threads' bins
  uint64_t toth, totl;    // the histogram's total
  uint64_t ah, al;        // found bin: the sum of the bins above it
  uint64_t bh, bl;        // found bin: its own sum
  int digit;              // found bin (-1: none)
};

// One pass over the row's logits (LIST: over the keys in the LDS list):
// f(l) for each.  From memory each thread takes groups of consecutive ids
// (16 bytes: 8 bf16 or 4 fp32), kKFUnroll groups per step; in rows of whole
// aligned groups the next
// step's loads are in flight while the current step is processed (loads
// past the row re-read its first group and are not processed, so every load
// is unconditional).
template <bool BF16>
constexpr int kf_group() { return BF16 ? 8 : 4; }
template <bool BF16>
constexpr int kf_unroll() { return BF16 ? 4 : 8; }  // 64 or 128 bytes per thread per step
template <bool BF16, int U = kf_unroll<BF16>()>
struct KFRaw {
  u32x4 v[U];  // 8 bf16 or 4 fp32 logits per group
};
template <bool BF16, int U>
__device__ __forceinline__ void kf_issue(const Params& P, int64_t off, int base, KFRaw<BF16, U>& r) {
  constexpr int E = kf_group<BF16>();
#pragma unroll
  for (int g = 0; g < U; ++g) {
    int y0 = base + E * (g * kKF + (int)threadIdx.x);
    y0 = y0 < P.V ? y0 : 0;
    if constexpr (BF16) r.v[g] = *(const u32x4*)((const uint16_t*)P.logits + off + y0);
    else r.v[g] = *(const u32x4*)((const float*)P.logits + off + y0);
  }
}
template <bool BF16, int U, typename F>
__device__ __forceinline__ void kf_fold(const KFRaw<BF16, U>& r, int base, int V, F&& f) {
  constexpr int E = kf_group<BF16>();
#pragma unroll
  for (int g = 0; g < U; ++g) {
    const int y0 = base + E * (g * kKF + (int)threadIdx.x);
    if (y0 < V) {
      const uint32_t w[4] = {r.v[g].x, r.v[g].y, r.v[g].z, r.v[g].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (BF16) {
          f(__uint_as_float(w[i] << 16));
          f(__uint_as_float(w[i] & 0xffff0000u));
        } else {
          f(__uint_as_float(w[i]));
        }
      }
    }
  }
}
// U: groups per thread per step (loads in flight).
template <bool BF16, int U = kf_unroll<BF16>(), typename F>
__device__ __forceinline__ void kf_pass_mem(const Params& P, int64_t row, F&& f) {
  const int tid = threadIdx.x;
  const int V = P.V;
  const int64_t off = row * P.lstride;
  constexpr int E = kf_group<BF16>();
  constexpr int step = E * kKF * U;
  if (P.aligned && (V % E) == 0) {
    KFRaw<BF16, U> a, b;
    kf_issue<BF16, U>(P, off, 0, a);
#pragma unroll 1
    for (int base = 0;;) {
      kf_issue<BF16, U>(P, off, base + step, b);
      kf_fold<BF16, U>(a, base, V, f);
      base += step;
      if (base >= V) break;
      kf_issue<BF16, U>(P, off, base + step, a);
      kf_fold<BF16, U>(b, base, V, f);
      base += step;
      if (base >= V) break;
    }
    return;
  }
  constexpr int sstep = 4 * kKF * kKFUnroll;
#pragma unroll 1
  for (int base = 0; base < V; base += sstep) {
    float l[kKFUnroll][4];
#pragma unroll
    for (int g = 0; g < kKFUnroll; ++g) {
      const int y0 = base + 4 * (g * kKF + tid);
#pragma unroll
      for (int i = 0; i < 4; ++i) l[g][i] = (y0 + i < V) ? load_logit<BF16>(P, row, y0 + i) : 0.f;
    }
#pragma unroll
    for (int g = 0; g < kKFUnroll; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (base + 4 * (g * kKF + tid) + i < V) f(l[g][i]);
  }
}
template <bool BF16, bool LIST, typename F>
__device__ __forceinline__ void kf_pass(const Params& P, int64_t row, const KFShared& s, F&& f) {
  if (LIST) {
    const int n = min(s.nlist, kKFList);
    for (int i = (int)threadIdx.x; i < n; i += kKF) f(kf_val(s.list[i]));
    return;
  }
  kf_pass_mem<BF16>(P, row, f);
}

__device__ __forceinline__ void kf_clear(KFShared& s) {
  for (int i = threadIdx.x; i < kKFBins; i += kKF) {
    s.hh[i] = 0;
    s.hl[i] = 0;
  }
  __syncthreads();
}

// The first bin from the top of a complete histogram of `nbins` bins at
// which the sum of the bins at or above it reaches (nh, nl) (a normalised
// fixed-point value, or a count in nl; with frac > 0 the need is frac times
// the histogram's total plus (xh, xl), the mass of the ids left out of the
// histogram, instead): s.digit, s.ah/al (bins above), s.bh/bl (the bin) and
// s.toth/totl.  Every thread calls it after the barrier that
// ends the histogram's pass; it ends with a barrier.  Thread t owns bins
// [t per, (t + 1) per); the sums of the bins above a thread's come from a
// suffix scan within its wave and the totals of the waves above.
template <bool MASS>
__device__ __forceinline__ void kf_find(KFShared& s, int nbins, uint64_t& nh, uint64_t& nl, float frac,
                                        uint64_t xh = 0, uint64_t xl = 0) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = nbins / kKF;
  uint64_t sh = 0, sl = 0;
  for (int j = 0; j < per; ++j) {
    if (MASS) sh += s.hh[tid * per + j];
    sl += s.hl[tid * per + j];
  }
  uint64_t ih = sh, il = sl;  // sums over the wave's lanes >= lane
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t vh = __shfl_down(ih, o, 64), vl = __shfl_down(il, o, 64);
    if (lane + o < 64) {
      ih += vh;
      il += vl;
    }
  }
  if (lane == 0) {
    s.wh[wave] = ih;
    s.wl[wave] = il;
  }
  if (tid == 0) s.digit = -1;
  __syncthreads();
  uint64_t rh = ih - sh, rl = il - sl, th = 0, tl = 0;
  for (int w = 0; w < kKFWaves; ++w) {
    const uint64_t a = s.wh[w], b = s.wl[w];
    th += a;
    tl += b;
    if (w > wave) {
      rh += a;
      rl += b;
    }
  }
  if (frac > 0.f) kf_fix((double)frac * kf_float(th + xh, tl + xl), nh, nl);
  for (int j = per - 1; j >= 0; --j) {
    const uint64_t ph = rh, pl = rl;
    const uint64_t bh = MASS ? s.hh[tid * per + j] : 0, bl = s.hl[tid * per + j];
    rh += bh;
    rl += bl;
    if (!kf_ge(ph, pl, nh, nl) && kf_ge(rh, rl, nh, nl)) {
      s.digit = tid * per + j;
      s.ah = ph;
      s.al = pl;
      s.bh = bh;
      s.bl = bl;
    }
  }
  if (tid == 0) {
    s.toth = th;
    s.totl = tl;
  }
  __syncthreads();
}

// Mass of a key's logit, in fixed point.
__device__ __forceinline__ void kf_mass(float l, double md, double cd, const double* tab, uint64_t& h, uint64_t& lo) {
  kf_fix(exp2_f64_nonpos(((double)l - md) * cd, tab), h, lo);
}

// Radix descent over the keys >= kmin, from memory or from the LDS list
// (LIST): the count descent (MASS false)
// finds the key at which the count from the top reaches (nh, nl); the mass
// descent finds the group at which the mass from the top reaches its need
// (frac > 0: frac times the set's mass), adding the masses above the found
// group, and the group's own, to (ch, cl).  Returns the key (0: not found).
// It starts at level L0 under the prefix pre0 of the levels above (keys all
// under it).  A widened bf16 logit's key has its low 16 bits set by its
// sign, so for bf16 the second level's prefix is already one logit.
template <bool BF16, bool LIST, bool MASS>
__device__ __forceinline__ uint32_t kf_descent(const Params& P, int64_t row, KFShared& s, const double* tab, double md, double cd,
                               uint32_t kmin, uint64_t nh, uint64_t nl, float frac, uint64_t& ch, uint64_t& cl,
                               int L0 = 0, uint32_t pre0 = 0) {
  uint32_t pre = pre0;
  for (int L = L0; L < 3; ++L) {
    kf_clear(s);
    const int sh = kf_shift(L);
    const uint32_t mask = (1u << kf_width(L)) - 1u;
    kf_pass<BF16, LIST>(P, row, s, [&](float l) {
      const uint32_t key = kf_key(l);
      if (key >= kmin && kf_under(key, L, pre)) {
        const int d = (int)((key >> sh) & mask);
        if (MASS) {
          uint64_t h, lo;
          kf_mass(l, md, cd, tab, h, lo);
          atomicAdd((unsigned long long*)&s.hh[d], (unsigned long long)h);
          atomicAdd((unsigned long long*)&s.hl[d], (unsigned long long)lo);
        } else {
          atomicAdd((unsigned long long*)&s.hl[d], 1ull);
        }
      }
    });
    __syncthreads();
    kf_find<MASS>(s, 1 << kf_width(L), nh, nl, L == 0 ? frac : 0.f);
    const int d = s.digit;
    if (d < 0) return 0;  // only for rows the decision step reports as non-finite
    kf_sub(nh, nl, s.ah, s.al);
    ch += s.ah;
    cl += s.al;
    pre = (pre << kf_width(L)) | (uint32_t)d;
    if (L == 2 || (BF16 && L == 1)) {
      ch += s.bh;
      cl += s.bl;
      if (L == 1) return (pre << 10) | (((pre >> 21) & 1u) ? 0u : 0x3FFu);
    }
  }
  return pre;
}

// Copy the row's keys with kf_key(l) in [lo, hi] into the LDS list (one
// atomic per wave for the positions).
template <bool BF16>
__device__ __forceinline__ void kf_collect(const Params& P, int64_t row, KFShared& s, uint32_t lo, uint32_t hi) {
  if (threadIdx.x == 0) s.nlist = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  kf_pass<BF16, false>(P, row, s, [&](float l) {
    const uint32_t key = kf_key(l);
    const bool take = key >= lo && key <= hi;
    const uint64_t mask = __ballot(take);
    if (mask) {
      const int leader = __builtin_ctzll(mask);
      int base = 0;
      if (lane == leader) base = atomicAdd(&s.nlist, __popcll(mask));
      base = __shfl(base, leader, 64);
      if (take) {
        const int i = base + __popcll(mask & ((1ull << lane) - 1ull));
        if (i < kKFList) s.list[i] = key;
      }
    }
  });
  __syncthreads();
}

struct KFRow {
  KFShared s;
  double tab[64];  // 2^(j/64)
  float red_m[kKFWaves];
  uint64_t red_h[kKFWaves], red_l[kKFWaves];
  uint32_t kx0;    // top-p alone: key of the lower bound on the cut (0: none)
};

// Block sums of per-thread fixed-point parts; every thread gets them.
__device__ __forceinline__ void kf_block_sum(uint64_t& h, uint64_t& l, uint64_t* red_h, uint64_t* red_l) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int o = 32; o > 0; o >>= 1) {
    h += __shfl_xor(h, o, 64);
    l += __shfl_xor(l, o, 64);
  }
  if (lane == 0) {
    red_h[wave] = h;
    red_l[wave] = l;
  }
  __syncthreads();
  h = l = 0;
  for (int i = 0; i < kKFWaves; ++i) {
    h += red_h[i];
    l += red_l[i];
  }
  __syncthreads();  // the per-wave sums may be reused
}

// Full key of the 16-bit key k of a widened bf16 logit (its low 16 bits
// follow from its sign).
__device__ __forceinline__ uint32_t kf_key16_full(uint32_t k) { return (k << 16) | ((k & 0x8000u) ? 0u : 0xFFFFu); }

// Top-p alone: the cut of row `row` and the mass at or above it (ch, cl);
// 0 for a row with no finite cut (non-finite rows).
// A lower bound on the cut from the statistics pass: the ids below x0 carry
// at most V 2^((x0 - m) cd) = (1 - tp) S / 4 of the mass, S the row's sum
// from the partials (within 1e-6 of the total), so the cut lies at or
// above x0.  Those ids only add to the total whose top_p fraction is the
// need: their masses are summed in registers and only the others are
// histogrammed.  bf16 rows whose keys from the bound to the max span at most
// kKFBins logit values count each value instead (a value's mass is its
// count times the mass of one) and find the cut in that table, with no
// second pass over the row.  Every way sums the same integers as the plain
// descent (the need comes from the same total), so it finds the same cut
// and kept mass; when the histogrammed mass cannot reach the need, the row
// is taken again with every id in the histogram.
template <bool BF16>
__device__ __forceinline__ uint32_t kf_top_p(const Params& P, int64_t row, KFRow& w, double md, double cd, float tp,
                                             uint64_t& ch, uint64_t& cl) {
  KFShared& s = w.s;
  const double* tab = w.tab;
  const int tid = threadIdx.x;
  if (tid < 64) {
    double sd = 0.0;
    if (tid < P.Q) {
      const Partial& pt = P.part[row * P.CPR + tid];
      const double ps = __longlong_as_double((long long)pt.s);
      const float pm = __uint_as_float((uint32_t)pt.m_amax);
      if (pm != -INFINITY) sd = ps * exp2_f64_nonpos(((double)pm - md) * cd, tab);
    }
    sd = wave_sum_d(sd);
    if (tid == 0) {
      const double x0 = md + log2(0.25 * (1.0 - (double)tp) * sd / (double)P.V) / cd;
      const float xf = (float)(x0 - fabs(x0) * 0x1p-20 - 0x1p-100);  // at or below x0
      w.kx0 = (sd > 0.0 && fabs(x0) < 1e30 && fabsf(xf) < 1e30f) ? kf_key(xf) : 0u;
    }
  }
  __syncthreads();
  uint32_t kx = w.kx0;
  uint64_t xh = 0, xl = 0;  // mass of the ids left out of the histogram
  uint64_t nh = 0, nl = 0;
  if constexpr (BF16) {
    const uint32_t k16hi = kf_key((float)md) >> 16;
    const uint32_t span = (uint32_t)kKFBins - 1u;
    const uint32_t k16lo = max(kx >> 16, k16hi >= span ? k16hi - span : 0u);
    if (kx != 0u) {
      uint32_t* cnt = s.list;  // counts of the values k16lo + i
      for (int i = tid; i < kKFBins; i += kKF) cnt[i] = 0u;
      __syncthreads();
      kf_pass<BF16, false>(P, row, s, [&](float l) {
        const uint32_t k = (kf_key(l) >> 16) - k16lo;  // wraps for keys below the table
        if (k < (uint32_t)kKFBins) {
          atomicAdd(&cnt[k], 1u);
        } else {
          uint64_t h, lo;
          kf_mass(l, md, cd, tab, h, lo);
          xh += h;
          xl += lo;
        }
      });
      __syncthreads();
      for (int i = tid; i < kKFBins; i += kKF) {
        const uint32_t c = cnt[i];
        uint64_t h = 0, lo = 0;
        if (c) kf_mass(kf_val(kf_key16_full(k16lo + (uint32_t)i)), md, cd, tab, h, lo);
        s.hh[i] = h * c;
        s.hl[i] = lo * c;
      }
      kf_block_sum(xh, xl, w.red_h, w.red_l);  // its barriers also complete the table
      kf_find<true>(s, kKFBins, nh, nl, tp, xh, xl);
      if (s.digit >= 0) {
        ch = s.ah + s.bh;
        cl = s.al + s.bl;
        return kf_key16_full(k16lo + (uint32_t)s.digit);
      }
      xh = xl = 0;
      nh = nl = 0;
    }
  }
  // first level of the masses from memory, the ids below the bound apart
  for (;;) {
    kf_clear(s);
    kf_pass<BF16, false>(P, row, s, [&](float l) {
      const uint32_t key = kf_key(l);
      uint64_t h, lo;
      kf_mass(l, md, cd, tab, h, lo);
      if (key >= kx) {
        atomicAdd((unsigned long long*)&s.hh[key >> 21], (unsigned long long)h);
        atomicAdd((unsigned long long*)&s.hl[key >> 21], (unsigned long long)lo);
      } else {
        xh += h;
        xl += lo;
      }
    });
    kf_block_sum(xh, xl, w.red_h, w.red_l);  // its barriers also complete the histogram
    kf_find<true>(s, kKFBins, nh, nl, tp, xh, xl);
    if (s.digit >= 0 || kx == 0u) break;
    kx = 0u;  // the bound did not hold: again with every id in the histogram
    xh = xl = 0;
    nh = nl = 0;
  }
  const int d = s.digit;
  if (d < 0) return 0u;
  kf_sub(nh, nl, s.ah, s.al);
  const uint64_t ah = s.ah, al = s.al;
  // the bin's keys to the list; the list's counter tells whether they fit
  kf_collect<BF16>(P, row, s, (uint32_t)d << 21, ((uint32_t)d << 21) | 0x1FFFFFu);
  if (s.nlist <= kKFList) {
    ch = ah;
    cl = al;
    // the need left within the bin, from the second level
    return kf_descent<BF16, true, true>(P, row, s, tab, md, cd, 0u, nh, nl, 0.f, ch, cl, 1, (uint32_t)d);
  }
  ch = cl = 0;
  return kf_descent<BF16, false, true>(P, row, s, tab, md, cd, 0u, 0, 0, tp, ch, cl);
}

// The thresholds of filtered row `row` (temperature Tf, top-k tk, top-p tp)
// from passes over the row.
template <bool BF16>
__device__ __forceinline__ void kf_row(const Params& P, int64_t row, float Tf, int tk, float tp, KFRow& w) {
  KFShared& s = w.s;
  double* tab = w.tab;
  float* red_m = w.red_m;
  uint64_t *red_h = w.red_h, *red_l = w.red_l;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool use_k = tk > 0 && tk < P.V, use_p = tp > 0.f && tp < 1.f;
  // the row max, from the statistics pass's partials
  float m = -INFINITY;
  if (tid < P.Q) m = __uint_as_float((uint32_t)P.part[row * P.CPR + tid].m_amax);
  if (tid < 64) {
    m = wave_max(m);
    if (lane == 0) red_m[0] = m;
    tab[tid] = exp2((double)tid / 64.0);
  }
  kf_clear(s);
  const double md = (double)red_m[0], cd = 1.4426950408889634074 / (double)Tf;
  // first level, from memory: top-k counts, or top-p masses
  uint64_t ch = 0, cl = 0;  // mass above the current prefix (top-p)
  uint64_t nh = 0, nl = 0;
  bool listed = false;
  uint32_t kmin = 0;
  if (use_k) {
    // 32-bit counters (in the list's first entries) for the pass, then widened
    for (int i = tid; i < kKFBins; i += kKF) s.list[i] = 0;
    __syncthreads();
    kf_pass<BF16, false>(P, row, s, [&](float l) { atomicAdd(&s.list[kf_key(l) >> 21], 1u); });
    __syncthreads();
    for (int i = tid; i < kKFBins; i += kKF) s.hl[i] = s.list[i];
    __syncthreads();
    nl = (uint64_t)tk;
    kf_find<false>(s, kKFBins, nh, nl, 0.f);
    const int d = s.digit < 0 ? 0 : s.digit;  // always found: the counts reach k
    // every key in or above bin d: the top-k set and the rest of bin d
    const uint64_t n = (s.ah + s.al) + (s.bh + s.bl);
    if (n <= (uint64_t)kKFList) {
      kf_collect<BF16>(P, row, s, (uint32_t)d << 21, 0xFFFFFFFFu);
      listed = true;
      kmin = kf_descent<BF16, true, false>(P, row, s, tab, md, cd, 0u, 0, (uint64_t)tk, 0.f, ch, cl);
    } else {
      kmin = kf_descent<BF16, false, false>(P, row, s, tab, md, cd, 0u, 0, (uint64_t)tk, 0.f, ch, cl);
    }
    ch = cl = 0;
  }
  uint32_t kcut = kmin;
  double S;
  if (use_p) {
    uint32_t cut;
    if (use_k) {
      cut = listed ? kf_descent<BF16, true, true>(P, row, s, tab, md, cd, kmin, 0, 0, tp, ch, cl)
                   : kf_descent<BF16, false, true>(P, row, s, tab, md, cd, kmin, 0, 0, tp, ch, cl);
    } else {
      cut = kf_top_p<BF16>(P, row, w, md, cd, tp, ch, cl);
    }
    if (cut) {
      kcut = cut;
      S = kf_float(ch + (cl >> 32), cl & 0xFFFFFFFFull);
    } else {
      S = __builtin_nan("");  // only for rows the decision step reports as non-finite
    }
  } else {
    // top-k alone: the fixed-point mass of the keys >= kmin
    uint64_t th = 0, tl = 0;
    auto add = [&](float l) {
      if (kf_key(l) >= kmin) {
        uint64_t h, lo;
        kf_mass(l, md, cd, tab, h, lo);
        th += h;
        tl += lo;
      }
    };
    if (listed) kf_pass<BF16, true>(P, row, s, add);
    else kf_pass<BF16, false>(P, row, s, add);
    for (int o = 32; o > 0; o >>= 1) {
      th += __shfl_xor(th, o, 64);
      tl += __shfl_xor(tl, o, 64);
    }
    if (lane == 0) {
      red_h[wave] = th;
      red_l[wave] = tl;
    }
    __syncthreads();
    th = tl = 0;
    for (int w = 0; w < kKFWaves; ++w) {
      th += red_h[w];
      tl += red_l[w];
    }
    S = kf_float(th + (tl >> 32), tl & 0xFFFFFFFFull);
  }
  if (tid == 0) {
    P.filt[row].s = S;
    P.filt[row].tau = kcut ? kf_val(kcut) : -INFINITY;
  }
}


// ------------------------------------------------ thresholds from candidates
// The top-k rows whose statistics segments published candidates: one
// workgroup of kKC threads per row, in four steps.
//  1. g', the k-th largest of the published keys (see the top-k candidates
//     of the statistics pass; 0 when fewer than k are published).
//  2. The groups to read: the published groups >= g', and every group of
//     the lanes whose second key is >= g'.
//  3. Their logits >= g': exactly the row's logits >= g', a set that holds
//     every logit >= tau, so the k-th largest of the set is tau and the
//     masses at or above tau are the row's.
//  4. tau, the top-p cut (the first group of equal logits from the top at
//     which the mass reaches top_p times the top-k set's mass) and the kept
//     sum S' (the fixed-point mass at or above the cut).  These are integer
//     sums, whatever the method or the order, so they equal the row passes'.
//     Sets of up to kKC logits are settled by ranking each key against the
//     others, a key per thread; larger ones by radix descents over 8-bit
//     digits.
// A row whose groups or logits exceed the LDS takes the row passes.
constexpr int kKC = kKF;          // threads of a candidate-thresholds workgroup
constexpr int kDig = 256;         // digits of a radix level (thread t < kDig owns digit t)
constexpr int kKCList = 4096;     // logits >= g' the LDS holds
constexpr int kKCGroups = 1024;   // groups to read the LDS holds
constexpr int kKCBatch = 4;       // loads in flight per thread
constexpr int kKCPub = 1024;      // lane records the LDS holds (more: read from memory at each use)
struct KCShared {
  u32x4 pub[kKCPub];              // the row's lane records
  uint32_t list[kKCList + 4];     // logits' keys (then zeros past them for the ranking)
  uint32_t grp[kKCGroups];        // ids of the groups to read
  uint64_t hh[kKC + 4], hl[kKC + 4];  // per digit: mass (integer parts, fraction parts) or counts (hl);
                                      // ranked selection: per key (zeros past the keys)
  uint64_t wh[kKC / 64], wl[kKC / 64];
  double tab[64];
  uint64_t ah, al, bh, bl;        // found digit: sums of the digits above it, and its own
  uint32_t cnt[kDig];             // per digit: counts (selection of g')
  uint32_t cw[kKC / 64];
  int above;                      // found digit: count of the digits above it
  uint32_t tau, cut;              // ranked selection: tau and the cut (0: none)
  uint64_t cut_h, cut_l;          // ... and the mass at or above the cut
  int rg[kKC], re[kKC];           // ranked selection: partial counts per thread
  uint64_t ps[6][kKC];            // ... and partial mass sums (total, at or above, above; two parts each)
  int digit;
  int nlist, ngrp;
  float m;
};

// One level of a descent: the first digit from the top at which the sum of
// the digits at or above it reaches (nh, nl) (with frac > 0: frac times the
// histogram's total).  Thread t owns digit t.  Called by every thread after
// the barrier that ends the histogram; ends with a barrier.
template <bool MASS>
__device__ __forceinline__ void kc_find(KCShared& s, uint64_t& nh, uint64_t& nl, float frac) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool owner = tid < kDig;
  const uint64_t bh = (MASS && owner) ? s.hh[tid] : 0, bl = owner ? s.hl[tid] : 0;
  uint64_t ih = bh, il = bl;  // sums over the wave's lanes >= lane
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t vh = __shfl_down(ih, o, 64), vl = __shfl_down(il, o, 64);
    if (lane + o < 64) {
      ih += vh;
      il += vl;
    }
  }
  if (lane == 0) {
    s.wh[wave] = ih;
    s.wl[wave] = il;
  }
  __syncthreads();
  uint64_t ah = ih - bh, al = il - bl, th = 0, tl = 0;
#pragma unroll
  for (int w = 0; w < kKC / 64; ++w) {
    th += s.wh[w];
    tl += s.wl[w];
    if (w > wave) {
      ah += s.wh[w];
      al += s.wl[w];
    }
  }
  if (frac > 0.f) kf_fix((double)frac * kf_float(th, tl), nh, nl);
  if (owner && !kf_ge(ah, al, nh, nl) && kf_ge(ah + bh, al + bl, nh, nl)) {
    s.digit = tid;
    s.ah = ah;
    s.al = al;
    s.bh = bh;
    s.bl = bl;
  }
  __syncthreads();
}

// Radix descent over the listed keys >= kmin, 8 bits a level: the count
// descent (MASS false) finds the key at which the count from the top reaches
// (nh, nl); the mass descent finds the group at which the mass from the top
// reaches its need (frac > 0: frac times the set's mass), adding the masses
// of the keys above it and of the group itself to (ch, cl).  Returns the key
// (0: not found).  bf16 logits' keys end in 16 bits that the upper 16 fix (0
// for a sign bit of 1, else all ones), so two levels settle them.
template <bool BF16, bool MASS>
__device__ __forceinline__ uint32_t kc_descent(KCShared& s, int n, double md, double cd, uint32_t kmin, uint64_t nh,
                                               uint64_t nl, float frac, uint64_t& ch, uint64_t& cl) {
  const int tid = threadIdx.x;
  constexpr int LV = BF16 ? 2 : 4;
  uint32_t pre = 0;
  for (int L = 0; L < LV; ++L) {
    const int sh = 24 - 8 * L;
    if (tid < kDig) {
      s.hh[tid] = 0;
      s.hl[tid] = 0;
    }
    if (tid == 0) s.digit = -1;
    __syncthreads();
    for (int i = tid; i < n; i += kKC) {
      const uint32_t key = s.list[i];
      if (key >= kmin && (L == 0 || (key >> (sh + 8)) == pre)) {
        const int d = (int)((key >> sh) & 255u);
        if (MASS) {
          uint64_t h, lo;
          kf_mass(kf_val(key), md, cd, s.tab, h, lo);
          atomicAdd((unsigned long long*)&s.hh[d], (unsigned long long)h);
          atomicAdd((unsigned long long*)&s.hl[d], (unsigned long long)lo);
        } else {
          atomicAdd((unsigned long long*)&s.hl[d], 1ull);
        }
      }
    }
    __syncthreads();
    kc_find<MASS>(s, nh, nl, L == 0 ? frac : 0.f);
    const int d = s.digit;
    if (d < 0) return 0;  // only for rows the decision step reports as non-finite
    kf_sub(nh, nl, s.ah, s.al);
    ch += s.ah;
    cl += s.al;
    if (L == LV - 1) {
      ch += s.bh;
      cl += s.bl;
    }
    pre = (pre << 8) | (uint32_t)d;
  }
  if (BF16) pre = (pre << 16) | ((pre & 0x8000u) ? 0u : 0xFFFFu);
  return pre;
}

// Lane record i of the row: from LDS when the records were cached there.
__device__ __forceinline__ u32x4 kc_pub(const KCShared& s, const u32x4* pub, int npub, int i) {
  if (i >= npub) return u32x4{0u, 0u, 0u, 0u};
  return npub <= kKCPub ? s.pub[i] : pub[i];
}

// The k-th largest of the row's published keys with its lower 16 bits
// cleared -- the key itself for bf16 logits, whose keys' lower 16 bits the
// upper ones fix, and at most it for fp32 logits -- or 0 when fewer than k
// keys are published: a radix descent over two 8-bit digits with 32-bit
// counts.
template <bool BF16>
__device__ __forceinline__ uint32_t kc_kth_pub(KCShared& s, const u32x4* pub, int npub, int k) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int LV = 2;
  uint32_t pre = 0;
  int need = k;
  for (int L = 0; L < LV; ++L) {
    const int sh = 24 - 8 * L;
    if (tid < kDig) s.cnt[tid] = 0;
    if (tid == 0) s.digit = -1;
    __syncthreads();
    for (int i0 = 0; i0 < npub; i0 += kKC * kKCBatch) {
      u32x4 e[kKCBatch];
#pragma unroll
      for (int u = 0; u < kKCBatch; ++u) e[u] = kc_pub(s, pub, npub, i0 + u * kKC + tid);
#pragma unroll
      for (int u = 0; u < kKCBatch; ++u) {
        const uint32_t ks[2] = {e[u].x, e[u].z};
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const bool on = ks[q] != 0u && (L == 0 || (ks[q] >> (sh + 8)) == pre);
          if (on) atomicAdd(&s.cnt[(ks[q] >> sh) & 255u], 1u);
        }
      }
    }
    __syncthreads();
    const uint32_t c = tid < kDig ? s.cnt[tid] : 0u;
    uint32_t in = c;  // counts of the wave's digits >= this one
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t v = (uint32_t)__shfl_down((int)in, o, 64);
      if (lane + o < 64) in += v;
    }
    if (lane == 0) s.cw[wave] = in;
    __syncthreads();
    uint32_t above = in - c;
#pragma unroll
    for (int w = 0; w < kKC / 64; ++w)
      if (w > wave) above += s.cw[w];
    if (tid < kDig && above < (uint32_t)need && above + c >= (uint32_t)need) {
      s.digit = tid;
      s.above = (int)above;
    }
    __syncthreads();
    const int d = s.digit;
    if (d < 0) return 0u;
    need -= s.above;
    pre = (pre << 8) | (uint32_t)d;
  }
  return BF16 ? (pre << 16) | ((pre & 0x8000u) ? 0u : 0xFFFFu) : pre << 16;
}

__device__ __forceinline__ void wave_sum_u64(uint64_t& h, uint64_t& l) {
  for (int o = 32; o > 0; o >>= 1) {
    h += __shfl_xor(h, o, 64);
    l += __shfl_xor(l, o, 64);
  }
}

// Step 4 for n <= kKC listed keys, by ranking: every key is compared with
// every listed key, the comparisons split over all threads (thread t takes
// key t % Kp and part t / Kp of the others, Kp = n rounded up to a multiple
// of 64) and the parts summed in LDS.  tau is the key with fewer than k
// keys above it and at least k at or above it; each key of the top-k set
// sums the masses above it and at or above it, and the cut is the key whose
// mass at or above reaches the need while the mass above does not.  kcut = 0
// (and S a NaN under top-p) for a row without them, as the descents give.
// The list must hold zeros in [n, n + 4).
__device__ __forceinline__ void kc_rank(KCShared& s, int n, int tk, bool use_p, float tp, double md, double cd,
                                        uint32_t& kcut, double& Sum) {
  const int tid = threadIdx.x;
  const int Kp = (n + 63) & ~63;
  const int Pn = kKC / Kp;                 // parts of the comparisons per key
  const int i = tid % Kp, part = tid / Kp;
  const bool act = part < Pn;
  const int n4 = (n + 3) >> 2;             // groups of 4 keys (zeros past n)
  const int q0 = act ? part * n4 / Pn : 0, q1 = act ? (part + 1) * n4 / Pn : 0;
  const uint32_t v = (act && i < n) ? s.list[i] : 0u;
  int g = 0, e = 0;
  for (int q = q0; q < q1; ++q) {
    const u32x4 k4 = *(const u32x4*)&s.list[4 * q];  // zeros count nowhere (v >= 1)
    g += (int)(k4.x > v) + (int)(k4.y > v) + (int)(k4.z > v) + (int)(k4.w > v);
    e += (int)(k4.x >= v) + (int)(k4.y >= v) + (int)(k4.z >= v) + (int)(k4.w >= v);
  }
  s.rg[tid] = g;
  s.re[tid] = e;
  if (tid == 0) {
    s.tau = 0u;
    s.cut = 0u;
  }
  __syncthreads();
  const bool own = part == 0 && i < n;  // the thread that settles key i
  if (own) {
    for (int p = 1; p < Pn; ++p) {
      g += s.rg[p * Kp + i];
      e += s.re[p * Kp + i];
    }
    if (g < tk && tk <= e) s.tau = v;  // every such thread holds the same key
  }
  __syncthreads();
  const uint32_t tau = s.tau;
  if (tau == 0u) {
    kcut = 0;
    Sum = use_p ? __builtin_nan("") : 0.0;
    return;
  }
  if (tid < Kp + 4) {
    uint64_t h = 0, l = 0;
    if (tid < n && s.list[tid] >= tau) kf_mass(kf_val(s.list[tid]), md, cd, s.tab, h, l);
    s.hh[tid] = h;  // zeros past n
    s.hl[tid] = l;
  }
  __syncthreads();
  uint64_t th = 0, tl = 0, ch = 0, cl = 0, ah = 0, al = 0;
  for (int q = q0; q < q1; ++q) {
    const u32x4 k4 = *(const u32x4*)&s.list[4 * q];
    const uint32_t kq[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint64_t hj = s.hh[4 * q + u], lj = s.hl[4 * q + u];
      th += hj;
      tl += lj;
      if (kq[u] >= v) {
        ch += hj;
        cl += lj;
      }
      if (kq[u] > v) {
        ah += hj;
        al += lj;
      }
    }
  }
  s.ps[0][tid] = th;
  s.ps[1][tid] = tl;
  s.ps[2][tid] = ch;
  s.ps[3][tid] = cl;
  s.ps[4][tid] = ah;
  s.ps[5][tid] = al;
  __syncthreads();
  if (own) {
    for (int p = 1; p < Pn; ++p) {
      th += s.ps[0][p * Kp + i];
      tl += s.ps[1][p * Kp + i];
      ch += s.ps[2][p * Kp + i];
      cl += s.ps[3][p * Kp + i];
      ah += s.ps[4][p * Kp + i];
      al += s.ps[5][p * Kp + i];
    }
  }
  if (!use_p) {
    // the set's total, as summed by the thread of key 0
    th = s.ps[0][0];
    tl = s.ps[1][0];
    for (int p = 1; p < Pn; ++p) {
      th += s.ps[0][p * Kp];
      tl += s.ps[1][p * Kp];
    }
    kcut = tau;
    Sum = kf_float(th + (tl >> 32), tl & 0xFFFFFFFFull);
    return;
  }
  uint64_t nh, nl;
  kf_fix((double)tp * kf_float(th, tl), nh, nl);
  if (own && v >= tau && kf_ge(ch, cl, nh, nl) && !kf_ge(ah, al, nh, nl)) {
    s.cut = v;  // every such thread holds the same key and sums
    s.cut_h = ch;
    s.cut_l = cl;
  }
  __syncthreads();
  kcut = s.cut;
  Sum = kcut ? kf_float(s.cut_h + (s.cut_l >> 32), s.cut_l & 0xFFFFFFFFull) : __builtin_nan("");
}

// Appends x to arr for every lane of the wave with `take`, one atomic on the
// count *n per wave (positions past cap are counted, not written, so that
// the caller sees the overflow).  Every lane of the wave calls it.
__device__ __forceinline__ void wave_append(uint32_t* arr, int* n, int cap, bool take, uint32_t x) {
  const uint64_t m = __ballot(take);
  if (m == 0) return;
  const int leader = __builtin_ctzll(m);
  int base = 0;
  if ((int)(threadIdx.x & 63) == leader) base = atomicAdd(n, __popcll(m));
  base = __shfl(base, leader, 64);
  if (take) {
    const int p = base + lanes_below(m);
    if (p < cap) arr[p] = x;
  }
}

// The thresholds of top-k row `row` from its candidates; false (every
// thread alike, nothing written) when they do not fit the LDS.  rec holds
// the row's lane records when they fit the LDS cache (loaded by the caller
// ahead of its checks), pm the row's partial maxima.
template <bool BF16>
__device__ __forceinline__ bool kc_try(const Params& P, int64_t row, float Tf, int tk, float tp, uint64_t pm,
                                       const u32x4* rec, KCShared& s) {
  const int tid = threadIdx.x;
  const int Q = P.Q;
  const bool use_p = tp > 0.f && tp < 1.f;
  const u32x4* pub = P.cand + row * Q * kWG;
  const int npub = Q * kWG;
  if (npub <= kKCPub)
#pragma unroll
    for (int j = 0; j < kKCPub / kKC; ++j)
      if (j * kKC + tid < npub) s.pub[j * kKC + tid] = rec[j];
  // wave 0: the row max from the partials
  if (tid < 64) {
    float m = tid < Q ? __uint_as_float((uint32_t)pm) : -INFINITY;
    m = wave_max(m);
    s.tab[tid] = exp2((double)tid / 64.0);
    if (tid == 0) {
      s.m = m;
      s.ngrp = 0;
      s.nlist = 0;
    }
  }
  // 1. g'
  const uint32_t g = kc_kth_pub<BF16>(s, pub, npub, tk);
  // 2. the groups to read
  for (int i0 = 0; i0 < npub; i0 += kKC * kKCBatch) {
    u32x4 e[kKCBatch];
#pragma unroll
    for (int u = 0; u < kKCBatch; ++u) e[u] = kc_pub(s, pub, npub, i0 + u * kKC + tid);
#pragma unroll
    for (int u = 0; u < kKCBatch; ++u) {
      const int i = i0 + u * kKC + tid;
      const int seg = i / kWG, t = i - seg * kWG;
      const bool both = e[u].z != 0u && e[u].z >= g;
      if (both) {
        // both of the lane's groups are >= g': every group of the lane
        const int s0 = (int)((int64_t)seg * P.nsub / Q), s1 = (int)((int64_t)(seg + 1) * P.nsub / Q);
        const int p = atomicAdd(&s.ngrp, s1 - s0);
        for (int sub = s0; sub < s1; ++sub)
          if (p + sub - s0 < kKCGroups) s.grp[p + sub - s0] = (uint32_t)(sub * kWG + t);
      }
      wave_append(s.grp, &s.ngrp, kKCGroups, !both && e[u].x != 0u && e[u].x >= g, e[u].y * kWG + t);
    }
  }
  __syncthreads();
  if (s.ngrp > kKCGroups) return false;
  {
    // 3. their logits >= g', kKCBatch loads of 16 bytes in flight per thread
    constexpr int EPV = BF16 ? 8 : 4;
    const int ng = s.ngrp;
    const int64_t off = row * P.lstride;
    for (int i0 = 0; i0 < ng * kVecPerThread; i0 += kKC * kKCBatch) {
      u32x4 v[kKCBatch];
      int e0[kKCBatch];
#pragma unroll
      for (int u = 0; u < kKCBatch; ++u) {
        const int i = i0 + u * kKC + tid;
        e0[u] = P.V;
        v[u] = u32x4{0u, 0u, 0u, 0u};
        if (i < ng * kVecPerThread) {
          const int gi = i / kVecPerThread, j = i - gi * kVecPerThread;
          const uint32_t gid = s.grp[gi];
          const int64_t e64 = (int64_t)(gid / kWG) * P.SUB + (int64_t)(j * kWG + (int)(gid % kWG)) * EPV;
          if (e64 < P.V) {
            e0[u] = (int)e64;
            if (P.aligned && e0[u] + EPV <= P.V)
              v[u] = BF16 ? *(const u32x4*)((const uint16_t*)P.logits + off + e0[u])
                          : *(const u32x4*)((const float*)P.logits + off + e0[u]);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kKCBatch; ++u) {
        float l[EPV];
        if (P.aligned && e0[u] + EPV <= P.V) {
          const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            if (BF16) {
              l[2 * h] = __uint_as_float(w[h] << 16);
              l[2 * h + 1] = __uint_as_float(w[h] & 0xffff0000u);
            } else {
              l[h] = __uint_as_float(w[h]);
            }
          }
        } else {
#pragma unroll
          for (int e = 0; e < EPV; ++e) l[e] = e0[u] + e < P.V ? load_logit<BF16>(P, row, e0[u] + e) : -INFINITY;
        }
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const uint32_t key = kf_key(l[e]);
          wave_append(s.list, &s.nlist, kKCList, e0[u] + e < P.V && key >= g, key);
        }
      }
    }
    __syncthreads();
  }
  if (s.nlist > kKCList) return false;
  // 4. tau, the cut and S'
  const int n = s.nlist;
  const double md = (double)s.m, cd = 1.4426950408889634074 / (double)Tf;
  uint32_t kcut = 0;
  double S = 0.0;
  if (n <= kKC) {
    if (tid < 4) s.list[n + tid] = 0u;
    __syncthreads();
    kc_rank(s, n, tk, use_p, tp, md, cd, kcut, S);
  } else {
    uint64_t ch = 0, cl = 0;
    const uint32_t kmin = kc_descent<BF16, false>(s, n, md, cd, 0u, 0, (uint64_t)tk, 0.f, ch, cl);
    ch = cl = 0;
    kcut = kmin;
    if (use_p) {
      const uint32_t cut = kc_descent<BF16, true>(s, n, md, cd, kmin, 0, 0, tp, ch, cl);
      kcut = cut;
      S = cut ? kf_float(ch + (cl >> 32), cl & 0xFFFFFFFFull) : __builtin_nan("");
    } else {
      // top-k alone: the fixed-point mass of the keys >= kmin
      const int lane = tid & 63, wave = tid >> 6;
      uint64_t th = 0, tl = 0;
      for (int i = tid; i < n; i += kKC) {
        const uint32_t key = s.list[i];
        if (key >= kmin) {
          uint64_t h, lo;
          kf_mass(kf_val(key), md, cd, s.tab, h, lo);
          th += h;
          tl += lo;
        }
      }
      wave_sum_u64(th, tl);
      if (lane == 0) {
        s.wh[wave] = th;
        s.wl[wave] = tl;
      }
      __syncthreads();
      th = tl = 0;
#pragma unroll
      for (int w = 0; w < kKC / 64; ++w) {
        th += s.wh[w];
        tl += s.wl[w];
      }
      S = kf_float(th + (tl >> 32), tl & 0xFFFFFFFFull);
    }
  }
  if (tid == 0) {
    P.filt[row].s = S;
    P.filt[row].tau = kcut ? kf_val(kcut) : -INFINITY;
  }
  return true;
}

// ------------------------------------------------ top-p from value counts
// bf16 rows filtered by top-p alone, in calls without top-k: a bf16 logit
// is one of 65536 bit patterns and equal logits have equal masses, so one
// pass counts each pattern (16-bit counters, two to a word: 128 KB of LDS)
// and the masses come from the counts: a value's mass is its count times
// the mass of one, the same integers as the sums id by id.  The total, the
// need and the cut then come from the table alone: the masses of chunks of
// 128 values in key order (16 lanes a chunk), the chunk of the cut by a scan
// over the chunks (one per thread), the value by a scan within it.  -0 is
// counted with +0 (one group of equal logits).  A count past 65535 carries
// into its neighbour; the counts then no longer add up to V and the row
// takes the passes over the row instead.
constexpr int kKTVals = 65536;
constexpr int kKTWords = kKTVals / 2;
constexpr int kKTChunk = kKTVals / kKF;  // values per chunk: one chunk per thread
static_assert(kKTChunk == 128 && kKF == 512, "a chunk is 16 lanes of 8 values; 4 chunks a wave");
struct KTShared {
  alignas(16) uint32_t tbl[kKTWords];    // counts of bit patterns 2i (low half) and 2i + 1
  uint64_t ph[kKF], pl[kKF];             // per chunk: mass (integer, fraction parts)
  uint64_t red_h[kKFWaves], red_l[kKFWaves];
  uint32_t red_c[kKFWaves];
  double tab[64];
  uint64_t ah, al;                       // chunk of the cut: mass of the chunks above it
  float m;
  int chunk;                             // chunk of the cut (-1: none)
};
// Bit pattern of the bf16 logit whose 16-bit key is k (keys order like the
// values: positive patterns follow the negative ones, which run backwards).
__device__ __forceinline__ uint32_t kt_raw(uint32_t k) { return k >= 0x8000u ? k - 0x8000u : 0xFFFFu - k; }
__device__ __forceinline__ uint32_t kt_count(const KTShared& t, uint32_t raw) {
  return (t.tbl[raw >> 1] >> ((raw & 1u) << 4)) & 0xFFFFu;
}

// Thresholds of bf16 row `row` under top-p tp alone from its value counts;
// false (nothing written) when a count overflowed.
__device__ __forceinline__ bool kt_row(const Params& P, int64_t row, float Tf, float tp, KTShared& t) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float m = -INFINITY;
  if (tid < P.Q) m = __uint_as_float((uint32_t)P.part[row * P.CPR + tid].m_amax);
  if (tid < 64) {
    m = wave_max(m);
    if (tid == 0) {
      t.m = m;
      t.chunk = -1;
    }
    t.tab[tid] = exp2((double)tid / 64.0);
  }
  for (int i = tid; i < kKTWords / 4; i += kKF) ((u32x4*)t.tbl)[i] = u32x4{0u, 0u, 0u, 0u};
  t.ph[tid] = 0;
  t.pl[tid] = 0;
  __syncthreads();
  const double md = (double)t.m, cd = 1.4426950408889634074 / (double)Tf;
  kf_pass_mem<true>(P, row, [&](float l) {
    const uint32_t raw = __float_as_uint(l) >> 16;
    atomicAdd(&t.tbl[raw >> 1], 1u << ((raw & 1u) << 4));
  });
  __syncthreads();
  if (tid == 0) {
    // -0 (pattern 0x8000, low half of word 0x4000) joins +0 (pattern 0)
    const uint32_t c = t.tbl[0x4000] & 0xFFFFu;
    t.tbl[0x4000] -= c;
    t.tbl[0] += c;
  }
  __syncthreads();
  // chunk masses: in pass j wave w takes the chunks 32 j + w + 8 g (g = 0..3,
  // so a band of populated chunks spreads over the waves), a group of 16
  // lanes per chunk, 8 consecutive values (one 16-byte word of counts) per
  // lane; a negative chunk's patterns run backwards, which a sum does not
  // see.  A wave with a populated value computes all its eight masses
  // without branches, so that their latencies overlap.
  uint32_t cnt = 0;
  for (int j = 0; j < kKF / (4 * kKFWaves); ++j) {
    const int kc = 4 * kKFWaves * j + wave + kKFWaves * (lane >> 4), part = lane & 15;
    const uint32_t k0 = (uint32_t)(kc * kKTChunk + 8 * part);  // keys k0 .. k0 + 7
    const uint32_t r0 = k0 >= 0x8000u ? k0 - 0x8000u : 0xFFF8u - k0;  // lowest pattern of the eight
    const u32x4 q = *(const u32x4*)&t.tbl[r0 >> 1];
    if (__ballot((q.x | q.y | q.z | q.w) != 0u) == 0ull) continue;
    const uint32_t wq[4] = {q.x, q.y, q.z, q.w};
    uint64_t sh = 0, sl = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t c = (wq[i >> 1] >> ((i & 1) << 4)) & 0xFFFFu;
      uint64_t h, lo;
      kf_mass(__uint_as_float((r0 + (uint32_t)i) << 16), md, cd, t.tab, h, lo);
      sh += h * c;
      sl += lo * c;
      cnt += c;
    }
    for (int o = 8; o > 0; o >>= 1) {
      sh += __shfl_xor(sh, o, 64);
      sl += __shfl_xor(sl, o, 64);
    }
    if (part == 0) {
      t.ph[kc] = sh;
      t.pl[kc] = sl;
    }
  }
  for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
  if (lane == 0) t.red_c[wave] = cnt;
  __syncthreads();  // also completes the chunks' masses
  cnt = 0;
  for (int w = 0; w < kKFWaves; ++w) cnt += t.red_c[w];
  if (cnt != (uint32_t)P.V) return false;  // every thread alike
  // the chunk of the cut: the first from the top at which the mass at or
  // above it reaches the need (chunk tid; the chunks above are tid + 1..)
  const uint64_t bh = t.ph[tid], bl = t.pl[tid];
  uint64_t ih = bh, il = bl;  // sums over the wave's lanes >= lane
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t vh = __shfl_down(ih, o, 64), vl = __shfl_down(il, o, 64);
    if (lane + o < 64) {
      ih += vh;
      il += vl;
    }
  }
  if (lane == 0) {
    t.red_h[wave] = ih;
    t.red_l[wave] = il;
  }
  __syncthreads();
  uint64_t rh = ih - bh, rl = il - bl, th = 0, tl = 0;
  for (int w = 0; w < kKFWaves; ++w) {
    th += t.red_h[w];
    tl += t.red_l[w];
    if (w > wave) {
      rh += t.red_h[w];
      rl += t.red_l[w];
    }
  }
  uint64_t nh, nl;
  kf_fix((double)tp * kf_float(th, tl), nh, nl);
  if (!kf_ge(rh, rl, nh, nl) && kf_ge(rh + bh, rl + bl, nh, nl)) {
    t.chunk = tid;
    t.ah = rh;
    t.al = rl;
  }
  __syncthreads();
  const int c = t.chunk;
  if (wave == 0) {
    uint32_t cut = 0;
    uint64_t ch = 0, cl = 0;
    if (c >= 0) {
      // lane j: keys 128 c + 2 j and 128 c + 2 j + 1 (the higher one first)
      const uint32_t k0 = (uint32_t)(c * kKTChunk + 2 * lane);
      const uint32_t p0 = kt_raw(k0), p1 = kt_raw(k0 + 1u);
      const uint32_t c0 = kt_count(t, p0), c1 = kt_count(t, p1);
      uint64_t h0 = 0, l0 = 0, h1 = 0, l1 = 0;
      if (c0) {
        kf_mass(__uint_as_float(p0 << 16), md, cd, t.tab, h0, l0);
        h0 *= c0;
        l0 *= c0;
      }
      if (c1) {
        kf_mass(__uint_as_float(p1 << 16), md, cd, t.tab, h1, l1);
        h1 *= c1;
        l1 *= c1;
      }
      uint64_t sh = h0 + h1, sl = l0 + l1;  // then: sums over lanes >= lane
      const uint64_t oh = sh, ol = sl;
      for (int o = 1; o < 64; o <<= 1) {
        const uint64_t vh = __shfl_down(sh, o, 64), vl = __shfl_down(sl, o, 64);
        if (lane + o < 64) {
          sh += vh;
          sl += vl;
        }
      }
      const uint64_t ah = t.ah + (sh - oh), al = t.al + (sl - ol);  // mass above this lane's keys
      int hit = -1;
      if (!kf_ge(ah, al, nh, nl) && kf_ge(ah + h1, al + l1, nh, nl)) hit = 1;
      else if (!kf_ge(ah + h1, al + l1, nh, nl) && kf_ge(ah + h1 + h0, al + l1 + l0, nh, nl)) hit = 0;
      const uint64_t hm = __ballot(hit >= 0);
      if (hm) {
        const int src = __builtin_ctzll(hm);
        const uint64_t xh = hit == 1 ? ah + h1 : ah + h1 + h0, xl = hit == 1 ? al + l1 : al + l1 + l0;
        cut = __shfl(kf_key16_full(k0 + (hit == 1 ? 1u : 0u)), src, 64);
        ch = __shfl(xh, src, 64);
        cl = __shfl(xl, src, 64);
      }
    }
    if (lane == 0) {
      P.filt[row].s = cut ? kf_float(ch + (cl >> 32), cl & 0xFFFFFFFFull) : __builtin_nan("");
      P.filt[row].tau = cut ? kf_val(cut) : -INFINITY;
    }
  }
  return true;
}

// Thresholds of the filtered rows (stochastic, r <= k_b for chains): one
// workgroup per row; top-k rows with candidates take them from those, the
// rest (top-p alone, larger top-k, candidates that do not fit) from passes
// over the row, or (TABLE: bf16 calls without top-k) from value counts.
union KFLds {
  KCShared c;
  KFRow f;
};
union KFTLds {
  KTShared t;
  KFRow f;
};
static_assert(kKC == kKF && kKC >= kDig && kKC % 64 == 0, "one workgroup shape for both thresholds paths");

template <bool BF16>
__global__ __launch_bounds__(kKF, 4) void kf_kernel(Params P) {
  __shared__ KFLds u;
  const int tid = threadIdx.x;
  const int b = (int)(blockIdx.x / (uint32_t)P.R);
  const int r = (int)(blockIdx.x - (uint32_t)b * (uint32_t)P.R);
  const int64_t row = (int64_t)b * P.R + r;
  const int Q = P.Q;
  // the row's partials and lane records are loaded ahead of the checks (in
  // bounds for every row of a filtered call; used by candidate rows only)
  uint64_t pm = 0;
  if (tid < Q) pm = P.part[row * P.CPR + tid].m_amax;
  u32x4 rec[kKCPub / kKC];
  const int npub = Q * kWG;
  const u32x4* pub = P.cand + row * Q * kWG;
#pragma unroll
  for (int j = 0; j < kKCPub / kKC; ++j)
    rec[j] = (P.top_k && npub <= kKCPub && j * kKC + tid < npub) ? pub[j * kKC + tid] : u32x4{0u, 0u, 0u, 0u};
  const float Tf = temp_of(P, b);
  const int tk = P.top_k ? P.top_k[b] : 0;
  const float tp = P.top_p ? P.top_p[b] : 1.f;
  int xi;
  const int kb = P.mode == MODE_CHAIN ? chain_kb(P, b, xi) : P.R;
  if (!request_filtered(P, b, Tf)) return;
  if (P.mode == MODE_CHAIN && r > kb) return;  // a tree reads all its rows
  if (kc_row(P, tk) && kc_try<BF16>(P, row, Tf, tk, tp, pm, rec, u.c)) return;
  __syncthreads();  // the shared memory changes roles
  kf_row<BF16>(P, row, Tf, tk, tp, u.f);
}

// The thresholds pass of a bf16 call with top-p and no top-k: value counts
// (one workgroup per CU: the table takes 128 KB of LDS).
__global__ __launch_bounds__(kKF, 2) void kft_kernel(Params P) {
  __shared__ KFTLds u;
  const int b = (int)(blockIdx.x / (uint32_t)P.R);
  const int r = (int)(blockIdx.x - (uint32_t)b * (uint32_t)P.R);
  const int64_t row = (int64_t)b * P.R + r;
  const float Tf = temp_of(P, b);
  const float tp = P.top_p[b];
  int xi;
  const int kb = P.mode == MODE_CHAIN ? chain_kb(P, b, xi) : P.R;
  if (!request_filtered(P, b, Tf)) return;
  if (P.mode == MODE_CHAIN && r > kb) return;  // a tree reads all its rows
  if (kt_row(P, row, Tf, tp, u.t)) return;
  __syncthreads();  // the shared memory changes roles
  kf_row<true>(P, row, Tf, 0, tp, u.f);
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
  int SUB, nsub, Q, Qp, G, CPR, C3, G3, CI, CHr;
  size_t gat_off, part_off, k3_off, r_off, f_off, cs_off, total;
};

// Work split of a call (a function of the shape alone, so results never
// depend on the device or the schedule): every row in Q segments, the
// fewest that give kK1Workgroups workgroups, but no more than are resident
// at once (at most 64 and at most one per sub-chunk; one when there are
// more rows than that).
static Shape shape_of(int64_t bs, int64_t R, int64_t V, int dtype, bool races, size_t data_off = kDataOffset) {
  Shape s;
  s.SUB = (dtype == SV_BF16 ? 8 : 4) * kVecPerThread * kWG;
  s.nsub = (int)((V + s.SUB - 1) / s.SUB);
  int64_t q = (kK1Workgroups + bs * R - 1) / (bs * R);
  if (q > kK1Resident / (bs * R)) q = kK1Resident / (bs * R);
  if (q > s.nsub) q = s.nsub;
  if (q > 64) q = 64;
  if (q < 1) q = 1;
  s.Q = (int)q;
  s.Qp = 1;
  while (s.Qp < s.Q) s.Qp *= 2;
  s.G = (int)(bs * R * q);
  s.CPR = q;
  s.C3 = races ? (int)((V + kK3Chunk - 1) / kK3Chunk) : 0;
  s.G3 = 1;
  if (races && bs * s.C3 > 2 * kK3Slots) s.G3 = (int)((bs * s.C3 + kK3Slots - 1) / kK3Slots);
  if (s.G3 > s.C3 && s.C3 > 0) s.G3 = s.C3;
  s.CI = races ? (s.C3 + s.G3 - 1) / s.G3 : 0;
  // block rule: residual-mass items per row of rows 1..R-2, about two
  // rounds of resident workgroups over the batch, whole chunks each
  s.CHr = 0;
  if (races && R >= 3) {
    int64_t ch = kKRWorkgroups / (bs * (R - 2));
    if (ch > s.C3) ch = s.C3;
    if (ch < 1) ch = 1;
    s.CHr = (int)ch;
  }
  s.gat_off = data_off;
  s.part_off = s.gat_off + align256(sizeof(Gather) * SV_MAX_NODES * (size_t)bs);
  s.k3_off = s.part_off + align256(sizeof(Partial) * (size_t)(bs * R * s.CPR));
  s.r_off = s.k3_off + align256(sizeof(K3Rec) * (size_t)(bs * s.C3));
  s.f_off = s.r_off + align256(sizeof(double) * (size_t)(bs * (R - 1) * s.CHr));
  s.cs_off = s.f_off + (races ? align256(sizeof(FiltRec) * (size_t)(bs * R)) : 0);
  // The race-chunk sums (unfiltered calls) and the top-k candidates
  // (filtered calls: a record per thread of every statistics segment) share
  // one area.
  const size_t cs_bytes = align256(sizeof(CSum) * kCSumShares * (size_t)(bs * R * s.C3));
  const size_t cand_bytes = align256(sizeof(u32x4) * kWG * (size_t)(bs * R * s.Q));
  s.total = s.cs_off + (races ? std::max(cs_bytes, cand_bytes) : 0);
  return s;
}

typedef void (*KernelFn)(Params);

struct Kernels {
  KernelFn k1, k23, fused, kr, kf, k23c, k1f, kft;
};

template <int MODE, bool BF16>
static Kernels kernels_for() {
  KernelFn k1f = nullptr;  // row-statistics calls have no filters
  if constexpr (MODE != MODE_ROWS) k1f = k1f_kernel<MODE, BF16>;
  KernelFn kft = nullptr;  // value counts: bf16 only
  if constexpr (BF16) kft = kft_kernel;
  return Kernels{k1_kernel<MODE, BF16>, k23_kernel<MODE, BF16>,  fused_kernel<MODE, BF16>, kr_kernel<BF16>,
                 kf_kernel<BF16>,         k23c_kernel<MODE, BF16>, k1f, kft};
}

static Kernels select_kernels(int mode, bool bf16) {
  if (mode == MODE_CHAIN) return bf16 ? kernels_for<MODE_CHAIN, true>() : kernels_for<MODE_CHAIN, false>();
  if (mode == MODE_TREE) return bf16 ? kernels_for<MODE_TREE, true>() : kernels_for<MODE_TREE, false>();
  return bf16 ? kernels_for<MODE_ROWS, true>() : kernels_for<MODE_ROWS, false>();
}

// Workgroups of fused kernel `slot` (mode * 2 + bf16) resident on the
// current device at once, queried once per device and kernel.
static std::atomic<int> g_resident[64][6];
static sv_status resident_workgroups(const void* kernel, int slot, int& out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64 || slot < 0 || slot >= 6) return SV_ERR_LAUNCH;
  const int cached = g_resident[dev][slot].load();
  if (cached > 0) {
    out = cached;
    return SV_OK;
  }
  int cu = 0, occ = 0;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return SV_ERR_LAUNCH;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, kWG, 0) != hipSuccess) return SV_ERR_LAUNCH;
  if (cu <= 0 || occ <= 0) return SV_ERR_LAUNCH;
  out = cu * occ;
  g_resident[dev][slot].store(out);
  return SV_OK;
}

static sv_status launch(Params& P, const Shape& S, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (ws == nullptr) return SV_ERR_INVALID_ARGUMENT;
  if (ws_bytes < S.total) return SV_ERR_WORKSPACE_TOO_SMALL;
  if (((uintptr_t)ws & 255u) != 0) return SV_ERR_INVALID_ARGUMENT;
  uint8_t* base = (uint8_t*)ws;
  P.ctrl = (Ctrl*)base;
  P.sync = (Sync*)(base + kSyncOffset);
  P.gat = (Gather*)(base + S.gat_off);
  P.part = (Partial*)(base + S.part_off);
  P.k3 = (K3Rec*)(base + S.k3_off);
  P.rpart = (double*)(base + S.r_off);
  P.filt = (FiltRec*)(base + S.f_off);
  P.csum = (CSum*)(base + S.cs_off);
  P.cand = (u32x4*)(base + S.cs_off);
  P.CHr = S.CHr;
  P.SUB = S.SUB;
  P.nsub = S.nsub;
  P.Q = S.Q;
  P.Qp = S.Qp;
  P.G = S.G;
  P.CPR = S.CPR;
  P.C3 = S.C3;
  P.G3 = S.G3;
  P.CI = S.CI;
  const bool filtered = P.mode != MODE_ROWS && (P.top_k != nullptr || P.top_p != nullptr);
  // Race-chunk sums: when every sampling job can only race over p (the
  // bonus) or p with ids removed -- one-hot chains and trees -- and no
  // filter changes p, the statistics pass publishes the chunk sums and one
  // decision/sampling item per request races from them.
  // (every schedule folds these calls' rows alike, so that they give the
  // same results)
  P.csum_fold = P.mode != MODE_ROWS && (P.mode == MODE_TREE || P.draft_kind == SV_DRAFT_ONEHOT);
  P.csum_on = P.csum_fold && !filtered && !(P.flags & SV_FLAG_FUSED);
  const int64_t grid23 = (int64_t)P.bs * P.CI;
  if (grid23 + P.G > (int64_t)INT32_MAX) return SV_ERR_UNSUPPORTED;
  const int64_t gridr = (int64_t)P.bs * (P.k >= 2 ? P.k - 1 : 0) * P.CHr;
  if (gridr > (int64_t)INT32_MAX) return SV_ERR_UNSUPPORTED;
  const int64_t gridf = (int64_t)P.bs * P.R;  // thresholds: one workgroup per row
  // Schedule: phased unless fused is asked for (phased measures faster on
  // the shapes benchmarked so far).
  P.sched = (P.flags & SV_FLAG_FUSED) ? SCHED_FUSED : SCHED_PHASED;
  const Kernels K = select_kernels(P.mode, P.dtype == SV_BF16);
  // fused: every K1 item first, then the sampling chunks (a lag of the
  // whole batch; smaller lags interleave them, SV_FUSED_LAG, for tuning)
  P.lag = P.bs;
  if (P.sched == SCHED_FUSED && P.mode != MODE_ROWS) {
    const char* e = getenv("SV_FUSED_LAG");
    if (e && *e) {
      const int l = atoi(e);
      if (l >= 0 && l < P.bs) P.lag = l;
    }
  }
  if (P.mode == MODE_ROWS) {
    hipLaunchKernelGGL(K.k1, dim3((unsigned)P.G), dim3(kWG), 0, stream, P);
  } else if (P.sched == SCHED_PHASED) {
    if (!(P.flags & SV_FLAG_DECIDE_ONLY)) {
      // top-k calls: the statistics pass also publishes candidate groups
      const bool cand = filtered && P.top_k != nullptr && !(P.flags & SV_FLAG_KF_ROWS);
      hipLaunchKernelGGL(cand ? K.k1f : K.k1, dim3((unsigned)P.G), dim3(kWG), 0, stream, P);
    }
    if (!(P.flags & SV_FLAG_STATS_ONLY)) {
      // bf16 calls with top-p and no top-k: thresholds from value counts
      if (filtered)
        hipLaunchKernelGGL((K.kft && P.top_k == nullptr) ? K.kft : K.kf, dim3((unsigned)gridf), dim3(kKF), 0, stream,
                           P);
      if ((P.flags & SV_FLAG_BLOCK) && P.k >= 2 && P.draft_kind == SV_DRAFT_PROBS)
        hipLaunchKernelGGL(K.kr, dim3((unsigned)gridr), dim3(kWG), 0, stream, P);
      if (P.csum_on) hipLaunchKernelGGL(K.k23c, dim3((unsigned)P.bs), dim3(kWG), 0, stream, P);
      else hipLaunchKernelGGL(K.k23, dim3((unsigned)grid23), dim3(kWG), 0, stream, P);
    }
  } else {
    hipLaunchKernelGGL(K.fused, dim3((unsigned)(P.G + grid23)), dim3(kWG), 0, stream, P);
  }
  if (hipGetLastError() != hipSuccess) return SV_ERR_LAUNCH;
  return SV_OK;
}

static bool aligned16(const void* p, int64_t stride_bytes) {
  return ((uintptr_t)p & 15u) == 0 && (stride_bytes & 15) == 0;
}

// Scratch of sv_verify_chain_noalloc: a fixed device array in place of the
// caller's workspace, for callers that cannot allocate.  Its layout is the
// workspace's, with a per-request counter area for SV_SCRATCH_MAX_BATCH
// requests.  Each device holds its own copy; the host learns its address
// with hipGetSymbolAddress once per device (the array's name is not a device
// address in host code).
static __device__ __align__(256) uint8_t scratch[SV_SCRATCH_BYTES];
constexpr size_t kScratchDataOffset = kSyncOffset + sizeof(Sync) * SV_SCRATCH_MAX_BATCH;
static std::atomic<void*> g_scratch[64];

static sv_status scratch_address(void*& out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return SV_ERR_LAUNCH;
  void* p = g_scratch[dev].load();
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SV_ERR_LAUNCH;
    g_scratch[dev].store(p);
  }
  out = p;
  return SV_OK;
}

// An enum-typed value from a caller, read as the int it holds: a caller may
// pass any value, and reading an enum outside its enumerators' range is
// undefined in C++.
template <typename E>
static int enum_int(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "C enums are int-sized");
  int v;
  memcpy(&v, &e, sizeof v);
  return v;
}

}  // namespace sv

using namespace sv;

extern "C" {

int32_t sv_abi_version(void) { return SV_ABI_VERSION; }

const char* sv_status_string(sv_status s) {
  switch (enum_int(s)) {
    case SV_OK: return "ok";
    case SV_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SV_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case SV_ERR_UNSUPPORTED: return "unsupported";
    case SV_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

static bool dtype_ok(const sv_dtype& d) { return enum_int(d) == SV_F32 || enum_int(d) == SV_BF16; }

static const uint32_t kKnownFlags =
    SV_FLAG_PHASED | SV_FLAG_FP64_RACE | SV_FLAG_FUSED | SV_FLAG_STATS_ONLY | SV_FLAG_DECIDE_ONLY | SV_FLAG_BLOCK |
    SV_FLAG_KF_ROWS;
// At most one of PHASED, FUSED, STATS_ONLY, DECIDE_ONLY, except PHASED with
// one of the split-phase bits.
static bool one_schedule(uint32_t flags) {
  const uint32_t split = flags & (SV_FLAG_STATS_ONLY | SV_FLAG_DECIDE_ONLY);
  if (split == (SV_FLAG_STATS_ONLY | SV_FLAG_DECIDE_ONLY)) return false;
  if ((flags & SV_FLAG_FUSED) && (split || (flags & SV_FLAG_PHASED))) return false;
  return true;
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

// Checks a chain descriptor on the host and fills the launch parameters.
static sv_status chain_params(const sv_chain_desc* d, Params& P) {
  if (d == nullptr) return SV_ERR_INVALID_ARGUMENT;
  if (d->batch < 1 || d->batch > SV_MAX_BATCH || d->max_draft < 0 || d->max_draft > SV_MAX_DRAFT ||
      d->vocab < 1 || d->vocab > SV_MAX_VOCAB)
    return SV_ERR_INVALID_ARGUMENT;
  if (!dtype_ok(d->logits_dtype)) return SV_ERR_UNSUPPORTED;
  if (enum_int(d->draft_kind) != SV_DRAFT_PROBS && enum_int(d->draft_kind) != SV_DRAFT_ONEHOT)
    return SV_ERR_UNSUPPORTED;
  if (d->flags & ~kKnownFlags) return SV_ERR_UNSUPPORTED;
  if (!one_schedule(d->flags)) return SV_ERR_INVALID_ARGUMENT;
  if ((d->flags & SV_FLAG_BLOCK) && (d->flags & SV_FLAG_FUSED)) return SV_ERR_UNSUPPORTED;
  if ((d->top_k != nullptr || d->top_p != nullptr) && (d->flags & SV_FLAG_FUSED)) return SV_ERR_UNSUPPORTED;
  if (d->logits == nullptr || d->temperature == nullptr || d->seed == nullptr || d->accept_len == nullptr ||
      d->tokens == nullptr)
    return SV_ERR_INVALID_ARGUMENT;
  if (d->max_draft > 0 && d->draft_ids == nullptr) return SV_ERR_INVALID_ARGUMENT;
  if (d->logits_row_stride < d->vocab) return SV_ERR_INVALID_ARGUMENT;
  const bool probs = d->draft_kind == SV_DRAFT_PROBS;
  if (probs && d->max_draft > 0 && (d->draft_probs == nullptr || d->q_row_stride < d->vocab))
    return SV_ERR_INVALID_ARGUMENT;
  const size_t esz = d->logits_dtype == SV_BF16 ? 2 : 4;
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
  P.top_k = d->top_k;
  P.top_p = d->top_p;
  return SV_OK;
}

sv_status sv_verify_chain(const sv_chain_desc* d, void* ws, size_t ws_bytes, void* stream) {
  Params P;
  const sv_status st = chain_params(d, P);
  if (st != SV_OK) return st;
  const Shape S = shape_of(P.bs, P.R, P.V, P.dtype, true);
  return launch(P, S, ws, ws_bytes, (hipStream_t)stream);
}

sv_status sv_verify_chain_noalloc(const sv_chain_desc* d, void* stream) {
  Params P;
  sv_status st = chain_params(d, P);
  if (st != SV_OK) return st;
  if (P.bs > SV_SCRATCH_MAX_BATCH) return SV_ERR_WORKSPACE_TOO_SMALL;
  const Shape S = shape_of(P.bs, P.R, P.V, P.dtype, true, kScratchDataOffset);
  if (S.total > (size_t)SV_SCRATCH_BYTES) return SV_ERR_WORKSPACE_TOO_SMALL;
  void* base = nullptr;
  st = scratch_address(base);
  if (st != SV_OK) return st;
  // The control block and this call's per-request counters must start at
  // zero.  A completed call leaves them so, but one that gave up a bounded
  // wait does not, and the array outlives every caller: clear them with the
  // fill kernel (no memset node, so the call may be captured in a graph).
  const size_t clear = kSyncOffset + sizeof(Sync) * (size_t)P.bs;
  const unsigned blocks = (unsigned)((clear / 16 + kWG - 1) / kWG);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(kWG), 0, (hipStream_t)stream, (uint8_t*)base, clear);
  if (hipGetLastError() != hipSuccess) return SV_ERR_LAUNCH;
  return launch(P, S, base, (size_t)SV_SCRATCH_BYTES, (hipStream_t)stream);
}

sv_status sv_verify_tree(const sv_tree_desc* d, void* ws, size_t ws_bytes, void* stream) {
  if (d == nullptr) return SV_ERR_INVALID_ARGUMENT;
  if (d->batch < 1 || d->batch > SV_MAX_BATCH || d->num_nodes < 1 || d->num_nodes > SV_MAX_NODES ||
      d->vocab < 1 || d->vocab > SV_MAX_VOCAB)
    return SV_ERR_INVALID_ARGUMENT;
  if (!dtype_ok(d->logits_dtype)) return SV_ERR_UNSUPPORTED;
  if (d->flags & ~kKnownFlags) return SV_ERR_UNSUPPORTED;
  if (d->flags & SV_FLAG_BLOCK) return SV_ERR_UNSUPPORTED;
  if ((d->top_k != nullptr || d->top_p != nullptr) && (d->flags & SV_FLAG_FUSED)) return SV_ERR_UNSUPPORTED;
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
  P.top_k = d->top_k;
  P.top_p = d->top_p;
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
