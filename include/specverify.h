/* specverify.h - C ABI of libspecverify: batched lossless verification of
 * speculative-decoding drafts on AMD Instinct MI355X (gfx950).
 *
 * What is computed.  For each request the target model has produced one
 * logit row per verified position.  The target distribution of a row is
 * p = softmax(logits / T) (temperature T > 0), or the point mass on the
 * argmax when T <= 0 (greedy).  Page "投机解码" (Speculative decoding,
 * rustineverything.app), section "接受规则为什么不改变分布" (why the acceptance
 * rule keeps the distribution), states the rule implemented here:
 *   - chain drafts are accepted left to right, draft x with probability
 *     min(1, p(x)/q(x)) (sub-section "采样：标准拒绝采样", standard rejection
 *     sampling); at the first rejection one token is drawn from
 *     max(0, p - q) normalised, the remaining drafts are dropped; if every
 *     draft is accepted a bonus token is drawn from the next row's p;
 *   - a one-hot ("target-only") draft has q(x) = 1, so x is accepted with
 *     probability p(x) and the residual is p with x removed (sub-section
 *     "默认路径：草稿当 one-hot");
 *   - greedy rows accept x iff x is the target argmax and emit the argmax
 *     (sub-section "贪心");
 *   - a draft tree is walked from the root: one coin per level, the
 *     children tried in increasing node index while their target
 *     probabilities accumulate; if none is accepted the next token is drawn
 *     from p with the tried children removed (sub-section "SGLang 默认：只看目标
 *     概率，可以验证一棵树", with both relaxation thresholds at their exact value 1).
 *   - q(x) <= 0 accepts iff p(x) > 0 (section "对照：mistral.rs").
 *
 * Randomness is a counter-based Philox4x32-10 stream (Salmon et al., SC'11)
 * keyed by the request's 64-bit seed: the coin of row r of request b is
 * word 0 of counter (0, r, b, 0); the sampling noise of vocabulary id y is
 * word (y & 3) of counter (y >> 2, r, b, 1) and that of id chunk c is word 0
 * of counter (c, r, b, 2); a word w maps to the uniform (2*(w >> 9) + 1) /
 * 2^24.  Every sample is a two-level exponential race: the ids are cut into
 * chunks of 2048; the chunk maximising W_c / E_c (W_c the chunk's weight
 * sum, E = -ln U) wins, then the id of that chunk maximising w(y) / E_y,
 * ties to the smaller index at both levels.  This draws y with probability
 * w(y) / sum w exactly, and a call is a pure function of its inputs:
 * replaying it replays the result.
 *
 * Conventions.  Every data pointer is DEVICE memory unless marked [host].
 * Logit rows are row-major: element y of row i is at logits + i*row_stride
 * + y (in elements).  bf16 logits are widened exactly; all arithmetic that
 * decides an outcome is fp32 with fp64 accumulation and fp64 re-evaluation
 * of near-ties.  `stream` is a hipStream_t (NULL = the default stream).
 * Calls only enqueue work: they never allocate, never synchronise, keep no
 * state between calls and may be made from any host thread.  Results are
 * valid once the stream reaches that point.
 *
 * Errors.  Problems visible on the host (NULL pointers, bad sizes, a
 * workspace that is too small, unsupported values) return a non-zero
 * sv_status and enqueue nothing.  Problems in the data set req_status[b]
 * (an SV_REQ_* code); that request then reports accept_len 0 and tokens all
 * -1, and every other request is unaffected.
 *
 * Workspace.  Each call needs a caller-owned device workspace of at least
 * the size returned by the matching *_workspace_bytes function.  It holds
 * scheduling counters and partial results; it must be zero-filled once
 * before its first use (sv_workspace_init does that on a stream), and every
 * completed call leaves it ready for the next one, whatever the shapes.
 * Calls that share a workspace must not overlap in time (use one workspace
 * per stream).  After a call reports SV_REQ_INTERNAL for any request,
 * re-initialise the workspace.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SV_ABI_VERSION 3

/* Limits of one call. */
#define SV_MAX_BATCH 65536   /* requests per call */
#define SV_MAX_DRAFT 63      /* chain drafts per request (k) */
#define SV_MAX_NODES 64      /* tree nodes per request, root included (N) */
#define SV_MAX_VOCAB (1 << 24)

typedef enum {
  SV_OK = 0,
  SV_ERR_INVALID_ARGUMENT = 1,
  SV_ERR_WORKSPACE_TOO_SMALL = 2,
  SV_ERR_UNSUPPORTED = 3,
  SV_ERR_LAUNCH = 4
} sv_status;

typedef enum { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

typedef enum {
  SV_DRAFT_PROBS = 0,  /* q given as full fp32 rows: standard rejection sampling */
  SV_DRAFT_ONEHOT = 1  /* q one-hot at the draft token ("target-only") */
} sv_draft_kind;

/* Per-request status codes written to req_status. */
enum {
  SV_REQ_OK = 0,
  SV_REQ_BAD_DRAFT_ID = 1,     /* a used draft id outside [0, V), or below -1 */
  SV_REQ_BAD_TREE = 2,         /* parent[0] != -1, parent[i] not in [0, i), node token outside [0, V),
                                  or two children of one node with the same token */
  SV_REQ_NONFINITE = 3,        /* a read row holds NaN or +inf, or is entirely -inf */
  SV_REQ_BAD_TEMPERATURE = 4,  /* temperature is NaN or infinite */
  SV_REQ_INTERNAL = 5          /* internal scheduling timeout; re-initialise the workspace */
};

/* Option bits for the `flags` fields.  At most one schedule bit (PHASED or
 * FUSED) may be set (else SV_ERR_INVALID_ARGUMENT); without one the library
 * picks the schedule it measures fastest.  Both give bit-identical results. */
#define SV_FLAG_PHASED 1u    /* two stream-ordered launches: row statistics, then decisions and sampling */
#define SV_FLAG_FP64_RACE 2u /* evaluate every sampling race entirely in fp64 (slow; a test aid) */
#define SV_FLAG_FUSED 4u     /* one launch: the decision/sampling workgroups wait for their rows' statistics */
/* Split-phase use of the phased schedule: a call with STATS_ONLY runs only
 * the row-statistics pass, the one launch that reads every target logit
 * (outputs untouched); a following call with DECIDE_ONLY, the same
 * descriptor and workspace, on the same stream, runs the rest (filter
 * thresholds, block residuals, decisions and sampling) and writes the
 * outputs.  Together they equal
 * one plain call; other work may be queued between them.  Neither may be
 * combined with SV_FLAG_FUSED or with each other. */
#define SV_FLAG_STATS_ONLY 8u
#define SV_FLAG_DECIDE_ONLY 16u
/* Block verification for the stochastic requests of a chain call (page "The
 * speculative decoding zoo", the passage on vLLM's "block" rejection method,
 * after Sun et al. 2024, which it cites).  The drafts are judged as a block:
 * with prefix weights w_0 = 1, w_{i+1} = min(w_i p_i(x_i) / q_i(x_i), 1)
 * (q one-hot at the draft for SV_DRAFT_ONEHOT; q(x) = 0 gives ratio +inf if
 * p(x) > 0, else 0) and residual masses r_i = sum_y max(w_i p_i(y) - q_i(y), 0),
 * prefix length i = 1..kb passes with probability h_i = r_i / (r_i + 1 - w_i)
 * (1 when that denominator is 0) for i < kb and h_kb = w_kb.  The accepted
 * length a is the longest prefix whose coin passes (eta_i <= h_i, eta_i the
 * coin of row i - 1; 0 if none), and the emitted token is drawn from
 * max(w_a p_a - q_a, 0) (all zero: p_a), or from p_kb when a = kb.  One draft
 * gives the standard rule.  Greedy requests are unaffected.  The residual
 * masses of rows 1..kb-1 take one more pass over those target and q rows
 * (a third launch); not available with SV_FLAG_FUSED (SV_ERR_UNSUPPORTED)
 * nor for trees (SV_ERR_UNSUPPORTED).  With STATS_ONLY / DECIDE_ONLY the
 * extra pass belongs to the DECIDE_ONLY call. */
#define SV_FLAG_BLOCK 32u
/* Top-k thresholds from passes over the whole rows.  Without it, for top-k
 * values up to 128 the row-statistics pass also keeps the groups of logits
 * the kept set can come from, and the thresholds come from those alone (one
 * read of each row in all); rows where ties defeat that are read again.
 * Both give bit-identical results; this bit is a test and measurement aid. */
#define SV_FLAG_KF_ROWS 64u

typedef struct {
  int32_t batch;              /* bs, 1..SV_MAX_BATCH */
  int32_t max_draft;          /* k, 0..SV_MAX_DRAFT; rows per request R = k + 1 */
  int32_t vocab;              /* V, 1..SV_MAX_VOCAB */
  sv_dtype logits_dtype;
  const void* logits;         /* [bs][k+1] rows of V; row b*(k+1)+r is the target after r drafts */
  int64_t logits_row_stride;  /* elements between rows, >= V */
  sv_draft_kind draft_kind;
  const float* draft_probs;   /* [bs][k] rows of V (SV_DRAFT_PROBS), row b*k+i is q_i; NULL for one-hot */
  int64_t q_row_stride;       /* elements between q rows, >= V */
  const int32_t* draft_ids;   /* [bs][k]; the first -1 ends a request's chain (later slots ignored) */
  const float* temperature;   /* [bs]; <= 0 selects greedy */
  const uint64_t* seed;       /* [bs]; Philox key of the request */
  int32_t* accept_len;        /* [bs] out: drafts accepted (bonus excluded) */
  int32_t* tokens;            /* [bs][k+1] out: accepted drafts, then the emitted token, -1 after */
  int32_t* req_status;        /* [bs] out, may be NULL */
  double* p_draft;            /* [bs][k] out, may be NULL: p_i(x_i) for used slots, NaN elsewhere
                                 (greedy rows: 1 at the argmax, else 0) */
  uint32_t flags;             /* SV_FLAG_* bits, 0 by default */
  /* Top-k / top-p filtering of the target (page "投机解码", section
   * "接受规则为什么不改变分布": p is the target after temperature and the
   * top-k / top-p sampling parameters).  Per request, both may be NULL (no
   * filtering).  top_k[b] keeps the tokens whose logit is at least the k-th
   * largest of the row (ties at it kept); top_p[b] then keeps, within that
   * set, the fewest groups of equal logits, highest first, whose probability
   * mass reaches top_p[b] times the set's mass.  The kept set is {l >= tau}
   * for one threshold tau per row; p is restricted to it and renormalised,
   * on every row read (0..k_b) of a stochastic request, so the ratio test,
   * the residual and the bonus all see the filtered p.  top_k <= 0 or >= V,
   * and top_p outside (0, 1) (NaN included), switch a filter off; greedy
   * requests ignore both.  q is taken as given (the drafter's own, already
   * filtered if it filters).  A call with either array non-NULL takes one
   * more launch (the thresholds of every row read, one workgroup each)
   * between the statistics and the decisions; not available with
   * SV_FLAG_FUSED (SV_ERR_UNSUPPORTED).  With STATS_ONLY / DECIDE_ONLY the
   * thresholds belong to the DECIDE_ONLY call, and both calls must pass the
   * same arrays.  The arrays are read on the device (device pointers). */
  const int32_t* top_k;       /* [bs] or NULL */
  const float* top_p;         /* [bs] or NULL */
} sv_chain_desc;

typedef struct {
  int32_t batch;              /* bs, 1..SV_MAX_BATCH */
  int32_t num_nodes;          /* N, 1..SV_MAX_NODES, the root included */
  int32_t vocab;
  sv_dtype logits_dtype;
  const void* logits;         /* [bs][N] rows of V; row b*N+n is the target after node n */
  int64_t logits_row_stride;
  const int32_t* node_tokens; /* [bs][N]; the token node n proposes (entry 0 ignored) */
  const int32_t* parent;      /* [bs][N]; parent[0] = -1, 0 <= parent[i] < i */
  const float* temperature;   /* [bs]; <= 0 selects greedy */
  const uint64_t* seed;       /* [bs] */
  int32_t* accept_len;        /* [bs] out: accepted nodes (root excluded) */
  int32_t* accept_path;       /* [bs][N] out: accepted node ids from the root down, -1 after */
  int32_t* tokens;            /* [bs][N] out: accepted nodes' tokens, then the emitted token, -1 after */
  int32_t* req_status;        /* [bs] out, may be NULL */
  uint32_t flags;
  /* Top-k / top-p filtering of the target, as for chains (sv_chain_desc):
   * every row of a filtered stochastic request (all N) is filtered, so the
   * walk's sibling sums and the residual use the filtered p.  NULL: off. */
  const int32_t* top_k;       /* [bs] or NULL */
  const float* top_p;         /* [bs] or NULL */
} sv_tree_desc;

/* Bytes of workspace a call of the given shape needs (0 if the shape is
 * outside the limits). */
size_t sv_chain_workspace_bytes(int32_t batch, int32_t max_draft, int32_t vocab, sv_dtype logits_dtype);
size_t sv_tree_workspace_bytes(int32_t batch, int32_t num_nodes, int32_t vocab, sv_dtype logits_dtype);
size_t sv_row_stats_workspace_bytes(int32_t rows, int32_t vocab, sv_dtype logits_dtype);

/* Zero-fill `bytes` of workspace on `stream` (a fill kernel, safe to
 * capture in a graph). */
sv_status sv_workspace_init(void* workspace, size_t bytes, void* stream);

/* Chain verification (standard, one-hot or greedy per request). */
sv_status sv_verify_chain(const sv_chain_desc* desc /* [host] */, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Chain verification without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  It is sv_verify_chain with the
 * workspace replaced by a fixed array of SV_SCRATCH_BYTES in the library's
 * device memory (one per GPU, held until the process ends); it allocates
 * nothing.  Shapes whose workspace would not fit it, and batches above
 * SV_SCRATCH_MAX_BATCH, return SV_ERR_WORKSPACE_TOO_SMALL and enqueue
 * nothing.  Each call first clears the array's control block and its
 * requests' counters with a small fill kernel (so a call after one that
 * reported SV_REQ_INTERNAL needs no reset).  Every call on one GPU uses that
 * GPU's one array: calls that may overlap in time on the same GPU (other
 * streams, other host threads) race and must be serialised by the caller.
 * Same descriptor, flags, results and errors as sv_verify_chain otherwise. */
#define SV_SCRATCH_BYTES (8u << 20)
#define SV_SCRATCH_MAX_BATCH 1024
sv_status sv_verify_chain_noalloc(const sv_chain_desc* desc /* [host] */, void* stream);

/* Target-only tree verification (stochastic or greedy per request). */
sv_status sv_verify_tree(const sv_tree_desc* desc /* [host] */, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Row statistics of `rows` logit rows (the streaming pass on its own):
 * row_max = max_y l(y); row_argmax = the smallest y attaining it (raw
 * logits); row_sumexp = sum_y exp((l(y) - row_max) / T_i) for T_i > 0 (NaN
 * for greedy rows), so p(y) = exp((l(y) - row_max)/T_i) / row_sumexp;
 * row_status = SV_REQ_OK or SV_REQ_NONFINITE.  temperature is per row.
 * Outputs may be NULL individually. */
sv_status sv_row_stats(int32_t rows, int32_t vocab, sv_dtype logits_dtype, const void* logits,
                       int64_t logits_row_stride, const float* temperature, float* row_max,
                       int32_t* row_argmax, double* row_sumexp, int32_t* row_status, void* workspace,
                       size_t workspace_bytes, void* stream);

const char* sv_status_string(sv_status status);
int32_t sv_abi_version(void);

/* Survival top-k draft budget: which draft positions of a batch to verify
 * this step (page "New approaches to speculative decoding: block drafts,
 * load-aware verification and PD disaggregation", section "Deciding how
 * much to verify by load", with the cost model of its section "The higher
 * the load, the smaller K should be"; page "The speculative decoding zoo",
 * section "The finer loop: DSpark's confidence budget").
 *
 * Slot (b, j) scores the chance that request b's drafts 0..j all pass: the
 * fp32 product of confidence[b][0..j], each confidence clamped to [0, 1]
 * (NaN counts as 0), for j < num_steps[b] (clamped to [0, K]; NULL: K).  Slots
 * are ranked by score, higher first; ties go to the earlier position, then
 * to the smaller request index, so every request's admitted slots form a
 * prefix.  Admitting the top B slots is worth
 *   rate(B) = (base_tokens + sum of their scores) / cost[B];
 * the budget B* is the first B in 0..min(max_budget, slots) with the largest
 * rate (sums in fp64; a NaN rate never wins; none that beats -inf: B* = 0).
 * Outputs: budget[0] = B*, draft_len[b] = admitted positions of request b
 * (pad its draft ids after that with -1 for sv_verify_chain), rate[0] =
 * rate(B*).  bs * K must not exceed SV_PLAN_MAX_SLOTS (else
 * SV_ERR_UNSUPPORTED).
 *
 * workspace: device memory of at least sv_plan_workspace_bytes(bs, K) bytes
 * (the same for every shape), 256-byte aligned (else SV_ERR_INVALID_ARGUMENT /
 * SV_ERR_WORKSPACE_TOO_SMALL), of any contents (it carries the ranked slots
 * from one launch of the call to the next and needs no clearing); calls of
 * any shape may reuse it as long as they do not overlap (calls that overlap
 * need their own).  The caller owns it. */
#define SV_PLAN_MAX_SLOTS 8192

typedef struct {
  int32_t batch;              /* bs >= 1 */
  int32_t max_steps;          /* K, 1..64: confidence columns per request */
  const float* confidence;    /* [bs][K] */
  const int32_t* num_steps;   /* [bs] drafted positions per request, or NULL */
  int32_t max_budget;         /* >= 0: the cost table covers budgets 0..max_budget */
  const double* cost;         /* [max_budget + 1] cost of a step that verifies B draft positions */
  double base_tokens;         /* tokens a step yields with no draft position verified */
  int32_t* budget;            /* [1] out: B* */
  int32_t* draft_len;         /* [bs] out */
  double* rate;               /* [1] out, may be NULL */
  void* workspace;            /* device, see above */
  size_t workspace_bytes;
} sv_plan_desc;

/* Workspace bytes of a plan of bs requests and K positions (0 for shapes
 * sv_plan_budget rejects). */
size_t sv_plan_workspace_bytes(int32_t batch, int32_t max_steps);
sv_status sv_plan_budget(const sv_plan_desc* desc /* [host] */, void* stream);

/* Accepted-path KV compaction after tree verification (page "投机解码", section
 * "与调度、KV 的交互", sub-section "SGLang：按最坏情况预留，结束时归还"; page "Draft
 * sources: draft models, n-gram, suffix decoding", section "SGLang's suffix
 * automaton, in tree"): a tree's accepted path is scattered over the tree's
 * KV slots and is moved so that the accepted tokens follow the committed
 * prefix contiguously.
 *
 * For each request b with accepted nodes p_1..p_a (accept_len and
 * accept_path as sv_verify_tree writes them; node 0, the root, is already in
 * place), for i = 1..a in order, every layer's row at slot node_slot[p_i] is
 * copied to slot node_slot[i] (no copy when p_i = i).  Row l, s of the pool
 * is the row_bytes at kv + l*layer_stride + s*slot_stride (bytes; all
 * multiples of 16 and kv 16-byte aligned, else SV_ERR_UNSUPPORTED).  A
 * request whose accept_len is outside [0, N), whose path does not rise from
 * node 1 up inside the tree, or whose slots fall outside the pool is left
 * untouched and reports moved = -1; otherwise moved[b] = the rows moved per
 * layer.  Different requests must not share slots.  Device pointers except
 * the descriptor. */
typedef struct {
  int32_t batch;              /* bs, 1..SV_MAX_BATCH */
  int32_t num_nodes;          /* N, 1..SV_MAX_NODES */
  const int32_t* accept_len;  /* [bs] */
  const int32_t* accept_path; /* [bs][N] */
  const int64_t* node_slot;   /* [bs][N] KV slot of each node's token */
  void* kv;                   /* the pool, modified in place */
  int32_t num_layers;         /* >= 1 */
  int64_t num_slots;          /* slots per layer */
  int64_t slot_stride;        /* bytes between slots, >= row_bytes */
  int64_t layer_stride;       /* bytes between layers, >= num_slots * slot_stride when num_layers > 1 */
  int64_t row_bytes;          /* bytes of one token's row in one layer */
  int32_t* moved;             /* [bs] out, may be NULL */
} sv_compact_desc;

sv_status sv_compact_kv(const sv_compact_desc* desc /* [host] */, void* stream);

/* Measurement aid, not part of verification: streams `bytes` (a multiple
 * of 16, 16-byte aligned) from `src` with the row-statistics pass's access
 * pattern (16-byte nontemporal loads, contiguous shares of `workgroups`
 * workgroups of 256 threads) and XOR-folds them, writing one word per
 * workgroup to sink[workgroups].  Its bandwidth is the attainable read
 * ceiling that the verification kernels are quoted against.  Device
 * pointers; SV_ERR_INVALID_ARGUMENT for bad sizes or alignment. */
sv_status sv_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
