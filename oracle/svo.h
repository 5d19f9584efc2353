/* svo.h - reference oracle for batched lossless draft verification.
 *
 * TEST INFRASTRUCTURE ONLY.  This header and svo.c form a plain, slow,
 * single-threaded CPU implementation of what the GPU library computes.  It
 * exists so that tests, the smoke check and the benchmark's CPU-baseline leg
 * can compare the HIP path against an independent implementation.  Nothing
 * in the product path may include, link or call it.  It shares no code,
 * header, table or constant with the HIP library.
 *
 * Every pointer is host memory.  Floating-point work is done in double;
 * bf16 inputs are widened exactly.
 */
#ifndef SVO_H
#define SVO_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Per-request status codes (same numbering as the library's, defined here
 * independently). */
enum {
  SVO_REQ_OK = 0,
  SVO_REQ_BAD_DRAFT_ID = 1,
  SVO_REQ_BAD_TREE = 2,
  SVO_REQ_NONFINITE = 3,
  SVO_REQ_BAD_TEMPERATURE = 4
};

enum { SVO_F32 = 0, SVO_BF16 = 1 };
enum { SVO_DRAFT_PROBS = 0, SVO_DRAFT_ONEHOT = 1 };
/* Acceptance rule of stochastic chain requests: left-to-right rejection
 * sampling, or block verification (greedy requests ignore it). */
enum { SVO_RULE_STANDARD = 0, SVO_RULE_BLOCK = 1 };

/* Philox4x32-10 block function: 10 rounds of the Philox-4x32 bijection keyed
 * by key[0..1], applied to the 128-bit counter ctr[0..3]. */
void svo_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);

/* Uniform in the open interval (0,1) from one 32-bit word: (2*(w>>9)+1)/2^24. */
double svo_uniform(uint32_t w);

/* The coin for row r of request b, and the race noise word for vocab id y. */
double svo_coin(uint64_t seed, int32_t b, int32_t r);
double svo_noise_uniform(uint64_t seed, int32_t b, int32_t r, int32_t y);
/* Chunk noise of the two-level race: word 0 of counter (c, r, b, 2). */
double svo_chunk_uniform(uint64_t seed, int32_t b, int32_t r, int32_t c);

/* Ids per chunk of the sampling race.  A constant of the sampler's
 * definition (the race first picks a chunk by its weight sum, then an id
 * inside it), fixed with that definition: two levels keep the per-id Philox
 * noise to one chunk per sample.  Any implementation of the same sampler
 * must use the same value to give the same tokens. */
#define SVO_RACE_CHUNK 2048

/* The two-level exponential race over w[0..V) with `chunk` ids per chunk
 * (the verifiers use SVO_RACE_CHUNK); *margin (may be NULL) receives the
 * smaller relative top-two key gap of the two levels. */
int32_t svo_race(const double* w, int32_t V, int32_t chunk, uint64_t seed, int32_t b, int32_t r, double* margin);

/* Row statistics of `rows` logit rows.  Row i starts at element i*row_stride.
 * temperature[i] <= 0 or non-finite means greedy (no sum is formed; sumexp = NaN).
 * Outputs (any may be NULL): row_max, row_argmax (smallest index of the max,
 * on raw logits), row_sumexp = sum_y exp((l_y - max)/T) summed left to right,
 * row_status (SVO_REQ_OK or SVO_REQ_NONFINITE). */
void svo_row_stats(int32_t rows, int32_t vocab, int32_t dtype, const void* logits, int64_t row_stride,
                   const float* temperature, double* row_max, int32_t* row_argmax, double* row_sumexp,
                   int32_t* row_status);

typedef struct {
  int32_t batch, max_draft, vocab;          /* bs, k, V */
  int32_t logits_dtype;                     /* SVO_F32 or SVO_BF16 (raw uint16 bits) */
  const void* logits;                       /* row (b*(k+1)+r) at element offset row*logits_row_stride */
  int64_t logits_row_stride;
  int32_t draft_kind;                       /* SVO_DRAFT_PROBS or SVO_DRAFT_ONEHOT */
  const float* draft_probs;                 /* row (b*k+i) at offset row*q_row_stride; NULL for one-hot */
  int64_t q_row_stride;
  const int32_t* draft_ids;                 /* [bs][k]; -1 ends the chain */
  const float* temperature;                 /* [bs]; <= 0 => greedy */
  const uint64_t* seed;                     /* [bs] */
  int32_t* accept_len;                      /* [bs] out */
  int32_t* tokens;                          /* [bs][k+1] out */
  int32_t* req_status;                      /* [bs] out, may be NULL */
  double* p_draft;                          /* [bs][k] out: p_i(x_i), NaN where unused; may be NULL */
  double* min_margin;                       /* [bs] out: smallest decision margin; may be NULL */
  int32_t* n_decisions;                     /* [bs] out: decisions taken; may be NULL */
  int32_t rule;                             /* SVO_RULE_STANDARD or SVO_RULE_BLOCK */
  const int32_t* top_k;                     /* [bs] or NULL: top-k of each stochastic request (<= 0: off) */
  const float* top_p;                       /* [bs] or NULL: top-p (outside (0, 1): off) */
  double* cut_margin;                       /* [bs] out, may be NULL: smallest relative gap of a top-p cut
                                               (its cumulative mass against the target, either side;
                                               +inf without one) */
} svo_chain_args;

typedef struct {
  int32_t batch, num_nodes, vocab;          /* bs, N (root included), V */
  int32_t logits_dtype;
  const void* logits;                       /* row (b*N+n): target distribution after node n */
  int64_t logits_row_stride;
  const int32_t* node_tokens;               /* [bs][N]; entry 0 ignored */
  const int32_t* parent;                    /* [bs][N]; parent[0] = -1, 0 <= parent[i] < i */
  const float* temperature;
  const uint64_t* seed;
  int32_t* accept_len;                      /* [bs] out: accepted nodes, root excluded */
  int32_t* accept_path;                     /* [bs][N] out: accepted node ids, -1 padded */
  int32_t* tokens;                          /* [bs][N] out: accepted tokens, then the emitted one */
  int32_t* req_status;
  double* min_margin;
  int32_t* n_decisions;
  /* Test-only relaxation knobs of the target-only tree rule.  1.0 is the
   * exact rule; any other value makes the rule lossy and exists only so the
   * statistical tests can show they detect a changed distribution. */
  double threshold_acc, threshold_single;
  /* Top-k / top-p filtering of the stochastic requests' target rows, as for
   * chains (NULL: off). */
  const int32_t* top_k;
  const float* top_p;
  double* cut_margin;                       /* [bs] out, may be NULL: as for chains */
} svo_tree_args;

void svo_verify_chain(const svo_chain_args* a);
void svo_verify_tree(const svo_tree_args* a);

/* Survival top-k draft budget: which draft positions of a batch to verify. */
typedef struct {
  int32_t batch, max_steps;                 /* bs, K */
  const float* confidence;                  /* [bs][K] per-position confidences */
  const int32_t* num_steps;                 /* [bs] drafted positions (clamped to [0, K]); NULL: K each */
  int32_t max_budget;                       /* cost table covers budgets 0..max_budget */
  const double* cost;                       /* [max_budget + 1] step cost when B positions are verified */
  double base_tokens;                       /* tokens a step yields with no draft position verified */
  int32_t* budget;                          /* [1] out: the chosen budget B* */
  int32_t* draft_len;                       /* [bs] out: admitted positions of each request (a prefix) */
  double* rate;                             /* [1] out: (base + gain(B*)) / cost[B*] */
  double* margin;                           /* [1] out, may be NULL: relative gap to the next distinct rate */
} svo_plan_args;

void svo_plan_budget(const svo_plan_args* a);

/* Accepted-path KV compaction after tree verification. */
typedef struct {
  int32_t batch, num_nodes;                 /* bs, N */
  const int32_t* accept_len;                /* [bs] */
  const int32_t* accept_path;               /* [bs][N] accepted node ids from the root down */
  const int64_t* node_slot;                 /* [bs][N] KV slot of each node */
  uint8_t* kv;                              /* layer l, slot s at kv + l*layer_stride + s*slot_stride */
  int32_t num_layers;
  int64_t num_slots, slot_stride, layer_stride, row_bytes;
  int32_t* moved;                           /* [bs] out, may be NULL: rows moved per layer (-1: request skipped) */
} svo_compact_args;

void svo_compact_kv(const svo_compact_args* a);

#ifdef __cplusplus
}
#endif

#endif
