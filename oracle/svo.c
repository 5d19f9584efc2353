/* svo.c - reference oracle for batched lossless draft verification.
 *
 * TEST INFRASTRUCTURE ONLY: a plain, slow, single-threaded CPU statement of
 * what the GPU library computes.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it.  It shares no code with the HIP
 * library.  All floating-point arithmetic is double precision; bf16 logits
 * are widened exactly; the loops follow the method's steps in order with no
 * blocking, fusion or reordering.
 *
 * Sources (the pages are cited by title and section):
 *  [SD]  "投机解码" (Speculative decoding), rustineverything.app:
 *        section "接受规则为什么不改变分布" (why the acceptance rule keeps the
 *        distribution) with its sub-sections "贪心" (greedy), "采样：标准拒绝采样"
 *        (standard rejection sampling), "默认路径：草稿当 one-hot" (one-hot
 *        default), "SGLang 默认：只看目标概率，可以验证一棵树" (target-only tree);
 *        section "对照：mistral.rs" (the q <= 0 rule).
 *  [ZOO] "The speculative decoding zoo" (section 6.6), mlinterviewnotes.com:
 *        "DFlash - the draft that borrows everything" (greedy prefix match);
 *        the passage on vLLM's rejection methods (after "Multi-layer EAGLE
 *        and STANDALONE"): the "block" rule's acceptance function.
 *  [BLK] Sun et al. 2024, block verification (arXiv 2403.10444), which the
 *        page cites for the prefix weight's clipped recursion.
 *  [NEW] "New approaches to speculative decoding: block drafts, load-aware
 *        verification and PD disaggregation", anrans.github.io (AI infra
 *        handbooks): section "Deciding how much to verify by load" (the
 *        adaptive-verification planner and its worked example) and "The
 *        higher the load, the smaller K should be" (its cost model); with
 *        [ZOO] "The finer loop: DSpark's confidence budget" (the global
 *        top-k of survival scores, the earlier-position-first tie rule and
 *        the argmax of expected tokens over the cost table).
 *  [KV]  "投机解码" (Speculative decoding), rustineverything.app, section
 *        "与调度、KV 的交互" (interaction with scheduling and KV), sub-section
 *        "SGLang：按最坏情况预留，结束时归还": with topk > 1 the accepted path
 *        is not contiguous in the tree and its KV is moved to contiguous
 *        positions after verification; and "Draft sources: draft models,
 *        n-gram, suffix decoding" (mlinterviewnotes.com, section 6.3),
 *        "SGLang's suffix automaton, in tree": a tree's accepted path is
 *        scattered, so its KV is moved into the target cache.
 *  [PHX] Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
 *        1, 2, 3", SC'11 (Philox4x32-10), which the pages do not fix.
 *
 * Readings where the pages leave a step open (all listed in the design notes):
 *  - randomness is a counter-based Philox4x32-10 stream keyed by the request
 *    seed; the coin for row r of request b is word 0 of counter (0, r, b, 0);
 *    the race noise for vocab id y is word (y & 3) of counter (y>>2, r, b, 1);
 *    the chunk noise for chunk c is word 0 of counter (c, r, b, 2);
 *  - uniforms are (2*(w>>9)+1)/2^24, inside (0,1) and exact in fp32;
 *  - the acceptance test is strict (u*q < p); q(x) <= 0 accepts iff p(x) > 0;
 *  - block verification: the prefix weight is clipped at 1 at every step
 *    ([BLK]); its test is eta <= h as the page's kernel writes it, with
 *    eta_i the coin of draft row i - 1;
 *  - the residual / bonus sample is a two-level exponential race: the ids
 *    are cut into chunks of SVO_RACE_CHUNK; the chunk c maximising
 *    W_c / E_c (W_c its weight sum, E_c = -ln U_c) is chosen, then the id y
 *    of that chunk maximising w(y) / E_y, ties to the smaller index at both
 *    levels; an all-zero residual falls back to p;
 *  - argmax ties go to the smallest index, on raw logits;
 *  - T <= 0 means greedy, a non-finite T is rejected;
 *  - draft id -1 ends the chain; NaN/+inf logits or an all -inf row are
 *    rejected, -inf is a masked token.
 */
#include "svo.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 [PHX]: each round multiplies counter words 0 and 2 by the
 * two round multipliers, and the new counter is
 *   (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0));
 * between rounds the key is bumped by the two Weyl constants. */
#define SVO_PHILOX_M0 0xD2511F53u
#define SVO_PHILOX_M1 0xCD9E8D57u
#define SVO_PHILOX_W0 0x9E3779B9u
#define SVO_PHILOX_W1 0xBB67AE85u

void svo_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += SVO_PHILOX_W0;
      k1 += SVO_PHILOX_W1;
    }
    uint64_t prod0 = (uint64_t)SVO_PHILOX_M0 * (uint64_t)c0;
    uint64_t prod1 = (uint64_t)SVO_PHILOX_M1 * (uint64_t)c2;
    uint32_t hi0 = (uint32_t)(prod0 >> 32), lo0 = (uint32_t)prod0;
    uint32_t hi1 = (uint32_t)(prod1 >> 32), lo1 = (uint32_t)prod1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

double svo_uniform(uint32_t w) {
  uint32_t j = w >> 9; /* 23 bits */
  return (double)(2u * j + 1u) / 16777216.0; /* 2^24 */
}

static void seed_key(uint64_t seed, uint32_t key[2]) {
  key[0] = (uint32_t)(seed & 0xffffffffu);
  key[1] = (uint32_t)(seed >> 32);
}

double svo_coin(uint64_t seed, int32_t b, int32_t r) {
  uint32_t key[2], ctr[4] = {0u, (uint32_t)r, (uint32_t)b, 0u}, out[4];
  seed_key(seed, key);
  svo_philox4x32_10(ctr, key, out);
  return svo_uniform(out[0]);
}

double svo_chunk_uniform(uint64_t seed, int32_t b, int32_t r, int32_t c) {
  uint32_t key[2], ctr[4] = {(uint32_t)c, (uint32_t)r, (uint32_t)b, 2u}, out[4];
  seed_key(seed, key);
  svo_philox4x32_10(ctr, key, out);
  return svo_uniform(out[0]);
}

double svo_noise_uniform(uint64_t seed, int32_t b, int32_t r, int32_t y) {
  uint32_t key[2], ctr[4] = {(uint32_t)y >> 2, (uint32_t)r, (uint32_t)b, 1u}, out[4];
  seed_key(seed, key);
  svo_philox4x32_10(ctr, key, out);
  return svo_uniform(out[y & 3]);
}

/* ------------------------------------------------------------------------ */
/* Logit rows. */

static double logit_at(int32_t dtype, const void* base, int64_t idx) {
  if (dtype == SVO_BF16) {
    uint16_t h = ((const uint16_t*)base)[idx];
    uint32_t bits = (uint32_t)h << 16; /* bf16 is the top half of an fp32 */
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
  }
  return (double)((const float*)base)[idx];
}

/* One row's statistics: m = max, amax = smallest index attaining m, and for a
 * stochastic row S = sum_y exp((l_y - m)/T), left to right.  The target
 * distribution is p(y) = exp((l_y - m)/T)/S: the softmax of the tempered
 * logits ([SD] "接受规则为什么不改变分布": p is taken after temperature). */
typedef struct {
  double m, S;    /* S: the sum over the kept tokens (all tokens when the row is not filtered) */
  double tau;     /* tokens with a logit below tau are filtered out (-inf: none) */
  int32_t amax;
  int32_t status;
} row_stat;

static row_stat scan_row(int32_t dtype, const void* logits, int64_t row_off, int32_t V, double T, int stochastic) {
  row_stat st;
  st.m = -INFINITY;
  st.tau = -INFINITY;
  st.amax = 0;
  st.S = NAN;
  st.status = SVO_REQ_OK;
  for (int32_t y = 0; y < V; ++y) {
    double l = logit_at(dtype, logits, row_off + y);
    if (isnan(l) || (isinf(l) && l > 0)) st.status = SVO_REQ_NONFINITE;
    if (l > st.m) { /* strict: the first index of the max is kept */
      st.m = l;
      st.amax = y;
    }
  }
  if (st.m == -INFINITY) st.status = SVO_REQ_NONFINITE; /* every token masked */
  if (st.status != SVO_REQ_OK) return st;
  if (stochastic) {
    double S = 0.0;
    for (int32_t y = 0; y < V; ++y) S += exp((logit_at(dtype, logits, row_off + y) - st.m) / T);
    st.S = S;
  }
  return st;
}

static int is_finite_num(double x) { return !isnan(x) && !isinf(x); }

static double p_of(int32_t dtype, const void* logits, int64_t row_off, const row_stat* st, double T, int32_t y) {
  const double l = logit_at(dtype, logits, row_off + y);
  if (l < st->tau) return 0.0;
  return exp((l - st->m) / T) / st->S;
}

/* Top-k / top-p filtering of a stochastic row's target ([SD]
 * "接受规则为什么不改变分布": p is the target after temperature and top-k / top-p).
 * Top-k keeps the tokens whose logit is at least the k-th largest logit
 * (ties at it are kept); top-p then keeps, among those, the fewest
 * highest-probability tokens whose probability mass reaches p times the
 * top-k mass, whole groups of equal logits at a time (so the kept set is
 * again "logit >= threshold").  The row's p becomes p restricted to the kept
 * tokens and renormalised: st->tau is the threshold and st->S the kept sum
 * (left to right).  k <= 0 or k >= V, and p outside (0, 1), switch a filter
 * off.  *margin gets the top-p decision's relative gap (how far the chosen
 * group's cumulative mass, and the one before it, are from the target). */
static int cmp_desc(const void* x, const void* y) {
  const double a = *(const double*)x, b = *(const double*)y;
  return a > b ? -1 : (a < b ? 1 : 0);
}

static void filter_row(row_stat* st, int32_t dtype, const void* logits, int64_t row_off, int32_t V, double T,
                       int32_t topk, float topp, double* margin) {
  const int use_k = topk > 0 && topk < V, use_p = topp > 0.0f && topp < 1.0f;
  *margin = INFINITY;
  if (!use_k && !use_p) return;
  double* v = (double*)malloc(sizeof(double) * (size_t)V);
  for (int32_t y = 0; y < V; ++y) v[y] = logit_at(dtype, logits, row_off + y);
  qsort(v, (size_t)V, sizeof(double), cmp_desc);
  double tau = use_k ? v[topk - 1] : -INFINITY;
  if (use_p) {
    int32_t n = 0;
    double pk = 0.0;
    while (n < V && v[n] >= tau) pk += exp((v[n++] - st->m) / T);
    const double target = (double)topp * pk;
    double cum = 0.0;
    for (int32_t i = 0; i < n;) {
      int32_t j = i;
      double g = 0.0;
      while (j < n && v[j] == v[i]) g += exp((v[j++] - st->m) / T);
      const double prev = cum;
      cum += g;
      if (cum >= target) {
        tau = v[i];
        const double g1 = (cum - target) / target, g0 = (target - prev) / target;
        *margin = g1 < g0 ? g1 : g0;
        break;
      }
      i = j;
    }
  }
  free(v);
  double S = 0.0;
  for (int32_t y = 0; y < V; ++y) {
    const double l = logit_at(dtype, logits, row_off + y);
    if (l >= tau) S += exp((l - st->m) / T);
  }
  st->S = S;
  st->tau = tau;
}

void svo_row_stats(int32_t rows, int32_t vocab, int32_t dtype, const void* logits, int64_t row_stride,
                   const float* temperature, double* row_max, int32_t* row_argmax, double* row_sumexp,
                   int32_t* row_status) {
  for (int32_t i = 0; i < rows; ++i) {
    double T = (double)temperature[i];
    row_stat st = scan_row(dtype, logits, (int64_t)i * row_stride, vocab, T, T > 0.0 && is_finite_num(T));
    if (row_max) row_max[i] = st.m;
    if (row_argmax) row_argmax[i] = st.amax;
    if (row_sumexp) row_sumexp[i] = st.S;
    if (row_status) row_status[i] = st.status;
  }
}

/* ------------------------------------------------------------------------ */
/* Exponential race over non-negative weights, two levels.
 *
 * One level: y* = argmax_y w(y) / E_y with E_y = -ln U_y independent Exp(1)
 * variables gives P(y* = y) = w(y) / sum w, an exact sample of the
 * normalised weights (the Gumbel-max trick of the vLLM resample step quoted
 * in [SD] "采样：标准拒绝采样" is the same race in log space).
 *
 * Two levels: the ids are cut into consecutive chunks of `chunk` ids; first
 * the chunks race with their weight sums W_c and the chunk noise, then the
 * ids of the winning chunk race with their own weights and the id noise.
 * The chunk wins with probability W_c / sum W and, given the chunk, the id
 * with probability w(y) / W_c (the two noise streams are independent), so
 * the sample is still exact; a single chunk is the one-level race.
 *
 * Ties go to the smaller chunk and the smaller id.  Writes the smaller of
 * the two levels' relative gaps between their two largest keys to *margin
 * (the gap is 1 for a level with a single positive key). */
static double top_gap(double k1, double k2) {
  if (k2 < 0.0) k2 = 0.0;
  return (k1 > 0.0) ? (k1 - k2) / k1 : 0.0;
}

int32_t svo_race(const double* w, int32_t V, int32_t chunk, uint64_t seed, int32_t b, int32_t r,
                 double* margin) {
  const int32_t nchunk = (V + chunk - 1) / chunk;
  int32_t cbest = -1;
  double k1 = -1.0, k2 = -1.0;
  for (int32_t c = 0; c < nchunk; ++c) {
    const int32_t y1 = (c + 1) * chunk < V ? (c + 1) * chunk : V;
    double W = 0.0;
    for (int32_t y = c * chunk; y < y1; ++y) W += w[y];
    const double key = W / -log(svo_chunk_uniform(seed, b, r, c));
    if (key > k1) {
      k2 = k1;
      k1 = key;
      cbest = c;
    } else if (key > k2) {
      k2 = key;
    }
  }
  const double gap_chunk = top_gap(k1, k2);
  int32_t best = -1;
  k1 = -1.0;
  k2 = -1.0;
  const int32_t y0 = cbest * chunk, y1 = (cbest + 1) * chunk < V ? (cbest + 1) * chunk : V;
  for (int32_t y = y0; y < y1; ++y) {
    const double key = w[y] / -log(svo_noise_uniform(seed, b, r, y));
    if (key > k1) {
      k2 = k1;
      k1 = key;
      best = y;
    } else if (key > k2) {
      k2 = key;
    }
  }
  const double gap_id = top_gap(k1, k2);
  if (margin) *margin = gap_chunk < gap_id ? gap_chunk : gap_id;
  return best;
}

static int32_t race(const double* w, int32_t V, uint64_t seed, int32_t b, int32_t r, double* margin) {
  return svo_race(w, V, SVO_RACE_CHUNK, seed, b, r, margin);
}

/* Sample from normalize(w); if every weight is zero, from p instead. */
static int32_t emit_from(double* w, const double* p, int32_t V, uint64_t seed, int32_t b, int32_t r, double* margin) {
  double total = 0.0;
  for (int32_t y = 0; y < V; ++y) total += w[y];
  if (!(total > 0.0)) memcpy(w, p, sizeof(double) * (size_t)V);
  return race(w, V, seed, b, r, margin);
}

static double rel_gap(double a, double b) {
  double hi = a > b ? a : b;
  if (hi <= 0.0) return INFINITY;
  return fabs(a - b) / hi;
}

/* ------------------------------------------------------------------------ */
/* Block verification ([ZOO], the passage on vLLM's "block" rejection
 * method, which points to [BLK]).  Instead of
 * testing each draft against its own ratio, the rule keeps a prefix weight
 * w_i (w_0 = 1, w_{i+1} = min(w_i p_i(x_i) / q_i(x_i), 1): the page's
 * "prefix joint ratio", clipped at 1 at every step as in [BLK]) and,
 * for every prefix length i = 1..kb, an acceptance probability
 *   h_i = r_i / (r_i + 1 - w_i)   (1 when the denominator is 0),  i < kb,
 *   h_kb = w_kb,
 * where r_i = sum_y max(w_i p_i(y) - q_i(y), 0) is the residual mass at the
 * next position.  With one uniform eta_i per prefix length, the accepted
 * length is the largest i with eta_i <= h_i (0 if none), and the emitted
 * token is drawn from max(w_a p_a - q_a, 0) (a < kb) or from p_kb.  A
 * one-hot draft has q_i the point mass at x_i.  eta_i is the coin of the
 * draft's row, coin(b, i - 1), so one draft gives the standard rule up to
 * the comparison's tie.  Every decision's relative gap is logged. */

/* q_i(y) of draft row i of request b (one-hot drafts: the point mass at x). */
static double q_of(const svo_chain_args* a, int32_t b, int32_t i, int32_t x, int32_t y) {
  if (a->draft_kind == SVO_DRAFT_ONEHOT) return y == x ? 1.0 : 0.0;
  return (double)a->draft_probs[((int64_t)b * a->max_draft + i) * a->q_row_stride + y];
}

/* w(y) = max(w_i p_i(y) - q_i(y), 0) for every y; prow holds p_i. */
static void block_residual(const svo_chain_args* a, int32_t b, int32_t i, int32_t x, double wi, const double* prow,
                           double* w) {
  for (int32_t y = 0; y < a->vocab; ++y) {
    double d = wi * prow[y] - q_of(a, b, i, x, y);
    w[y] = d > 0.0 ? d : 0.0;
  }
}

/* Fills wpre[0..kb] and returns the accepted length. */
static int32_t block_decisions(const svo_chain_args* a, int32_t b, int32_t kb, const row_stat* st, const double* px,
                               double* wpre, double* min_margin, int32_t* n_dec) {
  const int32_t R = a->max_draft + 1, V = a->vocab;
  const int32_t* x = a->draft_ids + (int64_t)b * a->max_draft;
  const double T = (double)a->temperature[b];
  wpre[0] = 1.0;
  for (int32_t i = 0; i < kb; ++i) {
    double q = q_of(a, b, i, x[i], x[i]);
    double ratio = q > 0.0 ? px[i] / q : (px[i] > 0.0 ? INFINITY : 0.0);
    double w = wpre[i] * ratio;
    if (wpre[i] == 0.0 || ratio == 0.0) w = 0.0;
    wpre[i + 1] = w < 1.0 ? w : 1.0;
  }
  int32_t tau = 0;
  for (int32_t i = 1; i <= kb; ++i) {
    double h;
    if (i < kb) {
      int64_t off = ((int64_t)b * R + i) * a->logits_row_stride;
      double r = 0.0;
      for (int32_t y = 0; y < V; ++y) {
        double d = wpre[i] * p_of(a->logits_dtype, a->logits, off, &st[i], T, y) - q_of(a, b, i, x[i], y);
        if (d > 0.0) r += d;
      }
      double den = r + 1.0 - wpre[i];
      h = den > 0.0 ? r / den : 1.0;
    } else {
      h = wpre[kb];
    }
    double eta = svo_coin(a->seed[b], b, i - 1);
    ++*n_dec;
    double g = rel_gap(eta, h);
    if (g < *min_margin) *min_margin = g;
    if (eta <= h) tau = i;
  }
  return tau;
}

/* ------------------------------------------------------------------------ */
/* Chain verification of one request.
 *
 * [SD] "采样：标准拒绝采样": accept x_i with probability min(1, p(x_i)/q(x_i)),
 * left to right; on the first rejection sample from max(0, p - q)/Z and drop
 * the remaining drafts; when all k are accepted sample one more token from
 * row k.  The ratio test is done as u*q(x) < p(x) (strict), as in the
 * quoted engine kernels.  [SD] "对照：mistral.rs": q(x) <= 0 accepts iff
 * p(x) > 0.  [SD] "默认路径：草稿当 one-hot": with a one-hot draft q(x) = 1, so
 * the test is u < p(x) and the residual is p with x zeroed.  [SD] "贪心"
 * and [ZOO] DFlash: with T = 0 a draft is accepted iff it equals the target
 * argmax, a rejection emits the argmax, and the bonus is the argmax of the
 * next row. */
static void chain_one(const svo_chain_args* a, int32_t b, double* w, double* prow) {
  const int32_t k = a->max_draft, V = a->vocab, R = k + 1;
  int32_t* tok = a->tokens + (int64_t)b * R;
  double* pd = a->p_draft ? a->p_draft + (int64_t)b * k : NULL;
  double min_margin = INFINITY;
  int32_t n_dec = 0;
  int32_t status = SVO_REQ_OK;

  for (int32_t i = 0; i < R; ++i) tok[i] = -1;
  if (pd)
    for (int32_t i = 0; i < k; ++i) pd[i] = NAN;
  a->accept_len[b] = 0;

  /* 1. validation */
  double T = (double)a->temperature[b];
  const int32_t* x = a->draft_ids + (int64_t)b * k;
  int32_t kb = k;
  for (int32_t i = 0; i < k; ++i)
    if (x[i] == -1) {
      kb = i;
      break;
    }
  if (!is_finite_num(T)) status = SVO_REQ_BAD_TEMPERATURE;
  for (int32_t i = 0; i < kb && status == SVO_REQ_OK; ++i)
    if (x[i] < 0 || x[i] >= V) status = SVO_REQ_BAD_DRAFT_ID;
  const int greedy = (T <= 0.0);

  /* 2. row statistics of the rows that are read: 0..kb */
  row_stat st[R > 0 ? R : 1];
  if (status == SVO_REQ_OK) {
    for (int32_t r = 0; r <= kb; ++r) {
      st[r] = scan_row(a->logits_dtype, a->logits, ((int64_t)b * R + r) * a->logits_row_stride, V, T, !greedy);
      if (st[r].status != SVO_REQ_OK) status = st[r].status;
    }
  }
  double cut_margin = INFINITY;
  if (status == SVO_REQ_OK && !greedy && (a->top_k || a->top_p)) {
    for (int32_t r = 0; r <= kb; ++r) {
      double g;
      filter_row(&st[r], a->logits_dtype, a->logits, ((int64_t)b * R + r) * a->logits_row_stride, V, T,
                 a->top_k ? a->top_k[b] : 0, a->top_p ? a->top_p[b] : 1.0f, &g);
      if (g < cut_margin) cut_margin = g;
    }
  }
  if (status != SVO_REQ_OK) {
    if (a->req_status) a->req_status[b] = status;
    if (a->min_margin) a->min_margin[b] = INFINITY;
    if (a->cut_margin) a->cut_margin[b] = INFINITY;
    if (a->n_decisions) a->n_decisions[b] = 0;
    return;
  }

  /* p_i(x_i) for every used draft slot */
  double px[k > 0 ? k : 1];
  for (int32_t i = 0; i < kb; ++i) {
    int64_t off = ((int64_t)b * R + i) * a->logits_row_stride;
    if (greedy)
      px[i] = (x[i] == st[i].amax) ? 1.0 : 0.0; /* point mass at the argmax */
    else
      px[i] = p_of(a->logits_dtype, a->logits, off, &st[i], T, x[i]);
    if (pd) pd[i] = px[i];
  }

  /* 3. decisions: block verification, or left to right stopping at the
   *    first rejection */
  int32_t acc = 0;
  double wpre[k + 1];  /* block rule: prefix weights w_0..w_kb */
  wpre[0] = 1.0;
  if (!greedy && a->rule == SVO_RULE_BLOCK) {
    acc = block_decisions(a, b, kb, st, px, wpre, &min_margin, &n_dec);
    for (int32_t i = 0; i < acc; ++i) tok[i] = x[i];
  }
  for (int32_t i = 0; i < kb && (greedy || a->rule != SVO_RULE_BLOCK); ++i) {
    int accept;
    ++n_dec;
    if (greedy) {
      accept = (x[i] == st[i].amax);
    } else if (a->draft_kind == SVO_DRAFT_ONEHOT) {
      double u = svo_coin(a->seed[b], b, i);
      accept = (u < px[i]);
      double g = rel_gap(u, px[i]);
      if (g < min_margin) min_margin = g;
    } else {
      double q = (double)a->draft_probs[((int64_t)b * k + i) * a->q_row_stride + x[i]];
      if (q <= 0.0) {
        accept = (px[i] > 0.0);
      } else {
        double u = svo_coin(a->seed[b], b, i);
        accept = (u * q < px[i]);
        double g = rel_gap(u * q, px[i]);
        if (g < min_margin) min_margin = g;
      }
    }
    if (!accept) break;
    tok[acc] = x[i];
    ++acc;
  }

  /* 4. one token from row acc: the residual after a rejection, the bonus
   *    after full acceptance */
  int32_t emitted;
  ++n_dec;
  if (greedy) {
    emitted = st[acc].amax;
  } else {
    int64_t off = ((int64_t)b * R + acc) * a->logits_row_stride;
    for (int32_t y = 0; y < V; ++y) prow[y] = p_of(a->logits_dtype, a->logits, off, &st[acc], T, y);
    if (acc < kb && a->rule == SVO_RULE_BLOCK) {
      /* block rule: the residual of the prefix-weighted target,
       * max(w_acc p - q, 0), q the draft row (one-hot: the point mass) */
      block_residual(a, b, acc, x[acc], wpre[acc], prow, w);
    } else if (acc < kb && a->draft_kind == SVO_DRAFT_PROBS) {
      const float* qrow = a->draft_probs + ((int64_t)b * k + acc) * a->q_row_stride;
      for (int32_t y = 0; y < V; ++y) {
        double d = prow[y] - (double)qrow[y];
        w[y] = d > 0.0 ? d : 0.0;
      }
    } else if (acc < kb) {
      for (int32_t y = 0; y < V; ++y) w[y] = prow[y];
      w[x[acc]] = 0.0;
    } else {
      for (int32_t y = 0; y < V; ++y) w[y] = prow[y];
    }
    double g;
    emitted = emit_from(w, prow, V, a->seed[b], b, acc, &g);
    if (g < min_margin) min_margin = g;
  }
  tok[acc] = emitted;
  a->accept_len[b] = acc;
  if (a->req_status) a->req_status[b] = SVO_REQ_OK;
  if (a->min_margin) a->min_margin[b] = min_margin;
  if (a->cut_margin) a->cut_margin[b] = cut_margin;
  if (a->n_decisions) a->n_decisions[b] = n_dec;
}

void svo_verify_chain(const svo_chain_args* a) {
  double* w = (double*)malloc(sizeof(double) * (size_t)(a->vocab > 0 ? a->vocab : 1));
  double* prow = (double*)malloc(sizeof(double) * (size_t)(a->vocab > 0 ? a->vocab : 1));
  for (int32_t b = 0; b < a->batch; ++b) chain_one(a, b, w, prow);
  free(w);
  free(prow);
}

/* ------------------------------------------------------------------------ */
/* Target-only tree verification of one request ([SD] "SGLang 默认：只看目标概率，
 * 可以验证一棵树").  Node 0 is the root; row n is the target distribution after
 * node n.  At each level one coin u is drawn; the children of the current
 * node are tried in increasing node index, accumulating their target
 * probabilities, and child j is accepted if p(tok_j) > 0 and u < acc_j.  If
 * none is accepted, the tried children's probability is removed from p and
 * the next token is drawn from what is left; at a leaf the bonus is drawn
 * from p.  Greedy mode follows the argmax through the tree. */
static void tree_one(const svo_tree_args* a, int32_t b, double* w, double* prow) {
  const int32_t N = a->num_nodes, V = a->vocab;
  int32_t* path = a->accept_path + (int64_t)b * N;
  int32_t* tok = a->tokens + (int64_t)b * N;
  const int32_t* ntok = a->node_tokens + (int64_t)b * N;
  const int32_t* par = a->parent + (int64_t)b * N;
  double min_margin = INFINITY;
  int32_t n_dec = 0;
  int32_t status = SVO_REQ_OK;

  for (int32_t i = 0; i < N; ++i) {
    path[i] = -1;
    tok[i] = -1;
  }
  a->accept_len[b] = 0;

  double T = (double)a->temperature[b];
  if (!is_finite_num(T)) status = SVO_REQ_BAD_TEMPERATURE;
  if (status == SVO_REQ_OK) {
    if (par[0] != -1) status = SVO_REQ_BAD_TREE;
    for (int32_t i = 1; i < N && status == SVO_REQ_OK; ++i) {
      if (par[i] < 0 || par[i] >= i) status = SVO_REQ_BAD_TREE;
      if (ntok[i] < 0 || ntok[i] >= V) status = SVO_REQ_BAD_TREE;
    }
    for (int32_t i = 1; i < N && status == SVO_REQ_OK; ++i)
      for (int32_t j = i + 1; j < N; ++j)
        if (par[i] == par[j] && ntok[i] == ntok[j]) status = SVO_REQ_BAD_TREE;
  }
  const int greedy = (T <= 0.0);
  row_stat st[N > 0 ? N : 1];
  if (status == SVO_REQ_OK) {
    for (int32_t n = 0; n < N; ++n) {
      st[n] = scan_row(a->logits_dtype, a->logits, ((int64_t)b * N + n) * a->logits_row_stride, V, T, !greedy);
      if (st[n].status != SVO_REQ_OK) status = st[n].status;
    }
  }
  double cut_margin = INFINITY;
  if (status == SVO_REQ_OK && !greedy && (a->top_k || a->top_p)) {
    for (int32_t n = 0; n < N; ++n) {
      double g;
      filter_row(&st[n], a->logits_dtype, a->logits, ((int64_t)b * N + n) * a->logits_row_stride, V, T,
                 a->top_k ? a->top_k[b] : 0, a->top_p ? a->top_p[b] : 1.0f, &g);
      if (g < cut_margin) cut_margin = g;
    }
  }
  if (status != SVO_REQ_OK) {
    if (a->req_status) a->req_status[b] = status;
    if (a->min_margin) a->min_margin[b] = INFINITY;
    if (a->cut_margin) a->cut_margin[b] = INFINITY;
    if (a->n_decisions) a->n_decisions[b] = 0;
    return;
  }

  int32_t cur = 0, len = 0, emitted = -1;
  for (;;) {
    int64_t off = ((int64_t)b * N + cur) * a->logits_row_stride;
    int32_t nchild = 0;
    for (int32_t c = cur + 1; c < N; ++c)
      if (par[c] == cur) ++nchild;
    ++n_dec;
    if (greedy) {
      int32_t next = -1;
      for (int32_t c = cur + 1; c < N; ++c)
        if (par[c] == cur && ntok[c] == st[cur].amax) next = c;
      if (next < 0) {
        emitted = st[cur].amax;
        break;
      }
      path[len] = next;
      tok[len] = ntok[next];
      ++len;
      cur = next;
      continue;
    }
    if (nchild == 0) { /* leaf: bonus token from p_cur */
      for (int32_t y = 0; y < V; ++y) prow[y] = p_of(a->logits_dtype, a->logits, off, &st[cur], T, y);
      for (int32_t y = 0; y < V; ++y) w[y] = prow[y];
      double g;
      emitted = emit_from(w, prow, V, a->seed[b], b, cur, &g);
      if (g < min_margin) min_margin = g;
      break;
    }
    double u = svo_coin(a->seed[b], b, cur);
    double acc = 0.0;
    int32_t next = -1;
    for (int32_t c = cur + 1; c < N; ++c) {
      if (par[c] != cur) continue;
      double pc = p_of(a->logits_dtype, a->logits, off, &st[cur], T, ntok[c]);
      acc += pc;
      double g = rel_gap(u, acc);
      if (g < min_margin) min_margin = g;
      if (pc > 0.0 && (u < acc / a->threshold_acc || pc >= a->threshold_single)) {
        next = c;
        break;
      }
    }
    if (next >= 0) {
      path[len] = next;
      tok[len] = ntok[next];
      ++len;
      cur = next;
      continue;
    }
    /* no child accepted: p with every tried child's token removed */
    for (int32_t y = 0; y < V; ++y) prow[y] = p_of(a->logits_dtype, a->logits, off, &st[cur], T, y);
    for (int32_t y = 0; y < V; ++y) w[y] = prow[y];
    for (int32_t c = cur + 1; c < N; ++c)
      if (par[c] == cur) w[ntok[c]] = 0.0;
    ++n_dec;
    double g;
    emitted = emit_from(w, prow, V, a->seed[b], b, cur, &g);
    if (g < min_margin) min_margin = g;
    break;
  }
  tok[len] = emitted;
  a->accept_len[b] = len;
  if (a->req_status) a->req_status[b] = SVO_REQ_OK;
  if (a->min_margin) a->min_margin[b] = min_margin;
  if (a->cut_margin) a->cut_margin[b] = cut_margin;
  if (a->n_decisions) a->n_decisions[b] = n_dec;
}

void svo_verify_tree(const svo_tree_args* a) {
  double* w = (double*)malloc(sizeof(double) * (size_t)(a->vocab > 0 ? a->vocab : 1));
  double* prow = (double*)malloc(sizeof(double) * (size_t)(a->vocab > 0 ? a->vocab : 1));
  for (int32_t b = 0; b < a->batch; ++b) tree_one(a, b, w, prow);
  free(w);
  free(prow);
}

/* ------------------------------------------------------------------------ */
/* Survival top-k draft budget ([NEW] "Deciding how much to verify by load";
 * [ZOO] "The finer loop: DSpark's confidence budget").  A (request,
 * position) slot's score is the chance that the request's drafts all pass up
 * to that position: the product of its confidences so far (in fp32, as the
 * pages' cumprod of fp32 confidences); the slots are ranked by score, higher first,
 * ties to the earlier position and then to the smaller request index (the
 * deterministic tie rule [ZOO] asks for, which makes every request's
 * admitted slots a prefix).  Admitting the top B slots yields
 * base + (sum of their scores) expected tokens at cost[B]; the budget is the
 * B in 0..min(max_budget, slots) that maximises their ratio (the first
 * maximum).  Confidences are clamped to [0, 1] (NaN counts as 0), so scores
 * never increase along a request. */
typedef struct {
  float s;
  int32_t j, b;
} plan_slot;

static int plan_order(const void* x, const void* y) {
  const plan_slot* p = (const plan_slot*)x;
  const plan_slot* q = (const plan_slot*)y;
  if (p->s != q->s) return p->s > q->s ? -1 : 1;
  if (p->j != q->j) return p->j < q->j ? -1 : 1;
  return p->b < q->b ? -1 : (p->b > q->b ? 1 : 0);
}

void svo_plan_budget(const svo_plan_args* a) {
  const int32_t bs = a->batch, K = a->max_steps;
  plan_slot* slot = (plan_slot*)malloc(sizeof(plan_slot) * (size_t)(bs * K > 0 ? bs * K : 1));
  int32_t n = 0;
  for (int32_t b = 0; b < bs; ++b) {
    int32_t len = a->num_steps ? a->num_steps[b] : K;
    if (len < 0) len = 0;
    if (len > K) len = K;
    float s = 1.0f;
    for (int32_t j = 0; j < len; ++j) {
      float c = a->confidence[(int64_t)b * K + j];
      if (!(c > 0.0f)) c = 0.0f; /* NaN and negatives */
      if (c > 1.0f) c = 1.0f;
      s = s * c;
      slot[n].s = s;
      slot[n].j = j;
      slot[n].b = b;
      ++n;
    }
  }
  qsort(slot, (size_t)n, sizeof(plan_slot), plan_order);
  const int32_t bmax = a->max_budget < n ? a->max_budget : n;
  double* rate = (double*)malloc(sizeof(double) * (size_t)(bmax + 1));
  double gain = 0.0, best = -INFINITY;
  int32_t bstar = 0;
  for (int32_t B = 0; B <= bmax; ++B) {
    if (B > 0) gain += (double)slot[B - 1].s;
    rate[B] = (a->base_tokens + gain) / a->cost[B];
    if (rate[B] > best) {
      best = rate[B];
      bstar = B;
    }
  }
  double gap = INFINITY;
  for (int32_t B = 0; B <= bmax; ++B)
    if (B != bstar && rate[B] != best && best > 0.0) {
      double g = (best - rate[B]) / best;
      if (g < gap) gap = g;
    }
  for (int32_t b = 0; b < bs; ++b) a->draft_len[b] = 0;
  for (int32_t r = 0; r < bstar; ++r) a->draft_len[slot[r].b] += 1;
  *a->budget = bstar;
  *a->rate = best;
  if (a->margin) *a->margin = gap;
  free(rate);
  free(slot);
}

/* ------------------------------------------------------------------------ */
/* Accepted-path KV compaction ([KV]).  After tree verification the accepted
 * nodes p_1..p_a (from the root down; node 0, the root, is already in
 * place) hold their KV rows wherever the tree put them.  Their rows move,
 * in path order, to the slots of nodes 1..a, so the accepted tokens follow
 * the committed prefix contiguously: for i = 1..a, every layer's row at
 * node_slot[p_i] is copied to node_slot[i] (a no-op when p_i = i).  Node
 * ids grow along a path, so p_i >= i and a copy never reads a slot that an
 * earlier copy of the same request wrote; doing them in order is the
 * definition.  A request whose accept_len or path lies outside the tree,
 * or whose slots lie outside the pool, is left untouched (moved = -1). */
void svo_compact_kv(const svo_compact_args* a) {
  const int32_t N = a->num_nodes;
  for (int32_t b = 0; b < a->batch; ++b) {
    const int32_t len = a->accept_len[b];
    const int32_t* path = a->accept_path + (int64_t)b * N;
    const int64_t* slot = a->node_slot + (int64_t)b * N;
    int ok = len >= 0 && len < N;
    for (int32_t i = 0; ok && i < len; ++i) {
      const int32_t p = path[i];
      if (p < i + 1 || p >= N || (i > 0 && p <= path[i - 1])) ok = 0;
      else if (slot[p] < 0 || slot[p] >= a->num_slots || slot[i + 1] < 0 || slot[i + 1] >= a->num_slots) ok = 0;
    }
    if (!ok) {
      if (a->moved) a->moved[b] = -1;
      continue;
    }
    int32_t moved = 0;
    for (int32_t i = 0; i < len; ++i) {
      const int32_t p = path[i];
      if (p == i + 1) continue;
      ++moved;
      for (int32_t l = 0; l < a->num_layers; ++l) {
        uint8_t* base = a->kv + (int64_t)l * a->layer_stride;
        memmove(base + slot[i + 1] * a->slot_stride, base + slot[p] * a->slot_stride, (size_t)a->row_bytes);
      }
    }
    if (a->moved) a->moved[b] = moved;
  }
}
