/*
 * Reference ("oracle") for single-query paged decode attention with GQA.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct CPU
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no code, header, table or helper with the HIP library under
 * paged_kv_decode_amd/, and the library never calls it.
 *
 * What is computed (the operation the AstrAI commit log for
 * csrc/kernels/attn_paged_decode_split_kv_mma.cuh builds kernels for, and the
 * "Paged attention" row of the b12x 0.30.0 kernel inventory lists as
 * decode over BF16 or FP8-E4M3 paged KV caches with GQA):
 *
 *   for every sequence b and query head h, with G = Hq / Hkv query heads per
 *   KV head, kv(h) = floor(h / G) and L = seq_lens[b]:
 *     token t in [0, L) lives in physical page p = block_table[b][t / ps],
 *     slot t % ps; its key/value rows are K[p][slot][kv(h)][:] and V[...].
 *     s_t   = scale * sum_d q[b][h][d] * k_t[d]
 *     m     = max_t s_t,  Z = sum_t exp(s_t - m)
 *     lse   = m + ln Z                       (natural log)
 *     out[d]= sum_t exp(s_t - m) * v_t[d] / Z
 *   L = 0 gives out = 0 and lse = -inf (no page is read).
 *
 * Everything is fp64, two-pass (max first, then sums), in token order, with no
 * tiling, blocking or fusion.  BF16 values are decoded from their bit patterns
 * (the upper half of an IEEE binary32), FP8 values from the OCP E4M3FN
 * definition (bias 7, no infinities, S.1111.111 is NaN) and multiplied by the
 * per-KV-head fp32 scale.
 *
 * The split form (pkd_oracle_paged_decode_split) cuts each sequence into
 * num_splits contiguous ranges, computes each range by the same definition and
 * recombines the ranges with the log-sum-exp merge (pkd_oracle_lse_merge).  It
 * exists to pin the merge algebra that split-KV decoding relies on (the AstrAI
 * log's split partials; the b12x "split-KV or direct output" variants and its
 * PagedPersistentMergeKernel; the merge_attn_states row of the sglang
 * fuse/overlap catalogue, vLLM section).
 *
 * Several query tokens per sequence (pkd_oracle_paged_decode_multi): the
 * speculative-verify / extend form that the b12x "Paged attention" row lists
 * beside decode, and that the AstrAI log's causal offset (the position of the
 * first query token) describes.  Each sequence b has q_len query tokens whose
 * rows are q[b][i][h][:], i in [0, q_len); the query tokens are the last
 * q_len positions of the sequence, so token i sits at position L - q_len + i.
 * Without the causal mask every query token attends over all L tokens; with
 * it, query token i attends over tokens t <= L - q_len + i only, i.e. over the
 * first clamp(L - q_len + i + 1, 0, L) tokens (none when that is <= 0: out =
 * 0, lse = -inf).  Each query token is then exactly the single-token
 * definition above over its visible tokens.  q_len = 1 without the mask is the
 * single-token decode.
 *
 * Sliding window and attention sinks (pkd_oracle_paged_decode_ext): the b12x
 * "Paged attention" row lists sliding-window attention and an attention-sink
 * bias among its variants.  With a window W > 0, query token i (at position
 * p = L - q_len + i) attends only over positions t > p - W (besides the causal
 * limit, if any); for plain decode that is the last W tokens.  With sinks,
 * query head h has a logit sink[h] that joins the softmax denominator without
 * a value row:
 *     out = sum_t exp(s_t) v_t / (exp(sink[h]) + sum_t exp(s_t)),
 *     lse = ln(exp(sink[h]) + sum_t exp(s_t)),
 * so a token that sees no position gets out = 0 and lse = sink[h].  The
 * oracle computes the plain result over the visible tokens, then folds the sink
 * in: lse' = ln(e^lse + e^sink), out' = out * e^(lse - lse').
 *
 * The file also defines the paged KV append that fills the cache
 * (pkd_oracle_kv_append), the decode metadata preparation that builds the
 * block table and lengths (pkd_oracle_decode_metadata) and decode over a
 * contiguous, strided KV layout (pkd_oracle_contiguous_decode), at the end.
 *
 * Work is spread over an optional pthread pool by (sequence, KV head) items.
 * The items are independent and each is computed in a fixed order, so the
 * result is bitwise identical for any thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Status codes returned by the oracle entry points. */
#define PKD_ORACLE_OK 0
#define PKD_ORACLE_BAD_ARG (-1)
#define PKD_ORACLE_BAD_PAGE (-2)   /* a used block-table entry is outside [0, num_pages) */
#define PKD_ORACLE_BAD_LEN (-3)    /* seq_len < 0 or > max_pages_per_seq * page_size */
#define PKD_ORACLE_NO_MEM (-4)

/* ---- scalar decoders ---------------------------------------------------- */

/* bfloat16: the 16 high-order bits of an IEEE-754 binary32. */
double pkd_oracle_bf16_value(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP 8-bit floating point, E4M3FN variant: 1 sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits.  Exponent field 0 encodes subnormals
 * (m/8 * 2^-6); exponent 15 with mantissa 7 is NaN; there is no infinity. */
double pkd_oracle_fp8e4m3_value(uint8_t code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double mag;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, 1 - 7);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* ---- problem description ------------------------------------------------ */

typedef struct {
  int batch, hq, hkv, head_dim, page_size, num_pages, max_pages, kv_fp8;
  const uint16_t* q;          /* [B][Hq][D] bf16 bits */
  const void* k_cache;        /* [num_pages][ps][Hkv][D], bf16 bits or fp8 codes */
  const void* v_cache;
  const int32_t* block_table; /* [B][max_pages] */
  const int32_t* seq_lens;    /* [B] */
  const float* k_scale;       /* [Hkv], fp8 only */
  const float* v_scale;
  double scale;
  int num_splits;             /* 0: plain definition; >= 1: split form */
  double* out;                /* [B][q_len][Hq][D] */
  double* lse;                /* [B][q_len][Hq] */
  int q_len;                  /* query tokens per sequence, >= 1 */
  int causal;                 /* 0: every query token sees all L tokens; 1: causal mask */
  int window;                 /* 0: no window; > 0: positions t > p - window only */
  const float* sinks;         /* [Hq] sink logits, or NULL */
  /* Contiguous (strided) layout, used when kv_strides is not NULL: key
   * element (b, t, g, d) is k_cache[b*s[0] + t*s[1] + g*s[2] + d] (s =
   * kv_strides, in elements) and no block table is used; page_size is then
   * the token capacity of each sequence.  q_strides (or NULL: dense) likewise
   * places query row (b, i, h) at q[b*s[0] + i*s[1] + h*s[2]]. */
  const int64_t* kv_strides;
  const int64_t* q_strides;
} problem;

/* Value of element d of token t's key (is_v = 0) or value (is_v = 1) row for
 * KV head g of sequence b; the page lookup is the per-token one described
 * above.  Page validity is checked by the caller. */
static double kv_elem(const problem* P, int is_v, int b, int t, int g, int d) {
  int64_t idx;
  if (P->kv_strides) {
    idx = (int64_t)b * P->kv_strides[0] + (int64_t)t * P->kv_strides[1] + (int64_t)g * P->kv_strides[2] + d;
  } else {
    int32_t page = P->block_table[(int64_t)b * P->max_pages + t / P->page_size];
    int slot = t % P->page_size;
    idx = (((int64_t)page * P->page_size + slot) * P->hkv + g) * P->head_dim + d;
  }
  if (P->kv_fp8) {
    const uint8_t* c = (const uint8_t*)(is_v ? P->v_cache : P->k_cache);
    const float* sc = is_v ? P->v_scale : P->k_scale;
    return pkd_oracle_fp8e4m3_value(c[idx]) * (double)sc[g];
  }
  const uint16_t* c = (const uint16_t*)(is_v ? P->v_cache : P->k_cache);
  return pkd_oracle_bf16_value(c[idx]);
}

/* Tokens visible to query token qi of sequence b: all L without the causal
 * mask, else those at positions <= L - q_len + qi. */
static int visible_tokens(const problem* P, int b, int qi) {
  const int L = P->seq_lens[b];
  if (!P->causal) return L;
  const int v = L - P->q_len + qi + 1;
  return v < 0 ? 0 : (v > L ? L : v);
}

/* First position visible to query token qi of sequence b (the window's lower
 * end; 0 without a window), never past visible_tokens. */
static int first_visible(const problem* P, int b, int qi) {
  const int V = visible_tokens(P, b, qi);
  if (P->window <= 0) return 0;
  const int p = P->seq_lens[b] - P->q_len + qi;  /* the query token's position */
  int lo = p - P->window + 1;
  if (lo < 0) lo = 0;
  return lo < V ? lo : V;
}

/* Folds query head h's sink logit into a finished row (see the top of the
 * file): lse' = ln(e^lse + e^sink), out' = out e^(lse - lse'). */
static double apply_sink(const problem* P, int h, double lse, double* o) {
  if (!P->sinks) return lse;
  const double sk = (double)P->sinks[h];
  if (sk == -INFINITY) return lse;
  if (lse == -INFINITY) {
    for (int d = 0; d < P->head_dim; ++d) o[d] = 0.0;
    return sk;
  }
  const double mx = lse > sk ? lse : sk;
  const double l2 = mx + log(exp(lse - mx) + exp(sk - mx));
  const double f = exp(lse - l2);
  for (int d = 0; d < P->head_dim; ++d) o[d] *= f;
  return l2;
}

/* Attention of query token qi, head h of sequence b over tokens [t0, t1), by
 * the plain two-pass definition.  Writes D values to o and returns the
 * natural-log LSE; an empty range gives o = 0 and lse = -inf.  `s` is caller
 * scratch of at least t1 - t0 doubles. */
static double attend_range(const problem* P, int b, int qi, int h, int t0, int t1, double* o, double* s) {
  const int D = P->head_dim;
  const int G = P->hq / P->hkv;
  const int g = h / G;
  const uint16_t* qrow = P->q_strides ? P->q + (int64_t)b * P->q_strides[0] + (int64_t)qi * P->q_strides[1] +
                                             (int64_t)h * P->q_strides[2]
                                       : P->q + (((int64_t)b * P->q_len + qi) * P->hq + h) * D;
  for (int d = 0; d < D; ++d) o[d] = 0.0;
  if (t1 <= t0) return -INFINITY;

  double m = -INFINITY;
  for (int t = t0; t < t1; ++t) {
    double acc = 0.0;
    for (int d = 0; d < D; ++d) acc += pkd_oracle_bf16_value(qrow[d]) * kv_elem(P, 0, b, t, g, d);
    s[t - t0] = P->scale * acc;
    if (s[t - t0] > m) m = s[t - t0];
  }
  double z = 0.0;
  for (int t = t0; t < t1; ++t) {
    double w = exp(s[t - t0] - m);
    z += w;
    for (int d = 0; d < D; ++d) o[d] += w * kv_elem(P, 1, b, t, g, d);
  }
  for (int d = 0; d < D; ++d) o[d] /= z;
  return m + log(z);
}

/* Log-sum-exp merge of S partial results of one row: each partial j is a
 * normalised output o_j (D values) with its log-sum-exp lse_j.  The merged
 * row is the attention over the union of the partials' token ranges:
 *   M = max_j lse_j;  lse = M + ln sum_j exp(lse_j - M);
 *   out = sum_j exp(lse_j - lse) * o_j.
 * A partial with lse_j = -inf (an empty range) has weight 0; if every partial
 * is empty the row is out = 0, lse = -inf. */
static double merge_row(int S, int D, const double* o_part, const double* lse_part, double* out) {
  double M = -INFINITY;
  for (int j = 0; j < S; ++j)
    if (lse_part[j] > M) M = lse_part[j];
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  if (M == -INFINITY) return -INFINITY;
  double z = 0.0;
  for (int j = 0; j < S; ++j) z += exp(lse_part[j] - M);
  double lse = M + log(z);
  for (int j = 0; j < S; ++j) {
    double w = exp(lse_part[j] - lse);
    for (int d = 0; d < D; ++d) out[d] += w * o_part[(int64_t)j * D + d];
  }
  return lse;
}

void pkd_oracle_lse_merge(int64_t rows, int num_splits, int head_dim, const double* o_part,
                          const double* lse_part, double* out, double* lse) {
  for (int64_t r = 0; r < rows; ++r)
    lse[r] = merge_row(num_splits, head_dim, o_part + r * num_splits * head_dim,
                       lse_part + r * num_splits, out + r * head_dim);
}

/* ---- work items ---------------------------------------------------------- */

typedef struct {
  const problem* P;
  int next;           /* shared item counter, guarded by mu */
  int status;
  pthread_mutex_t mu;
} pool;

static int check_sequence(const problem* P, int b) {
  int L = P->seq_lens[b];
  if (L < 0 || (int64_t)L > (int64_t)P->max_pages * P->page_size) return PKD_ORACLE_BAD_LEN;
  if (P->kv_strides) return PKD_ORACLE_OK;
  int used = (L + P->page_size - 1) / P->page_size;
  for (int i = 0; i < used; ++i) {
    int32_t p = P->block_table[(int64_t)b * P->max_pages + i];
    if (p < 0 || p >= P->num_pages) return PKD_ORACLE_BAD_PAGE;
  }
  return PKD_ORACLE_OK;
}

/* One item = one (sequence, KV head): all G query heads of that KV head. */
static int run_item(const problem* P, int item) {
  const int G = P->hq / P->hkv;
  const int D = P->head_dim;
  const int b = item / P->hkv;
  const int g = item % P->hkv;
  const int L = P->seq_lens[b];
  double* s = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
  if (!s) return PKD_ORACLE_NO_MEM;
  int S = P->num_splits;
  double* op = NULL;
  double* lp = NULL;
  if (S >= 1) {
    op = (double*)malloc(sizeof(double) * (size_t)S * D);
    lp = (double*)malloc(sizeof(double) * (size_t)S);
    if (!op || !lp) {
      free(s); free(op); free(lp);
      return PKD_ORACLE_NO_MEM;
    }
  }
  for (int qi = 0; qi < P->q_len; ++qi) {
    const int V = visible_tokens(P, b, qi);
    const int lo = first_visible(P, b, qi);
    for (int h = g * G; h < (g + 1) * G; ++h) {
      const int64_t row = ((int64_t)b * P->q_len + qi) * P->hq + h;
      double* o = P->out + row * D;
      double* l = P->lse + row;
      if (S < 1) {
        *l = attend_range(P, b, qi, h, lo, V, o, s);
      } else {
        /* split j covers [lo + j*c, min(lo + (j+1)*c, V)) with c = ceil((V - lo) / S) */
        int c = (V - lo + S - 1) / S;
        for (int j = 0; j < S; ++j) {
          int t0 = lo + j * c, t1 = lo + (j + 1) * c;
          if (t0 > V) t0 = V;
          if (t1 > V) t1 = V;
          lp[j] = attend_range(P, b, qi, h, t0, t1, op + (int64_t)j * D, s);
        }
        *l = merge_row(S, D, op, lp, o);
      }
      *l = apply_sink(P, h, *l, o);
    }
  }
  free(s); free(op); free(lp);
  return PKD_ORACLE_OK;
}

static void* worker(void* arg) {
  pool* W = (pool*)arg;
  const int n_items = W->P->batch * W->P->hkv;
  for (;;) {
    pthread_mutex_lock(&W->mu);
    int item = W->next++;
    pthread_mutex_unlock(&W->mu);
    if (item >= n_items) break;
    int st = run_item(W->P, item);
    if (st != PKD_ORACLE_OK) {
      pthread_mutex_lock(&W->mu);
      W->status = st;
      pthread_mutex_unlock(&W->mu);
    }
  }
  return NULL;
}

static int run(problem* P, int nthreads) {
  if (P->batch < 0 || P->hq < 1 || P->hkv < 1 || P->hq % P->hkv != 0 || P->head_dim < 1 ||
      P->page_size < 1 || P->max_pages < 0 || P->num_pages < 0 || !P->out || !P->lse ||
      P->q_len < 1 || (P->causal != 0 && P->causal != 1))
    return PKD_ORACLE_BAD_ARG;
  if (P->kv_fp8 && (!P->k_scale || !P->v_scale)) return PKD_ORACLE_BAD_ARG;
  for (int b = 0; b < P->batch; ++b) {
    int st = check_sequence(P, b);
    if (st != PKD_ORACLE_OK) return st;
  }
  pool W;
  W.P = P;
  W.next = 0;
  W.status = PKD_ORACLE_OK;
  pthread_mutex_init(&W.mu, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads == 1) {
    worker(&W);
  } else {
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th) return PKD_ORACLE_NO_MEM;
    int started = 0;
    for (int i = 0; i < nthreads; ++i)
      if (pthread_create(&th[i], NULL, worker, &W) == 0) ++started;
    if (started == 0) worker(&W);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    free(th);
  }
  pthread_mutex_destroy(&W.mu);
  return W.status;
}

/* Plain definition.  q: bf16 bits [B][Hq][D]; k_cache/v_cache: bf16 bits or
 * (kv_fp8 != 0) fp8 E4M3FN codes, [num_pages][page_size][Hkv][D];
 * block_table [B][max_pages]; seq_lens [B]; k_scale/v_scale [Hkv] for fp8.
 * out [B][Hq][D] and lse [B][Hq] are fp64.  Returns 0 or a negative status. */
int pkd_oracle_paged_decode(int batch, int hq, int hkv, int head_dim, int page_size, int num_pages,
                            int max_pages, int kv_fp8, const uint16_t* q, const void* k_cache,
                            const void* v_cache, const int32_t* block_table,
                            const int32_t* seq_lens, const float* k_scale, const float* v_scale,
                            double scale, double* out, double* lse, int nthreads) {
  problem P = {batch, hq, hkv, head_dim, page_size, num_pages, max_pages, kv_fp8,
               q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, scale,
               0, out, lse, 1, 0};
  return run(&P, nthreads);
}

/* Split form: same arguments plus num_splits >= 1. */
int pkd_oracle_paged_decode_split(int batch, int hq, int hkv, int head_dim, int page_size,
                                  int num_pages, int max_pages, int kv_fp8, const uint16_t* q,
                                  const void* k_cache, const void* v_cache,
                                  const int32_t* block_table, const int32_t* seq_lens,
                                  const float* k_scale, const float* v_scale, double scale,
                                  int num_splits, double* out, double* lse, int nthreads) {
  if (num_splits < 1) return PKD_ORACLE_BAD_ARG;
  problem P = {batch, hq, hkv, head_dim, page_size, num_pages, max_pages, kv_fp8,
               q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, scale,
               num_splits, out, lse, 1, 0};
  return run(&P, nthreads);
}

/* The plain definition for a list of rows only (see the _rows entries). */
static int rows_only(problem* P, int n_rows, const int64_t* rows, double* out, double* lse) {
  if (P->batch < 0 || P->hq < 1 || P->hkv < 1 || P->hq % P->hkv != 0 || P->head_dim < 1 ||
      P->page_size < 1 || P->q_len < 1 || (P->causal != 0 && P->causal != 1) || n_rows < 0 ||
      !rows || !out || !lse)
    return PKD_ORACLE_BAD_ARG;
  if (P->kv_fp8 && (!P->k_scale || !P->v_scale)) return PKD_ORACLE_BAD_ARG;
  const int64_t per_seq = (int64_t)P->q_len * P->hq;
  for (int i = 0; i < n_rows; ++i) {
    int64_t r = rows[i];
    if (r < 0 || r >= (int64_t)P->batch * per_seq) return PKD_ORACLE_BAD_ARG;
    int b = (int)(r / per_seq);
    int qi = (int)((r % per_seq) / P->hq);
    int h = (int)(r % P->hq);
    int st = check_sequence(P, b);
    if (st != PKD_ORACLE_OK) return st;
    int V = visible_tokens(P, b, qi);
    int lo = first_visible(P, b, qi);
    double* s = (double*)malloc(sizeof(double) * (size_t)(V > 0 ? V : 1));
    if (!s) return PKD_ORACLE_NO_MEM;
    double* o = out + (int64_t)i * P->head_dim;
    lse[i] = apply_sink(P, h, attend_range(P, b, qi, h, lo, V, o, s), o);
    free(s);
  }
  return PKD_ORACLE_OK;
}

/* Plain definition for a chosen list of (sequence, query head) rows only:
 * rows[i] = b * Hq + h.  out is [n_rows][D] and lse [n_rows], fp64.  Used to
 * spot-check full-size problems without computing every row.  Single thread,
 * rows in the given order. */
int pkd_oracle_paged_decode_rows(int batch, int hq, int hkv, int head_dim, int page_size,
                                 int num_pages, int max_pages, int kv_fp8, const uint16_t* q,
                                 const void* k_cache, const void* v_cache,
                                 const int32_t* block_table, const int32_t* seq_lens,
                                 const float* k_scale, const float* v_scale, double scale,
                                 int n_rows, const int64_t* rows, double* out, double* lse) {
  problem P = {batch, hq, hkv, head_dim, page_size, num_pages, max_pages, kv_fp8,
               q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, scale,
               0, out, lse, 1, 0};
  return rows_only(&P, n_rows, rows, out, lse);
}

/* Several query tokens per sequence (see the top of this file).  q: bf16 bits
 * [B][q_len][Hq][D]; out [B][q_len][Hq][D] and lse [B][q_len][Hq], fp64;
 * causal is 0 or 1; the other arguments as for pkd_oracle_paged_decode. */
int pkd_oracle_paged_decode_multi(int batch, int hq, int hkv, int head_dim, int page_size,
                                  int num_pages, int max_pages, int kv_fp8, int q_len, int causal,
                                  const uint16_t* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_table, const int32_t* seq_lens,
                                  const float* k_scale, const float* v_scale, double scale,
                                  double* out, double* lse, int nthreads) {
  problem P = {batch, hq, hkv, head_dim, page_size, num_pages, max_pages, kv_fp8,
               q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, scale,
               0, out, lse, q_len, causal};
  return run(&P, nthreads);
}

/* Several query tokens, causal mask, sliding window and sinks (see the top of
 * the file): window >= 0 (0 = none), sinks [hq] fp32 or NULL; other arguments
 * as for pkd_oracle_paged_decode_multi. */
int pkd_oracle_paged_decode_ext(int batch, int hq, int hkv, int head_dim, int page_size, int num_pages,
                                int max_pages, int kv_fp8, int q_len, int causal, int window,
                                const float* sinks, const uint16_t* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_table, const int32_t* seq_lens, const float* k_scale,
                                const float* v_scale, double scale, double* out, double* lse, int nthreads) {
  if (window < 0) return PKD_ORACLE_BAD_ARG;
  problem P = {batch, hq, hkv, head_dim, page_size, num_pages, max_pages, kv_fp8,
               q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, scale,
               0, out, lse, q_len, causal, window, sinks};
  return run(&P, nthreads);
}

/* pkd_oracle_paged_decode_ext for a list of rows only (rows as in _multi_rows). */
int pkd_oracle_paged_decode_ext_rows(int batch, int hq, int hkv, int head_dim, int page_size, int num_pages,
                                     int max_pages, int kv_fp8, int q_len, int causal, int window,
                                     const float* sinks, const uint16_t* q, const void* k_cache,
                                     const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                                     const float* k_scale, const float* v_scale, double scale, int n_rows,
                                     const int64_t* rows, double* out, double* lse) {
  if (window < 0) return PKD_ORACLE_BAD_ARG;
  problem P = {batch, hq, hkv, head_dim, page_size, num_pages, max_pages, kv_fp8,
               q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, scale,
               0, out, lse, q_len, causal, window, sinks};
  return rows_only(&P, n_rows, rows, out, lse);
}

/* pkd_oracle_paged_decode_multi for a list of rows only: rows[i] =
 * (b * q_len + i) * Hq + h; out [n_rows][D], lse [n_rows]; single thread. */
int pkd_oracle_paged_decode_multi_rows(int batch, int hq, int hkv, int head_dim, int page_size,
                                       int num_pages, int max_pages, int kv_fp8, int q_len,
                                       int causal, const uint16_t* q, const void* k_cache,
                                       const void* v_cache, const int32_t* block_table,
                                       const int32_t* seq_lens, const float* k_scale,
                                       const float* v_scale, double scale, int n_rows,
                                       const int64_t* rows, double* out, double* lse) {
  problem P = {batch, hq, hkv, head_dim, page_size, num_pages, max_pages, kv_fp8,
               q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, scale,
               0, out, lse, q_len, causal};
  return rows_only(&P, n_rows, rows, out, lse);
}

/* Plain definition restricted to one token range per sequence: row
 * (b, h) attends over tokens [t_begin[b], t_end[b]) only (an empty range gives
 * out = 0, lse = -inf).  Used to check split partials one split at a time.
 * out [B][Hq][D], lse [B][Hq]; single thread. */
int pkd_oracle_paged_decode_ranges(int batch, int hq, int hkv, int head_dim, int page_size,
                                   int num_pages, int max_pages, int kv_fp8, const uint16_t* q,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, const int32_t* seq_lens,
                                   const float* k_scale, const float* v_scale, double scale,
                                   const int32_t* t_begin, const int32_t* t_end, double* out,
                                   double* lse) {
  problem P = {batch, hq, hkv, head_dim, page_size, num_pages, max_pages, kv_fp8,
               q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, scale,
               0, out, lse, 1, 0};
  if (batch < 0 || hq < 1 || hkv < 1 || hq % hkv != 0 || head_dim < 1 || page_size < 1 ||
      !t_begin || !t_end || !out || !lse)
    return PKD_ORACLE_BAD_ARG;
  if (kv_fp8 && (!k_scale || !v_scale)) return PKD_ORACLE_BAD_ARG;
  for (int b = 0; b < batch; ++b) {
    int st = check_sequence(&P, b);
    if (st != PKD_ORACLE_OK) return st;
    int t0 = t_begin[b], t1 = t_end[b];
    if (t0 < 0 || t1 > seq_lens[b]) return PKD_ORACLE_BAD_ARG;
    double* s = (double*)malloc(sizeof(double) * (size_t)(t1 > t0 ? t1 - t0 : 1));
    if (!s) return PKD_ORACLE_NO_MEM;
    for (int h = 0; h < hq; ++h)
      lse[(int64_t)b * hq + h] =
          attend_range(&P, b, 0, h, t0, t1, out + ((int64_t)b * hq + h) * head_dim, s);
    free(s);
  }
  return PKD_ORACLE_OK;
}

/* ---- paged KV append (row f2) -------------------------------------------------
 *
 * Writing new K/V rows into the paged cache: the step before decode, which the
 * sglang fuse/overlap catalogue lists as fused FP8 quantisation + paged K/V
 * cache write (section 1, the TRTLLM FP8 KV row) and as RoPE fused with the KV
 * cache store (section 1; section 14, the vLLM rope + cache rows).  Token n's
 * rows k_new[n][h][:], v_new[n][h][:] (bf16) go to slot slot_mapping[n] of the
 * pool, i.e. page slot / page_size, position slot % page_size; a slot outside
 * [0, num_pages * page_size) (padding tokens use -1) writes nothing.  With a
 * RoPE table, K is first rotated in the NeoX "rotate half" form: for d < D/2,
 * with c = cos_sin[pos][d] and s = cos_sin[pos][D/2 + d],
 *     k'[d]       = k[d] c - k[d + D/2] s
 *     k'[d + D/2] = k[d + D/2] c + k[d] s
 * (a position outside [0, max_position) writes nothing).  The cache value is
 * then k' rounded to bf16, or for an FP8 cache the E4M3FN code of
 * clamp(k' / scale[h], -448, 448), rounded to nearest, ties to the even code.
 *
 * Unlike the attention definition above, these steps are carried out in fp32
 * exactly as written, because they end in a rounding to a code: the GPU kernel
 * takes the same decisions in the same precision (products rounded to fp32,
 * then one fused multiply-add, then an fp32 division by the scale), so that
 * the codes can be compared bit for bit.
 */

/* bf16 bits of an fp32 value, round to nearest even (finite inputs). */
uint16_t pkd_oracle_bf16_round(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* E4M3FN code of x (|x| <= 448 after the caller's clamp): the nearest finite
 * code by the decoder above, ties to the even code; the sign bit from x. */
uint8_t pkd_oracle_fp8e4m3_encode(float x) {
  const int neg = signbit(x) != 0;
  const double a = fabs((double)x);
  int best = 0;
  double best_err = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) { /* 0x7F is NaN */
    const double err = fabs(pkd_oracle_fp8e4m3_value((uint8_t)c) - a);
    if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      best_err = err;
    }
  }
  return (uint8_t)(best | (neg ? 0x80 : 0));
}

/* A bf16 value as fp32 (exact: every bf16 value is an fp32 value). */
static float bf16_float(uint16_t bits) { return (float)pkd_oracle_bf16_value(bits); }

static void store_row(int kv_fp8, void* cache, int64_t elem0, const float* y, int D, float scale) {
  if (kv_fp8) {
    uint8_t* c = (uint8_t*)cache;
    for (int d = 0; d < D; ++d) {
      float q = y[d] / scale;
      if (q > 448.0f) q = 448.0f;
      if (q < -448.0f) q = -448.0f;
      c[elem0 + d] = pkd_oracle_fp8e4m3_encode(q);
    }
  } else {
    uint16_t* c = (uint16_t*)cache;
    for (int d = 0; d < D; ++d) c[elem0 + d] = pkd_oracle_bf16_round(y[d]);
  }
}

/* k_new, v_new: bf16 bits [n_tokens][hkv][head_dim]; slot_mapping [n_tokens];
 * positions [n_tokens] and cos_sin [max_position][head_dim] fp32, or both NULL
 * for no RoPE; k_cache / v_cache [num_pages][page_size][hkv][head_dim] of bf16
 * bits or FP8 codes, updated in place; k_scale / v_scale [hkv] for FP8. */
int pkd_oracle_kv_append(int hkv, int head_dim, int page_size, int num_pages, int kv_fp8, int64_t n_tokens,
                         const uint16_t* k_new, const uint16_t* v_new, const int64_t* slot_mapping,
                         const int64_t* positions, const float* cos_sin, int max_position, void* k_cache,
                         void* v_cache, const float* k_scale, const float* v_scale) {
  const int D = head_dim;
  if (hkv < 1 || D < 2 || D % 2 != 0 || page_size < 1 || num_pages < 0 || n_tokens < 0 || !k_new || !v_new ||
      !slot_mapping || !k_cache || !v_cache || ((positions == NULL) != (cos_sin == NULL)))
    return PKD_ORACLE_BAD_ARG;
  if (kv_fp8 && (!k_scale || !v_scale)) return PKD_ORACLE_BAD_ARG;
  float* y = (float*)malloc(sizeof(float) * (size_t)D);
  if (!y) return PKD_ORACLE_NO_MEM;
  const int64_t capacity = (int64_t)num_pages * page_size;
  for (int64_t n = 0; n < n_tokens; ++n) {
    const int64_t slot = slot_mapping[n];
    if (slot < 0 || slot >= capacity) continue;
    const int64_t pos = positions ? positions[n] : 0;
    if (positions && (pos < 0 || pos >= max_position)) continue;
    for (int h = 0; h < hkv; ++h) {
      const int64_t src = (n * hkv + h) * (int64_t)D;
      const int64_t dst = (slot * hkv + h) * (int64_t)D;  /* page * ps + position, then head */
      for (int d = 0; d < D; ++d) y[d] = bf16_float(k_new[src + d]);
      if (positions) {
        const float* cs = cos_sin + pos * (int64_t)D;
        for (int d = 0; d < D / 2; ++d) {
          const float x0 = bf16_float(k_new[src + d]), x1 = bf16_float(k_new[src + d + D / 2]);
          const float c = cs[d], s = cs[D / 2 + d];
          const float t0 = x1 * s, t1 = x0 * s;
          y[d] = fmaf(x0, c, -t0);
          y[d + D / 2] = fmaf(x1, c, t1);
        }
      }
      store_row(kv_fp8, k_cache, dst, y, D, kv_fp8 ? k_scale[h] : 1.0f);
      for (int d = 0; d < D; ++d) y[d] = bf16_float(v_new[src + d]);
      store_row(kv_fp8, v_cache, dst, y, D, kv_fp8 ? v_scale[h] : 1.0f);
    }
  }
  free(y);
  return PKD_ORACLE_OK;
}

/* ---- decode metadata preparation ----------------------------------------
 *
 * The fused decode metadata setup of the sglang fuse/overlap catalogue
 * (section 1, the flashattention backend's normal_decode_set_metadata row):
 * from the serving runtime's per-request token map it builds what decode
 * reads, in the order the row lists its steps.
 *
 * Inputs: req_to_token [req_rows][req_stride] int32, the KV slot
 * (page * page_size + position in the page) of every token of every request
 * row; req_pool_indices [batch] int64, the request row of batch entry b;
 * seq_lens [batch] int64, its cached tokens before this step; extend, the
 * tokens this step adds to every sequence.
 *
 *   seq-len cast/add:  L_b = seq_lens[b] + extend, stored as int32
 *                      (cache_seqlens[b]);
 *   prefix sum:        cu_seqlens_k[0] = 0, cu_seqlens_k[b + 1] =
 *                      cu_seqlens_k[b] + L_b;
 *   req-to-token gather and page-table divide: for every page j of
 *                      sequence b (j < ceil(L_b / page_size)),
 *                      page_table[b][j] = req_to_token[r_b][j * page_size]
 *                      / page_size (the page of the page's first token; a
 *                      negative slot gives -1); entries past the last page
 *                      are -1;
 *   SWA metadata (window W > 0): the pages from the first one that holds a
 *                      visible position, f_b = max(L_b - q_len - W + 1, 0)
 *                      / page_size, on: swa_page_table[b][j] =
 *                      page_table[b][f_b + j], swa_seqlens[b] = L_b - f_b *
 *                      page_size (the same sequence with its first f_b pages
 *                      dropped, which decode with the same window reads as
 *                      the full one).
 *
 * A batch entry whose request row is outside [0, req_rows) or whose L_b is
 * outside [0, min(max_pages * page_size, req_stride)] is invalid: it is
 * counted, its lengths are written as 0 and its table rows as -1.  Returns the
 * count of invalid entries, or a negative status for bad arguments.
 */
static int64_t slot_page(int32_t slot, int page_size) { return slot >= 0 ? slot / page_size : -1; }

int pkd_oracle_decode_metadata(int batch, int req_rows, int req_stride, int page_size, int max_pages, int q_len,
                               int window, int extend, const int32_t* req_to_token,
                               const int64_t* req_pool_indices, const int64_t* seq_lens, int32_t* cache_seqlens,
                               int32_t* cu_seqlens_k, int32_t* page_table, int32_t* swa_seqlens,
                               int32_t* swa_page_table) {
  if (batch < 0 || req_rows < 1 || req_stride < 1 || page_size < 1 || max_pages < 1 || q_len < 1 || window < 0 ||
      extend < 0 || !req_to_token || !req_pool_indices || !seq_lens || !cache_seqlens || !cu_seqlens_k ||
      !page_table || (window > 0 && (!swa_seqlens || !swa_page_table)))
    return PKD_ORACLE_BAD_ARG;
  int bad = 0;
  int64_t run = 0;
  cu_seqlens_k[0] = 0;
  for (int b = 0; b < batch; ++b) {
    const int64_t r = req_pool_indices[b];
    const int64_t L = seq_lens[b] + extend;
    const int valid = r >= 0 && r < req_rows && L >= 0 && L <= (int64_t)max_pages * page_size && L <= req_stride;
    bad += !valid;
    const int64_t len = valid ? L : 0;
    cache_seqlens[b] = (int32_t)len;
    run += len;
    cu_seqlens_k[b + 1] = (int32_t)run;
    const int64_t n_pages = (len + page_size - 1) / page_size;
    for (int j = 0; j < max_pages; ++j)
      page_table[(int64_t)b * max_pages + j] =
          j < n_pages ? (int32_t)slot_page(req_to_token[r * req_stride + (int64_t)j * page_size], page_size) : -1;
    if (window > 0) {
      int64_t lo = len - q_len - window + 1;
      if (lo < 0) lo = 0;
      const int64_t f = valid ? lo / page_size : 0;
      swa_seqlens[b] = (int32_t)(len - f * page_size);
      for (int j = 0; j < max_pages; ++j)
        swa_page_table[(int64_t)b * max_pages + j] =
            j < n_pages - f ? page_table[(int64_t)b * max_pages + f + j] : -1;
    }
  }
  return bad;
}

/* ---- contiguous KV decode ----------------------------------------------
 *
 * The same attention (several query tokens, causal mask, window, sinks) over
 * K/V held in one contiguous tensor per cache rather than in pages: the
 * contiguous decode kernels of the AstrAI commit log, with its stride-based
 * addressing for Q, K/V and O (any layout, e.g. [B][L][Hkv][D] or
 * [B][Hkv][L][D], read in place).  k_cache / v_cache: element (b, t, g, d) at
 * b*kv_strides[0] + t*kv_strides[1] + g*kv_strides[2] + d; q row (b, i, h) at
 * b*q_strides[0] + i*q_strides[1] + h*q_strides[2] (strides in elements, the
 * head dimension contiguous).  seq_lens[b] <= max_seq_len.  out [B][q_len][Hq][D]
 * and lse [B][q_len][Hq] (fp64, dense) as for the paged entries.
 */
int pkd_oracle_contiguous_decode(int batch, int hq, int hkv, int head_dim, int max_seq_len, int kv_fp8, int q_len,
                                 int causal, int window, const float* sinks, const uint16_t* q,
                                 const int64_t* q_strides, const void* k_cache, const void* v_cache,
                                 const int64_t* kv_strides, const int32_t* seq_lens, const float* k_scale,
                                 const float* v_scale, double scale, double* out, double* lse, int nthreads) {
  if (window < 0 || max_seq_len < 1 || !q_strides || !kv_strides) return PKD_ORACLE_BAD_ARG;
  problem P = {batch, hq, hkv, head_dim, max_seq_len, 1, 1, kv_fp8,
               q, k_cache, v_cache, NULL, seq_lens, k_scale, v_scale, scale,
               0, out, lse, q_len, causal, window, sinks, kv_strides, q_strides};
  return run(&P, nthreads);
}
