/*
 * kda_oracle.c -- plain fp64 CPU oracle for Kimi Delta Attention (KDA).
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark load this library. It shares no code, header, table or
 * helper with the HIP path, and the HIP path never loads it.
 *
 * Sources (web pages; cited by title and section):
 *  [P1] vLLM PR #50649 "[ROCm][Bugfix] Kimi-K3 Fix KDA NaN on mixed batches and
 *       racy autotune config", section Purpose: decode rows of a mixed batch go
 *       to the recurrent kernel; the chunk kernel uses a WY recompute_w_u step.
 *  [P2] prhub report on vLLM PR #51682 "Give the AMD packed KDA decode kernel the
 *       state-index stride", sections Implementation breakdown and Key source
 *       excerpts: the packed-decode argument set (mixed_qkv, raw_g, raw_beta,
 *       A_log, dt_bias, lower_bound, initial_state, state_indices), the state
 *       slot read as state_indices[i * stride] widened to 64 bits, and the slot
 *       stride taken from the state pool.
 *  [P3] vLLM PR #60683 (latency_specialized decode for Kimi-K3 on MI355X),
 *       sections Purpose and Refusal and steps: spec-verify steps of at most 8
 *       rows made of whole requests of k+1 rows; padded requests use a null
 *       state slot.
 *
 * The pages name the KDA recurrence but print no formula. The recurrence used
 * here is the gated delta rule with a per-channel decay, in this order per
 * token: decay, delta-rule write, readout. The gate formula is a reading of the
 * argument names in [P2] (Mamba-style A_log / dt_bias, optional lower bound).
 * Every reading is listed with the design notes.
 *
 * Everything is computed in double precision from the exact bf16 / fp32 input
 * bytes. Parallel loops (OpenMP) only split independent (sequence, head) pairs;
 * the arithmetic of each pair is the plain loop below.
 */
#include "kda_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- inputs -- */

/* bf16 is the top half of an IEEE binary32; widening is exact. */
double kda_oracle_bf16_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* ------------------------------------------------------------------ gate -- */

/* softplus(x) = log(1 + e^x), in the overflow-free form max(x,0)+log1p(e^-|x|). */
static double softplus(double x) { return fmax(x, 0.0) + log1p(exp(-fabs(x))); }

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* Per-channel log-decay g (<= 0) for one token, head and key channel.
 * [P2] Key source excerpts: the gate is fused from raw_g, A_log (per head),
 * dt_bias (per key channel) and an optional lower_bound.
 * Reading: x = raw_g + dt_bias, a = exp(A_log);
 *   no lower bound:   g = -a * softplus(x)
 *   lower bound lb:   g = lb * sigmoid(a * x)          (so lb < g < 0)   */
double kda_oracle_gate(double raw_g, double A_log, double dt_bias,
                       int32_t has_lower_bound, double lower_bound) {
  double x = raw_g + dt_bias;
  double a = exp(A_log);
  if (has_lower_bound) return lower_bound * sigmoid(a * x);
  return -a * softplus(x);
}

/* Write strength beta = sigmoid(raw_beta) (reading: raw_ is a pre-activation). */
double kda_oracle_beta(double raw_beta) { return sigmoid(raw_beta); }

/* ------------------------------------------------------- recurrent form -- */

/* The token-by-token recurrence on one (sequence, head), from the pre-gated
 * per-token values. Layouts: q,k,g [T][K]; v,o [T][V]; beta [T];
 * S [K][V] row-major, read as the initial state and overwritten with the
 * final state.  Per token t:
 *   1. decay:       S <- diag(exp(g_t)) S
 *   2. delta write: u = beta_t (v_t - S^T k_t);  S <- S + k_t u^T
 *   3. readout:     o_t = scale S^T q_t   (with the updated S)            */
void kda_oracle_recurrent_pregated(int32_t T, int32_t K, int32_t V,
                                   const double* q, const double* k,
                                   const double* v, const double* g,
                                   const double* beta, double scale,
                                   double* S, double* o) {
  double* u = (double*)malloc(sizeof(double) * (size_t)V);
  for (int32_t t = 0; t < T; ++t) {
    const double* qt = q + (size_t)t * K;
    const double* kt = k + (size_t)t * K;
    const double* vt = v + (size_t)t * V;
    const double* gt = g + (size_t)t * K;
    /* 1. decay */
    for (int32_t i = 0; i < K; ++i) {
      double a = exp(gt[i]);
      for (int32_t j = 0; j < V; ++j) S[(size_t)i * V + j] *= a;
    }
    /* 2. delta-rule write */
    for (int32_t j = 0; j < V; ++j) {
      double sk = 0.0;
      for (int32_t i = 0; i < K; ++i) sk += S[(size_t)i * V + j] * kt[i];
      u[j] = beta[t] * (vt[j] - sk);
    }
    for (int32_t i = 0; i < K; ++i)
      for (int32_t j = 0; j < V; ++j) S[(size_t)i * V + j] += kt[i] * u[j];
    /* 3. readout */
    for (int32_t j = 0; j < V; ++j) {
      double s = 0.0;
      for (int32_t i = 0; i < K; ++i) s += S[(size_t)i * V + j] * qt[i];
      o[(size_t)t * V + j] = scale * s;
    }
  }
  free(u);
}

/* --------------------------------------------------------- chunked form -- */

/* The same result through the chunked (WY) form named in [P1] Purpose
 * (chunk_kda_with_fused_gate and its recompute_w_u step). Chunks of C tokens;
 * the last one may be shorter. Within a chunk of n tokens, starting state S:
 *   gam_t     = sum_{s<=t} g_s                        (per channel)
 *   A[t][s]   = beta_t sum_i k_ti k_si e^{gam_ti-gam_si}       s < t
 *   Tm        = (I + A)^{-1}                         (unit lower triangular)
 *   W         = Tm diag(beta) (K o e^{gam})          ("recompute_w")
 *   U         = Tm diag(beta) V                      ("recompute_u")
 *   Vn        = U - W S                              (the chunk's delta writes)
 *   P[t][s]   = sum_i q_ti k_si e^{gam_ti-gam_si}              s <= t
 *   O         = scale [ (Q o e^{gam}) S + P Vn ]
 *   S        <- diag(e^{gam_n-1}) S + (K o e^{gam_n-1 - gam})^T Vn
 * Every exponential is taken of a pairwise difference gam_t - gam_s with s <= t
 * (never factorised), so none can overflow.                                */
void kda_oracle_chunked_pregated(int32_t T, int32_t K, int32_t V, int32_t C,
                                 const double* q, const double* k,
                                 const double* v, const double* g,
                                 const double* beta, double scale, double* S,
                                 double* o) {
  double* gam = (double*)malloc(sizeof(double) * (size_t)C * K);
  double* A = (double*)calloc((size_t)C * C, sizeof(double));
  double* Tm = (double*)calloc((size_t)C * C, sizeof(double));
  double* P = (double*)calloc((size_t)C * C, sizeof(double));
  double* W = (double*)malloc(sizeof(double) * (size_t)C * K);
  double* U = (double*)malloc(sizeof(double) * (size_t)C * V);
  double* Vn = (double*)malloc(sizeof(double) * (size_t)C * V);
  double* Snew = (double*)malloc(sizeof(double) * (size_t)K * V);

  for (int32_t c0 = 0; c0 < T; c0 += C) {
    int32_t n = (T - c0 < C) ? (T - c0) : C;
    const double* qc = q + (size_t)c0 * K;
    const double* kc = k + (size_t)c0 * K;
    const double* vc = v + (size_t)c0 * V;
    const double* gc = g + (size_t)c0 * K;
    const double* bc = beta + c0;

    /* cumulative log-decay within the chunk (inclusive) */
    for (int32_t i = 0; i < K; ++i) {
      double acc = 0.0;
      for (int32_t t = 0; t < n; ++t) {
        acc += gc[(size_t)t * K + i];
        gam[(size_t)t * K + i] = acc;
      }
    }
    /* A (strictly lower) and P (lower, with diagonal) */
    for (int32_t t = 0; t < n; ++t) {
      for (int32_t s = 0; s <= t; ++s) {
        double a = 0.0, p = 0.0;
        for (int32_t i = 0; i < K; ++i) {
          double e = exp(gam[(size_t)t * K + i] - gam[(size_t)s * K + i]);
          a += kc[(size_t)t * K + i] * kc[(size_t)s * K + i] * e;
          p += qc[(size_t)t * K + i] * kc[(size_t)s * K + i] * e;
        }
        A[(size_t)t * C + s] = (s < t) ? bc[t] * a : 0.0;
        P[(size_t)t * C + s] = p;
      }
    }
    /* Tm = (I + A)^{-1}, row by row: Tm_t = e_t - sum_{s<t} A_ts Tm_s */
    for (int32_t t = 0; t < n; ++t) {
      for (int32_t j = 0; j < n; ++j) {
        double x = (j == t) ? 1.0 : 0.0;
        for (int32_t s = 0; s < t; ++s) x -= A[(size_t)t * C + s] * Tm[(size_t)s * C + j];
        Tm[(size_t)t * C + j] = x;
      }
    }
    /* W = Tm diag(beta) (K o e^gam),  U = Tm diag(beta) V */
    for (int32_t t = 0; t < n; ++t) {
      for (int32_t i = 0; i < K; ++i) {
        double x = 0.0;
        for (int32_t s = 0; s < n; ++s)
          x += Tm[(size_t)t * C + s] * bc[s] * kc[(size_t)s * K + i] *
               exp(gam[(size_t)s * K + i]);
        W[(size_t)t * K + i] = x;
      }
      for (int32_t j = 0; j < V; ++j) {
        double x = 0.0;
        for (int32_t s = 0; s < n; ++s)
          x += Tm[(size_t)t * C + s] * bc[s] * vc[(size_t)s * V + j];
        U[(size_t)t * V + j] = x;
      }
    }
    /* Vn = U - W S */
    for (int32_t t = 0; t < n; ++t)
      for (int32_t j = 0; j < V; ++j) {
        double x = U[(size_t)t * V + j];
        for (int32_t i = 0; i < K; ++i) x -= W[(size_t)t * K + i] * S[(size_t)i * V + j];
        Vn[(size_t)t * V + j] = x;
      }
    /* O = scale [ (Q o e^gam) S + P Vn ] */
    for (int32_t t = 0; t < n; ++t)
      for (int32_t j = 0; j < V; ++j) {
        double x = 0.0;
        for (int32_t i = 0; i < K; ++i)
          x += qc[(size_t)t * K + i] * exp(gam[(size_t)t * K + i]) * S[(size_t)i * V + j];
        for (int32_t s = 0; s <= t; ++s) x += P[(size_t)t * C + s] * Vn[(size_t)s * V + j];
        o[(size_t)(c0 + t) * V + j] = scale * x;
      }
    /* S <- diag(e^{gam_last}) S + (K o e^{gam_last - gam})^T Vn */
    const double* gl = gam + (size_t)(n - 1) * K;
    for (int32_t i = 0; i < K; ++i)
      for (int32_t j = 0; j < V; ++j) {
        double x = exp(gl[i]) * S[(size_t)i * V + j];
        for (int32_t s = 0; s < n; ++s)
          x += kc[(size_t)s * K + i] * exp(gl[i] - gam[(size_t)s * K + i]) *
               Vn[(size_t)s * V + j];
        Snew[(size_t)i * V + j] = x;
      }
    memcpy(S, Snew, sizeof(double) * (size_t)K * V);
  }
  free(gam); free(A); free(Tm); free(P); free(W); free(U); free(Vn); free(Snew);
}

/* ------------------------------------------------------ batch semantics -- */

/* Widens one (sequence, head) slice of the packed inputs and applies the gate.
 * mixed_qkv row layout: [q | k | v], each head-major (head h's q at columns
 * h*K .. h*K+K-1, k after all H*K q columns, v after all H*K k columns). */
static void gather_head(int32_t row0, int32_t n, int32_t h, int32_t H,
                        int32_t K, int32_t V, const uint16_t* qkv,
                        int64_t qkv_row_stride, const uint16_t* raw_g,
                        const uint16_t* raw_beta, const float* A_log,
                        const float* dt_bias, int32_t has_lb, double lb,
                        double* q, double* k, double* v, double* g,
                        double* beta) {
  for (int32_t t = 0; t < n; ++t) {
    const uint16_t* row = qkv + (int64_t)(row0 + t) * qkv_row_stride;
    for (int32_t i = 0; i < K; ++i) {
      q[(size_t)t * K + i] = kda_oracle_bf16_to_double(row[(size_t)h * K + i]);
      k[(size_t)t * K + i] = kda_oracle_bf16_to_double(row[(size_t)H * K + (size_t)h * K + i]);
      double rg = kda_oracle_bf16_to_double(raw_g[(int64_t)(row0 + t) * H * K + (size_t)h * K + i]);
      g[(size_t)t * K + i] =
          kda_oracle_gate(rg, (double)A_log[h], (double)dt_bias[(size_t)h * K + i], has_lb, lb);
    }
    for (int32_t j = 0; j < V; ++j)
      v[(size_t)t * V + j] = kda_oracle_bf16_to_double(row[(size_t)2 * H * K + (size_t)h * V + j]);
    beta[t] = kda_oracle_beta(kda_oracle_bf16_to_double(raw_beta[(int64_t)(row0 + t) * H + h]));
  }
}

/* One (sequence, head) pair: n rows starting at row0, slot `slot` (< 0: null
 * slot), head h. */
static void run_sequence_head(int32_t row0, int32_t n, int64_t slot, int32_t read_initial,
                              int32_t h, int32_t H, int32_t K, int32_t V,
                              const kda_oracle_args_t* a, int32_t form, double* out,
                              double* final_state) {
  if (n <= 0) return;
  if (slot < 0) {
    /* Null slot ([P3] Refusal and steps: padded requests): no pool access,
     * zero output rows. */
    for (int32_t t = 0; t < n; ++t)
      for (int32_t j = 0; j < V; ++j) out[(int64_t)(row0 + t) * H * V + (int64_t)h * V + j] = 0.0;
    return;
  }
  double* q = (double*)malloc(sizeof(double) * (size_t)n * K);
  double* k = (double*)malloc(sizeof(double) * (size_t)n * K);
  double* g = (double*)malloc(sizeof(double) * (size_t)n * K);
  double* v = (double*)malloc(sizeof(double) * (size_t)n * V);
  double* o = (double*)malloc(sizeof(double) * (size_t)n * V);
  double* beta = (double*)malloc(sizeof(double) * (size_t)n);
  double* S = (double*)malloc(sizeof(double) * (size_t)K * V);
  float* tile = a->pool + slot * a->slot_stride + (int64_t)h * K * V;
  for (int64_t x = 0; x < (int64_t)K * V; ++x) S[x] = read_initial ? (double)tile[x] : 0.0;
  gather_head(row0, n, h, H, K, V, a->mixed_qkv, a->qkv_row_stride, a->raw_g,
              a->raw_beta, a->A_log, a->dt_bias, a->has_lower_bound,
              a->lower_bound, q, k, v, g, beta);
  if (form <= 0)
    kda_oracle_recurrent_pregated(n, K, V, q, k, v, g, beta, a->scale, S, o);
  else
    kda_oracle_chunked_pregated(n, K, V, form, q, k, v, g, beta, a->scale, S, o);
  for (int32_t t = 0; t < n; ++t)
    for (int32_t j = 0; j < V; ++j)
      out[(int64_t)(row0 + t) * H * V + (int64_t)h * V + j] = o[(size_t)t * V + j];
  for (int64_t x = 0; x < (int64_t)K * V; ++x) tile[x] = (float)S[x];
  if (final_state)
    memcpy(final_state + (int64_t)h * K * V, S, sizeof(double) * (size_t)K * V);
  free(q); free(k); free(g); free(v); free(o); free(beta); free(S);
}

void kda_oracle_set_threads(int32_t n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int32_t kda_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Packed decode and spec-verify ([P2] Key source excerpts; [P3] Refusal and
 * steps): num_seqs groups of tokens_per_seq consecutive rows; group n uses slot
 * state_indices[n * index_stride]. Only the state after the group's last
 * token is written back. */
int32_t kda_oracle_decode_packed(int32_t num_seqs, int32_t tokens_per_seq,
                                 int32_t H, int32_t K, int32_t V,
                                 const kda_oracle_args_t* a, int32_t form,
                                 double* out, double* final_state) {
  if (num_seqs < 0 || tokens_per_seq < 1 || H < 1 || K < 1 || V < 1) return 1;
  if (final_state)
    for (int64_t x = 0; x < (int64_t)num_seqs * H * K * V; ++x) final_state[x] = 0.0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t nh = 0; nh < (int64_t)num_seqs * H; ++nh) {
    int32_t n = (int32_t)(nh / H), h = (int32_t)(nh % H);
    int64_t slot = (int64_t)a->state_indices[(int64_t)n * a->index_stride];
    double* fs = final_state ? final_state + (int64_t)n * H * K * V : NULL;
    run_sequence_head(n * tokens_per_seq, tokens_per_seq, slot, 1, h, H, K, V, a, form, out, fs);
  }
  return 0;
}

/* Speculative decoding with a state per token ([P2] Purpose: with speculative
 * decoding the KDA state slot is column 0 of a block table that has
 * 1 + num_speculative_blocks columns; [P3] Refusal and steps: a padded
 * request carries a null slot and one accepted token). Reading taken here:
 * request n owns tokens_per_seq consecutive rows and block-table row
 * table[n * index_stride + c * col_stride]. Its initial state is the slot in
 * column num_accepted[n] - 1 (clamped to 0 .. tokens_per_seq - 1); after its
 * token t the state is stored into the slot in column t, unless that entry
 * is < 0. A request whose initial entry is < 0 reads and writes no slot and
 * outputs zeros. states (optional): fp64 [num_seqs][tokens_per_seq][H][K][V],
 * the state after every token (zeros for such a request). */
int32_t kda_oracle_spec_decode(int32_t num_seqs, int32_t tokens_per_seq,
                               int32_t H, int32_t K, int32_t V,
                               const kda_oracle_args_t* a, int64_t col_stride,
                               const int32_t* num_accepted, double* out,
                               double* states) {
  if (num_seqs < 0 || tokens_per_seq < 1 || H < 1 || K < 1 || V < 1 || col_stride < 1) return 1;
  const int32_t T = tokens_per_seq;
  const int64_t KV = (int64_t)K * V;
  if (states)
    for (int64_t x = 0; x < (int64_t)num_seqs * T * H * KV; ++x) states[x] = 0.0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t nh = 0; nh < (int64_t)num_seqs * H; ++nh) {
    const int32_t n = (int32_t)(nh / H), h = (int32_t)(nh % H);
    const int32_t* row = a->state_indices + (int64_t)n * a->index_stride;
    int32_t acc = num_accepted[n];
    if (acc < 1) acc = 1;
    if (acc > T) acc = T;
    const int64_t s0 = (int64_t)row[(int64_t)(acc - 1) * col_stride];
    const int32_t row0 = n * T;
    if (s0 < 0) {
      for (int32_t t = 0; t < T; ++t)
        for (int32_t j = 0; j < V; ++j) out[(int64_t)(row0 + t) * H * V + (int64_t)h * V + j] = 0.0;
      continue;
    }
    double* q = (double*)malloc(sizeof(double) * (size_t)T * K);
    double* k = (double*)malloc(sizeof(double) * (size_t)T * K);
    double* g = (double*)malloc(sizeof(double) * (size_t)T * K);
    double* v = (double*)malloc(sizeof(double) * (size_t)T * V);
    double* o = (double*)malloc(sizeof(double) * (size_t)V);
    double* beta = (double*)malloc(sizeof(double) * (size_t)T);
    double* S = (double*)malloc(sizeof(double) * (size_t)KV);
    const float* init = a->pool + s0 * a->slot_stride + (int64_t)h * KV;
    for (int64_t x = 0; x < KV; ++x) S[x] = (double)init[x];
    gather_head(row0, T, h, H, K, V, a->mixed_qkv, a->qkv_row_stride, a->raw_g, a->raw_beta,
                a->A_log, a->dt_bias, a->has_lower_bound, a->lower_bound, q, k, v, g, beta);
    for (int32_t t = 0; t < T; ++t) {
      /* one token of the recurrence, then its state goes to column t */
      kda_oracle_recurrent_pregated(1, K, V, q + (size_t)t * K, k + (size_t)t * K,
                                    v + (size_t)t * V, g + (size_t)t * K, beta + t, a->scale, S, o);
      for (int32_t j = 0; j < V; ++j) out[(int64_t)(row0 + t) * H * V + (int64_t)h * V + j] = o[j];
      if (states) memcpy(states + (((int64_t)n * T + t) * H + h) * KV, S, sizeof(double) * (size_t)KV);
      const int64_t st = (int64_t)row[(int64_t)t * col_stride];
      if (st >= 0) {
        float* tile = a->pool + st * a->slot_stride + (int64_t)h * KV;
        for (int64_t x = 0; x < KV; ++x) tile[x] = (float)S[x];
      }
    }
    free(q); free(k); free(g); free(v); free(o); free(beta); free(S);
  }
  return 0;
}

/* Varlen prefill: sequence i covers rows cu_seqlens[i] .. cu_seqlens[i+1]-1
 * and uses slot state_indices[i * index_stride]. The initial state is read from
 * the slot unless has_initial_state[i] == 0 (then it is zero). A zero-length
 * sequence touches nothing. */
int32_t kda_oracle_prefill(int32_t num_seqs, const int32_t* cu_seqlens,
                           const uint8_t* has_initial_state, int32_t H,
                           int32_t K, int32_t V, const kda_oracle_args_t* a,
                           int32_t form, double* out, double* final_state) {
  if (num_seqs < 0 || H < 1 || K < 1 || V < 1) return 1;
  for (int32_t i = 0; i < num_seqs; ++i)
    if (cu_seqlens[i + 1] < cu_seqlens[i]) return 1;
  if (final_state)
    for (int64_t x = 0; x < (int64_t)num_seqs * H * K * V; ++x) final_state[x] = 0.0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t ih = 0; ih < (int64_t)num_seqs * H; ++ih) {
    int32_t i = (int32_t)(ih / H), h = (int32_t)(ih % H);
    int64_t slot = (int64_t)a->state_indices[(int64_t)i * a->index_stride];
    int32_t n = cu_seqlens[i + 1] - cu_seqlens[i];
    int32_t read_initial = has_initial_state ? (has_initial_state[i] != 0) : 1;
    double* fs = final_state ? final_state + (int64_t)i * H * K * V : NULL;
    run_sequence_head(cu_seqlens[i], n, slot, read_initial, h, H, K, V, a, form, out, fs);
  }
  return 0;
}

/* Gated RMSNorm output epilogue. [P3] Purpose lists "gated RMSNorm" as the
 * step after the KDA recurrence inside one decode kernel, with no formula.
 * Reading: per token row and head, over the head's V output channels,
 *   y_j = o_j / sqrt(mean_j' o_j'^2 + eps) * w_j * act(z_j)
 * with a per-channel weight w shared by the heads, a gate input z (bf16, laid
 * out head-major like the output: channel j of head h at h*V + j) and
 * act(z) = sigmoid(z) (activation 0) or z * sigmoid(z) (activation 1).
 * o is updated in place. */
void kda_oracle_gated_rmsnorm(int64_t rows, int32_t H, int32_t V, double* o,
                              const uint16_t* z, int64_t z_row_stride,
                              const float* w, double eps, int32_t activation) {
  for (int64_t r = 0; r < rows; ++r) {
    for (int32_t h = 0; h < H; ++h) {
      double* oh = o + ((size_t)r * H + h) * V;
      const uint16_t* zh = z + (size_t)r * z_row_stride + (size_t)h * V;
      double ss = 0.0;
      for (int32_t j = 0; j < V; ++j) ss += oh[j] * oh[j];
      const double inv = 1.0 / sqrt(ss / V + eps);
      for (int32_t j = 0; j < V; ++j) {
        const double zv = kda_oracle_bf16_to_double(zh[j]);
        const double act = activation == 1 ? zv * sigmoid(zv) : sigmoid(zv);
        oh[j] = oh[j] * inv * (double)w[j] * act;
      }
    }
  }
}

/* Short causal conv prologue. [P3] Purpose lists a "spec conv" step before
 * the KDA recurrence, with no formula. Reading: a depthwise causal
 * convolution of width W along each sequence, per channel of the [q | k | v]
 * pre-activations (D = 2*H*K + H*V channels, head-major as in mixed_qkv):
 *   a[t][c] = bias[c] + sum_{i<W} w[c][i] * x[t - (W-1) + i][c]
 * where inputs before the sequence's first row come from its conv state
 * (the W-1 previous inputs, oldest first; zero without an initial state or
 * on a null slot), then y = silu(a) = a * sigmoid(a), then q and k of each
 * head are divided by sqrt(sum of squares over the head + l2_eps). The new
 * conv state is the last W-1 inputs of the sequence (older ones from the old
 * state when the sequence is shorter than W-1); it is written back unless
 * the slot is null or the sequence is empty.
 *   x: bf16 bits [rows][D]; w: fp32 [D][W]; bias: fp32 [D] or NULL;
 *   state: fp64 [slots][W-1][D] (in/out, indexed like the KDA pool);
 *   y: fp64 [rows][D]. */
void kda_oracle_short_conv(int32_t num_seqs, const int32_t* cu_seqlens,
                           const uint8_t* has_initial_state, int32_t H,
                           int32_t K, int32_t V, int32_t W, const uint16_t* x,
                           const float* w, const float* bias, double l2_eps,
                           double* state, const int32_t* indices,
                           int64_t index_stride, double* y) {
  const int32_t D = 2 * H * K + H * V;
  const int32_t P = W - 1;
  double* hist = (double*)malloc(sizeof(double) * (size_t)(P + 1));
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t bos = cu_seqlens[s], len = cu_seqlens[s + 1] - cu_seqlens[s];
    const int64_t slot = (int64_t)indices[(int64_t)s * index_stride];
    const int init = slot >= 0 && (has_initial_state == NULL || has_initial_state[s] != 0);
    double* st = slot >= 0 ? state + (size_t)slot * P * D : NULL;
    for (int32_t c = 0; c < D; ++c) {
      /* hist[j] = input at relative position j - P, j < P */
      for (int32_t j = 0; j < P; ++j) hist[j] = init ? st[(size_t)j * D + c] : 0.0;
      for (int32_t t = 0; t < len; ++t) {
        double a = bias ? (double)bias[c] : 0.0;
        for (int32_t i = 0; i < W; ++i) {
          const int32_t pos = t - P + i;
          const double xv = pos >= 0 ? kda_oracle_bf16_to_double(x[(size_t)(bos + pos) * D + c])
                                     : hist[P + pos];
          a += (double)w[(size_t)c * W + i] * xv;
        }
        y[(size_t)(bos + t) * D + c] = a * sigmoid(a);
      }
      if (slot >= 0 && len > 0) {
        for (int32_t j = 0; j < P; ++j) {
          const int32_t pos = len - P + j;
          st[(size_t)j * D + c] = pos >= 0 ? kda_oracle_bf16_to_double(x[(size_t)(bos + pos) * D + c])
                                           : hist[P + pos];
        }
      }
    }
    /* L2 norm of q and k per head. */
    for (int32_t t = 0; t < len; ++t) {
      double* yr = y + (size_t)(bos + t) * D;
      for (int32_t part = 0; part < 2; ++part)
        for (int32_t h = 0; h < H; ++h) {
          double* v = yr + (size_t)part * H * K + (size_t)h * K;
          double ss = 0.0;
          for (int32_t i = 0; i < K; ++i) ss += v[i] * v[i];
          const double inv = 1.0 / sqrt(ss + l2_eps);
          for (int32_t i = 0; i < K; ++i) v[i] *= inv;
        }
    }
  }
  free(hist);
}
