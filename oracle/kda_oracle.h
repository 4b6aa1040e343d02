/*
 * kda_oracle.h -- fp64 CPU oracle for KDA. TEST INFRASTRUCTURE ONLY: nothing on
 * the product path includes or loads this. Shares nothing with the HIP path.
 */
#ifndef KDA_ORACLE_H
#define KDA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Host-side inputs of a batch, in the same byte formats the HIP path takes:
 * bf16 as raw uint16 bits, fp32 pool, int32 slot indices. */
typedef struct {
  const uint16_t* mixed_qkv;   /* [rows][qkv_row_stride], [q | k | v] head-major */
  int64_t qkv_row_stride;      /* elements */
  const uint16_t* raw_g;       /* [rows][H*K] */
  const uint16_t* raw_beta;    /* [rows][H] */
  const float* A_log;          /* [H] */
  const float* dt_bias;        /* [H*K] */
  int32_t has_lower_bound;
  double lower_bound;
  double scale;
  float* pool;                 /* [slots][slot_stride]; head h at h*K*V, [K][V] */
  int64_t slot_stride;         /* elements */
  const int32_t* state_indices;/* entry i at state_indices[i*index_stride]; <0 null */
  int64_t index_stride;        /* elements */
} kda_oracle_args_t;

double kda_oracle_bf16_to_double(uint16_t bits);
double kda_oracle_gate(double raw_g, double A_log, double dt_bias,
                       int32_t has_lower_bound, double lower_bound);
double kda_oracle_beta(double raw_beta);

void kda_oracle_recurrent_pregated(int32_t T, int32_t K, int32_t V,
                                   const double* q, const double* k,
                                   const double* v, const double* g,
                                   const double* beta, double scale,
                                   double* S, double* o);
void kda_oracle_chunked_pregated(int32_t T, int32_t K, int32_t V, int32_t C,
                                 const double* q, const double* k,
                                 const double* v, const double* g,
                                 const double* beta, double scale, double* S,
                                 double* o);

void kda_oracle_set_threads(int32_t n);
int32_t kda_oracle_max_threads(void);

/* form <= 0: recurrent form; form = C > 0: chunked form with chunk size C.
 * out: fp64 [rows][H][V]; final_state (optional): fp64 [seqs][H][K][V]. */
int32_t kda_oracle_decode_packed(int32_t num_seqs, int32_t tokens_per_seq,
                                 int32_t H, int32_t K, int32_t V,
                                 const kda_oracle_args_t* a, int32_t form,
                                 double* out, double* final_state);
/* Spec decode with a state per token: initial state from block-table column
 * num_accepted[n] - 1, the state after token t stored into column t.
 * states (optional): fp64 [seqs][tokens_per_seq][H][K][V]. */
int32_t kda_oracle_spec_decode(int32_t num_seqs, int32_t tokens_per_seq,
                               int32_t H, int32_t K, int32_t V,
                               const kda_oracle_args_t* a, int64_t col_stride,
                               const int32_t* num_accepted, double* out,
                               double* states);
int32_t kda_oracle_prefill(int32_t num_seqs, const int32_t* cu_seqlens,
                           const uint8_t* has_initial_state, int32_t H,
                           int32_t K, int32_t V, const kda_oracle_args_t* a,
                           int32_t form, double* out, double* final_state);

/* Gated RMSNorm epilogue (reading R20), in place on fp64 outputs:
 * o: [rows][H][V]; z: bf16 bits, row r at z + r*z_row_stride, head h at h*V;
 * w: fp32 [V]; activation 0 = sigmoid(z), 1 = z*sigmoid(z). */
void kda_oracle_gated_rmsnorm(int64_t rows, int32_t H, int32_t V, double* o,
                              const uint16_t* z, int64_t z_row_stride,
                              const float* w, double eps, int32_t activation);

/* Short causal conv prologue (reading R22), varlen over cu_seqlens:
 * x: bf16 bits [rows][D] (D = 2HK + HV); w: fp32 [D][W]; bias: fp32 [D] or
 * NULL; state: fp64 [slots][W-1][D] (in/out; entry i of indices at
 * i*index_stride, negative = null); y: fp64 [rows][D]. */
void kda_oracle_short_conv(int32_t num_seqs, const int32_t* cu_seqlens,
                           const uint8_t* has_initial_state, int32_t H,
                           int32_t K, int32_t V, int32_t W, const uint16_t* x,
                           const float* w, const float* bias, double l2_eps,
                           double* state, const int32_t* indices,
                           int64_t index_stride, double* y);

#ifdef __cplusplus
}
#endif
#endif
