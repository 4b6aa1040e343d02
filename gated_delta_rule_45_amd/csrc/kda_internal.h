// kda_internal.h -- launch descriptors shared between the C-ABI front end and
// the kernel translation units. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// Gated RMSNorm output epilogue (gate == nullptr: none):
// y = o / sqrt(mean(o^2) + eps) * weight * act(gate) per row and head.
struct OutNorm {
  const uint16_t* gate;     // bf16 [rows][gate_row_stride], head h at h*V
  int64_t gate_row_stride;  // elements
  const float* weight;      // [V]
  float eps;
  int32_t activation;       // 0: sigmoid(z), 1: z * sigmoid(z)
};

// Applies the epilogue in place to bf16 out [rows][H][V].
hipError_t launch_gated_rmsnorm(const OutNorm& n, uint16_t* out, int64_t rows, int32_t H,
                                int32_t V, hipStream_t stream);

// One packed-decode / spec-verify launch.
// Short conv prologue fused into the decode staging (x null: none): q, k
// and v come from the pre-activations x through the conv, request n's
// tokens forming one conv sequence on conv-state slot indices[n] (its state
// slot).
struct DecodeConv {
  const uint16_t* x;         // bf16 [rows][x_row_stride], channels [q | k | v]
  int64_t x_row_stride;      // elements
  const float* weight;       // [D][width]
  const float* bias;         // [D] or null
  int32_t width;             // 2..4
  float l2_eps;
  uint16_t* conv_state;      // bf16 pool; slot s at s*conv_slot_stride: [width-1][D]
  int64_t conv_slot_stride;  // elements
};

struct DecodeParams {
  const uint16_t* qkv;      // bf16 [rows][qkv_row_stride]
  int64_t qkv_row_stride;   // elements
  const uint16_t* raw_g;    // bf16 [rows][H*K]
  const uint16_t* raw_beta; // bf16 [rows][H]
  const float* A_log;       // [H]
  const float* dt_bias;     // [H*K]
  float lower_bound;
  float scale;
  int32_t has_lb;
  float* pool;
  int64_t slot_stride;
  const int32_t* indices;
  int64_t index_stride;
  // Spec decode with a state per token (null for plain decode): request n
  // starts from the slot in column num_accepted[n]-1 of its index row and
  // stores its state after token t into column t (entry n*index_stride +
  // c*index_col_stride).
  const int32_t* num_accepted;
  int64_t index_col_stride;
  uint16_t* out;            // bf16 [rows][H][V]
  OutNorm norm;             // fused into the kernel when a workgroup holds whole rows
  DecodeConv conv;          // x null: mixed_qkv holds q, k, v
  int32_t num_seqs;
  int32_t tokens_per_seq;
  int32_t H;
  int32_t V;
  int64_t num_tiles;        // num_seqs * H * (V / VT)
};

// One short-conv prologue call (varlen over cu_seqlens).
struct ConvParams {
  const uint16_t* x;            // bf16 [rows][x_row_stride], channels [q | k | v]
  int64_t x_row_stride;         // elements
  const float* weight;          // [D][width]
  const float* bias;            // [D] or null
  int32_t width;                // 2..4
  float l2_eps;
  uint16_t* conv_state;         // bf16 pool; slot s at s*conv_slot_stride: [width-1][D]
  int64_t conv_slot_stride;     // elements
  const int32_t* indices;       // entry i at indices[i*index_stride]; < 0: null
  int64_t index_stride;
  const int32_t* cu_seqlens;    // [num_seqs+1] (unused when uniform_len > 0)
  int32_t uniform_len;          // > 0: sequence i is rows i*uniform_len .. (i+1)*uniform_len - 1
  const uint8_t* has_initial_state;  // may be null (all 1)
  uint16_t* out;                // bf16 [rows][out_row_stride] (mixed_qkv)
  int64_t out_row_stride;       // elements
  int32_t num_seqs;
  int64_t num_rows;
  int32_t H;
  int32_t K;
  int32_t V;
};

hipError_t launch_short_conv(const ConvParams& p, hipStream_t stream);
// Only the conv-state pass of launch_short_conv (the new states from x and
// the old states), for callers that computed the conv outputs themselves.
hipError_t launch_conv_state(const ConvParams& p, hipStream_t stream);

// Picks the column-tile width for a decode launch and launches it.
hipError_t launch_decode(DecodeParams p, int K, hipStream_t stream);

// One chunked-prefill call (all sequences of one varlen batch).
struct PrefillParams {
  const uint16_t* qkv;
  int64_t qkv_row_stride;
  const uint16_t* raw_g;
  const uint16_t* raw_beta;
  const float* A_log;
  const float* dt_bias;
  float lower_bound;
  float scale;
  int32_t has_lb;
  float* pool;
  int64_t slot_stride;
  const int32_t* indices;
  int64_t index_stride;
  uint16_t* out;
  OutNorm norm;             // output epilogue, applied in the state passes (gate null: none)
  const int32_t* cu_seqlens;
  const uint8_t* has_initial_state;  // may be null
  int32_t num_seqs;
  int64_t num_tokens;
  int32_t H;
  int32_t K;
  int32_t V;
  void* workspace;
  size_t workspace_bytes;
};

// Workspace of a prefill call: the full size (plan, segment maps and chunk
// records) and the smallest that runs (without records: long sequences then
// run their intra part twice).
size_t prefill_workspace_bytes(int32_t num_seqs, int64_t num_tokens, int32_t H,
                               int32_t K, int32_t V);
size_t prefill_workspace_min_bytes(int32_t num_seqs, int64_t num_tokens, int32_t H,
                                   int32_t K, int32_t V);
// The segment-map area of that workspace: its byte offset, the bytes of one
// map item (M as bf16 hi then lo MFMA fragments, K*K*4 bytes, then B as
// fp32 [K][V]) and the number of items (H times the map bound).
void prefill_workspace_maps(int32_t num_seqs, int64_t num_tokens, int32_t H, int32_t K, int32_t V,
                            size_t* offset, size_t* item_bytes, int64_t* items);
// after_plan (optional) is recorded on the stream once the plan kernel is
// launched, before the map and state passes.
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream, hipEvent_t after_plan = nullptr);

}  // namespace kda
