/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention (KDA) library.
 *
 * KDA keeps, per sequence and head, an fp32 K x V state S. Per token it decays
 * S per key channel by alpha = exp(g), writes the value with a beta-scaled
 * delta rule, and reads out o = scale * S^T q (decay, write, readout):
 *     S <- diag(alpha) S ;  u = beta (v - S^T k) ;  S <- S + k u^T ;  o = scale S^T q
 * The gate g and beta are fused from raw inputs inside the kernels:
 *     x = raw_g + dt_bias ,  a = exp(A_log[h])
 *     g = -a * softplus(x)              (no lower bound)
 *     g = lower_bound * sigmoid(a * x)  (with a lower bound)
 *     beta = sigmoid(raw_beta)
 * Sources: vLLM PR #51682 (prhub report), "Key source excerpts" and
 * "Implementation breakdown" give the packed-decode argument set and the
 * strided slot addressing; vLLM PR #50649, "Purpose", gives the chunked prefill
 * with its WY recompute_w_u step and the rule that decode rows of a mixed
 * batch never go through the chunk path; vLLM PR #60683, "Purpose" and
 * "Refusal and steps", gives spec-verify steps of at most 8 rows with padded
 * requests on a null state slot. The gate formula is a reading of the argument
 * names (the pages print no formula).
 *
 * Conventions for every entry point:
 *  - All data pointers are DEVICE pointers owned by the caller. Inputs are only
 *    read, the state pool is read and written in place, outputs are written.
 *  - No computing call allocates or frees memory, synchronises the host, or
 *    reads device memory from the host; every launch goes on `stream` (NULL =
 *    the default stream). Calls can therefore be captured in a HIP graph. (Only
 *    kda_overlap_create and kda_overlap_destroy, which manage a caller-owned
 *    handle, create or free anything.)
 *  - Arguments are validated on the host before anything is launched. On any
 *    failed check nothing is launched, the call returns a non-zero status, and
 *    kda_last_error() lists every failed check (not just the first).
 *  - Device-side values are the caller's guarantee: slot numbers must be
 *    < num_slots and unique within one call (not checked), and cu_seqlens
 *    must start at 0, be non-decreasing and end at num_tokens (checked on the
 *    device by the prefill, which then writes NaN rows and sets its status
 *    word instead of computing).
 *  - bf16 outputs are rounded to nearest even; the state stays fp32.
 *  - Supported head dims: K, V in {64, 128}. Layout alignment: mixed_qkv, raw_g,
 *    out and the pool must be 16-byte aligned, qkv_row_stride a multiple of 8
 *    and at most 2^24 elements (kernels address up to 64 rows with 32-bit
 *    byte offsets), and slot_stride a multiple of 4 elements.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size or stride, bad value */
  KDA_ERR_UNSUPPORTED = 2,      /* valid but not built: head dim, alignment   */
  KDA_ERR_WORKSPACE = 3,        /* workspace missing or too small             */
  KDA_ERR_HIP = 4               /* a HIP launch reported an error             */
} kda_status_t;

/* Gate and readout parameters (vLLM PR #51682 report, Key source excerpts:
 * A_log, dt_bias, lower_bound). */
typedef struct {
  const float* A_log;      /* device fp32 [H]                                   */
  const float* dt_bias;    /* device fp32 [H*K]                                 */
  int32_t has_lower_bound; /* 0: no lower bound ("None")                        */
  float lower_bound;       /* used when has_lower_bound; must be <= 0, finite   */
  float scale;             /* o = scale * S^T q; finite                         */
} kda_gate_t;

/* State pool, updated in place (vLLM PR #51682 report, Implementation
 * breakdown: the slot of sequence i is state_indices[i * stride], read as a
 * 64-bit offset; the slot stride comes from the pool tensor). */
typedef struct {
  float* pool;             /* device fp32; slot s, head h at
                              pool + s*slot_stride + h*K*V, [K][V] row-major    */
  int64_t slot_stride;     /* elements between slots, >= H*K*V                  */
  int64_t num_slots;       /* >= 1                                              */
  const int32_t* indices;  /* device int32; entry i at indices[i*index_stride];
                              a negative entry is a null slot                   */
  int64_t index_stride;    /* elements, >= 1 (a strided view such as column 0
                              of a block table is accepted without a copy)      */
} kda_state_t;

/* Gated RMSNorm output epilogue (vLLM PR #60683, Purpose: in the decode
 * kernels a gated RMSNorm follows the KDA recurrence; the page prints no
 * formula, so this is a reading). With norm != NULL a call writes, per output
 * row and head, over the head's V channels,
 *     y_j = o_j / sqrt(mean_j' o_j'^2 + eps) * weight[j] * act(gate_j)
 * instead of o, where act(z) = sigmoid(z) (KDA_NORM_SIGMOID) or
 * z * sigmoid(z) (KDA_NORM_SILU). Null-slot rows stay zero. The norm is taken
 * over o in fp32 inside the decode kernel when one workgroup holds a head's
 * whole row of V channels; otherwise (narrow decode column tiles, prefill)
 * one more pass applies it to the call's bf16 output in place. */
enum { KDA_NORM_SIGMOID = 0, KDA_NORM_SILU = 1 };
typedef struct {
  const void* gate;        /* device bf16 [rows][gate_row_stride]; gate input of
                              head h, channel j at h*V + j; row r pairs with
                              output row r of the call                        */
  int64_t gate_row_stride; /* elements, >= H*V, a multiple of 8               */
  const float* weight;     /* device fp32 [V], shared by the heads            */
  float eps;               /* > 0, finite                                     */
  int32_t activation;      /* KDA_NORM_SIGMOID or KDA_NORM_SILU               */
} kda_out_norm_t;

/*
 * Packed decode and spec-verify (vLLM PR #51682 report, Key source excerpts:
 * fused_recurrent_kda_packed_decode; vLLM PR #60683, Refusal and steps).
 *
 * num_seqs sequences of tokens_per_seq (1..8) consecutive rows each; rows =
 * num_seqs * tokens_per_seq. Sequence n uses slot indices[n*index_stride]: its
 * state is read, the tokens are applied in order, and only the state after the
 * last token is written back. A null slot (negative entry) reads and writes no
 * state and yields zero output rows.
 *   mixed_qkv  bf16 [rows][qkv_row_stride]; per row [q | k | v], each
 *              head-major: q of head h at h*K, k at H*K + h*K, v at 2*H*K + h*V.
 *              qkv_row_stride >= 2*H*K + H*V.
 *   raw_g      bf16 [rows][H*K], contiguous.
 *   raw_beta   bf16 [rows][H], contiguous.
 *   norm       optional output epilogue (NULL: none); gate and weight
 *              16-byte aligned.
 *   out        bf16 [rows][H][V], contiguous.
 * Errors: KDA_ERR_INVALID_ARGUMENT, KDA_ERR_UNSUPPORTED, KDA_ERR_HIP.
 */
kda_status_t kda_decode_packed(int32_t num_seqs, int32_t tokens_per_seq,
                               int32_t H, int32_t K, int32_t V,
                               const void* mixed_qkv, int64_t qkv_row_stride,
                               const void* raw_g, const void* raw_beta,
                               const kda_gate_t* gate, const kda_state_t* state,
                               const kda_out_norm_t* norm, void* out,
                               hipStream_t stream);

/*
 * Speculative decoding with a state per token (vLLM PR #51682 report,
 * Purpose: with speculative decoding the KDA state slot is column 0 of a
 * block table with 1 + num_speculative_blocks columns; vLLM PR #60683,
 * Refusal and steps: a padded request carries a null slot and one accepted
 * token).
 *
 * As kda_decode_packed, except for the state slots. state->indices is a
 * device int32 block table: request n's column c is
 * indices[n*index_stride + c*index_col_stride], and every request must have
 * tokens_per_seq columns. The initial state is read from the slot in column
 * num_accepted_tokens[n] - 1 (device int32 [num_seqs]; values outside
 * 1..tokens_per_seq are clamped into it), and the state after the request's
 * token t is written to the slot in column t; a null entry there skips that
 * write. A request whose initial entry is null reads and writes no state and
 * yields zero output rows. Slots of different requests must be distinct
 * (caller's guarantee, as for the other entry points).
 * Errors: KDA_ERR_INVALID_ARGUMENT (also for index_col_stride < 1 or a NULL
 * num_accepted_tokens), KDA_ERR_UNSUPPORTED, KDA_ERR_HIP.
 */
kda_status_t kda_spec_decode(int32_t num_seqs, int32_t tokens_per_seq,
                             int32_t H, int32_t K, int32_t V,
                             const void* mixed_qkv, int64_t qkv_row_stride,
                             const void* raw_g, const void* raw_beta,
                             const kda_gate_t* gate, const kda_state_t* state,
                             int64_t index_col_stride,
                             const int32_t* num_accepted_tokens,
                             const kda_out_norm_t* norm, void* out,
                             hipStream_t stream);

/* Value of a prefill call's status word (workspace offset 0) when its
 * cu_seqlens break the contract. */
#define KDA_PREFILL_BAD_CU_SEQLENS 1

/* Bytes of device workspace for kda_chunk_prefill at these sizes (a pure
 * host computation; returns 0 for invalid sizes): the plan, the segment
 * maps of long sequences and a record per chunk of them. With the records
 * the second pass over a long sequence's later segments reads each chunk's
 * WY operands (the chunked delta rule of the vLLM PR #50649 kernel,
 * Purpose: W, U and the query operands) instead of building them again. */
size_t kda_chunk_prefill_workspace_size(int32_t num_seqs, int64_t num_tokens,
                                        int32_t H, int32_t K, int32_t V);

/* The smallest workspace kda_chunk_prefill accepts at these sizes: the plan
 * and the segment maps, without the chunk records (long sequences then
 * build their WY operands in both passes). Same results up to the rounding
 * of the segment split; 0 for invalid sizes. */
size_t kda_chunk_prefill_workspace_min_size(int32_t num_seqs, int64_t num_tokens,
                                            int32_t H, int32_t K, int32_t V);

/* Diagnostics (a pure host computation): where the segment maps of a
 * long-sequence prefill live in a workspace of these sizes. *offset is the
 * byte offset of the map area, *item_bytes the size of one map item (the
 * affine map S_out = M S_in + B of one segment of one head, chunked form of
 * the delta rule in the vLLM PR #50649 kernel, Purpose: M as bf16 MFMA
 * fragments, a hi part then a lo part, K*K*4 bytes together, then B as
 * fp32 [K][V]; after the call B holds the next segment's initial state),
 * *items the number of items the area holds (items beyond the ones a call
 * plans are left as they were). All three outputs are host pointers owned
 * by the caller. Errors: KDA_ERR_INVALID_ARGUMENT, KDA_ERR_UNSUPPORTED. */
kda_status_t kda_chunk_prefill_workspace_maps(int32_t num_seqs,
                                              int64_t num_tokens, int32_t H,
                                              int32_t K, int32_t V,
                                              size_t* offset,
                                              size_t* item_bytes,
                                              int64_t* items);

/*
 * Chunked prefill at chunk size 64 (vLLM PR #50649, Purpose:
 * chunk_kda_with_fused_gate and recompute_w_u).
 *
 * Varlen: sequence i covers rows cu_seqlens[i] .. cu_seqlens[i+1]-1 (device
 * int32 [num_seqs+1], cu_seqlens[num_seqs] == num_tokens) and uses slot
 * indices[i*index_stride]. Its initial state is read from the slot unless
 * has_initial_state[i] == 0 (device uint8 [num_seqs]; NULL means all 1), in
 * which case it starts from zero. The final state is written to the slot. A
 * zero-length sequence or a null slot touches no state (null: zero output).
 * Chunks never cross sequences; the last chunk of a sequence may be partial.
 * Row formats and norm as for kda_decode_packed; out is bf16 [num_tokens][H][V].
 * workspace: device scratch of kda_chunk_prefill_workspace_size() bytes
 * (at least kda_chunk_prefill_workspace_min_size(); below the full size
 * long sequences run without chunk records), 256-byte aligned, owned by the
 * caller; its contents are not needed before the call. After the call (in stream order) the int32 at workspace
 * offset 0 is a status word: 0 when cu_seqlens kept to the contract
 * (cu_seqlens[0] == 0, non-decreasing, cu_seqlens[num_seqs] == num_tokens),
 * else KDA_PREFILL_BAD_CU_SEQLENS; in that case every output row of the call
 * is set to NaN and no state slot is read or written.
 * Errors: KDA_ERR_INVALID_ARGUMENT, KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE,
 * KDA_ERR_HIP.
 */
kda_status_t kda_chunk_prefill(int32_t num_seqs, int64_t num_tokens,
                               const int32_t* cu_seqlens,
                               const uint8_t* has_initial_state,
                               int32_t H, int32_t K, int32_t V,
                               const void* mixed_qkv, int64_t qkv_row_stride,
                               const void* raw_g, const void* raw_beta,
                               const kda_gate_t* gate, const kda_state_t* state,
                               const kda_out_norm_t* norm, void* out,
                               void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* Size of the static device scratch of kda_chunk_prefill_noalloc, per GPU. */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * kda_chunk_prefill without any allocation, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. Same arguments, semantics and errors as
 * kda_chunk_prefill, minus the workspace: the call uses the library's own
 * static device buffer of KDA_NOALLOC_SCRATCH_BYTES (64 MiB), one per GPU,
 * which each GPU the library runs on holds until the process ends. Sizes
 * whose kda_chunk_prefill_workspace_min_size() exceeds it are rejected with
 * KDA_ERR_WORKSPACE before anything is launched; sizes whose
 * kda_chunk_prefill_workspace_size() fits run exactly as kda_chunk_prefill
 * with a full workspace, the others without chunk records. The call allocates and frees
 * nothing (no hipMalloc, no allocating library routine); the first call for a
 * GPU looks up the buffer's device address (hipGetSymbolAddress), so make that
 * first call outside graph capture. The kernels write every scratch word they
 * read, so the buffer needs no clearing between calls, but every call on one
 * GPU shares it: calls that overlap in time on one GPU (on different streams
 * or from different host threads) race on it and must be ordered by the
 * caller.
 */
kda_status_t kda_chunk_prefill_noalloc(int32_t num_seqs, int64_t num_tokens,
                                       const int32_t* cu_seqlens,
                                       const uint8_t* has_initial_state,
                                       int32_t H, int32_t K, int32_t V,
                                       const void* mixed_qkv, int64_t qkv_row_stride,
                                       const void* raw_g, const void* raw_beta,
                                       const kda_gate_t* gate, const kda_state_t* state,
                                       const kda_out_norm_t* norm, void* out,
                                       hipStream_t stream);

/* Bytes of device workspace kda_mixed_batch needs. */
size_t kda_mixed_batch_workspace_size(int32_t num_decodes, int32_t num_prefills,
                                      int64_t num_prefill_tokens, int32_t H,
                                      int32_t K, int32_t V);

/*
 * Overlap resources of kda_mixed_batch, created and owned by the caller: a
 * side stream (default priority, non-blocking) and two events on the device
 * current at creation. kda_overlap_create allocates them, so call it once,
 * outside graph capture, and keep the handle; kda_overlap_destroy frees them
 * (NULL is a no-op). A handle serves one call at a time: callers that issue
 * mixed batches concurrently (several host threads, or a capture beside
 * eager calls) each need their own.
 * Errors: KDA_ERR_INVALID_ARGUMENT (NULL out pointer), KDA_ERR_HIP.
 */
typedef struct kda_overlap_s* kda_overlap_t;
kda_status_t kda_overlap_create(kda_overlap_t* overlap);
kda_status_t kda_overlap_destroy(kda_overlap_t overlap);

/*
 * Mixed decode + prefill batch in one call (vLLM PR #50649, Purpose: the
 * decode rows of a mixed non-speculative batch go to the recurrent kernel,
 * never to the chunk kernel, which returned NaN for them).
 *
 * Rows [0, num_decodes) are single-token decodes; decode d uses slot
 * indices[d*index_stride]. Rows [num_decodes, num_decodes+num_prefill_tokens)
 * are num_prefills prefill sequences described by prefill_cu_seqlens (device
 * int32 [num_prefills+1], relative to row num_decodes); prefill i uses slot
 * indices[(num_decodes+i)*index_stride] and has_initial_state[i] (NULL = all
 * 1). Decode rows go to the recurrent decode kernel, prefill rows to the chunk
 * pipeline, with no host synchronisation. The call is ordered on `stream` as
 * a whole. With overlap == NULL both parts run on `stream`. With a handle from
 * kda_overlap_create (same device as `stream`, else KDA_ERR_INVALID_ARGUMENT)
 * and both kinds of rows, the decode kernel runs on the handle's side stream,
 * forked from `stream` after the prefill's plan kernel and joined back before
 * the call's work on `stream` ends, so it shares the chip with the prefill's
 * chunk passes; a capture of `stream` captures both branches. out is bf16
 * [num_decodes+num_prefill_tokens][H][V]; norm (optional) as for
 * kda_decode_packed, its gate rows paired with the output rows; the
 * workspace's status word as for kda_chunk_prefill.
 * Errors: as kda_chunk_prefill.
 */
kda_status_t kda_mixed_batch(int32_t num_decodes, int32_t num_prefills,
                             int64_t num_prefill_tokens,
                             const int32_t* prefill_cu_seqlens,
                             const uint8_t* has_initial_state,
                             int32_t H, int32_t K, int32_t V,
                             const void* mixed_qkv, int64_t qkv_row_stride,
                             const void* raw_g, const void* raw_beta,
                             const kda_gate_t* gate, const kda_state_t* state,
                             const kda_out_norm_t* norm, void* out,
                             void* workspace, size_t workspace_bytes,
                             kda_overlap_t overlap, hipStream_t stream);

/* Short causal conv prologue (vLLM PR #60683, Purpose: in the decode
 * kernels a conv step precedes the KDA recurrence; the page prints no
 * formula, so this is a reading). It produces mixed_qkv from the [q | k | v]
 * pre-activations x (D = 2*H*K + H*V channels, head-major as in mixed_qkv).
 * Per sequence and channel c:
 *     a[t][c] = bias[c] + sum_{i<width} weight[c*width + i] * x[t-(width-1)+i][c]
 * where the inputs before the sequence's first row come from its conv state
 * (the width-1 previous inputs, oldest first), read as zero on a null slot
 * or when has_initial_state[i] == 0. Then y = silu(a) = a*sigmoid(a), and q
 * and k of each head are divided by sqrt(sum of squares + l2_eps). The new
 * conv state, the sequence's last width-1 inputs (older ones from the old
 * state for a shorter sequence), is written back bit for bit unless the
 * slot is null or the sequence empty. */
typedef struct {
  const float* weight;      /* device fp32 [D][width], 16-byte aligned          */
  const float* bias;        /* device fp32 [D] (16-byte aligned), or NULL       */
  int32_t width;            /* 2..4                                             */
  float l2_eps;             /* > 0, finite                                      */
  void* conv_state;         /* device bf16 pool, 16-byte aligned; slot s at
                               conv_state + s*conv_slot_stride: [width-1][D]    */
  int64_t conv_slot_stride; /* elements, >= (width-1)*D, a multiple of 8        */
  int64_t num_slots;        /* >= 1                                             */
} kda_short_conv_t;

/*
 * Varlen: sequence i covers rows cu_seqlens[i] .. cu_seqlens[i+1]-1 (device
 * int32 [num_seqs+1], cu_seqlens[num_seqs] == num_rows; a decode batch is
 * sequences of one row, a spec-verify step sequences of tokens_per_seq rows)
 * and uses conv-state slot indices[i*index_stride] (the same slot numbers as
 * the KDA state pool). has_initial_state: device uint8 [num_seqs] or NULL.
 *   x          bf16 [num_rows][x_row_stride], x_row_stride >= D, multiple of 8.
 *   mixed_qkv  bf16 [num_rows][qkv_row_stride] output, qkv_row_stride >= D,
 *              multiple of 8; must not overlap x.
 * Errors: KDA_ERR_INVALID_ARGUMENT, KDA_ERR_UNSUPPORTED, KDA_ERR_HIP.
 */
kda_status_t kda_short_conv(int32_t num_seqs, int64_t num_rows,
                            const int32_t* cu_seqlens,
                            const uint8_t* has_initial_state,
                            int32_t H, int32_t K, int32_t V,
                            const void* x, int64_t x_row_stride,
                            const kda_short_conv_t* conv,
                            const int32_t* indices, int64_t index_stride,
                            void* mixed_qkv, int64_t qkv_row_stride,
                            hipStream_t stream);

/*
 * Packed decode with the short conv prologue fused (vLLM PR #60683, Purpose:
 * its decode kernel runs the conv step, the KDA recurrence and the gated
 * RMSNorm as one kernel). As kda_decode_packed, except that q, k and v come
 * from the [q | k | v] pre-activations x through the conv of
 * kda_short_conv, and mixed_qkv is never materialised:
 *   x     bf16 [num_seqs*tokens_per_seq][x_row_stride], x_row_stride >= D
 *         (D = 2*H*K + H*V), a multiple of 8, 16-byte aligned;
 *   conv  weights, bias, width, l2_eps and the bf16 conv-state pool, as for
 *         kda_short_conv; conv->num_slots >= state->num_slots.
 * Request n's tokens form one conv sequence whose conv-state slot is its KDA
 * state slot (state->indices); the conv state is read as the request's
 * initial state and replaced by its last width-1 inputs. A null slot reads
 * and writes neither state and yields zero output rows. The staged q, k and
 * v are bit-identical to those a kda_short_conv call writes into mixed_qkv
 * (same arithmetic, bf16 rounding included), and the decode kernel that
 * consumes them is kda_decode_packed's per-token kernel, also for requests of
 * several tokens (the spec-verify block form is not used on this path).
 * One launch when a workgroup holds whole heads (num_seqs*H >= 512, or
 * >= 256 with V = 64); otherwise the new conv states are written by a
 * second, small launch after the decode kernel.
 * Errors: as kda_decode_packed and kda_short_conv (row-input checks name x).
 */
kda_status_t kda_conv_decode_packed(int32_t num_seqs, int32_t tokens_per_seq,
                                    int32_t H, int32_t K, int32_t V,
                                    const void* x, int64_t x_row_stride,
                                    const kda_short_conv_t* conv,
                                    const void* raw_g, const void* raw_beta,
                                    const kda_gate_t* gate, const kda_state_t* state,
                                    const kda_out_norm_t* norm, void* out,
                                    hipStream_t stream);

/* Static name of a status code. */
const char* kda_status_string(kda_status_t status);

/* Detail of the last failed call on the calling thread: every failed check,
 * separated by "; ". Empty after a successful call. The pointer stays valid
 * until the next call on the same thread. */
const char* kda_last_error(void);

/* Library version string. */
const char* kda_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
