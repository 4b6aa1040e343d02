// kda_api.hip -- C-ABI front end: argument validation, launch planning and the
// mixed-batch router. Every entry point validates everything on the host
// first, launches nothing when any check fails, and reports every failed
// check at once (the all-reasons error convention of vLLM PR #60683, Refusal
// and steps). No entry point allocates, frees, synchronises or reads device
// memory from the host.
#include <cmath>
#include <cstdio>
#include <mutex>
#include <new>
#include <string>

#include "kda.h"
#include "kda_internal.h"

// Overlap resources of kda_mixed_batch, created and owned by the caller: a
// side stream for the decode rows and the two events that fork it from the
// caller's stream and join it back, all on one device.
struct kda_overlap_s {
  int device;
  hipStream_t stream;
  hipEvent_t fork, join;
};

namespace {

thread_local std::string g_last_error;

class Checks {
 public:
  void require(bool ok, kda_status_t code, const std::string& msg) {
    if (ok) return;
    if (!msg_.empty()) msg_ += "; ";
    msg_ += msg;
    // The most specific code wins: invalid argument over the others.
    if (status_ == KDA_OK || code == KDA_ERR_INVALID_ARGUMENT) status_ = code;
  }
  kda_status_t finish() {
    g_last_error = msg_;
    return status_;
  }
  bool ok() const { return status_ == KDA_OK; }

 private:
  kda_status_t status_ = KDA_OK;
  std::string msg_;
};

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Workspace of kda_chunk_prefill_noalloc: one static buffer per GPU, held
// until the process ends. In host code `scratch` names a host-side stand-in,
// not device memory; its device address on each GPU comes from
// hipGetSymbolAddress (looked up once per device, with that device current)
// and only that address is ever handed to kernels.
constexpr size_t kNoallocScratchBytes = KDA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device a call's work runs on: the stream's (the current device for
// the null stream).
hipError_t stream_device(hipStream_t stream, int* dev) {
  if (stream == nullptr) return hipGetDevice(dev);
  hipDevice_t d = 0;
  const hipError_t e = hipStreamGetDevice(stream, &d);
  if (e == hipSuccess) *dev = static_cast<int>(d);
  return e;
}

// Device address of the scratch on the GPU that `stream` runs on, looked up
// on the first call for that GPU with that GPU current (and the caller's
// current device restored).
hipError_t noalloc_scratch(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = stream_device(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t er = hipSetDevice(cur);
      if (e == hipSuccess) e = er;
    }
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// Checks shared by all entry points. rows: number of token rows the call reads.
// qkv_name and stride_name name the row input and its row stride in
// messages (mixed_qkv, or x for the conv entry).
void check_common(Checks& c, int64_t rows, int32_t H, int32_t K, int32_t V,
                  const void* mixed_qkv, int64_t qkv_row_stride, const void* raw_g,
                  const void* raw_beta, const kda_gate_t* gate, const kda_state_t* state,
                  const void* out, const std::string& qkv_name = "mixed_qkv",
                  const std::string& stride_name = "qkv_row_stride") {
  const auto INV = KDA_ERR_INVALID_ARGUMENT;
  const auto UNS = KDA_ERR_UNSUPPORTED;
  c.require(H >= 1, INV, "H must be >= 1");
  c.require(K >= 1 && V >= 1, INV, "K and V must be >= 1");
  c.require(K == 64 || K == 128 || K < 1, UNS, "K must be 64 or 128");
  c.require(V == 64 || V == 128 || V < 1, UNS, "V must be 64 or 128");
  c.require(gate != nullptr, INV, "gate must not be NULL");
  c.require(state != nullptr, INV, "state must not be NULL");
  if (gate) {
    c.require(gate->A_log != nullptr, INV, "gate->A_log must not be NULL");
    c.require(gate->dt_bias != nullptr, INV, "gate->dt_bias must not be NULL");
    c.require(std::isfinite(gate->scale), INV, "gate->scale must be finite");
    if (gate->has_lower_bound)
      c.require(std::isfinite(gate->lower_bound) && gate->lower_bound <= 0.0f, INV,
                "gate->lower_bound must be finite and <= 0");
  }
  if (state) {
    c.require(state->index_stride >= 1, INV,
              "state->index_stride must be >= 1 (a non-positive stride is rejected)");
    c.require(state->indices != nullptr, INV, "state->indices must not be NULL");
    c.require(state->pool != nullptr, INV, "state->pool must not be NULL");
    c.require(state->num_slots >= 1, INV, "state->num_slots must be >= 1");
    if (H >= 1 && K >= 1 && V >= 1)
      c.require(state->slot_stride >= static_cast<int64_t>(H) * K * V, INV,
                "state->slot_stride must be >= H*K*V");
    c.require(aligned(state->pool, 16), UNS, "state->pool must be 16-byte aligned");
    c.require(state->slot_stride % 4 == 0, UNS, "state->slot_stride must be a multiple of 4");
  }
  if (rows > 0) {
    c.require(mixed_qkv != nullptr, INV, qkv_name + " must not be NULL");
    c.require(raw_g != nullptr, INV, "raw_g must not be NULL");
    c.require(raw_beta != nullptr, INV, "raw_beta must not be NULL");
    c.require(out != nullptr, INV, "out must not be NULL");
    if (H >= 1 && K >= 1 && V >= 1)
      c.require(qkv_row_stride >= 2 * static_cast<int64_t>(H) * K + static_cast<int64_t>(H) * V, INV,
                stride_name + " must be >= 2*H*K + H*V");
    c.require(qkv_row_stride % 8 == 0, UNS, stride_name + " must be a multiple of 8");
    c.require(qkv_row_stride <= (int64_t{1} << 24), UNS,
              stride_name + " must be <= 2^24 (kernels address 64 rows with 32-bit offsets)");
    c.require(aligned(mixed_qkv, 16), UNS, qkv_name + " must be 16-byte aligned");
    c.require(aligned(raw_g, 16), UNS, "raw_g must be 16-byte aligned");
    c.require(aligned(raw_beta, 2), UNS, "raw_beta must be 2-byte aligned");
    c.require(aligned(out, 16), UNS, "out must be 16-byte aligned");
  }
}

// The optional output epilogue: rows gate rows pair with the call's output rows.
void check_norm(Checks& c, int64_t rows, int32_t H, int32_t V, const kda_out_norm_t* norm) {
  if (norm == nullptr) return;
  const auto INV = KDA_ERR_INVALID_ARGUMENT;
  const auto UNS = KDA_ERR_UNSUPPORTED;
  c.require(norm->activation == KDA_NORM_SIGMOID || norm->activation == KDA_NORM_SILU, INV,
            "norm->activation must be KDA_NORM_SIGMOID or KDA_NORM_SILU");
  c.require(std::isfinite(norm->eps) && norm->eps > 0.0f, INV, "norm->eps must be finite and > 0");
  if (rows > 0) {
    c.require(norm->gate != nullptr, INV, "norm->gate must not be NULL");
    c.require(norm->weight != nullptr, INV, "norm->weight must not be NULL");
    if (H >= 1 && V >= 1)
      c.require(norm->gate_row_stride >= static_cast<int64_t>(H) * V, INV,
                "norm->gate_row_stride must be >= H*V");
    c.require(norm->gate_row_stride % 8 == 0, UNS, "norm->gate_row_stride must be a multiple of 8");
    c.require(aligned(norm->gate, 16), UNS, "norm->gate must be 16-byte aligned");
    c.require(aligned(norm->weight, 16), UNS, "norm->weight must be 16-byte aligned");
  }
}

kda::OutNorm out_norm(const kda_out_norm_t* norm, int64_t first_row) {
  kda::OutNorm n{};
  if (norm == nullptr) return n;
  n.gate = static_cast<const uint16_t*>(norm->gate) + first_row * norm->gate_row_stride;
  n.gate_row_stride = norm->gate_row_stride;
  n.weight = norm->weight;
  n.eps = norm->eps;
  n.activation = norm->activation;
  return n;
}

kda::DecodeParams decode_params(int32_t num_seqs, int32_t tps, int32_t H, int32_t V,
                                const void* mixed_qkv, int64_t qkv_row_stride, const void* raw_g,
                                const void* raw_beta, const kda_gate_t* gate,
                                const kda_state_t* state, void* out) {
  kda::DecodeParams p{};
  p.qkv = static_cast<const uint16_t*>(mixed_qkv);
  p.qkv_row_stride = qkv_row_stride;
  p.raw_g = static_cast<const uint16_t*>(raw_g);
  p.raw_beta = static_cast<const uint16_t*>(raw_beta);
  p.A_log = gate->A_log;
  p.dt_bias = gate->dt_bias;
  p.has_lb = gate->has_lower_bound ? 1 : 0;
  p.lower_bound = gate->lower_bound;
  p.scale = gate->scale;
  p.pool = state->pool;
  p.slot_stride = state->slot_stride;
  p.indices = state->indices;
  p.index_stride = state->index_stride;
  p.out = static_cast<uint16_t*>(out);
  p.num_seqs = num_seqs;
  p.tokens_per_seq = tps;
  p.H = H;
  p.V = V;
  return p;
}

kda_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) {
    g_last_error.clear();
    return KDA_OK;
  }
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return KDA_ERR_HIP;
}

// The conv weights, bias and state pool.
void check_conv(Checks& c, const kda_short_conv_t* conv, int32_t H, int32_t K, int32_t V) {
  const auto INV = KDA_ERR_INVALID_ARGUMENT;
  const auto UNS = KDA_ERR_UNSUPPORTED;
  c.require(conv != nullptr, INV, "conv must not be NULL");
  if (conv == nullptr) return;
  const int64_t D = 2 * static_cast<int64_t>(H) * K + static_cast<int64_t>(H) * V;
  c.require(conv->width >= 2 && conv->width <= 4, UNS, "conv->width must be 2, 3 or 4");
  c.require(std::isfinite(conv->l2_eps) && conv->l2_eps > 0.0f, INV, "conv->l2_eps must be finite and > 0");
  c.require(conv->weight != nullptr, INV, "conv->weight must not be NULL");
  c.require(aligned(conv->weight, 16), UNS, "conv->weight must be 16-byte aligned");
  c.require(conv->bias == nullptr || aligned(conv->bias, 16), UNS, "conv->bias must be 16-byte aligned");
  c.require(conv->conv_state != nullptr, INV, "conv->conv_state must not be NULL");
  c.require(aligned(conv->conv_state, 16), UNS, "conv->conv_state must be 16-byte aligned");
  c.require(conv->num_slots >= 1, INV, "conv->num_slots must be >= 1");
  if (H >= 1)
    c.require(conv->conv_slot_stride >= (conv->width - 1) * D, INV,
              "conv->conv_slot_stride must be >= (width-1)*D");
  c.require(conv->conv_slot_stride % 8 == 0, UNS, "conv->conv_slot_stride must be a multiple of 8");
}

kda::PrefillParams prefill_params(int32_t num_seqs, int64_t num_tokens, const int32_t* cu_seqlens,
                                  const uint8_t* has_initial_state, int32_t H, int32_t K,
                                  int32_t V, const void* mixed_qkv, int64_t qkv_row_stride,
                                  const void* raw_g, const void* raw_beta,
                                  const kda_gate_t* gate, const kda_state_t* state, void* out,
                                  void* workspace, size_t workspace_bytes) {
  kda::PrefillParams p{};
  p.qkv = static_cast<const uint16_t*>(mixed_qkv);
  p.qkv_row_stride = qkv_row_stride;
  p.raw_g = static_cast<const uint16_t*>(raw_g);
  p.raw_beta = static_cast<const uint16_t*>(raw_beta);
  p.A_log = gate->A_log;
  p.dt_bias = gate->dt_bias;
  p.has_lb = gate->has_lower_bound ? 1 : 0;
  p.lower_bound = gate->lower_bound;
  p.scale = gate->scale;
  p.pool = state->pool;
  p.slot_stride = state->slot_stride;
  p.indices = state->indices;
  p.index_stride = state->index_stride;
  p.out = static_cast<uint16_t*>(out);
  p.cu_seqlens = cu_seqlens;
  p.has_initial_state = has_initial_state;
  p.num_seqs = num_seqs;
  p.num_tokens = num_tokens;
  p.H = H;
  p.K = K;
  p.V = V;
  p.workspace = workspace;
  p.workspace_bytes = workspace_bytes;
  return p;
}

void check_prefill_specific(Checks& c, int32_t num_seqs, int64_t num_tokens,
                            const int32_t* cu_seqlens, int32_t H, int32_t K, int32_t V,
                            void* workspace, size_t workspace_bytes) {
  const auto INV = KDA_ERR_INVALID_ARGUMENT;
  c.require(num_seqs >= 0, INV, "num_seqs must be >= 0");
  c.require(num_tokens >= 0, INV, "num_tokens must be >= 0");
  c.require(num_tokens <= 0x7fffffffLL, INV, "num_tokens must fit in int32");
  if (num_seqs > 0) c.require(cu_seqlens != nullptr, INV, "cu_seqlens must not be NULL");
  c.require(num_tokens == 0 || num_seqs > 0, INV, "num_tokens > 0 needs num_seqs > 0");
  if (num_seqs > 0 && num_tokens > 0 && H >= 1 && (K == 64 || K == 128) && (V == 64 || V == 128)) {
    const size_t need = kda::prefill_workspace_min_bytes(num_seqs, num_tokens, H, K, V);
    c.require(workspace != nullptr && workspace_bytes >= need, KDA_ERR_WORKSPACE,
              "workspace must be at least kda_chunk_prefill_workspace_min_size() bytes (" +
                  std::to_string(need) + ")");
    c.require(aligned(workspace, 256), KDA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
}

}  // namespace

extern "C" {

kda_status_t kda_decode_packed(int32_t num_seqs, int32_t tokens_per_seq, int32_t H, int32_t K,
                               int32_t V, const void* mixed_qkv, int64_t qkv_row_stride,
                               const void* raw_g, const void* raw_beta, const kda_gate_t* gate,
                               const kda_state_t* state, const kda_out_norm_t* norm, void* out,
                               hipStream_t stream) {
  Checks c;
  const auto INV = KDA_ERR_INVALID_ARGUMENT;
  c.require(num_seqs >= 0, INV, "num_seqs must be >= 0");
  c.require(tokens_per_seq >= 1 && tokens_per_seq <= 8, INV,
            "tokens_per_seq must be in 1..8 (spec-verify steps have at most 8 rows per request)");
  const int64_t rows = static_cast<int64_t>(num_seqs) * tokens_per_seq;
  c.require(rows <= 0x7fffffffLL, INV, "num_seqs * tokens_per_seq must fit in int32");
  check_common(c, rows, H, K, V, mixed_qkv, qkv_row_stride, raw_g, raw_beta, gate, state, out);
  check_norm(c, rows, H, V, norm);
  if (!c.ok()) return c.finish();
  if (num_seqs == 0) return c.finish();
  kda::DecodeParams p = decode_params(num_seqs, tokens_per_seq, H, V, mixed_qkv, qkv_row_stride,
                                      raw_g, raw_beta, gate, state, out);
  p.norm = out_norm(norm, 0);
  return hip_status(kda::launch_decode(p, K, stream), "decode launch");
}

kda_status_t kda_conv_decode_packed(int32_t num_seqs, int32_t tokens_per_seq, int32_t H, int32_t K,
                                    int32_t V, const void* x, int64_t x_row_stride,
                                    const kda_short_conv_t* conv, const void* raw_g,
                                    const void* raw_beta, const kda_gate_t* gate,
                                    const kda_state_t* state, const kda_out_norm_t* norm, void* out,
                                    hipStream_t stream) {
  Checks c;
  const auto INV = KDA_ERR_INVALID_ARGUMENT;
  c.require(num_seqs >= 0, INV, "num_seqs must be >= 0");
  c.require(tokens_per_seq >= 1 && tokens_per_seq <= 8, INV,
            "tokens_per_seq must be in 1..8 (spec-verify steps have at most 8 rows per request)");
  const int64_t rows = static_cast<int64_t>(num_seqs) * tokens_per_seq;
  c.require(rows <= 0x7fffffffLL, INV, "num_seqs * tokens_per_seq must fit in int32");
  check_common(c, rows, H, K, V, x, x_row_stride, raw_g, raw_beta, gate, state, out, "x", "x_row_stride");
  check_norm(c, rows, H, V, norm);
  check_conv(c, conv, H, K, V);
  if (conv && state)
    c.require(conv->num_slots >= state->num_slots, INV,
              "conv->num_slots must be >= state->num_slots (the conv state shares the slot numbers)");
  if (!c.ok()) return c.finish();
  if (num_seqs == 0) return c.finish();
  kda::DecodeParams p = decode_params(num_seqs, tokens_per_seq, H, V, nullptr, x_row_stride, raw_g,
                                      raw_beta, gate, state, out);
  p.norm = out_norm(norm, 0);
  p.conv.x = static_cast<const uint16_t*>(x);
  p.conv.x_row_stride = x_row_stride;
  p.conv.weight = conv->weight;
  p.conv.bias = conv->bias;
  p.conv.width = conv->width;
  p.conv.l2_eps = conv->l2_eps;
  p.conv.conv_state = static_cast<uint16_t*>(conv->conv_state);
  p.conv.conv_slot_stride = conv->conv_slot_stride;
  return hip_status(kda::launch_decode(p, K, stream), "conv decode launch");
}

kda_status_t kda_spec_decode(int32_t num_seqs, int32_t tokens_per_seq, int32_t H, int32_t K,
                             int32_t V, const void* mixed_qkv, int64_t qkv_row_stride,
                             const void* raw_g, const void* raw_beta, const kda_gate_t* gate,
                             const kda_state_t* state, int64_t index_col_stride,
                             const int32_t* num_accepted_tokens, const kda_out_norm_t* norm,
                             void* out, hipStream_t stream) {
  Checks c;
  const auto INV = KDA_ERR_INVALID_ARGUMENT;
  c.require(num_seqs >= 0, INV, "num_seqs must be >= 0");
  c.require(tokens_per_seq >= 1 && tokens_per_seq <= 8, INV,
            "tokens_per_seq must be in 1..8 (spec-verify steps have at most 8 rows per request)");
  const int64_t rows = static_cast<int64_t>(num_seqs) * tokens_per_seq;
  c.require(rows <= 0x7fffffffLL, INV, "num_seqs * tokens_per_seq must fit in int32");
  c.require(index_col_stride >= 1, INV, "index_col_stride must be >= 1");
  c.require(num_accepted_tokens != nullptr, INV, "num_accepted_tokens must not be NULL");
  check_common(c, rows, H, K, V, mixed_qkv, qkv_row_stride, raw_g, raw_beta, gate, state, out);
  check_norm(c, rows, H, V, norm);
  if (!c.ok()) return c.finish();
  if (num_seqs == 0) return c.finish();
  kda::DecodeParams p = decode_params(num_seqs, tokens_per_seq, H, V, mixed_qkv, qkv_row_stride,
                                      raw_g, raw_beta, gate, state, out);
  p.norm = out_norm(norm, 0);
  p.num_accepted = num_accepted_tokens;
  p.index_col_stride = index_col_stride;
  return hip_status(kda::launch_decode(p, K, stream), "spec decode launch");
}

size_t kda_chunk_prefill_workspace_size(int32_t num_seqs, int64_t num_tokens, int32_t H, int32_t K,
                                        int32_t V) {
  if (num_seqs < 0 || num_tokens < 0 || H < 1 || !(K == 64 || K == 128) || !(V == 64 || V == 128))
    return 0;
  return kda::prefill_workspace_bytes(num_seqs, num_tokens, H, K, V);
}

size_t kda_chunk_prefill_workspace_min_size(int32_t num_seqs, int64_t num_tokens, int32_t H, int32_t K,
                                            int32_t V) {
  if (num_seqs < 0 || num_tokens < 0 || H < 1 || !(K == 64 || K == 128) || !(V == 64 || V == 128))
    return 0;
  return kda::prefill_workspace_min_bytes(num_seqs, num_tokens, H, K, V);
}

kda_status_t kda_chunk_prefill_workspace_maps(int32_t num_seqs, int64_t num_tokens, int32_t H, int32_t K,
                                              int32_t V, size_t* offset, size_t* item_bytes,
                                              int64_t* items) {
  Checks c;
  c.require(num_seqs >= 0 && num_tokens >= 0 && H >= 1, KDA_ERR_INVALID_ARGUMENT,
            "num_seqs, num_tokens must be >= 0 and H >= 1");
  c.require((K == 64 || K == 128) && (V == 64 || V == 128), KDA_ERR_UNSUPPORTED, "K and V must be 64 or 128");
  c.require(offset != nullptr && item_bytes != nullptr && items != nullptr, KDA_ERR_INVALID_ARGUMENT,
            "offset, item_bytes and items are required");
  if (!c.ok()) return c.finish();
  kda::prefill_workspace_maps(num_seqs, num_tokens, H, K, V, offset, item_bytes, items);
  return c.finish();
}

kda_status_t kda_chunk_prefill(int32_t num_seqs, int64_t num_tokens, const int32_t* cu_seqlens,
                               const uint8_t* has_initial_state, int32_t H, int32_t K, int32_t V,
                               const void* mixed_qkv, int64_t qkv_row_stride, const void* raw_g,
                               const void* raw_beta, const kda_gate_t* gate,
                               const kda_state_t* state, const kda_out_norm_t* norm, void* out,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Checks c;
  check_common(c, num_tokens, H, K, V, mixed_qkv, qkv_row_stride, raw_g, raw_beta, gate, state, out);
  check_prefill_specific(c, num_seqs, num_tokens, cu_seqlens, H, K, V, workspace, workspace_bytes);
  check_norm(c, num_tokens, H, V, norm);
  if (!c.ok()) return c.finish();
  if (num_seqs == 0 || num_tokens == 0) return c.finish();
  kda::PrefillParams p =
      prefill_params(num_seqs, num_tokens, cu_seqlens, has_initial_state, H, K, V, mixed_qkv,
                     qkv_row_stride, raw_g, raw_beta, gate, state, out, workspace, workspace_bytes);
  p.norm = out_norm(norm, 0);
  return hip_status(kda::launch_prefill(p, stream), "prefill launch");
}

kda_status_t kda_chunk_prefill_noalloc(int32_t num_seqs, int64_t num_tokens,
                                       const int32_t* cu_seqlens,
                                       const uint8_t* has_initial_state, int32_t H, int32_t K,
                                       int32_t V, const void* mixed_qkv, int64_t qkv_row_stride,
                                       const void* raw_g, const void* raw_beta,
                                       const kda_gate_t* gate, const kda_state_t* state,
                                       const kda_out_norm_t* norm, void* out,
                                       hipStream_t stream) {
  Checks c;
  check_common(c, num_tokens, H, K, V, mixed_qkv, qkv_row_stride, raw_g, raw_beta, gate, state, out);
  size_t need = 0;
  if (num_seqs > 0 && num_tokens > 0 && H >= 1 && (K == 64 || K == 128) && (V == 64 || V == 128))
    need = kda::prefill_workspace_min_bytes(num_seqs, num_tokens, H, K, V);
  c.require(need <= kNoallocScratchBytes, KDA_ERR_WORKSPACE,
            "these sizes need " + std::to_string(need) + " bytes of workspace, more than the " +
                std::to_string(kNoallocScratchBytes) + " bytes of the static scratch (KDA_NOALLOC_SCRATCH_BYTES)");
  // The size check above stands in for the workspace argument's checks.
  void* ws = reinterpret_cast<void*>(uintptr_t{256});
  check_prefill_specific(c, num_seqs, num_tokens, cu_seqlens, H, K, V, ws, SIZE_MAX);
  check_norm(c, num_tokens, H, V, norm);
  if (!c.ok()) return c.finish();
  if (num_seqs == 0 || num_tokens == 0) return c.finish();
  const hipError_t e = noalloc_scratch(stream, &ws);
  if (e != hipSuccess) return hip_status(e, "prefill (no-alloc): scratch address");
  kda::PrefillParams p =
      prefill_params(num_seqs, num_tokens, cu_seqlens, has_initial_state, H, K, V, mixed_qkv,
                     qkv_row_stride, raw_g, raw_beta, gate, state, out, ws, kNoallocScratchBytes);
  p.norm = out_norm(norm, 0);
  return hip_status(kda::launch_prefill(p, stream), "prefill (no-alloc) launch");
}

size_t kda_mixed_batch_workspace_size(int32_t num_decodes, int32_t num_prefills,
                                      int64_t num_prefill_tokens, int32_t H, int32_t K,
                                      int32_t V) {
  if (num_decodes < 0) return 0;
  return kda_chunk_prefill_workspace_size(num_prefills, num_prefill_tokens, H, K, V);
}

kda_status_t kda_overlap_create(kda_overlap_t* overlap) {
  Checks c;
  c.require(overlap != nullptr, KDA_ERR_INVALID_ARGUMENT, "overlap must not be NULL");
  if (!c.ok()) return c.finish();
  *overlap = nullptr;
  kda_overlap_s* o = new (std::nothrow) kda_overlap_s{0, nullptr, nullptr, nullptr};
  if (o == nullptr) {
    g_last_error = "kda_overlap_create: out of host memory";
    return KDA_ERR_HIP;
  }
  hipError_t e = hipGetDevice(&o->device);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&o->stream, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&o->fork, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&o->join, hipEventDisableTiming);
  if (e != hipSuccess) {
    kda_overlap_destroy(o);
    return hip_status(e, "kda_overlap_create");
  }
  *overlap = o;
  g_last_error.clear();
  return KDA_OK;
}

kda_status_t kda_overlap_destroy(kda_overlap_t overlap) {
  if (overlap == nullptr) return KDA_OK;
  hipError_t e = hipSuccess, ei;
  if (overlap->join && (ei = hipEventDestroy(overlap->join)) != hipSuccess) e = ei;
  if (overlap->fork && (ei = hipEventDestroy(overlap->fork)) != hipSuccess) e = ei;
  if (overlap->stream && (ei = hipStreamDestroy(overlap->stream)) != hipSuccess) e = ei;
  delete overlap;
  return hip_status(e, "kda_overlap_destroy");
}

kda_status_t kda_mixed_batch(int32_t num_decodes, int32_t num_prefills, int64_t num_prefill_tokens,
                             const int32_t* prefill_cu_seqlens, const uint8_t* has_initial_state,
                             int32_t H, int32_t K, int32_t V, const void* mixed_qkv,
                             int64_t qkv_row_stride, const void* raw_g, const void* raw_beta,
                             const kda_gate_t* gate, const kda_state_t* state,
                             const kda_out_norm_t* norm, void* out, void* workspace,
                             size_t workspace_bytes, kda_overlap_t overlap, hipStream_t stream) {
  Checks c;
  const auto INV = KDA_ERR_INVALID_ARGUMENT;
  c.require(num_decodes >= 0, INV, "num_decodes must be >= 0");
  const int64_t rows = static_cast<int64_t>(num_decodes) + num_prefill_tokens;
  c.require(rows <= 0x7fffffffLL, INV, "num_decodes + num_prefill_tokens must fit in int32");
  check_common(c, rows, H, K, V, mixed_qkv, qkv_row_stride, raw_g, raw_beta, gate, state, out);
  check_prefill_specific(c, num_prefills, num_prefill_tokens, prefill_cu_seqlens, H, K, V,
                         workspace, workspace_bytes);
  check_norm(c, rows, H, V, norm);
  if (overlap != nullptr) {
    int dev = -1;
    const hipError_t e = stream_device(stream, &dev);
    c.require(e == hipSuccess && dev == overlap->device, INV,
              "overlap was created on another device than the one `stream` runs on");
  }
  if (!c.ok()) return c.finish();

  // Decode rows [0, D) go to the recurrent kernel, one token per request;
  // prefill rows [D, D + P) to the chunk pipeline on the shifted views (only
  // host pointer arithmetic; device data is never read here). The two parts
  // touch disjoint slots and rows. With the caller's overlap resources the
  // decode rows run on its side stream, forked from `stream` once the
  // prefill's plan kernel is launched and joined back after the decode
  // kernel: the HBM-bound decode kernel then shares the chip with the
  // prefill's chunk passes. Without them both run on `stream`, decode first.
  const bool has_decode = num_decodes > 0;
  const bool has_prefill = num_prefills > 0 && num_prefill_tokens > 0;
  auto launch_decode_rows = [&](hipStream_t s) -> hipError_t {
    kda::DecodeParams p = decode_params(num_decodes, 1, H, V, mixed_qkv, qkv_row_stride, raw_g,
                                        raw_beta, gate, state, out);
    p.norm = out_norm(norm, 0);
    return kda::launch_decode(p, K, s);
  };
  auto launch_prefill_rows = [&](hipStream_t s, hipEvent_t after_plan) -> hipError_t {
    const int64_t D = num_decodes;
    const uint16_t* qkv = static_cast<const uint16_t*>(mixed_qkv) + D * qkv_row_stride;
    const uint16_t* rg = static_cast<const uint16_t*>(raw_g) + D * H * K;
    const uint16_t* rb = static_cast<const uint16_t*>(raw_beta) + D * H;
    uint16_t* o = static_cast<uint16_t*>(out) + D * H * V;
    kda_state_t st = *state;
    st.indices = state->indices + D * state->index_stride;
    kda::PrefillParams p =
        prefill_params(num_prefills, num_prefill_tokens, prefill_cu_seqlens, has_initial_state, H,
                       K, V, qkv, qkv_row_stride, rg, rb, gate, &st, o, workspace, workspace_bytes);
    p.norm = out_norm(norm, D);
    return kda::launch_prefill(p, s, after_plan);
  };
  if (has_decode && has_prefill && overlap != nullptr) {
    // The fork is recorded inside the prefill launch, after its plan
    // kernel; once the side stream waits on it, it is joined back whatever
    // fails in between, so it never outlives the call's work on `stream`
    // (and a capture of `stream` stays joined).
    const hipError_t ep = launch_prefill_rows(stream, overlap->fork);
    if (ep != hipSuccess) return hip_status(ep, "mixed batch: prefill launch");
    hipError_t e;
    if ((e = hipStreamWaitEvent(overlap->stream, overlap->fork, 0)) != hipSuccess)
      return hip_status(e, "mixed batch: fork");
    const hipError_t ed = launch_decode_rows(overlap->stream);
    if ((e = hipEventRecord(overlap->join, overlap->stream)) != hipSuccess) return hip_status(e, "mixed batch: join");
    if ((e = hipStreamWaitEvent(stream, overlap->join, 0)) != hipSuccess) return hip_status(e, "mixed batch: join");
    if (ed != hipSuccess) return hip_status(ed, "mixed batch: decode launch");
  } else {
    if (has_decode) {
      const hipError_t e = launch_decode_rows(stream);
      if (e != hipSuccess) return hip_status(e, "mixed batch: decode launch");
    }
    if (has_prefill) {
      const hipError_t e = launch_prefill_rows(stream, nullptr);
      if (e != hipSuccess) return hip_status(e, "mixed batch: prefill launch");
    }
  }
  g_last_error.clear();
  return KDA_OK;
}

kda_status_t kda_short_conv(int32_t num_seqs, int64_t num_rows, const int32_t* cu_seqlens,
                            const uint8_t* has_initial_state, int32_t H, int32_t K, int32_t V,
                            const void* x, int64_t x_row_stride, const kda_short_conv_t* conv,
                            const int32_t* indices, int64_t index_stride, void* mixed_qkv,
                            int64_t qkv_row_stride, hipStream_t stream) {
  Checks c;
  const auto INV = KDA_ERR_INVALID_ARGUMENT;
  const auto UNS = KDA_ERR_UNSUPPORTED;
  c.require(num_seqs >= 0, INV, "num_seqs must be >= 0");
  c.require(num_rows >= 0 && num_rows <= 0x7fffffffLL, INV, "num_rows must be in 0..2^31-1");
  c.require(num_rows == 0 || num_seqs > 0, INV, "num_rows > 0 needs num_seqs > 0");
  if (num_seqs > 0) c.require(cu_seqlens != nullptr, INV, "cu_seqlens must not be NULL");
  c.require(H >= 1, INV, "H must be >= 1");
  c.require(K == 64 || K == 128, UNS, "K must be 64 or 128");
  c.require(V == 64 || V == 128, UNS, "V must be 64 or 128");
  c.require(indices != nullptr || num_seqs == 0, INV, "indices must not be NULL");
  c.require(index_stride >= 1, INV, "index_stride must be >= 1 (a non-positive stride is rejected)");
  check_conv(c, conv, H, K, V);
  const int64_t D = 2 * static_cast<int64_t>(H) * K + static_cast<int64_t>(H) * V;
  if (num_rows > 0) {
    c.require(x != nullptr, INV, "x must not be NULL");
    c.require(mixed_qkv != nullptr, INV, "mixed_qkv must not be NULL");
    if (H >= 1) {
      c.require(x_row_stride >= D, INV, "x_row_stride must be >= 2*H*K + H*V");
      c.require(qkv_row_stride >= D, INV, "qkv_row_stride must be >= 2*H*K + H*V");
    }
    c.require(x_row_stride % 8 == 0 && qkv_row_stride % 8 == 0, UNS,
              "x_row_stride and qkv_row_stride must be multiples of 8");
    c.require(aligned(x, 16) && aligned(mixed_qkv, 16), UNS, "x and mixed_qkv must be 16-byte aligned");
    if (x && mixed_qkv && x_row_stride >= 1 && qkv_row_stride >= 1) {
      const auto xa = reinterpret_cast<uintptr_t>(x), oa = reinterpret_cast<uintptr_t>(mixed_qkv);
      const uintptr_t xe = xa + static_cast<uintptr_t>(num_rows * x_row_stride * 2);
      const uintptr_t oe = oa + static_cast<uintptr_t>(num_rows * qkv_row_stride * 2);
      c.require(xe <= oa || oe <= xa, INV, "mixed_qkv must not overlap x");
    }
  }
  if (!c.ok()) return c.finish();
  if (num_seqs == 0) return c.finish();
  kda::ConvParams p{};
  p.x = static_cast<const uint16_t*>(x);
  p.x_row_stride = x_row_stride;
  p.weight = conv->weight;
  p.bias = conv->bias;
  p.width = conv->width;
  p.l2_eps = conv->l2_eps;
  p.conv_state = static_cast<uint16_t*>(conv->conv_state);
  p.conv_slot_stride = conv->conv_slot_stride;
  p.indices = indices;
  p.index_stride = index_stride;
  p.cu_seqlens = cu_seqlens;
  p.has_initial_state = has_initial_state;
  p.out = static_cast<uint16_t*>(mixed_qkv);
  p.out_row_stride = qkv_row_stride;
  p.num_seqs = num_seqs;
  p.num_rows = num_rows;
  p.H = H;
  p.K = K;
  p.V = V;
  return hip_status(kda::launch_short_conv(p, stream), "short conv launch");
}

const char* kda_status_string(kda_status_t status) {
  switch (status) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE";
    case KDA_ERR_HIP: return "KDA_ERR_HIP";
  }
  return "KDA_ERR_UNKNOWN";
}

const char* kda_last_error(void) { return g_last_error.c_str(); }

const char* kda_version(void) { return "kda-mi355x 0.1 (gfx950)"; }

}  // extern "C"
