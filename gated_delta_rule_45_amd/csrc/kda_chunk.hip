// kda_chunk.hip -- chunked prefill (placeholder until the chunk kernels land).
#include "kda_internal.h"

namespace kda {

size_t prefill_workspace_bytes(int32_t num_seqs, int64_t num_tokens, int32_t H, int32_t K,
                               int32_t V) {
  (void)K; (void)V;
  const int64_t chunks = num_tokens / 64 + num_seqs;
  return static_cast<size_t>(chunks) * H * 256 + 256;
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  (void)p; (void)stream;
  return hipErrorNotSupported;
}

}  // namespace kda
