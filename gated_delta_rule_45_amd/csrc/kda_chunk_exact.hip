// kda_chunk_exact.hip -- the exact-path variants of the chunked-prefill map,
// scan and state kernels (the chunk operands of chunk_kda_with_fused_gate,
// vLLM PR #50649, Purpose, for gates too steep for the factored form).
//
// The kernels are the templates of kda_chunk.hip with EXACT = true, compiled
// in a translation unit of their own so that they keep the default machine
// scheduler: the exact path's diagonal blocks hold more live values than the
// factored path, and the iterative ILP scheduler used for kda_chunk.hip
// spills several hundred VGPRs on them. kda_chunk.hip's launch_prefill runs
// the plan and then calls launch_prefill_exact when some chunk may need the
// exact form.
#define KDA_CHUNK_EXACT_PART 1
#include "kda_chunk.hip"
