// kda_norm.hip -- gated RMSNorm output epilogue as a pass over a call's bf16
// output, in place (vLLM PR #60683, Purpose, names a gated RMSNorm after the
// KDA recurrence; the formula is a reading):
//   y_j = o_j / sqrt(mean_j' o_j'^2 + eps) * weight[j] * act(gate_j)
// per row and head over the head's V channels, act(z) = sigmoid(z) or
// z * sigmoid(z). Used where no workgroup of the producing kernel holds a
// head's whole row (narrow decode column tiles); the prefill state pass
// applies it itself.
//
// HBM-bound elementwise work with one reduction per (row, head): a group of
// V/8 lanes owns a (row, head), each lane 8 consecutive channels (one 16-byte
// load of o, one of the gate, two of the weight), and the sum of squares is
// a butterfly within the group.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kNormThreads = 256;

template <int V>
__global__ __launch_bounds__(kNormThreads) void gated_rmsnorm_kernel(const OutNorm n, uint16_t* out,
                                                                     int64_t pairs, int32_t H) {
  constexpr int LP = V / 8;                  // lanes per (row, head)
  constexpr int PPB = kNormThreads / LP;     // (row, head) pairs per workgroup
  static_assert(64 % LP == 0, "a group stays inside one wave");
  const int64_t pair = static_cast<int64_t>(blockIdx.x) * PPB + threadIdx.x / LP;
  const int l = threadIdx.x % LP;
  // Lanes past the last pair take part in the butterfly on zeros and store
  // nothing; no lane leaves before the shuffles.
  const bool valid = pair < pairs;
  const int64_t pr = valid ? pair : pairs - 1;
  const int64_t row = pr / H;
  const int h = static_cast<int>(pr % H);
  uint16_t* o = out + pr * V + 8 * l;
  const uint16_t* z = n.gate + row * n.gate_row_stride + static_cast<int64_t>(h) * V + 8 * l;
  float ov[8], zv[8];
  load_bf16<8>(o, ov);
  load_bf16<8>(z, zv);
  const f32x4 w0 = *reinterpret_cast<const f32x4*>(n.weight + 8 * l);
  const f32x4 w1 = *reinterpret_cast<const f32x4*>(n.weight + 8 * l + 4);
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) ss = fmaf(ov[j], ov[j], ss);
  if (!valid) ss = 0.f;
#pragma unroll
  for (int off = 1; off < LP; off <<= 1) ss += __shfl_xor(ss, off);
  const float inv = 1.0f / sqrtf(ss * (1.0f / V) + n.eps);
  float y[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float sg = sigmoid_f32(zv[j]);
    const float act = n.activation == 1 ? zv[j] * sg : sg;
    y[j] = ov[j] * inv * (j < 4 ? w0[j] : w1[j - 4]) * act;
  }
  if (valid) {
    uint4 v;
    v.x = pack_bf16x2(y[0], y[1]);
    v.y = pack_bf16x2(y[2], y[3]);
    v.z = pack_bf16x2(y[4], y[5]);
    v.w = pack_bf16x2(y[6], y[7]);
    *reinterpret_cast<uint4*>(o) = v;
  }
}

}  // namespace

hipError_t launch_gated_rmsnorm(const OutNorm& n, uint16_t* out, int64_t rows, int32_t H, int32_t V,
                                hipStream_t stream) {
  const int64_t pairs = rows * H;
  if (pairs <= 0) return hipSuccess;
  const int64_t ppb = kNormThreads / (V / 8);
  const int64_t blocks = (pairs + ppb - 1) / ppb;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (V == 64)
    gated_rmsnorm_kernel<64><<<dim3(static_cast<unsigned>(blocks)), dim3(kNormThreads), 0, stream>>>(n, out, pairs, H);
  else
    gated_rmsnorm_kernel<128><<<dim3(static_cast<unsigned>(blocks)), dim3(kNormThreads), 0, stream>>>(n, out, pairs, H);
  return hipGetLastError();
}

}  // namespace kda
