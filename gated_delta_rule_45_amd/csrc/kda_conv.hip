// kda_conv.hip -- short causal conv prologue: mixed_qkv from the [q | k | v]
// pre-activations (vLLM PR #60683, Purpose, names a conv step before the
// KDA recurrence; the formula is a reading). Per sequence and channel c of
// D = 2*H*K + H*V:
//   a[t][c] = bias[c] + sum_{i<W} w[c][i] * x[t - (W-1) + i][c]
// with inputs before the sequence's first row taken from its conv state (the
// W-1 previous inputs, oldest first; zero on a null slot or without an
// initial state), y = silu(a), then q and k of each head divided by
// sqrt(sum of squares + l2_eps).
//
// Two launches on one stream:
//  1. conv_rows_kernel: one workgroup per (block of up to 32 consecutive
//     rows, 2048 channels). Lane tau of round r owns channels
//     8(256 r + tau) .. +7: its 8 x W taps and bias are loaded once, and a
//     window of the last W inputs (16-byte bf16 loads of x rows, or of the
//     conv state for positions before a sequence) slides down the rows,
//     refilled at every sequence start. A head's q (or k)
//     channels are K/8 consecutive lanes of one round (head and section
//     boundaries are multiples of K/8 chunks, and 256 is a multiple of K/8),
//     so the L2 norm is a butterfly over those lanes.
//  2. conv_state_kernel: one workgroup per sequence, after every row has read
//     the old states: the new conv state is the last W-1 inputs of the
//     sequence (older ones from the old state when it is shorter), copied
//     bit for bit.
// HBM-bound: every input row is read once from HBM (the W taps of
// neighbouring rows hit in L2) and every output row written once.
#include <algorithm>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kConvThreads = 256;

__device__ __forceinline__ int find_seq(const int32_t* cu, int32_t N, int64_t t) {
  int lo = 0, hi = N;  // the last i with cu[i] <= t
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

template <int K, int V, int W>
__global__ __launch_bounds__(kConvThreads) void conv_rows_kernel(const ConvParams p, int rows_per_block) {
  constexpr int G = K / 8;  // lanes per q or k head
  const int H = p.H;
  const int Dn = 2 * H * K + H * V;
  const int nch = Dn / 8;
  const int rounds = (nch + kConvThreads - 1) / kConvThreads;
  const int r = static_cast<int>(blockIdx.x % rounds);
  const int64_t t0 = static_cast<int64_t>(blockIdx.x / rounds) * rows_per_block;
  const int64_t t1 = min<int64_t>(t0 + rows_per_block, p.num_rows);
  if (t0 >= t1) return;
  const int tid = threadIdx.x;
  const int ch = r * kConvThreads + tid;
  const bool live = ch < nch;
  const int c0 = 8 * (live ? ch : 0);

  // Taps and bias of the lane's 8 channels, loaded once for all rows:
  // w[c0 + j][i] at (c0 + j) * W + i.
  float wt[8 * W], bias[8];
#pragma unroll
  for (int q = 0; q < 2 * W; ++q) {
    const f32x4 v = live ? *reinterpret_cast<const f32x4*>(p.weight + static_cast<int64_t>(c0) * W + 4 * q)
                         : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) wt[4 * q + j] = v[j];
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) bias[j] = 0.f;
  if (live && p.bias != nullptr) {
    const f32x4 b0 = *reinterpret_cast<const f32x4*>(p.bias + c0);
    const f32x4 b1 = *reinterpret_cast<const f32x4*>(p.bias + c0 + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bias[j] = b0[j];
      bias[4 + j] = b1[j];
    }
  }

  // Sequence of the first row; the window holds the inputs at positions
  // pos-(W-1) .. pos of the current row, refilled at every sequence start.
  int s = find_seq(p.cu_seqlens, p.num_seqs, t0);
  int64_t bos = uniform(static_cast<int64_t>(p.cu_seqlens[s]));
  int64_t eos = uniform(static_cast<int64_t>(p.cu_seqlens[s + 1]));
  float win[W][8];
  bool fresh = true;
  for (int64_t t = t0; t < t1; ++t) {
    while (t >= eos && s + 1 < p.num_seqs) {  // next non-empty sequence (uniform)
      ++s;
      bos = uniform(static_cast<int64_t>(p.cu_seqlens[s]));
      eos = uniform(static_cast<int64_t>(p.cu_seqlens[s + 1]));
      fresh = true;
    }
    if (t < bos || t >= eos || eos > p.num_rows) return;  // cu_seqlens outside the contract
    const int pos = static_cast<int>(t - bos);
    if (fresh) {
      const int64_t slot = uniform(static_cast<int64_t>(p.indices[static_cast<int64_t>(s) * p.index_stride]));
      const bool init = slot >= 0 && (p.has_initial_state == nullptr ||
                                      uniform(static_cast<int32_t>(p.has_initial_state[s])) != 0);
      const uint16_t* st = p.conv_state + (init ? slot : 0) * p.conv_slot_stride;
#pragma unroll
      for (int i = 0; i < W - 1; ++i) {
        const int src = pos - (W - 1) + i;
        if (live && src >= 0)
          load_bf16<8>(p.x + (bos + src) * p.x_row_stride + c0, win[i]);
        else if (live && init)
          load_bf16<8>(st + static_cast<int64_t>(W - 1 + src) * Dn + c0, win[i]);
        else {
#pragma unroll
          for (int j = 0; j < 8; ++j) win[i][j] = 0.f;
        }
      }
      fresh = false;
    } else {
#pragma unroll
      for (int i = 0; i < W - 1; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) win[i][j] = win[i + 1][j];
    }
    if (live) {
      load_bf16<8>(p.x + t * p.x_row_stride + c0, win[W - 1]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) win[W - 1][j] = 0.f;
    }
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float acc = bias[j];
#pragma unroll
      for (int i = 0; i < W; ++i) acc = fmaf(wt[j * W + i], win[i][j], acc);
      y[j] = live ? acc * sigmoid_f32(acc) : 0.f;
    }
    // L2 norm of q and k heads: a butterfly over the head's G lanes. Every
    // lane takes part (v lanes and lanes past the end included).
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = fmaf(y[j], y[j], ss);
#pragma unroll
    for (int off = 1; off < G; off <<= 1) ss += __shfl_xor(ss, off);
    if (live) {
      if (c0 < 2 * H * K) {
        const float inv = 1.0f / sqrtf(ss + p.l2_eps);
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] *= inv;
      }
      uint4 o;
      o.x = pack_bf16x2(y[0], y[1]);
      o.y = pack_bf16x2(y[2], y[3]);
      o.z = pack_bf16x2(y[4], y[5]);
      o.w = pack_bf16x2(y[6], y[7]);
      *reinterpret_cast<uint4*>(p.out + t * p.out_row_stride + c0) = o;
    }
  }
}

template <int W>
__global__ __launch_bounds__(kConvThreads) void conv_state_kernel(const ConvParams p, int Dn) {
  const int s = blockIdx.x;
  if (s >= p.num_seqs) return;
  const int64_t bos = p.uniform_len > 0 ? static_cast<int64_t>(s) * p.uniform_len
                                        : uniform(static_cast<int64_t>(p.cu_seqlens[s]));
  const int64_t eos = p.uniform_len > 0 ? bos + p.uniform_len : uniform(static_cast<int64_t>(p.cu_seqlens[s + 1]));
  const int64_t len = eos - bos;
  if (len <= 0 || bos < 0 || eos > p.num_rows) return;  // nothing to store
  const int64_t slot = uniform(static_cast<int64_t>(p.indices[static_cast<int64_t>(s) * p.index_stride]));
  if (slot < 0) return;
  const bool init = p.has_initial_state == nullptr || uniform(static_cast<int32_t>(p.has_initial_state[s])) != 0;
  uint16_t* st = p.conv_state + slot * p.conv_slot_stride;
  const int nch = Dn / 8;
  for (int ch = threadIdx.x; ch < nch; ch += kConvThreads) {
    const int c0 = 8 * ch;
    // Read every new row first (some come from the old state), then write.
    uint4 rows[W - 1];
#pragma unroll
    for (int j = 0; j < W - 1; ++j) {
      const int64_t q = len - (W - 1) + j;  // position of new row j
      if (q >= 0)
        rows[j] = *reinterpret_cast<const uint4*>(p.x + (bos + q) * p.x_row_stride + c0);
      else if (init)
        rows[j] = *reinterpret_cast<const uint4*>(st + (W - 1 + q) * Dn + c0);
      else
        rows[j] = uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < W - 1; ++j) *reinterpret_cast<uint4*>(st + static_cast<int64_t>(j) * Dn + c0) = rows[j];
  }
}

template <int K, int V>
hipError_t launch_kv(const ConvParams& p, hipStream_t stream) {
  const int Dn = 2 * p.H * K + p.H * V;
  const int rounds = (Dn / 8 + kConvThreads - 1) / kConvThreads;
  // Rows per workgroup: enough workgroups to fill the chip, up to 32 rows
  // sharing one load of the taps.
  const int rpb = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(32, p.num_rows / 256)));
  const int64_t blocks = (p.num_rows + rpb - 1) / rpb * rounds;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks)), seqs(static_cast<unsigned>(p.num_seqs));
  switch (p.width) {
    case 2:
      if (blocks > 0) conv_rows_kernel<K, V, 2><<<grid, kConvThreads, 0, stream>>>(p, rpb);
      conv_state_kernel<2><<<seqs, kConvThreads, 0, stream>>>(p, Dn);
      break;
    case 3:
      if (blocks > 0) conv_rows_kernel<K, V, 3><<<grid, kConvThreads, 0, stream>>>(p, rpb);
      conv_state_kernel<3><<<seqs, kConvThreads, 0, stream>>>(p, Dn);
      break;
    default:
      if (blocks > 0) conv_rows_kernel<K, V, 4><<<grid, kConvThreads, 0, stream>>>(p, rpb);
      conv_state_kernel<4><<<seqs, kConvThreads, 0, stream>>>(p, Dn);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_conv_state(const ConvParams& p, hipStream_t stream) {
  if (p.num_seqs <= 0) return hipSuccess;
  const int Dn = 2 * p.H * p.K + p.H * p.V;
  const dim3 seqs(static_cast<unsigned>(p.num_seqs));
  switch (p.width) {
    case 2: conv_state_kernel<2><<<seqs, kConvThreads, 0, stream>>>(p, Dn); break;
    case 3: conv_state_kernel<3><<<seqs, kConvThreads, 0, stream>>>(p, Dn); break;
    default: conv_state_kernel<4><<<seqs, kConvThreads, 0, stream>>>(p, Dn); break;
  }
  return hipGetLastError();
}

hipError_t launch_short_conv(const ConvParams& p, hipStream_t stream) {
  if (p.num_seqs <= 0) return hipSuccess;
  if (p.K == 64 && p.V == 64) return launch_kv<64, 64>(p, stream);
  if (p.K == 64 && p.V == 128) return launch_kv<64, 128>(p, stream);
  if (p.K == 128 && p.V == 64) return launch_kv<128, 64>(p, stream);
  return launch_kv<128, 128>(p, stream);
}

}  // namespace kda
