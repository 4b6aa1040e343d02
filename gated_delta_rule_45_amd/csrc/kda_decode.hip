// kda_decode.hip -- packed single-token decode and <=8-token spec-verify.
//
// Packed decode (vLLM PR #51682 report, Key source excerpts): one state slot
// per request, addressed through a possibly strided index view; spec-verify
// (vLLM PR #60683, Refusal and steps): whole requests of tokens_per_seq rows,
// padded requests on a null slot. Spec decode with a state per token (vLLM
// PR #51682 report, Purpose: the state slot is column 0 of a block table with
// 1 + num_speculative_blocks columns): the initial state comes from column
// num_accepted-1 and the state after token t is stored into column t.
//
// Work split. The V columns of a state evolve independently (u_j depends only
// on column j), so a workgroup owns a (request, head, VT-column) tile of the
// fp32 K x V state and needs no other workgroup. Its four waves split the K
// rows: wave w owns rows [w*K/4, (w+1)*K/4). Inside a wave, lane
// (rg, cg) = (lane / CG, lane % CG) holds the RPL consecutive rows
// w*K/4 + rg*RPL + r of columns 4cg..4cg+3 as float4s. With VT = 128 one
// wave-wide load covers RG whole 512-byte rows, and every wave streams a
// contiguous 16 KiB block of the state; a lane's rows are addressed from one
// base with immediate offsets. The tile is read once and written once; all tokens of a request are
// applied in registers in between. Bound by HBM bandwidth (about 0.9 flop per
// state byte), so no MFMA.
//
// The per-token inputs (q, k, the decay alpha = exp(g) from the fused gate,
// v, beta) for all tokens of the request are staged in LDS up front, while
// the state loads are in flight, so the token loop never waits on memory.
//
// Per token, with S' = diag(alpha) S:
//   u = beta (v - S'^T k),   o = scale (S'^T q + u (k.q)),   S = S' + k u^T
// which is the decay / delta-write / readout order in one pass over the tile.
// The K-reductions are a per-lane partial, a butterfly over the wave's row
// groups (DPP rotations and lane swaps, no LDS traffic), and a sum of the
// four waves' partials through LDS (one barrier per token; the partial
// buffer alternates between tokens).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kWaves = 4;
constexpr int kMaxTokens = 8;

// Sum of x over the lanes that share lane % CG (CG = 4, 8, 16 or 32): a
// butterfly on VALU lane permutations, no LDS traffic. Inside a 16-lane row
// the lanes l, l + CG, ... mod 16 are summed by DPP rotations of the row;
// the rows are then combined by swaps of rows 1, 3 with rows 0, 2
// (v_permlane16_swap) and of the two halves (v_permlane32_swap). Every
// lane must be active.
template <int CG>
__device__ __forceinline__ float sum_row_groups(float x) {
  static_assert(CG == 4 || CG == 8 || CG == 16 || CG == 32, "column groups");
  if constexpr (CG == 4)
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false));  // row_ror:4
  if constexpr (CG <= 8)
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));  // row_ror:8
  if constexpr (CG <= 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace

template <int K, int V, int VT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 8)))
void decode_kernel(const DecodeParams p) {
  constexpr int RW = K / kWaves;   // rows per wave
  constexpr int CG = VT / 4;       // column groups of 4 columns
  constexpr int RG = 64 / CG;      // row groups per wave
  constexpr int RPL = RW / RG;     // rows per lane
  static_assert(CG * RG == 64 && RPL * RG == RW && RPL >= 1, "tile does not fit");

  __shared__ float s_q[kMaxTokens][K];
  __shared__ float s_k[kMaxTokens][K];
  __shared__ float s_a[kMaxTokens][K];
  __shared__ float s_v[kMaxTokens][VT];
  __shared__ float s_b[kMaxTokens];
  __shared__ float s_red[2][kWaves][2 * VT + 4];
  // Gated RMSNorm epilogue operands (only a whole-row tile can apply it).
  constexpr bool kRow = VT == V;
  __shared__ float s_z[kRow ? kMaxTokens : 1][kRow ? VT : 1];
  __shared__ float s_w[kRow ? VT : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int H = p.H;
  const int tps = p.tokens_per_seq;
  constexpr int tiles = V / VT;
  const int64_t bid = blockIdx.x;
  const int tile = static_cast<int>(bid % tiles);
  const int64_t nh = bid / tiles;
  const int h = static_cast<int>(nh % H);
  const int n = static_cast<int>(nh / H);
  const int64_t row0 = static_cast<int64_t>(n) * tps;
  const int cg = lane % CG;
  const int rg = lane / CG;
  const int col = tile * VT + cg * 4;

  // State slot of this request: a strided 1-D view, widened to 64 bits. With
  // a state per token, the initial slot is the one in column num_accepted-1
  // (clamped to the request's columns) and every token's slot is read now.
  const int32_t* irow = p.indices + static_cast<int64_t>(n) * p.index_stride;
  const bool per_token = p.num_accepted != nullptr;
  int init_col = 0;
  if (per_token) init_col = min(max(uniform(p.num_accepted[n]), 1), tps) - 1;
  const int64_t slot = uniform(static_cast<int64_t>(irow[init_col * p.index_col_stride]));

  if (slot < 0) {
    // Null slot (the same for the whole workgroup): no state traffic, zero rows.
    for (int e = tid; e < tps * VT; e += blockDim.x) {
      const int t = e / VT, j = e % VT;
      p.out[((row0 + t) * H + h) * static_cast<int64_t>(V) + tile * VT + j] = 0;
    }
    return;
  }

  // 1. Issue the state loads first: one buffer resource over this head's
  //    K x V tile, a per-lane offset, and per-row scalar offsets.
  const __amdgpu_buffer_rsrc_t tile_rsrc =
      make_rsrc(p.pool + slot * p.slot_stride + static_cast<int64_t>(h) * K * V, K * V * 4);
  const int voff = ((w * RW + rg * RPL) * V + col) * 4;
  f32x4 S[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) S[r] = buffer_load_f32x4<kStreamPolicy>(tile_rsrc, voff, r * V * 4);

  // 2. Stage every token's q, k, alpha, v-tile and beta in LDS.
  {
    const float a = __expf(p.A_log[h]);
    const bool has_lb = p.has_lb != 0;
    if (tps >= 3) {
      // Long requests: every load is issued before the first use (buffer
      // loads over the request's rows; elements past its tokens read zero
      // and are not stored), one memory round trip instead of one per pass.
      constexpr int NE = (kMaxTokens * K + 255) / 256;   // q/k/raw_g elements per thread
      constexpr int NV = (kMaxTokens * VT + 255) / 256;  // v elements per thread
      const int rs = static_cast<int>(p.qkv_row_stride) * 2;  // bytes per mixed_qkv row
      const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.qkv + row0 * p.qkv_row_stride, static_cast<uint32_t>(tps * rs));
      const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.raw_g + row0 * (H * K), static_cast<uint32_t>(tps * H * K * 2));
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.raw_beta + row0 * H, static_cast<uint32_t>(tps * H * 2));
      uint16_t qb[NE], kb[NE], gb[NE], vb[NV];
      float db[NE];
#pragma unroll
      for (int u = 0; u < NE; ++u) {
        const int e = tid + 256 * u;
        const int t = e / K, i = e % K;
        qb[u] = __builtin_amdgcn_raw_buffer_load_b16(rq, t * rs + (h * K + i) * 2, 0, 0);
        kb[u] = __builtin_amdgcn_raw_buffer_load_b16(rq, t * rs + (H * K + h * K + i) * 2, 0, 0);
        gb[u] = __builtin_amdgcn_raw_buffer_load_b16(rg, (t * H * K + h * K + i) * 2, 0, 0);
        db[u] = p.dt_bias[h * K + i];
      }
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int e = tid + 256 * u;
        const int t = e / VT, j = e % VT;
        vb[u] = __builtin_amdgcn_raw_buffer_load_b16(rq, t * rs + (2 * H * K + h * V + tile * VT + j) * 2, 0, 0);
      }
      const uint16_t bb = __builtin_amdgcn_raw_buffer_load_b16(rb, (tid * H + h) * 2, 0, 0);
#pragma unroll
      for (int u = 0; u < NE; ++u) {
        const int e = tid + 256 * u;
        if (e < tps * K) {
          const int t = e / K, i = e % K;
          s_q[t][i] = bf16_to_f32(qb[u]);
          s_k[t][i] = bf16_to_f32(kb[u]);
          s_a[t][i] = __expf(gate_log_decay(bf16_to_f32(gb[u]), db[u], a, has_lb, p.lower_bound));
        }
      }
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int e = tid + 256 * u;
        if (e < tps * VT) s_v[e / VT][e % VT] = bf16_to_f32(vb[u]);
      }
      if (tid < tps) s_b[tid] = sigmoid_f32(bf16_to_f32(bb));
    } else {
      // One or two tokens: a single pass, with fewer instructions in the
      // way of the state loads.
      for (int e = tid; e < tps * K; e += blockDim.x) {
        const int t = e / K, i = e % K;
        const int64_t row = row0 + t;
        const uint16_t* qkv = p.qkv + row * p.qkv_row_stride;
        s_q[t][i] = bf16_to_f32(qkv[h * K + i]);
        s_k[t][i] = bf16_to_f32(qkv[H * K + h * K + i]);
        const float g = gate_log_decay(bf16_to_f32(p.raw_g[row * (H * K) + h * K + i]),
                                       p.dt_bias[h * K + i], a, has_lb, p.lower_bound);
        s_a[t][i] = __expf(g);
      }
      for (int e = tid; e < tps * VT; e += blockDim.x) {
        const int t = e / VT, j = e % VT;
        s_v[t][j] = bf16_to_f32(p.qkv[(row0 + t) * p.qkv_row_stride + 2 * H * K + h * V + tile * VT + j]);
      }
      if (tid < tps) s_b[tid] = sigmoid_f32(bf16_to_f32(p.raw_beta[(row0 + tid) * H + h]));
    }
    if constexpr (kRow) {
      if (p.norm.gate != nullptr) {
        for (int e = tid; e < tps * VT; e += blockDim.x) {
          const int t = e / VT, j = e % VT;
          s_z[t][j] = bf16_to_f32(p.norm.gate[(row0 + t) * p.norm.gate_row_stride + h * V + j]);
        }
        if (tid < VT) s_w[tid] = p.norm.weight[tid];
      }
    }
  }
  __syncthreads();

  // 3. Token loop, all in registers.
  for (int t = 0; t < tps; ++t) {
    f32x4 kS = {0.f, 0.f, 0.f, 0.f};
    f32x4 qS = {0.f, 0.f, 0.f, 0.f};
    float kq = 0.f;
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      const int row = w * RW + rg * RPL + r;
      const float alpha = s_a[t][row];
      const float kk = s_k[t][row];
      const float qq = s_q[t][row];
      S[r] *= alpha;
      kS += kk * S[r];
      qS += qq * S[r];
      kq = fmaf(kk, qq, kq);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      kS[c] = sum_row_groups<CG>(kS[c]);
      qS[c] = sum_row_groups<CG>(qS[c]);
    }
    kq = sum_row_groups<CG>(kq);
    float(*red)[2 * VT + 4] = s_red[t & 1];
    if (rg == 0) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        red[w][cg * 4 + c] = kS[c];
        red[w][VT + cg * 4 + c] = qS[c];
      }
      if (cg == 0) red[w][2 * VT] = kq;
    }
    __syncthreads();
    kS = f32x4{0.f, 0.f, 0.f, 0.f};
    qS = f32x4{0.f, 0.f, 0.f, 0.f};
    kq = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        kS[c] += red[ww][cg * 4 + c];
        qS[c] += red[ww][VT + cg * 4 + c];
      }
      kq += red[ww][2 * VT];
    }
    const float beta = s_b[t];
    f32x4 u;
#pragma unroll
    for (int c = 0; c < 4; ++c) u[c] = beta * (s_v[t][cg * 4 + c] - kS[c]);
#pragma unroll
    for (int r = 0; r < RPL; ++r) S[r] += s_k[t][w * RW + rg * RPL + r] * u;
    if (per_token) {
      // The state after token t goes to column t's slot (none when null).
      const int64_t st = uniform(static_cast<int64_t>(irow[t * p.index_col_stride]));
      if (st >= 0) {
        const __amdgpu_buffer_rsrc_t tr =
            make_rsrc(p.pool + st * p.slot_stride + static_cast<int64_t>(h) * K * V, K * V * 4);
#pragma unroll
        for (int r = 0; r < RPL; ++r) buffer_store_f32x4<kStreamPolicy>(S[r], tr, voff, r * V * 4);
      }
    }
    if (w == 0) {
      const float s = p.scale;
      f32x4 ov;
#pragma unroll
      for (int c = 0; c < 4; ++c) ov[c] = s * fmaf(u[c], kq, qS[c]);
      if constexpr (kRow) {
        // Gated RMSNorm over the head's V outputs: every row group of wave 0
        // holds the whole row (4 columns per lane), so a butterfly over the
        // CG lanes of a group gives the sum of squares.
        if (p.norm.gate != nullptr) {
          float ss = ov[0] * ov[0] + ov[1] * ov[1] + ov[2] * ov[2] + ov[3] * ov[3];
#pragma unroll
          for (int off = 1; off < CG; off <<= 1) ss += __shfl_xor(ss, off);
          const float inv = 1.0f / sqrtf(ss * (1.0f / V) + p.norm.eps);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float zv = s_z[t][cg * 4 + c];
            const float sg = sigmoid_f32(zv);
            ov[c] *= inv * s_w[cg * 4 + c] * (p.norm.activation == 1 ? zv * sg : sg);
          }
        }
      }
      if (rg == 0) {
        uint16_t* o = p.out + ((row0 + t) * H + h) * static_cast<int64_t>(V) + col;
        *reinterpret_cast<uint2*>(o) = make_uint2(pack_bf16x2(ov[0], ov[1]), pack_bf16x2(ov[2], ov[3]));
      }
    }
  }

  // 4. Store the final state (with a state per token it is already stored).
  if (!per_token) {
#pragma unroll
    for (int r = 0; r < RPL; ++r) buffer_store_f32x4<kStreamPolicy>(S[r], tile_rsrc, voff, r * V * 4);
  }
}

template <int K, int V>
static hipError_t launch_kv(const DecodeParams& p, int vt, hipStream_t stream) {
  const int64_t blocks = static_cast<int64_t>(p.num_seqs) * p.H * (V / vt);
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(blocks)), block(64 * kWaves);
  switch (vt) {
    case 16: decode_kernel<K, V, 16><<<grid, block, 0, stream>>>(p); break;
    case 32: decode_kernel<K, V, 32><<<grid, block, 0, stream>>>(p); break;
    case 64: decode_kernel<K, V, 64><<<grid, block, 0, stream>>>(p); break;
    default:
      if constexpr (V == 128) decode_kernel<K, V, 128><<<grid, block, 0, stream>>>(p);
      break;
  }
  return hipGetLastError();
}

// Column-tile choice: whole rows (VT = V) when there are enough (request,
// head) pairs to fill the chip; narrower tiles for small batches, so that a
// spec-verify step of a single request still spreads over the 256 CUs.
hipError_t launch_decode(DecodeParams p, int K, hipStream_t stream) {
  const int64_t pairs = static_cast<int64_t>(p.num_seqs) * p.H;
  int vt = 128;
  if (pairs < 512) vt = 64;
  if (pairs < 256) vt = 32;
  if (pairs < 128) vt = 16;
  if (vt > p.V) vt = p.V;
  p.num_tiles = pairs * (p.V / vt);
  // The output epilogue runs inside the kernel when a workgroup holds whole
  // rows; otherwise as a pass over the output after it.
  const OutNorm norm = p.norm;
  const bool separate = norm.gate != nullptr && vt != p.V;
  if (separate) p.norm.gate = nullptr;
  hipError_t e;
  if (K == 64)
    e = p.V == 64 ? launch_kv<64, 64>(p, vt, stream) : launch_kv<64, 128>(p, vt, stream);
  else
    e = p.V == 64 ? launch_kv<128, 64>(p, vt, stream) : launch_kv<128, 128>(p, vt, stream);
  if (e != hipSuccess || !separate) return e;
  return launch_gated_rmsnorm(norm, p.out, static_cast<int64_t>(p.num_seqs) * p.tokens_per_seq, p.H,
                              p.V, stream);
}

}  // namespace kda
