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
// Requests of at least this many tokens on tiles of at most 32 columns take
// the block (WY) form of the token chain.
constexpr int kBlockMinTokens = 2;

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

namespace {

// x rotated right by N lanes inside each 16-lane row (DPP row_ror).
template <int N>
__device__ __forceinline__ float row_ror(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xf, 0xf, false));
}

// One step of a recursive halving over the row-group bits of the lane
// index: lanes with bit B clear keep the lower HALF of their value list and
// lanes with it set the upper half, each adding the partner's copy of the
// half it keeps. Bits 2 and 3 pair lanes by DPP rotations inside a 16-lane
// row (a rotation by 4 or 8 flips that bit; the step for the next bit
// completes the coverage); bits 4 and 5 by v_permlane16_swap /
// v_permlane32_swap, which leave the kept half's two copies in the two
// operands. Every lane must be active.
template <int B, int HALF, int N>
__device__ __forceinline__ void halve_step(float (&x)[N], int lane) {
  if constexpr (B < 4) {
    const bool hi = (lane >> B) & 1;
#pragma unroll
    for (int v = 0; v < HALF; ++v) {
      const float keep = hi ? x[HALF + v] : x[v];
      const float send = hi ? x[v] : x[HALF + v];
      x[v] = keep + row_ror<(B == 2 ? 4 : 8)>(send);
    }
  } else {
#pragma unroll
    for (int v = 0; v < HALF; ++v) {
      const uint32_t lo = __float_as_uint(x[v]), up = __float_as_uint(x[HALF + v]);
      const auto r = B == 4 ? __builtin_amdgcn_permlane16_swap(lo, up, false, false)
                            : __builtin_amdgcn_permlane32_swap(lo, up, false, false);
      x[v] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
  }
}

// Sums of the N values over the wave's row groups (lanes that share
// lane % CG), N / (64 / CG) of them left per lane: block B of the list, the
// lowest row-group bit being B's most significant bit.
template <int CG, int N>
__device__ __forceinline__ void halve_row_groups(float (&x)[N], int lane) {
  constexpr int first = CG == 4 ? 2 : CG == 8 ? 3 : CG == 16 ? 4 : 5;
  static_assert((64 / CG) <= N, "fewer values than row groups");
  if constexpr (first <= 2) halve_step<2, (N >> (3 - first))>(x, lane);
  if constexpr (first <= 3) halve_step<3, (N >> (4 - first))>(x, lane);
  if constexpr (first <= 4) halve_step<4, (N >> (5 - first))>(x, lane);
  halve_step<5, (N >> (6 - first))>(x, lane);
}

}  // namespace

// Spec-verify blocks of 2..8 tokens on narrow column tiles (the latency
// case: few requests, one workgroup per CU). The per-token chain of the
// decode kernel (a K-reduction, a cross-wave exchange and a barrier per
// token) is replaced by the WY form of the block. With G_t the running sum
// of the log decays through token t (per key channel):
//   S'_t^T k_t = X_t + sum_{s<t} A_ts u_s,   X_t = S0^T (e^{G_t} * k_t),
//   S_t^T q_t  = Y_t + sum_{s<=t} P_ts u_s,  Y_t = S0^T (e^{G_t} * q_t),
//   A_ts = sum_i k_s[i] k_t[i] e^{G_t[i] - G_s[i]},  P_ts likewise with q_t,
// so u_t = beta_t (v_t - X_t - sum_{s<t} A_ts u_s) and
// o_t = scale (Y_t + sum_{s<=t} P_ts u_s). Every reduction against the state
// is taken at once from S0, then summed over the waves through LDS. On
// 16-column tiles [X | Y] is a 16-column by 16-entry product over the K
// rows, run on fp32 MFMA with the state held in the operand layout; on
// 32-column tiles it is one recursive halving over the wave's row groups,
// with the state held as float4 rows. The scalars A and P are formed while
// the state loads are in flight; the u recurrence is per-column scalar work; and the
// state then takes its tokens in registers, S = diag(e^{g_t}) S + k_t u_t^T
// (stored after every token with a state per token). The exponents
// G_t - G_s are never positive. NT is the token capacity (4 or 8).
template <int K, int V, int VT, int NT>
__global__ __launch_bounds__(256) void spec_block_kernel(const DecodeParams p) {
  constexpr int RW = K / kWaves;
  // MFMA layout (VT = 16): lane (g, m) = (lane / 16, lane % 16) of wave w
  // holds rows w RW + g NSTEP + s, s < NSTEP, of column m. Step s of the
  // [X | Y] product takes from it the A element S0[row][m] and the B element
  // ckq[row][m] of contraction index g (v_mfma_f32_16x16x4_f32).
  constexpr bool kMfma = VT == 16;
  constexpr int NSTEP = RW / 4;
  // Row-group layout (VT = 32): lane (rg, cg) = (lane / CG, lane % CG)
  // holds rows w RW + rg RPL + r, r < RPL, of columns 4cg .. 4cg + 3.
  constexpr int CG = VT / 4;
  constexpr int RG = 64 / CG;
  constexpr int RPL = RW / RG;
  constexpr int NVAL = 8 * NT;       // X and Y for NT tokens and 4 columns
  constexpr int NKEEP = NVAL / RG;   // of them held by a lane after the halving
  static_assert(kMfma ? NSTEP % 4 == 0 : (CG * RG == 64 && RPL * RG == RW && RPL >= 1 && NKEEP >= 1),
                "tile does not fit");
  constexpr int NS = kMfma ? NSTEP : 4 * RPL;  // state floats per lane
  // Factored A/P (below) on the MFMA layout with 8 token places; with 4 the
  // per-channel form has only 16 entries and costs less.
  constexpr bool kApMfma = kMfma && NT == 8;
  // A/P work split: LO lanes per entry (t, s), s < t, and LD per diagonal.
  constexpr int NO = NT * (NT - 1) / 2;
  constexpr int LO = NT == 8 ? 8 : 16;
  constexpr int LD = NT == 8 ? 4 : 16;
  static_assert(NO * LO + NT * LD <= 256 && (NO * LO) % LD == 0 && K % (4 * LO) == 0 && K % (4 * LD) == 0,
                "A/P lanes");
  // Wave-summed [X | Y] per column: entry t is X_t and 8 + t is Y_t. Row
  // strides are padded against LDS bank conflicts.
  constexpr int SS = 20;
  constexpr int QS = 17;  // MFMA B rows: e^{G_t} k_t at t, e^{G_t} q_t at 8 + t
  constexpr int kUParts = 4;  // threads per column in the u/o phase
  static_assert(VT * kUParts <= 256 && NT % kUParts == 0, "u/o threads");

  __shared__ __align__(16) float s_q[NT][K];
  __shared__ __align__(16) float s_k[NT][K];
  __shared__ __align__(16) float s_a[NT][K];   // e^{g_t}
  __shared__ __align__(16) float s_G[NT][K];   // G_t
  __shared__ __align__(16) float s_ck[kMfma ? 1 : NT][kMfma ? 1 : K];  // e^{G_t} k_t
  __shared__ __align__(16) float s_cq[kMfma ? 1 : NT][kMfma ? 1 : K];  // e^{G_t} q_t
  __shared__ float s_ckq[kMfma ? K : 1][kMfma ? QS : 1];
  __shared__ float s_kinv[kApMfma ? K : 1][kApMfma ? QS : 1];  // e^{-G_s} k_s at s (factored A/P)
  __shared__ __align__(16) float s_v[NT][VT];
  __shared__ __align__(16) float s_u[NT][VT];
  __shared__ __align__(16) float s_b[NT];
  __shared__ __align__(16) float s_A[NT][NT];
  __shared__ __align__(16) float s_P[NT][NT];
  __shared__ __align__(16) float s_xy[kWaves][kMfma ? 1 : CG][kMfma ? 1 : NVAL];
  __shared__ float s_xym[kWaves][kMfma ? VT : 1][kMfma ? QS : 1];
  __shared__ float s_apm[kWaves][kApMfma ? 16 : 1][kApMfma ? QS : 1];
  __shared__ __align__(16) float s_sum[VT][SS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int H = p.H;
  const int T = p.tokens_per_seq;
  constexpr int tiles = V / VT;
  const int64_t bid = blockIdx.x;
  const int tile = static_cast<int>(bid % tiles);
  const int64_t nh = bid / tiles;
  const int h = static_cast<int>(nh % H);
  const int n = static_cast<int>(nh / H);
  const int64_t row0 = static_cast<int64_t>(n) * T;
  const int cg = lane % CG;
  const int rg = lane / CG;
  const int col = tile * VT + cg * 4;
  const int g4 = lane >> 4, m16 = lane & 15;
  const int srow = w * RW + g4 * NSTEP;  // MFMA layout: the lane's first row
  // Factored A/P on the MFMA layout: with a lower bound lb every running sum
  // satisfies -NT |lb| <= G <= 0, so e^{G_t} and e^{-G_s} stay within
  // [e^-60, e^60] when NT |lb| <= 60 (products with key components stay
  // far above the fp32 denormal range), and e^{G_t - G_s} = e^{G_t} e^{-G_s}
  // makes [A | P] the product [e^G k | e^G q]^T (e^{-G} k) over the keys.
  const bool ap_mfma = kApMfma && p.has_lb != 0 && -p.lower_bound * NT <= 60.f;

  // 1. Per-token input loads, then the slot and the state loads: the inputs
  //    arrive first (loads complete in order), the slot lookup overlaps
  //    them, and the A/P work below overlaps the state's memory latency. Thread i < K owns key channel i for every
  //    token (the running sum G runs down its tokens); the others stage v
  //    and beta. Loads past the request's rows read zero, so padded tokens
  //    carry q = k = 0 and g = 0.
  constexpr int NVE = (NT * VT + 255 - K) / (256 - K);  // v elements per staging thread
  const int rs = static_cast<int>(p.qkv_row_stride) * 2;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.qkv + row0 * p.qkv_row_stride, static_cast<uint32_t>(T * rs));
  uint16_t qb[NT], kb[NT], gb[NT], vb[NVE], bb = 0;
  float db = 0.f;
  if (tid < K) {
    const int i = tid;
    const __amdgpu_buffer_rsrc_t rgt = make_rsrc(p.raw_g + row0 * (H * K), static_cast<uint32_t>(T * H * K * 2));
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      qb[t] = __builtin_amdgcn_raw_buffer_load_b16(rq, t * rs + (h * K + i) * 2, 0, 0);
      kb[t] = __builtin_amdgcn_raw_buffer_load_b16(rq, t * rs + (H * K + h * K + i) * 2, 0, 0);
      gb[t] = __builtin_amdgcn_raw_buffer_load_b16(rgt, (t * H * K + h * K + i) * 2, 0, 0);
    }
    db = p.dt_bias[h * K + i];
  } else {
    const int j0 = tid - K;
#pragma unroll
    for (int u = 0; u < NVE; ++u) {
      const int e = j0 + u * (256 - K);
      const int t = e / VT, j = e % VT;
      vb[u] = __builtin_amdgcn_raw_buffer_load_b16(rq, (e < NT * VT ? t * rs : T * rs) + (2 * H * K + h * V + tile * VT + j) * 2, 0, 0);
    }
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.raw_beta + row0 * H, static_cast<uint32_t>(T * H * 2));
    bb = __builtin_amdgcn_raw_buffer_load_b16(rb, (min(j0, NT) * H + h) * 2, 0, 0);
  }

  const int32_t* irow = p.indices + static_cast<int64_t>(n) * p.index_stride;
  const bool per_token = p.num_accepted != nullptr;
  int init_col = 0;
  if (per_token) init_col = min(max(uniform(p.num_accepted[n]), 1), T) - 1;
  const int64_t slot = uniform(static_cast<int64_t>(irow[init_col * p.index_col_stride]));
  if (slot < 0) {
    // Null slot: zero rows; the input loads are drained before the exit.
    __builtin_amdgcn_s_waitcnt(0);
    for (int e = tid; e < T * VT; e += blockDim.x) {
      const int t = e / VT, j = e % VT;
      p.out[((row0 + t) * H + h) * static_cast<int64_t>(V) + tile * VT + j] = 0;
    }
    return;
  }

  const __amdgpu_buffer_rsrc_t tile_rsrc =
      make_rsrc(p.pool + slot * p.slot_stride + static_cast<int64_t>(h) * K * V, K * V * 4);
  const int voff = kMfma ? (srow * V + tile * VT + m16) * 4 : ((w * RW + rg * RPL) * V + col) * 4;
  float S[NS];
  if constexpr (kMfma) {
#pragma unroll
    for (int st = 0; st < NSTEP; ++st)
      S[st] = __builtin_bit_cast(float,
                                 __builtin_amdgcn_raw_buffer_load_b32(tile_rsrc, voff, st * V * 4, kStreamPolicy));
  } else {
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      const f32x4 x = buffer_load_f32x4<kStreamPolicy>(tile_rsrc, voff, r * V * 4);
#pragma unroll
      for (int c = 0; c < 4; ++c) S[4 * r + c] = x[c];
    }
  }

  // 2. Inputs to LDS: q, k, e^{g}, G and the weighted rows e^{G} k, e^{G} q.
  {
    if (tid < K) {
      const int i = tid;
      const float a = __expf(p.A_log[h]);
      const bool has_lb = p.has_lb != 0;
      float G = 0.f;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float q = bf16_to_f32(qb[t]);
        const float k = bf16_to_f32(kb[t]);
        const float g = t < T ? gate_log_decay(bf16_to_f32(gb[t]), db, a, has_lb, p.lower_bound) : 0.f;
        G += g;
        const float eG = __expf(G);
        s_q[t][i] = q;
        s_k[t][i] = k;
        s_a[t][i] = __expf(g);
        s_G[t][i] = G;
        if constexpr (kMfma) {
          s_ckq[i][t] = eG * k;
          s_ckq[i][8 + t] = eG * q;
          if constexpr (kApMfma) {
            if (ap_mfma) s_kinv[i][t] = k * __expf(-G);
          }
        } else {
          s_ck[t][i] = eG * k;
          s_cq[t][i] = eG * q;
        }
      }
      if constexpr (kMfma) {
#pragma unroll
        for (int t = NT; t < 8; ++t) {
          s_ckq[i][t] = 0.f;
          s_ckq[i][8 + t] = 0.f;
        }
        if constexpr (kApMfma) {
          if (ap_mfma) {
#pragma unroll
            for (int t = NT; t < 16; ++t) s_kinv[i][t] = 0.f;
          }
        }
      }
    } else {
      const int j0 = tid - K;
#pragma unroll
      for (int u = 0; u < NVE; ++u) {
        const int e = j0 + u * (256 - K);
        if (e < NT * VT) s_v[e / VT][e % VT] = bf16_to_f32(vb[u]);
      }
      if (j0 < NT) s_b[j0] = j0 < T ? sigmoid_f32(bf16_to_f32(bb)) : 0.f;
    }
  }
  lds_barrier();

  // 3. A and P. For s < t, A_ts and P_ts share the factor e^{G_t - G_s}
  //    (one exponential per channel for both): LO lanes per such entry, the
  //    entries row by row; then LD lanes per diagonal entry P_tt = k_t . q_t.
  //    The lanes of an entry read neighbouring float4s, and each entry
  //    starts at its own offset, so the entries of a wave spread over the
  //    LDS banks. (The factored form takes A and P from MFMA in step 4.)
  if (!ap_mfma) {
    int te = -1, se = 0, part = 0, ent = 0;
    bool diag = false;
    if (tid < NO * LO) {
      ent = tid / LO;
      part = tid % LO;
      int rem = ent;
#pragma unroll
      for (int x = 1; x < NT; ++x)
        if (te < 0) {
          if (rem < x) { te = x; se = rem; } else { rem -= x; }
        }
    } else if (tid < NO * LO + NT * LD) {
      te = se = (tid - NO * LO) / LD;
      part = (tid - NO * LO) % LD;
      diag = true;
    }
    float accA = 0.f, accP = 0.f;
    if (te >= 0 && te < T) {
      if (!diag) {
        constexpr int NF = K / (4 * LO);  // float4s per lane
#pragma unroll
        for (int m = 0; m < NF; ++m) {
          const int i = (((m + ent) % NF) * LO + part) * 4;
          const float4 ks = *reinterpret_cast<const float4*>(&s_k[se][i]);
          const float4 kt = *reinterpret_cast<const float4*>(&s_k[te][i]);
          const float4 qt = *reinterpret_cast<const float4*>(&s_q[te][i]);
          const float4 gt = *reinterpret_cast<const float4*>(&s_G[te][i]);
          const float4 gs = *reinterpret_cast<const float4*>(&s_G[se][i]);
          const float e0 = ks.x * __expf(gt.x - gs.x), e1 = ks.y * __expf(gt.y - gs.y);
          const float e2 = ks.z * __expf(gt.z - gs.z), e3 = ks.w * __expf(gt.w - gs.w);
          accA = fmaf(e0, kt.x, fmaf(e1, kt.y, fmaf(e2, kt.z, fmaf(e3, kt.w, accA))));
          accP = fmaf(e0, qt.x, fmaf(e1, qt.y, fmaf(e2, qt.z, fmaf(e3, qt.w, accP))));
        }
      } else {
        constexpr int NF = K / (4 * LD);
#pragma unroll
        for (int m = 0; m < NF; ++m) {
          const int i = (m * LD + part) * 4;
          const float4 kt = *reinterpret_cast<const float4*>(&s_k[te][i]);
          const float4 qt = *reinterpret_cast<const float4*>(&s_q[te][i]);
          accP = fmaf(kt.x, qt.x, fmaf(kt.y, qt.y, fmaf(kt.z, qt.z, fmaf(kt.w, qt.w, accP))));
        }
      }
    }
    // Sums over an entry's lanes (aligned groups of 4, 8 or 16): the quad,
    // then the other quad of the half row, then the other half of the row.
    auto dpp = [](float x, int ctrl_id) {
      switch (ctrl_id) {
        case 0: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, false));  // quad [1,0,3,2]
        case 1: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xf, 0xf, false));  // quad [2,3,0,1]
        case 2: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xf, 0xf, false));  // row_half_mirror
        default: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xf, 0xf, false));  // row_mirror
      }
    };
    float sA[3], sP[3];  // sums over 4, 8 and 16 lanes
    accA += dpp(accA, 0);
    accP += dpp(accP, 0);
    sA[0] = accA + dpp(accA, 1);
    sP[0] = accP + dpp(accP, 1);
    sA[1] = sA[0] + dpp(sA[0], 2);
    sP[1] = sP[0] + dpp(sP[0], 2);
    sA[2] = sA[1] + dpp(sA[1], 3);
    sP[2] = sP[1] + dpp(sP[1], 3);
    constexpr int lo = LO == 4 ? 0 : LO == 8 ? 1 : 2;
    constexpr int ld = LD == 4 ? 0 : LD == 8 ? 1 : 2;
    if (part == 0 && te >= 0) {
      if (diag) {
        s_P[te][te] = sP[ld];
      } else {
        s_A[te][se] = sA[lo];
        s_P[te][se] = sP[lo];
      }
    }
  }

  // 4. X_t and Y_t from S0, per wave, then to LDS for the sum over the
  //    waves. MFMA layout: NSTEP fp32 MFMA steps over the wave's rows (lane
  //    (g, m) ends with entry m of columns 4g .. 4g + 3). Row-group layout:
  //    per-lane partials over the lane's rows, halved over the row groups.
  if constexpr (kMfma) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < NSTEP; ++st)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(S[st], s_ckq[srow + st][m16], acc, 0, 0, 0);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) s_xym[w][4 * g4 + jj][m16] = acc[jj];
    if constexpr (kApMfma) {
      if (ap_mfma) {
        // [A | P] partials over the wave's keys: lane (g, m) ends with
        // column s = m of rows 4g .. 4g + 3 (rows t: A_ts, 8 + t: P_ts).
        f32x4 ap = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < NSTEP; ++st)
          ap = __builtin_amdgcn_mfma_f32_16x16x4f32(s_ckq[srow + st][m16], s_kinv[srow + st][m16], ap, 0, 0, 0);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) s_apm[w][4 * g4 + jj][m16] = ap[jj];
      }
    }
  } else {
    float xy[NVAL];
#pragma unroll
    for (int v = 0; v < NVAL; ++v) xy[v] = 0.f;
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      const int row = w * RW + rg * RPL + r;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float ck = s_ck[t][row], cq = s_cq[t][row];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          xy[t * 4 + c] = fmaf(ck, S[4 * r + c], xy[t * 4 + c]);
          xy[(NT + t) * 4 + c] = fmaf(cq, S[4 * r + c], xy[(NT + t) * 4 + c]);
        }
      }
    }
    halve_row_groups<CG>(xy, lane);
    int blk = 0;
#pragma unroll
    for (int b = 2; b < 6; ++b)
      if ((1 << b) >= CG) blk = blk * 2 + ((lane >> b) & 1);
#pragma unroll
    for (int v = 0; v < NKEEP; ++v) s_xy[w][cg][blk * NKEEP + v] = xy[v];
  }
  lds_barrier();

  // 5. Sums over the waves (every thread), then u and o, one thread per
  //    column of the tile.
  for (int e = tid; e < VT * 2 * NT; e += 256) {
    const int jj = e / (2 * NT), v = e % (2 * NT);
    const int kind = v / NT, t = v % NT;
    float x = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      if constexpr (kMfma)
        x += s_xym[ww][jj][kind * 8 + t];
      else
        x += s_xy[ww][jj / 4][v * 4 + jj % 4];
    }
    s_sum[jj][kind * 8 + t] = x;
  }
  if constexpr (kApMfma) {
    if (ap_mfma && tid < NT * NT) {
      const int t = tid / NT, s2 = tid % NT;
      float a = 0.f, pp = 0.f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        a += s_apm[ww][t][s2];
        pp += s_apm[ww][8 + t][s2];
      }
      s_A[t][s2] = a;
      s_P[t][s2] = pp;
    }
  }
  lds_barrier();
  if (tid < VT * kUParts) {
    // kUParts threads per column: each runs the column's u recurrence (a
    // short dependent chain) and forms o and stores u for the token places
    // t = part (mod kUParts). Every operand is read before the first result
    // is written.
    const int j = tid / kUParts, part = tid % kUParts;
    constexpr int NOWN = NT / kUParts;
    float X[NT], A[NT][NT], b[NT], Yo[NOWN], Po[NOWN][NT];
#pragma unroll
    for (int t4 = 0; t4 < NT; t4 += 4) {
      const float4 xv = *reinterpret_cast<const float4*>(&s_sum[j][t4]);
      const float4 bv = *reinterpret_cast<const float4*>(&s_b[t4]);
      X[t4] = xv.x; X[t4 + 1] = xv.y; X[t4 + 2] = xv.z; X[t4 + 3] = xv.w;
      b[t4] = bv.x; b[t4 + 1] = bv.y; b[t4 + 2] = bv.z; b[t4 + 3] = bv.w;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float4 av = *reinterpret_cast<const float4*>(&s_A[t][t4]);
        A[t][t4] = av.x; A[t][t4 + 1] = av.y; A[t][t4 + 2] = av.z; A[t][t4 + 3] = av.w;
      }
#pragma unroll
      for (int i = 0; i < NOWN; ++i) {
        const float4 pv = *reinterpret_cast<const float4*>(&s_P[part + kUParts * i][t4]);
        Po[i][t4] = pv.x; Po[i][t4 + 1] = pv.y; Po[i][t4 + 2] = pv.z; Po[i][t4 + 3] = pv.w;
      }
    }
#pragma unroll
    for (int i = 0; i < NOWN; ++i) Yo[i] = s_sum[j][8 + part + kUParts * i];
    float u[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float x = s_v[t][j] - X[t];
#pragma unroll
      for (int s2 = 0; s2 < t; ++s2) x = fmaf(-A[t][s2], u[s2], x);
      u[t] = b[t] * x;
    }
#pragma unroll
    for (int i = 0; i < NOWN; ++i) {
      const int t = part + kUParts * i;
      if (t < T) {
        float y = Yo[i];
#pragma unroll
        for (int s2 = 0; s2 < NT; ++s2) y = fmaf(s2 <= t ? Po[i][s2] : 0.f, u[s2], y);
        p.out[((row0 + t) * H + h) * static_cast<int64_t>(V) + tile * VT + j] = f32_to_bf16_rne(p.scale * y);
        float ut = u[0];
#pragma unroll
        for (int s2 = 1; s2 < NT; ++s2) ut = s2 == t ? u[s2] : ut;
        s_u[t][j] = ut;
      }
    }
  }
  lds_barrier();

  // 6. The state takes the block's tokens in registers.
  auto store_state = [&](const __amdgpu_buffer_rsrc_t r) {
    if constexpr (kMfma) {
#pragma unroll
      for (int st = 0; st < NSTEP; ++st)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, S[st]), r, voff, st * V * 4,
                                              kStreamPolicy);
    } else {
#pragma unroll
      for (int r2 = 0; r2 < RPL; ++r2)
        buffer_store_f32x4<kStreamPolicy>(f32x4{S[4 * r2], S[4 * r2 + 1], S[4 * r2 + 2], S[4 * r2 + 3]}, r, voff,
                                          r2 * V * 4);
    }
  };
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (t < T) {
      if constexpr (kMfma) {
        const float ut = s_u[t][m16];
#pragma unroll
        for (int q4 = 0; q4 < NSTEP; q4 += 4) {
          const float4 av = *reinterpret_cast<const float4*>(&s_a[t][srow + q4]);
          const float4 kv = *reinterpret_cast<const float4*>(&s_k[t][srow + q4]);
          S[q4] = fmaf(kv.x, ut, S[q4] * av.x);
          S[q4 + 1] = fmaf(kv.y, ut, S[q4 + 1] * av.y);
          S[q4 + 2] = fmaf(kv.z, ut, S[q4 + 2] * av.z);
          S[q4 + 3] = fmaf(kv.w, ut, S[q4 + 3] * av.w);
        }
      } else {
        const f32x4 ut = *reinterpret_cast<const f32x4*>(&s_u[t][cg * 4]);
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
          const int row = w * RW + rg * RPL + r;
          const float al = s_a[t][row], kr = s_k[t][row];
#pragma unroll
          for (int c = 0; c < 4; ++c) S[4 * r + c] = fmaf(kr, ut[c], S[4 * r + c] * al);
        }
      }
      if (per_token) {
        const int64_t st = uniform(static_cast<int64_t>(irow[t * p.index_col_stride]));
        if (st >= 0) store_state(make_rsrc(p.pool + st * p.slot_stride + static_cast<int64_t>(h) * K * V, K * V * 4));
      }
    }
  }
  if (!per_token) store_state(tile_rsrc);
}

template <int K, int V>
static hipError_t launch_kv(const DecodeParams& p, int vt, hipStream_t stream) {
  const int64_t blocks = static_cast<int64_t>(p.num_seqs) * p.H * (V / vt);
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(blocks)), block(64 * kWaves);
  if (p.tokens_per_seq >= kBlockMinTokens && vt <= 32) {
    const bool nt4 = p.tokens_per_seq <= 4;
    if (vt == 16) {
      if (nt4) spec_block_kernel<K, V, 16, 4><<<grid, block, 0, stream>>>(p);
      else spec_block_kernel<K, V, 16, 8><<<grid, block, 0, stream>>>(p);
    } else {
      if (nt4) spec_block_kernel<K, V, 32, 4><<<grid, block, 0, stream>>>(p);
      else spec_block_kernel<K, V, 32, 8><<<grid, block, 0, stream>>>(p);
    }
    return hipGetLastError();
  }
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
  const bool block_form = p.tokens_per_seq >= kBlockMinTokens && vt <= 32;
  const bool separate = norm.gate != nullptr && (vt != p.V || block_form);
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
