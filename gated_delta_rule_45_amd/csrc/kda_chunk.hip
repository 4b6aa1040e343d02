// kda_chunk.hip -- chunked prefill at chunk size 64 (chunk_kda_with_fused_gate
// with its WY recompute_w_u step, vLLM PR #50649, Purpose).
//
// Within a chunk of n <= 64 tokens of one (sequence, head) that starts from
// state S, with gam_t = sum_{s<=t} g_s (per key channel), the recurrence is
// reached exactly by
//   A[t][s] = beta_t sum_i k_ti k_si e^{gam_ti - gam_si}   (s < t)
//   T       = (I + A)^{-1}
//   W       = T diag(beta) (K o e^gam),   U = T diag(beta) V     (recompute_w_u)
//   V'      = U - W S                                              (delta writes)
//   P[t][s] = sum_i q_ti k_si e^{gam_ti - gam_si}          (s <= t)
//   O       = scale [ (Q o e^gam) S + P V' ]
//   S      <- diag(e^{gam_last}) S + (K o e^{gam_last - gam})^T V'
//
// Launches on one stream, no host synchronisation (the map pass only when a
// call of these sizes can cut a sequence; see "segments" below):
//  1. plan:  chunk offsets and segments per sequence from the device
//            cu_seqlens.
//  2. intra: one workgroup per (chunk, head), all chunks in parallel (last
//            to first). Builds gam in registers, then A and P on bf16 MFMA
//            from factored operand tiles, the key channels in halves of 64
//            (or, in a second kernel for a chunk with a block that decays
//            too steeply, with pairwise fp32 exponentials on the diagonal
//            blocks), T by forward substitution plus fp32-MFMA block
//            products, then W and U on MFMA. It stores -W, scale Q o e^gam,
//            scale P, (K o e^{gam_last-gam})^T (bf16, laid out as MFMA A
//            operands), e^{gam_last} and U (fp32, in accumulator fragment
//            order) in the workspace.
//  3. map:   per non-final segment of a cut sequence, the affine map of
//            its chunks (below).
//  4. state: one workgroup per (segment, head, 64 value columns), looping over
//            the segment's chunks in order. The state lives in MFMA
//            accumulators (fp32) for the whole sequence; each chunk's A
//            operands are double-buffered in LDS, and the next chunk's are
//            copied in while the current one computes.
//
// Accumulator reuse. The bf16 16x16x32 MFMA leaves lane l with rows
// 4(l/16)+j (j < 4) of column l%16; its B operand wants rows 8(l/16)+j
// (j < 8). Two accumulator tiles (rows r0..r0+15 and r0+16..r0+31) therefore
// form a B operand directly if the contraction index is permuted within each
// 32-block: storage slot 8g+j holds index 4g+j (j < 4) or 16+4g+j-4 (j >= 4).
// The A operands that meet such a B operand (-W and Q o e^gam along channels,
// P and K^T along positions) are stored in that permuted order, so S and V'
// never leave registers.
#include <algorithm>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int C = 64;          // chunk size
constexpr int kThreads = 256;  // 4 waves per workgroup

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Index held in permuted storage slot s (0..31) of a 32-block.
__device__ __forceinline__ int perm_phys(int s) {
  const int g = s >> 3, j = s & 7;
  return j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4);
}

// Storage slot of index p (0..31) in a permuted 32-block.
__device__ __forceinline__ int perm_slot(int p) {
  const int hi = p >> 4, r = p & 15;
  return ((r >> 2) << 3) + (hi << 2) + (r & 3);
}

__device__ __forceinline__ uint16_t bf16_bits(float f) { return f32_to_bf16_rne(f); }

__device__ __forceinline__ bf16x8 to_bf16x8(const float* v) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = static_cast<__bf16>(v[j]);
  return r;
}

__device__ __forceinline__ bf16x8 pack_acc(f32x4 lo, f32x4 hi) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[j] = static_cast<__bf16>(lo[j]);
    r[4 + j] = static_cast<__bf16>(hi[j]);
  }
  return r;
}

// Residual of pack_acc: the bf16 rounding of (acc - hi), so hi + lo carries
// about 16 significant bits of the fp32 accumulators.
__device__ __forceinline__ bf16x8 pack_lo(f32x4 lo, f32x4 hi, bf16x8 h) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[j] = static_cast<__bf16>(lo[j] - static_cast<float>(h[j]));
    r[4 + j] = static_cast<__bf16>(hi[j] - static_cast<float>(h[4 + j]));
  }
  return r;
}

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

// Piece swizzle of the record's bf16 tiles. A row of N bf16 elements is
// N/8 16-byte pieces; piece p of row r is stored at piece p ^ swz<N>(r). The
// state kernel copies the record to LDS byte for byte and reads MFMA
// fragments of 16 consecutive rows at one logical piece: the swizzle puts
// those 16 reads in 16 different 16-byte bank groups (and any 8 consecutive
// rows in 8), for 256-byte rows (r & 15) and for 128-byte rows, whose odd
// rows start half way round the banks (r ^ r >> 3) & 7.
template <int N>
__device__ __forceinline__ int swz(int r) {
  static_assert(N / 8 >= 8, "rows of at least 8 pieces");
  if constexpr (N / 8 >= 16) return r & 15;
  else return (r ^ (r >> 3)) & 7;
}
// Element offset of logical (row, col) in a swizzled [rows][N] bf16 tile.
template <int N>
__device__ __forceinline__ int rec_elem(int r, int c) {
  return r * N + ((((c >> 3) ^ swz<N>(r)) << 3) | (c & 7));
}

// MFMA fragment (8 bf16) at logical (row, col) of a swizzled [rows][N] tile.
template <int N>
__device__ __forceinline__ bf16x8 frag(const uint16_t* tile, int r, int c) {
  return lds_frag(tile + rec_elem<N>(r, c));
}

// Per-(chunk, head) record in the workspace. The first five fields are
// copied to LDS as one contiguous block by the state kernel; its bf16 tiles
// are stored with the swizzle above.
template <int K, int V>
struct Rec {
  static constexpr size_t Wn = 0;                      // bf16 [C][K], -W, channels permuted
  static constexpr size_t Qg = Wn + C * K * 2;         // bf16 [C][K], scale Q o e^gam, channels permuted
  static constexpr size_t Pm = Qg + C * K * 2;         // bf16 [C][C], scale P, positions permuted
  static constexpr size_t KgT = Pm + C * C * 2;        // bf16 [K][C], positions permuted
  static constexpr size_t Eg = KgT + K * C * 2;        // fp32 [K], e^{gam_last}
  static constexpr size_t lds_part = Eg + K * 4;       // bytes copied to LDS
  static constexpr size_t Uf = (lds_part + 255) / 256 * 256;  // fp32 fragments [C/16][V/16][64][4]
  static constexpr size_t bytes = (Uf + C * V * 4 + 255) / 256 * 256;
};

// Waits until this wave's outstanding vector-memory operations (including
// LDS DMA) have completed: vmcnt = 0, other counters unconstrained.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__host__ __device__ inline int64_t max_chunks_for(int64_t num_tokens, int32_t num_seqs) {
  return num_tokens / C + num_seqs;
}

// Records, maps and starting states are laid out head-major: the chunks of
// one head follow each other, so a workgroup walking a head's chunks reads
// one contiguous stream.
__device__ __forceinline__ int64_t rec_index(int h, int c, const PrefillParams& p) {
  return static_cast<int64_t>(h) * max_chunks_for(p.num_tokens, p.num_seqs) + c;
}

// ------------------------------------------------------------- segments --
//
// The inter-chunk pass carries one state per (sequence, head) through the
// sequence's chunks, so a long sequence is a chain of dependent steps on a
// few workgroups. The chunk recurrence is affine in the state: after a run
// of chunks, S_out = M S_in + B with
//   M = prod_c (diag(e^{gam_last}) - (K o e^{gam_last - gam})^T W)   (K x K)
//   B = the state reached from S_in = 0                                (K x V)
// so a long sequence is cut into segments: a map pass computes (M, B) of
// every segment but the last in parallel, and in the state pass every
// segment first walks the maps of the segments before it
// (S_{j+1} = M_j S_j + B_j, a K x K by K x 16 product per wave and step)
// and then runs its own chunks, all segments in parallel.
//
// A sequence is cut into at most ceil(chunks / kSegMinChunks) segments of
// equal length (the last may be shorter), into no more segments than it
// takes for the cut sequences' state-pass workgroups to occupy kChipSlots
// slots (one per compute unit: its LDS image allows one workgroup per CU),
// and only into kMinCut segments or more: a map chunk costs about as much as
// a state chunk, so two segments would not shorten the chain.
constexpr int kSegMinChunks = 16;
constexpr int kMaxSegs = 16;  // <= kSegMinChunks: keeps the last segment non-empty
constexpr int kMinCut = 3;
constexpr int kChipSlots = 256;
static_assert(kMaxSegs <= kSegMinChunks, "segment count bound");

// Device-side plan of one prefill call, written by plan_kernel.
struct SegPlan {
  int32_t* chunk_start;  // [N+1] first chunk slot of each sequence
  int4* chunk_info;      // [max_chunks] per intra workgroup row j: {chunk slot, first token, tokens, 0}
                         // of chunk slot (chunks - 1 - j); tokens = 0 past the last chunk
  int32_t* seg_start;    // [N+1] first segment of each sequence
  int32_t* counts;       // [4]: segments, maps, long sequences, plan fits its bounds
  int32_t* seg_seq;      // [seg_bound] sequence of each segment
  int32_t* seg_long;     // [seg_bound] index of a cut sequence among the cut ones, else -1
  int32_t* map_seg;      // [map_bound] segment of each map item (a non-final segment)
  float* maps;           // [H][map_bound]: M (fp32 [K][K]) then B (fp32 [K][V])
  float* s0;             // [H][long_bound]: fp32 [K][V] initial state of each cut sequence
  int32_t seg_bound, map_bound, long_bound;
  int32_t max_segs;      // segments per sequence at most (host bound)
  int32_t fill_units;    // state-pass workgroups per segment (H * V / 64)
  int32_t max_chunks;    // chunk slots the records are sized for
  int32_t num_tokens;    // rows of the call (validated to fit in int32)
};

__device__ __forceinline__ int64_t map_index(int h, int mi, const SegPlan& pl) {
  return static_cast<int64_t>(h) * pl.map_bound + mi;
}
__device__ __forceinline__ int64_t s0_index(int h, int li, const SegPlan& pl) {
  return static_cast<int64_t>(h) * pl.long_bound + li;
}

// Workspace layout (byte offsets) for one call's sizes. Bounds: a cut
// sequence of len tokens has fewer than len / (64 kSegMinChunks) non-final
// segments, so a call has at most num_tokens / (64 kSegMinChunks) of them
// (and at most num_seqs (max_segs - 1)); each cut sequence has at least one.
struct Layout {
  int64_t seg_bound, map_bound, long_bound, max_segs, fill_units;
  size_t chunk_start, seg_start, counts, seg_seq, seg_long, map_seg, chunk_info;
  size_t flags, recs, maps, s0, total;
};

inline size_t round256(size_t x) { return (x + 255) / 256 * 256; }

inline size_t rec_bytes_for(int32_t K, int32_t V) {
  if (K == 64 && V == 64) return Rec<64, 64>::bytes;
  if (K == 64 && V == 128) return Rec<64, 128>::bytes;
  if (K == 128 && V == 64) return Rec<128, 64>::bytes;
  return Rec<128, 128>::bytes;
}

inline Layout layout_for(int32_t num_seqs, int64_t num_tokens, int32_t H, int32_t K, int32_t V) {
  Layout L{};
  const int64_t N = num_seqs;
  L.fill_units = static_cast<int64_t>(H) * (V / 64);
  L.max_segs = std::min<int64_t>(kMaxSegs, std::max<int64_t>(1, (kChipSlots + L.fill_units - 1) / L.fill_units));
  L.map_bound = L.max_segs < kMinCut ? 0 : std::min<int64_t>(num_tokens / (C * kSegMinChunks), N * (L.max_segs - 1));
  L.long_bound = L.map_bound;
  L.seg_bound = N + L.map_bound;
  size_t o = 0;
  L.chunk_start = o; o += (N + 1) * 4;
  L.seg_start = o;   o += (N + 1) * 4;
  L.counts = o;      o += 16;
  L.seg_seq = o;     o += L.seg_bound * 4;
  L.seg_long = o;    o += L.seg_bound * 4;
  L.map_seg = o;     o += L.map_bound * 4;
  const int64_t maxc = max_chunks_for(num_tokens, num_seqs);
  L.chunk_info = (o + 15) / 16 * 16;
  o = L.chunk_info + static_cast<size_t>(maxc) * 16;
  L.flags = round256(o);
  L.recs = L.flags + round256(static_cast<size_t>(maxc) * H);
  L.maps = L.recs + static_cast<size_t>(maxc) * H * rec_bytes_for(K, V);
  L.s0 = L.maps + static_cast<size_t>(L.map_bound) * H * (static_cast<size_t>(K) * K + static_cast<size_t>(K) * V) * 4;
  L.total = L.s0 + static_cast<size_t>(L.long_bound) * H * static_cast<size_t>(K) * V * 4;
  return L;
}

// ------------------------------------------------------------------ plan --

// Exclusive prefix sum of x over the workgroup (kThreads threads, 64-lane
// waves); `total` receives the sum. Every thread must call it.
__device__ __forceinline__ int block_exclusive_scan(int x, int* part, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(inc, d, 64);
    if (lane >= d) inc += y;
  }
  if (lane == 63) part[w] = inc;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int k = 0; k < kThreads / 64; ++k) {
    const int t = part[k];
    if (k < w) before += t;
    total += t;
  }
  __syncthreads();
  return before + inc - x;
}

__device__ __forceinline__ int chunks_of(const int32_t* cu, int i) {
  return (max(cu[i + 1] - cu[i], 0) + C - 1) / C;
}

__device__ __forceinline__ int segments_of(int nch, int target) {
  const int ns = min((nch + kSegMinChunks - 1) / kSegMinChunks, target);
  return ns >= kMinCut ? ns : 1;
}

// Chunk slots and segments of every sequence. The segment target is the
// number of segments each cut sequence needs for the cut sequences together
// to occupy the chip.
__global__ __launch_bounds__(kThreads) void plan_kernel(const int32_t* cu, int32_t N, SegPlan pl) {
  __shared__ int part[kThreads / 64];
  const int tid = threadIdx.x;
  const int per = (N + kThreads - 1) / kThreads;
  const int b = tid * per;
  const int e = min(N, b + per);
  int nl = 0;
  for (int i = b; i < e; ++i) nl += chunks_of(cu, i) > (kMinCut - 1) * kSegMinChunks;  // can be cut
  int n_long;
  block_exclusive_scan(nl, part, n_long);
  const int units = pl.fill_units * max(n_long, 1);
  const int target = min(pl.max_segs, max(1, (kChipSlots + units - 1) / units));

  int cc = 0, sc = 0, lc = 0;
  for (int i = b; i < e; ++i) {
    const int nch = chunks_of(cu, i);
    const int ns = segments_of(nch, target);
    cc += nch;
    sc += ns;
    lc += ns > 1;
  }
  int ctot, stot, ltot;
  int cb = block_exclusive_scan(cc, part, ctot);
  int sb = block_exclusive_scan(sc, part, stot);
  int lb = block_exclusive_scan(lc, part, ltot);
  const int mtot = stot - N;
  // Holds for cu_seqlens that keep to the contract; otherwise no segment
  // tables are written and the state pass does nothing.
  const bool fits = stot <= pl.seg_bound && mtot <= pl.map_bound && ltot <= pl.long_bound;
  // Intra rows past the last chunk do nothing (so do all rows if the
  // chunks outgrow the records).
  for (int jj = (ctot <= pl.max_chunks ? ctot : 0) + tid; jj < pl.max_chunks; jj += kThreads)
    pl.chunk_info[jj] = int4{0, 0, 0, 0};
  for (int i = b; i < e; ++i) {
    const int nch = chunks_of(cu, i);
    const int ns = segments_of(nch, target);
    pl.chunk_start[i] = cb;
    pl.seg_start[i] = sb;
    if (fits) {
      // Map items of sequence i start at sb - i (each earlier sequence has
      // one fewer than its segments); lb counts the earlier cut sequences.
      for (int s = 0; s < ns; ++s) {
        pl.seg_seq[sb + s] = i;
        pl.seg_long[sb + s] = ns > 1 ? lb : -1;
      }
      for (int s = 0; s + 1 < ns; ++s) pl.map_seg[sb - i + s] = sb + s;
    }
    cb += nch;
    sb += ns;
    lb += ns > 1;
  }
  __syncthreads();  // chunk_start[0 .. N-1] visible to every thread
  if (ctot <= pl.max_chunks) {
    // Intra row j takes chunk slot ctot - 1 - j (the chunks last to first);
    // slot c belongs to the last sequence whose first slot is <= c.
    for (int c = tid; c < ctot; c += kThreads) {
      int lo = 0, hi = N;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pl.chunk_start[mid] <= c) lo = mid; else hi = mid;
      }
      const int k = c - pl.chunk_start[lo];
      const int bos = cu[lo], eos = cu[lo + 1];
      const bool ok = bos >= 0 && eos <= pl.num_tokens;
      pl.chunk_info[ctot - 1 - c] = ok ? int4{c, bos + C * k, min(C, eos - bos - C * k), 0} : int4{0, 0, 0, 0};
    }
  }
  if (tid == 0) {
    pl.chunk_start[N] = ctot;
    pl.seg_start[N] = stot;
    pl.counts[0] = stot;
    pl.counts[1] = mtot;
    pl.counts[2] = ltot;
    pl.counts[3] = fits ? 1 : 0;
  }
}

// --------------------------------------------------------------- intra --

// Element offsets in XOR-swizzled row-major LDS tiles: the 16-byte pieces of
// row t are permuted by t, so the 16 rows an MFMA fragment touches fall in
// different banks (no padding, which keeps two workgroups per CU).
template <int N>  // bf16 tile [C][N]: 8 elements per piece
__device__ __forceinline__ int sw16(int t, int c) {
  constexpr int PM = (N / 8 > 16 ? 16 : N / 8) - 1;
  return t * N + ((((c >> 3) ^ (t & PM)) << 3) | (c & 7));
}
template <int N>  // fp32 tile [C][N]: 4 elements per piece
__device__ __forceinline__ int sw32(int t, int c) {
  constexpr int PM = (N / 4 > 16 ? 16 : N / 4) - 1;
  return t * N + ((((c >> 2) ^ (t & PM)) << 2) | (c & 3));
}

// Exact intra kernel LDS: 80 KiB at K = 128, two workgroups per CU.
//  k   bf16 [C][K] (sw16)  keys (zero rows past the chunk end)
//  q   bf16 [C][K] (sw16)  queries
//  u   union of
//        gam  fp32 [C][K] (sw32)  cumulative log-decay, and
//        kf   bf16 [C][K] space, placing x over gam's second half; its
//             first bytes hold beta after A/P, and
//        x    fp32 scratch: part totals, gam at block starts and per-block
//             decay ranges until gam is written; then (K o e^gam)^T, bf16
//             [K][C] (swz<C>), the B operand of W
//  at  fp32 [C][C] (sw32)  A^T
//                          strictly above the diagonal (at(s,t) = A[t][s]),
//                          T = (I + A)^{-1} strictly below it (unit
//                          diagonal implicit), beta on it
template <int K, int V>
struct IntraSmem {
  uint16_t k[C * K];
  uint16_t q[C * K];
  union {
    float gam[C * K];
    struct {
      uint16_t kf[C * K];
      float x[C * K / 2];
    } f;
  } u;
  float at[C * C];
};

// Layout of the x scratch (in floats).
template <int K>
struct XLayout {
  static constexpr int PARTS = kThreads / (K / 4);  // threads per channel quad in the gate scan
  static constexpr int tot = 0;               // [PARTS][K] partial sums of the gate scan
  static constexpr int bnd = tot + PARTS * K; // [4][K] gam at rows 16 I
  static constexpr int dmax = bnd + 4 * K;    // [4 blocks] largest decay range
  static constexpr int cij = dmax + 16;       // [10][K] e^{gam(16 I) - gam(16 J)}, J <= I
  static constexpr int end = cij + 10 * K;
  static_assert(end <= C * K / 2, "x scratch overflows its area");
};

// Factored-path bound on a 16-row block's decay range: every factored
// operand then lies in [e^-80, e^80], inside bf16/fp32 range.
constexpr float kMaxBlockDecay = 80.f;

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Steps common to both intra kernels once A^T (with beta on its diagonal)
// is in at, (K o e^gam)^T in wkt, beta in beta_l and the lane's v operands
// in vpre: T = (I + A)^{-1} in at, then W and U into the record.
template <int K, int V>
__device__ __forceinline__ void intra_inverse_wu(const PrefillParams& p, float* at, const uint16_t* wkt,
                                                 const float* beta_l,
                                                 const uint16_t (&vpre)[(V / 16 + 3) / 4][2][8],
                                                 char* rec, int w, int lane) {
  using R = Rec<K, V>;
  constexpr int NBU = (V / 16 + 3) / 4;
  const int m = lane & 15;
  const int g = lane >> 4;
  // ---- 5. T = (I + A)^{-1}: diagonal blocks by forward substitution -----
  // at(s, t) = A[t][s] for s < t; T strictly below the diagonal of at.
  if (lane < 16) {
    const int blk = w, jc = lane;
    float x[16];
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) {
      float v = (tt == jc) ? 1.f : 0.f;
#pragma unroll
      for (int s3 = 0; s3 < tt; ++s3) v = fmaf(-at[sw32<C>(16 * blk + s3, 16 * blk + tt)], x[s3], v);
      x[tt] = v;
    }
#pragma unroll
    for (int tt = 0; tt < 16; ++tt)
      if (tt > jc) at[sw32<C>(16 * blk + tt, 16 * blk + jc)] = x[tt];
  }
  lds_barrier();

  // ---- 6. off-diagonal blocks of T on fp32 MFMA ---------------------------
  // With the 32-row halves t (blocks 0, 1) and b (blocks 2, 3):
  //   T_10 = -T_11 A_10 T_00,  T_32 = -T_33 A_32 T_22,  T_bt = -T_bb (A_bt T_tt).
  // The 16x16x4 product pairs lane group g of step kk with contraction index
  // 4 g + kk, so an accumulator tile (rows 4 g + j) is the B operand of the
  // next product as it stands: step kk takes its element j = kk.
  {
    auto Tget = [&](int r, int cc) { return r > cc ? at[sw32<C>(r, cc)] : (r == cc ? 1.f : 0.f); };
    auto Aget = [&](int t, int s) { return s < t ? at[sw32<C>(s, t)] : 0.f; };  // A[t][s]
    // Operands are read into registers before their products (no LDS
    // writes intervene), so the reads overlap.
    if (w < 2) {
      const int I = 1 + 2 * w, J = 2 * w;
      float a[4], b[4], t[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        a[kk] = Aget(16 * I + m, 16 * J + 4 * g + kk);
        b[kk] = Tget(16 * J + 4 * g + kk, 16 * J + m);
        t[kk] = Tget(16 * I + m, 16 * I + 4 * g + kk);
      }
      f32x4 z = {0.f, 0.f, 0.f, 0.f}, tij = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) z = mfma4(a[kk], b[kk], z);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) tij = mfma4(t[kk], z[kk], tij);
#pragma unroll
      for (int j = 0; j < 4; ++j) at[sw32<C>(16 * I + 4 * g + j, 16 * J + m)] = -tij[j];
    }
    lds_barrier();
    {
      const int I = 2 + (w >> 1), J = w & 1;
      float a2[2][4], a3[2][4], b[2][4], t2[4], t3[4];
#pragma unroll
      for (int M = 0; M < 2; ++M)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          b[M][kk] = Tget(16 * M + 4 * g + kk, 16 * J + m);  // zero for M < J
          a2[M][kk] = Aget(32 + m, 16 * M + 4 * g + kk);
          a3[M][kk] = Aget(48 + m, 16 * M + 4 * g + kk);
        }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        t2[kk] = Tget(16 * I + m, 32 + 4 * g + kk);
        t3[kk] = Tget(48 + m, 48 + 4 * g + kk);
      }
      f32x4 y2 = {0.f, 0.f, 0.f, 0.f}, y3 = {0.f, 0.f, 0.f, 0.f}, tij = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int M = 0; M < 2; ++M)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          y2 = mfma4(a2[M][kk], b[M][kk], y2);
          y3 = mfma4(a3[M][kk], b[M][kk], y3);
        }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) tij = mfma4(t2[kk], y2[kk], tij);
      if (I == 3) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) tij = mfma4(t3[kk], y3[kk], tij);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) at[sw32<C>(16 * I + 4 * g + j, 16 * J + m)] = -tij[j];
    }
    lds_barrier();
  }

  // ---- 7. W = T diag(beta)(K o e^gam), U = T diag(beta) V on MFMA -------
  // beta is folded into the fp32 columns of T before the bf16 cast, so V
  // enters the product exactly as given. T is lower triangular, so rows
  // 0..31 need only positions 0..31.
  {
    // T diag(beta) as bf16 fragments: row 16 pb + m, positions 32 kb + 8 g
    // .. +7, read as two 16-byte pieces of at (T strictly below the
    // diagonal; the diagonal and above are masked by index).
    bf16x8 Tf[4][2];
#pragma unroll
    for (int pb = 0; pb < 4; ++pb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int row = 16 * pb + m;
        const int c0 = 32 * kb + 8 * g;
        const f32x4 t0 = *reinterpret_cast<const f32x4*>(&at[sw32<C>(row, c0)]);
        const f32x4 t1 = *reinterpret_cast<const f32x4*>(&at[sw32<C>(row, c0 + 4)]);
        const f32x4 b0 = *reinterpret_cast<const f32x4*>(&beta_l[c0]);
        const f32x4 b1 = *reinterpret_cast<const f32x4*>(&beta_l[c0 + 4]);
        float tv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int col = c0 + j;
          const float tval = j < 4 ? t0[j] : t1[j - 4];
          const float bcol = j < 4 ? b0[j] : b1[j - 4];
          tv[j] = (col < row ? tval : (col == row ? 1.f : 0.f)) * bcol;
        }
        Tf[pb][kb] = to_bf16x8(tv);
      }
    // -W^T = -(K o e^gam)^T (T diag(beta))^T: the same fragments with the
    // operands swapped leave lane (m, g) four consecutive channels
    // 16 nb + 4 g .. +3 of position 16 pb + m, which are four consecutive
    // slots of the record's permuted channel order: one 8-byte store each.
    {
      const __amdgpu_buffer_rsrc_t rwn = make_rsrc(rec + R::Wn, static_cast<uint32_t>(C * K * 2));
      typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
      for (int nb = w; nb < K / 16; nb += 4) {
        bf16x8 Bf[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) Bf[kb] = frag<C>(wkt, 16 * nb + m, 32 * kb + 8 * g);
        const int col = 32 * (nb >> 1) + 8 * g + 4 * (nb & 1);
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) {
          f32x4 D = mfma16(Bf[0], Tf[pb][0], f32x4{0.f, 0.f, 0.f, 0.f});
          if (pb >= 2) D = mfma16(Bf[1], Tf[pb][1], D);
          const u32x2 v = {pack_bf16x2(-D[0], -D[1]), pack_bf16x2(-D[2], -D[3])};
          __builtin_amdgcn_raw_buffer_store_b64(v, rwn, rec_elem<K>(16 * pb + m, col) * 2, 0, 0);
        }
      }
    }
    // U written straight out in accumulator fragment order.
    f32x4* uf = reinterpret_cast<f32x4*>(rec + R::Uf);
#pragma unroll
    for (int u = 0; u < NBU; ++u) {
      const int nb = w + 4 * u;
      if (nb >= V / 16) break;
      bf16x8 Bv[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 8; ++j) Bv[kb][j] = __builtin_bit_cast(__bf16, vpre[u][kb][j]);
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) {
        f32x4 D = mfma16(Tf[pb][0], Bv[0], f32x4{0.f, 0.f, 0.f, 0.f});
        if (pb >= 2) D = mfma16(Tf[pb][1], Bv[1], D);
        uf[(pb * (V / 16) + nb) * 64 + lane] = D;
      }
    }
  }
}

// One workgroup of the exact intra kernel, launched after the factored one
// on the same grid: it takes only the chunks the factored kernel flagged
// (some 16-row block decays by more than kMaxBlockDecay), with gam in LDS
// and pairwise exponentials on the diagonal blocks. Separate kernels keep
// the factored path's registers and LDS free of the exact path's.
template <int K, int V>
__device__ __forceinline__ void intra_exact(const PrefillParams& p, const int4* chunk_info,
                                            char* recs, uint8_t* exact_flags) {
  using R = Rec<K, V>;
  using SM = IntraSmem<K, V>;
  using XL = XLayout<K>;
  __shared__ SM sm;

  const int H = p.H;
  // Chunks are taken last to first: the state pass reads them first to
  // last, so its early chunks are the most recently written (still in the
  // memory-side cache when the records outgrow it). The plan gives row j
  // its chunk slot, first token and token count in one load (zero tokens
  // past the last chunk, or for cu_seqlens outside the contract).
  const int j = static_cast<int>(blockIdx.x / H);
  const int h = static_cast<int>(blockIdx.x % H);
  const int4 info = chunk_info[j];
  const int n = uniform(info.z);
  if (n <= 0) return;  // uniform
  const int c = uniform(info.x);
  const int64_t t0 = uniform(info.y);
  uint8_t* flag = exact_flags + static_cast<int64_t>(c) * H + h;
  if (*flag == 0) return;  // uniform: the factored kernel took this chunk

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);  // wave index, in a scalar register
  const int m = lane & 15;
  const int g = lane >> 4;
  constexpr int KP8 = K / 8;                     // 16-byte pieces per bf16 row
  constexpr int KPM = (KP8 > 16 ? 16 : KP8) - 1;

  char* rec = recs + rec_index(h, c, p) * static_cast<int64_t>(R::bytes);
  float* x = sm.u.f.x;
  uint16_t* wkt = reinterpret_cast<uint16_t*>(sm.u.f.x);

  // ---- 1. raw_g into registers, k and q tiles by LDS DMA -----------------
  // Rows past the chunk end read 0. The thread's raw_g arrives in its own
  // registers, so the gate scan waits only for those loads while the k and
  // q copies keep landing under it.
  // Thread (q4, part) owns channels 4 q4 .. 4 q4 + 3 at positions
  // part PP .. part PP + PP - 1: its tile reads and writes are 8 bytes wide,
  // and wave w holds exactly the 16-row block w.
  constexpr int NQ = K / 4;              // channel quads
  constexpr int NPART = XL::PARTS;       // 8 at K = 128, 16 at K = 64
  constexpr int PP = C / NPART;          // positions per thread: 8 or 4
  static_assert(NPART * PP == C && (64 / NQ) * PP == 16 && PP % 4 == 0, "a wave holds one 16-row block");
  const int q4 = tid % NQ, part = tid / NQ;
  const int c4 = 4 * q4;                 // the thread's first channel
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  u32x2 rgw[PP];
  float a_h, dtb[4];
  uint16_t rb_bits = 0;
  {
    const int64_t rs = p.qkv_row_stride * 2;  // bytes per mixed_qkv row
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.qkv + t0 * p.qkv_row_stride, static_cast<uint32_t>(n * rs));
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.raw_g + t0 * (H * K), static_cast<uint32_t>(n * H * K * 2));
#pragma unroll
    for (int i = 0; i < PP; ++i)
      rgw[i] = __builtin_amdgcn_raw_buffer_load_b64(rg, ((part * PP + i) * H * K + h * K + c4) * 2, 0, 0);
    // Per-head gate parameters and beta.
    a_h = __expf(p.A_log[h]);
#pragma unroll
    for (int j = 0; j < 4; ++j) dtb[j] = p.dt_bias[h * K + c4 + j];
    // beta of position tid (rows past the chunk end read 0; only tid < n is used).
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.raw_beta + t0 * H, static_cast<uint32_t>(n * H * 2));
    rb_bits = __builtin_amdgcn_raw_buffer_load_b16(rb, (tid * H + h) * 2, 0, 0);
    // Keep these loads ahead of the copies: loads complete in issue order,
    // so anything issued after the copies would wait for them.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < C * KP8 / kThreads; ++r) {
      const int ps = r * kThreads + tid;          // physical piece in the tile
      const int t = ps / KP8;
      const int pl = (ps % KP8) ^ (t & KPM);      // logical piece stored there
      const int slot = r * kThreads + (tid & ~63);
      const int qoff = static_cast<int>(t * rs) + (h * K + pl * 8) * 2;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, reinterpret_cast<uint4*>(sm.q) + slot, 16, qoff, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, reinterpret_cast<uint4*>(sm.k) + slot, 16, qoff + H * K * 2, 0, 0, 0);
    }
  }

  // ---- 2. gate and cumulative log-decay, in registers ---------------------
  const float beta_t = (tid < n) ? sigmoid_f32(bf16_to_f32(rb_bits)) : 0.f;
  // Each thread scans its PP positions; partial totals are added across
  // parts through x.
  float gm[PP][4];
  float gl[4] = {0.f, 0.f, 0.f, 0.f};
  {
    const float a = a_h;
    const bool has_lb = p.has_lb != 0;
    // All reads first (rows past the chunk end hold zeros), then a
    // branch-free scan; padded positions do not decay, so row 63 holds
    // gam_last.
    float rg[PP][4];
#pragma unroll
    for (int i = 0; i < PP; ++i) {
      rg[i][0] = __uint_as_float(rgw[i][0] << 16);
      rg[i][1] = __uint_as_float(rgw[i][0] & 0xffff0000u);
      rg[i][2] = __uint_as_float(rgw[i][1] << 16);
      rg[i][3] = __uint_as_float(rgw[i][1] & 0xffff0000u);
    }
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    if (has_lb) {
#pragma unroll
      for (int i = 0; i < PP; ++i) {
        const bool live = part * PP + i < n;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float gv = p.lower_bound * sigmoid_f32(a * (rg[i][j] + dtb[j]));
          acc[j] += live ? gv : 0.f;
          gm[i][j] = acc[j];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < PP; ++i) {
        const bool live = part * PP + i < n;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float gv = -a * softplus_f32(rg[i][j] + dtb[j]);
          acc[j] += live ? gv : 0.f;
          gm[i][j] = acc[j];
        }
      }
    }
    *reinterpret_cast<f32x4*>(&x[XL::tot + part * K + c4]) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    lds_barrier();  // partial totals visible
    float before[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q2 = 0; q2 < NPART; ++q2) {
      const f32x4 tq = *reinterpret_cast<const f32x4*>(&x[XL::tot + q2 * K + c4]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (q2 < part) before[j] += tq[j];
        gl[j] += tq[j];
      }
    }
    if (tid < C) sm.at[sw32<C>(tid, tid)] = beta_t;  // beta on the diagonal of at
#pragma unroll
    for (int i = 0; i < PP; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) gm[i][j] += before[j];
    // Block w's bound gam(16 w) is row 0 of the wave's first part (lanes
    // 0 .. NQ-1); its row 15 is the last row of the wave's last part, in
    // lane + 64 - NQ. The decay range is gam(16 w) - gam(16 w + 15).
    float d = 0.f;
    {
      float last[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) last[j] = __shfl_xor(gm[PP - 1][j], 64 - NQ);
      if (lane < NQ) {
        *reinterpret_cast<f32x4*>(&x[XL::bnd + w * K + c4]) = f32x4{gm[0][0], gm[0][1], gm[0][2], gm[0][3]};
#pragma unroll
        for (int j = 0; j < 4; ++j) d = fmaxf(d, gm[0][j] - last[j]);
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) d = fmaxf(d, __shfl_xor(d, off));
    if (lane == 0) x[XL::dmax + w] = d;
    if (part == 0)
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(rec + R::Eg) + c4) =
          f32x4{__expf(gl[0]), __expf(gl[1]), __expf(gl[2]), __expf(gl[3])};
  }
  wait_vmem();  // this thread's k and q copies (and every load before them) have landed
  lds_barrier();
  bool fast = true;
#pragma unroll
  for (int I = 0; I < 4; ++I) fast = fast && x[XL::dmax + I] <= kMaxBlockDecay;

  // K o e^gam of this thread's channels and positions, as bf16 pairs, kept
  // in registers until x is free.
  uint32_t wkp[4][PP / 2];

  {
    // ---- 3e/4e. exact path (a block decays by more than the bound) --------
    (void)fast;
    lds_barrier();  // every thread has read the decay ranges (gam overlays x)
#pragma unroll
    for (int i = 0; i < PP; ++i)
      *reinterpret_cast<f32x4*>(&sm.u.gam[sw32<K>(part * PP + i, c4)]) = f32x4{gm[i][0], gm[i][1], gm[i][2], gm[i][3]};
    lds_barrier();
    // Exact path, elementwise outputs: Q o e^gam and (K o e^{gl-gam})^T.
    {
      uint16_t* qg = reinterpret_cast<uint16_t*>(rec + R::Qg);
      for (int e = tid; e < C * KP8; e += kThreads) {
        const int t = e / KP8, pc = e % KP8;
        const int cb = (pc >> 2) * 32 + 4 * (pc & 3);  // storage piece pc holds channels cb..cb+3, cb+16..cb+19
        float qv[8], vals[8];
        {
          const uint2 w0 = *reinterpret_cast<const uint2*>(&sm.q[sw16<K>(t, cb)]);
          const uint2 w1 = *reinterpret_cast<const uint2*>(&sm.q[sw16<K>(t, cb + 16)]);
          qv[0] = __uint_as_float(w0.x << 16); qv[1] = __uint_as_float(w0.x & 0xffff0000u);
          qv[2] = __uint_as_float(w0.y << 16); qv[3] = __uint_as_float(w0.y & 0xffff0000u);
          qv[4] = __uint_as_float(w1.x << 16); qv[5] = __uint_as_float(w1.x & 0xffff0000u);
          qv[6] = __uint_as_float(w1.y << 16); qv[7] = __uint_as_float(w1.y & 0xffff0000u);
        }
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(&sm.u.gam[sw32<K>(t, cb)]);
        const f32x4 g1 = *reinterpret_cast<const f32x4*>(&sm.u.gam[sw32<K>(t, cb + 16)]);
  #pragma unroll
        for (int j = 0; j < 4; ++j) {
          vals[j] = p.scale * qv[j] * __expf(g0[j]);
          vals[4 + j] = p.scale * qv[4 + j] * __expf(g1[j]);
        }
        uint4 o;
        o.x = pack_bf16x2(vals[0], vals[1]); o.y = pack_bf16x2(vals[2], vals[3]);
        o.z = pack_bf16x2(vals[4], vals[5]); o.w = pack_bf16x2(vals[6], vals[7]);
        *reinterpret_cast<uint4*>(qg + rec_elem<K>(t, pc * 8)) = o;
      }
      uint16_t* kgt = reinterpret_cast<uint16_t*>(rec + R::KgT);
      for (int e = tid; e < K * (C / 8); e += kThreads) {
        const int ch = e / (C / 8), pc = e % (C / 8);
        const int base = (pc >> 2) * 32;
        const float gl = sm.u.gam[sw32<K>(C - 1, ch)];
        float vals[8];
  #pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int t = base + perm_phys((pc & 3) * 8 + j);
          vals[j] = bf16_to_f32(sm.k[sw16<K>(t, ch)]) * __expf(gl - sm.u.gam[sw32<K>(t, ch)]);
        }
        uint4 o;
        o.x = pack_bf16x2(vals[0], vals[1]); o.y = pack_bf16x2(vals[2], vals[3]);
        o.z = pack_bf16x2(vals[4], vals[5]); o.w = pack_bf16x2(vals[6], vals[7]);
        *reinterpret_cast<uint4*>(kgt + rec_elem<C>(ch, pc * 8)) = o;
      }
    }


    // Exact path, A and P by 16x16 blocks (I, J), J <= I.
    // Fast path for block-row I: one reference row r = 16 I + 7. For s in an
    // earlier block e^{gam_r - gam_s} <= 1; inside block I every factor lies
    // within e^{+-D}, D = the block's largest decay range over channels. If
    // D <= 80 every factor fits bf16 and every product with s <= t equals
    // e^{gam_t - gam_s} <= 1, so the whole block-row runs on MFMA. Otherwise
    // the exact scheme: reference 16 I for J < I (both factors <= 1) and
    // pairwise fp32 exponentials on the diagonal block.
    // A goes transposed into at (strictly above the diagonal); P goes straight
    // to the workspace (bf16, positions permuted), including the zero blocks
    // above the diagonal that the state kernel reads.
    {
      uint16_t* pm = reinterpret_cast<uint16_t*>(rec + R::Pm);
      const int blocks[4][3][2] = {{{3, 3}, {3, 0}, {0, 0}},
                                   {{2, 2}, {3, 1}, {1, 0}},
                                   {{1, 1}, {3, 2}, {-1, -1}},
                                   {{2, 1}, {2, 0}, {-1, -1}}};
      for (int bi = 0; bi < 3; ++bi) {
        const int I = blocks[w][bi][0], J = blocks[w][bi][1];
        if (I < 0) break;
        float dloc = 0.f;
        for (int ch = lane; ch < K; ch += 64)
          dloc = fmaxf(dloc, sm.u.gam[sw32<K>(16 * I, ch)] - sm.u.gam[sw32<K>(16 * I + 15, ch)]);
  #pragma unroll
        for (int off = 32; off > 0; off >>= 1) dloc = fmaxf(dloc, __shfl_xor(dloc, off));
        const bool fast = dloc <= 80.f;  // wave-uniform after the butterfly
        if (J < I || fast) {
          const int r = fast ? 16 * I + 7 : 16 * I;
          f32x4 dA = {0.f, 0.f, 0.f, 0.f}, dP = {0.f, 0.f, 0.f, 0.f};
  #pragma unroll
          for (int kb = 0; kb < K / 32; ++kb) {
            const int c0 = 32 * kb + 8 * g;
            const uint4 ka = *reinterpret_cast<const uint4*>(&sm.k[sw16<K>(16 * I + m, c0)]);
            const uint4 kbv = *reinterpret_cast<const uint4*>(&sm.k[sw16<K>(16 * J + m, c0)]);
            const uint4 qav = *reinterpret_cast<const uint4*>(&sm.q[sw16<K>(16 * I + m, c0)]);
            const uint32_t qaw[4] = {qav.x, qav.y, qav.z, qav.w};
            const f32x4 gt0 = *reinterpret_cast<const f32x4*>(&sm.u.gam[sw32<K>(16 * I + m, c0)]);
            const f32x4 gt1 = *reinterpret_cast<const f32x4*>(&sm.u.gam[sw32<K>(16 * I + m, c0 + 4)]);
            const f32x4 gr0 = *reinterpret_cast<const f32x4*>(&sm.u.gam[sw32<K>(r, c0)]);
            const f32x4 gr1 = *reinterpret_cast<const f32x4*>(&sm.u.gam[sw32<K>(r, c0 + 4)]);
            const f32x4 gs0 = *reinterpret_cast<const f32x4*>(&sm.u.gam[sw32<K>(16 * J + m, c0)]);
            const f32x4 gs1 = *reinterpret_cast<const f32x4*>(&sm.u.gam[sw32<K>(16 * J + m, c0 + 4)]);
            const uint32_t kaw[4] = {ka.x, ka.y, ka.z, ka.w};
            const uint32_t kbw[4] = {kbv.x, kbv.y, kbv.z, kbv.w};
            float ak[8], aq[8], bk[8];
  #pragma unroll
            for (int j = 0; j < 8; ++j) {
              const float gt = j < 4 ? gt0[j] : gt1[j - 4];
              const float gr = j < 4 ? gr0[j] : gr1[j - 4];
              const float gs = j < 4 ? gs0[j] : gs1[j - 4];
              const float kav = __uint_as_float(j & 1 ? (kaw[j >> 1] & 0xffff0000u) : (kaw[j >> 1] << 16));
              const float kbf = __uint_as_float(j & 1 ? (kbw[j >> 1] & 0xffff0000u) : (kbw[j >> 1] << 16));
              const float ea = __expf(gt - gr);
              ak[j] = kav * ea;
              aq[j] = __uint_as_float(j & 1 ? (qaw[j >> 1] & 0xffff0000u) : (qaw[j >> 1] << 16)) * ea;
              bk[j] = kbf * __expf(gr - gs);
            }
            const bf16x8 b = to_bf16x8(bk);
            dA = mfma16(to_bf16x8(ak), b, dA);
            dP = mfma16(to_bf16x8(aq), b, dP);
          }
          // Lane holds rows 16 I + 4 g + j of column s = 16 J + m. Entries
          // above the diagonal are dropped (they may be huge or non-finite).
          const int s2 = 16 * J + m;
  #pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int row = 16 * I + 4 * g + j;
            if (s2 < row) sm.at[sw32<C>(s2, row)] = sm.at[sw32<C>(row, row)] * dA[j];
            pm[rec_elem<C>(row, 32 * (s2 >> 5) + perm_slot(s2 & 31))] = bf16_bits(s2 <= row ? p.scale * dP[j] : 0.f);
          }
        } else {
          // Diagonal block pairwise: lane (t, cq) = (m, g) covers row t and a
          // quarter of the channels; partial sums are reduced over quarters.
          constexpr int CQ = K / 4;
          const int t = m, cq = g, row = 16 * I + t;
          float ares[16], pres[16];
#pragma unroll
          for (int s3 = 0; s3 < 16; ++s3) {
            ares[s3] = 0.f;
            pres[s3] = 0.f;
          }
          for (int i8 = 0; i8 < CQ; i8 += 8) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const int ch = cq * CQ + i8 + i;
              const float gt = sm.u.gam[sw32<K>(row, ch)];
              const float kt = bf16_to_f32(sm.k[sw16<K>(row, ch)]);
              const float qti = bf16_to_f32(sm.q[sw16<K>(row, ch)]);
#pragma unroll
              for (int s3 = 0; s3 < 16; ++s3) {
                const int srow = 16 * I + s3;
                // gam is non-increasing, so for s <= t the exponent is <= 0;
                // the min only keeps the masked s > t entries finite.
                const float ke = bf16_to_f32(sm.k[sw16<K>(srow, ch)]) *
                                 __expf(fminf(gt - sm.u.gam[sw32<K>(srow, ch)], 0.f));
                ares[s3] = fmaf(kt, ke, ares[s3]);
                pres[s3] = fmaf(qti, ke, pres[s3]);
              }
            }
          }
#pragma unroll
          for (int s3 = 0; s3 < 16; ++s3) {
            ares[s3] += __shfl_xor(ares[s3], 16);
            ares[s3] += __shfl_xor(ares[s3], 32);
            pres[s3] += __shfl_xor(pres[s3], 16);
            pres[s3] += __shfl_xor(pres[s3], 32);
          }
          if (cq == 0) {
            const float bt = sm.at[sw32<C>(row, row)];
#pragma unroll
            for (int s3 = 0; s3 < 16; ++s3) {
              const int col = 16 * I + s3;
              if (s3 < t) sm.at[sw32<C>(col, row)] = bt * ares[s3];
              pm[rec_elem<C>(row, 32 * (col >> 5) + perm_slot(col & 31))] = bf16_bits(s3 <= t ? p.scale * pres[s3] : 0.f);
            }
          }
        }
      }
      if (w == 3) {
        // Zero P blocks above the diagonal that the state kernel reads:
        // rows 0..15 x cols 16..31 and rows 32..47 x cols 48..63.
  #pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = 4 * g + j;
          pm[rec_elem<C>(row, perm_slot(16 + m))] = 0;
          pm[rec_elem<C>(32 + row, 32 + perm_slot(16 + m))] = 0;
        }
      }
    }

    // K o e^gam from the LDS tiles (k is unchanged on this path).
    float wk_even[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < PP; ++i) {
      const int t = part * PP + i;
      const uint2 kv = *reinterpret_cast<const uint2*>(&sm.k[sw16<K>(t, c4)]);
      const f32x4 gv = *reinterpret_cast<const f32x4*>(&sm.u.gam[sw32<K>(t, c4)]);
      const float kf[4] = {__uint_as_float(kv.x << 16), __uint_as_float(kv.x & 0xffff0000u),
                           __uint_as_float(kv.y << 16), __uint_as_float(kv.y & 0xffff0000u)};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float val = kf[j] * __expf(gv[j]);
        if (i & 1) wkp[j][i >> 1] = pack_bf16x2(wk_even[j], val);
        else wk_even[j] = val;
      }
    }
  }
  // v for the U phase, fetched now so its latency hides behind the inverse:
  // lane (m, g) needs v[t][16 nb + m] for t = 32 kb + 8 g + j, nb = w, w + 4.
  // 16-bit buffer loads over the chunk's rows: rows past its end read zero,
  // the lane part of the offset is fixed and the row part is scalar.
  constexpr int NBU = (V / 16 + 3) / 4;
  static_assert(V / 16 <= 4 * NBU && V / 16 > 4 * (NBU - 1), "every wave has NBU column blocks");
  uint16_t vpre[NBU][2][8];
  {
    const int rs = static_cast<int>(p.qkv_row_stride * 2);  // bytes per mixed_qkv row
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.qkv + t0 * p.qkv_row_stride, static_cast<uint32_t>(n * rs));
    const int vlane = (2 * H * K + h * V + m) * 2 + 8 * g * rs;
#pragma unroll
    for (int u = 0; u < NBU; ++u)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int nb = w + 4 * u;
          vpre[u][kb][j] = __builtin_amdgcn_raw_buffer_load_b16(rv, vlane + 32 * nb, (32 * kb + j) * rs, 0);
        }
  }


  lds_barrier();  // A^T complete; x (or gam) no longer read

  // beta of every position as a plain array in the first bytes of the kf
  // area (dead from here), for 16-byte reads in the W/U step.
  float* beta_l = reinterpret_cast<float*>(sm.u.f.kf);
  if (tid < C) beta_l[tid] = beta_t;

  // ---- 4. (K o e^gam)^T into x: 16-byte pieces of 8 positions -----------
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (PP == 8)
      *reinterpret_cast<uint4*>(wkt + rec_elem<C>(c4 + j, part * PP)) = uint4{wkp[j][0], wkp[j][1], wkp[j][2], wkp[j][3]};
    else
      *reinterpret_cast<uint2*>(wkt + rec_elem<C>(c4 + j, part * PP)) = uint2{wkp[j][0], wkp[j][1]};
  }

  intra_inverse_wu<K, V>(p, sm.at, wkt, beta_l, vpre, rec, w, lane);
}


// ------------------------------------------------------ intra, factored --
//
// The factored path works through the key channels in halves of 64, so one
// half's k, q and K o F tiles (24 KiB) are all the tile space it needs: 47
// KiB of LDS in all, three workgroups per CU. A and P accumulate over the
// halves in registers; after the last half the tile space holds
// (K o e^gam)^T for W. Chunks with a block that decays too steeply are
// flagged for the exact kernel (which recomputes the whole chunk).
constexpr int kHalf = 64;  // channels per half

template <int K, int V>
struct IntraHalfSmem {
  union {
    struct {
      uint16_t k[C * kHalf];   // keys, then K o R (sw16<kHalf>)
      uint16_t q[C * kHalf];   // queries, then Q o R
      uint16_t kf[C * kHalf];  // K o F
    } t;
    uint16_t wkt[K * C];       // (K o e^gam)^T, bf16 [K][C] (swz<C>), after A/P
  } u;
  float x[XLayout<kHalf>::end];  // one half's scan totals, bounds, ranges, c_IJ; then beta
  float at[C * C];               // as in the exact kernel: A^T, T, beta on the diagonal
};

template <int K, int V>
__device__ __forceinline__ void intra_factored(const PrefillParams& p, const int4* chunk_info,
                                               char* recs, uint8_t* exact_flags) {
  using R = Rec<K, V>;
  using SM = IntraHalfSmem<K, V>;
  using XL = XLayout<kHalf>;
  constexpr int NH = K / kHalf;  // halves
  __shared__ SM sm;

  const int H = p.H;
  const int j = static_cast<int>(blockIdx.x / H);
  const int h = static_cast<int>(blockIdx.x % H);
  const int4 info = chunk_info[j];
  const int n = uniform(info.z);
  if (n <= 0) return;  // uniform
  const int c = uniform(info.x);
  const int64_t t0 = uniform(info.y);
  uint8_t* flag = exact_flags + static_cast<int64_t>(c) * H + h;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int m = lane & 15;
  const int g = lane >> 4;
  char* rec = recs + rec_index(h, c, p) * static_cast<int64_t>(R::bytes);

  // Thread (q4, part) owns channels ch0 + 4 q4 .. + 3 of each half at
  // positions part PP .. part PP + PP - 1; wave w holds the 16-row block w.
  constexpr int NQ = kHalf / 4;         // 16 channel quads per half
  constexpr int NPART = XL::PARTS;      // 16 parts
  constexpr int PP = C / NPART;         // 4 positions per thread
  static_assert(NPART * PP == C && (64 / NQ) * PP == 16 && PP == 4, "a wave holds one 16-row block");
  constexpr int KP8 = kHalf / 8;        // 16-byte pieces per tile row
  const int q4 = tid % NQ, part = tid / NQ;
  const int c4 = 4 * q4;
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

  // raw_g of both halves, gate parameters and beta into registers first.
  const int rs = static_cast<int>(p.qkv_row_stride * 2);  // bytes per mixed_qkv row
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.qkv + t0 * p.qkv_row_stride, static_cast<uint32_t>(n * rs));
  u32x2 rgw[NH][PP];
  float dtb[NH][4];
  {
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.raw_g + t0 * (H * K), static_cast<uint32_t>(n * H * K * 2));
#pragma unroll
    for (int hf = 0; hf < NH; ++hf)
#pragma unroll
      for (int i = 0; i < PP; ++i)
        rgw[hf][i] = __builtin_amdgcn_raw_buffer_load_b64(rg, ((part * PP + i) * H * K + h * K + kHalf * hf + c4) * 2, 0, 0);
#pragma unroll
    for (int hf = 0; hf < NH; ++hf)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) dtb[hf][jj] = p.dt_bias[h * K + kHalf * hf + c4 + jj];
  }
  const float a_h = __expf(p.A_log[h]);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.raw_beta + t0 * H, static_cast<uint32_t>(n * H * 2));
  const uint16_t rb_bits = __builtin_amdgcn_raw_buffer_load_b16(rb, (tid * H + h) * 2, 0, 0);
  auto copy_tiles = [&](int hf) {  // one half's q and k columns by LDS DMA
#pragma unroll
    for (int r = 0; r < C * KP8 / kThreads; ++r) {
      const int ps = r * kThreads + tid;
      const int t = ps / KP8;
      const int pl = (ps % KP8) ^ (t & (KP8 - 1));
      const int slot = r * kThreads + (tid & ~63);
      const int qoff = t * rs + (h * K + kHalf * hf + pl * 8) * 2;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, reinterpret_cast<uint4*>(sm.u.t.q) + slot, 16, qoff, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, reinterpret_cast<uint4*>(sm.u.t.k) + slot, 16, qoff + H * K * 2, 0, 0, 0);
    }
  };
  __builtin_amdgcn_sched_barrier(0);
  copy_tiles(0);
  const float beta_t = (tid < n) ? sigmoid_f32(bf16_to_f32(rb_bits)) : 0.f;

  // The blocks (I, J), J <= I, of A and P each wave computes, with their
  // accumulators kept over the halves.
  const int blocks[4][3][2] = {{{3, 3}, {3, 0}, {0, 0}},
                               {{2, 2}, {3, 1}, {1, 0}},
                               {{1, 1}, {3, 2}, {-1, -1}},
                               {{2, 1}, {2, 0}, {-1, -1}}};
  f32x4 dA[3], dPt[3];
#pragma unroll
  for (int bi = 0; bi < 3; ++bi) {
    dA[bi] = f32x4{0.f, 0.f, 0.f, 0.f};
    dPt[bi] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  uint32_t wkp[NH][4][PP / 2];  // K o e^gam of the thread's channels, bf16 pairs
  const __amdgpu_buffer_rsrc_t rqg = make_rsrc(rec + R::Qg, static_cast<uint32_t>(C * K * 2));
  const __amdgpu_buffer_rsrc_t rkg = make_rsrc(rec + R::KgT, static_cast<uint32_t>(K * C * 2));

#pragma unroll
  for (int hf = 0; hf < NH; ++hf) {
    const int ch0 = kHalf * hf;
    if (hf > 0) {
      // Every wave is done with the previous half's tiles.
      lds_barrier();
      copy_tiles(hf);
    }
    // ---- gate and cumulative log-decay of the half, in registers ---------
    float gm[PP][4];
    float gl[4] = {0.f, 0.f, 0.f, 0.f};
    {
      const bool has_lb = p.has_lb != 0;
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < PP; ++i) {
        const bool live = part * PP + i < n;
        const float rg4[4] = {__uint_as_float(rgw[hf][i][0] << 16), __uint_as_float(rgw[hf][i][0] & 0xffff0000u),
                              __uint_as_float(rgw[hf][i][1] << 16), __uint_as_float(rgw[hf][i][1] & 0xffff0000u)};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float gv = gate_log_decay(rg4[jj], dtb[hf][jj], a_h, has_lb, p.lower_bound);
          acc[jj] += live ? gv : 0.f;
          gm[i][jj] = acc[jj];
        }
      }
      *reinterpret_cast<f32x4*>(&sm.x[XL::tot + part * kHalf + c4]) = f32x4{acc[0], acc[1], acc[2], acc[3]};
      lds_barrier();  // partial totals visible
      float before[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q2 = 0; q2 < NPART; ++q2) {
        const f32x4 tq = *reinterpret_cast<const f32x4*>(&sm.x[XL::tot + q2 * kHalf + c4]);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          if (q2 < part) before[jj] += tq[jj];
          gl[jj] += tq[jj];
        }
      }
      if (hf == 0 && tid < C) sm.at[sw32<C>(tid, tid)] = beta_t;  // beta on the diagonal of at
#pragma unroll
      for (int i = 0; i < PP; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) gm[i][jj] += before[jj];
      // Block w's bound gam(16 w) is row 0 of the wave's first part (lanes
      // 0 .. NQ-1); its row 15 is the last row of the wave's last part.
      float d = 0.f;
      {
        float last[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) last[jj] = __shfl_xor(gm[PP - 1][jj], 64 - NQ);
        if (lane < NQ) {
          *reinterpret_cast<f32x4*>(&sm.x[XL::bnd + w * kHalf + c4]) = f32x4{gm[0][0], gm[0][1], gm[0][2], gm[0][3]};
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) d = fmaxf(d, gm[0][jj] - last[jj]);
        }
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) d = fmaxf(d, __shfl_xor(d, off));
      if (lane == 0) sm.x[XL::dmax + w] = d;
      if (part == 0)
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(rec + R::Eg) + ch0 + c4) =
            f32x4{__expf(gl[0]), __expf(gl[1]), __expf(gl[2]), __expf(gl[3])};
    }
    wait_vmem();  // this half's k and q copies (and every load before them) have landed
    lds_barrier();
    bool fast = true;
#pragma unroll
    for (int I = 0; I < 4; ++I) fast = fast && sm.x[XL::dmax + I] <= kMaxBlockDecay;
    if (!fast) {  // uniform: the exact kernel takes the whole chunk
      if (tid == 0) *flag = 1;
      return;
    }
    // ---- factored operands of the half (see the exact kernel's notes) -----
    for (int e = tid; e < 10 * kHalf; e += kThreads) {
      const int pr = e / kHalf, cc = e % kHalf;
      const int I = pr < 1 ? 0 : pr < 3 ? 1 : pr < 6 ? 2 : 3;
      const int J = pr - I * (I + 1) / 2;
      sm.x[XL::cij + e] = __expf(sm.x[XL::bnd + I * kHalf + cc] - sm.x[XL::bnd + J * kHalf + cc]);
    }
    const f32x4 rho = *reinterpret_cast<const f32x4*>(&sm.x[XL::bnd + w * kHalf + c4]);
    float E[4], sE[4], G[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      E[jj] = __expf(rho[jj]);
      sE[jj] = p.scale * E[jj];
      G[jj] = __expf(gl[jj] - rho[jj]);
    }
    const int cg4 = ch0 + c4;  // the thread's first channel of the head
    const int r8 = (cg4 & 31) >> 2;
    const int qcol = 32 * (cg4 >> 5) + 8 * (r8 & 3) + 4 * (r8 >> 2);
    uint2 kq[PP], qq[PP];
#pragma unroll
    for (int i = 0; i < PP; ++i) {
      const int o = sw16<kHalf>(part * PP + i, c4);
      kq[i] = *reinterpret_cast<const uint2*>(&sm.u.t.k[o]);
      qq[i] = *reinterpret_cast<const uint2*>(&sm.u.t.q[o]);
    }
    float wk_even[4] = {0.f, 0.f, 0.f, 0.f};
    float kgv[4][PP];  // [channel][position]
#pragma unroll
    for (int i = 0; i < PP; ++i) {
      const int t = part * PP + i;
      const int o = sw16<kHalf>(t, c4);
      const float kv[4] = {__uint_as_float(kq[i].x << 16), __uint_as_float(kq[i].x & 0xffff0000u),
                           __uint_as_float(kq[i].y << 16), __uint_as_float(kq[i].y & 0xffff0000u)};
      const float qv[4] = {__uint_as_float(qq[i].x << 16), __uint_as_float(qq[i].x & 0xffff0000u),
                           __uint_as_float(qq[i].y << 16), __uint_as_float(qq[i].y & 0xffff0000u)};
      float kr[4], qr[4], kf[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float Rt = __expf(gm[i][jj] - rho[jj]), Ft = __builtin_amdgcn_rcpf(Rt);  // Rt >= e^-80
        kr[jj] = kv[jj] * Rt;
        qr[jj] = qv[jj] * Rt;
        kf[jj] = kv[jj] * Ft;
        kgv[jj][i] = kf[jj] * G[jj];
        if (i & 1) wkp[hf][jj][i >> 1] = pack_bf16x2(wk_even[jj], kr[jj] * E[jj]);
        else wk_even[jj] = kr[jj] * E[jj];
      }
      *reinterpret_cast<uint2*>(&sm.u.t.k[o]) = uint2{pack_bf16x2(kr[0], kr[1]), pack_bf16x2(kr[2], kr[3])};
      *reinterpret_cast<uint2*>(&sm.u.t.q[o]) = uint2{pack_bf16x2(qr[0], qr[1]), pack_bf16x2(qr[2], qr[3])};
      *reinterpret_cast<uint2*>(&sm.u.t.kf[o]) = uint2{pack_bf16x2(kf[0], kf[1]), pack_bf16x2(kf[2], kf[3])};
      const u32x2 qs = {pack_bf16x2(qr[0] * sE[0], qr[1] * sE[1]), pack_bf16x2(qr[2] * sE[2], qr[3] * sE[3])};
      __builtin_amdgcn_raw_buffer_store_b64(qs, rqg, rec_elem<K>(t, qcol) * 2, 0, 0);
    }
    {
      // (K o e^{gl - gam})^T: the 4 positions are 8 contiguous bytes of the
      // permuted order.
      const int tp = part * PP;
      const int pin = tp & 31;
      const int slot0 = pin < 16 ? 2 * pin : 2 * (pin - 16) + 4;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const u32x2 v = {pack_bf16x2(kgv[jj][0], kgv[jj][1]), pack_bf16x2(kgv[jj][2], kgv[jj][3])};
        __builtin_amdgcn_raw_buffer_store_b64(v, rkg, rec_elem<C>(cg4 + jj, 32 * (tp >> 5) + slot0) * 2, 0, 0);
      }
    }
    lds_barrier();
    // ---- A and P over the half's channels, accumulated --------------------
#pragma unroll
    for (int bi = 0; bi < 3; ++bi) {
      const int I = blocks[w][bi][0], J = blocks[w][bi][1];
      if (I >= 0) {  // wave-uniform
        const float* cv = sm.x + XL::cij + (I * (I + 1) / 2 + J) * kHalf;
        bf16x8 ak[kHalf / 32], aq[kHalf / 32], b[kHalf / 32];
#pragma unroll
        for (int kb = 0; kb < kHalf / 32; ++kb) {
          const int c0 = 32 * kb + 8 * g;
          ak[kb] = lds_frag(&sm.u.t.k[sw16<kHalf>(16 * I + m, c0)]);
          aq[kb] = lds_frag(&sm.u.t.q[sw16<kHalf>(16 * I + m, c0)]);
          b[kb] = lds_frag(&sm.u.t.kf[sw16<kHalf>(16 * J + m, c0)]);
        }
        if (J < I) {
#pragma unroll
          for (int kb = 0; kb < kHalf / 32; ++kb) {
            const f32x4 c0v = *reinterpret_cast<const f32x4*>(cv + 32 * kb + 8 * g);
            const f32x4 c1v = *reinterpret_cast<const f32x4*>(cv + 32 * kb + 8 * g + 4);
            float sc[8];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) sc[jj] = static_cast<float>(b[kb][jj]) * (jj < 4 ? c0v[jj] : c1v[jj - 4]);
            b[kb] = to_bf16x8(sc);
          }
        }
#pragma unroll
        for (int kb = 0; kb < kHalf / 32; ++kb) {
          dA[bi] = mfma16(ak[kb], b[kb], dA[bi]);
          dPt[bi] = mfma16(b[kb], aq[kb], dPt[bi]);
        }
      }
    }
  }
  if (tid == 0) *flag = 0;

  // ---- A^T into at, scale P into the record -------------------------------
  {
    const __amdgpu_buffer_rsrc_t rpm = make_rsrc(rec + R::Pm, static_cast<uint32_t>(C * C * 2));
#pragma unroll
    for (int bi = 0; bi < 3; ++bi) {
      const int I = blocks[w][bi][0], J = blocks[w][bi][1];
      if (I >= 0) {
        float bt[4];  // beta of the lane's rows (on the diagonal of at)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) bt[jj] = sm.at[sw32<C>(16 * I + 4 * g + jj, 16 * I + 4 * g + jj)];
        const int s2 = 16 * J + m;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int row = 16 * I + 4 * g + jj;
          sm.at[sw32<C>(s2, row)] = s2 == row ? bt[jj] : bt[jj] * dA[bi][jj];
        }
        const int prow = 16 * I + m;
        float pv[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) pv[jj] = 16 * J + 4 * g + jj <= prow ? p.scale * dPt[bi][jj] : 0.f;
        const u32x2 v = {pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])};
        __builtin_amdgcn_raw_buffer_store_b64(v, rpm, rec_elem<C>(prow, 32 * (J >> 1) + 8 * g + 4 * (J & 1)) * 2, 0, 0);
      }
    }
    if (w == 3) {
      const u32x2 z = {0u, 0u};
      __builtin_amdgcn_raw_buffer_store_b64(z, rpm, rec_elem<C>(m, 8 * g + 4) * 2, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b64(z, rpm, rec_elem<C>(32 + m, 32 + 8 * g + 4) * 2, 0, 0);
    }
  }
  // v for the U phase, fetched now so its latency hides behind the inverse.
  constexpr int NBU = (V / 16 + 3) / 4;
  static_assert(V / 16 <= 4 * NBU && V / 16 > 4 * (NBU - 1), "every wave has NBU column blocks");
  uint16_t vpre[NBU][2][8];
  {
    const int vlane = (2 * H * K + h * V + m) * 2 + 8 * g * rs;
#pragma unroll
    for (int u = 0; u < NBU; ++u)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int nb = w + 4 * u;
          vpre[u][kb][jj] = __builtin_amdgcn_raw_buffer_load_b16(rq, vlane + 32 * nb, (32 * kb + jj) * rs, 0);
        }
  }
  lds_barrier();  // A^T complete; tiles and x no longer read

  float* beta_l = sm.x;
  if (tid < C) beta_l[tid] = beta_t;
  uint16_t* wkt = sm.u.wkt;
  // (K o e^gam)^T: 8 bytes (4 positions) per channel and half.
#pragma unroll
  for (int hf = 0; hf < NH; ++hf)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      *reinterpret_cast<uint2*>(wkt + rec_elem<C>(kHalf * hf + c4 + jj, part * PP)) = uint2{wkp[hf][jj][0], wkp[hf][jj][1]};

  intra_inverse_wu<K, V>(p, sm.at, wkt, beta_l, vpre, rec, w, lane);
}

template <int K, int V>
__global__ __launch_bounds__(kThreads, 3) void chunk_intra_kernel(const PrefillParams p,
                                                                  const int4* chunk_info,
                                                                  char* recs, uint8_t* exact_flags) {
  intra_factored<K, V>(p, chunk_info, recs, exact_flags);
}

template <int K, int V>
__global__ __launch_bounds__(kThreads, 2) void chunk_intra_exact_kernel(const PrefillParams p,
                                                                        const int4* chunk_info,
                                                                        char* recs, uint8_t* exact_flags) {
  intra_exact<K, V>(p, chunk_info, recs, exact_flags);
}



// --------------------------------------------------------------- state --

// The LDS image of one record: the record's first lds_part bytes, byte for
// byte (tiles swizzled as written by the intra kernel).
template <int K, int V>
struct StateBuf {
  uint16_t wn[C * K];
  uint16_t qg[C * K];
  uint16_t pm[C * C];
  uint16_t kgt[K * C];
  float eg[K];
};

// Copy `Bytes` bytes (whole 16-byte pieces) from `src` to LDS at `dst` by
// buffer-to-LDS DMA: lane l of a wave writes its 16 bytes at the wave's LDS
// base + 16 l, so slot i takes piece i. Nothing passes through registers and
// no per-lane address math is needed; the copy runs until the next vmcnt
// wait. `wave` is the wave index in a scalar register.
template <int Bytes, int NT>
__device__ __forceinline__ void dma_copy(const char* src, void* dst_lds, int tid, int wave) {
  static_assert(Bytes % 16 == 0, "whole 16-byte pieces");
  constexpr int total = Bytes / 16;
  constexpr int full = total / NT, rem = total % NT;
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(src, static_cast<uint32_t>(Bytes));
  uint4* dst = reinterpret_cast<uint4*>(dst_lds) + wave * 64;
  const int voff = tid * 16;
#pragma unroll
  for (int r = 0; r < full; ++r)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, dst + r * NT, 16, voff, r * NT * 16, 0, 0);
  if constexpr (rem > 0) {
    // Only lanes whose slot lies inside the range take part (inactive lanes
    // write nothing).
    if (tid < rem)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, dst + full * NT, 16, voff, full * NT * 16, 0, 0);
  }
}

// Copy record `rec`'s LDS part into `b` with NT threads.
template <int K, int V, int NT>
__device__ __forceinline__ void dma_chunk(const char* rec, StateBuf<K, V>* b, int tid, int wave) {
  dma_copy<static_cast<int>(sizeof(StateBuf<K, V>)), NT>(rec, b, tid, wave);
}

// Output stores per lane per chunk: one 8-byte store per 16-position block.
constexpr int kOutStores = C / 16;

// Top of a chunk: this wave's copies and U loads for the chunk have landed
// (every vector-memory operation except the kOutStores output stores issued
// after them; they complete in order), its LDS reads are done, and all waves
// meet. Unlike __syncthreads this leaves the output stores in flight.
__device__ __forceinline__ void chunk_barrier() {
  static_assert(kOutStores < 16, "vmcnt field");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0070 | kOutStores);  // vmcnt = kOutStores, expcnt = 7, lgkmcnt = 0
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// NB = 2: the next chunk's record is copied into the second LDS buffer while
// the current one computes (one workgroup per CU at K = V = 128). NB = 1: one
// buffer, refilled once every wave has read it, so two workgroups share a CU
// and each one's copies overlap the other's MFMA phases; the host takes it
// when there are enough workgroups to give every CU two.
template <int K, int V, int NB>
__global__ __launch_bounds__(kThreads, NB == 1 ? 2 : 1) void chunk_state_kernel(const PrefillParams p,
                                                                                const SegPlan pl,
                                                                                const char* recs) {
  using R = Rec<K, V>;
  using B = StateBuf<K, V>;
  static_assert(sizeof(B) == R::lds_part, "LDS image is the record's first lds_part bytes");
  static_assert(R::lds_part % 16 == 0, "record LDS part must be whole 16-byte pieces");
  static_assert(NB == 1 || NB == 2, "one or two record buffers");
  constexpr int NVH = V / 64;  // workgroups per (segment, head): 64 columns each
  __shared__ B buf[NB];

  // The NVH workgroups of one (segment, head) read the same records: give
  // them indices that are equal modulo 8 so they run on the same XCD (one L2).
  // (Four waves per workgroup: every wave reads the whole of each record's
  // tiles from LDS, so more waves per workgroup would make LDS reads, not
  // the record copies, the bound.)
  const int bidx = blockIdx.x;
  int pair, vh;
  if constexpr (NVH == 2) {
    pair = (bidx / 16) * 8 + (bidx % 8);
    vh = (bidx / 8) % 2;
  } else {
    pair = bidx;
    vh = 0;
  }
  const int H = p.H;
  if (uniform(pl.counts[3]) == 0) return;  // cu_seqlens outside the contract
  const int gs = pair / H, h = pair % H;
  if (gs >= uniform(pl.counts[0])) return;
  // Records exist for at most max_chunks chunks (sized from the host's token
  // count); inconsistent cu_seqlens must not send us past them.
  if (pl.chunk_start[p.num_seqs] > max_chunks_for(p.num_tokens, p.num_seqs)) return;
  // Values loaded from wave-uniform addresses, kept in scalar registers.
  const int seq = uniform(pl.seg_seq[gs]);
  const int seg0 = uniform(pl.seg_start[seq]);
  const int nseg = uniform(pl.seg_start[seq + 1]) - seg0;
  const int sg = gs - seg0;
  const int cbase = uniform(pl.chunk_start[seq]);
  const int nch_seq = uniform(pl.chunk_start[seq + 1]) - cbase;
  const int seg_len = (nch_seq + nseg - 1) / nseg;
  const int cfirst = sg * seg_len;
  const int nch = min(nch_seq, cfirst + seg_len) - cfirst;
  const int c0 = cbase + cfirst;
  const bool last_seg = sg == nseg - 1;
  const int64_t bos = uniform(static_cast<int64_t>(p.cu_seqlens[seq]));
  const int64_t eos = uniform(static_cast<int64_t>(p.cu_seqlens[seq + 1]));
  if (nch <= 0 || eos > p.num_tokens || bos < 0) return;
  const int64_t tfirst = bos + static_cast<int64_t>(C) * cfirst;
  const int64_t tend = min<int64_t>(eos, tfirst + static_cast<int64_t>(C) * nch);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wave = uniform(w);
  const int m = lane & 15;
  const int g = lane >> 4;
  const int col0 = vh * 64 + 16 * w;
  const int64_t HV = static_cast<int64_t>(H) * V;

  const int64_t slot = uniform(static_cast<int64_t>(p.indices[static_cast<int64_t>(seq) * p.index_stride]));
  if (slot < 0) {
    // Null slot: zero output rows, no state traffic.
    for (int64_t t = tfirst; t < tend; ++t)
      if (tid < 64) p.out[t * HV + h * V + vh * 64 + tid] = 0;
    return;
  }

  float* st = p.pool + slot * p.slot_stride + static_cast<int64_t>(h) * K * V;
  // Every segment of a cut sequence starts from the copy of the slot's state
  // that the map pass made (the slot itself is written by the last segment
  // of this same launch); an uncut sequence from its slot.
  const int li = uniform(pl.seg_long[gs]);
  const float* s_in = li >= 0 ? pl.s0 + s0_index(h, li, pl) * K * V : st;
  const bool init = li >= 0 || p.has_initial_state == nullptr ||
                    uniform(static_cast<int32_t>(p.has_initial_state[seq])) != 0;
  // Without an initial state the range is empty and every load reads zero;
  // all loads are issued before the first use.
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(s_in, init ? static_cast<uint32_t>(K * V * 4) : 0u);
  f32x4 S[K / 16];
#pragma unroll
  for (int cb = 0; cb < K / 16; ++cb)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      S[cb][j] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(rs, ((16 * cb + 4 * g + j) * V + col0 + m) * 4, 0, 0));
  f32x4 Upre[4];
  auto rec_of = [&](int cc) {
    return recs + rec_index(h, c0 + cc, p) * static_cast<int64_t>(R::bytes);
  };
  // U fragments: lane's 16 bytes of tile (pb, col0 / 16) at a fixed offset.
  const int u_lane = ((col0 / 16) * 64 + lane) * 16;
  auto load_u = [&](int cc) {
    const __amdgpu_buffer_rsrc_t ru = make_rsrc(rec_of(cc) + R::Uf, static_cast<uint32_t>(C * V * 4));
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) Upre[pb] = buffer_load_f32x4<0>(ru, u_lane, pb * (V / 16) * 64 * 16);
  };
  // The first chunk's copy and U loads go out first, so the walk below
  // hides their latency.
  dma_chunk<K, V, kThreads>(rec_of(0), &buf[0], tid, wave);
  load_u(0);
  // Segment sg > 0 of a cut sequence walks the maps of the segments before
  // it: S <- M_j S + B_j. The wave holds all K rows of its 16 columns, so
  // two accumulator tiles form a bf16 B operand as in the chunk loop (the
  // contraction index permuted within each 32-block); lane (m, g)'s A
  // operand is then M[row m][32 kb + 4 g .. +3] and M[row m][32 kb + 16 +
  // 4 g .. +3], two float4s of the row-major fp32 M. Both operands are split
  // into bf16 hi + lo parts and the product is hi*hi + hi*lo + lo*hi (about
  // 16 significant bits, fp32 accumulation).
  if (li >= 0 && sg > 0) {
    const int mi0 = seg0 - seq;  // the sequence's first map item
    const int64_t item = static_cast<int64_t>(K) * K + static_cast<int64_t>(K) * V;
    constexpr int RT = K / 16, KB = K / 32;
    if constexpr (NB == 2) {
      // M goes through the idle second record buffer, 32 rows (two row
      // tiles) per stage, two stages in flight: the workgroup reads M from
      // L2 once instead of once per wave. Stage rows are stored with their
      // 16-byte pieces XOR-swizzled by the row (piece p of row r at p ^ (r &
      // 15)), so the 16 rows a fragment read touches fall in different banks.
      constexpr int QR = 32;                 // rows per stage
      constexpr int PPR = K / 4;             // 16-byte pieces per row
      constexpr int SBYTES = QR * K * 4;
      constexpr int SPS = K / QR;            // stages per map step
      static_assert(2 * SBYTES <= static_cast<int>(sizeof(B)), "two stages fit the idle buffer");
      static_assert((QR * PPR) % kThreads == 0, "whole DMA rounds");
      float* stage_buf = reinterpret_cast<float*>(&buf[1]);
      auto dma_stage = [&](int st) {  // stage st of the walk into its half of the buffer
        const float* M = pl.maps + map_index(h, mi0 + st / SPS, pl) * item + static_cast<int64_t>(st % SPS) * QR * K;
        const __amdgpu_buffer_rsrc_t rr = make_rsrc(M, static_cast<uint32_t>(SBYTES));
        uint4* dst = reinterpret_cast<uint4*>(stage_buf + (st & 1) * (SBYTES / 4));
#pragma unroll
        for (int r = 0; r < QR * PPR / kThreads; ++r) {
          const int ps = r * kThreads + tid;  // physical piece of the stage
          const int row = ps / PPR, pp = ps % PPR;
          const int pl = pp ^ (row & 15);     // logical piece stored there
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, dst + r * kThreads + (tid & ~63), 16,
                                                   (row * PPR + pl) * 16, 0, 0, 0);
        }
      };
      bf16x8 Sh[KB], Sl[KB];
      const int stages = sg * SPS;
      dma_stage(0);
      for (int st = 0; st < stages; ++st) {
        // Stage st has landed in every thread's pieces, and every wave is
        // done with the half stage st + 1 overwrites.
        wait_vmem();
        lds_barrier();
        if (st + 1 < stages) dma_stage(st + 1);
        const float* sb = stage_buf + (st & 1) * (SBYTES / 4);
        const float* Bm = pl.maps + map_index(h, mi0 + st / SPS, pl) * item + static_cast<int64_t>(K) * K;
        if (st % SPS == 0) {
          // Operands of this step: the state before it, as bf16 hi + lo.
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            Sh[kb] = pack_acc(S[2 * kb], S[2 * kb + 1]);
            Sl[kb] = pack_lo(S[2 * kb], S[2 * kb + 1], Sh[kb]);
          }
        }
#pragma unroll
        for (int t2 = 0; t2 < QR / 16; ++t2) {
          const int rt = (st % SPS) * (QR / 16) + t2;
          f32x4 acc;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) acc[jj] = Bm[(16 * rt + 4 * g + jj) * V + col0 + m];
          const float* row = sb + (16 * t2 + m) * K;
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            const f32x4 a0 = *reinterpret_cast<const f32x4*>(row + 4 * ((8 * kb + g) ^ m));
            const f32x4 a1 = *reinterpret_cast<const f32x4*>(row + 4 * ((8 * kb + 4 + g) ^ m));
            const bf16x8 ah = pack_acc(a0, a1);
            const bf16x8 al = pack_lo(a0, a1, ah);
            acc = mfma16(ah, Sh[kb], acc);
            acc = mfma16(ah, Sl[kb], acc);
            acc = mfma16(al, Sh[kb], acc);
          }
          // Row tile rt of the new state (the old tiles live on in Sh/Sl).
#pragma unroll
          for (int r2 = 0; r2 < RT; ++r2)
            if (r2 == rt) S[r2] = acc;
        }
      }
    } else {
      // Flattened over (step j, row tile rt); tile i + 1's operands are loaded
      // while tile i computes (the scheduling barriers keep that order).
      auto load_tile = [&](int i, f32x4 (&a)[KB][2], f32x4& b) {
        const float* M = pl.maps + map_index(h, mi0 + i / RT, pl) * item;
        const int rt = i % RT;
        const float* row = M + (16 * rt + m) * K + 4 * g;
  #pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          a[kb][0] = *reinterpret_cast<const f32x4*>(row + 32 * kb);
          a[kb][1] = *reinterpret_cast<const f32x4*>(row + 32 * kb + 16);
        }
        const float* Bm = M + static_cast<int64_t>(K) * K;
  #pragma unroll
        for (int jj = 0; jj < 4; ++jj) b[jj] = Bm[(16 * rt + 4 * g + jj) * V + col0 + m];
      };
      f32x4 a_cur[KB][2], a_nxt[KB][2], b_cur, b_nxt;
      bf16x8 Sh[KB], Sl[KB];
      load_tile(0, a_cur, b_cur);
      const int tiles = sg * RT;
      for (int i = 0; i < tiles; ++i) {
        const int rt = i % RT;
        if (rt == 0) {
          // Operands of this step: the state before it, as bf16 hi + lo.
  #pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            Sh[kb] = pack_acc(S[2 * kb], S[2 * kb + 1]);
            Sl[kb] = pack_lo(S[2 * kb], S[2 * kb + 1], Sh[kb]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (i + 1 < tiles) load_tile(i + 1, a_nxt, b_nxt);
        __builtin_amdgcn_sched_barrier(0);
        f32x4 acc = b_cur;
  #pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const bf16x8 ah = pack_acc(a_cur[kb][0], a_cur[kb][1]);
          const bf16x8 al = pack_lo(a_cur[kb][0], a_cur[kb][1], ah);
          acc = mfma16(ah, Sh[kb], acc);
          acc = mfma16(ah, Sl[kb], acc);
          acc = mfma16(al, Sh[kb], acc);
        }
        // Row tile rt of the new state (the old tiles live on in Sh/Sl).
  #pragma unroll
        for (int r2 = 0; r2 < RT; ++r2)
          if (r2 == rt) S[r2] = acc;
  #pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          a_cur[kb][0] = a_nxt[kb][0];
          a_cur[kb][1] = a_nxt[kb][1];
        }
        b_cur = b_nxt;
      }
    }
  }
  // Lane (m, g) of the transposed output tile of position block pb holds
  // channels col0 + 4 g .. + 3 of position 16 pb + m: 8 contiguous bytes.
  const int out_lane = static_cast<int>(m * HV + h * V + col0 + 4 * g) * 2;
  for (int cc = 0; cc < nch; ++cc) {
    const B& bf = buf[NB == 2 ? (cc & 1) : 0];
    // Chunk cc's buffer is complete once every wave's copy has landed; with
    // two buffers the barrier also means every wave is done with chunk
    // cc-1's buffer, which the next copy overwrites.
    chunk_barrier();
    f32x4 Vp[4];
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) Vp[pb] = Upre[pb];
    if (NB == 2 && cc + 1 < nch) {
      dma_chunk<K, V, kThreads>(rec_of(cc + 1), &buf[(cc + 1) & 1], tid, wave);
      load_u(cc + 1);
    }

    const int64_t t0 = tfirst + static_cast<int64_t>(C) * cc;
    const int n = static_cast<int>(min<int64_t>(C, eos - t0));

    // V' = U - W S (rows: positions) and O^T = S^T (Q o e^gam)^T (rows:
    // value channels), both contracting over key channels. S as a bf16
    // fragment is the B operand of the first and the A operand of the second.
    bf16x8 Sb[K / 32];
#pragma unroll
    for (int kb = 0; kb < K / 32; ++kb) Sb[kb] = pack_acc(S[2 * kb], S[2 * kb + 1]);
    // Fragments are read one position block ahead of the MFMAs that use
    // them (the scheduling barriers keep that order), so LDS latency hides
    // behind the previous block's MFMAs.
    bf16x8 wf[2][K / 32], qf[2][K / 32];
#pragma unroll
    for (int kb = 0; kb < K / 32; ++kb) {
      wf[0][kb] = frag<K>(bf.wn, m, 32 * kb + 8 * g);
      qf[0][kb] = frag<K>(bf.qg, m, 32 * kb + 8 * g);
    }
    bf16x8 pf[4][2];
    f32x4 Ot[4];
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
      __builtin_amdgcn_sched_barrier(0);
      if (pb + 1 < 4) {
#pragma unroll
        for (int kb = 0; kb < K / 32; ++kb) {
          wf[(pb + 1) & 1][kb] = frag<K>(bf.wn, 16 * (pb + 1) + m, 32 * kb + 8 * g);
          qf[(pb + 1) & 1][kb] = frag<K>(bf.qg, 16 * (pb + 1) + m, 32 * kb + 8 * g);
        }
      } else {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          pf[b][0] = frag<C>(bf.pm, 16 * b + m, 8 * g);
          if (b >= 2) pf[b][1] = frag<C>(bf.pm, 16 * b + m, 32 + 8 * g);
        }
      }
      Ot[pb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < K / 32; ++kb) {
        Vp[pb] = mfma16(wf[pb & 1][kb], Sb[kb], Vp[pb]);
        Ot[pb] = mfma16(Sb[kb], qf[pb & 1][kb], Ot[pb]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 kf[K / 16][2];
#pragma unroll
    for (int cb = 0; cb < K / 16; ++cb) {
      kf[cb][0] = frag<C>(bf.kgt, 16 * cb + m, 8 * g);
      kf[cb][1] = frag<C>(bf.kgt, 16 * cb + m, 32 + 8 * g);
    }
    // V' over positions: the output product takes it as hi + lo bf16 parts
    // (the rounding of V' would otherwise dominate the output error); the
    // state update takes the hi part.
    const bf16x8 Vb0 = pack_acc(Vp[0], Vp[1]);
    const bf16x8 Vb1 = pack_acc(Vp[2], Vp[3]);
    const bf16x8 Vl0 = pack_lo(Vp[0], Vp[1], Vb0);
    const bf16x8 Vl1 = pack_lo(Vp[2], Vp[3], Vb1);
    // O^T += V'^T P^T (P is lower triangular: positions 0..31 see only
    // positions 0..31).
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
      Ot[pb] = mfma16(Vb0, pf[pb][0], Ot[pb]);
      Ot[pb] = mfma16(Vl0, pf[pb][0], Ot[pb]);
      if (pb >= 2) {
        Ot[pb] = mfma16(Vb1, pf[pb][1], Ot[pb]);
        Ot[pb] = mfma16(Vl1, pf[pb][1], Ot[pb]);
      }
    }
    // Rows of the chunk as one buffer range: positions past its end fall
    // outside and their stores are dropped, so every lane issues exactly
    // kOutStores stores, the last vector-memory operations of the chunk.
    auto store_out = [&]() {
      const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.out + t0 * HV, static_cast<uint32_t>(n * HV * 2));
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) {
        const uint32_t lo = pack_bf16x2(Ot[pb][0], Ot[pb][1]);
        const uint32_t hi = pack_bf16x2(Ot[pb][2], Ot[pb][3]);
        typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo, hi}, ro, out_lane + static_cast<int>(16 * pb * HV * 2), 0, 0);
      }
    };
    if constexpr (NB == 2) store_out();
    // S <- diag(e^{gam_last}) S + (K o e^{gam_last - gam})^T V'.
#pragma unroll
    for (int cb = 0; cb < K / 16; ++cb) {
      const f32x4 e = *reinterpret_cast<const f32x4*>(&bf.eg[16 * cb + 4 * g]);
#pragma unroll
      for (int j = 0; j < 4; ++j) S[cb][j] *= e[j];
      S[cb] = mfma16(kf[cb][0], Vb0, S[cb]);
      S[cb] = mfma16(kf[cb][1], Vb1, S[cb]);
    }
    if constexpr (NB == 1) {
      // Every wave's reads of the buffer are done: refill it with the next
      // chunk, then store this chunk's output rows.
      if (cc + 1 < nch) {
        lds_barrier();
        dma_chunk<K, V, kThreads>(rec_of(cc + 1), &buf[0], tid, wave);
        load_u(cc + 1);
      }
      store_out();
    }
  }

  if (!last_seg) return;
#pragma unroll
  for (int cb = 0; cb < K / 16; ++cb)
#pragma unroll
    for (int j = 0; j < 4; ++j) st[(16 * cb + 4 * g + j) * V + col0 + m] = S[cb][j];
}

// ----------------------------------------------------------------- map --

// LDS image of the record parts the map pass reads: -W, and the
// contiguous (K o e^{gam_last - gam})^T and e^{gam_last}.
template <int K, int V>
struct MapBuf {
  uint16_t wn[C * K];
  uint16_t kgt[K * C];
  float eg[K];
};

// One workgroup per (map item, head, 64 columns of [M | B]), one 16-column
// MFMA tile per wave. (Two tiles per wave, each LDS fragment feeding two
// MFMAs, measured 5 % slower: half as many workgroups, each with longer
// chains per chunk.) Runs the chunk recurrence of one non-final segment
// (all of its chunks are full) from S = the identity's columns with U = 0
// (columns of M) or from S = 0 with the chunk's U (columns of B). There is
// no output; the rounding is the state pass's (bf16 S into W S, bf16 V' into
// the update, fp32 accumulation). Waves past column K + V only take part in
// the copies and barriers (K and V are multiples of 64, so a wave's columns
// all belong to M or all to B).
constexpr int kMapWaves = 4;
constexpr int kMapThreads = kMapWaves * 64;
constexpr int kMapCT = 1;  // 16-column tiles per wave

template <int K, int V>
__global__ __launch_bounds__(kMapThreads, 2) void chunk_map_kernel(const PrefillParams p,
                                                                   const SegPlan pl,
                                                                   const char* recs) {
  using R = Rec<K, V>;
  using B = MapBuf<K, V>;
  static_assert(R::Eg == R::KgT + static_cast<size_t>(K) * C * 2, "e^{gam_last} follows K^T in the record");
  static_assert(sizeof(B) == static_cast<size_t>(C) * K * 2 + static_cast<size_t>(K) * C * 2 + K * 4, "packed");
  constexpr int WCOLS = 16 * kMapCT;                                   // columns per wave
  constexpr int NW = (K + V + kMapWaves * WCOLS - 1) / (kMapWaves * WCOLS);  // workgroups per (item, head)
  constexpr int kKgtBytes = K * C * 2 + K * 4;
  __shared__ B buf[2];

  // The NW workgroups of one (item, head) read the same records: indices
  // equal modulo 8 put them on one XCD.
  const int bidx = blockIdx.x;
  const int pair = (bidx / (8 * NW)) * 8 + bidx % 8;
  const int sub = (bidx / 8) % NW;
  const int H = p.H;
  if (uniform(pl.counts[3]) == 0) return;
  const int mi = pair / H, h = pair % H;
  if (mi >= uniform(pl.counts[1])) return;
  if (pl.chunk_start[p.num_seqs] > max_chunks_for(p.num_tokens, p.num_seqs)) return;
  const int gs = uniform(pl.map_seg[mi]);
  const int seq = uniform(pl.seg_seq[gs]);
  const int seg0 = uniform(pl.seg_start[seq]);
  const int nseg = uniform(pl.seg_start[seq + 1]) - seg0;
  const int cbase = uniform(pl.chunk_start[seq]);
  const int nch_seq = uniform(pl.chunk_start[seq + 1]) - cbase;
  const int nch = (nch_seq + nseg - 1) / nseg;  // a non-final segment is full length
  const int c0 = cbase + (gs - seg0) * nch;
  const int64_t eos = uniform(static_cast<int64_t>(p.cu_seqlens[seq + 1]));
  if (eos > p.num_tokens) return;
  const int64_t slot = uniform(static_cast<int64_t>(p.indices[static_cast<int64_t>(seq) * p.index_stride]));
  if (slot < 0) return;  // a null slot carries no state

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wave = uniform(w);
  const int m = lane & 15;
  const int g = lane >> 4;
  const int gcol = sub * kMapWaves * WCOLS + WCOLS * wave;  // this wave's first column of [M | B]
  const bool active = gcol < K + V;
  const bool is_m = gcol < K;
  const int col0 = is_m ? gcol : gcol - K;

  f32x4 S[kMapCT][K / 16];
#pragma unroll
  for (int ct = 0; ct < kMapCT; ++ct)
#pragma unroll
    for (int cb = 0; cb < K / 16; ++cb)
#pragma unroll
      for (int j = 0; j < 4; ++j) S[ct][cb][j] = (is_m && 16 * cb + 4 * g + j == col0 + 16 * ct + m) ? 1.f : 0.f;

  auto rec_of = [&](int cc) {
    return recs + rec_index(h, c0 + cc, p) * static_cast<int64_t>(R::bytes);
  };
  auto dma = [&](int cc, B* b) {
    dma_copy<C * K * 2, kMapThreads>(rec_of(cc) + R::Wn, b->wn, tid, wave);
    dma_copy<kKgtBytes, kMapThreads>(rec_of(cc) + R::KgT, b->kgt, tid, wave);
  };
  f32x4 Upre[kMapCT][4];
  auto load_u = [&](int cc) {
    const __amdgpu_buffer_rsrc_t ru = make_rsrc(rec_of(cc) + R::Uf, static_cast<uint32_t>(C * V * 4));
#pragma unroll
    for (int ct = 0; ct < kMapCT; ++ct)
#pragma unroll
      for (int pb = 0; pb < 4; ++pb)
        Upre[ct][pb] = buffer_load_f32x4<0>(ru, (((col0 + 16 * ct) / 16) * 64 + lane) * 16, pb * (V / 16) * 64 * 16);
  };
  const bool takes_u = active && !is_m;
  // The first map item of a cut sequence copies the slot's initial state
  // (zero without one) for the state pass: its segments then never read the
  // slot that the last of them writes. The waves with columns of B cover
  // every value column once.
  if (takes_u && mi == seg0 - seq) {
    // Lane l copies 4 consecutive columns of the wave's WCOLS columns in
    // every 64 / (WCOLS / 4)-th row; every load is issued before the first
    // store.
    const int li = uniform(pl.seg_long[gs]);
    const bool init = p.has_initial_state == nullptr || uniform(static_cast<int32_t>(p.has_initial_state[seq])) != 0;
    const float* src = p.pool + slot * p.slot_stride + static_cast<int64_t>(h) * K * V;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, init ? static_cast<uint32_t>(K * V * 4) : 0u);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(pl.s0 + s0_index(h, li, pl) * K * V, static_cast<uint32_t>(K * V * 4));
    constexpr int LPR = WCOLS / 4;  // lanes per row
    constexpr int RPP = 64 / LPR;   // rows per pass
    static_assert(K % RPP == 0, "whole passes");
    const int lane_off = ((lane / LPR) * V + col0 + 4 * (lane % LPR)) * 4;
    f32x4 cp[K / RPP];
#pragma unroll
    for (int i = 0; i < K / RPP; ++i) cp[i] = buffer_load_f32x4<0>(rs, lane_off, i * RPP * V * 4);
#pragma unroll
    for (int i = 0; i < K / RPP; ++i) buffer_store_f32x4<0>(cp[i], rd, lane_off, i * RPP * V * 4);
  }
  dma(0, &buf[0]);
  if (takes_u) load_u(0);
  for (int cc = 0; cc < nch; ++cc) {
    const B& bf = buf[cc & 1];
    // Chunk cc's copy and U have landed in every wave, every wave's LDS
    // reads of chunk cc-1's buffer (which the next copy overwrites) are done,
    // and all waves meet.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt = 0, expcnt = 7, lgkmcnt = 0
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    f32x4 Vp[kMapCT][4];
#pragma unroll
    for (int ct = 0; ct < kMapCT; ++ct)
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) Vp[ct][pb] = is_m ? f32x4{0.f, 0.f, 0.f, 0.f} : Upre[ct][pb];
    if (cc + 1 < nch) {
      dma(cc + 1, &buf[(cc + 1) & 1]);
      if (takes_u) load_u(cc + 1);
    }
    if (!active) continue;
    // V' = U - W S over positions.
    bf16x8 Sh[kMapCT][K / 32];
#pragma unroll
    for (int ct = 0; ct < kMapCT; ++ct)
#pragma unroll
      for (int kb = 0; kb < K / 32; ++kb) Sh[ct][kb] = pack_acc(S[ct][2 * kb], S[ct][2 * kb + 1]);
    // Fragments are read one position block (or channel block) ahead of the
    // MFMAs that use them; the scheduling barriers keep that order, so LDS
    // latency hides behind the previous block's MFMAs.
    bf16x8 wf[2][K / 32];
#pragma unroll
    for (int kb = 0; kb < K / 32; ++kb) wf[0][kb] = frag<K>(bf.wn, m, 32 * kb + 8 * g);
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
      __builtin_amdgcn_sched_barrier(0);
      if (pb + 1 < 4) {
#pragma unroll
        for (int kb = 0; kb < K / 32; ++kb) wf[(pb + 1) & 1][kb] = frag<K>(bf.wn, 16 * (pb + 1) + m, 32 * kb + 8 * g);
      }
#pragma unroll
      for (int kb = 0; kb < K / 32; ++kb)
#pragma unroll
        for (int ct = 0; ct < kMapCT; ++ct) Vp[ct][pb] = mfma16(wf[pb & 1][kb], Sh[ct][kb], Vp[ct][pb]);
    }
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 Vb[kMapCT][2];
#pragma unroll
    for (int ct = 0; ct < kMapCT; ++ct) {
      Vb[ct][0] = pack_acc(Vp[ct][0], Vp[ct][1]);
      Vb[ct][1] = pack_acc(Vp[ct][2], Vp[ct][3]);
    }
    // S <- diag(e^{gam_last}) S + (K o e^{gam_last - gam})^T V'.
    bf16x8 kf[2][2];
    f32x4 ef[2];
    kf[0][0] = frag<C>(bf.kgt, m, 8 * g);
    kf[0][1] = frag<C>(bf.kgt, m, 32 + 8 * g);
    ef[0] = *reinterpret_cast<const f32x4*>(&bf.eg[4 * g]);
#pragma unroll
    for (int cb = 0; cb < K / 16; ++cb) {
      __builtin_amdgcn_sched_barrier(0);
      if (cb + 1 < K / 16) {
        kf[(cb + 1) & 1][0] = frag<C>(bf.kgt, 16 * (cb + 1) + m, 8 * g);
        kf[(cb + 1) & 1][1] = frag<C>(bf.kgt, 16 * (cb + 1) + m, 32 + 8 * g);
        ef[(cb + 1) & 1] = *reinterpret_cast<const f32x4*>(&bf.eg[16 * (cb + 1) + 4 * g]);
      }
#pragma unroll
      for (int ct = 0; ct < kMapCT; ++ct) {
#pragma unroll
        for (int j = 0; j < 4; ++j) S[ct][cb][j] *= ef[cb & 1][j];
        S[ct][cb] = mfma16(kf[cb & 1][0], Vb[ct][0], S[ct][cb]);
        S[ct][cb] = mfma16(kf[cb & 1][1], Vb[ct][1], S[ct][cb]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (!active) return;
  const int64_t item = map_index(h, mi, pl) * (static_cast<int64_t>(K) * K + static_cast<int64_t>(K) * V);
  float* dst = pl.maps + item + (is_m ? 0 : K * K);
  const int ld = is_m ? K : V;
#pragma unroll
  for (int ct = 0; ct < kMapCT; ++ct)
#pragma unroll
    for (int cb = 0; cb < K / 16; ++cb)
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[(16 * cb + 4 * g + j) * ld + col0 + 16 * ct + m] = S[ct][cb][j];
}

template <int K, int V>
hipError_t launch_kv(const PrefillParams& p, const Layout& L, const SegPlan& pl, uint8_t* exact_flags,
                     char* recs, hipStream_t stream, hipEvent_t after_intra) {
  const int64_t maxc = max_chunks_for(p.num_tokens, p.num_seqs);
  const int64_t intra_blocks = maxc * p.H;
  const int64_t seg_pairs = L.seg_bound * p.H;
  const int64_t state_blocks = (V / 64 == 2) ? (seg_pairs + 7) / 8 * 16 : seg_pairs;
  const int64_t map_blocks = (L.map_bound * p.H + 7) / 8 * 8 * ((K + V + 16 * kMapCT * kMapWaves - 1) / (16 * kMapCT * kMapWaves));
  if (intra_blocks > 0x7fffffff || state_blocks > 0x7fffffff || map_blocks > 0x7fffffff)
    return hipErrorInvalidValue;
  chunk_intra_kernel<K, V><<<dim3(static_cast<unsigned>(intra_blocks)), dim3(kThreads), 0, stream>>>(
      p, pl.chunk_info, recs, exact_flags);
  // With a lower bound lb every per-token log-decay lies in [lb, 0], so a
  // 16-row block decays by at most 15 |lb| and the factored kernel takes
  // every chunk once 15 |lb| <= kMaxBlockDecay: the exact kernel would only
  // read its flags and return.
  const bool all_factored = p.has_lb != 0 && 15.f * -p.lower_bound <= kMaxBlockDecay - 1.f;
  if (!all_factored)
    chunk_intra_exact_kernel<K, V><<<dim3(static_cast<unsigned>(intra_blocks)), dim3(kThreads), 0, stream>>>(
        p, pl.chunk_info, recs, exact_flags);
  if (after_intra != nullptr) {
    const hipError_t e = hipEventRecord(after_intra, stream);
    if (e != hipSuccess) return e;
  }
  if (L.map_bound > 0) {
    chunk_map_kernel<K, V><<<dim3(static_cast<unsigned>(map_blocks)), dim3(kMapThreads), 0, stream>>>(p, pl, recs);
  }
  // Every sequence is at least one segment: with enough of them for two
  // state workgroups per CU, one record buffer per workgroup lets two share
  // a CU.
  if (static_cast<int64_t>(p.num_seqs) * p.H * (V / 64) >= 2 * kChipSlots)
    chunk_state_kernel<K, V, 1><<<dim3(static_cast<unsigned>(state_blocks)), dim3(kThreads), 0, stream>>>(
        p, pl, recs);
  else
    chunk_state_kernel<K, V, 2><<<dim3(static_cast<unsigned>(state_blocks)), dim3(kThreads), 0, stream>>>(
        p, pl, recs);
  return hipGetLastError();
}

}  // namespace

size_t prefill_workspace_bytes(int32_t num_seqs, int64_t num_tokens, int32_t H, int32_t K,
                               int32_t V) {
  return layout_for(num_seqs, num_tokens, H, K, V).total;
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream, hipEvent_t after_intra) {
  const Layout L = layout_for(p.num_seqs, p.num_tokens, p.H, p.K, p.V);
  if (L.seg_bound > 0x7fffffff) return hipErrorInvalidValue;
  char* ws = static_cast<char*>(p.workspace);
  SegPlan pl;
  pl.chunk_start = reinterpret_cast<int32_t*>(ws + L.chunk_start);
  pl.seg_start = reinterpret_cast<int32_t*>(ws + L.seg_start);
  pl.counts = reinterpret_cast<int32_t*>(ws + L.counts);
  pl.seg_seq = reinterpret_cast<int32_t*>(ws + L.seg_seq);
  pl.seg_long = reinterpret_cast<int32_t*>(ws + L.seg_long);
  pl.map_seg = reinterpret_cast<int32_t*>(ws + L.map_seg);
  pl.maps = reinterpret_cast<float*>(ws + L.maps);
  pl.s0 = reinterpret_cast<float*>(ws + L.s0);
  pl.seg_bound = static_cast<int32_t>(L.seg_bound);
  pl.map_bound = static_cast<int32_t>(L.map_bound);
  pl.long_bound = static_cast<int32_t>(L.long_bound);
  pl.max_segs = static_cast<int32_t>(L.max_segs);
  pl.fill_units = static_cast<int32_t>(L.fill_units);
  pl.chunk_info = reinterpret_cast<int4*>(ws + L.chunk_info);
  pl.max_chunks = static_cast<int32_t>(max_chunks_for(p.num_tokens, p.num_seqs));
  pl.num_tokens = static_cast<int32_t>(p.num_tokens);
  uint8_t* flags = reinterpret_cast<uint8_t*>(ws + L.flags);
  char* recs = ws + L.recs;
  plan_kernel<<<1, kThreads, 0, stream>>>(p.cu_seqlens, p.num_seqs, pl);
  hipError_t e;
  if (p.K == 64 && p.V == 64) e = launch_kv<64, 64>(p, L, pl, flags, recs, stream, after_intra);
  else if (p.K == 64 && p.V == 128) e = launch_kv<64, 128>(p, L, pl, flags, recs, stream, after_intra);
  else if (p.K == 128 && p.V == 64) e = launch_kv<128, 64>(p, L, pl, flags, recs, stream, after_intra);
  else e = launch_kv<128, 128>(p, L, pl, flags, recs, stream, after_intra);
  // Output epilogue: a head's columns are spread over the state pass's waves
  // (and, at V = 128, over two workgroups), so the norm is a pass over the
  // output.
  if (e != hipSuccess || p.norm.gate == nullptr) return e;
  return launch_gated_rmsnorm(p.norm, p.out, p.num_tokens, p.H, p.V, stream);
}

}  // namespace kda
