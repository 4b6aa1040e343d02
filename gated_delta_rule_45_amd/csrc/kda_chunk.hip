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
// Fused design: one workgroup owns one (segment of a sequence, head) and all
// of its V value columns. For each chunk in order it builds the chunk's WY
// operands (gate scan, A, P, T, W, U: the "intra" part) in LDS and registers
// and then advances the state by them, writing the chunk's output. The
// operands never leave the workgroup, so the HBM traffic is the inputs read
// once, the outputs written once and the state read and written once; the
// next chunk's inputs are loaded while the current one computes.
//
// Launches on one stream, no host synchronisation:
//  1. plan:  validates cu_seqlens and splits long sequences into segments.
//  2. map:   (only when some sequence is cut) per non-final segment and head,
//            the affine map S_out = M S_in + B of the segment's chunks, with
//            the same per-chunk intra part (without the query operands).
//  3. scan:  (idem) per cut sequence and head, composes the maps in order
//            into every segment's initial state.
//  4. state: per segment and head: the segment's chunks from its initial
//            state, writing the outputs and (last segment) the final state.
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
#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// The launches of the exact path (kda_chunk_exact.hip): the map, scan and
// state kernels of a prefill whose gates may be steeper than the factored
// form allows, after the plan launch.
hipError_t launch_prefill_exact(const PrefillParams& p, hipStream_t stream);

namespace {

constexpr int C = 64;              // chunk size
constexpr int kWaves = 8;          // waves per fused workgroup (two per SIMD)
constexpr int kThreads = 64 * kWaves;
constexpr int kPlanThreads = 256;  // plan kernel

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
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

// Piece swizzle of the operand tiles the state step reads. A row of N bf16
// elements is N/8 16-byte pieces; piece p of row r is stored at piece
// p ^ swz<N>(r). MFMA fragments read 16 consecutive rows at one logical
// piece: the swizzle puts those 16 reads in 16 different 16-byte bank groups
// (and any 8 consecutive rows in 8), for 256-byte rows (r & 15) and for
// 128-byte rows, whose odd rows start half way round the banks
// (r ^ r >> 3) & 7.
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

// Element offsets in XOR-swizzled row-major LDS tiles of the intra part: the
// 16-byte pieces of row t are permuted by t, so the 16 rows an MFMA fragment
// touches fall in different banks.
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

// The thread index, hidden from the optimiser at each use. Inside the chunk
// loops every LDS and buffer address is a function of it; without this the
// compiler hoists all of those addresses out of the loop and keeps them live
// for its whole length, which runs the workgroup out of registers.
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  // The range survives, so divisions and remainders by powers of two stay
  // single shifts and masks.
  __builtin_assume(t >= 0 && t < kThreads);
  return t;
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// The words of the buffer resource make_rsrc builds, for the LDS copies
// below (wave-uniform: scalar registers).
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{static_cast<uint32_t>(uniform(static_cast<int32_t>(a))),
               static_cast<uint32_t>(uniform(static_cast<int32_t>(a >> 32))) & 0xffffu,
               static_cast<uint32_t>(uniform(static_cast<int32_t>(bytes))), 0x00020000u};
}

// Buffer-to-LDS copy of one 16-byte piece per lane: lane l's piece at byte
// offset voff + soff of the buffer lands at LDS byte lds_wave + 16 l
// (lds_wave and soff the same in every lane); offsets past the buffer's
// range land as zeros. The
// compiler is not told that this writes LDS: with the builtin form it makes
// the next LDS access of the wave wait until the copy has landed (it cannot
// tell the copy's tile from the others), which would serialise every
// prefetch. Each caller instead waits for its copies explicitly (vmcnt)
// before a barrier, ahead of any read of the tile, and issues them only
// after a barrier that ends every read of the tile's previous contents. M0
// is restored, so the compiler's own uses of it are unaffected.
__device__ __forceinline__ void lds_copy16(u32x4 rsrc, uint32_t lds_wave, int voff, uint32_t soff = 0) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_wave), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory");
}

// LDS byte address of a shared-memory pointer, read from lane 0.
__device__ __forceinline__ uint32_t lds_addr(const void* ptr) {
  return static_cast<uint32_t>(uniform(static_cast<int32_t>(reinterpret_cast<uintptr_t>(ptr))));
}

// Top of a chunk: this wave's vector-memory operations have completed except
// the last `Pending` (the previous chunk's output stores, issued after the
// loads of this chunk's inputs; they complete in issue order), its LDS
// operations are done, and all waves meet. Unlike __syncthreads this leaves
// the output stores in flight.
template <int Pending>
__device__ __forceinline__ void chunk_barrier() {
  static_assert(Pending >= 0 && Pending < 64, "vmcnt field");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0070 | (Pending & 15) | ((Pending >> 4) << 14));  // expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ------------------------------------------------------------- segments --
//
// The state pass carries one state per (sequence, head) through the
// sequence's chunks, so a long sequence is a chain of dependent steps on one
// workgroup. The chunk recurrence is affine in the state: after a run of
// chunks, S_out = M S_in + B with
//   M = prod_c (diag(e^{gam_last}) - (K o e^{gam_last - gam})^T W)   (K x K)
//   B = the state reached from S_in = 0                                (K x V)
// so a long sequence is cut into segments and run in two launches. The
// first runs segment 0's state pass (from the slot's state; its final state
// goes to B of map item 0) beside the maps (M, B) of segments 1 .. n - 2; the
// scan pass composes them in order into each later segment's initial state
// (S_{j+1} = M_j S_j + B_j, stored over B_j); the second launch runs the
// state pass of segments 1 .. n - 1 in parallel. Each launch has n - 1
// workgroups per cut (sequence, head).
//
// A sequence is cut into at most ceil(chunks / kSegMinChunks) segments of
// balanced lengths (they differ by at most one chunk; only the last chunk of
// the sequence may be partial, so every segment but the last is made of
// full chunks), into no more segments than it takes for the cut sequences'
// workgroups of one launch to occupy kChipSlots slots (one per compute
// unit: a workgroup's LDS takes most of a CU), and only into kMinCut
// segments or more without records: a map chunk costs about as much as a
// state chunk, so two segments would not shorten the chain. With records
// (the first launch keeps each chunk's operands for the second) two do.
constexpr int kSegMinChunks = 6;
constexpr int kMaxSegs = 16;
constexpr int kMinCut = 3;
constexpr int kChipSlots = 256;

// Device-side plan of one prefill call, written by plan_kernel. counts[0]
// is the call's status word (workspace offset 0): 0 when cu_seqlens keep to
// the contract, else KDA_PREFILL_BAD_CU_SEQLENS.
struct SegPlan {
  int32_t* counts;       // [4]: status, segments, maps, cut sequences
  int32_t* chunk_start;  // [N+1] first chunk of each sequence (in chunk units of the call)
  int32_t* seg_start;    // [N+1] first segment of each sequence
  int32_t* seg_seq;      // [seg_bound] sequence of each segment
  int32_t* seg_long;     // [seg_bound] index of a cut sequence among the cut ones, else -1
  int32_t* map_seg;      // [map_bound] segment of each map item (a non-final segment; the
                         // item of segment 0 runs that segment's state pass instead)
  int32_t* long_seq;     // [long_bound] sequence of each cut sequence
  float* maps;           // [H][map_bound]: M (as the scan's bf16 hi and lo A fragments, the
                         // size of fp32 [K][K]) then B (fp32 [K][V]); B of map item j ends up
                         // holding the initial state of segment j + 1
  uint8_t* recs;         // [H][rec_bound] chunk records (records mode only)
  int32_t seg_bound, map_bound, long_bound;
  int32_t rec_bound;     // chunk slots of the call at most
  int32_t max_segs;      // segments per sequence at most (host bound)
  int32_t num_tokens;    // rows of the call (validated to fit in int32)
  int32_t records;       // 1: the first launch writes chunk records, the second runs from them
};

constexpr int32_t kBadCuSeqlens = 1;

__device__ __forceinline__ int64_t map_index(int h, int mi, const SegPlan& pl) {
  return static_cast<int64_t>(h) * pl.map_bound + mi;
}

// Workspace layout (byte offsets) for one call's sizes. Bounds: a cut
// sequence of len tokens has fewer than len / (64 kSegMinChunks) non-final
// segments, so a call has at most num_tokens / (64 kSegMinChunks) of them
// (and at most num_seqs (max_segs - 1)); each cut sequence has at least one.
// The chunk records follow the maps; a workspace that ends before them
// (total_min bytes) runs without records.
struct Layout {
  int64_t seg_bound, map_bound, long_bound, max_segs, rec_bound;
  size_t counts, chunk_start, seg_start, seg_seq, seg_long, map_seg, long_seq, maps, total_min, recs, total;
};

inline size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// Bytes of one chunk record: -W, scale Q o e^gam, scale P, K~^T (bf16), e^{gam_last} (fp32 [K]), U (fp32 [C][V]).
__host__ __device__ constexpr size_t rec_bytes(int K, int V) {
  return static_cast<size_t>(C) * K * 2 * 2 + static_cast<size_t>(C) * C * 2 + static_cast<size_t>(K) * C * 2 +
         static_cast<size_t>(K) * 4 + static_cast<size_t>(C) * V * 4;
}

inline Layout layout_for(int32_t num_seqs, int64_t num_tokens, int32_t H, int32_t K, int32_t V) {
  Layout L{};
  const int64_t N = num_seqs;
  L.max_segs = std::min<int64_t>(kMaxSegs, (kChipSlots + H - 1) / H + 1);
  L.map_bound = L.max_segs < 2 ? 0 : std::min<int64_t>(num_tokens / (C * kSegMinChunks), N * (L.max_segs - 1));
  L.long_bound = L.map_bound;
  L.seg_bound = N + L.map_bound;
  size_t o = 0;
  L.counts = o;      o += 16;
  L.chunk_start = o; o += (N + 1) * 4;
  L.seg_start = o;   o += (N + 1) * 4;
  L.seg_seq = o;     o += L.seg_bound * 4;
  L.seg_long = o;    o += L.seg_bound * 4;
  L.map_seg = o;     o += L.map_bound * 4;
  L.long_seq = o;    o += L.long_bound * 4;
  L.maps = round256(o);
  L.total_min = L.maps + static_cast<size_t>(L.map_bound) * H * (static_cast<size_t>(K) * K + static_cast<size_t>(K) * V) * 4;
  // Records: one per chunk slot of a cut sequence (only those are written);
  // the chunk slots of a call number at most num_tokens / C + num_seqs.
  L.rec_bound = L.map_bound > 0 ? num_tokens / C + N : 0;
  L.recs = round256(L.total_min);
  L.total = L.recs + static_cast<size_t>(L.rec_bound) * H * rec_bytes(K, V);
  return L;
}

// ------------------------------------------------------------------ plan --

// Exclusive prefix sum of x over the workgroup (kPlanThreads threads, 64-lane
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
  for (int k = 0; k < kPlanThreads / 64; ++k) {
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

__device__ __forceinline__ int segments_of(int nch, int target, int min_cut) {
  const int ns = min((nch + kSegMinChunks - 1) / kSegMinChunks, target);
  return ns >= min_cut ? ns : 1;
}

#ifndef KDA_CHUNK_EXACT_PART
// Checks cu_seqlens (starts at 0, non-decreasing, ends at num_tokens) and
// plans chunks and segments of every sequence. The segment target is the
// number of segments each cut sequence needs for the cut sequences' n - 1
// workgroups per launch, with the uncut sequences' ones, to occupy the
// chip. With cu_seqlens outside the contract the status word
// is set and no segment exists: the state pass then writes NaN to every
// output row and touches no state.
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* cu, int32_t N, int32_t H, SegPlan pl) {
  __shared__ int part[kPlanThreads / 64];
  const int tid = threadIdx.x;
  const int per = (N + kPlanThreads - 1) / kPlanThreads;
  const int b = tid * per;
  const int e = min(N, b + per);
  // With records a second segment costs only its state steps in the second
  // launch, so two segments already shorten the chain.
  const int min_cut = pl.records ? 2 : kMinCut;
  int bad = 0, nl = 0, nw = 0;
  for (int i = b; i < e; ++i) {
    bad |= cu[i + 1] < cu[i];
    const int nch = chunks_of(cu, i);
    nl += nch > (min_cut - 1) * kSegMinChunks;  // can be cut
    nw += nch > 0 && nch <= (min_cut - 1) * kSegMinChunks;  // stays whole
  }
  if (tid == 0) bad |= cu[0] != 0 || cu[N] != pl.num_tokens;
  int nbad;
  block_exclusive_scan(bad, part, nbad);
  int n_long;
  block_exclusive_scan(nl, part, n_long);
  int n_whole;
  block_exclusive_scan(nw, part, n_whole);
  // Each launch holds a slot per (item, head); the uncut sequences' state
  // passes run in the second launch beside the later segments, so they take
  // slots from the cut sequences' budget there. Every cut sequence gets at
  // least min_cut segments. With records the first launch also holds the
  // last segment of every cut sequence (its records), so it has n workgroups
  // per cut (sequence, head) and the second one n - 1.
  const int slots = (kChipSlots + H - 1) / H;
  const int budget = slots - n_whole;
  const int per_long = max(min_cut - 1, budget / max(n_long, 1));
  const int target = pl.records ? min(pl.max_segs, max(min_cut, min(per_long + 1, slots / max(n_long, 1))))
                                : min(pl.max_segs, 1 + per_long);

  int cc = 0, sc = 0, lc = 0;
  for (int i = b; i < e; ++i) {
    const int nch = chunks_of(cu, i);
    const int ns = segments_of(nch, target, min_cut);
    cc += nch;
    sc += ns;
    lc += ns > 1;
  }
  int ctot, stot, ltot;
  int cb = block_exclusive_scan(cc, part, ctot);
  int sb = block_exclusive_scan(sc, part, stot);
  int lb = block_exclusive_scan(lc, part, ltot);
  const int mtot = stot - N;
  // The bounds hold for cu_seqlens that keep to the contract.
  const bool ok = nbad == 0 && stot <= pl.seg_bound && mtot <= pl.map_bound && ltot <= pl.long_bound;
  for (int i = b; i < e; ++i) {
    const int nch = chunks_of(cu, i);
    const int ns = segments_of(nch, target, min_cut);
    pl.chunk_start[i] = cb;
    pl.seg_start[i] = sb;
    if (ok) {
      // Map items of sequence i start at sb - i (each earlier sequence has
      // one fewer than its segments); lb counts the earlier cut sequences.
      for (int s = 0; s < ns; ++s) {
        pl.seg_seq[sb + s] = i;
        pl.seg_long[sb + s] = ns > 1 ? lb : -1;
      }
      for (int s = 0; s + 1 < ns; ++s) pl.map_seg[sb - i + s] = sb + s;
      if (ns > 1) pl.long_seq[lb] = i;
    }
    cb += nch;
    sb += ns;
    lb += ns > 1;
  }
  if (tid == 0) {
    pl.chunk_start[N] = ctot;
    pl.seg_start[N] = stot;
    pl.counts[0] = ok ? 0 : kBadCuSeqlens;
    pl.counts[1] = ok ? stot : 0;
    pl.counts[2] = ok ? mtot : 0;
    pl.counts[3] = ok ? ltot : 0;
  }
}
#endif  // KDA_CHUNK_EXACT_PART

// ------------------------------------------------------- the intra part --

// Factored-path bound on a 16-row block's decay range: every factored
// operand then lies in [e^-80, e^80], inside bf16/fp32 range.
constexpr float kMaxBlockDecay = 80.f;

// Thread roles of the intra part: thread (q4, part) owns channels 4 q4 ..
// 4 q4 + 3 at positions part PP .. part PP + PP - 1, so its tile reads and
// writes are 8 bytes wide and wave w holds rows 8 w .. 8 w + 7, half of the
// 16-row block w / 2.
template <int K>
struct Roles {
  static constexpr int NQ = K / 4;              // channel quads
  static constexpr int NPART = kThreads / NQ;   // 16 at K = 128, 32 at K = 64
  static constexpr int PP = C / NPART;          // positions per thread: 4 or 2
  static constexpr int KP8 = K / 8;             // 16-byte pieces per bf16 row
  static constexpr int RW = C / kWaves;         // rows per wave
  static_assert(NPART * PP == C && (64 / NQ) * PP == RW && RW == 8, "a wave holds 8 consecutive rows");
};

// fp32 scratch of the intra part (in floats). The 16-row blocks of a chunk
// are factored against rho_I = gam just before block I (the sum of the log
// decays of rows 0 .. 16 I - 1; rho_0 = 0), which every thread can form from
// the gate scan's partial totals without another exchange.
template <int K>
struct XLayout {
  static constexpr int NP = Roles<K>::NPART;
  static constexpr int tot = 0;                              // [NPART][K] partial sums of the gate scan
  static constexpr int cij = tot + NP * K;                   // [10][K] e^{rho_I - rho_J}, J <= I
  static constexpr int drange = cij + 10 * K;                // [4] largest decay over a block (rho_I - gam(16 I + 15))
  static constexpr int beta = drange + 16;                   // [C] beta per position
  static constexpr int gconst = beta + C;                    // [K] dt_bias, then e^{A_log} (fixed per head)
  static constexpr int end = gconst + K + 4;
};

// Factor pairs (I, J), J <= I, in the order of x.cij: pair pr = I (I+1)/2 + J.
__device__ __forceinline__ void cij_pair(int pr, int& I, int& J) {
  I = pr < 1 ? 0 : pr < 3 ? 1 : pr < 6 ? 2 : 3;
  J = pr - I * (I + 1) / 2;
}

// Operand tiles the state (or map) step reads, built per chunk. The bf16
// tiles are swizzled (rec_elem) for fragment reads.
template <int K, bool Q>
struct ChunkOps {
  uint16_t wn[C * K];            // -W, channels permuted
  uint16_t qg[Q ? C * K : 8];    // scale Q o e^gam, channels permuted
  uint16_t pm[Q ? C * C : 8];    // scale P, positions permuted
  uint16_t kgt[K * C];           // (K o e^{gam_last - gam})^T, positions permuted
  float eg[K];                   // e^{gam_last}
};

// LDS of a fused workgroup. Q: the state kernel (query operands and
// output); EXACT: chunks whose 16-row blocks decay too steeply for the
// factored operands take the exact path (only launched when the gate's
// bound does not rule them out).
template <int K, bool Q, bool EXACT>
struct FusedSmem {
  struct {
    ChunkOps<K, Q> ops;
  } r;
  union {
    struct {                     // factored path: raw keys and queries (copied in), then K o R and Q o R; K o F
      uint16_t k[C * K];
      uint16_t q[Q ? C * K : 8];
      uint16_t kf[C * K];
    } f;
    struct {                     // exact path: raw keys and queries, gam
      uint16_t k[C * K];
      uint16_t q[Q ? C * K : 8];
      float gam[EXACT ? C * K : 4];
    } e;
    uint16_t wkt[K * C];         // (K o e^gam)^T, bf16 [K][C] (swz<C>), after A/P (EXACT)
  } t;
  // Without the exact path (K o e^gam)^T has its own area, so the next
  // chunk's keys and queries can be copied into the tile area right after A/P.
  uint16_t wkt_own[EXACT ? 8 : K * C];
  float at[C * C];               // A^T strictly above the diagonal, then T = (I+A)^{-1} below it
  float x[XLayout<K>::end];
  float nrm[Q ? C * 8 : 1];      // output epilogue: sum of squares of each position over each wave's columns
  __device__ uint16_t* wkt() {
    if constexpr (EXACT) return t.wkt;
    else return wkt_own;
  }
  // bf16 T diag(beta), [C][C] (rec_elem<C>), for the W and U products: built
  // after A/P over K o F (or gam), which A/P was the last to read.
  __device__ uint16_t* tf() { return t.f.kf; }
};

// Chunk records. When a sequence is cut into segments, the first launch
// builds the intra part of every chunk of segments 1 .. n - 2 anyway (for the
// segment maps); with records it also builds the last segment's chunks, and
// writes every such chunk's state-step operands to the workspace: the
// ChunkOps tiles byte for byte as they sit in LDS, then U (fp32, lane (m, g)
// of wave w holding rows 16 pb + 4 g + j of value columns 16 w + m, as 16
// bytes at piece (4 w + pb) 64 + lane). The second launch then runs
// segments 1 .. n - 1 from the records alone. Records are head-major ([H]
// [chunk slot]), so a workgroup reads one contiguous stream.
template <int K, int V>
struct Rec {
  static constexpr int kOps = static_cast<int>(sizeof(ChunkOps<K, true>));  // bytes of the operand tiles
  static constexpr int kPieces = kOps / 16;
  static constexpr int kRounds = (kPieces + kThreads - 1) / kThreads;       // 16-byte pieces per thread
  static constexpr int kBytes = kOps + C * V * 4;                           // one record
  static constexpr int kBuf = kRounds * kThreads * 16;                      // LDS per record buffer
  static_assert(kOps % 16 == 0, "whole 16-byte pieces");
};

// LDS of a state pass that runs from records: two record buffers (the DMA
// rounds land whole, so each buffer is rounded up to them) and the output
// epilogue's exchange.
template <int K, int V>
struct RecSmem {
  uint4 ops[2][Rec<K, V>::kBuf / 16];
  float nrm[C * 8];
  __device__ const ChunkOps<K, true>& buf(int b) const {
    return *reinterpret_cast<const ChunkOps<K, true>*>(&ops[b][0]);
  }
};

// One chunk's register-held inputs, loaded a chunk ahead.
template <int K, int V>
struct ChunkIn {
  static constexpr int PP = Roles<K>::PP;
  u32x2 rgw[PP];                      // raw_g of the thread's 4 channels at its PP positions
  uint32_t rb;                        // raw beta (bf16 bits, zero-extended) of position tid
  u32x2 zg[4];                        // output epilogue gate of the lane's output elements (state pass)
  uint32_t vpre[2][8];                // v operands of U (waves w < V / 16, zero-extended): lane (m, g) needs
                                      // v[32 kb + 8 g + j][16 w + m]
};

// Where one chunk's rows are: first token and token count (n <= 64).
struct ChunkPos {
  int64_t t0;
  int n;
};

// Issues the register loads of chunk (t0, n) that the gate scan consumes:
// raw_g and raw beta. Rows past the chunk end read zero (buffer range).
template <int K, int V>
__device__ __forceinline__ void load_chunk_gate_regs(const PrefillParams& p, int h, ChunkPos cp, ChunkIn<K, V>& in) {
  using Ro = Roles<K>;
  const int H = p.H;
  const int tid = opaque_tid();
  const int q4 = tid % Ro::NQ, part = tid / Ro::NQ;
  const int c4 = 4 * q4;
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.raw_g + cp.t0 * (H * K), static_cast<uint32_t>(cp.n * H * K * 2));
#pragma unroll
  for (int i = 0; i < Ro::PP; ++i)
    in.rgw[i] = __builtin_amdgcn_raw_buffer_load_b64(rg, ((part * Ro::PP + i) * H * K + h * K + c4) * 2, 0, 0);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.raw_beta + cp.t0 * H, static_cast<uint32_t>(cp.n * H * 2));
  in.rb = __builtin_amdgcn_raw_buffer_load_b16(rb, (tid * H + h) * 2, 0, 0);
}

// Issues the loads of the v operands of chunk (t0, n) (waves w < V / 16).
template <int K, int V>
__device__ __forceinline__ void load_chunk_v_regs(const PrefillParams& p, int h, ChunkPos cp, ChunkIn<K, V>& in) {
  const int H = p.H;
  const int tid = opaque_tid(), lane = tid & 63, w = uniform(tid >> 6);
  const int m = lane & 15, g = lane >> 4;
  if (w < V / 16) {  // wave-uniform
    const int rs = static_cast<int>(p.qkv_row_stride * 2);  // bytes per mixed_qkv row
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.qkv + cp.t0 * p.qkv_row_stride, static_cast<uint32_t>(cp.n * rs));
    const int vlane = (2 * H * K + h * V + 16 * w + m) * 2 + 8 * g * rs;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        in.vpre[kb][j] = __builtin_amdgcn_raw_buffer_load_b16(rv, vlane, (32 * kb + j) * rs, 0);
  }
}

// Sum of x over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lane groups of a
// wave), in every lane and in the same order everywhere: the row swaps
// v_permlane16_swap / v_permlane32_swap with both operands x leave x of
// the partner row (group) in the second result.
__device__ __forceinline__ float sum_lane_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Makes the registers of a tile array look freshly written (waiting for
// any loads into them to land, here).
template <int N>
__device__ __forceinline__ void pin_regs(f32x4 (&a)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(a[i][j]));
}

// Issues the loads of the output epilogue's gate for chunk (t0, n): lane
// (m, g) of wave w takes channels 16 w + 4 g .. + 3 of positions 16 pb + m
// (rows past the chunk end read zero). Issued at the top of the chunk, so
// the intra part hides their latency.
template <int K, int V>
__device__ __forceinline__ void load_chunk_norm_regs(const PrefillParams& p, int h, ChunkPos cp, ChunkIn<K, V>& in) {
  const int tid = opaque_tid(), lane = tid & 63, w = uniform(tid >> 6);
  const int m = lane & 15, g = lane >> 4;
  const int64_t grs = p.norm.gate_row_stride;
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(p.norm.gate + cp.t0 * grs, static_cast<uint32_t>(cp.n * grs * 2));
  const int zl = static_cast<int>(m * grs + h * V + 16 * w + 4 * g) * 2;
#pragma unroll
  for (int pb = 0; pb < 4; ++pb)
    in.zg[pb] = __builtin_amdgcn_raw_buffer_load_b64(rz, zl + static_cast<int>(16 * pb * grs * 2), 0, 0);
}

// Holds the v operands as the 16 registers their loads write, late in a
// chunk: without this the compiler pairs them into bf16x2 right after the
// loads, which makes the wave wait there for the loads to land.
template <int K, int V>
__device__ __forceinline__ void pin_v_regs(ChunkIn<K, V>& in) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int j = 0; j < 8; ++j) asm volatile("" : "+v"(in.vpre[kb][j]));
}

// The same for the gate inputs (raw_g, raw beta), so that the next gate
// scan does not wait on whatever memory operations precede it.
template <int K, int V>
__device__ __forceinline__ void pin_gate_regs(ChunkIn<K, V>& in) {
#pragma unroll
  for (int i = 0; i < Roles<K>::PP; ++i) {
    uint32_t a = in.rgw[i][0], b = in.rgw[i][1];
    asm volatile("" : "+v"(a), "+v"(b));
    in.rgw[i] = u32x2{a, b};
  }
  asm volatile("" : "+v"(in.rb));
}

// All register loads of chunk (t0, n).
template <int K, int V>
__device__ __forceinline__ void load_chunk_regs(const PrefillParams& p, int h, ChunkPos cp, ChunkIn<K, V>& in) {
  load_chunk_gate_regs<K, V>(p, h, cp, in);
  load_chunk_v_regs<K, V>(p, h, cp, in);
}

// Copies chunk (t0, n)'s keys (and queries when Q) into the tile area by
// buffer-to-LDS DMA, 16-byte pieces XOR-swizzled by the row (sw16<K>); rows
// past the chunk end read zero.
template <int K, bool Q>
__device__ __forceinline__ void dma_chunk_tiles(const PrefillParams& p, int h, ChunkPos cp, uint16_t* k_lds,
                                                uint16_t* q_lds) {
  using Ro = Roles<K>;
  const int tid = opaque_tid();
  const int64_t rs = p.qkv_row_stride * 2;
  const u32x4 rq = rsrc_words(p.qkv + cp.t0 * p.qkv_row_stride, static_cast<uint32_t>(cp.n * rs));
  constexpr int KPM = (Ro::KP8 > 16 ? 16 : Ro::KP8) - 1;
  static_assert((C * Ro::KP8) % kThreads == 0, "whole DMA rounds");
#pragma unroll
  for (int r = 0; r < C * Ro::KP8 / kThreads; ++r) {
    const int ps = r * kThreads + tid;          // physical piece in the tile
    const int t = ps / Ro::KP8;
    const int pl = (ps % Ro::KP8) ^ (t & KPM);  // logical piece stored there
    const int slot = r * kThreads + (tid & ~63);
    const int qoff = static_cast<int>(t * rs) + (h * K + pl * 8) * 2;
    if constexpr (Q) lds_copy16(rq, lds_addr(reinterpret_cast<uint4*>(q_lds) + slot), qoff);
    lds_copy16(rq, lds_addr(reinterpret_cast<uint4*>(k_lds) + slot), qoff + p.H * K * 2);
  }
}

// The head's gate constants (dt_bias per channel, then e^{A_log}) into
// x.gconst, once per workgroup, ahead of the first barrier of the chunk loop.
template <int K>
__device__ __forceinline__ void stage_gate_consts(const PrefillParams& p, int h, float* x) {
  const int tid = threadIdx.x;
  if (tid < K) x[XLayout<K>::gconst + tid] = p.dt_bias[h * K + tid];
  if (tid == K) x[XLayout<K>::gconst + K] = __expf(p.A_log[h]);
}

// Gate and cumulative log-decay of the chunk, in registers: gm[i][j] = gam
// at the thread's position i and channel j, gl[j] = gam_last of channel j,
// rho[j] = rho of the thread's block. Writes beta to x.beta, e^{gam_last} to
// ops.eg, the factors c_IJ to x.cij and the blocks' decay ranges to
// x.drange; returns whether every block's range is within kMaxBlockDecay
// (the same value in every thread). Only the partial totals are exchanged
// (one barrier); the other outputs become visible at the next barrier.
template <int K, int V, bool Q, bool EXACT>
__device__ __forceinline__ bool gate_scan(const PrefillParams& p, int n, const ChunkIn<K, V>& in,
                                          FusedSmem<K, Q, EXACT>& sm, float (&gm)[Roles<K>::PP][4],
                                          float (&gl)[4], float (&rho)[4]) {
  using Ro = Roles<K>;
  using XL = XLayout<K>;
  constexpr int PP = Ro::PP, NQ = Ro::NQ, NPART = Ro::NPART;
  constexpr int PB = NPART / 4;  // parts per 16-row block
  const int tid = opaque_tid(), w = uniform(tid >> 6);
  const int q4 = tid % NQ, part = tid / NQ;
  const int c4 = 4 * q4;
  float* x = sm.x;
  const float a_h = x[XL::gconst + K];
  const f32x4 dtb = *reinterpret_cast<const f32x4*>(&x[XL::gconst + c4]);
  const float beta_t = (tid < n) ? sigmoid_f32(bf16_to_f32(static_cast<uint16_t>(in.rb))) : 0.f;
  // The thread's PP x 4 log-decays, with the gate form chosen once (the
  // form is uniform), so the independent exponentials interleave.
  float gv[PP][4];
  auto gates = [&](auto lb_form) {
#pragma unroll
    for (int i = 0; i < PP; ++i) {
      const float rg4[4] = {__uint_as_float(in.rgw[i][0] << 16), __uint_as_float(in.rgw[i][0] & 0xffff0000u),
                            __uint_as_float(in.rgw[i][1] << 16), __uint_as_float(in.rgw[i][1] & 0xffff0000u)};
#pragma unroll
      for (int j = 0; j < 4; ++j) gv[i][j] = gate_log_decay(rg4[j], dtb[j], a_h, decltype(lb_form)::value, p.lower_bound);
    }
  };
  if (p.has_lb != 0) gates(std::true_type{});
  else gates(std::false_type{});
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < PP; ++i) {
    // Padded positions do not decay, so row 63 holds gam_last.
    const bool live = part * PP + i < n;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[j] += live ? gv[i][j] : 0.f;
      gm[i][j] = acc[j];
    }
  }
  *reinterpret_cast<f32x4*>(&x[XL::tot + part * K + c4]) = f32x4{acc[0], acc[1], acc[2], acc[3]};
  lds_barrier();  // partial totals visible
  // Prefix sums over the parts: before this thread's part, before each
  // block (rho_I), and the total (gam_last).
  float before[4] = {0.f, 0.f, 0.f, 0.f}, pb[5][4], run[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q2 = 0; q2 < NPART; ++q2) {
    if (q2 % PB == 0) {  // a block boundary: rho of block q2 / PB
#pragma unroll
      for (int j = 0; j < 4; ++j) pb[q2 / PB][j] = run[j];
    }
    if (q2 == part) {
#pragma unroll
      for (int j = 0; j < 4; ++j) before[j] = run[j];
    }
    const f32x4 tq = *reinterpret_cast<const f32x4*>(&x[XL::tot + q2 * K + c4]);
#pragma unroll
    for (int j = 0; j < 4; ++j) run[j] += tq[j];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) pb[4][j] = run[j];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    gl[j] = pb[4][j];
    rho[j] = pb[0][j];
  }
#pragma unroll
  for (int I = 1; I < 4; ++I)
    if ((w >> 1) == I) {
#pragma unroll
      for (int j = 0; j < 4; ++j) rho[j] = pb[I][j];
    }
#pragma unroll
  for (int i = 0; i < PP; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) gm[i][j] += before[j];
  if (tid < C) x[XL::beta + tid] = beta_t;
  if (part == 0)
    *reinterpret_cast<f32x4*>(&sm.r.ops.eg[c4]) = f32x4{__expf(gl[0]), __expf(gl[1]), __expf(gl[2]), __expf(gl[3])};
  // c_IJ of the thread's channels for one pair (I, J) per part.
  if (part < 10) {
    int I, J;
    cij_pair(part, I, J);
    float c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float rI = pb[0][j], rJ = pb[0][j];
#pragma unroll
      for (int b2 = 1; b2 < 4; ++b2) {
        if (I == b2) rI = pb[b2][j];
        if (J == b2) rJ = pb[b2][j];
      }
      c[j] = __expf(rI - rJ);
    }
    *reinterpret_cast<f32x4*>(&x[XL::cij + part * K + c4]) = f32x4{c[0], c[1], c[2], c[3]};
  }
  if constexpr (!EXACT) {
    return true;
  } else {
    // Each wave's lanes cover every channel: the largest range of each
    // block by a butterfly, identical in every wave.
    bool fast = true;
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      float d = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) d = fmaxf(d, pb[I][j] - pb[I + 1][j]);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) d = fmaxf(d, __shfl_xor(d, off));
      if (tid == 0) x[XL::drange + I] = d;
      fast = fast && d <= kMaxBlockDecay;
    }
    return fast;
  }
}

// Off-diagonal blocks of A and P: waves 4..7 take (1,0) and (3,2), (2,1)
// and (3,0), (2,0), (3,1); waves 0..3 take the diagonal block (w, w).
__device__ __forceinline__ void offdiag_block(int w, int bi, int& I, int& J) {
  if (bi == 1 && w >= 6) {
    I = J = -1;
    return;
  }
  if (w == 4) { I = bi ? 3 : 1; J = bi ? 2 : 0; }
  else if (w == 5) { I = bi ? 3 : 2; J = bi ? 0 : 1; }
  else if (w == 6) { I = 2; J = 0; }
  else { I = 3; J = 1; }
}

// 16x16x16 fp32 product on the 16x16x4 MFMA: a = X^T and b = Y in
// accumulator form (lane (m, g) element j holds row 4 g + j of column m)
// give X Y in accumulator form. Step kk pairs lane group g with contraction
// index 4 g + kk, so an accumulator tile is a B operand as it stands and the
// accumulator form of X^T is the A operand of X.
__device__ __forceinline__ f32x4 mm16(const f32x4& a, const f32x4& b) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) acc = mfma4(a[kk], b[kk], acc);
  return acc;
}

// s I + x for a 16x16 tile x in accumulator form.
__device__ __forceinline__ f32x4 add_identity(f32x4 x, float s, int m, int g) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (4 * g + j == m) x[j] += s;
  return x;
}

// (I + N)^{-1} of a strictly lower triangular 16x16 block N, from N and N^T
// in accumulator form. N is nilpotent (N^16 = 0), so the Neumann series
// stops and factors into
//   (I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8),
// five levels of fp32 MFMA products instead of a 16-step substitution.
__device__ __forceinline__ f32x4 unit_lower_inverse(const f32x4& n, const f32x4& nt, int m, int g) {
  const f32x4 n2 = mm16(nt, n), n2t = mm16(n, nt);
  // ((I - N)(I + N^2))^T = (I + N^2)^T (I - N)^T
  const f32x4 w1t = mm16(add_identity(n2, 1.f, m, g), add_identity(-nt, 1.f, m, g));
  const f32x4 n4 = mm16(n2t, n2), n4t = mm16(n2, n2t);
  const f32x4 n8 = mm16(n4t, n4);
  const f32x4 y = mm16(add_identity(n4t, 1.f, m, g), add_identity(n8, 1.f, m, g));  // (I + N^4)(I + N^8)
  return mm16(w1t, y);
}

// P's block of rows 0..31 x columns 32..63 lies above the diagonal and is
// never read or written by a chunk; it is zeroed once per workgroup so that
// the chunk records, which copy the tiles byte for byte, carry no stale LDS
// contents.
template <int K, bool Q>
__device__ __forceinline__ void zero_p_unread(ChunkOps<K, Q>& ops) {
  if constexpr (Q) {
    const int tid = threadIdx.x;
    if (tid < 128) *reinterpret_cast<uint4*>(&ops.pm[rec_elem<C>(tid >> 2, 32 + 8 * (tid & 3))]) = uint4{0u, 0u, 0u, 0u};
  }
}

// Zero P blocks above the diagonal that the state step reads: rows 0..15 x
// cols 16..31 and rows 32..47 x cols 48..63.
template <int K, bool Q>
__device__ __forceinline__ void zero_p_blocks(ChunkOps<K, Q>& ops, int m, int g) {
  *reinterpret_cast<u32x2*>(&ops.pm[rec_elem<C>(m, 8 * g + 4)]) = u32x2{0u, 0u};
  *reinterpret_cast<u32x2*>(&ops.pm[rec_elem<C>(32 + m, 32 + 8 * g + 4)]) = u32x2{0u, 0u};
}

// Factored path (every 16-row block decays by <= kMaxBlockDecay on every
// channel, always so with a lower bound >= -5): with rho_I = gam just before
// block I, e^{gam_t - gam_s} = R_t F_s c_IJ with R_t = e^{gam_t - rho_I},
// F_s = e^{rho_J - gam_s}, c_IJ = e^{rho_I - rho_J} <= 1. One elementwise
// pass writes K o R, Q o R and K o F tiles, scale Q o e^gam and
// (K o e^{gam_last - gam})^T; A and P then run on bf16 MFMA from the tiles.
// Waves 0..3 take the diagonal blocks and invert theirs in (I + A) at once
// (in registers, unit_lower_inverse), waves 4..7 the off-diagonal blocks.
// Leaves A^T (times beta) of the off-diagonal blocks strictly above the
// diagonal of at and the diagonal blocks of T below it, scale P in ops.pm,
// and K o e^gam of the thread's elements in wkp; ends with the workgroup met.
template <int K, int V, bool Q, bool EXACT>
__device__ __forceinline__ void intra_factored(const PrefillParams& p, FusedSmem<K, Q, EXACT>& sm,
                                               const float (&gm)[Roles<K>::PP][4], const float (&gl)[4],
                                               const float (&rho)[4], uint32_t (&wkp)[4][Roles<K>::PP / 2]) {
  using Ro = Roles<K>;
  using XL = XLayout<K>;
  constexpr int PP = Ro::PP, NQ = Ro::NQ;
  const int tid = opaque_tid(), lane = tid & 63, w = uniform(tid >> 6);
  const int m = lane & 15, g = lane >> 4;
  const int q4 = tid % NQ, part = tid / NQ;
  const int c4 = 4 * q4;
  float* x = sm.x;
  auto& ops = sm.r.ops;
  float E[4], sE[4], G[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    E[jj] = __expf(rho[jj]);
    sE[jj] = p.scale * E[jj];
    G[jj] = __expf(gl[jj] - rho[jj]);
  }
  const int r8 = (c4 & 31) >> 2;
  const int qcol = 32 * (c4 >> 5) + 8 * (r8 & 3) + 4 * (r8 >> 2);  // permuted slot of channel c4
  uint2 kq[PP], qq[PP];
#pragma unroll
  for (int i = 0; i < PP; ++i) {
    const int o = sw16<K>(part * PP + i, c4);
    kq[i] = *reinterpret_cast<const uint2*>(&sm.t.f.k[o]);
    if constexpr (Q) qq[i] = *reinterpret_cast<const uint2*>(&sm.t.f.q[o]);
  }
  float wk_even[4] = {0.f, 0.f, 0.f, 0.f};
  float kgv[4][PP];  // [channel][position]
#pragma unroll
  for (int i = 0; i < PP; ++i) {
    const int t = part * PP + i;
    const int o = sw16<K>(t, c4);
    const float kv[4] = {__uint_as_float(kq[i].x << 16), __uint_as_float(kq[i].x & 0xffff0000u),
                         __uint_as_float(kq[i].y << 16), __uint_as_float(kq[i].y & 0xffff0000u)};
    float Rt[4], kr[4], kf[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      Rt[jj] = __expf(gm[i][jj] - rho[jj]);
      const float Ft = __builtin_amdgcn_rcpf(Rt[jj]);  // Rt >= e^-80
      kr[jj] = kv[jj] * Rt[jj];
      kf[jj] = kv[jj] * Ft;
      kgv[jj][i] = kf[jj] * G[jj];
      if (i & 1) wkp[jj][i >> 1] = pack_bf16x2(wk_even[jj], kr[jj] * E[jj]);
      else wk_even[jj] = kr[jj] * E[jj];
    }
    *reinterpret_cast<uint2*>(&sm.t.f.k[o]) = uint2{pack_bf16x2(kr[0], kr[1]), pack_bf16x2(kr[2], kr[3])};
    *reinterpret_cast<uint2*>(&sm.t.f.kf[o]) = uint2{pack_bf16x2(kf[0], kf[1]), pack_bf16x2(kf[2], kf[3])};
    if constexpr (Q) {
      const float qv[4] = {__uint_as_float(qq[i].x << 16), __uint_as_float(qq[i].x & 0xffff0000u),
                           __uint_as_float(qq[i].y << 16), __uint_as_float(qq[i].y & 0xffff0000u)};
      float qr[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) qr[jj] = qv[jj] * Rt[jj];
      *reinterpret_cast<uint2*>(&sm.t.f.q[o]) = uint2{pack_bf16x2(qr[0], qr[1]), pack_bf16x2(qr[2], qr[3])};
      *reinterpret_cast<u32x2*>(&ops.qg[rec_elem<K>(t, qcol)]) =
          u32x2{pack_bf16x2(qr[0] * sE[0], qr[1] * sE[1]), pack_bf16x2(qr[2] * sE[2], qr[3] * sE[3])};
    }
  }
  // (K o e^{gl - gam})^T: the thread's PP positions are PP consecutive slots
  // of the permuted order (PP <= 4, aligned).
  {
    static_assert(PP == 4 || PP == 2, "positions per thread");
    const int tp = part * PP;
    const int slot0 = 32 * (tp >> 5) + perm_slot(tp & 31);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      uint16_t* dst = &ops.kgt[rec_elem<C>(c4 + jj, slot0)];
      if constexpr (PP == 4)
        *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(kgv[jj][0], kgv[jj][1]), pack_bf16x2(kgv[jj][2], kgv[jj][3])};
      else
        *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(kgv[jj][0], kgv[jj][1]);
    }
  }
  lds_barrier();
  // ---- A and P over all channels ----------------------------------------
  // Block (I, J): lane (m, g) holds rows 16 I + 4 g + j of column 16 J + m.
  // Diagonal block (I, I): A, A^T (for the inverse) and P^T. Every
  // fragment is read before the products (the scheduling barrier keeps the
  // reads together, so their latencies overlap).
  auto ap_diag = [&](int I, f32x4& dA, f32x4& dPt, f32x4& dAt) {
    constexpr int KB = K / 32;
    bf16x8 ak[KB], bk[KB], aq[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int c0 = 32 * kb + 8 * g;
      ak[kb] = lds_frag(&sm.t.f.k[sw16<K>(16 * I + m, c0)]);
      bk[kb] = lds_frag(&sm.t.f.kf[sw16<K>(16 * I + m, c0)]);
      if constexpr (Q) aq[kb] = lds_frag(&sm.t.f.q[sw16<K>(16 * I + m, c0)]);
    }
    __builtin_amdgcn_sched_barrier(0);
    dA = f32x4{0.f, 0.f, 0.f, 0.f};
    dPt = f32x4{0.f, 0.f, 0.f, 0.f};
    dAt = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      dA = mfma16(ak[kb], bk[kb], dA);
      dAt = mfma16(bk[kb], ak[kb], dAt);
      if constexpr (Q) dPt = mfma16(bk[kb], aq[kb], dPt);
    }
  };
  // Off-diagonal block (I, J), J < I: the B operand (K o F rows of block J)
  // scaled by c_IJ per channel. All reads first, as above.
  auto ap_off = [&](int I, int J, f32x4& dA, f32x4& dPt) {
    constexpr int KB = K / 32;
    const float* cv = x + XL::cij + (I * (I + 1) / 2 + J) * K;
    bf16x8 ak[KB], bk[KB], aq[KB];
    f32x4 cs[KB][2];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int c0 = 32 * kb + 8 * g;
      ak[kb] = lds_frag(&sm.t.f.k[sw16<K>(16 * I + m, c0)]);
      bk[kb] = lds_frag(&sm.t.f.kf[sw16<K>(16 * J + m, c0)]);
      cs[kb][0] = *reinterpret_cast<const f32x4*>(cv + c0);
      cs[kb][1] = *reinterpret_cast<const f32x4*>(cv + c0 + 4);
      if constexpr (Q) aq[kb] = lds_frag(&sm.t.f.q[sw16<K>(16 * I + m, c0)]);
    }
    __builtin_amdgcn_sched_barrier(0);
    dA = f32x4{0.f, 0.f, 0.f, 0.f};
    dPt = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      float sc[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) sc[jj] = static_cast<float>(bk[kb][jj]) * cs[kb][jj >> 2][jj & 3];
      const bf16x8 b = to_bf16x8(sc);
      dA = mfma16(ak[kb], b, dA);
      if constexpr (Q) dPt = mfma16(b, aq[kb], dPt);
    }
  };
  // A^T (times beta) of an off-diagonal block into at.
  auto store_a = [&](int I, int J, const f32x4& dA) {
    const int s2 = 16 * J + m;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int row = 16 * I + 4 * g + jj;
      sm.at[sw32<C>(s2, row)] = x[XL::beta + row] * dA[jj];
    }
  };
  // Scale P into ops.pm.
  auto store_p = [&](int I, int J, const f32x4& dPt) {
    if constexpr (Q) {
      const int prow = 16 * I + m;
      float pv[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) pv[jj] = 16 * J + 4 * g + jj <= prow ? p.scale * dPt[jj] : 0.f;
      *reinterpret_cast<u32x2*>(&ops.pm[rec_elem<C>(prow, 32 * (J >> 1) + 8 * g + 4 * (J & 1))]) =
          u32x2{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])};
    }
  };
  if (w < 4) {
    // Diagonal block: N = diag(beta) A below the diagonal, inverted in
    // registers; T_II goes strictly below the diagonal of at.
    f32x4 dA, dPt, dAt;
    ap_diag(w, dA, dPt, dAt);
    store_p(w, w, dPt);
    const float beta_m = x[XL::beta + 16 * w + m];
    const f32x4 beta_r = *reinterpret_cast<const f32x4*>(&x[XL::beta + 16 * w + 4 * g]);
    f32x4 n, nt;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      n[jj] = m < 4 * g + jj ? beta_r[jj] * dA[jj] : 0.f;   // N[4 g + jj][m]
      nt[jj] = 4 * g + jj < m ? beta_m * dAt[jj] : 0.f;     // N[m][4 g + jj]
    }
    const f32x4 tb = unit_lower_inverse(n, nt, m, g);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      if (4 * g + jj > m) sm.at[sw32<C>(16 * w + 4 * g + jj, 16 * w + m)] = tb[jj];
  } else {
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
      int I, J;
      offdiag_block(w, bi, I, J);
      if (I >= 0) {  // wave-uniform
        f32x4 dA, dPt;
        ap_off(I, J, dA, dPt);
        store_a(I, J, dA);
        store_p(I, J, dPt);
      }
    }
    if constexpr (Q) {
      if (w == kWaves - 1) zero_p_blocks<K, Q>(ops, m, g);
    }
  }
  lds_barrier();  // A^T and the diagonal blocks of T complete; the tiles are no longer read
}

// Exact path (some 16-row block decays by more than kMaxBlockDecay): gam in
// LDS, A and P by 16x16 blocks with a reference row per block: off-diagonal
// blocks and diagonal blocks with a small decay range on bf16 MFMA (every
// factor <= 1 or within e^{+-80}), the other diagonal blocks by 4-row
// sub-blocks (between them on bf16 MFMA against a reference row per pass,
// within them pairwise in fp32). Same outputs as intra_factored (with the
// same block split), diagonal inverses included.
template <int K, int V, bool Q, bool EXACT>
__device__ __forceinline__ void intra_exact(const PrefillParams& p, FusedSmem<K, Q, EXACT>& sm,
                                            const float (&gm)[Roles<K>::PP][4], const float (&gl)[4],
                                            uint32_t (&wkp)[4][Roles<K>::PP / 2]) {
  using Ro = Roles<K>;
  using XL = XLayout<K>;
  constexpr int PP = Ro::PP, NQ = Ro::NQ;
  const int tid = opaque_tid(), lane = tid & 63, w = uniform(tid >> 6);
  const int m = lane & 15, g = lane >> 4;
  const int q4 = tid % NQ, part = tid / NQ;
  const int c4 = 4 * q4;
  float* x = sm.x;
  auto& ops = sm.r.ops;
  float* gam = sm.t.e.gam;
#pragma unroll
  for (int i = 0; i < PP; ++i)
    *reinterpret_cast<f32x4*>(&gam[sw32<K>(part * PP + i, c4)]) = f32x4{gm[i][0], gm[i][1], gm[i][2], gm[i][3]};
  // Elementwise outputs of the thread's own elements, from gam in registers
  // (every factor <= 1): scale Q o e^gam and (K o e^{gl - gam})^T; the
  // stores of gam above drain meanwhile.
  {
    const int r8 = (c4 & 31) >> 2;
    const int qcol = 32 * (c4 >> 5) + 8 * (r8 & 3) + 4 * (r8 >> 2);  // permuted slot of channel c4
    float kgv[4][PP];  // [channel][position]
#pragma unroll
    for (int i = 0; i < PP; ++i) {
      const int t = part * PP + i;
      const int o = sw16<K>(t, c4);
      const uint2 kq = *reinterpret_cast<const uint2*>(&sm.t.e.k[o]);
      const float kf[4] = {__uint_as_float(kq.x << 16), __uint_as_float(kq.x & 0xffff0000u),
                           __uint_as_float(kq.y << 16), __uint_as_float(kq.y & 0xffff0000u)};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) kgv[jj][i] = kf[jj] * __expf(gl[jj] - gm[i][jj]);
      if constexpr (Q) {
        const uint2 qq = *reinterpret_cast<const uint2*>(&sm.t.e.q[o]);
        const float qf[4] = {__uint_as_float(qq.x << 16), __uint_as_float(qq.x & 0xffff0000u),
                             __uint_as_float(qq.y << 16), __uint_as_float(qq.y & 0xffff0000u)};
        float qg[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) qg[jj] = p.scale * qf[jj] * __expf(gm[i][jj]);
        *reinterpret_cast<u32x2*>(&ops.qg[rec_elem<K>(t, qcol)]) =
            u32x2{pack_bf16x2(qg[0], qg[1]), pack_bf16x2(qg[2], qg[3])};
      }
    }
    static_assert(PP == 4 || PP == 2, "positions per thread");
    const int tp = part * PP;
    const int slot0 = 32 * (tp >> 5) + perm_slot(tp & 31);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      uint16_t* dst = &ops.kgt[rec_elem<C>(c4 + jj, slot0)];
      if constexpr (PP == 4)
        *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(kgv[jj][0], kgv[jj][1]), pack_bf16x2(kgv[jj][2], kgv[jj][3])};
      else
        *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(kgv[jj][0], kgv[jj][1]);
    }
  }
  lds_barrier();  // gam visible
  // A and P by 16x16 blocks (I, J), J <= I. For block-row I the reference
  // row r = 16 I + 7 when the block decays by at most 80 on every channel:
  // then every factor fits bf16 and every product with s <= t equals
  // e^{gam_t - gam_s} <= 1. Otherwise reference 16 I for J < I (both
  // factors <= 1) and 4-row sub-blocks on the diagonal block (below).
  // A goes transposed into at (strictly above the diagonal); P into ops.pm
  // (positions permuted), including the zero blocks above the diagonal that
  // the state step reads.
  auto do_block = [&](int I, int J) {
    const bool fast = x[XL::drange + I] <= kMaxBlockDecay;  // uniform
    if (J < I || fast) {
      const int r = fast ? 16 * I + 7 : 16 * I;
      f32x4 dA = {0.f, 0.f, 0.f, 0.f}, dP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < K / 32; ++kb) {
        const int c0 = 32 * kb + 8 * g;
        const uint4 ka = *reinterpret_cast<const uint4*>(&sm.t.e.k[sw16<K>(16 * I + m, c0)]);
        const uint4 kbv = *reinterpret_cast<const uint4*>(&sm.t.e.k[sw16<K>(16 * J + m, c0)]);
        const f32x4 gt0 = *reinterpret_cast<const f32x4*>(&gam[sw32<K>(16 * I + m, c0)]);
        const f32x4 gt1 = *reinterpret_cast<const f32x4*>(&gam[sw32<K>(16 * I + m, c0 + 4)]);
        const f32x4 gr0 = *reinterpret_cast<const f32x4*>(&gam[sw32<K>(r, c0)]);
        const f32x4 gr1 = *reinterpret_cast<const f32x4*>(&gam[sw32<K>(r, c0 + 4)]);
        const f32x4 gs0 = *reinterpret_cast<const f32x4*>(&gam[sw32<K>(16 * J + m, c0)]);
        const f32x4 gs1 = *reinterpret_cast<const f32x4*>(&gam[sw32<K>(16 * J + m, c0 + 4)]);
        const uint32_t kaw[4] = {ka.x, ka.y, ka.z, ka.w};
        const uint32_t kbw[4] = {kbv.x, kbv.y, kbv.z, kbv.w};
        uint32_t qaw[4] = {0u, 0u, 0u, 0u};
        if constexpr (Q) {
          const uint4 qav = *reinterpret_cast<const uint4*>(&sm.t.e.q[sw16<K>(16 * I + m, c0)]);
          qaw[0] = qav.x; qaw[1] = qav.y; qaw[2] = qav.z; qaw[3] = qav.w;
        }
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
        if constexpr (Q) dP = mfma16(to_bf16x8(aq), b, dP);
      }
      // Lane holds rows 16 I + 4 g + j of column s = 16 J + m. Entries above
      // the diagonal are dropped (they may be huge or non-finite).
      const int s2 = 16 * J + m;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 16 * I + 4 * g + j;
        if (s2 < row) sm.at[sw32<C>(s2, row)] = x[XL::beta + row] * dA[j];
        if constexpr (Q)
          ops.pm[rec_elem<C>(row, 32 * (s2 >> 5) + perm_slot(s2 & 31))] = bf16_bits(s2 <= row ? p.scale * dP[j] : 0.f);
      }
    } else {
      // Diagonal block whose range exceeds kMaxBlockDecay, by 4-row
      // sub-blocks. Between sub-blocks on bf16 MFMA: pass a = 1..3 takes
      // reference row r = 16 I + 4 a, so rows t >= r carry e^{gam_t - gam_r}
      // and columns s < r carry e^{gam_r - gam_s}, both <= 1; the pass's
      // other rows and columns keep the unscaled (finite) keys and are
      // dropped.
      // Lane group g keeps the rows 4 g .. 4 g + 3 of pass g. Within a
      // sub-block pairwise in fp32: lane (sb, tt, ss) = (l / 16, l / 4 % 4,
      // l % 4) forms entry (4 sb + tt, 4 sb + ss) over every channel.
      f32x4 dA = {0.f, 0.f, 0.f, 0.f}, dP = {0.f, 0.f, 0.f, 0.f};
      const int tm = 16 * I + m;
#pragma unroll 1
      for (int a = 1; a < 4; ++a) {
        const int r = 16 * I + 4 * a;
        const bool below = m >= 4 * a;  // row m of the block is at or after r
        f32x4 pA = {0.f, 0.f, 0.f, 0.f}, pP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < K / 32; ++kb) {
          const int c0 = 32 * kb + 8 * g;
          const uint4 kv = *reinterpret_cast<const uint4*>(&sm.t.e.k[sw16<K>(tm, c0)]);
          const f32x4 gt0 = *reinterpret_cast<const f32x4*>(&gam[sw32<K>(tm, c0)]);
          const f32x4 gt1 = *reinterpret_cast<const f32x4*>(&gam[sw32<K>(tm, c0 + 4)]);
          const f32x4 gr0 = *reinterpret_cast<const f32x4*>(&gam[sw32<K>(r, c0)]);
          const f32x4 gr1 = *reinterpret_cast<const f32x4*>(&gam[sw32<K>(r, c0 + 4)]);
          const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w};
          uint32_t qw[4] = {0u, 0u, 0u, 0u};
          if constexpr (Q) {
            const uint4 qv = *reinterpret_cast<const uint4*>(&sm.t.e.q[sw16<K>(tm, c0)]);
            qw[0] = qv.x; qw[1] = qv.y; qw[2] = qv.z; qw[3] = qv.w;
          }
          float ak[8], aq[8], bk[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float d = (j < 4 ? gt0[j] : gt1[j - 4]) - (j < 4 ? gr0[j] : gr1[j - 4]);
            const float e = __expf(-fabsf(d));  // e^{gam_t - gam_r} on rows after r, e^{gam_r - gam_s} before
            const float kf = __uint_as_float(j & 1 ? (kw[j >> 1] & 0xffff0000u) : (kw[j >> 1] << 16));
            const float qf = __uint_as_float(j & 1 ? (qw[j >> 1] & 0xffff0000u) : (qw[j >> 1] << 16));
            ak[j] = below ? kf * e : kf;
            aq[j] = below ? qf * e : qf;
            bk[j] = below ? kf : kf * e;
          }
          const bf16x8 b = to_bf16x8(bk);
          pA = mfma16(to_bf16x8(ak), b, pA);
          if constexpr (Q) pP = mfma16(to_bf16x8(aq), b, pP);
        }
        if (g == a) {
          dA = pA;
          dP = pP;
        }
      }
      // Lane (m, g) holds rows 16 I + 4 g + j of column s = 16 I + m: the
      // sub-blocks before g from the passes, P's zeros after g.
      const int s2 = 16 * I + m;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 16 * I + 4 * g + j;
        if ((m >> 2) < g) sm.at[sw32<C>(s2, row)] = x[XL::beta + row] * dA[j];
        if constexpr (Q) {
          if ((m >> 2) != g)
            ops.pm[rec_elem<C>(row, 32 * (s2 >> 5) + perm_slot(s2 & 31))] = bf16_bits((m >> 2) < g ? p.scale * dP[j] : 0.f);
        }
      }
      const int tt = (lane >> 2) & 3, ss = lane & 3, sb = lane >> 4;
      const int rt = 16 * I + 4 * sb + tt, rsrc = 16 * I + 4 * sb + ss;
      float aw = 0.f, pw = 0.f;
#pragma unroll 2
      for (int c0 = 0; c0 < K; c0 += 8) {
        const uint4 kt = *reinterpret_cast<const uint4*>(&sm.t.e.k[sw16<K>(rt, c0)]);
        const uint4 ks = *reinterpret_cast<const uint4*>(&sm.t.e.k[sw16<K>(rsrc, c0)]);
        const f32x4 gt0 = *reinterpret_cast<const f32x4*>(&gam[sw32<K>(rt, c0)]);
        const f32x4 gt1 = *reinterpret_cast<const f32x4*>(&gam[sw32<K>(rt, c0 + 4)]);
        const f32x4 gs0 = *reinterpret_cast<const f32x4*>(&gam[sw32<K>(rsrc, c0)]);
        const f32x4 gs1 = *reinterpret_cast<const f32x4*>(&gam[sw32<K>(rsrc, c0 + 4)]);
        const uint32_t ktw[4] = {kt.x, kt.y, kt.z, kt.w};
        const uint32_t ksw[4] = {ks.x, ks.y, ks.z, ks.w};
        uint32_t qtw[4] = {0u, 0u, 0u, 0u};
        if constexpr (Q) {
          const uint4 qt = *reinterpret_cast<const uint4*>(&sm.t.e.q[sw16<K>(rt, c0)]);
          qtw[0] = qt.x; qtw[1] = qt.y; qtw[2] = qt.z; qtw[3] = qt.w;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          // gam is non-increasing, so for s <= t the exponent is <= 0; the
          // min only keeps the dropped s > t entries finite.
          const float d = fminf((j < 4 ? gt0[j] : gt1[j - 4]) - (j < 4 ? gs0[j] : gs1[j - 4]), 0.f);
          const float ke = __uint_as_float(j & 1 ? (ksw[j >> 1] & 0xffff0000u) : (ksw[j >> 1] << 16)) * __expf(d);
          aw = fmaf(__uint_as_float(j & 1 ? (ktw[j >> 1] & 0xffff0000u) : (ktw[j >> 1] << 16)), ke, aw);
          if constexpr (Q)
            pw = fmaf(__uint_as_float(j & 1 ? (qtw[j >> 1] & 0xffff0000u) : (qtw[j >> 1] << 16)), ke, pw);
        }
      }
      if (ss < tt) sm.at[sw32<C>(rsrc, rt)] = x[XL::beta + rt] * aw;
      if constexpr (Q)
        ops.pm[rec_elem<C>(rt, 32 * (rsrc >> 5) + perm_slot(rsrc & 31))] = bf16_bits(ss <= tt ? p.scale * pw : 0.f);
    }
  };
  if (w < 4) {
    do_block(w, w);
    // The block's A^T entries were written by this wave's own lanes: LDS
    // operations of one wave complete in order, so no barrier is needed.
    // N = diag(beta) A below the diagonal comes back in accumulator form
    // and is inverted in registers as on the factored path; T_II goes
    // strictly below the diagonal of at.
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt = 0
    __builtin_amdgcn_wave_barrier();
    f32x4 n, nt;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int r = 4 * g + jj;
      n[jj] = m < r ? sm.at[sw32<C>(16 * w + m, 16 * w + r)] : 0.f;    // N[r][m]
      nt[jj] = r < m ? sm.at[sw32<C>(16 * w + r, 16 * w + m)] : 0.f;   // N[m][r]
    }
    const f32x4 tb = unit_lower_inverse(n, nt, m, g);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      if (4 * g + jj > m) sm.at[sw32<C>(16 * w + 4 * g + jj, 16 * w + m)] = tb[jj];
  } else {
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
      int I, J;
      offdiag_block(w, bi, I, J);
      if (I >= 0) do_block(I, J);  // wave-uniform
    }
    if constexpr (Q) {
      if (w == kWaves - 1) zero_p_blocks<K, Q>(ops, m, g);
    }
  }
  // K o e^gam of this thread's channels and positions, from the tiles.
  float wk_even[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < PP; ++i) {
    const int t = part * PP + i;
    const uint2 kv = *reinterpret_cast<const uint2*>(&sm.t.e.k[sw16<K>(t, c4)]);
    const f32x4 gv = *reinterpret_cast<const f32x4*>(&gam[sw32<K>(t, c4)]);
    const float kf[4] = {__uint_as_float(kv.x << 16), __uint_as_float(kv.x & 0xffff0000u),
                         __uint_as_float(kv.y << 16), __uint_as_float(kv.y & 0xffff0000u)};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float val = kf[j] * __expf(gv[j]);
      if (i & 1) wkp[j][i >> 1] = pack_bf16x2(wk_even[j], val);
      else wk_even[j] = val;
    }
  }
  lds_barrier();  // A^T complete; the tiles and gam are no longer read
}

// The rest of T = (I + A)^{-1} (its diagonal blocks are in at already),
// as the bf16 tile of T diag(beta) (sm.tf()), then
// W = T diag(beta)(K o e^gam) (as -W into ops.wn) and
// U = T diag(beta) V (into registers of waves w < V / 16: lane (m, g) holds
// rows 16 pb + 4 g + j of value columns 16 w + m in U[pb]). Starts with
// K o e^gam of the thread's elements in wkp (written here to the wkt tile)
// and the v operands in `in`; ends with the workgroup met.
template <int K, int V, bool Q, bool EXACT>
__device__ __forceinline__ void intra_inverse_wu(FusedSmem<K, Q, EXACT>& sm,
                                                 const uint32_t (&wkp)[4][Roles<K>::PP / 2],
                                                 const ChunkIn<K, V>& in, f32x4 (&U)[4]) {
  using Ro = Roles<K>;
  using XL = XLayout<K>;
  constexpr int PP = Ro::PP, NQ = Ro::NQ;
  const int tid = opaque_tid(), lane = tid & 63, w = uniform(tid >> 6);
  const int m = lane & 15, g = lane >> 4;
  const int q4 = tid % NQ, part = tid / NQ;
  const int c4 = 4 * q4;
  float* at = sm.at;
  const float* beta_l = sm.x + XL::beta;
  uint16_t* wkt = sm.wkt();
  uint16_t* tf = sm.tf();
  // (K o e^gam)^T into its tile: PP positions of a channel are 2 PP
  // contiguous bytes.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (PP == 4)
      *reinterpret_cast<uint2*>(wkt + rec_elem<C>(c4 + j, part * PP)) = uint2{wkp[j][0], wkp[j][1]};
    else
      *reinterpret_cast<uint32_t*>(wkt + rec_elem<C>(c4 + j, part * PP)) = wkp[j][0];
  }

  // ---- off-diagonal blocks of T on fp32 MFMA, in one phase ----------------
  // For J < I, T_IJ = -T_II sum_{J <= L < I} A_IL T_LJ. Wave w < 6 computes
  // block (I, J) = (1,0), (2,1), (3,2), (2,0), (3,1), (3,0) and, in its
  // registers, the lower-order blocks that one needs (every wave forms them
  // with the same operations, so the copies agree). The 16x16x4 product
  // pairs lane group g of step kk with contraction index 4 g + kk, so an
  // accumulator tile (rows 4 g + j) is the B operand of the next product as
  // it stands: step kk takes its element j = kk.
  if (w < 6) {
    // Operand values are read unconditionally (all in bounds), pinned, and
    // only then selected: a read under a lane-dependent condition becomes a
    // branch that waits for it on the spot. Every operand of the wave's
    // chain is read first (only the MFMAs are then dependent).
    auto pin4 = [](float (&v)[4]) { asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3])); };
    // A-operand values of block (I, L), L < I, of A: A[16 I + m][16 L + 4 g + kk]
    // (at holds A^T above the diagonal; no mask needed off the diagonal).
    auto a_blk = [&](int I, int L, float (&a)[4]) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) a[kk] = at[sw32<C>(16 * L + 4 * g + kk, 16 * I + m)];
    };
    // Raw values of the diagonal block T_LL as an A operand (row m, column
    // 4 g + kk) and as a B operand (row 4 g + kk, column m).
    auto t_raw_a = [&](int L, float (&v)[4]) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) v[kk] = at[sw32<C>(16 * L + m, 16 * L + 4 * g + kk)];
    };
    auto t_raw_b = [&](int L, float (&v)[4]) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) v[kk] = at[sw32<C>(16 * L + 4 * g + kk, 16 * L + m)];
    };
    // Unit lower triangular selection of a raw diagonal-block value at local
    // (row r, column c); sgn = -1 negates (the minus sign of the recurrence).
    auto t_sel = [](float (&v)[4], bool as_a, int m_, int g_, float sgn) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int r = as_a ? m_ : 4 * g_ + kk, c = as_a ? 4 * g_ + kk : m_;
        v[kk] = sgn * (r > c ? v[kk] : (r == c ? 1.f : 0.f));
      }
    };
    auto mm = [&](const float (&a)[4], const float (&b)[4], f32x4 acc) {  // both from registers
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) acc = mfma4(a[kk], b[kk], acc);
      return acc;
    };
    auto mm_acc = [&](const float (&a)[4], const f32x4& y, f32x4 acc) {   // B operand an accumulator tile
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) acc = mfma4(a[kk], y[kk], acc);
      return acc;
    };
    const f32x4 z0 = {0.f, 0.f, 0.f, 0.f};
    int I, J;
    f32x4 t;
    if (w < 3) {  // the first sub-diagonal: T_{J+1,J} = -T_{J+1,J+1} A_{J+1,J} T_JJ
      J = w;
      I = w + 1;
      float aIJ[4], bJJ[4], nTII[4];
      a_blk(I, J, aIJ);
      t_raw_b(J, bJJ);
      t_raw_a(I, nTII);
      pin4(aIJ); pin4(bJJ); pin4(nTII);
      t_sel(bJJ, false, m, g, 1.f);
      t_sel(nTII, true, m, g, -1.f);
      t = mm_acc(nTII, mm(aIJ, bJJ, z0), z0);
    } else if (w < 5) {  // T_20 (w = 3) and T_31 (w = 4), through T_{J+1,J}
      J = w - 3;
      I = J + 2;
      float a10[4], bJJ[4], nT11[4], a20[4], a21[4], nT22[4];
      a_blk(J + 1, J, a10);
      t_raw_b(J, bJJ);
      t_raw_a(J + 1, nT11);
      a_blk(I, J, a20);
      a_blk(I, J + 1, a21);
      t_raw_a(I, nT22);
      pin4(a10); pin4(bJJ); pin4(nT11); pin4(a20); pin4(a21); pin4(nT22);
      t_sel(bJJ, false, m, g, 1.f);
      t_sel(nT11, true, m, g, -1.f);
      t_sel(nT22, true, m, g, -1.f);
      const f32x4 t_mid = mm_acc(nT11, mm(a10, bJJ, z0), z0);  // T_{J+1,J}
      t = mm_acc(nT22, mm_acc(a21, t_mid, mm(a20, bJJ, z0)), z0);
    } else {  // T_30, through T_10 and T_20
      I = 3;
      J = 0;
      float a10[4], b00[4], nT11[4], a20[4], a21[4], nT22[4], a30[4], a31[4], a32[4], nT33[4];
      a_blk(1, 0, a10);
      t_raw_b(0, b00);
      t_raw_a(1, nT11);
      a_blk(2, 0, a20);
      a_blk(2, 1, a21);
      t_raw_a(2, nT22);
      a_blk(3, 0, a30);
      a_blk(3, 1, a31);
      a_blk(3, 2, a32);
      t_raw_a(3, nT33);
      pin4(a10); pin4(b00); pin4(nT11); pin4(a20); pin4(a21);
      pin4(nT22); pin4(a30); pin4(a31); pin4(a32); pin4(nT33);
      t_sel(b00, false, m, g, 1.f);
      t_sel(nT11, true, m, g, -1.f);
      t_sel(nT22, true, m, g, -1.f);
      t_sel(nT33, true, m, g, -1.f);
      const f32x4 p20 = mm(a20, b00, z0), p30 = mm(a30, b00, z0);  // independent of the chain
      const f32x4 t10 = mm_acc(nT11, mm(a10, b00, z0), z0);
      const f32x4 t20 = mm_acc(nT22, mm_acc(a21, t10, p20), z0);
      t = mm_acc(nT33, mm_acc(a32, t20, mm_acc(a31, t10, p30)), z0);
    }
    // T_IJ diag(beta) in bf16 into the T tile (lane: rows 16 I + 4 g + j of
    // column 16 J + m).
    const float bc = beta_l[16 * J + m];
#pragma unroll
    for (int j = 0; j < 4; ++j) tf[rec_elem<C>(16 * I + 4 * g + j, 16 * J + m)] = bf16_bits(t[j] * bc);
  } else {
    // Waves 6 and 7: the diagonal blocks of T diag(beta) (blocks 2 (w - 6)
    // and 2 (w - 6) + 1, from at) and the zero blocks above the diagonal that
    // the products read, (0, 1) and (2, 3).
    float tv[2][4];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) tv[b][j] = at[sw32<C>(16 * (2 * (w - 6) + b) + 4 * g + j, 16 * (2 * (w - 6) + b) + m)];
    asm volatile("" : "+v"(tv[0][0]), "+v"(tv[0][1]), "+v"(tv[0][2]), "+v"(tv[0][3]));
    asm volatile("" : "+v"(tv[1][0]), "+v"(tv[1][1]), "+v"(tv[1][2]), "+v"(tv[1][3]));
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int I = 2 * (w - 6) + b;
      const float bc = beta_l[16 * I + m];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * g + j;
        const float v = r > m ? tv[b][j] : (r == m ? 1.f : 0.f);  // read above, selected here
        tf[rec_elem<C>(16 * I + r, 16 * I + m)] = bf16_bits(v * bc);
      }
    }
    const int zr = 32 * (w - 6) + (lane >> 1), zp = 4 * (w - 6) + 2 + (lane & 1);
    if (lane < 32) *reinterpret_cast<uint4*>(&tf[rec_elem<C>(zr, zp * 8)]) = uint4{0u, 0u, 0u, 0u};
  }
  lds_barrier();

  // ---- W = T diag(beta)(K o e^gam), U = T diag(beta) V on MFMA -----------
  // beta is folded into the fp32 columns of T before the bf16 cast, so V
  // enters the product exactly as given. T is lower triangular, so rows
  // 0..31 need only positions 0..31. Wave w takes channel block w of W and
  // value block w of U. Each block of the tile was written by the wave that
  // formed it.
  const bool does_w = w < K / 16, does_u = w < V / 16;  // wave-uniform
  if (does_w || does_u) {
    // Rows 16 pb + m of T diag(beta) at columns 32 kb + 8 g .. + 7 (rows
    // 0..31 need only columns 0..31).
    bf16x8 Tf[4][2];
#pragma unroll
    for (int pb = 0; pb < 4; ++pb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        if (kb == 0 || pb >= 2) Tf[pb][kb] = frag<C>(tf, 16 * pb + m, 32 * kb + 8 * g);
    // -W^T = -(K o e^gam)^T (T diag(beta))^T: the same fragments with the
    // operands swapped leave lane (m, g) four consecutive channels
    // 16 nb + 4 g .. +3 of position 16 pb + m, which are four consecutive
    // slots of the permuted channel order: one 8-byte store each.
    if (does_w) {
      const int nb = w;
      bf16x8 Bf[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) Bf[kb] = frag<C>(wkt, 16 * nb + m, 32 * kb + 8 * g);
      const int col = 32 * (nb >> 1) + 8 * g + 4 * (nb & 1);
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) {
        f32x4 D = mfma16(Bf[0], Tf[pb][0], f32x4{0.f, 0.f, 0.f, 0.f});
        if (pb >= 2) D = mfma16(Bf[1], Tf[pb][1], D);
        *reinterpret_cast<u32x2*>(&sm.r.ops.wn[rec_elem<K>(16 * pb + m, col)]) =
            u32x2{pack_bf16x2(-D[0], -D[1]), pack_bf16x2(-D[2], -D[3])};
      }
    }
    if (does_u) {
      bf16x8 Bv[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 8; ++j) Bv[kb][j] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(in.vpre[kb][j]));
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) {
        f32x4 D = mfma16(Tf[pb][0], Bv[0], f32x4{0.f, 0.f, 0.f, 0.f});
        if (pb >= 2) D = mfma16(Tf[pb][1], Bv[1], D);
        U[pb] = D;
      }
    }
  }
  lds_barrier();  // -W complete; at and wkt no longer read
}

// The whole intra part of one chunk whose inputs have landed (tiles in LDS,
// the rest in `in`): operand tiles in sm.r.ops, U in registers. With
// has_next (`next` the following chunk of the same workgroup), its raw_g and
// beta loads go out as soon as the gate scan has consumed this chunk's, and
// (without the exact path) its keys and queries as soon as A/P is done. Ends
// with the workgroup met and the tile area free.
template <int K, int V, bool Q, bool EXACT>
__device__ __forceinline__ void intra_part(const PrefillParams& p, int h, int n, ChunkIn<K, V>& in,
                                           bool has_next, ChunkPos next, FusedSmem<K, Q, EXACT>& sm,
                                           f32x4 (&U)[4]) {
  using Ro = Roles<K>;
  float gm[Ro::PP][4], gl[4], rho[4];
  const bool fast = gate_scan<K, V, Q, EXACT>(p, n, in, sm, gm, gl, rho);
  if (has_next) load_chunk_gate_regs<K, V>(p, h, next, in);
  uint32_t wkp[4][Ro::PP / 2];
  if (fast) intra_factored<K, V, Q, EXACT>(p, sm, gm, gl, rho, wkp);  // uniform
  else if constexpr (EXACT) intra_exact<K, V, Q, EXACT>(p, sm, gm, gl, wkp);
  // The tile area is free from here on (EXACT: after W, see the caller).
  if constexpr (!EXACT) {
    if (has_next) dma_chunk_tiles<K, Q>(p, h, next, sm.t.f.k, sm.t.f.q);
  }
  intra_inverse_wu<K, V, Q, EXACT>(sm, wkp, in, U);
}

// Which chunks a segment runs: from the plan, for segment gs of the call.
struct SegRange {
  int seq, seg0, nseg, sg, c0;  // c0: the segment's first chunk within its sequence
  int nch;
  int64_t bos, eos;             // the sequence's rows
};

__device__ __forceinline__ SegRange segment_range(const PrefillParams& p, const SegPlan& pl, int gs) {
  SegRange r;
  r.seq = uniform(pl.seg_seq[gs]);
  r.seg0 = uniform(pl.seg_start[r.seq]);
  r.nseg = uniform(pl.seg_start[r.seq + 1]) - r.seg0;
  r.sg = gs - r.seg0;
  const int nch_seq = uniform(pl.chunk_start[r.seq + 1]) - uniform(pl.chunk_start[r.seq]);
  // Balanced split: segment sg takes chunks [sg nch / nseg, (sg + 1) nch / nseg).
  r.c0 = r.sg * nch_seq / r.nseg;
  r.nch = (r.sg + 1) * nch_seq / r.nseg - r.c0;
  r.bos = uniform(static_cast<int64_t>(p.cu_seqlens[r.seq]));
  r.eos = uniform(static_cast<int64_t>(p.cu_seqlens[r.seq + 1]));
  return r;
}

__device__ __forceinline__ ChunkPos chunk_pos(const SegRange& r, int cc) {
  ChunkPos cp;
  cp.t0 = r.bos + static_cast<int64_t>(C) * (r.c0 + cc);
  cp.n = static_cast<int>(min<int64_t>(C, r.eos - cp.t0));
  return cp;
}

// --------------------------------------------------------------- state --

// With cu_seqlens outside the contract, every output row of the call is set
// to NaN (no state is touched); the workgroups share the rows.
__device__ __forceinline__ void poison_output(const PrefillParams& p) {
  const int64_t total = p.num_tokens * p.H * p.V;  // bf16 elements
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < total; i += stride)
    p.out[i] = 0x7FC0;  // bf16 quiet NaN
}

// One chunk's state step on the calling wave's value columns 16 w .. 16 w +
// 15 (w < V / 16): V' = U - W S, the chunk's output (with the optional
// gated RMSNorm epilogue) and S <- diag(e^{gam_last}) S + K~^T V', from the
// operand tiles `ops` and U in Vp. zg holds the epilogue's gate of the
// lane's output elements, nw its weights; nrm is the epilogue's LDS
// exchange (all waves of the workgroup take part in its barrier, see the
// callers). pin() runs just before the output stores.
template <int K, int V, typename Pin>
__device__ __forceinline__ void state_step(const PrefillParams& p, int h, int w, ChunkPos cp,
                                           const ChunkOps<K, true>& ops, float* nrm, f32x4 (&S)[K / 16],
                                           f32x4 (&Vp)[4], const u32x2 (&zg)[4], f32x4 nw, bool has_norm,
                                           Pin&& pin) {
  const int64_t HV = static_cast<int64_t>(p.H) * V;
  const int col0 = 16 * w;
  const int m = opaque_tid() & 15, g = (opaque_tid() & 63) >> 4;
  // Lane (m, g) of the transposed output tile of position block pb holds
  // channels col0 + 4 g .. + 3 of position 16 pb + m: 8 contiguous bytes.
  const int out_lane = static_cast<int>(m * HV + h * V + col0 + 4 * g) * 2;

  // V' = U - W S (rows: positions) and O^T = S^T (Q o e^gam)^T (rows:
  // value channels), both contracting over key channels. S as a bf16
  // fragment is the B operand of the first and the A operand of the
  // second.
  bf16x8 Sb[K / 32];
#pragma unroll
  for (int kb = 0; kb < K / 32; ++kb) Sb[kb] = pack_acc(S[2 * kb], S[2 * kb + 1]);
  // Fragments are read one position block ahead of the MFMAs that use
  // them (the scheduling barriers keep that order), so LDS latency hides
  // behind the previous block's MFMAs.
  bf16x8 wf[2][K / 32], qf[2][K / 32];
#pragma unroll
  for (int kb = 0; kb < K / 32; ++kb) {
    wf[0][kb] = frag<K>(ops.wn, m, 32 * kb + 8 * g);
    qf[0][kb] = frag<K>(ops.qg, m, 32 * kb + 8 * g);
  }
  bf16x8 pf[4][2];
  f32x4 Ot[4];
#pragma unroll
  for (int pb = 0; pb < 4; ++pb) {
    __builtin_amdgcn_sched_barrier(0);
    if (pb + 1 < 4) {
#pragma unroll
      for (int kb = 0; kb < K / 32; ++kb) {
        wf[(pb + 1) & 1][kb] = frag<K>(ops.wn, 16 * (pb + 1) + m, 32 * kb + 8 * g);
        qf[(pb + 1) & 1][kb] = frag<K>(ops.qg, 16 * (pb + 1) + m, 32 * kb + 8 * g);
      }
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        pf[b][0] = frag<C>(ops.pm, 16 * b + m, 8 * g);
        if (b >= 2) pf[b][1] = frag<C>(ops.pm, 16 * b + m, 32 + 8 * g);
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
  // outside and their stores are dropped, so every lane issues exactly 4
  // stores, the last vector-memory operations of the chunk.
  if (has_norm) {
    // Sum of squares of each position over the wave's 16 columns (lanes
    // m, m + 16, m + 32, m + 48 hold one position), posted per wave by
    // lanes 0..15.
    float ss[4];
#pragma unroll
    for (int pb = 0; pb < 4; ++pb)
      ss[pb] = sum_lane_groups(Ot[pb][0] * Ot[pb][0] + Ot[pb][1] * Ot[pb][1] + Ot[pb][2] * Ot[pb][2] +
                               Ot[pb][3] * Ot[pb][3]);
    if (g == 0) {
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) nrm[(16 * pb + m) * 8 + w] = ss[pb];
    }
    lds_barrier();
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(&nrm[(16 * pb + m) * 8]);
      float tot = a[0] + a[1] + a[2] + a[3];
      if constexpr (V / 16 > 4) {
        const f32x4 b = *reinterpret_cast<const f32x4*>(&nrm[(16 * pb + m) * 8 + 4]);
        tot += b[0] + b[1] + b[2] + b[3];
      }
      // Hardware reciprocal square root (about 1 ulp; the result is cast to bf16).
      const float inv = __builtin_amdgcn_rsqf(tot * (1.0f / V) + p.norm.eps);
      const float z[4] = {__uint_as_float(zg[pb][0] << 16), __uint_as_float(zg[pb][0] & 0xffff0000u),
                          __uint_as_float(zg[pb][1] << 16), __uint_as_float(zg[pb][1] & 0xffff0000u)};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float sg = sigmoid_f32(z[j]);
        const float act = p.norm.activation == 1 ? z[j] * sg : sg;
        Ot[pb][j] = Ot[pb][j] * inv * nw[j] * act;
      }
    }
  }
  // The caller's registers for the next chunk (loads in flight) are held
  // here, ahead of the stores, so that nothing later waits on them.
  pin();
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.out + cp.t0 * HV, static_cast<uint32_t>(cp.n * HV * 2));
#pragma unroll
  for (int pb = 0; pb < 4; ++pb)
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack_bf16x2(Ot[pb][0], Ot[pb][1]), pack_bf16x2(Ot[pb][2], Ot[pb][3])},
                                          ro, out_lane + static_cast<int>(16 * pb * HV * 2), 0, 0);
  // S <- diag(e^{gam_last}) S + (K o e^{gam_last - gam})^T V'.
  bf16x8 kf[2][2];
  kf[0][0] = frag<C>(ops.kgt, m, 8 * g);
  kf[0][1] = frag<C>(ops.kgt, m, 32 + 8 * g);
#pragma unroll
  for (int cb = 0; cb < K / 16; ++cb) {
    __builtin_amdgcn_sched_barrier(0);
    if (cb + 1 < K / 16) {
      kf[(cb + 1) & 1][0] = frag<C>(ops.kgt, 16 * (cb + 1) + m, 8 * g);
      kf[(cb + 1) & 1][1] = frag<C>(ops.kgt, 16 * (cb + 1) + m, 32 + 8 * g);
    }
    const f32x4 e = *reinterpret_cast<const f32x4*>(&ops.eg[16 * cb + 4 * g]);
#pragma unroll
    for (int j = 0; j < 4; ++j) S[cb][j] *= e[j];
    S[cb] = mfma16(kf[cb & 1][0], Vb0, S[cb]);
    S[cb] = mfma16(kf[cb & 1][1], Vb1, S[cb]);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// The state pass of segment gs (rows sr) of head h on one workgroup, 8
// waves; wave w < V / 16 owns value columns 16 w .. 16 w + 15 of the state,
// kept in MFMA accumulators for the whole segment. Starts from the slot's
// state (segment 0 or an uncut sequence) or from B of map item sg - 1 (the
// scan's result); the final state goes to the slot (last segment) or, for
// segment 0 of a cut sequence, to B of map item 0.
template <int K, int V, bool EXACT>
__device__ __forceinline__ void state_segment(const PrefillParams& p, const SegPlan& pl, int gs,
                                              const SegRange& sr, int h, FusedSmem<K, true, EXACT>& sm) {
  const int H = p.H;
  const bool last_seg = sr.sg == sr.nseg - 1;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int m = lane & 15;
  const int g = lane >> 4;
  const bool has_cols = w < V / 16;  // wave-uniform
  const int col0 = 16 * w;
  const int64_t HV = static_cast<int64_t>(H) * V;
  const int64_t tfirst = sr.bos + static_cast<int64_t>(C) * sr.c0;
  const int64_t tend = min<int64_t>(sr.eos, tfirst + static_cast<int64_t>(C) * sr.nch);

  const int64_t slot = uniform(static_cast<int64_t>(p.indices[static_cast<int64_t>(sr.seq) * p.index_stride]));
  if (slot < 0) {
    // Null slot: zero output rows, no state traffic.
    for (int64_t t = tfirst; t < tend; ++t)
      for (int c = tid; c < V; c += kThreads) p.out[t * HV + h * V + c] = 0;
    return;
  }

  // The first chunk's inputs go out first, so the state loads below hide
  // their latency.
  ChunkIn<K, V> in;
  load_chunk_regs<K, V>(p, h, chunk_pos(sr, 0), in);
  dma_chunk_tiles<K, true>(p, h, chunk_pos(sr, 0), sm.t.f.k, sm.t.f.q);

  float* st = p.pool + slot * p.slot_stride + static_cast<int64_t>(h) * K * V;
  // B of the sequence's map item j (fp32 [K][V]).
  auto map_b = [&](int j) {
    return pl.maps + map_index(h, sr.seg0 - sr.seq + j, pl) * (static_cast<int64_t>(K) * K + static_cast<int64_t>(K) * V) +
           K * K;
  };
  const bool cut = uniform(pl.seg_long[gs]) >= 0;
  const bool from_scan = cut && sr.sg > 0;
  const float* s_in = from_scan ? map_b(sr.sg - 1) : st;
  const bool init = from_scan || p.has_initial_state == nullptr ||
                    uniform(static_cast<int32_t>(p.has_initial_state[sr.seq])) != 0;
  // Without an initial state (or without columns) the range is empty and
  // every load reads zero.
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(s_in, init && has_cols ? static_cast<uint32_t>(K * V * 4) : 0u);
  f32x4 S[K / 16];
#pragma unroll
  for (int cb = 0; cb < K / 16; ++cb)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      S[cb][j] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(rs, ((16 * cb + 4 * g + j) * V + col0 + m) * 4, 0, 0));
  // Wait for the state here, once: the compiler cannot tell inside the loop
  // that these loads are long done and would wait for every later load.
  pin_regs(S);

  stage_gate_consts<K>(p, h, sm.x);
  zero_p_unread<K, true>(sm.r.ops);
  // Gated RMSNorm output epilogue (optional; vLLM PR #60683, Purpose, places
  // it after the recurrence): y = o / sqrt(mean over the head's V channels
  // of o^2 + eps) * weight * act(gate), applied to the fp32 output before
  // its bf16 store. The workgroup holds every value column of its
  // positions, so one exchange of per-wave sums of squares per chunk does.
  const bool has_norm = p.norm.gate != nullptr;  // uniform
  f32x4 nw = {1.f, 1.f, 1.f, 1.f};               // the norm weights of the lane's four channels
  if (has_norm && has_cols) nw = *reinterpret_cast<const f32x4*>(p.norm.weight + col0 + 4 * g);
  const auto& ops = sm.r.ops;
  for (int cc = 0; cc < sr.nch; ++cc) {
    const ChunkPos cp = chunk_pos(sr, cc);
    // This chunk's inputs have landed (the previous chunk's 4 output stores
    // per lane, issued after them, may still be in flight) and every wave is
    // done with the previous chunk's operands.
    if (has_cols) chunk_barrier<4>();
    else chunk_barrier<0>();
    if (has_norm && has_cols) load_chunk_norm_regs<K, V>(p, h, cp, in);
    f32x4 Vp[4];
    const bool more = cc + 1 < sr.nch;
    const ChunkPos np = chunk_pos(sr, more ? cc + 1 : cc);
    intra_part<K, V, true, EXACT>(p, h, cp.n, in, more, np, sm, Vp);
    // The rest of the next chunk's inputs go out now: the registers and the
    // tile area are free, and the state step below hides their latency.
    if (more) {
      load_chunk_v_regs<K, V>(p, h, np, in);
      if constexpr (EXACT) dma_chunk_tiles<K, true>(p, h, np, sm.t.f.k, sm.t.f.q);
    }
    if (!has_cols) {
      pin_gate_regs<K, V>(in);            // (no v operands without columns)
      if (has_norm) lds_barrier();        // the epilogue's exchange below
      continue;
    }
    state_step<K, V>(p, h, w, cp, ops, sm.nrm, S, Vp, in.zg, nw, has_norm, [&] {
      // The next chunk's v operands have had the products above to land.
      // (Unconditional: the last chunk's pins are no-ops, but every path
      // through the loop then carries them.)
      pin_v_regs<K, V>(in);
      pin_gate_regs<K, V>(in);
    });
  }

  if (!has_cols) return;
  float* fin = last_seg ? st : (cut && sr.sg == 0 ? map_b(0) : nullptr);
  if (fin == nullptr) return;
#pragma unroll
  for (int cb = 0; cb < K / 16; ++cb)
#pragma unroll
    for (int j = 0; j < 4; ++j) fin[(16 * cb + 4 * g + j) * V + col0 + m] = S[cb][j];
}

// Address of the record of chunk cc of segment range sr, head h.
template <int K, int V>
__device__ __forceinline__ uint8_t* record_of(const SegPlan& pl, const SegRange& sr, int h, int cc) {
  const int64_t slot = static_cast<int64_t>(uniform(pl.chunk_start[sr.seq])) + sr.c0 + cc;
  return pl.recs + (static_cast<int64_t>(h) * pl.rec_bound + slot) * static_cast<int64_t>(rec_bytes(K, V));
}

// Buffer-to-LDS copy of a record's operand tiles into an LDS record buffer,
// Rec::kRounds 16-byte pieces per thread; pieces past the tiles land as
// zeros in the buffer's rounding.
template <int K, int V>
__device__ __forceinline__ void dma_record(const uint8_t* rec, const uint4* buf) {
  const u32x4 rr = rsrc_words(rec, static_cast<uint32_t>(Rec<K, V>::kOps));
  const int tid = opaque_tid();
#pragma unroll
  for (int r = 0; r < Rec<K, V>::kRounds; ++r)
    lds_copy16(rr, lds_addr(buf + r * kThreads + (tid & ~63)), (r * kThreads + tid) * 16);
}

// U of a record (waves w < V / 16): lane (m, g) gets rows 16 pb + 4 g + j of
// value columns 16 w + m.
template <int K, int V>
__device__ __forceinline__ void load_record_u(const uint8_t* rec, int w, f32x4 (&u)[4]) {
  const __amdgpu_buffer_rsrc_t ru = make_rsrc(rec + Rec<K, V>::kOps, static_cast<uint32_t>(C * V * 4));
  const int lane = opaque_tid() & 63;
#pragma unroll
  for (int pb = 0; pb < 4; ++pb)
    u[pb] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ru, ((4 * w + pb) * 64 + lane) * 16, 0, 0));
}

// The state pass of segment sg >= 1 of a cut sequence from its chunk
// records (records mode): the same state steps as state_segment, from the
// scan's initial state, with the next chunk's record copied into the idle
// LDS buffer (and its U and epilogue gate loaded) while the current one
// computes. The final state goes to the slot (last segment).
template <int K, int V>
__device__ __forceinline__ void state_records(const PrefillParams& p, const SegPlan& pl, const SegRange& sr, int h,
                                              RecSmem<K, V>& rm) {
  const int H = p.H;
  const bool last_seg = sr.sg == sr.nseg - 1;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int m = lane & 15;
  const int g = lane >> 4;
  const bool has_cols = w < V / 16;  // wave-uniform
  const int col0 = 16 * w;
  const int64_t HV = static_cast<int64_t>(H) * V;
  const int64_t tfirst = sr.bos + static_cast<int64_t>(C) * sr.c0;
  const int64_t tend = min<int64_t>(sr.eos, tfirst + static_cast<int64_t>(C) * sr.nch);

  const int64_t slot = uniform(static_cast<int64_t>(p.indices[static_cast<int64_t>(sr.seq) * p.index_stride]));
  if (slot < 0) {
    // Null slot: zero output rows, no state traffic (and no records were written).
    for (int64_t t = tfirst; t < tend; ++t)
      for (int c = tid; c < V; c += kThreads) p.out[t * HV + h * V + c] = 0;
    return;
  }
  const bool has_norm = p.norm.gate != nullptr;  // uniform
  f32x4 Un[4] = {};
  u32x2 zn[4] = {};
  // The first chunk's record goes out first, so the state loads below hide
  // its latency.
  auto issue = [&](int cc) {
    const uint8_t* rec = record_of<K, V>(pl, sr, h, cc);
    dma_record<K, V>(rec, rm.ops[cc & 1]);
    if (has_cols) {
      load_record_u<K, V>(rec, w, Un);
      if (has_norm) {
        const ChunkPos cp = chunk_pos(sr, cc);
        const int64_t grs = p.norm.gate_row_stride;
        const __amdgpu_buffer_rsrc_t rz =
            make_rsrc(p.norm.gate + cp.t0 * grs, static_cast<uint32_t>(cp.n * grs * 2));
        const int zl = static_cast<int>(m * grs + h * V + col0 + 4 * g) * 2;
#pragma unroll
        for (int pb = 0; pb < 4; ++pb)
          zn[pb] = __builtin_amdgcn_raw_buffer_load_b64(rz, zl + static_cast<int>(16 * pb * grs * 2), 0, 0);
      }
    }
  };
  issue(0);

  // From B of the sequence's map item sg - 1: the scan's result.
  const float* s_in = pl.maps + map_index(h, sr.seg0 - sr.seq + sr.sg - 1, pl) *
                                    (static_cast<int64_t>(K) * K + static_cast<int64_t>(K) * V) +
                      K * K;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(s_in, has_cols ? static_cast<uint32_t>(K * V * 4) : 0u);
  f32x4 S[K / 16];
#pragma unroll
  for (int cb = 0; cb < K / 16; ++cb)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      S[cb][j] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(rs, ((16 * cb + 4 * g + j) * V + col0 + m) * 4, 0, 0));
  f32x4 nw = {1.f, 1.f, 1.f, 1.f};
  if (has_norm && has_cols) nw = *reinterpret_cast<const f32x4*>(p.norm.weight + col0 + 4 * g);
  pin_regs(S);

  for (int cc = 0; cc < sr.nch; ++cc) {
    const ChunkPos cp = chunk_pos(sr, cc);
    // This chunk's record, U and gate have landed (the previous chunk's 4
    // output stores per lane, issued after them, may still be in flight) and
    // every wave is done with the other buffer.
    if (cc > 0 && has_cols) chunk_barrier<4>();
    else chunk_barrier<0>();
    f32x4 Vp[4];
    u32x2 zg[4];
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
      Vp[pb] = Un[pb];
      zg[pb] = zn[pb];
    }
    if (cc + 1 < sr.nch) issue(cc + 1);
    if (!has_cols) {
      if (has_norm) lds_barrier();  // the epilogue's exchange in the state step
      continue;
    }
    // (The next chunk's U and gate are first read at its top, after its
    // barrier: nothing to hold here.)
    state_step<K, V>(p, h, w, cp, rm.buf(cc & 1), rm.nrm, S, Vp, zg, nw, has_norm, [] {});
  }
  if (!has_cols || !last_seg) return;
  float* st = p.pool + slot * p.slot_stride + static_cast<int64_t>(h) * K * V;
#pragma unroll
  for (int cb = 0; cb < K / 16; ++cb)
#pragma unroll
    for (int j = 0; j < 4; ++j) st[(16 * cb + 4 * g + j) * V + col0 + m] = S[cb][j];
}

// Second launch: one workgroup per (segment, head), every segment but
// segment 0 of a cut sequence (run by the first launch). REC: the later
// segments of cut sequences run from their chunk records.
template <int K, int V, bool EXACT, bool REC>
__global__ __launch_bounds__(kThreads, 1) void chunk_state_kernel(const PrefillParams p, const SegPlan pl) {
  __shared__ union {
    FusedSmem<K, true, EXACT> fused;
    RecSmem<K, V> rec;
  } smu;
  const int H = p.H;
  if (uniform(pl.counts[0]) != 0) {
    poison_output(p);
    return;
  }
  const int gs = static_cast<int>(blockIdx.x) / H, h = static_cast<int>(blockIdx.x) % H;
  if (gs >= uniform(pl.counts[1])) return;
  const SegRange sr = segment_range(p, pl, gs);
  if (sr.nch <= 0) return;
  const bool cut = uniform(pl.seg_long[gs]) >= 0;
  if (sr.sg == 0 && cut) return;
  if (REC && cut) state_records<K, V>(p, pl, sr, h, smu.rec);
  else state_segment<K, V, EXACT>(p, pl, gs, sr, h, smu.fused);
}

// ---------------------------------------------------------------- scan --

// The A operand fragments of M for S <- M S + B: fragment (rt, kb) of lane
// (m, g) is row 16 rt + m at the permuted channel slots 8 g .. 8 g + 7 of
// block kb (channels 32 kb + 4 g + 0..3 and 32 kb + 16 + 4 g + 0..3), so an
// accumulator-held S is the B operand as it stands. Stored as bf16 hi parts
// ([RT][KB][64] fragments of 16 bytes) and then lo parts (the bf16 rounding
// of M - hi), together the size of M in fp32. From M in LDS (fp32 [K][K],
// pieces swizzled by row); all threads of the workgroup take part.
template <int K>
__device__ __forceinline__ void store_map_fragments(const float* mt, uint4* dst) {
  constexpr int NF = (K / 16) * (K / 32) * 64;  // fragments per part
  static_assert(NF % kThreads == 0, "whole rounds");
#pragma unroll
  for (int r0 = 0; r0 < NF / kThreads; ++r0) {
    const int f = r0 * kThreads + static_cast<int>(threadIdx.x);
    const int l = f & 63, kb = (f >> 6) % (K / 32), rt = (f >> 6) / (K / 32);
    const int row = 16 * rt + (l & 15), g = l >> 4;
    const int p0 = 8 * kb + g, p1 = 8 * kb + 4 + g;  // pieces of channels 32 kb + 4 g and 32 kb + 16 + 4 g
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(&mt[row * K + ((p0 ^ (row & 15)) << 2)]);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(&mt[row * K + ((p1 ^ (row & 15)) << 2)]);
    const bf16x8 hi = pack_acc(a0, a1);
    const bf16x8 lo = pack_lo(a0, a1, hi);
    dst[f] = __builtin_bit_cast(uint4, hi);
    dst[NF + f] = __builtin_bit_cast(uint4, lo);
  }
}

// One workgroup of four waves per (cut sequence, value column block of 16,
// head); the blocks of a head share an XCD (the index is head-fastest, so
// with H a multiple of 8 they fall on one L2 and each M is fetched once).
// Composes the segment maps in order: S_1 = B_0 (segment 0's final state),
// S_{j+1} = M_j S_j + B_j, stored over B_j (the workgroup's columns) for
// segment j + 1 of the state pass. Wave w computes row tiles RPW w .. RPW w
// + RPW - 1 of S_{j+1} (RPW = K / 64); S_j goes through LDS (one barrier
// per step), and M_{j+1}'s fragments and B_{j+1} are loaded while step j
// computes.
constexpr int kScanWaves = 4;
constexpr int kScanThreads = 64 * kScanWaves;

template <int K, int V>
__global__ __launch_bounds__(kScanThreads, 1) void chunk_scan_kernel(const PrefillParams p, const SegPlan pl) {
  constexpr int KB = K / 32, RT = K / 16, NCB = V / 16;
  constexpr int RPW = RT / kScanWaves;           // row tiles per wave
  constexpr int NF = RT * KB * 64;               // fragments per part of M
  constexpr int NSTORE = RPW * 4;                // stores per lane per step
  constexpr int SST = K + 4;                     // S in LDS: [16 columns][K rows], rows padded
  static_assert(RPW * kScanWaves == RT && (2 * NF) % kScanThreads == 0, "whole row tiles and DMA rounds");
  __shared__ uint4 mbuf[2][2 * NF];
  __shared__ float sbuf[2][16 * SST];
  const int H = p.H;
  if (uniform(pl.counts[0]) != 0) return;
  auto scan_item = [&](int bi) {
    const int h = bi % H, rest = bi / H;
    const int cbk = rest % NCB, li = rest / NCB;
    if (li >= uniform(pl.counts[3])) return;
    const int seq = uniform(pl.long_seq[li]);
    const int64_t slot = uniform(static_cast<int64_t>(p.indices[static_cast<int64_t>(seq) * p.index_stride]));
    if (slot < 0) return;  // no maps were made for a null slot
    const int seg0 = uniform(pl.seg_start[seq]);
    const int nmap = uniform(pl.seg_start[seq + 1]) - seg0 - 1;
    if (nmap < 2) return;
    const int mi0 = seg0 - seq;
    const int tid = threadIdx.x, lane = tid & 63, w = uniform(tid >> 6), m = lane & 15, g = lane >> 4;
    const int col0 = 16 * cbk;
    const int64_t item = static_cast<int64_t>(K) * K + static_cast<int64_t>(K) * V;
    auto dma_map = [&](int j) {
      const u32x4 rr = rsrc_words(pl.maps + map_index(h, mi0 + j, pl) * item, static_cast<uint32_t>(K * K * 4));
#pragma unroll
      for (int r = 0; r < 2 * NF / kScanThreads; ++r)
        lds_copy16(rr, lds_addr(&mbuf[j & 1][r * kScanThreads + (tid & ~63)]), (r * kScanThreads + tid) * 16);
    };
    auto b_of = [&](int j) { return pl.maps + map_index(h, mi0 + j, pl) * item + static_cast<int64_t>(K) * K; };
    // The wave's row tiles of B_j's columns: lane (m, g) holds rows 16 rt + 4 g
    // + jj of column col0 + m.
    auto load_rows = [&](const float* src, f32x4 (&b)[RPW]) {
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(src, static_cast<uint32_t>(K * V * 4));
#pragma unroll
      for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          b[r][jj] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                   rb, ((16 * (RPW * w + r) + 4 * g + jj) * V + col0 + m) * 4, 0, 0));
    };
    auto put_rows = [&](float* sb, const f32x4 (&b)[RPW]) {
#pragma unroll
      for (int r = 0; r < RPW; ++r)
        *reinterpret_cast<f32x4*>(&sb[m * SST + 16 * (RPW * w + r) + 4 * g]) = b[r];
    };
    dma_map(1);
    f32x4 S1[RPW], Bn[RPW];
    load_rows(b_of(0), S1);
    load_rows(b_of(1), Bn);
    pin_regs(S1);
    put_rows(sbuf[1], S1);
    for (int j = 1; j < nmap; ++j) {
      // M_j's fragments, B_j and every wave's rows of S_j have landed (only the
      // previous step's stores, the last vector-memory operations, may be in
      // flight), and every wave is done with step j - 1's buffers.
      if (j == 1) __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt 0, lgkmcnt 0
      else __builtin_amdgcn_s_waitcnt(0x0070 | (NSTORE & 15) | ((NSTORE >> 4) << 14));
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      f32x4 Bc[RPW];
#pragma unroll
      for (int r = 0; r < RPW; ++r) Bc[r] = Bn[r];
      if (j + 1 < nmap) {
        dma_map(j + 1);
        load_rows(b_of(j + 1), Bn);
      }
      // S_j as the B operand: lane (m, g) takes rows 16 cb + 4 g + jj.
      const float* sb = sbuf[j & 1];
      bf16x8 Sh[KB], Sl[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(&sb[m * SST + 32 * kb + 4 * g]);
        const f32x4 s1 = *reinterpret_cast<const f32x4*>(&sb[m * SST + 32 * kb + 16 + 4 * g]);
        Sh[kb] = pack_acc(s0, s1);
        Sl[kb] = pack_lo(s0, s1, Sh[kb]);
      }
      const uint4* mh = mbuf[j & 1];
      f32x4 Sn[RPW];
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const int rt = RPW * w + r;
        f32x4 acc = Bc[r];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const bf16x8 ah = __builtin_bit_cast(bf16x8, mh[(rt * KB + kb) * 64 + lane]);
          const bf16x8 al = __builtin_bit_cast(bf16x8, mh[NF + (rt * KB + kb) * 64 + lane]);
          acc = mfma16(ah, Sh[kb], acc);
          acc = mfma16(ah, Sl[kb], acc);
          acc = mfma16(al, Sh[kb], acc);
        }
        Sn[r] = acc;
      }
      put_rows(sbuf[(j + 1) & 1], Sn);
      // The state that segment j + 1 starts from, over B_j (the workgroup's
      // columns; the other columns belong to the head's other workgroups).
      float* Bm = b_of(j);
#pragma unroll
      for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) Bm[(16 * (RPW * w + r) + 4 * g + jj) * V + col0 + m] = Sn[r][jj];
    }
  };
  // One item per (cut sequence, 16 value columns, head). The grid holds at
  // most one workgroup per CU (idle ones would each cost a dispatch round),
  // so a workgroup steps through the items; a stride that is a multiple of
  // 8 keeps every item of a head on one XCD.
  const int items = uniform(pl.counts[3]) * H * NCB;
  for (int bi = blockIdx.x; bi < items; bi += gridDim.x) {
    if (bi != static_cast<int>(blockIdx.x)) __syncthreads();  // the previous item is done with the LDS
    scan_item(bi);
  }
}

// ----------------------------------------------------------------- map --

// Writes chunk cc's record (records mode): the operand tiles from LDS, 16
// bytes per piece (Rec::kRounds stores per thread; those past the tiles are
// dropped by the buffer range), then U from the registers of waves w < V /
// 16 (4 stores per lane).
template <int K, int V>
__device__ __forceinline__ void write_record(uint8_t* rec, const ChunkOps<K, true>& ops, const f32x4 (&U)[4], int w) {
  using R = Rec<K, V>;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(rec, static_cast<uint32_t>(R::kOps));
  const int tid = opaque_tid();
  const uint4* src = reinterpret_cast<const uint4*>(&ops);
#pragma unroll
  for (int r = 0; r < R::kRounds; ++r) {
    const int piece = r * kThreads + tid;
    const uint4 v = src[min(piece, R::kPieces - 1)];
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v.z, v.w}, ro, piece * 16, 0, 0);
  }
  if (w < V / 16) {  // wave-uniform
    const __amdgpu_buffer_rsrc_t ru = make_rsrc(rec + R::kOps, static_cast<uint32_t>(C * V * 4));
    const int lane = tid & 63;
#pragma unroll
    for (int pb = 0; pb < 4; ++pb)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, U[pb]), ru, ((4 * w + pb) * 64 + lane) * 16, 0,
                                             0);
  }
}

// A segment sg >= 1 of a cut sequence in the first launch: with do_map its
// map (M, B) into map item mi; with REC the records of its chunks (then Q:
// the intra part builds the query operands too). Every chunk of a map item's
// segment is full; a records-only segment (the last) may end in a partial
// chunk.
//   X = [I | 0] (the identity's columns, and zero); per chunk, with U = 0
//   for the columns of M and the chunk's U for those of B:
//   X <- e^{gam_last} o X + (K o e^{gam_last-gam})^T ([0 | U] - W X).
// Wave w owns M's column tile w (w < K / 16) and B's (w < V / 16). The
// rounding is the state pass's (bf16 X into W X, bf16 V' into the update,
// fp32 accumulation).
template <int K, int V, bool Q, bool EXACT, bool REC>
__device__ __forceinline__ void map_segment(const PrefillParams& p, const SegPlan& pl, int mi, const SegRange& sr,
                                            int h, FusedSmem<K, Q, EXACT>& sm, bool do_map) {
  static_assert(!REC || Q, "records carry the query operands");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int m = lane & 15;
  const int g = lane >> 4;
  const bool act[2] = {do_map && w < K / 16, do_map && w < V / 16};  // the wave's tile of M, of B (wave-uniform)

  ChunkIn<K, V> in;
  load_chunk_regs<K, V>(p, h, chunk_pos(sr, 0), in);
  dma_chunk_tiles<K, Q>(p, h, chunk_pos(sr, 0), sm.t.f.k, Q ? sm.t.f.q : nullptr);

  // X[0]: the wave's column tile of M (from the identity), X[1]: of B.
  f32x4 X[2][K / 16];
#pragma unroll
  for (int cb = 0; cb < K / 16; ++cb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      X[0][cb][j] = (16 * cb + 4 * g + j == 16 * w + m) ? 1.f : 0.f;
      X[1][cb][j] = 0.f;
    }
  stage_gate_consts<K>(p, h, sm.x);
  zero_p_unread<K, Q>(sm.r.ops);
  const auto& ops = sm.r.ops;
  for (int cc = 0; cc < sr.nch; ++cc) {
    pin_v_regs<K, V>(in);
    // This chunk's inputs have landed; with records, the previous chunk's
    // record stores (the last vector-memory operations) may be in flight.
    if (REC && cc > 0) {
      if (w < V / 16) chunk_barrier<Rec<K, V>::kRounds + 4>();
      else chunk_barrier<Rec<K, V>::kRounds>();
    } else {
      chunk_barrier<0>();
    }
    f32x4 U[4];
    const bool more = cc + 1 < sr.nch;
    const ChunkPos cp = chunk_pos(sr, cc);
    const ChunkPos np = chunk_pos(sr, more ? cc + 1 : cc);
    intra_part<K, V, Q, EXACT>(p, h, cp.n, in, more, np, sm, U);
    if (more) {
      load_chunk_v_regs<K, V>(p, h, np, in);
      if constexpr (EXACT) dma_chunk_tiles<K, Q>(p, h, np, sm.t.f.k, Q ? sm.t.f.q : nullptr);
    }
    if constexpr (REC) write_record<K, V>(record_of<K, V>(pl, sr, h, cc), ops, U, w);
    if (!act[0] && !act[1]) continue;
    const int m = opaque_tid() & 15, g = (opaque_tid() & 63) >> 4;
    // V' = [0 | U] - W X over positions.
    f32x4 Vp[2][4];
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
      Vp[0][pb] = f32x4{0.f, 0.f, 0.f, 0.f};
      Vp[1][pb] = U[pb];
    }
    bf16x8 Xb[2][K / 32];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int kb = 0; kb < K / 32; ++kb) Xb[x][kb] = pack_acc(X[x][2 * kb], X[x][2 * kb + 1]);
    bf16x8 wf[2][K / 32];
#pragma unroll
    for (int kb = 0; kb < K / 32; ++kb) wf[0][kb] = frag<K>(ops.wn, m, 32 * kb + 8 * g);
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
      __builtin_amdgcn_sched_barrier(0);
      if (pb + 1 < 4) {
#pragma unroll
        for (int kb = 0; kb < K / 32; ++kb) wf[(pb + 1) & 1][kb] = frag<K>(ops.wn, 16 * (pb + 1) + m, 32 * kb + 8 * g);
      }
#pragma unroll
      for (int kb = 0; kb < K / 32; ++kb)
#pragma unroll
        for (int x = 0; x < 2; ++x)
          if (act[x]) Vp[x][pb] = mfma16(wf[pb & 1][kb], Xb[x][kb], Vp[x][pb]);
    }
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 Vb[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      Vb[x][0] = pack_acc(Vp[x][0], Vp[x][1]);
      Vb[x][1] = pack_acc(Vp[x][2], Vp[x][3]);
    }
    // X <- diag(e^{gam_last}) X + (K o e^{gam_last - gam})^T V'.
#pragma unroll
    for (int cb = 0; cb < K / 16; ++cb) {
      const bf16x8 kf0 = frag<C>(ops.kgt, 16 * cb + m, 8 * g);
      const bf16x8 kf1 = frag<C>(ops.kgt, 16 * cb + m, 32 + 8 * g);
      const f32x4 e = *reinterpret_cast<const f32x4*>(&ops.eg[16 * cb + 4 * g]);
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        if (!act[x]) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) X[x][cb][j] *= e[j];
        X[x][cb] = mfma16(kf0, Vb[x][0], X[x][cb]);
        X[x][cb] = mfma16(kf1, Vb[x][1], X[x][cb]);
      }
    }
  }
  if (!do_map) return;  // uniform
  float* dst = pl.maps + map_index(h, mi, pl) * (static_cast<int64_t>(K) * K + static_cast<int64_t>(K) * V);
  // B as fp32 [K][V].
  if (act[1]) {
#pragma unroll
    for (int cb = 0; cb < K / 16; ++cb)
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[K * K + (16 * cb + 4 * g + j) * V + 16 * w + m] = X[1][cb][j];
  }
  // M as the scan's MFMA A operands, split into bf16 hi and lo parts: a
  // waves' column tiles go through LDS (fp32 [K][K], 16-byte pieces of row
  // r XOR-swizzled by r) and come back as row fragments.
  float* mt = reinterpret_cast<float*>(&sm);
  static_assert(sizeof(FusedSmem<K, Q, EXACT>) >= sizeof(float) * K * K, "M fits the workgroup's LDS");
  __syncthreads();  // every wave is done with the last chunk's operands
  if (act[0]) {
#pragma unroll
    for (int cb = 0; cb < K / 16; ++cb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * cb + 4 * g + j, c = 16 * w + m;
        mt[r * K + ((((c >> 2) ^ (r & 15)) << 2) | (c & 3))] = X[0][cb][j];
      }
  }
  __syncthreads();
  store_map_fragments<K>(mt, reinterpret_cast<uint4*>(dst));
}

// First launch: one workgroup per (map item = a non-final segment of a cut
// sequence, head), 8 waves, and with REC one more per (cut sequence, head)
// for the sequence's last segment (records only). Segment 0 runs its state
// pass (state_segment); segments 1 .. n - 2 their maps (map_segment), with
// REC also their records.
template <int K, int V, bool EXACT, bool REC>
__global__ __launch_bounds__(kThreads, 1) void chunk_map_kernel(const PrefillParams p, const SegPlan pl) {
  __shared__ union {
    FusedSmem<K, true, EXACT> state;
    FusedSmem<K, false, EXACT> map;
  } smu;
  const int H = p.H;
  if (uniform(pl.counts[0]) != 0) return;
  const int mi = static_cast<int>(blockIdx.x) / H, h = static_cast<int>(blockIdx.x) % H;
  const int nmaps = uniform(pl.counts[2]);
  int gs;
  bool do_map = true;
  if (mi < nmaps) {
    gs = uniform(pl.map_seg[mi]);
  } else {
    if (!REC) return;
    const int li = mi - nmaps;
    if (li >= uniform(pl.counts[3])) return;
    gs = uniform(pl.seg_start[uniform(pl.long_seq[li]) + 1]) - 1;
    do_map = false;
  }
  const SegRange sr = segment_range(p, pl, gs);
  if (sr.sg == 0) {  // segment 0's state pass instead of its map
    state_segment<K, V, EXACT>(p, pl, gs, sr, h, smu.state);
    return;
  }
  const int64_t slot = uniform(static_cast<int64_t>(p.indices[static_cast<int64_t>(sr.seq) * p.index_stride]));
  if (slot < 0) return;  // a null slot carries no state
  if constexpr (REC) map_segment<K, V, true, EXACT, true>(p, pl, mi, sr, h, smu.state, do_map);
  else map_segment<K, V, false, EXACT, false>(p, pl, mi, sr, h, smu.map, true);
}

template <int K, int V, bool EXACT>
hipError_t launch_kv(const PrefillParams& p, const Layout& L, const SegPlan& pl, hipStream_t stream) {
  const int64_t state_blocks = L.seg_bound * p.H;
  // With records the first launch also runs the last segment of every cut
  // sequence (one item per cut sequence after the map items).
  const int64_t map_blocks = (L.map_bound + (pl.records ? L.long_bound : 0)) * p.H;
  const int64_t scan_blocks = L.long_bound * p.H * (V / 16);
  if (state_blocks > 0x7fffffff || map_blocks > 0x7fffffff || scan_blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (map_blocks > 0) {
    // The scan kernel steps through its items (one workgroup per CU at
    // most): only the plan knows how many there are.
    const unsigned scan_grid = static_cast<unsigned>(std::min<int64_t>(scan_blocks, kChipSlots));
    if (pl.records)
      chunk_map_kernel<K, V, EXACT, true><<<dim3(static_cast<unsigned>(map_blocks)), dim3(kThreads), 0, stream>>>(p, pl);
    else
      chunk_map_kernel<K, V, EXACT, false><<<dim3(static_cast<unsigned>(map_blocks)), dim3(kThreads), 0, stream>>>(p, pl);
    chunk_scan_kernel<K, V><<<dim3(scan_grid), dim3(kScanThreads), 0, stream>>>(p, pl);
  }
  if (pl.records)
    chunk_state_kernel<K, V, EXACT, true><<<dim3(static_cast<unsigned>(state_blocks)), dim3(kThreads), 0, stream>>>(p, pl);
  else
    chunk_state_kernel<K, V, EXACT, false><<<dim3(static_cast<unsigned>(state_blocks)), dim3(kThreads), 0, stream>>>(p, pl);
  return hipGetLastError();
}

// With a lower bound lb every per-token log-decay lies in (lb, 0), so a
// block's factors (over its 16 rows from the gam just before it) span less
// than 16 |lb| and every chunk takes the factored path once
// 16 |lb| <= kMaxBlockDecay: the kernels without the exact path (less LDS)
// then suffice.
#ifndef KDA_CHUNK_EXACT_PART
bool all_factored(const PrefillParams& p) { return p.has_lb != 0 && 16.f * -p.lower_bound <= kMaxBlockDecay; }
#endif

template <bool EXACT>
hipError_t launch_kernels(const PrefillParams& p, const Layout& L, const SegPlan& pl, hipStream_t stream) {
  if (p.K == 64 && p.V == 64) return launch_kv<64, 64, EXACT>(p, L, pl, stream);
  if (p.K == 64 && p.V == 128) return launch_kv<64, 128, EXACT>(p, L, pl, stream);
  if (p.K == 128 && p.V == 64) return launch_kv<128, 64, EXACT>(p, L, pl, stream);
  return launch_kv<128, 128, EXACT>(p, L, pl, stream);
}

// The plan's pointers into the workspace.
SegPlan plan_for(const PrefillParams& p, const Layout& L) {
  char* ws = static_cast<char*>(p.workspace);
  SegPlan pl;
  pl.counts = reinterpret_cast<int32_t*>(ws + L.counts);
  pl.chunk_start = reinterpret_cast<int32_t*>(ws + L.chunk_start);
  pl.seg_start = reinterpret_cast<int32_t*>(ws + L.seg_start);
  pl.seg_seq = reinterpret_cast<int32_t*>(ws + L.seg_seq);
  pl.seg_long = reinterpret_cast<int32_t*>(ws + L.seg_long);
  pl.map_seg = reinterpret_cast<int32_t*>(ws + L.map_seg);
  pl.long_seq = reinterpret_cast<int32_t*>(ws + L.long_seq);
  pl.maps = reinterpret_cast<float*>(ws + L.maps);
  // Records when the workspace holds them (a workspace of total_min bytes
  // runs without) and some sequence can be cut.
  pl.records = p.workspace_bytes >= L.total && L.rec_bound > 0 ? 1 : 0;
  pl.recs = pl.records ? reinterpret_cast<uint8_t*>(ws + L.recs) : nullptr;
  pl.rec_bound = static_cast<int32_t>(L.rec_bound);
  pl.seg_bound = static_cast<int32_t>(L.seg_bound);
  pl.map_bound = static_cast<int32_t>(L.map_bound);
  pl.long_bound = static_cast<int32_t>(L.long_bound);
  pl.max_segs = static_cast<int32_t>(L.max_segs);
  pl.num_tokens = static_cast<int32_t>(p.num_tokens);
  return pl;
}

}  // namespace

#ifndef KDA_CHUNK_EXACT_PART

size_t prefill_workspace_bytes(int32_t num_seqs, int64_t num_tokens, int32_t H, int32_t K,
                               int32_t V) {
  return layout_for(num_seqs, num_tokens, H, K, V).total;
}

size_t prefill_workspace_min_bytes(int32_t num_seqs, int64_t num_tokens, int32_t H, int32_t K,
                                   int32_t V) {
  return layout_for(num_seqs, num_tokens, H, K, V).total_min;
}

void prefill_workspace_maps(int32_t num_seqs, int64_t num_tokens, int32_t H, int32_t K, int32_t V,
                            size_t* offset, size_t* item_bytes, int64_t* items) {
  const Layout L = layout_for(num_seqs, num_tokens, H, K, V);
  *offset = L.maps;
  *item_bytes = (static_cast<size_t>(K) * K + static_cast<size_t>(K) * V) * 4;
  *items = L.map_bound * H;
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream, hipEvent_t after_plan) {
  const Layout L = layout_for(p.num_seqs, p.num_tokens, p.H, p.K, p.V);
  if (L.seg_bound > 0x7fffffff || L.rec_bound > 0x7fffffff) return hipErrorInvalidValue;
  const SegPlan pl = plan_for(p, L);
  plan_kernel<<<1, kPlanThreads, 0, stream>>>(p.cu_seqlens, p.num_seqs, p.H, pl);
  if (after_plan != nullptr) {
    const hipError_t e = hipEventRecord(after_plan, stream);
    if (e != hipSuccess) return e;
  }
  // The output epilogue (p.norm) is applied inside the state passes.
  return all_factored(p) ? launch_kernels<false>(p, L, pl, stream) : launch_prefill_exact(p, stream);
}

#else  // KDA_CHUNK_EXACT_PART

hipError_t launch_prefill_exact(const PrefillParams& p, hipStream_t stream) {
  const Layout L = layout_for(p.num_seqs, p.num_tokens, p.H, p.K, p.V);
  return launch_kernels<true>(p, L, plan_for(p, L), stream);
}

#endif  // KDA_CHUNK_EXACT_PART

}  // namespace kda
