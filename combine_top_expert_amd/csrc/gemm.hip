// Grouped GEMMs of the gated-SiLU expert MLP on CDNA4 matrix cores.
//
//   moe_grouped_gemm_w13:  G = A W13[e]^T   (+ fused SiLU(gate)*up epilogue)
//   moe_grouped_gemm_w2 :  O = Z W2[e]^T
//
// ("SGLang Expert Compute Backend" §1.1 expert MLP, §2.3-§2.6 grouped work
// set and scheduling, §3.5 block-FP8 accumulation, §3.6 non-interleaved
// gate/up, §4.4 fused SiLU + group quantisation.)
//
// Work set.  Expert e contributes ceil(counts[e]/BM) row tiles; every row
// tile meets nb_count column blocks.  Only these tiles exist -- nothing is
// launched or computed for capacity rows beyond counts[e] (the page's
// "compact task organisation").  Each workgroup rebuilds the tile map from
// counts in LDS and walks it persistently; tiles are ordered expert-major,
// then band of 8 row tiles, then column block, then row tile, so the tiles
// that share a weight block or an activation tile run close together, and
// the ordered tile range is cut into 8 contiguous chunks, one per XCD
// (workgroup i runs on XCD i mod 8), so both operands are fetched from HBM
// into one XCD's L2 and reused there.
//
// Tile.  BM = 128 rows x two 128-column "halves" of W rows.  For W13 the
// halves are the gate block n0 + [0,128) and the matching up block
// I + n0 + [0,128), so one lane holds gate and up of the same (row, column)
// and SiLU(gate)*up needs no data exchange.  For W2 the halves are two
// adjacent 128-column blocks.
//
// Waves.  Twelve waves, three per SIMD.  Waves 8-11 are producers: they
// only move K stages HBM -> LDS with direct-to-LDS buffer loads (lane l's
// bytes land at base + size*l), so a wave held at a load issue by the
// memory pipeline never holds up matrix work.  Waves 0-7 are consumers in
// a 2 x 4 grid, each owning 64 rows x (32 columns of each half) = 16 MFMA
// 16x16 tiles; they only read LDS and multiply.
//
// K loop.  One stage = 128 bytes of K per row: 128 FP8, 64 bf16 or 32 fp32
// values -- for FP8 exactly one activation / weight scale group.  Each
// lane's MFMA operand is 32 contiguous bytes of one row of the stage, so
// the same LDS fragment feeds one 16x16x128 FP8 MFMA, two 16x16x32 bf16
// MFMAs or eight 16x16x4 fp32 MFMAs (both operands use the same K mapping,
// so the dot products pair up).  The weight fragment is the matrix unit's
// first operand and the activation fragment its second, so a lane's four
// results of a 16x16 tile are four consecutive output columns of ONE
// activation row: a lane needs one activation scale per 16-row block.
//
// Ring and phases.  Three stages live in an LDS ring.  Consumer waves 0-3
// and 4-7 form two groups that alternate a read phase (fragment reads of a
// stage) and a matrix phase (its products), one phase apart, so each SIMD
// has one consumer on the matrix core while the other reads; a workgroup
// barrier, taken by all twelve waves, closes every phase.  In the two
// phases of stream stage G the producers issue stage G + 2 (into the slot
// of G - 1, whose last reader finished in the phase before) and then wait
// (vmcnt) for their loads of G + 1, which the consumers first read after
// the second barrier.
//
// FP8 scaling.  Per stage g every 16x16 FP8 product P_g is formed from a
// zero accumulator and folded in as acc += P_g * (a_scale[row, g] *
// w_scale[block, g]), fp32.  Both scales travel with the stage: the
// activation scales of the 128 rows and the two weight-block scales are
// staged into LDS beside the operands.

#include <algorithm>

#include "moe_common.h"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int i4 __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kConsumers = 8;      // consumer waves, 2 x 4 grid
constexpr int kProducers = 4;      // staging waves
constexpr int kThreads = (kConsumers + kProducers) * MOE_WAVE;
constexpr int BM = 128;            // rows per tile
constexpr int BH = 128;            // columns per half
constexpr int KB = 128;            // bytes of K per stage and row
constexpr int kMaxL = 1024;
constexpr int NST = 3;             // LDS ring depth
constexpr int kBand = 8;           // row tiles per band of the tile order
constexpr int A_BYTES = BM * KB;                   // 16 KB
constexpr int B_BYTES = 2 * BH * KB;               // 32 KB
constexpr int AS_BYTES = BM * 4;                   // FP8 activation scales of the stage
constexpr int WS_BYTES = 16;                       // FP8 weight scales of the two halves (+ pad)
constexpr int STAGE = A_BYTES + B_BYTES + AS_BYTES + WS_BYTES;
constexpr int kRsrcWord3 = 0x00020000;             // raw buffer: 32-bit data format
static_assert(STAGE % 16 == 0, "stage slots must stay 16-byte aligned");

enum Dt { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2 };
enum Epi { EPI_STORE_F32 = 0, EPI_STORE_BF16 = 1, EPI_SILU_F32 = 2, EPI_SILU_BF16 = 3, EPI_SILU_FP8 = 4,
           EPI_SCATTER_F32 = 5, EPI_SILU_BWD = 6 };

struct GemmArgs {
  const uint8_t* A;      // [rows_cap, K] elements
  const float* As;       // [rows_cap, K/128] (FP8)
  const uint8_t* W;      // [L, N, K]
  const float* Ws;       // [L, N/128, K/128] (FP8)
  const int32_t* counts;
  const int32_t* offsets;
  int L;
  int K;                 // reduction length in elements
  int N;                 // W rows per expert
  int nb_count;          // column blocks per expert
  int nb_stride;         // W row step between column blocks
  int half_stride;       // W row offset of half 1 from half 0
  int64_t rows_cap;
  void* out;
  float* out_scales;     // Z scales [rows_cap, I/128] (FP8 SiLU epilogue)
  int ldo;               // output row length in elements
  float* part;           // K-split partial sums [grid][BM][2*BH] fp32, or null (no split)
  int* desc;             // [grid][kDescInts]: the K-split piece each workgroup ran
  int w_packed;          // W in the packed layout (moe_pack_w13), else [L, N, K]
  // EPI_SILU_BWD (gate/up GEMM recomputing G for the SiLU*up backward):
  const uint8_t* dz;         // [rows_cap, I] dZ, fp32 (dz_f32) or bf16
  int dz_f32;
  int out_f32;               // dG in out [rows_cap, 2I]: fp32, else bf16
  // EPI_SCATTER_F32 (down GEMM adding weighted rows into token sums):
  const int32_t* row_src;    // [rows_cap]: t * topk + k of each valid row
  const float* route_w;      // [T, topk] router weights
  float* y_acc;              // [T, ldo] fp32 token sums
  int topk;
};

constexpr int kDescInts = 16;
constexpr int kPartFloats = BM * 2 * BH;           // one workgroup's partial tile
constexpr int kMinPieces = 4;                      // K split only into >= 4 pieces
// K split only for reductions of at least this many stages: the long gate/up
// GEMMs, whose last round costs most; the host then launches the second
// kernel, which costs a few microseconds even when no piece exists
constexpr int kMinSplitStages = 32;

// Rows of expert e that exist: counts[e] clipped to the buffer, so a tile
// never reaches past rows_cap even for inconsistent counts/offsets.
__device__ __forceinline__ int eff_count(int64_t off, int cnt, int64_t rows_cap) {
  if (off < 0 || off >= rows_cap) return 0;
  return static_cast<int>(max<int64_t>(0, min<int64_t>(cnt, rows_cap - off)));
}

// counts / offsets of a workgroup-uniform expert through the scalar cache:
// scalar loads complete on lgkmcnt, so they never add to the vmcnt queue
// that tracks the staged loads
typedef const __attribute__((address_space(4))) int32_t* cint_ptr;
__device__ __forceinline__ int32_t uniform_load(const int32_t* base, int i) {
  return ((cint_ptr)base)[i];
}

// s_waitcnt immediate for "vmcnt <= n" with the other counters left alone
template <int N> struct VmCnt {
  static constexpr int imm = (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8);
};

// Workgroup barrier that is also a compiler fence: no memory access moves
// across it.
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

// End of a consumer's read phase: its fragment reads of the stage are
// complete (the slot may be re-staged after the barrier) and the fragments
// pass through the barrier as register operands, so no product that uses
// them can be scheduled before it.
#define MOE_WAIT_BARRIER_FRAGS(af, bf, sa, sw)                                                \
  asm volatile("s_waitcnt lgkmcnt(0)\n s_barrier"                                            \
               : "+v"(af[0]), "+v"(af[1]), "+v"(af[2]), "+v"(af[3]), "+v"(bf[0][0]),          \
                 "+v"(bf[0][1]), "+v"(bf[1][0]), "+v"(bf[1][1]), "+v"(sa), "+v"(sw)            \
               :                                                                             \
               : "memory")

// End of a matrix phase: the accumulators pass through the barrier, so the
// products of the phase stay between its two barriers.
#define MOE_BARRIER_ACC(acc)                                                                  \
  asm volatile("s_barrier"                                                                   \
               : "+v"(acc[0][0][0]), "+v"(acc[0][0][1]), "+v"(acc[0][1][0]), "+v"(acc[0][1][1]), \
                 "+v"(acc[1][0][0]), "+v"(acc[1][0][1]), "+v"(acc[1][1][0]), "+v"(acc[1][1][1]), \
                 "+v"(acc[2][0][0]), "+v"(acc[2][0][1]), "+v"(acc[2][1][0]), "+v"(acc[2][1][1]), \
                 "+v"(acc[3][0][0]), "+v"(acc[3][0][1]), "+v"(acc[3][1][0]), "+v"(acc[3][1][1])  \
               :                                                                             \
               : "memory")

// One 16x16 product over one stage: w = 16 weight rows (first operand),
// a = 16 activation rows (second operand); lane l holds 32 bytes of row
// l & 15 at K bytes 32 * (l >> 4).  Result: lane l, element r = output
// column 4 * (l >> 4) + r of activation row l & 15.
template <int DT>
__device__ __forceinline__ v4f mma_stage(const v8i& w, const v8i& a, v4f acc) {
  if constexpr (DT == DT_FP8) {
    // formats 0/0 = fp8 e4m3 for both operands; scale bytes 127 = 2^0
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, a, acc, 0, 0, 0, 127, 0, 127);
  } else if constexpr (DT == DT_BF16) {
    const i4 wl = __builtin_shufflevector(w, w, 0, 1, 2, 3), wh = __builtin_shufflevector(w, w, 4, 5, 6, 7);
    const i4 al = __builtin_shufflevector(a, a, 0, 1, 2, 3), ah = __builtin_shufflevector(a, a, 4, 5, 6, 7);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, wl), __builtin_bit_cast(v8bf, al),
                                                 acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, wh), __builtin_bit_cast(v8bf, ah),
                                                  acc, 0, 0, 0);
  } else {
#pragma unroll
    for (int m = 0; m < 8; ++m)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(w[m]), __int_as_float(a[m]), acc, 0, 0, 0);
    return acc;
  }
}

__shared__ __attribute__((aligned(16))) uint8_t s_ring[NST * STAGE];
__shared__ int s_mt_prefix[kMaxL + 1];
__shared__ float s_amax[4][BM];
__shared__ int s_part[kThreads];

// Tile id -> (expert, column block, row tile).  s_mt_prefix[e] = sum of row
// tiles of experts < e; tile ids are expert-major, then band of kBand row
// tiles, then column block, then row tile inside the band.  With one
// workgroup per CU, an XCD's 32 workgroups run 32 consecutive tiles at a
// time, roughly in step along K: with bands they cover about 8 row tiles x
// 4 column blocks, so each activation tile and each weight block of the
// round comes from HBM once and is shared through L2 (the row-tile-inner
// order alone made the 32 tiles of a large expert share one weight block
// but stream 32 activation tiles, re-reading every activation tile once per
// column block).
__device__ __forceinline__ void decode_tile(int L, int nb_count, int t, int& e, int& nb, int& mt) {
  int lo = 0, hi = L;           // largest e with s_mt_prefix[e]*nb_count <= t
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_mt_prefix[mid] * nb_count <= t) lo = mid; else hi = mid;
  }
  e = lo;
  const int mte = s_mt_prefix[e + 1] - s_mt_prefix[e];
  const int local = t - s_mt_prefix[e] * nb_count;
  const int b = local / (kBand * nb_count);
  const int r = local - b * kBand * nb_count;
  const int gm = min(kBand, mte - b * kBand);   // row tiles of this band
  nb = r / gm;
  mt = b * kBand + (r - nb * gm);
}

// One work item, workgroup-uniform: a tile, or one K-range piece of it.
struct Tile {
  int e, nb, rows_valid, n0;
  int64_t row0;
  bool half1;
  int ws0, ws1;                        // FP8: first weight-scale index of each half
  int ks0, nks;                        // K stages [ks0, ks0 + nks)
  int split;                           // -1: whole tile; else the piece's index
};

// 32 bytes of one LDS row for an MFMA operand: 16-byte chunks at c0 and c1
__device__ __forceinline__ v8i lds_frag(const uint8_t* row, int c0, int c1) {
  const i4 lo = *reinterpret_cast<const i4*>(row + c0);
  const i4 hi = *reinterpret_cast<const i4*>(row + c1);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int DT, int EPI>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(GemmArgs p) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform by construction; readfirstlane tells the compiler so, which
  // keeps the staged-load offsets in scalar registers (no per-load loop)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int ESZ = DT == DT_FP8 ? 1 : (DT == DT_BF16 ? 2 : 4);
  constexpr bool kFp8 = DT == DT_FP8;
  // direct-to-LDS loads per producer per stage (producer 0 issues one more,
  // the weight scales, first)
  constexpr int NLOAD = kFp8 ? 13 : 12;

  // ---- tile map: row tiles per expert, prefix over experts (block scan)
  {
    const int per = (p.L + kThreads - 1) / kThreads;
    const int e0 = tid * per;
    int s = 0;
    for (int e = e0; e < min(e0 + per, p.L); ++e)
      s += (eff_count(p.offsets[e], p.counts[e], p.rows_cap) + BM - 1) / BM;
    s_part[tid] = s;
    __syncthreads();
    for (int d = 1; d < kThreads; d <<= 1) {
      const int v = tid >= d ? s_part[tid - d] : 0;
      __syncthreads();
      s_part[tid] += v;
      __syncthreads();
    }
    int run = s_part[tid] - s;     // exclusive prefix of this thread's range
    for (int e = e0; e < min(e0 + per, p.L); ++e) {
      s_mt_prefix[e] = run;
      run += (eff_count(p.offsets[e], p.counts[e], p.rows_cap) + BM - 1) / BM;
    }
    if (tid == kThreads - 1) s_mt_prefix[p.L] = s_part[kThreads - 1];
    __syncthreads();
  }
  const int n_tiles = s_mt_prefix[p.L] * p.nb_count;
  const int kstages = p.K * ESZ / KB;
  const int kgroups = p.K / 128;              // FP8 scale groups along K
  const int64_t lda = static_cast<int64_t>(p.K) * ESZ;
  const bool stream = kstages >= 2;

  // Work plan.  The workgroups form 8 XCD groups (workgroup i runs on XCD
  // i mod 8); each group takes a contiguous chunk of the ordered tiles and
  // walks it in whole rounds, slot j taking tiles j, j + slots, ...  When a
  // workspace is bound (K of at least kMinSplitStages stages) and the
  // chunk's last round would leave at least three quarters of its slots
  // idle, each tile of that round is split along K into S = slots / tail
  // pieces (at least two stages a piece); a piece leaves its fp32 sums in
  // the workspace and a second kernel adds the pieces in order and applies
  // the epilogue.  (With fewer idle slots the saved time does not cover the
  // second launch and the partial traffic.)
  int c_begin, c_len, slots, slot, bstride;
  if (gridDim.x >= 8 && (gridDim.x & 7) == 0) {
    const int xcd = blockIdx.x & 7;
    slots = gridDim.x >> 3;
    slot = blockIdx.x >> 3;
    bstride = 8;
    c_begin = static_cast<int>((static_cast<int64_t>(n_tiles) * xcd) >> 3);
    c_len = static_cast<int>((static_cast<int64_t>(n_tiles) * (xcd + 1)) >> 3) - c_begin;
  } else {
    slots = gridDim.x;
    slot = blockIdx.x;
    bstride = 1;
    c_begin = 0;
    c_len = n_tiles;
  }
  const int full = c_len / slots;
  const int tail = c_len - full * slots;
  int S = 1;
  if (p.part != nullptr && stream && tail > 0) {
    S = min(slots / tail, kstages / 2);
    if (S < kMinPieces) S = 1;
  }
  S = __builtin_amdgcn_readfirstlane(S);
  const int my_full = full + ((S == 1 && slot < tail) ? 1 : 0);
  const bool has_piece = S > 1 && slot < tail * S;
  const int piece_tile = c_begin + full * slots + (has_piece ? slot / S : 0);
  const int piece_split = has_piece ? slot % S : 0;
  const int piece_ks0 = __builtin_amdgcn_readfirstlane(piece_split * kstages / S);
  const int piece_nks = __builtin_amdgcn_readfirstlane((piece_split + 1) * kstages / S) - piece_ks0;
  const int my_items = my_full + (has_piece ? 1 : 0);
  const int total = my_full * kstages + (has_piece ? piece_nks : 0);

  auto make_tile = [&](int t) {
    Tile c;
    int e, nb, mt;
    decode_tile(p.L, p.nb_count, t, e, nb, mt);
    c.e = __builtin_amdgcn_readfirstlane(e);
    c.nb = __builtin_amdgcn_readfirstlane(nb);
    mt = __builtin_amdgcn_readfirstlane(mt);
    const int64_t off = uniform_load(p.offsets, c.e);
    c.rows_valid = min(BM, eff_count(off, uniform_load(p.counts, c.e), p.rows_cap) - mt * BM);
    c.row0 = off + static_cast<int64_t>(mt) * BM;
    c.n0 = c.nb * p.nb_stride;
    c.half1 = c.n0 + p.half_stride < p.N;
    const int bpe = p.N / 128;                 // weight-scale block rows per expert
    c.ws0 = (c.e * bpe + c.n0 / 128) * kgroups;
    c.ws1 = (c.e * bpe + (c.half1 ? c.n0 + p.half_stride : c.n0) / 128) * kgroups;
    c.ks0 = 0;
    c.nks = kstages;
    c.split = -1;
    return c;
  };
  // item ti of this workgroup: its whole tiles, then its piece
  auto make_item = [&](int ti) {
    if (ti < my_full) return make_tile(c_begin + slot + ti * slots);
    Tile c = make_tile(piece_tile);
    c.ks0 = piece_ks0;
    c.nks = piece_nks;
    c.split = piece_split;
    return c;
  };
  // what the reduce kernel needs of this workgroup's piece
  if (p.desc != nullptr && tid == 0) {
    int* d = p.desc + static_cast<int64_t>(blockIdx.x) * kDescInts;
    if (has_piece) {
      const Tile c = make_tile(piece_tile);
      d[0] = 1;
      d[1] = S;
      d[2] = piece_split;
      d[3] = bstride;
      d[4] = c.rows_valid;
      d[5] = c.n0;
      d[6] = c.nb;
      d[7] = c.half1 ? 1 : 0;
      d[8] = static_cast<int>(static_cast<uint32_t>(c.row0));
      d[9] = static_cast<int>(c.row0 >> 32);
    } else {
      d[0] = 0;
    }
  }

  // The workgroup's items form one stream of stages: stage g lives in ring
  // slot g % NST, and item ti's stages follow those of item ti - 1.  With
  // kstages >= 2 (every item then has at least two stages), the first two
  // stages of the next item are staged during the last two stages of the
  // current one, so an item starts with its operands on the way instead of
  // refilling the pipeline.
  Tile cur{}, nxt{};
  if (my_items > 0) cur = make_item(0);
  if (my_items > 1) nxt = make_item(1);

  if (wave >= kConsumers) {
    // ================================================================ producers
    // Stage layout: chunk c (16 bytes) of row r sits at chunk c ^ swz(r) with
    // swz(r) = (r & 7) ^ ((r >> 3) & 1), which repeats every 16 rows; with it
    // the consumers' fragment reads (16 rows x 2 chunks per lane group) hit
    // every LDS bank once.  A direct-to-LDS load still writes 1 KB
    // contiguously: lane l fills row l >> 3 of an 8-row group, physical chunk
    // l & 7, so it fetches chunk (l & 7) ^ (l >> 3) ^ (group & 1).
    //   producer w stages A rows 32w + [0,32), W rows 64w + [0,64) (w < 2:
    //   half 0, else half 1), FP8 activation-scale positions 32w + [0,32),
    //   and producer 0 the two weight scales.  Scale position 64m + 4q + i
    //   holds row 64m + 16i + q, so a consumer lane of row group m reads the
    //   four scales of its rows 16i + q with one 16-byte read.
    const int pw = wave - kConsumers;
    const int srow = lane >> 3;
    const int voff_e = static_cast<int>(srow * lda) + (((lane & 7) ^ srow) << 4);
    const int voff_o = static_cast<int>(srow * lda) + (((lane & 7) ^ srow ^ 1) << 4);
    // packed W: rows of one tile stage are 128 bytes apart
    const int pvoff_e = srow * KB + (((lane & 7) ^ srow) << 4);
    const int pvoff_o = srow * KB + (((lane & 7) ^ srow ^ 1) << 4);
    const int64_t w_expert_bytes = p.w_packed ? static_cast<int64_t>(p.nb_count) * kstages * (2 * BH) * KB
                                              : p.N * lda;
    const int spos = 32 * (pw & 1) + (lane & 31);
    const int soff = (64 * (pw >> 1) + 16 * (spos & 3) + (spos >> 2)) * kgroups * 4;
    // Buffer resources: A over the whole expert-major buffer, W over one
    // expert's [N, K] block.  Rows past the end of a resource read as 0, so a
    // tail tile may read past its expert's last row without a clamp; those
    // rows are never stored.
    const int a_records = static_cast<int>(p.rows_cap * lda);
    const __amdgpu_buffer_rsrc_t rS = kFp8 ? __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(p.As), 0, static_cast<int>(p.rows_cap * kgroups * 4), kRsrcWord3)
                                           : __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.A), 0, 0,
                                                                               kRsrcWord3);
    typedef __attribute__((address_space(3))) void* lds_void;

    // half 0 / half 1 of this producer's loads of K stage ks of tile c into
    // ring slot s (FP8: 7 + 6 loads, plus the weight scales on producer 0)
    auto issue_half = [&](const Tile& c, int s, int ks, int half) {
      const __amdgpu_buffer_rsrc_t rW = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(p.W + static_cast<int64_t>(c.e) * w_expert_bytes), 0,
          static_cast<int>(w_expert_bytes), kRsrcWord3);
      uint8_t* st = s_ring + s * STAGE;
      if constexpr (kFp8) {
        if (half == 0 && pw == 0 && lane < 2) {
          const __amdgpu_buffer_rsrc_t rWs = __builtin_amdgcn_make_buffer_rsrc(
              const_cast<float*>(p.Ws), 0, p.L * (p.N / 128) * kgroups * 4, kRsrcWord3);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rWs, (lds_void)(st + A_BYTES + B_BYTES + AS_BYTES), 4,
                                                   (lane ? c.ws1 : c.ws0) * 4, ks * 4, 0, 0);
        }
      }
      const int a_off = static_cast<int>((c.row0 + 32 * pw) * lda) + ks * KB;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * half + jj;
        // 8-row groups wholly past the tile's valid rows (an expert's tail,
        // most of a decode tile) load through a resource of zero records:
        // the load still counts (the vmcnt bookkeeping stays fixed) but
        // every access is out of range, reads zeros and touches no memory;
        // those rows' results are never stored.  The resource is built per
        // load from the base pointer, so only the pointer and the record
        // count stay in registers.
        const bool live = 32 * pw + 8 * j < c.rows_valid;
        const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(p.A), 0, live ? a_records : 0, kRsrcWord3);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void)(st + (32 * pw + 8 * j) * KB), 16,
                                                 (j & 1) ? voff_o : voff_e,
                                                 a_off + static_cast<int>(8 * j * lda), 0, 0);
      }
      if (p.w_packed) {
        // tile stage (nb, ks) of the expert: 2*BH rows x 128 bytes, contiguous
        const int w_off = ((c.nb * kstages + ks) * (2 * BH) + 64 * pw) * KB;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int j = 4 * half + jj;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rW, (lds_void)(st + A_BYTES + (64 * pw + 8 * j) * KB), 16,
                                                   (j & 1) ? pvoff_o : pvoff_e, w_off + 8 * j * KB, 0, 0);
        }
      } else {
        const int w_off =
            static_cast<int>((c.n0 + (pw >> 1) * (c.half1 ? p.half_stride : 0) + 64 * (pw & 1)) * lda) + ks * KB;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int j = 4 * half + jj;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rW, (lds_void)(st + A_BYTES + (64 * pw + 8 * j) * KB), 16,
                                                   (j & 1) ? voff_o : voff_e,
                                                   w_off + static_cast<int>(8 * j * lda), 0, 0);
        }
      }
      if constexpr (kFp8) {
        if (half == 0 && lane < 32)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, (lds_void)(st + A_BYTES + B_BYTES + 128 * pw), 4, soff,
                                                   static_cast<int>(c.row0 * kgroups * 4) + ks * 4, 0, 0);
      }
    };

    int base = 0;                              // stream index of the item's first stage
    for (int ti = 0; ti < my_items; ++ti) {
      const int nks = cur.nks;
      auto staged = [&](int g) { return g < total && (stream || g < base + nks); };
      auto issue_g = [&](int g, int half) {
        const int ks = g - base;
        if (ks < nks) issue_half(cur, g % NST, cur.ks0 + ks, half);
        else issue_half(nxt, g % NST, nxt.ks0 + ks - nks, half);
      };
      if (ti == 0 || !stream) {
        __builtin_amdgcn_s_waitcnt(VmCnt<0>::imm);
        wg_barrier();                          // the ring is idle
        issue_g(base, 0);
        issue_g(base, 1);
        if (staged(base + 1)) {
          issue_g(base + 1, 0);
          issue_g(base + 1, 1);
          __builtin_amdgcn_s_waitcnt(VmCnt<NLOAD>::imm);
        } else {
          __builtin_amdgcn_s_waitcnt(VmCnt<0>::imm);
        }
        wg_barrier();                          // stage 0 has landed
      }
      for (int ks = 0; ks < nks; ++ks) {
        const int g = base + ks;
        const bool s2 = staged(g + 2);
        if (s2) issue_g(g + 2, 0);
        wg_barrier();
        if (s2) {
          issue_g(g + 2, 1);
          __builtin_amdgcn_s_waitcnt(VmCnt<NLOAD>::imm);   // stage g + 1 has landed
        } else if (staged(g + 1)) {
          __builtin_amdgcn_s_waitcnt(VmCnt<0>::imm);
        }
        wg_barrier();
      }
      wg_barrier();                            // the item's last phase
      if constexpr (EPI == EPI_SILU_FP8) {
        if (cur.split < 0) wg_barrier();       // consumers' row-amax exchange
      }
      base += nks;
      cur = nxt;
      if (ti + 2 < my_items) nxt = make_item(ti + 2);
    }
    return;
  }

  // ================================================================== consumers
  const int wm = wave >> 2;      // 64-row slice of the tile = consumer group
  const int wn = wave & 3;       // 32-column slice of each half
  // fragment reads: row (lane & 15) of a 16-row block, bytes 32*(lane>>4)..+32
  const int frow = lane & 15;
  const int fsw = (frow & 7) ^ (frow >> 3);
  const int fc0 = ((2 * (lane >> 4)) ^ fsw) << 4;
  const int fc1 = ((2 * (lane >> 4) + 1) ^ fsw) << 4;
  const int a_frag = (wm * 64 + frow) * KB;
  const int b_frag = A_BYTES + (wn * 32 + frow) * KB;
  const int s_frag = A_BYTES + B_BYTES + wm * 256 + frow * 16;
  const int w_frag = A_BYTES + B_BYTES + AS_BYTES;

  int base = 0;
  for (int ti = 0; ti < my_items; ++ti) {
    const int nks = cur.nks;
    const int nb = cur.nb, rows_valid = cur.rows_valid, n0 = cur.n0;
    const int64_t row0 = cur.row0;
    const bool half1 = cur.half1;

    v4f acc[4][2][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][h][j] = v4f{0.f, 0.f, 0.f, 0.f};

    if (ti == 0 || !stream) {
      wg_barrier();                            // producers: ring idle
      wg_barrier();                            // producers: stage 0 landed
    }
    // Group g reads stage ks in phase 2*ks + g and multiplies it in phase
    // 2*ks + g + 1 (group 1 waits out phase 0, group 0 the last phase).
    if (wm == 1) wg_barrier();
    for (int ks = 0; ks < nks; ++ks) {
      const uint8_t* sb = s_ring + ((base + ks) % NST) * STAGE;
      v8i af[4], bf[2][2];
      i4 sa;
      f2 sw;
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = lds_frag(sb + a_frag + i * 16 * KB, fc0, fc1);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 2; ++j) bf[h][j] = lds_frag(sb + b_frag + (h * BH + j * 16) * KB, fc0, fc1);
      if constexpr (kFp8) {
        sa = *reinterpret_cast<const i4*>(sb + s_frag);
        sw = *reinterpret_cast<const f2*>(sb + w_frag);
      } else {
        sa = i4{0, 0, 0, 0};
        sw = f2{0.f, 0.f};
      }
      MOE_WAIT_BARRIER_FRAGS(af, bf, sa, sw);
      if constexpr (kFp8) {
        // 16 products P, each folded in as acc += P * (sa * sw) while the
        // matrix core works on later products.  Product n covers row block
        // i = n >> 2, half h = (n >> 1) & 1, column block j = n & 1.
        // Two products ahead: the fold of product n follows the matrix op of
        // product n + 2, far enough behind product n for its result to be
        // ready without a stall (one product ahead, every fold waits on the
        // matrix op issued just before it).  Scheduling fences pin the order.
        const v4f zero = {0.f, 0.f, 0.f, 0.f};
        v4f pr[3];
        float f = 0.f;
        pr[0] = mma_stage<DT>(bf[0][0], af[0], zero);
        pr[1] = mma_stage<DT>(bf[0][1], af[0], zero);
#pragma unroll
        for (int n = 0; n < 16; ++n) {
          if (n + 2 < 16) {
            const int m = n + 2;
            pr[m % 3] = mma_stage<DT>(bf[(m >> 1) & 1][m & 1], af[m >> 2], zero);
          }
          __builtin_amdgcn_sched_barrier(0);
          const int i = n >> 2, h = (n >> 1) & 1, j = n & 1;
          if (j == 0) f = __int_as_float(sa[i]) * sw[h];
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][h][j][r] = fmaf(pr[n % 3][r], f, acc[i][h][j][r]);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i][h][j] = mma_stage<DT>(bf[h][j], af[i], acc[i][h][j]);
      }
      MOE_BARRIER_ACC(acc);
    }
    if (wm == 0) wg_barrier();

    // ---- epilogue.  Lane holds, for row block i, half h, column block j,
    // activation row 64*wm + 16*i + (lane & 15) and columns
    // 32*wn + 16*j + 4*(lane >> 4) + r of the half, r = 0..3.
    const int mrow = wm * 64 + frow;
    const int ncol = wn * 32 + 4 * (lane >> 4);
    if (cur.split >= 0) {
      // a K piece: its fp32 sums go to this workgroup's partial tile,
      // row-major [BM][2*BH] (half h at columns h*BH + [0,BH))
      float* pp = p.part + static_cast<int64_t>(blockIdx.x) * kPartFloats;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (mrow + 16 * i >= rows_valid) continue;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            *reinterpret_cast<v4f*>(pp + (mrow + 16 * i) * (2 * BH) + h * BH + ncol + 16 * j) = acc[i][h][j];
      }
    } else if constexpr (EPI == EPI_SCATTER_F32) {
      // out[q, n] * w[t, k] added into y_acc[t, n] (t, k the row's route):
      // the combine's weighted sum made in the down GEMM's epilogue, summed
      // in whatever order the atomic adds arrive
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = mrow + 16 * i;
        if (row >= rows_valid) continue;
        const int src = p.row_src[row0 + row];
        const float w = p.route_w[src];
        float* yrow = p.y_acc + static_cast<int64_t>(src / p.topk) * p.ldo;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (h == 1 && !half1) continue;
          const int ncol0 = n0 + h * p.half_stride;
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              unsafeAtomicAdd(yrow + ncol0 + ncol + 16 * j + r, acc[i][h][j][r] * w);
        }
      }
    } else if constexpr (EPI == EPI_STORE_F32 || EPI == EPI_STORE_BF16) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (h == 1 && !half1) continue;
        const int ncol0 = n0 + h * p.half_stride;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = mrow + 16 * i;
          if (row >= rows_valid) continue;
          if constexpr (EPI == EPI_STORE_F32) {
            const int64_t o = (row0 + row) * p.ldo + ncol0 + ncol;
#pragma unroll
            for (int j = 0; j < 2; ++j) *reinterpret_cast<v4f*>(static_cast<float*>(p.out) + o + 16 * j) = acc[i][h][j];
          } else {
            // lanes 16 apart (column groups q, q ^ 1) trade one 4-column
            // block, so each lane stores 8 contiguous columns (16 bytes)
            const bool odd = (lane >> 4) & 1;
            const v4f give = odd ? acc[i][h][0] : acc[i][h][1];
            v4f got;
#pragma unroll
            for (int r = 0; r < 4; ++r) got[r] = __shfl_xor(give[r], 16);
            const v4f lo = odd ? got : acc[i][h][0];
            const v4f hi = odd ? acc[i][h][1] : got;
            const int c0 = odd ? 16 + 4 * ((lane >> 4) - 1) : 4 * (lane >> 4);
            const int64_t o = (row0 + row) * p.ldo + ncol0 + wn * 32 + c0;
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) + o) = make_uint4(
                static_cast<uint32_t>(moe::f32_to_bf16(lo[0])) | (static_cast<uint32_t>(moe::f32_to_bf16(lo[1])) << 16),
                static_cast<uint32_t>(moe::f32_to_bf16(lo[2])) | (static_cast<uint32_t>(moe::f32_to_bf16(lo[3])) << 16),
                static_cast<uint32_t>(moe::f32_to_bf16(hi[0])) | (static_cast<uint32_t>(moe::f32_to_bf16(hi[1])) << 16),
                static_cast<uint32_t>(moe::f32_to_bf16(hi[2])) | (static_cast<uint32_t>(moe::f32_to_bf16(hi[3])) << 16));
          }
        }
      }
    } else if constexpr (EPI == EPI_SILU_BWD) {
      // dG of the tile's 128 Z columns from its gate and up sums and dZ:
      // gate gradients to dG columns nb*128 + c, up gradients to I + nb*128 + c.
      // Every dZ load of the tile is issued before the first is used.
      const int64_t zcol = static_cast<int64_t>(nb) * BH + ncol;
      float dz[4][2][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = mrow + 16 * i;
        const int64_t q = row0 + min(row, rows_valid - 1);     // rows past the valid ones read a valid row
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (p.dz_f32) {
            const v4f v = *reinterpret_cast<const v4f*>(p.dz + (q * (p.ldo / 2) + zcol + 16 * j) * 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) dz[i][j][r] = v[r];
          } else {
            const uint2 v = *reinterpret_cast<const uint2*>(p.dz + (q * (p.ldo / 2) + zcol + 16 * j) * 2);
            dz[i][j][0] = __uint_as_float(v.x << 16);
            dz[i][j][1] = __uint_as_float(v.x & 0xffff0000u);
            dz[i][j][2] = __uint_as_float(v.y << 16);
            dz[i][j][3] = __uint_as_float(v.y & 0xffff0000u);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = mrow + 16 * i;
        if (row >= rows_valid) continue;
        const int64_t o = (row0 + row) * p.ldo + zcol;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          float dgt[4], dup[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) moe::silu_mul_grad(acc[i][0][j][r], acc[i][1][j][r], dz[i][j][r], dgt[r], dup[r]);
          if (p.out_f32) {
            float* d = static_cast<float*>(p.out) + o + 16 * j;
            *reinterpret_cast<v4f*>(d) = v4f{dgt[0], dgt[1], dgt[2], dgt[3]};
            *reinterpret_cast<v4f*>(d + p.half_stride) = v4f{dup[0], dup[1], dup[2], dup[3]};
          } else {
            uint16_t* d = static_cast<uint16_t*>(p.out) + o + 16 * j;
            *reinterpret_cast<uint2*>(d) = make_uint2(
                static_cast<uint32_t>(moe::f32_to_bf16(dgt[0])) | (static_cast<uint32_t>(moe::f32_to_bf16(dgt[1])) << 16),
                static_cast<uint32_t>(moe::f32_to_bf16(dgt[2])) | (static_cast<uint32_t>(moe::f32_to_bf16(dgt[3])) << 16));
            *reinterpret_cast<uint2*>(d + p.half_stride) = make_uint2(
                static_cast<uint32_t>(moe::f32_to_bf16(dup[0])) | (static_cast<uint32_t>(moe::f32_to_bf16(dup[1])) << 16),
                static_cast<uint32_t>(moe::f32_to_bf16(dup[2])) | (static_cast<uint32_t>(moe::f32_to_bf16(dup[3])) << 16));
          }
        }
      }
    } else {
      // Z = SiLU(gate) * up, columns nb*128 + [0,128) of Z
      float z[4][2][4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) z[i][j][r] = moe::silu(acc[i][0][j][r]) * acc[i][1][j][r];
      const int64_t zcol0 = static_cast<int64_t>(nb) * BH;
      if constexpr (EPI == EPI_SILU_FP8) {
        // per-row amax over the 128 Z columns: 8 in-lane, 4 lanes, 4 waves
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float m = 0.f;
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(z[i][j][r]));
          m = fmaxf(m, __shfl_xor(m, 16));
          m = fmaxf(m, __shfl_xor(m, 32));
          if (lane < 16) s_amax[wn][mrow + 16 * i] = m;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = mrow + 16 * i;
          const float amax = moe::fp8_group_amax_clamp(
              fmaxf(fmaxf(s_amax[0][row], s_amax[1][row]), fmaxf(s_amax[2][row], s_amax[3][row])));
          const float inv = moe::fp8_group_inv(amax);
          if (row >= rows_valid) continue;
          uint8_t* zrow = static_cast<uint8_t*>(p.out) + (row0 + row) * p.ldo + zcol0;
#pragma unroll
          for (int j = 0; j < 2; ++j)
            *reinterpret_cast<uint32_t*>(zrow + ncol + 16 * j) = moe::f32x4_to_e4m3(
                z[i][j][0] * inv, z[i][j][1] * inv, z[i][j][2] * inv, z[i][j][3] * inv);
          if (wn == 0 && lane < 16)
            p.out_scales[(row0 + row) * (p.ldo / 128) + nb] = moe::fp8_group_scale(amax);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = mrow + 16 * i;
          if (row >= rows_valid) continue;
          const int64_t o = (row0 + row) * p.ldo + zcol0 + ncol;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            if constexpr (EPI == EPI_SILU_F32) {
              *reinterpret_cast<v4f*>(static_cast<float*>(p.out) + o + 16 * j) =
                  v4f{z[i][j][0], z[i][j][1], z[i][j][2], z[i][j][3]};
            } else {
              const uint2 w = make_uint2(
                  static_cast<uint32_t>(moe::f32_to_bf16(z[i][j][0])) |
                      (static_cast<uint32_t>(moe::f32_to_bf16(z[i][j][1])) << 16),
                  static_cast<uint32_t>(moe::f32_to_bf16(z[i][j][2])) |
                      (static_cast<uint32_t>(moe::f32_to_bf16(z[i][j][3])) << 16));
              *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + o + 16 * j) = w;
            }
          }
        }
      }
    }
    base += nks;
    cur = nxt;
    if (ti + 2 < my_items) nxt = make_item(ti + 2);
  }
}

// Second kernel of a K-split last round: workgroup b of the GEMM's grid
// left a piece in partial tile b.  Blocks (b, y) of a tile's first piece add
// the tile's S pieces in piece order (partial tiles b, b + bstride, ...) for
// rows 8y .. 8y + 7 and apply the GEMM's epilogue to the valid ones.  A
// half-wave of 32 lanes takes one row, 4 columns per lane per half.
constexpr int kReduceThreads = 256;
constexpr int kReduceRows = 2 * (kReduceThreads / MOE_WAVE);   // rows per block
constexpr int kReduceBatch = 8;                                 // pieces loaded before adding

template <int EPI>
__global__ __launch_bounds__(kReduceThreads) void gemm_piece_reduce_kernel(GemmArgs p) {
  if constexpr (EPI == EPI_SCATTER_F32) return;     // never split: launched without a workspace
  const int* d = p.desc + static_cast<int64_t>(blockIdx.x) * kDescInts;
  if (d[0] == 0 || d[2] != 0) return;              // no piece, or not a tile's first one
  const int S = d[1], bstride = d[3], rows_valid = d[4], n0 = d[5], nb = d[6];
  const bool half1 = d[7] != 0;
  const int64_t row0 = static_cast<int64_t>(static_cast<uint32_t>(d[8])) | (static_cast<int64_t>(d[9]) << 32);
  const int lane = threadIdx.x & 63;
  const int c4 = 4 * (lane & 31);
  const int r = blockIdx.y * kReduceRows + 2 * (threadIdx.x / MOE_WAVE) + (lane >> 5);
  if (r < rows_valid) {
    // pieces are added in order 0, 1, ..., S-1; the loads of a batch of
    // kReduceBatch pieces are all issued before the first add, so a thread
    // waits for one memory round trip per batch rather than per piece
    const float* src = p.part + static_cast<int64_t>(blockIdx.x) * kPartFloats + r * (2 * BH) + c4;
    const int64_t pstride = static_cast<int64_t>(bstride) * kPartFloats;
    v4f g[2];
    for (int k0 = 0; k0 < S; k0 += kReduceBatch) {
      v4f v[kReduceBatch][2];
#pragma unroll
      for (int u = 0; u < kReduceBatch; ++u)
        if (k0 + u < S)
#pragma unroll
          for (int h = 0; h < 2; ++h) v[u][h] = *reinterpret_cast<const v4f*>(src + (k0 + u) * pstride + h * BH);
#pragma unroll
      for (int u = 0; u < kReduceBatch; ++u)
        if (k0 + u < S)
#pragma unroll
          for (int h = 0; h < 2; ++h) g[h] = (k0 + u == 0) ? v[u][h] : g[h] + v[u][h];
    }
    if constexpr (EPI == EPI_STORE_F32 || EPI == EPI_STORE_BF16) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (h == 1 && !half1) continue;
        const int64_t o = (row0 + r) * p.ldo + n0 + h * p.half_stride + c4;
        if constexpr (EPI == EPI_STORE_F32) {
          *reinterpret_cast<v4f*>(static_cast<float*>(p.out) + o) = g[h];
        } else {
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + o) = make_uint2(
              static_cast<uint32_t>(moe::f32_to_bf16(g[h][0])) | (static_cast<uint32_t>(moe::f32_to_bf16(g[h][1])) << 16),
              static_cast<uint32_t>(moe::f32_to_bf16(g[h][2])) | (static_cast<uint32_t>(moe::f32_to_bf16(g[h][3])) << 16));
        }
      }
    } else if constexpr (EPI == EPI_SILU_BWD) {
      const int64_t q = row0 + r;
      const int64_t zc = q * (p.ldo / 2) + static_cast<int64_t>(nb) * BH + c4;
      float dz[4];
      if (p.dz_f32) {
        const v4f v = *reinterpret_cast<const v4f*>(p.dz + zc * 4);
#pragma unroll
        for (int k = 0; k < 4; ++k) dz[k] = v[k];
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(p.dz + zc * 2);
        dz[0] = __uint_as_float(v.x << 16);
        dz[1] = __uint_as_float(v.x & 0xffff0000u);
        dz[2] = __uint_as_float(v.y << 16);
        dz[3] = __uint_as_float(v.y & 0xffff0000u);
      }
      float dgt[4], dup[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) moe::silu_mul_grad(g[0][k], g[1][k], dz[k], dgt[k], dup[k]);
      const int64_t o = q * p.ldo + static_cast<int64_t>(nb) * BH + c4;
      if (p.out_f32) {
        *reinterpret_cast<v4f*>(static_cast<float*>(p.out) + o) = v4f{dgt[0], dgt[1], dgt[2], dgt[3]};
        *reinterpret_cast<v4f*>(static_cast<float*>(p.out) + o + p.half_stride) = v4f{dup[0], dup[1], dup[2], dup[3]};
      } else {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + o) = make_uint2(
            static_cast<uint32_t>(moe::f32_to_bf16(dgt[0])) | (static_cast<uint32_t>(moe::f32_to_bf16(dgt[1])) << 16),
            static_cast<uint32_t>(moe::f32_to_bf16(dgt[2])) | (static_cast<uint32_t>(moe::f32_to_bf16(dgt[3])) << 16));
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + o + p.half_stride) = make_uint2(
            static_cast<uint32_t>(moe::f32_to_bf16(dup[0])) | (static_cast<uint32_t>(moe::f32_to_bf16(dup[1])) << 16),
            static_cast<uint32_t>(moe::f32_to_bf16(dup[2])) | (static_cast<uint32_t>(moe::f32_to_bf16(dup[3])) << 16));
      }
    } else {
      float z[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) z[k] = moe::silu(g[0][k]) * g[1][k];
      const int64_t o = (row0 + r) * p.ldo + static_cast<int64_t>(nb) * BH + c4;
      if constexpr (EPI == EPI_SILU_FP8) {
        float m = fmaxf(fmaxf(fabsf(z[0]), fabsf(z[1])), fmaxf(fabsf(z[2]), fabsf(z[3])));
        m = fmaxf(m, __shfl_xor(m, 1));
        m = fmaxf(m, __shfl_xor(m, 2));
        m = fmaxf(m, __shfl_xor(m, 4));
        m = fmaxf(m, __shfl_xor(m, 8));
        m = fmaxf(m, __shfl_xor(m, 16));
        const float amax = moe::fp8_group_amax_clamp(m);
        const float inv = moe::fp8_group_inv(amax);
        *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(p.out) + o) =
            moe::f32x4_to_e4m3(z[0] * inv, z[1] * inv, z[2] * inv, z[3] * inv);
        if ((lane & 31) == 0) p.out_scales[(row0 + r) * (p.ldo / 128) + nb] = moe::fp8_group_scale(amax);
      } else if constexpr (EPI == EPI_SILU_F32) {
        *reinterpret_cast<v4f*>(static_cast<float*>(p.out) + o) = v4f{z[0], z[1], z[2], z[3]};
      } else {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + o) = make_uint2(
            static_cast<uint32_t>(moe::f32_to_bf16(z[0])) | (static_cast<uint32_t>(moe::f32_to_bf16(z[1])) << 16),
            static_cast<uint32_t>(moe::f32_to_bf16(z[2])) | (static_cast<uint32_t>(moe::f32_to_bf16(z[3])) << 16));
      }
    }
  }
}

// W13 [L, 2I, H] -> packed [L][I/128][H*esz/128][2*BH rows][KB bytes]: tile
// stage (nb, ks) holds gate rows nb*128 + [0,128) then up rows
// I + nb*128 + [0,128), bytes [ks*128, ks*128 + 128) of each, so the
// gate/up GEMM stages it with 1 KB contiguous loads.  One thread per
// 16-byte chunk.
__global__ __launch_bounds__(256) void pack_w13_kernel(const uint8_t* __restrict__ w, int64_t n_chunks, int I,
                                                      int row_bytes, uint8_t* __restrict__ out) {
  const int ks_count = row_bytes / KB;
  const int nb_count = I / BH;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n_chunks;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int c16 = static_cast<int>(i & 7);
    int64_t q = i >> 3;
    const int r = static_cast<int>(q % (2 * BH));
    q /= 2 * BH;
    const int ks = static_cast<int>(q % ks_count);
    q /= ks_count;
    const int nb = static_cast<int>(q % nb_count);
    const int64_t e = q / nb_count;
    const int64_t wrow = (r < BH ? 0 : I) + static_cast<int64_t>(nb) * BH + (r & (BH - 1));
    const uint4 v = *reinterpret_cast<const uint4*>(w + (e * 2 * I + wrow) * row_bytes + ks * KB + c16 * 16);
    *reinterpret_cast<uint4*>(out + i * 16) = v;
  }
}

int gemm_grid(int64_t max_tiles) {
  int grid = static_cast<int>(std::min<int64_t>(max_tiles, moe_host::device_cu_count()));
  if (grid >= 8) grid &= ~7;
  return grid;
}

template <int DT, int EPI>
moe_status launch(const GemmArgs& a, int max_mtiles, hipStream_t stream) {
  const int64_t max_tiles = static_cast<int64_t>(max_mtiles) * a.nb_count;
  if (max_tiles <= 0) return MOE_OK;
  const int grid = gemm_grid(max_tiles);
  grouped_gemm_kernel<DT, EPI><<<grid, kThreads, 0, stream>>>(a);
  MOE_LAUNCH_CHECK();
  if (a.part != nullptr) {
    gemm_piece_reduce_kernel<EPI><<<dim3(grid, BM / kReduceRows), kReduceThreads, 0, stream>>>(a);
    MOE_LAUNCH_CHECK();
  }
  return MOE_OK;
}

// workspace layout: partial tiles [grid][kPartFloats] fp32, then
// descriptors [grid][kDescInts]
size_t workspace_bytes_for_grid(int grid) {
  return static_cast<size_t>(grid) * (kPartFloats * sizeof(float) + kDescInts * sizeof(int));
}

// Point the K-split at the caller's workspace; MOE_ERR_WORKSPACE if it is
// given but too small for the launch's grid.
moe_status bind_workspace(GemmArgs& g, int max_mtiles, int elem_bytes, void* ws, size_t ws_bytes) {
  g.part = nullptr;
  g.desc = nullptr;
  if (ws == nullptr) return MOE_OK;
  const int64_t max_tiles = static_cast<int64_t>(max_mtiles) * g.nb_count;
  if (max_tiles <= 0) return MOE_OK;
  const int grid = gemm_grid(max_tiles);
  if (ws_bytes < workspace_bytes_for_grid(grid)) return MOE_ERR_WORKSPACE;
  MOE_CHECK((reinterpret_cast<uintptr_t>(ws) & 15) == 0, MOE_ERR_INVALID_ARG);
  // too few K stages for a split: no second launch
  if (static_cast<int64_t>(g.K) * elem_bytes / KB < kMinSplitStages) return MOE_OK;
  g.part = static_cast<float*>(ws);
  g.desc = reinterpret_cast<int*>(static_cast<uint8_t*>(ws) + static_cast<size_t>(grid) * kPartFloats * sizeof(float));
  return MOE_OK;
}

int dt_index(moe_dtype d) { return d == MOE_F32 ? DT_F32 : (d == MOE_BF16 ? DT_BF16 : DT_FP8); }

template <int EPI>
moe_status dispatch_dt(moe_dtype dt, const GemmArgs& a, int max_mtiles, hipStream_t s) {
  switch (dt_index(dt)) {
    case DT_F32: return launch<DT_F32, EPI>(a, max_mtiles, s);
    case DT_BF16: return launch<DT_BF16, EPI>(a, max_mtiles, s);
    default: return launch<DT_FP8, EPI>(a, max_mtiles, s);
  }
}

int max_row_tiles(int64_t rows_cap, int L) {
  return static_cast<int>(std::min<int64_t>(rows_cap / BM + L, (rows_cap + BM - 1) / BM + L));
}

// Staged loads address A and one expert's W through 32-bit buffer
// resources with signed 32-bit offsets: both must span less than 2 GiB.
bool offsets_fit(int64_t K_bytes, int64_t N, int64_t rows_cap) {
  const int64_t lim = int64_t(1) << 31;
  return K_bytes * N < lim && K_bytes * (rows_cap + BM) < lim;
}

}  // namespace

extern "C" moe_status moe_pack_w13(const void* w13, moe_dtype w_dt, int L, int H, int I, void* w13_packed,
                                   hipStream_t stream) {
  MOE_CHECK(L >= 1 && H > 0 && I > 0 && moe_host::valid_dtype(w_dt), MOE_ERR_INVALID_ARG);
  MOE_CHECK(H % 128 == 0 && I % 128 == 0, MOE_ERR_UNSUPPORTED);
  MOE_CHECK(w13 && w13_packed && w13 != w13_packed, MOE_ERR_INVALID_ARG);
  MOE_CHECK(((reinterpret_cast<uintptr_t>(w13) | reinterpret_cast<uintptr_t>(w13_packed)) & 15) == 0,
            MOE_ERR_INVALID_ARG);
  const int row_bytes = H * moe_host::elem_bytes(w_dt);
  const int64_t n_chunks = static_cast<int64_t>(L) * 2 * I * row_bytes / 16;
  const int grid = static_cast<int>(std::min<int64_t>((n_chunks + 255) / 256, 65536));
  pack_w13_kernel<<<grid, 256, 0, stream>>>(static_cast<const uint8_t*>(w13), n_chunks, I, row_bytes,
                                           static_cast<uint8_t*>(w13_packed));
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

extern "C" moe_status moe_grouped_gemm_w13(const void* a, moe_dtype a_dt, const float* a_scales,
                                           const void* w13, moe_dtype w_dt, const float* w13_scales,
                                           moe_weight_layout w13_layout,
                                           const int32_t* counts, const int32_t* offsets, int L,
                                           int64_t rows_cap, int H, int I, moe_w13_epilogue epi,
                                           void* out, moe_dtype out_dt, float* out_scales,
                                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  MOE_CHECK(L >= 1 && L <= kMaxL && rows_cap >= 0 && H > 0 && I > 0, MOE_ERR_INVALID_ARG);
  MOE_CHECK(moe_host::valid_dtype(a_dt) && moe_host::valid_dtype(w_dt) && moe_host::valid_dtype(out_dt),
            MOE_ERR_INVALID_ARG);
  MOE_CHECK(epi == MOE_EPI_STORE_G || epi == MOE_EPI_SILU_MUL, MOE_ERR_INVALID_ARG);
  MOE_CHECK(w13_layout == MOE_W_ROW_MAJOR || w13_layout == MOE_W_PACKED, MOE_ERR_INVALID_ARG);
  MOE_CHECK(a_dt == w_dt, MOE_ERR_UNSUPPORTED);
  MOE_CHECK(H % 128 == 0 && I % 128 == 0, MOE_ERR_UNSUPPORTED);
  MOE_CHECK(epi == MOE_EPI_SILU_MUL || out_dt == MOE_F32, MOE_ERR_UNSUPPORTED);
  MOE_CHECK(offsets_fit(static_cast<int64_t>(H) * moe_host::elem_bytes(a_dt), 2 * static_cast<int64_t>(I),
                        rows_cap),
            MOE_ERR_UNSUPPORTED);
  MOE_CHECK(a_dt != MOE_FP8_E4M3 || H <= 128 * 128, MOE_ERR_UNSUPPORTED);
  if (rows_cap == 0) return MOE_OK;
  MOE_CHECK(a && w13 && counts && offsets && out, MOE_ERR_INVALID_ARG);
  MOE_CHECK(a_dt != MOE_FP8_E4M3 || (a_scales && w13_scales), MOE_ERR_INVALID_ARG);
  MOE_CHECK(!(epi == MOE_EPI_SILU_MUL && out_dt == MOE_FP8_E4M3) || out_scales, MOE_ERR_INVALID_ARG);
  GemmArgs g{};
  g.A = static_cast<const uint8_t*>(a);
  g.As = a_scales;
  g.W = static_cast<const uint8_t*>(w13);
  g.Ws = w13_scales;
  g.counts = counts;
  g.offsets = offsets;
  g.L = L;
  g.K = H;
  g.N = 2 * I;
  g.nb_count = I / BH;
  g.nb_stride = BH;
  g.half_stride = I;
  g.rows_cap = rows_cap;
  g.out = out;
  g.out_scales = out_scales;
  g.w_packed = w13_layout == MOE_W_PACKED;
  const int mt = max_row_tiles(rows_cap, L);
  const moe_status ws_st = bind_workspace(g, mt, moe_host::elem_bytes(a_dt), workspace, workspace_bytes);
  if (ws_st != MOE_OK) return ws_st;
  if (epi == MOE_EPI_STORE_G) {
    g.ldo = 2 * I;
    return dispatch_dt<EPI_STORE_F32>(a_dt, g, mt, stream);
  }
  g.ldo = I;
  switch (out_dt) {
    case MOE_F32: return dispatch_dt<EPI_SILU_F32>(a_dt, g, mt, stream);
    case MOE_BF16: return dispatch_dt<EPI_SILU_BF16>(a_dt, g, mt, stream);
    default: return dispatch_dt<EPI_SILU_FP8>(a_dt, g, mt, stream);
  }
}

extern "C" moe_status moe_grouped_gemm_w13_silu_backward(const void* a, moe_dtype a_dt, const void* w13,
                                                        moe_dtype w_dt, moe_weight_layout w13_layout,
                                                        const int32_t* counts, const int32_t* offsets, int L,
                                                        int64_t rows_cap, int H, int I, const void* dz,
                                                        moe_dtype dz_dt, void* dg, moe_dtype dg_dt,
                                                        void* workspace, size_t workspace_bytes,
                                                        hipStream_t stream) {
  MOE_CHECK(L >= 1 && L <= kMaxL && rows_cap >= 0 && H > 0 && I > 0, MOE_ERR_INVALID_ARG);
  MOE_CHECK(moe_host::valid_dtype(a_dt) && moe_host::valid_dtype(w_dt) && moe_host::valid_dtype(dz_dt) &&
                moe_host::valid_dtype(dg_dt),
            MOE_ERR_INVALID_ARG);
  MOE_CHECK(w13_layout == MOE_W_ROW_MAJOR || w13_layout == MOE_W_PACKED, MOE_ERR_INVALID_ARG);
  MOE_CHECK(a_dt == w_dt && a_dt != MOE_FP8_E4M3, MOE_ERR_UNSUPPORTED);
  MOE_CHECK(dz_dt != MOE_FP8_E4M3 && dg_dt != MOE_FP8_E4M3, MOE_ERR_UNSUPPORTED);
  MOE_CHECK(H % 128 == 0 && I % 128 == 0, MOE_ERR_UNSUPPORTED);
  MOE_CHECK(offsets_fit(static_cast<int64_t>(H) * moe_host::elem_bytes(a_dt), 2 * static_cast<int64_t>(I),
                        rows_cap),
            MOE_ERR_UNSUPPORTED);
  if (rows_cap == 0) return MOE_OK;
  MOE_CHECK(a && w13 && counts && offsets && dz && dg, MOE_ERR_INVALID_ARG);
  GemmArgs g{};
  g.A = static_cast<const uint8_t*>(a);
  g.W = static_cast<const uint8_t*>(w13);
  g.counts = counts;
  g.offsets = offsets;
  g.L = L;
  g.K = H;
  g.N = 2 * I;
  g.nb_count = I / BH;
  g.nb_stride = BH;
  g.half_stride = I;
  g.rows_cap = rows_cap;
  g.out = dg;
  g.ldo = 2 * I;
  g.dz = static_cast<const uint8_t*>(dz);
  g.dz_f32 = dz_dt == MOE_F32;
  g.out_f32 = dg_dt == MOE_F32;
  g.w_packed = w13_layout == MOE_W_PACKED;
  const int mt = max_row_tiles(rows_cap, L);
  const moe_status ws_st = bind_workspace(g, mt, moe_host::elem_bytes(a_dt), workspace, workspace_bytes);
  if (ws_st != MOE_OK) return ws_st;
  // bf16 and fp32 only: the backward has no FP8 form
  if (a_dt == MOE_F32) return launch<DT_F32, EPI_SILU_BWD>(g, mt, stream);
  return launch<DT_BF16, EPI_SILU_BWD>(g, mt, stream);
}

extern "C" moe_status moe_grouped_gemm_w2(const void* z, moe_dtype z_dt, const float* z_scales,
                                          const void* w2, moe_dtype w_dt, const float* w2_scales,
                                          const int32_t* counts, const int32_t* offsets, int L,
                                          int64_t rows_cap, int H, int I, void* out,
                                          moe_dtype out_dt, void* workspace, size_t workspace_bytes,
                                          hipStream_t stream) {
  MOE_CHECK(L >= 1 && L <= kMaxL && rows_cap >= 0 && H > 0 && I > 0, MOE_ERR_INVALID_ARG);
  MOE_CHECK(moe_host::valid_dtype(z_dt) && moe_host::valid_dtype(w_dt) && moe_host::valid_dtype(out_dt),
            MOE_ERR_INVALID_ARG);
  MOE_CHECK(z_dt == w_dt, MOE_ERR_UNSUPPORTED);
  MOE_CHECK(H % 128 == 0 && I % 128 == 0, MOE_ERR_UNSUPPORTED);
  MOE_CHECK(out_dt == MOE_F32 || out_dt == MOE_BF16, MOE_ERR_UNSUPPORTED);
  MOE_CHECK(offsets_fit(static_cast<int64_t>(I) * moe_host::elem_bytes(z_dt), H, rows_cap),
            MOE_ERR_UNSUPPORTED);
  MOE_CHECK(z_dt != MOE_FP8_E4M3 || I <= 128 * 128, MOE_ERR_UNSUPPORTED);
  if (rows_cap == 0) return MOE_OK;
  MOE_CHECK(z && w2 && counts && offsets && out, MOE_ERR_INVALID_ARG);
  MOE_CHECK(z_dt != MOE_FP8_E4M3 || (z_scales && w2_scales), MOE_ERR_INVALID_ARG);
  GemmArgs g{};
  g.A = static_cast<const uint8_t*>(z);
  g.As = z_scales;
  g.W = static_cast<const uint8_t*>(w2);
  g.Ws = w2_scales;
  g.counts = counts;
  g.offsets = offsets;
  g.L = L;
  g.K = I;
  g.N = H;
  g.nb_count = (H + 2 * BH - 1) / (2 * BH);
  g.nb_stride = 2 * BH;
  g.half_stride = BH;
  g.rows_cap = rows_cap;
  g.out = out;
  g.ldo = H;
  const int mt = max_row_tiles(rows_cap, L);
  const moe_status ws_st = bind_workspace(g, mt, moe_host::elem_bytes(z_dt), workspace, workspace_bytes);
  if (ws_st != MOE_OK) return ws_st;
  if (out_dt == MOE_F32) return dispatch_dt<EPI_STORE_F32>(z_dt, g, mt, stream);
  return dispatch_dt<EPI_STORE_BF16>(z_dt, g, mt, stream);
}

namespace {

// y_acc = 0, 16 bytes per thread, grid-stride (a fill kernel rather than a
// memset node, so the call can be captured in a graph)
__global__ __launch_bounds__(256) void zero_f32_kernel(float* __restrict__ p, int64_t n4) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n4;
       i += static_cast<int64_t>(gridDim.x) * 256)
    reinterpret_cast<float4*>(p)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// y = y_acc rounded to bf16 (RNE) or copied (fp32), 4 values per thread
__global__ __launch_bounds__(256) void finish_rows_kernel(const float* __restrict__ acc, int64_t n4, void* y,
                                                         int y_bf16) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n4;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const float4 v = reinterpret_cast<const float4*>(acc)[i];
    if (y_bf16) {
      reinterpret_cast<uint2*>(y)[i] = make_uint2(
          static_cast<uint32_t>(moe::f32_to_bf16(v.x)) | (static_cast<uint32_t>(moe::f32_to_bf16(v.y)) << 16),
          static_cast<uint32_t>(moe::f32_to_bf16(v.z)) | (static_cast<uint32_t>(moe::f32_to_bf16(v.w)) << 16));
    } else {
      reinterpret_cast<float4*>(y)[i] = v;
    }
  }
}

}  // namespace

extern "C" moe_status moe_grouped_gemm_w2_combine(const void* z, moe_dtype z_dt, const float* z_scales,
                                                  const void* w2, moe_dtype w_dt, const float* w2_scales,
                                                  const int32_t* counts, const int32_t* offsets, int L,
                                                  int64_t rows_cap, int H, int I, const int32_t* row_src,
                                                  const float* topk_weights, int T, int K, float* y_acc,
                                                  void* y, moe_dtype y_dt, hipStream_t stream) {
  MOE_CHECK(L >= 1 && L <= kMaxL && rows_cap >= 0 && H > 0 && I > 0 && T >= 0 && K > 0, MOE_ERR_INVALID_ARG);
  MOE_CHECK(moe_host::valid_dtype(z_dt) && moe_host::valid_dtype(w_dt) && moe_host::valid_dtype(y_dt),
            MOE_ERR_INVALID_ARG);
  MOE_CHECK(z_dt == w_dt, MOE_ERR_UNSUPPORTED);
  MOE_CHECK(H % 128 == 0 && I % 128 == 0, MOE_ERR_UNSUPPORTED);
  MOE_CHECK(y_dt == MOE_F32 || y_dt == MOE_BF16, MOE_ERR_UNSUPPORTED);
  MOE_CHECK(offsets_fit(static_cast<int64_t>(I) * moe_host::elem_bytes(z_dt), H, rows_cap),
            MOE_ERR_UNSUPPORTED);
  MOE_CHECK(z_dt != MOE_FP8_E4M3 || I <= 128 * 128, MOE_ERR_UNSUPPORTED);
  if (T == 0) return MOE_OK;
  // every argument is checked before the first launch
  MOE_CHECK(y_acc && y, MOE_ERR_INVALID_ARG);
  MOE_CHECK(((reinterpret_cast<uintptr_t>(y_acc) | reinterpret_cast<uintptr_t>(y)) & 15) == 0, MOE_ERR_INVALID_ARG);
  if (rows_cap > 0) {
    MOE_CHECK(z && w2 && counts && offsets && row_src && topk_weights, MOE_ERR_INVALID_ARG);
    MOE_CHECK(z_dt != MOE_FP8_E4M3 || (z_scales && w2_scales), MOE_ERR_INVALID_ARG);
  }
  const int64_t n4 = static_cast<int64_t>(T) * H / 4;
  const int fill_grid = static_cast<int>(std::min<int64_t>((n4 + 255) / 256, 8192));
  zero_f32_kernel<<<fill_grid, 256, 0, stream>>>(y_acc, n4);
  MOE_LAUNCH_CHECK();
  if (rows_cap > 0) {
    GemmArgs g{};
    g.A = static_cast<const uint8_t*>(z);
    g.As = z_scales;
    g.W = static_cast<const uint8_t*>(w2);
    g.Ws = w2_scales;
    g.counts = counts;
    g.offsets = offsets;
    g.L = L;
    g.K = I;
    g.N = H;
    g.nb_count = (H + 2 * BH - 1) / (2 * BH);
    g.nb_stride = 2 * BH;
    g.half_stride = BH;
    g.rows_cap = rows_cap;
    g.ldo = H;
    g.row_src = row_src;
    g.route_w = topk_weights;
    g.y_acc = y_acc;
    g.topk = K;
    const moe_status st = dispatch_dt<EPI_SCATTER_F32>(z_dt, g, max_row_tiles(rows_cap, L), stream);
    if (st != MOE_OK) return st;
  }
  finish_rows_kernel<<<fill_grid, 256, 0, stream>>>(y_acc, n4, y, y_dt == MOE_BF16 ? 1 : 0);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

extern "C" size_t moe_grouped_gemm_workspace_bytes(void) {
  return workspace_bytes_for_grid(gemm_grid(int64_t(1) << 30));
}
