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
// then column block, then row tile, so the row tiles that share a weight
// block run back to back, and the ordered tile range is cut into 8
// contiguous chunks, one per XCD (workgroup i runs on XCD i mod 8), so a
// weight block is fetched from HBM into one XCD's L2 and reused there.
//
// Tile.  BM = 128 rows x two 128-column "halves" of W rows.  For W13 the
// halves are the gate block n0 + [0,128) and the matching up block
// I + n0 + [0,128), so one lane holds gate and up of the same (row, column)
// and SiLU(gate)*up needs no data exchange.  For W2 the halves are two
// adjacent 128-column blocks.  Eight waves (two per SIMD, so one wave's LDS
// reads overlap the other's matrix work) in a 2x4 grid each own 64 rows x
// (32 columns of each half) = 16 MFMA 16x16 tiles.
//
// K loop.  One stage = 128 bytes of K per row: 128 FP8, 64 bf16 or 32 fp32
// values -- for FP8 exactly one activation / weight scale group.  Each
// lane's MFMA operand is 32 contiguous bytes of one row of the stage, so
// the same LDS fragment feeds one 16x16x128 FP8 MFMA, two 16x16x32 bf16
// MFMAs or eight 16x16x4 fp32 MFMAs (A and B use the same K mapping, so the
// dot products pair up).
//
// Stages move HBM -> LDS by direct-to-LDS loads (global_load_lds_dwordx4:
// lane l's 16 bytes land at base + 16*l), three stages deep, so two stages
// are in flight while the third is multiplied and no VGPR holds staged data.
// A stage row is 128 bytes in a 16-byte XOR swizzle (chunk c of row r at
// chunk c ^ ((r >> 1) & 7), bank-conflict free on the 64-bank LDS); the
// swizzle is applied by choosing which source chunk each lane fetches.  Fragment reads are issued as ds_read_b128 in inline
// assembly that ends with its own lgkmcnt wait, so the compiler never
// inserts a full vmcnt wait (which would drain the loads still in flight);
// stage completion is tracked by hand with vmcnt and a workgroup barrier.
//
// FP8 scaling.  Per stage g every 16x16 FP8 product P_g is formed from a
// zero accumulator and folded in as acc += P_g * (a_scale[row, g] *
// w_scale[block, g]), fp32.

#include <algorithm>

#include "moe_common.h"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));   // 16 bytes in 4 VGPRs

constexpr int kThreads = 512;
constexpr int BM = 128;            // rows per tile
constexpr int BH = 128;            // columns per half
constexpr int KB = 128;            // bytes of K per stage and row
constexpr int kMaxL = 1024;
constexpr int NST = 3;             // LDS ring depth
constexpr int A_BYTES = BM * KB;                   // 16 KB
constexpr int B_BYTES = 2 * BH * KB;               // 32 KB
constexpr int AS_BYTES = BM * 4;                   // FP8 activation scales
constexpr int STAGE = A_BYTES + B_BYTES + AS_BYTES;
constexpr int kRsrcWord3 = 0x00020000;             // raw buffer: 32-bit data format

enum Dt { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2 };
enum Epi { EPI_STORE_F32 = 0, EPI_STORE_BF16 = 1, EPI_SILU_F32 = 2, EPI_SILU_BF16 = 3, EPI_SILU_FP8 = 4 };

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
};

// Rows of expert e that exist: counts[e] clipped to the buffer, so a tile
// never reaches past rows_cap even for inconsistent counts/offsets.
__device__ __forceinline__ int eff_count(const GemmArgs& p, int e) {
  const int64_t off = p.offsets[e];
  if (off < 0 || off >= p.rows_cap) return 0;
  return static_cast<int>(max<int64_t>(0, min<int64_t>(p.counts[e], p.rows_cap - off)));
}

// s_waitcnt immediate for "vmcnt <= n" with the other counters left alone
template <int N> struct VmCnt {
  static constexpr int imm = (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8);
};

// byte address of a __shared__ object inside the workgroup's LDS
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  typedef const __attribute__((address_space(3))) uint8_t* lds_ptr;
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)(p)));
}

// Fragment reads of one stage for one wave, issued without waiting: A (4
// row sub-tiles) and B (half, 16-column sub-tile) at (0,0) (0,1) (1,0)
// (1,1); for FP8 the activation scales of the wave's 64 rows.  The
// registers are only consumed after MOE_WAIT_BARRIER_FRAGS, which waits for
// them (lgkmcnt) and carries them as operands.
#define MOE_DS_AB(af, bf, a0, a1, b0, b1)                                                    \
  asm volatile(                                                                            \
      "ds_read_b128 %0, %16\n ds_read_b128 %1, %17\n"                                      \
      "ds_read_b128 %2, %16 offset:2048\n ds_read_b128 %3, %17 offset:2048\n"              \
      "ds_read_b128 %4, %16 offset:4096\n ds_read_b128 %5, %17 offset:4096\n"              \
      "ds_read_b128 %6, %16 offset:6144\n ds_read_b128 %7, %17 offset:6144\n"              \
      "ds_read_b128 %8, %18\n ds_read_b128 %9, %19\n"                                      \
      "ds_read_b128 %10, %18 offset:2048\n ds_read_b128 %11, %19 offset:2048\n"            \
      "ds_read_b128 %12, %18 offset:16384\n ds_read_b128 %13, %19 offset:16384\n"          \
      "ds_read_b128 %14, %18 offset:18432\n ds_read_b128 %15, %19 offset:18432"             \
      : "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(af[3]), "=&v"(af[4]), "=&v"(af[5]), \
        "=&v"(af[6]), "=&v"(af[7]), "=&v"(bf[0]), "=&v"(bf[1]), "=&v"(bf[2]), "=&v"(bf[3]), \
        "=&v"(bf[4]), "=&v"(bf[5]), "=&v"(bf[6]), "=&v"(bf[7])                              \
      : "v"(a0), "v"(a1), "v"(b0), "v"(b1))

#define MOE_DS_S(sv, s0)                                                                    \
  asm volatile(                                                                            \
      "ds_read_b128 %0, %4\n ds_read_b128 %1, %4 offset:64\n"                              \
      "ds_read_b128 %2, %4 offset:128\n ds_read_b128 %3, %4 offset:192"                    \
      : "=&v"(sv[0]), "=&v"(sv[1]), "=&v"(sv[2]), "=&v"(sv[3])                              \
      : "v"(s0))

#define MOE_WAIT_BARRIER_FRAGS(af, bf, sv)                                                  \
  asm volatile("s_waitcnt lgkmcnt(0)\n s_barrier"                                          \
               : "+v"(af[0]), "+v"(af[1]), "+v"(af[2]), "+v"(af[3]), "+v"(af[4]), "+v"(af[5]), \
                 "+v"(af[6]), "+v"(af[7]), "+v"(bf[0]), "+v"(bf[1]), "+v"(bf[2]), "+v"(bf[3]), \
                 "+v"(bf[4]), "+v"(bf[5]), "+v"(bf[6]), "+v"(bf[7]), "+v"(sv[0]), "+v"(sv[1]), \
                 "+v"(sv[2]), "+v"(sv[3])                                                   \
               :                                                                           \
               : "memory")

// Workgroup barriers that also pin register values: the compiler may move
// matrix instructions (they touch no memory) across a plain barrier, which
// would blur the phases; routing the fragments (resp. accumulators) through
// the barrier keeps the products of a phase between its two barriers.
#define MOE_BARRIER_ACC(acc, WAIT)                                                          \
  asm volatile(WAIT "s_barrier"                                                            \
               : "+v"(acc[0][0][0]), "+v"(acc[0][0][1]), "+v"(acc[0][1][0]), "+v"(acc[0][1][1]), \
                 "+v"(acc[1][0][0]), "+v"(acc[1][0][1]), "+v"(acc[1][1][0]), "+v"(acc[1][1][1]), \
                 "+v"(acc[2][0][0]), "+v"(acc[2][0][1]), "+v"(acc[2][1][0]), "+v"(acc[2][1][1]), \
                 "+v"(acc[3][0][0]), "+v"(acc[3][0][1]), "+v"(acc[3][1][0]), "+v"(acc[3][1][1])  \
               :                                                                           \
               : "memory")

template <int DT>
__device__ __forceinline__ v4f mma_stage(const u4& alo, const u4& ahi, const u4& blo,
                                         const u4& bhi, v4f acc) {
  if constexpr (DT == DT_FP8) {
    const v8i a = {int(alo.x), int(alo.y), int(alo.z), int(alo.w), int(ahi.x), int(ahi.y), int(ahi.z), int(ahi.w)};
    const v8i b = {int(blo.x), int(blo.y), int(blo.z), int(blo.w), int(bhi.x), int(bhi.y), int(bhi.z), int(bhi.w)};
    // formats 0/0 = fp8 e4m3 for A and B; scale bytes 127 = 2^0
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, 127, 0, 127);
  } else if constexpr (DT == DT_BF16) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, alo),
                                                 __builtin_bit_cast(v8bf, blo), acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, ahi),
                                                  __builtin_bit_cast(v8bf, bhi), acc, 0, 0, 0);
  } else {
    const float a[8] = {__uint_as_float(alo.x), __uint_as_float(alo.y), __uint_as_float(alo.z),
                        __uint_as_float(alo.w), __uint_as_float(ahi.x), __uint_as_float(ahi.y),
                        __uint_as_float(ahi.z), __uint_as_float(ahi.w)};
    const float b[8] = {__uint_as_float(blo.x), __uint_as_float(blo.y), __uint_as_float(blo.z),
                        __uint_as_float(blo.w), __uint_as_float(bhi.x), __uint_as_float(bhi.y),
                        __uint_as_float(bhi.z), __uint_as_float(bhi.w)};
#pragma unroll
    for (int m = 0; m < 8; ++m) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[m], b[m], acc, 0, 0, 0);
    return acc;
  }
}

__shared__ __attribute__((aligned(16))) uint8_t s_ring[NST * STAGE];
__shared__ int s_mt_prefix[kMaxL + 1];
__shared__ float s_amax[4][BM];
__shared__ int s_part[kThreads];

// Tile id -> (expert, column block, row tile).  s_mt_prefix[e] = sum of row
// tiles of experts < e; tile ids are expert-major, then column block, then
// row tile.
__device__ __forceinline__ void decode_tile(int L, int nb_count, int t, int& e, int& nb, int& mt) {
  int lo = 0, hi = L;           // largest e with s_mt_prefix[e]*nb_count <= t
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_mt_prefix[mid] * nb_count <= t) lo = mid; else hi = mid;
  }
  e = lo;
  const int mte = s_mt_prefix[e + 1] - s_mt_prefix[e];
  const int local = t - s_mt_prefix[e] * nb_count;
  nb = local / mte;
  mt = local - nb * mte;
}

// Staging context of one tile, workgroup-uniform.
struct Tile {
  int e, nb, rows_valid, n0;
  int64_t row0;
  bool half1;
  int a_row_off, w_row_off, s_row_off;
  int ws0, ws1;                        // FP8: first weight-scale index of each half
};

template <int DT, int EPI>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(GemmArgs p) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform by construction; readfirstlane tells the compiler so, which
  // keeps the staged-load offsets in scalar registers (no per-load loop)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2;      // 64-row slice of the tile = wave group (0: waves 0-3, 1: 4-7)
  const int wn = wave & 3;       // 32-column slice of each half
  constexpr int ESZ = DT == DT_FP8 ? 1 : (DT == DT_BF16 ? 2 : 4);
  constexpr bool kFp8 = DT == DT_FP8;
  constexpr int NLOAD = kFp8 ? 7 : 6;      // direct-to-LDS loads per wave per stage

  // ---- tile map: row tiles per expert, prefix over experts (block scan)
  {
    const int per = (p.L + kThreads - 1) / kThreads;
    const int e0 = tid * per;
    int s = 0;
    for (int e = e0; e < min(e0 + per, p.L); ++e) s += (eff_count(p, e) + BM - 1) / BM;
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
      run += (eff_count(p, e) + BM - 1) / BM;
    }
    if (tid == kThreads - 1) s_mt_prefix[p.L] = s_part[kThreads - 1];
    __syncthreads();
  }
  const int n_tiles = s_mt_prefix[p.L] * p.nb_count;
  int t_begin, t_end, t_step;
  if (gridDim.x >= 8 && (gridDim.x & 7) == 0) {
    const int xcd = blockIdx.x & 7;
    const int per_xcd = gridDim.x >> 3;
    t_begin = static_cast<int>((static_cast<int64_t>(n_tiles) * xcd) >> 3) + (blockIdx.x >> 3);
    t_end = static_cast<int>((static_cast<int64_t>(n_tiles) * (xcd + 1)) >> 3);
    t_step = per_xcd;
  } else {
    t_begin = blockIdx.x;
    t_end = n_tiles;
    t_step = gridDim.x;
  }

  const int kstages = p.K * ESZ / KB;
  const int kgroups = p.K / 128;              // FP8 scale groups along K
  const int64_t lda = static_cast<int64_t>(p.K) * ESZ;

  // Stage layout: chunk c (16 bytes) of row r sits at chunk c ^ swz(r) with
  // swz(r) = (r & 7) ^ ((r >> 3) & 1), which repeats every 16 rows.  With it
  // the fragment reads below (16 rows x 4 chunk pairs per instruction) run
  // at the full LDS rate with no bank conflicts (measured: 256 B/clk per CU
  // with 8 waves; the same reads without the (r >> 3) term, or with
  // (r >> 1) & 7, reach 160 B/clk).  A direct-to-LDS load still writes 1 KB
  // contiguously: lane l fills row srow = l >> 3 of an 8-row group g,
  // physical chunk l & 7, so it fetches chunk (l & 7) ^ srow ^ (g & 1).
  const int srow = lane >> 3;
  const int voff_e = static_cast<int>(srow * lda) + (((lane & 7) ^ srow) << 4);
  const int voff_o = static_cast<int>(srow * lda) + (((lane & 7) ^ srow ^ 1) << 4);
  const int soff = (lane & 15) * kgroups * 4;    // A-scale row of this lane (FP8)
  // fragment reads: row (lane & 15) of a 16-row block, bytes 32*(lane>>4)..+32
  const int frow = lane & 15;
  const int fsw = (frow & 7) ^ (frow >> 3);
  const int fc0 = ((2 * (lane >> 4)) ^ fsw) << 4;
  const int fc1 = ((2 * (lane >> 4) + 1) ^ fsw) << 4;
  const uint32_t ring = lds_u32(s_ring);

  // Per-tile staging context (see Tile).  The tile decode reads LDS, so
  // readfirstlane marks its results workgroup-uniform.
  auto make_tile = [&](int t) {
    Tile c;
    int e, nb, mt;
    decode_tile(p.L, p.nb_count, t, e, nb, mt);
    c.e = __builtin_amdgcn_readfirstlane(e);
    c.nb = __builtin_amdgcn_readfirstlane(nb);
    mt = __builtin_amdgcn_readfirstlane(mt);
    c.rows_valid = min(BM, eff_count(p, c.e) - mt * BM);
    c.row0 = static_cast<int64_t>(p.offsets[c.e]) + static_cast<int64_t>(mt) * BM;
    c.n0 = c.nb * p.nb_stride;
    c.half1 = c.n0 + p.half_stride < p.N;
    // this wave stages A rows 16*wave + [0,16) and W-tile rows 32*wave +
    // [0,32) (waves 0-3: half 0, waves 4-7: half 1)
    c.a_row_off = static_cast<int>((c.row0 + 16 * wave) * lda);
    c.w_row_off = static_cast<int>((c.n0 + (wave >> 2) * (c.half1 ? p.half_stride : 0) + 32 * (wave & 3)) * lda);
    c.s_row_off = static_cast<int>((c.row0 + 16 * wave) * kgroups * 4);
    const int bpe = p.N / 128;                 // weight-scale block rows per expert
    c.ws0 = (c.e * bpe + c.n0 / 128) * kgroups;
    c.ws1 = (c.e * bpe + (c.half1 ? c.n0 + p.half_stride : c.n0) / 128) * kgroups;
    return c;
  };
  // Buffer resources: A over the whole expert-major buffer, W over one
  // expert's [N, K] block.  Rows past the end of a resource read as 0, so a
  // tail tile may read past its expert's last row without a clamp; those
  // rows are never stored.
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.A), 0, static_cast<int>(p.rows_cap * lda), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rS = kFp8 ? __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(p.As), 0, static_cast<int>(p.rows_cap * kgroups * 4), kRsrcWord3) : rA;
  // issue this wave's direct-to-LDS loads of K stage ks of tile c into slot s
  auto issue = [&](const Tile& c, int s, int ks) {
    const __amdgpu_buffer_rsrc_t rW = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(p.W + static_cast<int64_t>(c.e) * p.N * lda), 0,
        static_cast<int>(p.N * lda), kRsrcWord3);
    uint8_t* st = s_ring + s * STAGE;
    typedef __attribute__((address_space(3))) void* lds_void;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rA, (lds_void)(st + (16 * wave + 8 * j) * KB), 16, j ? voff_o : voff_e,
          c.a_row_off + static_cast<int>(8 * j * lda) + ks * KB, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rW, (lds_void)(st + A_BYTES + (32 * wave + 8 * j) * KB), 16, (j & 1) ? voff_o : voff_e,
          c.w_row_off + static_cast<int>(8 * j * lda) + ks * KB, 0, 0);
    if constexpr (kFp8) {
      if (lane < 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rS, (lds_void)(st + A_BYTES + B_BYTES + 16 * wave * 4), 4, soff, c.s_row_off + ks * 4, 0, 0);
    }
  };

  // The workgroup's tiles form one stream of stages: stage g is K stage
  // g % kstages of its (g / kstages)-th tile and lives in ring slot g % NST.
  // With kstages >= 2, the first two stages of the next tile are staged
  // during the last two stages of the current one, so a tile starts with its
  // operands on the way instead of refilling the pipeline.
  const int my_tiles = t_begin < t_end ? (t_end - t_begin + t_step - 1) / t_step : 0;
  const int total = my_tiles * kstages;
  const bool stream = kstages >= 2;
  // FP8 weight scales of a tile: lane g holds group g (and 64 + g) of each
  // half; read per stage with readlane
  auto load_wscales = [&](const Tile& c, float (&v)[2][2]) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int g = lane + 64 * q;
      v[0][q] = g < kgroups ? p.Ws[c.ws0 + g] : 0.f;
      v[1][q] = g < kgroups ? p.Ws[c.ws1 + g] : 0.f;
    }
  };
  Tile cur{}, nxt{};
  float vsw[2][2] = {{0.f, 0.f}, {0.f, 0.f}}, vsw_n[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
  if (my_tiles > 0) {
    cur = make_tile(t_begin);
    if constexpr (kFp8) load_wscales(cur, vsw);
  }
  if (my_tiles > 1) {
    nxt = make_tile(t_begin + t_step);
    if constexpr (kFp8) load_wscales(nxt, vsw_n);
  }
  const uint32_t a_frag = (wm * 64 + frow) * KB;
  const uint32_t b_frag = A_BYTES + (wn * 32 + frow) * KB;
  const uint32_t s_frag = A_BYTES + B_BYTES + (wm * 64 + (lane >> 4) * 4) * 4;

  for (int ti = 0; ti < my_tiles; ++ti) {
    const int base = ti * kstages;             // stream index of this tile's stage 0
    const int e = cur.e, nb = cur.nb, rows_valid = cur.rows_valid, n0 = cur.n0;
    const int64_t row0 = cur.row0;
    const bool half1 = cur.half1;
    // stage g of the stream exists / is staged by the code below
    auto staged = [&](int g) { return g < total && (stream || g < base + kstages); };
    auto issue_g = [&](int g) {
      const int ks = g - base;
      if (ks < kstages) issue(cur, g % NST, ks); else issue(nxt, g % NST, ks - kstages);
    };
    (void)e;

    v4f acc[4][2][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][h][j] = v4f{0.f, 0.f, 0.f, 0.f};

    if (ti == 0 || !stream) {
      // nothing of a previous tile is still landing in the ring
      __builtin_amdgcn_s_waitcnt(VmCnt<0>::imm);
      __syncthreads();
      issue_g(base);
      if (staged(base + 1)) {
        issue_g(base + 1);
        __builtin_amdgcn_s_waitcnt(VmCnt<NLOAD>::imm);
      } else {
        __builtin_amdgcn_s_waitcnt(VmCnt<0>::imm);
      }
      __builtin_amdgcn_s_barrier();  // stage 0 has landed for every wave
    }

    // Two wave groups take turns.  Every phase ends with a workgroup
    // barrier; in each phase one group stages and reads while the other runs
    // the matrix products of the stage it read in the phase before, so each
    // SIMD always has one wave feeding the matrix core and one moving data.
    // Group g reads stage ks in phase 2*ks + g and multiplies it in phase
    // 2*ks + g + 1 (group 1 waits out phase 0, group 0 the last phase).  In
    // its read phase for stream stage G a wave also issues its share of
    // stage G + 2 (into the slot of G - 1, which group 1 finished reading in
    // the phase before) and, before the closing barrier, waits for its own
    // loads of stage G + 1 -- so neither staging issue nor waits ever sit in
    // a matrix phase.  Stage G + 1 is first read after both groups' waits.
    if (wm == 1) __builtin_amdgcn_s_barrier();
    for (int ks = 0; ks < kstages; ++ks) {
      const int g = base + ks;
      // fragment reads first (no wait), then the staging loads: a wave is
      // held at a staging load until the memory pipeline takes it, and the
      // reads complete meanwhile
      const uint32_t sb = ring + (g % NST) * STAGE;
      u4 af[8], bf[8], sv[4];
      MOE_DS_AB(af, bf, sb + a_frag + fc0, sb + a_frag + fc1, sb + b_frag + fc0, sb + b_frag + fc1);
      if constexpr (kFp8) {
        MOE_DS_S(sv, sb + s_frag);
      } else {
        sv[0] = sv[1] = sv[2] = sv[3] = u4{0, 0, 0, 0};
      }
      if (staged(g + 2)) issue_g(g + 2);
      if (staged(g + 2))
        __builtin_amdgcn_s_waitcnt(VmCnt<NLOAD>::imm);
      else if (staged(g + 1))
        __builtin_amdgcn_s_waitcnt(VmCnt<0>::imm);
      MOE_WAIT_BARRIER_FRAGS(af, bf, sv);
      if constexpr (kFp8) {
        const int qq = ks >> 6;
        float sw[2];
        sw[0] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
            __builtin_bit_cast(int, qq ? vsw[0][1] : vsw[0][0]), ks & 63));
        sw[1] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
            __builtin_bit_cast(int, qq ? vsw[1][1] : vsw[1][0]), ks & 63));
        // 16 independent products P, each folded in as acc += P * (sa * sw).
        // Software-pipelined over the 8 (row sub-tile, half) pairs: the two
        // products of pair n + 1 are issued before the fp32 folds of pair n,
        // so the matrix core works while the vector ALU folds.
        v4f pr[2][2];
        auto products = [&](int n, v4f* out) {
          const int i = n >> 1, h = n & 1;
#pragma unroll
          for (int j = 0; j < 2; ++j)
            out[j] = mma_stage<DT>(af[2 * i], af[2 * i + 1], bf[4 * h + 2 * j],
                                   bf[4 * h + 2 * j + 1], v4f{0.f, 0.f, 0.f, 0.f});
        };
        products(0, pr[0]);
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          if (n + 1 < 8) products(n + 1, pr[(n + 1) & 1]);
          const int i = n >> 1, h = n & 1;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float f = __uint_as_float(sv[i][r]) * sw[h];
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][h][j][r] = fmaf(pr[n & 1][j][r], f, acc[i][h][j][r]);
          }
          // keep the issue order: 2 matrix ops, then this pair's 12 vector ops
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
        }
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[i][h][j] = mma_stage<DT>(af[2 * i], af[2 * i + 1], bf[4 * h + 2 * j],
                                           bf[4 * h + 2 * j + 1], acc[i][h][j]);
      }
      MOE_BARRIER_ACC(acc, "");
    }
    if (wm == 0) __builtin_amdgcn_s_barrier();

    // ---- epilogue.  Lane holds rows i*16 + (lane>>4)*4 + r, columns
    // j*16 + (lane&15) of its 32-column slice of each half.
    const int rbase = wm * 64 + (lane >> 4) * 4;
    const int cbase = wn * 32 + (lane & 15);
    if constexpr (EPI == EPI_STORE_F32 || EPI == EPI_STORE_BF16) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (h == 1 && !half1) continue;
        const int ncol0 = n0 + h * p.half_stride;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = rbase + i * 16 + r;
            if (row >= rows_valid) continue;
            const int64_t o = (row0 + row) * p.ldo + ncol0;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const int c = cbase + j * 16;
              if constexpr (EPI == EPI_STORE_F32)
                static_cast<float*>(p.out)[o + c] = acc[i][h][j][r];
              else
                static_cast<uint16_t*>(p.out)[o + c] = moe::f32_to_bf16(acc[i][h][j][r]);
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
        // per-row amax over the 128 Z columns: 2 in-lane, 16 lanes, 4 waves
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float m = fmaxf(fabsf(z[i][0][r]), fabsf(z[i][1][r]));
            m = moe::group16_max(m);
            if ((lane & 15) == 0) s_amax[wn][rbase + i * 16 + r] = m;
          }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = rbase + i * 16 + r;
            const float amax = moe::fp8_group_amax_clamp(
                fmaxf(fmaxf(s_amax[0][row], s_amax[1][row]), fmaxf(s_amax[2][row], s_amax[3][row])));
            const float inv = moe::fp8_group_inv(amax);
            if (row >= rows_valid) continue;
            uint8_t* zrow = static_cast<uint8_t*>(p.out) + (row0 + row) * p.ldo + zcol0;
#pragma unroll
            for (int j = 0; j < 2; ++j)
              zrow[cbase + j * 16] = static_cast<uint8_t>(moe::f32x2_to_e4m3(z[i][j][r] * inv, 0.f));
            if (wn == 0 && (lane & 15) == 0)
              p.out_scales[(row0 + row) * (p.ldo / 128) + nb] = moe::fp8_group_scale(amax);
          }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = rbase + i * 16 + r;
            if (row >= rows_valid) continue;
            const int64_t o = (row0 + row) * p.ldo + zcol0;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              if constexpr (EPI == EPI_SILU_F32)
                static_cast<float*>(p.out)[o + cbase + j * 16] = z[i][j][r];
              else
                static_cast<uint16_t*>(p.out)[o + cbase + j * 16] = moe::f32_to_bf16(z[i][j][r]);
            }
          }
      }
    }
    // the next tile's first stages are already on their way
    cur = nxt;
    if constexpr (kFp8) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int q = 0; q < 2; ++q) vsw[h][q] = vsw_n[h][q];
    }
    if (ti + 2 < my_tiles) {
      nxt = make_tile(t_begin + (ti + 2) * t_step);
      if constexpr (kFp8) load_wscales(nxt, vsw_n);
    }
  }
}

template <int DT, int EPI>
moe_status launch(const GemmArgs& a, int max_mtiles, hipStream_t stream) {
  const int64_t max_tiles = static_cast<int64_t>(max_mtiles) * a.nb_count;
  if (max_tiles <= 0) return MOE_OK;
  const int cus = moe_host::device_cu_count();
  int grid = static_cast<int>(std::min<int64_t>(max_tiles, cus));
  if (grid >= 8) grid &= ~7;
  grouped_gemm_kernel<DT, EPI><<<grid, kThreads, 0, stream>>>(a);
  MOE_LAUNCH_CHECK();
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

extern "C" moe_status moe_grouped_gemm_w13(const void* a, moe_dtype a_dt, const float* a_scales,
                                           const void* w13, moe_dtype w_dt, const float* w13_scales,
                                           const int32_t* counts, const int32_t* offsets, int L,
                                           int64_t rows_cap, int H, int I, moe_w13_epilogue epi,
                                           void* out, moe_dtype out_dt, float* out_scales,
                                           hipStream_t stream) {
  MOE_CHECK(L >= 1 && L <= kMaxL && rows_cap >= 0 && H > 0 && I > 0, MOE_ERR_INVALID_ARG);
  MOE_CHECK(moe_host::valid_dtype(a_dt) && moe_host::valid_dtype(w_dt) && moe_host::valid_dtype(out_dt),
            MOE_ERR_INVALID_ARG);
  MOE_CHECK(epi == MOE_EPI_STORE_G || epi == MOE_EPI_SILU_MUL, MOE_ERR_INVALID_ARG);
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
  const int mt = max_row_tiles(rows_cap, L);
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

extern "C" moe_status moe_grouped_gemm_w2(const void* z, moe_dtype z_dt, const float* z_scales,
                                          const void* w2, moe_dtype w_dt, const float* w2_scales,
                                          const int32_t* counts, const int32_t* offsets, int L,
                                          int64_t rows_cap, int H, int I, void* out,
                                          moe_dtype out_dt, hipStream_t stream) {
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
  if (out_dt == MOE_F32) return dispatch_dt<EPI_STORE_F32>(z_dt, g, mt, stream);
  return dispatch_dt<EPI_STORE_BF16>(z_dt, g, mt, stream);
}
