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
// adjacent 128-column blocks.  Four waves in a 2x2 grid each own 64 rows x
// (64 columns of each half) = 32 MFMA 16x16 tiles.
//
// K loop.  One stage = 128 bytes of K per row: 128 FP8, 64 bf16 or 32 fp32
// values -- for FP8 exactly one activation / weight scale group.  Each
// lane's MFMA operand is 32 contiguous bytes of one row of the stage, so
// the same LDS fragment feeds one 16x16x128 FP8 MFMA, two 16x16x32 bf16
// MFMAs or eight 16x16x4 fp32 MFMAs (A and B use the same K mapping, so the
// dot products pair up).  Stages are double-buffered in LDS with a 16-byte
// XOR swizzle (chunk c of row r at chunk c ^ (r & 7)) so fragment reads and
// stage writes are bank-conflict free; the next stage is fetched into
// registers while the current one is multiplied.
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

constexpr int kThreads = 256;
constexpr int BM = 128;            // rows per tile
constexpr int BH = 128;            // columns per half
constexpr int KB = 128;            // bytes of K per stage and row
constexpr int kMaxL = 1024;

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

struct Stage {
  uint8_t a[BM * KB];          // 16 KB
  uint8_t b[2 * BH * KB];      // 32 KB
  float as[BM];                // A scales of this stage (FP8)
};

struct Smem {
  Stage st[2];
  int mt_prefix[kMaxL + 1];    // row-tile prefix over experts
  float amax[2][BM];           // FP8 SiLU epilogue: per-row amax of each wave column
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * KB + ((chunk ^ (row & 7)) << 4); }

// 32 bytes of row `row`, K quarter `kq` (bytes 32*kq .. 32*kq+31) of a stage
__device__ __forceinline__ void frag(const uint8_t* base, int row, int kq, u4& lo, u4& hi) {
  lo = *reinterpret_cast<const u4*>(base + swz(row, 2 * kq));
  hi = *reinterpret_cast<const u4*>(base + swz(row, 2 * kq + 1));
}

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

// Rows of expert e that exist: counts[e] clipped to the buffer, so a tile
// never reaches past rows_cap even for inconsistent counts/offsets.
__device__ __forceinline__ int eff_count(const GemmArgs& p, int e) {
  const int64_t off = p.offsets[e];
  if (off < 0 || off >= p.rows_cap) return 0;
  return static_cast<int>(max<int64_t>(0, min<int64_t>(p.counts[e], p.rows_cap - off)));
}

// Tile id -> (expert, column block, row tile).  mt_prefix[e] = sum of row
// tiles of experts < e; tile ids are expert-major, then column block, then
// row tile.
__device__ __forceinline__ void decode_tile(const Smem& sm, int L, int nb_count, int t, int& e,
                                            int& nb, int& mt) {
  int lo = 0, hi = L;           // largest e with mt_prefix[e]*nb_count <= t
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (sm.mt_prefix[mid] * nb_count <= t) lo = mid; else hi = mid;
  }
  e = lo;
  const int mte = sm.mt_prefix[e + 1] - sm.mt_prefix[e];
  const int local = t - sm.mt_prefix[e] * nb_count;
  nb = local / mte;
  mt = local - nb * mte;
}

template <int DT, int EPI>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1;       // 64-row slice
  const int wn = wave >> 1;      // 64-column slice of each half
  constexpr int ESZ = DT == DT_FP8 ? 1 : (DT == DT_BF16 ? 2 : 4);

  // ---- tile map: row tiles per expert, prefix over experts (block scan)
  {
    __shared__ int part[kThreads];
    const int per = (p.L + kThreads - 1) / kThreads;
    const int e0 = tid * per;
    int s = 0;
    for (int e = e0; e < min(e0 + per, p.L); ++e) s += (eff_count(p, e) + BM - 1) / BM;
    part[tid] = s;
    __syncthreads();
    for (int d = 1; d < kThreads; d <<= 1) {
      const int v = tid >= d ? part[tid - d] : 0;
      __syncthreads();
      part[tid] += v;
      __syncthreads();
    }
    int run = part[tid] - s;     // exclusive prefix of this thread's range
    for (int e = e0; e < min(e0 + per, p.L); ++e) {
      sm.mt_prefix[e] = run;
      run += (eff_count(p, e) + BM - 1) / BM;
    }
    if (tid == kThreads - 1) sm.mt_prefix[p.L] = part[kThreads - 1];
    __syncthreads();
  }
  const int n_tiles = sm.mt_prefix[p.L] * p.nb_count;
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

  for (int t = t_begin; t < t_end; t += t_step) {
    int e, nb, mt;
    decode_tile(sm, p.L, p.nb_count, t, e, nb, mt);
    const int rows_valid = min(BM, eff_count(p, e) - mt * BM);
    const int64_t row0 = static_cast<int64_t>(p.offsets[e]) + static_cast<int64_t>(mt) * BM;
    const int n0 = nb * p.nb_stride;
    const bool half1 = n0 + p.half_stride < p.N;
    const uint8_t* Wexp = p.W + static_cast<int64_t>(e) * p.N * lda;

    // global source pointers of this thread's stage chunks
    const int cch = tid & 7;
    const uint8_t* asrc[4];
    const uint8_t* bsrc[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 32 * i;
      asrc[i] = p.A + (row0 + min(r, rows_valid - 1)) * lda + cch * 16;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = (tid >> 3) + 32 * i;
      const int h = r >> 7;
      const int rr = r & 127;
      const int wrow = (h && half1) ? n0 + p.half_stride + rr : n0 + rr;
      bsrc[i] = Wexp + static_cast<int64_t>(wrow) * lda + cch * 16;
    }
    const float* assrc = nullptr;
    if constexpr (DT == DT_FP8)
      assrc = p.As + (row0 + min(tid & (BM - 1), rows_valid - 1)) * kgroups;
    const float* wsb0 = nullptr;
    const float* wsb1 = nullptr;
    if constexpr (DT == DT_FP8) {
      const float* wse = p.Ws + static_cast<int64_t>(e) * (p.N / 128) * kgroups;
      wsb0 = wse + static_cast<int64_t>(n0 / 128) * kgroups;
      wsb1 = wse + static_cast<int64_t>((half1 ? n0 + p.half_stride : n0) / 128) * kgroups;
    }

    u4 ra[4], rb[8];
    float ras = 0.f;
    auto fetch = [&](int ks) {
#pragma unroll
      for (int i = 0; i < 4; ++i) ra[i] = *reinterpret_cast<const u4*>(asrc[i] + ks * KB);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        rb[i] = __builtin_nontemporal_load(reinterpret_cast<const u4*>(bsrc[i] + ks * KB));
      if constexpr (DT == DT_FP8) {
        if (tid < BM) ras = assrc[ks];
      }
    };
    auto commit = [&](int s) {
      Stage& st = sm.st[s];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u4*>(st.a + swz((tid >> 3) + 32 * i, cch)) = ra[i];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<u4*>(st.b + swz((tid >> 3) + 32 * i, cch)) = rb[i];
      if constexpr (DT == DT_FP8) {
        if (tid < BM) st.as[tid] = ras;
      }
    };

    v4f acc[4][2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][h][j] = v4f{0.f, 0.f, 0.f, 0.f};

    __syncthreads();               // previous tile's readers of stage 0 are done
    fetch(0);
    commit(0);
    for (int ks = 0; ks < kstages; ++ks) {
      __syncthreads();             // stage ks&1 complete; stage (ks+1)&1 free
      const bool more = ks + 1 < kstages;
      if (more) fetch(ks + 1);
      const Stage& st = sm.st[ks & 1];
      u4 alo[4], ahi[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) frag(st.a, wm * 64 + i * 16 + (lane & 15), lane >> 4, alo[i], ahi[i]);
      float sa[4][4];
      float sw[2] = {1.f, 1.f};
      if constexpr (DT == DT_FP8) {
        const int g = ks;                  // one stage == one scale group
        sw[0] = wsb0[g];
        sw[1] = wsb1[g];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 v = *reinterpret_cast<const float4*>(&st.as[wm * 64 + i * 16 + (lane >> 4) * 4]);
          sa[i][0] = v.x; sa[i][1] = v.y; sa[i][2] = v.z; sa[i][3] = v.w;
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u4 blo[4], bhi[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          frag(st.b, h * BH + wn * 64 + j * 16 + (lane & 15), lane >> 4, blo[j], bhi[j]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (DT == DT_FP8) {
            float f[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) f[r] = sa[i][r] * sw[h];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const v4f pj = mma_stage<DT>(alo[i], ahi[i], blo[j], bhi[j], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[i][h][j][r] = fmaf(pj[r], f[r], acc[i][h][j][r]);
            }
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][h][j] = mma_stage<DT>(alo[i], ahi[i], blo[j], bhi[j], acc[i][h][j]);
          }
        }
      }
      if (more) commit((ks + 1) & 1);
    }

    // ---- epilogue.  Lane holds rows i*16 + (lane>>4)*4 + r, column j*16 + (lane&15).
    const int rbase = wm * 64 + (lane >> 4) * 4;
    const int cbase = wn * 64 + (lane & 15);
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
            for (int j = 0; j < 4; ++j) {
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
      float z[4][4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) z[i][j][r] = moe::silu(acc[i][0][j][r]) * acc[i][1][j][r];
      const int64_t zcol0 = static_cast<int64_t>(nb) * BH;
      if constexpr (EPI == EPI_SILU_FP8) {
        // per-row amax over the 128 Z columns: 4 in-lane, 16 lanes, 2 waves
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float m = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) m = fmaxf(m, fabsf(z[i][j][r]));
            m = moe::group16_max(m);
            if ((lane & 15) == 0) sm.amax[wn][rbase + i * 16 + r] = m;
          }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = rbase + i * 16 + r;
            const float amax = moe::fp8_group_amax_clamp(fmaxf(sm.amax[0][row], sm.amax[1][row]));
            const float inv = moe::fp8_group_inv(amax);
            if (row >= rows_valid) continue;
            uint8_t* zrow = static_cast<uint8_t*>(p.out) + (row0 + row) * p.ldo + zcol0;
#pragma unroll
            for (int j = 0; j < 4; ++j)
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
            for (int j = 0; j < 4; ++j) {
              if constexpr (EPI == EPI_SILU_F32)
                static_cast<float*>(p.out)[o + cbase + j * 16] = z[i][j][r];
              else
                static_cast<uint16_t*>(p.out)[o + cbase + j * 16] = moe::f32_to_bf16(z[i][j][r]);
            }
          }
      }
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
  const size_t smem = sizeof(Smem);
  static bool attr_set = false;   // one kernel instance per template pair
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&grouped_gemm_kernel<DT, EPI>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem)) != hipSuccess)
      return MOE_ERR_HIP;
    attr_set = true;
  }
  grouped_gemm_kernel<DT, EPI><<<grid, kThreads, smem, stream>>>(a);
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
