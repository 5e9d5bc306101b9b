// Backward of the MoE path: combine backward, SiLU*up backward and the weight
// transpose that lets the grouped GEMM compute both data gradients.
//
// ("XTuner Domino EP": the DeepEP part's complete run path, whose backward
// consumes the saved routing in reverse order, and the UltraEP part's
// backward sketch -- combine backward, the grouped GEMMs' gradients, inverse
// permutation.  The formulas are the derivatives of the forward definition
// of "SGLang、NCCL 与 MoE EP" §1.1 and "SGLang Expert Compute Backend" §1.1,
// §3.6.)
//
//   d_out[q]  = w[t,k] * dy[t]                 combine backward (a dispatch)
//   d_w[t,k]  = <dy[t], out[q]>                router-weight gradient
//   dZ        = d_out W2[e]     = d_out (W2[e]^T)^T    grouped GEMM, W2 transposed
//   dG        = SiLU*up backward of (G, dZ)
//   dA        = dG W13[e]      = dG (W13[e]^T)^T       grouped GEMM, W13 transposed
//   dx[t]     = sum_k dA[q(t,k)]               permute backward (unit-weight combine)

#include <algorithm>

#include "moe_common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / MOE_WAVE;

template <bool kF32>
__device__ __forceinline__ void load8(const uint8_t* row, int c, float* v) {
  // 8 values starting at column 8c
  if constexpr (kF32) {
    const uint4 a = reinterpret_cast<const uint4*>(row)[2 * c];
    const uint4 b = reinterpret_cast<const uint4*>(row)[2 * c + 1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(w[i]);
  } else {
    const uint4 a = reinterpret_cast<const uint4*>(row)[c];
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
}

template <bool kF32>
__device__ __forceinline__ void store8(uint8_t* row, int c, const float* v) {
  if constexpr (kF32) {
    reinterpret_cast<float4*>(row)[2 * c] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(row)[2 * c + 1] = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    uint4 o;
    o.x = moe::f32_to_bf16(v[0]) | (uint32_t(moe::f32_to_bf16(v[1])) << 16);
    o.y = moe::f32_to_bf16(v[2]) | (uint32_t(moe::f32_to_bf16(v[3])) << 16);
    o.z = moe::f32_to_bf16(v[4]) | (uint32_t(moe::f32_to_bf16(v[5])) << 16);
    o.w = moe::f32_to_bf16(v[6]) | (uint32_t(moe::f32_to_bf16(v[7])) << 16);
    reinterpret_cast<uint4*>(row)[c] = o;
  }
}

// One wave per token.  Its local routes are walked in k order; for each, the
// wave streams dy[t] and out[q] in 8-column chunks, writes
// d_out[q] = w * dy[t] (one fp32 product, rounded to the output format) and
// sums dy * out in fp32, reduced across the wave for d_w[t,k].  Routes
// without a local row get d_w = 0 and write no row.
template <bool kDyF32, bool kOutF32, bool kDoF32>
__global__ __launch_bounds__(kThreads) void combine_backward_kernel(
    const uint8_t* __restrict__ dy, const uint8_t* __restrict__ out, const int32_t* __restrict__ slot_of,
    const float* __restrict__ w, int T, int K, int H, int64_t rows_cap, uint8_t* __restrict__ d_out,
    float* __restrict__ d_w) {
  const int lane = moe::lane_id();
  const int t = blockIdx.x * kWavesPerBlock + threadIdx.x / MOE_WAVE;
  if (t >= T) return;
  const int s_l = lane < K ? slot_of[static_cast<int64_t>(t) * K + lane] : -1;
  const float w_l = lane < K ? w[static_cast<int64_t>(t) * K + lane] : 0.f;
  const bool local = s_l >= 0 && s_l < rows_cap;
  const uint64_t routes = __ballot(local);
  const int nchunk = H / 8;
  const uint8_t* dyrow = dy + static_cast<int64_t>(t) * H * (kDyF32 ? 4 : 2);
  float dw_l = 0.f;
  for (uint64_t m = routes; m; m &= m - 1) {
    const int k = __builtin_ctzll(m);
    const int q = __builtin_amdgcn_readlane(s_l, k);
    const float wk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w_l), k));
    const uint8_t* orow = out + static_cast<int64_t>(q) * H * (kOutF32 ? 4 : 2);
    uint8_t* drow = d_out + static_cast<int64_t>(q) * H * (kDoF32 ? 4 : 2);
    float dot = 0.f;
    for (int c = lane; c < nchunk; c += MOE_WAVE) {
      float g[8], o[8], d[8];
      load8<kDyF32>(dyrow, c, g);
      load8<kOutF32>(orow, c, o);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        dot = fmaf(g[i], o[i], dot);
        d[i] = wk * g[i];
      }
      store8<kDoF32>(drow, c, d);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dot += __shfl_xor(dot, off);
    if (lane == k) dw_l = dot;
  }
  if (lane < K) d_w[static_cast<int64_t>(t) * K + lane] = dw_l;
}

// All-bf16 combine backward for H <= 4096: the lane's 8 chunks of dy[t] are
// loaded once and stay in registers for every route of the token, and a
// route's 8 chunks of out[q] (non-temporal: read once) are all issued before
// any is used.  Per lane the products run in the same order as above, so d_out
// and d_w are bit-identical to the general kernel.
constexpr int kCbNper = 8;
__global__ __launch_bounds__(kThreads) void combine_backward_bf16_reg_kernel(
    const uint4* __restrict__ dy, const uint4* __restrict__ out, const int32_t* __restrict__ slot_of,
    const float* __restrict__ w, int T, int K, int H, int64_t rows_cap, uint4* __restrict__ d_out,
    float* __restrict__ d_w) {
  const int lane = moe::lane_id();
  const int t = blockIdx.x * kWavesPerBlock + threadIdx.x / MOE_WAVE;
  if (t >= T) return;
  const int s_l = lane < K ? slot_of[static_cast<int64_t>(t) * K + lane] : -1;
  const float w_l = lane < K ? w[static_cast<int64_t>(t) * K + lane] : 0.f;
  const uint64_t routes = __ballot(s_l >= 0 && s_l < rows_cap);
  const int nchunk = H / 8;
  const uint4* dyrow = dy + static_cast<int64_t>(t) * nchunk;
  uint4 g[kCbNper];
#pragma unroll
  for (int j = 0; j < kCbNper; ++j) {
    const int c = lane + MOE_WAVE * j;
    g[j] = c < nchunk ? dyrow[c] : make_uint4(0, 0, 0, 0);
  }
  float dw_l = 0.f;
  for (uint64_t m = routes; m; m &= m - 1) {
    const int k = __builtin_ctzll(m);
    const int q = __builtin_amdgcn_readlane(s_l, k);
    const float wk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w_l), k));
    const uint4* orow = out + static_cast<int64_t>(q) * nchunk;
    uint4* drow = d_out + static_cast<int64_t>(q) * nchunk;
    uint4 o[kCbNper];
#pragma unroll
    for (int j = 0; j < kCbNper; ++j) {
      const int c = lane + MOE_WAVE * j;
      o[j] = c < nchunk ? moe::load_nt16(orow + c) : make_uint4(0, 0, 0, 0);
    }
    float dot = 0.f;
#pragma unroll
    for (int j = 0; j < kCbNper; ++j) {
      const int c = lane + MOE_WAVE * j;
      if (c >= nchunk) break;
      float gf[8], of[8], d[8];
      load8<false>(reinterpret_cast<const uint8_t*>(&g[j]), 0, gf);
      load8<false>(reinterpret_cast<const uint8_t*>(&o[j]), 0, of);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        dot = fmaf(gf[i], of[i], dot);
        d[i] = wk * gf[i];
      }
      store8<false>(reinterpret_cast<uint8_t*>(drow + c), 0, d);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dot += __shfl_xor(dot, off);
    if (lane == k) dw_l = dot;
  }
  if (lane < K) d_w[static_cast<int64_t>(t) * K + lane] = dw_l;
}

// d_gate = dz * up * s * (1 + gate * (1 - s)), d_up = dz * SiLU(gate),
// s = sigmoid(gate) (moe::silu_mul_grad); one wave per valid row, 4 columns
// per lane per step.
constexpr int kSiluBwBatch = 6;
template <bool kDzF32, bool kDgF32>
__global__ __launch_bounds__(kThreads) void silu_mul_backward_kernel(
    const float* __restrict__ g, const uint8_t* __restrict__ dz, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, int L, int64_t rows_cap, int I, uint8_t* __restrict__ dg) {
  const int lane = moe::lane_id();
  const int64_t q = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + threadIdx.x / MOE_WAVE;
  if (q >= rows_cap) return;
  // expert of row q: largest e with offsets[e] <= q; padding rows are skipped
  int lo = 0, hi = L;
  if (q < offsets[0]) return;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= q) lo = mid; else hi = mid;
  }
  if (q >= static_cast<int64_t>(offsets[lo]) + counts[lo]) return;
  const float* grow = g + q * 2 * I;
  const uint8_t* zrow = dz + q * I * (kDzF32 ? 4 : 2);
  uint8_t* drow = dg + q * 2 * I * (kDgF32 ? 4 : 2);
  // a lane's steps in batches of kSiluBwBatch: every load of a batch is issued
  // before any of its values is used
  const int nstep = I / 4;
  for (int base = lane; base < nstep; base += MOE_WAVE * kSiluBwBatch) {
    float4 gt[kSiluBwBatch], up[kSiluBwBatch];
    float z[kSiluBwBatch][4];
#pragma unroll
    for (int b = 0; b < kSiluBwBatch; ++b) {
      const int c = base + MOE_WAVE * b;
      const bool live = c < nstep;
      gt[b] = live ? reinterpret_cast<const float4*>(grow)[c] : make_float4(0.f, 0.f, 0.f, 0.f);
      up[b] = live ? reinterpret_cast<const float4*>(grow + I)[c] : make_float4(0.f, 0.f, 0.f, 0.f);
      if constexpr (kDzF32) {
        const float4 v = live ? reinterpret_cast<const float4*>(zrow)[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        z[b][0] = v.x; z[b][1] = v.y; z[b][2] = v.z; z[b][3] = v.w;
      } else {
        const uint2 v = live ? reinterpret_cast<const uint2*>(zrow)[c] : make_uint2(0, 0);
        z[b][0] = __uint_as_float(v.x << 16); z[b][1] = __uint_as_float(v.x & 0xffff0000u);
        z[b][2] = __uint_as_float(v.y << 16); z[b][3] = __uint_as_float(v.y & 0xffff0000u);
      }
    }
#pragma unroll
    for (int b = 0; b < kSiluBwBatch; ++b) {
      const int c = base + MOE_WAVE * b;
      if (c >= nstep) break;
      const float ga[4] = {gt[b].x, gt[b].y, gt[b].z, gt[b].w}, ua[4] = {up[b].x, up[b].y, up[b].z, up[b].w};
      float dgate[4], dup[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) moe::silu_mul_grad(ga[i], ua[i], z[b][i], dgate[i], dup[i]);
      if constexpr (kDgF32) {
        reinterpret_cast<float4*>(drow)[c] = make_float4(dgate[0], dgate[1], dgate[2], dgate[3]);
        reinterpret_cast<float4*>(drow + I * 4)[c] = make_float4(dup[0], dup[1], dup[2], dup[3]);
      } else {
        reinterpret_cast<uint2*>(drow)[c] = make_uint2(
            moe::f32_to_bf16(dgate[0]) | (uint32_t(moe::f32_to_bf16(dgate[1])) << 16),
            moe::f32_to_bf16(dgate[2]) | (uint32_t(moe::f32_to_bf16(dgate[3])) << 16));
        reinterpret_cast<uint2*>(drow + I * 2)[c] = make_uint2(
            moe::f32_to_bf16(dup[0]) | (uint32_t(moe::f32_to_bf16(dup[1])) << 16),
            moe::f32_to_bf16(dup[2]) | (uint32_t(moe::f32_to_bf16(dup[3])) << 16));
      }
    }
  }
}

// w [L, N, K] -> wt [L, K, N], 64 x 64 element tiles through LDS (padded row
// against bank conflicts); ESZ = element bytes (2 or 4).
template <typename TE>
__global__ __launch_bounds__(kThreads) void transpose_kernel(const TE* __restrict__ w, int N, int K,
                                                            TE* __restrict__ wt) {
  __shared__ TE tile[64][65];
  const int e = blockIdx.z;
  const int n0 = blockIdx.y * 64, k0 = blockIdx.x * 64;
  const TE* src = w + static_cast<int64_t>(e) * N * K;
  TE* dst = wt + static_cast<int64_t>(e) * N * K;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += kThreads / 64) {
    const int n = n0 + r, k = k0 + tx;
    if (n < N && k < K) tile[r][tx] = src[static_cast<int64_t>(n) * K + k];
  }
  __syncthreads();
  for (int r = ty; r < 64; r += kThreads / 64) {
    const int k = k0 + r, n = n0 + tx;
    if (n < N && k < K) dst[static_cast<int64_t>(k) * N + n] = tile[tx][r];
  }
}

// bf16 transpose for N, K multiples of 64: thread t loads 16 bytes (8
// elements) of rows t/8 and t/8 + 32 of the 64 x 64 tile, and writes 8
// consecutive n of output rows k = t/8 and t/8 + 32 (8 lanes cover one output
// row's 128 bytes), gathered from the LDS tile (row stride 66 elements).
__global__ __launch_bounds__(kThreads) void transpose_bf16_vec_kernel(const uint16_t* __restrict__ w, int N,
                                                                    int K, uint16_t* __restrict__ wt) {
  constexpr int kStride = 66;
  __shared__ uint16_t tile[64 * kStride];
  const int e = blockIdx.z;
  const int n0 = blockIdx.y * 64, k0 = blockIdx.x * 64;
  const uint16_t* src = w + static_cast<int64_t>(e) * N * K;
  uint16_t* dst = wt + static_cast<int64_t>(e) * N * K;
  const int c = threadIdx.x & 7, r0 = threadIdx.x >> 3;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = r0 + 32 * h;
    const uint4 v = *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(n0 + r) * K + k0 + 8 * c);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)       // 4-byte LDS writes: the row stride keeps them aligned
      *reinterpret_cast<uint32_t*>(&tile[r * kStride + 8 * c + 2 * i]) = u[i];
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int k = r0 + 32 * h;
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = tile[(8 * c + 2 * i) * kStride + k] | (uint32_t(tile[(8 * c + 2 * i + 1) * kStride + k]) << 16);
    *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(k0 + k) * N + n0 + 8 * c) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// ---------------------------------------------------------------- weight gradients
// C[e] = B_e^T A_e over expert e's valid rows: B [rows_cap, N], A [rows_cap, K]
// -> C [L, N, K] fp32.
//
// fp32 operands: one workgroup per (expert, 128 x 128 tile of C); rows are
// reduced in chunks of 32.  Each chunk of B (32 x 128) and A (32 x 128) is
// staged into LDS transposed ([column][row], rows contiguous) so that a
// 16x16x4 matrix-core operand -- 4 consecutive rows of one column, one per
// lane group -- is one 4-byte read per lane.  Wave w owns C rows
// 64*(w & 1) + [0,64) and columns 64*(w >> 1) + [0,64): 4 x 4 tiles of
// 16 x 16.  Rows past the expert's count stage as zeros.
typedef float v4f_t __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf_t __attribute__((ext_vector_type(8)));
constexpr int kWgTile = 128;
constexpr int kWgRows = 32;
constexpr int kWgStride = kWgRows + 8;       // LDS row stride in elements (padding vs bank conflicts)

__global__ __launch_bounds__(kThreads) void wgrad_f32_kernel(const float* __restrict__ b, const float* __restrict__ a,
                                                        const int32_t* __restrict__ counts,
                                                        const int32_t* __restrict__ offsets, int64_t rows_cap,
                                                        int N, int K, float* __restrict__ c) {
  __shared__ __attribute__((aligned(16))) float sB[kWgTile * kWgStride];
  __shared__ __attribute__((aligned(16))) float sA[kWgTile * kWgStride];
  const int e = blockIdx.z;
  const int n0 = blockIdx.y * kWgTile, k0 = blockIdx.x * kWgTile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t off = offsets[e];
  int cnt = 0;
  if (off >= 0 && off < rows_cap) cnt = static_cast<int>(min<int64_t>(counts[e], rows_cap - off));
  // staging: thread t moves rows 2*(t / 16) and 2*(t / 16) + 1, columns 8*(t % 16) + [0,8)
  const int sr = 2 * (tid >> 4), sc = 8 * (tid & 15);
  v4f_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f_t{0.f, 0.f, 0.f, 0.f};
  const int wn = 64 * (wave & 1), wk = 64 * (wave >> 1);
  for (int r0 = 0; r0 < cnt; r0 += kWgRows) {
    // 8 elements = 32 B per row and operand
    constexpr int kVec = 2;
    uint4 vb[2][kVec], va[2][kVec];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = r0 + sr + h;
      const bool live = r < cnt;
      const uint4* brow = reinterpret_cast<const uint4*>(b + (off + r) * static_cast<int64_t>(N) + n0 + sc);
      const uint4* arow = reinterpret_cast<const uint4*>(a + (off + r) * static_cast<int64_t>(K) + k0 + sc);
#pragma unroll
      for (int v = 0; v < kVec; ++v) {
        vb[h][v] = live ? brow[v] : make_uint4(0, 0, 0, 0);
        va[h][v] = live ? arow[v] : make_uint4(0, 0, 0, 0);
      }
    }
    __syncthreads();                               // the previous chunk's reads are done
    // rows sr and sr + 1 of one column are adjacent in LDS: one 8-byte write
    // per column and operand
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t* b0 = reinterpret_cast<const uint32_t*>(&vb[0][0]);
      const uint32_t* b1 = reinterpret_cast<const uint32_t*>(&vb[1][0]);
      const uint32_t* a0 = reinterpret_cast<const uint32_t*>(&va[0][0]);
      const uint32_t* a1 = reinterpret_cast<const uint32_t*>(&va[1][0]);
      *reinterpret_cast<uint2*>(&sB[(sc + i) * kWgStride + sr]) = make_uint2(b0[i], b1[i]);
      *reinterpret_cast<uint2*>(&sA[(sc + i) * kWgStride + sr]) = make_uint2(a0[i], a1[i]);
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kWgRows / 4; ++s) {
      float fb[4], fa[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fb[i] = sB[(wn + 16 * i + (lane & 15)) * kWgStride + 4 * s + (lane >> 4)];
        fa[i] = sA[(wk + 16 * i + (lane & 15)) * kWgStride + 4 * s + (lane >> 4)];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(fb[i], fa[j], acc[i][j], 0, 0, 0);
    }
  }
  // lane holds C[n = 16i + 4*(lane >> 4) + r][k = 16j + (lane & 15)] of the wave's 64 x 64
  float* ce = c + static_cast<int64_t>(e) * N * K;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = n0 + wn + 16 * i + 4 * (lane >> 4) + r;
#pragma unroll
      for (int j = 0; j < 4; ++j) ce[static_cast<int64_t>(n) * K + k0 + wk + 16 * j + (lane & 15)] = acc[i][j][r];
    }
}

// bf16 weight gradients, staged by direct global-to-LDS loads.  A ring of
// kW3Stages stages, each 32 rows x 256 columns of both operands in row-major
// order (512 bytes per row, the layout in memory), keeps kW3Stages - 1 chunks
// of loads in flight while one is multiplied.  Within a row the 16-byte chunk
// c sits at position c ^ 2 * (row & 3) ^ 8 * ((row >> 3) & 1): the four rows
// a 16-lane group's transposed read touches fall in four different 32-byte
// bank windows, and the two groups served together (rows 8 apart) in
// different 128-byte halves of the banks.  A matrix-core
// operand (8 consecutive rows of one column) is two transposed LDS reads
// (ds_read_b64_tr_b16: within 16 lanes, lane 4*d + q names row d, columns
// 4q..4q+3, and lane j receives column j of those four rows).  Rows past the
// expert's count read as zeros through the bound of a buffer resource made
// per chunk (based at the chunk's first row, so offsets stay small for any
// expert size).  Eight waves: wave w owns C rows 128*(w & 1) + [0,128) and
// columns 64*(w >> 1) + [0,64) of the 256 x 256 tile (8 x 4 MFMA tiles, 128
// accumulators), so two waves fit on a SIMD.  N and K need only be multiples
// of 128: columns past them stage garbage that only the waves owning those
// columns would read, and those waves skip both the products and the stores.
// Blocks are numbered expert-major, then n tile, then k tile.
constexpr int kW3Threads = 512;
constexpr int kW3Tile = 256;                           // C tile: 256 x 256
constexpr int kW3Rows = 32;
constexpr int kW3Stages = 4;
constexpr int kW3OpBytes = kW3Rows * kW3Tile * 2;       // one operand of one stage: 16 KB
constexpr int kW3StageBytes = 2 * kW3OpBytes;
constexpr int kW3LoadsPerChunk = 4;                     // per thread: 2 per operand
constexpr uint32_t kW3RsrcWord3 = 0x00020000u;

template <int N> struct W3VmCnt {
  static constexpr int imm = (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8);
};

typedef __attribute__((address_space(3))) void* lds_void_t;

// byte offset, within one operand of a stage, of this lane's first transposed
// read for the 16 columns starting at col0 (the second read is 4 rows = 2048
// bytes further)
__device__ __forceinline__ int chunk_swizzle(int row) {
  // rows 4 apart share it (the second transposed read is 2048 bytes on)
  return 2 * (row & 3) ^ 8 * ((row >> 3) & 1);
}

__device__ __forceinline__ int tr_offset(int col0, int lane) {
  const int g = lane >> 4, d = (lane >> 2) & 3, q = lane & 3;
  const int c = (col0 >> 3) + (q >> 1);                 // logical 16-byte chunk
  const int row = 8 * g + d;
  return row * 512 + ((c ^ chunk_swizzle(row)) << 4) + ((q & 1) << 3);
}

// Transposed reads are written as inline assembly: as compiler builtins they
// would make the compiler wait for every outstanding global-to-LDS load (it
// cannot tell that they target other stages).  Their results are used only
// after lds_wait() below, which passes them through an explicit lgkmcnt wait.
typedef int v2i_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ v8bf_t tr_fragment(uint32_t addr) {
  v2i_t lo, hi;
  // early-clobber outputs: the first read's destination must not share a
  // register with the address the second read still needs
  asm volatile("ds_read_b64_tr_b16 %0, %2\n\tds_read_b64_tr_b16 %1, %2 offset:2048"
               : "=&v"(lo), "=&v"(hi)
               : "v"(addr));
  const v2i_t both[2] = {lo, hi};
  return *reinterpret_cast<const v8bf_t*>(both);
}

__device__ __forceinline__ void lds_wait(v8bf_t (&f)[4]) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(f[0]), "+v"(f[1]), "+v"(f[2]), "+v"(f[3]));
}

__global__ __launch_bounds__(kW3Threads, 1) void wgrad_bf16_lds_kernel(
    const uint16_t* __restrict__ b, const uint16_t* __restrict__ a, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, int64_t rows_cap, int N, int K, int tiles_n, int tiles_k,
    float* __restrict__ c) {
  __shared__ __attribute__((aligned(16))) uint8_t s_ring[kW3Stages * kW3StageBytes];
  const int per_e = tiles_n * tiles_k;
  const int e = blockIdx.x / per_e;
  const int rem = blockIdx.x - e * per_e;
  const int n0 = (rem / tiles_k) * kW3Tile, k0 = (rem % tiles_k) * kW3Tile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t off = offsets[e];
  int cnt = 0;
  if (off >= 0 && off < rows_cap) cnt = static_cast<int>(min<int64_t>(counts[e], rows_cap - off));
  const int wn = 128 * (wave & 1), wk = 64 * (wave >> 1);
  const bool active = n0 + wn < N && k0 + wk < K;
  // load j of this wave covers rows 4*wave + 2j + [0,2) of a chunk: the
  // lane's row is 4*wave + 2j + (lane >> 5), its chunk position lane & 31
  int vB[2], vA[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 4 * wave + 2 * j + (lane >> 5);
    const int cl = (lane & 31) ^ chunk_swizzle(row);
    vB[j] = row * N * 2 + n0 * 2 + cl * 16;
    vA[j] = row * K * 2 + k0 * 2 + cl * 16;
  }
  auto issue = [&](int chunk) {
    uint8_t* st = s_ring + (chunk % kW3Stages) * kW3StageBytes;
    const int r0 = chunk * kW3Rows;
    const int rows = min(kW3Rows, cnt - r0);            // reads of rows past the count return 0
    const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(b + (off + r0) * N), 0, rows * N * 2, kW3RsrcWord3);
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a + (off + r0) * K), 0, rows * K * 2, kW3RsrcWord3);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_void_t)(st + (4 * wave + 2 * j) * 512), 16, vB[j], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void_t)(st + kW3OpBytes + (4 * wave + 2 * j) * 512), 16,
                                               vA[j], 0, 0, 0);
    }
  };
  const uint32_t lds_ring = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t)s_ring));
  uint32_t ob[8], oa[4];
#pragma unroll
  for (int x = 0; x < 8; ++x) ob[x] = tr_offset(wn + 16 * x, lane);
#pragma unroll
  for (int y = 0; y < 4; ++y) oa[y] = kW3OpBytes + tr_offset(wk + 16 * y, lane);
  v4f_t acc[8][4];
#pragma unroll
  for (int x = 0; x < 8; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = v4f_t{0.f, 0.f, 0.f, 0.f};
  const int nchunks = (cnt + kW3Rows - 1) / kW3Rows;
  for (int ch = 0; ch < kW3Stages - 1 && ch < nchunks; ++ch) issue(ch);
  for (int i = 0; i < nchunks; ++i) {
    // this thread's loads of chunk i have landed once at most the loads of
    // the chunks issued after it are outstanding
    const int after = min(kW3Stages - 2, nchunks - 1 - i);
    if (after >= 2) __builtin_amdgcn_s_waitcnt(W3VmCnt<2 * kW3LoadsPerChunk>::imm);
    else if (after == 1) __builtin_amdgcn_s_waitcnt(W3VmCnt<kW3LoadsPerChunk>::imm);
    else __builtin_amdgcn_s_waitcnt(W3VmCnt<0>::imm);
    // chunk i visible; chunk i - 1 fully read (its reads completed before its
    // products).  A bare barrier: no fence, which would wait for every load.
    asm volatile("s_barrier" ::: "memory");
    if (i + kW3Stages - 1 < nchunks) issue(i + kW3Stages - 1);
    if (active) {
      const uint32_t st = lds_ring + (i % kW3Stages) * kW3StageBytes;
      v8bf_t fa[4], fb0[4], fb1[4];
#pragma unroll
      for (int y = 0; y < 4; ++y) fa[y] = tr_fragment(st + oa[y]);
#pragma unroll
      for (int x = 0; x < 4; ++x) fb0[x] = tr_fragment(st + ob[x]);
      lds_wait(fa);
      lds_wait(fb0);
#pragma unroll
      for (int x = 0; x < 4; ++x) fb1[x] = tr_fragment(st + ob[4 + x]);
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb0[x], fa[y], acc[x][y], 0, 0, 0);
      lds_wait(fb1);
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y)
          acc[4 + x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb1[x], fa[y], acc[4 + x][y], 0, 0, 0);
    }
  }
  if (!active) return;
  // lane holds C[n = 16x + 4 * (lane >> 4) + r][k = 16y + (lane & 15)]: each
  // store writes 64 contiguous bytes of 4 rows (16-byte stores across 16 rows
  // measured slower)
  float* ce = c + static_cast<int64_t>(e) * N * K;
#pragma unroll
  for (int x = 0; x < 8; ++x)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = n0 + wn + 16 * x + 4 * (lane >> 4) + r;
#pragma unroll
      for (int y = 0; y < 4; ++y)
        __builtin_nontemporal_store(acc[x][y][r], &ce[static_cast<int64_t>(n) * K + k0 + wk + 16 * y + (lane & 15)]);
    }
}

}  // namespace

extern "C" moe_status moe_grouped_gemm_wgrad(const void* b, const void* a, moe_dtype dt,
                                             const int32_t* counts, const int32_t* offsets, int L,
                                             int64_t rows_cap, int N, int K, float* c, hipStream_t stream) {
  MOE_CHECK(L >= 1 && L <= 65535 && rows_cap >= 0 && N > 0 && K > 0 && moe_host::valid_dtype(dt),
            MOE_ERR_INVALID_ARG);
  MOE_CHECK(dt != MOE_FP8_E4M3, MOE_ERR_UNSUPPORTED);
  MOE_CHECK(N % kWgTile == 0 && K % kWgTile == 0, MOE_ERR_UNSUPPORTED);
  MOE_CHECK(c && counts && offsets && (rows_cap == 0 || (a && b)), MOE_ERR_INVALID_ARG);
  MOE_CHECK(((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b) | reinterpret_cast<uintptr_t>(c)) & 15) == 0,
            MOE_ERR_INVALID_ARG);
  const dim3 grid(K / kWgTile, N / kWgTile, L);
  if (dt == MOE_F32)
    wgrad_f32_kernel<<<grid, kThreads, 0, stream>>>(static_cast<const float*>(b), static_cast<const float*>(a),
                                                       counts, offsets, rows_cap, N, K, c);
  else {
    const int tn = (N + kW3Tile - 1) / kW3Tile, tk = (K + kW3Tile - 1) / kW3Tile;
    const int64_t blocks = static_cast<int64_t>(L) * tn * tk;
    MOE_CHECK(blocks <= INT32_MAX, MOE_ERR_UNSUPPORTED);
    MOE_CHECK(32LL * std::max(N, K) * 2 < (int64_t(1) << 31), MOE_ERR_UNSUPPORTED);   // per-chunk offsets
    wgrad_bf16_lds_kernel<<<static_cast<unsigned>(blocks), kW3Threads, 0, stream>>>(
        static_cast<const uint16_t*>(b), static_cast<const uint16_t*>(a), counts, offsets, rows_cap, N, K, tn, tk, c);
  }
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

extern "C" moe_status moe_combine_backward(const void* dy, moe_dtype dy_dt, const void* expert_out,
                                           moe_dtype eo_dt, const int32_t* slot_of,
                                           const float* topk_weights, int T, int K, int H, int64_t rows_cap,
                                           void* d_out, moe_dtype d_out_dt, float* d_weights,
                                           hipStream_t stream) {
  MOE_CHECK(T >= 0 && K > 0 && H > 0 && rows_cap >= 0, MOE_ERR_INVALID_ARG);
  MOE_CHECK(moe_host::valid_dtype(dy_dt) && moe_host::valid_dtype(eo_dt) && moe_host::valid_dtype(d_out_dt),
            MOE_ERR_INVALID_ARG);
  MOE_CHECK(dy_dt != MOE_FP8_E4M3 && eo_dt != MOE_FP8_E4M3 && d_out_dt != MOE_FP8_E4M3, MOE_ERR_UNSUPPORTED);
  MOE_CHECK(H % 8 == 0 && K <= 64, MOE_ERR_UNSUPPORTED);
  if (T == 0) return MOE_OK;
  MOE_CHECK(dy && slot_of && topk_weights && d_weights && (rows_cap == 0 || (expert_out && d_out)),
            MOE_ERR_INVALID_ARG);
  const int grid = (T + kWavesPerBlock - 1) / kWavesPerBlock;
  auto* g = static_cast<const uint8_t*>(dy);
  auto* o = static_cast<const uint8_t*>(expert_out);
  auto* d = static_cast<uint8_t*>(d_out);
  const int sel = (dy_dt == MOE_F32 ? 4 : 0) | (eo_dt == MOE_F32 ? 2 : 0) | (d_out_dt == MOE_F32 ? 1 : 0);
#define MOE_CB(A, B, C)                                                                                 \
  combine_backward_kernel<A, B, C><<<grid, kThreads, 0, stream>>>(g, o, slot_of, topk_weights, T, K, H, \
                                                                  rows_cap, d, d_weights)
  if (sel == 0 && H <= 8 * MOE_WAVE * kCbNper) {
    combine_backward_bf16_reg_kernel<<<grid, kThreads, 0, stream>>>(
        static_cast<const uint4*>(dy), static_cast<const uint4*>(expert_out), slot_of, topk_weights, T, K, H,
        rows_cap, static_cast<uint4*>(d_out), d_weights);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
  }
  switch (sel) {
    case 0: MOE_CB(false, false, false); break;
    case 1: MOE_CB(false, false, true); break;
    case 2: MOE_CB(false, true, false); break;
    case 3: MOE_CB(false, true, true); break;
    case 4: MOE_CB(true, false, false); break;
    case 5: MOE_CB(true, false, true); break;
    case 6: MOE_CB(true, true, false); break;
    default: MOE_CB(true, true, true); break;
  }
#undef MOE_CB
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

extern "C" moe_status moe_silu_mul_backward(const float* g, const void* dz, moe_dtype dz_dt,
                                            const int32_t* counts, const int32_t* offsets, int L,
                                            int64_t rows_cap, int I, void* dg, moe_dtype dg_dt,
                                            hipStream_t stream) {
  MOE_CHECK(L >= 1 && rows_cap >= 0 && I > 0, MOE_ERR_INVALID_ARG);
  MOE_CHECK(moe_host::valid_dtype(dz_dt) && moe_host::valid_dtype(dg_dt), MOE_ERR_INVALID_ARG);
  MOE_CHECK(dz_dt != MOE_FP8_E4M3 && dg_dt != MOE_FP8_E4M3, MOE_ERR_UNSUPPORTED);
  MOE_CHECK(I % 4 == 0, MOE_ERR_UNSUPPORTED);
  if (rows_cap == 0) return MOE_OK;
  MOE_CHECK(g && dz && dg && counts && offsets, MOE_ERR_INVALID_ARG);
  const int64_t grid64 = (rows_cap + kWavesPerBlock - 1) / kWavesPerBlock;
  MOE_CHECK(grid64 <= 0x7fffffff, MOE_ERR_UNSUPPORTED);
  const int grid = static_cast<int>(grid64);
  auto* z = static_cast<const uint8_t*>(dz);
  auto* d = static_cast<uint8_t*>(dg);
  if (dz_dt == MOE_F32 && dg_dt == MOE_F32)
    silu_mul_backward_kernel<true, true><<<grid, kThreads, 0, stream>>>(g, z, counts, offsets, L, rows_cap, I, d);
  else if (dz_dt == MOE_F32)
    silu_mul_backward_kernel<true, false><<<grid, kThreads, 0, stream>>>(g, z, counts, offsets, L, rows_cap, I, d);
  else if (dg_dt == MOE_F32)
    silu_mul_backward_kernel<false, true><<<grid, kThreads, 0, stream>>>(g, z, counts, offsets, L, rows_cap, I, d);
  else
    silu_mul_backward_kernel<false, false><<<grid, kThreads, 0, stream>>>(g, z, counts, offsets, L, rows_cap, I, d);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

extern "C" moe_status moe_transpose_weights(const void* w, moe_dtype w_dt, int L, int N, int K, void* wt,
                                            hipStream_t stream) {
  MOE_CHECK(L >= 1 && N > 0 && K > 0 && moe_host::valid_dtype(w_dt), MOE_ERR_INVALID_ARG);
  MOE_CHECK(w_dt != MOE_FP8_E4M3, MOE_ERR_UNSUPPORTED);
  MOE_CHECK(w && wt && w != wt, MOE_ERR_INVALID_ARG);
  MOE_CHECK(L <= 65535, MOE_ERR_UNSUPPORTED);
  const dim3 grid((K + 63) / 64, (N + 63) / 64, L);
  if (w_dt == MOE_F32)
    transpose_kernel<float><<<grid, kThreads, 0, stream>>>(static_cast<const float*>(w), N, K,
                                                           static_cast<float*>(wt));
  else if (N % 64 == 0 && K % 64 == 0 && ((reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(wt)) & 15) == 0)
    transpose_bf16_vec_kernel<<<grid, kThreads, 0, stream>>>(static_cast<const uint16_t*>(w), N, K,
                                                             static_cast<uint16_t*>(wt));
  else
    transpose_kernel<uint16_t><<<grid, kThreads, 0, stream>>>(static_cast<const uint16_t*>(w), N, K,
                                                              static_cast<uint16_t*>(wt));
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}
