// moe_permute: token rows -> expert-major buffer, optionally quantised to
// block FP8 on the way ("SGLang、NCCL 与 MoE EP" §2.3.4 and §2.3.5;
// "DeepEP 架构与实现笔记" §9.4 and §11).
//
// A wavefront reads a token's routes once (lane k = route k), reads its row
// (for bf16 -> FP8 one 1024-column part of it, for a same-dtype copy one
// 2 KB part) from HBM once, quantises it once (the code of a row does not
// depend on which expert receives it) and stores it to each of its local
// slots.  A 128-column FP8
// group is covered by 16 lanes of 8 values (bf16 input) or 32 lanes of 4
// values (fp32 input); its amax is a butterfly max inside those lanes.
// Tokens without a local route read nothing.
//
// The bf16 and copy kernels run one wave per workgroup and read the token
// rows with ordinary (cache-allocating) loads: measured inside the whole
// layer on MI355X, both beat four-wave workgroups and non-temporal loads.
// Copies store non-temporally: ordinary stores shorten the copy but leave
// dirty lines that the next GEMM then pays for, with no net gain.

#include "moe_common.h"

namespace {

constexpr int kThreads = 256;                 // fp32 -> FP8 kernel
constexpr int kTokPerBlock = kThreads / MOE_WAVE;
constexpr int kUnroll = 16;          // 16-byte chunks per lane in flight (a 4096-column fp32 row)

template <typename TIn> struct Vec;
template <> struct Vec<uint16_t> {  // 8 bf16 per 16-byte chunk
  static constexpr int N = 8;
  static __device__ __forceinline__ void to_f32(const uint4& r, float* f) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <> struct Vec<float> {     // 4 fp32 per 16-byte chunk
  static constexpr int N = 4;
  static __device__ __forceinline__ void to_f32(const uint4& r, float* f) {
    f[0] = __uint_as_float(r.x);
    f[1] = __uint_as_float(r.y);
    f[2] = __uint_as_float(r.z);
    f[3] = __uint_as_float(r.w);
  }
};

template <int LANES> __device__ __forceinline__ float group_max(float v) {
  v = moe::group16_max(v);
  if constexpr (LANES == 32) v = fmaxf(v, __shfl_xor(v, 16));
  return v;
}

// fp32 -> block FP8: one wave per token, up to 16 16-byte chunks per lane in
// flight; a 128-column group is 32 lanes of 4 values.
__global__ __launch_bounds__(kThreads) void permute_f32_fp8_kernel(const float* __restrict__ x, int T, int K,
                                                                  int H, const int32_t* __restrict__ slot_of,
                                                                  int64_t rows_cap, uint8_t* __restrict__ buf,
                                                                  float* __restrict__ scales) {
  constexpr int EPC = Vec<float>::N;            // elements per 16-byte chunk
  constexpr int LPG = 128 / EPC;                // lanes per 128-column group
  const int wave = threadIdx.x / MOE_WAVE;
  const int lane = moe::lane_id();
  const int t = blockIdx.x * kTokPerBlock + wave;
  if (t >= T) return;
  // lane k holds route k of the token; ballot bit k marks a local slot
  const int s_l = lane < K ? slot_of[static_cast<int64_t>(t) * K + lane] : -1;
  const uint64_t routes = __ballot(s_l >= 0 && s_l < rows_cap);
  if (!routes) return;

  const int nchunk = H / EPC;
  const uint4* xrow = reinterpret_cast<const uint4*>(x + static_cast<int64_t>(t) * H);
  const int groups = H / 128;

  for (int c0 = 0; c0 < nchunk; c0 += MOE_WAVE * kUnroll) {
    uint4 raw[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = c0 + u * MOE_WAVE + lane;
      raw[u] = c < nchunk ? moe::load_nt16(xrow + c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int cw = c0 + u * MOE_WAVE;          // wave-uniform chunk base
      if (cw >= nchunk) break;
      const int c = cw + lane;
      const bool live = c < nchunk;
      float f[EPC];
      Vec<float>::to_f32(raw[u], f);
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < EPC; ++i) amax = fmaxf(amax, fabsf(f[i]));
      amax = moe::fp8_group_amax_clamp(group_max<LPG>(amax));
      const float inv = moe::fp8_group_inv(amax);
      const uint32_t code = moe::f32x4_to_e4m3(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv);
      const float scale = moe::fp8_group_scale(amax);
      const int g = c / LPG;
      for (uint64_t m = routes; m; m &= m - 1) {
        const int s = __builtin_amdgcn_readlane(s_l, __builtin_ctzll(m));
        if (!live) continue;
        *reinterpret_cast<uint32_t*>(buf + static_cast<int64_t>(s) * H + c * EPC) = code;
        if ((lane % LPG) == 0) scales[static_cast<int64_t>(s) * groups + g] = scale;
      }
    }
  }
}

// Same-dtype copy (bf16 or fp32): one wave per (token, 2 KB part of its
// row); lane l moves the 16-byte chunks 128p + 64u + l, so each load and
// store instruction covers 1 KB of a row contiguously.
constexpr int kCopyLoads = 2;
constexpr int kCopyChunks = kCopyLoads * MOE_WAVE;

__global__ __launch_bounds__(MOE_WAVE) void permute_copy_kernel(const uint8_t* __restrict__ x, int T, int K,
                                                               int row_bytes, const int32_t* __restrict__ slot_of,
                                                               int64_t rows_cap, uint8_t* __restrict__ buf,
                                                               int parts) {
  const int lane = moe::lane_id();
  const int item = blockIdx.x;                            // (token, part)
  const int t = item / parts;
  const int p = item - t * parts;
  if (t >= T) return;
  const int s_l = lane < K ? slot_of[static_cast<int64_t>(t) * K + lane] : -1;
  const uint64_t routes = __ballot(s_l >= 0 && s_l < rows_cap);
  if (!routes) return;
  const int nchunk = row_bytes / 16;
  const uint4* xrow = reinterpret_cast<const uint4*>(x + static_cast<int64_t>(t) * row_bytes);
  uint4 raw[kCopyLoads];
#pragma unroll
  for (int u = 0; u < kCopyLoads; ++u) {
    const int c = p * kCopyChunks + u * MOE_WAVE + lane;
    raw[u] = c < nchunk ? xrow[c] : make_uint4(0, 0, 0, 0);
  }
  for (uint64_t m = routes; m; m &= m - 1) {
    const int s = __builtin_amdgcn_readlane(s_l, __builtin_ctzll(m));
    uint4* dst = reinterpret_cast<uint4*>(buf + static_cast<int64_t>(s) * row_bytes);
#pragma unroll
    for (int u = 0; u < kCopyLoads; ++u) {
      const int c = p * kCopyChunks + u * MOE_WAVE + lane;
      if (c < nchunk) moe::store_nt16(dst + c, raw[u]);
    }
  }
}

// bf16 -> block FP8, the main path.  A wave takes one 1024-column part of a
// token's row: lane l converts the 8-value chunks 128p + l and 128p + 64 + l,
// so each load instruction reads 1 KB of the row contiguously and each code
// store writes 512 contiguous bytes.  A 128-column group is 16 lanes of one
// load; its amax is a 4-step butterfly.  Many short waves (7 per row at
// H = 7168) keep loads and stores of different tokens in flight together.
constexpr int kPartLoads = 2;                       // 16-byte chunks per lane
constexpr int kPartChunks = kPartLoads * MOE_WAVE;  // 8-column chunks per part

__global__ __launch_bounds__(MOE_WAVE) void permute_bf16_fp8_kernel(const uint16_t* __restrict__ x, int T,
                                                                   int K, int H,
                                                                   const int32_t* __restrict__ slot_of,
                                                                   int64_t rows_cap, uint8_t* __restrict__ buf,
                                                                   float* __restrict__ scales, int parts) {
  const int lane = moe::lane_id();
  const int item = blockIdx.x;                            // (token, part)
  const int t = item / parts;
  const int p = item - t * parts;
  if (t >= T) return;
  const int s_l = lane < K ? slot_of[static_cast<int64_t>(t) * K + lane] : -1;
  const uint64_t routes = __ballot(s_l >= 0 && s_l < rows_cap);
  if (!routes) return;

  const int nchunk = H / 8;
  const int groups = H / 128;
  const uint4* xrow = reinterpret_cast<const uint4*>(x + static_cast<int64_t>(t) * H);
  int c[kPartLoads];
  bool live[kPartLoads];
  uint4 raw[kPartLoads];
#pragma unroll
  for (int h = 0; h < kPartLoads; ++h) {
    c[h] = p * kPartChunks + h * MOE_WAVE + lane;
    live[h] = c[h] < nchunk;
    raw[h] = live[h] ? xrow[c[h]] : make_uint4(0, 0, 0, 0);
  }
  uint2 codes[kPartLoads];
  float scale[kPartLoads];
#pragma unroll
  for (int h = 0; h < kPartLoads; ++h) {
    float f[8];
    Vec<uint16_t>::to_f32(raw[h], f);
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
    amax = moe::fp8_group_amax_clamp(moe::group16_max(amax));
    const float inv = moe::fp8_group_inv(amax);
    codes[h] = make_uint2(moe::f32x4_to_e4m3(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv),
                          moe::f32x4_to_e4m3(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv));
    scale[h] = moe::fp8_group_scale(amax);
  }
  for (uint64_t m = routes; m; m &= m - 1) {
    const int s = __builtin_amdgcn_readlane(s_l, __builtin_ctzll(m));
    uint8_t* dst = buf + static_cast<int64_t>(s) * H;
#pragma unroll
    for (int h = 0; h < kPartLoads; ++h) {
      if (!live[h]) continue;
      *reinterpret_cast<uint2*>(dst + c[h] * 8) = codes[h];
      if ((lane & 15) == 0) scales[static_cast<int64_t>(s) * groups + (c[h] >> 4)] = scale[h];
    }
  }
}

}  // namespace

extern "C" moe_status moe_permute(const void* x, moe_dtype x_dt, int T, int K, int H,
                                  const int32_t* slot_of, int64_t rows_cap, void* buf,
                                  moe_dtype buf_dt, float* buf_scales, hipStream_t stream) {
  MOE_CHECK(T >= 0 && K > 0 && H > 0 && rows_cap >= 0, MOE_ERR_INVALID_ARG);
  MOE_CHECK(moe_host::valid_dtype(x_dt) && moe_host::valid_dtype(buf_dt), MOE_ERR_INVALID_ARG);
  MOE_CHECK(H % 128 == 0 && K <= 64, MOE_ERR_UNSUPPORTED);
  MOE_CHECK(x_dt == MOE_F32 || x_dt == MOE_BF16, MOE_ERR_UNSUPPORTED);
  MOE_CHECK(buf_dt == x_dt || buf_dt == MOE_FP8_E4M3, MOE_ERR_UNSUPPORTED);
  if (T == 0 || rows_cap == 0) return MOE_OK;
  MOE_CHECK(x && slot_of && buf, MOE_ERR_INVALID_ARG);
  MOE_CHECK(buf_dt != MOE_FP8_E4M3 || buf_scales, MOE_ERR_INVALID_ARG);
  auto* b = static_cast<uint8_t*>(buf);
  auto item_grid = [&](int parts, int per_block, int& grid) -> bool {
    const int64_t g = (static_cast<int64_t>(T) * parts + per_block - 1) / per_block;
    grid = static_cast<int>(g);
    return g <= 0x7fffffff;
  };
  int grid = 0;
  if (buf_dt == x_dt) {
    const int row_bytes = H * (x_dt == MOE_BF16 ? 2 : 4);
    const int parts = (row_bytes / 16 + kCopyChunks - 1) / kCopyChunks;
    MOE_CHECK(item_grid(parts, 1, grid), MOE_ERR_UNSUPPORTED);
    permute_copy_kernel<<<grid, MOE_WAVE, 0, stream>>>(static_cast<const uint8_t*>(x), T, K, row_bytes, slot_of,
                                                       rows_cap, b, parts);
  } else if (x_dt == MOE_BF16) {
    const int parts = (H / 8 + kPartChunks - 1) / kPartChunks;
    MOE_CHECK(item_grid(parts, 1, grid), MOE_ERR_UNSUPPORTED);
    permute_bf16_fp8_kernel<<<grid, MOE_WAVE, 0, stream>>>(static_cast<const uint16_t*>(x), T, K, H, slot_of,
                                                           rows_cap, b, buf_scales, parts);
  } else {
    MOE_CHECK(item_grid(1, kTokPerBlock, grid), MOE_ERR_UNSUPPORTED);
    permute_f32_fp8_kernel<<<grid, kThreads, 0, stream>>>(static_cast<const float*>(x), T, K, H, slot_of,
                                                          rows_cap, b, buf_scales);
  }
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}
