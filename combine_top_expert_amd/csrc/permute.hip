// moe_permute: token rows -> expert-major buffer, optionally quantised to
// block FP8 on the way ("SGLang、NCCL 与 MoE EP" §2.3.4 and §2.3.5;
// "DeepEP 架构与实现笔记" §9.4 and §11).
//
// One wavefront per token.  The token's routes are read once (lane k =
// route k); its row is read from HBM once, with up to 256 bytes per lane in
// flight, quantised once (the code of a row does not depend on which expert
// receives it), and stored to each of its local slots.  A 128-column FP8
// group is covered by 8 lanes of 16 values (bf16 input, 16-byte code stores)
// or 32 lanes of 4 values (fp32 input); its amax is a butterfly max inside
// those lanes.  Tokens without a local route read nothing.

#include "moe_common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kTokPerBlock = kThreads / MOE_WAVE;
constexpr int kUnroll = 16;          // 16-byte chunks per lane in flight (a 8192-column bf16 row)

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

template <typename TIn, bool kFp8>
__global__ __launch_bounds__(kThreads) void permute_kernel(const TIn* __restrict__ x, int T, int K,
                                                           int H, const int32_t* __restrict__ slot_of,
                                                           int64_t rows_cap, uint8_t* __restrict__ buf,
                                                           float* __restrict__ scales) {
  constexpr int EPC = Vec<TIn>::N;              // elements per 16-byte chunk
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
  const int out_row_bytes = kFp8 ? H : H * static_cast<int>(sizeof(TIn));
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
      if constexpr (kFp8) {
        float f[EPC];
        Vec<TIn>::to_f32(raw[u], f);
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < EPC; ++i) amax = fmaxf(amax, fabsf(f[i]));
        amax = moe::fp8_group_amax_clamp(group_max<LPG>(amax));
        const float inv = moe::fp8_group_inv(amax);
        uint32_t codes[EPC / 4];
#pragma unroll
        for (int i = 0; i < EPC / 4; ++i)
          codes[i] = moe::f32x4_to_e4m3(f[4 * i] * inv, f[4 * i + 1] * inv, f[4 * i + 2] * inv,
                                        f[4 * i + 3] * inv);
        const float scale = moe::fp8_group_scale(amax);
        const int g = c / LPG;
        for (uint64_t m = routes; m; m &= m - 1) {
          const int s = __builtin_amdgcn_readlane(s_l, __builtin_ctzll(m));
          if (!live) continue;
          uint8_t* dst = buf + static_cast<int64_t>(s) * out_row_bytes + c * EPC;
          if constexpr (EPC == 8) {
            *reinterpret_cast<uint2*>(dst) = make_uint2(codes[0], codes[1]);
          } else {
            *reinterpret_cast<uint32_t*>(dst) = codes[0];
          }
          if ((lane % LPG) == 0) scales[static_cast<int64_t>(s) * groups + g] = scale;
        }
      } else {
        for (uint64_t m = routes; m; m &= m - 1) {
          const int s = __builtin_amdgcn_readlane(s_l, __builtin_ctzll(m));
          if (!live) continue;
          uint4* dst = reinterpret_cast<uint4*>(buf + static_cast<int64_t>(s) * out_row_bytes) + c;
          moe::store_nt16(dst, raw[u]);
        }
      }
    }
  }
}

// bf16 -> block FP8, the main path: each lane converts 16 consecutive
// values (two 16-byte loads) into one 16-byte store of codes per local slot,
// so a 128-column group is 8 lanes and a wave stores 1 KB per instruction.
constexpr int kUnroll2 = 8;          // 32-byte lane units in flight (a 8192-column row)

__global__ __launch_bounds__(kThreads) void permute_bf16_fp8_kernel(const uint16_t* __restrict__ x, int T,
                                                                   int K, int H,
                                                                   const int32_t* __restrict__ slot_of,
                                                                   int64_t rows_cap, uint8_t* __restrict__ buf,
                                                                   float* __restrict__ scales) {
  const int wave = threadIdx.x / MOE_WAVE;
  const int lane = moe::lane_id();
  const int t = blockIdx.x * kTokPerBlock + wave;
  if (t >= T) return;
  const int s_l = lane < K ? slot_of[static_cast<int64_t>(t) * K + lane] : -1;
  const uint64_t routes = __ballot(s_l >= 0 && s_l < rows_cap);
  if (!routes) return;

  const int nunit = H / 16;                       // 32-byte units of the input row
  const uint4* xrow = reinterpret_cast<const uint4*>(x + static_cast<int64_t>(t) * H);
  const int groups = H / 128;
  for (int d0 = 0; d0 < nunit; d0 += MOE_WAVE * kUnroll2) {
    uint4 raw[kUnroll2][2];
#pragma unroll
    for (int u = 0; u < kUnroll2; ++u) {
      const int d = d0 + u * MOE_WAVE + lane;
      const bool live = d < nunit;
      raw[u][0] = live ? moe::load_nt16(xrow + 2 * d) : make_uint4(0, 0, 0, 0);
      raw[u][1] = live ? moe::load_nt16(xrow + 2 * d + 1) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll2; ++u) {
      const int dw = d0 + u * MOE_WAVE;           // wave-uniform unit base
      if (dw >= nunit) break;
      const int d = dw + lane;
      const bool live = d < nunit;
      float f[16];
      Vec<uint16_t>::to_f32(raw[u][0], f);
      Vec<uint16_t>::to_f32(raw[u][1], f + 8);
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
      amax = fmaxf(amax, __shfl_xor(amax, 1));
      amax = fmaxf(amax, __shfl_xor(amax, 2));
      amax = fmaxf(amax, __shfl_xor(amax, 4));
      amax = moe::fp8_group_amax_clamp(amax);
      const float inv = moe::fp8_group_inv(amax);
      uint4 codes;
      codes.x = moe::f32x4_to_e4m3(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv);
      codes.y = moe::f32x4_to_e4m3(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv);
      codes.z = moe::f32x4_to_e4m3(f[8] * inv, f[9] * inv, f[10] * inv, f[11] * inv);
      codes.w = moe::f32x4_to_e4m3(f[12] * inv, f[13] * inv, f[14] * inv, f[15] * inv);
      const float scale = moe::fp8_group_scale(amax);
      const int g = d >> 3;
      for (uint64_t m = routes; m; m &= m - 1) {
        const int s = __builtin_amdgcn_readlane(s_l, __builtin_ctzll(m));
        if (!live) continue;
        moe::store_nt16(buf + static_cast<int64_t>(s) * H + d * 16, codes);
        if ((lane & 7) == 0) scales[static_cast<int64_t>(s) * groups + g] = scale;
      }
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
  const int grid = (T + kTokPerBlock - 1) / kTokPerBlock;
  auto* b = static_cast<uint8_t*>(buf);
  if (x_dt == MOE_BF16) {
    auto* xi = static_cast<const uint16_t*>(x);
    if (buf_dt == MOE_FP8_E4M3)
      permute_bf16_fp8_kernel<<<grid, kThreads, 0, stream>>>(xi, T, K, H, slot_of, rows_cap, b, buf_scales);
    else
      permute_kernel<uint16_t, false><<<grid, kThreads, 0, stream>>>(xi, T, K, H, slot_of, rows_cap, b, nullptr);
  } else {
    auto* xi = static_cast<const float*>(x);
    if (buf_dt == MOE_FP8_E4M3)
      permute_kernel<float, true><<<grid, kThreads, 0, stream>>>(xi, T, K, H, slot_of, rows_cap, b, buf_scales);
    else
      permute_kernel<float, false><<<grid, kThreads, 0, stream>>>(xi, T, K, H, slot_of, rows_cap, b, nullptr);
  }
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}
