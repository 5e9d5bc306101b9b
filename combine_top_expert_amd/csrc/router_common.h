// Device helpers of the router top-K (moe_router_topk): the score keys and
// one wavefront's top-K of one token.
#pragma once

#include "moe_common.h"

namespace moe_router {

// order-preserving image of an fp32 value: larger float -> larger key;
// every NaN maps below -inf, -0 and +0 map together
__device__ __forceinline__ uint32_t score_key(float v) {
  if (v != v) return 0u;
  uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave reductions by DPP modifiers of ordinary VALU operations.  Inside each
// 16-lane row: swap neighbours, swap pairs, mirror within 8, mirror within
// 16 -- each step combines two disjoint groups, so every lane ends with its
// row's result.  Across rows: row 1 takes lane 15 and row 3 lane 47 (rows
// 0+1, 2+3), then rows 2 and 3 take lane 31, so lane 63 holds the wave's
// result, read once into a uniform value.
template <int CTRL, int ROWS = 0xF> __device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(static_cast<int>(old), static_cast<int>(v), CTRL, ROWS, 0xF, false));
}
template <int CTRL, int ROWS = 0xF> __device__ __forceinline__ float dpp_f32(float old, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, ROWS, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // lane i <- lane 7 - i within 8
constexpr int kDppMirror = 0x140;       // lane i <- lane 15 - i within 16
constexpr int kDppBcast15 = 0x142;      // next row <- lane 15 of the row
constexpr int kDppBcast31 = 0x143;      // rows 2, 3 <- lane 31

// Reductions inside each 16-lane row only (four DPP steps).
__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kDppXor1>(v, v));
  v = max(v, dpp_u32<kDppXor2>(v, v));
  v = max(v, dpp_u32<kDppHalfMirror>(v, v));
  return max(v, dpp_u32<kDppMirror>(v, v));
}
__device__ __forceinline__ float row_max_f32(float v) {
  v = fmaxf(v, dpp_f32<kDppXor1>(v, v));
  v = fmaxf(v, dpp_f32<kDppXor2>(v, v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v, v));
  return fmaxf(v, dpp_f32<kDppMirror>(v, v));
}
__device__ __forceinline__ float row_sum_f32(float v) {
  v += dpp_f32<kDppXor1>(0.f, v);
  v += dpp_f32<kDppXor2>(0.f, v);
  v += dpp_f32<kDppHalfMirror>(0.f, v);
  return v + dpp_f32<kDppMirror>(0.f, v);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kDppXor1>(v, v));
  v = max(v, dpp_u32<kDppXor2>(v, v));
  v = max(v, dpp_u32<kDppHalfMirror>(v, v));
  v = max(v, dpp_u32<kDppMirror>(v, v));
  v = max(v, dpp_u32<kDppBcast15, 0xA>(v, v));
  v = max(v, dpp_u32<kDppBcast31, 0xC>(v, v));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, dpp_f32<kDppXor1>(v, v));
  v = fmaxf(v, dpp_f32<kDppXor2>(v, v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v, v));
  v = fmaxf(v, dpp_f32<kDppMirror>(v, v));
  v = fmaxf(v, dpp_f32<kDppBcast15, 0xA>(v, v));
  v = fmaxf(v, dpp_f32<kDppBcast31, 0xC>(v, v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// lanes outside the enabled rows add 0 (old operand 0)
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dpp_f32<kDppXor1>(0.f, v);
  v += dpp_f32<kDppXor2>(0.f, v);
  v += dpp_f32<kDppHalfMirror>(0.f, v);
  v += dpp_f32<kDppMirror>(0.f, v);
  v += dpp_f32<kDppBcast15, 0xA>(0.f, v);
  v += dpp_f32<kDppBcast31, 0xC>(0.f, v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Top-K of one token's scores by one wavefront.  Lane l holds experts l,
// l+64, ... as 32-bit keys: the order-preserving image of the score (logit +
// bias, one fp32 add), with every NaN mapped to 1, below every number, and
// 0 for an absent or retired entry.  Each of the K rounds takes the
// wave-wide maximum key; among the entries holding it the lowest expert id
// wins (expert l + 64j: the lowest j with a holder, then its lowest lane, by
// ballot), and its owner retires it.  Lane k < K returns round k's expert in
// *id and its renormalised softmax weight in *w (over the K selected
// values: the score, or the unbiased logit when the bias only steers the
// selection).
template <int NPL>
__device__ __forceinline__ void token_topk(const float* __restrict__ row, const float* __restrict__ bias, int E,
                                           int K, int bias_in_weights, int lane, int* id, float* w) {
  uint32_t key[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int e = lane + MOE_WAVE * j;
    key[j] = 0;
    if (e < E) {
      const float v = bias ? row[e] + bias[e] : row[e];
      key[j] = max(score_key(v), 1u);
    }
  }
  int my_id = -1;
  for (int k = 0; k < K; ++k) {
    uint32_t best = 0;
#pragma unroll
    for (int j = 0; j < NPL; ++j) best = max(best, key[j]);
    const uint32_t win = wave_max_u32(best);
    int e = -1;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const uint64_t holders = __ballot(key[j] == win);
      if (e < 0 && holders) {
        const int owner = __builtin_ctzll(holders);
        e = MOE_WAVE * j + owner;
        if (lane == owner) key[j] = 0;
      }
    }
    if (lane == k) my_id = e;
  }
  float my_v = 0.0f;
  if (lane < K) my_v = (bias && bias_in_weights) ? row[my_id] + bias[my_id] : row[my_id];
  const float m = wave_max_f32(lane < K ? my_v : -INFINITY);
  const float p = lane < K ? expf(my_v - m) : 0.0f;
  const float s = wave_sum_f32(p);
  *id = my_id;
  *w = p / s;
}

}  // namespace moe_router
