// Device helpers of the router top-K, shared by moe_router_topk and the
// router fused with the dispatch layout's count pass.
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

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
#pragma unroll
  for (int d = 1; d < MOE_WAVE; d <<= 1) {
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(k), d);
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(k >> 32), d);
    const uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
    k = o > k ? o : k;
  }
  return k;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int d = 1; d < MOE_WAVE; d <<= 1) v = fmaxf(v, __shfl_xor(v, d));
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int d = 1; d < MOE_WAVE; d <<= 1) v += __shfl_xor(v, d);
  return v;
}

// Top-K of one token's scores by one wavefront.  Lane l holds experts l,
// l+64, ...; each of the K rounds takes the wave-wide maximum of a 64-bit
// key -- the order-preserving image of the score (logit + bias, one fp32
// add) in the high word and the complement of the expert id in the low word,
// so equal scores go to the lower id -- and the owner retires the winner.
// Lane k < K returns round k's expert in *id and its renormalised softmax
// weight in *w (over the K selected values: the score, or the unbiased
// logit when the bias only steers the selection).
template <int NPL>
__device__ __forceinline__ void token_topk(const float* __restrict__ row, const float* __restrict__ bias, int E,
                                           int K, int bias_in_weights, int lane, int* id, float* w) {
  uint64_t key[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int e = lane + MOE_WAVE * j;
    key[j] = 0;                                  // absent: below every real entry
    if (e < E) {
      const float v = bias ? row[e] + bias[e] : row[e];
      // low word 0xffffffff - e > 0, so a present entry (even a NaN score,
      // high word 0) always beats an absent or retired one (key 0)
      key[j] = (static_cast<uint64_t>(score_key(v)) << 32) | (0xffffffffu - static_cast<uint32_t>(e));
    }
  }
  int my_id = -1;
  for (int k = 0; k < K; ++k) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < NPL; ++j) best = key[j] > best ? key[j] : best;
    const uint64_t win = wave_max_u64(best);
    const int e = static_cast<int>(0xffffffffu - static_cast<uint32_t>(win));
    // keys are unique (the expert id is part of them): the owner retires it
#pragma unroll
    for (int j = 0; j < NPL; ++j) key[j] = key[j] == win ? 0 : key[j];
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
