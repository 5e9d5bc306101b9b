// moe_router_topk: router logits -> top-K expert ids and renormalised
// softmax weights, the TopKOutput the dispatch path starts from ("SGLang、
// NCCL 与 MoE EP" §1.1: router scores, a selection policy returns K ids and
// weights; §3.6: topk_ids [T,K], topk_weights [T,K]).
//
// One wavefront per token.  Lane l holds the scores of experts l, l+64, ...
// (score = logit + bias, one fp32 add).  Each of the K rounds takes the
// wave-wide maximum of a 64-bit key -- an order-preserving integer image of
// the score in the high word (NaN lowest, -0 folded onto +0) and the
// complement of the expert id in the low word, so equal scores go to the
// lower id -- and retires the winner.  Lane k keeps round k's expert; the K
// lanes then form exp(v - max) and its sum with wave reductions, and divide.

#include "moe_common.h"
#include "router_common.h"

namespace {

using namespace moe_router;

constexpr int kThreads = 256;
constexpr int kTokPerBlock = kThreads / MOE_WAVE;
constexpr int kMaxE = 1024;
constexpr int kMaxK = 64;

template <int NPL>   // scores per lane: E <= 64 * NPL
__global__ __launch_bounds__(kThreads) void router_topk_kernel(const float* __restrict__ logits,
                                                               const float* __restrict__ bias, int T,
                                                               int E, int K, int bias_in_weights,
                                                               int32_t* __restrict__ ids,
                                                               float* __restrict__ weights) {
  const int lane = moe::lane_id();
  const int t = blockIdx.x * kTokPerBlock + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + static_cast<int64_t>(t) * E;
  int my_id;
  float my_w;
  token_topk<NPL>(row, bias, E, K, bias_in_weights, lane, &my_id, &my_w);
  if (lane < K) {
    ids[static_cast<int64_t>(t) * K + lane] = my_id;
    weights[static_cast<int64_t>(t) * K + lane] = my_w;
  }
}

// One token per kSeg-lane segment (16: four tokens per wave).  Lane s of a
// segment holds experts s, s+kSeg, ...; a round is a local maximum plus
// log2(kSeg) in-segment exchange steps, and the softmax reductions stay in
// the segment.
// Keys and ties as above, so the ids are the same; the weights' sum runs in a
// different order (within an ulp or so).
template <int kSeg, int NPL>   // lanes per token, scores per lane: E <= kSeg * NPL
__global__ __launch_bounds__(kThreads) void router_topk_seg_kernel(const float* __restrict__ logits,
                                                                   const float* __restrict__ bias, int T,
                                                                   int E, int K, int bias_in_weights,
                                                                   int32_t* __restrict__ ids,
                                                                   float* __restrict__ weights) {
  const int lane = moe::lane_id();
  const int sl = lane & (kSeg - 1);
  const int t = (blockIdx.x * kTokPerBlock + (threadIdx.x >> 6)) * (MOE_WAVE / kSeg) + lane / kSeg;
  const bool tok = t < T;                      // the whole segment agrees
  const float* row = logits + static_cast<int64_t>(tok ? t : 0) * E;
  uint64_t key[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int e = sl + kSeg * j;
    key[j] = 0;
    if (tok && e < E) {
      const float v = bias ? row[e] + bias[e] : row[e];
      key[j] = (static_cast<uint64_t>(score_key(v)) << 32) | (0xffffffffu - static_cast<uint32_t>(e));
    }
  }
  int my_id = 0;
  for (int k = 0; k < K; ++k) {
    uint64_t win = 0;
#pragma unroll
    for (int j = 0; j < NPL; ++j) win = key[j] > win ? key[j] : win;
#pragma unroll
    for (int d = 1; d < kSeg; d <<= 1) {
      const uint32_t lo = __shfl_xor(static_cast<uint32_t>(win), d);
      const uint32_t hi = __shfl_xor(static_cast<uint32_t>(win >> 32), d);
      const uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
      win = o > win ? o : win;
    }
    // keys are unique (the expert id is part of them): the owner retires it
#pragma unroll
    for (int j = 0; j < NPL; ++j) key[j] = key[j] == win ? 0 : key[j];
    if (sl == k) my_id = static_cast<int>(0xffffffffu - static_cast<uint32_t>(win));
  }
  const bool mine = tok && sl < K;
  const float my_v = mine ? ((bias && bias_in_weights) ? row[my_id] + bias[my_id] : row[my_id]) : 0.0f;
  float m = mine ? my_v : -INFINITY;
#pragma unroll
  for (int d = 1; d < kSeg; d <<= 1) m = fmaxf(m, __shfl_xor(m, d));
  const float p = mine ? expf(my_v - m) : 0.0f;
  float sum = p;
#pragma unroll
  for (int d = 1; d < kSeg; d <<= 1) sum += __shfl_xor(sum, d);
  if (mine) {
    ids[static_cast<int64_t>(t) * K + sl] = my_id;
    weights[static_cast<int64_t>(t) * K + sl] = p / sum;
  }
}

template <int kSeg, int NPL>
void launch_seg(const float* logits, const float* bias, int T, int E, int K, int biw, int32_t* ids,
                float* w, hipStream_t stream) {
  constexpr int kTokPerBlockSeg = kTokPerBlock * (MOE_WAVE / kSeg);
  const int grid = (T + kTokPerBlockSeg - 1) / kTokPerBlockSeg;
  router_topk_seg_kernel<kSeg, NPL><<<grid, kThreads, 0, stream>>>(logits, bias, T, E, K, biw, ids, w);
}

template <int NPL>
void launch(const float* logits, const float* bias, int T, int E, int K, int biw, int32_t* ids,
            float* w, hipStream_t stream) {
  const int grid = (T + kTokPerBlock - 1) / kTokPerBlock;
  router_topk_kernel<NPL><<<grid, kThreads, 0, stream>>>(logits, bias, T, E, K, biw, ids, w);
}

}  // namespace

extern "C" moe_status moe_router_topk(const float* logits, const float* bias, int T, int E, int K,
                                      int bias_in_weights, int32_t* topk_ids, float* topk_weights,
                                      hipStream_t stream) {
  MOE_CHECK(T >= 0 && E >= 1 && K >= 1 && K <= E, MOE_ERR_INVALID_ARG);
  MOE_CHECK(E <= kMaxE && K <= kMaxK, MOE_ERR_UNSUPPORTED);
  if (T == 0) return MOE_OK;
  MOE_CHECK(logits && topk_ids && topk_weights, MOE_ERR_INVALID_ARG);
  const int biw = bias_in_weights ? 1 : 0;
  // 16-lane segments where they measured faster: E <= 128 at any T, wider E
  // once T gives enough tokens (at E = 256: 16.4 vs 13.4 us for 8192 tokens,
  // 24.7 vs 43.4 us for 32768)
  if (K <= 16 && E <= 256 && (E <= 128 || T >= 16384)) {
    if (E <= 64) launch_seg<16, 4>(logits, bias, T, E, K, biw, topk_ids, topk_weights, stream);
    else if (E <= 128) launch_seg<16, 8>(logits, bias, T, E, K, biw, topk_ids, topk_weights, stream);
    else launch_seg<16, 16>(logits, bias, T, E, K, biw, topk_ids, topk_weights, stream);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
  }
  if (E <= 64) launch<1>(logits, bias, T, E, K, biw, topk_ids, topk_weights, stream);
  else if (E <= 128) launch<2>(logits, bias, T, E, K, biw, topk_ids, topk_weights, stream);
  else if (E <= 256) launch<4>(logits, bias, T, E, K, biw, topk_ids, topk_weights, stream);
  else if (E <= 512) launch<8>(logits, bias, T, E, K, biw, topk_ids, topk_weights, stream);
  else launch<16>(logits, bias, T, E, K, biw, topk_ids, topk_weights, stream);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}
