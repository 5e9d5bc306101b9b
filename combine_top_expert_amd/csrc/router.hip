// moe_router_topk: router logits -> top-K expert ids and renormalised
// softmax weights, the TopKOutput the dispatch path starts from ("SGLang、
// NCCL 与 MoE EP" §1.1: router scores, a selection policy returns K ids and
// weights; §3.6: topk_ids [T,K], topk_weights [T,K]).
//
// One wavefront per token.  Lane l holds the scores of experts l, l+64, ...
// (score = logit + bias, one fp32 add) as order-preserving 32-bit keys (NaN
// lowest, -0 folded onto +0).  Each of the K rounds takes the wave-wide
// maximum key (DPP steps inside 16-lane rows, two exchanges across rows);
// among its holders the lowest expert id wins, found by ballot, so equal
// scores go to the lower id; the owner retires it.  Lane k keeps round k's
// expert; the K lanes then form exp(v - max) and its sum with wave
// reductions, and divide.

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

// One token per 16-lane segment (four tokens per wave), the segment being
// one DPP row.  Lane s of a segment holds experts s, s+16, ... as the keys
// above; a round is a local maximum plus the four in-row DPP steps, and the
// lowest expert id among the holders of the maximum is found from the
// segment's bits of one ballot per key slot.  The softmax reductions stay in
// the row.  Same ids as the wave-per-token kernel; the weights' sum runs in
// the same order within 16 lanes.
constexpr int kSeg = 16;
template <int NPL>   // scores per lane: E <= 16 * NPL
__global__ __launch_bounds__(kThreads) void router_topk_seg_kernel(const float* __restrict__ logits,
                                                                   const float* __restrict__ bias, int T,
                                                                   int E, int K, int bias_in_weights,
                                                                   int32_t* __restrict__ ids,
                                                                   float* __restrict__ weights) {
  const int lane = moe::lane_id();
  const int sl = lane & (kSeg - 1);
  const int seg_shift = lane & ~(kSeg - 1);      // the segment's first lane
  const int t = (blockIdx.x * kTokPerBlock + (threadIdx.x >> 6)) * (MOE_WAVE / kSeg) + lane / kSeg;
  const bool tok = t < T;                        // the whole segment agrees
  const float* row = logits + static_cast<int64_t>(tok ? t : 0) * E;
  uint32_t key[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int e = sl + kSeg * j;
    key[j] = 0;
    if (tok && e < E) {
      const float v = bias ? row[e] + bias[e] : row[e];
      key[j] = max(score_key(v), 1u);
    }
  }
  int my_id = 0;
  for (int k = 0; k < K; ++k) {
    uint32_t best = 0;
#pragma unroll
    for (int j = 0; j < NPL; ++j) best = max(best, key[j]);
    const uint32_t win = row_max_u32(best);
    int e = -1;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const uint32_t holders = static_cast<uint32_t>(__ballot(key[j] == win) >> seg_shift) & 0xffffu;
      if (e < 0 && holders) {
        const int owner = __builtin_ctz(holders);
        e = kSeg * j + owner;
        if (sl == owner) key[j] = 0;
      }
    }
    if (sl == k) my_id = e;
  }
  const bool mine = tok && sl < K;
  const float my_v = mine ? ((bias && bias_in_weights) ? row[my_id] + bias[my_id] : row[my_id]) : 0.0f;
  const float m = row_max_f32(mine ? my_v : -INFINITY);
  const float p = mine ? expf(my_v - m) : 0.0f;
  const float sum = row_sum_f32(p);
  if (mine) {
    ids[static_cast<int64_t>(t) * K + sl] = my_id;
    weights[static_cast<int64_t>(t) * K + sl] = p / sum;
  }
}

template <int NPL>
void launch_seg(const float* logits, const float* bias, int T, int E, int K, int biw, int32_t* ids,
                float* w, hipStream_t stream) {
  constexpr int kTokPerBlockSeg = kTokPerBlock * (MOE_WAVE / kSeg);
  const int grid = (T + kTokPerBlockSeg - 1) / kTokPerBlockSeg;
  router_topk_seg_kernel<NPL><<<grid, kThreads, 0, stream>>>(logits, bias, T, E, K, biw, ids, w);
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
  // 16-lane segments where they measured faster: E <= 128 (131072 tokens:
  // 21.3 vs 44.0 us at E = 64, 39.5 vs 61.0 us at E = 128; equal at 8192-16384
  // tokens).  At E = 256 the wave per token wins at every size (8192 tokens:
  // 8.2 vs 13.9 us; 131072: 80 vs 196 us).
  if (K <= 16 && E <= 128) {
    if (E <= 64) launch_seg<4>(logits, bias, T, E, K, biw, topk_ids, topk_weights, stream);
    else launch_seg<8>(logits, bias, T, E, K, biw, topk_ids, topk_weights, stream);
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
