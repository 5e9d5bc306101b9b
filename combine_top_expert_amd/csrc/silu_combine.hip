// moe_silu_mul and moe_combine.
//
// silu_mul: Z = SiLU(gate) * up on the valid rows of an expert-major fp32
// G buffer ("SGLang Expert Compute Backend" §3.6: non-interleaved gate/up,
// activation applied to valid expert rows only, Z re-quantised with its own
// per-128 scales before the down GEMM).  One wavefront per row; a
// 128-column Z group spans 32 lanes x 4 values.
//
// combine: y[t] = sum_k w[t,k] * out[slot_of[t,k]] ("SGLang、NCCL 与 MoE EP"
// §1.1 and §2.3.6; "DeepEP 架构与实现笔记" §9.4 combine_convert).  One
// wavefront per token.  The token's routes are read once (lane k = route k)
// and its local routes walked in k order; for each, every lane has 8
// 8-column chunks of the source row in flight at once (a whole 4096-column
// bf16 row per wave per round trip).  Products and sums are separate fp32
// operations in k order (no fused multiply-add), so the result equals a
// plain fp32 evaluation of the sum term by term.

#include "moe_common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / MOE_WAVE;

// expert of row q, or -1 if q is a padding row
__device__ __forceinline__ bool valid_row(const int32_t* counts, const int32_t* offsets, int L,
                                          int64_t q) {
  int lo = 0, hi = L;          // largest e with offsets[e] <= q
  if (q < offsets[0]) return false;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= q) lo = mid; else hi = mid;
  }
  return q < static_cast<int64_t>(offsets[lo]) + counts[lo];
}

constexpr int kSiluBatch = 6;
template <int ZDT>  // 0 f32, 1 bf16, 2 fp8
__global__ __launch_bounds__(kThreads) void silu_mul_kernel(const float* __restrict__ g,
                                                            const int32_t* __restrict__ counts,
                                                            const int32_t* __restrict__ offsets,
                                                            int L, int64_t rows_cap, int I,
                                                            uint8_t* __restrict__ z,
                                                            float* __restrict__ zs) {
  const int lane = moe::lane_id();
  const int64_t q = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
  if (q >= rows_cap || !valid_row(counts, offsets, L, q)) return;
  const float4* grow = reinterpret_cast<const float4*>(g + q * 2 * I);
  const int nchunk = I / 4;                       // 4 columns per lane-step
  // steps in batches of kSiluBatch: a batch's loads are issued before any is used
  for (int cb = 0; cb < nchunk; cb += MOE_WAVE * kSiluBatch) {
    float4 gtb[kSiluBatch], upb[kSiluBatch];
#pragma unroll
    for (int b = 0; b < kSiluBatch; ++b) {
      const int c = cb + MOE_WAVE * b + lane;
      gtb[b] = upb[b] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c < nchunk) {
        gtb[b] = grow[c];
        upb[b] = grow[nchunk + c];
      }
    }
#pragma unroll
    for (int b = 0; b < kSiluBatch; ++b) {
      const int c0 = cb + MOE_WAVE * b;
      if (c0 >= nchunk) break;                      // wave-uniform
      const int c = c0 + lane;
      const bool live = c < nchunk;                 // nchunk % 32 == 0: groups stay whole
      const float4 gt = gtb[b], up = upb[b];
      const float v[4] = {moe::silu(gt.x) * up.x, moe::silu(gt.y) * up.y, moe::silu(gt.z) * up.z,
                          moe::silu(gt.w) * up.w};
      if constexpr (ZDT == 2) {
        float m = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
        m = moe::group16_max(m);
        m = fmaxf(m, __shfl_xor(m, 16));
        const float amax = moe::fp8_group_amax_clamp(m);
        const float inv = moe::fp8_group_inv(amax);
        if (live) {
          reinterpret_cast<uint32_t*>(z + q * I)[c] =
              moe::f32x4_to_e4m3(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
          if ((lane & 31) == 0) zs[q * (I / 128) + c / 32] = moe::fp8_group_scale(amax);
        }
      } else if constexpr (ZDT == 1) {
        if (live) {
          const uint32_t lo = moe::f32_to_bf16(v[0]) | (uint32_t(moe::f32_to_bf16(v[1])) << 16);
          const uint32_t hi = moe::f32_to_bf16(v[2]) | (uint32_t(moe::f32_to_bf16(v[3])) << 16);
          reinterpret_cast<uint2*>(z + q * I * 2)[c] = make_uint2(lo, hi);
        }
      } else {
        if (live) reinterpret_cast<float4*>(z + q * I * 4)[c] = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
  }
}

constexpr int kMaxK = 64;
constexpr int kCPL = 4;                         // 8-column chunks per lane in one part
constexpr int kPartChunks = kCPL * MOE_WAVE;    // 2048 columns per part

template <bool kInBf16, bool kOutBf16>
__global__ __launch_bounds__(kThreads) void combine_kernel(const uint8_t* __restrict__ eo,
                                                           const int32_t* __restrict__ slot_of,
                                                           const float* __restrict__ w, int T,
                                                           int K, int H, int64_t rows_cap,
                                                           uint8_t* __restrict__ y, int parts) {
  const int lane = moe::lane_id();
  const int item = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);   // (token, part)
  const int t = item / parts;
  const int p = item - t * parts;
  if (t >= T) return;
  constexpr int IB = kInBf16 ? 2 : 4;
  constexpr int OB = kOutBf16 ? 2 : 4;
  constexpr int NV = IB == 2 ? 1 : 2;            // 16-byte loads per 8-column chunk
  // lane k holds route k of the token; the routes with a local row form a
  // bit mask in k order (ballot bit k = lane k)
  const int s_l = lane < K ? slot_of[static_cast<int64_t>(t) * K + lane] : -1;
  // null weights: every route weighs 1 (permute backward); 1 * v is exact
  const float w_l = lane < K ? (w != nullptr ? w[static_cast<int64_t>(t) * K + lane] : 1.f) : 0.f;
  uint64_t m = __ballot(s_l >= 0 && s_l < rows_cap);
  const int nchunk = H / 8;
  const int c0 = p * kPartChunks + lane;         // chunk u of this lane: c0 + 64u

  float acc[kCPL][8];
#pragma unroll
  for (int u = 0; u < kCPL; ++u)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[u][i] = 0.f;
  auto load = [&](int s, uint4 (*r)[NV]) {
    const uint4* row = reinterpret_cast<const uint4*>(eo + static_cast<int64_t>(s) * H * IB);
#pragma unroll
    for (int u = 0; u < kCPL; ++u) {
      const int c = c0 + u * MOE_WAVE;
#pragma unroll
      for (int v = 0; v < NV; ++v)
        r[u][v] = c < nchunk ? moe::load_nt16(row + static_cast<int64_t>(c) * NV + v) : make_uint4(0, 0, 0, 0);
    }
  };
  auto accumulate = [&](const uint4 (*r)[NV], float wk) {
#pragma unroll
    for (int u = 0; u < kCPL; ++u) {
      float v[8];
      if constexpr (kInBf16) {
        const uint32_t ww[4] = {r[u][0].x, r[u][0].y, r[u][0].z, r[u][0].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = __uint_as_float(ww[i] << 16);
          v[2 * i + 1] = __uint_as_float(ww[i] & 0xffff0000u);
        }
      } else {
        const uint32_t ww[8] = {r[u][0].x, r[u][0].y, r[u][0].z, r[u][0].w,
                                r[u][NV - 1].x, r[u][NV - 1].y, r[u][NV - 1].z, r[u][NV - 1].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(ww[i]);
      }
      {
        // product and sum rounded separately, in k order (no FMA contraction)
#pragma clang fp contract(off)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[u][i] = acc[u][i] + wk * v[i];
      }
    }
  };
  auto route = [&](int k, int& s, float& wk) {
    s = __builtin_amdgcn_readlane(s_l, k);
    wk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w_l), k));
  };
  // walk the local routes in increasing k; the next route's loads are issued
  // before this route's sums
  if (m) {
    uint4 cur[kCPL][NV], nxt[kCPL][NV];
    int s;
    float wk;
    route(__builtin_ctzll(m), s, wk);
    load(s, cur);
    for (;;) {
      m &= m - 1;
      const bool more = m != 0;
      int s2 = 0;
      float wk2 = 0.f;
      if (more) {
        route(__builtin_ctzll(m), s2, wk2);
        load(s2, nxt);
      }
      accumulate(cur, wk);
      if (!more) break;
      for (int u = 0; u < kCPL; ++u)
        for (int v = 0; v < NV; ++v) cur[u][v] = nxt[u][v];
      wk = wk2;
    }
  }
  uint8_t* yrow = y + static_cast<int64_t>(t) * H * OB;
#pragma unroll
  for (int u = 0; u < kCPL; ++u) {
    const int c = c0 + u * MOE_WAVE;
    if (c >= nchunk) continue;
    uint8_t* dst = yrow + static_cast<int64_t>(c) * 8 * OB;
    if constexpr (kOutBf16) {
      uint4 o;
      o.x = moe::f32_to_bf16(acc[u][0]) | (uint32_t(moe::f32_to_bf16(acc[u][1])) << 16);
      o.y = moe::f32_to_bf16(acc[u][2]) | (uint32_t(moe::f32_to_bf16(acc[u][3])) << 16);
      o.z = moe::f32_to_bf16(acc[u][4]) | (uint32_t(moe::f32_to_bf16(acc[u][5])) << 16);
      o.w = moe::f32_to_bf16(acc[u][6]) | (uint32_t(moe::f32_to_bf16(acc[u][7])) << 16);
      moe::store_nt16(dst, o);
    } else {
      reinterpret_cast<float4*>(dst)[0] = make_float4(acc[u][0], acc[u][1], acc[u][2], acc[u][3]);
      reinterpret_cast<float4*>(dst)[1] = make_float4(acc[u][4], acc[u][5], acc[u][6], acc[u][7]);
    }
  }
}

}  // namespace

extern "C" moe_status moe_silu_mul(const float* g, const int32_t* counts, const int32_t* offsets,
                                   int L, int64_t rows_cap, int I, void* z, moe_dtype z_dt,
                                   float* z_scales, hipStream_t stream) {
  MOE_CHECK(L >= 1 && rows_cap >= 0 && I > 0, MOE_ERR_INVALID_ARG);
  MOE_CHECK(moe_host::valid_dtype(z_dt), MOE_ERR_INVALID_ARG);
  MOE_CHECK(I % 128 == 0, MOE_ERR_UNSUPPORTED);
  if (rows_cap == 0) return MOE_OK;
  MOE_CHECK(g && counts && offsets && z, MOE_ERR_INVALID_ARG);
  MOE_CHECK(z_dt != MOE_FP8_E4M3 || z_scales, MOE_ERR_INVALID_ARG);
  const int64_t grid = (rows_cap + kRowsPerBlock - 1) / kRowsPerBlock;
  MOE_CHECK(grid <= 0x7fffffff, MOE_ERR_UNSUPPORTED);
  auto* zo = static_cast<uint8_t*>(z);
  if (z_dt == MOE_F32)
    silu_mul_kernel<0><<<grid, kThreads, 0, stream>>>(g, counts, offsets, L, rows_cap, I, zo, nullptr);
  else if (z_dt == MOE_BF16)
    silu_mul_kernel<1><<<grid, kThreads, 0, stream>>>(g, counts, offsets, L, rows_cap, I, zo, nullptr);
  else
    silu_mul_kernel<2><<<grid, kThreads, 0, stream>>>(g, counts, offsets, L, rows_cap, I, zo, z_scales);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

namespace {

moe_status combine_launch(const void* expert_out, moe_dtype eo_dt, const int32_t* slot_of,
                          const float* topk_weights, int T, int K, int H, int64_t rows_cap, void* y,
                          moe_dtype y_dt, hipStream_t stream) {
  MOE_CHECK(T >= 0 && K > 0 && H > 0 && rows_cap >= 0, MOE_ERR_INVALID_ARG);
  MOE_CHECK(moe_host::valid_dtype(eo_dt) && moe_host::valid_dtype(y_dt), MOE_ERR_INVALID_ARG);
  MOE_CHECK(eo_dt != MOE_FP8_E4M3 && y_dt != MOE_FP8_E4M3, MOE_ERR_UNSUPPORTED);
  MOE_CHECK(H % 8 == 0 && K <= kMaxK, MOE_ERR_UNSUPPORTED);
  if (T == 0) return MOE_OK;
  MOE_CHECK(slot_of && y && (rows_cap == 0 || expert_out), MOE_ERR_INVALID_ARG);
  const int parts = (H / 8 + kPartChunks - 1) / kPartChunks;
  const int64_t grid64 = (static_cast<int64_t>(T) * parts + kRowsPerBlock - 1) / kRowsPerBlock;
  MOE_CHECK(grid64 <= 0x7fffffff, MOE_ERR_UNSUPPORTED);
  const int grid = static_cast<int>(grid64);
  auto* eo = static_cast<const uint8_t*>(expert_out);
  auto* yo = static_cast<uint8_t*>(y);
  const bool ib = eo_dt == MOE_BF16, ob = y_dt == MOE_BF16;
  if (ib && ob)
    combine_kernel<true, true><<<grid, kThreads, 0, stream>>>(eo, slot_of, topk_weights, T, K, H, rows_cap, yo, parts);
  else if (ib)
    combine_kernel<true, false><<<grid, kThreads, 0, stream>>>(eo, slot_of, topk_weights, T, K, H, rows_cap, yo, parts);
  else if (ob)
    combine_kernel<false, true><<<grid, kThreads, 0, stream>>>(eo, slot_of, topk_weights, T, K, H, rows_cap, yo, parts);
  else
    combine_kernel<false, false><<<grid, kThreads, 0, stream>>>(eo, slot_of, topk_weights, T, K, H, rows_cap, yo, parts);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_combine(const void* expert_out, moe_dtype eo_dt, const int32_t* slot_of,
                                  const float* topk_weights, int T, int K, int H, int64_t rows_cap,
                                  void* y, moe_dtype y_dt, hipStream_t stream) {
  MOE_CHECK(T == 0 || topk_weights, MOE_ERR_INVALID_ARG);
  return combine_launch(expert_out, eo_dt, slot_of, topk_weights, T, K, H, rows_cap, y, y_dt, stream);
}

extern "C" moe_status moe_permute_backward(const void* d_buf, moe_dtype d_buf_dt, const int32_t* slot_of,
                                           int T, int K, int H, int64_t rows_cap, void* dx, moe_dtype dx_dt,
                                           hipStream_t stream) {
  return combine_launch(d_buf, d_buf_dt, slot_of, nullptr, T, K, H, rows_cap, dx, dx_dt, stream);
}
