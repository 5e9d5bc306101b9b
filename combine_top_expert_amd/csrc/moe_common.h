// Shared device helpers for the gfx950 MoE kernels: number formats,
// wavefront primitives, argument checks.  Wave64 throughout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_ep.h"

#define MOE_WAVE 64

#define MOE_CHECK(cond, code)                                                    \
  do {                                                                           \
    if (!(cond)) return (code);                                                  \
  } while (0)

#define MOE_LAUNCH_CHECK()                                                       \
  do {                                                                           \
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;                     \
  } while (0)

namespace moe {

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// ------------------------------------------------------------------ e4m3fn
// Two fp32 values -> two OCP e4m3fn codes packed in the low 16 bits.  The
// hardware conversion rounds to nearest even; magnitudes are clamped to the
// format's largest finite value 448 first so no input can become NaN.
__device__ __forceinline__ uint32_t f32x2_to_e4m3(float a, float b) {
  a = fminf(fmaxf(a, -448.0f), 448.0f);
  b = fminf(fmaxf(b, -448.0f), 448.0f);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xffffu;
}

// Four fp32 values -> four e4m3fn codes in one dword (value i in byte i).
__device__ __forceinline__ uint32_t f32x4_to_e4m3(float a, float b, float c, float d) {
  return f32x2_to_e4m3(a, b) | (f32x2_to_e4m3(c, d) << 16);
}

// The per-group FP8 activation recipe: amax over the group (clamped at
// 1e-4), factor 448/amax and scale amax/448, each a correctly rounded fp32
// operation (HIP's fp32 '/' is IEEE-correct unless fast-math is requested).
__device__ __forceinline__ float fp8_group_amax_clamp(float amax) { return fmaxf(amax, 1e-4f); }
__device__ __forceinline__ float fp8_group_inv(float amax) { return 448.0f / amax; }
__device__ __forceinline__ float fp8_group_scale(float amax) { return amax / 448.0f; }

// ------------------------------------------------------------------ wave helpers
__device__ __forceinline__ int lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// number of set bits of `m` in lanes below this one
__device__ __forceinline__ int mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0));
}

// max over aligned groups of 16 lanes (xor butterfly inside each group)
__device__ __forceinline__ float group16_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 1));
  v = fmaxf(v, __shfl_xor(v, 2));
  v = fmaxf(v, __shfl_xor(v, 4));
  v = fmaxf(v, __shfl_xor(v, 8));
  return v;
}

// SiLU(v) = v / (1 + e^-v) with the hardware exp2 (v_exp_f32) and
// reciprocal (v_rcp_f32): a few ulp of fp32, far below the FP8 step of the
// Z quantisation that follows, at a tenth of the instructions of the
// correctly rounded expf and divide.  Saturates cleanly: e^-v overflowing
// to inf gives 0 (large negative v), underflowing to 0 gives v.
__device__ __forceinline__ float silu(float v) {
  const float e = __builtin_amdgcn_exp2f(v * -1.44269504088896341f);   // e^-v = 2^(-v log2 e)
  return v * __builtin_amdgcn_rcpf(1.0f + e);
}

// Gradient of z = SiLU(g) * u for one element, given dz:
//   d_up = dz * SiLU(g),  d_gate = dz * u * s * (1 + g * (1 - s)),  s = sigmoid(g),
// s from the same hardware exp2 and reciprocal as silu().  Contraction is off
// so that every kernel that calls it (the SiLU*up backward and the gate/up
// GEMM's backward epilogue) gets the same bits from the same g, u, dz.
__device__ __forceinline__ void silu_mul_grad(float g, float u, float dz, float& dgate, float& dup) {
#pragma clang fp contract(off)
  const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.44269504088896341f));
  dup = dz * (g * s);
  dgate = dz * u * s * (1.0f + g * (1.0f - s));
}

// 16-byte loads/stores that bypass cache retention (streamed once)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_nt16(void* p, const uint4& v) {
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}

}  // namespace moe

// ------------------------------------------------------------------ host helpers
namespace moe_host {

inline bool valid_dtype(int d) { return d == MOE_F32 || d == MOE_BF16 || d == MOE_FP8_E4M3; }

inline int elem_bytes(moe_dtype d) { return d == MOE_F32 ? 4 : (d == MOE_BF16 ? 2 : 1); }

// Compute units of the current device (cached per device id).
__attribute__((visibility("hidden"))) int device_cu_count();

}  // namespace moe_host
