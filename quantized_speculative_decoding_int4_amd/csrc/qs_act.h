// Device helpers for activations: per-token INT4 quantization (W4A4) and the row
// standardisation between the linears of a chain.  Shared by the per-linear kernels
// (linear.hip) and the persistent pass kernel (pass.hip).
#pragma once

#include "qs_device.h"

namespace qs {

// Quantize one 8-element block (16 bytes of fp16) with scale s to clamp(rint(x / s), -QMAX - 1,
// QMAX) (QMAX = 7: INT4 codes; 127: INT8 codes); returns the 8 codes in operand byte order (low
// dword, high dword) and in logical order.
template <int QMAX = 7>
__device__ __forceinline__ void quant_block8(const uint4 v, float s, uint2& op, uint2& logical) {
  const uint16_t* h = reinterpret_cast<const uint16_t*>(&v);
  uint32_t lo_op = 0, hi_op = 0, lo_lg = 0, hi_lg = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    int qv = 0;
    if (s != 0.0f) {
      float r = __builtin_rintf(h2f(h[e]) / s);
      r = fminf((float)QMAX, fmaxf(-(float)QMAX - 1.0f, r));
      qv = (int)r;
    }
    const uint32_t b = (uint32_t)(qv & 0xFF);
    const int p = ((e & 3) << 1) | ((e >> 2) & 1);
    if (p < 4) lo_op |= b << (8 * p); else hi_op |= b << (8 * (p - 4));
    if (e < 4) lo_lg |= b << (8 * e); else hi_lg |= b << (8 * (e - 4));
  }
  op = make_uint2(lo_op, hi_op);
  logical = make_uint2(lo_lg, hi_lg);
}

// ---- input standardisation between the linears of a chain
// x -> fp16((x - mean) / std) per row over the K columns read (population std from fp32 sums);
// a row with zero spread maps to zeros.
__device__ __forceinline__ void norm_params(float sum, float sq, int K, float& mu, float& inv) {
  mu = sum / (float)K;
  float var = sq / (float)K - mu * mu;
  var = var > 0.0f ? var : 0.0f;
  const float sd = sqrtf(var);
  inv = sd > 0.0f ? 1.0f / sd : 0.0f;
}
__device__ __forceinline__ uint16_t norm_h(float x, float mu, float inv) {
  return inv == 0.0f ? (uint16_t)0 : f2h((x - mu) * inv);
}
// Standardise 8 fp16 values.
__device__ __forceinline__ uint4 norm_block8(uint4 v, float mu, float inv) {
  uint16_t* h = reinterpret_cast<uint16_t*>(&v);
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = norm_h(h2f(h[e]), mu, inv);
  return v;
}
// Per-thread statistics of 8 fp16 values: sum, sum of squares, max, min.
__device__ __forceinline__ void stats_block8(const uint4 v, float& sum, float& sq, float& mx, float& mn) {
  const uint16_t* h = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float f = h2f(h[e]);
    sum += f;
    sq += f * f;
    mx = fmaxf(mx, f);
    mn = fminf(mn, f);
  }
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace qs
