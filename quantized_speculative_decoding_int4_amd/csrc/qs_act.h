// Device helpers for activations: per-token INT4 quantization (W4A4) and the row
// standardisation between the linears of a chain.  Shared by the per-linear kernels
// (linear.hip), the batched kernel (gemm.hip) and the persistent pass kernel (pass.hip).
//
// Two arithmetics of the standardisation, one per kind of mode:
//  * W4A16 folds it into the epilogue, y = (sum_k v w - mu sum_k w) / sd, with the row statistics
//    in fp32 (its products are fp32 anyway);
//  * the integer modes quantize the standardised fp16 row, so its rounding decides codes: the
//    statistics, the standardised value and its rounding to fp16 are computed in fp64 and rounded
//    once, correctly, to fp16 -- the float64 definition's own result, whatever the summation order
//    (a different order moves the fp64 value by ~1e-16, which changes an fp16 rounding only for a
//    value within that distance of a midpoint).
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
// ---- exact (fp64) standardisation of the integer modes

// Correctly rounded fp64 -> fp16 (round to nearest even).  Converting through fp32 with two
// round-to-nearest steps is wrong whenever the fp32 value lands exactly on an fp16 midpoint; rounding
// the first step to odd instead (truncate, then set the last bit if anything was dropped) makes the
// second step exact, since fp32 keeps at least two more bits than fp16 (24 >= 11 + 2), normal or not.
__device__ __forceinline__ uint16_t f64_to_f16_rn(double d) {
  const float f = (float)d;  // round to nearest even
  uint32_t b = __float_as_uint(f);
  const double back = (double)f;
  if (back != d) {                           // inexact (or NaN, which stays NaN)
    if (__builtin_fabs(back) > __builtin_fabs(d)) b -= 1u;  // was rounded away from zero: one step back
    b |= 1u;                                 // sticky bit: round to odd
  }
  return f2h(__uint_as_float(b));
}

// Per-thread fp64 sum and sum of squares (exact products) and fp32 max / min of 8 fp16 values.
__device__ __forceinline__ void stats_block8_64(const uint4 v, double& sum, double& sq, float& mx, float& mn) {
  const uint16_t* h = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float f = h2f(h[e]);
    const double d = (double)f;
    sum += d;
    sq += d * d;
    mx = fmaxf(mx, f);
    mn = fminf(mn, f);
  }
}
// Row mean and 1/std (population) in fp64.  A row with zero spread (max == min, the exact test)
// maps to zeros: inv = 0.
__device__ __forceinline__ void norm_params64(double sum, double sq, float mx, float mn, int K, double& mu,
                                              double& inv) {
  mu = sum / (double)K;
  double var = sq / (double)K - mu * mu;
  var = var > 0.0 ? var : 0.0;
  inv = (mx != mn && var > 0.0) ? 1.0 / __builtin_sqrt(var) : 0.0;
}
__device__ __forceinline__ uint16_t norm_h64(float x, double mu, double inv) {
  return inv == 0.0 ? (uint16_t)0 : f64_to_f16_rn(((double)x - mu) * inv);
}
__device__ __forceinline__ uint4 norm_block8_64(uint4 v, double mu, double inv) {
  uint16_t* h = reinterpret_cast<uint16_t*>(&v);
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = norm_h64(h2f(h[e]), mu, inv);
  return v;
}

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace qs
