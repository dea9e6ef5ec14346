// Cross-lane helpers and the softmax-statistics triple shared by the verify kernels and the
// LM-head epilogue of the batched linear: per set of logits, (max, sum of exp(l - max), lowest
// index attaining the max), merged associatively in a fixed order, so every result is
// deterministic and ties resolve to the lowest index.
#pragma once

#include <hip/hip_runtime.h>

#include "qs_device.h"

namespace qs {

// Lane moves of 32- and 64-bit values (a double moves as its two halves).
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) { return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false); }
template <int CTRL>
__device__ __forceinline__ float dpp_v(float x) { return __int_as_float(dpp_i<CTRL>(__float_as_int(x))); }
template <int CTRL>
__device__ __forceinline__ double dpp_v(double x) {
  const long long b = __double_as_longlong(x);
  const unsigned lo = (unsigned)dpp_i<CTRL>((int)(unsigned)b), hi = (unsigned)dpp_i<CTRL>((int)(b >> 32));
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
__device__ __forceinline__ float readlane_v(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ __forceinline__ double readlane_v(double x, int l) {
  const long long b = __double_as_longlong(x);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)b, l);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(b >> 32), l);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
// (max, sum of exp(l - max), lowest index attaining max) of a set of logits, and its merge.
struct Msi {
  float m, s;
  int i;
};
// By value, field by field: a select between two structs in memory would keep them in scratch.
__device__ __forceinline__ Msi msi_merge(const Msi a, const Msi b) {
  const float am = a.m, bm = b.m, as = a.s, bs = b.s;
  const int ai = a.i, bi = b.i;
  const bool tb = bm > am || (bm == am && bi < ai);
  const float m = tb ? bm : am;
  const int i = tb ? bi : ai;
  // The winner's scale factor is 1: one exponential per merge.  Empty sets (m = -inf) add nothing.
  const float lo = tb ? am : bm;
  const float e = lo == -INFINITY ? 0.0f : __expf(lo - m);
  const float sum = m == -INFINITY ? 0.0f : (tb ? as * e + bs : as + bs * e);
  return Msi{m, sum, i};
}
template <int CTRL>
__device__ __forceinline__ Msi msi_dpp(const Msi x) {
  return Msi{dpp_v<CTRL>(x.m), dpp_v<CTRL>(x.s), dpp_i<CTRL>(x.i)};
}
__device__ __forceinline__ Msi msi_readlane(const Msi x, int l) {
  return Msi{readlane_v(x.m, l), readlane_v(x.s, l), __builtin_amdgcn_readlane(x.i, l)};
}
// Merge over the 64 lanes (all active): pairs, quads, halves of 8 and rows of 16 by DPP (the
// merge is symmetric, so both partners hold the same result), then rows 0-3 from lanes 0, 16,
// 32, 48.  Result in every lane.
__device__ __forceinline__ Msi wave_msi(Msi x) {
  x = msi_merge(x, msi_dpp<0xB1>(x));   // quad_perm [1,0,3,2]
  x = msi_merge(x, msi_dpp<0x4E>(x));   // quad_perm [2,3,0,1]
  x = msi_merge(x, msi_dpp<0x141>(x));  // row_half_mirror
  x = msi_merge(x, msi_dpp<0x140>(x));  // row_mirror
  return msi_merge(msi_merge(msi_readlane(x, 0), msi_readlane(x, 16)),
                   msi_merge(msi_readlane(x, 32), msi_readlane(x, 48)));
}
}  // namespace qs
