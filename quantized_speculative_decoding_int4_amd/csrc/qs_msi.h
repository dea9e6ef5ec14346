// Cross-lane helpers and the softmax-statistics triple shared by the verify kernels and the
// LM-head epilogue of the batched linear: per set of logits, (max, sum of exp(l - max), lowest
// index attaining the max), merged associatively in a fixed order, so every result is
// deterministic and ties resolve to the lowest index.
#pragma once

#include <hip/hip_runtime.h>

#include "qs_device.h"

namespace qs {

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
