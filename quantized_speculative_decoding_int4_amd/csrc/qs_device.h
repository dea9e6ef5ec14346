// Device-side helpers shared by the gfx950 kernels of libqspec: MFMA operand
// types, the INT4 nibble expansion for both modes, and wave reductions.
//
// Packed weight layout (one buffer serves both modes):
//   The [N, K] code matrix is cut into tiles of 16 rows x 128 k (one scale
//   group).  Tile (rb, g), rb = n / 16, g = k / 128, is 1024 contiguous bytes at
//   byte offset (rb * G + g) * 1024, G = K / 128, so a 16-row block streams its
//   whole K range contiguously.  Inside a tile, wave lane l (0..63) owns the 16
//   bytes at l * 16: row n = 16 rb + (l & 15), k in [128 g + 32 (l >> 4), +32),
//   i.e. exactly the B-operand fragment that lane feeds a 16x16 MFMA.  The four
//   dwords of a lane hold k offsets 0-7, 8-15, 16-23, 24-31; inside a dword the
//   code of k offset e sits in nibble pos(e) = (e & 1) * 4 + (e >> 1), stored
//   offset-binary (u = q + 8).  This order lets two AND-OR operations per half
//   dword produce fp16 pairs already in k order (see unpack_f16x8).
//   Scales: s_packed[(rb * G + g) * 16 + (n & 15)].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qs {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef double double4_t __attribute__((ext_vector_type(4)));
typedef int int4_t __attribute__((ext_vector_type(4)));

constexpr int kGroup = 128;
constexpr int kTileBytes = 1024;

__device__ __forceinline__ float h2f(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}
__device__ __forceinline__ uint16_t f2h(float f) {  // round to nearest even
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// 8 offset-binary nibbles (one packed dword, layout above) -> 8 fp16 codes q in
// k order.  (0x6400 | v) is the fp16 value 1024 + v for v < 1024, so
//   low nibble  : (1024 + u)        - 1032       = q
//   high nibble : (1024 + 16 u) / 16 - 72        = q
// Both are exact in fp16.  `magic` must be 0x64006400 (see fp16_magic_vgpr).
__device__ __forceinline__ half8_t unpack_f16x8(uint32_t w, uint32_t magic) {
  const uint32_t w8 = w >> 8;
  const uint32_t a = (w & 0x000F000Fu) | magic;   // k0, k1
  const uint32_t b = (w & 0x00F000F0u) | magic;   // k2, k3
  const uint32_t c = (w8 & 0x000F000Fu) | magic;  // k4, k5
  const uint32_t d = (w8 & 0x00F000F0u) | magic;  // k6, k7
  const half2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
  const half2_t sc = {(_Float16)0.0625f, (_Float16)0.0625f};
  const half2_t off2 = {(_Float16)72.0f, (_Float16)72.0f};
  const half2_t ha = __builtin_bit_cast(half2_t, a) - off;
  const half2_t hb = __builtin_bit_cast(half2_t, b) * sc - off2;
  const half2_t hc = __builtin_bit_cast(half2_t, c) - off;
  const half2_t hd = __builtin_bit_cast(half2_t, d) * sc - off2;
  uint4 u;
  u.x = __builtin_bit_cast(uint32_t, ha);
  u.y = __builtin_bit_cast(uint32_t, hb);
  u.z = __builtin_bit_cast(uint32_t, hc);
  u.w = __builtin_bit_cast(uint32_t, hd);
  return __builtin_bit_cast(half8_t, u);
}

// 0x64006400 held in a VGPR: lets (w & mask) | magic fuse into one v_and_or_b32 (VOP3 on this
// target cannot encode two literal operands).
__device__ __forceinline__ uint32_t fp16_magic_vgpr() {
  uint32_t v;
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(v));
  return v;
}

// Two packed dwords (k offsets 0-15 of a lane's slice) -> 16 int8 operands
// holding 16 * q (two's-complement nibble in the high half of each byte).
// Byte order of the result, as k offsets: 0,4,1,5, 2,6,3,7, 8,12,9,13, 10,14,11,15.
// The activation operand is stored in the same order (qs_xq_pos).
__device__ __forceinline__ int4_t unpack_i8x16(uint32_t w0, uint32_t w1) {
  const uint32_t t0 = w0 ^ 0x88888888u;  // offset-binary -> two's complement nibbles
  const uint32_t t1 = w1 ^ 0x88888888u;
  int4_t r;
  r[0] = (int)((t0 << 4) & 0xF0F0F0F0u);
  r[1] = (int)(t0 & 0xF0F0F0F0u);
  r[2] = (int)((t1 << 4) & 0xF0F0F0F0u);
  r[3] = (int)(t1 & 0xF0F0F0F0u);
  return r;
}

// Byte position, inside a 16-byte activation operand chunk, of k offset j (0..15).
__host__ __device__ __forceinline__ int xq_pos(int j) {
  return (j & 8) | ((j & 3) << 1) | ((j >> 2) & 1);
}

// ---- lane moves of 32- and 64-bit values (a double moves as its two halves) -------
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

// ---- wave (64-lane) reductions -------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// Data-parallel-primitive (DPP) reductions: four in-row steps (pairs, quads, halves of 8, rows of
// 16) leave every lane with its 16-lane row's result; the four rows are then combined from lanes
// 0, 16, 32 and 48.  Fixed order, all 64 lanes active, result in every lane.
template <typename Op>
__device__ __forceinline__ float wave_reduce_dpp(float v, Op op) {
  auto dpp = [](float x, int ctrl) {
    switch (ctrl) {  // the control word must be a constant
      case 0: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
      case 1: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
      case 2: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
      default: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
    }
  };
  v = op(v, dpp(v, 0));  // quad_perm [1,0,3,2]
  v = op(v, dpp(v, 1));  // quad_perm [2,3,0,1]
  v = op(v, dpp(v, 2));  // row_half_mirror
  v = op(v, dpp(v, 3));  // row_mirror
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return op(op(r0, r1), op(r2, r3));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  return wave_reduce_dpp(v, [](float a, float b) { return a + b; });
}
__device__ __forceinline__ float wave_max_dpp(float v) {
  return wave_reduce_dpp(v, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float wave_min_dpp(float v) {
  return wave_reduce_dpp(v, [](float a, float b) { return fminf(a, b); });
}
// fp64 sum over the 64 lanes, same fixed order as wave_reduce_dpp; result in every lane.
__device__ __forceinline__ double wave_sum_dpp64(double v) {
  v += dpp_v<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_v<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_v<0x141>(v);  // row_half_mirror
  v += dpp_v<0x140>(v);  // row_mirror
  return (readlane_v(v, 0) + readlane_v(v, 16)) + (readlane_v(v, 32) + readlane_v(v, 48));
}
// fp64 sum over lanes 0..7 (first three in-row steps), returned from lane 0.
__device__ __forceinline__ double lanes8_sum_dpp64(double v) {
  v += dpp_v<0xB1>(v);
  v += dpp_v<0x4E>(v);
  v += dpp_v<0x141>(v);
  return readlane_v(v, 0);
}
// Result of op over lanes 0..7 (after the first three in-row steps), returned from lane 0.
template <typename Op>
__device__ __forceinline__ float lanes8_reduce_dpp(float v, Op op) {
  v = op(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
  v = op(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
  v = op(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
}

// (value, index) max with the lowest index winning ties.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(v, o, 64);
    const int oi = __shfl_xor(i, o, 64);
    if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
  }
}

}  // namespace qs
