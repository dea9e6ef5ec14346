// Batched linear: the verify pass over many sequences, where the target scores B * (gamma + 1)
// positions at once ([P3] "draft modelとtarget modelの処理フロー"; modes from [P1] "QSpec の W4A4
// モードと W4A16 モード"), and every per-linear call from 5 rows (W4A16) or 2 rows (W4A4, W4A8) on.
// W4A16 expands the INT4 codes to fp16 in registers, runs v_mfma_f32_16x16x32_f16 over each
// 128-wide group and scales the group's fp32 sum by its scale in fp32 (the products are exact, as
// in the definition); the integer modes run v_mfma_i32_16x16x64_i8 on the quantized activations
// and scale each group's exact i32 sum in fp64, where every term, every sum of terms and the
// product with the row scale are exact while log2(K / 128) + the binades spanned by an output row's
// scales <= 13, so the output is the exact value rounded once.
//
// Work split.  A workgroup of 4 waves owns an output tile of MT * 16 rows (MT = 1, 2 or 4 MFMA
// row tiles) x 256 columns (16 packed row blocks, 4 per wave) over a range of K, one 128-wide group
// at a time:
//   * the group's activation rows are staged once in LDS (double-buffered, rows padded by 16 bytes
//     so the fragment reads of 16 rows hit distinct banks) and read by all 4 waves;
//   * each wave keeps D groups of its 4 weight tiles in flight in a register ring, expands each
//     fragment once and feeds it to MT MFMAs, while each activation fragment feeds 4 MFMAs;
//   * linears with few output tiles split K over workgroups; the last workgroup of a tile to finish
//     sums the splits' partials in split order (device-coherent slots, self-resetting counters);
//   * the workgroup order is remapped so that the row tiles of one column block run on one XCD
//     and share its L2;
//   * optional epilogues: the row standardisation of a chain's input (W4A16, applied after the
//     contraction) and the LM-head's Top-1 (per-tile softmax statistics merged by the last tile).

#include "qs_act.h"
#include "qs_msi.h"
#include "qs_device.h"
#include "qs_internal.h"

#include <type_traits>

namespace qs {

constexpr int kGemmWaves = 4;
constexpr int kGemmMaxMt = 2;                   // 16-row MFMA tiles per workgroup: 1 or 2
constexpr int kGemmMaxRows = kGemmMaxMt * 16;
constexpr int kGemmNt = 4;                      // 16-column row blocks per wave
constexpr int kGemmBlocks = kGemmWaves * kGemmNt;  // row blocks per workgroup (256 columns)
constexpr int kGemmMaxSplits = 16;
constexpr int kGemmMinGroupsPerSplit = 4;
constexpr int kGemmMaxCounters = 1024;           // split runs have fewer than 256 output tiles

// Partial slot of one (K split, output tile) workgroup, device-coherent, read back only by the
// tile's last-arriving workgroup: the accumulators in register order ([wave][mt][nt][lane] float4 or,
// for the integer modes, double4), then the column sums of the expanded weights ([wave][nt][16
// columns]) and the row sums (sum, sum of squares) of the staged activations ([rows] float2).
// Sized for the largest row tile.
constexpr int kSlotAcc = kGemmWaves * kGemmMaxMt * kGemmNt * 64 * 32;
constexpr int kSlotCs = kSlotAcc;
constexpr int kSlotStats = kSlotCs + kGemmWaves * kGemmNt * 16 * 4;
constexpr int kSlotBytes = kSlotStats + kGemmMaxRows * 8;
static_assert(kSlotBytes % 256 == 0, "slots stay 256-byte aligned");

// 16-row tiles per workgroup: the smallest tile that covers M up to 32 rows, 32 rows beyond that.
// Rows past 32 are re-read weight tiles that hit the XCD's L2 (see the XCD-aware order below).
// 64-row W4A16 tiles (each expanded weight fragment feeding four MFMAs) measured slower over the
// Llama-3-8B-shaped stack -- M = 128 5.18 against 4.71 ms per pass, M = 64 4.05 against 3.38 --
// because their registers leave room for one group of weights in flight, not two.
static int gemm_mt(int mode, int M) {
  (void)mode;
  return M <= 16 ? 1 : 2;
}
// Waves per SIMD the register budget allows: 16-row tiles and W4A16 32-row tiles with a 2-group
// ring fit three (at most 168 registers, the standardisation and the Top-1 epilogue included); a
// deeper ring and the 32-row integer tile's fp64 accumulators need two.
template <int MODE, bool NORM, int MT, int D, bool STATS>
constexpr int kGemmOcc = ((MODE == 0 && D <= 2) || MT == 1) ? 3 : 2;

struct GemmArgs {
  const uint16_t* x;   // W4A16: fp16 activations [M][ldx]
  int ldx;
  const int8_t* xq;    // W4A4: operand-ordered codes [M][K]
  const float* sxf;    // W4A4: per-row scale (fp32 value of the fp16 scale) [M]
  const uint4* w;      // packed tiles
  const uint16_t* sc;  // packed scales
  int M, N, K;
  int gps;             // 128-wide groups per K split
  int splits;
  unsigned char* slots;  // splits > 1: partial slots [split][tile]
  unsigned* cnt;         // splits > 1: arrival counter per output tile (zero at launch, left zero)
  float* y;            // fp32 output [M][N] ...
  uint16_t* y16;       // ... or fp16 output with row stride ldy (both NULL: not written)
  int ldy;
  // Top-1 epilogue (LM-head): per-(row, column tile, wave) softmax-statistics partials
  // [M][tiles][4], merged by top1_merge_kernel
  unsigned char* stats;
};

__device__ __forceinline__ void gemm_lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <typename F, int... Is>
__device__ __forceinline__ void gemm_static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void gemm_static_for(F&& f) {
  gemm_static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Device-coherent (SC1) 16-byte and 8-byte accesses to the partial slots, through a buffer
// resource over the slot array (offsets stay below 2^31: at most 256 tiles x 16 splits x 67 KB).
constexpr int kGemmSc1 = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gemm_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ void slot_store4(unsigned char* base, int off, float4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(int4_t, v), gemm_rsrc(base), off, 0, kGemmSc1);
}
__device__ __forceinline__ float4_t slot_load4(const unsigned char* base, int off) {
  return __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(gemm_rsrc(base), off, 0, kGemmSc1));
}
__device__ __forceinline__ void slot_store1(unsigned char* base, int off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(v), gemm_rsrc(base), off, 0, kGemmSc1);
}
__device__ __forceinline__ float slot_load1(const unsigned char* base, int off) {
  return __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(gemm_rsrc(base), off, 0, kGemmSc1));
}
// Accumulators of either width: float4 in 16 bytes, double4 in 32.
__device__ __forceinline__ void slot_store_acc(unsigned char* base, int idx, float4_t v) { slot_store4(base, idx * 16, v); }
__device__ __forceinline__ float4_t slot_load_acc(const unsigned char* base, int idx, float4_t) {
  return slot_load4(base, idx * 16);
}
__device__ __forceinline__ void slot_store_acc(unsigned char* base, int idx, double4_t v) {
  const int4_t* p = reinterpret_cast<const int4_t*>(&v);
  __builtin_amdgcn_raw_buffer_store_b128(p[0], gemm_rsrc(base), idx * 32, 0, kGemmSc1);
  __builtin_amdgcn_raw_buffer_store_b128(p[1], gemm_rsrc(base), idx * 32 + 16, 0, kGemmSc1);
}
__device__ __forceinline__ double4_t slot_load_acc(const unsigned char* base, int idx, double4_t) {
  int4_t p[2];
  p[0] = __builtin_amdgcn_raw_buffer_load_b128(gemm_rsrc(base), idx * 32, 0, kGemmSc1);
  p[1] = __builtin_amdgcn_raw_buffer_load_b128(gemm_rsrc(base), idx * 32 + 16, 0, kGemmSc1);
  return __builtin_bit_cast(double4_t, p);
}
// Output value of an accumulator: W4A16 as accumulated; the integer modes' exact fp64 value times the
// row scale, rounded once (to fp32 here, or to fp16 by out16).
__device__ __forceinline__ float out32(float v, float) { return v; }
__device__ __forceinline__ float out32(double v, float sx) { return (float)(v * (double)sx); }
__device__ __forceinline__ uint16_t out16(float v, float) { return f2h(v); }
__device__ __forceinline__ uint16_t out16(double v, float sx) { return f64_to_f16_rn(v * (double)sx); }

// Sum of the 32 codes q of one lane's fragment (four packed dwords, offset-binary nibbles).
__device__ __forceinline__ int fragment_code_sum(const uint4 w) {
  unsigned u = __builtin_amdgcn_udot8(w.x, 0x11111111u, 0u, false);
  u = __builtin_amdgcn_udot8(w.y, 0x11111111u, u, false);
  u = __builtin_amdgcn_udot8(w.z, 0x11111111u, u, false);
  u = __builtin_amdgcn_udot8(w.w, 0x11111111u, u, false);
  return (int)u - 32 * 8;
}

// Top-1 epilogue of one output tile (see STATS below) over the values as stored: value(mt, nt, j,
// ml) is the output of accumulator element j of (mt, nt) at tile row ml.  Each wave reduces its 64
// columns of every row to one (max, sum of exp, first argmax) partial and stores it with a plain
// store: no barrier, no arrival, so the workgroup retires as soon as its stores are issued.  The
// partials of a row, [row][column tile][wave] in column order, are merged by top1_merge_kernel.
template <int MT, typename F>
__device__ __forceinline__ void gemm_top1_epilogue(const GemmArgs& a, F&& value, int m0, int rb0, int by, int lane,
                                                   int wave) {
  const size_t parts = (size_t)gridDim.y * kGemmWaves;  // partials per row
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ml = mt * 16 + 4 * (lane >> 4) + j;
      Msi t{-INFINITY, 0.0f, 0x7fffffff};  // rows past M: computed, never stored
#pragma unroll
      for (int nt = 0; nt < kGemmNt; ++nt) {
        const int n = (rb0 + nt) * 16 + (lane & 15);
        if (n < a.N) t = msi_merge(t, Msi{value(mt, nt, j, ml), 1.0f, n});
      }
      // the 16 lanes holding this row: pairs, quads, halves of 8, rows of 16
      t = msi_merge(t, msi_dpp<0xB1>(t));
      t = msi_merge(t, msi_dpp<0x4E>(t));
      t = msi_merge(t, msi_dpp<0x141>(t));
      t = msi_merge(t, msi_dpp<0x140>(t));
      if ((lane & 15) == 0 && m0 + ml < a.M)
        reinterpret_cast<float4_t*>(a.stats)[(size_t)(m0 + ml) * parts + (size_t)by * kGemmWaves + wave] =
            float4_t{t.m, t.s, __int_as_float(t.i), 0.0f};
    }
  }
}

// Row m's Top-1 from its `parts` partials, one workgroup per row: thread t merges partials t, t +
// 256, ... in order (eight loaded before any is merged, one round trip up to 2048 partials), then
// a fixed-order merge over the lanes and the four waves.
__global__ __launch_bounds__(256) void top1_merge_kernel(const float4_t* __restrict__ stats, int parts,
                                                         int32_t* __restrict__ top1, float* __restrict__ top1_prob) {
  __shared__ Msi wt[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = (int)blockIdx.x;
  const float4_t* row = stats + (size_t)m * parts;
  constexpr int kPer = 8;
  Msi t{-INFINITY, 0.0f, 0x7fffffff};
  for (int c0 = 0; c0 < parts; c0 += 256 * kPer) {
    float4_t v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int c = c0 + 256 * k + (int)threadIdx.x;
      v[k] = row[c < parts ? c : parts - 1];
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k)
      if (c0 + 256 * k + (int)threadIdx.x < parts) t = msi_merge(t, Msi{v[k][0], v[k][1], __float_as_int(v[k][2])});
  }
  t = wave_msi(t);
  if (lane == 0) wt[wave] = t;
  __syncthreads();
  if (threadIdx.x == 0) {
    t = msi_merge(msi_merge(wt[0], wt[1]), msi_merge(wt[2], wt[3]));
    top1[m] = t.i;
    if (top1_prob) top1_prob[m] = 1.0f / t.s;
  }
}

// MODE 0 (W4A16) with NORM: the input rows are standardised over their K columns, applied after
// the contraction as y = (sum_k x w - mu sum_k w) / sd.  The row sums come from the activations as
// they are staged, the weight sums sum_k w from the packed codes, so no separate pass over the
// activations is needed.  MT: 16-row tiles per workgroup; D: groups of weights in flight per wave
// (a register ring: the weights do not depend on the activations, so they are fetched D groups
// ahead of their use).
//
// STATS (the LM-head's Top-1 epilogue): besides (or instead of) storing the logits, each wave
// reduces every row's values over its 64 columns to (max, sum of exp(v - max), first argmax) and
// stores that partial; top1_merge_kernel merges a row's partials in column order into its Top-1
// and Top-1 probability 1 / sum exp(v - max).  So a greedy step never reads the logits back.
template <int MODE, bool NORM, int MT, int D, bool STATS>
__global__ __launch_bounds__(kGemmWaves * 64, (kGemmOcc<MODE, NORM, MT, D, STATS>)) void gemm_kernel(const GemmArgs a) {
  static_assert(MODE == 0 || !NORM, "standardisation is fused for W4A16 only");
  using Acc = std::conditional_t<MODE == 0, float4_t, double4_t>;
  constexpr int kRows = MT * 16;
  constexpr int kRowB = MODE == 0 ? 256 : 128;  // activation bytes per row and group
  constexpr int kPitch = kRowB + 16;
  constexpr int kTotalPieces = kRows * kRowB / 16;  // 16-byte copies per group
  constexpr int kPieces = (kTotalPieces + kGemmWaves * 64 - 1) / (kGemmWaves * 64);
  constexpr int kSteps = MODE == 0 ? 4 : 2;     // MFMA k-steps per group
  static_assert(!NORM || kTotalPieces % (kGemmWaves * 64) == 0, "row statistics assume whole pieces");
  __shared__ __align__(16) unsigned char abuf[2][kRows * kPitch];
  __shared__ float row_mu[kRows], row_inv[kRows];
  __shared__ int last_sh;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int G = a.K >> 7;
  const int nrb = (a.N + 15) >> 4;
  // XCD-aware order: workgroup L of the launch runs on XCD L % 8, so consecutive logical indices
  // (the row tiles of one column block, then its neighbours) are given to one XCD and share its L2.
  int bx, by, split;
  {
    const int mtiles = (int)gridDim.x, ntiles = (int)gridDim.y;
    const int total = mtiles * ntiles * (int)gridDim.z;
    const int L = (int)(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
    const int xcd = L & 7, idx = L >> 3, per = total >> 3, rem = total & 7;
    const int lg = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    bx = lg % mtiles;
    by = (lg / mtiles) % ntiles;
    split = lg / (mtiles * ntiles);
  }
  const int m0 = bx * kRows;
  const int rb0 = by * kGemmBlocks + wave * kGemmNt;
  const int g0 = split * a.gps;
  const int g1 = g0 + a.gps < G ? g0 + a.gps : G;

  // Activation staging: thread t copies pieces t + 256 j of the [rows][kRowB] chunk.  Rows past
  // M copy row M-1: result row i depends only on operand row i, and those rows are not stored.
  // (W4A16: piece t + 256 j is row t / 16 + 16 j, so the 16 lanes of a DPP row share a row.)
  // Sources as 32-bit byte offsets from the (uniform) activation base: at most 256 rows of 64 Ki
  // fp16 columns, and they keep the register count low enough that nothing is spilled.
  const unsigned char* const abase =
      MODE == 0 ? reinterpret_cast<const unsigned char*>(a.x) : reinterpret_cast<const unsigned char*>(a.xq);
  uint32_t asrc[kPieces];
  uint32_t adst[kPieces];
  bool aon[kPieces];
#pragma unroll
  for (int j = 0; j < kPieces; ++j) {
    const int p = (int)threadIdx.x + j * kGemmWaves * 64;
    aon[j] = p < kTotalPieces;
    const int pc = aon[j] ? p : 0;
    const int row = pc / (kRowB / 16), col = pc - row * (kRowB / 16);
    const int r = m0 + row < a.M ? m0 + row : a.M - 1;
    asrc[j] = (uint32_t)(r * (MODE == 0 ? 2 * a.ldx : a.K) + col * 16);
    adst[j] = (uint32_t)(row * kPitch + col * 16);
  }
  // A native vector type: an array of HIP's uint4 struct is copied with memcpy and stays in
  // scratch memory instead of registers.
  int4_t areg[kPieces];
  float rsum[kPieces], rsq[kPieces];
#pragma unroll
  for (int j = 0; j < kPieces; ++j) rsum[j] = rsq[j] = 0.0f;
  auto a_load = [&](int g) __attribute__((always_inline)) {
    const int gg = g < g1 ? g : g1 - 1;
#pragma unroll
    for (int j = 0; j < kPieces; ++j)
      if (aon[j]) areg[j] = *reinterpret_cast<const int4_t*>(abase + asrc[j] + (size_t)gg * kRowB);
  };
  // store the staged group into LDS buffer b; `real` = it is a group of this split (not a re-read
  // past the end)
  auto a_store = [&](int b, bool real) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kPieces; ++j)
      if (aon[j]) *reinterpret_cast<int4_t*>(&abuf[b][adst[j]]) = areg[j];
    if constexpr (NORM) {
      if (real) {
#pragma unroll
        for (int j = 0; j < kPieces; ++j) {  // fp16 pairs: products exact, sums in fp32
          const half8_t h = __builtin_bit_cast(half8_t, areg[j]);
          const half2_t one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const half2_t p = {h[2 * e], h[2 * e + 1]};
            rsum[j] = __builtin_amdgcn_fdot2(p, one, rsum[j], false);
            rsq[j] = __builtin_amdgcn_fdot2(p, p, rsq[j], false);
          }
        }
      }
    }
  };

  // Weight row blocks past N read block 0 (never stored).  Tile indices fit 32 bits (N / 16 * K / 128).
  uint32_t wbase[kGemmNt];
#pragma unroll
  for (int nt = 0; nt < kGemmNt; ++nt) {
    const int rb = rb0 + nt < nrb ? rb0 + nt : 0;
    wbase[nt] = (uint32_t)(rb * G);
  }
  uint4 wr[D][kGemmNt];
  uint16_t sr[D][kGemmNt];
  // Unconditional (a group past the range re-reads the last one), so the loads in flight are the
  // same at every slot and the compiler waits for exactly the oldest.
  auto w_issue = [&](int slot, int g) __attribute__((always_inline)) {
    const int gg = g < g1 ? g : g1 - 1;
#pragma unroll
    for (int nt = 0; nt < kGemmNt; ++nt) {
      const size_t t = wbase[nt] + (uint32_t)gg;
      wr[slot][nt] = a.w[t * 64 + lane];
      sr[slot][nt] = a.sc[t * 16 + (lane & 15)];
    }
  };

  Acc acc[MT][kGemmNt];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < kGemmNt; ++nt) acc[mt][nt] = Acc{0, 0, 0, 0};
  float csum[kGemmNt];  // NORM: this lane's share of sum_k w for column lane & 15 of each block
#pragma unroll
  for (int nt = 0; nt < kGemmNt; ++nt) csum[nt] = 0.0f;

  a_load(g0);
  gemm_static_for<D>([&](auto ic) __attribute__((always_inline)) { w_issue(decltype(ic)::value, g0 + decltype(ic)::value); });
  a_store(0, true);
  gemm_lds_barrier();
  const uint32_t magic = fp16_magic_vgpr();
  // fragment offset of this lane inside a staged row: k = 32 (lane >> 4) + step * (32 or 16)
  const uint32_t lane_off = (uint32_t)((lane & 15) * kPitch + (MODE == 0 ? 64 : 32) * (lane >> 4));

  for (int g = g0; g < g1; g += D) {
    gemm_static_for<D>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      const int gi = g + i;
      if (gi < g1) {
        const int cur = (gi - g0) & 1;
        a_load(gi + 1);  // next group's activations, stored after this group's math
        const unsigned char* ab = abuf[cur];
        if constexpr (MODE == 0) {
          // each group's exact products summed in fp32 by the MFMAs, then scaled by the group's scale.
          // The group's A fragments (every row tile and k-step) are read once and held; the blocks
          // are then taken one at a time, so only one block's group sums are live.
          half8_t av[MT][kSteps];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int t = 0; t < kSteps; ++t)
              av[mt][t] = *reinterpret_cast<const half8_t*>(ab + lane_off + mt * 16 * kPitch + 16 * t);
#pragma unroll
          for (int nt = 0; nt < kGemmNt; ++nt) {
            float4_t dg[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) dg[mt] = float4_t{0.f, 0.f, 0.f, 0.f};
            const uint4 wv = wr[i][nt];
#pragma unroll
            for (int t = 0; t < kSteps; ++t) {
              const half8_t b = unpack_f16x8(t == 0 ? wv.x : t == 1 ? wv.y : t == 2 ? wv.z : wv.w, magic);
#pragma unroll
              for (int mt = 0; mt < MT; ++mt) dg[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[mt][t], b, dg[mt], 0, 0, 0);
            }
            const float s = h2f(sr[i][nt]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt][nt] += s * dg[mt];
            if constexpr (NORM)  // exact product; the weights' own sum, unrounded
              csum[nt] += s * (float)fragment_code_sum(wv);
          }
        } else {
          int4_t dg[MT][kGemmNt];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < kGemmNt; ++nt) dg[mt][nt] = int4_t{0, 0, 0, 0};
#pragma unroll
          for (int t2 = 0; t2 < kSteps; ++t2) {
            int4_t b[kGemmNt];
#pragma unroll
            for (int nt = 0; nt < kGemmNt; ++nt) {
              const uint4 wv = wr[i][nt];
              b[nt] = t2 == 0 ? unpack_i8x16(wv.x, wv.y) : unpack_i8x16(wv.z, wv.w);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              const int4_t av = *reinterpret_cast<const int4_t*>(ab + lane_off + mt * 16 * kPitch + 16 * t2);
#pragma unroll
              for (int nt = 0; nt < kGemmNt; ++nt)
                dg[mt][nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, b[nt], dg[mt][nt], 0, 0, 0);
            }
          }
#pragma unroll
          for (int nt = 0; nt < kGemmNt; ++nt) {
            const double s = (double)h2f(sr[i][nt]) * 0.0625;  // operands carry 16 q: exact rescale
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
              for (int j = 0; j < 4; ++j) acc[mt][nt][j] += s * (double)dg[mt][nt][j];  // exact in fp64
          }
        }
        w_issue(i, gi + D);  // refill this slot after consuming it
        a_store(cur ^ 1, gi + 1 < g1);
        gemm_lds_barrier();
      }
    });
  }

  // ---- this split's column and row sums (NORM)
  if constexpr (NORM) {
    // columns: lanes l, l + 16, l + 32, l + 48 hold the four k quarters of column l & 15
#pragma unroll
    for (int nt = 0; nt < kGemmNt; ++nt) {
      const float c0 = __shfl(csum[nt], lane & 15, 64), c1 = __shfl(csum[nt], (lane & 15) + 16, 64);
      const float c2 = __shfl(csum[nt], (lane & 15) + 32, 64), c3 = __shfl(csum[nt], (lane & 15) + 48, 64);
      csum[nt] = (c0 + c1) + (c2 + c3);
    }
    // rows: the 16 lanes of a DPP row share a row; lane 16 r + 0 keeps the result
#pragma unroll
    for (int j = 0; j < kPieces; ++j) {
      auto row16 = [](float v) {
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
        return v;
      };
      rsum[j] = row16(rsum[j]);
      rsq[j] = row16(rsq[j]);
    }
  }

  // ---- K splits: publish this split's partials; the tile's last arrival sums all splits in split
  // order (deterministic whichever workgroup arrives last) and writes the output.
  const int tile = by * (int)gridDim.x + bx;
  if (a.splits > 1) {
    const int tiles = (int)(gridDim.x * gridDim.y);
    unsigned char* my = a.slots + ((size_t)split * tiles + tile) * kSlotBytes;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < kGemmNt; ++nt)
        slot_store_acc(my, ((wave * MT + mt) * kGemmNt + nt) * 64 + lane, acc[mt][nt]);
    if constexpr (NORM) {
      if (lane < 16) {
#pragma unroll
        for (int nt = 0; nt < kGemmNt; ++nt) slot_store1(my, kSlotCs + ((wave * kGemmNt + nt) * 16 + lane) * 4, csum[nt]);
      }
      if ((lane & 15) == 0) {
#pragma unroll
        for (int j = 0; j < kPieces; ++j) {
          const int row = (int)(threadIdx.x >> 4) + 16 * j;
          slot_store1(my, kSlotStats + row * 8, rsum[j]);
          slot_store1(my, kSlotStats + row * 8 + 4, rsq[j]);
        }
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's partials are in memory
    __syncthreads();
    if (threadIdx.x == 0) {
      const unsigned old = __hip_atomic_fetch_add(a.cnt + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int last = old + 1u == (unsigned)a.splits;
      if (last) __hip_atomic_store(a.cnt + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last_sh = last;
    }
    __syncthreads();
    if (!last_sh) return;
    // sum every split's partial (this workgroup's own included, as stored) in split order, so the
    // result does not depend on which workgroup arrives last; two splits' loads are in flight at once
    for (int s = 0; s < a.splits; s += 2) {
      const bool two = s + 1 < a.splits;
      const unsigned char* p0 = a.slots + ((size_t)s * tiles + tile) * kSlotBytes;
      const unsigned char* p1 = a.slots + ((size_t)(two ? s + 1 : s) * tiles + tile) * kSlotBytes;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < kGemmNt; ++nt) {
          const int idx = ((wave * MT + mt) * kGemmNt + nt) * 64 + lane;
          const Acc v0 = slot_load_acc(p0, idx, Acc{}), v1 = slot_load_acc(p1, idx, Acc{});
          Acc t = s == 0 ? v0 : acc[mt][nt] + v0;
          if (two) t += v1;
          acc[mt][nt] = t;
        }
      if constexpr (NORM) {
#pragma unroll
        for (int nt = 0; nt < kGemmNt; ++nt) {
          const int off = kSlotCs + ((wave * kGemmNt + nt) * 16 + (lane & 15)) * 4;
          const float v0 = slot_load1(p0, off), v1 = slot_load1(p1, off);
          float t = s == 0 ? v0 : csum[nt] + v0;
          if (two) t += v1;
          csum[nt] = t;
        }
#pragma unroll
        for (int j = 0; j < kPieces; ++j) {
          const int off = kSlotStats + ((int)(threadIdx.x >> 4) + 16 * j) * 8;
          const float s0 = slot_load1(p0, off), q0 = slot_load1(p0, off + 4);
          const float s1 = slot_load1(p1, off), q1 = slot_load1(p1, off + 4);
          float ts = s == 0 ? s0 : rsum[j] + s0, tq = s == 0 ? q0 : rsq[j] + q0;
          if (two) {
            ts += s1;
            tq += q1;
          }
          rsum[j] = ts;
          rsq[j] = tq;
        }
      }
    }
  }
  if constexpr (NORM) {
    if ((lane & 15) == 0) {
#pragma unroll
      for (int j = 0; j < kPieces; ++j) {
        const int row = (int)(threadIdx.x >> 4) + 16 * j;
        float mu, inv;
        norm_params(rsum[j], rsq[j], a.K, mu, inv);
        row_mu[row] = mu;
        row_inv[row] = inv;
      }
    }
    __syncthreads();
  }

  // Epilogue: lane holds rows 4 (lane >> 4) + j of each row tile, column lane & 15 of each block.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ml = mt * 16 + 4 * (lane >> 4) + j;
      const int m = m0 + ml;
      if (m >= a.M) continue;
      const float sx = MODE == 1 ? a.sxf[m] : 1.0f;
      float mu = 0.0f, inv = 1.0f;
      if constexpr (NORM) {
        mu = row_mu[ml];
        inv = row_inv[ml];
      }
#pragma unroll
      for (int nt = 0; nt < kGemmNt; ++nt) {
        const int n = (rb0 + nt) * 16 + (lane & 15);
        if (n >= a.N) continue;
        if constexpr (NORM) {
          const float v = (acc[mt][nt][j] - mu * csum[nt]) * inv;
          if (a.y16)
            a.y16[(size_t)m * a.ldy + n] = f2h(v);
          else if (a.y)
            a.y[(size_t)m * a.N + n] = v;
        } else {
          if (a.y16)
            a.y16[(size_t)m * a.ldy + n] = out16(acc[mt][nt][j], sx);
          else if (a.y)
            a.y[(size_t)m * a.N + n] = out32(acc[mt][nt][j], sx);
        }
      }
    }
  }
  if constexpr (STATS) {
    // the values as stored: standardised (NORM) or with the integer modes' row scale applied
    auto value = [&](int mt, int nt, int j, int ml) __attribute__((always_inline)) {
      if constexpr (NORM) {
        return (acc[mt][nt][j] - row_mu[ml] * csum[nt]) * row_inv[ml];
      } else {
        const int m = m0 + ml < a.M ? m0 + ml : a.M - 1;
        return out32(acc[mt][nt][j], MODE == 1 ? a.sxf[m] : 1.0f);
      }
    };
    gemm_top1_epilogue<MT>(a, value, m0, rb0, by, lane, wave);
  }
}

__global__ __launch_bounds__(256) void gemm_clear_kernel(unsigned* __restrict__ cnt, int n) {
  for (int i = threadIdx.x; i < n; i += 256) cnt[i] = 0u;
}

// ------------------------------------------------------------------ host side

// K splits for an M x N x K linear: enough workgroups for a 256-CU part, at least
// kGemmMinGroupsPerSplit groups per split.
static int gemm_tiles(int mode, int M, int N) {
  const int rows = gemm_mt(mode, M) * 16;
  return (((N + 15) / 16 + kGemmBlocks - 1) / kGemmBlocks) * ((M + rows - 1) / rows);
}

int gemm_splits(int mode, int M, int N, int K) {
  const int tiles = gemm_tiles(mode, M, N);
  const int G = K / kGroup;
  int s = 1;
  // The integer modes' fp64 partial slots are twice as large and their last arrival sums them in
  // fp64, so they split less: over the Llama-3-8B-shaped stack (W4A4 pass ms, M = 4 / 24 / 64 / 128)
  // at most 128 workgroups and 8 groups per split gave 2.97 / 3.90 / 4.29 / 5.38 against
  // 3.36 / 4.75 / 5.28 / 5.19 with the W4A16 rule, and at M = 128 16 groups per split 4.92.
  const bool wide = mode != QS_W4A16 && M > 64;
  const int target = mode == QS_W4A16 || wide ? 256 : 128;
  const int min_groups = mode == QS_W4A16 ? kGemmMinGroupsPerSplit : wide ? 16 : 8;
  while (s < kGemmMaxSplits && tiles * s < target && G / (2 * s) >= min_groups) s *= 2;
  return s;
}

size_t gemm_counter_bytes() { return align_up((size_t)kGemmMaxCounters * 4, 256); }

size_t gemm_top1_bytes(int M, int N) {
  const size_t ntiles = (size_t)((N + 15) / 16 + kGemmBlocks - 1) / kGemmBlocks;
  return align_up((size_t)M * ntiles * kGemmWaves * 16, 256);
}

size_t gemm_workspace(int mode, int M, int N, int K) {
  const int s = gemm_splits(mode, M, N, K);
  if (s <= 1) return 0;
  return (size_t)s * gemm_tiles(mode, M, N) * kSlotBytes;
}

int launch_gemm_clear(unsigned* cnt, hipStream_t st) {
  hipLaunchKernelGGL(gemm_clear_kernel, dim3(1), dim3(256), 0, st, cnt, kGemmMaxCounters);
  return launch_status();
}

template <int MODE, bool NORM, int MT, int D>
static void gemm_launch_one(const GemmArgs& a, dim3 grid, hipStream_t st) {
  if (a.stats) {
    hipLaunchKernelGGL((gemm_kernel<MODE, NORM, MT, D, true>), grid, dim3(kGemmWaves * 64), 0, st, a);
    return;
  }
  hipLaunchKernelGGL((gemm_kernel<MODE, NORM, MT, D, false>), grid, dim3(kGemmWaves * 64), 0, st, a);
}

// Weight ring depth per row tile: 16-row tiles a 3-group (W4A16, whose per-group sums take registers)
// or 4-group ring, 32-row tiles a QS_GEMM_MT2_RING-group ring.  Deeper 32-row rings (at two waves
// per SIMD) measured no faster: W4A16 M = 128 4.74 / 4.85 / 4.82 ms with 2 / 3 / 4 groups.
#ifndef QS_GEMM_MT2_RING
#define QS_GEMM_MT2_RING 2
#endif
template <int MODE, bool NORM>
static void gemm_launch_mt(const GemmArgs& a, int mt, dim3 grid, hipStream_t st) {
  if (mt == 1)
    gemm_launch_one<MODE, NORM, 1, MODE == 0 ? 3 : 4>(a, grid, st);
  else
    gemm_launch_one<MODE, NORM, 2, QS_GEMM_MT2_RING>(a, grid, st);
}

int launch_gemm(int mode, bool norm, const uint16_t* x, int ldx, const int8_t* xq, const float* sxf,
                const uint8_t* wp, const uint16_t* sp, int M, int N, int K, float* y, uint16_t* y16, int ldy,
                unsigned* cnt, void* ws, size_t ws_bytes, hipStream_t st, const GemmTop1* t1) {
  if (t1 && (!t1->stats || !t1->top1)) return QS_ERR_INVALID_ARG;
  if (mode != QS_W4A16 && norm) return QS_ERR_INVALID_ARG;
  // split K only when the caller's scratch holds the partial slots and the (zeroed) counters;
  // results then differ from the unsplit order by fp32 rounding only
  const size_t need = gemm_workspace(mode, M, N, K);
  const int splits = need > 0 && cnt != nullptr && ws != nullptr && ws_bytes >= need ? gemm_splits(mode, M, N, K) : 1;
  const int G = K / kGroup;
  const int mt = gemm_mt(mode, M);
  GemmArgs a{};
  a.x = x;
  a.ldx = ldx;
  a.xq = xq;
  a.sxf = sxf;
  a.w = reinterpret_cast<const uint4*>(wp);
  a.sc = sp;
  a.M = M;
  a.N = N;
  a.K = K;
  a.gps = (G + splits - 1) / splits;
  a.splits = (G + a.gps - 1) / a.gps;
  a.slots = a.splits > 1 ? static_cast<unsigned char*>(ws) : nullptr;
  a.cnt = a.splits > 1 ? cnt : nullptr;
  a.y = y;
  a.y16 = y16;
  a.ldy = ldy;
  if (t1) a.stats = t1->stats;
  const int nrb = (N + 15) / 16;
  const dim3 grid((M + mt * 16 - 1) / (mt * 16), (nrb + kGemmBlocks - 1) / kGemmBlocks, a.splits);
  if (a.splits > 1 && (int)(grid.x * grid.y) > kGemmMaxCounters) return QS_ERR_UNSUPPORTED;
  if (mode == QS_W4A16) {
    if (norm)
      gemm_launch_mt<0, true>(a, mt, grid, st);
    else
      gemm_launch_mt<0, false>(a, mt, grid, st);
  } else {
    gemm_launch_mt<1, false>(a, mt, grid, st);
  }
  if (t1) {
    const int rc = launch_status();
    if (rc != QS_OK) return rc;
    hipLaunchKernelGGL(top1_merge_kernel, dim3((unsigned)M), dim3(256), 0, st,
                       reinterpret_cast<const float4_t*>(t1->stats), (int)grid.y * kGemmWaves, t1->top1,
                       t1->top1_prob);
  }
  return launch_status();
}

}  // namespace qs
