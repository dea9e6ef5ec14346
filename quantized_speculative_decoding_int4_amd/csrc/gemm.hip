// Batched linear (M >= 16 activation rows): the verify pass over many sequences, where the
// target scores B * (gamma + 1) positions at once ([P3] "draft modelとtarget modelの処理フロー";
// modes from [P1] "QSpec の W4A4 モードと W4A16 モード").  Same arithmetic as the streaming
// linear: W4A16 expands the INT4 codes to fp16 in registers and runs v_mfma_f32_16x16x32_f16,
// W4A4 runs v_mfma_i32_16x16x64_i8 on the quantized activations; both scale each 128-wide group
// partial sum in fp32.
//
// Work split.  A workgroup of 4 waves owns an output tile of 64 rows (4 MFMA row tiles) x 256
// columns (16 packed row blocks, 4 per wave) over a range of K, one 128-wide group at a time:
//   * the 64 activation rows of the group are staged once in LDS (double-buffered, rows padded by
//     16 bytes so the fragment reads of 16 rows hit distinct banks) and read by all 4 waves;
//   * each wave keeps its 4 weight tiles of the group (and of the next one) in registers, expands
//     each fragment once and feeds it to 4 MFMAs (one per row tile), while each activation
//     fragment feeds 4 MFMAs (one per weight tile): per 16-cycle MFMA about 3 VALU operations and
//     256 bytes of LDS reads, which the SIMD and LDS sustain together.
// The row tile is the fastest-varying workgroup index, so the workgroups that read the same weight
// tiles for different rows run back to back and the second read is served by the caches.

#include "qs_device.h"
#include "qs_internal.h"

#include <type_traits>

namespace qs {

constexpr int kGemmWaves = 4;
constexpr int kGemmMt = 4;                      // 16-row MFMA tiles per workgroup (all waves)
constexpr int kGemmRows = kGemmMt * 16;         // 64 activation rows per workgroup
constexpr int kGemmNt = 4;                      // 16-column row blocks per wave
constexpr int kGemmBlocks = kGemmWaves * kGemmNt;  // row blocks per workgroup (256 columns)
constexpr int kGemmMaxSplits = 16;

struct GemmArgs {
  const uint16_t* x;   // W4A16: fp16 activations [M][ldx]
  int ldx;
  const int8_t* xq;    // W4A4: operand-ordered codes [M][K]
  const float* sxf;    // W4A4: per-row scale (fp32 value of the fp16 scale) [M]
  const uint4* w;      // packed tiles
  const uint16_t* sc;  // packed scales
  int M, N, K;
  int gps;             // 128-wide groups per K split
  float* part;         // splits > 1: fp32 partials [split][M][N]
  float* y;            // splits == 1: fp32 output [M][N] ...
  uint16_t* y16;       // ... or fp16 output with row stride ldy
  int ldy;
};

__device__ __forceinline__ void gemm_lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <typename F>
__device__ __forceinline__ void gemm_static_for_2(F&& f) {
  f(std::integral_constant<int, 0>{});
  f(std::integral_constant<int, 1>{});
}

template <int MODE>
__global__ __launch_bounds__(kGemmWaves * 64) void gemm_kernel(const GemmArgs a) {
  constexpr int kRowB = MODE == 0 ? 256 : 128;  // activation bytes per row and group
  constexpr int kPitch = kRowB + 16;
  constexpr int kPieces = kGemmRows * kRowB / 16 / (kGemmWaves * 64);  // 16-byte copies per thread
  constexpr int kSteps = MODE == 0 ? 4 : 2;     // MFMA k-steps per group
  __shared__ __align__(16) unsigned char abuf[2][kGemmRows * kPitch];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int G = a.K >> 7;
  const int nrb = (a.N + 15) >> 4;
  const int m0 = (int)blockIdx.x * kGemmRows;
  const int rb0 = (int)blockIdx.y * kGemmBlocks + wave * kGemmNt;
  const int g0 = (int)blockIdx.z * a.gps;
  const int g1 = g0 + a.gps < G ? g0 + a.gps : G;

  // Activation staging: thread t copies pieces t + 256 j of the [64 rows][kRowB] chunk.  Rows past
  // M copy row M-1: result row i depends only on operand row i, and those rows are not stored.
  const unsigned char* asrc[kPieces];
  uint32_t adst[kPieces];
#pragma unroll
  for (int j = 0; j < kPieces; ++j) {
    const int p = (int)threadIdx.x + j * kGemmWaves * 64;
    const int row = p / (kRowB / 16), col = p - row * (kRowB / 16);
    const int r = m0 + row < a.M ? m0 + row : a.M - 1;
    asrc[j] = MODE == 0 ? reinterpret_cast<const unsigned char*>(a.x + (size_t)r * a.ldx) + col * 16
                        : reinterpret_cast<const unsigned char*>(a.xq + (size_t)r * a.K) + col * 16;
    adst[j] = (uint32_t)(row * kPitch + col * 16);
  }
  // A native vector type: an array of HIP's uint4 struct is copied with memcpy and stays in
  // scratch memory instead of registers.
  int4_t areg[kPieces];
  auto a_load = [&](int g) __attribute__((always_inline)) {
    const int gg = g < g1 ? g : g1 - 1;
#pragma unroll
    for (int j = 0; j < kPieces; ++j)
      areg[j] = *reinterpret_cast<const int4_t*>(asrc[j] + (size_t)gg * kRowB);
  };
  auto a_store = [&](int b) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kPieces; ++j) *reinterpret_cast<int4_t*>(&abuf[b][adst[j]]) = areg[j];
  };

  // Weight row blocks past N read block 0 (never stored).
  size_t wbase[kGemmNt];
#pragma unroll
  for (int nt = 0; nt < kGemmNt; ++nt) {
    const int rb = rb0 + nt < nrb ? rb0 + nt : 0;
    wbase[nt] = (size_t)rb * G;
  }
  uint4 wr[2][kGemmNt];
  uint16_t sr[2][kGemmNt];
  // Unconditional (a group past the range re-reads the last one), so the loads in flight are the
  // same at every slot and the compiler waits for exactly the oldest.
  auto w_issue = [&](int slot, int g) __attribute__((always_inline)) {
    const int gg = g < g1 ? g : g1 - 1;
#pragma unroll
    for (int nt = 0; nt < kGemmNt; ++nt) {
      const size_t t = wbase[nt] + gg;
      wr[slot][nt] = a.w[t * 64 + lane];
      sr[slot][nt] = a.sc[t * 16 + (lane & 15)];
    }
  };

  float4_t acc[kGemmMt][kGemmNt];
#pragma unroll
  for (int mt = 0; mt < kGemmMt; ++mt)
#pragma unroll
    for (int nt = 0; nt < kGemmNt; ++nt) acc[mt][nt] = float4_t{0.f, 0.f, 0.f, 0.f};

  a_load(g0);
  w_issue(0, g0);
  w_issue(1, g0 + 1);
  a_store(0);
  gemm_lds_barrier();
  const uint32_t magic = fp16_magic_vgpr();
  // fragment offset of this lane inside a staged row: k = 32 (lane >> 4) + step * (32 or 16)
  const uint32_t lane_off = (uint32_t)((lane & 15) * kPitch + (MODE == 0 ? 64 : 32) * (lane >> 4));

  for (int g = g0; g < g1; g += 2) {
    gemm_static_for_2([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      const int gi = g + i;
      if (gi < g1) {
        const int cur = (gi - g0) & 1;
        a_load(gi + 1);  // next group's activations, stored after this group's math
        const unsigned char* ab = abuf[cur];
        if constexpr (MODE == 0) {
          float4_t dg[kGemmMt][kGemmNt];
#pragma unroll
          for (int mt = 0; mt < kGemmMt; ++mt)
#pragma unroll
            for (int nt = 0; nt < kGemmNt; ++nt) dg[mt][nt] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int t = 0; t < kSteps; ++t) {
            half8_t b[kGemmNt];
#pragma unroll
            for (int nt = 0; nt < kGemmNt; ++nt) {
              const uint4 wv = wr[i][nt];
              const uint32_t wt = t == 0 ? wv.x : t == 1 ? wv.y : t == 2 ? wv.z : wv.w;
              b[nt] = unpack_f16x8(wt, magic);
            }
#pragma unroll
            for (int mt = 0; mt < kGemmMt; ++mt) {
              const half8_t av = *reinterpret_cast<const half8_t*>(ab + lane_off + mt * 16 * kPitch + 16 * t);
#pragma unroll
              for (int nt = 0; nt < kGemmNt; ++nt)
                dg[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, b[nt], dg[mt][nt], 0, 0, 0);
            }
          }
#pragma unroll
          for (int nt = 0; nt < kGemmNt; ++nt) {
            const float s = h2f(sr[i][nt]);
#pragma unroll
            for (int mt = 0; mt < kGemmMt; ++mt) acc[mt][nt] += s * dg[mt][nt];
          }
        } else {
          int4_t dg[kGemmMt][kGemmNt];
#pragma unroll
          for (int mt = 0; mt < kGemmMt; ++mt)
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
            for (int mt = 0; mt < kGemmMt; ++mt) {
              const int4_t av = *reinterpret_cast<const int4_t*>(ab + lane_off + mt * 16 * kPitch + 16 * t2);
#pragma unroll
              for (int nt = 0; nt < kGemmNt; ++nt)
                dg[mt][nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, b[nt], dg[mt][nt], 0, 0, 0);
            }
          }
#pragma unroll
          for (int nt = 0; nt < kGemmNt; ++nt) {
            const float s = h2f(sr[i][nt]);
#pragma unroll
            for (int mt = 0; mt < kGemmMt; ++mt)
#pragma unroll
              for (int j = 0; j < 4; ++j) acc[mt][nt][j] += s * (float)(dg[mt][nt][j] >> 4);  // operands carry 16 q
          }
        }
        w_issue(i, gi + 2);  // refill this slot after consuming it
        a_store(cur ^ 1);
        gemm_lds_barrier();
      }
    });
  }

  // Epilogue: lane holds rows 4 (lane >> 4) + j of each row tile, column lane & 15 of each block.
  const bool split = a.part != nullptr;
#pragma unroll
  for (int mt = 0; mt < kGemmMt; ++mt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + mt * 16 + 4 * (lane >> 4) + j;
      if (m >= a.M) continue;
      const float sx = MODE == 1 ? a.sxf[m] : 1.0f;
#pragma unroll
      for (int nt = 0; nt < kGemmNt; ++nt) {
        const int n = (rb0 + nt) * 16 + (lane & 15);
        if (n >= a.N) continue;
        float v = acc[mt][nt][j];
        if constexpr (MODE == 1) v *= sx;
        if (split)
          a.part[((size_t)blockIdx.z * a.M + m) * a.N + n] = v;
        else if (a.y16)
          a.y16[(size_t)m * a.ldy + n] = f2h(v);
        else
          a.y[(size_t)m * a.N + n] = v;
      }
    }
  }
}

// out[m][n] = sum over splits s (in order) of part[s][m][n], as fp32 y or fp16 y16 (row stride ldy).
__global__ __launch_bounds__(256) void gemm_reduce_kernel(const float* __restrict__ part, int splits, int M,
                                                          int N, float* __restrict__ y,
                                                          uint16_t* __restrict__ y16, int ldy) {
  const size_t total = (size_t)M * N;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    float v = part[i];
    for (int s = 1; s < splits; ++s) v += part[(size_t)s * total + i];
    const size_t m = i / (size_t)N, n = i - m * (size_t)N;
    if (y16)
      y16[m * (size_t)ldy + n] = f2h(v);
    else
      y[i] = v;
  }
}

// ------------------------------------------------------------------ host side

// K splits for an M x N x K linear: enough workgroups for a 256-CU part, at least 2 groups per split.
int gemm_splits(int M, int N, int K) {
  const int tiles = (((N + 15) / 16 + kGemmBlocks - 1) / kGemmBlocks) * ((M + kGemmRows - 1) / kGemmRows);
  const int G = K / kGroup;
  int s = 1;
  while (s < kGemmMaxSplits && tiles * s < 256 && G / (2 * s) >= 2) s *= 2;
  return s;
}

size_t gemm_workspace(int M, int N, int K) {
  const int s = gemm_splits(M, N, K);
  return s > 1 ? align_up((size_t)s * M * N * 4, 256) : 0;
}

int launch_gemm(int mode, const uint16_t* x, int ldx, const int8_t* xq, const float* sxf, const uint8_t* wp,
                const uint16_t* sp, int M, int N, int K, float* y, uint16_t* y16, int ldy, void* ws,
                size_t ws_bytes, hipStream_t st) {
  // split K only when the caller's scratch holds the partials (results then differ from the
  // unsplit order by fp32 rounding only)
  const size_t need = gemm_workspace(M, N, K);
  const int splits = need > 0 && ws != nullptr && ws_bytes >= need ? gemm_splits(M, N, K) : 1;
  const int G = K / kGroup;
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
  a.part = splits > 1 ? static_cast<float*>(ws) : nullptr;
  a.y = y;
  a.y16 = y16;
  a.ldy = ldy;
  const int nrb = (N + 15) / 16;
  const dim3 grid((M + kGemmRows - 1) / kGemmRows, (nrb + kGemmBlocks - 1) / kGemmBlocks, (G + a.gps - 1) / a.gps);
  if (mode == QS_W4A16)
    hipLaunchKernelGGL(gemm_kernel<0>, grid, dim3(kGemmWaves * 64), 0, st, a);
  else
    hipLaunchKernelGGL(gemm_kernel<1>, grid, dim3(kGemmWaves * 64), 0, st, a);
  int rc = launch_status();
  if (rc != QS_OK || grid.z == 1) return rc;
  const size_t total = (size_t)M * N;
  size_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(gemm_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a.part, (int)grid.z, M, N, y,
                     y16, ldy);
  return launch_status();
}

}  // namespace qs
