// INT4 weight packing and the dual-mode quantized linear for gfx950.
//
// One packed weight set serves both execution modes of QSpec ([P1] qiita.com,
// "QSpec実行時の2つの量子化による推論の一致率を調べる", sections "W4A16", "W4A4"
// and the mode tree of "QSpec の W4A4 モードと W4A16 モード"):
//   W4A16 (verify): codes expanded to fp16 in registers, fp16 MFMA
//                   (v_mfma_f32_16x16x32_f16), fp32 accumulation, the group
//                   scale applied in fp32 to each 128-wide partial sum.
//   W4A4  (draft) : activations quantized per token to INT4, codes expanded to
//                   int8, int8 MFMA (v_mfma_i32_16x16x64_i8) with exact i32
//                   group sums, fp32 epilogue.  gfx950 has no int4 MFMA.
//
// At decode sizes (M <= 16 rows) the kernel is a weight stream: each 64-lane
// wave pulls whole 1 KiB tiles (one 16 B global_load_dwordx4 per lane, 1 KiB
// per wave instruction, fully coalesced) through a ring of PF outstanding
// tiles, expands nibbles in VGPRs and feeds the tile straight into the MFMA as
// its B operand; activations sit in LDS (or, for large M, are read from L2).
// A workgroup of 8 waves covers R = 8 / S row blocks, S waves splitting K, and
// reduces the S partials through LDS in a fixed order (deterministic).

#include "qs_device.h"
#include "qs_internal.h"

namespace qs {

// ------------------------------------------------------------------ packing

__global__ __launch_bounds__(256) void pack_weights_kernel(const int8_t* __restrict__ q,
                                                           const uint16_t* __restrict__ s,
                                                           int N, int K,
                                                           uint32_t* __restrict__ wp,
                                                           uint16_t* __restrict__ sp,
                                                           size_t total_dwords) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total_dwords) return;
  const int G = K / kGroup;
  const size_t tile = idx >> 8;          // 256 dwords per tile
  const int within = (int)(idx & 255);
  const int lane = within >> 2, t = within & 3;
  const int rb = (int)(tile / G), g = (int)(tile % G);
  const int n = rb * 16 + (lane & 15);
  const int kbase = g * kGroup + 32 * (lane >> 4) + 8 * t;
  uint32_t word = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    int v = 0;
    if (n < N) {
      v = q[(size_t)n * K + kbase + e];
      v = v < -8 ? -8 : (v > 7 ? 7 : v);
    }
    const uint32_t u = (uint32_t)(v + 8);
    const int pos = (e & 1) * 4 + (e >> 1);
    word |= u << (4 * pos);
  }
  wp[idx] = word;
  if (within < 16) {
    const int n2 = rb * 16 + within;
    sp[tile * 16 + within] = n2 < N ? s[(size_t)n2 * G + g] : (uint16_t)0;
  }
}

int launch_pack(const int8_t* q, const uint16_t* s, int N, int K, uint8_t* wp, uint16_t* sp,
                hipStream_t st) {
  const size_t nrb = (size_t)(N + 15) / 16;
  const size_t total = nrb * (size_t)(K / kGroup) * 256;
  const size_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)blocks), dim3(256), 0, st, q, s, N, K,
                     reinterpret_cast<uint32_t*>(wp), sp, total);
  return launch_status();
}

// ------------------------------------------------------------------ activation quantization
// Per-token symmetric INT4: s = fp16(fp32(max|x|) / 7), xq = clamp(rint(x / s), -8, 7), with the
// correctly rounded fp32 quotient (exact for the rounding decision: the quotient of two fp16 values
// is either an exact half-integer tie or at least 2^-13 away from one) and round-half-even rint.

// Quantize one 8-element block (16 bytes of fp16) with scale s; returns the 8 codes in
// operand byte order (low dword, high dword) and in logical order.
__device__ __forceinline__ void quant_block8(const uint4 v, float s, uint2& op, uint2& logical) {
  const uint16_t* h = reinterpret_cast<const uint16_t*>(&v);
  uint32_t lo_op = 0, hi_op = 0, lo_lg = 0, hi_lg = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    int qv = 0;
    if (s != 0.0f) {
      float r = __builtin_rintf(h2f(h[e]) / s);
      r = fminf(7.0f, fmaxf(-8.0f, r));
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

// Stand-alone quantizer for large M: one workgroup per row.  Writes operand-ordered codes and the
// fp32 value of the fp16 scale to the workspace, and optionally the logical codes / fp16 scales.
__global__ __launch_bounds__(256) void act_quant_kernel(const uint16_t* __restrict__ x, int K,
                                                        int8_t* __restrict__ xq_op,
                                                        float* __restrict__ sx_f,
                                                        int8_t* __restrict__ xq_out,
                                                        uint16_t* __restrict__ sx_out) {
  __shared__ float red[4];
  __shared__ float s_sh;
  const int m = blockIdx.x;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)m * K);
  const int nb = K / 8;
  float mx = 0.0f;
  for (int i = threadIdx.x; i < nb; i += 256) {
    const uint4 v = xr[i];
    const uint16_t* h = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
    for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(h2f(h[e])));
  }
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const uint16_t s16 = f2h(amax / 7.0f);
    s_sh = h2f(s16);
    sx_f[m] = s_sh;
    if (sx_out) sx_out[m] = s16;
  }
  __syncthreads();
  const float s = s_sh;
  for (int i = threadIdx.x; i < nb; i += 256) {
    uint2 op, lg;
    quant_block8(xr[i], s, op, lg);
    *reinterpret_cast<uint2*>(xq_op + (size_t)m * K + 8 * i) = op;
    if (xq_out) *reinterpret_cast<uint2*>(xq_out + (size_t)m * K + 8 * i) = lg;
  }
}

// ------------------------------------------------------------------ streaming linear

enum { MODE_W4A16 = 0, MODE_W4A4 = 1 };
constexpr int kNW = 8;        // waves per workgroup
constexpr int kThreads = kNW * 64;
constexpr int kPF = 8;        // tiles in flight per wave

struct LinearArgs {
  const uint16_t* x;   // fp16 [M][K]
  const int8_t* xq;    // W4A4 with separate quantizer: operand-ordered codes [M][K]
  const float* sxf;    // W4A4 with separate quantizer: scales (fp32 value of fp16) [M]
  const uint4* w;      // packed tiles
  const uint16_t* sc;  // packed scales
  float* y;            // [M][N]
  int32_t* acc_out;    // optional [M][N][G]
  int8_t* xq_out;      // optional logical codes (fused quantizer, written by block 0)
  uint16_t* sx_out;    // optional fp16 scales (fused quantizer, written by block 0)
  int M, N, K;
};

// MODE: MODE_W4A16 / MODE_W4A4.  MT: 16-row activation tiles per wave (M <= 16 MT).
// S: waves splitting K.  XLDS: activations staged in LDS (W4A4: quantized in the prologue).
template <int MODE, int MT, int S, bool XLDS>
__global__ __launch_bounds__(kThreads) void linear_stream_kernel(LinearArgs a) {
  constexpr int R = kNW / S;
  extern __shared__ __align__(16) unsigned char dyn_lds[];
  __shared__ float4_t red[S > 1 ? kNW : 1][64];
  __shared__ float sx_lds[16];
  __shared__ float amax_red[8][kNW];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = wave / S, sidx = wave % S;
  const int M = a.M, N = a.N, K = a.K;
  const int G = K / kGroup;
  const int nrb = (N + 15) / 16;
  const int nsets = (nrb + R - 1) / R;
  const int per = (G + S - 1) / S;            // uniform item count per set for every wave
  const int g0 = sidx * per;
  const int my_sets = blockIdx.x < (unsigned)nsets ? (nsets - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
  const int total = my_sets * per;

  // ---- item -> (row block, group) and the prefetch ring
  uint4 buf[kPF];
  uint16_t sbuf[kPF];
  auto item_tile = [&](int it, int& rb, int& g) -> bool {
    const int si = it / per, gi = it - si * per;
    const int set = (int)blockIdx.x + si * (int)gridDim.x;
    rb = set * R + r;
    g = g0 + gi;
    return rb < nrb && g < G;
  };
  auto issue = [&](int it, int slot) {
    int rb, g;
    if (it < total && item_tile(it, rb, g)) {
      const size_t tile = (size_t)rb * G + g;
      buf[slot] = a.w[tile * 64 + lane];
      sbuf[slot] = a.sc[tile * 16 + (lane & 15)];
    }
  };
#pragma unroll
  for (int i = 0; i < kPF; ++i) issue(i, i);

  // ---- prologue: stage activations
  if constexpr (XLDS) {
    if constexpr (MODE == MODE_W4A16) {
      const uint4* src = reinterpret_cast<const uint4*>(a.x);
      uint4* dst = reinterpret_cast<uint4*>(dyn_lds);
      const int n16 = M * K / 8;
      for (int i = threadIdx.x; i < n16; i += kThreads) dst[i] = src[i];
    } else {
      const int nb = K / 8;
      for (int m = 0; m < M; ++m) {
        const uint4* xr = reinterpret_cast<const uint4*>(a.x + (size_t)m * K);
        float mx = 0.0f;
        for (int i = threadIdx.x; i < nb; i += kThreads) {
          const uint4 v = xr[i];
          const uint16_t* h = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
          for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(h2f(h[e])));
        }
        mx = wave_max(mx);
        if (lane == 0) amax_red[m][wave] = mx;
      }
      __syncthreads();
      if (threadIdx.x < M) {
        float amax = 0.0f;
#pragma unroll
        for (int w = 0; w < kNW; ++w) amax = fmaxf(amax, amax_red[threadIdx.x][w]);
        const uint16_t s16 = f2h(amax / 7.0f);
        sx_lds[threadIdx.x] = h2f(s16);
        if (blockIdx.x == 0 && a.sx_out) a.sx_out[threadIdx.x] = s16;
      }
      __syncthreads();
      int8_t* xq_lds = reinterpret_cast<int8_t*>(dyn_lds);
      for (int m = 0; m < M; ++m) {
        const uint4* xr = reinterpret_cast<const uint4*>(a.x + (size_t)m * K);
        const float s = sx_lds[m];
        for (int i = threadIdx.x; i < nb; i += kThreads) {
          uint2 op, lg;
          quant_block8(xr[i], s, op, lg);
          *reinterpret_cast<uint2*>(xq_lds + (size_t)m * K + 8 * i) = op;
          if (blockIdx.x == 0 && a.xq_out)
            *reinterpret_cast<uint2*>(a.xq_out + (size_t)m * K + 8 * i) = lg;
        }
      }
    }
    __syncthreads();
  }

  float4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = float4_t{0.f, 0.f, 0.f, 0.f};

  const int arow = lane & 15;      // A-operand row (activation row within a 16-row tile)
  const int kq = 32 * (lane >> 4);  // lane's k offset inside a group

  for (int base = 0; base < total; base += kPF) {
#pragma unroll
    for (int i = 0; i < kPF; ++i) {
      const int it = base + i;
      if (it < total) {
        int rb, g;
        const bool valid = item_tile(it, rb, g);
        const uint4 wv = buf[i];
        const float s = h2f(sbuf[i]);
        issue(it + kPF, i);
        if (valid) {
          const int kb = g * kGroup + kq;
          if constexpr (MODE == MODE_W4A16) {
            float4_t dg[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) dg[mt] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const uint32_t wt = t == 0 ? wv.x : t == 1 ? wv.y : t == 2 ? wv.z : wv.w;
              const half8_t b = unpack_f16x8(wt);
#pragma unroll
              for (int mt = 0; mt < MT; ++mt) {
                const int m = mt * 16 + arow;
                half8_t av = {};
                if (m < M) {
                  if constexpr (XLDS)
                    av = *reinterpret_cast<const half8_t*>(
                        reinterpret_cast<const _Float16*>(dyn_lds) + (size_t)m * K + kb + 8 * t);
                  else
                    av = *reinterpret_cast<const half8_t*>(
                        reinterpret_cast<const _Float16*>(a.x) + (size_t)m * K + kb + 8 * t);
                }
                dg[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, b, dg[mt], 0, 0, 0);
              }
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] += s * dg[mt];
          } else {
            int4_t dg[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) dg[mt] = int4_t{0, 0, 0, 0};
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
              const int4_t b = t2 == 0 ? unpack_i8x16(wv.x, wv.y) : unpack_i8x16(wv.z, wv.w);
#pragma unroll
              for (int mt = 0; mt < MT; ++mt) {
                const int m = mt * 16 + arow;
                int4_t av = {0, 0, 0, 0};
                if (m < M) {
                  const int8_t* src = XLDS ? reinterpret_cast<const int8_t*>(dyn_lds) : a.xq;
                  av = *reinterpret_cast<const int4_t*>(src + (size_t)m * K + kb + 16 * t2);
                }
                dg[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, b, dg[mt], 0, 0, 0);
              }
            }
            const int n = rb * 16 + (lane & 15);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const int gsum = dg[mt][j] >> 4;  // operands carry 16 * q: exact
                acc[mt][j] += s * (float)gsum;
                if (a.acc_out) {
                  const int m = mt * 16 + 4 * (lane >> 4) + j;
                  if (m < M && n < N) a.acc_out[((size_t)m * N + n) * G + g] = gsum;
                }
              }
            }
          }
        }
        // ---- end of this wave's share of a row-block set: reduce over S and store
        if (it - (it / per) * per == per - 1) {
          int rb2, g2;
          item_tile(it - (per - 1), rb2, g2);  // row block of this set (independent of g)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            float4_t v = acc[mt];
            if constexpr (S > 1) {
              red[wave][lane] = v;
              __syncthreads();
              if (sidx == 0) {
#pragma unroll
                for (int s2 = 1; s2 < S; ++s2) v += red[wave + s2][lane];
              }
              __syncthreads();
            }
            if (sidx == 0 && rb2 < nrb) {
              const int n = rb2 * 16 + (lane & 15);
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const int m = mt * 16 + 4 * (lane >> 4) + j;
                if (m < M && n < N) {
                  float out = v[j];
                  if constexpr (MODE == MODE_W4A4) out *= XLDS ? sx_lds[m] : a.sxf[m];
                  a.y[(size_t)m * N + n] = out;
                }
              }
            }
          }
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[mt] = float4_t{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
  }
}

// ------------------------------------------------------------------ launch selection

constexpr int kFusedMaxM = 8;            // W4A4: quantize inside the GEMM up to this many rows
constexpr size_t kMaxLdsStage = 131072;  // bytes of activations staged in LDS

static bool w4a4_fused(int M, int K) { return M <= kFusedMaxM && (size_t)M * K <= kMaxLdsStage; }
static bool w4a16_lds(int M, int K) { return M <= 4 && (size_t)M * K * 2 <= kMaxLdsStage; }

size_t linear_workspace(int mode, int M, int N, int K) {
  (void)N;
  if (mode != QS_W4A4 || w4a4_fused(M, K)) return 0;
  return align_up((size_t)M * K, 256) + align_up((size_t)M * 4, 256);
}

template <int MODE, int MT, int S, bool XLDS>
static int launch_one(const LinearArgs& a, size_t lds, hipStream_t st) {
  auto fn = linear_stream_kernel<MODE, MT, S, XLDS>;
  const DeviceInfo* di = device_info();
  const int nrb = (a.N + 15) / 16;
  const int R = kNW / S;
  const int nsets = (nrb + R - 1) / R;
  const int per_cu = lds > 65536 ? 1 : 2;
  const int grid = nsets < di->num_cus * per_cu ? nsets : di->num_cus * per_cu;
  if (lds > 65536) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return QS_ERR_HIP;
  }
  hipLaunchKernelGGL(fn, dim3(grid), dim3(kThreads), lds, st, a);
  return launch_status();
}

// Choose how many waves split K: enough waves to cover the chip, at least 2 groups per wave.
static int pick_split(int N, int K) {
  const int nrb = (N + 15) / 16;
  const int G = K / kGroup;
  int s = 1;
  while (s < 8 && nrb * s < 4096 && G / (2 * s) >= 2) s *= 2;
  return s;
}

template <int MODE, int MT, bool XLDS>
static int launch_split(const LinearArgs& a, size_t lds, hipStream_t st) {
  switch (pick_split(a.N, a.K)) {
    case 1: return launch_one<MODE, MT, 1, XLDS>(a, lds, st);
    case 2: return launch_one<MODE, MT, 2, XLDS>(a, lds, st);
    case 4: return launch_one<MODE, MT, 4, XLDS>(a, lds, st);
    default: return launch_one<MODE, MT, 8, XLDS>(a, lds, st);
  }
}

// Activation rows per launch of the streaming kernel (larger M is processed in chunks).
constexpr int kMaxRowsPerLaunch = 128;

template <int MODE>
static int launch_mt(const LinearArgs& a, hipStream_t st) {
  const int mt = (a.M + 15) / 16;
  if (mt <= 1) return launch_split<MODE, 1, false>(a, 0, st);
  if (mt <= 2) return launch_split<MODE, 2, false>(a, 0, st);
  if (mt <= 4) return launch_split<MODE, 4, false>(a, 0, st);
  return launch_split<MODE, 8, false>(a, 0, st);
}

// Rows [m0, m0 + rows) of a linear without LDS staging.
template <int MODE>
static int launch_rows(LinearArgs a, int m0, int rows, hipStream_t st) {
  const int G = a.K / kGroup;
  a.M = rows;
  a.x = a.x ? a.x + (size_t)m0 * a.K : nullptr;
  a.xq = a.xq ? a.xq + (size_t)m0 * a.K : nullptr;
  a.sxf = a.sxf ? a.sxf + m0 : nullptr;
  a.y += (size_t)m0 * a.N;
  a.acc_out = a.acc_out ? a.acc_out + (size_t)m0 * a.N * G : nullptr;
  return launch_mt<MODE>(a, st);
}

template <int MODE>
static int launch_chunked(const LinearArgs& a, hipStream_t st) {
  for (int m0 = 0; m0 < a.M; m0 += kMaxRowsPerLaunch) {
    const int rows = a.M - m0 < kMaxRowsPerLaunch ? a.M - m0 : kMaxRowsPerLaunch;
    const int rc = launch_rows<MODE>(a, m0, rows, st);
    if (rc != QS_OK) return rc;
  }
  return QS_OK;
}

int launch_linear(int mode, const uint16_t* x, const uint8_t* wp, const uint16_t* sp, float* y,
                  int M, int N, int K, int8_t* xq_out, uint16_t* sx_out, int32_t* acc_out,
                  void* ws, size_t ws_bytes, hipStream_t st) {
  LinearArgs a{};
  a.x = x;
  a.w = reinterpret_cast<const uint4*>(wp);
  a.sc = sp;
  a.y = y;
  a.acc_out = acc_out;
  a.xq_out = xq_out;
  a.sx_out = sx_out;
  a.M = M;
  a.N = N;
  a.K = K;
  if (mode == QS_W4A16) {
    if (w4a16_lds(M, K)) return launch_split<MODE_W4A16, 1, true>(a, (size_t)M * K * 2, st);
    return launch_chunked<MODE_W4A16>(a, st);
  }
  if (w4a4_fused(M, K)) return launch_split<MODE_W4A4, 1, true>(a, (size_t)M * K, st);
  const size_t need = linear_workspace(mode, M, N, K);
  if (ws == nullptr || ws_bytes < need) return QS_ERR_WORKSPACE;
  int8_t* xq_op = static_cast<int8_t*>(ws);
  float* sxf = reinterpret_cast<float*>(static_cast<unsigned char*>(ws) + align_up((size_t)M * K, 256));
  hipLaunchKernelGGL(act_quant_kernel, dim3(M), dim3(256), 0, st, x, K, xq_op, sxf, xq_out, sx_out);
  const int rc = launch_status();
  if (rc != QS_OK) return rc;
  a.xq = xq_op;
  a.sxf = sxf;
  a.xq_out = nullptr;
  a.sx_out = nullptr;
  return launch_chunked<MODE_W4A4>(a, st);
}

}  // namespace qs
