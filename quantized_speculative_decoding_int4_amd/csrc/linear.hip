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
//                   group sums, scaled and summed in fp64 (exact) and rounded
//                   once to the fp32 output.  gfx950 has no int4 MFMA.
//
// At decode sizes (M <= 16 rows) the kernel is a weight stream: each 64-lane
// wave pulls whole 1 KiB tiles (one 16 B global_load_dwordx4 per lane, 1 KiB
// per wave instruction, fully coalesced) through a ring of PF outstanding
// tiles, expands nibbles in VGPRs and feeds the tile straight into the MFMA as
// its B operand; activations sit in LDS (or, for large M, are read from L2).
// A workgroup of 8 waves covers R = 8 / S row blocks, S waves splitting K, and
// reduces the S partials through LDS in a fixed order (deterministic).

#include "qs_act.h"
#include "qs_device.h"
#include "qs_internal.h"

#include <type_traits>

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

// Stand-alone quantizer (INT4 codes for W4A4, QMAX = 7; INT8 codes for W4A8, QMAX = 127): one
// workgroup of kAqThreads per row (wide, so the serial statistics and quantization of one row
// are short).  Writes operand-ordered codes and the fp32 value of the fp16 scale to the workspace,
// and optionally the logical codes / fp16 scales.
constexpr int kAqThreads = 1024;
template <int QMAX>
__global__ __launch_bounds__(kAqThreads) void act_quant_kernel(const uint16_t* __restrict__ x, int K, int ldx,
                                                               int norm_in, int8_t* __restrict__ xq_op,
                                                               float* __restrict__ sx_f,
                                                               int8_t* __restrict__ xq_out,
                                                               uint16_t* __restrict__ sx_out) {
  constexpr int kW = kAqThreads / 64;
  __shared__ double red64[2][kW];
  __shared__ float red[2][kW];
  __shared__ float s_sh;
  __shared__ double mu_sh, inv_sh;
  const int m = blockIdx.x;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)m * ldx);
  const int nb = K / 8;
  double sum = 0.0, sq = 0.0;
  float mx = -INFINITY, mn = INFINITY;
  for (int i = threadIdx.x; i < nb; i += kAqThreads) stats_block8_64(xr[i], sum, sq, mx, mn);
  sum = wave_sum_dpp64(sum);
  sq = wave_sum_dpp64(sq);
  mx = wave_max_dpp(mx);
  mn = wave_min_dpp(mn);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { red64[0][w] = sum; red64[1][w] = sq; red[0][w] = mx; red[1][w] = mn; }
  __syncthreads();
  if (threadIdx.x == 0) {
    double tsum = red64[0][0], tsq = red64[1][0];
    float xmax = red[0][0], xmin = red[1][0];
    for (int j = 1; j < kW; ++j) {  // fixed order
      tsum += red64[0][j];
      tsq += red64[1][j];
      xmax = fmaxf(xmax, red[0][j]);
      xmin = fminf(xmin, red[1][j]);
    }
    double mu = 0.0, inv = 0.0;
    float amax;
    if (norm_in) {
      norm_params64(tsum, tsq, xmax, xmin, K, mu, inv);
      amax = fmaxf(h2f(norm_h64(xmax, mu, inv)), -h2f(norm_h64(xmin, mu, inv)));
    } else {
      amax = fmaxf(xmax, -xmin);
    }
    const uint16_t s16 = f2h(amax / (float)QMAX);
    s_sh = h2f(s16);
    mu_sh = mu;
    inv_sh = inv;
    sx_f[m] = s_sh;
    if (sx_out) sx_out[m] = s16;
  }
  __syncthreads();
  const float s = s_sh;
  for (int i = threadIdx.x; i < nb; i += kAqThreads) {
    uint2 op, lg;
    uint4 v = xr[i];
    if (norm_in) v = norm_block8_64(v, mu_sh, inv_sh);
    quant_block8<QMAX>(v, s, op, lg);
    *reinterpret_cast<uint2*>(xq_op + (size_t)m * K + 8 * i) = op;
    if (xq_out) *reinterpret_cast<uint2*>(xq_out + (size_t)m * K + 8 * i) = lg;
  }
}

// ------------------------------------------------------------------ streaming linear

enum { MODE_W4A16 = 0, MODE_W4A4 = 1 };
#ifndef QS_STREAM_WAVES
#define QS_STREAM_WAVES 8
#endif
#ifndef QS_STREAM_RING
#define QS_STREAM_RING 8
#endif
#ifndef QS_STREAM_WG_PER_CU
#define QS_STREAM_WG_PER_CU 2
#endif
constexpr int kNW = QS_STREAM_WAVES;   // waves per workgroup
constexpr int kThreads = kNW * 64;
constexpr int kPF = QS_STREAM_RING;    // tiles in flight per wave

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
  uint16_t* y16;       // if set: write fp16(y) here (row stride ldy) instead of y
  int M, N, K;
  int ldx;             // row stride of x (elements), >= K
  int ldy;             // row stride of y16 (elements)
  int norm_in;         // standardise each input row over its K columns first (chain stages > 0)
};

// MODE: MODE_W4A16 / MODE_W4A4.  MT: 16-row activation tiles per wave (M <= 16 MT).
// S: waves splitting K.  XLDS: activations staged in LDS (W4A4: quantized in the prologue).
//
// Work of one wave: for each row-block set handled by its workgroup, `per` consecutive 1 KiB tiles
// of its row block (its share of K).  The wave walks this stream with a ring of kPF outstanding
// tile loads that runs across set boundaries; the stream is padded to whole rings with dummy items
// that re-read an already cached tile and are not computed, so every load is unconditional and the
// compiler can wait for exactly the oldest outstanding tile.  All control flow is wave-uniform.
template <int MODE, int MT, int S, bool XLDS>
__global__ __launch_bounds__(kThreads) void linear_stream_kernel(LinearArgs a) {
  constexpr int R = kNW / S;
  // W4A16 accumulates in fp32; the integer modes scale their exact i32 group sums in fp64 (exact).
  using Acc = std::conditional_t<MODE == MODE_W4A16, float4_t, double4_t>;
  extern __shared__ __align__(16) unsigned char dyn_lds[];
  __shared__ Acc red[S > 1 ? kNW : 1][64];
  __shared__ float sx_lds[16];     // W4A4: row scales; W4A16 with norm_in: row mean [0, 8), 1/std [8, 16)
  __shared__ float amax_red[8][kNW];
  __shared__ double row64[2][8];   // W4A4 with norm_in: row mean, 1/std (fp64)
  __shared__ __align__(16) uint32_t zero_pad[16];  // A-operand source for lanes beyond M
  __shared__ __align__(16) uint32_t ones_pad[16];  // W4A16 with norm_in: fp16 1.0 pairs (row sums of W)

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int r = wave / S, sidx = wave - (wave / S) * S;
  const int M = a.M, N = a.N, K = a.K;
  const int G = K / kGroup;
  const int nrb = (N + 15) / 16;
  const int nsets = (nrb + R - 1) / R;
  const int per = (G + S - 1) / S;           // uniform item count per set for every wave
  const int g0 = sidx * per;
  const int gcnt = G - g0 < per ? G - g0 : per;  // valid groups of this wave (may be <= 0)
  const int grid = (int)gridDim.x, bid = (int)blockIdx.x;
  const int my_sets = bid < nsets ? (nsets - 1 - bid) / grid + 1 : 0;
  const int total = (my_sets * per + kPF - 1) / kPF * kPF;  // padded to whole rings
  const size_t set_stride = (size_t)grid * R * G;              // tiles between consecutive sets

  if (threadIdx.x < 16) {
    zero_pad[threadIdx.x] = 0u;
    ones_pad[threadIdx.x] = 0x3C003C00u;
  }

  // ---- load cursor (scalar): set index, item within set, tile index
  int l_gi = 0, l_si = 0;
  size_t l_tile = (size_t)(bid * R + r) * G + g0;
  const uint4* __restrict__ wbase = a.w + lane;
  const uint16_t* __restrict__ sbase = a.sc + (lane & 15);
  uint4 buf[kPF];
  uint16_t sbuf[kPF];
  auto issue = [&](int slot) {
    const int rb = (bid + l_si * grid) * R + r;
    const bool ok = l_si < my_sets && rb < nrb && l_gi < gcnt;
    const size_t t = ok ? l_tile : 0;   // dummy items re-read tile 0
    buf[slot] = wbase[t * 64];
    sbuf[slot] = sbase[t * 16];
    ++l_tile;
    if (++l_gi == per) { l_gi = 0; ++l_si; l_tile += set_stride - per; }
  };
#pragma unroll
  for (int i = 0; i < kPF; ++i) issue(i);

  // ---- prologue: stage activations
  if constexpr (XLDS) {
    if constexpr (MODE == MODE_W4A16) {
      uint4* dst = reinterpret_cast<uint4*>(dyn_lds);
      const int per_row = K / 8;
      const int n16 = M * per_row;
      float rs[4] = {0.f, 0.f, 0.f, 0.f}, rq[4] = {0.f, 0.f, 0.f, 0.f};
      for (int i = threadIdx.x; i < n16; i += kThreads) {
        const int m = i / per_row, j = i - m * per_row;
        const uint4 v = *reinterpret_cast<const uint4*>(a.x + (size_t)m * a.ldx + 8 * j);
        dst[i] = v;
        if (a.norm_in) {
          float su = 0.f, sq = 0.f, mx = 0.f, mn = 0.f;
          stats_block8(v, su, sq, mx, mn);
#pragma unroll
          for (int r2 = 0; r2 < 4; ++r2)
            if (m == r2) { rs[r2] += su; rq[r2] += sq; }
        }
      }
      if (a.norm_in) {
#pragma unroll
        for (int r2 = 0; r2 < 4; ++r2) {
          const float su = wave_sum(rs[r2]), sq = wave_sum(rq[r2]);
          if (lane == 0) { amax_red[r2][wave] = su; amax_red[4 + r2][wave] = sq; }
        }
        __syncthreads();
        if (threadIdx.x < M) {  // applied in the epilogue: (sum_k x w - mu sum_k w) * inv
          float su = 0.f, sq = 0.f;
#pragma unroll
          for (int w = 0; w < kNW; ++w) { su += amax_red[threadIdx.x][w]; sq += amax_red[4 + threadIdx.x][w]; }
          float mu, inv;
          norm_params(su, sq, K, mu, inv);
          sx_lds[threadIdx.x] = mu;
          sx_lds[8 + threadIdx.x] = inv;
        }
      }
    } else {
      const int nb = K / 8;
      __shared__ double stat_sum[2][8][kNW];
      __shared__ float stat_mm[2][8][kNW];
      for (int m = 0; m < M; ++m) {
        const uint4* xr = reinterpret_cast<const uint4*>(a.x + (size_t)m * a.ldx);
        double su = 0.0, sq = 0.0;
        float mx = -INFINITY, mn = INFINITY;
        for (int i = threadIdx.x; i < nb; i += kThreads) stats_block8_64(xr[i], su, sq, mx, mn);
        su = wave_sum_dpp64(su);
        sq = wave_sum_dpp64(sq);
        mx = wave_max(mx);
        mn = wave_min(mn);
        if (lane == 0) {
          stat_sum[0][m][wave] = su;
          stat_sum[1][m][wave] = sq;
          stat_mm[0][m][wave] = mx;
          stat_mm[1][m][wave] = mn;
        }
      }
      __syncthreads();
      if (threadIdx.x < M) {
        const int m = threadIdx.x;
        double su = 0.0, sq = 0.0;
        float xmax = -INFINITY, xmin = INFINITY;
#pragma unroll
        for (int w = 0; w < kNW; ++w) {
          su += stat_sum[0][m][w];
          sq += stat_sum[1][m][w];
          xmax = fmaxf(xmax, stat_mm[0][m][w]);
          xmin = fminf(xmin, stat_mm[1][m][w]);
        }
        double mu = 0.0, inv = 0.0;
        float amax;
        if (a.norm_in) {
          norm_params64(su, sq, xmax, xmin, K, mu, inv);
          amax = fmaxf(h2f(norm_h64(xmax, mu, inv)), -h2f(norm_h64(xmin, mu, inv)));
        } else {
          amax = fmaxf(xmax, -xmin);
        }
        const uint16_t s16 = f2h(amax / 7.0f);
        sx_lds[m] = h2f(s16);
        row64[0][m] = mu;
        row64[1][m] = inv;
        if (blockIdx.x == 0 && a.sx_out) a.sx_out[m] = s16;
      }
      __syncthreads();
      int8_t* xq_lds = reinterpret_cast<int8_t*>(dyn_lds);
      for (int m = 0; m < M; ++m) {
        const uint4* xr = reinterpret_cast<const uint4*>(a.x + (size_t)m * a.ldx);
        const float s = sx_lds[m];
        const double mu = row64[0][m], inv = row64[1][m];
        for (int i = threadIdx.x; i < nb; i += kThreads) {
          uint2 op, lg;
          uint4 v = xr[i];
          if (a.norm_in) v = norm_block8_64(v, mu, inv);
          quant_block8(v, s, op, lg);
          *reinterpret_cast<uint2*>(xq_lds + (size_t)m * K + 8 * i) = op;
          if (blockIdx.x == 0 && a.xq_out)
            *reinterpret_cast<uint2*>(a.xq_out + (size_t)m * K + 8 * i) = lg;
        }
      }
    }
  }
  __syncthreads();

  Acc acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = Acc{0, 0, 0, 0};

  const int arow = lane & 15;       // A-operand row (activation row within a 16-row tile)
  const int kq = 32 * (lane >> 4);  // lane's k offset inside a group
  // LDS byte address of this lane's A operand at group 0 (or the zero pad for rows beyond M).
  const uint32_t zero_addr = (uint32_t)(uintptr_t)zero_pad;
  const uint32_t lds_base = (uint32_t)(uintptr_t)dyn_lds;
  constexpr int kElt = MODE == MODE_W4A16 ? 2 : 1;  // bytes per staged activation element
  // W4A16 with norm_in: operand row M reads all-ones, so output row M is sum_k w[n, k] (M <= 4 here)
  const bool ones_row = MODE == MODE_W4A16 && XLDS && a.norm_in && arow == M;
  const uint32_t a_lane = arow < M ? lds_base + (uint32_t)((arow * K + kq) * kElt)
                                   : ones_row ? (uint32_t)(uintptr_t)ones_pad : zero_addr;
  const uint32_t a_step = arow < M ? (uint32_t)(kGroup * kElt) : 0u;  // per group

  const uint32_t magic = fp16_magic_vgpr();
  int c_gi = 0, c_si = 0;
  for (int base = 0; base < total; base += kPF) {
#pragma unroll
    for (int i = 0; i < kPF; ++i) {
      const uint4 wv = buf[i];
      const float s = h2f(sbuf[i]);
      issue(i);
      const int rb = (bid + c_si * grid) * R + r;
      const bool valid = c_si < my_sets && rb < nrb && c_gi < gcnt;
      if (valid) {
        const int g = g0 + c_gi;
        const int kb = g * kGroup + kq;
        if constexpr (MODE == MODE_W4A16) {
          float4_t dg[MT];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) dg[mt] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint32_t wt = t == 0 ? wv.x : t == 1 ? wv.y : t == 2 ? wv.z : wv.w;
            const half8_t b = unpack_f16x8(wt, magic);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              half8_t av;
              if constexpr (XLDS) {
                const uint32_t addr = a_lane + (uint32_t)g * a_step + 16u * t;
                av = *reinterpret_cast<const __attribute__((address_space(3))) half8_t*>(
                    (size_t)addr);
              } else {
                const int m = mt * 16 + arow;
                av = half8_t{};
                if (m < M)
                  av = *reinterpret_cast<const half8_t*>(
                      reinterpret_cast<const _Float16*>(a.x) + (size_t)m * a.ldx + kb + 8 * t);
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
              int4_t av;
              if constexpr (XLDS) {
                const uint32_t addr = a_lane + (uint32_t)g * a_step + 16u * t2;
                av = *reinterpret_cast<const __attribute__((address_space(3))) int4_t*>((size_t)addr);
              } else {
                const int m = mt * 16 + arow;
                av = int4_t{0, 0, 0, 0};
                if (m < M) av = *reinterpret_cast<const int4_t*>(a.xq + (size_t)m * K + kb + 16 * t2);
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
              acc[mt][j] += (double)s * (double)gsum;  // exact in fp64
              if (a.acc_out) {
                const int m = mt * 16 + 4 * (lane >> 4) + j;
                if (m < M && n < N) a.acc_out[((size_t)m * N + n) * G + g] = gsum;
              }
            }
          }
        }
      }
      // ---- end of this wave's share of a row-block set: reduce over S and store
      if (++c_gi == per) {
        c_gi = 0;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          Acc v = acc[mt];
          if constexpr (S > 1) {
            red[wave][lane] = v;
            __syncthreads();
            if (sidx == 0) {
#pragma unroll
              for (int s2 = 1; s2 < S; ++s2) v += red[wave + s2][lane];
            }
            __syncthreads();
          }
          if (sidx == 0 && c_si < my_sets && rb < nrb) {
            const int n = rb * 16 + (lane & 15);
            float rowsum = 0.f;  // W4A16 with norm_in: sum_k w[n, k] from operand row M
            if constexpr (MODE == MODE_W4A16 && XLDS) {
              if (a.norm_in) {
                const int q = M & 3;
                const float vq = q == 0 ? v[0] : q == 1 ? v[1] : q == 2 ? v[2] : v[3];
                rowsum = __shfl(vq, (lane & 15) + 16 * (M >> 2), 64);
              }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int m = mt * 16 + 4 * (lane >> 4) + j;
              if (m < M && n < N) {
                float out;
                uint16_t h;
                if constexpr (MODE == MODE_W4A4) {  // exact product, rounded once
                  const double o64 = v[j] * (double)(XLDS ? sx_lds[m] : a.sxf[m]);
                  out = (float)o64;
                  h = f64_to_f16_rn(o64);
                } else {
                  out = v[j];
                  if constexpr (XLDS) {
                    if (a.norm_in) out = (out - sx_lds[m] * rowsum) * sx_lds[8 + m];
                  }
                  h = f2h(out);
                }
                if (a.y16) a.y16[(size_t)m * a.ldy + n] = h;
                else a.y[(size_t)m * N + n] = out;
              }
            }
          }
          acc[mt] = Acc{0, 0, 0, 0};
        }
        ++c_si;
      }
    }
  }
}

// ------------------------------------------------------------------ launch selection

constexpr int kFusedMaxM = 8;            // W4A4: quantize inside the GEMM up to this many rows
constexpr size_t kMaxLdsStage = 131072;  // bytes of activations staged in LDS

static bool w4a4_fused(int M, int K) { return M <= kFusedMaxM && (size_t)M * K <= kMaxLdsStage; }
static bool w4a16_lds(int M, int K) { return M <= 4 && (size_t)M * K * 2 <= kMaxLdsStage; }

// From this many rows on (and without the per-group accumulator output) a linear runs as the
// register-tiled batched kernel of gemm.hip instead of the streaming kernel: above the rows the
// LDS-staged streaming kernel takes (W4A16, up to 4) or the single-row fused one (W4A4).  Measured
// on the Llama-3-8B-shaped stack, the batched kernel's 16-row tile is faster from these row counts
// on (M = 6 and 8: 2.3 instead of 2.7-2.9 ms per W4A16 pass; W4A4 M = 4: 2.8 instead of 2.8-4.2).
static int gemm_min_rows(int mode) { return mode == QS_W4A16 ? 5 : mode == QS_W4A4 ? 2 : 1; }
static bool use_gemm(int mode, int M, const int32_t* acc_out) {
  return M >= gemm_min_rows(mode) && acc_out == nullptr;
}

// Scratch of one linear: the standardised (W4A16) or quantized (W4A4) activations when they are
// staged in memory, then the K-split partials of the batched kernel.  Sized for the case without
// the per-group accumulator output (it only ever makes the need smaller).
static size_t staging_bytes(int mode, int M, int K, bool norm_in) {
  (void)norm_in;
  if (mode == QS_W4A16) return 0;  // both W4A16 kernels standardise in their epilogue
  if (mode == QS_W4A4 && w4a4_fused(M, K) && !use_gemm(mode, M, nullptr)) return 0;
  return align_up((size_t)M * K, 256) + align_up((size_t)M * 4, 256);
}

// Layout of a linear's workspace: [K-split arrival counters (batched kernel)] [staging] [K-split
// partial slots].  The counters come first so that every linear of a chain finds them at the same
// place: they are cleared once per chain call and every batched launch leaves them at zero.
static size_t counter_bytes(int mode, int M) { return use_gemm(mode, M, nullptr) ? gemm_counter_bytes() : 0; }

size_t linear_workspace(int mode, int M, int N, int K, bool norm_in) {
  const size_t stage = staging_bytes(mode, M, K, norm_in);
  return counter_bytes(mode, M) + stage + (use_gemm(mode, M, nullptr) ? gemm_workspace(mode, M, N, K) : 0);
}

int linear_clear_counters(int mode, int M, void* ws, hipStream_t st) {
  if (counter_bytes(mode, M) == 0) return QS_OK;
  return launch_gemm_clear(static_cast<unsigned*>(ws), st);
}

template <int MODE, int MT, int S, bool XLDS>
static int launch_one(const LinearArgs& a, size_t lds, hipStream_t st) {
  auto fn = linear_stream_kernel<MODE, MT, S, XLDS>;
  const DeviceInfo* di = device_info();
  const int nrb = (a.N + 15) / 16;
  const int R = kNW / S;
  const int nsets = (nrb + R - 1) / R;
  const int per_cu = lds > 65536 ? 1 : QS_STREAM_WG_PER_CU;
  const int grid = nsets < di->num_cus * per_cu ? nsets : di->num_cus * per_cu;
  if (lds > 65536) {
    // Raise the dynamic-LDS limit once per instance (before any graph capture uses it).
    static int lds_limit = 0;
    if ((int)lds > lds_limit) {
      if (hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kMaxLdsStage) != hipSuccess) {
        (void)hipGetLastError();  // report it here, not at the caller's next HIP call
        return QS_ERR_HIP;
      }
      lds_limit = (int)kMaxLdsStage;
    }
  }
  hipLaunchKernelGGL(fn, dim3(grid), dim3(kThreads), lds, st, a);
  return launch_status();
}

// Choose how many waves split K: enough waves to cover the chip, at least 2 groups per wave.
static int pick_split(int N, int K) {
  const int nrb = (N + 15) / 16;
  const int G = K / kGroup;
  int s = 1;
  while (s < 8 && s < kNW && nrb * s < 4096 && G / (2 * s) >= 2) s *= 2;
  return s;
}

template <int MODE, int MT, bool XLDS>
static int launch_split(const LinearArgs& a, size_t lds, hipStream_t st) {
  switch (pick_split(a.N, a.K)) {
    case 1: return launch_one<MODE, MT, 1, XLDS>(a, lds, st);
    case 2: return launch_one<MODE, MT, 2, XLDS>(a, lds, st);
    case 4:
      if constexpr (kNW >= 4) return launch_one<MODE, MT, 4, XLDS>(a, lds, st);
      return QS_ERR_UNSUPPORTED;
    default:
      if constexpr (kNW >= 8) return launch_one<MODE, MT, 8, XLDS>(a, lds, st);
      return QS_ERR_UNSUPPORTED;
  }
}

// Activation rows per launch of the streaming kernel (larger M is processed in chunks; 128-row
// launches would not fit the registers).
constexpr int kMaxRowsPerLaunch = 64;

template <int MODE>
static int launch_mt(const LinearArgs& a, hipStream_t st) {
  const int mt = (a.M + 15) / 16;
  if (mt <= 1) return launch_split<MODE, 1, false>(a, 0, st);
  if (mt <= 2) return launch_split<MODE, 2, false>(a, 0, st);
  return launch_split<MODE, 4, false>(a, 0, st);
}

// Rows [m0, m0 + rows) of a linear without LDS staging.
template <int MODE>
static int launch_rows(LinearArgs a, int m0, int rows, hipStream_t st) {
  const int G = a.K / kGroup;
  a.M = rows;
  a.x = a.x ? a.x + (size_t)m0 * a.ldx : nullptr;
  a.xq = a.xq ? a.xq + (size_t)m0 * a.K : nullptr;
  a.sxf = a.sxf ? a.sxf + m0 : nullptr;
  if (a.y) a.y += (size_t)m0 * a.N;
  if (a.y16) a.y16 += (size_t)m0 * a.ldy;
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

// LM-head with the Top-1 epilogue: [counters (zero before the first call, left zero)] [INT4/INT8
// codes and scales for the integer modes] [K-split slots] [per-tile softmax-statistics partials].
static size_t top1_stage_bytes(int mode, int M, int K) {
  return mode == QS_W4A16 ? 0 : align_up((size_t)M * K, 256) + align_up((size_t)M * 4, 256);
}

size_t lmhead_top1_workspace(int mode, int M, int V, int K) {
  return gemm_counter_bytes() + top1_stage_bytes(mode, M, K) + gemm_workspace(mode, M, V, K) +
         gemm_top1_bytes(M, V);
}

int launch_lmhead_top1(int mode, const uint16_t* x, int ldx, int norm, const uint8_t* wp, const uint16_t* sp,
                       float* logits, int M, int V, int K, int32_t* top1, float* top1_prob, void* ws, hipStream_t st) {
  unsigned char* base = static_cast<unsigned char*>(ws);
  unsigned* cnt = reinterpret_cast<unsigned*>(base);
  unsigned char* stg = base + gemm_counter_bytes();
  unsigned char* slots = stg + top1_stage_bytes(mode, M, K);
  const size_t slot_bytes = gemm_workspace(mode, M, V, K);
  GemmTop1 t1{slots + slot_bytes, top1, top1_prob};
  if (mode == QS_W4A16)
    return launch_gemm(QS_W4A16, norm != 0, x, ldx, nullptr, nullptr, wp, sp, M, V, K, logits, nullptr, V, cnt,
                       slots, slot_bytes, st, &t1);
  int8_t* xq_op = reinterpret_cast<int8_t*>(stg);
  float* sxf = reinterpret_cast<float*>(stg + align_up((size_t)M * K, 256));
  if (mode == QS_W4A4)
    hipLaunchKernelGGL(act_quant_kernel<7>, dim3(M), dim3(kAqThreads), 0, st, x, K, ldx, norm, xq_op, sxf, nullptr,
                       nullptr);
  else
    hipLaunchKernelGGL(act_quant_kernel<127>, dim3(M), dim3(kAqThreads), 0, st, x, K, ldx, norm, xq_op, sxf, nullptr,
                       nullptr);
  const int rc = launch_status();
  if (rc != QS_OK) return rc;
  return launch_gemm(mode, false, nullptr, 0, xq_op, sxf, wp, sp, M, V, K, logits, nullptr, V, cnt, slots,
                     slot_bytes, st, &t1);
}

int launch_linear(int mode, const uint16_t* x, const uint8_t* wp, const uint16_t* sp, float* y,
                  int M, int N, int K, int8_t* xq_out, uint16_t* sx_out, int32_t* acc_out,
                  void* ws, size_t ws_bytes, hipStream_t st) {
  LinearIO io{};
  io.x = x;
  io.ldx = K;
  io.y = y;
  return launch_linear_io(mode, io, wp, sp, M, N, K, xq_out, sx_out, acc_out, ws, ws_bytes, st);
}

int launch_linear_io(int mode, const LinearIO& io, const uint8_t* wp, const uint16_t* sp, int M, int N,
                     int K, int8_t* xq_out, uint16_t* sx_out, int32_t* acc_out, void* ws,
                     size_t ws_bytes, hipStream_t st) {
  const uint16_t* x = io.x;
  LinearArgs a{};
  a.x = x;
  a.w = reinterpret_cast<const uint4*>(wp);
  a.sc = sp;
  a.y = io.y;
  a.y16 = io.y16;
  a.ldx = io.ldx;
  a.ldy = io.ldy;
  a.acc_out = acc_out;
  a.xq_out = xq_out;
  a.sx_out = sx_out;
  a.M = M;
  a.N = N;
  a.K = K;
  a.norm_in = io.norm_in;
  // the staging part is required; the batched kernel's split partials are optional (without them it
  // does not split K)
  const size_t pre = counter_bytes(mode, M);
  const size_t need = staging_bytes(mode, M, K, io.norm_in != 0);
  if (need > 0 && (ws == nullptr || ws_bytes < pre + need)) return QS_ERR_WORKSPACE;
  const bool gemm = use_gemm(mode, M, acc_out);
  unsigned char* stg = ws ? static_cast<unsigned char*>(ws) + pre : nullptr;
  unsigned* cnt = pre > 0 && ws != nullptr && ws_bytes >= pre ? static_cast<unsigned*>(ws) : nullptr;
  if (cnt && !io.counters_zero) {
    // counters of a workspace not known to be clear; only needed if the GEMM splits K
    if (gemm && gemm_workspace(mode, M, N, K) > 0 && ws_bytes >= pre + need + gemm_workspace(mode, M, N, K)) {
      const int rc = launch_gemm_clear(cnt, st);
      if (rc != QS_OK) return rc;
    }
  }
  void* gws = ws ? stg + need : nullptr;
  const size_t gws_bytes = ws && ws_bytes > pre + need ? ws_bytes - pre - need : 0;
  if (mode == QS_W4A16) {
    if (w4a16_lds(M, K)) return launch_split<MODE_W4A16, 1, true>(a, (size_t)M * K * 2, st);
    // the batched kernel also takes the standardised rows that do not fit the LDS stage (it
    // standardises in its epilogue; without a workspace it does not split K)
    if (gemm || io.norm_in)
      return launch_gemm(QS_W4A16, io.norm_in != 0, a.x, a.ldx, nullptr, nullptr, wp, sp, M, N, K, a.y, a.y16,
                         a.y16 ? a.ldy : N, cnt, gws, gws_bytes, st);
    return launch_chunked<MODE_W4A16>(a, st);
  }
  // W4A4 and W4A8 share the integer kernels: only the activation codes' range differs (the fused
  // quantization of the streaming kernel is INT4 only)
  if (mode == QS_W4A4 && w4a4_fused(M, K) && !gemm) return launch_split<MODE_W4A4, 1, true>(a, (size_t)M * K, st);
  int8_t* xq_op = reinterpret_cast<int8_t*>(stg);
  float* sxf = reinterpret_cast<float*>(stg + align_up((size_t)M * K, 256));
  if (mode == QS_W4A4)
    hipLaunchKernelGGL(act_quant_kernel<7>, dim3(M), dim3(kAqThreads), 0, st, x, K, io.ldx, io.norm_in, xq_op, sxf,
                       xq_out, sx_out);
  else
    hipLaunchKernelGGL(act_quant_kernel<127>, dim3(M), dim3(kAqThreads), 0, st, x, K, io.ldx, io.norm_in, xq_op, sxf,
                       xq_out, sx_out);
  const int rc = launch_status();
  if (rc != QS_OK) return rc;
  if (gemm)
    return launch_gemm(mode, false, nullptr, 0, xq_op, sxf, wp, sp, M, N, K, a.y, a.y16, a.y16 ? a.ldy : N,
                       cnt, gws, gws_bytes, st);
  a.xq = xq_op;
  a.sxf = sxf;
  a.xq_out = nullptr;
  a.sx_out = nullptr;
  return launch_chunked<MODE_W4A4>(a, st);
}

}  // namespace qs
