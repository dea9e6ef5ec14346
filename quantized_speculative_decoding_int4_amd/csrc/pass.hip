// Persistent pass kernel: one launch runs up to kMaxStages linears of a chain
// (the W4A4 draft pass at M = batch rows or the W4A16 verify pass at M = 4 rows,
// [P3] "draft modelとtarget modelの処理フロー"; modes from [P1] "QSpec の W4A4
// モードと W4A16 モード").
//
// Why persistent: at decode sizes a linear moves 2-60 MB of weights, so a
// stand-alone launch spends a large share of its time ramping up and draining
// (on MI355X a kernel that only reads 8 MB takes ~7 us).  Here one workgroup per
// compute unit stays resident for all stages.  Every wave owns a flattened
// stream of 1 KiB weight tiles across all stages of the launch and keeps a ring
// of kPRing tile loads in flight; weights do not depend on activations, so the
// ring runs ahead into the next stage while the workgroups wait at the grid
// barrier between stages and stage the next activations in LDS.  HBM keeps
// streaming through the dependency.
//
// Stage hand-over without cache maintenance: stage outputs are written with
// device-coherent stores (they bypass the per-XCD L2 on the way to memory) and
// read back with device-coherent loads, so neither side needs the L2 write-back
// and invalidate of an agent-scope release/acquire (measured at about 3.5 us per
// boundary on MI355X).  The grid barrier is a flag per workgroup gathered by
// workgroup 0, which then publishes a `go` word; every wait has a wall-clock
// deadline that sets an error word and makes the workgroup exit, so no wave can
// wait forever even if the workgroups were not all resident.
//
// Tile math per stage is the one of linear.hip: a wave's share of a 16-row block
// (S waves split K), expansion of the nibbles in VGPRs, MFMA with the staged
// activations as A operand, fp32 group scaling, fixed-order reduction over the
// S waves through LDS.
//
// W4A16 stages take the raw fp16 input and apply the row standardisation after
// the contraction: with mean mu and 1/std inv of input row m,
//   sum_k w[n,k] (x[m,k] - mu) inv = (sum_k w[n,k] x[m,k] - mu sum_k w[n,k]) inv,
// and sum_k w[n,k] comes for free from an all-ones row placed in the zero padding
// of the 16-row A operand.  The input therefore goes to LDS by direct DMA and its
// statistics are computed while the contraction runs.  This skips the fp16
// rounding of the standardised input (a relative 2^-12 per term).  W4A4 stages
// must quantise the standardised row first, so they stage through registers:
// statistics, scale, quantisation, then LDS.

#include "qs_act.h"
#include "qs_device.h"
#include "qs_internal.h"

#include <atomic>
#include <type_traits>

namespace qs {

// Compile-time loop: calls f(std::integral_constant<int, I>) for I = B..E-1, so ring slots are
// addressed with constant indices and stay in registers however long the ring is.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

#ifndef QS_PASS_STREAM_WAVES
#define QS_PASS_STREAM_WAVES 8
#endif
#ifndef QS_PASS_CTRL_WAVES
#define QS_PASS_CTRL_WAVES 8
#endif
#ifndef QS_PASS_RING
#define QS_PASS_RING 16
#endif
constexpr int kSW = QS_PASS_STREAM_WAVES;  // streaming waves: weight ring + MFMA (split S x R)
constexpr int kCW = QS_PASS_CTRL_WAVES;    // control waves: reductions, stores, barriers, staging
constexpr int kPW = kSW;                   // waves sharing the tiles of a row-block set
constexpr int kCT = 64 * kCW;              // control threads
constexpr int kPThreads = 64 * (kSW + kCW);
constexpr int kPRing = QS_PASS_RING;       // tiles in flight per streaming wave (two loads each)
constexpr size_t kPassLdsStage = 114688;   // activations staged per stage: M * K * element bytes
constexpr int kPassSlots = 4;              // row-block sets a workgroup may own per stage
constexpr int kSc1 = 16;                   // cache-policy bit SC1: device-coherent access
constexpr uint32_t kBufWord3 = 0x00020000u;  // raw 32-bit buffer resource, no swizzle

struct PassStage {
  const uint4* w;      // packed tiles
  const uint16_t* sc;  // packed scales
  int N, K;
  int s_log2;          // S = 1 << s_log2 streaming waves split K of one row block
  int nsets;           // row-block sets: ceil(nrb / R), R = kSW / S
};

struct PassArgs {
  const uint16_t* x;  // input of the launch's first stage, fp16, row stride ldx0
  int ldx0;
  int norm0;          // standardise the first stage's input rows
  uint16_t* act0;     // ping-pong fp16 stage outputs (row stride = that stage's N)
  uint16_t* act1;
  int act_first;      // act buffer written by the launch's first stage
  float* out;         // fp32 output of the launch's last stage when last_is_final
  int last_is_final;
  unsigned* flags;    // per-workgroup arrival epochs (kFlagStride apart), zeroed before the launch
  unsigned* go;       // released epoch, zeroed before the launch
  unsigned* error;    // set to 1 if a barrier wait passed its deadline
  long long deadline; // wall-clock ticks allowed per barrier wait
  int M;
  int n_stages;
  PassStage st[kMaxPassStages];
};

// Stage i of the running launch, read straight from the kernel-argument segment with scalar loads
// (the argument is the kernel's first and only one, at offset 0).  Indexing the by-value argument
// with a run-time index would copy the whole table to per-lane scratch, and scratch loads share
// the vector-memory counter with the weight ring, so every use would wait for the entire ring.
__device__ __forceinline__ PassStage stage_at(int i) {
  typedef const __attribute__((address_space(4))) PassArgs* KArgs;
  const KArgs k = (KArgs)__builtin_amdgcn_kernarg_segment_ptr();
  const int u = __builtin_amdgcn_readfirstlane(i);
  PassStage p;
  p.w = k->st[u].w;
  p.sc = k->st[u].sc;
  p.N = k->st[u].N;
  p.K = k->st[u].K;
  p.s_log2 = k->st[u].s_log2;
  p.nsets = k->st[u].nsets;
  return p;
}

// Per-wave view of one stage.
struct StageView {
  const uint4* w;
  const uint16_t* sc;
  int G, per, gcnt, nrb, my_sets, R, r, sidx, S;
  size_t tile0, set_stride;
};

// Sets of workgroup bid: bid, bid + grid, ... below nsets.  nsets <= kPassSlots * grid (host
// check), so the count is found with compares instead of a division, which keeps the stage
// bookkeeping that is repeated at every ring slot short.
__device__ __forceinline__ int stage_sets(const PassStage& ps, int bid, int grid) {
  static_assert(kPassSlots == 4, "stage_sets assumes at most four sets per workgroup");
  if (bid >= ps.nsets) return 0;
  const int x = ps.nsets - 1 - bid;
  return 1 + (x >= grid) + (x >= 2 * grid) + (x >= 3 * grid);
}

__device__ __forceinline__ StageView stage_view(const PassStage& ps, int wave, int bid, int grid) {
  StageView v;
  v.w = ps.w;
  v.sc = ps.sc;
  v.S = 1 << ps.s_log2;
  v.R = kPW >> ps.s_log2;
  v.r = wave >> ps.s_log2;
  v.sidx = wave & (v.S - 1);
  v.G = ps.K >> 7;  // K / kGroup
  v.per = (v.G + v.S - 1) >> ps.s_log2;
  const int g0 = v.sidx * v.per;
  v.gcnt = v.G - g0 < v.per ? v.G - g0 : v.per;
  v.nrb = (ps.N + 15) >> 4;
  v.my_sets = stage_sets(ps, bid, grid);
  v.tile0 = (size_t)(bid * v.R + v.r) * v.G + g0;
  v.set_stride = (size_t)grid * v.R * v.G;
  return v;
}

// Workgroup barrier for LDS exchange only.  __syncthreads() also orders global memory, which on
// this target means waiting for every outstanding vector memory operation -- it would drain the
// weight rings.  LDS traffic is complete once lgkmcnt reaches zero.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Grid barrier between stages, free of contended atomics: workgroup b release-stores the epoch
// into its own flag (one 128-byte line each); the control threads of workgroup 0 each watch flags
// and, once all have arrived, workgroup 0 release-stores the epoch into the `go` word that every
// workgroup acquires.  Each wait has a wall-clock deadline; passing it sets the error word.
constexpr int kFlagStride = 32;  // uint32 words between flags (128 bytes)

__device__ __forceinline__ bool wait_at_least(const unsigned* p, unsigned v, const PassArgs& a) {
  if (a.deadline <= 0) {  // a zero limit fails at once (exercises the time-out path)
    __hip_atomic_store(a.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return false;
  }
  const long long t0 = wall_clock64();
  while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < v) {
    __builtin_amdgcn_s_sleep(1);
    if (wall_clock64() - t0 > a.deadline) {
      __hip_atomic_store(a.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
  }
  return true;
}

// 16 bytes per lane from global memory straight into LDS (lane l writes lds_addr + 16 l), with a
// device-coherent read.  Written as inline assembly: when the compiler sees an LDS-DMA anywhere in
// the kernel it makes every LDS read wait for all outstanding vector loads, which would drain the
// weight rings of the streaming waves.  The caller waits (s_waitcnt vmcnt(0)) before using the data;
// loads the compiler does not know about only make its own waits stricter, since loads complete in
// order.  lds_addr must be the same in all lanes.
__device__ __forceinline__ void dma_to_lds_sc1(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off sc1"
               :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds_addr)) : "memory", "m0");
}

// 16 bytes from a device-coherent read of base + byte offset (base the same in all lanes).
__device__ __forceinline__ uint4 load_sc1(const void* base, uint32_t off, uint32_t extent) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)extent, (int)kBufWord3);
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kSc1));
}

// LDS barriers every wave executes at a stage boundary:
//   A partials parked | B outputs stored | C arrivals seen (workgroup 0) | D go seen |
//   staging: W4A16 G activations in LDS; W4A4 E statistics | F row parameters | G codes in LDS
// and the staging barriers once before the first stage.  The last stage ends after B.
// Streaming waves only pass through them.
template <int MODE>
constexpr int kStagingBarriers = MODE == 0 ? 1 : 3;

template <int MODE>
__global__ __launch_bounds__(kPThreads) void pass_kernel(const PassArgs a) {
  extern __shared__ __align__(16) unsigned char dyn_lds[];
  __shared__ float4_t red[kPassSlots][kSW][64];  // per-set partials of one stage
  __shared__ float row_a[8], row_b[8], row_c[8];   // per-row mean, 1/std, W4A4 scale
  __shared__ float stat_red[4][2 * kCW];           // staging statistics per reduction unit
  __shared__ __align__(16) uint32_t zero_pad[16];
  __shared__ __align__(16) uint32_t ones_pad[16];  // fp16 1.0 pairs: the W4A16 row-sum operand
  __shared__ int fail_sh;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int bid = (int)blockIdx.x, grid = (int)gridDim.x;
  const int M = a.M;
  constexpr int kElt = MODE == 0 ? 2 : 1;

  if (wave < kSW) {
    // ======================= streaming waves =======================
    int ls = 0, l_si = 0, l_gi = 0;
    StageView lv = stage_view(stage_at(0), wave, bid, grid);
    size_t l_tile = lv.tile0;
    auto l_skip_empty = [&]() {  // stages without sets for this workgroup load nothing
      while (ls < a.n_stages && lv.my_sets == 0) {
        if (ls + 1 < a.n_stages) {
          ++ls;
          lv = stage_view(stage_at(ls), wave, bid, grid);
          l_tile = lv.tile0;
        } else {
          ls = a.n_stages;
        }
      }
    };
    l_skip_empty();
    uint4 buf[kPRing];
    uint16_t sbuf[kPRing];
    // Loads are unconditional so the compiler can wait for exactly the oldest ring slot; past the
    // last stage (lv keeps the last stage's view) the ring re-reads tile 0, which is never consumed.
    auto issue = [&](int slot) __attribute__((always_inline)) {
      const bool live = ls < a.n_stages;
      const int rb = (bid + l_si * grid) * lv.R + lv.r;
      const bool ok = live && rb < lv.nrb && l_gi < lv.gcnt;
      const size_t t = ok ? l_tile : 0;
      buf[slot] = lv.w[t * 64 + lane];
      sbuf[slot] = lv.sc[t * 16 + (lane & 15)];
      if (live) {
        ++l_tile;
        if (__builtin_expect(++l_gi == lv.per, 0)) {  // rare: keeps the ring loop's hot code compact
          l_gi = 0;
          l_tile += lv.set_stride - lv.per;
          if (++l_si == lv.my_sets) {
            l_si = 0;
            if (ls + 1 < a.n_stages) {
              ++ls;
              lv = stage_view(stage_at(ls), wave, bid, grid);
              l_tile = lv.tile0;
              l_skip_empty();
            } else {
              ls = a.n_stages;
            }
          }
        }
      }
    };
    static_for<0, kPRing>([&](auto ic) __attribute__((always_inline)) { issue(decltype(ic)::value); });

    static_for<0, kStagingBarriers<MODE>>([&](auto) { lds_barrier(); });

    const int arow = lane & 15;
    const int kq = 32 * (lane >> 4);
    const uint32_t zero_addr = (uint32_t)(uintptr_t)zero_pad;
    const uint32_t pad_addr = MODE == 0 ? (uint32_t)(uintptr_t)ones_pad : zero_addr;
    const uint32_t lds_base = (uint32_t)(uintptr_t)dyn_lds;
    int cs = 0, c_si = 0, c_gi = 0;
    StageView cv = stage_view(stage_at(0), wave, bid, grid);
    uint32_t a_lane = 0, a_step = 0;
    auto set_a = [&]() {
      const int K = stage_at(cs).K;
      a_lane = arow < M ? lds_base + (uint32_t)((arow * K + kq) * kElt) : arow == M ? pad_addr : zero_addr;
      a_step = arow < M ? (uint32_t)(kGroup * kElt) : 0u;
    };
    set_a();
    // Pass the boundary barriers of finished stages until a stage with sets for this workgroup.
    auto next_stage = [&]() __attribute__((always_inline)) {
      while (true) {
        lds_barrier();  // A
        lds_barrier();  // B
        if (cs + 1 >= a.n_stages) { cs = a.n_stages; return; }
        lds_barrier();  // C
        lds_barrier();  // D
        if (__builtin_amdgcn_readfirstlane(fail_sh)) { cs = a.n_stages; return; }
        static_for<0, kStagingBarriers<MODE>>([&](auto) { lds_barrier(); });
        ++cs;
        cv = stage_view(stage_at(cs), wave, bid, grid);
        set_a();
        if (cv.my_sets > 0) return;
      }
    };
    if (cv.my_sets == 0) next_stage();

    const uint32_t magic = fp16_magic_vgpr();
    float4_t acc = float4_t{0.f, 0.f, 0.f, 0.f};
    while (cs < a.n_stages) {
      static_for<0, kPRing>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        const uint4 wv = buf[i];
        const float s = h2f(sbuf[i]);
        bool stage_done = false;
        if (cs < a.n_stages) {
          const int rb = (bid + c_si * grid) * cv.R + cv.r;
          if (__builtin_expect(rb < cv.nrb && c_gi < cv.gcnt, 1)) {
            const uint32_t g = (uint32_t)(cv.sidx * cv.per + c_gi);
            if constexpr (MODE == 0) {
              float4_t dg = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                const uint32_t wt = t == 0 ? wv.x : t == 1 ? wv.y : t == 2 ? wv.z : wv.w;
                const half8_t b = unpack_f16x8(wt, magic);
                const uint32_t addr = a_lane + g * a_step + 16u * t;
                const half8_t av =
                    *reinterpret_cast<const __attribute__((address_space(3))) half8_t*>((size_t)addr);
                dg = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, b, dg, 0, 0, 0);
              }
              acc += s * dg;
            } else {
              int4_t dg = int4_t{0, 0, 0, 0};
#pragma unroll
              for (int t2 = 0; t2 < 2; ++t2) {
                const int4_t b = t2 == 0 ? unpack_i8x16(wv.x, wv.y) : unpack_i8x16(wv.z, wv.w);
                const uint32_t addr = a_lane + g * a_step + 16u * t2;
                const int4_t av =
                    *reinterpret_cast<const __attribute__((address_space(3))) int4_t*>((size_t)addr);
                dg = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, b, dg, 0, 0, 0);
              }
#pragma unroll
              for (int j = 0; j < 4; ++j) acc[j] += s * (float)(dg[j] >> 4);  // operands carry 16 q
            }
          }
          if (__builtin_expect(++c_gi == cv.per, 0)) {
            // end of a set: park the partial in LDS slot c_si (read by the control waves)
            c_gi = 0;
            red[c_si][wave][lane] = acc;
            acc = float4_t{0.f, 0.f, 0.f, 0.f};
            if (++c_si == cv.my_sets) {
              c_si = 0;
              stage_done = true;
            }
          }
        }
        // Refill the slot once its tile is consumed, so the new load reuses the slot's registers
        // (a refill into fresh registers makes the compiler copy the ring at the loop back-edge,
        // and each copy waits for a pending load).  Unconditional, so the number of loads in
        // flight is known at every slot; issued before the stage boundary so the ring stays full
        // through it.
        issue(i);
        if (__builtin_expect(stage_done, 0)) next_stage();
      });
    }
    return;
  }

  // ======================= control waves =======================
  const int ct = (int)threadIdx.x - 64 * kSW;  // 0 .. kCT-1
  const int cw = wave - kSW;
  if (ct == 0) fail_sh = 0;
  if (ct < 16) {
    zero_pad[ct] = 0u;
    ones_pad[ct] = 0x3C003C00u;
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)dyn_lds;
  // W4A4 staging layout: rows spread over groups of control threads (gsz threads per row).
  const int mp = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8;
  const int gsz = kCT / mp;                   // threads per row
  const int unit = gsz < 64 ? gsz : 64;       // lanes per reduction unit (32 or 64)
  const int my_row = ct / gsz;
  const int row_tid = ct - my_row * gsz;
  const int my_unit = ct / unit;              // reduction unit index (< 2 * kCW)
  const int units_per_row = gsz / unit;
  constexpr int kXBatch = 8;

  auto unit_sum = [&](float v) {
    for (int o = unit >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
  };
  auto unit_max = [&](float v) {
    for (int o = unit >> 1; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
  };
  auto unit_min = [&](float v) {
    for (int o = unit >> 1; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
    return v;
  };
  auto stage_input = [&](int s) -> const uint16_t* {
    return s == 0 ? a.x : (((a.act_first + s - 1) & 1) ? a.act1 : a.act0);
  };

  // Stage s input -> LDS, ending with the staging barriers (work only if this workgroup has sets).
  auto prologue = [&](int s, bool has) {
    const int K = stage_at(s).K;
    const uint16_t* x = stage_input(s);
    const int ldx = s == 0 ? a.ldx0 : stage_at(s - 1).N;
    const int norm = s == 0 ? a.norm0 : 1;
    if constexpr (MODE == 0) {
      // Raw fp16 rows straight into LDS, [M][K] row-major: one 1 KiB chunk per wave instruction.
      if (has) {
        const int total = M * K;
        const int nch = (total + 511) / 512;
        for (int ch = cw; ch < nch; ch += kCW) {
          const int e = ch * 512 + lane * 8;
          if (e < total) {
            const int row = e / K, col = e - row * K;
            dma_to_lds_sc1(x + (size_t)row * ldx + col, lds_base + (uint32_t)ch * 1024u);
          }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      lds_barrier();  // G
      // Row statistics for the epilogue, one control wave per row, while the contraction runs.
      if (has && cw < M) {
        float mu = 0.f, inv = 1.f;
        if (norm) {
          const uint4* r = reinterpret_cast<const uint4*>(dyn_lds) + (size_t)cw * (K / 8);
          float su = 0.f, sq = 0.f, mx = -INFINITY, mn = INFINITY;
          for (int i = lane; i < K / 8; i += 64) stats_block8(r[i], su, sq, mx, mn);
          su = wave_sum(su);
          sq = wave_sum(sq);
          norm_params(su, sq, K, mu, inv);
        }
        if (lane == 0) {
          row_a[cw] = mu;
          row_b[cw] = inv;
        }
      }
    } else {
      const int nb = K / 8;
      const bool active = has && my_row < M;
      const bool one_batch = nb <= kXBatch * gsz;
      const uint32_t rows_bytes = (uint32_t)(((M - 1) * ldx + K) * 2);
      const uint32_t row_off = (uint32_t)((my_row < M ? my_row : 0) * ldx * 2);
      uint4 v[kXBatch];
      auto load_batch = [&](int base) {
#pragma unroll
        for (int j = 0; j < kXBatch; ++j) {
          const int i = base + row_tid + j * gsz;
          if (i < nb) v[j] = load_sc1(x, row_off + (uint32_t)i * 16u, rows_bytes);
        }
      };
      float su = 0.f, sq = 0.f, mx = -INFINITY, mn = INFINITY;
      if (active) {
        for (int base = 0; base < nb; base += kXBatch * gsz) {
          load_batch(base);
#pragma unroll
          for (int j = 0; j < kXBatch; ++j) {
            const int i = base + row_tid + j * gsz;
            if (i < nb) stats_block8(v[j], su, sq, mx, mn);
          }
        }
      }
      su = unit_sum(su);
      sq = unit_sum(sq);
      mx = unit_max(mx);
      mn = unit_min(mn);
      if ((ct & (unit - 1)) == 0) {
        stat_red[0][my_unit] = su;
        stat_red[1][my_unit] = sq;
        stat_red[2][my_unit] = mx;
        stat_red[3][my_unit] = mn;
      }
      lds_barrier();  // E
      if (has && ct < M) {
        const int m = ct;
        float tsu = 0.f, tsq = 0.f, xmax = -INFINITY, xmin = INFINITY;
        for (int u = m * units_per_row; u < (m + 1) * units_per_row; ++u) {
          tsu += stat_red[0][u];
          tsq += stat_red[1][u];
          xmax = fmaxf(xmax, stat_red[2][u]);
          xmin = fminf(xmin, stat_red[3][u]);
        }
        float mu = 0.f, inv = 0.f;
        if (norm) norm_params(tsu, tsq, K, mu, inv);
        row_a[m] = mu;
        row_b[m] = inv;
        const float amax = norm ? fmaxf(h2f(norm_h(xmax, mu, inv)), -h2f(norm_h(xmin, mu, inv)))
                                : fmaxf(xmax, -xmin);
        row_c[m] = h2f(f2h(amax / 7.0f));
      }
      lds_barrier();  // F
      if (active) {
        int8_t* xq = reinterpret_cast<int8_t*>(dyn_lds) + (size_t)my_row * K;
        const float mu = row_a[my_row], inv = row_b[my_row], sc = row_c[my_row];
        for (int base = 0; base < nb; base += kXBatch * gsz) {
          if (!one_batch) load_batch(base);
#pragma unroll
          for (int j = 0; j < kXBatch; ++j) {
            const int i = base + row_tid + j * gsz;
            if (i < nb) {
              uint4 w = v[j];
              if (norm) w = norm_block8(w, mu, inv);
              uint2 op, lg;
              quant_block8(w, sc, op, lg);
              *reinterpret_cast<uint2*>(xq + (size_t)i * 8) = op;
            }
          }
        }
      }
      lds_barrier();  // G
    }
  };

  prologue(0, stage_sets(stage_at(0), bid, grid) > 0);
  for (int s = 0; s < a.n_stages; ++s) {
    lds_barrier();  // A: the streaming waves have parked the partials of stage s
    const PassStage ps = stage_at(s);
    const int sets = stage_sets(ps, bid, grid);
    const bool final_out = a.last_is_final && s + 1 == a.n_stages;
    if (sets > 0) {
      // sum, in a fixed order, the S partials of each (set, row block) and store the outputs
      const int S = 1 << ps.s_log2, R = kSW >> ps.s_log2;
      const int nrb = (ps.N + 15) >> 4, N = ps.N;
      const int norm = s == 0 ? a.norm0 : 1;
      uint16_t* o16 = ((a.act_first + s) & 1) ? a.act1 : a.act0;
      for (int p = cw; p < sets * R; p += kCW) {
        const int si = p / R, r2 = p - si * R;
        const int rb = (bid + si * grid) * R + r2;
        float4_t v = red[si][r2 * S][lane];
        for (int s2 = 1; s2 < S; ++s2) v += red[si][r2 * S + s2][lane];
        float rowsum = 0.f;  // W4A16: sum_k w[n,k] from the all-ones operand row M
        if constexpr (MODE == 0) {
          const int q = M & 3;
          const float vq = q == 0 ? v[0] : q == 1 ? v[1] : q == 2 ? v[2] : v[3];
          rowsum = __shfl(vq, (lane & 15) + 16 * (M >> 2), 64);
        }
        const int n = rb * 16 + (lane & 15);
        if (rb < nrb && n < N) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int m = 4 * (lane >> 4) + j;
            if (m < M) {
              float outv = v[j];
              if constexpr (MODE == 0) {
                if (norm) outv = (outv - row_a[m] * rowsum) * row_b[m];
              } else {
                outv *= row_c[m];
              }
              if (final_out)
                a.out[(size_t)m * N + n] = outv;
              else  // device-coherent store: read by other workgroups after the grid barrier
                __hip_atomic_store(o16 + (size_t)m * N + n, f2h(outv), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
          }
        }
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's output stores have completed
    lds_barrier();  // B
    if (s + 1 >= a.n_stages) return;
    const unsigned epoch = (unsigned)(s + 1);
    if (ct == 0)
      __hip_atomic_store(a.flags + (size_t)bid * kFlagStride, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (bid == 0) {
      for (int t = ct; t < grid; t += kCT)
        if (!wait_at_least(a.flags + (size_t)t * kFlagStride, epoch, a)) fail_sh = 1;
    }
    lds_barrier();  // C
    if (ct == 0) {
      if (bid == 0 && !fail_sh)
        __hip_atomic_store(a.go, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (!fail_sh && !wait_at_least(a.go, epoch, a)) fail_sh = 1;
    }
    lds_barrier();  // D
    if (__builtin_amdgcn_readfirstlane(fail_sh)) return;
    prologue(s + 1, stage_sets(stage_at(s + 1), bid, grid) > 0);
  }
}

__global__ void pass_reset_kernel(unsigned* flags, int n_flags, unsigned* go, unsigned* error,
                                  int clear_error) {
  for (int i = threadIdx.x; i < n_flags; i += blockDim.x) flags[(size_t)i * 32] = 0u;
  if (threadIdx.x == 0) {
    go[0] = 0u;
    if (clear_error) error[0] = 0u;
  }
}

// ------------------------------------------------------------------ host side

static int pick_pass_split(int N, int K, int grid);

bool pass_eligible(int mode, int M, const qs_linear_desc* c, int n) {
  // W4A4 above one row: every workgroup would quantize all rows itself and the fp16 exchange grows
  // with M; measured on MI355X, one launch per linear is as fast from M = 2 on.
  if (mode == QS_W4A16 ? M > 4 : M > 1) return false;
  const int grid = device_info()->num_cus;
  if (grid < 1 || grid > kMaxPassWorkgroups) return false;
  for (int i = 0; i < n; ++i) {
    if ((size_t)M * c[i].K * (mode == QS_W4A16 ? 2 : 1) > kPassLdsStage) return false;
    if (pick_pass_split(c[i].N, c[i].K, grid) < 0) return false;
  }
  return true;
}

// K-split S per stage: fewest tiles per wave, subject to at most kPassSlots sets per workgroup;
// ties go to the smaller S (fewer, longer sets).  Returns -1 if no S fits.
static int pick_pass_split(int N, int K, int grid) {
  const int nrb = (N + 15) / 16, G = K / kGroup;
  int best = -1;
  long best_items = -1;
  for (int sl = 0; (1 << sl) <= kPW; ++sl) {
    const int S = 1 << sl, R = kPW / S;
    const long nsets = (nrb + R - 1) / R;
    if (nsets > (long)kPassSlots * grid) continue;
    const long items = (nsets + grid - 1) / grid * ((G + S - 1) / S);
    if (best_items < 0 || items < best_items) { best_items = items; best = sl; }
  }
  return best;
}

int pass_launch_count(int n) { return (n + kMaxPassStages - 1) / kMaxPassStages; }

static std::atomic<int> g_barrier_timeout_us{200000};
int pass_barrier_timeout_us() { return g_barrier_timeout_us.load(); }
void set_pass_barrier_timeout_us(int us) { g_barrier_timeout_us.store(us); }

int launch_pass(int mode, const uint16_t* x, int M, const qs_linear_desc* c, int n, float* out,
                uint16_t* act0, uint16_t* act1, unsigned* ctrl, hipStream_t st) {
  const DeviceInfo* di = device_info();
  const int grid = di->num_cus;
  auto fn0 = pass_kernel<0>;
  auto fn1 = pass_kernel<1>;
  const void* fn = mode == QS_W4A16 ? reinterpret_cast<const void*>(fn0) : reinterpret_cast<const void*>(fn1);
  static int lds_set[2] = {0, 0};
  if (!lds_set[mode]) {
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kPassLdsStage) != hipSuccess)
      return QS_ERR_HIP;
    lds_set[mode] = 1;
  }
  // At least 80 KiB of dynamic LDS: together with the static arrays no two workgroups fit on one
  // CU, so the num_cus workgroups spread one per CU.
  size_t lds = 81920;
  for (int i = 0; i < n; ++i) {
    const size_t b = (size_t)M * c[i].K * (mode == QS_W4A16 ? 2 : 1);
    lds = b > lds ? b : lds;
  }

  const int launches = pass_launch_count(n);
  const int per_launch = (n + launches - 1) / launches;
  int act_first = 0;
  for (int s0 = 0, li = 0; s0 < n; s0 += per_launch, ++li) {
    const int cnt = n - s0 < per_launch ? n - s0 : per_launch;
    PassArgs a{};
    if (s0 == 0) {
      a.x = x;
      a.ldx0 = c[0].K;
      a.norm0 = 0;
    } else {
      a.x = ((act_first + 1) & 1) ? act1 : act0;  // output of stage s0-1
      a.ldx0 = c[s0 - 1].N;
      a.norm0 = 1;
    }
    a.act0 = act0;
    a.act1 = act1;
    a.act_first = act_first;
    a.out = out;
    a.last_is_final = s0 + cnt == n;
    a.go = ctrl;
    a.error = ctrl + 1;
    a.flags = ctrl + kFlagStride;
    a.deadline = (long long)di->clock_khz * pass_barrier_timeout_us() / 1000;  // wall-clock ticks
    a.M = M;
    a.n_stages = cnt;
    for (int i = 0; i < cnt; ++i) {
      const qs_linear_desc& d = c[s0 + i];
      PassStage& p = a.st[i];
      p.w = reinterpret_cast<const uint4*>(d.w_packed);
      p.sc = d.s_packed;
      p.N = d.N;
      p.K = d.K;
      p.s_log2 = pick_pass_split(d.N, d.K, grid);
      const int R = kPW >> p.s_log2;
      p.nsets = ((d.N + 15) / 16 + R - 1) / R;
    }
    hipLaunchKernelGGL(pass_reset_kernel, dim3(1), dim3(256), 0, st, ctrl + kFlagStride, grid, ctrl, ctrl + 1,
                       li == 0 ? 1 : 0);
    int rc = launch_status();
    if (rc != QS_OK) return rc;
    if (mode == QS_W4A16)
      hipLaunchKernelGGL(pass_kernel<0>, dim3(grid), dim3(kPThreads), lds, st, a);
    else
      hipLaunchKernelGGL(pass_kernel<1>, dim3(grid), dim3(kPThreads), lds, st, a);
    rc = launch_status();
    if (rc != QS_OK) return rc;
    act_first = (act_first + cnt) & 1;
  }
  return QS_OK;
}

}  // namespace qs
