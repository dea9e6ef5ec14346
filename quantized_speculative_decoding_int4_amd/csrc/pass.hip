// Persistent pass kernel: one launch runs up to kMaxPassStages linears of a chain
// (the W4A4 draft pass at up to 4 rows or the W4A16 verify pass at up to 14 rows,
// [P3] "draft modelとtarget modelの処理フロー"; modes from [P1] "QSpec の W4A4
// モードと W4A16 モード"; W4A8 from [P2] "3.中核となる技術的要素").  The integer modes W4A4
// and W4A8 share one kernel body and differ only in the activation code range (7 or 127).
//
// Why persistent: at decode sizes a linear moves 2-60 MB of weights, so a
// stand-alone launch spends a large share of its time ramping up and draining
// (on MI355X a kernel that only reads 8 MB takes ~7 us).  Here one workgroup per
// compute unit stays resident for all stages.  Every wave owns a flattened
// stream of 1 KiB weight tiles across all stages of the launch and keeps a ring
// of kPRing tile loads in flight; weights do not depend on activations, so the
// ring runs ahead into the next stage while the workgroups wait for the stage's
// input and stage it in LDS.  HBM keeps streaming through the dependency.
//
// Stage hand-over.  Every stage of a pass writes its fp16 output to a buffer of
// its own with device-coherent stores, and the next stage reads it with
// device-coherent loads (both go past the per-XCD L2 to memory), so no L2
// write-back or invalidate is needed (an agent-scope release/acquire costs about
// 3.5 us per boundary on MI355X).  Two ways to know the input is complete:
//  * W4A4 and W4A8 (up to 4 rows, 8-112 KiB of input): the data carries the signal.  The output
//    buffers start filled with the pattern 0xFFFF (a NaN the epilogue never
//    emits: it rewrites that one pattern as the canonical NaN 0x7E00).  A
//    consumer fetches its input as soon as its own stage is done and reads again
//    every 16-byte piece that still holds the pattern.  Each piece is written by
//    one workgroup in 2-byte stores, so a piece read while it is being written
//    shows the pattern in the halves not yet written.  This saves the producer's
//    wait for its store acknowledgements and the two hops of a grid barrier.
//  * W4A16 (up to 14 rows, up to 112 KiB of staged input): a grid barrier, then one fetch.
//    Where M rows of a linear's K do not fit in LDS, the linear runs as several table entries,
//    each over a K chunk that does; they sum into the same outputs with no barrier in between.
//    A premature fetch of that much data costs a second full round trip, which
//    measured slower than the barrier.  Workgroup b stores an epoch into its own
//    flag once its outputs are acknowledged, and every workgroup watches all the
//    flags (one round trip; a relay through a `go` word published by workgroup 0
//    measured 2.4% slower over the verify pass).
// Every wait has a wall-clock deadline that sets an error word and makes the
// workgroup exit, so no wave can wait forever.  The final output is filled with
// NaN before the pass starts: a workgroup writes its part of it only after every
// wait it made succeeded, so after a time-out each output value is either the
// correct one or NaN -- never a value left from an earlier call.
//
// Tile math per stage is the one of linear.hip: a wave's share of a 16-row block
// (S waves split K), expansion of the nibbles in VGPRs, MFMA with the staged
// activations as A operand, fp32 group scaling, fixed-order reduction over the
// S waves through LDS.
//
// W4A16 stages take the raw fp16 input (the 16-bit activations of the product)
// and apply the row standardisation after the contraction: with mean mu and 1/std
// inv of input row m,
//   sum_k w[n,k] (x[m,k] - mu) inv = (sum_k w[n,k] x[m,k] - mu sum_k w[n,k]) inv,
// and sum_k w[n,k] comes for free from an all-ones row placed in the zero padding
// of the 16-row A operand.  The input therefore goes to LDS as it arrives and its
// statistics are computed while the contraction runs.  The integer modes must
// quantise the standardised row first, so they stage through registers:
// statistics, scale, quantisation, then LDS -- all exact: fp64 statistics and a
// correctly rounded fp16 standardised value (qs_act.h), and fp64 group scaling of
// the exact i32 sums (each term s * acc is exact in fp64, and so are their sums
// and the product with the row scale while log2(K / 128) + the binades spanned by
// a row's scales <= 13), rounded once to the fp16 stage output or the fp32 result.

#include "qs_act.h"
#include "qs_device.h"
#include "qs_internal.h"
#include "qs_msi.h"

#include <atomic>
#include <vector>
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
// Measured on MI355X over the 129-linear stack: rings of 4 to 12 tiles give the same pass time
// within 1-2%, a 16-deep ring is 3-4% slower in both modes -- the deeper prefetch's HBM traffic
// delays the latency-bound stage hand-over more than the prefetch shortens the next stage.
#define QS_PASS_RING 8
#endif
constexpr int kSW = QS_PASS_STREAM_WAVES;  // streaming waves: weight ring + MFMA (split S x R)
constexpr int kCW = QS_PASS_CTRL_WAVES;    // control waves: reductions, stores, barriers, staging
constexpr int kPW = kSW;                   // waves sharing the tiles of a row-block set
constexpr int kCT = 64 * kCW;              // control threads
constexpr int kPThreads = 64 * (kSW + kCW);
constexpr int kPRing = QS_PASS_RING;       // tiles in flight per streaming wave (two loads each)
constexpr size_t kPassLdsStage = 114688;   // W4A16: activations staged per stage, M * K * 2 bytes
// Integer modes: their fp64 partials take 64 KiB of static LDS, so the staged codes (M * K bytes)
// get at most this much dynamic LDS.
constexpr size_t kPassLdsStageInt = 81920;
// At least this much dynamic LDS per workgroup: with the static arrays no two workgroups fit on one
// CU, so the launch spreads one workgroup per CU.
constexpr size_t kPassLdsMin = 81920;
constexpr int kPassSlots = 4;              // row-block sets a workgroup may own per stage
constexpr int kCtrlSlots = (kPassSlots * kPW + kCW - 1) / kCW;  // (set, row block) pairs per control wave
constexpr uint16_t kEmpty = 0xFFFFu;       // pattern of a stage output not yet written
// Shared activation codes not yet written: W4A4 stores a byte per code and -128 is no INT4 code; W4A8
// codes take every byte value, so W4A8 stores 16 bits per code and -32768 marks the empty ones.
constexpr uint32_t kCodeEmpty = 0x80808080u;
constexpr uint32_t kCodeEmpty16 = 0x80008000u;
constexpr int kSc1 = 16;                   // cache-policy bit SC1: device-coherent access
constexpr uint32_t kBufWord3 = 0x00020000u;  // raw 32-bit buffer resource, no swizzle

// One entry of a launch's stage table: a linear, or one K chunk of a linear whose M staged input
// rows do not fit in LDS at once (W4A16 at K = 14336 above four rows).  A chunked linear's entries sum into the
// same outputs: every chunk but the last hands its partial sums on in the control waves' registers,
// the last one writes the outputs; a grid barrier follows only a linear's last chunk.
struct PassStage {
  const uint4* w;      // packed tiles
  const uint16_t* sc;  // packed scales
  uint16_t* y16;       // fp16 output [M][N], filled with kEmpty before the launch (not the last stage)
  int N, K;            // K: columns of this entry's chunk
  int s_log2;          // S = 1 << s_log2 streaming waves split K of one row block
  int nsets;           // row-block sets: ceil(nrb / R), R = kSW / S
  int gfull;           // 128-wide groups of the whole linear (tiles per row block)
  int chunk;           // bits 0-15: the chunk's first group; bit 16: first chunk; bit 17: last chunk;
                       // bits 24-31: entries back to the producer's last chunk (0: the launch input)
};
__device__ __forceinline__ int chunk_g0(const PassStage& p) { return p.chunk & 0xFFFF; }
__device__ __forceinline__ bool chunk_first(const PassStage& p) { return ((p.chunk >> 16) & 1) != 0; }
__device__ __forceinline__ bool chunk_last(const PassStage& p) { return ((p.chunk >> 17) & 1) != 0; }
__device__ __forceinline__ int chunk_back(const PassStage& p) { return (p.chunk >> 24) & 0xFF; }

struct PassArgs {
  const uint16_t* x;  // input of the launch's first stage, fp16, row stride ldx0 (complete at launch)
  int ldx0;
  int norm0;          // standardise the first stage's input rows
  float* out;         // fp32 output of the launch's last stage when last_is_final (nullable)
  int last_is_final;
  // Top-1 epilogue of the final stage (the LM-head), when top1 is not NULL: per row, the lowest
  // index of the largest output and 1 / sum exp(y - max).  Each workgroup reduces its columns to
  // a (max, sum of exp, argmax) partial per row in t1_stats [M][grid] (16 bytes each); the last
  // workgroup to arrive at t1_cnt (zero at pass start) merges them.
  int32_t* top1;
  float* top1_prob;   // nullable
  unsigned char* t1_stats;
  unsigned* t1_cnt;
  unsigned* flags;    // W4A16: per-workgroup arrival epochs (kFlagStride apart), zero at pass start
  unsigned epoch0;    // W4A16: epochs of this launch's boundaries are epoch0 + 1, epoch0 + 2, ...
  unsigned* error;    // set to 1 if a wait passed its deadline
  long long deadline; // wall-clock ticks allowed per wait
  // Boundary timestamps (nullable): wall-clock ticks per (pass-wide entry trace_e0 + s, workgroup),
  // four per entry -- input staged, partials parked (stage done), outputs stored, hand-over done.
  unsigned long long* trace;
  int trace_e0;
  int M;
  int n_stages;
  PassStage st[kMaxPassStages];
  // Shared activation codes (integer modes above one row), [M][K] in MFMA operand order, empty before
  // the pass (W4A4: bytes, kCodeEmpty; W4A8: 16-bit, kCodeEmpty16): those of the fp16 stage output at
  // byte offset o of the stage-output area (stage_base) are at codes_base + o / 2 (W4A4) or + o
  // (W4A8); those of the launch's input at codes_in.  After the stage table, which keeps its offset
  // in the argument segment.
  const unsigned char* stage_base;
  int8_t* codes_base;
  int8_t* codes_in;  // codes of the launch's input
};
static_assert(sizeof(PassArgs) <= 4096, "the stage table travels in the 4 KiB kernel-argument segment");

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
  p.y16 = k->st[u].y16;
  p.N = k->st[u].N;
  p.K = k->st[u].K;
  p.s_log2 = k->st[u].s_log2;
  p.nsets = k->st[u].nsets;
  p.gfull = k->st[u].gfull;
  p.chunk = k->st[u].chunk;
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
  v.tile0 = (size_t)(bid * v.R + v.r) * ps.gfull + chunk_g0(ps) + g0;  // tiles of a row block: gfull apart
  v.set_stride = (size_t)grid * v.R * ps.gfull;
  return v;
}

// Workgroup barrier for LDS exchange only.  __syncthreads() also orders global memory, which on
// this target means waiting for every outstanding vector memory operation -- it would drain the
// weight rings.  LDS traffic is complete once lgkmcnt reaches zero.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// True if any of the 8 halves of v holds kEmpty: ~v then has a zero halfword, which the
// borrow test (w - 0x00010001) & ~w & 0x80008000 detects (exactly, for the "any" question).
__device__ __forceinline__ bool has_empty(const uint4 v) {
  auto zero_half = [](uint32_t w) { return (w - 0x00010001u) & ~w & 0x80008000u; };
  return (zero_half(~v.x) | zero_half(~v.y) | zero_half(~v.z) | zero_half(~v.w)) != 0u;
}

// True if any byte (CB = 1) or 16-bit word (CB = 2) of v holds the empty code: v ^ kCodeEmpty(16)
// then has a zero byte or word.
template <int CB>
__device__ __forceinline__ bool has_code_empty(const uint4 v) {
  auto zero_part = [](uint32_t w) {
    if constexpr (CB == 1) {
      w ^= kCodeEmpty;
      return (w - 0x01010101u) & ~w & 0x80808080u;
    } else {
      w ^= kCodeEmpty16;
      return (w - 0x00010001u) & ~w & 0x80008000u;
    }
  };
  return (zero_part(v.x) | zero_part(v.y) | zero_part(v.z) | zero_part(v.w)) != 0u;
}

// Buffer resource over extent bytes at base (base the same in all lanes); reads past the extent
// return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t sc1_rsrc(const void* base, uint32_t extent) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)extent, (int)kBufWord3);
}
// 16 bytes from a device-coherent read at byte offset voff (per lane) + soff (uniform).
__device__ __forceinline__ uint4 load_sc1(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kSc1));
}

// 16 bytes per active lane from global memory straight into LDS (lane l writes lds_addr + 16 l),
// with a device-coherent read.  Written as inline assembly: when the compiler sees an LDS-DMA
// anywhere in the kernel it makes every LDS read wait for all outstanding vector loads, which would
// drain the weight rings of the streaming waves.  The caller waits (s_waitcnt vmcnt(0)) before
// using the data; loads the compiler does not know about only make its own waits stricter, since
// loads complete in order.  lds_addr must be the same in all lanes.
__device__ __forceinline__ void dma_to_lds_sc1(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off sc1"
               :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds_addr)) : "memory", "m0");
}

// LDS barriers every wave executes at a stage boundary:
//   A partials parked |
//   W4A16 grid barrier: B outputs stored | C all arrivals seen |
//   staging: W4A16 G activations in LDS; W4A4 E statistics | F row parameters | G codes in LDS
// and the staging barriers once before the first stage.  The last stage ends after A.
// Streaming waves only pass through them.
constexpr int kGridBarriers = 2;
template <int MODE>
constexpr int kStagingBarriers = MODE == 0 ? 1 : 3;
// Largest activation code of the integer modes: 7 (W4A4, INT4 codes), 127 (W4A8, INT8 codes).
template <int MODE>
constexpr int kPassQmax = MODE == 2 ? 127 : 7;
// The integer-mode passes of 2-4 rows stage every input through the shared codes (stage_in4s).
// Measured on the Llama-3-8B-shaped stack, 4-row draft pass: W4A4 1.94 ms, W4A8 2.02 ms (16-bit
// codes), against 2.41 ms with every workgroup quantising all rows (3 rows: 1.92 / 1.97 against
// 2.34; 2 rows: 1.79 either way).  The one-row pass keeps stage_in4: shared codes took the W4A4 one
// from 1.38 to 1.64 ms (1.45 ms when used only into the 14336-wide down projection), the extra
// exchange costing more than the quantisation of one row it saves.
template <int MODE, bool WIDE>
constexpr bool kPassShared = MODE != 0 && WIDE;

// W4A16 grid barrier between stages, free of contended atomics: workgroup b stores the epoch into
// its own flag (one 128-byte line each) once its outputs are acknowledged, and the control threads
// of every workgroup each watch flags until all have arrived.  All of these are device-coherent
// accesses.
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

// Top-1 epilogue of the final stage, run by every control wave of every workgroup (also one
// without columns in the stage, so that all workgroups arrive).  No workgroup barrier: the
// streaming waves may already have ended.  The wave's 16-lane rows are merged by DPP; the last
// control wave of the workgroup to arrive (an LDS counter) merges the waves' partials in wave
// order and publishes the workgroup's partial per row; the last workgroup to arrive merges the
// partials of all workgroups, lanes strided over them, then a fixed-order lane merge.
struct Top1Out {
  int32_t* top1;
  float* top1_prob;
  unsigned char* stats;
  unsigned* cnt;
};
__device__ __forceinline__ void top1_epilogue(const Top1Out o, Msi (&t1v)[4], float4_t (*t1_wave)[16],
                                              unsigned* t1_arrive, int cw, int lane, int bid, int grid, int M) {
  // lane l holds rows 4 (l >> 4) + j of its column; the 16 lanes of a DPP row share those rows
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    Msi t = t1v[j];
    t = msi_merge(t, msi_dpp<0xB1>(t));
    t = msi_merge(t, msi_dpp<0x4E>(t));
    t = msi_merge(t, msi_dpp<0x141>(t));
    t = msi_merge(t, msi_dpp<0x140>(t));
    if ((lane & 15) == 0) t1_wave[cw][4 * (lane >> 4) + j] = float4_t{t.m, t.s, __int_as_float(t.i), 0.0f};
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's partials are in LDS
  unsigned old = 0u;
  if (lane == 0) old = __hip_atomic_fetch_add(t1_arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  old = (unsigned)__builtin_amdgcn_readfirstlane((int)old);
  asm volatile("" ::: "memory");
  if (old != (unsigned)(kCW - 1)) return;
  // the workgroup's last control wave: lane m merges row m over the waves, in wave order
  const __amdgpu_buffer_rsrc_t rs = sc1_rsrc(o.stats, (uint32_t)(M * grid * 16));
  if (lane < M) {
    Msi t{-INFINITY, 0.0f, 0x7fffffff};
    for (int w = 0; w < kCW; ++w) {
      const float4_t v = t1_wave[w][lane];
      t = msi_merge(t, Msi{v[0], v[1], __float_as_int(v[2])});
    }
    const float4_t pv{t.m, t.s, __int_as_float(t.i), 0.0f};
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(int4_t, pv), rs, (lane * grid + bid) * 16, 0, kSc1);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the partials are in memory
  unsigned prev = 0u;
  if (lane == 0) prev = __hip_atomic_fetch_add(o.cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  prev = (unsigned)__builtin_amdgcn_readfirstlane((int)prev);
  asm volatile("" ::: "memory");
  if (prev + 1u != (unsigned)grid) return;
  // the last workgroup: every row over all workgroups (lane c takes workgroups c, c + 64, ...), four
  // rows at a time.  A round's partials are all loaded before any is merged, so they cost one round
  // trip (buffer loads past the extent return zeros and are not merged).
  constexpr int kPer = 4;  // workgroups per lane and round
  for (int m0 = 0; m0 < M; m0 += 4) {
    Msi t4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) t4[r] = Msi{-INFINITY, 0.0f, 0x7fffffff};
    for (int c0 = 0; c0 < grid; c0 += 64 * kPer) {
      float4_t v[4][kPer];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
          const int c = c0 + 64 * k + lane;
          v[r][k] = m0 + r < M ? __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                                  rs, ((m0 + r) * grid + c) * 16, 0, kSc1))
                               : float4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int k = 0; k < kPer; ++k)
          if (c0 + 64 * k + lane < grid) t4[r] = msi_merge(t4[r], Msi{v[r][k][0], v[r][k][1], __float_as_int(v[r][k][2])});
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (m0 + r < M) {
        const Msi t = wave_msi(t4[r]);
        if (lane == 0) {
          o.top1[m0 + r] = t.i;
          if (o.top1_prob) o.top1_prob[m0 + r] = 1.0f / t.s;
        }
      }
    }
  }
}

// WIDE (integer modes, more than one row): the inputs are staged through the shared codes
// (stage_in4s) instead of being quantised whole in every workgroup (stage_in4).  A separate instance:
// both stagings in one kernel spill registers.
// TRACE: record the boundary timestamps of PassArgs::trace (a separate instance, so the passes that do
// not record them carry no check).
template <int MODE, bool WIDE, bool TRACE>
__global__ __launch_bounds__(kPThreads) void pass_kernel(const PassArgs a) {
  // Partials of the streaming waves: fp32 (W4A16) or fp64 (the integer modes: exact sums).
  using Acc = std::conditional_t<MODE == 0, float4_t, double4_t>;
  extern __shared__ __align__(16) unsigned char dyn_lds[];
  __shared__ Acc red[kPassSlots][kSW][64];         // per-set partials of one stage
  __shared__ float row_a[16], row_b[16], row_c[16];  // W4A16: per-row mean, 1/std; integer modes: scale
  __shared__ float row_su[16], row_sq[16];          // W4A16 chunked linear: row sums of earlier chunks
  __shared__ double row_mu64[8], row_inv64[8];     // integer modes: per-row mean, 1/std (fp64)
  __shared__ double stat_sum[2][2 * kCW];          // integer staging: fp64 sum, sum of squares per unit
  __shared__ float stat_mm[2][2 * kCW];            // integer staging: max, min per unit
  __shared__ __align__(16) uint32_t zero_pad[16];
  __shared__ __align__(16) uint32_t ones_pad[16];  // fp16 1.0 pairs: the W4A16 row-sum operand
  __shared__ int fail_sh;
  __shared__ float4_t t1_wave[kCW][16];            // Top-1 epilogue: per control wave and row
  __shared__ unsigned t1_arrive;                   // control waves done with their Top-1 partials

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
        if (cs + 1 >= a.n_stages) { cs = a.n_stages; return; }
        if constexpr (MODE == 0) {  // B C, after a linear's last chunk (the control waves' condition)
          if (chunk_last(stage_at(cs))) static_for<0, kGridBarriers>([&](auto) { lds_barrier(); });
        }
        static_for<0, kStagingBarriers<MODE>>([&](auto) { lds_barrier(); });
        if (__builtin_amdgcn_readfirstlane(fail_sh)) { cs = a.n_stages; return; }
        ++cs;
        cv = stage_view(stage_at(cs), wave, bid, grid);
        set_a();
        if (cv.my_sets > 0) return;
      }
    };
    if (cv.my_sets == 0) next_stage();

    const uint32_t magic = fp16_magic_vgpr();
    Acc acc = Acc{0, 0, 0, 0};
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
              const double s16 = (double)s * 0.0625;  // operands carry 16 q: exact rescale
#pragma unroll
              for (int j = 0; j < 4; ++j) acc[j] += s16 * (double)dg[j];  // exact in fp64
            }
          }
          if (__builtin_expect(++c_gi == cv.per, 0)) {
            // end of a set: park the partial in LDS slot c_si (read by the control waves)
            c_gi = 0;
            red[c_si][wave][lane] = acc;
            acc = Acc{0, 0, 0, 0};
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
  if (ct == 0) {
    fail_sh = 0;
    t1_arrive = 0u;
  }
  if (ct < 16) {
    zero_pad[ct] = 0u;
    ones_pad[ct] = 0x3C003C00u;
  }
  // Input rows spread over groups of control threads: gsz threads per row (M <= 4, so gsz >= 128),
  // thread row_tid of a group holds pieces row_tid, row_tid + gsz, ... of its row.  Reduction units
  // are whole waves.
  const int mp = M <= 1 ? 1 : M <= 2 ? 2 : 4;
  const int gsz = kCT / mp;
  const int my_row = ct / gsz;
  const int row_tid = ct - my_row * gsz;
  const int units_per_row = gsz / 64;
  const uint32_t lds_base = (uint32_t)(uintptr_t)dyn_lds;

  // Stage s input -> LDS, ending with the staging barriers (work only if this workgroup has sets).
  auto wait_failed = [&](long long t0) {
    if (a.deadline > 0 && wall_clock64() - t0 <= a.deadline) return false;  // a zero limit fails at once
    __hip_atomic_store(a.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    fail_sh = 1;
    return true;
  };

  // Input of entry s: the launch input, or the output of the producer's last chunk.
  auto input_of = [&](const PassStage& ps, int s, const uint16_t** x, int* ldx, int* norm) {
    const int back = chunk_back(ps);
    if (back == 0) {
      *x = a.x;
      *ldx = a.ldx0;
      *norm = a.norm0;
    } else {
      const PassStage pr = stage_at(s - back);
      *x = pr.y16;
      *ldx = pr.N;
      *norm = 1;
    }
  };

  // Integer modes: the row statistics of the staged input (this thread's sums, max, min) combined over
  // the row's waves, then the row parameters (mean, 1/std, code scale) in LDS, behind barriers E
  // and F; computed where `want`.
  auto finish_params = [&](double su, double sq, float mx, float mn, int K, int norm, bool want)
      __attribute__((always_inline)) {
    su = wave_sum_dpp64(su);
    sq = wave_sum_dpp64(sq);
    mx = wave_max_dpp(mx);
    mn = wave_min_dpp(mn);
    if (lane == 0) {
      stat_sum[0][cw] = su;
      stat_sum[1][cw] = sq;
      stat_mm[0][cw] = mx;
      stat_mm[1][cw] = mn;
    }
    lds_barrier();  // E
    // Row parameters, one wave per row: lane u reads the statistics of the row's u-th wave.
    if (want && cw < M) {
      const int m = cw;
      const bool mine = lane < units_per_row;
      const int u = m * units_per_row + (mine ? lane : 0);
      const double tsu = lanes8_sum_dpp64(mine ? stat_sum[0][u] : 0.0);
      const double tsq = lanes8_sum_dpp64(mine ? stat_sum[1][u] : 0.0);
      const float xmax = lanes8_reduce_dpp(mine ? stat_mm[0][u] : -INFINITY, [](float p, float q) { return fmaxf(p, q); });
      const float xmin = lanes8_reduce_dpp(mine ? stat_mm[1][u] : INFINITY, [](float p, float q) { return fminf(p, q); });
      if (lane == 0) {
        double mu = 0.0, inv = 0.0;
        if (norm) norm_params64(tsu, tsq, xmax, xmin, K, mu, inv);
        row_mu64[m] = mu;
        row_inv64[m] = inv;
        const float amax = norm ? fmaxf(h2f(norm_h64(xmax, mu, inv)), -h2f(norm_h64(xmin, mu, inv)))
                                : fmaxf(xmax, -xmin);
        row_c[m] = h2f(f2h(amax / (float)kPassQmax<MODE>));
      }
    }
    lds_barrier();  // F
  };

  // W4A16 (input complete: after the grid barrier, or from the previous launch): raw fp16 rows of
  // this entry's K chunk straight into LDS, [M][K] row-major, by direct DMA, 64 pieces (1 KiB) per
  // wave instruction.  The row statistics for the epilogue are taken after barrier G, while the
  // contraction runs, by one control wave per row (needed at barrier A); a chunked linear sums
  // them over its chunks and forms the row parameters at its last chunk.
  auto stage_in16 = [&](int s, bool has) __attribute__((always_inline)) {
    const PassStage ps = stage_at(s);
    const int K = ps.K;
    const uint16_t* xin;
    int ldx, norm;
    input_of(ps, s, &xin, &ldx, &norm);
    const uint16_t* x = xin + chunk_g0(ps) * kGroup;  // the chunk's first column
    const int nb = K / 8;  // pieces per row
    if (has) {
      // the wave's chunks q = cw, cw + kCW, ... of M * cpr: (row, 64-piece column block), no division
      const int cpr = (nb + 63) >> 6;
      int m = 0, c = cw;
      while (c >= cpr) { c -= cpr; ++m; }
      while (m < M) {
        const int pi = (c << 6) + lane;
        if (pi < nb) dma_to_lds_sc1(x + (size_t)m * ldx + 8 * pi, lds_base + (uint32_t)(m * K + 8 * (c << 6)) * 2u);
        c += kCW;
        while (c >= cpr) { c -= cpr; ++m; }
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    lds_barrier();  // G
    for (int m = cw; has && m < M; m += kCW) {
      float mu = 0.f, inv = 1.f;
      if (norm) {
        const uint4* r = reinterpret_cast<const uint4*>(dyn_lds) + (size_t)m * nb;
        float su = 0.f, sq = 0.f, mx = 0.f, mn = 0.f;
        for (int i0 = 0; i0 < nb; i0 += 256) {  // four LDS reads in flight per lane
          uint4 v[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int i = i0 + 64 * u + lane;
            v[u] = i < nb ? r[i] : make_uint4(0u, 0u, 0u, 0u);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) stats_block8(v[u], su, sq, mx, mn);  // zero pieces add nothing
        }
        su = wave_sum_dpp(su);
        sq = wave_sum_dpp(sq);
        if (!chunk_first(ps)) {  // the linear's earlier chunks (this wave's own row, in LDS)
          su += row_su[m];
          sq += row_sq[m];
        }
        if (!chunk_last(ps)) {
          if (lane == 0) {
            row_su[m] = su;
            row_sq[m] = sq;
          }
          continue;
        }
        norm_params(su, sq, ps.gfull * kGroup, mu, inv);
      }
      if (lane == 0) {
        row_a[m] = mu;
        row_b[m] = inv;
      }
    }
  };

  // The integer modes at one row: the row staged through registers (statistics, scale,
  // quantisation, then LDS).  From the launch's second stage on, the input is being written by other
  // workgroups: pieces that still hold kEmpty are read again until all hold data or the deadline
  // passes.  Each thread holds P pieces, P a compile-time bucket of the stage's pieces per thread
  // chosen with a uniform branch.  The loads are unconditional: a load under a condition is merged
  // with the old value by a select, and the compiler then keeps two copies of all pieces live.
  // Pieces past this thread's count are read (next row, or zeros past the buffer resource's extent)
  // and not used.  Rows wider than P pieces per thread would be taken in H rounds of P pieces: each
  // round loaded (polled) and added to the statistics, then, after the row parameters, every round
  // but the last reloaded to be quantised.  The passes call it with H = 1 only (it staged the wider
  // rows of 3-4 rows before the shared codes); the round loop stays because the kernel written
  // without it compiled to another schedule that made the one-row draft pass 2% slower.
  auto stage_in4 = [&](auto pc, auto hc, int s, bool has) __attribute__((always_inline)) {
    constexpr int P = decltype(pc)::value;
    constexpr int H = decltype(hc)::value;
    const PassStage ps = stage_at(s);
    const int K = ps.K;  // integer modes take whole linears (no chunks)
    const uint16_t* x;
    int ldx, norm;
    input_of(ps, s, &x, &ldx, &norm);
    const int nb = K / 8;  // pieces per row
    // A whole wave serves one row (gsz >= 128), so `active` is wave-uniform.
    const bool active = has && my_row < M;
    const int np = row_tid < nb ? (nb - row_tid + gsz - 1) / gsz : 0;  // this thread's pieces
    // piece j of this thread: byte offset voff + j * pstride
    const __amdgpu_buffer_rsrc_t rs = sc1_rsrc(x, (uint32_t)(((M - 1) * ldx + K) * 2));
    const uint32_t voff = (uint32_t)(((my_row < M ? my_row : 0) * ldx + 8 * row_tid) * 2);
    const uint32_t pstride = (uint32_t)gsz * 16u;
    uint4 v[P];
    double su = 0.0, sq = 0.0;
    float mx = -INFINITY, mn = INFINITY;
#pragma unroll 1
    for (int h = 0; h < H; ++h) {
      const int nh = np - h * P;  // this round's pieces (may be <= 0)
      if (active) {
#pragma unroll
        for (int j = 0; j < P; ++j) v[j] = load_sc1(rs, voff, (uint32_t)(h * P + j) * pstride);
        if (s > 0) {
          auto pending = [&]() {
            uint32_t m = 0;
#pragma unroll
            for (int j = 0; j < P; ++j)
              if (j < nh && has_empty(v[j])) m |= 1u << j;
            return m;
          };
          const long long t0 = wall_clock64();
          while (a.deadline <= 0 || __any(pending() != 0u)) {
            if (wait_failed(t0)) break;
            __builtin_amdgcn_s_sleep(1);
#pragma unroll
            for (int j = 0; j < P; ++j)
              v[j] = load_sc1(rs, voff, (uint32_t)(h * P + j) * pstride);  // data, once there, stays
          }
        }
#pragma unroll
        for (int j = 0; j < P; ++j)
          if (j < nh) stats_block8_64(v[j], su, sq, mx, mn);
      }
    }
    su = wave_sum_dpp64(su);
    sq = wave_sum_dpp64(sq);
    mx = wave_max_dpp(mx);
    mn = wave_min_dpp(mn);
    if (lane == 0) {
      stat_sum[0][cw] = su;
      stat_sum[1][cw] = sq;
      stat_mm[0][cw] = mx;
      stat_mm[1][cw] = mn;
    }
    lds_barrier();  // E
    // Row parameters, one wave per row: lane u reads the statistics of the row's u-th wave.
    if (has && cw < M) {
      const int m = cw;
      const bool mine = lane < units_per_row;
      const int u = m * units_per_row + (mine ? lane : 0);
      const double tsu = lanes8_sum_dpp64(mine ? stat_sum[0][u] : 0.0);
      const double tsq = lanes8_sum_dpp64(mine ? stat_sum[1][u] : 0.0);
      const float xmax = lanes8_reduce_dpp(mine ? stat_mm[0][u] : -INFINITY, [](float p, float q) { return fmaxf(p, q); });
      const float xmin = lanes8_reduce_dpp(mine ? stat_mm[1][u] : INFINITY, [](float p, float q) { return fminf(p, q); });
      if (lane == 0) {
        double mu = 0.0, inv = 0.0;
        if (norm) norm_params64(tsu, tsq, xmax, xmin, K, mu, inv);
        row_mu64[m] = mu;
        row_inv64[m] = inv;
        const float amax = norm ? fmaxf(h2f(norm_h64(xmax, mu, inv)), -h2f(norm_h64(xmin, mu, inv)))
                                : fmaxf(xmax, -xmin);
        row_c[m] = h2f(f2h(amax / (float)kPassQmax<MODE>));
      }
    }
    lds_barrier();  // F
    if (active) {
      int8_t* xq = reinterpret_cast<int8_t*>(dyn_lds) + (size_t)my_row * K + 8 * row_tid;
      const double mu = row_mu64[my_row], inv = row_inv64[my_row];
      const float sc = row_c[my_row];
#pragma unroll 1
      for (int h = H - 1; h >= 0; --h) {  // the last round first: its pieces are still in registers
        const int nh = np - h * P;
        if (h < H - 1) {
#pragma unroll
          for (int j = 0; j < P; ++j) v[j] = load_sc1(rs, voff, (uint32_t)(h * P + j) * pstride);
        }
#pragma unroll
        for (int j = 0; j < P; ++j) {
          if (j < nh) {
            uint4 w = v[j];
            if (norm) w = norm_block8_64(w, mu, inv);
            uint2 op, lg;
            quant_block8<kPassQmax<MODE>>(w, sc, op, lg);
            *reinterpret_cast<uint2*>(xq + (h * P + j) * (pstride / 2)) = op;
          }
        }
      }
    }
    lds_barrier();  // G
  };

  // The integer modes above one row, with shared codes: the row statistics as in stage_in4 (rounds
  // of P pieces per thread, each polled until complete and added up, none kept), then each
  // workgroup standardises and quantises only its share of the rows -- pieces [bid * per, (bid + 1)
  // * per) of the M * K / 8 pieces, at most one per control thread -- and stores the codes to the
  // stage's code buffer with device-coherent stores (W4A4 a byte per code, W4A8 16 bits).  It then
  // reads the whole code buffer (16-byte pieces, polled until none holds the empty code) into LDS.
  // Every workgroup takes part, with or without sets in the stage, so that all shares get written;
  // only those with sets read the codes.  This replaces the per-workgroup quantisation of all M * K
  // values (whose time grows with the rows and with K) by one more all-to-all exchange.
  auto stage_in4s = [&](auto pc, int s, bool has) __attribute__((always_inline)) {
    constexpr int P = decltype(pc)::value;
    const PassStage ps = stage_at(s);
    const int K = ps.K;
    const uint16_t* x;
    int ldx, norm;
    input_of(ps, s, &x, &ldx, &norm);
    const int nb = K / 8;
    const bool part = !fail_sh;
    const bool active = part && my_row < M;
    const int np = row_tid < nb ? (nb - row_tid + gsz - 1) / gsz : 0;
    const int H = ((nb + gsz - 1) / gsz + P - 1) / P;  // rounds (uniform)
    const __amdgpu_buffer_rsrc_t rs = sc1_rsrc(x, (uint32_t)(((M - 1) * ldx + K) * 2));
    const uint32_t voff = (uint32_t)(((my_row < M ? my_row : 0) * ldx + 8 * row_tid) * 2);
    const uint32_t pstride = (uint32_t)gsz * 16u;
    const int per = (M * nb + grid - 1) / grid;  // <= gsz (host check): one piece per thread at most
    const int q0 = bid * per - my_row * nb;      // this row's share: pieces [q0, q0 + per) of the row
    uint4 mine = make_uint4(0u, 0u, 0u, 0u);
    int mine_idx = -1;
    double su = 0.0, sq = 0.0;
    float mx = -INFINITY, mn = INFINITY;
#pragma unroll 1
    for (int h = 0; h < H; ++h) {
      const int nh = np - h * P;
      if (active) {
        uint4 v[P];
#pragma unroll
        for (int j = 0; j < P; ++j) v[j] = load_sc1(rs, voff, (uint32_t)(h * P + j) * pstride);
        if (s > 0) {
          auto pending = [&]() {
            uint32_t m = 0;
#pragma unroll
            for (int j = 0; j < P; ++j)
              if (j < nh && has_empty(v[j])) m |= 1u << j;
            return m;
          };
          const long long t0 = wall_clock64();
          while (a.deadline <= 0 || __any(pending() != 0u)) {
            if (wait_failed(t0)) break;
            __builtin_amdgcn_s_sleep(1);
#pragma unroll
            for (int j = 0; j < P; ++j) v[j] = load_sc1(rs, voff, (uint32_t)(h * P + j) * pstride);
          }
        }
#pragma unroll
        for (int j = 0; j < P; ++j) {
          if (j < nh) {
            stats_block8_64(v[j], su, sq, mx, mn);
            const int idx = row_tid + (h * P + j) * gsz;
            if (idx >= q0 && idx < q0 + per) {
              mine = v[j];
              mine_idx = idx;
            }
          }
        }
      }
    }
    finish_params(su, sq, mx, mn, K, norm, part);
    constexpr int CB = MODE == 1 ? 1 : 2;  // bytes per shared code
    int8_t* const codes =
        chunk_back(ps) == 0 ? a.codes_in
                            : a.codes_base + (reinterpret_cast<const unsigned char*>(x) - a.stage_base) * CB / 2;
    // A workgroup one of whose waits failed publishes nothing (its statistics may be incomplete), so
    // every other workgroup's wait for the codes fails too and no output is computed from them.
    if (active && mine_idx >= 0 && !fail_sh) {
      uint4 w = mine;
      if (norm) w = norm_block8_64(w, row_mu64[my_row], row_inv64[my_row]);
      uint2 op, lg;
      quant_block8<kPassQmax<MODE>>(w, row_c[my_row], op, lg);
      const __amdgpu_buffer_rsrc_t rw = sc1_rsrc(codes, (uint32_t)(M * K * CB));
      if constexpr (CB == 1) {
        typedef int v2i_t __attribute__((ext_vector_type(2)));
        __builtin_amdgcn_raw_buffer_store_b64(v2i_t{(int)op.x, (int)op.y}, rw, my_row * K + 8 * mine_idx, 0, kSc1);
      } else {  // each code byte sign-extended to 16 bits, same order
        auto widen = [](uint32_t b) {  // bytes 0, 1 of b -> 16-bit words 0, 1
          return ((uint32_t)((int32_t)(b << 24) >> 24) & 0xFFFFu) | ((uint32_t)((int32_t)(b << 16) >> 24) << 16);
        };
        const int4_t v16 = int4_t{(int)widen(op.x), (int)widen(op.x >> 16), (int)widen(op.y), (int)widen(op.y >> 16)};
        __builtin_amdgcn_raw_buffer_store_b128(v16, rw, (my_row * K + 8 * mine_idx) * 2, 0, kSc1);
      }
    }
    if (has && !fail_sh) {
      constexpr int Q = 4;  // 16-byte code pieces per thread and round (8 spilled registers)
      const int nq = M * K * CB / 16;
      const __amdgpu_buffer_rsrc_t rc = sc1_rsrc(codes, (uint32_t)(M * K * CB));
#pragma unroll 1
      for (int b0 = 0; b0 < nq; b0 += Q * kCT) {
        uint4 c[Q];
#pragma unroll
        for (int u = 0; u < Q; ++u) c[u] = load_sc1(rc, (uint32_t)(b0 + u * kCT + ct) * 16u, 0u);  // zeros past the end
        auto pending = [&]() {
          uint32_t m = 0;
#pragma unroll
          for (int u = 0; u < Q; ++u)
            if (has_code_empty<CB>(c[u])) m |= 1u << u;
          return m;
        };
        const long long t0 = wall_clock64();
        while (a.deadline <= 0 || __any(pending() != 0u)) {
          if (wait_failed(t0)) break;
          __builtin_amdgcn_s_sleep(1);
#pragma unroll
          for (int u = 0; u < Q; ++u) c[u] = load_sc1(rc, (uint32_t)(b0 + u * kCT + ct) * 16u, 0u);
        }
#pragma unroll
        for (int u = 0; u < Q; ++u) {
          const int q = b0 + u * kCT + ct;
          if (q < nq) {
            if constexpr (CB == 1) {
              reinterpret_cast<uint4*>(dyn_lds)[q] = c[u];
            } else {  // the low byte of each 16-bit code
              auto narrow = [](uint32_t lo, uint32_t hi) {
                return (lo & 0xFFu) | ((lo >> 8) & 0xFF00u) | ((hi & 0xFFu) << 16) | ((hi & 0xFF0000u) << 8);
              };
              reinterpret_cast<uint2*>(dyn_lds)[q] = make_uint2(narrow(c[u].x, c[u].y), narrow(c[u].z, c[u].w));
            }
          }
        }
      }
    }
    lds_barrier();  // G
  };

  auto prologue = [&](int s) {
    const bool has = stage_sets(stage_at(s), bid, grid) > 0 && !fail_sh;
    if constexpr (MODE == 0) {
      stage_in16(s, has);
    } else {
      if constexpr (kPassShared<MODE, WIDE>) {
        stage_in4s(std::integral_constant<int, 4>{}, s, has);  // rounds of 4 pieces (8 spilled registers)
      } else {  // one row: at most 8 pieces per thread (host check)
        const int npmax = (stage_at(s).K / 8 + gsz - 1) / gsz;
        using one = std::integral_constant<int, 1>;
        if (npmax <= 2)
          stage_in4(std::integral_constant<int, 2>{}, one{}, s, has);
        else if (npmax <= 4)
          stage_in4(std::integral_constant<int, 4>{}, one{}, s, has);
        else
          stage_in4(std::integral_constant<int, 8>{}, one{}, s, has);
      }
    }
  };

  // one timestamp of the running entry, from the first control thread (trace instances only)
  auto trace_mark = [&](int s, int k) __attribute__((always_inline)) {
    if constexpr (TRACE) {
      if (ct == 0)
        a.trace[((size_t)(a.trace_e0 + s) * (size_t)grid + (size_t)bid) * 4 + k] = (unsigned long long)wall_clock64();
    }
  };

  constexpr int kCarry = MODE == 0 ? kCtrlSlots : 1;
  Acc carry[kCarry];  // W4A16 chunked linears: this wave's partial sums of the earlier chunks
#pragma unroll
  for (int pi = 0; pi < kCarry; ++pi) carry[pi] = Acc{0, 0, 0, 0};
  for (int s = 0; s < a.n_stages; ++s) {
    prologue(s);
    if (__builtin_amdgcn_readfirstlane(fail_sh)) return;
    trace_mark(s, 0);
    lds_barrier();  // A: the streaming waves have parked the partials of stage s
    trace_mark(s, 1);
    const PassStage ps = stage_at(s);
    const int sets = stage_sets(ps, bid, grid);
    const bool final_out = a.last_is_final && s + 1 == a.n_stages;
    const bool want_t1 = final_out && a.top1 != nullptr;
    // Top-1 partials of this lane's rows 4 (lane >> 4) + j, column lane & 15
    Msi t1v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) t1v[j] = Msi{-INFINITY, 0.0f, 0x7fffffff};
    if (sets > 0) {
      // sum, in a fixed order, the S partials of each (set, row block) and store the outputs; a
      // chunked linear's earlier chunks are added from `carry` (same (set, row block) per slot pi
      // in every chunk, since its chunks share one split) and only its last chunk stores
      const int S = 1 << ps.s_log2, R = kSW >> ps.s_log2;
      const int nrb = (ps.N + 15) >> 4, N = ps.N;
      const int norm = chunk_back(ps) == 0 ? a.norm0 : 1;
      const bool first = chunk_first(ps), last = chunk_last(ps);
#pragma unroll
      for (int pi = 0; pi < kCtrlSlots; ++pi) {
        const int p = cw + pi * kCW;
        if (p >= sets * R) break;
        const int si = p / R, r2 = p - si * R;
        const int rb = (bid + si * grid) * R + r2;
        Acc v = red[si][r2 * S][lane];
        for (int s2 = 1; s2 < S; ++s2) v += red[si][r2 * S + s2][lane];
        if constexpr (MODE == 0) {
          if (!first) v += carry[pi % kCarry];
          if (!last) {
            carry[pi % kCarry] = v;
            continue;
          }
        }
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
              float outv;
              uint16_t h;
              if constexpr (MODE == 0) {
                outv = v[j];
                if (norm) outv = (outv - row_a[m] * rowsum) * row_b[m];
                h = f2h(outv);
              } else {  // exact product, rounded once
                const double o64 = v[j] * (double)row_c[m];
                outv = (float)o64;
                h = f64_to_f16_rn(o64);
              }
              if (final_out) {
                if (a.out) a.out[(size_t)m * N + n] = outv;
                if (want_t1) t1v[j] = msi_merge(t1v[j], Msi{outv, 1.0f, n});
              } else {  // device-coherent store, read by other workgroups in the next stage
                if (h == kEmpty) h = 0x7E00u;
                __hip_atomic_store(ps.y16 + (size_t)m * N + n, h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              }
            }
          }
        }
      }
    }
    if (want_t1) top1_epilogue(Top1Out{a.top1, a.top1_prob, a.t1_stats, a.t1_cnt}, t1v, t1_wave, &t1_arrive, cw, lane,
                               bid, grid, M);
    bool marked = false;
    if constexpr (MODE == 0) {
      // grid barrier after a linear's last chunk: all outputs of the linear are in memory (the
      // streaming waves take the same condition)
      if (s + 1 < a.n_stages && chunk_last(ps)) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's output stores have completed
        lds_barrier();  // B
        trace_mark(s, 2);
        const unsigned epoch = a.epoch0 + (unsigned)(s + 1);
        if (ct == 0)
          __hip_atomic_store(a.flags + (size_t)bid * kFlagStride, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // every workgroup watches all flags itself: one round trip, no `go` relay
        for (int t = ct; t < grid; t += kCT)
          if (!wait_at_least(a.flags + (size_t)t * kFlagStride, epoch, a)) fail_sh = 1;
        lds_barrier();  // C
        trace_mark(s, 3);
        marked = true;
      }
    }
    if (!marked) {  // no grid barrier: the integer modes' data-carried hand-over, or the last entry
      trace_mark(s, 2);
      trace_mark(s, 3);
    }
  }
}

// Start of a pass: fills the stage outputs with kEmpty (integer modes; device-coherent stores) and the
// n16c 16-byte pieces after them (the shared codes) with cfill, the
// final output with NaN and the Top-1 outputs with -1 and NaN, and zeroes the control words (the
// Top-1 arrival counter and the error word, then n_flags arrival flags kFlagStride apart).
__global__ __launch_bounds__(256) void pass_reset_kernel(uint4* bufs, uint32_t n16, uint32_t n16c, uint32_t cfill,
                                                         unsigned* ctrl, int n_flags,
                                                         float* out, uint32_t n_out, int32_t* top1, float* top1_prob,
                                                         int n_top1) {
  if (blockIdx.x == 0 && top1) {
    for (int i = threadIdx.x; i < n_top1; i += 256) {
      top1[i] = -1;
      if (top1_prob) top1_prob[i] = __builtin_nanf("");
    }
  }
  if (blockIdx.x == 0) {
    if (threadIdx.x < 2) __hip_atomic_store(ctrl + threadIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int i = threadIdx.x; i < n_flags; i += 256)
      __hip_atomic_store(ctrl + (size_t)(i + 1) * kFlagStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(bufs, (short)0, (int)((n16 + n16c) * 16u), (int)kBufWord3);
  const int4_t e = int4_t{-1, -1, -1, -1};
  const int ce = (int)cfill;
  const int4_t ec = int4_t{ce, ce, ce, ce};
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < n16 + n16c; i += gridDim.x * 256u)
    __builtin_amdgcn_raw_buffer_store_b128(i < n16 ? e : ec, r, (int)(i * 16u), 0, kSc1);
  if (out) {
    for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < n_out; i += gridDim.x * 256u)
      out[i] = __builtin_nanf("");
  }
}

// ------------------------------------------------------------------ host side

static int pick_pass_split(int N, int K, int grid);

// K chunks of a linear at M rows: W4A16 stages M fp16 rows of each chunk in LDS, so K is split
// into equal chunks of whole groups that fit; the integer modes take whole linears.  -1: no fit.
static int pass_chunks(int mode, int M, int K) {
  if (mode != QS_W4A16) return (size_t)M * K <= kPassLdsStageInt ? 1 : -1;
  const int gmax = (int)(kPassLdsStage / ((size_t)M * kGroup * 2));  // groups per chunk
  if (gmax < 1) return -1;
  const int G = K / kGroup;
  return (G + gmax - 1) / gmax;
}
// Groups in each chunk of a linear split into nch chunks (the last may be shorter).
static int chunk_groups(int K, int nch) { return (K / kGroup + nch - 1) / nch; }

// Workgroup share of the shared-code staging fits: at most one 16-byte piece per control thread.
static bool pass_share_fits(int M, int K, int grid) {
  const int gsz = kCT / (M <= 1 ? 1 : M <= 2 ? 2 : 4);
  return (M * (K / 8) + grid - 1) / grid <= gsz;
}
// The pass stages its inputs through the shared codes (kPassShared): the integer modes above one row.
static bool pass_shared_codes(int mode, int M) { return (mode == QS_W4A4 || mode == QS_W4A8) && M > 1; }
static size_t pass_code_bytes(int mode) { return mode == QS_W4A8 ? 2 : 1; }  // per shared code

bool pass_eligible(int mode, int M, const qs_linear_desc* c, int n) {
  if (M > pass_max_rows(mode)) return false;
  const int grid = device_info()->num_cus;
  if (grid < 1 || grid > kMaxPassWorkgroups) return false;
  const int gsz = kCT / (M <= 1 ? 1 : M <= 2 ? 2 : 4);  // control threads per input row
  for (int i = 0; i < n; ++i) {
    const int nch = pass_chunks(mode, M, c[i].K);
    if (nch < 1 || nch > kMaxPassStages) return false;
    if (mode != QS_W4A16 && M <= 1 && c[i].K / 8 > 8 * gsz) return false;  // one-row staging: 8 pieces per thread
    if (pass_shared_codes(mode, M) && !pass_share_fits(M, c[i].K, grid)) return false;
    if (pick_pass_split(c[i].N, chunk_groups(c[i].K, nch) * kGroup, grid) < 0) return false;
  }
  return true;
}

// W4A16 takes up to 14 rows (row M of the 16-row MFMA operand is the all-ones row of the
// standardisation's weight sums).  Measured over the Llama-3-8B-shaped stack: 5, 6, 8, 12 rows
// 1.41, 1.40, 1.43, 1.90 ms per pass against 2.1-2.3 ms with one launch per linear; at 15 rows every
// 4096-wide linear needs two K chunks and the pass took 2.25 ms against 2.12 ms.
//
// The integer modes take up to 4 rows (the row statistics are taken in every workgroup, so the
// staging grows with M): W4A4 pass 1.38 / 1.79 / 1.92 / 1.94 ms at 1 / 2 / 3 / 4 rows (shared codes
// above one row; 2.34 / 2.41 ms at 3 / 4 rows with every workgroup quantising all rows), W4A8
// 1.39 / 1.80 / 1.97 / 2.02 ms, against 2.97 ms with one launch per linear at 4 rows.
int pass_max_rows(int mode) { return mode == QS_W4A16 ? 14 : (mode == QS_W4A4 || mode == QS_W4A8) ? 4 : 0; }

size_t pass_stage_bytes(int M, const qs_linear_desc* c, int n) {
  size_t b = 0;
  for (int i = 0; i + 1 < n; ++i) b += align_up((size_t)M * c[i].N * 2, 256);
  return b;
}
// Stage outputs and, for the integer modes above one row, the shared codes after them: one byte (W4A4)
// or two (W4A8) per fp16 output, at half or all of its offset (so each stage's codes start 128-byte
// aligned), then the codes of the pass's input.
size_t pass_area_bytes(int mode, int M, const qs_linear_desc* c, int n) {
  const size_t sb = pass_stage_bytes(M, c, n);
  if (!pass_shared_codes(mode, M)) return sb;
  const size_t cb = pass_code_bytes(mode);
  return sb + sb * cb / 2 + align_up((size_t)M * c[0].K * cb, 256);
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

// Launch boundaries (first linear of each launch, then n): linears are packed in order into
// launches of at most kMaxPassStages entries, balanced in entries, never splitting a linear's chunks.
static std::vector<int> pass_launch_plan(int mode, int M, const qs_linear_desc* c, int n) {
  std::vector<int> nch(n);
  int total = 0;
  for (int i = 0; i < n; ++i) total += nch[i] = pass_chunks(mode, M, c[i].K);
  const int launches = (total + kMaxPassStages - 1) / kMaxPassStages;
  const int target = (total + launches - 1) / launches;
  std::vector<int> first{0};
  int in_launch = 0;
  for (int i = 0; i < n; ++i) {
    if (in_launch > 0 && in_launch + nch[i] > target) {
      first.push_back(i);
      in_launch = 0;
    }
    in_launch += nch[i];
  }
  first.push_back(n);
  return first;
}

int pass_launch_count(int mode, int M, const qs_linear_desc* c, int n) {
  return (int)pass_launch_plan(mode, M, c, n).size() - 1;
}

size_t pass_top1_bytes(int M) { return align_up((size_t)M * kMaxPassWorkgroups * 16, 256); }

static std::atomic<int> g_barrier_timeout_us{200000};
int pass_barrier_timeout_us() { return g_barrier_timeout_us.load(); }
void set_pass_barrier_timeout_us(int us) { g_barrier_timeout_us.store(us); }

int pass_entry_count(int mode, int M, const qs_linear_desc* c, int n) {
  int e = 0;
  for (int i = 0; i < n; ++i) e += pass_chunks(mode, M, c[i].K);
  return e;
}

int launch_pass(int mode, const uint16_t* x, int M, const qs_linear_desc* c, int n, float* out,
                unsigned* ctrl, uint16_t* stage_out, hipStream_t st, const PassTop1* t1,
                unsigned long long* trace) {
  const DeviceInfo* di = device_info();
  const int grid = di->num_cus;
  const bool wide = mode != QS_W4A16 && M > 1;
  // 0 W4A16, 1 W4A4, 2 W4A8, 3 W4A4 wide, 4 W4A8 wide; + 5: the same recording boundary timestamps
  const int variant = mode + (wide ? 2 : 0) + (trace ? 5 : 0);
  const void* fns[10] = {reinterpret_cast<const void*>(pass_kernel<0, false, false>),
                         reinterpret_cast<const void*>(pass_kernel<1, false, false>),
                         reinterpret_cast<const void*>(pass_kernel<2, false, false>),
                         reinterpret_cast<const void*>(pass_kernel<1, true, false>),
                         reinterpret_cast<const void*>(pass_kernel<2, true, false>),
                         reinterpret_cast<const void*>(pass_kernel<0, false, true>),
                         reinterpret_cast<const void*>(pass_kernel<1, false, true>),
                         reinterpret_cast<const void*>(pass_kernel<2, false, true>),
                         reinterpret_cast<const void*>(pass_kernel<1, true, true>),
                         reinterpret_cast<const void*>(pass_kernel<2, true, true>)};
  static int lds_set[10] = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
  if (!lds_set[variant]) {
    const int limit = (int)(mode == QS_W4A16 ? kPassLdsStage : kPassLdsStageInt);
    if (hipFuncSetAttribute(fns[variant], hipFuncAttributeMaxDynamicSharedMemorySize, limit) != hipSuccess) {
      (void)hipGetLastError();  // report it here, not at the caller's next HIP call
      return QS_ERR_HIP;
    }
    lds_set[variant] = 1;
  }
  size_t lds = kPassLdsMin;
  for (int i = 0; i < n; ++i) {
    const int nch = pass_chunks(mode, M, c[i].K);
    const size_t b = (size_t)M * chunk_groups(c[i].K, nch) * kGroup * (mode == QS_W4A16 ? 2 : 1);
    lds = b > lds ? b : lds;
  }

  // Stage outputs of the whole pass -> kEmpty, shared codes -> empty, error word -> 0.
  const size_t sb = pass_stage_bytes(M, c, n);
  if (pass_area_bytes(mode, M, c, n) > (size_t)0x7FFFFF00) return QS_ERR_UNSUPPORTED;  // one buffer resource spans them
  const uint32_t n16 = mode != QS_W4A16 ? (uint32_t)(sb / 16) : 0u;  // W4A16 stages hand over at a grid barrier
  const uint32_t n16c = (uint32_t)((pass_area_bytes(mode, M, c, n) - sb) / 16);  // shared codes
  const uint32_t cfill = mode == QS_W4A8 ? kCodeEmpty16 : kCodeEmpty;
  const size_t n_out = out ? (size_t)M * c[n - 1].N : 0;
  if (n_out > 0xFFFFFFFFu) return QS_ERR_UNSUPPORTED;
  const size_t work = (size_t)n16 + n16c + n_out / 4;
  const unsigned rblocks = (unsigned)((work + 255) / 256 < 1024 ? (work + 255) / 256 : 1024);
  hipLaunchKernelGGL(pass_reset_kernel, dim3(rblocks > 0 ? rblocks : 1), dim3(256), 0, st,
                     reinterpret_cast<uint4*>(stage_out), n16, n16c, cfill, ctrl, mode == QS_W4A16 ? grid : 0, out,
                     (uint32_t)n_out, t1 ? t1->top1 : nullptr, t1 ? t1->top1_prob : nullptr, M);
  int rc = launch_status();
  if (rc != QS_OK) return rc;

  // Output of linear i at the running offset: outputs are laid out in chain order.
  unsigned char* const base = reinterpret_cast<unsigned char*>(stage_out);
  size_t off = 0;            // offset of the next linear's output
  uint16_t* prev = nullptr;  // output of the linear before the launch's first
  const std::vector<int> plan = pass_launch_plan(mode, M, c, n);
  int entry0 = 0;  // pass-wide index of the launch's first entry (epochs count entries)
  for (size_t l = 0; l + 1 < plan.size(); ++l) {
    const int i0 = plan[l], i1 = plan[l + 1];
    PassArgs a{};
    if (i0 == 0) {
      a.x = x;
      a.ldx0 = c[0].K;
      a.norm0 = 0;
    } else {
      a.x = prev;  // written by the previous launch
      a.ldx0 = c[i0 - 1].N;
      a.norm0 = 1;
    }
    a.out = out;
    a.last_is_final = i1 == n;
    if (t1 && a.last_is_final) {
      a.top1 = t1->top1;
      a.top1_prob = t1->top1_prob;
      a.t1_stats = t1->stats;
      a.t1_cnt = ctrl;  // the control region's first word
    }
    a.error = ctrl + 1;
    a.flags = ctrl + kFlagStride;
    a.epoch0 = (unsigned)entry0;
    a.trace = trace;
    a.trace_e0 = entry0;
    a.stage_base = base;
    a.codes_base = reinterpret_cast<int8_t*>(base + sb);
    // the launch's input: the pass input's own code area, or the codes of the previous launch's output
    const size_t cb = pass_code_bytes(mode);
    a.codes_in = i0 == 0 ? reinterpret_cast<int8_t*>(base + sb + sb * cb / 2)
                         : reinterpret_cast<int8_t*>(base + sb + (reinterpret_cast<unsigned char*>(prev) - base) * cb / 2);
    a.deadline = (long long)di->clock_khz * pass_barrier_timeout_us() / 1000;  // wall-clock ticks
    a.M = M;
    int e = 0;
    for (int i = i0; i < i1; ++i) {
      const qs_linear_desc& d = c[i];
      uint16_t* y16 = nullptr;
      if (i + 1 < n) {
        y16 = reinterpret_cast<uint16_t*>(base + off);
        off += align_up((size_t)M * d.N * 2, 256);
      }
      const int G = d.K / kGroup, nch = pass_chunks(mode, M, d.K), gc = chunk_groups(d.K, nch);
      const int sl = pick_pass_split(d.N, gc * kGroup, grid);  // one split for all chunks
      const int R = kPW >> sl;
      for (int j = 0; j < nch; ++j, ++e) {
        PassStage& p = a.st[e];
        const int g0 = j * gc;
        p.w = reinterpret_cast<const uint4*>(d.w_packed);
        p.sc = d.s_packed;
        p.y16 = y16;
        p.N = d.N;
        p.K = (G - g0 < gc ? G - g0 : gc) * kGroup;
        p.s_log2 = sl;
        p.nsets = ((d.N + 15) / 16 + R - 1) / R;
        p.gfull = G;
        const int back = i == i0 ? 0 : j + 1;  // the previous linear's last chunk
        p.chunk = g0 | (j == 0 ? 1 << 16 : 0) | (j + 1 == nch ? 1 << 17 : 0) | (back << 24);
      }
      if (y16) prev = y16;
    }
    a.n_stages = e;
    entry0 += e;
    switch (variant) {
      case 0: hipLaunchKernelGGL((pass_kernel<0, false, false>), dim3(grid), dim3(kPThreads), lds, st, a); break;
      case 1: hipLaunchKernelGGL((pass_kernel<1, false, false>), dim3(grid), dim3(kPThreads), lds, st, a); break;
      case 2: hipLaunchKernelGGL((pass_kernel<2, false, false>), dim3(grid), dim3(kPThreads), lds, st, a); break;
      case 3: hipLaunchKernelGGL((pass_kernel<1, true, false>), dim3(grid), dim3(kPThreads), lds, st, a); break;
      case 4: hipLaunchKernelGGL((pass_kernel<2, true, false>), dim3(grid), dim3(kPThreads), lds, st, a); break;
      case 5: hipLaunchKernelGGL((pass_kernel<0, false, true>), dim3(grid), dim3(kPThreads), lds, st, a); break;
      case 6: hipLaunchKernelGGL((pass_kernel<1, false, true>), dim3(grid), dim3(kPThreads), lds, st, a); break;
      case 7: hipLaunchKernelGGL((pass_kernel<2, false, true>), dim3(grid), dim3(kPThreads), lds, st, a); break;
      case 8: hipLaunchKernelGGL((pass_kernel<1, true, true>), dim3(grid), dim3(kPThreads), lds, st, a); break;
      default: hipLaunchKernelGGL((pass_kernel<2, true, true>), dim3(grid), dim3(kPThreads), lds, st, a); break;
    }
    rc = launch_status();
    if (rc != QS_OK) return rc;
  }
  return QS_OK;
}

}  // namespace qs
