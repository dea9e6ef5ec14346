// Verify/accept kernels for gfx950: softmax statistics, Top-1, greedy prefix
// acceptance, sampling acceptance and residual resampling.
//
// Method ([P3] kasblo.com, "Speculative Decodingとは？LLM生成を速くする方法"):
//   "greedy decodingでは一致するprefixを採用する" -- accept draft tokens while they
//   equal the target's argmax, replace the first mismatch by the target token,
//   add the target's extra token when all match;
//   "samplingでもtargetの確率分布を保つ" -- accept draft x with probability
//   min(1, p(x)/q(x)); on rejection draw from max(0, p - q) normalised.
//
// Layout of the work: a row of V logits (V = 128256 for the Llama-3 vocab) is
// split into chunks of 8192 logits for the statistics and 2048 for the draw,
// one 256-thread workgroup per (row, chunk) -- enough workgroups to fill the
// chip even for a single sequence.  Each statistics workgroup produces (max,
// sum exp(l - max), first argmax) in one pass: every thread forms its own
// triple, and triples are merged (max; lowest index among equal maxima; sums
// rescaled to the larger max) by DPP row steps and lane reads inside a wave,
// then across the 4 waves in LDS, in a fixed order.  The last workgroup of a
// sequence to finish merges the chunk partials the same way (so argmax ties
// resolve to the lowest index and the result is deterministic) and applies the
// acceptance rule.  Sampling then re-reads only the two rows per sequence that
// the final token is drawn from.  Draft ids are bounds-checked before use.
//
// Precision: statistics, Top-1 and acceptance probabilities are fp32.  The
// draw is fp64 end to end: the residual max(0, p - q) cancels wherever the two
// models agree, and its normalised values must hold 1e-5 even when the
// residual mass Z is a few 1e-4, where fp32 rounding of p alone (1e-7
// relative) moves them by 1e-7 / Z.  So the draw pass sums exp(l - max) of the
// two drawn-from rows in fp64 itself, and the finisher of a sequence forms the
// normalisers from those sums before any value is normalised.

#include "qs_msi.h"
#include "qs_device.h"
#include "qs_internal.h"

namespace qs {

constexpr int kVThreads = 256;
// Statistics workgroups take 8192 logits (32 per thread): at the batched scale the whole grid is
// then resident at once, so the arrival atomic each workgroup waits on before it retires is paid
// once, not once per round of workgroups.  Draw workgroups take 2048 (8 per thread): their fp64
// exponentials are slow, and a sequence's draw runs two of them back to back (its chunk sums, then
// the search inside the chosen chunk), so shorter chunks shorten that path.
// (16 and 64 per thread measured the same at B = 16, gamma = 7, warm and cold.)
constexpr int kStatPerThread = 32;
constexpr int kStatChunk = kVThreads * kStatPerThread;
constexpr int kPerThread = 8;
constexpr int kChunk = kVThreads * kPerThread;

// Chunk partial, 16 bytes: (max, lowest index attaining it, sum over the chunk of exp(l - max)).
struct Part {
  int w[4];
};

// What the final token of a sequence is drawn from.  The fp32 normalisers only classify slots as
// p > q; the draw itself uses fp64 normalisers formed from the draw pass's own sums.
struct SeqInfo {
  int n;         // accepted count (row of the final draw)
  int use_res;   // 1: draw from the residual max(0, p - q); 0: from p
  float mp, mq;  // row maxima: target row n, draft row n (when n < gamma)
  float sp, sq;  // fp32 normalisers sum exp(l - max) of the same rows
  int pad[2];
};

// Per-chunk fp64 sums of the unnormalised a_j = exp(lp_j - mp) and b_j = exp(lq_j - mq) of the
// drawn-from rows: over the chunk (a, b) and over its slots with p_j > q_j (ap, bp).  With
// S_p = sum a and S_q = sum b over the row, the chunk's residual mass is ap / S_p - bp / S_q and
// its p mass a / S_p.
struct Mass4 {
  double a, b, ap, bp;
};

static inline int stat_chunks(int V) { return (V + kStatChunk - 1) / kStatChunk; }
static inline int draw_chunks(int V) { return (V + kChunk - 1) / kChunk; }

// Workspace: first the per-sequence arrival counters, two 32-bit words in a 256-byte line of its
// own for each of up to QS_MAX_VERIFY_SEQS sequences (the atomics of different sequences would
// otherwise queue on one line), at a fixed place whatever the call's shape (zero before the first
// use; every call leaves them zero), then the chunk partials, per-sequence decisions and the fp64
// chunk sums of the draw.
constexpr int kCounterStride = 64;  // 32-bit words per sequence: one 256-byte line each
constexpr size_t kCounterBytes = (size_t)QS_MAX_VERIFY_SEQS * kCounterStride * 4;
size_t verify_counter_bytes() { return kCounterBytes; }
size_t verify_workspace(int B, int gamma, int V) {
  if (B > QS_MAX_VERIFY_SEQS) B = QS_MAX_VERIFY_SEQS;  // larger batches run block by block
  const size_t Cs = (size_t)stat_chunks(V), Cd = (size_t)draw_chunks(V);
  const size_t rows = (size_t)B * (2 * (size_t)gamma + 1);
  return kCounterBytes + align_up(rows * Cs * sizeof(Part), 256) + align_up((size_t)B * sizeof(SeqInfo), 256) +
         align_up((size_t)B * Cd * sizeof(Mass4), 256);
}

struct VerifyWs {
  Part* parts;
  SeqInfo* info;
  Mass4* csum;
  unsigned* cnt;   // arrivals at the statistics step (sequence b at cnt[kCounterStride b])
  unsigned* cnt2;  // arrivals at the draw step (sequence b at cnt2[kCounterStride b])
};
static VerifyWs carve(void* ws, int B, int gamma, int V) {
  const size_t Cs = (size_t)stat_chunks(V);
  const size_t rows = (size_t)B * (2 * (size_t)gamma + 1);
  unsigned char* p = static_cast<unsigned char*>(ws);
  VerifyWs w;
  w.cnt = reinterpret_cast<unsigned*>(p);
  w.cnt2 = w.cnt + kCounterStride / 2;
  p += kCounterBytes;
  w.parts = reinterpret_cast<Part*>(p);
  p += align_up(rows * Cs * sizeof(Part), 256);
  w.info = reinterpret_cast<SeqInfo*>(p);
  p += align_up((size_t)B * sizeof(SeqInfo), 256);
  w.csum = reinterpret_cast<Mass4*>(p);
  return w;
}

// e^x in fp64 for x <= 0, to 1e-14 relative: Cody-Waite reduction x = n ln2 + r, |r| <= ln2 / 2,
// with ln2 split in a 24-bit head (n * head is exact) and a tail, then the Taylor series of e^r
// to degree 11 (truncation below 7e-15).  Below -708 the result is 0 (e^-708 < 3e-308); -inf
// gives 0.  The sampling path needs about 1e-12 relative, well short of a correctly rounded exp,
// so this takes 15 fp64 operations where a general-purpose one takes several times that.
__device__ __forceinline__ double exp_nonpos_f64(double x) {
  constexpr double kLog2e = 0x1.71547652b82fep0;
  constexpr double kLn2Hi = 0x1.62e43p-1;
  constexpr double kLn2Lo = -0x1.05c610ca86c39p-29;
  const bool tiny = x < -708.0;
  const double xc = tiny ? -708.0 : x;
  const double n = __builtin_rint(xc * kLog2e);
  double r = __builtin_fma(-n, kLn2Hi, xc);
  r = __builtin_fma(-n, kLn2Lo, r);
  double p = 1.0 / 39916800.0;  // 1/11!
  p = __builtin_fma(p, r, 1.0 / 3628800.0);
  p = __builtin_fma(p, r, 1.0 / 362880.0);
  p = __builtin_fma(p, r, 1.0 / 40320.0);
  p = __builtin_fma(p, r, 1.0 / 5040.0);
  p = __builtin_fma(p, r, 1.0 / 720.0);
  p = __builtin_fma(p, r, 1.0 / 120.0);
  p = __builtin_fma(p, r, 1.0 / 24.0);
  p = __builtin_fma(p, r, 1.0 / 6.0);
  p = __builtin_fma(p, r, 0.5);
  p = __builtin_fma(p, r, 1.0);
  p = __builtin_fma(p, r, 1.0);
  return tiny ? 0.0 : __builtin_ldexp(p, (int)n);
}
// exp(l - m) in fp64 for fp32 logits l <= m: both convert exactly and their difference is exact.
__device__ __forceinline__ double exp_diff64(float l, float m) { return exp_nonpos_f64((double)l - (double)m); }

// Sum over the 64 lanes (all active) by the same DPP row steps as the merge below; every lane.
__device__ __forceinline__ double wave_sum_f64(double x) {
  x += dpp_v<0xB1>(x);
  x += dpp_v<0x4E>(x);
  x += dpp_v<0x141>(x);
  x += dpp_v<0x140>(x);
  return (readlane_v(x, 0) + readlane_v(x, 16)) + (readlane_v(x, 32) + readlane_v(x, 48));
}

// This thread's triple over n logits v[] with indices ix[] (-inf entries are absent).
template <int N>
__device__ __forceinline__ Msi thread_msi(const float (&v)[N], const int (&ix)[N]) {
  Msi t{-INFINITY, 0.0f, 0x7fffffff};
#pragma unroll
  for (int j = 0; j < N; ++j)
    if (v[j] > t.m) { t.m = v[j]; t.i = ix[j]; }  // indices increase with j: first maximum
  if (t.m != -INFINITY) {
#pragma unroll
    for (int j = 0; j < N; ++j) t.s += __expf(v[j] - t.m);
  }
  return t;
}

// Block-wide (max, argmax) for 256 threads.
__device__ __forceinline__ void block_argmax(float& v, int& i, float* sv, int* si) {
  wave_argmax(v, i);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) { sv[w] = v; si[w] = i; }
  __syncthreads();
  v = sv[0];
  i = si[0];
#pragma unroll
  for (int k = 1; k < kVThreads / 64; ++k)
    if (sv[k] > v || (sv[k] == v && si[k] < i)) { v = sv[k]; i = si[k]; }
  __syncthreads();
}
// Loads this thread's PT logits of chunk [lo, lo + n) in increasing index order.
// VEC: 16-byte loads (row base 16-byte aligned, V % 4 == 0); thread t owns float4 slots
// t, t + 256, t + 512, t + 768.  Otherwise scalar slots t + 256 j.  Missing -> -inf.
template <bool VEC, int PT>
__device__ __forceinline__ void load_chunk(const float* __restrict__ row, int lo, int n, float (&v)[PT],
                                           int (&ix)[PT]) {
  if constexpr (VEC) {
#pragma unroll
    for (int j = 0; j < PT / 4; ++j) {
      const int e = 4 * ((int)threadIdx.x + kVThreads * j);
      float4 f = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      if (e < n) f = *reinterpret_cast<const float4*>(row + lo + e);  // n % 4 == 0
      v[4 * j + 0] = f.x; v[4 * j + 1] = f.y; v[4 * j + 2] = f.z; v[4 * j + 3] = f.w;
#pragma unroll
      for (int q = 0; q < 4; ++q) ix[4 * j + q] = lo + e + q;
    }
  } else {
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const int e = (int)threadIdx.x + kVThreads * j;
      v[j] = e < n ? row[lo + e] : -INFINITY;
      ix[j] = lo + e;
    }
  }
}

// ---- device-coherent hand-off between the workgroups of one launch
// Partials written by the workgroups of a sequence are stored with device-coherent (SC1) stores;
// each workgroup waits for its store, then counts itself on a per-sequence counter that is zero
// when the call starts.  The workgroup that brings the count to T (the sequence's workgroup
// count) arrived last: it reads the partials back with device-coherent loads (no L2 maintenance
// needed), finishes the sequence and sets the counter back to zero for the next call.  So the
// counters must be zero before the workspace is first used, and every call leaves them zero.
constexpr int kSc1Bit = 16;  // cache-policy bit SC1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coh_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}
// A partial as the words (m, s, i, 0).
__device__ __forceinline__ void store_part_coh(Part* parts, size_t k, const Msi& r) {
  const int4_t v = int4_t{__float_as_int(r.m), __float_as_int(r.s), r.i, 0};
  __builtin_amdgcn_raw_buffer_store_b128(v, coh_rsrc(parts), (int)(k * sizeof(Part)), 0, kSc1Bit);
}
// Vector elements are copied to scalars before any reinterpretation: a bit_cast applied to a
// vector element directly was lowered to a read of element 0 by this compiler.
__device__ __forceinline__ Msi load_part_coh(const Part* parts, size_t k) {
  const int4_t v = __builtin_bit_cast(int4_t, __builtin_amdgcn_raw_buffer_load_b128(coh_rsrc(parts), (int)(k * sizeof(Part)), 0, kSc1Bit));
  const int e0 = v[0], e1 = v[1], e2 = v[2];
  return Msi{__int_as_float(e0), __int_as_float(e1), e2};
}
// Thread 0 publishes, all threads learn whether this workgroup finishes the sequence (and, if so,
// the counter is already back at zero: no other workgroup of this call touches it again).
__device__ __forceinline__ bool last_of_sequence(unsigned* cnt, unsigned total, int* sh) {
  if (threadIdx.x == 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this workgroup's partial is in memory
    const unsigned old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = old + 1u == total;
    if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *sh = last;
  }
  __syncthreads();
  return *sh != 0;
}

// (max, sum exp, first argmax) of this workgroup's chunk [lo, lo + n) of row src; valid in thread 0.
template <bool VEC>
__device__ __forceinline__ Msi chunk_stats(const float* __restrict__ src, int lo, int n) {
  float v[kStatPerThread];
  int ix[kStatPerThread];
  load_chunk<VEC, kStatPerThread>(src, lo, n, v, ix);
  const Msi t = wave_msi(thread_msi(v, ix));
  __shared__ Msi wt[kVThreads / 64];
  if ((threadIdx.x & 63) == 0) wt[threadIdx.x >> 6] = t;
  __syncthreads();
  return msi_merge(msi_merge(wt[0], wt[1]), msi_merge(wt[2], wt[3]));
}

// Merge the C partials of one row (chunk order kept lane-locally) with a 64-lane wave.
__device__ __forceinline__ Msi merge_row_coh(const Part* __restrict__ parts, size_t row, int C) {
  const int lane = threadIdx.x & 63;
  Msi t{-INFINITY, 0.0f, 0x7fffffff};
  for (int c = lane; c < C; c += 64) t = msi_merge(t, load_part_coh(parts, row * (size_t)C + c));
  return wave_msi(t);
}

constexpr int kMaxGammaShared = 63;  // gamma bound of the per-sequence steps (rows in LDS)
constexpr int kWaves = kVThreads / 64;

// Greedy verify, one launch: workgroup (row, chunk) of B * (gamma + 1) rows; the last workgroup
// of a sequence merges its rows (Top-1, top1_prob) and applies the prefix rule.
template <bool VEC>
__global__ __launch_bounds__(kVThreads) void greedy_kernel(const float* __restrict__ tgt, int gamma, int V, int C,
                                                           Part* __restrict__ parts,
                                                           unsigned* __restrict__ cnt,
                                                           const int32_t* __restrict__ draft,
                                                           int32_t* __restrict__ t_out, float* __restrict__ p1_out,
                                                           int32_t* __restrict__ n_acc, int32_t* __restrict__ out) {
  __shared__ int last_sh;
  __shared__ int t_sh[kMaxGammaShared + 1];
  const size_t bid = blockIdx.x;
  const int rows = gamma + 1;
  const int row = (int)(bid / C), c = (int)(bid % C);
  const int b = row / rows;
  const int lo = c * kStatChunk;
  const int n = V - lo < kStatChunk ? V - lo : kStatChunk;
  const Msi r = chunk_stats<VEC>(tgt + (size_t)row * V, lo, n);
  if (threadIdx.x == 0) store_part_coh(parts, bid, r);
  if (!last_of_sequence(cnt + kCounterStride * b, (unsigned)(rows * C), &last_sh)) return;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int i = w; i < rows; i += kWaves) {
    const size_t rr = (size_t)b * rows + i;
    const Msi t = merge_row_coh(parts, rr, C);
    if (lane == 0) {
      t_sh[i] = t.i;
      t_out[rr] = t.i;
      if (p1_out) p1_out[rr] = 1.0f / t.s;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int na = 0;
    while (na < gamma && draft[(size_t)b * gamma + na] == t_sh[na]) ++na;
    int32_t* o = out + (size_t)b * rows;
    for (int i = 0; i < na; ++i) o[i] = draft[(size_t)b * gamma + i];
    o[na] = t_sh[na];
    for (int i = na + 1; i < rows; ++i) o[i] = -1;
    n_acc[b] = na;
  }
}

// Tree-shaped greedy verify, one launch: workgroup (row, chunk) of B * T rows (row t of a sequence
// holds the target's scores after node t; node 0 is the root).  The last workgroup of a sequence
// merges its rows' Top-1 and walks the tree in node order (a parent precedes its children): node
// t >= 1 is accepted iff its parent is valid (in [0, t)) and accepted and its token equals the
// parent row's Top-1.  The deepest accepted node wins (lowest index on equal depth); the committed
// tokens are those along its root path, then its own Top-1 (the greedy prefix rule applied to every
// root-to-node path).
template <bool VEC>
__global__ __launch_bounds__(kVThreads) void tree_greedy_kernel(const float* __restrict__ tgt, int T, int V, int C,
                                                                Part* __restrict__ parts,
                                                                unsigned* __restrict__ cnt,
                                                                const int32_t* __restrict__ tokens,
                                                                const int32_t* __restrict__ parent,
                                                                int32_t* __restrict__ t_out,
                                                                int32_t* __restrict__ n_acc,
                                                                int32_t* __restrict__ out,
                                                                int32_t* __restrict__ out_nodes) {
  __shared__ int last_sh;
  __shared__ int t_sh[kMaxGammaShared + 1];
  __shared__ int depth[kMaxGammaShared + 1], par[kMaxGammaShared + 1], path[kMaxGammaShared + 1];
  const size_t bid = blockIdx.x;
  const int row = (int)(bid / C), c = (int)(bid % C);
  const int b = row / T;
  const int lo = c * kStatChunk;
  const int n = V - lo < kStatChunk ? V - lo : kStatChunk;
  const Msi r = chunk_stats<VEC>(tgt + (size_t)row * V, lo, n);
  if (threadIdx.x == 0) store_part_coh(parts, bid, r);
  if (!last_of_sequence(cnt + kCounterStride * b, (unsigned)(T * C), &last_sh)) return;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int i = w; i < T; i += kWaves) {
    const size_t rr = (size_t)b * T + i;
    const Msi t = merge_row_coh(parts, rr, C);
    if (lane == 0) {
      t_sh[i] = t.i;
      t_out[rr] = t.i;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int32_t* tok = tokens + (size_t)b * T;
    const int32_t* pa = parent + (size_t)b * T;
    depth[0] = 0;  // -1: not accepted
    int win = 0;
    for (int t = 1; t < T; ++t) {
      const int p = pa[t];
      par[t] = p;
      depth[t] = -1;
      if (p >= 0 && p < t && depth[p] >= 0 && tok[t] == t_sh[p]) {
        depth[t] = depth[p] + 1;
        if (depth[t] > depth[win]) win = t;
      }
    }
    const int na = depth[win];
    for (int node = win, i = na - 1; i >= 0; --i) {  // root path, filled from the end
      path[i] = node;
      node = par[node];
    }
    int32_t* o = out + (size_t)b * T;
    int32_t* on = out_nodes ? out_nodes + (size_t)b * T : nullptr;
    for (int i = 0; i < T; ++i) {
      o[i] = i < na ? tok[path[i]] : i == na ? t_sh[win] : -1;
      if (on) on[i] = i < na ? path[i] : -1;
    }
    n_acc[b] = na;
  }
}

// Sampling verify, first launch: workgroup (row, chunk) of the B (gamma + 1) target rows, then
// the B gamma draft rows; the last workgroup of a sequence merges its 2 gamma + 1 rows, computes
// every a_i = min(1, p(d_i) / q(d_i)), finds the first rejection and records what the final token
// is drawn from.  All fp32: an acceptance probability needs 1e-5 absolute, which fp32 holds.
template <bool VEC>
__global__ __launch_bounds__(kVThreads) void sample_stats_kernel(
    const float* __restrict__ tgt, const float* __restrict__ drf, int B, int gamma, int V, int C,
    Part* __restrict__ parts, unsigned* __restrict__ cnt, const int32_t* __restrict__ draft,
    const float* __restrict__ u_acc, float* __restrict__ a_out, int32_t* __restrict__ n_acc,
    int32_t* __restrict__ out, SeqInfo* __restrict__ info) {
  __shared__ int last_sh;
  __shared__ float mp[kMaxGammaShared + 1], sp[kMaxGammaShared + 1];
  __shared__ float mq[kMaxGammaShared + 1], sq[kMaxGammaShared + 1];
  __shared__ float a_sh[kMaxGammaShared + 1];
  const size_t bid = blockIdx.x;
  const int rows_t = gamma + 1;
  const int row = (int)(bid / C), c = (int)(bid % C);
  const bool is_t = row < B * rows_t;
  const int b = is_t ? row / rows_t : (row - B * rows_t) / gamma;
  const float* src = is_t ? tgt + (size_t)row * V : drf + (size_t)(row - B * rows_t) * V;
  const int lo = c * kStatChunk;
  const int n = V - lo < kStatChunk ? V - lo : kStatChunk;
  const Msi r = chunk_stats<VEC>(src, lo, n);
  if (threadIdx.x == 0) store_part_coh(parts, bid, r);
  if (!last_of_sequence(cnt + kCounterStride * b, (unsigned)((2 * gamma + 1) * C), &last_sh)) return;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int i = w; i < 2 * gamma + 1; i += kWaves) {
    // target rows of all sequences come first in the parts array, then draft rows
    const size_t rr = i <= gamma ? (size_t)b * rows_t + i : (size_t)B * rows_t + (size_t)b * gamma + (i - rows_t);
    const Msi t = merge_row_coh(parts, rr, C);
    if (lane == 0) {
      if (i <= gamma) { mp[i] = t.m; sp[i] = t.s; } else { mq[i - rows_t] = t.m; sq[i - rows_t] = t.s; }
    }
  }
  __syncthreads();
  if (threadIdx.x < gamma) {
    const int i = threadIdx.x;
    const int d = draft[(size_t)b * gamma + i];
    float a = 0.0f;
    if (d >= 0 && d < V) {
      const float lp = tgt[((size_t)b * rows_t + i) * V + d];
      const float lq = drf[((size_t)b * gamma + i) * V + d];
      const float pp = __expf(lp - mp[i]) / sp[i];
      const float qq = __expf(lq - mq[i]) / sq[i];
      if (pp <= 0.0f) a = 0.0f;
      else if (qq <= 0.0f) a = 1.0f;
      else a = fminf(1.0f, pp / qq);
    }
    a_sh[i] = a;
    a_out[(size_t)b * gamma + i] = a;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int na = 0;
    while (na < gamma && u_acc[(size_t)b * gamma + na] < a_sh[na]) ++na;
    int32_t* o = out + (size_t)b * rows_t;
    for (int i = 0; i < na; ++i) o[i] = draft[(size_t)b * gamma + i];
    n_acc[b] = na;
    SeqInfo si{};
    si.n = na;
    si.use_res = na < gamma ? 1 : 0;
    si.mp = mp[na];
    si.sp = sp[na];
    si.mq = na < gamma ? mq[na] : 0.0f;
    si.sq = na < gamma ? sq[na] : 1.0f;
    info[b] = si;
  }
}

// This thread's slots of a chunk of the drawn-from rows, unnormalised, in fp64: a_j = exp(lp_j - mp)
// and b_j = exp(lq_j - mq) (0 when drawing from p).  Missing slots give 0.
template <bool VEC>
__device__ __forceinline__ void draw_exps(const SeqInfo& si, const float* __restrict__ prow,
                                          const float* __restrict__ qrow, int lo, int n,
                                          double (&a)[kPerThread], double (&bq)[kPerThread],
                                          int (&ix)[kPerThread]) {
  float lp[kPerThread];
  load_chunk<VEC, kPerThread>(prow, lo, n, lp, ix);
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) a[j] = exp_diff64(lp[j], si.mp);
  if (si.use_res) {
    float lq[kPerThread];
    int ix2[kPerThread];
    load_chunk<VEC, kPerThread>(qrow, lo, n, lq, ix2);
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) bq[j] = exp_diff64(lq[j], si.mq);
  } else {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) bq[j] = 0.0;
  }
}

// The chunk's Mass4, valid in thread 0.  A slot counts as p > q when a_j sq > b_j sp with the fp32
// normalisers; a slot put on the wrong side has |p_j - q_j| within their rounding (1e-7 p_j), so
// it moves the chunk's residual mass by no more than that.
template <bool VEC>
__device__ __forceinline__ Mass4 chunk_mass(const SeqInfo& si, const float* __restrict__ prow,
                                            const float* __restrict__ qrow, int lo, int n) {
  double a[kPerThread], bq[kPerThread];
  int ix[kPerThread];
  draw_exps<VEC>(si, prow, qrow, lo, n, a, bq, ix);
  const double sp = si.sp, sq = si.sq;
  double za = 0.0, zb = 0.0, zap = 0.0, zbp = 0.0;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    za += a[j];
    zb += bq[j];
    const bool pos = a[j] * sq > bq[j] * sp;
    zap += pos ? a[j] : 0.0;
    zbp += pos ? bq[j] : 0.0;
  }
  za = wave_sum_f64(za);
  zb = wave_sum_f64(zb);
  zap = wave_sum_f64(zap);
  zbp = wave_sum_f64(zbp);
  __shared__ Mass4 wm[kWaves];
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = Mass4{za, zb, zap, zbp};
  __syncthreads();
  return Mass4{(wm[0].a + wm[1].a) + (wm[2].a + wm[3].a), (wm[0].b + wm[1].b) + (wm[2].b + wm[3].b),
               (wm[0].ap + wm[1].ap) + (wm[2].ap + wm[3].ap), (wm[0].bp + wm[1].bp) + (wm[2].bp + wm[3].bp)};
}

// The draw of a sequence from its chunk sums (wave 0 only; ld(k) gives chunk k's Mass4): the fp64
// normalisers S_p, S_q, every chunk's mass of the drawn-from distribution (residual, or p when
// the residual vanished), their total, then an inclusive scan 64 chunks at a time; the first chunk
// whose inclusive prefix passes u times the total, else the last chunk with mass.  The same
// arithmetic in every caller, so every workgroup of a sequence agrees.
struct Draw {
  double prefix, target, z;  // mass before the chunk, u times the total, the total
  double inv_sp, inv_sq;     // 1 / S_p, and 1 / S_q (0 when drawing from p)
  int chunk, usep;
};
template <typename LD>
__device__ __forceinline__ Draw find_chunk(LD&& ld_any, int C, float u, int use_res) {
  const int lane = threadIdx.x & 63;
  // Up to 64 chunks (V <= 131072) every lane reads its chunk's sums once; beyond, each pass reads.
  const bool one = C <= 64;
  Mass4 mine{0.0, 0.0, 0.0, 0.0};
  if (one && lane < C) mine = ld_any(lane);
  auto ld = [&](int k) { return one ? mine : ld_any(k); };  // with one, k is this lane
  double ta = 0.0, tb = 0.0;
  for (int k = lane; k < C; k += 64) { const Mass4 v = ld(k); ta += v.a; tb += v.b; }
  ta = wave_sum_f64(ta);
  tb = wave_sum_f64(tb);
  Draw d;
  d.inv_sp = 1.0 / ta;
  d.inv_sq = use_res ? 1.0 / tb : 0.0;
  auto mass = [&](const Mass4& v, bool usep) {
    return usep ? v.a * d.inv_sp : fmax(0.0, v.ap * d.inv_sp - v.bp * d.inv_sq);
  };
  double zr = 0.0;
  for (int k = lane; k < C; k += 64) zr += mass(ld(k), false);
  zr = wave_sum_f64(zr);
  d.usep = !(zr > 0.0);   // residual mass vanished: draw from p
  d.z = d.usep ? ta * d.inv_sp : zr;
  d.target = (double)u * d.z;
  double carry = 0.0, pre = 0.0, pre_last = 0.0;
  int chunk = -1, last_nz = 0;
  for (int k0 = 0; k0 < C; k0 += 64) {
    const int k = k0 + lane;
    double zk = 0.0;
    if (k < C) zk = mass(ld(k), d.usep);
    double incl = zk;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const double t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    incl += carry;
    const double excl = incl - zk;
    const unsigned long long hit = __ballot(k < C && incl > d.target);
    if (chunk < 0 && hit != 0ull) {
      const int l = __ffsll((long long)hit) - 1;
      chunk = k0 + l;
      pre = __shfl(excl, l, 64);
    }
    const unsigned long long nz = __ballot(k < C && zk > 0.0);
    if (nz != 0ull) {
      const int l = 63 - __clzll((long long)nz);
      last_nz = k0 + l;
      pre_last = __shfl(excl, l, 64);
    }
    carry = __shfl(incl, 63, 64);
  }
  if (chunk < 0) { chunk = last_nz; pre = pre_last; }
  d.chunk = chunk;
  d.prefix = pre;
  return d;
}

// Normalised values of the drawn-from distribution for this thread's slots (fp64, exact
// normalisers): the residual max(0, p_j - q_j), or p_j.
template <bool VEC>
__device__ __forceinline__ void final_values(const SeqInfo& si, const Draw& d, const float* __restrict__ prow,
                                             const float* __restrict__ qrow, int lo, int n,
                                             double (&r)[kPerThread], int (&ix)[kPerThread]) {
  double a[kPerThread], bq[kPerThread];
  draw_exps<VEC>(si, prow, qrow, lo, n, a, bq, ix);
#pragma unroll
  for (int j = 0; j < kPerThread; ++j)
    r[j] = d.usep ? a[j] * d.inv_sp : fmax(0.0, a[j] * d.inv_sp - bq[j] * d.inv_sq);
}

// Inverse-CDF search inside chunk [lo, lo + n) given the mass before it; all threads; returns the
// token (valid in every thread).  Slots of a thread are not contiguous in the VEC layout, so the
// scan is slot-major: slot group j covers indices [4*256*j, 4*256*(j+1)).
template <bool VEC>
__device__ __forceinline__ int draw_in_chunk(const SeqInfo& si, const Draw& d, const float* __restrict__ prow,
                                             const float* __restrict__ qrow, int lo, int n) {
  __shared__ float sv[4];
  __shared__ int si_[4];
  __shared__ double wsum[4];
  double r[kPerThread];
  int ix[kPerThread];
  final_values<VEC>(si, d, prow, qrow, lo, n, r, ix);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  double base = d.prefix;
  int found = 0x7fffffff;
  int last_pos = -1;
  constexpr int kGroups = VEC ? kPerThread / 4 : kPerThread;
  constexpr int kPerGroup = VEC ? 4 : 1;
#pragma unroll
  for (int j = 0; j < kGroups; ++j) {
    double loc[kPerGroup];
    double tsum = 0.0;
#pragma unroll
    for (int q = 0; q < kPerGroup; ++q) { tsum += r[j * kPerGroup + q]; loc[q] = tsum; }
    // exclusive scan of tsum across the 256 threads (thread order = index order inside group j)
    double incl = tsum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const double t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    double wpre = 0.0;
    for (int k = 0; k < w; ++k) wpre += wsum[k];
    const double gtot = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
    const double excl = base + wpre + (incl - tsum);
#pragma unroll
    for (int q = 0; q < kPerGroup; ++q) {
      const int idx = ix[j * kPerGroup + q];
      if (idx < lo + n) {
        if (found == 0x7fffffff && excl + loc[q] > d.target && r[j * kPerGroup + q] > 0.0) found = idx;
        if (r[j * kPerGroup + q] > 0.0) last_pos = idx;
      }
    }
    base += gtot;
  }
  // smallest found index; else the last index with positive mass
  float fv = found == 0x7fffffff ? -1.0f : 1.0f;
  int fi = found == 0x7fffffff ? 0x7fffffff : found;
  block_argmax(fv, fi, sv, si_);
  int token = fi;
  if (fv < 0.0f) {
    float lv = last_pos >= 0 ? (float)last_pos : -1.0f;
    int li = last_pos;
    block_argmax(lv, li, sv, si_);
    token = li >= 0 ? li : lo;
  }
  return token;
}

__device__ __forceinline__ void write_final(int32_t* __restrict__ out, int b, int gamma, const SeqInfo& si, int token) {
  int32_t* o = out + (size_t)b * (gamma + 1);
  o[si.n] = token;
  for (int i = si.n + 1; i <= gamma; ++i) o[i] = -1;
}

// Mass4 of chunk k of a sequence's sums, device-coherent (two 16-byte words).
__device__ __forceinline__ void store_mass_coh(Mass4* cs, size_t k, const Mass4& m) {
  const long long a = __double_as_longlong(m.a), b = __double_as_longlong(m.b);
  const long long ap = __double_as_longlong(m.ap), bp = __double_as_longlong(m.bp);
  const int off = (int)(k * sizeof(Mass4));
  __builtin_amdgcn_raw_buffer_store_b128(int4_t{(int)(unsigned)a, (int)(a >> 32), (int)(unsigned)b, (int)(b >> 32)},
                                         coh_rsrc(cs), off, 0, kSc1Bit);
  __builtin_amdgcn_raw_buffer_store_b128(int4_t{(int)(unsigned)ap, (int)(ap >> 32), (int)(unsigned)bp, (int)(bp >> 32)},
                                         coh_rsrc(cs), off + 16, 0, kSc1Bit);
}
__device__ __forceinline__ double join_f64(int lo, int hi) {
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}
__device__ __forceinline__ Mass4 load_mass_coh(const Mass4* cs, int k) {
  const int off = k * (int)sizeof(Mass4);
  const int4_t u = __builtin_bit_cast(int4_t, __builtin_amdgcn_raw_buffer_load_b128(coh_rsrc(cs), off, 0, kSc1Bit));
  const int4_t v = __builtin_bit_cast(int4_t, __builtin_amdgcn_raw_buffer_load_b128(coh_rsrc(cs), off + 16, 0, kSc1Bit));
  const int u0 = u[0], u1 = u[1], u2 = u[2], u3 = u[3];  // through scalars (see load_part_coh)
  const int v0 = v[0], v1 = v[1], v2 = v[2], v3 = v[3];
  return Mass4{join_f64(u0, u1), join_f64(u2, u3), join_f64(v0, v1), join_f64(v2, v3)};
}

// Sampling verify, second launch when the final distribution is not requested: workgroup
// (sequence, chunk) sums its chunk of the drawn-from rows; the last workgroup of a sequence finds
// the chunk of the draw and searches it.
template <bool VEC>
__global__ __launch_bounds__(kVThreads) void sample_draw_kernel(
    const float* __restrict__ tgt, const float* __restrict__ drf, int gamma, int V, int C,
    const SeqInfo* __restrict__ info, Mass4* __restrict__ csum, unsigned* __restrict__ cnt,
    const float* __restrict__ u_fin, int32_t* __restrict__ out) {
  __shared__ int last_sh;
  __shared__ Draw dsh;
  const size_t bid = blockIdx.x;
  const int b = (int)(bid / C), c = (int)(bid % C);
  const SeqInfo si = info[b];
  const float* prow = tgt + ((size_t)b * (gamma + 1) + si.n) * V;
  const float* qrow = si.use_res ? drf + ((size_t)b * gamma + si.n) * V : prow;
  const int lo = c * kChunk;
  const int n = V - lo < kChunk ? V - lo : kChunk;
  const Mass4 z = chunk_mass<VEC>(si, prow, qrow, lo, n);
  if (threadIdx.x == 0) store_mass_coh(csum, bid, z);
  if (!last_of_sequence(cnt + kCounterStride * b, (unsigned)C, &last_sh)) return;
  if (threadIdx.x < 64) {
    const Mass4* cs = csum + (size_t)b * C;
    const Draw d = find_chunk([&](int k) { return load_mass_coh(cs, k); }, C, u_fin[b], si.use_res);
    if (threadIdx.x == 0) dsh = d;
  }
  __syncthreads();
  const Draw d = dsh;
  const int clo = d.chunk * kChunk;
  const int cn = V - clo < kChunk ? V - clo : kChunk;
  const int token = draw_in_chunk<VEC>(si, d, prow, qrow, clo, cn);
  if (threadIdx.x == 0) write_final(out, b, gamma, si, token);
}

// Sampling verify with the final distribution f: per-chunk sums, then every workgroup of a
// sequence finds the chunk of the draw, writes its chunk of f, and the owner of the draw's chunk
// searches it.
template <bool VEC>
__global__ __launch_bounds__(kVThreads) void residual_sum_kernel(const float* __restrict__ tgt,
                                                                 const float* __restrict__ drf, int gamma,
                                                                 int V, int C,
                                                                 const SeqInfo* __restrict__ info,
                                                                 Mass4* __restrict__ csum) {
  const size_t bid = blockIdx.x;
  const int b = (int)(bid / C), c = (int)(bid % C);
  const SeqInfo si = info[b];
  const float* prow = tgt + ((size_t)b * (gamma + 1) + si.n) * V;
  const float* qrow = si.use_res ? drf + ((size_t)b * gamma + si.n) * V : prow;
  const int lo = c * kChunk;
  const int n = V - lo < kChunk ? V - lo : kChunk;
  const Mass4 z = chunk_mass<VEC>(si, prow, qrow, lo, n);
  if (threadIdx.x == 0) csum[bid] = z;
}

template <bool VEC>
__global__ __launch_bounds__(kVThreads) void sample_final_kernel(
    const float* __restrict__ tgt, const float* __restrict__ drf, int gamma, int V, int C,
    const SeqInfo* __restrict__ info, const Mass4* __restrict__ csum, const float* __restrict__ u_fin,
    int32_t* __restrict__ out, float* __restrict__ fdist) {
  __shared__ Draw dsh;
  const size_t bid = blockIdx.x;
  const int b = (int)(bid / C), c = (int)(bid % C);
  const SeqInfo si = info[b];
  if (threadIdx.x < 64) {
    const Mass4* cs = csum + (size_t)b * C;
    const Draw d = find_chunk([&](int k) { return cs[k]; }, C, u_fin[b], si.use_res);
    if (threadIdx.x == 0) dsh = d;
  }
  __syncthreads();
  const Draw d = dsh;
  const float* prow = tgt + ((size_t)b * (gamma + 1) + si.n) * V;
  const float* qrow = si.use_res ? drf + ((size_t)b * gamma + si.n) * V : prow;
  const int lo = c * kChunk;
  const int n = V - lo < kChunk ? V - lo : kChunk;
  {  // this workgroup's chunk of f
    double r[kPerThread];
    int ix[kPerThread];
    final_values<VEC>(si, d, prow, qrow, lo, n, r, ix);
    const double inv_z = 1.0 / d.z;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j)
      if (ix[j] < lo + n) fdist[(size_t)b * V + ix[j]] = (float)(r[j] * inv_z);
  }
  if (c != d.chunk) return;
  const int token = draw_in_chunk<VEC>(si, d, prow, qrow, lo, n);
  if (threadIdx.x == 0) write_final(out, b, gamma, si, token);
}

static bool vec_ok(const float* p, int V) { return p != nullptr && V % 4 == 0 && aligned16(p); }

static int greedy_block(const float* tgt, const int32_t* d, int B, int gamma, int V, int32_t* t,
                        float* p1, int32_t* n_acc, int32_t* out, void* ws, hipStream_t st) {
  const int C = stat_chunks(V);
  VerifyWs w = carve(ws, B, gamma, V);
  const size_t rows = (size_t)B * (gamma + 1);
  const size_t blocks = rows * C;
  if (vec_ok(tgt, V))
    hipLaunchKernelGGL(greedy_kernel<true>, dim3((unsigned)blocks), dim3(kVThreads), 0, st, tgt, gamma, V, C,
                       w.parts, w.cnt, d, t, p1, n_acc, out);
  else
    hipLaunchKernelGGL(greedy_kernel<false>, dim3((unsigned)blocks), dim3(kVThreads), 0, st, tgt, gamma, V, C,
                       w.parts, w.cnt, d, t, p1, n_acc, out);
  return launch_status();
}

static int tree_block(const float* tgt, const int32_t* tok, const int32_t* par, int B, int T, int V, int32_t* t,
                      int32_t* n_acc, int32_t* out, int32_t* nodes, void* ws, hipStream_t st) {
  const int C = stat_chunks(V);
  VerifyWs w = carve(ws, B, T - 1, V);
  const size_t blocks = (size_t)B * T * C;
  if (vec_ok(tgt, V))
    hipLaunchKernelGGL(tree_greedy_kernel<true>, dim3((unsigned)blocks), dim3(kVThreads), 0, st, tgt, T, V, C,
                       w.parts, w.cnt, tok, par, t, n_acc, out, nodes);
  else
    hipLaunchKernelGGL(tree_greedy_kernel<false>, dim3((unsigned)blocks), dim3(kVThreads), 0, st, tgt, T, V, C,
                       w.parts, w.cnt, tok, par, t, n_acc, out, nodes);
  return launch_status();
}

static int sample_block(const float* tgt, const float* drf, const int32_t* d, const float* u_acc,
                        const float* u_fin, int B, int gamma, int V, float* a, int32_t* n_acc,
                        int32_t* out, float* fdist, void* ws, hipStream_t st) {
  const int Cs = stat_chunks(V), C = draw_chunks(V);
  VerifyWs w = carve(ws, B, gamma, V);
  const size_t rows_t = (size_t)B * (gamma + 1), rows_d = (size_t)B * gamma;
  const size_t blocks = (rows_t + rows_d) * Cs;
  const bool vec = vec_ok(tgt, V) && (gamma == 0 || vec_ok(drf, V));
  const size_t fb = (size_t)B * C;
  if (vec)
    hipLaunchKernelGGL(sample_stats_kernel<true>, dim3((unsigned)blocks), dim3(kVThreads), 0, st, tgt, drf, B,
                       gamma, V, Cs, w.parts, w.cnt, d, u_acc, a, n_acc, out, w.info);
  else
    hipLaunchKernelGGL(sample_stats_kernel<false>, dim3((unsigned)blocks), dim3(kVThreads), 0, st, tgt, drf, B,
                       gamma, V, Cs, w.parts, w.cnt, d, u_acc, a, n_acc, out, w.info);
  int rc = launch_status();
  if (rc != QS_OK) return rc;
  if (fdist == nullptr) {
    if (vec)
      hipLaunchKernelGGL(sample_draw_kernel<true>, dim3((unsigned)fb), dim3(kVThreads), 0, st, tgt, drf, gamma, V,
                         C, w.info, w.csum, w.cnt2, u_fin, out);
    else
      hipLaunchKernelGGL(sample_draw_kernel<false>, dim3((unsigned)fb), dim3(kVThreads), 0, st, tgt, drf, gamma, V,
                         C, w.info, w.csum, w.cnt2, u_fin, out);
    return launch_status();
  }
  if (vec) {
    hipLaunchKernelGGL(residual_sum_kernel<true>, dim3((unsigned)fb), dim3(kVThreads), 0, st, tgt, drf,
                       gamma, V, C, w.info, w.csum);
    rc = launch_status();
    if (rc != QS_OK) return rc;
    hipLaunchKernelGGL(sample_final_kernel<true>, dim3((unsigned)fb), dim3(kVThreads), 0, st, tgt, drf,
                       gamma, V, C, w.info, w.csum, u_fin, out, fdist);
  } else {
    hipLaunchKernelGGL(residual_sum_kernel<false>, dim3((unsigned)fb), dim3(kVThreads), 0, st, tgt, drf,
                       gamma, V, C, w.info, w.csum);
    rc = launch_status();
    if (rc != QS_OK) return rc;
    hipLaunchKernelGGL(sample_final_kernel<false>, dim3((unsigned)fb), dim3(kVThreads), 0, st, tgt, drf,
                       gamma, V, C, w.info, w.csum, u_fin, out, fdist);
  }
  return launch_status();
}

// Greedy acceptance from Top-1 ids already computed (the LM-head epilogue of a verify pass): one
// thread per sequence applies the prefix rule of greedy_kernel.  A negative Top-1 (what a timed-out
// pass leaves) matches no draft token.
__global__ __launch_bounds__(256) void accept_greedy_kernel(const int32_t* __restrict__ t,
                                                            const int32_t* __restrict__ draft, int B, int gamma,
                                                            int32_t* __restrict__ n_acc, int32_t* __restrict__ out) {
  const int b = (int)(blockIdx.x * 256 + threadIdx.x);
  if (b >= B) return;
  const int rows = gamma + 1;
  const int32_t* tb = t + (size_t)b * rows;
  const int32_t* db = draft + (size_t)b * gamma;  // not read when gamma = 0
  int na = 0;
  while (na < gamma && tb[na] >= 0 && db[na] == tb[na]) ++na;
  int32_t* o = out + (size_t)b * rows;
  for (int i = 0; i < na; ++i) o[i] = db[i];
  o[na] = tb[na];
  for (int i = na + 1; i < rows; ++i) o[i] = -1;
  n_acc[b] = na;
}

int launch_accept_greedy(const int32_t* t, const int32_t* d, int B, int gamma, int32_t* n_acc, int32_t* out,
                         hipStream_t st) {
  hipLaunchKernelGGL(accept_greedy_kernel, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, st, t, d, B, gamma,
                     n_acc, out);
  return launch_status();
}

// Sequences are independent: a batch beyond the counter slots runs as consecutive blocks of at
// most QS_MAX_VERIFY_SEQS sequences on the stream, each reusing the same workspace in turn.
int launch_verify_greedy(const float* tgt, const int32_t* d, int B, int gamma, int V, int32_t* t,
                         float* p1, int32_t* n_acc, int32_t* out, void* ws, hipStream_t st) {
  for (int b0 = 0; b0 < B; b0 += QS_MAX_VERIFY_SEQS) {
    const int nb = B - b0 < QS_MAX_VERIFY_SEQS ? B - b0 : QS_MAX_VERIFY_SEQS;
    const size_t r0 = (size_t)b0 * (gamma + 1);
    const int rc = greedy_block(tgt + r0 * V, d ? d + (size_t)b0 * gamma : d, nb, gamma, V, t + r0,
                                p1 ? p1 + r0 : p1, n_acc + b0, out + r0, ws, st);
    if (rc != QS_OK) return rc;
  }
  return QS_OK;
}

int launch_verify_tree_greedy(const float* tgt, const int32_t* tok, const int32_t* par, int B, int T, int V,
                              int32_t* t, int32_t* n_acc, int32_t* out, int32_t* nodes, void* ws, hipStream_t st) {
  for (int b0 = 0; b0 < B; b0 += QS_MAX_VERIFY_SEQS) {
    const int nb = B - b0 < QS_MAX_VERIFY_SEQS ? B - b0 : QS_MAX_VERIFY_SEQS;
    const size_t r0 = (size_t)b0 * T;
    const int rc = tree_block(tgt + r0 * V, tok + r0, par + r0, nb, T, V, t + r0, n_acc + b0, out + r0,
                              nodes ? nodes + r0 : nodes, ws, st);
    if (rc != QS_OK) return rc;
  }
  return QS_OK;
}

int launch_verify_sample(const float* tgt, const float* drf, const int32_t* d, const float* u_acc,
                         const float* u_fin, int B, int gamma, int V, float* a, int32_t* n_acc,
                         int32_t* out, float* fdist, void* ws, hipStream_t st) {
  for (int b0 = 0; b0 < B; b0 += QS_MAX_VERIFY_SEQS) {
    const int nb = B - b0 < QS_MAX_VERIFY_SEQS ? B - b0 : QS_MAX_VERIFY_SEQS;
    const size_t r0 = (size_t)b0 * (gamma + 1), d0 = (size_t)b0 * gamma;
    const int rc = sample_block(tgt + r0 * V, drf ? drf + d0 * V : drf, d ? d + d0 : d, u_acc ? u_acc + d0 : u_acc,
                                u_fin + b0, nb, gamma, V, a ? a + d0 : a, n_acc + b0, out + r0,
                                fdist ? fdist + (size_t)b0 * V : fdist, ws, st);
    if (rc != QS_OK) return rc;
  }
  return QS_OK;
}

}  // namespace qs
