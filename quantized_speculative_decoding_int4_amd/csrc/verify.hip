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
// split into chunks of kChunk elements, one 256-thread workgroup per
// (row, chunk) -- enough workgroups to fill the chip even for a single
// sequence.  Each workgroup produces (max, sum exp(l - max), first argmax)
// with 64-lane shuffle reductions and an LDS step across its 4 waves.  A small
// per-sequence kernel merges the chunk partials in chunk order (so argmax ties
// resolve to the lowest index and the result is deterministic) and applies the
// acceptance rule.  Sampling then re-reads only the one row per sequence that
// the final token is drawn from.  Draft ids are bounds-checked before use.

#include "qs_device.h"
#include "qs_internal.h"

namespace qs {

constexpr int kVThreads = 256;
constexpr int kPerThread = 16;
constexpr int kChunk = kVThreads * kPerThread;  // 4096 logits per workgroup

struct Part {
  float m;    // chunk maximum
  float s;    // sum over the chunk of exp(l - m)
  int idx;    // lowest index attaining m
  int pad;
};

struct SeqInfo {
  int n;        // accepted count (row of the final draw)
  int use_res;  // 1: draw from the residual max(0, p - q); 0: from p
  float mp, sp;  // target row n: max and normaliser
  float mq, sq;  // draft row n (when n < gamma)
  int pad[2];
};

static inline int n_chunks(int V) { return (V + kChunk - 1) / kChunk; }

size_t verify_workspace(int B, int gamma, int V) {
  const size_t C = (size_t)n_chunks(V);
  const size_t rows = (size_t)B * (2 * (size_t)gamma + 1);
  return align_up(rows * C * sizeof(Part), 256) + align_up((size_t)B * sizeof(SeqInfo), 256) +
         align_up((size_t)B * C * sizeof(float2), 256);
}

struct VerifyWs {
  Part* parts;
  SeqInfo* info;
  float2* csum;
};
static VerifyWs carve(void* ws, int B, int gamma, int V) {
  const size_t C = (size_t)n_chunks(V);
  const size_t rows = (size_t)B * (2 * (size_t)gamma + 1);
  unsigned char* p = static_cast<unsigned char*>(ws);
  VerifyWs w;
  w.parts = reinterpret_cast<Part*>(p);
  p += align_up(rows * C * sizeof(Part), 256);
  w.info = reinterpret_cast<SeqInfo*>(p);
  p += align_up((size_t)B * sizeof(SeqInfo), 256);
  w.csum = reinterpret_cast<float2*>(p);
  return w;
}

// Block-wide (max, argmax) then sum reduction helpers for 256 threads.
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
__device__ __forceinline__ float block_sum(float v, float* sv) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) sv[w] = v;
  __syncthreads();
  float t = 0.0f;
#pragma unroll
  for (int k = 0; k < kVThreads / 64; ++k) t += sv[k];  // fixed order
  __syncthreads();
  return t;
}

// Loads this thread's kPerThread logits of chunk [lo, lo + n) in increasing index order.
// VEC: 16-byte loads (row base 16-byte aligned, V % 4 == 0); thread t owns float4 slots
// t, t + 256, t + 512, t + 768.  Otherwise scalar slots t + 256 j.  Missing -> -inf.
template <bool VEC>
__device__ __forceinline__ void load_chunk(const float* __restrict__ row, int lo, int n,
                                           float (&v)[kPerThread], int (&ix)[kPerThread]) {
  if constexpr (VEC) {
#pragma unroll
    for (int j = 0; j < kPerThread / 4; ++j) {
      const int e = 4 * ((int)threadIdx.x + kVThreads * j);
      float4 f = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      if (e < n) f = *reinterpret_cast<const float4*>(row + lo + e);  // n % 4 == 0
      v[4 * j + 0] = f.x; v[4 * j + 1] = f.y; v[4 * j + 2] = f.z; v[4 * j + 3] = f.w;
#pragma unroll
      for (int q = 0; q < 4; ++q) ix[4 * j + q] = lo + e + q;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int e = (int)threadIdx.x + kVThreads * j;
      v[j] = e < n ? row[lo + e] : -INFINITY;
      ix[j] = lo + e;
    }
  }
}

// Partial softmax statistics of (row, chunk) = (bid / C, bid % C).  Rows [0, rows0) come from
// buf0, rows [rows0, rows0 + rows1) from buf1.
template <bool VEC>
__global__ __launch_bounds__(kVThreads) void row_stats_kernel(const float* __restrict__ buf0, int rows0,
                                                              const float* __restrict__ buf1, int V,
                                                              int C, Part* __restrict__ parts) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const size_t bid = blockIdx.x;
  const int row = (int)(bid / C), c = (int)(bid % C);
  const float* src = row < rows0 ? buf0 + (size_t)row * V : buf1 + (size_t)(row - rows0) * V;
  const int lo = c * kChunk;
  const int n = V - lo < kChunk ? V - lo : kChunk;
  float v[kPerThread];
  int ix[kPerThread];
  load_chunk<VEC>(src, lo, n, v, ix);
  float m = -INFINITY;
  int mi = 0x7fffffff;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j)
    if (v[j] > m) { m = v[j]; mi = ix[j]; }
  block_argmax(m, mi, sv, si);
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) s += __expf(v[j] - m);
  s = block_sum(s, sv);
  if (threadIdx.x == 0) parts[bid] = Part{m, s, mi, 0};
}

// Merge the C partials of one row with a 64-lane wave (chunk order preserved).
__device__ __forceinline__ void merge_row(const Part* __restrict__ p, int C, float& M, float& S,
                                          int& idx) {
  const int lane = threadIdx.x & 63;
  float m = -INFINITY;
  int mi = 0x7fffffff;
  for (int c = lane; c < C; c += 64) {
    const Part q = p[c];
    if (q.m > m || (q.m == m && q.idx < mi)) { m = q.m; mi = q.idx; }
  }
  wave_argmax(m, mi);
  float s = 0.0f;
  for (int c = lane; c < C; c += 64) {
    const Part q = p[c];
    s += q.s * __expf(q.m - m);
  }
  S = wave_sum(s);
  M = m;
  idx = mi;
}

constexpr int kMaxGammaShared = 63;  // gamma bound of the per-sequence kernels (rows in LDS)

__global__ __launch_bounds__(kVThreads) void greedy_finish_kernel(const Part* __restrict__ parts, int C,
                                                                  int gamma, int V,
                                                                  const int32_t* __restrict__ draft,
                                                                  int32_t* __restrict__ t_out,
                                                                  float* __restrict__ p1_out,
                                                                  int32_t* __restrict__ n_acc,
                                                                  int32_t* __restrict__ out) {
  __shared__ int t_sh[kMaxGammaShared + 1];
  const int b = blockIdx.x;
  const int rows = gamma + 1;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int i = w; i < rows; i += kVThreads / 64) {
    const size_t row = (size_t)b * rows + i;
    float M, S;
    int idx;
    merge_row(parts + row * C, C, M, S, idx);
    if (lane == 0) {
      t_sh[i] = idx;
      t_out[row] = idx;
      if (p1_out) p1_out[row] = 1.0f / S;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int n = 0;
    while (n < gamma && draft[(size_t)b * gamma + n] == t_sh[n]) ++n;
    int32_t* o = out + (size_t)b * rows;
    for (int i = 0; i < n; ++i) o[i] = draft[(size_t)b * gamma + i];
    o[n] = t_sh[n];
    for (int i = n + 1; i < rows; ++i) o[i] = -1;
    n_acc[b] = n;
  }
}

// Per sequence: merge statistics of target rows 0..gamma and draft rows 0..gamma-1,
// compute every a_i, find the first rejection.
__global__ __launch_bounds__(kVThreads) void sample_decide_kernel(
    const Part* __restrict__ parts, int C, int gamma, int V, const float* __restrict__ tgt,
    const float* __restrict__ drf, const int32_t* __restrict__ draft, const float* __restrict__ u_acc,
    float* __restrict__ a_out, int32_t* __restrict__ n_acc, int32_t* __restrict__ out,
    SeqInfo* __restrict__ info) {
  __shared__ float mp[kMaxGammaShared + 1], sp[kMaxGammaShared + 1];
  __shared__ float mq[kMaxGammaShared + 1], sq[kMaxGammaShared + 1];
  __shared__ float a_sh[kMaxGammaShared + 1];
  const int b = blockIdx.x;
  const int B = gridDim.x;
  const int rows_t = gamma + 1;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int i = w; i < 2 * gamma + 1; i += kVThreads / 64) {
    // target rows of all sequences come first in the parts array, then draft rows
    const size_t row = i <= gamma ? (size_t)b * rows_t + i
                                  : (size_t)B * rows_t + (size_t)b * gamma + (i - rows_t);
    float M, S;
    int idx;
    merge_row(parts + row * C, C, M, S, idx);
    if (lane == 0) {
      if (i <= gamma) { mp[i] = M; sp[i] = S; } else { mq[i - rows_t] = M; sq[i - rows_t] = S; }
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
      const float p = __expf(lp - mp[i]) / sp[i];
      const float q = __expf(lq - mq[i]) / sq[i];
      if (p <= 0.0f) a = 0.0f;
      else if (q <= 0.0f) a = 1.0f;
      else a = fminf(1.0f, p / q);
    }
    a_sh[i] = a;
    a_out[(size_t)b * gamma + i] = a;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int n = 0;
    while (n < gamma && u_acc[(size_t)b * gamma + n] < a_sh[n]) ++n;
    int32_t* o = out + (size_t)b * rows_t;
    for (int i = 0; i < n; ++i) o[i] = draft[(size_t)b * gamma + i];
    n_acc[b] = n;
    SeqInfo si{};
    si.n = n;
    si.use_res = n < gamma ? 1 : 0;
    si.mp = mp[n];
    si.sp = sp[n];
    si.mq = n < gamma ? mq[n] : 0.0f;
    si.sq = n < gamma ? sq[n] : 1.0f;
    info[b] = si;
  }
}

// Values of the distribution the final token is drawn from, for this thread's slots of a chunk:
// r_j = max(0, p_j - q_j) (residual) and p_j.
template <bool VEC>
__device__ __forceinline__ void final_values(const SeqInfo& si, const float* __restrict__ prow,
                                             const float* __restrict__ qrow, int lo, int n,
                                             float (&r)[kPerThread], float (&p)[kPerThread],
                                             int (&ix)[kPerThread]) {
  float lp[kPerThread];
  load_chunk<VEC>(prow, lo, n, lp, ix);
  const float inv_sp = 1.0f / si.sp;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) p[j] = __expf(lp[j] - si.mp) * inv_sp;
  if (si.use_res) {
    float lq[kPerThread];
    int ix2[kPerThread];
    load_chunk<VEC>(qrow, lo, n, lq, ix2);
    const float inv_sq = 1.0f / si.sq;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) r[j] = fmaxf(0.0f, p[j] - __expf(lq[j] - si.mq) * inv_sq);
  } else {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) r[j] = p[j];
  }
}

template <bool VEC>
__global__ __launch_bounds__(kVThreads) void residual_sum_kernel(const float* __restrict__ tgt,
                                                                 const float* __restrict__ drf, int gamma,
                                                                 int V, int C,
                                                                 const SeqInfo* __restrict__ info,
                                                                 float2* __restrict__ csum) {
  __shared__ float sv[4];
  const size_t bid = blockIdx.x;
  const int b = (int)(bid / C), c = (int)(bid % C);
  const SeqInfo si = info[b];
  const float* prow = tgt + ((size_t)b * (gamma + 1) + si.n) * V;
  const float* qrow = si.use_res ? drf + ((size_t)b * gamma + si.n) * V : prow;
  const int lo = c * kChunk;
  const int n = V - lo < kChunk ? V - lo : kChunk;
  float r[kPerThread], p[kPerThread];
  int ix[kPerThread];
  final_values<VEC>(si, prow, qrow, lo, n, r, p, ix);
  float zr = 0.0f, zp = 0.0f;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) { zr += r[j]; zp += p[j]; }
  zr = block_sum(zr, sv);
  zp = block_sum(zp, sv);
  if (threadIdx.x == 0) csum[bid] = make_float2(zr, zp);
}

// Inverse-CDF draw: every workgroup of sequence b recomputes the same chunk prefix (same order,
// same arithmetic); the workgroup owning the crossing chunk searches inside it.  With final_dist,
// every workgroup also writes its chunk of f.
template <bool VEC>
__global__ __launch_bounds__(kVThreads) void sample_final_kernel(
    const float* __restrict__ tgt, const float* __restrict__ drf, int gamma, int V, int C,
    const SeqInfo* __restrict__ info, const float2* __restrict__ csum, const float* __restrict__ u_fin,
    int32_t* __restrict__ out, float* __restrict__ fdist) {
  __shared__ float sh_prefix, sh_target, sh_z;
  __shared__ int sh_chunk, sh_usep;
  __shared__ float sv[4];
  __shared__ int si_[4];
  const size_t bid = blockIdx.x;
  const int b = (int)(bid / C), c = (int)(bid % C);
  const SeqInfo si = info[b];
  if (threadIdx.x == 0) {
    const float2* cs = csum + (size_t)b * C;
    float zr = 0.0f, zp = 0.0f;
    for (int k = 0; k < C; ++k) { zr += cs[k].x; zp += cs[k].y; }
    const int usep = !(zr > 0.0f);   // residual mass vanished: draw from p
    const float z = usep ? zp : zr;
    const float target = u_fin[b] * z;
    float run = 0.0f;
    int chunk = -1, last_nz = 0;
    float pre = 0.0f, pre_last = 0.0f;
    for (int k = 0; k < C; ++k) {
      const float zk = usep ? cs[k].y : cs[k].x;
      if (zk > 0.0f) { last_nz = k; pre_last = run; }
      if (chunk < 0 && run + zk > target) { chunk = k; pre = run; }
      run += zk;
    }
    if (chunk < 0) { chunk = last_nz; pre = pre_last; }
    sh_prefix = pre;
    sh_target = target;
    sh_z = z;
    sh_chunk = chunk;
    sh_usep = usep;
  }
  __syncthreads();
  const int usep = sh_usep;
  const float* prow = tgt + ((size_t)b * (gamma + 1) + si.n) * V;
  const float* qrow = si.use_res ? drf + ((size_t)b * gamma + si.n) * V : prow;
  const int lo = c * kChunk;
  const int n = V - lo < kChunk ? V - lo : kChunk;
  const bool mine = c == sh_chunk;
  if (!mine && fdist == nullptr) return;
  float r[kPerThread], p[kPerThread];
  int ix[kPerThread];
  final_values<VEC>(si, prow, qrow, lo, n, r, p, ix);
  if (usep) {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) r[j] = p[j];
  }
  if (fdist) {
    const float inv_z = 1.0f / sh_z;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j)
      if (ix[j] < lo + n) fdist[(size_t)b * V + ix[j]] = r[j] * inv_z;
  }
  if (!mine) return;
  // Inclusive scan of r over the chunk in index order.  Slots of a thread are not contiguous
  // in the VEC layout, so scan slot-major: slot group j covers indices [4*256*j, 4*256*(j+1)).
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __shared__ float wsum[4];
  float base = sh_prefix;
  const float target = sh_target;
  int found = 0x7fffffff;
  int last_pos = -1;
  constexpr int kGroups = VEC ? kPerThread / 4 : kPerThread;
  constexpr int kPerGroup = VEC ? 4 : 1;
#pragma unroll
  for (int j = 0; j < kGroups; ++j) {
    float loc[kPerGroup];
    float tsum = 0.0f;
#pragma unroll
    for (int q = 0; q < kPerGroup; ++q) { tsum += r[j * kPerGroup + q]; loc[q] = tsum; }
    // exclusive scan of tsum across the 256 threads (thread order = index order inside group j)
    float incl = tsum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    float wpre = 0.0f;
    for (int k = 0; k < w; ++k) wpre += wsum[k];
    const float gtot = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
    const float excl = base + wpre + (incl - tsum);
#pragma unroll
    for (int q = 0; q < kPerGroup; ++q) {
      const int idx = ix[j * kPerGroup + q];
      if (idx < lo + n) {
        if (found == 0x7fffffff && excl + loc[q] > target && r[j * kPerGroup + q] > 0.0f) found = idx;
        if (r[j * kPerGroup + q] > 0.0f) last_pos = idx;
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
  if (threadIdx.x == 0) {
    int32_t* o = out + (size_t)b * (gamma + 1);
    o[si.n] = token;
    for (int i = si.n + 1; i <= gamma; ++i) o[i] = -1;
  }
}

static bool vec_ok(const float* p, int V) { return p != nullptr && V % 4 == 0 && aligned16(p); }

int launch_verify_greedy(const float* tgt, const int32_t* d, int B, int gamma, int V, int32_t* t,
                         float* p1, int32_t* n_acc, int32_t* out, void* ws, hipStream_t st) {
  const int C = n_chunks(V);
  VerifyWs w = carve(ws, B, gamma, V);
  const size_t rows = (size_t)B * (gamma + 1);
  const size_t blocks = rows * C;
  if (vec_ok(tgt, V))
    hipLaunchKernelGGL(row_stats_kernel<true>, dim3((unsigned)blocks), dim3(kVThreads), 0, st, tgt,
                       (int)rows, tgt, V, C, w.parts);
  else
    hipLaunchKernelGGL(row_stats_kernel<false>, dim3((unsigned)blocks), dim3(kVThreads), 0, st, tgt,
                       (int)rows, tgt, V, C, w.parts);
  int rc = launch_status();
  if (rc != QS_OK) return rc;
  hipLaunchKernelGGL(greedy_finish_kernel, dim3(B), dim3(kVThreads), 0, st, w.parts, C, gamma, V, d, t,
                     p1, n_acc, out);
  return launch_status();
}

int launch_verify_sample(const float* tgt, const float* drf, const int32_t* d, const float* u_acc,
                         const float* u_fin, int B, int gamma, int V, float* a, int32_t* n_acc,
                         int32_t* out, float* fdist, void* ws, hipStream_t st) {
  const int C = n_chunks(V);
  VerifyWs w = carve(ws, B, gamma, V);
  const size_t rows_t = (size_t)B * (gamma + 1), rows_d = (size_t)B * gamma;
  const size_t blocks = (rows_t + rows_d) * C;
  const bool vec = vec_ok(tgt, V) && (gamma == 0 || vec_ok(drf, V));
  if (vec)
    hipLaunchKernelGGL(row_stats_kernel<true>, dim3((unsigned)blocks), dim3(kVThreads), 0, st, tgt,
                       (int)rows_t, drf, V, C, w.parts);
  else
    hipLaunchKernelGGL(row_stats_kernel<false>, dim3((unsigned)blocks), dim3(kVThreads), 0, st, tgt,
                       (int)rows_t, drf, V, C, w.parts);
  int rc = launch_status();
  if (rc != QS_OK) return rc;
  hipLaunchKernelGGL(sample_decide_kernel, dim3(B), dim3(kVThreads), 0, st, w.parts, C, gamma, V, tgt,
                     drf, d, u_acc, a, n_acc, out, w.info);
  rc = launch_status();
  if (rc != QS_OK) return rc;
  const size_t fb = (size_t)B * C;
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

}  // namespace qs
