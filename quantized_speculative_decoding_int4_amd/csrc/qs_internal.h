// Host-side declarations shared by the translation units of libqspec.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/qspec.h"

namespace qs {

// Cached facts about the current device (checked once per device).
struct DeviceInfo {
  int ok;              // 1 if the device is a gfx950
  int num_cus;         // compute units
  long long clock_khz; // rate of the device wall clock (wall_clock64), kHz
};
const DeviceInfo* device_info();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Launch helpers implemented in linear.hip / verify.hip.
int launch_pack(const int8_t* q, const uint16_t* s, int N, int K, uint8_t* wp,
                uint16_t* sp, hipStream_t st);
size_t linear_workspace(int mode, int M, int N, int K, bool norm_in);
int launch_linear(int mode, const uint16_t* x, const uint8_t* wp, const uint16_t* sp,
                  float* y, int M, int N, int K, int8_t* xq_out, uint16_t* sx_out,
                  int32_t* acc_out, void* ws, size_t ws_bytes, hipStream_t st);

// LM-head with the fused Top-1 epilogue (batched kernel at any M): x fp16 [M][ldx], its rows
// standardised first when norm (the chain's last stage); logits nullable.  The workspace starts
// with the batched kernel's arrival counters (zero before the call, left zero).
size_t lmhead_top1_workspace(int mode, int M, int V, int K);
int launch_lmhead_top1(int mode, const uint16_t* x, int ldx, int norm, const uint8_t* wp, const uint16_t* sp,
                       float* logits, int M, int V, int K, int32_t* top1, float* top1_prob, void* ws, hipStream_t st);

// Input/output placement of one linear inside a chain: x with row stride ldx, optionally
// standardised per row; output either fp32 y [M][N] or fp16(y) into y16 with row stride ldy.
struct LinearIO {
  const uint16_t* x;
  int ldx;
  float* y;
  uint16_t* y16;
  int ldy;
  int norm_in;  // standardise each input row over its K columns first
  int counters_zero;  // the workspace's K-split counters are known to be zero (chain calls)
};
int launch_linear_io(int mode, const LinearIO& io, const uint8_t* wp, const uint16_t* sp, int M, int N,
                     int K, int8_t* xq_out, uint16_t* sx_out, int32_t* acc_out, void* ws,
                     size_t ws_bytes, hipStream_t st);

// Clears the K-split counters at the start of a linear's workspace (before the first linear of a
// chain call); a no-op for row counts that never use the batched kernel.
int linear_clear_counters(int mode, int M, void* ws, hipStream_t st);

// Batched linear (gemm.hip), M >= 16 rows: x fp16 [M][ldx] (W4A16, standardised per row inside
// the kernel when norm) or operand-ordered codes xq [M][K] with fp32 row scales sxf (W4A4); output
// fp32 y [M][N] or fp16 y16 (row stride ldy).  K is split over workgroups when cnt (zeroed arrival
// counters, left zero) and ws (partial slots of gemm_workspace bytes) are given.
size_t gemm_counter_bytes();
size_t gemm_workspace(int mode, int M, int N, int K);
int launch_gemm_clear(unsigned* cnt, hipStream_t st);
// Top-1 epilogue of the batched kernel (LM-head): stats holds gemm_top1_bytes of partials, top1 [M],
// top1_prob [M] (nullable), written by a merge launch that follows the linear's.
struct GemmTop1 {
  unsigned char* stats;
  int32_t* top1;
  float* top1_prob;
};
size_t gemm_top1_bytes(int M, int N);
int launch_gemm(int mode, bool norm, const uint16_t* x, int ldx, const int8_t* xq, const float* sxf,
                const uint8_t* wp, const uint16_t* sp, int M, int N, int K, float* y, uint16_t* y16, int ldy,
                unsigned* cnt, void* ws, size_t ws_bytes, hipStream_t st, const GemmTop1* t1 = nullptr);

// Persistent pass kernel (pass.hip): one resident workgroup per CU runs up to kMaxPassStages
// linears of a chain per launch.
constexpr int kMaxPassStages = 72;
constexpr int kMaxPassWorkgroups = 1024;
// Control region of a persistent pass in the workspace: the Top-1 arrival counter and the error
// word, then one 128-byte arrival flag per workgroup.
constexpr size_t kPassCtrlBytes = 128 + (size_t)kMaxPassWorkgroups * 128;
bool pass_eligible(int mode, int M, const qs_linear_desc* c, int n);
int pass_max_rows(int mode);   // most rows a persistent pass takes in this mode
int pass_launch_count(int mode, int M, const qs_linear_desc* c, int n);  // launches of a persistent pass
// fp16 outputs of all stages but the last, each 256-byte aligned, in chain order
size_t pass_stage_bytes(int M, const qs_linear_desc* c, int n);
// the stage outputs, then (W4A4) one code byte per output at half the output's offset
size_t pass_area_bytes(int mode, int M, const qs_linear_desc* c, int n);
int pass_barrier_timeout_us();  // wall-clock limit of one wait for a stage's input (process-wide)
void set_pass_barrier_timeout_us(int us);
// Top-1 of the final stage (the LM-head): top1 [M], top1_prob [M] (nullable), and stats, the
// partials of pass_top1_bytes(M) bytes.
struct PassTop1 {
  int32_t* top1;
  float* top1_prob;
  unsigned char* stats;
};
size_t pass_top1_bytes(int M);
// out nullable when t1 is given; trace (nullable) receives pass_entry_count(...) x grid x 4 boundary
// timestamps (wall-clock ticks), [entry][workgroup][4]
int launch_pass(int mode, const uint16_t* x, int M, const qs_linear_desc* c, int n, float* out,
                unsigned* ctrl, uint16_t* stage_out, hipStream_t st, const PassTop1* t1 = nullptr,
                unsigned long long* trace = nullptr);
int pass_entry_count(int mode, int M, const qs_linear_desc* c, int n);  // stage-table entries of a pass

size_t verify_workspace(int B, int gamma, int V);
size_t verify_counter_bytes();  // the arrival counters at the start of a verify workspace
int launch_verify_greedy(const float* tgt, const int32_t* d, int B, int gamma, int V,
                         int32_t* t, float* p1, int32_t* n_acc, int32_t* out, void* ws,
                         hipStream_t st);
int launch_accept_greedy(const int32_t* t, const int32_t* d, int B, int gamma, int32_t* n_acc, int32_t* out,
                         hipStream_t st);
int launch_verify_tree_greedy(const float* tgt, const int32_t* tok, const int32_t* par, int B, int T, int V,
                              int32_t* t, int32_t* n_acc, int32_t* out, int32_t* nodes, void* ws, hipStream_t st);
int launch_verify_sample(const float* tgt, const float* drf, const int32_t* d,
                         const float* u_acc, const float* u_fin, int B, int gamma, int V,
                         float* a, int32_t* n_acc, int32_t* out, float* fdist, void* ws,
                         hipStream_t st);

inline int launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? QS_OK : QS_ERR_HIP;
}

}  // namespace qs
