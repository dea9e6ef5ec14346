// qs_chain_forward: one forward pass of a stack of quantized linears (the draft
// pass in W4A4 or the verify pass in W4A16), as persistent pass launches or
// linear by linear on one stream.  Intermediate activations stay in the
// workspace as fp16; each stage after the first standardises its input rows
// inside its own prologue; only the final stage (the LM-head) writes fp32.
// qs_chain_forward_top1 also reduces the final stage's outputs to each row's
// Top-1 and its probability inside that stage's epilogue, so a greedy step
// needs no second pass over the logits.

#include "qs_internal.h"

namespace qs {

static bool chain_ok(const qs_linear_desc* c, int n) {
  if (!c || n < 1) return false;
  for (int i = 0; i < n; ++i) {
    if (!c[i].w_packed || !c[i].s_packed || c[i].N < 1 || c[i].K < QS_GROUP || c[i].K % QS_GROUP ||
        c[i].K > 65536)
      return false;
    if (!aligned16(c[i].w_packed)) return false;
    if (i > 0 && (c[i].K > c[i - 1].N || c[i - 1].N % 8)) return false;
  }
  return true;
}

static size_t act_bytes(int M, const qs_linear_desc* c, int n) {
  int maxn = 8;
  for (int i = 0; i + 1 < n; ++i) maxn = c[i].N > maxn ? c[i].N : maxn;
  return align_up((size_t)M * maxn * 2, 256);
}

// Workspace: two fp16 ping-pong buffers for the launch-per-linear path, then the per-linear scratch
// or the control words of the persistent pass, then (for row counts a persistent pass takes) the
// stage outputs of the persistent pass and, for the integer modes above one row, its shared
// activation codes (pass_area_bytes).
static size_t scratch_bytes(int mode, int M, const qs_linear_desc* c, int n) {
  size_t q = 0;
  for (int i = 0; i < n; ++i) {
    const size_t w = linear_workspace(mode, M, c[i].N, c[i].K, i > 0);
    q = w > q ? w : q;
  }
  return align_up(q > kPassCtrlBytes ? q : kPassCtrlBytes, 256);
}

size_t chain_workspace(int mode, int M, const qs_linear_desc* c, int n) {
  const size_t stages = M <= pass_max_rows(mode) ? pass_area_bytes(mode, M, c, n) : 0;
  return 2 * act_bytes(M, c, n) + scratch_bytes(mode, M, c, n) + stages;
}

// Top-1 region after the chain workspace: the pass's per-workgroup partials, or the LM-head
// Top-1 launch's own workspace (arrival counters, staging, partials) on the per-linear path.
static size_t top1_bytes(int mode, int M, const qs_linear_desc* c, int n) {
  const size_t p = pass_top1_bytes(M);
  const size_t l = lmhead_top1_workspace(mode, M, c[n - 1].N, c[n - 1].K);
  return align_up(p > l ? p : l, 256);
}

// One pass of the chain; t1 (nullable) asks for the final stage's Top-1, with its region at t1_ws.
static int chain_run(int mode, const uint16_t* x, int M, const qs_linear_desc* chain, int n, float* out,
                     int32_t* top1, float* top1_prob, void* ws, size_t ws_bytes, hipStream_t st,
                     unsigned long long* trace = nullptr) {
  const size_t ab = act_bytes(M, chain, n);
  uint16_t* buf[2] = {reinterpret_cast<uint16_t*>(ws),
                      reinterpret_cast<uint16_t*>(static_cast<unsigned char*>(ws) + ab)};
  void* qws = static_cast<unsigned char*>(ws) + 2 * ab;
  const size_t main_bytes = chain_workspace(mode, M, chain, n);
  unsigned char* t1_ws = static_cast<unsigned char*>(ws) + main_bytes;
  const size_t qws_bytes = main_bytes - 2 * ab;
  if (pass_eligible(mode, M, chain, n)) {
    uint16_t* stage_out =
        reinterpret_cast<uint16_t*>(static_cast<unsigned char*>(qws) + scratch_bytes(mode, M, chain, n));
    PassTop1 t1{top1, top1_prob, t1_ws};
    return launch_pass(mode, x, M, chain, n, out, static_cast<unsigned*>(qws), stage_out, st,
                       top1 ? &t1 : nullptr, trace);
  }
  const uint16_t* in = x;
  int ldx = chain[0].K;
  // every linear's workspace starts at qws, so its K-split counters are shared: clear them once
  int rc = linear_clear_counters(mode, M, qws, st);
  if (rc != QS_OK) return rc;
  if (top1) {  // the LM-head Top-1 launch's counters start at zero
    rc = launch_gemm_clear(reinterpret_cast<unsigned*>(t1_ws), st);
    if (rc != QS_OK) return rc;
  }
  for (int i = 0; i < n; ++i) {
    if (top1 && i + 1 == n)
      return launch_lmhead_top1(mode, in, ldx, i > 0, chain[i].w_packed, chain[i].s_packed, out, M, chain[i].N,
                                chain[i].K, top1, top1_prob, t1_ws, st);
    LinearIO io{};
    io.x = in;
    io.ldx = ldx;
    io.norm_in = i > 0;
    io.counters_zero = 1;
    if (i + 1 == n) {
      io.y = out;
    } else {
      io.y16 = buf[i & 1];
      io.ldy = chain[i].N;
    }
    rc = launch_linear_io(mode, io, chain[i].w_packed, chain[i].s_packed, M, chain[i].N, chain[i].K, nullptr,
                          nullptr, nullptr, qws, qws_bytes, st);
    if (rc != QS_OK) return rc;
    in = buf[i & 1];
    ldx = chain[i].N;
  }
  return QS_OK;
}

}  // namespace qs

using namespace qs;

extern "C" {

size_t qs_chain_workspace_bytes(int mode, int M, const qs_linear_desc* chain, int n) {
  if ((mode != QS_W4A16 && mode != QS_W4A4 && mode != QS_W4A8) || M < 1 || M > QS_MAX_M || !chain_ok(chain, n)) return 0;
  return chain_workspace(mode, M, chain, n);
}

int qs_chain_pass_launches(int mode, int M, const qs_linear_desc* chain, int n) {
  if (mode != QS_W4A16 && mode != QS_W4A4 && mode != QS_W4A8) return QS_ERR_INVALID_ARG;
  if (!chain_ok(chain, n) || M < 1) return QS_ERR_INVALID_ARG;
  if (M > QS_MAX_M) return QS_ERR_UNSUPPORTED;
  if (!device_info()->ok) return QS_ERR_DEVICE;
  return pass_eligible(mode, M, chain, n) ? pass_launch_count(mode, M, chain, n) : 0;
}

size_t qs_chain_trace_bytes(int mode, int M, const qs_linear_desc* chain, int n) {
  if ((mode != QS_W4A16 && mode != QS_W4A4 && mode != QS_W4A8) || M < 1 || M > QS_MAX_M || !chain_ok(chain, n)) return 0;
  if (!device_info()->ok || !pass_eligible(mode, M, chain, n)) return 0;
  return (size_t)pass_entry_count(mode, M, chain, n) * (size_t)device_info()->num_cus * 4 * sizeof(unsigned long long);
}

int qs_chain_forward_trace(int mode, const uint16_t* x, int M, const qs_linear_desc* chain, int n, float* out,
                           void* ws, size_t ws_bytes, unsigned long long* trace, size_t trace_bytes, void* stream) {
  if (mode != QS_W4A16 && mode != QS_W4A4 && mode != QS_W4A8) return QS_ERR_INVALID_ARG;
  if (!x || !out || !trace || !chain_ok(chain, n) || M < 1) return QS_ERR_INVALID_ARG;
  if (M > QS_MAX_M) return QS_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(trace)) return QS_ERR_MISALIGNED;
  if (!ws || ws_bytes < chain_workspace(mode, M, chain, n)) return QS_ERR_WORKSPACE;
  if (!aligned16(ws)) return QS_ERR_MISALIGNED;
  if (!device_info()->ok) return QS_ERR_DEVICE;
  if (!pass_eligible(mode, M, chain, n)) return QS_ERR_UNSUPPORTED;  // nothing to trace: one launch per linear
  if (trace_bytes < qs_chain_trace_bytes(mode, M, chain, n)) return QS_ERR_WORKSPACE;
  return chain_run(mode, x, M, chain, n, out, nullptr, nullptr, ws, ws_bytes, static_cast<hipStream_t>(stream),
                   trace);
}

int qs_set_barrier_timeout_us(int us) {
  if (us < 0) return QS_ERR_INVALID_ARG;
  set_pass_barrier_timeout_us(us);
  return QS_OK;
}

int qs_chain_pass_status(int mode, int M, const qs_linear_desc* chain, int n, void* ws, size_t ws_bytes,
                         int* timed_out, void* stream) {
  if (mode != QS_W4A16 && mode != QS_W4A4 && mode != QS_W4A8) return QS_ERR_INVALID_ARG;
  if (!timed_out || !chain_ok(chain, n) || M < 1) return QS_ERR_INVALID_ARG;
  if (M > QS_MAX_M) return QS_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < chain_workspace(mode, M, chain, n)) return QS_ERR_WORKSPACE;
  if (!device_info()->ok) return QS_ERR_DEVICE;
  *timed_out = 0;
  if (!pass_eligible(mode, M, chain, n)) return QS_OK;  // one launch per linear: no waits
  hipStream_t st = static_cast<hipStream_t>(stream);
  // control region after the two activation buffers; its second word is the error word
  unsigned* err = reinterpret_cast<unsigned*>(static_cast<unsigned char*>(ws) + 2 * act_bytes(M, chain, n)) + 1;
  unsigned word = 0;
  if (hipMemcpyAsync(&word, err, sizeof(word), hipMemcpyDeviceToHost, st) != hipSuccess) return QS_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return QS_ERR_HIP;
  *timed_out = word != 0 ? 1 : 0;
  return QS_OK;
}

int qs_chain_forward(int mode, const uint16_t* x, int M, const qs_linear_desc* chain, int n, float* out,
                     void* ws, size_t ws_bytes, void* stream) {
  if (mode != QS_W4A16 && mode != QS_W4A4 && mode != QS_W4A8) return QS_ERR_INVALID_ARG;
  if (!x || !out || !chain_ok(chain, n) || M < 1) return QS_ERR_INVALID_ARG;
  if (M > QS_MAX_M) return QS_ERR_UNSUPPORTED;
  if (!aligned16(x)) return QS_ERR_MISALIGNED;
  if (!ws || ws_bytes < chain_workspace(mode, M, chain, n)) return QS_ERR_WORKSPACE;
  if (!aligned16(ws)) return QS_ERR_MISALIGNED;
  if (!device_info()->ok) return QS_ERR_DEVICE;
  return chain_run(mode, x, M, chain, n, out, nullptr, nullptr, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

size_t qs_chain_top1_workspace_bytes(int mode, int M, const qs_linear_desc* chain, int n) {
  if ((mode != QS_W4A16 && mode != QS_W4A4 && mode != QS_W4A8) || M < 1 || M > QS_MAX_M || !chain_ok(chain, n)) return 0;
  return chain_workspace(mode, M, chain, n) + top1_bytes(mode, M, chain, n);
}

int qs_chain_forward_top1(int mode, const uint16_t* x, int M, const qs_linear_desc* chain, int n, float* out,
                          int32_t* top1, float* top1_prob, void* ws, size_t ws_bytes, void* stream) {
  if (mode != QS_W4A16 && mode != QS_W4A4 && mode != QS_W4A8) return QS_ERR_INVALID_ARG;
  if (!x || !top1 || !chain_ok(chain, n) || M < 1) return QS_ERR_INVALID_ARG;
  if (M > QS_MAX_M) return QS_ERR_UNSUPPORTED;
  if (!aligned16(x)) return QS_ERR_MISALIGNED;
  if (!ws || ws_bytes < chain_workspace(mode, M, chain, n) + top1_bytes(mode, M, chain, n)) return QS_ERR_WORKSPACE;
  if (!aligned16(ws)) return QS_ERR_MISALIGNED;
  if (!device_info()->ok) return QS_ERR_DEVICE;
  return chain_run(mode, x, M, chain, n, out, top1, top1_prob, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

}  // extern "C"
