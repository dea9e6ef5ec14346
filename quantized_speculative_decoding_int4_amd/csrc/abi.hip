// extern "C" entry points of libqspec (declared and documented in include/qspec.h):
// host-side argument checks, then the launchers in linear.hip / verify.hip.

#include <climits>
#include <cstring>
#include <mutex>

#include "qs_internal.h"

namespace qs {

const DeviceInfo* device_info() {
  constexpr int kMaxDevices = 64;
  static DeviceInfo cache[kMaxDevices];
  static bool filled[kMaxDevices];
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    static DeviceInfo bad{0, 0, 0};
    return &bad;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!filled[dev]) {
    hipDeviceProp_t prop;
    DeviceInfo d{0, 0, 0};
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess) {
      d.ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
      d.num_cus = prop.multiProcessorCount;
      int khz = 0;
      if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
        khz = 100000;
      d.clock_khz = khz;
    }
    cache[dev] = d;
    filled[dev] = true;
  }
  return &cache[dev];
}

static bool linear_shape_ok(int M, int N, int K) {
  return M >= 1 && N >= 1 && K >= QS_GROUP && K % QS_GROUP == 0 && K <= 65536 &&
         (size_t)N * (size_t)K / 2 < ((size_t)1 << 40);
}

static constexpr int kMaxGamma = 63;
static constexpr int kMaxVocab = 1 << 24;

}  // namespace qs

using namespace qs;

extern "C" {

const char* qs_status_string(int status) {
  switch (status) {
    case QS_OK: return "ok";
    case QS_ERR_INVALID_ARG: return "invalid argument (null pointer, shape or mode)";
    case QS_ERR_UNSUPPORTED: return "shape outside the supported range";
    case QS_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case QS_ERR_WORKSPACE: return "workspace missing or too small";
    case QS_ERR_HIP: return "HIP runtime error at launch";
    case QS_ERR_DEVICE: return "current device is not a gfx950 GPU";
    default: return "unknown status";
  }
}

size_t qs_packed_weight_bytes(int N, int K) {
  if (N < 1 || K < QS_GROUP || K % QS_GROUP) return 0;
  return (size_t)((N + 15) / 16) * 16 * (size_t)K / 2;
}

size_t qs_packed_scale_bytes(int N, int K) {
  if (N < 1 || K < QS_GROUP || K % QS_GROUP) return 0;
  return (size_t)((N + 15) / 16) * 16 * (size_t)(K / QS_GROUP) * 2;
}

int qs_pack_weights(const int8_t* q, const uint16_t* s, int N, int K, uint8_t* w_packed,
                    uint16_t* s_packed, void* stream) {
  if (!q || !s || !w_packed || !s_packed) return QS_ERR_INVALID_ARG;
  if (!linear_shape_ok(1, N, K)) return QS_ERR_INVALID_ARG;
  if (!aligned16(w_packed)) return QS_ERR_MISALIGNED;
  if (!device_info()->ok) return QS_ERR_DEVICE;
  return launch_pack(q, s, N, K, w_packed, s_packed, static_cast<hipStream_t>(stream));
}

int qs_linear_w4a16(const uint16_t* x, const uint8_t* w_packed, const uint16_t* s_packed, float* y,
                    int M, int N, int K, void* stream) {
  if (!x || !w_packed || !s_packed || !y) return QS_ERR_INVALID_ARG;
  if (!linear_shape_ok(M, N, K)) return QS_ERR_INVALID_ARG;
  if (M > QS_MAX_M) return QS_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(w_packed)) return QS_ERR_MISALIGNED;
  if (!device_info()->ok) return QS_ERR_DEVICE;
  return launch_linear(QS_W4A16, x, w_packed, s_packed, y, M, N, K, nullptr, nullptr, nullptr, nullptr,
                       0, static_cast<hipStream_t>(stream));
}

size_t qs_linear_workspace_bytes(int mode, int M, int N, int K) {
  if ((mode != QS_W4A16 && mode != QS_W4A4 && mode != QS_W4A8) || !linear_shape_ok(M, N, K) || M > QS_MAX_M)
    return 0;
  return linear_workspace(mode, M, N, K, false);
}

static int linear_int_mode(int mode, const uint16_t* x, const uint8_t* w_packed, const uint16_t* s_packed,
                           float* y, int M, int N, int K, int8_t* xq_out, uint16_t* sx_out, int32_t* acc_out,
                           void* ws, size_t ws_bytes, void* stream) {
  if (!x || !w_packed || !s_packed || !y) return QS_ERR_INVALID_ARG;
  if (!linear_shape_ok(M, N, K)) return QS_ERR_INVALID_ARG;
  if (M > QS_MAX_M) return QS_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(w_packed)) return QS_ERR_MISALIGNED;
  if (xq_out && ((reinterpret_cast<uintptr_t>(xq_out) & 7u) != 0)) return QS_ERR_MISALIGNED;
  const size_t need = linear_workspace(mode, M, N, K, false);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return QS_ERR_WORKSPACE;
  if (ws && !aligned16(ws)) return QS_ERR_MISALIGNED;
  if (!device_info()->ok) return QS_ERR_DEVICE;
  return launch_linear(mode, x, w_packed, s_packed, y, M, N, K, xq_out, sx_out, acc_out, ws, ws_bytes,
                       static_cast<hipStream_t>(stream));
}

int qs_linear_w4a4(const uint16_t* x, const uint8_t* w_packed, const uint16_t* s_packed, float* y, int M,
                   int N, int K, int8_t* xq_out, uint16_t* sx_out, int32_t* acc_out, void* ws,
                   size_t ws_bytes, void* stream) {
  return linear_int_mode(QS_W4A4, x, w_packed, s_packed, y, M, N, K, xq_out, sx_out, acc_out, ws, ws_bytes,
                         stream);
}

int qs_linear_w4a8(const uint16_t* x, const uint8_t* w_packed, const uint16_t* s_packed, float* y, int M,
                   int N, int K, int8_t* xq_out, uint16_t* sx_out, int32_t* acc_out, void* ws,
                   size_t ws_bytes, void* stream) {
  return linear_int_mode(QS_W4A8, x, w_packed, s_packed, y, M, N, K, xq_out, sx_out, acc_out, ws, ws_bytes,
                         stream);
}

int qs_lmhead(int mode, const uint16_t* x, const uint8_t* w_packed, const uint16_t* s_packed,
              float* logits, int M, int V, int K, void* ws, size_t ws_bytes, void* stream) {
  if (mode != QS_W4A16 && mode != QS_W4A4 && mode != QS_W4A8) return QS_ERR_INVALID_ARG;
  if (mode == QS_W4A16)
    return qs_linear_w4a16(x, w_packed, s_packed, logits, M, V, K, stream);
  return linear_int_mode(mode, x, w_packed, s_packed, logits, M, V, K, nullptr, nullptr, nullptr, ws, ws_bytes,
                         stream);
}

size_t qs_lmhead_top1_workspace_bytes(int mode, int M, int V, int K) {
  if ((mode != QS_W4A16 && mode != QS_W4A4 && mode != QS_W4A8) || !linear_shape_ok(M, V, K) || M > QS_MAX_M)
    return 0;
  return lmhead_top1_workspace(mode, M, V, K);
}

int qs_lmhead_top1(int mode, const uint16_t* x, const uint8_t* w_packed, const uint16_t* s_packed, float* logits,
                   int M, int V, int K, int32_t* top1, float* top1_prob, void* ws, size_t ws_bytes, void* stream) {
  if (mode != QS_W4A16 && mode != QS_W4A4 && mode != QS_W4A8) return QS_ERR_INVALID_ARG;
  if (!x || !w_packed || !s_packed || !top1 || !linear_shape_ok(M, V, K)) return QS_ERR_INVALID_ARG;
  if (M > QS_MAX_M) return QS_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(w_packed)) return QS_ERR_MISALIGNED;
  if (!ws || ws_bytes < lmhead_top1_workspace(mode, M, V, K)) return QS_ERR_WORKSPACE;
  if (!aligned16(ws)) return QS_ERR_MISALIGNED;
  if (!device_info()->ok) return QS_ERR_DEVICE;
  return launch_lmhead_top1(mode, x, K, 0, w_packed, s_packed, logits, M, V, K, top1, top1_prob, ws,
                            static_cast<hipStream_t>(stream));
}

size_t qs_verify_workspace_bytes(int B, int gamma, int V) {
  if (B < 1 || gamma < 0 || gamma > kMaxGamma || V < 1 || V > kMaxVocab) return 0;
  return verify_workspace(B, gamma, V);
}

static int verify_common_checks(const float* tgt, int B, int gamma, int V, void* ws, size_t ws_bytes) {
  if (!tgt) return QS_ERR_INVALID_ARG;
  if (B < 1 || gamma < 0 || V < 1) return QS_ERR_INVALID_ARG;
  if (gamma > kMaxGamma || V > kMaxVocab) return QS_ERR_UNSUPPORTED;
  const size_t C = (size_t)((V + 2047) / 2048);  // the finest chunking of a row
  const size_t Bb = B < QS_MAX_VERIFY_SEQS ? (size_t)B : (size_t)QS_MAX_VERIFY_SEQS;  // one block's grid
  if (Bb * (2 * (size_t)gamma + 1) * C > (size_t)INT_MAX) return QS_ERR_UNSUPPORTED;
  const size_t need = verify_workspace(B, gamma, V);
  if (ws == nullptr || ws_bytes < need) return QS_ERR_WORKSPACE;
  if (!aligned16(ws)) return QS_ERR_MISALIGNED;
  return QS_OK;
}

int qs_verify_greedy(const float* tgt_logits, const int32_t* draft_ids, int B, int gamma, int V,
                     int32_t* tgt_top1, float* top1_prob, int32_t* n_accept, int32_t* out_tokens, void* ws,
                     size_t ws_bytes, void* stream) {
  int rc = verify_common_checks(tgt_logits, B, gamma, V, ws, ws_bytes);
  if (rc != QS_OK) return rc;
  if (!tgt_top1 || !n_accept || !out_tokens || (gamma > 0 && !draft_ids)) return QS_ERR_INVALID_ARG;
  if (!device_info()->ok) return QS_ERR_DEVICE;
  return launch_verify_greedy(tgt_logits, draft_ids, B, gamma, V, tgt_top1, top1_prob, n_accept, out_tokens,
                              ws, static_cast<hipStream_t>(stream));
}

int qs_accept_greedy(const int32_t* tgt_top1, const int32_t* draft_ids, int B, int gamma, int32_t* n_accept,
                     int32_t* out_tokens, void* stream) {
  if (!tgt_top1 || !n_accept || !out_tokens || (gamma > 0 && !draft_ids)) return QS_ERR_INVALID_ARG;
  if (B < 1 || gamma < 0) return QS_ERR_INVALID_ARG;
  if (gamma > kMaxGamma) return QS_ERR_UNSUPPORTED;
  if (!device_info()->ok) return QS_ERR_DEVICE;
  return launch_accept_greedy(tgt_top1, draft_ids, B, gamma, n_accept, out_tokens, static_cast<hipStream_t>(stream));
}

int qs_verify_tree_greedy(const float* tgt_logits, const int32_t* tokens, const int32_t* parent, int B, int T,
                          int V, int32_t* tgt_top1, int32_t* n_accept, int32_t* out_tokens, int32_t* out_nodes,
                          void* ws, size_t ws_bytes, void* stream) {
  if (T < 1) return QS_ERR_INVALID_ARG;
  int rc = verify_common_checks(tgt_logits, B, T - 1, V, ws, ws_bytes);
  if (rc != QS_OK) return rc;
  if (!tgt_top1 || !n_accept || !out_tokens || (T > 1 && (!tokens || !parent))) return QS_ERR_INVALID_ARG;
  if (!device_info()->ok) return QS_ERR_DEVICE;
  return launch_verify_tree_greedy(tgt_logits, tokens, parent, B, T, V, tgt_top1, n_accept, out_tokens, out_nodes,
                                   ws, static_cast<hipStream_t>(stream));
}

int qs_verify_sample(const float* tgt_logits, const float* drf_logits, const int32_t* draft_ids,
                     const float* u_accept, const float* u_final, int B, int gamma, int V, float* accept_prob,
                     int32_t* n_accept, int32_t* out_tokens, float* final_dist, void* ws, size_t ws_bytes,
                     void* stream) {
  int rc = verify_common_checks(tgt_logits, B, gamma, V, ws, ws_bytes);
  if (rc != QS_OK) return rc;
  if (!u_final || !n_accept || !out_tokens) return QS_ERR_INVALID_ARG;
  if (gamma > 0 && (!drf_logits || !draft_ids || !u_accept || !accept_prob)) return QS_ERR_INVALID_ARG;
  if (!device_info()->ok) return QS_ERR_DEVICE;
  return launch_verify_sample(tgt_logits, drf_logits, draft_ids, u_accept, u_final, B, gamma, V, accept_prob,
                              n_accept, out_tokens, final_dist, ws, static_cast<hipStream_t>(stream));
}

}  // extern "C"
