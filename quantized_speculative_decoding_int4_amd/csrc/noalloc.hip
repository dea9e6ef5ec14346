// qs_verify_greedy_noalloc: the greedy verify of qs_verify_greedy for callers that cannot allocate
// or pass device memory of their own (code under graph capture, tight serving loops, harnesses
// that forbid allocation).  Its scratch -- the per-sequence arrival counters and the statistics
// partials that qs_verify_greedy keeps in the caller's workspace -- lives in a file-scope device
// array of fixed size, one copy per GPU, held until the process ends.
//
// The array's name is only a host-side stand-in: host code uses the device address that
// hipGetSymbolAddress returns for the current device, looked up once per device and cached.  On a
// device's first call the counter region is cleared by a kernel (graph-capture safe); every call
// leaves the counters at zero again, and the partials are fully rewritten by each call.  All calls
// on one GPU share the array, so calls that overlap in time on one GPU race.

#include <mutex>

#include "qs_internal.h"

namespace qs {

constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;  // 8 MiB per GPU
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

__global__ __launch_bounds__(256) void noalloc_clear_kernel(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Device address of this GPU's scratch array; *fresh is set on the first lookup for the device.
static void* scratch_address(bool* fresh, int* rc) {
  constexpr int kMaxDevices = 64;
  static void* addr[kMaxDevices];
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *rc = QS_ERR_HIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  *fresh = false;
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      *rc = QS_ERR_HIP;
      return nullptr;
    }
    addr[dev] = p;
    *fresh = true;
  }
  *rc = QS_OK;
  return addr[dev];
}

}  // namespace qs

using namespace qs;

extern "C" {

size_t qs_verify_greedy_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

int qs_verify_greedy_noalloc(const float* tgt_logits, const int32_t* draft_ids, int B, int gamma, int V,
                             int32_t* tgt_top1, float* top1_prob, int32_t* n_accept, int32_t* out_tokens,
                             void* stream) {
  if (!tgt_logits || !tgt_top1 || !n_accept || !out_tokens || (gamma > 0 && !draft_ids)) return QS_ERR_INVALID_ARG;
  if (B < 1 || gamma < 0 || V < 1) return QS_ERR_INVALID_ARG;
  const size_t need = qs_verify_workspace_bytes(B, gamma, V);
  if (need == 0) return QS_ERR_UNSUPPORTED;
  if (need > kNoAllocScratchBytes) return QS_ERR_UNSUPPORTED;  // beyond the fixed scratch
  if (!device_info()->ok) return QS_ERR_DEVICE;
  bool fresh = false;
  int rc = QS_OK;
  void* ws = scratch_address(&fresh, &rc);
  if (rc != QS_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (fresh) {  // counters start at zero (every later call leaves them zero)
    const size_t n16 = verify_counter_bytes() / 16;
    hipLaunchKernelGGL(noalloc_clear_kernel, dim3(256), dim3(256), 0, st, static_cast<uint4*>(ws), n16);
    rc = launch_status();
    if (rc != QS_OK) return rc;
  }
  return qs_verify_greedy(tgt_logits, draft_ids, B, gamma, V, tgt_top1, top1_prob, n_accept, out_tokens, ws,
                          need, stream);
}

}  // extern "C"
