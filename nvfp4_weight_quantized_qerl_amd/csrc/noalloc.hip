// qerl_linear_decode_noalloc: qerl_linear_decode for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).  The layer's scratch (noisy
// activations, LoRA-down partials and t, split-K partial sums) lives in a
// file-scope device array of kScratchBytes instead of a caller workspace.
//
// Each GPU the library runs on holds its own copy of the array for the
// life of the process.  Its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and kept; host code only
// ever passes that address, never the array's name (which in host code is
// a host-side stand-in).  Nothing in the scratch needs to start at zero:
// every call writes each byte it later reads.  All calls on one GPU share
// its array, so calls that overlap on one GPU (several streams or host
// threads at once) race and must be serialised by the caller.
#include <mutex>

#include "qerl.h"
#include "qerl_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;   // 64 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (looked up on first use).
qerl_status scratch_for_current_device(void* stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QERL_ERR_HIP;
  if (stream) {
    int sdev = -1;
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess)
      return QERL_ERR_HIP;
    if (sdev != dev) return QERL_ERR_RANGE;   // the stream must belong to the current device
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QERL_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QERL_OK;
}

}  // namespace

extern "C" {

size_t qerl_linear_noalloc_scratch_bytes(void) { return kScratchBytes; }

qerl_status qerl_linear_decode_noalloc(const void* x, int64_t m, const void* codes,
                                       const void* scales, const float* gscale, int64_t n,
                                       int64_t k, const void* lora_a, const void* lora_b,
                                       int32_t r, float lora_scale, const float* z, void* y,
                                       void* stream) {
  // Sizes beyond the array are refused before anything is enqueued.
  const int32_t r_eff = (r > 0 && lora_a && lora_b) ? r : 0;
  const size_t need = qerl_linear_workspace_bytes(m, n, k, r_eff);
  if (need > kScratchBytes) return QERL_ERR_WORKSPACE;
  void* ws = nullptr;
  const qerl_status s = scratch_for_current_device(stream, &ws);
  if (s != QERL_OK) return s;
  return qerl_linear_decode(x, m, codes, scales, gscale, n, k, lora_a, lora_b, r, lora_scale, z,
                            y, ws, kScratchBytes, stream);
}

}  // extern "C"
