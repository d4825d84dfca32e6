// Attention stub between the fused q/k/v layer and the output projection of
// a decode step (the pages' layers W_q, W_k, W_v, W_o [QeRL summary, §3.4
// "Layer coverage"]; attention itself is the model's, not the pages').
// Every token row is attended over a context of one position: its own key
// and value.  The softmax of a single score is exactly 1, so the output of
// query head h is the value of its key/value head h / (hq / hkv) (grouped
// query attention), copied bit for bit:
//     out[i, h dh + e] = qkv[i, (hq + hkv + h / (hq / hkv)) dh + e]
// qkv holds the q heads, then the k heads, then the v heads of each row.
#include "qerl_device.h"
#include "qerl_internal.h"

namespace qerl {
namespace {

// One thread per 8 output values (16 bytes).
__global__ __launch_bounds__(256) void attn_stub_kernel(const uint16_t* __restrict__ qkv,
                                                        int64_t m, int hq, int hkv, int dh,
                                                        uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_row = (int64_t)hq * dh / 8;
  if (i >= m * per_row) return;
  const int64_t row = i / per_row;
  const int64_t col = (i - row * per_row) * 8;          // output column
  const int h = (int)(col / dh), e = (int)(col - (int64_t)h * dh);
  const int g = h / (hq / hkv);                         // its key/value head
  const int64_t ld = (int64_t)(hq + 2 * hkv) * dh;
  const uint16_t* src = qkv + row * ld + (int64_t)(hq + hkv + g) * dh + e;
  *reinterpret_cast<uint4*>(out + row * (int64_t)hq * dh + col) =
      *reinterpret_cast<const uint4*>(src);
}

}  // namespace

hipError_t launch_attention_stub(const uint16_t* qkv, int64_t m, int hq, int hkv, int dh,
                                 uint16_t* out, hipStream_t stream) {
  const int64_t threads = m * (int64_t)hq * dh / 8;
  hipLaunchKernelGGL(attn_stub_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     stream, qkv, m, hq, hkv, dh, out);
  return hipGetLastError();
}

}  // namespace qerl
