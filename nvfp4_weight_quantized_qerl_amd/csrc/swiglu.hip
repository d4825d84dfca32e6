// Gated feed-forward activation between the fused gate/up layer and the
// down layer of the Qwen2.5 feed-forward block (W_gate, W_up, W_down
// [QeRL summary, §3.4 "Layer coverage"]):
//     out[m, j] = bf16( SiLU(g[m, j]) * u[m, j] ),  SiLU(g) = g / (1 + exp(-g))
// where g and u are the two halves of the fused gate/up output [m, 2 d]
// (gate in columns 0 .. d-1, up in d .. 2d-1).  fp32 arithmetic (the
// exponential and the division by the hardware's approximations), one
// rounding to bf16.  HBM-bound: 6 bytes per output element; each thread
// handles eight consecutive outputs with 16-byte loads and stores.
#include "qerl_act.h"
#include "qerl_device.h"
#include "qerl_internal.h"

namespace qerl {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void swiglu_kernel(const uint16_t* __restrict__ gu, int64_t m,
                                                     int64_t d, uint16_t* __restrict__ out) {
  const int64_t per_row = d / 8;
  const int64_t total = m * per_row;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t row = i / per_row, j = 8 * (i - row * per_row);
    const u32x4 g = *reinterpret_cast<const u32x4*>(gu + row * 2 * d + j);
    const u32x4 u = *reinterpret_cast<const u32x4*>(gu + row * 2 * d + d + j);
    const uint4 o = swiglu8(__builtin_bit_cast(uint4, g), __builtin_bit_cast(uint4, u));
    *reinterpret_cast<u32x4*>(out + row * d + j) = __builtin_bit_cast(u32x4, o);
  }
}

}  // namespace

hipError_t launch_swiglu(const uint16_t* gu, int64_t m, int64_t d, uint16_t* out,
                         hipStream_t stream) {
  const int64_t threads = m * (d / 8);
  const int64_t groups = std::min<int64_t>((threads + 255) / 256, 16 * (int64_t)device_cu_count());
  hipLaunchKernelGGL(swiglu_kernel, dim3((unsigned)groups), dim3(256), 0, stream, gu, m, d, out);
  return hipGetLastError();
}

}  // namespace qerl
