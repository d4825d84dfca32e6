// LoRA-down reduction: t = bf16(sum over the K chunks of the partial sums
// s x_t A^T) [QeRL summary, §3.4, Eq. 2 (LoRA side branch)].  Shared by
// its own launch (linear.hip) and by the extra workgroups that a whole
// decode call appends to a split-K contraction launch (decode_m128.h,
// decode_lds.h), so both give the same bits.
#pragma once

#include "qerl_device.h"

namespace qerl {

struct TReduceArgs {
  const float* tpart;   // [kchunks, mpad, rpad32] fp32 partials (s applied)
  uint16_t* t;          // [mpad, rpad16] bf16
  int64_t mpad;
  int rpad32, rpad16, kchunks;
  // t is read by other workgroups of the same launch: stored at device
  // scope (past the per-XCD L2s)
  int coherent;
};

// Output i = row * rpad16 + j.  Chunk c goes to partial sum c % 4 (the
// loads of a batch of 16 chunks are issued before the first add), then
// (s0 + s1) + (s2 + s3): a fixed order.
__device__ __forceinline__ void treduce_one(const TReduceArgs& a, int64_t i) {
  const int64_t mrow = i / a.rpad16;
  const int j = (int)(i - mrow * a.rpad16);
  const float* src = a.tpart + mrow * a.rpad32 + j;
  const int64_t stride = a.mpad * a.rpad32;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int c0 = 0; c0 < a.kchunks; c0 += 16) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      v[u] = c0 + u < a.kchunks ? src[(int64_t)(c0 + u) * stride] : 0.0f;
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (c0 + u < a.kchunks) acc[u & 3] += v[u];
  }
  const uint16_t tb = f32_to_bf16_bits((acc[0] + acc[1]) + (acc[2] + acc[3]));
  if (a.coherent)
    __hip_atomic_store(a.t + i, tb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    a.t[i] = tb;
}

// Outputs first, first + stride, ... of the mpad x rpad16.
__device__ __forceinline__ void treduce_strided(const TReduceArgs& a, int64_t first,
                                                int64_t stride) {
  const int64_t total = a.mpad * a.rpad16;
  for (int64_t i = first; i < total; i += stride) treduce_one(a, i);
}

}  // namespace qerl
