// Elementwise helpers shared by several kernels, so that every kernel that
// forms these values forms them bit-identically:
//   noisy8   the AQN-noised activations x_t = bf16(x (1 + z)) [QeRL summary,
//            §3.4, Eq. 12], used by the prepare and by the dA contraction
//            of the backward;
//   swiglu8  the gated feed-forward activation bf16(SiLU(gate) up) (Qwen2.5
//            feed-forward block; W_gate, W_up, W_down [§3.4 "Layer
//            coverage"]), used by the SwiGLU kernel and by the prepare that
//            forms the down layer's input from the fused gate/up output.
#pragma once

#include "qerl_device.h"

namespace qerl {

// x_t = bf16(x (1 + z)) of 8 consecutive channels from their noise z0, z1.
__device__ __forceinline__ uint4 noisy8(uint4 xv, float4 z0, float4 z1) {
  xv.x = pack_bf16x2(bf16_to_f32(xv.x & 0xffffu) * (1.0f + z0.x),
                     bf16_to_f32(xv.x >> 16) * (1.0f + z0.y));
  xv.y = pack_bf16x2(bf16_to_f32(xv.y & 0xffffu) * (1.0f + z0.z),
                     bf16_to_f32(xv.y >> 16) * (1.0f + z0.w));
  xv.z = pack_bf16x2(bf16_to_f32(xv.z & 0xffffu) * (1.0f + z1.x),
                     bf16_to_f32(xv.z >> 16) * (1.0f + z1.y));
  xv.w = pack_bf16x2(bf16_to_f32(xv.w & 0xffffu) * (1.0f + z1.z),
                     bf16_to_f32(xv.w >> 16) * (1.0f + z1.w));
  return xv;
}

// SiLU(g) = g / (1 + exp(-g)) in fp32 with the hardware exponential and
// reciprocal (each within a few fp32 ulps, far below one bf16 ulp, the
// precision the result is rounded to).
__device__ __forceinline__ float silu_f32(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// bf16(SiLU(g) * u) of eight consecutive channels from their gate and up
// values (bf16 pairs, channel i in half i % 2 of dword i / 2): one rounding.
__device__ __forceinline__ uint4 swiglu8(uint4 g, uint4 u) {
  uint4 o;
  o.x = pack_bf16x2(silu_f32(bf16_to_f32(g.x & 0xffffu)) * bf16_to_f32(u.x & 0xffffu),
                    silu_f32(bf16_to_f32(g.x >> 16)) * bf16_to_f32(u.x >> 16));
  o.y = pack_bf16x2(silu_f32(bf16_to_f32(g.y & 0xffffu)) * bf16_to_f32(u.y & 0xffffu),
                    silu_f32(bf16_to_f32(g.y >> 16)) * bf16_to_f32(u.y >> 16));
  o.z = pack_bf16x2(silu_f32(bf16_to_f32(g.z & 0xffffu)) * bf16_to_f32(u.z & 0xffffu),
                    silu_f32(bf16_to_f32(g.z >> 16)) * bf16_to_f32(u.z >> 16));
  o.w = pack_bf16x2(silu_f32(bf16_to_f32(g.w & 0xffffu)) * bf16_to_f32(u.w & 0xffffu),
                    silu_f32(bf16_to_f32(g.w >> 16)) * bf16_to_f32(u.w >> 16));
  return o;
}

}  // namespace qerl
