// MXFP4 variant: E2M1 codes with one E8M0 (power-of-two) scale per 32
// elements [QeRL summary, §3.4, the formats compared beside NVFP4; the
// scale rule is the OCP Microscaling (MX) v1.0 one]:
//   X    = 2^(floor(log2 amax_b) - 2),  byte = that exponent + 127 in [0, 254]
//   code = sign | RNE_E2M1,sat(|w| / X), ties to even, saturating at 6
// Every threshold t X (t an E2M1 midpoint) is a power of two times a value
// of at most 3 bits, exact in fp32 (subnormals included: the library is
// built without denormal flushing), so comparing the bf16 |w| with it in
// fp32 decides each code exactly.
//
// mx_to_nv re-expresses the scales in the NVFP4 layout of this library (an
// E4M3 per 16 elements and an FP32 tensor scale), which lets the NVFP4
// kernels run the MXFP4 layer exactly: S = 2^(E_max - 8) and each 16-block
// scale 2^(e - E_max + 8), an E4M3 power of two when e >= E_max - 17; a
// block below that with a nonzero code sets the range flag.
#include <algorithm>

#include "qerl_device.h"
#include "qerl_internal.h"

namespace qerl {
namespace {

__global__ void mx_reset(uint32_t* slot, int32_t* flag) {
  *slot = 0u;
  if (flag) *flag = 0;
}

__global__ void mx_flag_reset(int32_t* flag) { *flag = 0; }

// One thread per 32-element block, grid-stride.
__global__ __launch_bounds__(256) void mx_encode(const uint4* __restrict__ w, int64_t nblocks,
                                                 uint4* __restrict__ codes,
                                                 uint8_t* __restrict__ scales,
                                                 int32_t* __restrict__ flag) {
  const float mids[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblocks;
       b += (int64_t)gridDim.x * blockDim.x) {
    uint32_t words[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = w[4 * b + i];
      words[4 * i] = v.x;
      words[4 * i + 1] = v.y;
      words[4 * i + 2] = v.z;
      words[4 * i + 3] = v.w;
    }
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = max(amax, max(words[i] & 0x7fffu, (words[i] >> 16) & 0x7fffu));
    if (amax >= 0x7f80u && flag) atomicOr(flag, 1);   // inf or NaN
    int byte = 0;
    if (amax != 0) {
      const int ef = (int)(amax >> 7);
      const int lg = ef ? ef - 127 : (31 - __clz((int)(amax & 0x7fu))) - 133;   // floor(log2 amax)
      byte = min(254, max(0, lg - 2 + 127));
    }
    float thr[7];
#pragma unroll
    for (int t = 0; t < 7; ++t) thr[t] = ldexpf(mids[t], byte - 127);
    uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t bits = (words[i >> 1] >> (16 * (i & 1))) & 0xffffu;
      const float a = bf16_to_f32(bits & 0x7fffu);
      uint32_t c = 0;
      if (amax != 0) {
#pragma unroll
        for (int t = 0; t < 7; ++t) c += ((t & 1) ? (a >= thr[t]) : (a > thr[t])) ? 1u : 0u;
      }
      c |= (bits >> 15) << 3;
      out[i >> 3] |= c << (4 * (i & 7));
    }
    codes[b] = make_uint4(out[0], out[1], out[2], out[3]);
    scales[b] = (uint8_t)byte;
  }
}

__global__ __launch_bounds__(256) void mx_max_byte(const uint8_t* __restrict__ s, int64_t count,
                                                   uint32_t* __restrict__ slot) {
  uint32_t m = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * blockDim.x)
    m = max(m, (uint32_t)s[i]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if ((threadIdx.x & 63) == 0 && m) atomicMax(slot, m);
}

// One thread per 16-element block: E4M3 power of two of its 32-block scale.
__global__ __launch_bounds__(256) void mx_to_nv(const uint8_t* __restrict__ codes,
                                                const uint8_t* __restrict__ s8, int64_t n16,
                                                const uint32_t* __restrict__ slot,
                                                uint8_t* __restrict__ s4,
                                                int32_t* __restrict__ flag) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= n16) return;
  const int rel = (int)s8[b >> 1] - (int)*slot + 8;          // e - E_max + 8 <= 8
  uint32_t code;
  if (rel >= -6) {
    code = (uint32_t)(rel + 7) << 3;
  } else if (rel >= -9) {
    code = 1u << (rel + 9);
  } else {
    code = 0;
    const uint2 cv = *reinterpret_cast<const uint2*>(codes + 8 * b);
    if (((cv.x | cv.y) & 0x77777777u) && flag) atomicOr(flag, 1);   // nonzero code lost
  }
  s4[b] = (uint8_t)code;
}

__global__ void mx_scale(uint32_t* slot) {
  // S = 2^(E_max - 8), E_max = max byte - 127; exact in fp32 (>= 2^-135)
  const int e = (int)*slot - 127 - 8;
  *reinterpret_cast<float*>(slot) = ldexpf(1.0f, e);
}

// Non-power-of-two check of NVFP4 block scales (E4M3 bytes), 16 per thread:
// a byte is zero or a power of two when its mantissa is 0 (normal) or a
// single set bit with exponent field 0 (subnormal m 2^-9, m = 1, 2 or 4),
// and its sign is clear; NaN (0x7f) is neither.
__global__ __launch_bounds__(256) void pow2_check(const uint8_t* __restrict__ scales,
                                                  int64_t nbytes, int32_t* __restrict__ flag) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  bool bad = false;
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 16; i < nbytes;
       i += 16 * stride) {
    const int64_t cnt = min<int64_t>(16, nbytes - i);
    for (int64_t j = 0; j < cnt; ++j) {
      const uint32_t b = scales[i + j];
      const uint32_t e = (b >> 3) & 0xfu, m = b & 7u;
      const bool ok = !(b & 0x80u) && b != 0x7fu && (e ? m == 0u : (m & (m - 1u)) == 0u);
      bad = bad || !ok;
    }
  }
  if (bad) atomicOr(flag, 1);
}

}  // namespace

hipError_t launch_quantize_mxfp4(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                                 uint8_t* scales, int32_t* flag, hipStream_t stream) {
  const int64_t nblocks = n * k / 32;
  if (flag) hipLaunchKernelGGL(mx_flag_reset, dim3(1), dim3(1), 0, stream, flag);
  const int64_t g = std::min<int64_t>((nblocks + 255) / 256, 8 * (int64_t)device_cu_count());
  hipLaunchKernelGGL(mx_encode, dim3((unsigned)g), dim3(256), 0, stream,
                     reinterpret_cast<const uint4*>(w), nblocks, reinterpret_cast<uint4*>(codes),
                     scales, flag);
  return hipGetLastError();
}

hipError_t launch_mxfp4_to_nvfp4(const uint8_t* codes, const uint8_t* s8, int64_t n, int64_t k,
                                 uint8_t* s4, float* gscale, int32_t* flag, hipStream_t stream) {
  uint32_t* slot = reinterpret_cast<uint32_t*>(gscale);
  hipLaunchKernelGGL(mx_reset, dim3(1), dim3(1), 0, stream, slot, flag);
  const int64_t n32 = n * k / 32, n16 = n * k / 16;
  const int64_t g = std::min<int64_t>((n32 + 255) / 256, 4 * (int64_t)device_cu_count());
  hipLaunchKernelGGL(mx_max_byte, dim3((unsigned)g), dim3(256), 0, stream, s8, n32, slot);
  hipLaunchKernelGGL(mx_to_nv, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, stream, codes,
                     s8, n16, (const uint32_t*)slot, s4, flag);
  hipLaunchKernelGGL(mx_scale, dim3(1), dim3(1), 0, stream, slot);
  return hipGetLastError();
}

hipError_t launch_check_pow2_scales(const uint8_t* scales, int64_t n, int64_t k, int32_t* flag,
                                   hipStream_t stream) {
  const int64_t nbytes = n * (k / 16);
  hipLaunchKernelGGL(mx_flag_reset, dim3(1), dim3(1), 0, stream, flag);
  const int64_t grid =
      std::max<int64_t>(1, std::min<int64_t>((nbytes + 16 * 256 - 1) / (16 * 256),
                                             (int64_t)device_cu_count() * 4));
  hipLaunchKernelGGL(pow2_check, dim3((unsigned)grid), dim3(256), 0, stream, scales, nbytes, flag);
  return hipGetLastError();
}

}  // namespace qerl
