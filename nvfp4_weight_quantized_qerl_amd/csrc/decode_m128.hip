// Instantiations of the single-pass 128-token decode contraction.
#include "decode_m128.h"

namespace qerl {
namespace d128 {

Kernel pick(bool p2, bool tiled) {
  if (tiled) return p2 ? decode_m128<true, true> : decode_m128<false, true>;
  return p2 ? decode_m128<true, false> : decode_m128<false, false>;
}

namespace {

// One thread per 16-byte code slot of a tile (2048 B of codes = 128 slots)
// and its 2-byte scale slot.
__global__ __launch_bounds__(256) void tile128_kernel(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales,
                                                      int64_t n, int64_t k, int64_t nblocks,
                                                      int64_t ntiles, uint8_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= ntiles * 128) return;
  const int64_t tile = i >> 7;
  const int slot = (int)(i & 127);
  const int64_t st = tile / nblocks, b = tile - st * nblocks;
  const int c = slot & 31, hk = slot >> 5;          // hk = 2 kh + h
  const int64_t row = 32 * st + c;
  uint4 cv = make_uint4(0u, 0u, 0u, 0u);
  uint32_t sv = 0u;
  if (row < n) {
    const int64_t kb = 64 * b + 16 * hk;            // code byte of the slot's 32 channels
    cv = *reinterpret_cast<const uint4*>(codes + row * (k / 2) + kb);
    const uint8_t* sp = scales + row * (k / 16) + 8 * b + 2 * hk;
    sv = (uint32_t)sp[0] | ((uint32_t)sp[1] << 8);
  }
  uint8_t* t = out + tile * kTileBytes;
  *reinterpret_cast<uint4*>(t + 16 * slot) = cv;
  t[2048 + 2 * slot] = (uint8_t)(sv & 0xffu);
  t[2048 + 2 * slot + 1] = (uint8_t)(sv >> 8);
}

}  // namespace

size_t tile128_bytes(int64_t n, int64_t k) {
  return (size_t)((n + 31) / 32) * (size_t)(k / kBlock) * kTileBytes;
}

hipError_t launch_tile128(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k,
                          uint8_t* out, hipStream_t stream) {
  const int64_t nblocks = k / kBlock, ntiles = (n + 31) / 32 * nblocks;
  const int64_t threads = ntiles * 128;
  hipLaunchKernelGGL(tile128_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                     codes, scales, n, k, nblocks, ntiles, out);
  return hipGetLastError();
}

}  // namespace d128
}  // namespace qerl
