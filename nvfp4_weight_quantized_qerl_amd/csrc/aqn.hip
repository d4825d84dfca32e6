// AQN noise vector z ~ N(0, sigma^2 I) of length d [QeRL summary, §3.4,
// Eq. 7], resampled per forward pass by changing call_id.
//
// Generator (not on the pages, which ask only for Gaussian noise):
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC'11) with key (seed, stream_id) and counter
// (j / 4, call_id, 0, 0); each 4-word output feeds two Box-Muller pairs
// (Box and Muller, 1958), all in fp64; z_j = RN_fp32(sigma * n_j).
// One thread per counter value; no state, so any slice of z can be
// recomputed independently.
//
// Several vectors in one launch: vector v (blockIdx.y) takes call id
// call0 + v * call_step and counter word 2 = v * row_step, so the same
// kernel draws a batch of per-call vectors (row_step 0: each is the vector
// qerl_aqn_sample gives for its call id) or one vector per token row of a
// call (call_step 0, row_step 1: row 0 is the shared vector).
#include "qerl_device.h"
#include "qerl_internal.h"

namespace qerl {
namespace {

constexpr uint64_t kM0 = 0xD2E7470EE14C6C93ull;
constexpr uint64_t kM1 = 0xCA5A826395121157ull;
constexpr uint64_t kW0 = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kW1 = 0xBB67AE8584CAA73Bull;

__device__ __forceinline__ void philox4x64_10(uint64_t c[4], uint64_t k0,
                                              uint64_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    if (round) { k0 += kW0; k1 += kW1; }
    const uint64_t lo0 = kM0 * c[0], hi0 = __umul64hi(kM0, c[0]);
    const uint64_t lo1 = kM1 * c[2], hi1 = __umul64hi(kM1, c[2]);
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
  }
}

__device__ __forceinline__ void box_muller(uint64_t ra, uint64_t rb,
                                           double* n0, double* n1) {
  const double u1 = (double)((ra >> 11) + 1) * 0x1p-53;   // (0, 1]
  const double u2 = (double)(rb >> 11) * 0x1p-53;         // [0, 1)
  const double rad = sqrt(-2.0 * log(u1));
  const double ang = 2.0 * M_PI * u2;
  *n0 = rad * cos(ang);
  *n1 = rad * sin(ang);
}

__global__ __launch_bounds__(256) void aqn_sample_kernel(
    uint64_t seed, uint64_t stream_id, uint64_t call0, uint64_t call_step,
    uint64_t row_step, double sigma, int64_t d, float* __restrict__ z) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (4 * q >= d) return;
  const uint64_t v = blockIdx.y;
  z += (int64_t)v * d;
  uint64_t c[4] = {(uint64_t)q, call0 + v * call_step, v * row_step, 0ull};
  philox4x64_10(c, seed, stream_id);
  double n[4];
  box_muller(c[0], c[1], &n[0], &n[1]);
  box_muller(c[2], c[3], &n[2], &n[3]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t j = 4 * q + i;
    if (j < d) z[j] = (float)(sigma * n[i]);
  }
}

}  // namespace

hipError_t launch_aqn_sample(uint64_t seed, uint64_t stream_id, uint64_t call0,
                             uint64_t call_step, uint64_t row_step, int64_t count,
                             double sigma, int64_t d, float* z, hipStream_t stream) {
  const int64_t quads = (d + 3) / 4;
  const int64_t grid = (quads + 255) / 256;
  hipLaunchKernelGGL(aqn_sample_kernel, dim3((unsigned)grid, (unsigned)count), dim3(256), 0,
                     stream, seed, stream_id, call0, call_step, row_step, sigma, d, z);
  return hipGetLastError();
}

}  // namespace qerl
