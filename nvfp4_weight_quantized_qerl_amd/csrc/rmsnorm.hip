// Noisy RMSNorm, the producer of a linear layer's noisy input
// [QeRL summary, §3.4 "Noise Merging", Eq. 10]:
//     y[m, i] = bf16( (w_i + z_i) * (x[m, i] * rsqrt(mean_j x[m, j]^2 + delta)) )
// The AQN noise vector z is added to the RMSNorm scale w; the
// normalisation is unchanged.  One z serves every row of the call.
//
// One wave per token row; the rows are spread over the waves of the
// launch.  Lane l holds the 16-byte chunks (8 channels each) l, l + 64,
// ... of the row.  For rows of up to 64 * kNch chunks (kNch <= 10 per lane)
// a wave first forms w + z of its lanes' channels in fp32 (once: they are
// the same for every row), then per row issues all of the row's loads,
// sums the squares across the wave with lane exchanges in a fixed order and
// scales the row from registers.  Longer rows go in groups of 64 * kNch
// chunks and are read a second time for the scaling.  HBM-bound: 4 bytes
// per element of x and y, plus w and z once per call.
#include "qerl_device.h"
#include "qerl_internal.h"

namespace qerl {
namespace {


struct NormArgs {
  const uint16_t* x;      // may be y itself: a lane reads each chunk before it writes it
  const uint16_t* __restrict__ w;
  const float* __restrict__ z;
  uint16_t* y;
  int64_t m, d;
  float delta;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ float sumsq8(u32x4 v) {
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float lo = bf16_to_f32(v[e] & 0xffffu), hi = bf16_to_f32(v[e] >> 16);
    s += lo * lo;
    s += hi * hi;
  }
  return s;
}

// Eight outputs (w + z) * (x * r) of one chunk, packed to bf16.
__device__ __forceinline__ u32x4 scale8(u32x4 xv, u32x4 wv, f32x4 z0, f32x4 z1, float r) {
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float zl = e < 2 ? z0[2 * e] : z1[2 * e - 4];
    const float zh = e < 2 ? z0[2 * e + 1] : z1[2 * e - 3];
    const float lo = (bf16_to_f32(wv[e] & 0xffffu) + zl) * (bf16_to_f32(xv[e] & 0xffffu) * r);
    const float hi = (bf16_to_f32(wv[e] >> 16) + zh) * (bf16_to_f32(xv[e] >> 16) * r);
    o[e] = pack_bf16x2(lo, hi);
  }
  return o;
}

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ f32x4 ldf4(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}

// kNch: 16-byte chunks per lane held in registers at once (a row of up to
// 512 kNch channels in one group); sized to the row so that the registers,
// and with them the waves resident per CU, follow the row length.
template <int kNch>
__global__ __launch_bounds__(256) void rmsnorm_kernel(NormArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  const int64_t nch = a.d / 8;
  const int64_t row_first = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (nch <= 64 * kNch) {
    // w + z of this lane's channels, the same for every row of the call.
    float wz[kNch][8];
#pragma unroll
    for (int i = 0; i < kNch; ++i) {
      const int64_t c = lane + 64 * i;
      u32x4 wv = 0u;
      f32x4 z0 = 0.0f, z1 = 0.0f;
      if (c < nch) {
        wv = ld16(a.w + 8 * c);
        if (a.z) {
          z0 = ldf4(a.z + 8 * c);
          z1 = ldf4(a.z + 8 * c + 4);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        wz[i][2 * e] = bf16_to_f32(wv[e] & 0xffffu) + (e < 2 ? z0[2 * e] : z1[2 * e - 4]);
        wz[i][2 * e + 1] = bf16_to_f32(wv[e] >> 16) + (e < 2 ? z0[2 * e + 1] : z1[2 * e - 3]);
      }
    }
    // x of the wave's next row is loaded while the current one is scaled.
    u32x4 xn[kNch];
    auto load_row = [&](int64_t row) {
#pragma unroll
      for (int i = 0; i < kNch; ++i) {
        xn[i] = 0u;
        const int64_t c = lane + 64 * i;
        if (row < a.m && c < nch) xn[i] = ld16(a.x + row * a.d + 8 * c);
      }
    };
    load_row(row_first);
    for (int64_t row = row_first; row < a.m; row += nwaves) {
      uint16_t* yr = a.y + row * a.d;
      u32x4 xv[kNch];
#pragma unroll
      for (int i = 0; i < kNch; ++i) xv[i] = xn[i];
      load_row(row + nwaves);
      float ss = 0.0f;
#pragma unroll
      for (int i = 0; i < kNch; ++i) ss += sumsq8(xv[i]);
      ss = wave_sum(ss);
      const float r = 1.0f / sqrtf(ss / (float)a.d + a.delta);
#pragma unroll
      for (int i = 0; i < kNch; ++i) {
        const int64_t c = lane + 64 * i;
        if (c < nch) {
          u32x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            o[e] = pack_bf16x2(wz[i][2 * e] * (bf16_to_f32(xv[i][e] & 0xffffu) * r),
                               wz[i][2 * e + 1] * (bf16_to_f32(xv[i][e] >> 16) * r));
          *reinterpret_cast<u32x4*>(yr + 8 * c) = o;
        }
      }
    }
    return;
  }
  // Rows longer than 512 kNch channels: sum of squares over groups of
  // 64 kNch chunks, then a second pass that re-reads the row.
  for (int64_t row = row_first; row < a.m; row += nwaves) {
    const uint16_t* xr = a.x + row * a.d;
    uint16_t* yr = a.y + row * a.d;
    float ss = 0.0f;
    for (int64_t c0 = 0; c0 < nch; c0 += 64 * kNch) {
      u32x4 xv[kNch];
#pragma unroll
      for (int i = 0; i < kNch; ++i) {
        xv[i] = 0u;
        const int64_t c = c0 + lane + 64 * i;
        if (c < nch) xv[i] = ld16(xr + 8 * c);
      }
#pragma unroll
      for (int i = 0; i < kNch; ++i) ss += sumsq8(xv[i]);
    }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)a.d + a.delta);
    for (int64_t c0 = 0; c0 < nch; c0 += 64 * kNch) {
#pragma unroll
      for (int i = 0; i < kNch; ++i) {
        const int64_t c = c0 + lane + 64 * i;
        if (c < nch) {
          f32x4 z0 = 0.0f, z1 = 0.0f;
          if (a.z) {
            z0 = ldf4(a.z + 8 * c);
            z1 = ldf4(a.z + 8 * c + 4);
          }
          *reinterpret_cast<u32x4*>(yr + 8 * c) =
              scale8(ld16(xr + 8 * c), ld16(a.w + 8 * c), z0, z1, r);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_rmsnorm_noisy(const uint16_t* x, int64_t m, int64_t d, const uint16_t* w,
                                const float* z, float delta, uint16_t* y, hipStream_t stream) {
  NormArgs a;
  a.x = x;
  a.w = w;
  a.z = z;
  a.y = y;
  a.m = m;
  a.d = d;
  a.delta = delta;
  // Four rows per workgroup and two workgroups per CU; each wave loops over
  // its rows with the next row's loads in flight.
  const int64_t groups = std::min<int64_t>((m + 3) / 4, 2 * (int64_t)device_cu_count());
  const int64_t per_lane = (d / 8 + 63) / 64;
  const dim3 grid((unsigned)groups), block(256);
  if (per_lane <= 2)
    hipLaunchKernelGGL(rmsnorm_kernel<2>, grid, block, 0, stream, a);
  else if (per_lane <= 4)
    hipLaunchKernelGGL(rmsnorm_kernel<4>, grid, block, 0, stream, a);
  else if (per_lane <= 7)
    hipLaunchKernelGGL(rmsnorm_kernel<7>, grid, block, 0, stream, a);
  else if (per_lane <= 8)
    hipLaunchKernelGGL(rmsnorm_kernel<8>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<10>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace qerl
