// NVFP4 quantizer: bf16 W[n, k] -> E2M1 codes, E4M3 block scales, FP32 S.
//
// The pages define NVFP4 by its dequantization W_hat = S_FP32 * (S_E4M3 (.)
// W_tilde) with one E4M3 scale per 16 contiguous elements [QeRL summary,
// §3.4, Eq. 6].  The quantizer is read from Eq. 1's "scale = range / q_max"
// at both levels, q_max = 6 for E2M1 [§3.4] and 448 for E4M3:
//   S    = RN_fp32(amax / 2688)
//   s_b  = RNE_E4M3(amax_b / (6 S)), saturating at 448
//   code = sign | RNE_E2M1(|w| / (s_b S)), saturating at 6, ties to even
// with the quotients taken exactly, so the encoding is unique.
//
// Four stream-ordered kernels:
//   reset    gscale slot <- 0 (it doubles as the amax accumulator)
//   amax     max over |w| as integers (bf16 bits & 0x7fff; for
//            non-negative floats integer order is value order) combined
//            with a global atomic max of the fp32 bit pattern
//   scale    one thread: non-finite flag, S = RN_fp32(amax / 2688)
//   encode   one thread per 16-element block (blocks are contiguous in
//            memory because k % 16 == 0), grid-stride; each workgroup
//            first tabulates the element keys of all 126 nonzero block-scale
//            codes (they depend only on the code and S)
//
// Exactness of `encode` (no rounding can change a decision):
//  * q = amax_b / (6 S) in fp64.  amax_b has 8 significant bits and 6 S at
//    most 26, so a quotient that is not exactly an E4M3 midpoint differs
//    from it by more than 2^-31 relative, far above fp64's 2^-53; an exact
//    midpoint is computed exactly.  Rounding q to E4M3 then uses rint
//    (round half to even) on the scaled mantissa.
//  * Element thresholds t * s_b * S (t = the E2M1 midpoints 0.25 ... 5)
//    have at most 31 significant bits: exact in fp64.  Comparing a bf16
//    |w| against a real threshold thr is the same as comparing its bit
//    pattern against the bits of RD_bf16(thr) (strictly greater), except
//    that "|w| >= thr" for a thr that is itself a bf16 needs the key one
//    lower.  A tie at the midpoint between codes i and i+1 goes to the
//    even one of the two, so the crossing test is "> thr" for even i and
//    ">= thr" for odd i.
#include <algorithm>

#include "qerl_device.h"
#include "qerl_internal.h"

namespace qerl {
namespace {

__global__ void qz_reset(uint32_t* slot) { *slot = 0u; }

__global__ __launch_bounds__(256) void qz_amax(const uint4* __restrict__ w,
                                               int64_t nvec,
                                               uint32_t* __restrict__ slot) {
  uint32_t m = 0;
  auto fold = [&](const uint4& v) {
    const uint32_t a = max(v.x & 0x7fffu, (v.x >> 16) & 0x7fffu);
    const uint32_t b = max(v.y & 0x7fffu, (v.y >> 16) & 0x7fffu);
    const uint32_t c = max(v.z & 0x7fffu, (v.z >> 16) & 0x7fffu);
    const uint32_t d = max(v.w & 0x7fffu, (v.w >> 16) & 0x7fffu);
    m = max(m, max(max(a, b), max(c, d)));
  };
  // Eight independent 16-byte loads per thread in flight per iteration.
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 7 * stride < nvec; i += 8 * stride) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = w[i + u * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) fold(v[u]);
  }
  for (; i < nvec; i += stride) fold(w[i]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  __shared__ uint32_t red[4];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) red[wid] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = max(max(red[0], red[1]), max(red[2], red[3]));
    if (r) atomicMax(slot, r << 16);   // fp32 bits of the bf16 magnitude
  }
}

__global__ void qz_scale(uint32_t* slot, int32_t* flag) {
  const uint32_t bits = *slot;
  const bool nonfinite = bits >= 0x7f800000u;
  if (flag) *flag = nonfinite ? 1 : 0;
  float S;
  if (nonfinite) {
    S = __uint_as_float(0x7fc00000u);
  } else {
    // amax / 2688 in fp64, then to fp32: the exact quotient is amax/21
    // times a power of two, never an fp32 midpoint nor within fp64
    // rounding of one, so this is the correctly rounded fp32 quotient.
    S = (float)((double)__uint_as_float(bits) / 2688.0);
  }
  *reinterpret_cast<float*>(slot) = S;
}

// Round q > 0 to OCP E4M3 (nearest, ties to even), saturating at 448.
__device__ __forceinline__ uint32_t e4m3_rne_code(double q) {
  if (q >= 448.0) return 0x7eu;
  if (q < 0x1p-6) return (uint32_t)rint(q * 512.0);   // subnormal m * 2^-9
  int e;
  double fr = frexp(q, &e);          // q = fr * 2^e, fr in [0.5, 1)
  double r = rint(fr * 16.0);        // (1 + f) * 8 in [8, 16]
  int E = e - 1;
  if (r == 16.0) { r = 8.0; E += 1; }
  uint32_t code = ((uint32_t)(E + 7) << 3) | ((uint32_t)r - 8u);
  return code > 0x7eu ? 0x7eu : code;
}

// bf16 key g such that (|w| bits > g) == (|w| > thr) if !ge, (|w| >= thr)
// if ge.  thr > 0 is exact in fp64.
__device__ __forceinline__ int32_t bf16_key(double thr, bool ge) {
  float f = __double2float_rz(thr);
  uint32_t kb = __float_as_uint(f) >> 16;            // RD to bf16
  bool exact = (double)__uint_as_float(kb << 16) == thr;
  return (int32_t)kb - ((ge && exact) ? 1 : 0);
}

// Element keys of every block-scale code, once per workgroup: key_tab[c][t]
// for E4M3 codes c = 1..126 and E2M1 midpoints t (code 0 never reads them).
// The keys depend only on c and S, so the fp64 work is done 127 times per
// workgroup instead of once per block.
constexpr int kCodes = 127;

__device__ __forceinline__ void build_keys(int16_t (*key_tab)[8], double S) {
  constexpr double mids[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
  for (int i = threadIdx.x; i < kCodes * 7; i += blockDim.x) {
    const int c = i / 7, t = i - 7 * (i / 7);
    if (c == 0) continue;
    const double unit = (double)e4m3_to_f32((uint32_t)c) * S;   // exact
    key_tab[c][t] = (int16_t)bf16_key(mids[t] * unit, (t & 1) != 0);
  }
}

// Grid-stride over 16-element blocks; each thread encodes one block per
// iteration (blocks are contiguous in memory because k % 16 == 0).
__global__ __launch_bounds__(256) void qz_encode(const uint4* __restrict__ w,
                                                 int64_t nblocks,
                                                 const float* __restrict__ gscale,
                                                 uint2* __restrict__ codes,
                                                 uint8_t* __restrict__ scales) {
  __shared__ int16_t key_tab[kCodes][8];
  const float S = *gscale;
  build_keys(key_tab, (double)S);
  __syncthreads();
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblocks; b += stride) {
    const uint4 lo = w[2 * b], hi = w[2 * b + 1];
    const uint32_t words[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    uint32_t mag[16];
    uint32_t amax_b = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      mag[2 * i] = words[i] & 0x7fffu;
      mag[2 * i + 1] = (words[i] >> 16) & 0x7fffu;
      amax_b = max(amax_b, max(mag[2 * i], mag[2 * i + 1]));
    }
    uint32_t scode = 0;
    if (S > 0.0f && amax_b != 0) {
      const double q = (double)bf16_to_f32(amax_b) / (6.0 * (double)S);
      scode = e4m3_rne_code(q);
    }
    int32_t key[7];
#pragma unroll
    for (int t = 0; t < 7; ++t) key[t] = scode ? (int32_t)key_tab[scode][t] : 0x7fff;
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int32_t a = (int32_t)mag[i];
      uint32_t c = 0;
#pragma unroll
      for (int t = 0; t < 7; ++t) c += (a > key[t]) ? 1u : 0u;
      const uint32_t sign = (words[i >> 1] >> ((i & 1) ? 31 : 15)) & 1u;
      c |= sign << 3;
      packed[i >> 3] |= c << (4 * (i & 7));
    }
    codes[b] = make_uint2(packed[0], packed[1]);
    scales[b] = (uint8_t)scode;
  }
}

}  // namespace

hipError_t launch_quantize(const uint16_t* w, int64_t n, int64_t k,
                           uint8_t* codes, uint8_t* scales, float* gscale,
                           int32_t* flag, hipStream_t stream) {
  uint32_t* slot = reinterpret_cast<uint32_t*>(gscale);
  const int64_t nvec = n * k / 8;
  const int64_t nblocks = n * k / 16;
  hipLaunchKernelGGL(qz_reset, dim3(1), dim3(1), 0, stream, slot);
  int64_t grid = (nvec + 255) / 256;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(qz_amax, dim3((unsigned)grid), dim3(256), 0, stream,
                     reinterpret_cast<const uint4*>(w), nvec, slot);
  hipLaunchKernelGGL(qz_scale, dim3(1), dim3(1), 0, stream, slot, flag);
  // Enough workgroups to fill the chip a few times over; each builds its
  // key table once and then loops over its blocks.
  const int64_t eg = std::min<int64_t>((nblocks + 255) / 256, (int64_t)device_cu_count() * 8);
  hipLaunchKernelGGL(qz_encode, dim3((unsigned)eg), dim3(256), 0, stream,
                     reinterpret_cast<const uint4*>(w), nblocks,
                     (const float*)gscale, reinterpret_cast<uint2*>(codes),
                     scales);
  return hipGetLastError();
}

}  // namespace qerl
