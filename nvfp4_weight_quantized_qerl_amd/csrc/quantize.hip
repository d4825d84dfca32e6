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
// Three stream-ordered kernels per tensor:
//   reset    gscale slot <- 0x80000000 (the slot doubles as the amax
//            accumulator; the top bit marks "still an amax")
//   amax     max over |w| as integers (bf16 bits & 0x7fff; for
//            non-negative floats integer order is value order), one global
//            atomic max per workgroup of 0x80000000 | (fp32 bits of the max)
//   encode   every workgroup forms the non-finite flag and S = RN_fp32(amax
//            / 2688) from the slot (or takes S from it if another workgroup
//            has already stored S there: S never has the top bit set), and
//            workgroup 0 stores S and the flag; then one thread per
//            16-element block (blocks are contiguous in memory because
//            k % 16 == 0), two blocks per iteration, grid-stride; each
//            workgroup first tabulates the element keys of all 126 nonzero
//            block-scale codes (they depend only on the code and S)
// A batch of tensors runs in count + 2 launches: the reset of the first two
// slots, the amax pass of the first tensor, then per tensor one launch with
// its encode pass beside the amax pass of the next (qz_pipe).
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

constexpr uint32_t kAmaxMark = 0x80000000u;

// Both passes run workgroups of kThreads; the amax pass uses at most one
// workgroup per CU: its per-workgroup atomics on the one slot are
// serialised where the slot lives, so there are few of them.
constexpr int kThreads = 512;

__global__ void qz_reset(uint32_t* a, uint32_t* b) {
  *a = kAmaxMark;
  if (b) *b = kAmaxMark;
}

// The amax pass over nvec 16-byte vectors, as workgroup wg of nwg.
__device__ __forceinline__ void amax_body(const uint4* __restrict__ w, int64_t nvec,
                                          uint32_t* __restrict__ slot, int64_t wg, int64_t nwg) {
  uint32_t m = 0;
  auto fold = [&](const uint4& v) {
    const uint32_t a = max(v.x & 0x7fffu, (v.x >> 16) & 0x7fffu);
    const uint32_t b = max(v.y & 0x7fffu, (v.y >> 16) & 0x7fffu);
    const uint32_t c = max(v.z & 0x7fffu, (v.z >> 16) & 0x7fffu);
    const uint32_t d = max(v.w & 0x7fffu, (v.w >> 16) & 0x7fffu);
    m = max(m, max(max(a, b), max(c, d)));
  };
  // Eight independent 16-byte loads per thread in flight per iteration.
  const int64_t stride = nwg * kThreads;
  int64_t i = wg * kThreads + threadIdx.x;
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
  __shared__ uint32_t red[kThreads / 64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) red[wid] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
#pragma unroll
    for (int u = 0; u < kThreads / 64; ++u) r = max(r, red[u]);
    if (r) atomicMax(slot, kAmaxMark | (r << 16));   // fp32 bits of the bf16 magnitude
  }
}

__global__ __launch_bounds__(kThreads) void qz_amax(const uint4* __restrict__ w, int64_t nvec,
                                                    uint32_t* __restrict__ slot) {
  amax_body(w, nvec, slot, blockIdx.x, gridDim.x);
}

// S and the non-finite flag from the slot: the marked amax (S is formed
// here), or S itself, stored by a workgroup that got there first.
__device__ __forceinline__ float scale_from_slot(uint32_t bits, bool* nonfinite) {
  if (!(bits & kAmaxMark)) {
    const float S = __uint_as_float(bits);
    *nonfinite = S != S;
    return S;
  }
  bits &= ~kAmaxMark;
  *nonfinite = bits >= 0x7f800000u;
  if (*nonfinite) return __uint_as_float(0x7fc00000u);
  // amax / 2688 in fp64, then to fp32: the exact quotient is amax/21 times a
  // power of two, never an fp32 midpoint nor within fp64 rounding of one,
  // so this is the correctly rounded fp32 quotient.
  return (float)((double)__uint_as_float(bits) / 2688.0);
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

typedef int16_t i16x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// One 16-element block: E4M3 block-scale code and the 16 packed E2M1 codes.
// The element codes are counted two at a time in 16-bit halves: a bf16 word
// pair masked with 0x7fff7fff holds the two magnitudes, and key - |w| (both
// in [-1, 0x7fff]) is negative exactly when |w| > key.
__device__ __forceinline__ uint32_t encode_block(const uint4& lo, const uint4& hi, float S,
                                                 const int16_t (*key_tab)[8], uint2* out) {
  const uint32_t words[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  uint32_t amax_b = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    amax_b = max(amax_b, max(words[i] & 0x7fffu, (words[i] >> 16) & 0x7fffu));
  uint32_t scode = 0;
  if (S > 0.0f && amax_b != 0) {
    const double q = (double)bf16_to_f32(amax_b) / (6.0 * (double)S);
    scode = e4m3_rne_code(q);
  }
  i16x2 key[7];
#pragma unroll
  for (int t = 0; t < 7; ++t) {
    const int16_t kt = scode ? key_tab[scode][t] : (int16_t)0x7fff;
    key[t] = i16x2{kt, kt};
  }
  uint32_t packed[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t mw = words[i] & 0x7fff7fffu;
    const i16x2 a = __builtin_bit_cast(i16x2, mw);
    u16x2 cnt = u16x2{0, 0};
#pragma unroll
    for (int t = 0; t < 7; ++t) cnt += __builtin_bit_cast(u16x2, key[t] - a) >> (uint16_t)15;
    // the two codes (0..7) with their sign bits (bf16 bit 15 -> code bit 3)
    const uint32_t c2 = __builtin_bit_cast(uint32_t, cnt) | ((words[i] >> 12) & 0x00080008u);
    packed[i >> 2] |= ((c2 & 0xfu) | ((c2 >> 12) & 0xf0u)) << (8 * (i & 3));
  }
  *out = make_uint2(packed[0], packed[1]);
  return scode;
}

struct EncodeJob {
  const uint4* w;
  int64_t nblocks;
  uint32_t* slot;   // the amax slot, S on return
  int32_t* flag;    // nullable
  uint2* codes;
  uint8_t* scales;
};

// The encode pass as workgroup wg of nwg: S and the flag from the slot
// (workgroup 0 stores them), the key table, then a grid-stride over the
// 16-element blocks, two per thread per iteration (their four loads issued
// together); blocks are contiguous in memory because k % 16 == 0.
__device__ __forceinline__ void encode_body(const EncodeJob& j, int64_t wg, int64_t nwg,
                                            int16_t (*key_tab)[8]) {
  bool nonfinite = false;
  const float S = scale_from_slot(*j.slot, &nonfinite);
  build_keys(key_tab, (double)S);
  __syncthreads();
  if (wg == 0 && threadIdx.x == 0) {
    *reinterpret_cast<float*>(j.slot) = S;
    if (j.flag) *j.flag = nonfinite ? 1 : 0;
  }
  const int64_t stride = nwg * kThreads;
  int64_t b = wg * kThreads + threadIdx.x;
  for (; b + stride < j.nblocks; b += 2 * stride) {
    const uint4 lo0 = j.w[2 * b], hi0 = j.w[2 * b + 1];
    const uint4 lo1 = j.w[2 * (b + stride)], hi1 = j.w[2 * (b + stride) + 1];
    uint2 c0, c1;
    const uint32_t s0 = encode_block(lo0, hi0, S, key_tab, &c0);
    const uint32_t s1 = encode_block(lo1, hi1, S, key_tab, &c1);
    j.codes[b] = c0;
    j.scales[b] = (uint8_t)s0;
    j.codes[b + stride] = c1;
    j.scales[b + stride] = (uint8_t)s1;
  }
  if (b < j.nblocks) {
    uint2 c0;
    const uint32_t s0 = encode_block(j.w[2 * b], j.w[2 * b + 1], S, key_tab, &c0);
    j.codes[b] = c0;
    j.scales[b] = (uint8_t)s0;
  }
}

__global__ __launch_bounds__(kThreads) void qz_encode(EncodeJob j) {
  __shared__ int16_t key_tab[kCodes][8];
  encode_body(j, blockIdx.x, gridDim.x, key_tab);
}

// One launch of the batched quantizer: the encode pass of tensor i on
// ewgs workgroups, the amax pass of tensor i + 1 on awgs workgroups (0 for
// the last tensor), spread evenly through the grid so that the two run side
// by side, and the reset of the slot of tensor i + 2 (nullable).  Tensor i
// was read by its amax pass in the launch before, so its second read
// mostly hits the last-level cache.
__global__ __launch_bounds__(kThreads) void qz_pipe(EncodeJob e, int64_t ewgs, const uint4* aw,
                                                    int64_t anvec, uint32_t* aslot, int64_t awgs,
                                                    uint32_t* reset) {
  __shared__ int16_t key_tab[kCodes][8];
  if (reset && blockIdx.x == 0 && threadIdx.x == 0) *reset = kAmaxMark;
  const int64_t G = ewgs + awgs, b = blockIdx.x;
  const int64_t na0 = b * awgs / G, na1 = (b + 1) * awgs / G;   // amax workgroups before b, b + 1
  if (na1 > na0) amax_body(aw, anvec, aslot, na0, awgs);
  else encode_body(e, b - na0, ewgs, key_tab);
}

int64_t amax_wgs(int64_t nvec) {
  return std::max<int64_t>(1, std::min<int64_t>((nvec + kThreads - 1) / kThreads,
                                                (int64_t)device_cu_count()));
}

// Enough encode workgroups to fill the chip a few times over; each builds
// its key table once and then loops over its blocks.
int64_t encode_wgs(int64_t nblocks) {
  return std::max<int64_t>(1, std::min<int64_t>((nblocks + kThreads - 1) / kThreads,
                                                (int64_t)device_cu_count() * 4));
}

EncodeJob encode_job(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes, uint8_t* scales,
                     float* gscale, int32_t* flag) {
  EncodeJob j;
  j.w = reinterpret_cast<const uint4*>(w);
  j.nblocks = n * k / 16;
  j.slot = reinterpret_cast<uint32_t*>(gscale);
  j.flag = flag;
  j.codes = reinterpret_cast<uint2*>(codes);
  j.scales = scales;
  return j;
}

}  // namespace

hipError_t launch_quantize(const uint16_t* w, int64_t n, int64_t k,
                           uint8_t* codes, uint8_t* scales, float* gscale,
                           int32_t* flag, hipStream_t stream) {
  uint32_t* slot = reinterpret_cast<uint32_t*>(gscale);
  const int64_t nvec = n * k / 8;
  hipLaunchKernelGGL(qz_reset, dim3(1), dim3(1), 0, stream, slot, nullptr);
  hipLaunchKernelGGL(qz_amax, dim3((unsigned)amax_wgs(nvec)), dim3(kThreads), 0, stream,
                     reinterpret_cast<const uint4*>(w), nvec, slot);
  const EncodeJob j = encode_job(w, n, k, codes, scales, gscale, flag);
  hipLaunchKernelGGL(qz_encode, dim3((unsigned)encode_wgs(j.nblocks)), dim3(kThreads), 0, stream,
                     j);
  return hipGetLastError();
}

hipError_t launch_quantize_batch(int count, const uint16_t* const* w, const int64_t* n,
                                 const int64_t* k, uint8_t* const* codes, uint8_t* const* scales,
                                 float* const* gscale, int32_t* const* flag, hipStream_t stream) {
  auto slot = [&](int i) { return reinterpret_cast<uint32_t*>(gscale[i]); };
  auto nvec = [&](int i) { return n[i] * k[i] / 8; };
  hipLaunchKernelGGL(qz_reset, dim3(1), dim3(1), 0, stream, slot(0),
                     count > 1 ? slot(1) : nullptr);
  hipLaunchKernelGGL(qz_amax, dim3((unsigned)amax_wgs(nvec(0))), dim3(kThreads), 0, stream,
                     reinterpret_cast<const uint4*>(w[0]), nvec(0), slot(0));
  for (int i = 0; i < count; ++i) {
    const EncodeJob e = encode_job(w[i], n[i], k[i], codes[i], scales[i], gscale[i],
                                   flag ? flag[i] : nullptr);
    const int64_t ewgs = encode_wgs(e.nblocks);
    const bool next = i + 1 < count;
    const int64_t awgs = next ? amax_wgs(nvec(i + 1)) : 0;
    hipLaunchKernelGGL(qz_pipe, dim3((unsigned)(ewgs + awgs)), dim3(kThreads), 0, stream, e, ewgs,
                       next ? reinterpret_cast<const uint4*>(w[i + 1]) : nullptr,
                       next ? nvec(i + 1) : 0, next ? slot(i + 1) : nullptr, awgs,
                       i + 2 < count ? slot(i + 2) : nullptr);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace qerl
