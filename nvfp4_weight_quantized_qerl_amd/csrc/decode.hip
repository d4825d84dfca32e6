// Decode contraction: launches over the m rows in chunks of at most
// 32 * dec_mt rows.  Per chunk, one contraction kernel -- the LDS-staged
// one (decode_lds.h) where its shape conditions hold, else the general one
// (decode_kernel.h) -- and, when K is split across workgroups, the
// finishing kernel below.
#include <algorithm>

#include "decode_kernel.h"
#include "decode_lds.h"
#include "qerl_internal.h"

namespace qerl {

namespace {

decode::DecodeKernel pick_decode(int mt, int nt) {
  switch (mt) {
    case 1: return decode::pick_mt1(nt);
    case 2: return decode::pick_mt2(nt);
    case 4: return decode::pick_mt4(nt);
    default: return nullptr;
  }
}

struct FinishArgs {
  const float* __restrict__ ypart;      // [split, rows, n] fp32 partial sums of acc
  const float* __restrict__ gscale;
  const uint16_t* __restrict__ t;       // [rows, rpad16] bf16 s x_t A^T of this chunk
  const uint16_t* __restrict__ lora_b;  // [n, r] bf16
  uint16_t* __restrict__ y;             // [m_valid, n] rows of this chunk
  int64_t n;
  int split, rows, m_valid, r, rpad16, lora_vec, vec4;
};

constexpr int kFinishBatch = 16;   // partial sums loaded together per thread

// y[m, j] = bf16(S * sum_s ypart[s, m, j] + sum_i t[m, i] B[j, i]): the
// epilogue of a split-K contraction [QeRL summary, §3.4, Eq. 6 (S) and
// Eq. 2 (LoRA side branch)].  The splits are summed in split order, then
// scaled, then the LoRA term is added in i order.  One thread per token row
// and four consecutive columns; every load of a thread is independent of
// the others, so a thread waits about one memory latency per batch of
// kFinishBatch splits.
__global__ __launch_bounds__(256) void splitk_finish(FinishArgs a) {
  const int64_t groups = (a.n + 3) / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= groups * a.m_valid) return;
  const int m = (int)(idx / groups);
  const int64_t col = (idx - (int64_t)m * groups) * 4;
  const int ncol = (int)min<int64_t>(4, a.n - col);
  const bool vec = a.vec4 && ncol == 4;
  const float* src = a.ypart + (int64_t)m * a.n + col;
  const int64_t sstride = (int64_t)a.rows * a.n;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = 0; s0 < a.split; s0 += kFinishBatch) {
    float4 part[kFinishBatch];
#pragma unroll
    for (int u = 0; u < kFinishBatch; ++u) {
      part[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (s0 + u < a.split) {
        const float* ps = src + (int64_t)(s0 + u) * sstride;
        if (vec) {
          part[u] = *reinterpret_cast<const float4*>(ps);
        } else {
          part[u].x = ps[0];
          if (ncol > 1) part[u].y = ps[1];
          if (ncol > 2) part[u].z = ps[2];
          if (ncol > 3) part[u].w = ps[3];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kFinishBatch; ++u) {
      if (s0 + u < a.split) {
        acc[0] += part[u].x;
        acc[1] += part[u].y;
        acc[2] += part[u].z;
        acc[3] += part[u].w;
      }
    }
  }
  const float S = *a.gscale;
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] *= S;
  if (a.r > 0) {
    const uint16_t* trow = a.t + (int64_t)m * a.rpad16;
#pragma unroll 4
    for (int i0 = 0; i0 < a.r; i0 += 8) {
      // t[m, i0 .. i0+7] (t is padded to rpad16 columns with zeros)
      const uint4 tv = *reinterpret_cast<const uint4*>(trow + i0);
      const float tf[8] = {bf16_to_f32(tv.x & 0xffffu), bf16_to_f32(tv.x >> 16),
                           bf16_to_f32(tv.y & 0xffffu), bf16_to_f32(tv.y >> 16),
                           bf16_to_f32(tv.z & 0xffffu), bf16_to_f32(tv.z >> 16),
                           bf16_to_f32(tv.w & 0xffffu), bf16_to_f32(tv.w >> 16)};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (c >= ncol) break;
        const uint16_t* brow = a.lora_b + (col + c) * a.r + i0;
        float bf[8];
        if (a.lora_vec) {
          const uint4 bv = *reinterpret_cast<const uint4*>(brow);
          const uint32_t bw[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            bf[2 * e] = bf16_to_f32(bw[e] & 0xffffu);
            bf[2 * e + 1] = bf16_to_f32(bw[e] >> 16);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) bf[e] = i0 + e < a.r ? bf16_to_f32(brow[e]) : 0.0f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[c] += tf[e] * bf[e];
      }
    }
  }
  uint16_t* dst = a.y + (int64_t)m * a.n + col;
  if (vec) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
  } else {
    for (int c = 0; c < ncol; ++c) dst[c] = f32_to_bf16_bits(acc[c]);
  }
}

hipError_t launch_finish(const LinearPlan& p, int split, int rows, int m_valid,
                         const float* ypart, const float* gscale, const uint16_t* t,
                         const uint16_t* lora_b, int r, int lora_vec, uint16_t* y,
                         hipStream_t stream) {
  FinishArgs f;
  f.ypart = ypart;
  f.gscale = gscale;
  f.t = t;
  f.lora_b = lora_b;
  f.y = y;
  f.n = p.n;
  f.split = split;
  f.rows = rows;
  f.m_valid = m_valid;
  f.r = r;
  f.rpad16 = p.rpad16;
  f.lora_vec = lora_vec;
  f.vec4 = p.n % 4 == 0 && (reinterpret_cast<uintptr_t>(y) & 7) == 0;
  const int64_t threads = (p.n + 3) / 4 * m_valid;
  hipLaunchKernelGGL(splitk_finish, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     stream, f);
  return hipGetLastError();
}

// LDS-staged contraction (decode_lds.h) for one chunk of <= 64 rows, when
// k is a multiple of 256.
hipError_t run_decode_lds(const LinearPlan& p, int mt, const uint8_t* codes,
                          const uint8_t* scales, const float* gscale, const uint16_t* t,
                          const uint16_t* lora_b, int r, int lora_vec, const uint16_t* xt,
                          uint16_t* y, int m_valid, int64_t m0_chunk, char* ws,
                          hipStream_t stream) {
  dlds::Kernel kern = mt == 1 ? dlds::pick_mt1(p.dec_nt) : dlds::pick_mt2(p.dec_nt);
  if (!kern) return hipErrorInvalidConfiguration;
  dlds::Args a;
  a.xt = xt;
  a.codes = codes;
  a.scales = scales;
  a.gscale = gscale;
  a.t = t;
  a.lora_b = lora_b;
  a.y = y;
  a.ypart = reinterpret_cast<float*>(ws + p.off_ypart);
  a.n = p.n;
  a.k = p.k;
  const int split = lds_split(p);
  a.nblocks = p.k / 256;
  a.m_valid = m_valid;
  a.rows = p.dec_rows;
  a.split = split;
  a.r = r;
  a.rpad16 = p.rpad16;
  a.lora_vec = lora_vec;
  hipLaunchKernelGGL(kern, dim3((unsigned)p.dec_groups, (unsigned)split), dim3(512), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || split == 1) return e;
  return launch_finish(p, split, 32 * mt, m_valid, a.ypart, gscale, t, lora_b, r, lora_vec, y,
                       stream);
}

}  // namespace

hipError_t run_decode_chunks(const LinearPlan& p, const uint8_t* codes,
                             const uint8_t* scales, const float* gscale,
                             const uint16_t* lora_b, uint16_t* y, char* ws,
                             hipStream_t stream) {
  decode::DecodeArgs a;
  a.codes = codes;
  a.scales = scales;
  a.gscale = gscale;
  a.lora_b = lora_b;
  a.ypart = reinterpret_cast<float*>(ws + p.off_ypart);
  a.n = p.n;
  a.k = p.k;
  a.nfull = p.k / 64;
  a.tail_steps = (int)((p.k % 64) / 16);
  a.units_per_split = p.dec_kblk_per_split;
  a.rows = p.dec_rows;
  a.split = p.dec_split;
  a.r = (lora_b && p.r > 0) ? p.r : 0;
  a.rpad16 = p.rpad16;
  a.lora_vec = (a.r % 8 == 0) && ((reinterpret_cast<uintptr_t>(lora_b) & 15) == 0);
  const uint16_t* xt = reinterpret_cast<const uint16_t*>(ws + p.off_xt);
  const uint16_t* t = reinterpret_cast<const uint16_t*>(ws + p.off_t);
  int64_t m0 = 0;
  while (m0 < p.m) {
    const int64_t tiles_left = (p.mpad - m0) / 32;
    int mt = p.dec_mt;
    if (tiles_left < mt) mt = tiles_left >= 2 ? 2 : 1;
    a.xt = xt + m0 * p.k;
    a.t = t + m0 * p.rpad16;
    a.y = y + m0 * p.n;
    a.m_valid = (int)std::min<int64_t>(32 * mt, p.m - m0);
    hipError_t e;
    if (mt <= 2 && p.k % 256 == 0 && p.dec_nt <= 5) {
      e = run_decode_lds(p, mt, codes, scales, gscale, a.t, lora_b, a.r, a.lora_vec, a.xt,
                         a.y, a.m_valid, m0, ws, stream);
    } else {
      decode::DecodeKernel kern = pick_decode(mt, p.dec_nt);
      if (!kern) return hipErrorInvalidConfiguration;
      hipLaunchKernelGGL(kern, dim3((unsigned)p.dec_groups, (unsigned)p.dec_split),
                         dim3(256), 0, stream, a);
      e = hipGetLastError();
      if (e == hipSuccess && p.dec_split > 1)
        e = launch_finish(p, p.dec_split, 32 * mt, a.m_valid, a.ypart, gscale, a.t, lora_b,
                          a.r, a.lora_vec, a.y, stream);
    }
    if (e != hipSuccess) return e;
    m0 += 32 * mt;
  }
  return hipSuccess;
}

hipError_t launch_linear_decode_main(const LinearPlan& p, const uint8_t* codes,
                                     const uint8_t* scales, const float* gscale,
                                     const uint16_t* lora_b, uint16_t* y, char* ws,
                                     hipStream_t stream) {
  return run_decode_chunks(p, codes, scales, gscale, lora_b, y, ws, stream);
}

}  // namespace qerl
