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
  const float* __restrict__ tpart;      // [kchunks, mpad, rpad32] (chunk rows), or null
  const uint16_t* __restrict__ lora_b;  // [n, r] bf16
  uint16_t* __restrict__ y;             // [m_valid, n] rows of this chunk
  int64_t n, tpart_stride;
  int split, rows, m_valid, r, rpad16, rpad32, kchunks, lora_vec;
};

constexpr int kFinishRows = 4;  // token rows per thread

// y[m, j] = bf16(S * sum_s ypart[s, m, j] + sum_i t[m, i] B[j, i]): the
// epilogue of a split-K contraction [QeRL summary, §3.4, Eq. 6 (S) and
// Eq. 2 (LoRA side branch)].  The splits are summed in split order.  One
// thread per output column j and kFinishRows token rows; t of those rows
// sits in LDS, either read from t or, when the prepare step left only the
// chunk partials, summed from them here in chunk order and rounded to
// bf16.  Every thread issues its partial-sum loads before the LDS staging.
__global__ __launch_bounds__(256) void splitk_finish(FinishArgs a) {
  __shared__ float t_lds[kFinishRows * 128];
  const int m0 = blockIdx.y * kFinishRows;
  const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool live = col < a.n;
  const int mrows = min(kFinishRows, a.m_valid - m0);
  float acc[kFinishRows];
#pragma unroll
  for (int mm = 0; mm < kFinishRows; ++mm) acc[mm] = 0.0f;
  if (live) {
    const float* src = a.ypart + (int64_t)m0 * a.n + col;
    const int64_t sstride = (int64_t)a.rows * a.n;
#pragma unroll 4
    for (int s = 0; s < a.split; ++s) {
#pragma unroll
      for (int mm = 0; mm < kFinishRows; ++mm)
        if (mm < mrows) acc[mm] += src[s * sstride + (int64_t)mm * a.n];
    }
  }
  // The LoRA B row of this column, loaded before the LDS staging when it is
  // 16-byte aligned and short (r <= 64), so that all global loads of the
  // thread are in flight together.
  constexpr int kBPre = 8;
  const bool bpre = a.lora_vec && a.r <= 8 * kBPre;
  uint4 bv[kBPre];
  if (live && bpre) {
    const uint4* brow4 = reinterpret_cast<const uint4*>(a.lora_b + col * a.r);
#pragma unroll
    for (int q = 0; q < kBPre; ++q)
      bv[q] = 8 * q < a.r ? brow4[q] : make_uint4(0u, 0u, 0u, 0u);
  }
  if (a.tpart) {
    // Items (mm, jj) of t, kFinishRows x r <= 512 of them, 128 per pass:
    // the two thread halves sum the even and the odd chunks (eight loads
    // in flight per thread), then the halves are combined in chunk-pair
    // order and rounded to bf16.
    __shared__ float half_sum[2][128];
    const int items = kFinishRows * a.r;
    const int hf = threadIdx.x >> 7, it = threadIdx.x & 127;
    for (int base = 0; base < items; base += 128) {
      const int i = base + it;
      float v = 0.0f;
      if (i < items) {
        const int mm = i / a.r, jj = i % a.r;
        if (m0 + mm < a.m_valid) {
          const float* tp = a.tpart + (int64_t)(m0 + mm) * a.rpad32 + jj;
          float p4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
          int c = hf;
          for (; c + 14 < a.kchunks; c += 16) {
#pragma unroll
            for (int u = 0; u < 8; ++u) p4[u & 3] += tp[(int64_t)(c + 2 * u) * a.tpart_stride];
          }
          for (; c < a.kchunks; c += 2) p4[0] += tp[(int64_t)c * a.tpart_stride];
          v = (p4[0] + p4[1]) + (p4[2] + p4[3]);
        }
      }
      half_sum[hf][it] = v;
      __syncthreads();
      if (hf == 0 && i < items) {
        const int mm = i / a.r, jj = i % a.r;
        t_lds[mm * 128 + jj] = bf16_to_f32(f32_to_bf16_bits(half_sum[0][it] + half_sum[1][it]));
      }
      __syncthreads();
    }
    // Columns jj >= r of t_lds are never read (the LoRA loop stops at r).
  } else {
    for (int i = threadIdx.x; i < kFinishRows * 128; i += 256) {
      const int mm = i / 128, jj = i % 128;
      t_lds[i] = (m0 + mm < a.m_valid && jj < a.r)
                     ? bf16_to_f32(a.t[(int64_t)(m0 + mm) * a.rpad16 + jj])
                     : 0.0f;
    }
  }
  __syncthreads();
  if (!live) return;
  const float S = *a.gscale;
#pragma unroll
  for (int mm = 0; mm < kFinishRows; ++mm) acc[mm] *= S;
  if (bpre) {
#pragma unroll
    for (int q = 0; q < kBPre; ++q) {
      if (8 * q >= a.r) break;
      const uint32_t bw[4] = {bv[q].x, bv[q].y, bv[q].z, bv[q].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float b0 = bf16_to_f32(bw[e] & 0xffffu), b1 = bf16_to_f32(bw[e] >> 16);
#pragma unroll
        for (int mm = 0; mm < kFinishRows; ++mm)
          acc[mm] += t_lds[mm * 128 + 8 * q + 2 * e] * b0 + t_lds[mm * 128 + 8 * q + 2 * e + 1] * b1;
      }
    }
  }
  const uint16_t* brow = a.lora_b + col * a.r;
  for (int i0 = bpre ? a.r : 0; i0 < a.r; i0 += 8) {
    uint32_t bw[4];
    if (a.lora_vec) {
      const uint4 v = *reinterpret_cast<const uint4*>(brow + i0);
      bw[0] = v.x; bw[1] = v.y; bw[2] = v.z; bw[3] = v.w;
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = i0 + 2 * q < a.r ? brow[i0 + 2 * q] : 0u;
        const uint32_t hi = i0 + 2 * q + 1 < a.r ? brow[i0 + 2 * q + 1] : 0u;
        bw[q] = lo | (hi << 16);
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float b0 = bf16_to_f32(bw[q] & 0xffffu), b1 = bf16_to_f32(bw[q] >> 16);
#pragma unroll
      for (int mm = 0; mm < kFinishRows; ++mm)
        acc[mm] += t_lds[mm * 128 + i0 + 2 * q] * b0 + t_lds[mm * 128 + i0 + 2 * q + 1] * b1;
    }
  }
#pragma unroll
  for (int mm = 0; mm < kFinishRows; ++mm)
    if (mm < mrows) a.y[(int64_t)(m0 + mm) * a.n + col] = f32_to_bf16_bits(acc[mm]);
}

// m0_chunk: first token row of the chunk (for the LoRA-down partials).
hipError_t launch_finish(const LinearPlan& p, int split, int rows, int m_valid, int64_t m0_chunk,
                         const float* ypart, const float* gscale, const uint16_t* t,
                         const uint16_t* lora_b, int r, int lora_vec, uint16_t* y,
                         const char* ws, hipStream_t stream) {
  FinishArgs f;
  f.ypart = ypart;
  f.gscale = gscale;
  f.t = t;
  f.tpart = (r > 0 && !prepare_reduces_t(p))
                ? reinterpret_cast<const float*>(ws + p.off_tpart) + m0_chunk * p.rpad32
                : nullptr;
  f.tpart_stride = p.mpad * p.rpad32;
  f.lora_b = lora_b;
  f.y = y;
  f.n = p.n;
  f.split = split;
  f.rows = rows;
  f.m_valid = m_valid;
  f.r = r;
  f.rpad16 = p.rpad16;
  f.rpad32 = p.rpad32;
  f.kchunks = p.kchunks;
  f.lora_vec = lora_vec;
  const dim3 grid((unsigned)((p.n + 255) / 256),
                  (unsigned)((m_valid + kFinishRows - 1) / kFinishRows));
  hipLaunchKernelGGL(splitk_finish, grid, dim3(256), 0, stream, f);
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
  const int64_t nblocks = p.k / 256;
  const int64_t per = (nblocks + p.dec_split - 1) / p.dec_split;
  const int split = (int)((nblocks + per - 1) / per);
  a.blocks_per_split = per;
  a.m_valid = m_valid;
  a.rows = p.dec_rows;
  a.split = split;
  a.r = r;
  a.rpad16 = p.rpad16;
  a.lora_vec = lora_vec;
  hipLaunchKernelGGL(kern, dim3((unsigned)p.dec_groups, (unsigned)split), dim3(512), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || split == 1) return e;
  return launch_finish(p, split, 32 * mt, m_valid, m0_chunk, a.ypart, gscale, t, lora_b, r,
                       lora_vec, y, ws, stream);
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
        e = launch_finish(p, p.dec_split, 32 * mt, a.m_valid, m0, a.ypart, gscale, a.t, lora_b,
                          a.r, a.lora_vec, a.y, ws, stream);
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
