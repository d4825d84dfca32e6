// Decode contraction: launch of decode_main (decode_kernel.h) over the m
// rows in chunks of at most 32 * dec_mt rows.
#include <algorithm>

#include "decode_kernel.h"
#include "decode_lds.h"
#include "qerl_internal.h"

namespace qerl {

static decode::DecodeKernel pick_decode(int mt, int nt, int rt) {
  switch (mt) {
    case 1: return decode::pick_mt1(nt, rt);
    case 2: return decode::pick_mt2(nt, rt);
    case 4: return decode::pick_mt4(nt, rt);
    default: return nullptr;
  }
}

// LDS-staged contraction (decode_lds.h) for one chunk of <= 64 rows, when
// k is a multiple of 256 and the LoRA-down is precomputed.
static hipError_t run_decode_lds(const LinearPlan& p, int mt, const uint8_t* codes,
                                 const uint8_t* scales, const float* gscale,
                                 const uint16_t* t, const uint16_t* lora_b, int r,
                                 int lora_vec, const uint16_t* xt, uint16_t* y, int m_valid,
                                 char* ws, hipStream_t stream) {
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
  a.cnt = reinterpret_cast<uint32_t*>(ws + p.off_cnt);
  a.n = p.n;
  a.k = p.k;
  const int64_t nblocks = p.k / 256;
  int64_t per = (nblocks + p.dec_split - 1) / p.dec_split;
  const int64_t split = (nblocks + per - 1) / per;
  a.blocks_per_split = per;
  a.m_valid = m_valid;
  a.rows = p.dec_rows;
  a.split = (int)split;
  a.r = r;
  a.rpad16 = p.rpad16;
  a.lora_vec = lora_vec;
  hipLaunchKernelGGL(kern, dim3((unsigned)p.dec_groups, (unsigned)split), dim3(512), 0, stream, a);
  return hipGetLastError();
}

hipError_t run_decode_chunks(const LinearPlan& p, const uint8_t* codes,
                             const uint8_t* scales, const float* gscale,
                             const uint16_t* lora_a, float lora_scale,
                             const uint16_t* lora_b, uint16_t* y, char* ws,
                             hipStream_t stream) {
  decode::DecodeArgs a;
  a.codes = codes;
  a.scales = scales;
  a.gscale = gscale;
  a.lora_a = lora_a;
  a.lora_b = lora_b;
  a.ypart = reinterpret_cast<float*>(ws + p.off_ypart);
  a.tpart = reinterpret_cast<float*>(ws + p.off_tsplit);
  a.cnt = reinterpret_cast<uint32_t*>(ws + p.off_cnt);
  a.n = p.n;
  a.k = p.k;
  a.nfull = p.k / 64;
  a.tail_steps = (int)((p.k % 64) / 16);
  a.units_per_split = p.dec_kblk_per_split;
  a.rows = p.dec_rows;
  a.split = p.dec_split;
  a.r = (lora_b && p.r > 0) ? p.r : 0;
  a.rpad16 = p.rpad16;
  a.rpad32 = p.rpad32;
  a.lora_scale = lora_scale;
  a.lora_vec = (a.r % 8 == 0) && ((reinterpret_cast<uintptr_t>(lora_b) & 15) == 0);
  const int rt = a.r > 0 ? p.dec_rt : 0;
  if (rt > 0 && !lora_a) return hipErrorInvalidValue;
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
    if (mt <= 2 && rt == 0 && p.k % 256 == 0 && p.dec_nt <= 5) {
      const hipError_t e = run_decode_lds(p, mt, codes, scales, gscale, a.t, lora_b, a.r,
                                          a.lora_vec, a.xt, a.y, a.m_valid, ws, stream);
      if (e != hipSuccess) return e;
      m0 += 32 * mt;
      continue;
    }
    decode::DecodeKernel kern = pick_decode(mt, p.dec_nt, rt);
    if (!kern) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kern, dim3((unsigned)p.dec_groups, (unsigned)p.dec_split),
                       dim3(256), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    m0 += 32 * mt;
  }
  return hipSuccess;
}

hipError_t launch_linear_decode_main(const LinearPlan& p, const uint8_t* codes,
                                     const uint8_t* scales, const float* gscale,
                                     const uint16_t* lora_a, float lora_scale,
                                     const uint16_t* lora_b, uint16_t* y, char* ws,
                                     hipStream_t stream) {
  return run_decode_chunks(p, codes, scales, gscale, lora_a, lora_scale, lora_b, y, ws,
                           stream);
}

}  // namespace qerl
