// Decode contraction: launches over the m rows in chunks.  Per chunk, one
// contraction kernel -- the single-pass 128-token one (decode_m128.h) for
// chunks of three or four 32-row tiles when k % 128 == 0, else the
// LDS-staged one (decode_lds.h) where its shape conditions hold, else the
// general one (decode_kernel.h) -- and, when K is split across
// workgroups, the finishing kernel below.
#include <algorithm>

#include "decode_kernel.h"
#include "decode_lds.h"
#include "decode_m128.h"
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
  const float* __restrict__ ypart;      // [split, prows, n] fp32 partial sums of acc
  const float* __restrict__ gscale;
  const uint16_t* __restrict__ t;       // [rows, rpad16] bf16 s x_t A^T of this chunk
  const uint16_t* __restrict__ lora_b;  // [n, r] bf16
  uint16_t* __restrict__ y;             // [m_valid, n] rows of this chunk
  int64_t n;
  int split, rows, prows, m_valid, r, rpad16, lora_vec;   // rows <= prows finished
};

constexpr int kFinishBatch = 16;   // splits whose partial sums a thread loads together

// LoRA B operand of one MFMA step: B[col, j0 .. j0 + 7] (zeros past r or
// past the last column).
__device__ __forceinline__ uint4 finish_b(const FinishArgs& a, int64_t col, int j0) {
  if (col >= a.n || j0 >= a.r) return make_uint4(0u, 0u, 0u, 0u);
  const uint16_t* src = a.lora_b + col * a.r + j0;
  if (a.lora_vec) return *reinterpret_cast<const uint4*>(src);
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = (j0 + 2 * i < a.r) ? src[2 * i] : 0u;
    const uint32_t hi = (j0 + 2 * i + 1 < a.r) ? src[2 * i + 1] : 0u;
    w[i] = lo | (hi << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// y[m, j] = bf16(S * sum_s ypart[s, m, j] + sum_i t[m, i] B[j, i]): the
// epilogue of a split-K contraction [QeRL summary, §3.4, Eq. 6 (S) and
// Eq. 2 (LoRA side branch)].  One workgroup per 32 x 32 output tile (32
// token rows x 32 columns).  First every thread sums the splits of one
// token row and four columns in split order (16-byte loads, kFinishBatch
// splits in flight) into an LDS copy of the tile; then wave 0 reads the
// tile in the 32x32x16 MFMA accumulator layout (lane l: column l % 32),
// scales it by S and adds t B^T with MFMAs whose operands it loaded at the
// start, so B is read once per 32 token rows.
__global__ __launch_bounds__(256) void splitk_finish(FinishArgs a) {
  __shared__ float sums[32][33];
  const int lane = threadIdx.x & 63, c = lane & 31, h = lane >> 5;
  const int wave = threadIdx.x >> 6;
  const int64_t ctiles = (a.n + 31) / 32;
  const int u = (int)(blockIdx.x / ctiles);                  // token tile
  const int64_t col0 = (int64_t)(blockIdx.x - (int64_t)u * ctiles) * 32;

  // LoRA operands of wave 0 (r <= 128: at most eight 16-wide steps).
  uint4 tv[8], bv[8];
  if (wave == 0 && a.r > 0) {
    const uint16_t* trow = a.t + (int64_t)(32 * u + c) * a.rpad16 + 8 * h;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      tv[i] = make_uint4(0u, 0u, 0u, 0u);
      bv[i] = make_uint4(0u, 0u, 0u, 0u);
      if (16 * i < a.rpad16) {
        tv[i] = *reinterpret_cast<const uint4*>(trow + 16 * i);
        bv[i] = finish_b(a, col0 + c, 16 * i + 8 * h);
      }
    }
  }

  // Split sums: thread -> token row rr, columns cq .. cq + 3 of the tile.
  const int rr = threadIdx.x >> 3, cq = 4 * (threadIdx.x & 7);
  const int64_t col = col0 + cq;
  const int ncol = (int)max<int64_t>(0, min<int64_t>(4, a.n - col));
  const bool vec = ncol == 4 && a.n % 4 == 0;
  const float* src = a.ypart + (int64_t)(32 * u + rr) * a.n + col;
  const int64_t sstride = (int64_t)a.prows * a.n;
  float4 acc4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int s0 = 0; s0 < a.split; s0 += kFinishBatch) {
    float4 part[kFinishBatch];
#pragma unroll
    for (int b = 0; b < kFinishBatch; ++b) {
      part[b] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (s0 + b < a.split) {
        const float* ps = src + (int64_t)(s0 + b) * sstride;
        if (vec) {
          part[b] = *reinterpret_cast<const float4*>(ps);
        } else {
          if (ncol > 0) part[b].x = ps[0];
          if (ncol > 1) part[b].y = ps[1];
          if (ncol > 2) part[b].z = ps[2];
          if (ncol > 3) part[b].w = ps[3];
        }
      }
    }
#pragma unroll
    for (int b = 0; b < kFinishBatch; ++b) {
      if (s0 + b < a.split) {
        acc4.x += part[b].x;
        acc4.y += part[b].y;
        acc4.z += part[b].z;
        acc4.w += part[b].w;
      }
    }
  }
  sums[rr][cq] = acc4.x;
  sums[rr][cq + 1] = acc4.y;
  sums[rr][cq + 2] = acc4.z;
  sums[rr][cq + 3] = acc4.w;
  __syncthreads();
  if (wave != 0) return;

  const float S = *a.gscale;
  f32x16_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = S * sums[acc_row(v, lane)][c];
  if (a.r > 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (16 * i < a.rpad16) acc = mfma_bf16(tv[i], bv[i], acc);
  }
  if (col0 + c >= a.n) return;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int m = 32 * u + acc_row(v, lane);
    if (m < a.m_valid) a.y[(int64_t)m * a.n + col0 + c] = f32_to_bf16_bits(acc[v]);
  }
}

// rows: token rows to finish (a multiple of 32, at most prows, the rows of
// one split's partial tile block).
hipError_t launch_finish(const LinearPlan& p, int split, int rows, int m_valid,
                         const float* ypart, const float* gscale, const uint16_t* t,
                         const uint16_t* lora_b, int r, int lora_vec, uint16_t* y,
                         hipStream_t stream, int prows = 0) {
  FinishArgs f;
  f.ypart = ypart;
  f.gscale = gscale;
  f.t = t;
  f.lora_b = lora_b;
  f.y = y;
  f.n = p.n;
  f.split = split;
  f.rows = rows;
  f.prows = prows ? prows : rows;
  f.m_valid = m_valid;
  f.r = r;
  f.rpad16 = p.rpad16;
  f.lora_vec = lora_vec;
  const int64_t tiles = (p.n + 31) / 32 * (rows / 32);
  hipLaunchKernelGGL(splitk_finish, dim3((unsigned)tiles), dim3(256), 0, stream, f);
  return hipGetLastError();
}

// Workgroups appended to a split contraction launch of `wgs` workgroups to
// sum the LoRA-down partials: up to 8, on CU slots the contraction leaves
// free (one workgroup per CU: both kernels hold most of the LDS).
int reduce_wgs(int wgs) {
  return (int)std::max<int64_t>(0, std::min<int64_t>(8, (int64_t)device_cu_count() - wgs));
}

// Kernel of the chunk of a decode call that starts at token row m0: the
// 128-token kernel, the LDS-staged one or the general one, with its K
// split and token tiles.
enum class ChunkKernel { kM128, kLds, kMain };
struct ChunkChoice {
  ChunkKernel kind;
  int mt, split;
};

ChunkChoice choose_chunk(const LinearPlan& p, int64_t m0) {
  const int64_t tiles_left = (p.mpad - m0) / 32;
  if (p.m128 && (tiles_left >= 3 || p.tiled)) return {ChunkKernel::kM128, 4, p.m128_split};
  int mt = p.dec_mt;
  if (tiles_left < mt) mt = tiles_left >= 2 ? 2 : 1;
  if (mt <= 2 && p.k % 256 == 0 && p.dec_nt <= 5) return {ChunkKernel::kLds, mt, lds_split(p)};
  return {ChunkKernel::kMain, mt, p.dec_split};
}

// LDS-staged contraction (decode_lds.h) for one chunk of <= 64 rows, when
// k is a multiple of 256.
hipError_t run_decode_lds(const LinearPlan& p, int mt, const uint8_t* codes,
                          const uint8_t* scales, const float* gscale, const uint16_t* t,
                          const uint16_t* lora_b, int r, int lora_vec, const uint16_t* xt,
                          uint16_t* y, int m_valid, int64_t m0_chunk, char* ws,
                          hipStream_t stream, const TReduceArgs* tr) {
  dlds::Kernel kern = mt == 1 ? dlds::pick_mt1(p.dec_nt, p.pow2_scales)
                              : dlds::pick_mt2(p.dec_nt, p.pow2_scales);
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
  a.groups = p.dec_groups;
  a.tr_wgs = tr ? reduce_wgs(p.dec_groups * split) : 0;
  a.tr = tr ? *tr : TReduceArgs{};
  // Unsplit, the epilogue reads t: the reduction workgroups go first and
  // the contraction workgroups wait for them (sync words cleared by the
  // call's prepare).
  a.tsync = (a.tr_wgs > 0 && split == 1) ? reinterpret_cast<unsigned*>(ws + p.off_sync) : nullptr;
  a.tr.coherent = a.tsync ? 1 : 0;
  hipLaunchKernelGGL(kern, dim3((unsigned)(p.dec_groups * split + a.tr_wgs)), dim3(512), 0,
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || split == 1) return e;
  return launch_finish(p, split, 32 * mt, m_valid, a.ypart, gscale, t, lora_b, r, lora_vec, y,
                       stream);
}

// Single-pass contraction (decode_m128.h) of one chunk of up to 128 rows:
// xrows rows of x_t (and t) exist, m_valid of them are output rows.
hipError_t run_decode_m128(const LinearPlan& p, const uint8_t* codes, const uint8_t* scales,
                           const float* gscale, const uint16_t* t, const uint16_t* lora_b, int r,
                           int lora_vec, const uint16_t* xt, uint16_t* y, int xrows, int m_valid,
                           char* ws, hipStream_t stream, const TReduceArgs* tr) {
  d128::Args a;
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
  a.nblocks = p.k / d128::kBlock;
  a.xrows = xrows;
  a.m_valid = m_valid;
  a.split = p.m128_split;
  a.r = r;
  a.rpad16 = p.rpad16;
  a.lora_vec = lora_vec;
  a.groups = p.m128_groups;
  a.tr_wgs = tr ? reduce_wgs(p.m128_groups * a.split) : 0;
  a.tr = tr ? *tr : TReduceArgs{};
  // Unsplit, the epilogue reads t: the reduction workgroups go first and
  // the contraction workgroups wait for them (sync words cleared by the
  // call's prepare).
  a.tsync = (a.tr_wgs > 0 && a.split == 1) ? reinterpret_cast<unsigned*>(ws + p.off_sync)
                                           : nullptr;
  a.tr.coherent = a.tsync ? 1 : 0;
  hipLaunchKernelGGL(d128::pick(p.pow2_scales, p.tiled),
                     dim3((unsigned)(p.m128_groups * a.split + a.tr_wgs)), dim3(512), 0, stream,
                     a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.split == 1) return e;
  return launch_finish(p, a.split, (int)((xrows + 31) / 32 * 32), m_valid, a.ypart, gscale, t,
                       lora_b, r, lora_vec, y, stream, d128::kTokens);
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
  // The LoRA-down partials are summed into t by the first launch's extra
  // workgroups when the prepare left that to it, else t is already there.
  const TReduceArgs trs = treduce_args(p, ws);
  const TReduceArgs* tr = (a.r > 0 && p.t_in_contraction) ? &trs : nullptr;
  if (tr && !t_reduce_can_merge(p)) {
    hipError_t e = launch_treduce(p, ws, stream);
    if (e != hipSuccess) return e;
    tr = nullptr;
  }
  int64_t m0 = 0;
  while (m0 < p.m) {
    const ChunkChoice ch = choose_chunk(p, m0);
    if (ch.kind == ChunkKernel::kM128) {
      const int xrows = (int)std::min<int64_t>(d128::kTokens, p.mpad - m0);
      const int m_valid = (int)std::min<int64_t>(d128::kTokens, p.m - m0);
      hipError_t e = run_decode_m128(p, codes, scales, gscale, t + m0 * p.rpad16, lora_b, a.r,
                                     a.lora_vec, xt + m0 * p.k, y + m0 * p.n, xrows, m_valid, ws,
                                     stream, tr);
      if (e != hipSuccess) return e;
      tr = nullptr;
      m0 += d128::kTokens;
      continue;
    }
    const int mt = ch.mt;
    a.xt = xt + m0 * p.k;
    a.t = t + m0 * p.rpad16;
    a.y = y + m0 * p.n;
    a.m_valid = (int)std::min<int64_t>(32 * mt, p.m - m0);
    hipError_t e;
    if (ch.kind == ChunkKernel::kLds) {
      e = run_decode_lds(p, mt, codes, scales, gscale, a.t, lora_b, a.r, a.lora_vec, a.xt,
                         a.y, a.m_valid, m0, ws, stream, tr);
      tr = nullptr;
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

bool t_reduce_can_merge(const LinearPlan& p) {
  const ChunkChoice ch = choose_chunk(p, 0);
  const int groups = ch.kind == ChunkKernel::kM128 ? p.m128_groups : p.dec_groups;
  return ch.kind != ChunkKernel::kMain && reduce_wgs(groups * ch.split) > 0;
}

hipError_t tile128(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k,
                   uint8_t* out, hipStream_t stream) {
  return d128::launch_tile128(codes, scales, n, k, out, stream);
}

size_t tile128_bytes(int64_t n, int64_t k) { return d128::tile128_bytes(n, k); }

hipError_t launch_linear_decode_main(const LinearPlan& p, const uint8_t* codes,
                                     const uint8_t* scales, const float* gscale,
                                     const uint16_t* lora_b, uint16_t* y, char* ws,
                                     hipStream_t stream) {
  return run_decode_chunks(p, codes, scales, gscale, lora_b, y, ws, stream);
}

}  // namespace qerl
