// Linear layer, shared part: launch plan, workspace layout and the prepare
// step that both the decode and the prefill contraction consume.
//
// The layer [QeRL summary, §3.4, Eq. 2 (LoRA on the quantized weight) and
// Eq. 10-12 (AQN noise folded into the RMSNorm scale, i.e. a multiplier
// (1 + z_j) on input channel j shared by every token of the call)]:
//     x_t = x (.) (1 + z)
//     y   = bf16( S * (x_t W0^T) + (s x_t A^T) B^T ),  W0 = e2m1 (.) s_b
// S (the FP32 tensor scale) is applied to the fp32 accumulator once in the
// epilogue, so the dequantized weight W0 = e2m1 * s_b is exact in bf16.
//
// prepare writes x_t = bf16(x * (1 + z)) to the workspace, rows padded to a
// multiple of 32 with zeros so the contraction kernels need no row masks,
// and, with a LoRA branch, the LoRA-down t:
//   prep_kernel (four waves per 32 rows x 512-wide K chunk): x_t, read
//           and written one row per instruction, and tpart = x_t A^T over
//           the chunk (bf16 MFMA, fp32, operands through LDS);
//   treduce: t = bf16(sum over chunks of tpart), summed in a fixed order
//           so the result is deterministic; a launch of its own, or (whole
//           decode calls whose first contraction launch has CU slots to
//           spare) workgroups of that launch running the same routine.
// Without a LoRA branch a single elementwise kernel (xt_kernel) writes x_t.
#include <algorithm>

#include "qerl_act.h"
#include "qerl_device.h"
#include "qerl_internal.h"
#include "treduce.h"

namespace qerl {

int device_cu_count() {
  static int cached = [] {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount,
                              dev) != hipSuccess || cus <= 0)
      return 256;
    return cus;
  }();
  return cached;
}

namespace {

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t rup(int64_t a, int64_t b) { return cdiv(a, b) * b; }

// K range of one prepare workgroup (four waves of a quarter each) for the
// LoRA-down of other operands (launch_lora_down).
constexpr int64_t kPrepChunk = 512;

// K range of one prepare workgroup of a linear call (mtiles 32-row tiles,
// rtiles 32-wide rank tiles): 512 channels, halved (down to 128) while the
// launch has fewer than 256 workgroups and the K chunks -- the partial sums
// the LoRA-down reduction adds per output -- stay at most kMaxPrepChunks.
// Narrow chunks give the latency-bound prepare of a decode call more
// workgroups; the reduction's loads grow with the chunk count.  (Measured on
// whole decode steps: 128 for K = 5120 and 3584, 256 for K = 18944, 512 for
// K = 27648 and for prefill-sized m.)
constexpr int64_t kMaxPrepChunks = 80;
int64_t prep_chunk(int64_t k, int64_t mtiles, int64_t rtiles) {
  int64_t ch = 512;
  while (ch > 128 && mtiles * cdiv(k, ch) * rtiles < 256 && cdiv(k, ch / 2) <= kMaxPrepChunks)
    ch /= 2;
  return ch;
}

// Largest weight subtile count NT per wave that the decode kernels hold in
// registers without spilling, for MT token tiles (from the compiler's
// resource report: the general kernel spills at MT = 4, NT = 3).
int decode_nt_max(int mt) { return mt == 1 ? 6 : (mt == 2 ? 5 : 2); }

// Decode rows per workgroup and split-K choice for one m tile count.
void plan_decode(LinearPlan* p, int mt) {
  const int cu = device_cu_count();
  const int ntmax = decode_nt_max(mt);
  const int64_t n = p->n;
  const int64_t units = cdiv(p->k, 64);     // 64-wide K blocks (last may be partial)
  const int64_t rows_per_cu = cdiv(n, cu);
  int rows, split;
  if (rows_per_cu >= 64 || units < 8) {
    const int64_t rounds = cdiv(rows_per_cu, 32 * ntmax);
    rows = (int)rup(cdiv(n, rounds * cu), 16);
    rows = std::min(rows, 32 * ntmax);
    split = 1;
  } else {
    double best = -1.0;
    rows = 32 * ntmax;
    split = 1;
    for (int cand = 64; cand <= 32 * ntmax; cand += 16) {
      const int64_t groups = cdiv(n, cand);
      int64_t s = std::max<int64_t>(1, cu / groups);
      s = std::min<int64_t>(s, std::max<int64_t>(1, units / 4));
      const int64_t wgs = groups * s;
      // CU occupancy times the share of the streamed 32-row subtiles that
      // belongs to the workgroup (the rest is loaded and discarded).
      const double util = (double)wgs / (double)(cu * cdiv(wgs, cu)) *
                          (double)cand / (double)(32 * cdiv(cand, 32));
      if (util > best + 1e-9 || (util > best - 1e-9 && cand > rows)) {
        best = util;
        rows = cand;
        split = (int)s;
      }
    }
  }
  int64_t per = cdiv(units, split);
  split = (int)cdiv(units, per);
  p->dec_mt = mt;
  p->dec_rows = rows;
  p->dec_nt = (int)cdiv(rows, 32);
  p->dec_groups = (int)cdiv(n, rows);
  p->dec_split = split;
  p->dec_kblk_per_split = per;
}

// Single-pass 128-token contraction: 256 weight rows per workgroup; K is
// split across workgroups when the row groups alone leave CUs idle (one
// round of workgroups, at least two 128-wide blocks per split).  The split
// count minimises a cost fitted to whole calls on the 32B shapes at 128
// tokens (qkv 7168 x 5120, o 5120 x 5120, down 5120 x 27648; splits 2-12):
// about 1.16 us per K block of the longest split, plus 0.215 us per split
// and 1000 output columns for writing and summing the fp32 partials, plus
// one more launch (the finish) when K is split.
void plan_m128(LinearPlan* p) {
  const int cu = device_cu_count();
  const int64_t groups = cdiv(p->n, 256);
  const int64_t nblocks = p->k / 128;
  int64_t split = 1;
  if (groups * 4 < cu * 3) {
    const int64_t smax = std::max<int64_t>(1, std::min<int64_t>(cu / groups, nblocks / 2));
    double best = 0.0;
    for (int64_t s = 1; s <= smax; ++s) {
      const double cost = 1.16 * (double)cdiv(nblocks, s) + 0.215e-3 * (double)(s * p->n) +
                          (s > 1 ? 4.0 : 0.0);
      if (s == 1 || cost < best) {
        best = cost;
        split = s;
      }
    }
  }
  p->m128 = true;
  p->m128_groups = (int)groups;
  p->m128_split = (int)split;
}

}  // namespace

bool make_linear_plan(int64_t m, int64_t n, int64_t k, int r, LinearPlan* p, bool tiled) {
  if (m < 1 || n < 1 || k < 16 || k % 16 || r < 0 || r > 128) return false;
  if (tiled && (k % 128 || ((n + 31) / 32) * (k / 128) * 2304 >= ((int64_t)1 << 31))) return false;
  *p = LinearPlan{};
  p->m = m;
  p->n = n;
  p->k = k;
  p->r = r;
  p->mpad = rup(m, 32);
  p->rpad32 = r ? (int)rup(r, 32) : 0;
  p->rpad16 = r ? (int)rup(r, 16) : 0;
  const int64_t mtiles = p->mpad / 32;
  p->kchunk = prep_chunk(k, mtiles, std::max(1, p->rpad32 / 32));
  p->kchunks = (int)cdiv(k, p->kchunk);
  // Token tiles per decode launch: 1, 2 or 4 (the instantiated kernels);
  // run_decode_chunks takes smaller chunks for the remainder.
  // With k % 256 == 0 the LDS-staged kernel (up to two tiles) is used even
  // for more rows, one 64-row chunk after the other: it streams the weights
  // fast enough that two passes beat one pass of the general kernel.
  // With k % 128 == 0 and at least three token tiles the single-pass
  // 128-token kernel takes chunks of 128 rows, and the kernels planned here
  // only a remainder of one or two tiles.
  // (Its buffer descriptors take 32-bit byte counts: codes under 2 GB.)
  const bool m128 = tiled || (k % 128 == 0 && mtiles >= 3 && n * (k / 2) < ((int64_t)1 << 31));
  const int mt_cap = (m128 || k % 256 == 0) ? 2 : 4;
  const int mt = std::min(mt_cap, mtiles >= 4 ? 4 : (mtiles >= 2 ? 2 : 1));
  plan_decode(p, mt);
  if (m128) plan_m128(p);
  p->tiled = tiled;
  p->pf_tile_m = 128;
  p->pf_tile_n = 128;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = (size_t)rup((int64_t)(off + bytes), 256);
    return o;
  };
  p->off_xt = take((size_t)p->mpad * k * 2);
  p->off_tpart = take(r ? (size_t)p->kchunks * p->mpad * p->rpad32 * 4 : 0);
  p->off_t = take(r ? (size_t)p->mpad * p->rpad16 * 2 : 0);
  p->off_sync = take(8);
  size_t ypart = p->dec_split > 1 ? (size_t)p->dec_split * 32 * p->dec_mt * n * 4 : 0;
  if (p->m128 && p->m128_split > 1)
    ypart = std::max(ypart, (size_t)p->m128_split * 128 * n * 4);
  p->off_ypart = take(ypart);
  p->total = off;
  return true;
}

namespace {

struct PrepArgs {
  const uint16_t* __restrict__ x;  // [m, ldx]; with swiglu, gate in 0 .. k-1 and up in k .. 2k-1
  int64_t ldx;
  int swiglu;                      // the layer input is bf16(SiLU(gate) * up)
  const float* __restrict__ z;     // [k] shared by the rows, or [m, k] one row per token
  int64_t z_ld;                    // 0: shared; k: one noise row per token
  const uint16_t* __restrict__ a;
  uint16_t* __restrict__ xt;     // null: x_t is not written (only the LoRA-down partials)
  float* __restrict__ tpart;
  unsigned* sync;                  // two words cleared by the first workgroup, or null
  int64_t m, mpad, k;
  int r, rpad32;
  float lora_scale;
};

// One workgroup: 32 rows x one CH-wide K chunk x RT 32-wide rank tiles
// (the launches use RT = 1 and one rank tile per grid z).
//   x_t: wave w reads and writes rows 8 w .. 8 w + 7, RPI rows of the chunk
//        per instruction (CH / 8 lanes per row, each holding eight
//        channels); the rows also go to an LDS tile, 16-byte chunk q of row
//        rr stored at q ^ (rr mod 16) so that the MFMA reads below (lane =
//        row) hit 16 different bank groups per 16 lanes.
//   LoRA-down: wave w takes the CH / 4 channels at w CH / 4:
//        STEPS 32x32x16 MFMAs per 32 rows of A, operands x_t from the LDS tile
//        and A from global memory (issued first, so their latency passes
//        under the x_t work).
// The four waves' LoRA-down tiles are summed through LDS and wave 0 writes
// the chunk's partial tpart[chunk, rows, rpad32].
template <int RT, int CH>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs p) {
  constexpr int STEPS = CH / 64;     // 16-deep steps per wave
  constexpr int QPR = CH / 8;        // 16-byte chunks per row
  constexpr int RPI = 64 / QPR;                   // rows per load instruction
  static_assert(QPR >= 16 && QPR <= 64 && 64 % QPR == 0, "chunk of 128 to 512 channels");
  __shared__ __attribute__((aligned(16))) uint4 xs[32 * QPR];
  __shared__ float red[3 * (RT > 0 ? RT : 1) * 16 * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, c = lane & 31;
  const int64_t kc = (int64_t)blockIdx.y * CH;
  const int64_t row0 = (int64_t)blockIdx.x * 32;
  if (p.sync && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x < 2)
    p.sync[threadIdx.x] = 0u;

  // A operands of this wave's channels (lane: row j = 32 t + c of A, from
  // the rank tiles of this workgroup: blockIdx.z picks RT tiles of 32).
  const int64_t kb = kc + (CH / 4) * wave;
  const int rank0 = 32 * RT * (int)blockIdx.z;
  uint4 av[RT > 0 ? RT : 1][STEPS];
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int64_t k0 = kb + 16 * s + 8 * h;
    const bool in = kb + 16 * s < p.k;   // k % 16 == 0: the whole step is in range
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int j = rank0 + 32 * t + c;
      av[t][s] = (in && j < p.r) ? *reinterpret_cast<const uint4*>(p.a + (int64_t)j * p.k + k0)
                                 : make_uint4(0u, 0u, 0u, 0u);
    }
  }

  // x_t rows, coalesced: lane l holds channels 8 (l mod QPR) .. + 7 of row
  // 8 wave + RPI i + l / QPR.
  const int q = lane % QPR, sub = lane / QPR;
  const int64_t kl = kc + 8 * q;          // this lane's channels
  const bool kin = kl < p.k;              // k % 8 == 0: all eight in range or none
  float4 z0 = make_float4(0.0f, 0.0f, 0.0f, 0.0f), z1 = z0;
  if (kin && p.z && p.z_ld == 0) {
    z0 = *reinterpret_cast<const float4*>(p.z + kl);
    z1 = *reinterpret_cast<const float4*>(p.z + kl + 4);
  }
  constexpr int NX = 8 / RPI;             // load instructions per wave
  uint4 xv[NX];
#pragma unroll
  for (int i = 0; i < NX; ++i) {
    const int64_t mrow = row0 + 8 * wave + RPI * i + sub;
    xv[i] = (kin && mrow < p.m) ? *reinterpret_cast<const uint4*>(p.x + mrow * p.ldx + kl)
                                : make_uint4(0u, 0u, 0u, 0u);
  }
  if (p.swiglu) {
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int64_t mrow = row0 + 8 * wave + RPI * i + sub;
      const uint4 up = (kin && mrow < p.m)
                           ? *reinterpret_cast<const uint4*>(p.x + mrow * p.ldx + p.k + kl)
                           : make_uint4(0u, 0u, 0u, 0u);
      xv[i] = swiglu8(xv[i], up);      // rows past m: SiLU(0) * 0 = 0
    }
  }
#pragma unroll
  for (int i = 0; i < NX; ++i) {
    const int rr = 8 * wave + RPI * i + sub;
    const int64_t mrow = row0 + rr;
    if (mrow < p.m && p.z) {
      if (p.z_ld && kin) {
        const float* zr = p.z + mrow * p.z_ld + kl;     // this token's own noise row
        xv[i] = noisy8(xv[i], *reinterpret_cast<const float4*>(zr),
                       *reinterpret_cast<const float4*>(zr + 4));
      } else {
        xv[i] = noisy8(xv[i], z0, z1);
      }
    }
    if (kin && p.xt && blockIdx.z == 0) *reinterpret_cast<uint4*>(p.xt + mrow * p.k + kl) = xv[i];
    xs[rr * QPR + (q ^ (rr & 15))] = xv[i];
  }
  if (RT == 0) return;
  __syncthreads();

  f32x16_t acc[RT > 0 ? RT : 1];
#pragma unroll
  for (int t = 0; t < (RT > 0 ? RT : 1); ++t) acc[t] = zero16();
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const uint4 xa = xs[c * QPR + (((QPR / 4) * wave + 2 * s + h) ^ (c & 15))];
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[t] = mfma_bf16(xa, av[t][s], acc[t]);
  }
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) red[(((wave - 1) * RT + t) * 16 + v) * 64 + lane] = acc[t][v];
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int t = 0; t < RT; ++t) {
#pragma unroll
    for (int w = 0; w < 3; ++w)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[t][v] += red[((w * RT + t) * 16 + v) * 64 + lane];
    float* dst = p.tpart + ((int64_t)blockIdx.y * p.mpad + row0) * p.rpad32 + rank0 + 32 * t + c;
#pragma unroll
    for (int v = 0; v < 16; ++v) dst[(int64_t)acc_row(v, lane) * p.rpad32] = p.lora_scale * acc[t][v];
  }
}

// x_t = bf16(x (1 + z)) only (no LoRA branch): 8 elements per thread; rows
// m..mpad-1 are written as zeros.
__global__ __launch_bounds__(256) void xt_kernel(PrepArgs p) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (p.sync && i < 2) p.sync[i] = 0u;
  const int64_t per_row = p.k / 8;
  if (i >= p.mpad * per_row) return;
  const int64_t mrow = i / per_row, k0 = (i % per_row) * 8;
  uint4 xv = make_uint4(0u, 0u, 0u, 0u);
  if (mrow < p.m) {
    xv = *reinterpret_cast<const uint4*>(p.x + mrow * p.ldx + k0);
    if (p.swiglu) xv = swiglu8(xv, *reinterpret_cast<const uint4*>(p.x + mrow * p.ldx + p.k + k0));
    if (p.z) {
      const float* zr = p.z + mrow * p.z_ld + k0;
      xv = noisy8(xv, *reinterpret_cast<const float4*>(zr),
                  *reinterpret_cast<const float4*>(zr + 4));
    }
  }
  *reinterpret_cast<uint4*>(p.xt + mrow * p.k + k0) = xv;
}

// t = bf16(sum over chunks of tpart) (the partials carry s already): one
// thread per (row, j), the chunks summed in the fixed order of treduce_one.
__global__ __launch_bounds__(256) void treduce_kernel(TReduceArgs a) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < a.mpad * a.rpad16) treduce_one(a, i);
}

}  // namespace

int lds_split(const LinearPlan& p) {
  return (int)std::min<int64_t>(p.dec_split, std::max<int64_t>(1, p.k / 256));
}

hipError_t launch_lora_down(const uint16_t* x, int64_t m, int64_t mpad, int64_t k,
                            const uint16_t* a_rk, int r, float scale, float* tpart,
                            uint16_t* t, hipStream_t stream) {
  PrepArgs a;
  a.x = x;
  a.ldx = k;
  a.swiglu = 0;
  a.z = nullptr;
  a.z_ld = 0;
  a.a = a_rk;
  a.xt = nullptr;
  a.tpart = tpart;
  a.sync = nullptr;
  a.m = m;
  a.mpad = mpad;
  a.k = k;
  a.r = r;
  a.rpad32 = (int)rup(r, 32);
  a.lora_scale = scale;
  const int kchunks = (int)cdiv(k, kPrepChunk);
  // One 32-wide rank tile per workgroup (grid z): a workgroup loads a
  // quarter of A at rank 128 and finishes sooner; x is read once per tile.
  const dim3 grid((unsigned)(mpad / 32), (unsigned)kchunks, (unsigned)(a.rpad32 / 32));
  if (a.rpad32 < 32 || a.rpad32 > 128) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prep_kernel<1, (int)kPrepChunk>), grid, dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  TReduceArgs tr;
  tr.tpart = tpart;
  tr.t = t;
  tr.mpad = mpad;
  tr.rpad32 = a.rpad32;
  tr.rpad16 = (int)rup(r, 16);
  tr.kchunks = kchunks;
  tr.coherent = 0;
  hipLaunchKernelGGL(treduce_kernel, dim3((unsigned)cdiv(mpad * tr.rpad16, 256)), dim3(256), 0,
                     stream, tr);
  return hipGetLastError();
}

TReduceArgs treduce_args(const LinearPlan& p, char* ws) {
  TReduceArgs tr;
  tr.tpart = reinterpret_cast<const float*>(ws + p.off_tpart);
  tr.t = reinterpret_cast<uint16_t*>(ws + p.off_t);
  tr.mpad = p.mpad;
  tr.rpad32 = p.rpad32;
  tr.rpad16 = p.rpad16;
  tr.kchunks = p.kchunks;
  tr.coherent = 0;
  return tr;
}

hipError_t launch_treduce(const LinearPlan& p, char* ws, hipStream_t stream) {
  const TReduceArgs tr = treduce_args(p, ws);
  hipLaunchKernelGGL(treduce_kernel, dim3((unsigned)cdiv(p.mpad * p.rpad16, 256)), dim3(256), 0,
                     stream, tr);
  return hipGetLastError();
}

hipError_t launch_linear_prepare(const LinearPlan& p, const uint16_t* x,
                                 const float* z, const uint16_t* lora_a,
                                 float lora_scale, char* ws,
                                 hipStream_t stream, bool swiglu_input, bool write_xt,
                                 bool z_rows, bool reduce_t, unsigned* clear_sync) {
  PrepArgs a;
  a.x = x;
  a.ldx = swiglu_input ? 2 * p.k : p.k;
  a.swiglu = swiglu_input ? 1 : 0;
  a.z = z;
  a.z_ld = (z && z_rows) ? p.k : 0;
  a.a = lora_a;
  a.xt = write_xt ? reinterpret_cast<uint16_t*>(ws + p.off_xt) : nullptr;
  a.tpart = reinterpret_cast<float*>(ws + p.off_tpart);
  a.sync = clear_sync;
  a.m = p.m;
  a.mpad = p.mpad;
  a.k = p.k;
  a.r = p.r;
  a.rpad32 = p.rpad32;
  a.lora_scale = lora_scale;
  if (p.r == 0 || !lora_a) {
    if (!write_xt) return hipSuccess;
    const int64_t threads = p.mpad * p.k / 8;
    hipLaunchKernelGGL(xt_kernel, dim3((unsigned)cdiv(threads, 256)), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  // One 32-wide rank tile per workgroup (grid z); the tile-0 workgroups
  // also write x_t.
  const dim3 grid((unsigned)(p.mpad / 32), (unsigned)p.kchunks, (unsigned)(p.rpad32 / 32));
  if (p.rpad32 < 32 || p.rpad32 > 128) return hipErrorInvalidValue;
  switch (p.kchunk) {
    case 128: hipLaunchKernelGGL((prep_kernel<1, 128>), grid, dim3(256), 0, stream, a); break;
    case 256: hipLaunchKernelGGL((prep_kernel<1, 256>), grid, dim3(256), 0, stream, a); break;
    case 512: hipLaunchKernelGGL((prep_kernel<1, 512>), grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !reduce_t) return e;
  return launch_treduce(p, ws, stream);
}

}  // namespace qerl
