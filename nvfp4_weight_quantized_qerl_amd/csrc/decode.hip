// Decode contraction: y = bf16(S * x_t W0^T + t B^T) for a few rollout
// tokens (m <= 128 per launch), W0 = E2M1 codes (.) E4M3 block scales
// dequantized in registers [QeRL summary, §3.4, Eq. 6; the pages' kernel
// does the dequantization and the product "in a single fused operation"
// with no dequantized weight buffer].
//
// The layer is bound by the weight stream (0.5625 B per weight): every
// byte of codes and scales is read from HBM exactly once, with 128-bit
// loads, and turned into bf16 MFMA operands in registers.
//
// Work decomposition (one workgroup = 4 waves = one CU's share):
//   * a workgroup owns `rows` consecutive weight rows (output features) and
//     a range of 64-wide K blocks; the rows are sized so that the grid is a
//     whole number of waves of workgroups over the CUs;
//   * its 4 waves split the K range four ways, so each wave reads its own
//     slice of the noisy activations x_t straight from L2 (no LDS copy and
//     no duplicated activation traffic inside a CU), keeps accumulators for
//     all of the workgroup's rows x all m (NT x MT tiles of 32 x 32) and
//     streams the weights of its K slice;
//   * the four partial accumulators are summed through LDS, each wave
//     owning a quarter of the tiles, then the owner applies the epilogue:
//     acc * S, plus the LoRA up-projection t B^T as extra bf16 MFMA steps
//     (t = bf16(s x_t A^T) from the prepare step), round to bf16, store;
//   * when the rows of a layer are too few to fill the GPU (down
//     projections), K is also split across workgroups: each writes fp32
//     partials, and the last workgroup of a row group to arrive (counted
//     with an atomic) sums them in split order -- deterministic -- and
//     runs the epilogue.  No workgroup ever waits for another.
//
// K layout inside a 64-wide block: lane (h = lane/32) of an MFMA holds
// k = k0 + 32h + 8j + 0..7 at step j = 0..3, for both operands, so every
// lane reads 16 contiguous bytes of codes per row and 64 contiguous bytes
// of x_t per token row (the dot product does not depend on which lane
// carries which k, only that A and B agree).
#include <algorithm>

#include "qerl_device.h"
#include "qerl_internal.h"

namespace qerl {
namespace {

struct DecodeArgs {
  const uint16_t* xt;      // [MT*32, k] bf16 rows of this m chunk
  const uint8_t* codes;    // [n, k/2]
  const uint8_t* scales;   // [n, k/16]
  const float* gscale;
  const uint16_t* t;       // [MT*32, rpad16] bf16 (s x_t A^T) or null
  const uint16_t* lora_b;  // [n, r] bf16
  uint16_t* y;             // [m_valid, n] rows of this m chunk
  float* ypart;            // [split, MT*32, n] fp32 partials
  uint32_t* cnt;           // [groups] arrival counters (zero on entry)
  int64_t n, k;
  int64_t units_per_split; // 64-wide K blocks per split
  int64_t nfull;           // full 64-wide K blocks
  int tail_steps;          // 16-wide steps in the last partial block
  int m_valid, rows, split, r, rpad16, lora_vec;
};

__device__ __forceinline__ uint32_t comp(const uint4& v, int j) {
  return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
}

// Eight LoRA B values B[row][j0 .. j0+7] (zero past r) as a bf16 MFMA operand.
__device__ __forceinline__ uint4 load_lora_b(const DecodeArgs& a, int64_t row,
                                             bool live, int j0) {
  if (!live || j0 >= a.r) return make_uint4(0u, 0u, 0u, 0u);
  const uint16_t* src = a.lora_b + row * a.r + j0;
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

// acc (already the full K sum of one 32x32 tile) -> S * acc + LoRA -> y.
__device__ __forceinline__ void epilogue_tile(const DecodeArgs& a,
                                              f32x16_t acc, float S, int u,
                                              int64_t row, bool live,
                                              int lane) {
  const int h = lane >> 5, c = lane & 31;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] *= S;
  if (a.r > 0) {
    const uint16_t* trow = a.t + (int64_t)(32 * u + c) * a.rpad16;
    for (int j0 = 0; j0 < a.rpad16; j0 += 16) {
      const uint4 tv = *reinterpret_cast<const uint4*>(trow + j0 + 8 * h);
      const uint4 bv = load_lora_b(a, row, live, j0 + 8 * h);
      acc = mfma_bf16(tv, bv, acc);
    }
  }
  if (!live) return;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int mrow = 32 * u + acc_row(v, lane);
    if (mrow < a.m_valid) a.y[(int64_t)mrow * a.n + row] = f32_to_bf16_bits(acc[v]);
  }
}

template <int MT, int NT>
__global__ __launch_bounds__(256, 1) void decode_main(DecodeArgs a) {
  constexpr int NP = MT * NT;
  constexpr int ROUNDS = (NP + 3) / 4;
  __shared__ float red[12 * 16 * 64];
  __shared__ int is_last;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, c = lane & 31;
  const int64_t row0 = (int64_t)blockIdx.x * a.rows;
  const int64_t row_end = min(a.n, row0 + (int64_t)a.rows);
  const int split_id = blockIdx.y;
  const int64_t units = a.nfull + (a.tail_steps ? 1 : 0);
  const int64_t ub = (int64_t)split_id * a.units_per_split;
  const int64_t ue = min(units, ub + a.units_per_split);
  const int64_t q = (ue - ub + 3) / 4;
  const int64_t wb = ub + wave * q;
  const int64_t we = min(ue, wb + q);

  const int64_t kbytes = a.k / 2, kscales = a.k / 16;
  const uint8_t* crow[NT];
  const uint8_t* srow[NT];
  bool live[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int64_t row = row0 + 32 * t + c;
    live[t] = row < row_end;
    const int64_t safe = live[t] ? row : row0;
    crow[t] = a.codes + safe * kbytes + 16 * h;
    srow[t] = a.scales + safe * kscales + 2 * h;
  }
  const uint16_t* xrow = a.xt + (int64_t)c * a.k + 32 * h;

  f32x16_t acc[NT][MT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int u = 0; u < MT; ++u) acc[t][u] = zero16();

  auto load = [&](int64_t kb, uint4 (&cw)[NT], uint32_t (&sw)[NT],
                  uint4 (&xa)[MT][4]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      cw[t] = live[t] ? *reinterpret_cast<const uint4*>(crow[t] + kb * 32)
                      : make_uint4(0u, 0u, 0u, 0u);
      sw[t] = live[t] ? (uint32_t)*reinterpret_cast<const uint16_t*>(srow[t] + kb * 4)
                      : 0u;
    }
#pragma unroll
    for (int u = 0; u < MT; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xa[u][i] = *reinterpret_cast<const uint4*>(xrow + (int64_t)32 * u * a.k +
                                                   kb * 64 + 8 * i);
  };
  auto compute = [&](const uint4 (&cw)[NT], const uint32_t (&sw)[NT],
                     const uint4 (&xa)[MT][4]) {
    float sb0[NT], sb1[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      sb0[t] = e4m3_to_f32(sw[t] & 0xffu);
      sb1[t] = e4m3_to_f32((sw[t] >> 8) & 0xffu);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint4 b = dequant8_bf16(comp(cw[t], j), j < 2 ? sb0[t] : sb1[t]);
#pragma unroll
        for (int u = 0; u < MT; ++u) acc[t][u] = mfma_bf16(xa[u][j], b, acc[t][u]);
      }
    }
  };

  const int64_t fe = min(we, a.nfull);
  if (wb < fe) {
    uint4 cwA[NT], cwB[NT];
    uint32_t swA[NT], swB[NT];
    uint4 xaA[MT][4], xaB[MT][4];
    load(wb, cwA, swA, xaA);
    for (int64_t kb = wb; kb < fe; kb += 2) {
      if (kb + 1 < fe) load(kb + 1, cwB, swB, xaB);
      compute(cwA, swA, xaA);
      if (kb + 2 < fe) load(kb + 2, cwA, swA, xaA);
      if (kb + 1 < fe) compute(cwB, swB, xaB);
    }
  }
  // The last, partial K block (k % 64 != 0) in 16-wide steps.
  if (a.tail_steps && wb <= a.nfull && a.nfull < we) {
    for (int s = 0; s < a.tail_steps; ++s) {
      const int64_t k0 = a.nfull * 64 + 16 * s;
      uint4 xs[MT];
#pragma unroll
      for (int u = 0; u < MT; ++u)
        xs[u] = *reinterpret_cast<const uint4*>(a.xt + (int64_t)(32 * u + c) * a.k + k0 + 8 * h);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        uint32_t cw = 0u, sb = 0u;
        if (live[t]) {
          const int64_t row = row0 + 32 * t + c;
          cw = *reinterpret_cast<const uint32_t*>(a.codes + row * kbytes + (k0 + 8 * h) / 2);
          sb = a.scales[row * kscales + k0 / 16];
        }
        const uint4 b = dequant8_bf16(cw, e4m3_to_f32(sb));
#pragma unroll
        for (int u = 0; u < MT; ++u) acc[t][u] = mfma_bf16(xs[u], b, acc[t][u]);
      }
    }
  }

  // Sum the four waves' partial tiles; tile p = t*MT + u belongs to wave p%4.
#pragma unroll
  for (int rnd = 0; rnd < ROUNDS; ++rnd) {
#pragma unroll
    for (int p = 4 * rnd; p < NP && p < 4 * rnd + 4; ++p) {
      const int owner = p & 3;
      if (wave != owner) {
        const int rank = wave - (wave > owner ? 1 : 0);
        float* dst = red + ((p - 4 * rnd) * 3 + rank) * 1024 + lane;
#pragma unroll
        for (int v = 0; v < 16; ++v) dst[v * 64] = acc[p / MT][p % MT][v];
      }
    }
    __syncthreads();
#pragma unroll
    for (int p = 4 * rnd; p < NP && p < 4 * rnd + 4; ++p) {
      if (wave == (p & 3)) {
#pragma unroll
        for (int rank = 0; rank < 3; ++rank) {
          const float* src = red + ((p - 4 * rnd) * 3 + rank) * 1024 + lane;
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[p / MT][p % MT][v] += src[v * 64];
        }
      }
    }
    __syncthreads();
  }

  const float S = *a.gscale;
  if (a.split == 1) {
#pragma unroll
    for (int p = 0; p < NP; ++p)
      if (wave == (p & 3))
        epilogue_tile(a, acc[p / MT][p % MT], S, p % MT, row0 + 32 * (p / MT) + c,
                      live[p / MT], lane);
    return;
  }

  const int64_t mrows = 32 * MT;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    if (wave == (p & 3) && live[p / MT]) {
      const int64_t row = row0 + 32 * (p / MT) + c;
      float* dst = a.ypart + ((int64_t)split_id * mrows + 32 * (p % MT)) * a.n + row;
#pragma unroll
      for (int v = 0; v < 16; ++v) dst[(int64_t)acc_row(v, lane) * a.n] = acc[p / MT][p % MT][v];
    }
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(a.cnt + blockIdx.x, 1u, __ATOMIC_ACQ_REL,
                                                __HIP_MEMORY_SCOPE_AGENT);
    is_last = (old == (uint32_t)(a.split - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    if (wave == (p & 3)) {
      const int64_t row = row0 + 32 * (p / MT) + c;
      f32x16_t sum = zero16();
      if (live[p / MT]) {
        for (int s = 0; s < a.split; ++s) {
          const float* src = a.ypart + ((int64_t)s * mrows + 32 * (p % MT)) * a.n + row;
#pragma unroll
          for (int v = 0; v < 16; ++v) sum[v] += src[(int64_t)acc_row(v, lane) * a.n];
        }
      }
      epilogue_tile(a, sum, S, p % MT, row, live[p / MT], lane);
    }
  }
  if (threadIdx.x == 0) a.cnt[blockIdx.x] = 0u;
}

typedef void (*DecodeKernel)(DecodeArgs);

DecodeKernel pick_decode(int mt, int nt) {
  if (mt == 1) {
    switch (nt) {
      case 1: return decode_main<1, 1>;
      case 2: return decode_main<1, 2>;
      case 3: return decode_main<1, 3>;
      case 4: return decode_main<1, 4>;
      case 5: return decode_main<1, 5>;
      case 6: return decode_main<1, 6>;
    }
  } else if (mt == 2) {
    switch (nt) {
      case 1: return decode_main<2, 1>;
      case 2: return decode_main<2, 2>;
      case 3: return decode_main<2, 3>;
      case 4: return decode_main<2, 4>;
      case 5: return decode_main<2, 5>;
    }
  } else if (mt == 4) {
    switch (nt) {
      case 1: return decode_main<4, 1>;
      case 2: return decode_main<4, 2>;
      case 3: return decode_main<4, 3>;
    }
  }
  return nullptr;
}

}  // namespace

// Runs the decode contraction over the m rows in chunks of at most
// 32 * dec_mt rows (one launch per chunk).
hipError_t run_decode_chunks(const LinearPlan& p, const uint8_t* codes,
                             const uint8_t* scales, const float* gscale,
                             const uint16_t* lora_b, uint16_t* y, char* ws,
                             hipStream_t stream) {
  DecodeArgs a;
  a.codes = codes;
  a.scales = scales;
  a.gscale = gscale;
  a.lora_b = lora_b;
  a.ypart = reinterpret_cast<float*>(ws + p.off_ypart);
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
  a.lora_vec = (a.r % 8 == 0) && ((reinterpret_cast<uintptr_t>(lora_b) & 15) == 0);
  const uint16_t* xt = reinterpret_cast<const uint16_t*>(ws + p.off_xt);
  const uint16_t* t = reinterpret_cast<const uint16_t*>(ws + p.off_t);
  int64_t m0 = 0;
  while (m0 < p.m) {
    const int64_t tiles_left = (p.mpad - m0) / 32;
    int mt = p.dec_mt;
    if (tiles_left < mt) mt = tiles_left >= 2 ? 2 : 1;
    DecodeKernel kern = pick_decode(mt, p.dec_nt);
    if (!kern) return hipErrorInvalidConfiguration;
    a.xt = xt + m0 * p.k;
    a.t = t + m0 * p.rpad16;
    a.y = y + m0 * p.n;
    a.m_valid = (int)std::min<int64_t>(32 * mt, p.m - m0);
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
                                     const uint16_t* lora_b, uint16_t* y, char* ws,
                                     hipStream_t stream) {
  return run_decode_chunks(p, codes, scales, gscale, lora_b, y, ws, stream);
}

}  // namespace qerl
