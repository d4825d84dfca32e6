// Decode contraction kernel (template; instantiated by decode_mt*.hip): y = bf16(S * x_t W0^T + t B^T) for a few rollout
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
//     projections), K is also split across workgroups: each writes its
//     fp32 partial tiles, and a separate finishing kernel sums them in
//     split order (deterministic) and applies the epilogue.  A workgroup
//     never waits for another: on gfx950 the device-scope fences an
//     in-kernel hand-off needs write back and invalidate the L2.
//
// K layout inside a 64-wide block: lane (h = lane/32) of an MFMA holds
// k = k0 + 32h + 8j + 0..7 at step j = 0..3, for both operands, so every
// lane reads 16 contiguous bytes of codes per row and 64 contiguous bytes
// of x_t per token row (the dot product does not depend on which lane
// carries which k, only that A and B agree).
#pragma once

#include "qerl_device.h"

namespace qerl {
namespace decode {

struct DecodeArgs {
  const uint16_t* xt;      // [MT*32, k] bf16 rows of this m chunk
  const uint8_t* codes;    // [n, k/2]
  const uint8_t* scales;   // [n, k/16]
  const float* gscale;
  const uint16_t* t;       // [MT*32, rpad16] bf16 s x_t A^T (precomputed) or null
  const uint16_t* lora_b;  // [n, r] bf16
  uint16_t* y;             // [m_valid, n] rows of this m chunk
  float* ypart;            // [split, MT*32, n] fp32 partials
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

// acc (the full K sum of one 32x32 tile) -> S * acc + t B^T -> y.
// t_lds holds bf16(s x_t A^T) for the chunk's rows, row stride rpad16.
__device__ __forceinline__ void epilogue_tile(const DecodeArgs& a, f32x16_t acc,
                                              float S, int u, int64_t row, bool live,
                                              int lane, const uint16_t* t_lds) {
  const int h = lane >> 5, c = lane & 31;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] *= S;
  if (a.r > 0) {
    const uint16_t* trow = t_lds + (32 * u + c) * a.rpad16;
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

// Buffer resource over [p, p + bytes): loads past the end return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 bload128(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                          uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff,
                                                                         (int)soff, 0));
}

__device__ __forceinline__ uint32_t bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                            uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0);
}

__device__ __forceinline__ uint32_t bload8(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                           uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, (int)soff, 0);
}

__device__ __forceinline__ uint32_t bload32(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                            uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}

// Activation registers of one 64-wide K block: x_t of MT token tiles.
template <int MT>
struct XStage {
  uint4 x[MT][4];
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Asynchronous copy global -> LDS of 16 bytes per lane: lane l's data lands
// at dst + 16 l.  dst must be wave-uniform.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* dst, uint32_t voff,
                                      uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)dst, 16, (int)voff, (int)soff, 0, 0);
}



// MT token tiles x NT weight subtiles of 32 x 32.
//
// Software pipeline per wave: the NVFP4 weight blocks (the HBM stream) go
// global -> LDS by direct-to-LDS buffer loads into three LDS stages (no
// register cost), and are issued two K blocks ahead of their MFMAs; the
// activation blocks (L2-resident) go to registers, one block
// ahead, in the order X(kb+1), W(kb+2), MFMA(kb).  Loads of a wave retire
// in issue order, so waiting for X(kb) never waits for W(kb+1): two weight
// blocks stay in flight while a block is computed.  Loads are never
// predicated (the block index is clamped; rows past the matrix read zeros
// through the buffer bounds), which keeps the waits a fixed distance
// behind the loads.
template <int MT, int NT>
__global__ __launch_bounds__(256, 1) void decode_main(DecodeArgs a) {
  constexpr int NA = NT;               // accumulator rows
  constexpr int NP = MT * NA;          // 32x32 tiles per wave
  constexpr int ROUNDS = (NP + 3) / 4;
  __shared__ float red[12 * 16 * 64];
  __shared__ __attribute__((aligned(16))) uint16_t t_lds[MT * 32 * 128];
  __shared__ __attribute__((aligned(16))) uint4 wl0[4 * NT * 64], wl1[4 * NT * 64],
      wl2[4 * NT * 64];

  const int lane = threadIdx.x & 63;
  // Wave-uniform (the compiler cannot see that threadIdx.x / 64 is): keeps
  // every K-block offset and LDS stage address in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
  const int mrows = 32 * MT;

  // Precomputed LoRA-down t: stage it in LDS for the epilogue.
  if (a.r > 0) {
    const int words = mrows * a.rpad16 / 8;
    for (int i = threadIdx.x; i < words; i += 256)
      reinterpret_cast<uint4*>(t_lds)[i] = reinterpret_cast<const uint4*>(a.t)[i];
  }

  const uint32_t kbytes = (uint32_t)(a.k / 2), kscales = (uint32_t)(a.k / 16);
  const uint32_t xrow_bytes = (uint32_t)a.k * 2;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.codes + row0 * kbytes,
                                              (uint32_t)((a.n - row0) * kbytes));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scales + row0 * kscales,
                                              (uint32_t)((a.n - row0) * kscales));
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.xt, (uint32_t)mrows * xrow_bytes);
  // Row offsets go into the per-lane offset, which the buffer range check
  // covers (rows past the end of a tensor read as zeros); the uniform
  // offset carries only the position along K.
  const uint32_t vw = (uint32_t)c * kbytes + 16u * h;      // + 32 t kbytes, K: + 32 kb
  const uint32_t vs = (uint32_t)c * kscales + 2u * h;      // + 32 t kscales, K: + 4 kb
  const uint32_t vx = (uint32_t)c * xrow_bytes + 64u * h;  // + 32 u row + 128 kb + 16 i
  bool live[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) live[t] = row0 + 32 * t + c < row_end;

  f32x16_t acc[NA][MT];
#pragma unroll
  for (int t = 0; t < NA; ++t)
#pragma unroll
    for (int u = 0; u < MT; ++u) acc[t][u] = zero16();

  const int wslot = wave * NT * 64;
  // Block scales (2 bytes per lane and subtile) go to registers, issued with
  // the codes of the same block.
  auto load_w = [&](int64_t kb, uint4* wl, uint32_t (&sw)[NT]) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
      sw[t] = bload16(rs, vs + 32u * t * kscales, 4u * (uint32_t)kb);
#pragma unroll
    for (int t = 0; t < NT; ++t)
      dma16(rw, wl + wslot + t * 64, vw + 32u * t * kbytes, 32u * (uint32_t)kb);
  };
  auto load_x = [&](int64_t kb, XStage<MT>& st) {
#pragma unroll
    for (int u = 0; u < MT; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        st.x[u][i] = bload128(rx, vx, 32u * u * xrow_bytes + 128u * (uint32_t)kb + 16u * i);
  };
  auto compute = [&](const uint4* wl, const uint32_t (&sw)[NT], const XStage<MT>& xs) {
    uint4 w[NT];
    float sb0[NT], sb1[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      w[t] = wl[wslot + t * 64 + lane];
      sb0[t] = e4m3_to_f32(sw[t] & 0xffu);
      sb1[t] = e4m3_to_f32((sw[t] >> 8) & 0xffu);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint4 b = dequant8_bf16(comp(w[t], j), j < 2 ? sb0[t] : sb1[t]);
#pragma unroll
        for (int u = 0; u < MT; ++u) acc[t][u] = mfma_bf16(xs.x[u][j], b, acc[t][u]);
      }
    }
  };

  const int64_t fe = min(we, a.nfull);
  if (wb < fe) {
    XStage<MT> x0, x1;
    uint32_t sl0[NT], sl1[NT], sl2[NT];
    const int64_t last = fe - 1;
    load_w(wb, wl0, sl0);
    load_x(wb, x0);
    load_w(min(wb + 1, last), wl1, sl1);
    // Block kb + i uses weight stage i % 3 (codes in LDS, scales in
    // registers) and activation stage i % 2; period 6.
    // The scheduling barriers keep each group of loads ahead of the MFMAs
    // (the scheduler would otherwise sink them into the compute, and the
    // in-order waits for them would then also wait for the weight copies).
#define QERL_DECODE_STEP(XN, WN, SN, WC, SC, XC, OFF)                 \
  __builtin_amdgcn_sched_barrier(0);                                 \
  load_x(min(kb + (OFF) + 1, last), XN);                             \
  load_w(min(kb + (OFF) + 2, last), WN, SN);                         \
  __builtin_amdgcn_sched_barrier(0);                                 \
  compute(WC, SC, XC);                                               \
  if (kb + (OFF) + 1 >= fe) break;
    for (int64_t kb = wb;; kb += 6) {
      QERL_DECODE_STEP(x1, wl2, sl2, wl0, sl0, x0, 0)
      QERL_DECODE_STEP(x0, wl0, sl0, wl1, sl1, x1, 1)
      QERL_DECODE_STEP(x1, wl1, sl1, wl2, sl2, x0, 2)
      QERL_DECODE_STEP(x0, wl2, sl2, wl0, sl0, x1, 3)
      QERL_DECODE_STEP(x1, wl0, sl0, wl1, sl1, x0, 4)
      QERL_DECODE_STEP(x0, wl1, sl1, wl2, sl2, x1, 5)
    }
#undef QERL_DECODE_STEP
    // Let the clamped tail copies land before the LDS is reused or freed.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  // The last, partial K block (k % 64 != 0) in 16-wide steps.
  if (a.tail_steps && wb <= a.nfull && a.nfull < we) {
    const uint32_t vx16 = (uint32_t)c * xrow_bytes + 16u * h;
    for (int s = 0; s < a.tail_steps; ++s) {
      const uint32_t k0 = (uint32_t)(a.nfull * 64 + 16 * s);
      uint4 xs[MT];
#pragma unroll
      for (int u = 0; u < MT; ++u) xs[u] = bload128(rx, vx16, 32u * u * xrow_bytes + 2u * k0);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint32_t cw = bload32(rw, (uint32_t)(32 * t + c) * kbytes + 4u * h, k0 / 2);
        const uint32_t sb = bload8(rs, (uint32_t)(32 * t + c) * kscales, k0 / 16);
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
    for (int p = 0; p < MT * NT; ++p)
      if (wave == (p & 3))
        epilogue_tile(a, acc[p / MT][p % MT], S, p % MT, row0 + 32 * (p / MT) + c,
                      live[p / MT], lane, t_lds);
    return;
  }
  // Split K: this workgroup's fp32 partial tiles; the finishing kernel
  // sums the splits and applies the epilogue.
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    if (wave == (p & 3) && live[p / MT]) {
      const int64_t row = row0 + 32 * (p / MT) + c;
      float* dst = a.ypart + ((int64_t)split_id * mrows + 32 * (p % MT)) * a.n + row;
#pragma unroll
      for (int v = 0; v < 16; ++v) dst[(int64_t)acc_row(v, lane) * a.n] = acc[p / MT][p % MT][v];
    }
  }
}

typedef void (*DecodeKernel)(DecodeArgs);

// decode_main<MT, NT> if it holds its accumulators and operands in
// registers without spilling (NT <= 6, 5 and 2 for MT = 1, 2 and 4, the
// limits the planner keeps to; the compiler's resource report shows scratch
// at MT = 2, NT = 6 and MT = 4, NT = 3), else null.
template <int MT, int NT>
DecodeKernel kernel_or_null() {
  if constexpr (NT >= 1 && NT <= (MT == 1 ? 6 : (MT == 2 ? 5 : 2))) {
    return decode_main<MT, NT>;
  } else {
    return nullptr;
  }
}

template <int MT>
DecodeKernel pick_mt(int nt) {
  switch (nt) {
    case 1: return kernel_or_null<MT, 1>();
    case 2: return kernel_or_null<MT, 2>();
    case 3: return kernel_or_null<MT, 3>();
    case 4: return kernel_or_null<MT, 4>();
    case 5: return kernel_or_null<MT, 5>();
    case 6: return kernel_or_null<MT, 6>();
    default: return nullptr;
  }
}

DecodeKernel pick_mt1(int nt);
DecodeKernel pick_mt2(int nt);
DecodeKernel pick_mt4(int nt);

}  // namespace decode
}  // namespace qerl
