// Prefill contraction kernel (template; instantiated by prefill.hip):
//     y = bf16(S * x_t W0^T + t B^T),  W0 = E2M1 codes (.) E4M3 block scales
// for many tokens [QeRL summary, §3.4, Eq. 6 (NVFP4 dequantization, S
// applied to the fp32 accumulator) and Eq. 2 (LoRA side branch, t =
// bf16(s x_t A^T) from the prepare step)].  This is a dense contraction, so
// it runs as a bf16 MFMA GEMM whose weight tiles are dequantized into LDS;
// no dequantized weight tensor ever exists in HBM.
//
// Tiling.  A workgroup of WGM x WGN waves owns a BM x BN output tile (BM =
// WGM * WM token rows, BN = WGN * WN weight rows) and walks K in steps of
// 64.  Per step:
//   A (x_t, bf16)  BM x 64 -> LDS by direct-to-LDS buffer loads, 8 rows x
//                  128 B per instruction;
//   B (NVFP4)      BN x 64 codes (32 B per row) + 4 scales per row -> VGPRs
//                  one step ahead, dequantized once per workgroup into a
//                  bf16 BN x 64 LDS tile (each 32-wide row half by one
//                  thread: 16 B of codes, two scales, four 16-byte writes).
// Both LDS tiles store the eight 16-byte chunks of a row XOR-swizzled by
// the row index (chunk c of row r at c ^ (r mod 8)), so the MFMA operand
// reads (lane = row) hit eight different bank groups per eight lanes.
//
// Pipeline (double-buffered LDS).  Iteration i: issue the copies of
// A(i+1) and the code/scale loads of B(i+1); run the MFMAs of step i from
// LDS; wait for the loads; dequantize B(i+1) into the other buffer; one
// barrier.  The barrier also makes A(i+1) visible (every wave waited for
// its own copies first).
//
// Each wave accumulates a WM x WN tile in MT x NW blocks of 32 x 32
// (v_mfma_f32_32x32x16_bf16); the epilogue scales by S, adds the LoRA-up
// with a few more MFMA steps and stores bf16.
#pragma once

#include "qerl_device.h"

namespace qerl {
namespace prefill {

struct Args {
  const uint16_t* xt;      // [mpad, k] bf16 x_t
  const uint8_t* codes;    // [n, k/2]
  const uint8_t* scales;   // [n, k/16]
  const float* gscale;
  const uint16_t* t;       // [mpad, rpad16] bf16 s x_t A^T, or null (r == 0)
  const uint16_t* lora_b;  // [n, r] bf16
  uint16_t* y;             // [m, n]
  int64_t m, mpad, n, k;
  int r, rpad16, lora_vec;
  int tiles_n;             // N tiles per M tile row of the grid
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Buffer resource over [p, p + bytes), bytes clamped to 2^32 - 1; loads
// past the end read zeros.  Both arguments must be wave-uniform; the
// readfirstlane keeps the descriptor in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint64_t bytes) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(
      (int)(bytes > 0xffffffffull ? 0xffffffffu : (uint32_t)bytes));
  void* base = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)n, 0x00020000);
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* dst, uint32_t voff,
                                      uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)dst, 16, (int)voff, (int)soff, 0, 0);
}

__device__ __forceinline__ uint4 bload128(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                          uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff,
                                                                         (int)soff, 0));
}

__device__ __forceinline__ uint2 bload64(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                         uint32_t soff) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff,
                                                                       (int)soff, 0));
}

__device__ __forceinline__ uint32_t bload8(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                           uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, (int)soff, 0);
}

// Eight LoRA B values B[row][j0 .. j0+7] (zero past r or n) as an operand.
__device__ __forceinline__ uint4 lora_b8(const Args& a, int64_t row, int j0) {
  if (row >= a.n || j0 >= a.r) return make_uint4(0u, 0u, 0u, 0u);
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

// WPE is the number of waves per SIMD the registers are planned for (the
// second launch bound): 1 gives a wave up to 512 registers (accumulators
// in AGPRs), 2 lets two workgroups of four waves share a CU when their LDS
// tiles fit (two double-buffered tiles of (BM + BN) x 128 B each).
template <int WGM, int WGN, int WM, int WN, int WPE>
__global__ __launch_bounds__(64 * WGM * WGN, WPE)
void gemm(Args a) {
  constexpr int WAVES = WGM * WGN;
  constexpr int THREADS = 64 * WAVES;
  constexpr int BM = WGM * WM, BN = WGN * WN;
  constexpr int MT = WM / 32, NW = WN / 32;
  constexpr int A_COPIES = BM / 8;                 // 1 KB copies per step
  static_assert(A_COPIES % WAVES == 0, "equal copies per wave");
  constexpr int A_PER_WAVE = A_COPIES / WAVES;
  constexpr int B_ITEMS = 2 * BN;                  // (row, 32-wide half) per step
  constexpr int B_PER_THREAD = (B_ITEMS + THREADS - 1) / THREADS;

  __shared__ __attribute__((aligned(16))) uint4 as[2][BM * 8];
  __shared__ __attribute__((aligned(16))) uint4 bs[2][BN * 8];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int h = lane >> 5, c = lane & 31;
  // Tile coordinates, kept in scalar registers (the buffer descriptors
  // built from them must be wave-uniform, or every load becomes a loop).
  const int tm = __builtin_amdgcn_readfirstlane((int)blockIdx.x / a.tiles_n);
  const int tn = __builtin_amdgcn_readfirstlane((int)blockIdx.x - tm * a.tiles_n);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int nsteps = (int)((a.k + 63) / 64);

  // A: rows m0 .. m0+BM-1 of x_t; rows past mpad read zeros.
  const uint32_t xrow = (uint32_t)(a.k * 2);
  const int64_t arows = a.mpad - m0;
  const __amdgpu_buffer_rsrc_t ra =
      rsrc(a.xt + m0 * a.k, (uint64_t)(arows > 0 ? arows : 0) * xrow);
  // Copy j of this wave: rows 8 (wave * A_PER_WAVE + j) .. +7, lane = (row, chunk).
  const uint32_t ar = (uint32_t)(lane >> 3);
  const uint32_t avoff = ar * xrow + 16u * (((uint32_t)lane & 7u) ^ ar);

  // B: rows n0 .. n0+BN-1 of the codes and scales; rows past n read zeros.
  const uint32_t kbytes = (uint32_t)(a.k / 2), kscales = (uint32_t)(a.k / 16);
  const int64_t brows = a.n - n0;
  const __amdgpu_buffer_rsrc_t rw = rsrc(a.codes + n0 * kbytes, (uint64_t)brows * kbytes);
  const __amdgpu_buffer_rsrc_t rs = rsrc(a.scales + n0 * kscales, (uint64_t)brows * kscales);

  // Uniform offsets along K go into the scalar offset operand.
  auto koff = [](int step, uint32_t bytes_per_step) __attribute__((always_inline)) {
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)(bytes_per_step * (uint32_t)step));
  };
  auto copy_a = [&](int step, uint4* dst) __attribute__((always_inline)) {
    const uint32_t so = koff(step, 128u);
#pragma unroll
    for (int j = 0; j < A_PER_WAVE; ++j) {
      const int cp = wave * A_PER_WAVE + j;
      dma16(ra, dst + cp * 64, avoff + 8u * cp * xrow, so);
    }
  };
  uint4 bcode[B_PER_THREAD];
  uint32_t bscale[B_PER_THREAD];
  // A buffer load that crosses the end of its range reads zeros in full,
  // so every load here covers one 16-wide group (8 B of codes, 1 scale):
  // with k % 16 == 0 each is either wholly inside the tensor or wholly
  // past its end (the last row's partial last step).
  auto load_b = [&](int step) __attribute__((always_inline)) {
    const uint32_t so_c = koff(step, 32u), so_s = koff(step, 4u);
#pragma unroll
    for (int i = 0; i < B_PER_THREAD; ++i) {
      const int item = tid + i * THREADS;
      const int row = item >> 1, half = item & 1;
      if (item < B_ITEMS) {
        const uint32_t vc = (uint32_t)row * kbytes + 16u * half;
        const uint32_t vs = (uint32_t)row * kscales + 2u * half;
        const uint2 c0 = bload64(rw, vc, so_c), c1 = bload64(rw, vc + 8u, so_c);
        bcode[i] = make_uint4(c0.x, c0.y, c1.x, c1.y);
        bscale[i] = bload8(rs, vs, so_s) | (bload8(rs, vs + 1u, so_s) << 8);
      }
    }
  };
  // Scales of 16-wide groups at or past k are zeroed (their codes may be
  // the next row's), so a partial last step contributes nothing there.
  auto store_b = [&](int step, uint4* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < B_PER_THREAD; ++i) {
      const int item = tid + i * THREADS;
      const int row = item >> 1, half = item & 1;
      if (item < B_ITEMS) {
        const int64_t g0 = step * 4 + 2 * half;          // first 16-wide group
        const float s0 = 16 * g0 < a.k ? e4m3_to_f32(bscale[i] & 0xffu) : 0.0f;
        const float s1 = 16 * (g0 + 1) < a.k ? e4m3_to_f32((bscale[i] >> 8) & 0xffu) : 0.0f;
        const int sw = row & 7;
        uint4* drow = dst + row * 8;
        drow[(4 * half + 0) ^ sw] = dequant8_bf16(bcode[i].x, s0);
        drow[(4 * half + 1) ^ sw] = dequant8_bf16(bcode[i].y, s0);
        drow[(4 * half + 2) ^ sw] = dequant8_bf16(bcode[i].z, s1);
        drow[(4 * half + 3) ^ sw] = dequant8_bf16(bcode[i].w, s1);
      }
    }
  };

  f32x16_t acc[MT][NW];
#pragma unroll
  for (int u = 0; u < MT; ++u)
#pragma unroll
    for (int t = 0; t < NW; ++t) acc[u][t] = zero16();

  // Operand reads run one 16-deep MFMA step ahead of the MFMAs (two sets of
  // fragments live); the scheduling barriers keep the compiler from
  // hoisting all four steps' reads, which would spill.
  auto read_frags = [&](const uint4* as, const uint4* bs, int kk, uint4 (&af)[MT],
                        uint4 (&bf)[NW]) __attribute__((always_inline)) {
    const int ch = 2 * kk + h;
#pragma unroll
    for (int u = 0; u < MT; ++u) {
      const int r = wm * WM + 32 * u + c;
      af[u] = as[r * 8 + (ch ^ (r & 7))];
    }
#pragma unroll
    for (int t = 0; t < NW; ++t) {
      const int r = wn * WN + 32 * t + c;
      bf[t] = bs[r * 8 + (ch ^ (r & 7))];
    }
  };
  auto compute = [&](const uint4* as, const uint4* bs) __attribute__((always_inline)) {
    uint4 af[2][MT], bf[2][NW];
    read_frags(as, bs, 0, af[0], bf[0]);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk < 3) read_frags(as, bs, kk + 1, af[(kk + 1) & 1], bf[(kk + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < MT; ++u)
#pragma unroll
        for (int t = 0; t < NW; ++t)
          acc[u][t] = mfma_bf16(af[kk & 1][u], bf[kk & 1][t], acc[u][t]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Prologue: step 0 into buffer 0.
  copy_a(0, as[0]);
  load_b(0);
  __builtin_amdgcn_s_waitcnt(0x0f70);             // vmcnt(0): B(0) in registers
  store_b(0, bs[0]);
  __syncthreads();

  // One K step per iteration; the buffer index alternates at run time so
  // that the accumulators stay in the same registers across iterations.
  for (int step = 0; step < nsteps; ++step) {
    const int cur = step & 1;
    const bool more = step + 1 < nsteps;
    if (more) {
      copy_a(step + 1, as[cur ^ 1]);
      load_b(step + 1);
    }
    compute(as[cur], bs[cur]);
    if (more) {
      __builtin_amdgcn_s_waitcnt(0x0f70);           // vmcnt(0): A and B of step + 1
      store_b(step + 1, bs[cur ^ 1]);
    }
    __syncthreads();
  }

  // Epilogue, one 32 x 32 block at a time (so that only one block's
  // accumulators leave the AGPRs at once): S * acc + t B^T (bf16 MFMA over
  // r), round to bf16, store.
  const float S = *a.gscale;
#pragma unroll
  for (int u = 0; u < MT; ++u) {
    const int64_t trow = m0 + wm * WM + 32 * u + c;
#pragma unroll
    for (int t = 0; t < NW; ++t) {
      const int64_t col = n0 + wn * WN + 32 * t + c;
      f32x16_t o = acc[u][t];
#pragma unroll
      for (int v = 0; v < 16; ++v) o[v] *= S;
      for (int j0 = 0; j0 < a.r; j0 += 16) {
        const uint4 tf = trow < a.mpad
                             ? *reinterpret_cast<const uint4*>(a.t + trow * a.rpad16 + j0 + 8 * h)
                             : make_uint4(0u, 0u, 0u, 0u);
        o = mfma_bf16(tf, lora_b8(a, col, j0 + 8 * h), o);
      }
      if (col < a.n) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = m0 + wm * WM + 32 * u + acc_row(v, lane);
          if (row < a.m) a.y[row * a.n + col] = f32_to_bf16_bits(o[v]);
        }
      }
    }
  }
}

}  // namespace prefill
}  // namespace qerl
