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
// the row index (chunk c of row r at c ^ ((r / 2) mod 8)).  The LDS has 64
// banks of 4 bytes and serves a 16-byte-per-lane access 16 lanes per clock;
// with 128-byte rows, lanes r and r + 1 differ in bank half and the key
// (r / 2) mod 8 separates the eight rows of each parity, so the MFMA operand
// reads (lane = row) and the dequantized-tile writes are conflict-free.
//
// Pipeline (double-buffered LDS, weight registers two steps ahead).
// Iteration i: issue the copies of A(i+1) and the code/scale loads of
// B(i+2); run the MFMAs of step i from LDS while dequantizing B(i+1) (loaded
// during step i-1) into the other buffer, a quarter beside each 16-deep
// MFMA step; wait for A(i+1); one barrier.  The barrier also makes A(i+1)
// visible (every wave waited for its own copies first).
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

  // Separate arrays per buffer: the compiler tracks direct-to-LDS copies
  // per array, and would otherwise wait for every load in flight before
  // reading the buffer that is not being filled.
  __shared__ __attribute__((aligned(16))) uint4 as0[BM * 8], as1[BM * 8];
  __shared__ __attribute__((aligned(16))) uint4 bs0[BN * 8], bs1[BN * 8];

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
  // Copy j of this wave: rows 8 cp .. 8 cp + 7 (cp = wave * A_PER_WAVE + j),
  // lane = (row, chunk position); the swizzle key ((8 cp + ar) / 2) mod 8
  // depends on the parity of cp.
  const uint32_t ar = (uint32_t)(lane >> 3);
  const uint32_t avoff_e = ar * xrow + 16u * (((uint32_t)lane & 7u) ^ ((ar >> 1) & 7u));
  const uint32_t avoff_o = ar * xrow + 16u * (((uint32_t)lane & 7u) ^ (((ar >> 1) + 4u) & 7u));

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
      dma16(ra, dst + cp * 64, ((cp & 1) ? avoff_o : avoff_e) + 8u * cp * xrow, so);
    }
  };
  // B registers: bn receives the loads of step s + 2 while bc (step s + 1)
  // is dequantized during the MFMAs of step s.
  // (The two scale bytes stay in separate registers, so that each load
  // result lives until it is used and nothing has to wait for it early.)
  uint4 bn_code[B_PER_THREAD], bc_code[B_PER_THREAD];
  uint32_t bn_s0[B_PER_THREAD], bn_s1[B_PER_THREAD], bc_s0[B_PER_THREAD], bc_s1[B_PER_THREAD];
  // Every thread issues the same number of loads (items past the tile
  // repeat the last item and are not stored), so the vmcnt waits below are
  // exact.  A buffer load that crosses the end of its range reads zeros in
  // full, so every load covers one 16-wide group (8 B of codes, 1 scale):
  // with k % 16 == 0 each is either wholly inside the tensor or wholly past
  // its end (the last row's partial last step).
  constexpr int B_LOADS = 4 * B_PER_THREAD;        // vector loads per thread per step
  auto load_b = [&](int step) __attribute__((always_inline)) {
    const uint32_t so_c = koff(step, 32u), so_s = koff(step, 4u);
#pragma unroll
    for (int i = 0; i < B_PER_THREAD; ++i) {
      const int item = min(tid + i * THREADS, B_ITEMS - 1);
      const int row = item >> 1, half = item & 1;
      const uint32_t vc = (uint32_t)row * kbytes + 16u * half;
      const uint32_t vs = (uint32_t)row * kscales + 2u * half;
      const uint2 c0 = bload64(rw, vc, so_c), c1 = bload64(rw, vc + 8u, so_c);
      bn_code[i] = make_uint4(c0.x, c0.y, c1.x, c1.y);
      bn_s0[i] = bload8(rs, vs, so_s);
      bn_s1[i] = bload8(rs, vs + 1u, so_s);
    }
  };
  // Dequantize chunk q (8 codes = one 16-byte LDS chunk) of every item of
  // bc (step `step`) into dst.  Scales of 16-wide groups at or past k are
  // zeroed (their codes may be the next row's), so a partial last step
  // contributes nothing there.
  auto store_b_chunk = [&](int step, uint4* dst, int q) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < B_PER_THREAD; ++i) {
      const int item = tid + i * THREADS;
      if (B_ITEMS % THREADS == 0 || item < B_ITEMS) {
        const int row = item >> 1, half = item & 1;
        const int g = step * 4 + 2 * half + (q >> 1);     // 16-wide group
        const uint32_t sbyte = q < 2 ? bc_s0[i] : bc_s1[i];
        const float sb = 16 * (int64_t)g < a.k ? e4m3_to_f32(sbyte) : 0.0f;
        const uint32_t cw = q == 0 ? bc_code[i].x
                            : (q == 1 ? bc_code[i].y : (q == 2 ? bc_code[i].z : bc_code[i].w));
        dst[row * 8 + ((4 * half + q) ^ ((row >> 1) & 7))] = dequant8_bf16(cw, sb);
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
  // hoisting all four steps' reads, which would spill.  Chunk kk of the
  // next step's weight tile is dequantized beside the MFMAs of step kk.
  auto read_frags = [&](const uint4* as, const uint4* bs, int kk, uint4 (&af)[MT],
                        uint4 (&bf)[NW]) __attribute__((always_inline)) {
    const int ch = 2 * kk + h;
#pragma unroll
    for (int u = 0; u < MT; ++u) {
      const int r = wm * WM + 32 * u + c;
      af[u] = as[r * 8 + (ch ^ ((r >> 1) & 7))];
    }
#pragma unroll
    for (int t = 0; t < NW; ++t) {
      const int r = wn * WN + 32 * t + c;
      bf[t] = bs[r * 8 + (ch ^ ((r >> 1) & 7))];
    }
  };
  auto compute = [&](const uint4* as, const uint4* bs, int next_step,
                     uint4* bs_next) __attribute__((always_inline)) {
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
      store_b_chunk(next_step, bs_next, kk);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Prologue: step 0 into buffer 0, the loads of step 1 in flight.
  copy_a(0, as0);
  load_b(0);
  __builtin_amdgcn_s_waitcnt(0x0f70);             // vmcnt(0)
#pragma unroll
  for (int i = 0; i < B_PER_THREAD; ++i) {
    bc_code[i] = bn_code[i];
    bc_s0[i] = bn_s0[i];
    bc_s1[i] = bn_s1[i];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) store_b_chunk(0, bs0, q);
  if (nsteps > 1) load_b(1);
  __syncthreads();

  // Step S: wait for B(S+1) (loaded one step ago), move it to bc, issue
  // A(S+1) and B(S+2), run the MFMAs of S while dequantizing B(S+1) into the
  // other buffer, wait for A(S+1) (B(S+2) may stay in flight), barrier.  On
  // the last step the dequantized tile is stale and never read.  Buffers
  // are named at compile time (two steps per loop iteration, the odd first
  // step peeled) and no iteration leaves early, so the accumulators keep
  // their registers.
#define QERL_PF_STEP(S, ACUR, BCUR, ANXT, BNXT)                                  \
  {                                                                             \
    __builtin_amdgcn_s_waitcnt(0x0f70);                                         \
    _Pragma("unroll") for (int i = 0; i < B_PER_THREAD; ++i) {                  \
      bc_code[i] = bn_code[i];                                                  \
      bc_s0[i] = bn_s0[i];                                                      \
      bc_s1[i] = bn_s1[i];                                                      \
    }                                                                           \
    if ((S) + 1 < nsteps) copy_a((S) + 1, ANXT);                                \
    if ((S) + 2 < nsteps) load_b((S) + 2);                                      \
    compute(ACUR, BCUR, (S) + 1, BNXT);                                         \
    if ((S) + 2 < nsteps)                                                       \
      __builtin_amdgcn_s_waitcnt((B_LOADS & 15) | ((B_LOADS >> 4) << 14) | 0x0f70); \
    else                                                                        \
      __builtin_amdgcn_s_waitcnt(0x0f70);                                       \
    __syncthreads();                                                            \
  }
  if (nsteps & 1) {
    QERL_PF_STEP(0, as0, bs0, as1, bs1)
    for (int step = 1; step < nsteps; step += 2) {
      QERL_PF_STEP(step, as1, bs1, as0, bs0)
      QERL_PF_STEP(step + 1, as0, bs0, as1, bs1)
    }
  } else {
    for (int step = 0; step < nsteps; step += 2) {
      QERL_PF_STEP(step, as0, bs0, as1, bs1)
      QERL_PF_STEP(step + 1, as1, bs1, as0, bs0)
    }
  }
#undef QERL_PF_STEP

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
