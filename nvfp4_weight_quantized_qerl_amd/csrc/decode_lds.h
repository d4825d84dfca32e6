// Decode contraction, LDS-staged variant (template; instantiated by
// decode_lds_mt*.hip).  Same operation as decode_kernel.h:
//     y = bf16(S * x_t W0^T + t B^T),  W0 = E2M1 codes (.) E4M3 scales
// [QeRL summary, §3.4, Eq. 6 (NVFP4 dequantization) and Eq. 2 (LoRA)],
// for m <= 64 tokens and k a multiple of 256.
//
// Memory path.  A workgroup owns `rows` weight rows and a range of
// 256-wide K blocks.  Each block is copied global -> LDS by direct-to-LDS
// buffer loads that the four waves issue together:
//   codes   8 rows x 128 B per instruction (one cache line per row)
//   scales  64 rows x 16 B per instruction
//   x_t     2 rows x 512 B per instruction
// so every load instruction touches few cache lines.  Inside a row the
// 16-byte chunks are stored XOR-swizzled by the row index: chunk q of code
// row r (128 B) at q ^ ((r / 2) mod 8), chunk q of x_t row r (512 B) at
// q ^ (r mod 16).  The LDS has 64 banks of 4 bytes and serves 16-byte
// accesses 16 lanes per clock; with these keys the MFMA-layout reads
// (lane = row) of 16 consecutive rows hit 16 different bank groups.
//
// Pipeline.  Codes and scales are triple-buffered, x_t double-buffered.
// Iteration i: the four copying waves wait for their copies of block i
// (s_waitcnt with the weight copies of block i+1 still in flight),
// s_barrier (now every copy of block i has landed and every wave has
// finished block i-1), the copying waves issue the copies of x_t(i+1) and
// weights(i+2) into the stages block i-1 used, then block i is computed.
// The raw s_barrier is used instead of __syncthreads, whose memory fence
// would wait for every copy in flight.  The wait's count (the W_PER_WAVE
// weight copies of block i+1 may be outstanding) needs the x_t copies of a
// block issued before its weight copies; scheduling barriers keep them so.
//
// Waves.  Eight waves, two per SIMD so that one wave's LDS and VALU
// latencies are covered by the other's MFMAs: wave w takes K quarter w % 4
// of every block and row half w / 4 of the workgroup's weight subtiles.
#pragma once

#include <type_traits>

#include "qerl_device.h"
#include "treduce.h"

namespace qerl {
namespace dlds {

struct Args {
  const uint16_t* xt;      // [MT*32, k] bf16 rows of this m chunk
  const uint8_t* codes;    // [n, k/2]
  const uint8_t* scales;   // [n, k/16]
  const float* gscale;
  const uint16_t* t;       // [MT*32, rpad16] bf16 s x_t A^T, or null
  const uint16_t* lora_b;  // [n, r] bf16
  uint16_t* y;             // [m_valid, n]
  float* ypart;            // [split, MT*32, n] fp32 partials
  int64_t n, k;
  int64_t nblocks;           // 256-wide K blocks (k / 256), spread evenly over the splits
  int m_valid, rows, split, r, rpad16, lora_vec;
  // Grid: groups * split contraction workgroups (workgroup g + groups * s
  // owns row group g and K split s), then tr_wgs workgroups that sum the
  // LoRA-down partials into t (split > 1 only: the finish reads t).
  int groups, tr_wgs;
  TReduceArgs tr;
  // Unsplit with tr_wgs > 0: the reduction workgroups come first in the
  // grid instead (workgroup tr_wgs + g owns row group g), store t at device
  // scope and count themselves in tsync[0] (zero at launch); after the main
  // loop the contraction workgroups wait for the count and load t.  tsync[1]
  // is set if that wait gave up.  Null otherwise.
  unsigned* tsync;
};

// A wait for t gives up after this many polls (about a second); the output
// is then undefined and tsync[1] is set.
constexpr uint32_t kTWaitLimit = 1u << 20;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 16 bytes per lane global -> LDS; lane l's data lands at dst + 16 l.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* dst, uint32_t voff,
                                      uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)dst, 16, (int)voff, (int)soff, 0, 0);
}

// s_waitcnt vmcnt(N) (gfx9 encoding; expcnt and lgkmcnt left free).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
}

__device__ __forceinline__ void barrier_nofence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t comp(const uint4& v, int j) {
  return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
}

__device__ __forceinline__ uint4 load_lora_b(const Args& a, int64_t row, bool live, int j0) {
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

// acc (full K sum of one 32x32 tile) -> S * acc + t B^T -> y.  row: the
// weight row (output column) of this lane; row_end: end of the workgroup's
// rows.  A tile with all 32 columns and all 32 token rows in range goes out
// through the wave's LDS scratch (2 KB): written in the MFMA layout, read
// back as 32 B of one token row per lane, stored with 16-byte stores.
__device__ __forceinline__ void epilogue_tile(const Args& a, f32x16_t acc, float S, int u,
                                              int64_t row, bool live, int lane,
                                              const uint16_t* t_lds, int64_t row_end,
                                              uint16_t* scratch, bool b_pre, uint4 b0,
                                              uint4 b1) {
  const int h = lane >> 5, c = lane & 31;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] *= S;
  if (a.r > 0) {
    const uint16_t* trow = t_lds + (32 * u + c) * a.rpad16;
    if (b_pre) {
      // r <= 32, B loaded ahead (b1 is zero when r <= 16).  The operands come
      // by value: an array whose address is taken would live in scratch.
      acc = mfma_bf16(*reinterpret_cast<const uint4*>(trow + 8 * h), b0, acc);
      if (a.rpad16 > 16)
        acc = mfma_bf16(*reinterpret_cast<const uint4*>(trow + 16 + 8 * h), b1, acc);
    } else {
      for (int j0 = 0; j0 < a.rpad16; j0 += 16) {
        const uint4 tv = *reinterpret_cast<const uint4*>(trow + j0 + 8 * h);
        const uint4 bv = load_lora_b(a, row, live, j0 + 8 * h);
        acc = mfma_bf16(tv, bv, acc);
      }
    }
  }
  const int64_t col0 = row - c;                    // first column of the tile
  if (col0 + 32 <= row_end && 32 * u + 32 <= a.m_valid && a.n % 8 == 0 &&
      (reinterpret_cast<uintptr_t>(a.y) & 15) == 0) {
#pragma unroll
    for (int v = 0; v < 16; ++v) scratch[acc_row(v, lane) * 32 + c] = f32_to_bf16_bits(acc[v]);
    // The same wave reads its own writes back: LDS operations of one wave
    // complete in order.
    const int r = lane >> 1, half = lane & 1;
    const uint4 lo = *reinterpret_cast<const uint4*>(scratch + r * 32 + 16 * half);
    const uint4 hi = *reinterpret_cast<const uint4*>(scratch + r * 32 + 16 * half + 8);
    uint16_t* dst = a.y + (int64_t)(32 * u + r) * a.n + col0 + 16 * half;
    *reinterpret_cast<uint4*>(dst) = lo;
    *reinterpret_cast<uint4*>(dst + 8) = hi;
    return;
  }
  if (!live) return;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int mrow = 32 * u + acc_row(v, lane);
    if (mrow < a.m_valid) a.y[(int64_t)mrow * a.n + row] = f32_to_bf16_bits(acc[v]);
  }
}

// P2: every block scale is a power of two (an MXFP4 weight in the NVFP4
// layout), so one v_cvt_scalef32_pk_bf16_fp4 turns two codes straight into
// their exact bf16 products with the scale; otherwise the general route.
template <int MT, int NT, bool P2 = false>
__global__ __launch_bounds__(512, 1) void decode_lds(Args a) {
  constexpr int XROWS = 32 * MT;              // token rows
  constexpr int WROWS = 32 * NT;              // weight rows staged per block
  constexpr int NT0 = (NT + 1) / 2;           // weight subtiles of row half 0
  constexpr int NT1 = NT - NT0;               // ... and of row half 1
  constexpr int CODE_INSTR = WROWS / 8;       // 8 rows per code copy
  constexpr int XINSTR = XROWS / 2;           // 2 rows per x_t copy
  constexpr int W_PER_WAVE = CODE_INSTR / 4 + 1;   // code copies + one scale copy
  static_assert(CODE_INSTR % 4 == 0 && XINSTR % 4 == 0, "copies split evenly over 4 waves");
  // Reduction slices of 16 x 64 floats live in the two x_t stages after the
  // main loop: 8 * MT slices, half per row half, 3 per reduced tile.
  constexpr int SPH = 4 * MT;                 // slices per row half
  constexpr int TPR = SPH / 3;                // tiles reduced per round and half
  constexpr int ROUNDS = (NT0 * MT + TPR - 1) / TPR;

  __shared__ __attribute__((aligned(16))) uint4 wc0[WROWS * 8], wc1[WROWS * 8], wc2[WROWS * 8];
  __shared__ __attribute__((aligned(16))) uint4 sc0[256], sc1[256], sc2[256];
  __shared__ __attribute__((aligned(16))) uint4 xs0[XROWS * 32], xs1[XROWS * 32];
  __shared__ __attribute__((aligned(16))) uint16_t t_lds[XROWS * 128];

  int bid = __builtin_amdgcn_readfirstlane((int)blockIdx.x);
  if (a.tsync) {
    if (bid < a.tr_wgs) {
      treduce_strided(a.tr, (int64_t)bid * 512 + threadIdx.x, (int64_t)a.tr_wgs * 512);
      // every wave's t stores have completed before the count goes up
      wait_vmcnt<0>();
      __syncthreads();
      if (threadIdx.x == 0)
        __hip_atomic_fetch_add(a.tsync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    bid -= a.tr_wgs;
  } else if (bid >= a.groups * a.split) {
    treduce_strided(a.tr, (int64_t)(bid - a.groups * a.split) * 512 + threadIdx.x,
                    (int64_t)a.tr_wgs * 512);
    return;
  }
  const int lane = threadIdx.x & 63;
  // Wave-uniform values the compiler cannot prove uniform by itself.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = wave & 3;                     // K quarter of every block
  const int hf = wave >> 2;                   // row half: subtiles [0, NT0) or [NT0, NT)
  const int tbase = hf ? NT0 : 0;
  const int h = lane >> 5, c = lane & 31;
  const int split_id = bid / a.groups;
  const int64_t row0 = (int64_t)(bid - split_id * a.groups) * a.rows;
  const int64_t row_end = min(a.n, row0 + (int64_t)a.rows);
  // Blocks [bb, be) of this split: the splits differ by at most one block.
  const int64_t bb = (int64_t)split_id * a.nblocks / a.split;
  const int64_t be = (int64_t)(split_id + 1) * a.nblocks / a.split;

  const float S = *a.gscale;     // first needed in the epilogue
  // t is read only by the unsplit epilogue (with K split the finishing
  // kernel adds t B^T, and t may still be being summed by this launch's
  // reduction workgroups; with tsync it is loaded after the main loop).
  if (a.r > 0 && a.split == 1 && !a.tsync) {
    const int words = XROWS * a.rpad16 / 8;
    for (int i = threadIdx.x; i < words; i += 512)
      reinterpret_cast<uint4*>(t_lds)[i] = reinterpret_cast<const uint4*>(a.t)[i];
  }

  const uint32_t kbytes = (uint32_t)(a.k / 2), kscales = (uint32_t)(a.k / 16);
  const uint32_t xrow = (uint32_t)a.k * 2;
  const __amdgpu_buffer_rsrc_t rw = rsrc(a.codes + row0 * kbytes, (uint32_t)((a.n - row0) * kbytes));
  // The scale copies cover 256 rows per block (64 per wave); only the
  // WROWS rows of this workgroup are in range, so the others read zeros
  // without fetching the next workgroups' scales.
  const __amdgpu_buffer_rsrc_t rs =
      rsrc(a.scales + row0 * kscales,
           (uint32_t)(min(a.n - row0, (int64_t)WROWS) * kscales));
  const __amdgpu_buffer_rsrc_t rx = rsrc(a.xt, (uint32_t)XROWS * xrow);

  // Copies are issued by waves 0..3 (see the file comment for the layout).
  // codes copy j of wave q covers rows 8 (q + 4 j) .. +7
  // (swizzle key of row r: (r / 2) mod 8 = (4 q + cr / 2) mod 8 for these rows)
  const uint32_t cr = (uint32_t)(lane >> 3);
  const uint32_t vcode = (8u * q + cr) * kbytes +
                         16u * ((uint32_t)(lane & 7) ^ ((4u * (uint32_t)q + (cr >> 1)) & 7u));
  // scales copy of wave q covers rows 64 q .. +63
  const uint32_t vscale = (64u * q + lane) * kscales;
  // x_t copy j of wave q covers rows 2 (q + 4 j) and 2 (q + 4 j) + 1
  // (swizzle key of row r: r mod 16 = (xr + 8 (j mod 2)) mod 16)
  const uint32_t xr = 2u * q + (uint32_t)(lane >> 5);
  const uint32_t vx_e = xr * xrow + 16u * ((uint32_t)(lane & 31) ^ (xr & 15u));
  const uint32_t vx_o = xr * xrow + 16u * ((uint32_t)(lane & 31) ^ ((xr + 8u) & 15u));

  auto copy_w = [&](int64_t blk, uint4* wc, uint4* sc) {
#pragma unroll
    for (int j = 0; j < CODE_INSTR / 4; ++j)
      // The row offset stays in the per-lane offset, which the buffer range
      // check covers: rows past the end of the tensor read as zeros.
      dma16(rw, wc + (q + 4 * j) * 64, vcode + 32u * j * kbytes, 128u * (uint32_t)blk);
    dma16(rs, sc + q * 64, vscale, 16u * (uint32_t)blk);
  };
  auto copy_x = [&](int64_t blk, uint4* xs) {
#pragma unroll
    for (int j = 0; j < XINSTR / 4; ++j)
      dma16(rx, xs + (q + 4 * j) * 64, (j & 1) ? vx_o : vx_e, 8u * j * xrow + 512u * (uint32_t)blk);
  };

  f32x16_t acc[NT0][MT];
#pragma unroll
  for (int t = 0; t < NT0; ++t)
#pragma unroll
    for (int u = 0; u < MT; ++u) acc[t][u] = zero16();

  // This wave computes K quarter q of the block for NTH weight subtiles
  // starting at TB.
  auto compute = [&](auto nth, int TB, const uint4* wc, const uint4* sc,
                     const uint4* xs) __attribute__((always_inline)) {
    constexpr int NTH = decltype(nth)::value;
    uint4 w[NTH > 0 ? NTH : 1];
    float sb0[NTH > 0 ? NTH : 1], sb1[NTH > 0 ? NTH : 1];
    uint4 xa[4][MT];
#pragma unroll
    for (int t = 0; t < NTH; ++t) {
      const int r = 32 * (TB + t) + c;
      w[t] = wc[r * 8 + ((2 * q + h) ^ ((r >> 1) & 7))];
      const uint32_t sw = reinterpret_cast<const uint16_t*>(sc)[r * 8 + 2 * q + h];
      sb0[t] = e4m3_to_f32(sw & 0xffu);
      sb1[t] = e4m3_to_f32((sw >> 8) & 0xffu);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int u = 0; u < MT; ++u) {
        const int r = 32 * u + c;
        xa[j][u] = xs[r * 32 + ((8 * q + 4 * h + j) ^ (r & 15))];
      }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int t = 0; t < NTH; ++t) {
        const uint4 b = P2 ? dequant8_bf16_pow2(comp(w[t], j), j < 2 ? sb0[t] : sb1[t])
                           : dequant8_bf16(comp(w[t], j), j < 2 ? sb0[t] : sb1[t]);
#pragma unroll
        for (int u = 0; u < MT; ++u) acc[t][u] = mfma_bf16(xa[j][u], b, acc[t][u]);
      }
    }
  };
  auto compute_half = [&](const uint4* wc, const uint4* sc,
                          const uint4* xs) __attribute__((always_inline)) {
    if (hf == 0)
      compute(std::integral_constant<int, NT0>{}, 0, wc, sc, xs);
    else
      compute(std::integral_constant<int, NT1>{}, NT0, wc, sc, xs);
  };

  if (bb < be) {
    const int64_t last = be - 1;
    if (hf == 0) {
      copy_w(bb, wc0, sc0);
      __builtin_amdgcn_sched_barrier(0);
      copy_x(bb, xs0);
      __builtin_amdgcn_sched_barrier(0);
      copy_w(min(bb + 1, last), wc1, sc1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Block bb + i uses weight stage i % 3 and x_t stage i % 2; period 6.
#define QERL_LDS_STEP(OFF, WC, SC, XS, XN, WN, SN)                         \
  if (hf == 0) wait_vmcnt<W_PER_WAVE>();                                    \
  barrier_nofence();                                                        \
  if (hf == 0) {                                                            \
    copy_x(min(blk + (OFF) + 1, last), XN);                                 \
    __builtin_amdgcn_sched_barrier(0);                                      \
    copy_w(min(blk + (OFF) + 2, last), WN, SN);                             \
    __builtin_amdgcn_sched_barrier(0);                                      \
  }                                                                         \
  compute_half(WC, SC, XS);                                                 \
  if (blk + (OFF) + 1 >= be) break;
    for (int64_t blk = bb;; blk += 6) {
      QERL_LDS_STEP(0, wc0, sc0, xs0, xs1, wc2, sc2)
      QERL_LDS_STEP(1, wc1, sc1, xs1, xs0, wc0, sc0)
      QERL_LDS_STEP(2, wc2, sc2, xs0, xs1, wc1, sc1)
      QERL_LDS_STEP(3, wc0, sc0, xs1, xs0, wc2, sc2)
      QERL_LDS_STEP(4, wc1, sc1, xs0, xs1, wc0, sc0)
      QERL_LDS_STEP(5, wc2, sc2, xs1, xs0, wc1, sc1)
    }
#undef QERL_LDS_STEP
  }
  // Every copy has landed and every wave is done with the stages.
  wait_vmcnt<0>();
  barrier_nofence();
  if (a.tsync) {
    // t comes from this launch's first workgroups (dispatched before this
    // one, so the wait ends); loaded at device scope (aux 16: sc1).  The
    // reduction rounds below end with barriers, so t_lds is complete before
    // the epilogue reads it.
    if (threadIdx.x == 0) {
      for (uint32_t it = 0;
           __hip_atomic_load(a.tsync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
           (unsigned)a.tr_wgs;
           ++it) {
        if (it >= kTWaitLimit) {
          __hip_atomic_store(a.tsync + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    __syncthreads();
    if (a.r > 0) {
      const int words = XROWS * a.rpad16 / 8;
      const __amdgpu_buffer_rsrc_t rt = rsrc(a.t, (uint32_t)(words * 16));
      for (int i = threadIdx.x; i < words; i += 512)
        reinterpret_cast<uint4*>(t_lds)[i] =
            __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rt, 16 * i, 0, 16));
    }
  }

  // Sum the four K quarters of each row half through the (now free) x_t
  // stages.  Half hf uses slices [hf * SPH, (hf + 1) * SPH); per round TPR
  // tiles of the half are reduced, tile p by wave q == p % TPR.
  auto slice = [&](int s) -> float* {
    return s < 4 * MT ? reinterpret_cast<float*>(xs0) + s * 1024
                      : reinterpret_cast<float*>(xs1) + (s - 4 * MT) * 1024;
  };
  const int ntile = (hf ? NT1 : NT0) * MT;
  auto owns = [&](int p) { return p < ntile && q == p % TPR; };
  auto tile_row = [&](int p) { return row0 + 32 * (tbase + p / MT) + c; };
  auto tile_live = [&](int p) { return tile_row(p) < row_end; };

  // LoRA B operands of the owned output tiles (r <= 32: two 16-wide
  // steps), loaded before the cross-wave reduction so that their latency
  // passes during it.  Wave q owns tiles q, q + TPR, ...: tile p's operands
  // go to slot p / TPR.
  constexpr int NOWN = (NT0 * MT + TPR - 1) / TPR;
  uint4 bpre[NOWN][2];
  const bool b_pre = a.split == 1 && a.r > 0 && a.rpad16 <= 32;
  if (b_pre) {
#pragma unroll
    for (int p = 0; p < NT0 * MT; ++p) {
      if (owns(p)) {
        bpre[p / TPR][0] = load_lora_b(a, tile_row(p), tile_live(p), 8 * h);
        bpre[p / TPR][1] = a.rpad16 > 16 ? load_lora_b(a, tile_row(p), tile_live(p), 16 + 8 * h)
                                         : make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }

#pragma unroll
  for (int rnd = 0; rnd < ROUNDS; ++rnd) {
#pragma unroll
    for (int p = TPR * rnd; p < NT0 * MT && p < TPR * rnd + TPR; ++p) {
      const int owner = p - TPR * rnd;
      if (p < ntile && q != owner) {
        const int rank = q - (q > owner ? 1 : 0);
        float* dst = slice(hf * SPH + owner * 3 + rank) + lane;
#pragma unroll
        for (int v = 0; v < 16; ++v) dst[v * 64] = acc[p / MT][p % MT][v];
      }
    }
    __syncthreads();
#pragma unroll
    for (int p = TPR * rnd; p < NT0 * MT && p < TPR * rnd + TPR; ++p) {
      const int owner = p - TPR * rnd;
      if (p < ntile && q == owner) {
#pragma unroll
        for (int rank = 0; rank < 3; ++rank) {
          const float* src = slice(hf * SPH + owner * 3 + rank) + lane;
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[p / MT][p % MT][v] += src[v * 64];
        }
      }
    }
    __syncthreads();
  }
  if (a.split == 1) {
    // Every slice is free after the last round; wave (q, hf) takes slice
    // hf * SPH + q (q < 4 <= SPH) as its transpose scratch.
    uint16_t* scratch = reinterpret_cast<uint16_t*>(slice(hf * SPH + q));
#pragma unroll
    for (int p = 0; p < NT0 * MT; ++p)
      if (owns(p))
        epilogue_tile(a, acc[p / MT][p % MT], S, p % MT, tile_row(p), tile_live(p), lane, t_lds,
                      row_end, scratch, b_pre, bpre[p / TPR][0], bpre[p / TPR][1]);
    return;
  }

  // Split K: this workgroup's fp32 partial tiles; the finishing kernel
  // sums the splits and applies the epilogue.
#pragma unroll
  for (int p = 0; p < NT0 * MT; ++p) {
    if (owns(p) && tile_live(p)) {
      float* dst = a.ypart + ((int64_t)split_id * XROWS + 32 * (p % MT)) * a.n + tile_row(p);
#pragma unroll
      for (int v = 0; v < 16; ++v) dst[(int64_t)acc_row(v, lane) * a.n] = acc[p / MT][p % MT][v];
    }
  }
}

typedef void (*Kernel)(Args);

template <int MT, bool P2 = false>
Kernel pick_nt(int nt) {
  switch (nt) {
    case 1: return decode_lds<MT, 1, P2>;
    case 2: return decode_lds<MT, 2, P2>;
    case 3: return decode_lds<MT, 3, P2>;
    case 4: return decode_lds<MT, 4, P2>;
    case 5: return decode_lds<MT, 5, P2>;
    default: return nullptr;
  }
}

Kernel pick_mt1(int nt, bool p2);
Kernel pick_mt2(int nt, bool p2);

}  // namespace dlds
}  // namespace qerl
