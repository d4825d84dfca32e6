// Decode contraction for up to 128 rollout tokens in one pass over the
// weights (template; instantiated by decode_m128.hip):
//     y = bf16(S * x_t W0^T + t B^T),  W0 = E2M1 codes (.) E4M3 scales
// [QeRL summary, §3.4, Eq. 6 (NVFP4 dequantization, S applied to the fp32
// accumulator) and Eq. 2 (LoRA side branch, t = bf16(s x_t A^T) from the
// prepare step)], for k a multiple of 128.
//
// At 128 tokens every dequantized weight value feeds 128 multiply-adds, so
// the contraction is bound by the bf16 MFMA rate rather than by the weight
// stream.  The layout is chosen so that (a) each dequantized MFMA operand
// is used by four MFMAs (all 128 tokens), keeping the dequantization VALU
// work at half the MFMA time, and (b) every MFMA reads at most half a KB of
// LDS operand bytes per 32x32x16 step.
//
// Work decomposition.  A workgroup of eight waves owns 256 weight rows and
// a range of 128-wide K blocks.  Wave w takes K half kh = w / 4 of every
// block (64 channels, four 16-deep MFMA steps) and row group rg = w % 4 (64
// rows = two 32-row subtiles), for all 128 tokens (four 32-token tiles):
// eight 32x32 accumulators.  At the end the two K halves of each row group
// are summed through LDS; the K-half-0 wave finishes token tiles 0-1 and
// its partner tiles 2-3.
//
// Memory path.  x_t goes global -> LDS by direct-to-LDS buffer loads (the
// four row groups share it): 4 token rows x 256 B per instruction, 16-byte
// chunk q of row r stored at q ^ (r mod 16), so the MFMA reads (lane = token
// row) of 16 consecutive rows hit 16 different bank groups.  The weights
// are not shared between waves and go straight to registers, two blocks
// ahead: one 16-byte load per lane and subtile carries the codes of the
// lane's 32 channels of the block, one 2-byte load their two block scales.
// Inside a wave's 64 channels, lane half h holds channels 32h + 8s .. +7 at
// step s for both operands (the dot product does not depend on which lane
// carries which channel, only that A and B agree), which makes the codes
// of a lane contiguous.
//
// Pipeline.  x_t has four LDS stages and the weights four register sets;
// both run two blocks ahead.  Block i: issue the copies of x_t(i+2) and
// the loads of W(i+2); steps 0-2; wait for this wave's copies of x_t(i+1)
// (s_waitcnt with the 12 later operations still in flight) and s_barrier
// (every wave's copies of x_t(i+1) have landed and every wave is past
// block i-1, whose stage the next block's copies overwrite); step 3, whose
// shadow holds the first read of x_t(i+1).
// The operand reads and dequantization of each 16-deep step are
// interleaved with the MFMAs of the previous one.
//
// When the weight rows are too few to fill the GPU, K is also split
// across workgroups: each writes its fp32 partial tiles (written through
// to memory) and a separate finishing kernel sums them in split order and
// applies the epilogue.  A whole call's launch also runs the LoRA-down
// reduction (t) in a few extra workgroups: appended when K is split (the
// finish reads t), first in the grid when it is not (the epilogue waits
// for them).
#pragma once

#include "qerl_device.h"
#include "treduce.h"

namespace qerl {
namespace d128 {

constexpr int kTokens = 128;     // token rows per launch
constexpr int kRows = 256;       // weight rows per workgroup
constexpr int kBlock = 128;      // K channels per pipeline block

// Tiled weight layout (qerl_nvfp4_tile128): for each 32-row subtile st and
// each 128-channel block b, a tile of kTileBytes at (st * nblocks + b) *
// kTileBytes holding
//   codes   2048 B: slot (kh, h, c) of 16 B at ((2 kh + h) * 32 + c) * 16 =
//           the codes of row 32 st + c, channels 128 b + 64 kh + 32 h + 0..31
//   scales   256 B at 2048: slot (kh, h, c) of 2 B at ((2 kh + h) * 32 + c) * 2
//           = the block scales of those 32 channels
// so the load of one wave (K half kh, lanes (h, c)) for one subtile and
// block is 1 KB of contiguous codes and 128 B of contiguous scales.  Rows
// past n are zero.
constexpr int kTileBytes = 2304;

struct Args {
  const uint16_t* xt;      // [xrows, k] bf16 rows of this m chunk
  const uint8_t* codes;    // [n, k/2], or the tiled weight (TILED)
  const uint8_t* scales;   // [n, k/16] (unused when TILED)
  const float* gscale;
  const uint16_t* t;       // [128, rpad16] bf16 s x_t A^T of this chunk, or null
  const uint16_t* lora_b;  // [n, r] bf16
  uint16_t* y;             // [m_valid, n] rows of this chunk
  float* ypart;            // [split, 128, n] fp32 partials (split > 1)
  int64_t n, k;
  int64_t nblocks;         // k / 128, spread evenly over the splits
  int xrows, m_valid, split, r, rpad16, lora_vec;
  // Grid: groups * split contraction workgroups (workgroup g + groups * s
  // owns row group g and K split s), then tr_wgs workgroups that sum the
  // LoRA-down partials into t (split > 1 only: the finish reads t).
  int groups, tr_wgs;
  TReduceArgs tr;
  // Unsplit with tr_wgs > 0: the reduction workgroups come first in the
  // grid instead (workgroup tr_wgs + g owns row group g), store t at device
  // scope and count themselves in tsync[0] (zero at launch); the epilogue
  // waits for the count before it reads t.  tsync[1] is set if that wait
  // gave up.  Null otherwise.
  unsigned* tsync;
};

// A wait for t gives up after this many polls (about a second); the output
// is then undefined and tsync[1] is set.
constexpr uint32_t kTWaitLimit = 1u << 20;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Buffer resource over [p, p + bytes): loads past the end read zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* dst, uint32_t voff,
                                      uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)dst, 16, (int)voff, (int)soff, 0, 0);
}

__device__ __forceinline__ uint4 bload128(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff,
                                                                         (int)soff, 0));
}

__device__ __forceinline__ uint32_t bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                            uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0);
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

__device__ __forceinline__ uint32_t word(const uint4& v, int j) {
  return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
}

// LoRA B operand: B[row][j0 .. j0+7] (zeros past r or for a dead row).
__device__ __forceinline__ uint4 lora_b8(const Args& a, int64_t row, bool live, int j0) {
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

template <bool P2 = false, bool TILED = false>
__global__ __launch_bounds__(512, 1) void decode_m128(Args a) {
  constexpr int MT = kTokens / 32;            // token tiles
  constexpr int NTW = 2;                      // weight subtiles per wave
  constexpr int XCOPIES = kTokens / 4 / 8;    // x_t copies per wave and block (4 rows each)
  // x_t stages: 128 rows x 16 chunks of 16 B (32 KB each).  After the main
  // loop the first two hold the reduction slots: 8 waves x two tiles x 1024
  // floats, tile t of every wave in stage t; the last two hold the bf16
  // output tiles of the unsplit epilogue, 8 KB per wave.
  __shared__ __attribute__((aligned(16))) uint4 xs0[kTokens * 16], xs1[kTokens * 16],
      xs2[kTokens * 16], xs3[kTokens * 16];

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
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kh = wave >> 2, rg = wave & 3;
  const int h = lane >> 5, c = lane & 31;
  const int split_id = bid / a.groups;
  const int64_t row0 = (int64_t)(bid - split_id * a.groups) * kRows;
  const int64_t bb = (int64_t)split_id * a.nblocks / a.split;
  const int64_t be = (int64_t)(split_id + 1) * a.nblocks / a.split;

  const uint32_t kbytes = (uint32_t)(a.k / 2), kscales = (uint32_t)(a.k / 16);
  const uint32_t xrow = (uint32_t)a.k * 2;
  // Standard layout: codes and scales from row row0 on.  Tiled layout: the
  // tiles from subtile row0 / 32 on, one descriptor for codes and scales.
  const int64_t sub0 = row0 / 32, nsub = (a.n + 31) / 32;
  const uint32_t tstride = (uint32_t)a.nblocks * kTileBytes;   // bytes per subtile
  const __amdgpu_buffer_rsrc_t rw =
      TILED ? rsrc(a.codes + sub0 * tstride, (uint32_t)((nsub - sub0) * tstride))
            : rsrc(a.codes + row0 * kbytes, (uint32_t)((a.n - row0) * kbytes));
  const __amdgpu_buffer_rsrc_t rs =
      TILED ? rw : rsrc(a.scales + row0 * kscales, (uint32_t)((a.n - row0) * kscales));
  const __amdgpu_buffer_rsrc_t rx = rsrc(a.xt, (uint32_t)a.xrows * xrow);

  // x_t copy j of this wave: LDS rows 4 (wave + 8 j) .. +3; lane l -> row
  // 4 (wave + 8 j) + l / 16, chunk position l % 16, which holds global chunk
  // (l % 16) ^ (row mod 16); row mod 16 does not depend on j.
  const uint32_t xr = 4u * (uint32_t)wave + (uint32_t)(lane >> 4);
  const uint32_t vx = xr * xrow + 16u * (((uint32_t)lane & 15u) ^ (xr & 15u));
  // Weight rows of this lane: 64 rg + 32 t + c; codes of K half kh, lane half h.
  uint32_t vc[NTW], vs[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    if (TILED) {
      const uint32_t tile = (2u * (uint32_t)rg + (uint32_t)t) * tstride;
      const uint32_t slot = (2u * (uint32_t)kh + (uint32_t)h) * 32u + (uint32_t)c;
      vc[t] = tile + 16u * slot;
      vs[t] = tile + 2048u + 2u * slot;
    } else {
      const uint32_t wr = 64u * (uint32_t)rg + 32u * (uint32_t)t + (uint32_t)c;
      vc[t] = wr * kbytes + 32u * (uint32_t)kh + 16u * (uint32_t)h;
      vs[t] = wr * kscales + 4u * (uint32_t)kh + 2u * (uint32_t)h;
    }
  }
  // Byte offset of block blk: codes and scales of the standard layout, or
  // the tile of the tiled one.
  const uint32_t cstep = TILED ? (uint32_t)kTileBytes : (uint32_t)(kBlock / 2);
  const uint32_t sstep = TILED ? (uint32_t)kTileBytes : (uint32_t)(kBlock / 16);

  auto copy_x = [&](int64_t blk, uint4* xs) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < XCOPIES; ++j)
      dma16(rx, xs + (wave + 8 * j) * 64, vx + 32u * (uint32_t)j * xrow,
            (uint32_t)(2 * kBlock) * (uint32_t)blk);
  };
  auto load_w = [&](int64_t blk, uint4 (&wv)[NTW], uint32_t (&sv)[NTW])
      __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NTW; ++t) wv[t] = bload128(rw, vc[t], cstep * (uint32_t)blk);
#pragma unroll
    for (int t = 0; t < NTW; ++t) sv[t] = bload16(rs, vs[t], sstep * (uint32_t)blk);
  };

  f32x16_t acc[NTW][MT];
#pragma unroll
  for (int t = 0; t < NTW; ++t)
#pragma unroll
    for (int u = 0; u < MT; ++u) acc[t][u] = zero16();

  // Operands of one 16-deep step: x_t fragments (lane = token row) read from
  // an LDS stage, and the dequantized weight fragments of the two subtiles.
  auto read_a = [&](const uint4* xs, int s, uint4 (&xa)[MT]) __attribute__((always_inline)) {
    const int q = 8 * kh + 4 * h + s;        // 16-byte chunk of the 256-byte row
#pragma unroll
    for (int u = 0; u < MT; ++u) xa[u] = xs[(32 * u + c) * 16 + (q ^ (c & 15))];
  };
  auto dequant_b = [&](const uint4 (&wv)[NTW], const uint32_t (&sv)[NTW], int s,
                       uint4 (&bf)[NTW]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const float sb = e4m3_to_f32((sv[t] >> (8 * (s >> 1))) & 0xffu);
      bf[t] = P2 ? dequant8_bf16_pow2(word(wv[t], s), sb) : dequant8_bf16(word(wv[t], s), sb);
    }
  };
  // One step: the MFMAs of the current operands, with the next step's LDS
  // reads and dequantization interleaved (one MFMA, then four VALU
  // instructions, the reads first), so that the matrix pipe stays busy
  // while the wave prepares what follows.
  auto mfmas = [&](const uint4 (&xa)[MT], const uint4 (&bf)[NTW]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int u = 0; u < MT; ++u) acc[t][u] = mfma_bf16(xa[u], bf[t], acc[t][u]);
  };
  auto interleave = []() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // DS reads
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // VALU
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < 7; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
  };

  if (bb < be) {
    const int64_t last = be - 1;
    // Block bb + i uses x_t stage i % 4 and weight registers i % 4; the
    // copies and loads run two blocks ahead.
    uint4 w0[NTW], w1[NTW], w2[NTW], w3[NTW];
    uint32_t s0[NTW], s1[NTW], s2[NTW], s3[NTW];
    uint4 xa0[MT], xa1[MT], b0[NTW], b1[NTW];
    // Issue order as in a steady-state block (x_t(i), W(i) pairs), so the
    // compiler's waits match the manual ones.
    copy_x(bb, xs0);
    __builtin_amdgcn_sched_barrier(0);
    load_w(bb, w0, s0);
    __builtin_amdgcn_sched_barrier(0);
    copy_x(min(bb + 1, last), xs1);
    __builtin_amdgcn_sched_barrier(0);
    load_w(min(bb + 1, last), w1, s1);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<12>();                        // x_t(bb) has landed
    barrier_nofence();
    read_a(xs0, 0, xa0);
    dequant_b(w0, s0, 0, b0);
    // Block at offset OFF of a group of four: W = its weights, XS its stage,
    // XN the next block's stage and WN its weights, X2 / W2 / S2 the stage
    // and registers that receive the block two ahead.
    //   top:        copies of x_t(i+2), then loads of W(i+2); the scheduling
    //               barriers keep every copy ahead of every load, which the
    //               count of the wait below (12 = the 4 + 4 + 4 operations
    //               issued after x_t(i+1)) relies on: with a load of W(i+1)
    //               moved before a copy of x_t(i+1), fewer than 12 would
    //               follow it and a wave could pass the barrier while its
    //               copy is still in flight
    //   steps 0-2:  MFMAs of steps 0, 1, 2 (reads and dequantization of
    //               steps 1, 2, 3)
    //   late:       wait for this wave's copies of x_t(i+1), s_barrier: every
    //               copy of x_t(i+1) has landed, and every wave is past block
    //               i-1, so the stage written at the next block's top is free;
    //               placed as late as it can be, just before the first read
    //               of x_t(i+1), to give the copies the most time
    //   step 3:     MFMAs of step 3 (reads and dequantization of the next
    //               block's step 0)
#define QERL_M128_BLOCK(OFF, W, S, XS, XN, WN, SN, X2, W2, S2)            \
  copy_x(min(blk + (OFF) + 2, last), X2);                                 \
  __builtin_amdgcn_sched_barrier(0);                                      \
  load_w(min(blk + (OFF) + 2, last), W2, S2);                             \
  __builtin_amdgcn_sched_barrier(0);                                      \
  read_a(XS, 1, xa1);                                                     \
  dequant_b(W, S, 1, b1);                                                 \
  mfmas(xa0, b0);                                                         \
  interleave();                                                           \
  read_a(XS, 2, xa0);                                                     \
  dequant_b(W, S, 2, b0);                                                 \
  mfmas(xa1, b1);                                                         \
  interleave();                                                           \
  read_a(XS, 3, xa1);                                                     \
  dequant_b(W, S, 3, b1);                                                 \
  mfmas(xa0, b0);                                                         \
  interleave();                                                           \
  wait_vmcnt<12>();                                                       \
  barrier_nofence();                                                      \
  read_a(XN, 0, xa0);                                                     \
  dequant_b(WN, SN, 0, b0);                                               \
  mfmas(xa1, b1);                                                         \
  interleave();
    // Past the last block the copies and loads repeat the last one (and the
    // next block's operands are read but never used), so every block issues
    // the same number and the vmcnt waits stay exact.  The loop has a single
    // exit (groups of four blocks, then up to three more): early exits from
    // an unrolled body made the compiler copy the accumulators.
    const int64_t nb = be - bb;
    int64_t blk = bb;
    for (int64_t i = 0; i < nb / 4; ++i, blk += 4) {
      QERL_M128_BLOCK(0, w0, s0, xs0, xs1, w1, s1, xs2, w2, s2)
      QERL_M128_BLOCK(1, w1, s1, xs1, xs2, w2, s2, xs3, w3, s3)
      QERL_M128_BLOCK(2, w2, s2, xs2, xs3, w3, s3, xs0, w0, s0)
      QERL_M128_BLOCK(3, w3, s3, xs3, xs0, w0, s0, xs1, w1, s1)
    }
    const int rem = (int)(nb & 3);
    if (rem > 0) {
      QERL_M128_BLOCK(0, w0, s0, xs0, xs1, w1, s1, xs2, w2, s2)
    }
    if (rem > 1) {
      QERL_M128_BLOCK(1, w1, s1, xs1, xs2, w2, s2, xs3, w3, s3)
    }
    if (rem > 2) {
      QERL_M128_BLOCK(2, w2, s2, xs2, xs3, w3, s3, xs0, w0, s0)
    }
#undef QERL_M128_BLOCK
    // An empty use of every weight register set: without it the compiler
    // deletes the loads of the last blocks whose values are never used,
    // and the mid-block waits, which count them, would then let the x_t
    // copies they are meant to wait for still be in flight.
    auto keep = [](const uint4 (&wv)[NTW], const uint32_t (&sv)[NTW])
        __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < NTW; ++t) asm volatile("" ::"v"(wv[t].x), "v"(sv[t]));
    };
    keep(w0, s0);
    keep(w1, s1);
    keep(w2, s2);
    keep(w3, s3);
  }
  wait_vmcnt<0>();
  __syncthreads();

  // Sum the two K halves: in round rho the K-half-1 wave of row group rg
  // hands token tile rho to its partner, and the K-half-0 wave hands token
  // tile 2 + rho to its partner.  Slot of (writer wave w, subtile t): 1024
  // floats at w * 1024 in stage t.
  float* slots[NTW] = {reinterpret_cast<float*>(xs0), reinterpret_cast<float*>(xs1)};
  const int partner = wave ^ 4;
#pragma unroll
  for (int rho = 0; rho < 2; ++rho) {
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      float* dst = slots[t] + wave * 1024 + lane;
      const f32x16_t v = kh ? acc[t][rho] : acc[t][2 + rho];
#pragma unroll
      for (int e = 0; e < 16; ++e) dst[e * 64] = v[e];
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const float* src = slots[t] + partner * 1024 + lane;
      if (kh == 0) {
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[t][rho][e] += src[e * 64];
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[t][2 + rho][e] += src[e * 64];
      }
    }
    __syncthreads();
  }

  // Epilogue of the owned tiles: token tiles 2 kh, 2 kh + 1.
  const int64_t row_end = min(a.n, row0 + (int64_t)kRows);
  if (a.split > 1) {
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const int64_t row = row0 + 64 * rg + 32 * t + c;
      if (row >= row_end) continue;
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) {
        const int u = 2 * kh + uu;
        const f32x16_t v = kh ? acc[t][2 + uu] : acc[t][uu];
        float* dst = a.ypart + ((int64_t)split_id * kTokens + 32 * u) * a.n + row;
        // Written through to memory (device-scope stores): the finishing
        // launch reads them from there anyway, and the kernel's end then
        // has no dirty L2 lines of partials to write back.
#pragma unroll
        for (int e = 0; e < 16; ++e)
          __hip_atomic_store(dst + (int64_t)acc_row(e, lane) * a.n, v[e], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    return;
  }
  const float S = *a.gscale;
  // With n a multiple of 8 and y 16-byte aligned, the wave's 64 token rows x
  // 64 columns of y pass through an 8 KB LDS tile of its own (stages 2 and 3
  // are idle after the K-half exchange) and leave as 16-byte stores that
  // cover whole 128-byte rows, instead of 2-byte stores that fill each line
  // in two halves from different instructions.
  const bool vec = a.n % 8 == 0 && (reinterpret_cast<uintptr_t>(a.y) & 15) == 0;
  uint16_t* ytile = reinterpret_cast<uint16_t*>(wave < 4 ? xs2 : xs3) + (wave & 3) * 4096;
  if (a.tsync) {
    // t comes from this launch's first workgroups (dispatched before this
    // one, so the wait ends); its rows are read at device scope below
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
    // t (rows past xrows as zeros) into LDS once per workgroup, loaded at
    // device scope (aux 16: sc1): token rows 0-63 in stage 0, 64-127 in
    // stage 1, nch + 1 16-byte chunks per row (an odd stride: the MFMA-layout
    // reads of 16 consecutive rows hit 16 different bank groups)
    if (a.r > 0) {
      const int nch = a.rpad16 / 8;
      const __amdgpu_buffer_rsrc_t rt = rsrc(a.t, (uint32_t)(a.xrows * a.rpad16 * 2));
      for (int ch = threadIdx.x; ch < kTokens * nch; ch += 512) {
        const int tr = ch / nch, q = ch - tr * nch;
        (tr < 64 ? xs0 : xs1)[(tr & 63) * (nch + 1) + q] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(rt, (tr * a.rpad16 + 8 * q) * 2, 0, 16));
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int64_t row = row0 + 64 * rg + 32 * t + c;
    const bool live = row < row_end;
#pragma unroll
    for (int uu = 0; uu < 2; ++uu) {
      const int u = 2 * kh + uu;
      f32x16_t v = kh ? acc[t][2 + uu] : acc[t][uu];
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] *= S;
      if (a.r > 0) {
        // t has xrows rows (rows past it are zero tokens)
        const bool trow_in = 32 * u + c < a.xrows;
        const uint16_t* trow = a.t + (int64_t)(32 * u + c) * a.rpad16 + 8 * h;
        const uint4* tl = (u < 2 ? xs0 : xs1) + ((32 * u + c) & 63) * (a.rpad16 / 8 + 1) + h;
        for (int j0 = 0; j0 < a.rpad16; j0 += 16) {
          const uint4 tv = a.tsync ? tl[j0 / 8]
                                   : (trow_in ? *reinterpret_cast<const uint4*>(trow + j0)
                                              : make_uint4(0u, 0u, 0u, 0u));
          v = mfma_bf16(tv, lora_b8(a, row, live, j0 + 8 * h), v);
        }
      }
      if (vec) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
          ytile[(32 * uu + acc_row(e, lane)) * 64 + 32 * t + c] = f32_to_bf16_bits(v[e]);
        continue;
      }
      if (!live) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int mrow = 32 * u + acc_row(e, lane);
        if (mrow < a.m_valid) a.y[(int64_t)mrow * a.n + row] = f32_to_bf16_bits(v[e]);
      }
    }
  }
  if (!vec) return;
  // 16-byte chunk q = lane + 64 j of the tile holds token row 64 kh + q / 8,
  // columns 8 (q % 8) .. 8 (q % 8) + 7 of the wave's block.  The wave reads
  // back only its own writes, and one wave's LDS operations complete in
  // order.  row_end and the columns are multiples of 8, so a chunk is either
  // wholly inside y or wholly past its end.
  const int64_t col0 = row0 + 64 * rg;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int q = lane + 64 * j;
    const int rr = q >> 3, cc = 8 * (q & 7);
    const uint4 val = *reinterpret_cast<const uint4*>(ytile + rr * 64 + cc);
    const int mrow = 64 * kh + rr;
    if (mrow < a.m_valid && col0 + cc < row_end)
      *reinterpret_cast<uint4*>(a.y + (int64_t)mrow * a.n + col0 + cc) = val;
  }
}

typedef void (*Kernel)(Args);

Kernel pick(bool p2, bool tiled);

// The tiled layout: its size, and the re-layout of a standard NVFP4 weight.
size_t tile128_bytes(int64_t n, int64_t k);
hipError_t launch_tile128(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k,
                          uint8_t* out, hipStream_t stream);

}  // namespace d128
}  // namespace qerl
