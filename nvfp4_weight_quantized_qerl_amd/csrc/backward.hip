// Backward of the NVFP4 + LoRA + AQN linear layer through the frozen
// quantized weight.  The rollout's log-probabilities are taken on the same
// quantized model and only the LoRA factors (and RMSNorm scales) are
// trained [QeRL summary, §3.4 "Low-Rank Adaptation"; Algorithm 1, inner
// updates]: the weight gets no gradient, the input does.  With
// x_t = x (.) (1 + z), t = s x_t A^T and gs = s dy B:
//     dx = bf16( (S dy W0 + gs A) (.) (1 + z) )     W_hat = S W0 (Eq. 6)
//     dA = gs^T x_t                                   [r, k] fp32
//     dB = dy^T t                                     [n, r] fp32
// Launches: the forward's prepare (t only), a transpose of B, the
// LoRA-down kernels on (dy, B^T) for gs, the dx contraction below, and for
// each of dA and dB an accumulation over 256-row chunks plus a reduction of
// the chunks in order.
//
// dx contraction (bwd_dx<MT>): a workgroup of eight waves owns 32 MT token
// rows x 256 output columns (input channels k); wave w the columns
// 32 w .. 32 w + 31.  The sum runs over the weight rows n in steps of 32:
// the workgroup copies the codes (32 rows x 128 B) and scales of the step,
// dequantizes them (E2M1 code x E4M3 scale, exact in bf16) into an LDS tile
// stored transposed, [k][n] with rows padded to 40 elements (80 B) so that
// the MFMA operand reads (lane = column k, eight consecutive n) of 16 lanes
// hit 16 different bank groups, and runs two 32x32x16 bf16 MFMAs per token
// tile.  A dequantizing lane takes two adjacent weight rows, so each of its
// transposed writes is one dword holding both rows of a column.  The dy tile of the step is copied to LDS with 16-byte loads (rows
// padded to 40 elements like the weight tile, two buffers) and read by the
// MFMAs with lane = token row.  The codes, scales and dy of the next step
// are loaded into registers while the current step's MFMAs run; two
// barriers per step.
#include <algorithm>

#include "qerl_act.h"
#include "qerl_device.h"
#include "qerl_internal.h"

namespace qerl {
namespace {

constexpr int kTileK = 256;     // output columns per workgroup (eight waves of 32)
constexpr int kThreads = 512;
constexpr int kCodeRow = kTileK / 2;     // code bytes of one weight row of the tile
constexpr int kCodeLds = kCodeRow + 4;   // its LDS row: 33 dwords, so rows 2p hit distinct banks
constexpr int kScaleRow = kTileK / 16;   // scale bytes of one weight row of the tile
constexpr int kScaleLds = kScaleRow + 4; // its LDS row: 5 dwords, so rows 2p hit distinct banks
constexpr int kStepN = 32;      // weight rows per step
constexpr int kLdsRow = 40;     // padded LDS row (elements) of the transposed tile

struct DxArgs {
  const uint16_t* __restrict__ dy;     // [m, n] bf16
  const uint8_t* __restrict__ codes;   // [n, k/2]
  const uint8_t* __restrict__ scales;  // [n, k/16]
  const float* __restrict__ gscale;
  const uint16_t* __restrict__ gs;     // [mpad, rpad16] bf16 s dy B, or null
  const uint16_t* __restrict__ lora_a; // [r, k] bf16
  const float* __restrict__ z;         // [k] or null
  uint16_t* __restrict__ dx;           // [m, k] bf16
  int64_t m, n, k;
  int r, rpad16;
};

template <int MT>
__global__ __launch_bounds__(kThreads) void bwd_dx(DxArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t wt[kTileK * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint8_t cs[kStepN * kCodeLds];
  __shared__ __attribute__((aligned(16))) uint8_t ss[kStepN * kScaleLds];
  // dy tile of the step, [32 MT rows][40] bf16, two buffers (step parity)
  __shared__ __attribute__((aligned(16))) uint16_t dys[2][32 * MT * kLdsRow];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 31, h = lane >> 5;
  const int64_t k0 = (int64_t)blockIdx.x * kTileK;
  const int64_t m0 = (int64_t)blockIdx.y * 32 * MT;
  const int64_t kbytes = a.k / 2, kscales = a.k / 16;
  // copy roles: thread -> weight row tid / 16 of the step, 8 code bytes at (tid % 16) * 8
  // (and the scale byte tid % 16 of the same row)
  const int lr = tid / (kCodeRow / 8), lb = (tid % (kCodeRow / 8)) * 8;
  // dequantization roles: thread -> weight rows 2 pp, 2 pp + 1 and, in each of two
  // passes, four columns 4 G .. 4 G + 3 with G = 4 (2 wave + pass) + lane / 16;
  // every transposed write is one dword (the two rows of a column), and the
  // four 16-lane groups of a wave land in four different 16-bank windows
  const int pp = lane & 15, gl = lane >> 4;
  uint32_t* wt32 = reinterpret_cast<uint32_t*>(wt);
  f32x16_t acc[MT];
#pragma unroll
  for (int u = 0; u < MT; ++u) acc[u] = zero16();

  // Global operands of one step, held in registers one step ahead: the
  // dy tile goes 16 bytes per thread-chunk (row ch / 4, columns 8 (ch % 4)).
  constexpr int DYCH = 32 * MT * 4;               // 16-byte chunks of the dy tile
  constexpr int DYPT = (DYCH + kThreads - 1) / kThreads;   // chunks per thread
  uint2 cv;
  uint8_t sv;
  uint4 dv[DYPT];
  auto load_step = [&](int64_t n0) {
    const int64_t row = n0 + lr;
    const int64_t byte0 = k0 / 2 + lb;            // 8 bytes = 16 columns
    cv = make_uint2(0u, 0u);
    if (row < a.n && 2 * byte0 < a.k)
      cv = *reinterpret_cast<const uint2*>(a.codes + row * kbytes + byte0);
    const int srow = tid / kScaleRow, sblk = tid % kScaleRow;
    const int64_t blk = k0 / 16 + sblk, row2 = n0 + srow;
    sv = (row2 < a.n && blk < kscales) ? a.scales[row2 * kscales + blk] : 0;
#pragma unroll
    for (int i = 0; i < DYPT; ++i) {
      const int ch = tid + kThreads * i;
      dv[i] = make_uint4(0u, 0u, 0u, 0u);
      const int64_t mrow = m0 + (ch >> 2), nn = n0 + 8 * (ch & 3);
      if (ch < DYCH && mrow < a.m && nn < a.n)
        dv[i] = *reinterpret_cast<const uint4*>(a.dy + mrow * a.n + nn);
    }
  };

  load_step(0);
  int par = 0;
  for (int64_t n0 = 0; n0 < a.n; n0 += kStepN, par ^= 1) {
    // Every wave has finished the previous step's MFMAs (which read wt and
    // the other dy buffer) and dequantization (which read cs) before it
    // passes the barrier below; this dy buffer was last read two steps ago.
    uint32_t* cdst = reinterpret_cast<uint32_t*>(cs + lr * kCodeLds + lb);
    cdst[0] = cv.x;
    cdst[1] = cv.y;
    ss[(tid / kScaleRow) * kScaleLds + tid % kScaleRow] = sv;
    uint16_t* dyb = dys[par];
#pragma unroll
    for (int i = 0; i < DYPT; ++i) {
      const int ch = tid + kThreads * i;
      if (ch < DYCH) *reinterpret_cast<uint4*>(dyb + (ch >> 2) * kLdsRow + 8 * (ch & 3)) = dv[i];
    }
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int G = 4 * (2 * wave + pass) + gl;       // four columns 4 G .. 4 G + 3
      const int r0 = 2 * pp;
      uint32_t lohi[2][2];                           // [row][bf16 pair of columns]
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const uint32_t c4 = *reinterpret_cast<const uint16_t*>(cs + (r0 + rr) * kCodeLds + 2 * G);
        const float sb = e4m3_to_f32(ss[(r0 + rr) * kScaleLds + (G >> 2)]);
        const f32x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c4, 1.0f, 0);
        const f32x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c4, 1.0f, 1);
        lohi[rr][0] = pack_bf16x2(v0[0] * sb, v0[1] * sb);
        lohi[rr][1] = pack_bf16x2(v1[0] * sb, v1[1] * sb);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t a0 = (lohi[0][i >> 1] >> (16 * (i & 1))) & 0xffffu;   // row r0
        const uint32_t a1 = (lohi[1][i >> 1] >> (16 * (i & 1))) & 0xffffu;   // row r0 + 1
        wt32[((4 * G + i) * kLdsRow + r0) >> 1] = a0 | (a1 << 16);
      }
    }
    __syncthreads();
    if (n0 + kStepN < a.n) load_step(n0 + kStepN);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const uint4 b = *reinterpret_cast<const uint4*>(wt + (32 * wave + c) * kLdsRow + 16 * s2 + 8 * h);
#pragma unroll
      for (int u = 0; u < MT; ++u) {
        const uint4 av = *reinterpret_cast<const uint4*>(dyb + (32 * u + c) * kLdsRow + 16 * s2 + 8 * h);
        acc[u] = mfma_bf16(av, b, acc[u]);
      }
    }
  }
  __syncthreads();

  const float S = *a.gscale;
  const int64_t col = k0 + 32 * wave + c;
  const bool live = col < a.k;
  const float zc = (live && a.z) ? a.z[col] : 0.0f;
#pragma unroll
  for (int u = 0; u < MT; ++u) {
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[u][v] *= S;
    if (a.gs) {
      for (int j0 = 0; j0 < a.rpad16; j0 += 16) {
        const uint4 gv = *reinterpret_cast<const uint4*>(a.gs + (m0 + 32 * u + c) * a.rpad16 + j0 + 8 * h);
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = j0 + 8 * h + 2 * i;
          const uint32_t lo = (live && j < a.r) ? a.lora_a[(int64_t)j * a.k + col] : 0u;
          const uint32_t hi = (live && j + 1 < a.r) ? a.lora_a[(int64_t)(j + 1) * a.k + col] : 0u;
          w[i] = lo | (hi << 16);
        }
        acc[u] = mfma_bf16(gv, make_uint4(w[0], w[1], w[2], w[3]), acc[u]);
      }
    }
    if (!live) continue;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t mrow = m0 + 32 * u + acc_row(v, lane);
      if (mrow < a.m) a.dx[mrow * a.k + col] = f32_to_bf16_bits(acc[u][v] * (1.0f + zc));
    }
  }
}

// part[mc][j][c] = sum over the token rows i of chunk mc (kOuterRows rows)
// of q[i, j] p[i, c], for columns c of p [m, cols] (row stride ldp) and
// j < r of q [.., ldq] (bf16), by 32x32x16 bf16 MFMAs with the tokens as the
// contraction.  A workgroup of four waves owns 128 columns (wave w: 32 w ..
// 32 w + 31) and all 32 RT values of j for one chunk.  Each step stages 32
// token rows of p and q in LDS as they are stored (16-byte copies, rows padded
// so that token rows 8 apart fall on different bank halves); the MFMA operands
// (lane = column or j, eight consecutive tokens) are gathered from there with
// 2-byte reads.  The next step's rows are loaded while the MFMAs run.  With
// a noise vector z the p rows are x and the contraction uses
// x_t = bf16(x (1 + z)), formed as they are loaded (noisy8, the prepare's
// arithmetic).
// outer_reduce sums the chunks in chunk order.
constexpr int kOuterRows = 256;
constexpr int kOuterCols = 128;            // columns per workgroup
constexpr int kOuterLds = kOuterCols + 8;  // LDS row of the p tile (elements)

template <int RT>
__global__ __launch_bounds__(256) void outer_mfma(const uint16_t* __restrict__ p, int64_t ldp,
                                                  const float* __restrict__ z,
                                                  const uint16_t* __restrict__ q, int64_t ldq,
                                                  int64_t m, int64_t cols, int r,
                                                  float* __restrict__ part) {
  constexpr int QW = 32 * RT;              // j values of the q tile
  constexpr int QLDS = QW + 8;
  constexpr int QCH = 32 * QW / 8;         // 16-byte chunks of the q tile
  constexpr int QPT = (QCH + 255) / 256;   // q chunks per thread
  __shared__ __attribute__((aligned(16))) uint16_t pt[32 * kOuterLds];
  __shared__ __attribute__((aligned(16))) uint16_t qt[32 * QLDS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 31, h = lane >> 5;
  const int64_t c0 = (int64_t)blockIdx.x * kOuterCols;
  const int mc = blockIdx.y;
  const int64_t i0 = (int64_t)mc * kOuterRows;
  const int64_t iend = min<int64_t>(m, i0 + kOuterRows);
  // copy roles: p chunk e (e = tid, tid + 256) -> token row e / 16, columns
  // 8 (e % 16) .. + 7; q chunk e (e = tid + 256 i < QCH) -> token row
  // e / (QW / 8), j = 8 (e % (QW / 8)) .. + 7
  uint4 pv[2], qv[QPT];
  auto load = [&](int64_t s) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = tid + 256 * i;
      const int64_t row = s + (e >> 4), col = c0 + 8 * (e & 15);
      pv[i] = make_uint4(0u, 0u, 0u, 0u);
      if (row < iend && col < cols)
        pv[i] = *reinterpret_cast<const uint4*>(p + row * ldp + col);
    }
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int e = tid + 256 * i;
      qv[i] = make_uint4(0u, 0u, 0u, 0u);
      const int64_t row = s + e / (QW / 8);
      const int j0 = 8 * (e % (QW / 8));
      if (e < QCH && row < iend && j0 < r) {
        const uint4 v = *reinterpret_cast<const uint4*>(q + row * ldq + j0);
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int x = 0; x < 8; ++x)            // j >= r reads as zero
          if (j0 + x >= r) w[x >> 1] &= (x & 1) ? 0x0000ffffu : 0xffff0000u;
        qv[i] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  };
  // Eight bf16 of column col (LDS row stride ld), token rows t0 .. t0 + 7.
  auto gather = [&](const uint16_t* tile, int ld, int col, int t0) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)tile[(t0 + 2 * e) * ld + col] | ((uint32_t)tile[(t0 + 2 * e + 1) * ld + col] << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
  };

  // noise of this thread's eight p columns (the same in every step); the
  // multiply is applied as the prefetched rows are stored, so that the
  // loads of the next step stay in flight during the MFMAs
  float4 z0 = make_float4(0.0f, 0.0f, 0.0f, 0.0f), z1 = z0;
  const int64_t zcol = c0 + 8 * (tid & 15);
  if (z && zcol < cols) {
    z0 = *reinterpret_cast<const float4*>(z + zcol);
    z1 = *reinterpret_cast<const float4*>(z + zcol + 4);
  }
  f32x16_t acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = zero16();
  load(i0);
  for (int64_t s = i0; s < iend; s += 32) {
    __syncthreads();                           // the previous step's gathers are done
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = tid + 256 * i;
      *reinterpret_cast<uint4*>(pt + (e >> 4) * kOuterLds + 8 * (e & 15)) =
          z ? noisy8(pv[i], z0, z1) : pv[i];
    }
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int e = tid + 256 * i;
      if (e < QCH) *reinterpret_cast<uint4*>(qt + (e / (QW / 8)) * QLDS + 8 * (e % (QW / 8))) = qv[i];
    }
    __syncthreads();
    if (s + 32 < iend) load(s + 32);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const uint4 b = gather(pt, kOuterLds, 32 * wave + c, 16 * s2 + 8 * h);
#pragma unroll
      for (int t = 0; t < RT; ++t)
        acc[t] = mfma_bf16(gather(qt, QLDS, 32 * t + c, 16 * s2 + 8 * h), b, acc[t]);
    }
  }
  // D[j][col]: lane l, element v holds col = l % 32, j = acc_row(v, l)
  const int64_t col = c0 + 32 * wave + c;
  if (col >= cols) return;
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int j = 32 * t + acc_row(v, lane);
      if (j < r) part[((int64_t)mc * r + j) * cols + col] = acc[t][v];
    }
}

// out[c * oc + j * oj] = sum over chunks mc (in order) of part[mc][j][c].
__global__ __launch_bounds__(256) void outer_reduce(const float* __restrict__ part, int mchunks,
                                                    int64_t cols, int r, float* __restrict__ out,
                                                    int64_t oc, int64_t oj) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= cols * r) return;
  const int j = (int)(e / cols);
  const int64_t c = e - (int64_t)j * cols;
  float sum = 0.0f;
  for (int mc = 0; mc < mchunks; ++mc) sum += part[((int64_t)mc * r + j) * cols + c];
  out[c * oc + (int64_t)j * oj] = sum;
}

__global__ __launch_bounds__(256) void transpose_b(const uint16_t* __restrict__ b, int64_t n,
                                                   int r, uint16_t* __restrict__ bt) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n * r) return;
  const int j = (int)(i / n);
  const int64_t row = i - (int64_t)j * n;
  bt[i] = b[row * r + j];      // bt [r, n]
}

inline int64_t rup64(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

}  // namespace

BackwardPlan make_backward_plan(int64_t m, int64_t n, int64_t k, int r) {
  BackwardPlan b{};
  make_linear_plan(m, n, k, r, &b.fwd);
  const int64_t mpad = b.fwd.mpad;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = (size_t)rup64((int64_t)(off + bytes), 256);
    return o;
  };
  const int rpad32 = r ? (int)rup64(r, 32) : 0, rpad16 = r ? (int)rup64(r, 16) : 0;
  // Of the forward's workspace the backward uses only the LoRA-down partials
  // and t (x_t is formed from x and z where it is needed, and not stored).
  b.fwd.off_xt = 0;
  b.fwd.off_sync = 0;
  b.fwd.off_ypart = 0;
  b.fwd.off_tpart = take(r ? (size_t)b.fwd.kchunks * mpad * b.fwd.rpad32 * 4 : 0);
  b.fwd.off_t = take(r ? (size_t)mpad * b.fwd.rpad16 * 2 : 0);
  b.off_bt = take(r ? (size_t)r * n * 2 : 0);
  b.off_gpart = take(r ? (size_t)((n + 511) / 512) * mpad * rpad32 * 4 : 0);
  b.off_gs = take(r ? (size_t)mpad * rpad16 * 2 : 0);
  b.mchunks = (int)((m + kOuterRows - 1) / kOuterRows);
  b.off_opart = take(r ? (size_t)b.mchunks * r * std::max(n, k) * 4 : 0);
  b.total = std::max<size_t>(off, 256);   // a size of 0 means invalid sizes
  return b;
}

hipError_t launch_linear_backward(const BackwardPlan& b, const uint16_t* dy, const uint8_t* codes,
                                  const uint8_t* scales, const float* gscale, const uint16_t* x,
                                  const uint16_t* lora_a, const uint16_t* lora_b, float lora_scale,
                                  const float* z, uint16_t* dx, float* da, float* db, char* ws,
                                  hipStream_t stream) {
  const LinearPlan& p = b.fwd;
  const int r = (lora_a && lora_b) ? p.r : 0;
  hipError_t e;
  // t = s x_t A^T (the forward's prepare, without storing x_t: the dA
  // contraction forms x_t from x and z as it loads them)
  e = launch_linear_prepare(p, x, z, r ? lora_a : nullptr, lora_scale, ws, stream, false, false);
  if (e != hipSuccess) return e;
  uint16_t* gs = nullptr;
  if (r) {
    uint16_t* bt = reinterpret_cast<uint16_t*>(ws + b.off_bt);
    hipLaunchKernelGGL(transpose_b, dim3((unsigned)((p.n * r + 255) / 256)), dim3(256), 0, stream,
                       lora_b, p.n, r, bt);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    gs = reinterpret_cast<uint16_t*>(ws + b.off_gs);
    e = launch_lora_down(dy, p.m, p.mpad, p.n, bt, r, lora_scale,
                         reinterpret_cast<float*>(ws + b.off_gpart), gs, stream);
    if (e != hipSuccess) return e;
  }
  DxArgs a;
  a.dy = dy;
  a.codes = codes;
  a.scales = scales;
  a.gscale = gscale;
  a.gs = gs;
  a.lora_a = lora_a;
  a.z = z;
  a.dx = dx;
  a.m = p.m;
  a.n = p.n;
  a.k = p.k;
  a.r = r;
  a.rpad16 = p.rpad16;
  const int64_t ktiles = (p.k + kTileK - 1) / kTileK;
  const int64_t mtiles = p.mpad / 32;
  if (mtiles >= 4 && mtiles % 4 == 0)
    hipLaunchKernelGGL(bwd_dx<4>, dim3((unsigned)ktiles, (unsigned)(mtiles / 4)), dim3(kThreads),
                       0, stream, a);
  else if (mtiles % 2 == 0)
    hipLaunchKernelGGL(bwd_dx<2>, dim3((unsigned)ktiles, (unsigned)(mtiles / 2)), dim3(kThreads),
                       0, stream, a);
  else
    hipLaunchKernelGGL(bwd_dx<1>, dim3((unsigned)ktiles, (unsigned)mtiles), dim3(kThreads), 0,
                       stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  float* opart = reinterpret_cast<float*>(ws + b.off_opart);
  auto outer = [&](const uint16_t* pp, int64_t ldp, const float* zz, const uint16_t* qq,
                   int64_t ldq, int64_t cols, float* out, int64_t oc, int64_t oj) {
    const dim3 grid((unsigned)((cols + kOuterCols - 1) / kOuterCols), (unsigned)b.mchunks);
    switch ((r + 31) / 32) {
      case 1: hipLaunchKernelGGL(outer_mfma<1>, grid, dim3(256), 0, stream, pp, ldp, zz, qq, ldq, p.m, cols, r, opart); break;
      case 2: hipLaunchKernelGGL(outer_mfma<2>, grid, dim3(256), 0, stream, pp, ldp, zz, qq, ldq, p.m, cols, r, opart); break;
      case 3: hipLaunchKernelGGL(outer_mfma<3>, grid, dim3(256), 0, stream, pp, ldp, zz, qq, ldq, p.m, cols, r, opart); break;
      default: hipLaunchKernelGGL(outer_mfma<4>, grid, dim3(256), 0, stream, pp, ldp, zz, qq, ldq, p.m, cols, r, opart); break;
    }
    hipError_t e2 = hipGetLastError();
    if (e2 != hipSuccess) return e2;
    hipLaunchKernelGGL(outer_reduce, dim3((unsigned)((cols * r + 255) / 256)), dim3(256), 0,
                       stream, opart, b.mchunks, cols, r, out, oc, oj);
    return hipGetLastError();
  };
  if (r && da) {
    // dA[j, col] = sum_i gs[i, j] x_t[i, col], x_t = bf16(x (1 + z)) formed on load
    e = outer(x, p.k, z, gs, (int64_t)p.rpad16, p.k, da, (int64_t)1, p.k);
    if (e != hipSuccess) return e;
  }
  if (r && db) {
    // dB[col, j] = sum_i dy[i, col] t[i, j]
    e = outer(dy, p.n, nullptr, reinterpret_cast<const uint16_t*>(ws + p.off_t),
              (int64_t)p.rpad16, p.n, db, (int64_t)r, (int64_t)1);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace qerl
