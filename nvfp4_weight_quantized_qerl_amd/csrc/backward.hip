// Backward of the NVFP4 + LoRA + AQN linear layer through the frozen
// quantized weight.  The rollout's log-probabilities are taken on the same
// quantized model and only the LoRA factors (and RMSNorm scales) are
// trained [QeRL summary, §3.4 "Low-Rank Adaptation"; Algorithm 1, inner
// updates]: the weight gets no gradient, the input does.  With
// x_t = x (.) (1 + z), t = s x_t A^T and gs = s dy B:
//     dx = bf16( (S dy W0 + gs A) (.) (1 + z) )     W_hat = S W0 (Eq. 6)
//     dA = gs^T x_t                                   [r, k] fp32
//     dB = dy^T t                                     [n, r] fp32
// Launches: the forward's prepare (x_t and t), a transpose of B, the
// LoRA-down kernels on (dy, B^T) for gs, the dx contraction below, and one
// accumulation kernel each for dA and dB.
//
// dx contraction (bwd_dx<MT>): a workgroup of four waves owns 32 MT token
// rows x 128 output columns (input channels k); wave w the columns
// 32 w .. 32 w + 31.  The sum runs over the weight rows n in steps of 32:
// the workgroup copies the codes (32 rows x 64 B) and scales of the step,
// dequantizes them (E2M1 code x E4M3 scale, exact in bf16) into an LDS tile
// stored transposed, [k][n] with rows padded to 40 elements (80 B) so that
// the MFMA operand reads (lane = column k, eight consecutive n) of 16 lanes
// hit 16 different bank groups, and runs two 32x32x16 bf16 MFMAs per token
// tile with dy read straight from global memory (lane = token row).
#include <algorithm>

#include "qerl_device.h"
#include "qerl_internal.h"

namespace qerl {
namespace {

constexpr int kTileK = 128;     // output columns per workgroup
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
__global__ __launch_bounds__(256) void bwd_dx(DxArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t wt[kTileK * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint8_t cs[kStepN * 64];
  __shared__ uint8_t ss[kStepN * 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 31, h = lane >> 5;
  const int64_t k0 = (int64_t)blockIdx.x * kTileK;
  const int64_t m0 = (int64_t)blockIdx.y * 32 * MT;
  const int64_t kbytes = a.k / 2, kscales = a.k / 16;
  // copy roles: thread -> weight row n0 + tid / 8, 8 code bytes at (tid % 8) * 8
  const int cr = tid >> 3, cb = (tid & 7) * 8;
  f32x16_t acc[MT];
#pragma unroll
  for (int u = 0; u < MT; ++u) acc[u] = zero16();

  for (int64_t n0 = 0; n0 < a.n; n0 += kStepN) {
    // stage codes and scales of rows n0 .. n0 + 31, columns k0 .. k0 + 127
    {
      const int64_t row = n0 + cr;
      const int64_t byte0 = k0 / 2 + cb;            // 8 bytes = 16 columns
      uint2 v = make_uint2(0u, 0u);
      if (row < a.n && 2 * byte0 < a.k)
        v = *reinterpret_cast<const uint2*>(a.codes + row * kbytes + byte0);
      *reinterpret_cast<uint2*>(cs + cr * 64 + cb) = v;
      if (tid < kStepN * 8) {
        const int srow = tid >> 3, sblk = tid & 7;
        const int64_t blk = k0 / 16 + sblk;
        const int64_t row2 = n0 + srow;
        ss[srow * 8 + sblk] = (row2 < a.n && blk < kscales) ? a.scales[row2 * kscales + blk] : 0;
      }
    }
    __syncthreads();
    // dequantize: thread -> row cr, 16 columns cb*2 .. cb*2 + 15 (one scale block)
    {
      const uint2 v = *reinterpret_cast<const uint2*>(cs + cr * 64 + cb);
      const float sb = e4m3_to_f32(ss[cr * 8 + (cb >> 3)]);
      const uint4 lo = dequant8_bf16(v.x, sb), hi = dequant8_bf16(v.y, sb);
      const uint32_t wds[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int col = 2 * cb + 2 * e;
        wt[col * kLdsRow + cr] = (uint16_t)(wds[e] & 0xffffu);
        wt[(col + 1) * kLdsRow + cr] = (uint16_t)(wds[e] >> 16);
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint4 b = *reinterpret_cast<const uint4*>(wt + (32 * wave + c) * kLdsRow + 16 * s + 8 * h);
      const int64_t nn = n0 + 16 * s + 8 * h;
#pragma unroll
      for (int u = 0; u < MT; ++u) {
        const int64_t mrow = m0 + 32 * u + c;
        uint4 av = make_uint4(0u, 0u, 0u, 0u);
        if (mrow < a.m && nn < a.n) av = *reinterpret_cast<const uint4*>(a.dy + mrow * a.n + nn);
        acc[u] = mfma_bf16(av, b, acc[u]);
      }
    }
    __syncthreads();
  }

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

// out[c, j] (strides oc, oj) = sum_i p[i, c] q[i, j] over the m rows i, for
// columns c of p [m, cols] (row stride ldp) and j < r of q [.., ldq] bf16;
// one thread per column, 32 values of j per launch row (blockIdx.y).
__global__ __launch_bounds__(256) void outer_acc(const uint16_t* __restrict__ p, int64_t ldp,
                                                 const uint16_t* __restrict__ q, int64_t ldq,
                                                 int64_t m, int64_t cols, int r,
                                                 float* __restrict__ out, int64_t oc,
                                                 int64_t oj) {
  const int64_t cidx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int j0 = 32 * blockIdx.y;
  if (cidx >= cols) return;
  float acc[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) acc[j] = 0.0f;
  for (int64_t i = 0; i < m; ++i) {
    const float pv = bf16_to_f32(p[i * ldp + cidx]);
    const uint16_t* qr = q + i * ldq + j0;
#pragma unroll
    for (int j = 0; j < 32; ++j) acc[j] += pv * bf16_to_f32(j0 + j < r ? qr[j] : 0u);
  }
#pragma unroll
  for (int j = 0; j < 32; ++j)
    if (j0 + j < r) out[cidx * oc + (int64_t)(j0 + j) * oj] = acc[j];
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
  size_t off = rup64((int64_t)b.fwd.total, 256);
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = (size_t)rup64((int64_t)(off + bytes), 256);
    return o;
  };
  const int rpad32 = r ? (int)rup64(r, 32) : 0, rpad16 = r ? (int)rup64(r, 16) : 0;
  b.off_bt = take(r ? (size_t)r * n * 2 : 0);
  b.off_gpart = take(r ? (size_t)((n + 511) / 512) * mpad * rpad32 * 4 : 0);
  b.off_gs = take(r ? (size_t)mpad * rpad16 * 2 : 0);
  b.total = off;
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
  // x_t and t = s x_t A^T (the forward's prepare)
  e = launch_linear_prepare(p, x, z, r ? lora_a : nullptr, lora_scale, ws, stream);
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
    hipLaunchKernelGGL(bwd_dx<4>, dim3((unsigned)ktiles, (unsigned)(mtiles / 4)), dim3(256), 0,
                       stream, a);
  else if (mtiles % 2 == 0)
    hipLaunchKernelGGL(bwd_dx<2>, dim3((unsigned)ktiles, (unsigned)(mtiles / 2)), dim3(256), 0,
                       stream, a);
  else
    hipLaunchKernelGGL(bwd_dx<1>, dim3((unsigned)ktiles, (unsigned)mtiles), dim3(256), 0, stream,
                       a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (r && da) {
    // dA[j, col] = sum_i gs[i, j] x_t[i, col]
    hipLaunchKernelGGL(outer_acc, dim3((unsigned)((p.k + 255) / 256), (unsigned)((r + 31) / 32)),
                       dim3(256), 0, stream, reinterpret_cast<const uint16_t*>(ws + p.off_xt),
                       p.k, gs, (int64_t)p.rpad16, p.m, p.k, r, da, (int64_t)1, p.k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (r && db) {
    // dB[col, j] = sum_i dy[i, col] t[i, j]
    hipLaunchKernelGGL(outer_acc, dim3((unsigned)((p.n + 255) / 256), (unsigned)((r + 31) / 32)),
                       dim3(256), 0, stream, dy, p.n,
                       reinterpret_cast<const uint16_t*>(ws + p.off_t), (int64_t)p.rpad16, p.m,
                       p.n, r, db, (int64_t)r, (int64_t)1);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace qerl
