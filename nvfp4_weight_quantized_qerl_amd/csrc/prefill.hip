// Prefill contraction entry point: the LDS-tiled NVFP4 GEMM of
// prefill_kernel.h for m > 64, the decode contraction for fewer tokens.
#include <algorithm>

#include "prefill_kernel.h"
#include "qerl_internal.h"

namespace qerl {

namespace {

typedef void (*GemmKernel)(prefill::Args);

struct TileConfig {
  int bm, bn;
  GemmKernel kern;
  int threads;
  int wgs_per_cu;   // workgroups that share a CU (LDS and registers)
  int rate;         // relative tile throughput, measured at M = 4096 on the
                    // Qwen2.5-7B qkv and down shapes
};

// Candidate tiles: (waves M x N, wave tile WM x WN, waves per SIMD).  None
// spills inside its main loop: the 256 x 256 tile keeps one 8-byte value in
// scratch (12 bytes per lane), stored once before the K loop and reloaded
// once after it; the other two use no scratch.
const TileConfig kConfigs[] = {
    {256, 256, prefill::gemm<2, 4, 128, 64, 2>, 512, 1, 550},
    {256, 192, prefill::gemm<2, 2, 128, 96, 1>, 256, 1, 430},
    {128, 128, prefill::gemm<2, 2, 64, 64, 2>, 256, 2, 470},
};

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Estimated time = whole rounds of workgroups over the CU slots x work per
// round / tile throughput; the smallest wins, ties go to the earlier entry.
const TileConfig& pick_tile(int64_t m, int64_t n) {
  const int cu = device_cu_count();
  const TileConfig* best = &kConfigs[0];
  double best_cost = -1.0;
  for (const TileConfig& c : kConfigs) {
    const int64_t tiles = cdiv(m, c.bm) * cdiv(n, c.bn);
    const int64_t rounds = cdiv(tiles, (int64_t)cu * c.wgs_per_cu);
    const double cost = (double)rounds * c.bm * c.bn * c.wgs_per_cu / c.rate;
    if (best_cost < 0.0 || cost < best_cost) {
      best_cost = cost;
      best = &c;
    }
  }
  return *best;
}

}  // namespace

hipError_t launch_linear_prefill_main(const LinearPlan& p, const uint8_t* codes,
                                      const uint8_t* scales, const float* gscale,
                                      const uint16_t* lora_b, uint16_t* y, char* ws,
                                      hipStream_t stream) {
  if (p.m <= 64) return run_decode_chunks(p, codes, scales, gscale, lora_b, y, ws, stream);
  const TileConfig& tc = pick_tile(p.m, p.n);
  prefill::Args a;
  a.xt = reinterpret_cast<const uint16_t*>(ws + p.off_xt);
  a.codes = codes;
  a.scales = scales;
  a.gscale = gscale;
  a.r = (lora_b && p.r > 0) ? p.r : 0;
  a.t = a.r ? reinterpret_cast<const uint16_t*>(ws + p.off_t) : nullptr;
  a.lora_b = lora_b;
  a.y = y;
  a.m = p.m;
  a.mpad = p.mpad;
  a.n = p.n;
  a.k = p.k;
  a.rpad16 = p.rpad16;
  a.lora_vec = (a.r % 8 == 0) && ((reinterpret_cast<uintptr_t>(lora_b) & 15) == 0);
  a.tiles_n = (int)cdiv(p.n, tc.bn);
  const int64_t tiles = cdiv(p.m, tc.bm) * a.tiles_n;
  hipLaunchKernelGGL(tc.kern, dim3((unsigned)tiles), dim3(tc.threads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace qerl
