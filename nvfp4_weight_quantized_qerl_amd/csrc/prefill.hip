// Prefill contraction entry point.  Until the LDS-tiled kernel covers a
// shape, the prefill path runs the decode contraction over m in chunks of
// 128 rows (same arithmetic, same result).
#include "qerl_internal.h"

namespace qerl {

hipError_t launch_linear_prefill_main(const LinearPlan& p, const uint8_t* codes,
                                      const uint8_t* scales, const float* gscale,
                                      const uint16_t* lora_b, uint16_t* y, char* ws,
                                      hipStream_t stream) {
  return run_decode_chunks(p, codes, scales, gscale, lora_b, y, ws, stream);
}

}  // namespace qerl
