// C ABI of libqerl (declared and documented in include/qerl.h): argument
// validation on the host, then asynchronous launches on the caller's
// stream.  No call allocates, frees or synchronises.
#include <cmath>

#include "qerl.h"
#include "qerl_internal.h"

namespace {

bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

qerl_status from_hip(hipError_t e) { return e == hipSuccess ? QERL_OK : QERL_ERR_HIP; }

// Shared validation of the linear-layer arguments; fills the plan.
qerl_status check_linear(const void* x, int64_t m, const void* codes,
                         const void* scales, const float* gscale, int64_t n,
                         int64_t k, int32_t r, float lora_scale, const float* z,
                         const void* y, void* ws, size_t ws_bytes,
                         qerl::LinearPlan* plan, bool tiled = false) {
  if (!codes || !scales || !gscale || !y || !ws) return QERL_ERR_NULL;
  if (m < 1 || n < 1 || k < 16 || k % 16) return QERL_ERR_SHAPE;
  if (r < 0 || r > 128 || !std::isfinite(lora_scale)) return QERL_ERR_RANGE;
  if ((x && !aligned(x, 16)) || !aligned(codes, 16) || !aligned(gscale, 4) ||
      !aligned(y, 2) || (z && !aligned(z, 16)) || !aligned(ws, 256))
    return QERL_ERR_ALIGN;
  if (tiled && k % 128) return QERL_ERR_SHAPE;
  if (!qerl::make_linear_plan(m, n, k, r, plan, tiled)) return QERL_ERR_SHAPE;
  if (ws_bytes < plan->total) return QERL_ERR_WORKSPACE;
  return QERL_OK;
}

qerl_status check_prepare(const void* x, const void* lora_a, int32_t r) {
  if (!x) return QERL_ERR_NULL;
  if (r > 0 && !lora_a) return QERL_ERR_NULL;
  if (lora_a && !aligned(lora_a, 16)) return QERL_ERR_ALIGN;
  return QERL_OK;
}

}  // namespace

extern "C" {

const char* qerl_status_string(int status) {
  switch (status) {
    case QERL_OK: return "QERL_OK";
    case QERL_ERR_NULL: return "QERL_ERR_NULL: a required pointer is NULL";
    case QERL_ERR_SHAPE: return "QERL_ERR_SHAPE: a size is out of range or k % 16 != 0";
    case QERL_ERR_ALIGN: return "QERL_ERR_ALIGN: a pointer is not aligned as required";
    case QERL_ERR_RANGE: return "QERL_ERR_RANGE: a scalar argument is out of range";
    case QERL_ERR_WORKSPACE: return "QERL_ERR_WORKSPACE: the workspace is too small";
    case QERL_ERR_HIP: return "QERL_ERR_HIP: the HIP runtime reported an error";
    default: return "unknown qerl_status";
  }
}

int qerl_abi_version(void) { return 12; }

qerl_status qerl_quantize_nvfp4(const void* w_bf16, int64_t n, int64_t k, void* codes,
                                void* scales, float* gscale, int32_t* nonfinite_flag,
                                void* stream) {
  if (!w_bf16 || !codes || !scales || !gscale) return QERL_ERR_NULL;
  if (n < 1 || k < 16 || k % 16) return QERL_ERR_SHAPE;
  if (!aligned(w_bf16, 16) || !aligned(codes, 16) || !aligned(gscale, 4) ||
      (nonfinite_flag && !aligned(nonfinite_flag, 4)))
    return QERL_ERR_ALIGN;
  return from_hip(qerl::launch_quantize(
      static_cast<const uint16_t*>(w_bf16), n, k, static_cast<uint8_t*>(codes),
      static_cast<uint8_t*>(scales), gscale, nonfinite_flag,
      static_cast<hipStream_t>(stream)));
}

qerl_status qerl_quantize_nvfp4_batch(int32_t count, const void* const* w_bf16, const int64_t* n,
                                      const int64_t* k, void* const* codes, void* const* scales,
                                      float* const* gscale, int32_t* const* nonfinite_flag,
                                      void* stream) {
  if (count < 1 || count > (1 << 20)) return QERL_ERR_SHAPE;
  if (!w_bf16 || !n || !k || !codes || !scales || !gscale) return QERL_ERR_NULL;
  for (int32_t i = 0; i < count; ++i) {
    if (!w_bf16[i] || !codes[i] || !scales[i] || !gscale[i]) return QERL_ERR_NULL;
    if (n[i] < 1 || k[i] < 16 || k[i] % 16) return QERL_ERR_SHAPE;
    if (!aligned(w_bf16[i], 16) || !aligned(codes[i], 16) || !aligned(gscale[i], 4) ||
        (nonfinite_flag && nonfinite_flag[i] && !aligned(nonfinite_flag[i], 4)))
      return QERL_ERR_ALIGN;
  }
  return from_hip(qerl::launch_quantize_batch(
      count, reinterpret_cast<const uint16_t* const*>(w_bf16), n, k,
      reinterpret_cast<uint8_t* const*>(codes), reinterpret_cast<uint8_t* const*>(scales), gscale,
      nonfinite_flag, static_cast<hipStream_t>(stream)));
}

qerl_status qerl_aqn_sigma(double sigma_start, double sigma_end, int32_t num_stages,
                           int32_t stage, double* sigma_out) {
  if (!sigma_out) return QERL_ERR_NULL;
  if (!(sigma_start > 0.0) || !(sigma_end > 0.0) || !std::isfinite(sigma_start) ||
      !std::isfinite(sigma_end) || num_stages < 1 || stage < 0 || stage > num_stages)
    return QERL_ERR_RANGE;
  if (stage == 0) {
    *sigma_out = 0.0;
  } else if (num_stages == 1) {
    *sigma_out = sigma_start;
  } else {
    const double ratio = sigma_end / sigma_start;
    *sigma_out = sigma_start *
                 std::pow(ratio, (double)(stage - 1) / (double)(num_stages - 1));
  }
  return QERL_OK;
}

qerl_status qerl_quantize_mxfp4(const void* w_bf16, int64_t n, int64_t k, void* codes,
                                void* scales_e8m0, int32_t* nonfinite_flag, void* stream) {
  if (!w_bf16 || !codes || !scales_e8m0) return QERL_ERR_NULL;
  if (n < 1 || k < 32 || k % 32) return QERL_ERR_SHAPE;
  if (!aligned(w_bf16, 16) || !aligned(codes, 16) || (nonfinite_flag && !aligned(nonfinite_flag, 4)))
    return QERL_ERR_ALIGN;
  return from_hip(qerl::launch_quantize_mxfp4(
      static_cast<const uint16_t*>(w_bf16), n, k, static_cast<uint8_t*>(codes),
      static_cast<uint8_t*>(scales_e8m0), nonfinite_flag, static_cast<hipStream_t>(stream)));
}

qerl_status qerl_mxfp4_to_nvfp4(const void* codes, const void* scales_e8m0, int64_t n, int64_t k,
                                void* scales_e4m3, float* gscale, int32_t* range_flag,
                                void* stream) {
  if (!codes || !scales_e8m0 || !scales_e4m3 || !gscale) return QERL_ERR_NULL;
  if (n < 1 || k < 32 || k % 32) return QERL_ERR_SHAPE;
  if (!aligned(codes, 16) || !aligned(gscale, 4) || (range_flag && !aligned(range_flag, 4)))
    return QERL_ERR_ALIGN;
  return from_hip(qerl::launch_mxfp4_to_nvfp4(
      static_cast<const uint8_t*>(codes), static_cast<const uint8_t*>(scales_e8m0), n, k,
      static_cast<uint8_t*>(scales_e4m3), gscale, range_flag, static_cast<hipStream_t>(stream)));
}

qerl_status qerl_aqn_sigma_schedule(int32_t mode, double sigma_start, double sigma_end,
                                    int32_t num_stages, int32_t stage, double* sigma_out) {
  if (!sigma_out) return QERL_ERR_NULL;
  if (mode < QERL_SCHEDULE_EXPONENTIAL || mode > QERL_SCHEDULE_LOGARITHMIC)
    return QERL_ERR_RANGE;
  if (mode == QERL_SCHEDULE_EXPONENTIAL)
    return qerl_aqn_sigma(sigma_start, sigma_end, num_stages, stage, sigma_out);
  if (!(sigma_start > 0.0) || !(sigma_end > 0.0) || !std::isfinite(sigma_start) ||
      !std::isfinite(sigma_end) || num_stages < 1 || stage < 0 || stage > num_stages)
    return QERL_ERR_RANGE;
  if (stage == 0) {
    *sigma_out = 0.0;
    return QERL_OK;
  }
  if (num_stages == 1) {
    *sigma_out = sigma_start;
    return QERL_OK;
  }
  const double frac = (double)(stage - 1) / (double)(num_stages - 1);
  const double drop = sigma_start - sigma_end;
  switch (mode) {
    case QERL_SCHEDULE_LINEAR:
      *sigma_out = sigma_start - drop * frac;
      break;
    case QERL_SCHEDULE_COSINE:
      *sigma_out = sigma_end + 0.5 * drop * (1.0 + std::cos(M_PI * frac));
      break;
    default:  // QERL_SCHEDULE_LOGARITHMIC
      *sigma_out = sigma_start - drop * (std::log((double)stage) / std::log((double)num_stages));
      break;
  }
  return QERL_OK;
}

qerl_status qerl_aqn_sample(uint64_t seed, uint64_t stream_id, uint64_t call_id,
                            double sigma, int64_t d, float* z_out, void* stream) {
  if (!z_out) return QERL_ERR_NULL;
  if (d < 1) return QERL_ERR_SHAPE;
  if (!(sigma >= 0.0) || !std::isfinite(sigma)) return QERL_ERR_RANGE;
  if (!aligned(z_out, 4)) return QERL_ERR_ALIGN;
  return from_hip(qerl::launch_aqn_sample(seed, stream_id, call_id, 0, 0, 1, sigma, d, z_out,
                                          static_cast<hipStream_t>(stream)));
}

qerl_status qerl_aqn_sample_batch(uint64_t seed, uint64_t stream_id, uint64_t call_id0,
                                  uint64_t call_stride, int64_t count, double sigma, int64_t d,
                                  float* z_out, void* stream) {
  if (!z_out) return QERL_ERR_NULL;
  if (d < 1 || count < 1 || count > 65535) return QERL_ERR_SHAPE;
  if (!(sigma >= 0.0) || !std::isfinite(sigma)) return QERL_ERR_RANGE;
  if (!aligned(z_out, 4)) return QERL_ERR_ALIGN;
  return from_hip(qerl::launch_aqn_sample(seed, stream_id, call_id0, call_stride, 0, count,
                                          sigma, d, z_out, static_cast<hipStream_t>(stream)));
}

qerl_status qerl_rmsnorm_noisy(const void* x, int64_t m, int64_t d, const void* w,
                               const float* z, float delta, void* y, void* stream) {
  if (!x || !w || !y) return QERL_ERR_NULL;
  if (m < 1 || d < 8 || d % 8) return QERL_ERR_SHAPE;
  if (!(delta >= 0.0f) || !std::isfinite(delta)) return QERL_ERR_RANGE;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16) || (z && !aligned(z, 16)))
    return QERL_ERR_ALIGN;
  return from_hip(qerl::launch_rmsnorm_noisy(
      static_cast<const uint16_t*>(x), m, d, static_cast<const uint16_t*>(w), z, delta,
      static_cast<uint16_t*>(y), static_cast<hipStream_t>(stream)));
}

qerl_status qerl_swiglu(const void* gate_up, int64_t m, int64_t d, void* out, void* stream) {
  if (!gate_up || !out) return QERL_ERR_NULL;
  if (m < 1 || d < 8 || d % 8) return QERL_ERR_SHAPE;
  if (!aligned(gate_up, 16) || !aligned(out, 16)) return QERL_ERR_ALIGN;
  return from_hip(qerl::launch_swiglu(static_cast<const uint16_t*>(gate_up), m, d,
                                      static_cast<uint16_t*>(out),
                                      static_cast<hipStream_t>(stream)));
}

size_t qerl_linear_backward_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t r) {
  if (m < 1 || n < 16 || n % 16 || k < 16 || k % 16 || r < 0 || r > 128) return 0;
  return qerl::make_backward_plan(m, n, k, r).total;
}

qerl_status qerl_linear_backward(const void* dy, int64_t m, const void* codes,
                                 const void* scales, const float* gscale, int64_t n, int64_t k,
                                 const void* x, const void* lora_a, const void* lora_b,
                                 int32_t r, float lora_scale, const float* z, void* dx,
                                 float* da, float* db, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (!dy || !codes || !scales || !gscale || !x || !dx || !workspace) return QERL_ERR_NULL;
  if (r > 0 && (!lora_a) != (!lora_b)) return QERL_ERR_NULL;
  if (m < 1 || n < 16 || n % 16 || k < 16 || k % 16) return QERL_ERR_SHAPE;
  if (r < 0 || r > 128 || !std::isfinite(lora_scale)) return QERL_ERR_RANGE;
  const int32_t r_eff = (r > 0 && lora_a && lora_b) ? r : 0;
  if (!aligned(dy, 16) || !aligned(x, 16) || !aligned(codes, 16) || !aligned(gscale, 4) ||
      !aligned(dx, 2) || (z && !aligned(z, 16)) || (r_eff && !aligned(lora_a, 16)) ||
      (da && !aligned(da, 4)) || (db && !aligned(db, 4)) || !aligned(workspace, 256))
    return QERL_ERR_ALIGN;
  const qerl::BackwardPlan plan = qerl::make_backward_plan(m, n, k, r_eff);
  if (workspace_bytes < plan.total) return QERL_ERR_WORKSPACE;
  return from_hip(qerl::launch_linear_backward(
      plan, static_cast<const uint16_t*>(dy), static_cast<const uint8_t*>(codes),
      static_cast<const uint8_t*>(scales), gscale, static_cast<const uint16_t*>(x),
      static_cast<const uint16_t*>(r_eff ? lora_a : nullptr),
      static_cast<const uint16_t*>(r_eff ? lora_b : nullptr), lora_scale, z,
      static_cast<uint16_t*>(dx), r_eff ? da : nullptr, r_eff ? db : nullptr,
      static_cast<char*>(workspace), static_cast<hipStream_t>(stream)));
}

size_t qerl_linear_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t r) {
  qerl::LinearPlan p;
  if (!qerl::make_linear_plan(m, n, k, r, &p)) return 0;
  return p.total;
}

static qerl_status linear_full(bool prefill, const void* x, int64_t m, const void* codes,
                               const void* scales, const float* gscale, int64_t n,
                               int64_t k, const void* lora_a, const void* lora_b,
                               int32_t r, float lora_scale, const float* z, void* y,
                               void* workspace, size_t workspace_bytes, void* stream,
                               bool pow2 = false, bool swiglu = false, bool tiled = false,
                               bool z_rows = false) {
  if (!x) return QERL_ERR_NULL;
  if (r > 0 && (!lora_a) != (!lora_b)) return QERL_ERR_NULL;
  const int32_t r_eff = (r > 0 && lora_a && lora_b) ? r : 0;
  if (r < 0 || r > 128) return QERL_ERR_RANGE;
  qerl::LinearPlan plan;
  qerl_status s = check_linear(x, m, codes, scales, gscale, n, k, r_eff, lora_scale, z, y,
                               workspace, workspace_bytes, &plan, tiled);
  if (s != QERL_OK) return s;
  s = check_prepare(x, r_eff ? lora_a : nullptr, r_eff);
  if (s != QERL_OK) return s;
  plan.pow2_scales = pow2;
  // When the first contraction launch splits K, its extra workgroups sum the
  // LoRA-down partials into t, which saves the reduction its own launch.
  plan.t_in_contraction =
      r_eff > 0 && (!prefill || plan.m <= 64) && qerl::t_reduce_can_merge(plan);
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  hipError_t e = qerl::launch_linear_prepare(
      plan, static_cast<const uint16_t*>(x), z, static_cast<const uint16_t*>(lora_a), lora_scale,
      ws, st, swiglu, true, z_rows, !plan.t_in_contraction,
      plan.t_in_contraction ? reinterpret_cast<unsigned*>(ws + plan.off_sync) : nullptr);
  if (e != hipSuccess) return QERL_ERR_HIP;
  const uint8_t* c = static_cast<const uint8_t*>(codes);
  const uint8_t* sc = static_cast<const uint8_t*>(scales);
  const uint16_t* b = r_eff ? static_cast<const uint16_t*>(lora_b) : nullptr;
  uint16_t* yy = static_cast<uint16_t*>(y);
  e = prefill ? qerl::launch_linear_prefill_main(plan, c, sc, gscale, b, yy, ws, st)
              : qerl::launch_linear_decode_main(plan, c, sc, gscale, b, yy, ws, st);
  return from_hip(e);
}

qerl_status qerl_linear_decode(const void* x, int64_t m, const void* codes,
                               const void* scales, const float* gscale, int64_t n,
                               int64_t k, const void* lora_a, const void* lora_b,
                               int32_t r, float lora_scale, const float* z, void* y,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return linear_full(false, x, m, codes, scales, gscale, n, k, lora_a, lora_b, r,
                     lora_scale, z, y, workspace, workspace_bytes, stream);
}

qerl_status qerl_linear_decode_swiglu(const void* gate_up, int64_t m, const void* codes,
                                      const void* scales, const float* gscale, int64_t n,
                                      int64_t k, const void* lora_a, const void* lora_b,
                                      int32_t r, float lora_scale, const float* z, void* y,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  return linear_full(false, gate_up, m, codes, scales, gscale, n, k, lora_a, lora_b, r,
                     lora_scale, z, y, workspace, workspace_bytes, stream, false, true);
}

qerl_status qerl_linear_prefill(const void* x, int64_t m, const void* codes,
                                const void* scales, const float* gscale, int64_t n,
                                int64_t k, const void* lora_a, const void* lora_b,
                                int32_t r, float lora_scale, const float* z, void* y,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return linear_full(true, x, m, codes, scales, gscale, n, k, lora_a, lora_b, r,
                     lora_scale, z, y, workspace, workspace_bytes, stream);
}

qerl_status qerl_linear_prepare(const void* x, int64_t m, int64_t n, int64_t k,
                                const void* lora_a, int32_t r, float lora_scale,
                                const float* z, void* workspace, size_t workspace_bytes,
                                void* stream) {
  if (!x || !workspace) return QERL_ERR_NULL;
  if (m < 1 || n < 1 || k < 16 || k % 16) return QERL_ERR_SHAPE;
  if (r < 0 || r > 128 || !std::isfinite(lora_scale)) return QERL_ERR_RANGE;
  qerl_status s = check_prepare(x, lora_a, r);
  if (s != QERL_OK) return s;
  if (!aligned(x, 16) || (z && !aligned(z, 16)) || !aligned(workspace, 256))
    return QERL_ERR_ALIGN;
  qerl::LinearPlan plan;
  if (!qerl::make_linear_plan(m, n, k, r, &plan)) return QERL_ERR_SHAPE;
  // It writes x_t, the LoRA-down partials and t, which come first in the
  // workspace of every linear entry point (standard or tiled).
  if (workspace_bytes < plan.off_ypart) return QERL_ERR_WORKSPACE;
  return from_hip(qerl::launch_linear_prepare(
      plan, static_cast<const uint16_t*>(x), z, static_cast<const uint16_t*>(lora_a),
      lora_scale, static_cast<char*>(workspace), static_cast<hipStream_t>(stream)));
}

static qerl_status linear_prepared(bool prefill, int64_t m, const void* codes,
                                   const void* scales, const float* gscale, int64_t n,
                                   int64_t k, const void* lora_b, int32_t r, void* y,
                                   void* workspace, size_t workspace_bytes, void* stream,
                                   bool pow2 = false, bool tiled = false) {
  if (r > 0 && !lora_b) return QERL_ERR_NULL;
  qerl::LinearPlan plan;
  qerl_status s = check_linear(nullptr, m, codes, scales, gscale, n, k, r, 1.0f, nullptr, y,
                               workspace, workspace_bytes, &plan, tiled);
  if (s != QERL_OK) return s;
  plan.pow2_scales = pow2;
  const uint8_t* c = static_cast<const uint8_t*>(codes);
  const uint8_t* sc = static_cast<const uint8_t*>(scales);
  const uint16_t* b = r > 0 ? static_cast<const uint16_t*>(lora_b) : nullptr;
  uint16_t* yy = static_cast<uint16_t*>(y);
  char* ws = static_cast<char*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return from_hip(prefill ? qerl::launch_linear_prefill_main(plan, c, sc, gscale, b, yy, ws, st)
                          : qerl::launch_linear_decode_main(plan, c, sc, gscale, b, yy, ws, st));
}

qerl_status qerl_linear_decode_prepared(int64_t m, const void* codes, const void* scales,
                                        const float* gscale, int64_t n, int64_t k,
                                        const void* lora_b, int32_t r, void* y,
                                        void* workspace, size_t workspace_bytes,
                                        void* stream) {
  return linear_prepared(false, m, codes, scales, gscale, n, k, lora_b, r, y, workspace,
                         workspace_bytes, stream);
}

qerl_status qerl_linear_prefill_prepared(int64_t m, const void* codes, const void* scales,
                                         const float* gscale, int64_t n, int64_t k,
                                         const void* lora_b, int32_t r, void* y,
                                         void* workspace, size_t workspace_bytes,
                                         void* stream) {
  return linear_prepared(true, m, codes, scales, gscale, n, k, lora_b, r, y, workspace,
                         workspace_bytes, stream);
}

qerl_status qerl_nvfp4_check_pow2_scales(const void* scales, int64_t n, int64_t k,
                                         int32_t* flag, void* stream) {
  if (!scales || !flag) return QERL_ERR_NULL;
  if (n < 1 || k < 16 || k % 16) return QERL_ERR_SHAPE;
  if (!aligned(flag, 4)) return QERL_ERR_ALIGN;
  return from_hip(qerl::launch_check_pow2_scales(static_cast<const uint8_t*>(scales), n, k, flag,
                                                 static_cast<hipStream_t>(stream)));
}

qerl_status qerl_linear_decode_mxfp4(const void* x, int64_t m, const void* codes,
                                     const void* scales, const float* gscale, int64_t n,
                                     int64_t k, const void* lora_a, const void* lora_b,
                                     int32_t r, float lora_scale, const float* z, void* y,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  return linear_full(false, x, m, codes, scales, gscale, n, k, lora_a, lora_b, r, lora_scale, z,
                     y, workspace, workspace_bytes, stream, true);
}

qerl_status qerl_linear_decode_prepared_mxfp4(int64_t m, const void* codes, const void* scales,
                                              const float* gscale, int64_t n, int64_t k,
                                              const void* lora_b, int32_t r, void* y,
                                              void* workspace, size_t workspace_bytes,
                                              void* stream) {
  return linear_prepared(false, m, codes, scales, gscale, n, k, lora_b, r, y, workspace,
                         workspace_bytes, stream, true);
}

qerl_status qerl_aqn_sample_rows(uint64_t seed, uint64_t stream_id, uint64_t call_id,
                                 double sigma, int64_t m, int64_t d, float* z_out,
                                 void* stream) {
  if (!z_out) return QERL_ERR_NULL;
  if (d < 1 || m < 1 || m > 65535) return QERL_ERR_SHAPE;
  if (!(sigma >= 0.0) || !std::isfinite(sigma)) return QERL_ERR_RANGE;
  if (!aligned(z_out, 4)) return QERL_ERR_ALIGN;
  return from_hip(qerl::launch_aqn_sample(seed, stream_id, call_id, 0, 1, m, sigma, d, z_out,
                                          static_cast<hipStream_t>(stream)));
}

qerl_status qerl_linear_decode_rownoise(const void* x, int64_t m, const void* codes,
                                        const void* scales, const float* gscale, int64_t n,
                                        int64_t k, const void* lora_a, const void* lora_b,
                                        int32_t r, float lora_scale, const float* z_rows,
                                        void* y, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  if (!z_rows) return QERL_ERR_NULL;
  return linear_full(false, x, m, codes, scales, gscale, n, k, lora_a, lora_b, r, lora_scale,
                     z_rows, y, workspace, workspace_bytes, stream, false, false, false, true);
}

qerl_status qerl_linear_prefill_rownoise(const void* x, int64_t m, const void* codes,
                                         const void* scales, const float* gscale, int64_t n,
                                         int64_t k, const void* lora_a, const void* lora_b,
                                         int32_t r, float lora_scale, const float* z_rows,
                                         void* y, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  if (!z_rows) return QERL_ERR_NULL;
  return linear_full(true, x, m, codes, scales, gscale, n, k, lora_a, lora_b, r, lora_scale,
                     z_rows, y, workspace, workspace_bytes, stream, false, false, false, true);
}

qerl_status qerl_attention_stub(const void* qkv, int64_t m, int32_t n_q_heads,
                                int32_t n_kv_heads, int32_t head_dim, void* out, void* stream) {
  if (!qkv || !out) return QERL_ERR_NULL;
  if (m < 1 || n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads || head_dim < 8 ||
      head_dim % 8)
    return QERL_ERR_SHAPE;
  if (!aligned(qkv, 16) || !aligned(out, 16)) return QERL_ERR_ALIGN;
  return from_hip(qerl::launch_attention_stub(static_cast<const uint16_t*>(qkv), m, n_q_heads,
                                              n_kv_heads, head_dim, static_cast<uint16_t*>(out),
                                              static_cast<hipStream_t>(stream)));
}

size_t qerl_nvfp4_tile128_bytes(int64_t n, int64_t k) {
  if (n < 1 || k < 128 || k % 128) return 0;
  return qerl::tile128_bytes(n, k);
}

qerl_status qerl_nvfp4_tile128(const void* codes, const void* scales, int64_t n, int64_t k,
                               void* tiled, void* stream) {
  if (!codes || !scales || !tiled) return QERL_ERR_NULL;
  if (n < 1 || k < 128 || k % 128) return QERL_ERR_SHAPE;
  if (((n + 31) / 32) * (k / 128) * 2304 >= ((int64_t)1 << 31)) return QERL_ERR_SHAPE;
  if (!aligned(codes, 16) || !aligned(tiled, 16)) return QERL_ERR_ALIGN;
  return from_hip(qerl::tile128(static_cast<const uint8_t*>(codes),
                                static_cast<const uint8_t*>(scales), n, k,
                                static_cast<uint8_t*>(tiled), static_cast<hipStream_t>(stream)));
}

size_t qerl_linear_tiled_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t r) {
  qerl::LinearPlan p;
  if (k % 128 || !qerl::make_linear_plan(m, n, k, r, &p, true)) return 0;
  return p.total;
}

qerl_status qerl_linear_decode_tiled(const void* x, int64_t m, const void* tiled,
                                     const float* gscale, int64_t n, int64_t k,
                                     const void* lora_a, const void* lora_b, int32_t r,
                                     float lora_scale, const float* z, void* y,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  return linear_full(false, x, m, tiled, tiled, gscale, n, k, lora_a, lora_b, r, lora_scale, z,
                     y, workspace, workspace_bytes, stream, false, false, true);
}

qerl_status qerl_linear_decode_tiled_prepared(int64_t m, const void* tiled, const float* gscale,
                                              int64_t n, int64_t k, const void* lora_b,
                                              int32_t r, void* y, void* workspace,
                                              size_t workspace_bytes, void* stream) {
  return linear_prepared(false, m, tiled, tiled, gscale, n, k, lora_b, r, y, workspace,
                         workspace_bytes, stream, false, true);
}

}  // extern "C"
