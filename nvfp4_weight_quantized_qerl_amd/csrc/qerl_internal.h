// Host-side internals of libqerl: launch planning and kernel launchers.
// Not part of the public ABI (include/qerl.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "treduce.h"

namespace qerl {

// Number of compute units of the current device (cached; 256 on MI355X,
// and 256 when no device is visible so that sizing works on a host).
int device_cu_count();

// ---------------------------------------------------------------- quantizer
hipError_t launch_quantize(const uint16_t* w, int64_t n, int64_t k,
                           uint8_t* codes, uint8_t* scales, float* gscale,
                           int32_t* flag, hipStream_t stream);
// `count` tensors in count + 2 launches (the encode pass of one tensor runs
// beside the amax pass of the next); flag may be null, as may its entries.
hipError_t launch_quantize_batch(int count, const uint16_t* const* w, const int64_t* n,
                                 const int64_t* k, uint8_t* const* codes, uint8_t* const* scales,
                                 float* const* gscale, int32_t* const* flag, hipStream_t stream);

// MXFP4 (E8M0 scale per 32): quantize, and re-express the scales in the
// NVFP4 layout (E4M3 per 16 + FP32 S) so the NVFP4 kernels run it exactly.
hipError_t launch_quantize_mxfp4(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                                 uint8_t* scales, int32_t* flag, hipStream_t stream);
hipError_t launch_mxfp4_to_nvfp4(const uint8_t* codes, const uint8_t* s8, int64_t n, int64_t k,
                                 uint8_t* s4, float* gscale, int32_t* flag, hipStream_t stream);
// flag <- 1 if any NVFP4 block scale of [n, k/16] is not zero or a power of
// two (the condition of the power-of-two decode path), else 0.
hipError_t launch_check_pow2_scales(const uint8_t* scales, int64_t n, int64_t k, int32_t* flag,
                                   hipStream_t stream);

// -------------------------------------------------------------------- noise
// `count` vectors of length d, vector v with call id call0 + v * call_step
// and Philox counter word 2 = v * row_step, stored one after the other.
hipError_t launch_aqn_sample(uint64_t seed, uint64_t stream_id, uint64_t call0,
                             uint64_t call_step, uint64_t row_step, int64_t count,
                             double sigma, int64_t d, float* z, hipStream_t stream);

// ------------------------------------------------------------------ rmsnorm
// y = bf16((w + z) * x / sqrt(mean(x^2) + delta)) per row of x [m, d].
hipError_t launch_rmsnorm_noisy(const uint16_t* x, int64_t m, int64_t d, const uint16_t* w,
                                const float* z, float delta, uint16_t* y, hipStream_t stream);

// out = bf16(SiLU(gate) * up) from the fused gate/up output [m, 2 d].
hipError_t launch_swiglu(const uint16_t* gu, int64_t m, int64_t d, uint16_t* out,
                         hipStream_t stream);

// ------------------------------------------------------------------- linear
// Workspace layout and launch shapes for one (m, n, k, r).
struct LinearPlan {
  int64_t m, n, k;
  int r;
  int64_t mpad;        // m rounded up to 32: rows of x_t and t
  int rpad32;          // r rounded up to 32 (LoRA-down MFMA tiles), 0 if r == 0
  int rpad16;          // r rounded up to 16: row stride of t (bf16)
  int kchunks;         // K chunks of the LoRA-down partial sums
  int64_t kchunk;      // multiple of 16
  // decode main kernel (per m-chunk of at most 128 rows)
  int dec_mt;          // 32-row m tiles per launch: 1, 2 or 4
  int dec_nt;          // 32-row n subtiles per wave
  int dec_rows;        // weight rows per workgroup (<= 32 * dec_nt)
  int dec_groups;      // row groups = ceil(n / dec_rows)
  int dec_split;       // K splits across workgroups
  int64_t dec_kblk_per_split;  // 64-wide K blocks per split
  // single-pass 128-token contraction (k % 128 == 0): chunks of up to 128
  // rows with at least three 32-row tiles; the kernels above take the rest
  bool m128;
  bool tiled;          // the weight is in the tiled layout: every chunk runs the
                       // 128-token kernel
  int m128_groups;     // 256-row groups = ceil(n / 256)
  int m128_split;      // K splits across workgroups
  // every block scale is a power of two (MXFP4 in the NVFP4 layout): the
  // LDS-staged decode kernel may use its single-instruction dequantization
  bool pow2_scales;
  // a whole decode call whose first contraction launch splits K: the prepare
  // leaves the LoRA-down partials and that launch's extra workgroups sum
  // them into t (set by the caller after t_reduce_can_merge)
  bool t_in_contraction;
  // prefill main kernel
  int pf_tile_m, pf_tile_n;
  // workspace byte offsets
  size_t off_xt, off_tpart, off_t, off_sync, off_ypart, total;
  // off_sync: two words that the prepare of a whole call clears: the count
  // of reduction workgroups done and the wait-timeout flag of an unsplit
  // 128-token launch that also sums t (decode_m128.h, Args::tsync)
};

// tiled: the plan of the tiled-layout entry points (k % 128 == 0).
bool make_linear_plan(int64_t m, int64_t n, int64_t k, int r, LinearPlan* p, bool tiled = false);

// With swiglu_input, x is the fused gate/up output [m, 2k] and the layer
// input is bf16(SiLU(gate) * up), formed as the rows are loaded.  Without
// write_xt only t is produced (x_t is not stored; nothing is launched
// without a LoRA branch).
// z_rows: z is [m, k], one noise row per token (else [k], shared).
// Without reduce_t only the LoRA-down partials are written; the contraction
// launch then sums them into t (LinearPlan::t_in_contraction).
// clear_sync: two words set to zero by the launch (needs a LoRA branch or
// write_xt, so that a kernel is launched).
hipError_t launch_linear_prepare(const LinearPlan& p, const uint16_t* x,
                                 const float* z, const uint16_t* lora_a,
                                 float lora_scale, char* ws,
                                 hipStream_t stream, bool swiglu_input = false,
                                 bool write_xt = true, bool z_rows = false,
                                 bool reduce_t = true, unsigned* clear_sync = nullptr);

// Single-position attention stub: out[i, h dh + e] = v[i, (h / (hq / hkv)) dh + e]
// of qkv [m, (hq + 2 hkv) dh] (q, then k, then v heads).
hipError_t launch_attention_stub(const uint16_t* qkv, int64_t m, int hq, int hkv, int dh,
                                 uint16_t* out, hipStream_t stream);

// t = bf16(scale x a_rk^T) for x [m, k] (rows m..mpad-1 read as zero) and
// a_rk [r, k]: the LoRA-down kernels on any operands (partials [ceil(k/512),
// mpad, rup(r,32)] fp32 in tpart, t [mpad, rup(r,16)] bf16).
hipError_t launch_lora_down(const uint16_t* x, int64_t m, int64_t mpad, int64_t k,
                            const uint16_t* a_rk, int r, float scale, float* tpart,
                            uint16_t* t, hipStream_t stream);

// LoRA-down reduction: launch_linear_prepare writes the chunk partials
// s x_t A^T (tpart) and then t = bf16(sum of the partials) (launch_treduce).
hipError_t launch_treduce(const LinearPlan& p, char* ws, hipStream_t stream);
TReduceArgs treduce_args(const LinearPlan& p, char* ws);

// Whether the first contraction launch of a decode call has CU slots to
// spare, so that it can also sum the LoRA-down partials into t: when it
// splits K (the contraction does not read t then; the finish does), or
// when it is unsplit (its workgroups wait for t after their main loop, on
// the sync words, which the prepare clears: launch_linear_prepare
// clear_sync).
bool t_reduce_can_merge(const LinearPlan& p);

// K splits of the LDS-staged decode kernel: the planned split, capped at
// the number of 256-wide K blocks.
int lds_split(const LinearPlan& p);

// The contraction kernels read x_t and the LoRA-down t = bf16(s x_t A^T)
// that launch_linear_prepare left in the workspace.
hipError_t launch_linear_decode_main(const LinearPlan& p, const uint8_t* codes,
                                     const uint8_t* scales, const float* gscale,
                                     const uint16_t* lora_b, uint16_t* y, char* ws,
                                     hipStream_t stream);

// Decode contraction over m in chunks of at most 128 rows (also the
// fallback of the prefill entry point for shapes its tiles do not cover).
hipError_t run_decode_chunks(const LinearPlan& p, const uint8_t* codes,
                             const uint8_t* scales, const float* gscale,
                             const uint16_t* lora_b, uint16_t* y, char* ws,
                             hipStream_t stream);

// Tiled layout of the 128-token decode kernel (decode_m128.h): size and
// re-layout of a standard NVFP4 weight (k % 128 == 0).
size_t tile128_bytes(int64_t n, int64_t k);
hipError_t tile128(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k,
                   uint8_t* out, hipStream_t stream);

hipError_t launch_linear_prefill_main(const LinearPlan& p, const uint8_t* codes,
                                      const uint8_t* scales, const float* gscale,
                                      const uint16_t* lora_b, uint16_t* y, char* ws,
                                      hipStream_t stream);

// ----------------------------------------------------------------- backward
// Workspace of the backward: the forward prepare's LoRA-down partials and t
// (fwd.off_tpart, fwd.off_t; no x_t), then B^T [r, n], the partials of
// s dy B, gs = bf16(s dy B) [mpad, rpad16] and the dA / dB chunk partials.
struct BackwardPlan {
  LinearPlan fwd;
  int mchunks;         // 256-row chunks of the dA / dB sums over the tokens
  size_t off_bt, off_gpart, off_gs, off_opart, total;
};

BackwardPlan make_backward_plan(int64_t m, int64_t n, int64_t k, int r);

hipError_t launch_linear_backward(const BackwardPlan& b, const uint16_t* dy, const uint8_t* codes,
                                  const uint8_t* scales, const float* gscale, const uint16_t* x,
                                  const uint16_t* lora_a, const uint16_t* lora_b, float lora_scale,
                                  const float* z, uint16_t* dx, float* da, float* db, char* ws,
                                  hipStream_t stream);

}  // namespace qerl
