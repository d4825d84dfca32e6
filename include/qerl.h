/*
 * qerl.h -- C ABI of the NVFP4 weight-only linear layer with a LoRA side
 * branch and Adaptive Quantization Noise (AQN), for AMD Instinct MI355X
 * (gfx950).
 *
 * The method is QeRL's rollout-phase linear layer, as described on the
 * page "QeRL: Beyond Efficiency -- Quantization-enhanced Reinforcement
 * Learning for LLMs" (the long summary page; cited below as
 * [QeRL summary, <section>, <equation>]).
 *
 * Conventions shared by every call
 *   - Tensors are plain device pointers owned by the caller.  The library
 *     never allocates, frees or retains them.
 *   - bf16 tensors are passed as pointers to their 16-bit patterns.
 *   - Matrices are row-major.  A weight W has the nn.Linear layout
 *     [n = output features, k = input features]; activations x are [m, k];
 *     outputs y are [m, n].
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every device call is asynchronous on that stream: it returns after
 *     validating its arguments and enqueueing its kernels, with no host
 *     synchronisation.  Device faults surface at the caller's next sync.
 *   - The return value reports host-side validation and launch errors
 *     only (qerl_status).  On an error nothing has been enqueued.
 *   - Calls are reentrant and thread-safe; the library keeps no mutable
 *     global state besides a per-process cache of device properties (and
 *     the per-device scratch array of qerl_linear_decode_noalloc, whose
 *     calls must not overlap on one GPU).
 *
 * NVFP4 storage [QeRL summary, §3.4, Eq. 6: W_hat = S_FP32 * (S_E4M3 (.)
 * W_tilde), one E4M3 scale per block of 16 contiguous elements and one
 * FP32 scale per tensor]:
 *   codes  uint8 [n, k/2]   two E2M1 codes per byte, the even k in the low
 *                           nibble; code bit 3 = sign, bits 2..0 index the
 *                           magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 [§3.4,
 *                           E2M1 level list]
 *   scales uint8 [n, k/16]  OCP FP8 E4M3 (bias 7, max 448) bit patterns;
 *                           scale j covers k = 16j .. 16j+15 of its row
 *   gscale float [1]        S_FP32, in device memory
 */
#ifndef QERL_H
#define QERL_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define QERL_API __attribute__((visibility("default")))
#else
#define QERL_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QERL_OK = 0,
  QERL_ERR_NULL = 1,      /* a required pointer is NULL                    */
  QERL_ERR_SHAPE = 2,     /* a size is out of range or k % 16 != 0         */
  QERL_ERR_ALIGN = 3,     /* a device pointer is not aligned as required   */
  QERL_ERR_RANGE = 4,     /* a scalar argument is out of range             */
  QERL_ERR_WORKSPACE = 5, /* the workspace is smaller than required        */
  QERL_ERR_HIP = 6        /* the HIP runtime refused a launch or a query   */
} qerl_status;

/* Human-readable name of a status code.  Never returns NULL. */
QERL_API const char* qerl_status_string(int status);

/* Version of this ABI; bumped when a signature or a layout changes. */
QERL_API int qerl_abi_version(void);

/*
 * qerl_quantize_nvfp4 -- bf16 weight [n, k] -> NVFP4 (codes, scales, S).
 *
 * Follows Eq. 6 [QeRL summary, §3.4] read as a quantizer (the pages print
 * only the dequantization; the rounding rules below are this library's
 * reading of Eq. 1's "scale = range / q_max" applied at both levels):
 *   amax  = max |w| over the tensor
 *   S     = RN_fp32(amax / (6 * 448))
 *   s_b   = RNE_E4M3(amax_b / (6 * S)), saturating at 448, per block
 *   code  = sign(w) | RNE_E2M1(|w| / (s_b * S)), saturating at 6, ties to
 *           the even code
 * where the quotients are taken exactly (the result is bit-exact and
 * unique).  S == 0 (all-zero tensor or underflow) gives zero scales and
 * sign-only codes.
 *
 *   w_bf16         device, [n, k] bf16, 16-byte aligned
 *   n, k           n >= 1, k >= 16, k % 16 == 0
 *   codes          device out, [n, k/2] bytes, 16-byte aligned
 *   scales         device out, [n, k/16] bytes
 *   gscale         device out, 1 float (also used as the amax
 *                  accumulator while the call runs)
 *   nonfinite_flag device out, nullable; set to 1 if w holds an inf or a
 *                  NaN, else 0.  When it is 1, codes/scales/gscale are
 *                  unspecified.
 * Three kernels are enqueued (reset, amax, encode).
 */
QERL_API qerl_status qerl_quantize_nvfp4(const void* w_bf16, int64_t n, int64_t k,
                                void* codes, void* scales, float* gscale,
                                int32_t* nonfinite_flag, void* stream);

/*
 * qerl_quantize_nvfp4_batch -- qerl_quantize_nvfp4 of `count` tensors in
 * one call, each with the same result (bit for bit) as its own call.  The
 * pages quantize a model's weights once, when it is loaded, and keep them
 * [QeRL summary, §3.2 and §3.3]; this is that bulk step.  count + 2 kernels
 * are enqueued: one launch per tensor runs the encode pass of tensor i
 * beside the amax pass of tensor i + 1, so tensor i's second read mostly
 * hits the last-level cache and no launch is spent on a separate pass.
 *   count              1 <= count <= 1 << 20
 *   w_bf16, n, k,      host arrays of `count` entries; entry i is as the
 *   codes, scales,     arguments of qerl_quantize_nvfp4 (device pointers,
 *   gscale             same shapes and alignment).  No two tensors' outputs
 *                      may overlap.
 *   nonfinite_flag     host array of `count` device pointers (entries
 *                      nullable), or NULL for no flags
 * Every entry is checked before anything is enqueued; the first bad entry
 * decides the status.  The host arrays are read during the call only.
 */
QERL_API qerl_status qerl_quantize_nvfp4_batch(int32_t count, const void* const* w_bf16,
                                               const int64_t* n, const int64_t* k,
                                               void* const* codes, void* const* scales,
                                               float* const* gscale,
                                               int32_t* const* nonfinite_flag, void* stream);

/*
 * qerl_aqn_sigma -- host, pure.  The AQN exponential decay schedule
 * [QeRL summary, §3.4, Eq. 8]:
 *   sigma(k) = sigma_start * (sigma_end / sigma_start)^((k-1)/(K-1)),
 * k = 1..K, with sigma(0) = 0 (stage 0 carries only quantization noise,
 * §3.4 "Stage 0") and sigma(1) = sigma_start when K == 1.
 *   sigma_start, sigma_end  > 0 (the paper uses 1e-2 and 5e-4)
 *   num_stages (K)          >= 1 (the paper uses 10)
 *   stage (k)               0 <= k <= K
 *   sigma_out               host out, non-NULL
 */
QERL_API qerl_status qerl_aqn_sigma(double sigma_start, double sigma_end,
                           int32_t num_stages, int32_t stage,
                           double* sigma_out);

/*
 * qerl_quantize_mxfp4 -- the MXFP4 variant of the weight format [QeRL
 * summary, §3.4, the formats compared beside NVFP4: E2M1 elements sharing
 * an E8M0 scale per 32]; the scale rule is the OCP Microscaling v1.0 one:
 *   X = 2^(floor(log2 amax_b) - 2) per 32 contiguous elements of a row,
 *   stored as the byte exponent + 127 (clamped to 0..254; 0 for a zero block),
 *   code = sign | RNE_E2M1(|w| / X), ties to even, saturating at 6.
 * Codes pack as for NVFP4 (two per byte, the even k in the low nibble).
 *   w_bf16          device, [n, k] bf16, 16-byte aligned
 *   n, k            n >= 1, k >= 32, k % 32 == 0
 *   codes           device out, [n, k/2] bytes, 16-byte aligned
 *   scales_e8m0     device out, [n, k/32] bytes
 *   nonfinite_flag  device out, nullable: 1 if w holds an inf or a NaN
 *                   (the outputs are then unspecified), else 0
 */
QERL_API qerl_status qerl_quantize_mxfp4(const void* w_bf16, int64_t n, int64_t k, void* codes,
                                         void* scales_e8m0, int32_t* nonfinite_flag,
                                         void* stream);

/*
 * qerl_mxfp4_to_nvfp4 -- the same MXFP4 weight in this library's NVFP4
 * layout, exactly: gscale = 2^(E_max - 8) (E_max the largest block
 * exponent) and each 16-element block scale the E4M3 power of two
 * 2^(e - E_max + 8) of its 32-block exponent e.  The codes are used as they
 * are, so (codes, scales_e4m3, gscale) go straight to qerl_linear_decode /
 * qerl_linear_prefill / qerl_linear_backward.  A block more than 17
 * octaves below the largest has no E4M3 power of two: its scale is written
 * as 0 and, if any of its codes is nonzero, *range_flag is set to 1.
 *   codes, scales_e8m0   from qerl_quantize_mxfp4 ([n, k/2], [n, k/32])
 *   scales_e4m3          device out, [n, k/16] bytes
 *   gscale               device out, 1 float
 *   range_flag           device out, nullable
 */
QERL_API qerl_status qerl_mxfp4_to_nvfp4(const void* codes, const void* scales_e8m0, int64_t n,
                                         int64_t k, void* scales_e4m3, float* gscale,
                                         int32_t* range_flag, void* stream);

/* Decay schedules of qerl_aqn_sigma_schedule. */
typedef enum {
  QERL_SCHEDULE_EXPONENTIAL = 0, /* Eq. 8, as qerl_aqn_sigma              */
  QERL_SCHEDULE_LINEAR = 1,
  QERL_SCHEDULE_COSINE = 2,
  QERL_SCHEDULE_LOGARITHMIC = 3
} qerl_schedule;

/*
 * qerl_aqn_sigma_schedule -- host, pure.  sigma at stage k under one of the
 * four decay schedules the pages compare [QeRL summary, §3.4, "Why
 * exponential decay" (Fig. 9, Fig. 15)], with t = (k-1)/(K-1):
 *   EXPONENTIAL  sigma_start (sigma_end / sigma_start)^t          (Eq. 8)
 *   LINEAR       sigma_start - (sigma_start - sigma_end) t
 *   COSINE       sigma_end + (sigma_start - sigma_end)(1 + cos(pi t)) / 2
 *   LOGARITHMIC  sigma_start - (sigma_start - sigma_end) ln(k) / ln(K)
 * Stage 0 gives 0 and K == 1 gives sigma_start, as for qerl_aqn_sigma.
 *   mode       a qerl_schedule value (else QERL_ERR_RANGE)
 *   other arguments and errors as qerl_aqn_sigma
 */
QERL_API qerl_status qerl_aqn_sigma_schedule(int32_t mode, double sigma_start,
                                             double sigma_end, int32_t num_stages,
                                             int32_t stage, double* sigma_out);

/*
 * qerl_aqn_sample -- the AQN noise vector z ~ N(0, sigma^2 I) of length
 * d (= the layer's input dimension) [QeRL summary, §3.4, Eq. 7], drawn
 * afresh per forward pass by changing call_id.
 * Generator: Philox4x64-10 (Salmon et al., SC'11) with key (seed,
 * stream_id) and counter (j/4, call_id, 0, 0); Box-Muller in fp64 on the
 * output words: u1 = ((r >> 11) + 1) 2^-53, u2 = (r >> 11) 2^-53,
 * n = sqrt(-2 ln u1) {cos, sin}(2 pi u2) from the pairs (r0, r1) and
 * (r2, r3); z_j = RN_fp32(sigma * n_j).  Element j depends only on
 * (seed, stream_id, call_id, j).
 *   sigma  >= 0 and finite (0 gives z == 0)
 *   d      >= 1
 *   z_out  device out, [d] float, 4-byte aligned
 */
QERL_API qerl_status qerl_aqn_sample(uint64_t seed, uint64_t stream_id,
                            uint64_t call_id, double sigma, int64_t d,
                            float* z_out, void* stream);

/*
 * qerl_aqn_sample_batch -- `count` noise vectors in one launch, for the
 * layers of a forward pass that each draw their own [QeRL summary, §3.4,
 * Eq. 7; "Per-block noise sharing" (Fig. 6): one vector per noise group of
 * every layer].  Row i of z_out [count, d] is bit-identical to
 * qerl_aqn_sample(seed, stream_id, call_id0 + i * call_stride, sigma, d).
 *   count  1 .. 65535
 *   z_out  device out, [count, d] float, 4-byte aligned
 * Other arguments and errors as qerl_aqn_sample.
 */
QERL_API qerl_status qerl_aqn_sample_batch(uint64_t seed, uint64_t stream_id,
                                           uint64_t call_id0, uint64_t call_stride,
                                           int64_t count, double sigma, int64_t d,
                                           float* z_out, void* stream);

/*
 * qerl_aqn_sample_rows -- one noise vector per token row of a call, the
 * variant in which each rollout of a batch sees its own draw of the noise
 * [QeRL summary, §3.4 "Noise injection frequency": a different sample per
 * rollout].  Row i of z_out [m, d] takes Philox counter (j/4, call_id, i, 0)
 * for element j, so row 0 is bit-identical to qerl_aqn_sample(seed,
 * stream_id, call_id, sigma, d).
 *   m      1 .. 65535 rows
 *   z_out  device out, [m, d] float, 4-byte aligned
 * Other arguments and errors as qerl_aqn_sample.
 */
QERL_API qerl_status qerl_aqn_sample_rows(uint64_t seed, uint64_t stream_id, uint64_t call_id,
                                          double sigma, int64_t m, int64_t d, float* z_out,
                                          void* stream);

/*
 * qerl_rmsnorm_noisy -- the noisy RMSNorm that produces a linear layer's
 * input [QeRL summary, §3.4 "Noise Merging", Eq. 10]:
 *     y[i, j] = bf16( (w_j + z_j) * x[i, j] / sqrt(mean_j' x[i, j']^2 + delta) )
 * The AQN noise z is added to the RMSNorm scale w, which multiplies the
 * normalised channel j by (1 + z_j / w_j) (Eq. 11); the layer that reads y
 * then runs with no noise of its own (z == NULL there).  The sum of squares
 * and the scaling are computed in fp32; y is rounded to nearest even.
 *   x      device, [m, d] bf16 rows, 16-byte aligned
 *   m      >= 1 rows
 *   d      >= 8, d % 8 == 0 (the normalised dimension)
 *   w      device, [d] bf16 RMSNorm scale, 16-byte aligned
 *   z      device, [d] float noise, 16-byte aligned; NULL means no noise
 *   delta  >= 0 and finite (a row of zeros with delta == 0 gives NaN)
 *   y      device out, [m, d] bf16, 16-byte aligned; may be x itself
 */
QERL_API qerl_status qerl_rmsnorm_noisy(const void* x, int64_t m, int64_t d,
                                        const void* w, const float* z, float delta,
                                        void* y, void* stream);

/*
 * qerl_swiglu -- the gated activation between the fused gate/up layer and
 * the down layer of the Qwen2.5 feed-forward block (W_gate, W_up, W_down
 * [QeRL summary, §3.4 "Layer coverage"]; the gating itself is the model's,
 * not stated on the pages):
 *     out[i, j] = bf16( SiLU(gate_up[i, j]) * gate_up[i, d + j] ),
 *     SiLU(g) = g / (1 + exp(-g)), computed in fp32.
 *   gate_up  device, [m, 2 d] bf16 (the fused layer's output: gate in
 *            columns 0 .. d-1, up in d .. 2d-1), 16-byte aligned
 *   m        >= 1
 *   d        >= 8, d % 8 == 0
 *   out      device out, [m, d] bf16, 16-byte aligned; must not overlap
 *            gate_up
 */
QERL_API qerl_status qerl_swiglu(const void* gate_up, int64_t m, int64_t d, void* out,
                                 void* stream);

/*
 * qerl_linear_workspace_bytes -- bytes of device workspace that
 * qerl_linear_decode / qerl_linear_prefill / qerl_linear_prepare need for
 * these sizes on the current device.  0 if the sizes are invalid.  The
 * workspace holds the noisy activations in bf16 ([m, k]), the LoRA
 * down-projection and, for some shapes, split-K partial sums; it is
 * O(m k + m n), never O(n k).
 */
QERL_API size_t qerl_linear_workspace_bytes(int64_t m, int64_t n, int64_t k,
                                   int32_t r);

/*
 * qerl_linear_decode -- y = bf16( x_t W_hat^T + s (x_t A^T) B^T ),
 *                       x_t = x (.) (1 + z)
 * The NVFP4 linear layer with its LoRA side branch [QeRL summary, §3.4,
 * Eq. 2: W_hat + B A, with A and B in bf16] and the AQN noise merged as a
 * per-input-channel multiplier [§3.4 "Noise Merging", Eq. 10-12: noise
 * folded into the RMSNorm scale multiplies channel j by (1 + z_j / w_j);
 * here the RMSNorm weight is taken as already applied to x, w == 1].
 * W_hat is dequantized in registers (Eq. 6); no dequantized weight buffer
 * exists.  Tuned for small m (rollout decode, m <= 128); any m >= 1 works.
 *
 *   x            device, [m, k] bf16, 16-byte aligned
 *   m            >= 1
 *   codes, scales, gscale   the NVFP4 weight [n, k] as produced by
 *                qerl_quantize_nvfp4 (codes 16-byte aligned)
 *   n, k         n >= 1, k >= 16, k % 16 == 0
 *   lora_a       device, [r, k] bf16, 16-byte aligned; NULL or r == 0
 *                means no LoRA branch
 *   lora_b       device, [n, r] bf16 (any alignment)
 *   r            0 <= r <= 128
 *   lora_scale   s (= alpha / r), finite
 *   z            device, [k] float AQN noise, 16-byte aligned; NULL means
 *                no noise (bit-identical to z == 0)
 *   y            device out, [m, n] bf16, 4-byte aligned
 *   workspace    device scratch of at least
 *                qerl_linear_workspace_bytes(m, n, k, r) bytes,
 *                256-byte aligned; its contents on entry do not matter
 * Concurrent calls must not share a workspace.  Within one call, the
 * workgroups of a contraction launch may wait (a bounded poll on words of
 * the workspace that the call's own prepare launch clears) for workgroups
 * of the same launch that are dispatched ahead of them; should a wait ever
 * give up (after about a second: only if those workgroups could not run),
 * y is undefined.
 */
QERL_API qerl_status qerl_linear_decode(const void* x, int64_t m, const void* codes,
                               const void* scales, const float* gscale,
                               int64_t n, int64_t k, const void* lora_a,
                               const void* lora_b, int32_t r,
                               float lora_scale, const float* z, void* y,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * qerl_linear_decode_swiglu -- qerl_linear_decode of the down layer of a
 * gated feed-forward block, taking the fused gate/up output instead of its
 * activation: the layer input is x = bf16(SiLU(gate) * up), the operation
 * of qerl_swiglu (Qwen2.5 feed-forward block; W_gate, W_up, W_down
 * [QeRL summary, §3.4 "Layer coverage"]), formed while the prepare loads
 * the rows, so the result is bit-identical to qerl_swiglu followed by
 * qerl_linear_decode and the activation is never written out.
 *   gate_up      device, [m, 2k] bf16, 16-byte aligned: gate in columns
 *                0 .. k-1, up in k .. 2k-1
 * Every other argument, the workspace size and the errors are those of
 * qerl_linear_decode for the layer (m, n, k, r).
 */
QERL_API qerl_status qerl_linear_decode_swiglu(const void* gate_up, int64_t m, const void* codes,
                                      const void* scales, const float* gscale,
                                      int64_t n, int64_t k, const void* lora_a,
                                      const void* lora_b, int32_t r,
                                      float lora_scale, const float* z, void* y,
                                      void* workspace, size_t workspace_bytes,
                                      void* stream);

/*
 * qerl_linear_decode_rownoise / qerl_linear_prefill_rownoise -- the same
 * operations and arguments as qerl_linear_decode / qerl_linear_prefill with
 * one noise row per token: x_t[i, j] = x[i, j] (1 + z_rows[i, j]) (the
 * per-rollout noise of qerl_aqn_sample_rows).
 *   z_rows   device, [m, k] float, rows 16-byte aligned (k % 16 == 0);
 *            required (non-NULL)
 */
QERL_API qerl_status qerl_linear_decode_rownoise(const void* x, int64_t m, const void* codes,
                                                 const void* scales, const float* gscale,
                                                 int64_t n, int64_t k, const void* lora_a,
                                                 const void* lora_b, int32_t r,
                                                 float lora_scale, const float* z_rows, void* y,
                                                 void* workspace, size_t workspace_bytes,
                                                 void* stream);

QERL_API qerl_status qerl_linear_prefill_rownoise(const void* x, int64_t m, const void* codes,
                                                  const void* scales, const float* gscale,
                                                  int64_t n, int64_t k, const void* lora_a,
                                                  const void* lora_b, int32_t r,
                                                  float lora_scale, const float* z_rows, void* y,
                                                  void* workspace, size_t workspace_bytes,
                                                  void* stream);

/*
 * qerl_attention_stub -- the attention step between the fused q/k/v layer
 * and the output projection of a decode layer (W_q, W_k, W_v, W_o [QeRL
 * summary, §3.4 "Layer coverage"]), reduced to a context of one position:
 * each token attends only to its own key and value, the softmax of a single
 * score is exactly 1, and query head h outputs the value of its key/value
 * head h / (n_q_heads / n_kv_heads) (grouped-query attention):
 *     out[i, h d + e] = qkv[i, (n_q_heads + n_kv_heads + h / g) d + e],
 *     g = n_q_heads / n_kv_heads, d = head_dim
 * The values are copied bit for bit.
 *   qkv    device, [m, (n_q_heads + 2 n_kv_heads) head_dim] bf16 (q heads,
 *          then k heads, then v heads), 16-byte aligned
 *   n_q_heads % n_kv_heads == 0; head_dim >= 8, head_dim % 8 == 0
 *   out    device out, [m, n_q_heads head_dim] bf16, 16-byte aligned
 */
QERL_API qerl_status qerl_attention_stub(const void* qkv, int64_t m, int32_t n_q_heads,
                                         int32_t n_kv_heads, int32_t head_dim, void* out,
                                         void* stream);

/*
 * qerl_linear_prefill -- the same operation and arguments as
 * qerl_linear_decode, tuned for large m (prompt prefill): NVFP4 tiles are
 * dequantized into LDS and contracted with bf16 MFMA.
 */
QERL_API qerl_status qerl_linear_prefill(const void* x, int64_t m, const void* codes,
                                const void* scales, const float* gscale,
                                int64_t n, int64_t k, const void* lora_a,
                                const void* lora_b, int32_t r,
                                float lora_scale, const float* z, void* y,
                                void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * The two halves of qerl_linear_decode / qerl_linear_prefill, for callers
 * that time or schedule them separately.
 *
 * qerl_linear_prepare writes into the workspace the noisy activations
 * x_t = bf16(x (.) (1 + z)) [QeRL summary, §3.4, Eq. 12] and, with a LoRA
 * branch (r > 0 and lora_a non-NULL), the scaled down-projection
 * t = bf16(s x_t A^T) [§3.4, Eq. 2].  Arguments as above; n is needed to
 * size the workspace.
 *
 * Its workspace may be one sized for any linear entry point with the same
 * (m, n, k, r) (qerl_linear_workspace_bytes or
 * qerl_linear_tiled_workspace_bytes).
 *
 * qerl_linear_decode_prepared / qerl_linear_prefill_prepared run the main
 * contraction y = bf16(S acc + t B^T) from a workspace that
 * qerl_linear_prepare filled with the same (m, n, k, r); x, z and lora_a
 * are not read again.  r == 0 or lora_b == NULL means no LoRA branch (r
 * must then also have been 0 for the prepare call).
 */
QERL_API qerl_status qerl_linear_prepare(const void* x, int64_t m, int64_t n,
                                         int64_t k, const void* lora_a, int32_t r,
                                         float lora_scale, const float* z,
                                         void* workspace, size_t workspace_bytes,
                                         void* stream);

QERL_API qerl_status qerl_linear_decode_prepared(
    int64_t m, const void* codes, const void* scales, const float* gscale,
    int64_t n, int64_t k, const void* lora_b, int32_t r, void* y,
    void* workspace, size_t workspace_bytes, void* stream);

QERL_API qerl_status qerl_linear_prefill_prepared(
    int64_t m, const void* codes, const void* scales, const float* gscale,
    int64_t n, int64_t k, const void* lora_b, int32_t r, void* y,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * qerl_nvfp4_check_pow2_scales -- *flag = 1 if any block scale of an NVFP4
 * weight is neither zero nor a positive power of two (the condition of
 * qerl_linear_decode_mxfp4 below), else 0.  A one-time check for a weight
 * that is to run on that path; qerl_mxfp4_to_nvfp4 output always passes.
 *   scales   device, [n, k/16] E4M3 bytes; n >= 1, k >= 16, k % 16 == 0
 *   flag     device out, 4-byte aligned, written by the call
 * Two kernels are enqueued (clear the flag, scan the scales).
 */
QERL_API qerl_status qerl_nvfp4_check_pow2_scales(const void* scales, int64_t n, int64_t k,
                                                  int32_t* flag, void* stream);

/*
 * qerl_linear_decode_mxfp4 / qerl_linear_decode_prepared_mxfp4 -- the
 * same operations and arguments as qerl_linear_decode /
 * qerl_linear_decode_prepared, for an MXFP4 weight in the NVFP4 layout
 * (qerl_mxfp4_to_nvfp4): every block scale is then a power of two, which
 * lets the decode kernel form each pair of bf16 weight values with one
 * scaled-conversion instruction.  The result is bit-identical to the
 * general call on the same arguments; block scales that are not powers of
 * two give wrong results (qerl_nvfp4_check_pow2_scales tells which weights
 * qualify).
 */
QERL_API qerl_status qerl_linear_decode_mxfp4(const void* x, int64_t m, const void* codes,
                                              const void* scales, const float* gscale,
                                              int64_t n, int64_t k, const void* lora_a,
                                              const void* lora_b, int32_t r, float lora_scale,
                                              const float* z, void* y, void* workspace,
                                              size_t workspace_bytes, void* stream);

QERL_API qerl_status qerl_linear_decode_prepared_mxfp4(
    int64_t m, const void* codes, const void* scales, const float* gscale, int64_t n, int64_t k,
    const void* lora_b, int32_t r, void* y, void* workspace, size_t workspace_bytes,
    void* stream);

/*
 * Tiled weight layout for the 128-token decode kernel.  A rollout engine
 * quantizes the model once and holds it [QeRL summary, §3.3 "Roadmap";
 * §3.2], so the stored NVFP4 weight may be re-laid once at load for the
 * kernel that reads it every token.  The tiled weight holds the same codes
 * and scales (same S) grouped in tiles of 32 rows x 128 channels
 * (2304 bytes: 2048 of codes, then 256 of block scales), tile (st, b) of
 * rows 32 st .. 32 st + 31 and channels 128 b .. 128 b + 127 at byte
 * (st * (k / 128) + b) * 2304.  Inside a tile, the 16 bytes at
 * ((2 kh + h) * 32 + c) * 16 are the codes of row 32 st + c, channels
 * 128 b + 64 kh + 32 h + 0..31 (two per byte, the even channel in the low
 * nibble), and the 2 bytes at 2048 + ((2 kh + h) * 32 + c) * 2 their two
 * block scales.  Rows past n are zero.  With this order one wave of the
 * kernel loads 1 KB of contiguous codes and 128 B of contiguous scales per
 * 32 rows and 128 channels, instead of 32 separate pieces of each.
 *
 * qerl_nvfp4_tile128_bytes -- size of the tiled weight: ceil(n/32) * (k/128)
 *   * 2304 bytes; 0 if n < 1 or k is not a positive multiple of 128.
 * qerl_nvfp4_tile128 -- re-lays (codes [n, k/2], scales [n, k/16]) as above.
 *   codes, tiled   device, 16-byte aligned; k % 128 == 0; tiled holds
 *                  qerl_nvfp4_tile128_bytes(n, k) bytes and must not overlap
 *                  codes or scales
 * qerl_linear_tiled_workspace_bytes -- workspace of the tiled entry points
 *   (0 if the sizes are invalid).
 * qerl_linear_decode_tiled / qerl_linear_decode_tiled_prepared -- the same
 *   operations and arguments as qerl_linear_decode / _prepared with the
 *   tiled weight in place of (codes, scales); k % 128 == 0.  Every chunk of
 *   up to 128 tokens runs the single-pass 128-token kernel, which gives
 *   results bit-identical to qerl_linear_decode for chunks of 65 to 128
 *   tokens.  The prepared half reads a workspace filled by
 *   qerl_linear_prepare with the same (m, n, k, r).
 */
QERL_API size_t qerl_nvfp4_tile128_bytes(int64_t n, int64_t k);

QERL_API qerl_status qerl_nvfp4_tile128(const void* codes, const void* scales, int64_t n,
                                        int64_t k, void* tiled, void* stream);

QERL_API size_t qerl_linear_tiled_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t r);

QERL_API qerl_status qerl_linear_decode_tiled(const void* x, int64_t m, const void* tiled,
                                              const float* gscale, int64_t n, int64_t k,
                                              const void* lora_a, const void* lora_b, int32_t r,
                                              float lora_scale, const float* z, void* y,
                                              void* workspace, size_t workspace_bytes,
                                              void* stream);

QERL_API qerl_status qerl_linear_decode_tiled_prepared(int64_t m, const void* tiled,
                                                       const float* gscale, int64_t n, int64_t k,
                                                       const void* lora_b, int32_t r, void* y,
                                                       void* workspace, size_t workspace_bytes,
                                                       void* stream);

/*
 * qerl_linear_decode_noalloc -- for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): qerl_linear_decode with the same arguments
 * minus the workspace, which is replaced by a device array inside the
 * library of qerl_linear_noalloc_scratch_bytes() bytes (64 MiB) per GPU,
 * held until the process ends.  It allocates and frees nothing.
 *   - Sizes whose workspace (qerl_linear_workspace_bytes) exceeds the
 *     array return QERL_ERR_WORKSPACE before anything is enqueued.
 *   - `stream` must belong to the current device (else QERL_ERR_RANGE);
 *     the array of the current device is used.
 *   - Every call on one GPU uses that GPU's single array: calls that
 *     overlap on one GPU (other streams, other host threads) race and must
 *     be serialised by the caller.  The array keeps the last call's
 *     contents; no call relies on them.
 * Results are bit-identical to qerl_linear_decode.
 */
QERL_API size_t qerl_linear_noalloc_scratch_bytes(void);

QERL_API qerl_status qerl_linear_decode_noalloc(const void* x, int64_t m, const void* codes,
                                                const void* scales, const float* gscale,
                                                int64_t n, int64_t k, const void* lora_a,
                                                const void* lora_b, int32_t r, float lora_scale,
                                                const float* z, void* y, void* stream);

/*
 * qerl_linear_backward -- gradients of the layer through the frozen NVFP4
 * weight.  The rollout's log-probabilities are taken on the same quantized
 * model and only the LoRA factors (and RMSNorm scales) are trained
 * [QeRL summary, §3.4 "Low-Rank Adaptation"; Algorithm 1, inner updates],
 * so W_hat gets no gradient.  With x_t = bf16(x (.) (1 + z)) as in the
 * forward, t = bf16(s x_t A^T) and gs = bf16(s dy B):
 *     dx = bf16( (dy W_hat + gs A) (.) (1 + z) )      [m, k]
 *     dA = gs^T x_t   (fp32, [r, k])     dB = dy^T t   (fp32, [n, r])
 * Sums in fp32.
 *   dy           device, [m, n] bf16 output gradient, 16-byte aligned
 *   m            >= 1
 *   codes, scales, gscale   the layer's NVFP4 weight [n, k]
 *   n, k         >= 16, multiples of 16
 *   x            device, [m, k] bf16 forward input, 16-byte aligned
 *   lora_a, lora_b, r, lora_scale, z   as in qerl_linear_decode
 *   dx           device out, [m, k] bf16
 *   da, db       device out, fp32 [r, k] and [n, r]; either may be NULL
 *                (not computed); both ignored without a LoRA branch
 *   workspace    at least qerl_linear_backward_workspace_bytes(m, n, k, r)
 *                bytes, 256-byte aligned
 */
QERL_API size_t qerl_linear_backward_workspace_bytes(int64_t m, int64_t n, int64_t k,
                                                     int32_t r);

QERL_API qerl_status qerl_linear_backward(const void* dy, int64_t m, const void* codes,
                                          const void* scales, const float* gscale,
                                          int64_t n, int64_t k, const void* x,
                                          const void* lora_a, const void* lora_b, int32_t r,
                                          float lora_scale, const float* z, void* dx,
                                          float* da, float* db, void* workspace,
                                          size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QERL_H */
