/*
 * fp8lin -- static per-tensor FP8 linear layers for AMD MI355X (gfx950).
 *
 * C ABI of the library libfp8lin.so. Every entry point is extern "C", takes
 * plain pointers and sizes, and returns an int32_t status (FP8LIN_OK = 0,
 * negative on error). No C++ exception crosses the ABI.
 *
 * The method (web pages, cited by title and section):
 *   [CF-157]    NVIDIA/cosmos-framework PR #157, "feat: load ModelOpt
 *               static-FP8 checkpoints via TorchAO".
 *   [DF-14664]  huggingface/diffusers PR #14664, "[Cosmos3] Mixed W8A8/W8A16
 *               denoising for ModelOpt FP8 checkpoints".
 *   [TRT-17476] NVIDIA/TensorRT-LLM PR #17476, "Load static FP8 Cosmos3
 *               Nano/Super checkpoints without re-quantizing them".
 *   [DF-15170]  huggingface/diffusers issue #15170, "Cosmos 3 docs: FP8
 *               snippet fails at the first W8A8 step without importing
 *               ModelOpt's FP8 GEMM backend".
 *
 * Conventions shared by all GPU entry points:
 *   - Tensor pointers are DEVICE pointers, allocated and owned by the caller.
 *     The library allocates no device memory and keeps no state between
 *     calls apart from the launch counters of fp8lin_launch_count().
 *   - Work is enqueued asynchronously on `stream` (NULL = the default
 *     stream); no call synchronizes the host with the device, and no call
 *     reads device memory from the host, so calls are safe to capture into a
 *     HIP graph.
 *   - Scales are HOST floats: static, load-time constants of the checkpoint.
 *     A scale must be finite and lie in [2^-126, 2^126] (so that its
 *     reciprocal is a normal float) -> otherwise FP8LIN_ESCALE.
 *   - All arguments are validated before anything is enqueued; a failing
 *     call enqueues nothing. rows/M == 0 is a valid no-op (FP8LIN_OK); the
 *     activation and output pointers may then be NULL (sizes, scales and
 *     the weight pointer are still checked).
 *   - Matrices are row-major. Activations x are [M, K], weights are
 *     [N, K] (out_features x in_features, the nn.Linear layout, bias=False
 *     as in [DF-15170] "Logs"), outputs y are [M, N] with row stride ldy
 *     elements.
 *   - E4M3 is the OCP FP8 "FN" format (bias 7, max 448, no infinities,
 *     NaN = S.1111.111), one byte per element.
 *   - Layout requirements (else FP8LIN_ELAYOUT): K and cols multiples of 16;
 *     N and ldy multiples of 8 with ldy >= N; every pointer 16-byte aligned.
 *   - Size limits (else FP8LIN_EUNSUPPORTED): M and rows < 2^31, cols
 *     < 2^24, M*K and rows*cols < 2^40; for the GEMMs K, N and ldy < 2^22
 *     and M <= 2^31 - 256.
 *   - A HIP launch error is reported as FP8LIN_EHIP.
 */
#ifndef FP8LIN_H
#define FP8LIN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP8LIN_OK = 0,
  FP8LIN_EINVAL = -1,       /* null pointer, negative size, unknown enum value */
  FP8LIN_ELAYOUT = -2,      /* alignment, divisibility or leading dimension */
  FP8LIN_EDTYPE = -3,       /* activation dtype this call does not accept */
  FP8LIN_ESCALE = -4,       /* bad scale, or unequal input scales in a group */
  FP8LIN_EPOLICY = -5,      /* step policy missing a field or holding a bad value */
  FP8LIN_EUNSUPPORTED = -6, /* size beyond the stated limits */
  FP8LIN_EHIP = -7          /* the HIP runtime rejected a launch */
} fp8lin_status;

typedef enum { FP8LIN_MODE_W8A8 = 0, FP8LIN_MODE_W8A16 = 1 } fp8lin_mode;

/* Element formats: bf16, OCP E4M3, IEEE binary16, IEEE binary32. */
typedef enum { FP8LIN_DT_BF16 = 0, FP8LIN_DT_E4M3 = 1, FP8LIN_DT_F16 = 2, FP8LIN_DT_F32 = 3 } fp8lin_dtype;

typedef enum { FP8LIN_TOWER_GENERATION = 0, FP8LIN_TOWER_REASONER = 1 } fp8lin_tower;

/* Values of the enumerated policy fields. A parser maps each JSON string it
 * recognises to its value and anything else to FP8LIN_POLICY_UNKNOWN. */
enum {
  FP8LIN_POLICY_UNKNOWN = -1,
  FP8LIN_POLICY_TYPE_FIRST_LAST_STEPS = 1, /* "type": "first_last_steps" */
  FP8LIN_POLICY_INDEX_SCHEDULER_STEP = 1,  /* "index_space": "scheduler_step" (0-based) */
  FP8LIN_POLICY_OVERLAP_A16 = 1            /* "overlap": "a16" */
};

/* present_mask bits: one per field of the policy document. */
enum {
  FP8LIN_PF_SCHEMA_VERSION = 1u << 0,
  FP8LIN_PF_TYPE = 1u << 1,
  FP8LIN_PF_INDEX_SPACE = 1u << 2,
  FP8LIN_PF_DEFAULT_MODE = 1u << 3,
  FP8LIN_PF_OVERLAP = 1u << 4,
  FP8LIN_PF_FIRST_STEPS = 1u << 5,
  FP8LIN_PF_LAST_STEPS = 1u << 6,
  FP8LIN_PF_REASONER = 1u << 7,
  FP8LIN_PF_ALL = 0xFFu,
  FP8LIN_PF_UNKNOWN_FIELD = 1u << 31 /* the document held a field not listed above */
};

/* quantization_config.runtime.diffusion_step_policy, as parsed from the
 * checkpoint ([DF-14664] "Behavior"; [TRT-17476] "Denoising-step activation
 * precision"). default_mode and reasoner_mode hold fp8lin_mode values
 * (default_mode must be FP8LIN_MODE_W8A8). */
typedef struct {
  int32_t schema_version; /* must be 1 */
  int32_t type;           /* FP8LIN_POLICY_TYPE_FIRST_LAST_STEPS */
  int32_t index_space;    /* FP8LIN_POLICY_INDEX_SCHEDULER_STEP */
  int32_t default_mode;   /* FP8LIN_MODE_W8A8 */
  int32_t overlap;        /* FP8LIN_POLICY_OVERLAP_A16 */
  int32_t first_steps;    /* >= 0: steps [0, first_steps) run W8A16 */
  int32_t last_steps;     /* >= 0: steps [num_steps - last_steps, num_steps) run W8A16 */
  int32_t reasoner_mode;  /* mode of the understanding tower, not step-gated */
  uint32_t present_mask;  /* FP8LIN_PF_* bits of the fields the document held */
} fp8lin_policy;

/*
 * Static per-tensor activation quantization ([CF-157] "Verification": the
 * quantizer divides by the exported input_scale, clamps, then rounds to FP8).
 *   q[i] = E4M3_RNE( clamp( fl32(x[i]) / input_scale, -448, 448 ) )
 * with the quotient the correctly rounded float32 division; ties go to the
 * even code, -0 and a negative value that rounds to zero give 0x80, a NaN
 * input gives 0x7F or 0xFF (its sign kept).
 *   x_bf16  device, bf16 [rows, cols], contiguous, read only
 *   q_e4m3  device, uint8 [rows, cols], contiguous, written
 *   cols    multiple of 16
 */
int32_t fp8lin_quantize_static(const void* x_bf16, void* q_e4m3, int64_t rows, int64_t cols,
                               float input_scale, hipStream_t stream);

/*
 * W8A8 GEMM ([CF-157] "Verification": a real FP8 x FP8 GEMM; [TRT-17476]
 * "Description": one weight scale and one input scale per projection):
 *   y[m, n] = bf16_RNE( (sum_k dec(qx[m, k]) * dec(qw[n, k])) * fl32(input_scale * weight_scale) )
 * FP8 products accumulate in float32 on the FP8 matrix cores; the output is
 * rounded to bf16 once.
 *   qx  device, E4M3 [M, K], contiguous        (from fp8lin_quantize_static)
 *   qw  device, E4M3 [N, K], contiguous        (the checkpoint weight)
 *   y   device, bf16 [M, ldy], columns [0, N) written, the rest untouched
 */
int32_t fp8lin_gemm_w8a8(const void* qx, const void* qw, void* y_bf16, int64_t M, int64_t N, int64_t K,
                         int64_t ldy, float input_scale, float weight_scale, hipStream_t stream);

/*
 * W8A16 GEMM for the steps the policy sends to 16-bit activations
 * ([TRT-17476] "Denoising-step activation precision": the resident FP8
 * weight is dequantized with its own weight_scale, input_scale is unused, no
 * dequantized weight copy is kept; [DF-14664] "Behavior"):
 *   y[m, n] = RNE( weight_scale * sum_k x[m, k] * dec(qw[n, k]) )
 * in the activation's 16-bit format. Weight tiles are staged in LDS as
 * E4M3 and converted exactly to bf16 (or binary16) on the way to the
 * matching matrix cores; no dequantized weight is written to memory.
 *   x_dtype  FP8LIN_DT_BF16 or FP8LIN_DT_F16 (the pages' 16-bit activation
 *            dtypes); an already-quantized activation (FP8LIN_DT_E4M3) is
 *            refused with FP8LIN_EDTYPE, as the pages' 16-bit path refuses
 *            one, and so is FP8LIN_DT_F32 (it needs the workspace of
 *            fp8lin_gemm_w8a16_f32)
 *   x   device, [M, K] of x_dtype, contiguous
 *   qw  device, E4M3 [N, K], contiguous
 *   y   device, [M, ldy] of x_dtype (binary16 overflows to an infinity)
 */
int32_t fp8lin_gemm_w8a16(const void* x, int32_t x_dtype, const void* qw, void* y_bf16, int64_t M, int64_t N,
                          int64_t K, int64_t ldy, float weight_scale, hipStream_t stream);

/*
 * W8A16 with a float32 activation ([DF-14664] "Tests" lists this case: the
 * weight is dequantized to the activation's dtype and the product is taken
 * in float32):
 *   y[m, n] = fl32( weight_scale * A ),  A = sum_k x[m, k] * dec(qw[n, k])
 * accumulated in float32. A first kernel splits every x value exactly into
 * three bf16 pieces (hi + mid + lo = x; exact for |x| >= 2^-110, and
 * non-finite values stay whole in hi) into the workspace, then the bf16
 * W8A16 kernel takes 3 K exact products per output and writes float32.
 * |y - exact| <= (3 K u / (1 - 3 K u)) * weight_scale * sum_k |x dec(qw)|
 * plus two float32 roundings, u = 2^-24.
 *   x          device, float32 [M, K], contiguous
 *   qw         device, E4M3 [N, K], contiguous
 *   y          device, float32 [M, ldy]
 *   workspace  device, at least fp8lin_w8a16_f32_workspace_bytes(M, K)
 *              bytes, 16-byte aligned; overwritten (caller-owned scratch;
 *              two calls in flight on different streams need two)
 *   K          multiple of 16, < 2^20 (else FP8LIN_EUNSUPPORTED)
 * Launches counted as FP8LIN_KERNEL_SPLIT and FP8LIN_KERNEL_GEMM_W8A16.
 */
int32_t fp8lin_gemm_w8a16_f32(const void* x_f32, const void* qw, void* y_f32, int64_t M, int64_t N, int64_t K,
                              int64_t ldy, float weight_scale, void* workspace, int64_t workspace_bytes,
                              hipStream_t stream);

/* Workspace bytes fp8lin_gemm_w8a16_f32 needs: M * 3 * 64 * ceil(K / 64) * 2
 * (three bf16 pieces per value, each row padded to 64 values); -1 for
 * sizes the call refuses. Host only. */
int64_t fp8lin_w8a16_f32_workspace_bytes(int64_t M, int64_t K);

/*
 * fp8lin_gemm_w8a8 with the K dimension split into `splits` slices, for
 * shapes whose 256 x 256 output tiles are too few to fill the device (at
 * M = 1024, N = 4096: 64 tiles for 256 compute units). Each slice's product
 * goes, unscaled, in float32 to its part of the workspace; a second kernel
 * sums the parts in slice order and writes
 *   y[m, n] = bf16_RNE( (sum_s partial_s[m, n]) * (input_scale * weight_scale) )
 * (the float32 summation order differs from fp8lin_gemm_w8a8's, so the two
 * may differ in the last bf16 bit; both meet the same tolerance).
 *   splits     1 (plain fp8lin_gemm_w8a8, workspace unused), 2 or 4; K a
 *              multiple of 16 * splits (else FP8LIN_ELAYOUT)
 *   workspace  device, >= splits * M * N * 4 bytes, 16-byte aligned,
 *              caller-owned scratch (else FP8LIN_EINVAL)
 * Other arguments and rules as fp8lin_gemm_w8a8. Launches counted as
 * FP8LIN_KERNEL_GEMM_W8A8 and FP8LIN_KERNEL_SPLITK_REDUCE.
 */
int32_t fp8lin_gemm_w8a8_splitk(const void* qx, const void* qw, void* y_bf16, int64_t M, int64_t N, int64_t K,
                                int64_t ldy, float input_scale, float weight_scale, int32_t splits, void* workspace,
                                int64_t workspace_bytes, hipStream_t stream);

/* The split count fp8lin_gemm_w8a8_splitk does best with on the current
 * device: 1. A split of the 256 x 256 kernel helps only where its tiles fill
 * at most half the compute units, and there the unsplit call runs on
 * 128 x 128 tiles (when 256 x 256 ones would keep at most 60% of the compute
 * units busy), which beats every split (1024 x 4096 x 4096: 1.75-1.79 against
 * 0.96-1.02 PFLOP/s with 2 slices). Kept so that callers need not change;
 * explicit split counts stay available. Host only. */
int32_t fp8lin_gemm_w8a8_splitk_choice(int64_t M, int64_t N, int64_t K);

/* Size of the library's static device scratch array (32 MiB), which each GPU
 * the library runs on holds until the process ends. */
#define FP8LIN_SCRATCH_BYTES (32 * 1024 * 1024)

/*
 * fp8lin_gemm_w8a8_splitk for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and the same result bit for bit, with the
 * float32 partials in the library's static scratch array instead of a
 * caller workspace. It calls no allocating routine; on a device's first call
 * it looks the array's device address up once (hipGetSymbolAddress).
 *   splits  1 (plain fp8lin_gemm_w8a8, no scratch), 2 or 4; K a multiple of
 *           16 * splits (else FP8LIN_ELAYOUT)
 * splits * M * N * 4 must not exceed FP8LIN_SCRATCH_BYTES (else
 * FP8LIN_EUNSUPPORTED, nothing enqueued): e.g. M = 1024, N = 4096 with 2
 * splits, or M = 512 with 4.
 * Every call on one GPU uses that GPU's one scratch array: calls that
 * overlap on a GPU (concurrent streams, several host threads) race and
 * give wrong results; calls in stream order on one stream are safe. The
 * partials are fully overwritten by every call, nothing needs clearing.
 * Other arguments, rules and launch counts as fp8lin_gemm_w8a8_splitk.
 */
int32_t fp8lin_gemm_w8a8_splitk_noalloc(const void* qx, const void* qw, void* y_bf16, int64_t M, int64_t N,
                                        int64_t K, int64_t ldy, float input_scale, float weight_scale, int32_t splits,
                                        hipStream_t stream);

/*
 * fp8lin_gemm_w8a16 with K split into `splits` slices, for shapes with too
 * few output tiles to fill the device (e.g. M = 1024 tokens of a 4096 ->
 * 4096 projection: 64 tiles of 256 x 256 for 256 compute units). The same
 * W8A16 product ([DF-14664] "Behavior": the 16-bit step keeps the FP8
 * weight and the 16-bit activation) computed as one launch over the
 * slices, each writing its unscaled float32 partial to `workspace`
 * ([splits][M][N] float32), then a reduction that sums the parts in slice
 * order and writes
 *   y[m, n] = bf16_RNE( (sum_s partial_s[m, n]) * weight_scale )
 * (the float32 summation order differs from fp8lin_gemm_w8a16's, so the
 * two may differ in the last bf16 bit; both meet the same tolerance).
 *   x_dtype    FP8LIN_DT_BF16 (binary16 activations: FP8LIN_EUNSUPPORTED
 *              when splits > 1, the reduction writes bf16; E4M3 or float32:
 *              FP8LIN_EDTYPE)
 *   splits     1 (plain fp8lin_gemm_w8a16, workspace unused), 2 or 4; K a
 *              multiple of 16 * splits (else FP8LIN_ELAYOUT)
 *   workspace  device, >= splits * M * N * 4 bytes, 16-byte aligned,
 *              caller-owned scratch (else FP8LIN_EINVAL)
 * Other arguments and rules as fp8lin_gemm_w8a16. Launches counted as
 * FP8LIN_KERNEL_GEMM_W8A16 and FP8LIN_KERNEL_SPLITK_REDUCE.
 */
int32_t fp8lin_gemm_w8a16_splitk(const void* x, int32_t x_dtype, const void* qw, void* y_bf16, int64_t M, int64_t N,
                                 int64_t K, int64_t ldy, float weight_scale, int32_t splits, void* workspace,
                                 int64_t workspace_bytes, hipStream_t stream);

/* The split count fp8lin_gemm_w8a16_splitk does best with on the current
 * device: 1, for the reason given at fp8lin_gemm_w8a8_splitk_choice
 * (1024 x 4096 x 4096: 1.0 PFLOP/s unsplit on 128 x 128 tiles against
 * 0.68-0.72 with 4 slices). Host only. */
int32_t fp8lin_gemm_w8a16_splitk_choice(int64_t M, int64_t N, int64_t K);

/*
 * The GEMMs of a shared-input projection group on an activation quantized
 * once ([TRT-17476] "What changed": every projection of the group consumes
 * the same FP8 tensor, each with its own weight_scale), in one launch:
 *   y[i][m, n] = bf16_RNE( (sum_k dec(qx[m, k]) * dec(qw[i][n, k]))
 *                          * (input_scale * weight_scale[i]) )
 * i.e. fp8lin_gemm_w8a8 for each i with ldy = n_out[i]; the tiles of all
 * projections share one grid, so the group fills the GPU as one GEMM would.
 *   qx            device, E4M3 [M, K], contiguous
 *   nproj         1..4
 *   qw[i]         device, E4M3 [n_out[i], K]
 *   n_out[i]      host array: output width of projection i (multiple of 8)
 *   weight_scale  host array [nproj]; input_scale: the group's one scale
 *   y[i]          device, bf16 [M, n_out[i]], contiguous
 *   The host arrays are read during the call only.
 */
int32_t fp8lin_gemm_w8a8_group(const void* qx, int64_t M, int64_t K, int32_t nproj, const void* const qw[],
                               const int64_t n_out[], const float weight_scale[], float input_scale,
                               void* const y_bf16[], hipStream_t stream);

/*
 * Shared-input projections: Q/K/V (nproj = 3) or gate/up (nproj = 2)
 * ([TRT-17476] "What changed": the group quantizes its shared activation once
 * and hands the same FP8 tensor to every projection, each with its own
 * weight_scale; the projections stay separate and write contiguous outputs,
 * "It is also faster"). The group's input scales must be bitwise equal
 * ("Description": the invariant the sharing rests on) -> else FP8LIN_ESCALE.
 *   mode FP8LIN_MODE_W8A8:  one quantization of x into qx_workspace, then one
 *                           grouped FP8 GEMM launch over all projections.
 *   mode FP8LIN_MODE_W8A16: the sharing stands down ("Denoising-step
 *                           activation precision"): no quantization, one
 *                           grouped W8A16 launch; qx_workspace may be NULL.
 *   x             device, bf16 [M, K]
 *   nproj         1..4
 *   qw[i]         device, E4M3 [n_out[i], K]
 *   n_out[i]      host array: output width of projection i (multiple of 8)
 *   weight_scale  host array [nproj]; input_scale host array [nproj]
 *   y[i]          device, bf16 [M, n_out[i]], contiguous (ldy = n_out[i])
 *   qx_workspace  device, M*K bytes; on return (W8A8) it holds the codes of x
 *   The host arrays are read during the call only.
 */
int32_t fp8lin_qkv_shared(const void* x_bf16, int64_t M, int64_t K, int32_t nproj, const void* const qw[],
                          const int64_t n_out[], const float weight_scale[], const float input_scale[],
                          void* const y_bf16[], void* qx_workspace, int32_t mode, hipStream_t stream);

/*
 * Two-input SwiGLU h = silu(gate) * up, silu(g) = g / (1 + exp(-g)), in
 * float32, from two separate tensors ([TRT-17476] "What changed": the split
 * MLP's SiLU(G) * U, quantized straight to FP8 for the down projection).
 *   out_dtype FP8LIN_DT_E4M3: out[i] = E4M3_RNE(clamp(h / out_scale, +-448))
 *                             (out_scale = the down projection's static
 *                             input scale; h is not rounded to bf16 first)
 *   out_dtype FP8LIN_DT_BF16: out[i] = bf16_RNE(h), for 16-bit steps;
 *                             out_scale is ignored
 *   gate, up  device, bf16 [rows, cols], contiguous (else the layout error)
 *   out       device, [rows, cols] of E4M3 bytes or bf16
 *   cols      multiple of 16
 */
int32_t fp8lin_swiglu_2in_quant(const void* gate_bf16, const void* up_bf16, void* out, int32_t out_dtype,
                                int64_t rows, int64_t cols, float out_scale, hipStream_t stream);

/*
 * The same two-input SwiGLU for either 16-bit input format ([TRT-17476]
 * "What changed": the split SwiGLU runs on BF16 and FP16 shapes):
 *   in_dtype   FP8LIN_DT_BF16 or FP8LIN_DT_F16 (else FP8LIN_EDTYPE)
 *   out_dtype  FP8LIN_DT_E4M3 (codes as above) or in_dtype (RNE of h in
 *              the input's format; binary16 overflows to an infinity);
 *              another format -> FP8LIN_EDTYPE
 *   gate, up   device, [rows, cols] of in_dtype, contiguous
 * With in_dtype = FP8LIN_DT_BF16 it is fp8lin_swiglu_2in_quant. Unknown
 * format values -> FP8LIN_EINVAL.
 */
int32_t fp8lin_swiglu_2in(const void* gate, const void* up, int32_t in_dtype, void* out, int32_t out_dtype,
                          int64_t rows, int64_t cols, float out_scale, hipStream_t stream);

/*
 * Gate/up projections and SwiGLU fused in one GEMM launch (W8A8): the split
 * gated MLP of [TRT-17476] "What changed" (gate and up on one shared FP8
 * activation, then silu(G) * U quantized for the down projection) without
 * the two bf16 [M, I] intermediates. For every element
 *   g = bf16_RNE( (sum_k dec(qx[m,k]) dec(qw_gate[n,k])) * (input_scale * gate_scale) )
 *   u = bf16_RNE( (sum_k dec(qx[m,k]) dec(qw_up[n,k]))   * (input_scale * up_scale) )
 *   h[m, n] = E4M3_RNE(clamp(silu(g) * u / out_scale, +-448))
 * i.e. exactly fp8lin_gemm_w8a8 for gate and for up followed by
 * fp8lin_swiglu_2in_quant(E4M3, out_scale) on their outputs; the bf16
 * rounding of g and u is kept so the result equals that unfused path bit
 * for bit.
 *   qx              device, E4M3 [M, K], contiguous (the activation quantized
 *                   once with input_scale)
 *   qw_gate, qw_up  device, E4M3 [I, K], contiguous
 *   h               device, E4M3 [M, I], contiguous
 *   I               multiple of 16 (else FP8LIN_ELAYOUT), < 2^22
 *   out_scale       the down projection's static input scale
 * Launch counted as FP8LIN_KERNEL_GATE_UP_SWIGLU.
 */
int32_t fp8lin_gate_up_swiglu_w8a8(const void* qx, int64_t M, int64_t K, const void* qw_gate, const void* qw_up,
                                   int64_t I, float input_scale, float gate_scale, float up_scale, float out_scale,
                                   void* h_e4m3, hipStream_t stream);

/*
 * The same fusion for 16-bit steps (W8A16): gate and up from a bf16
 * activation and the resident E4M3 weights ([TRT-17476] "Denoising-step
 * activation precision"), then the two-input SwiGLU with a bf16 output:
 *   g = bf16_RNE( gate_scale * sum_k x[m,k] dec(qw_gate[n,k]) )
 *   u = bf16_RNE( up_scale   * sum_k x[m,k] dec(qw_up[n,k]) )
 *   h[m, n] = bf16_RNE( silu(g) * u )
 * i.e. exactly fp8lin_gemm_w8a16 for gate and for up followed by
 * fp8lin_swiglu_2in_quant(FP8LIN_DT_BF16) on their outputs, bit for bit.
 * With a binary16 activation every bf16 above is binary16 (the chain
 * fp8lin_gemm_w8a16 + fp8lin_swiglu_2in in FP8LIN_DT_F16).
 *   x_dtype  FP8LIN_DT_BF16 or FP8LIN_DT_F16 (FP8LIN_DT_E4M3 and
 *            FP8LIN_DT_F32 -> FP8LIN_EDTYPE)
 *   x        device, [M, K] of x_dtype, contiguous
 *   qw_gate, qw_up  device, E4M3 [I, K], contiguous
 *   h        device, [M, I] of x_dtype, contiguous; I multiple of 16, < 2^22
 * Launch counted as FP8LIN_KERNEL_GATE_UP_SWIGLU.
 */
int32_t fp8lin_gate_up_swiglu_w8a16(const void* x_bf16, int32_t x_dtype, int64_t M, int64_t K, const void* qw_gate,
                                    const void* qw_up, int64_t I, float gate_scale, float up_scale, void* h_bf16,
                                    hipStream_t stream);

/*
 * Per-head QK RMSNorm followed by rotary position embedding, reading the
 * contiguous outputs of the separate Q and K projections ([TRT-17476] "It
 * is also faster": with split projections these ops read contiguous rows,
 * where the pages find the end-to-end gain; [DF-15170] "Logs": the
 * processor views a projection as [tokens, heads, head_dim] and receives a
 * precomputed rotary embedding). For every token t and head of D values x,
 * in float32:
 *   r = rsqrt(sum(x^2) / D + eps),  y = x * r * w
 *   out[i]       = y[i] * cos[t, i] - y[i + D/2] * sin[t, i]
 *   out[i + D/2] = y[i + D/2] * cos[t, i] + y[i] * sin[t, i],  i < D/2
 * rounded once to bf16 (the rotate-half RoPE form; the pages fix neither
 * eps nor the RoPE variant, so both are the caller's).
 *   q, k          device, bf16 [tokens, q_heads * D] / [tokens, k_heads * D],
 *                 contiguous; k may be NULL with k_heads = 0
 *   q_out, k_out  device, same shapes; may equal q / k (in place), must not
 *                 overlap them otherwise
 *   q_weight, k_weight  device, bf16 [D] RMSNorm weights, or NULL for 1
 *   cos, sin      device, float32 [tokens, D/2] rotary tables
 *   head_dim      64 or 128 (else FP8LIN_EUNSUPPORTED)
 *   eps           finite, > 0 (else FP8LIN_EINVAL)
 * Pointers 16-byte aligned. One launch for Q and K, counted as
 * FP8LIN_KERNEL_QK_NORM_ROPE; tokens = 0 is a no-op.
 */
int32_t fp8lin_qk_norm_rope(const void* q, const void* k, void* q_out, void* k_out, int64_t tokens, int32_t q_heads,
                            int32_t k_heads, int32_t head_dim, const void* q_weight, const void* k_weight,
                            const float* cos, const float* sin, float eps, hipStream_t stream);

/*
 * The grouped W8A8 QKV projections with the per-head QK RMSNorm + RoPE of
 * fp8lin_qk_norm_rope applied in the GEMM's epilogue to Q (group 0) and K
 * (group 1), heads of 128 values: the consumer of the contiguous split
 * outputs ([TRT-17476] "It is also faster") without its extra pass over Q
 * and K. Per output row and head, with y = bf16_RNE(acc * input_scale *
 * weight_scale) (the value fp8lin_gemm_w8a8_group writes):
 *   r = rsqrt(sum(y^2) / 128 + eps)
 *   out[d]      = y[d] r w[d] cos[m, d] - y[d + 64] r w[d + 64] sin[m, d]
 *   out[d + 64] = y[d + 64] r w[d + 64] cos[m, d] + y[d] r w[d] sin[m, d]
 * in float32, rounded once to bf16; group 2 (V) is the plain GEMM output.
 * Same arguments and rules as fp8lin_gemm_w8a8_group, plus:
 *   nproj          2 (Q, K) or 3 (Q, K, V)
 *   n_out[0], n_out[1]  multiples of 128 (else FP8LIN_ELAYOUT)
 *   q_norm_weight, k_norm_weight  device, bf16 [128], or NULL for 1
 *   cos, sin       device, float32 [M, 64] rotary tables, 16-byte aligned
 *   eps            finite, > 0 (else FP8LIN_EINVAL)
 * The result is within the float32 error bound of the exact norm and
 * rotation of y (the summation order differs from fp8lin_qk_norm_rope's,
 * so the two may differ in the last bf16 bit). One launch, counted as
 * FP8LIN_KERNEL_GEMM_W8A8.
 */
int32_t fp8lin_qkv_w8a8_norm_rope(const void* qx, int64_t M, int64_t K, int32_t nproj, const void* const qw[],
                                  const int64_t n_out[], const float weight_scale[], float input_scale,
                                  void* const y_bf16[], const void* q_norm_weight, const void* k_norm_weight,
                                  const float* cos, const float* sin, float eps, hipStream_t stream);

/*
 * Dynamic per-tensor activation quantization: the scale comes from the
 * tensor itself at run time instead of a calibrated checkpoint value (the
 * dynamically quantized FP8 path the pages keep beside the static one,
 * [TRT-17476] "What changed", "Test Coverage"). Two passes over x:
 *   amax = max |x| over the finite elements (NaN and +-Inf excluded)
 *   s    = max( fl32(amax) / 448, 2^-126 )     (float32, IEEE division; the
 *          max-calibration rule behind the printed amax of [DF-15170] "Logs")
 *   q    = the fp8lin_quantize_static codes of x with input scale s
 * and s is stored to *scale_out on the device (for fp8lin_gemm_w8a8_dev_scale);
 * the host never reads it, so there is no synchronization.
 *   x, q       device, as for fp8lin_quantize_static (cols multiple of 16)
 *   scale_out  device, one float (written)
 *   amax_ws    device, one 32-bit word of scratch (cleared and overwritten
 *              on the stream; calls sharing it must not overlap)
 * rows or cols == 0: nothing is launched and *scale_out is left as it was.
 * Launches counted as FP8LIN_KERNEL_AMAX and FP8LIN_KERNEL_QUANTIZE.
 */
int32_t fp8lin_quantize_dynamic(const void* x_bf16, void* q_e4m3, int64_t rows, int64_t cols, float* scale_out,
                                uint32_t* amax_ws, hipStream_t stream);

/*
 * fp8lin_gemm_w8a8 with the input scale read from device memory (the scale
 * fp8lin_quantize_dynamic stored): alpha = weight_scale * (*input_scale_dev),
 * the same float product as the static call's, so the results agree bit for
 * bit with fp8lin_gemm_w8a8 given that scale on the host. *input_scale_dev
 * must be a positive normal float (it is not validated on the host).
 *   input_scale_dev  device, one float, 4-byte aligned
 */
int32_t fp8lin_gemm_w8a8_dev_scale(const void* qx, const void* qw, void* y_bf16, int64_t M, int64_t N, int64_t K,
                                   int64_t ldy, const float* input_scale_dev, float weight_scale,
                                   hipStream_t stream);

/*
 * Fail-closed check of a parsed policy ([TRT-17476] "Denoising-step
 * activation precision": unknown or missing fields, schema_version other than
 * 1 and any other type / index_space / default_mode / overlap are refused).
 * Returns FP8LIN_OK or FP8LIN_EPOLICY (FP8LIN_EINVAL for p == NULL). Host only.
 */
int32_t fp8lin_policy_validate(const fp8lin_policy* p);

/*
 * Mode of one transformer call ([DF-14664] "Behavior"; [TRT-17476]
 * "Denoising-step activation precision"). A pure function of its arguments:
 *   p == NULL (no policy, runtime: null)      -> W8A8 on every step
 *   tower == FP8LIN_TOWER_REASONER            -> p->reasoner_mode
 *   num_steps == 1 (one-step carve-out)       -> W8A8
 *   step < first_steps or step >= num_steps - last_steps -> W8A16
 *   otherwise                                 -> W8A8
 * step is the 0-based scheduler step, 0 <= step < num_steps (else
 * FP8LIN_EINVAL); an invalid policy gives FP8LIN_EPOLICY. Host only.
 */
int32_t fp8lin_step_policy(const fp8lin_policy* p, int32_t tower, int32_t step, int32_t num_steps,
                           int32_t* mode_out);

/* Static, NUL-terminated description of a status code. Host only. */
const char* fp8lin_strerror(int32_t status);

/* Kinds counted by fp8lin_launch_count(). */
enum {
  FP8LIN_KERNEL_QUANTIZE = 0,
  FP8LIN_KERNEL_GEMM_W8A8 = 1,
  FP8LIN_KERNEL_GEMM_W8A16 = 2,
  FP8LIN_KERNEL_SWIGLU = 3,
  FP8LIN_KERNEL_GATE_UP_SWIGLU = 4,
  FP8LIN_KERNEL_AMAX = 5,
  FP8LIN_KERNEL_SPLIT = 6, /* float32 activation -> three bf16 pieces */
  FP8LIN_KERNEL_QK_NORM_ROPE = 7,
  FP8LIN_KERNEL_SPLITK_REDUCE = 8, /* sum of split-K partials */
  FP8LIN_KERNEL_KINDS = 9
};

/* Number of kernels of `kind` this process has enqueued through the library
 * (host-side atomic counter; -1 for an unknown kind). Lets a test check that a
 * shared group quantizes exactly once per call. Host only, thread-safe. */
int64_t fp8lin_launch_count(int32_t kind);

#ifdef __cplusplus
}
#endif

#endif /* FP8LIN_H */
