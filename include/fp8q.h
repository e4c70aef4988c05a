/*
 * fp8q -- the FP8 quantized linear layer of LLM inference on AMD Instinct
 * MI355X (gfx950): fused RMSNorm / SiLU-and-mul + dynamic FP8 quantization,
 * and the per-token and block-scaled FP8 GEMMs.
 *
 * The operations are the ones named on the page "Helion in vLLM: FP8
 * inference of Qwen3" (24-ai.news, 2026-06-10), section "Kernels integrated
 * into vLLM": rms_norm_dynamic_per_token_quant, rms_norm_per_block_quant,
 * silu_and_mul_dynamic_per_token_quant, silu_and_mul_per_block_quant,
 * dynamic_per_token_scaled_fp8_quant, per_token_group_fp8_quant, scaled_mm and
 * scaled_mm_blockwise.  The small-M split-K and swap-AB GEMM regimes follow
 * the page "Helion can accelerate vLLM LLM inference on NVIDIA GPUs"
 * (aihirek.info), section "One GEMM implementation handles several
 * algorithms"; the choice among them is a per-shape table (same page,
 * section "Autotuning picks the right variant").
 *
 * Formats (the pages say only "FP8"; these are the readings adopted):
 *   FP8   OCP e4m3 ("e4m3fn"): bias 7, max 448, no infinity, NaN 0x7F/0xFF.
 *   bf16  IEEE binary32 truncated to 16 bits, stored as uint16.
 *   scale fp32, scale = amax / 448 (IEEE division), q = e4m3(RN32(y / scale)),
 *         an all-zero group gets scale 0 and signed-zero codes.
 *   group 1 x 128 consecutive elements of a row; weight blocks 128 x 128.
 *
 * Conventions for every entry point
 *   - Outputs first, then inputs, then sizes and scalars, then the stream.
 *   - All pointers are DEVICE pointers owned by the caller; the library never
 *     allocates, frees or synchronizes, and keeps no state between calls.
 *   - All tensors are dense and row-major (no strides).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously on it; a successful return means the
 *     kernels were launched, not that they finished.
 *   - Arguments are checked on the host before any HIP call; a violation
 *     returns an error status and launches nothing.  M == 0 is a no-op that
 *     returns FP8Q_OK (pointers are then not inspected).
 *   - Every pointer must be 16-byte aligned.
 *   - Inputs must be finite; NaN or infinity in inputs is outside the
 *     contract (no fault, unspecified values).
 *   - Functions are reentrant; calls on one stream are ordered by the stream.
 *   - No C++ exception crosses this interface.
 */
#ifndef FP8Q_H
#define FP8Q_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8Q_VERSION 200 /* major*100 + minor */

typedef enum {
  FP8Q_OK = 0,
  FP8Q_ERR_INVALID_ARG = 1,       /* null pointer, negative size, bad eps */
  FP8Q_ERR_UNSUPPORTED_SHAPE = 2, /* size not a multiple the op needs     */
  FP8Q_ERR_ALIGNMENT = 3,         /* a pointer is not 16-byte aligned     */
  FP8Q_ERR_WORKSPACE = 4,         /* ws smaller than fp8q_workspace_size  */
  FP8Q_ERR_NO_DEVICE = 5,         /* no HIP device is usable              */
  FP8Q_ERR_ARCH = 6,              /* current device is not gfx950         */
  FP8Q_ERR_HIP = 7,               /* a HIP call failed, see last_hip_error*/
  FP8Q_ERR_BAD_MODE = 8,          /* unknown quantization mode            */
  FP8Q_ERR_BAD_CONFIG = 9         /* unknown or inapplicable GEMM config  */
} fp8q_status;

/* Quantization modes.  Dynamic modes compute the scale from the data and
 * WRITE it to `scale`; the static mode READS scale[0].
 *   amax/448 rule:  scale = RN32(amax / 448)
 *   UE8M0 rule:     scale = the smallest 2^e, e >= -127, with 448 * 2^e >= amax
 *                   (power-of-two scales, the format the page "Helion in
 *                   vLLM: FP8 inference of Qwen3", section "Practical
 *                   limits", names for DeepGEMM on B200); an all-zero group
 *                   gets 2^-127.
 * Codes are always q = e4m3(RN32(y / scale)), saturating. */
typedef enum {
  FP8Q_PER_TOKEN = 0,          /* one scale per row,    amax/448: scale [M]        (out) */
  FP8Q_GROUP128 = 1,           /* one scale per 1x128,  amax/448: scale [M, K/128] (out) */
  FP8Q_PER_TENSOR_STATIC = 2,  /* caller's scale for all elements: scale [1]      (in)
                                  scale[0] must be positive and finite             */
  FP8Q_PER_TOKEN_UE8M0 = 3,    /* one power-of-two scale per row:  scale [M]       (out) */
  FP8Q_GROUP128_UE8M0 = 4      /* one power-of-two scale per 1x128: [M, K/128]     (out) */
} fp8q_quant_mode;

typedef enum {
  FP8Q_OP_SCALED_MM = 0,
  FP8Q_OP_SCALED_MM_BLOCKWISE = 1,
  FP8Q_OP_SCALED_MM_INT8 = 2,          /* W8A8 INT8, fp8q_scaled_mm_int8 */
  FP8Q_OP_SCALED_MM_BLOCKWISE_UE8M0 = 3 /* fp8q_scaled_mm_blockwise_ue8m0 */
} fp8q_gemm_op;

/* ------------------------------------------------------------------------
 * Fused RMSNorm + dynamic FP8 quantization
 * (rms_norm_dynamic_per_token_quant / rms_norm_per_block_quant).
 *
 *   inv  = RN32(1 / sqrt(sum_k x[m,k]^2 / K + eps))   sum in fp64, the rest
 *                                                      in IEEE fp64
 *   y    = RN32(RN32(x[m,k] * w[k]) * inv)             no bf16 rounding of y
 *   then the quantizer of `mode` (fp8q_quant_mode).
 *
 *   q     [M, K]   e4m3 bytes            (out)
 *   scale fp32, shape and direction by mode (fp8q_quant_mode)
 *   x     [M, K]   bf16                  (in)
 *   w     [K]      bf16                  (in)
 *   eps   > 0, finite
 * Needs K > 0, K % 128 == 0 for the GROUP128 modes, K % 8 == 0 otherwise,
 * K <= 32768.
 * ---------------------------------------------------------------------- */
int fp8q_rmsnorm_quant(void* q, float* scale, const void* x, const void* w, int64_t M,
                       int64_t K, float eps, int mode, void* stream);

/* ------------------------------------------------------------------------
 * Fused SiLU-and-mul + dynamic FP8 quantization
 * (silu_and_mul_dynamic_per_token_quant / silu_and_mul_per_block_quant).
 *
 *   y[m,d] = RN32(silu(gate_up[m,d]) * gate_up[m,D+d]),  silu correctly
 *            rounded to fp32; then the quantizer as above.
 *
 *   q       [M, D]   e4m3 bytes           (out)
 *   scale   fp32, shape and direction by mode (fp8q_quant_mode)
 *   gate_up [M, 2D]  bf16, gate = columns [0,D), up = [D,2D)   (in)
 * Needs D > 0, D % 128 == 0 for the GROUP128 modes, D % 8 == 0 otherwise,
 * D <= 32768.
 * ---------------------------------------------------------------------- */
int fp8q_silu_mul_quant(void* q, float* scale, const void* gate_up, int64_t M, int64_t D,
                        int mode, void* stream);

/* ------------------------------------------------------------------------
 * Standalone FP8 quantization of a bf16 matrix
 * (dynamic_per_token_scaled_fp8_quant / per_token_group_fp8_quant, and the
 * static per-tensor form): the quantizer with an identity front end.
 * Arguments as for fp8q_rmsnorm_quant without w and eps.
 * ---------------------------------------------------------------------- */
int fp8q_quant(void* q, float* scale, const void* x, int64_t M, int64_t K, int mode,
               void* stream);

/* ------------------------------------------------------------------------
 * scaled_mm: per-token x per-channel scaled FP8 GEMM, "NT" layout.
 *
 *   y[m,n] = bf16( sa[m] * sb[n] * sum_k a[m,k] * b[n,k] )   fp32 accumulate
 *
 *   y  [M, N] bf16 (out)     a [M, K] e4m3 (in)   b [N, K] e4m3 (in)
 *   sa [M] fp32 (in)         sb [N] fp32 (in)
 *   ws / ws_bytes: device workspace of at least
 *                  fp8q_workspace_size(FP8Q_OP_SCALED_MM, M, N, K) bytes;
 *                  may be NULL when that size is 0.
 * Needs K % 128 == 0, N % 128 == 0, 0 < K <= 2^22, N > 0.
 * ---------------------------------------------------------------------- */
int fp8q_scaled_mm(void* y, const void* a, const void* b, const float* sa, const float* sb,
                   int64_t M, int64_t N, int64_t K, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * scaled_mm_blockwise: 1x128 activation x 128x128 weight block-scaled GEMM.
 *
 *   y[m,n] = bf16( sum_kb sa[m,kb] * sb[n/128,kb]
 *                          * sum_{k in block kb} a[m,k] * b[n,k] )
 *   products inside a 128-block are summed in fp32 before its scales apply.
 *
 *   y  [M, N] bf16 (out)    a [M, K] e4m3 (in)     b [N, K] e4m3 (in)
 *   sa [M, K/128] fp32 (in) sb [N/128, K/128] fp32 (in)
 *   (the argument order of fp8q_scaled_mm: operands, then their scales)
 *   ws / ws_bytes as for fp8q_scaled_mm (op FP8Q_OP_SCALED_MM_BLOCKWISE).
 * Needs K % 128 == 0, N % 128 == 0, 0 < K <= 2^22, N > 0.
 * ---------------------------------------------------------------------- */
int fp8q_scaled_mm_blockwise(void* y, const void* a, const void* b, const float* sa,
                             const float* sb, int64_t M, int64_t N, int64_t K, void* ws,
                             size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * W8A8 INT8: the same front ends and GEMM machinery with symmetric int8
 * operands (page "Helion can accelerate vLLM LLM inference on NVIDIA GPUs",
 * aihirek.info, section "Autotuning picks the right variant": W8A8_INT8
 * beside FP8_Dynamic and Block_FP8).
 *
 * Quantizers: as their FP8 counterparts with
 *   scale = RN32(amax / 127), q = clamp(rne(RN32(y / scale)), -127, 127),
 *   an all-zero row gets scale 0 and q = 0;
 *   q is int8 [M, K] (or [M, D]); modes FP8Q_PER_TOKEN (scale [M], out) and
 *   FP8Q_PER_TENSOR_STATIC (scale [1], in) only (else FP8Q_ERR_BAD_MODE).
 * GEMM (per-token x per-channel, "NT"):
 *   y[m,n] = bf16( sa[m] * sb[n] * sum_k a[m,k] * b[n,k] ),
 *   a int8 [M, K], b int8 [N, K], sa [M], sb [N] fp32; the integer sum is
 *   exact (int32, so K <= 131072); ws as for fp8q_scaled_mm with
 *   op FP8Q_OP_SCALED_MM_INT8.  Needs K % 128 == 0, N % 128 == 0, K <= 131072.
 * ---------------------------------------------------------------------- */
int fp8q_rmsnorm_quant_int8(void* q, float* scale, const void* x, const void* w, int64_t M,
                            int64_t K, float eps, int mode, void* stream);
int fp8q_silu_mul_quant_int8(void* q, float* scale, const void* gate_up, int64_t M,
                             int64_t D, int mode, void* stream);
int fp8q_quant_int8(void* q, float* scale, const void* x, int64_t M, int64_t K, int mode,
                    void* stream);
int fp8q_scaled_mm_int8(void* y, const void* a, const void* b, const float* sa,
                        const float* sb, int64_t M, int64_t N, int64_t K, void* ws,
                        size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * scaled_mm_blockwise for power-of-two (UE8M0) scales, e.g. activations from
 * the FP8Q_GROUP128_UE8M0 quantizer and weights with power-of-two block
 * scales.  Same arguments and result as fp8q_scaled_mm_blockwise.  The
 * eight-wave tiled kernels fold such scales exactly into the e4m3 -> f16
 * widening and drop the per-block scale multiply-add (page "Helion in vLLM:
 * FP8 inference of Qwen3", section "Practical limits", on UE8M0 scales);
 * wherever a scale is not a power of two, or the exponents of one token row
 * or weight block span more than 22 binades, those kernels take the general
 * path, so any scales give the fp8q_scaled_mm_blockwise result.  The other
 * variants (four-wave tiles, the weight-streaming kernel), where folding
 * measured no faster, run the general path throughout.
 * ---------------------------------------------------------------------- */
int fp8q_scaled_mm_blockwise_ue8m0(void* y, const void* a, const void* b, const float* sa,
                                   const float* sb, int64_t M, int64_t N, int64_t K, void* ws,
                                   size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * fp8q_scaled_mm_blockwise for callers that cannot allocate device memory:
 * code under HIP graph capture, serving loops and harnesses that forbid
 * hipMalloc.  Same operands, result and errors as fp8q_scaled_mm_blockwise
 * (the same kernels; results identical bit for bit), without ws/ws_bytes:
 * when the table's variant for the shape splits K across workgroups, its
 * fp32 partials go to a scratch array the library holds on each GPU it runs
 * on (FP8Q_NOALLOC_SCRATCH_BYTES, resident until the process ends) instead
 * of a caller workspace.  The call allocates nothing and records no memset
 * (every partial is written before it is read).
 * Returns FP8Q_ERR_WORKSPACE, before touching the device, when the shape's
 * variant needs more than FP8Q_NOALLOC_SCRATCH_BYTES of partials, i.e. when
 * fp8q_workspace_size(FP8Q_OP_SCALED_MM_BLOCKWISE, M, N, K) exceeds it (the
 * Qwen3 shapes need at most 32 MiB; a long K split across all columns of a
 * mid-size M can need more, e.g. 80 MiB at M=1024, N=5120, K=25600).
 * All calls on one GPU share its scratch array: calls whose executions
 * overlap on one GPU (concurrent streams, or threads) race on it and give
 * undefined results.  Calls ordered on one stream are safe.
 * ---------------------------------------------------------------------- */
#define FP8Q_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int fp8q_scaled_mm_blockwise_noalloc(void* y, const void* a, const void* b, const float* sa,
                                     const float* sb, int64_t M, int64_t N, int64_t K,
                                     void* stream);

/* Bytes of workspace the GEMM `op` needs for this shape with the table's
 * choice (0 when the chosen variant needs none).  Pure host function. */
size_t fp8q_workspace_size(int op, int64_t M, int64_t N, int64_t K);

/* ------------------------------------------------------------------------
 * Blockwise GEMM with SiLU-and-mul and group-128 quantization fused into its
 * epilogue: the MLP's gate_up projection followed by silu_mul_quant (the
 * blockwise GEMM and the per-block SiLU-and-mul quantizer of the page
 * "Helion in vLLM: FP8 inference of Qwen3", section "Kernels integrated into
 * vLLM", one after the other) in one kernel, without writing the bf16
 * gate_up product to memory.  The results are those of
 *
 *   fp8q_scaled_mm_blockwise(y, a, b, sa, sb, M, N, K, ...)   y bf16 [M, N]
 *   fp8q_silu_mul_quant(q, scale, y, M, N / 2, FP8Q_GROUP128, ...)
 *
 * with the GEMM's 128x256-tile variant (the two agree bit for bit).
 *
 *   q     [M, N/2]        e4m3 bytes          (out)
 *   scale [M, N/2/128]    fp32                (out)
 *   a, b, sa, sb as for fp8q_scaled_mm_blockwise; b holds N rows, the gate
 *   rows [0, N/2) then the up rows [N/2, N).
 * Needs N % 256 == 0, K % 128 == 0 and (N/2 + 128) * K < 2^32; no workspace.
 * Efficient for large M
 * (one workgroup per 128 tokens x 128 output columns); correct for every
 * M >= 0 (M == 0 is a no-op).  Errors as for fp8q_scaled_mm_blockwise.
 * ---------------------------------------------------------------------- */
int fp8q_scaled_mm_blockwise_silu_quant(void* q, float* scale, const void* a, const void* b,
                                        const float* sa, const float* sb, int64_t M, int64_t N,
                                        int64_t K, void* stream);

/* ------------------------------------------------------------------------
 * GEMM variants.  The same GEMMs with the variant forced instead of taken
 * from the per-shape table; used by tests (every variant is checked) and by
 * the table's tuner.  cfg < 0 means "use the table".  Variant names start
 * with the engine: f16_ (exact: e4m3 widened losslessly to f16; every FP8
 * variant), i8_ (int8 op only).  Then the kind: _tiled_m<BM>_n<BN>_w<WM>x<WN>
 * _st<stages> (LDS-staged tiles; _s<S>: K split over S workgroup rows, with
 * fp32 partials in the workspace; _p: raised wave priority), _tiled_..._h<S>
 * (hybrid: the column tiles that fill whole rounds of workgroups unsplit, the
 * remaining columns on 128x128 tiles split S ways; its column split, and so
 * its workspace size, depend on the current device's compute-unit count),
 * _skinny_t<T>_r<R>_k<W>_j<J> (weight-streaming kernel for up to 16*T
 * tokens).
 * Non-conforming opt-in: with the environment variable
 * FP8Q_NONCONFORMING_FP8_MFMA=1 set before the first GEMM call, the registry
 * also holds f8_ variants, which run the FP8 matrix instruction itself.  Its
 * datapath truncates products inside groups of 8 consecutive K, so their
 * results do NOT meet the GEMM accuracy contract of this library; they exist
 * only to measure that.  Without the variable they do not exist (num_configs
 * excludes them) and nothing selects them.
 * Returns FP8Q_ERR_BAD_CONFIG when cfg is unknown, cannot run this shape,
 * or belongs to another op.
 * ---------------------------------------------------------------------- */
int fp8q_gemm_num_configs(void);
const char* fp8q_gemm_config_name(int cfg);
int fp8q_gemm_config_for(int op, int64_t M, int64_t N, int64_t K); /* table lookup */
size_t fp8q_workspace_size_cfg(int cfg, int64_t M, int64_t N, int64_t K);
int fp8q_scaled_mm_cfg(void* y, const void* a, const void* b, const float* sa,
                       const float* sb, int64_t M, int64_t N, int64_t K, void* ws,
                       size_t ws_bytes, int cfg, void* stream);
int fp8q_scaled_mm_blockwise_cfg(void* y, const void* a, const void* b, const float* sa,
                                 const float* sb, int64_t M, int64_t N, int64_t K, void* ws,
                                 size_t ws_bytes, int cfg, void* stream);
int fp8q_scaled_mm_int8_cfg(void* y, const void* a, const void* b, const float* sa,
                            const float* sb, int64_t M, int64_t N, int64_t K, void* ws,
                            size_t ws_bytes, int cfg, void* stream);
int fp8q_scaled_mm_blockwise_ue8m0_cfg(void* y, const void* a, const void* b, const float* sa,
                                       const float* sb, int64_t M, int64_t N, int64_t K,
                                       void* ws, size_t ws_bytes, int cfg, void* stream);

/* ------------------------------------------------------------------------
 * Elementwise building blocks (also used to test the device arithmetic
 * exhaustively).
 *   fp8q_cvt_e4m3: q[i] = e4m3(x[i]) for fp32 x, round to nearest even,
 *                  saturating to +-448, sign of zero kept.
 *   fp8q_silu:     y[i] = fp32 silu(g[i]) correctly rounded, g bf16.
 * n >= 0; n == 0 is a no-op.
 * ---------------------------------------------------------------------- */
int fp8q_cvt_e4m3(void* q, const float* x, int64_t n, void* stream);
int fp8q_silu(float* y, const void* g, int64_t n, void* stream);

/* ------------------------------------------------------------------------
 * Launch shape the library picks for a quantizer call (a pure host function,
 * no device needed; for tests that check which kernel instantiations a
 * workload reaches).  front_end: 0 = fp8q_quant, 1 = fp8q_rmsnorm_quant,
 * 2 = fp8q_silu_mul_quant (K = D); mode as for those calls; num_cus the
 * device's compute-unit count.  Writes the threads per work unit (64, 128 or
 * 256), the 16-byte chunks each thread holds (the instantiation's CH) and
 * the workgroup count.  Errors: FP8Q_ERR_INVALID_ARG (M <= 0, K <= 0,
 * num_cus <= 0, null outputs, unknown front end), FP8Q_ERR_BAD_MODE,
 * FP8Q_ERR_UNSUPPORTED_SHAPE (as the call itself would return).
 * ---------------------------------------------------------------------- */
int fp8q_quant_launch_config(int front_end, int mode, int64_t M, int64_t K, int num_cus,
                             int* tpr, int* ch, int* grid);

/* Diagnostics. */
const char* fp8q_status_string(int status);
int fp8q_last_hip_error(void); /* hipError_t of this thread's last FP8Q_ERR_HIP */
int fp8q_version(void);

#ifdef __cplusplus
}
#endif
#endif /* FP8Q_H */
