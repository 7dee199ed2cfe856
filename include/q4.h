/*
 * q4.h — group-wise affine INT4 weight quantization (round to nearest) and the W4A16 matmul
 * that consumes it, for AMD MI355X (gfx950).  C ABI: plain pointers and sizes only.
 *
 * What is computed
 * ----------------
 * Quantization follows "DL S067 · Quantization — INT8, INT4, GPTQ, AWQ", §1 "The core math"
 * (asymmetric: scale = (beta - alpha) / (q_max - q_min), z = round(q_min - alpha / scale),
 * q = clip(round(x / scale) + z, q_min, q_max); symmetric: zero-point dropped and
 * scale = max|x| / q_max) applied per group of g consecutive weights along K within each
 * output row ("Model Quantization" §1 "Group-wise Quantization"; "DL S067" §2).  The matmul
 * is W4A16 in the sense of "LLM Weight Quantization - GPTQ, AWQ, SmoothQuant, FP8 &
 * INT4/INT8 Trade-offs", "The vocabulary": the 4-bit weights are dequantised inside the
 * kernel and the product runs on 16-bit operands.
 *
 * Exact rules (the pages leave these open; this library fixes them):
 *   - W is widened to fp32 (exact).  alpha = min(group, 0), beta = max(group, 0).
 *   - asymmetric: codes in [0, 15], s32 = fl32(fl32(beta - alpha) / 15);
 *     symmetric:  codes in [-8, 7],  s32 = fl32(max|x| / 7), z = 0.
 *   - scale = fp16_rne(min(s32, 65504)); a scale that rounds to 0 is stored as 1.0.
 *   - z = clamp(rint(-alpha / scale), 0, 15); q = clamp(rint(x / scale) + z, q_min, q_max),
 *     rint = round half to even of the exact quotient (equal to rint of the IEEE fp32
 *     quotient for every bf16 x and fp16 scale).
 *   - dequantised weight: scale * (q - z).  Y = X * dequant(W)^T, fp32 accumulation,
 *     Y rounded to bf16 (round to nearest even).
 * NaN or Inf inputs are outside the method's domain: outputs are then unspecified.
 *
 * Layouts (all row-major, contiguous, little-endian)
 *   W       bf16  [N, K]      weights, N output features, K input features
 *   packed  uint8 [N, K/2]    codes, two per byte, even k in the low nibble; symmetric codes
 *                             are 4-bit two's complement
 *   scales  fp16  [N, K/g]
 *   zeros   uint8 [N, K/g]    0 in symmetric mode
 *   X       bf16  [M, K]      activations
 *   Y       bf16  [M, N]
 *
 * Ownership, streams, errors
 *   - Every pointer is device memory allocated by the caller.  The library never allocates,
 *     frees or retains memory, and keeps no per-call state.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL means the default stream) and the
 *     call returns without synchronizing.  Kernel faults surface at the caller's next
 *     synchronization, as usual in HIP.  Calls are thread-safe.
 *   - Arguments are validated before anything is enqueued; on error a negative status is
 *     returned and nothing is launched.  A launch failure reported by the HIP runtime
 *     returns Q4_ERR_HIP.
 */
#ifndef Q4_H
#define Q4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q4_VERSION 10400  /* 1.4.0 */

typedef enum {
    Q4_ASYM = 0,   /* uint4 codes [0, 15] with a uint8 zero-point per group */
    Q4_SYM = 1     /* int4 codes [-8, 7], zero-point 0                      */
} q4_mode_t;

typedef enum {
    Q4_KERNEL_AUTO = 0,    /* choose by M, N, K, g (see q4_select_kernel)                           */
    Q4_KERNEL_GEMV = 1,    /* decode GEMV, M <= 2: fp32 wave reduction of exact fp16 (q - z) dots  */
    Q4_KERNEL_GEMM = 2,    /* bf16 MFMA GEMM on dequantised bf16 tiles, any M (K % 128 == 0 and a
                              power-of-two g >= 32: X staged in LDS, W dequantised in registers;
                              otherwise W dequantised into LDS)                                   */
    Q4_KERNEL_DECODE = 3   /* decode, 16 rows of X per launch: fp16 MFMA on exact (q - z) and exactly
                              scaled X (bf16 MFMA where X's range inside a K part exceeds fp16's),
                              fp32 per-group scaling                                              */
} q4_kernel_t;

typedef enum {
    Q4_DTYPE_BF16 = 0,     /* bfloat16 output */
    Q4_DTYPE_F16 = 1       /* IEEE binary16 output */
} q4_dtype_t;

typedef enum {
    Q4_SCALE_MUL = 0,      /* out = A * s per column */
    Q4_SCALE_DIV = 1       /* out = A / s per column */
} q4_scale_op_t;

enum {
    Q4_OK = 0,
    Q4_ERR_NULL = -1,      /* a required pointer is NULL                                    */
    Q4_ERR_SHAPE = -2,     /* N < 1, K < 1, M < 0, or a size beyond 2^31 - 1                */
    Q4_ERR_GROUP = -3,     /* g < 32, g % 32 != 0, or K % g != 0                             */
    Q4_ERR_MODE = -4,      /* mode, kernel selector or output type out of range              */
    Q4_ERR_ALIGN = -5,     /* W, X, packed or a dequantize output not 16-byte aligned; scales
                              or Y not 2-byte                                                 */
    Q4_ERR_HIP = -6,       /* the HIP runtime rejected a launch                              */
    Q4_ERR_ALIAS = -7,     /* an output buffer overlaps an input or another output          */
    Q4_ERR_UNSUPPORTED = -8, /* explicit kernel choice cannot run this shape (e.g. GEMV, M > 2) */
    Q4_ERR_WORKSPACE = -9, /* workspace smaller than the matching *_workspace_bytes() requires */
    Q4_ERR_VALUE = -10,    /* a numeric parameter out of range (GPTQ damping)                 */
    Q4_ERR_SCRATCH = -11   /* sizes need more scratch than the library's static buffer holds */
};

/*
 * Quantize W[N, K] (bf16) group-wise with round to nearest.
 * Source: "DL S067 · Quantization — INT8, INT4, GPTQ, AWQ", §1 (formulas) and §2 (groups).
 *
 *   W       device, bf16 [N, K], 16-byte aligned
 *   N, K    1 <= N, K <= 2^31 - 1
 *   g       group size: multiple of 32, K % g == 0 (g = K gives one group per row)
 *   mode    Q4_ASYM or Q4_SYM
 *   packed  device, uint8 [N, K/2], 16-byte aligned (output)
 *   scales  device, fp16  [N, K/g], 2-byte aligned (output)
 *   zeros   device, uint8 [N, K/g] (output; all 0 in symmetric mode)
 *   stream  hipStream_t or NULL
 * Returns Q4_OK or a negative status.  Outputs are bit-exact with the rules above.
 */
int q4_quantize_rtn(const void* W, int64_t N, int64_t K, int32_t g, int32_t mode,
                    void* packed, void* scales, void* zeros, void* stream);

/*
 * Y[M, N] = X[M, K] * dequant(packed, scales, zeros)^T, bf16 out, fp32 accumulation.
 * Source: W4A16 as defined in "LLM Weight Quantization - GPTQ, AWQ, SmoothQuant, FP8 &
 * INT4/INT8 Trade-offs", "The vocabulary"; dequantisation x_hat = scale * (q - z) from
 * "DL S067 · Quantization", §1.
 *
 *   X       device, bf16 [M, K], 16-byte aligned (may be NULL only when M == 0)
 *   M       0 <= M <= 2^31 - 1 (M == 0 returns Q4_OK and launches nothing)
 *   N, K, g, mode   as for q4_quantize_rtn; they must describe packed/scales/zeros
 *   packed, scales  device inputs as produced by q4_quantize_rtn
 *   zeros   device input; ignored and may be NULL in symmetric mode
 *   Y       device, bf16 [M, N], 2-byte aligned (output; must not overlap any input)
 * Accuracy: |Y - Y_exact| <= 8e-3 * sum_k |X[m,k] * x_hat[n,k]| + 1e-6 per element, where
 * Y_exact is the fp64 product with the dequantised weights.
 */
int q4_matmul(const void* X, int64_t M, int64_t N, int64_t K, int32_t g, int32_t mode,
              const void* packed, const void* scales, const void* zeros, void* Y, void* stream);

/*
 * out[N, K] = scale * (q - z) for every weight, rounded once (to nearest even) to bf16 or fp16:
 * the dequantisation of "DL S067 · Quantization — INT8, INT4, GPTQ, AWQ", §1 "The core math"
 * (x_hat = scale * (q - z)) with the per-group parameters of "Model Quantization" §1
 * "Group-wise Quantization".  For callers that feed the dequantised weights to another
 * library's GEMM.  The value before rounding is exact (an fp16 scale times an integer in
 * [-15, 15]), so the output is bit-exact; with Q4_DTYPE_F16 a product beyond the fp16 range
 * becomes +-Inf.
 *
 *   N, K, g, mode   as for q4_quantize_rtn; they must describe packed/scales/zeros
 *   packed, scales  device inputs as produced by q4_quantize_rtn (packed 16-byte aligned)
 *   zeros   device input; ignored and may be NULL in symmetric mode
 *   out     device, [N, K] of out_dtype, 16-byte aligned (output; must not overlap an input)
 *   out_dtype  Q4_DTYPE_BF16 or Q4_DTYPE_F16
 */
int q4_dequantize(int64_t N, int64_t K, int32_t g, int32_t mode, const void* packed,
                  const void* scales, const void* zeros, void* out, int32_t out_dtype,
                  void* stream);

/*
 * AWQ-style activation-aware scaling before RTN.
 * Source: "LLM Weight Quantization - GPTQ, AWQ, SmoothQuant, FP8 & INT4/INT8 Trade-offs",
 * "GPTQ vs AWQ: two ways to choose what error to keep" (the toy's activation-aware search) and
 * "DL S067 · Quantization", §5 "AWQ intuition": scale the weight columns of input channels with
 * large activations up by s before quantizing, divide the activations by s, and search the
 * exponent of s on calibration data by the layer's output error.  The kernels at serve time
 * are the plain ones: the quantized weights are those of W * s, and the caller folds 1/s into
 * the activations (or the previous layer).  Rules this library fixes:
 *   - a_j = mean over calibration rows of |X[m, j]| (fp32, fixed summation order), floored at
 *     2^-20 max_j a_j (an all-zero X gives s = 1);
 *   - alpha_i = i / (n_alpha - 1) (alpha = 0 when n_alpha == 1);
 *     s_j = a_j^alpha / sqrt(max_j a_j^alpha * min_j a_j^alpha), in fp32 (2^(alpha (log2 a_j -
 *     mean of log2 max a and log2 min a)), so within a few fp32 ulps of the exact value); s = 1
 *     exactly for alpha = 0;
 *   - scaled weights bf16(fl32(W[n, j] * s_j)) and scaled activations bf16(fl32(X[m, j] / s_j)):
 *     one IEEE fp32 product or quotient, then round to nearest even;
 *   - error_i = sum over the calibration outputs of (Y_i - Y_ref)^2 in fp64, Y_i the library's
 *     W4A16 product of the scaled activations and the quantized scaled weights, Y_ref the layer's
 *     unquantized output; the first smallest error wins.
 */

/* RTN quantization of W * s: as q4_quantize_rtn applied to bf16(fl32(W[n, k] * s[k])).
 *   s       device, fp32 [K], 16-byte aligned (input; must not overlap the outputs)
 *   other arguments and errors as for q4_quantize_rtn.  Outputs are bit-exact. */
int q4_quantize_rtn_scaled(const void* W, const void* s, int64_t N, int64_t K, int32_t g, int32_t mode,
                           void* packed, void* scales, void* zeros, void* stream);

/* out[r, c] = bf16(fl32(A[r, c] * s[c])) (Q4_SCALE_MUL) or bf16(fl32(A[r, c] / s[c]))
 * (Q4_SCALE_DIV): the activation side of AWQ-style scaling (X / s) or the weight side (W * s).
 *   A       device, bf16 [rows, cols], 16-byte aligned
 *   rows    0 <= rows <= 2^31 - 1 (rows == 0 returns Q4_OK and launches nothing)
 *   cols    8 <= cols <= 2^31 - 1, cols % 8 == 0 (else Q4_ERR_SHAPE)
 *   s       device, fp32 [cols], 16-byte aligned
 *   op      q4_scale_op_t (else Q4_ERR_MODE)
 *   out     device, bf16 [rows, cols], 16-byte aligned; may be A itself (in place), must not
 *           overlap A otherwise, nor s
 * Outputs are bit-exact (IEEE product / quotient, round to nearest even). */
int q4_scale_columns(const void* A, int64_t rows, int64_t cols, const void* s, int32_t op, void* out,
                     void* stream);

/* Bytes of device workspace q4_awq_search needs for these sizes, or a negative status
 * (Q4_ERR_SHAPE when M < 1 or n_alpha outside [1, 64], the q4_quantize_rtn errors otherwise).
 * Pure host function, no HIP call. */
int64_t q4_awq_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t g, int32_t n_alpha);

/* The activation-aware search and the final quantization, enqueued on `stream` without any
 * host synchronization (the best index is chosen on the device).
 *   X        device, bf16 [M, K] calibration activations, 16-byte aligned; 1 <= M <= 2^31 - 1
 *   Yref     device, bf16 [M, N], the layer's unquantized output on X (e.g. X W^T), 2-byte aligned
 *   W        device, bf16 [N, K] weights, 16-byte aligned
 *   N, K, g, mode   as for q4_quantize_rtn
 *   n_alpha  grid points in [1, 64] (11 gives the pages' grid 0, 0.1, ..., 1)
 *   workspace, workspace_bytes  device scratch of at least q4_awq_workspace_bytes(M, N, K, g,
 *            n_alpha) bytes, 256-byte aligned, owned by the caller; contents are overwritten
 *   s_out    device, fp32 [K], 16-byte aligned (output): the chosen alpha's scales
 *   packed, scales, zeros  outputs as for q4_quantize_rtn: the quantization of W * s_out
 *   errors   device, fp64 [n_alpha], 8-byte aligned (output): error_i per grid point
 *   best     device, int32 [1], 4-byte aligned (output): the chosen index i (alpha = i/(n_alpha-1))
 * No output may overlap an input, the workspace or another output (Q4_ERR_ALIAS).  Errors as
 * for q4_quantize_rtn and q4_matmul, plus Q4_ERR_WORKSPACE.  The outputs are deterministic. */
int q4_awq_search(const void* X, int64_t M, const void* Yref, const void* W, int64_t N, int64_t K,
                  int32_t g, int32_t mode, int32_t n_alpha, void* workspace, int64_t workspace_bytes,
                  void* s_out, void* packed, void* scales, void* zeros, void* errors, void* best,
                  void* stream);

/* For callers that cannot allocate device memory (code under stream capture, serving loops
 * that forbid hipMalloc): q4_awq_search with its scratch in a static device buffer of
 * q4_awq_static_scratch_bytes() bytes (64 MiB) that the library holds on each GPU it runs on
 * until the process ends, instead of a caller's workspace.  Arguments, outputs and errors as
 * for q4_awq_search without workspace and workspace_bytes, plus Q4_ERR_SCRATCH (returned before
 * any HIP call) when q4_awq_workspace_bytes(M, N, K, g, n_alpha) exceeds the buffer.  No call
 * allocates.  Calls on one GPU share its buffer: calls that overlap in time on one GPU (other
 * streams, other threads) race and must not be issued; calls in one stream are ordered. */
int64_t q4_awq_static_scratch_bytes(void);
int q4_awq_search_static(const void* X, int64_t M, const void* Yref, const void* W, int64_t N, int64_t K,
                         int32_t g, int32_t mode, int32_t n_alpha, void* s_out, void* packed, void* scales,
                         void* zeros, void* errors, void* best, void* stream);

/* As q4_matmul, but with an explicit kernel choice (q4_kernel_t).  Q4_KERNEL_GEMV requires
 * M == 1 and K <= 16384, or M == 2 and K <= 4096.  Q4_KERNEL_DECODE runs M > 16 as launches
 * of 16 rows of X and Y (the last one M mod 16 rows), each of which must fit the decode rule;
 * for a launch of M <= 16 rows it requires g in {32, 64, 128}, N * K / 2 < 2^32, and K split
 * into at most 8 equal ranges of KR
 * weights: KR = 32 P S with P = 4, 2 or 1 parts for M <= 4, <= 8 or <= 16, S = 16 slices (8
 * for g = 32 at M <= 8, and at M <= 4 for g = 64 or K a multiple of 1024 up to 8192), S
 * halved (down to P S = 16) while K is
 * not a multiple of KR or holds fewer than 4 ranges, and S = 32 for P = 1, g >= 64 and K a
 * multiple of 1024 above 4096; K % KR == 0, KR >= 512, and two stages of 16 rows x KR weights
 * per range fitting 160 KiB of LDS.  So K must be a multiple of 512, at most 4096 for g = 32
 * at M > 4, and at most 8192 otherwise (a multiple of 1024 above 4096 at M > 8).  Other shapes
 * return Q4_ERR_UNSUPPORTED.  Every kernel satisfies the same accuracy bound; callers use
 * this to pin a kernel. */
int q4_matmul_kernel(const void* X, int64_t M, int64_t N, int64_t K, int32_t g, int32_t mode,
                     const void* packed, const void* scales, const void* zeros, void* Y,
                     int32_t kernel, void* stream);

/* The kernel Q4_KERNEL_AUTO picks for this shape (Q4_KERNEL_GEMV, Q4_KERNEL_DECODE or
 * Q4_KERNEL_GEMM), or a negative status for an invalid shape: the GEMV for M == 1 (K <= 16384),
 * else the decode kernel where it fits (M <= 16), else the GEMV for M == 2 (K <= 4096), else
 * the decode kernel in 16-row launches where every launch fits and M <= 16 n, n = the number of
 * launches that take no longer than the GEMM by a cost model of MI355X (a launch 4.4 us plus
 * 0.001 us per k plus N K (1/2 + 3/g) bytes at 4.5 TB/s, the GEMM 0.0117 us per k), clamped to
 * 3 ... 6; else the GEMM.  Pure host function, no HIP call. */
int q4_select_kernel(int64_t M, int64_t N, int64_t K, int32_t g);

/*
 * W8A16: the same group-wise round-to-nearest with 8-bit codes, and its matmul.
 * Source: "LLM Weight Quantization - GPTQ, AWQ, SmoothQuant, FP8 & INT4/INT8 Trade-offs",
 * "Granularity and outliers" (W8A16: INT8 weights, 16-bit activations, the conservative choice)
 * with the formulas and INT8 ranges of "DL S067 · Quantization — INT8, INT4, GPTQ, AWQ", §1
 * "The core math".  The rules of q4_quantize_rtn hold with these changes:
 *   - asymmetric: codes in [0, 255], s32 = fl32(fl32(beta - alpha) / 255), z in [0, 255];
 *     symmetric:  codes in [-127, 127], s32 = fl32(max|x| / 127), z = 0;
 *   - g = K gives one scale per output row (per-channel).
 * Layouts
 *   codes   uint8 [N, K]      one code per byte; symmetric codes are int8 two's complement
 *   scales  fp16  [N, K/g];  zeros uint8 [N, K/g] (0 in symmetric mode)
 */

/* Quantize W[N, K] (bf16) group-wise to 8-bit codes.  Arguments, alignment (W and codes 16
 * bytes, scales 2), aliasing and errors as for q4_quantize_rtn, with codes [N, K].  Outputs are
 * bit-exact with the rules above. */
int q4_quantize_rtn8(const void* W, int64_t N, int64_t K, int32_t g, int32_t mode, void* codes,
                     void* scales, void* zeros, void* stream);

/* Y[M, N] = X[M, K] * dequant(codes, scales, zeros)^T, bf16 out, fp32 accumulation, with the
 * accuracy bound of q4_matmul.  Arguments as for q4_matmul_kernel, with codes [N, K] (16-byte
 * aligned) in place of packed.  kernel:
 *   Q4_KERNEL_AUTO  Q4_KERNEL_GEMV when it fits, else Q4_KERNEL_GEMM (see q4_select_kernel_w8);
 *   Q4_KERNEL_GEMV  decode GEMV for 1 <= M <= 4 with X staged in LDS, which needs
 *                   2.25 M K + 16 <= 160 KiB (e.g. M <= 4 at K = 16384, M <= 2 at K = 28672): exact
 *                   (q - z) in fp16 against x scaled by a power of two per 16 weights;
 *   Q4_KERNEL_GEMM  bf16 MFMA GEMM on dequantised bf16 tiles, any M;
 *   Q4_KERNEL_DECODE  not provided for 8-bit codes.
 * Q4_ERR_UNSUPPORTED when the chosen kernel cannot run the shape. */
int q4_matmul_w8(const void* X, int64_t M, int64_t N, int64_t K, int32_t g, int32_t mode,
                 const void* codes, const void* scales, const void* zeros, void* Y, int32_t kernel,
                 void* stream);

/* The kernel q4_matmul_w8 picks under Q4_KERNEL_AUTO (Q4_KERNEL_GEMV or Q4_KERNEL_GEMM; GEMM
 * for M == 0), or a negative status for an invalid shape.  Pure host function, no HIP call. */
int q4_select_kernel_w8(int64_t M, int64_t N, int64_t K, int32_t g);

/*
 * GPTQ: quantization that compensates each column's rounding error in the columns not yet
 * quantized, through the inverse Hessian of the layer's calibration inputs.
 * Source: "LLM Weight Quantization - GPTQ, AWQ, SmoothQuant, FP8 & INT4/INT8 Trade-offs",
 * "GPTQ vs AWQ: two ways to choose what error to keep" (table and toy); "Model Quantization",
 * §2.1 "GPTQ" (column-by-column quantization with a Cholesky factorisation of the inverse Hessian);
 * "DL S067 · Quantization", §4 "GPTQ intuition" (the update rule).  Rules this library fixes:
 *   - H = X^T X in fp32 over the M calibration rows, plus damp * mean(diag H) on the diagonal
 *     (damp = 0.01 in the pages' toy); an all-zero X gives H = I, i.e. plain RTN;
 *   - each group's scale and zero-point are RTN's on the original weights (fixed up front, as
 *     the toy fixes its row scale), so the output differs from q4_quantize_rtn in codes only;
 *   - columns are processed in order; the code of a compensated weight w' is
 *     clamp(rint(fl32(w' / scale)) + z), the same fp32 decision as RTN;
 *   - the compensation runs in fp32 (H, its Cholesky factor and the accumulated updates), so
 *     codes can differ from an exact evaluation where w' / scale lies close to a rounding
 *     boundary; the outputs are deterministic.
 * The matmul kernels consume the result like any q4_quantize_rtn output.
 */

/* Bytes of device workspace q4_gptq needs: 4 K^2 + 4 N K + 128 K bytes, each part rounded up to
 * 256; or a negative status (Q4_ERR_SHAPE when M < 1 or K > 32768, the q4_quantize_rtn errors
 * otherwise).  Pure host function, no HIP call. */
int64_t q4_gptq_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t g);

/* GPTQ of W on calibration activations X, enqueued on `stream` without host synchronization.
 *   X        device, bf16 [M, K] calibration activations, 16-byte aligned; 1 <= M <= 2^31 - 1
 *   W        device, bf16 [N, K] weights, 16-byte aligned; K <= 32768
 *   g, mode  as for q4_quantize_rtn
 *   damp     finite, >= 0 (else Q4_ERR_VALUE)
 *   workspace, workspace_bytes  device scratch of at least q4_gptq_workspace_bytes(M, N, K, g)
 *            bytes, 256-byte aligned, owned by the caller; contents are overwritten
 *   packed, scales, zeros  outputs as for q4_quantize_rtn
 *   info     device, int32 [1], 4-byte aligned (output): 0, or j + 1 when the Cholesky
 *            factorisation met a non-positive pivot at (reversed) column j, which it replaced
 *            by a tiny positive value so that the outputs are still written
 * No output may overlap an input, the workspace or another output (Q4_ERR_ALIAS); errors
 * otherwise as for q4_quantize_rtn plus Q4_ERR_WORKSPACE. */
int q4_gptq(const void* X, int64_t M, const void* W, int64_t N, int64_t K, int32_t g, int32_t mode, float damp,
            void* workspace, int64_t workspace_bytes, void* packed, void* scales, void* zeros, void* info,
            void* stream);

/* Static, NUL-terminated description of a status code; never NULL. */
const char* q4_status_string(int status);

/* Q4_VERSION of the built library. */
int q4_version(void);

#ifdef __cplusplus
}
#endif

#endif /* Q4_H */
