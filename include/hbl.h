/*
 * hbl.h -- C ABI of the H-BitLinear forward pass (BitNet v2) for AMD MI355X (gfx950).
 *
 * The layer (QbitAI article on BitNet v2, section 引入H-BitLinear模块; 新智元
 * article "微软再放LLM量化大招", sections BitNet v2：原生4位激活 and H-BitLinear模块):
 *
 *     y = dequant( Q_act( H_K . RMSNorm(x) / sqrt(K) ) . W_t^T )
 *
 *   RMSNorm    r_m = sqrt(mean_k x[m][k]^2 + 1e-6),  u = x * g / r_m   (g = 1 if gain == NULL)
 *   rotation   online Walsh-Hadamard transform over K, Sylvester order, scaled by 1/sqrt(K)
 *   INT8       per-token absmax:  G = max(max_k |xt|, 1e-5), q = round(xt * 127 / G), d = G / 127
 *   INT4       per-token absmean: G = max(mean_k |xt|, 1e-5), q = clamp(round(xt * sqrt7 / G), -8, 7),
 *              d = G / sqrt7
 *   weights    per-tensor absmean ternary: alpha = mean |W|, a = max(alpha, 1e-5),
 *              W_t = clamp(round(W / a), -1, 1)   (done once, offline)
 *   matmul     acc[m][n] = sum_k q[m][k] * W_t[n][k]   (exact int32)
 *   dequant    y[m][n] = acc[m][n] * (d[m] * a)
 * Rounding is round-half-to-even.  The HIP path computes the normalisation,
 * rotation and scales in fp32.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates or frees memory.  Tensors are dense row-major.
 *   - Every call is asynchronous on `stream` (NULL = default stream) and does
 *     no host synchronisation; outputs are valid once the stream reaches them.
 *   - Arguments are validated before anything is launched.  On any error
 *     nothing is launched and outputs are untouched.  Launch failures are
 *     reported as HBL_ERR_LAUNCH.  Nothing aborts or throws across the ABI.
 *   - M == 0 is valid: after the dtype and shape checks the call returns
 *     HBL_OK without launching anything (pointers may then be NULL).
 *   - Shapes: K is a power of two with 64 <= K <= 32768; N % 16 == 0 and
 *     N > 0; 0 <= M < 2^31; M * max(K, N) < 2^40.  Codes in the fp6 operand
 *     layout (bits = HBL_BITS_INT4_FP6) need K >= 256 (HBL_ERR_SHAPE below).
 *   - Alignment: every pointer must be 16-byte aligned (HBL_ERR_ALIGN).
 *   - The library keeps no mutable global state other than a per-device
 *     cache of device properties filled on first use; distinct streams may
 *     call concurrently with distinct workspaces.
 *   - Only gfx950 devices are supported (HBL_ERR_DEVICE otherwise).
 *
 * Data formats:
 *   packed ternary weights  N*K/4 bytes (uint8 [N][K/4] in size): one
 *       little-endian 32-bit word per 16 consecutive k of a row; the code of
 *       k0 + 4*j + i (i, j in 0..3) occupies bits 8*i + 2*j .. 8*i + 2*j + 1
 *       of the word of k0, with the 2-bit codes 0b00 = 0, 0b01 = +1,
 *       0b11 = -1 (0b10 never written).  The words are tiled: tiles of 16
 *       rows x TW k, TW = min(K, 256), in row-block-major order, and inside
 *       a tile the TW/16 words of each row contiguous, so with T = TW/16 word
 *       w of row n (k = 16w .. 16w+15) is word ((n/16)*(K/TW) + w/T)*16*T +
 *       (n%16)*T + w%T.  (Sixteen rows' 64-byte segments of one 256-k block
 *       are one contiguous KiB, read whole by the matmuls; for K <= 256 the
 *       layout is plain row-major.)
 *   INT8 activation codes   int8 [M][K], two's complement.
 *   INT4 activation codes   uint8 [M][K/2]: for each row, one little-endian
 *       32-bit word per 8 consecutive k; the code of k0 + 4*j + i (i in 0..3,
 *       j in 0..1) occupies bits 8*i + 4*j .. 8*i + 4*j + 3, as a 4-bit two's
 *       complement nibble.
 *   INT4 codes, fp6 operand layout (bits = HBL_BITS_INT4_FP6)   uint8 [K/128][M][96]
 *       (M*K*3/4 bytes): the same codes q in [-8, 7], each stored as the OCP
 *       fp6 e2m3 encoding of q/2 (sign bit 5, exponent bits 4..3 with bias 1,
 *       mantissa bits 2..0; every q/2 is exact).  Token m's codes of the k
 *       block [128*kb, 128*kb + 128) are the 96 bytes at (kb*M + m)*96: four
 *       24-byte little-endian groups, group j for k0 = 128*kb + 32*j; field p
 *       (p in 0..31) occupies bits 6*p .. 6*p + 5 of its group and holds the
 *       code of k0 + b + 4*d0 + 8*h + 16*d1, where p = h + 2*b + 8*d0 + 16*d1
 *       (b in 0..3; h, d0, d1 in 0..1).  This is the operand layout of the
 *       gfx950 fp6 x fp4 matrix instruction for the weights' packed order,
 *       blocked so that 128 k of consecutive tokens are contiguous; the INT4
 *       forward uses it internally for M > 64 and K >= 256.
 *   per-token dequant scales d   fp32 [M].
 *   per-tensor weight scale      fp32 [1] (alpha; the floor 1e-5 is applied on use).
 */
#ifndef HBL_H
#define HBL_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    HBL_OK = 0,
    HBL_ERR_NULL = 1,       /* a required pointer is NULL */
    HBL_ERR_SHAPE = 2,      /* M, K or N outside the supported set */
    HBL_ERR_DTYPE = 3,      /* unknown dtype or bit width */
    HBL_ERR_ALIGN = 4,      /* a pointer is not 16-byte aligned */
    HBL_ERR_WORKSPACE = 5,  /* workspace smaller than hbl_workspace_bytes() */
    HBL_ERR_LAUNCH = 6,     /* the HIP runtime reported an error at launch */
    HBL_ERR_DEVICE = 7,     /* no current device, or it is not gfx950 */
    HBL_ERR_SCRATCH = 8,    /* hbl_forward_noalloc: the problem needs more than
                               HBL_NOALLOC_SCRATCH_BYTES of scratch */
    /* range markers, never returned: with them every int is a value of the
       type, so C++ code may hold any value a C caller passes */
    HBL_STATUS_RANGE_MIN_ = -2147483647 - 1, HBL_STATUS_RANGE_MAX_ = 2147483647
} hbl_status;

/* Element types.  Any other value is rejected with HBL_ERR_DTYPE; the range
 * markers (never valid arguments) make every int a value of the type, so that
 * rejection is well defined in the C++ implementation. */
typedef enum {
    HBL_F32 = 0, HBL_BF16 = 1,
    HBL_DTYPE_RANGE_MIN_ = -2147483647 - 1, HBL_DTYPE_RANGE_MAX_ = 2147483647
} hbl_dtype;

/* Activation code formats (the `bits` argument of the stage calls). */
enum { HBL_BITS_INT4 = 4, HBL_BITS_INT4_FP6 = 6, HBL_BITS_INT8 = 8 };

/* Operation selector for hbl_workspace_bytes. */
enum { HBL_OP_QUANTIZE_WEIGHTS = 0, HBL_OP_MATMUL = 1, HBL_OP_QUANTIZE_WEIGHTS_ROTATED = 2,
       HBL_OP_FORWARD_INT4 = 4, HBL_OP_FORWARD_INT8 = 8, HBL_OP_BACKWARD = 16 };

/* Human-readable name of a status code (static string, never NULL). */
const char *hbl_status_string(hbl_status s);

/* Bytes of device workspace the operation needs for these sizes (0 for an
 * invalid op).  Host-only; never touches the device. */
size_t hbl_workspace_bytes(int op, int64_t M, int64_t K, int64_t N);

/*
 * Offline per-tensor absmean ternarisation of latent weights
 * (QbitAI article, section 引入H-BitLinear模块; 新智元 article, section
 * H-BitLinear模块: weights become {-1, 0, 1} with one absmean scale).
 *   w         fp32 [N][K] latent weights (device, read only)
 *   w_packed  uint8 [N][K/4] packed ternary codes (device, written)
 *   w_alpha   fp32 [1] alpha = mean|W| (device, written).  The sum of |W| is
 *             taken in fp64 in a fixed order (64-column blocks of each row
 *             left to right, the block sums in order, then the row sums in
 *             row order), so alpha is reproducible from call to call and
 *             within one fp32 ulp of the exactly rounded mean.
 *   workspace at least hbl_workspace_bytes(HBL_OP_QUANTIZE_WEIGHTS, 0, K, N) bytes.
 */
hbl_status hbl_quantize_weights(const float *w, int64_t N, int64_t K,
                                uint8_t *w_packed, float *w_alpha,
                                void *workspace, size_t ws_bytes, hipStream_t stream);

/*
 * Whole H-BitLinear forward with INT8 (per-token absmax) activations
 * (QbitAI article, section 引入H-BitLinear模块; 新智元 article, section
 * H-BitLinear模块).
 *   x         [M][K] activations, dtype x_dtype (fp32 or bf16)
 *   gain      fp32 [K] RMSNorm gain, or NULL for 1
 *   w_packed  uint8 [N][K/4] from hbl_quantize_weights;  w_alpha fp32 [1]
 *   y         [M][N] output, dtype y_dtype (fp32 or bf16; bf16 rounds to nearest even)
 *   workspace at least hbl_workspace_bytes(HBL_OP_FORWARD_INT8, M, K, N) bytes;
 *             holds the activation codes and scales between the two kernels
 *             (unused where the whole layer is one kernel: 1..4 tokens at
 *             K = 8192 / 16384 while M * K <= 16384, and up to 64 tokens at
 *             K <= 256; the size asked for is the same),
 *             and for 33..64 tokens with K = 32768 the split-K partial sums
 *             plus one arrival counter per 64-channel tile, which the first
 *             kernel of each call clears (the workspace needs no
 *             initialisation; calls sharing one workspace must be
 *             stream-ordered).
 */
hbl_status hbl_forward_int8(const void *x, hbl_dtype x_dtype, const float *gain,
                            const uint8_t *w_packed, const float *w_alpha,
                            int64_t M, int64_t K, int64_t N,
                            void *y, hbl_dtype y_dtype,
                            void *workspace, size_t ws_bytes, hipStream_t stream);

/* Same with INT4 (per-token absmean) activations; the arguments mean the same. */
hbl_status hbl_forward_int4(const void *x, hbl_dtype x_dtype, const float *gain,
                            const uint8_t *w_packed, const float *w_alpha,
                            int64_t M, int64_t K, int64_t N,
                            void *y, hbl_dtype y_dtype,
                            void *workspace, size_t ws_bytes, hipStream_t stream);

/*
 * The forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same kernels as hbl_forward_int8 (bits = 8) and hbl_forward_int4 (bits = 4),
 * with the same arguments and results, but no workspace argument.  Its
 * scratch (activation codes, scales, split-K partials and arrival counters)
 * is a static device array of HBL_NOALLOC_SCRATCH_BYTES that each GPU the
 * library runs on holds until the process ends; the call itself allocates
 * nothing.  A problem whose workspace (hbl_workspace_bytes(HBL_OP_FORWARD_INT8
 * or _INT4, M, K, N)) exceeds that size returns HBL_ERR_SCRATCH before
 * anything touches the device.  The array keeps the last call's contents; the
 * kernels clear what must start at zero.  Every call on one GPU shares that
 * GPU's array, so calls that may overlap on one GPU (different streams, or
 * different host threads without ordering) race: serialise them.
 */
#define HBL_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
hbl_status hbl_forward_noalloc(int bits, const void *x, hbl_dtype x_dtype, const float *gain,
                               const uint8_t *w_packed, const float *w_alpha,
                               int64_t M, int64_t K, int64_t N,
                               void *y, hbl_dtype y_dtype, hipStream_t stream);

/* ---- variants beside H-BitLinear ---- */

/*
 * BitLinear forward without the Hadamard rotation, for the layers whose
 * inputs are already close to Gaussian (attention and FFN input projections;
 * 新智元 article "微软再放LLM量化大招", section H-BitLinear模块):
 *     y = dequant( Q_act( RMSNorm(x) ) . W_t^T )
 * with the same quantisers, weights, formats and conventions as the H-BitLinear
 * forward.  bits is 8 or 4; the workspace is sized with HBL_OP_FORWARD_INT8 or
 * HBL_OP_FORWARD_INT4.  K must still be a power of two in [64, 32768].
 */
hbl_status hbl_bitlinear_forward(const void *x, hbl_dtype x_dtype, const float *gain,
                                 const uint8_t *w_packed, const float *w_alpha,
                                 int64_t M, int64_t K, int64_t N, int bits,
                                 void *y, hbl_dtype y_dtype,
                                 void *workspace, size_t ws_bytes, hipStream_t stream);

/* Stage 1 of that forward: RMSNorm -> per-token quantisation, no rotation.
 * Arguments and formats as hbl_quantize_act (bits 8, 4 or 6). */
hbl_status hbl_quantize_act_unrotated(const void *x, hbl_dtype x_dtype, const float *gain,
                                      int64_t M, int64_t K, int bits,
                                      void *codes, float *dscale, hipStream_t stream);

/*
 * Offline ternarisation of weights rotated like the activations (the weight +
 * activation rotation of 新智元 article, section 实验效果, table 5): each row
 * w[n] (one output channel over the K inputs) becomes H_K w[n] / sqrt(K), the
 * same orthonormal Sylvester transform the activations get, so the layer's
 * inner products are unchanged before quantisation; the rotated rows are then
 * ternarised exactly as hbl_quantize_weights does (alpha = mean |rotated W|).
 * Use the result with hbl_forward_int8 / hbl_forward_int4.
 *   w         fp32 [N][K] latent weights (device, read only)
 *   w_packed, w_alpha  as hbl_quantize_weights
 *   workspace at least hbl_workspace_bytes(HBL_OP_QUANTIZE_WEIGHTS_ROTATED, 0, K, N)
 *             bytes (holds the rotated rows, fp32, and the row sums).
 * The rotation runs in fp32, so codes can differ from an exact rotation where
 * |rotated w| / alpha lies within rounding of 0.5.
 */
hbl_status hbl_quantize_weights_rotated(const float *w, int64_t N, int64_t K,
                                        uint8_t *w_packed, float *w_alpha,
                                        void *workspace, size_t ws_bytes, hipStream_t stream);

/* ---- the two stages of the forward, exported for stage-wise checking ---- */

/*
 * Stage 1: RMSNorm -> Hadamard rotation -> per-token quantisation, one fused
 * kernel (新智元 article, section H-BitLinear模块: the transform is applied to
 * the activations before they are quantised).
 *   bits      8, 4 or HBL_BITS_INT4_FP6 (6: INT4 codes in the fp6 operand layout,
 *             K >= 256)
 *   codes     INT8: int8 [M][K];  INT4: uint8 [M][K/2];  6: uint8 [K/128][M][96]
 *             (formats above)
 *   dscale    fp32 [M] per-token dequant scales d
 */
hbl_status hbl_quantize_act(const void *x, hbl_dtype x_dtype, const float *gain,
                            int64_t M, int64_t K, int bits,
                            void *codes, float *dscale, hipStream_t stream);

/*
 * Stage 1 from the rotated activations: the per-token quantiser alone, on
 * xt = H_K RMSNorm(x) / sqrt(K) held by the caller (as hbl_rmsnorm_fwht
 * writes it).  The same quantisers as hbl_quantize_act (QbitAI article on
 * BitNet v2, section 引入H-BitLinear模块, and 新智元 article, section
 * H-BitLinear模块: INT8 per-token absmax, INT4 per-token absmean), with no
 * normalisation or transform in front.
 *   xt        fp32 [M][K], device, 16-byte aligned
 *   bits      8, 4 or HBL_BITS_INT4_FP6 (6, K >= 256); codes and dscale as
 *             for hbl_quantize_act
 * The fused hbl_quantize_act scales the unnormalised transform once, so its
 * codes may differ from these by one at rounding ties of the quantiser.
 * Errors: HBL_ERR_DTYPE (bits), HBL_ERR_SHAPE (K, or K < 256 with bits 6),
 * HBL_ERR_NULL, HBL_ERR_ALIGN, HBL_ERR_DEVICE, HBL_ERR_LAUNCH; M = 0 is a no-op.
 */
hbl_status hbl_quantize_rotated(const float *xt, int64_t M, int64_t K, int bits,
                                void *codes, float *dscale, hipStream_t stream);

/*
 * Stage 2: ternary integer matmul of the codes with dequant epilogue.
 *   codes, dscale as written by hbl_quantize_act;  y [M][N] of y_dtype.
 *   bits      8 and 4 run on the int8 matrix instruction (any M); 6 runs on
 *             the fp6 x fp4 instruction (made for prefill token counts; any
 *             M works, K >= 256).
 *   workspace at least hbl_workspace_bytes(HBL_OP_MATMUL, M, K, N) bytes (split-K
 *             scratch of the small-M path; may be NULL when that size is 0).
 *   Calls sharing one workspace must be stream-ordered.
 */
hbl_status hbl_matmul_dequant(const void *codes, int bits, const float *dscale,
                              const uint8_t *w_packed, const float *w_alpha,
                              int64_t M, int64_t K, int64_t N,
                              void *y, hbl_dtype y_dtype,
                              void *workspace, size_t ws_bytes, hipStream_t stream);

/* ---- debug views used by the parity tests ---- */

/* The rotated, normalised activations xt = H_K RMSNorm(x) / sqrt(K) as fp32
 * [M][K], computed by the same code as stage 1 stopped before quantisation. */
hbl_status hbl_rmsnorm_fwht(const void *x, hbl_dtype x_dtype, const float *gain,
                            int64_t M, int64_t K, float *xt, hipStream_t stream);

/* The exact int32 accumulators acc[m][n] = sum_k q[m][k] W_t[n][k] [M][N],
 * computed by the same matmul kernels as stage 2 without the dequant epilogue.
 * Workspace as for hbl_matmul_dequant. */
hbl_status hbl_gemm_ternary(const void *codes, int bits, const uint8_t *w_packed,
                            int64_t M, int64_t K, int64_t N, int32_t *acc,
                            void *workspace, size_t ws_bytes, hipStream_t stream);

/* Expand packed ternary weights to int8 [N][K] in {-1, 0, 1}. */
hbl_status hbl_unpack_weights(const uint8_t *w_packed, int64_t N, int64_t K,
                              int8_t *w_t, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Backward pass (QbitAI article on BitNet v2, section 引入H-BitLinear模块,
 * training paragraph): the straight-through estimator bypasses both
 * quantisers, and the gradient goes through the transposed Hadamard
 * transform, i.e. the transform itself (H symmetric, orthonormal after the
 * 1/sqrt(K) scale).  With the forward y = xh . Wh^T, xh = q * d (the forward's
 * codes and per-token scales), Wh = W_t * a:
 *     dxh = dy . Wh;   du = H_K dxh / sqrt(K)  (du = dxh when rotate == 0);
 *     dx  = g du / r - x (sum_i du_i g_i x_i) / (K r^3),  r = sqrt(mean x^2 + 1e-6);
 *     dgain[k] = sum_m du[m][k] x[m][k] / r_m;     dw = dy^T . xh   (fp32 [N][K]).
 * The HIP path multiplies bf16 operands on the bf16 matrix instruction with
 * fp32 accumulation: dy and the ternary weights are exact in bf16, xh = q * d
 * is rounded to bf16 (relative 2^-9) for the weight gradient.
 */

/* The weights of the input-gradient product: W_t^T as bf16 [K][N] (values
 * -1, 0, +1; the scale alpha is applied inside hbl_backward).  Computed once
 * per weight update from the packed ternary weights.  N % 32 == 0. */
hbl_status hbl_backward_weights(const uint8_t *w_packed, int64_t N, int64_t K, void *w_bf16_t,
                                hipStream_t stream);

/* Backward of the layer.  x [M][K] (x_dtype) and gain [K] (or NULL) are the
 * forward's input; codes/d the forward's activation codes (bits 8: int8
 * [M][K]; bits 4: the INT4 format above) and per-token scales; w_bf16_t from
 * hbl_backward_weights and w_alpha as in the forward; dy bf16 [M][N].
 * Outputs dx [M][K] (dx_dtype), dw fp32 [N][K], dgain fp32 [K] (only with a
 * gain; NULL to skip).  rotate = 1 for H-BitLinear, 0 for BitLinear.
 * M >= 1, N % 32 == 0; workspace at least
 * hbl_workspace_bytes(HBL_OP_BACKWARD, M, K, N) bytes. */
hbl_status hbl_backward(const void *x, hbl_dtype x_dtype, const float *gain, const void *codes, int bits,
                        const float *d, const void *w_bf16_t, const float *w_alpha, const void *dy,
                        int64_t M, int64_t K, int64_t N, int rotate, void *dx, hbl_dtype dx_dtype,
                        float *dw, float *dgain, void *workspace, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* HBL_H */
