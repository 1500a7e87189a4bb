/*
 * bnn.h: C ABI of libbnn, the MI355X (gfx950) forward pass of binarized
 * linear and conv2d layers, the W8A8 int8 conv, and the straight-through
 * backward of the binarized linear layer.
 *
 * The layers are those of bitorch-engine's binary layer pages:
 *   - BinaryLinearForward.forward(input, weight, bmm_type, scale_a, scale_w, is_train)
 *     (BinaryLinearForward page): the binary product multiplied by both scalar
 *     scales; the operation has no bias;
 *   - BinaryConv2dForward.forward(x, weight, scale_a, scale_w, is_train,
 *     kernel_size, stride, padding, dilation) (qconv/binary/cutlass/layer
 *     page): the native forward receives the host product of the two scalar
 *     scales and returns the output in the input's dtype;
 *   - BinaryLinearCuda.w_pack / BinaryConv2dCutlass.generate_quantized_weight:
 *     weights are bit-packed once, ahead of the forward, by a packing kernel.
 *
 * Arithmetic (the method): every activation and weight element maps to +1
 * when it is >= 0 and to -1 otherwise (so -0 -> +1 and NaN -> -1); signs
 * are packed 32 per uint32 word along the reduction axis, bit j of word q
 * holding element 32q + j, bit value 1 for +1; the dot product of two
 * packed rows of K signs is K - 2 * popcount(a XOR w), exactly. Conv2d is
 * the im2col lowering of the banghao.live blog post, section 2 (output size
 * floor((H + 2p - d(k-1) - 1)/s + 1)), computed implicitly, with padded
 * taps contributing 0. The integer accumulator is scaled by
 * (float)(scale_a * scale_w) in fp32 and rounded to the output dtype
 * (round to nearest even).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, allocated and owned by the
 *     caller; the library never allocates, frees or keeps a pointer after
 *     returning. Tensors are dense (contiguous, row-major in the stated
 *     layout).
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is
 *     enqueued on it and the call returns without synchronizing.
 *   - Arguments are validated before anything is enqueued: on any error the
 *     call returns a non-zero status, enqueues nothing and leaves every
 *     output untouched. BNN_ERR_HIP reports a failed kernel launch.
 *   - Packed words travel in int32/uint32 buffers. A reduction length K (or
 *     channel count C) that is not a multiple of 32 fills ceil(K/32) words,
 *     the last one holding K % 32 signs in its low bits and 0 above them, in
 *     both operands; the contraction still runs over the true K (the pages'
 *     CUTLASS layer asserts whole binary words; this ABI also takes the
 *     rest).
 *   - The library holds no state except the per-thread record of the path
 *     that the last call took (bnn_last_path).
 */
#ifndef BNN_H
#define BNN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BNN_OK = 0,
  BNN_ERR_NULL = 1,      /* a required pointer is NULL */
  BNN_ERR_SHAPE = 2,     /* a size is negative/zero where it may not be, a bias of the wrong length, empty conv output */
  BNN_ERR_DTYPE = 3,     /* dtype code not allowed for that argument */
  BNN_ERR_ALIGN = 4,     /* a pointer is not aligned as the call requires (16 bytes for tensors read in vectors) */
  BNN_ERR_WORKSPACE = 5, /* workspace missing or smaller than the *_workspace_bytes query */
  BNN_ERR_PATH = 6,      /* unknown path code, or the forced path cannot run this shape */
  BNN_ERR_HIP = 7        /* the HIP runtime reported an error on launch */
} bnn_status;

typedef enum {
  BNN_F32 = 0,
  BNN_F16 = 1,
  BNN_BF16 = 2,
  BNN_I32 = 3,        /* output only: the raw integer accumulators, unscaled */
  BNN_U32_PACKED = 4, /* input only: activations already packed by bnn_pack_sign / bnn_pack_sign_nchw */
  BNN_U8_PACKED = 5   /* input only: activations packed in 8-bit containers, the container type of the
                         CUTLASS conv layer (bits_binary_word = 8; BinaryConv2dCutlass.__init__ and
                         _check_forward on the qconv/binary/cutlass/layer page): a row (linear) or a
                         pixel (conv) is ceil(n/8) bytes, bit j of byte q = sign 8q + j (1 for +1),
                         bits past n 0 or ignored; n = k or c. With n % 32 == 0 the bytes are read in
                         place as 32-bit words (4-byte alignment needed, no workspace); otherwise
                         they are repacked into the workspace first. */
} bnn_dtype;

/* Kernel choice; mirrors the layers' bmm_type argument (BMM.ADAPTIVE is the default there). */
typedef enum {
  BNN_PATH_AUTO = 0,     /* BNN_PATH_MFMA_FP4 when its sums are exact (K <= 2^24), else BNN_PATH_MFMA
                            (measured fastest at every tested shape, small layers included) */
  BNN_PATH_XOR = 1,      /* XOR + popcount on the vector ALUs */
  BNN_PATH_MFMA = 2,     /* signs expanded to int8 +-1, contracted on the matrix cores (int32 sums) */
  BNN_PATH_MFMA_FP4 = 3  /* signs expanded to fp4 (e2m1) +-1.0, contracted on the matrix cores
                            with fp32 sums, exact for a reduction length K <= 2^24 (K = k for
                            bnn_gemm, kernel_size^2 * c for bnn_conv2d; larger K: BNN_ERR_PATH) */
} bnn_path;

/* Sign + pack of activations along rows.
 *   x        [rows, k] in x_dtype (BNN_F32/F16/BF16), aligned to its element size (the fast
 *            path needs 16-byte alignment and k % 32 == 0).
 *   x_packed [rows, ceil(k/32)] uint32 out; bit j of word q = (x[r][32q+j] >= 0), 0 past k.
 * k >= 1; rows == 0 is a no-op. */
bnn_status bnn_pack_sign(const void* x, int x_dtype, int64_t rows, int64_t k,
                         uint32_t* x_packed, void* stream);

/* 8-bit containers -> 32-bit words (weights or activations packed for the CUTLASS layer, whose
 * container type is uint8_t: BinaryConv2dCutlass.__init__ on the qconv/binary/cutlass/layer page).
 *   src  [rows, ceil(bits/8)] bytes, bit j of byte q = sign 8q + j; any alignment.
 *   dst  [rows, ceil(bits/32)] uint32 out, 4-byte aligned; word q = bytes 4q..4q+3 little-endian
 *        (bytes past the row read as 0) with the bits at or past `bits` cleared, so the words carry
 *        the zero tail the contractions expect even when the containers' unused bits are not 0.
 * Conv weights [o, kh, kw, ceil(c/8)] are rows = o*kh*kw, bits = c; NHWC activations rows =
 * n*h*w, bits = c; linear rows have bits = k. bits >= 1; rows == 0 is a no-op. */
bnn_status bnn_u8_to_words(const uint8_t* src, int64_t rows, int64_t bits, uint32_t* dst,
                           void* stream);

/* Sign + pack of NCHW activations along channels.
 *   x        [n, c, h, w] in x_dtype (BNN_F32/F16/BF16), aligned to its element size (a 16-byte
 *            aligned tensor whose pixel planes are a multiple of the 16-byte vector width takes
 *            the vector kernel, any other the element-wise one, e.g. a slice of a batch).
 *   x_packed [n, h, w, ceil(c/32)] uint32 out; bit j of word q = (x[n][32q+j][h][w] >= 0), 0 past c.
 * c >= 1. */
bnn_status bnn_pack_sign_nchw(const void* x, int x_dtype, int64_t n, int64_t c, int64_t h,
                              int64_t w, uint32_t* x_packed, void* stream);

/* Activation prologue of the layers (set_activation of BinaryLinearCuda and BinaryConv2dCutlass):
 * the input is shifted by the learnable bias_a before its sign is taken, and while scale_a is
 * still zero it is initialised to 2 * mean|x| (symmetric quantization) or 4 * mean|x|.
 *
 * Shifted sign + pack along rows (linear layers):
 *   x        [rows, k] in x_dtype (BNN_F32/F16/BF16), aligned to its element size.
 *   bias     bias_len == 1: one shift for every element; bias_len == k: bias[col] per input
 *            feature (the linear page gives the bias no shape). bias_dtype BNN_F32/F16/BF16,
 *            aligned to its element size.
 *   x_packed [rows, ceil(k/32)] uint32 out; bit j of word q = (x[r][32q+j] + bias >= 0), the sign of the
 *            exact sum: -0 + -0 -> +1, a NaN operand or opposite infinities -> -1 (the sign of a
 *            sum never depends on the precision the layer adds in).
 * k >= 1; bits past k are 0; bias_len 1 or k (else BNN_ERR_SHAPE); rows == 0 is a no-op. */
bnn_status bnn_pack_sign_shift(const void* x, int x_dtype, int64_t rows, int64_t k,
                               const void* bias, int bias_dtype, int64_t bias_len,
                               uint32_t* x_packed, void* stream);

/* Shifted sign + pack of NCHW activations along channels (the conv layer: bias_a has one value
 * per input channel, broadcast over batch and pixels).
 *   bias     [c] in bias_dtype (BNN_F32/F16/BF16), aligned to its element size.
 *   x_packed [n, h, w, ceil(c/32)]; bit j of word q = (x[n][32q+j][h][w] + bias[32q+j] >= 0), as above.
 * Shapes and alignment as bnn_pack_sign_nchw. */
bnn_status bnn_pack_sign_nchw_shift(const void* x, int x_dtype, int64_t n, int64_t c, int64_t h,
                                    int64_t w, const void* bias, int bias_dtype,
                                    uint32_t* x_packed, void* stream);

/* Lazy activation scale: *scale_out (one double, device memory, 8-byte aligned) =
 * factor * (sum_i |x[i]|) / count over count >= 1 elements of x (BNN_F32/F16/BF16, 16-byte
 * aligned; the unshifted input, any layout). The pages use factor 2 (symmetric) or 4. Each
 * |x[i]| is exact in double and the sum is taken in double in a fixed order that depends only on
 * count, so the result is the same on every run (it differs from a sequential sum by at most
 * about count * 2^-53 relative). A NaN element gives NaN, an infinite one +inf. The layer rounds
 * the result to its dtype; that cast is the caller's.
 *   workspace at least bnn_abs_mean_workspace_bytes(count) bytes of device memory, 8-byte aligned
 *             (partial sums; contents on return are unspecified).
 * count <= 0 -> BNN_ERR_SHAPE. */
bnn_status bnn_abs_mean_scale(const void* x, int x_dtype, int64_t count, double factor,
                              double* scale_out, void* workspace, size_t workspace_bytes,
                              void* stream);
size_t bnn_abs_mean_workspace_bytes(int64_t count);

/* One-pass prologue (the layer's first forward, while scale_a is still zero): bnn_pack_sign_shift
 * and bnn_abs_mean_scale of the same x in a single read of x (set_activation of BinaryLinearCuda:
 * the shifted sign feeds the contraction, the lazy scale_a = factor * mean|x| is taken of the
 * unshifted input). x_packed exactly as bnn_pack_sign_shift; *scale_out as bnn_abs_mean_scale
 * (a sum in double in a fixed order that depends only on rows and k, within about rows * k * 2^-53
 * relative of the sequential sum, the same on every run; it may differ in the last bits from
 * bnn_abs_mean_scale's, whose order is another). x 16-byte aligned; rows >= 1, k >= 1 (the mean of
 * no elements is undefined: BNN_ERR_SHAPE); bias and its length as bnn_pack_sign_shift.
 *   workspace at least bnn_pack_sign_shift_abs_mean_workspace_bytes(rows, k) bytes, 8-byte aligned.
 * Rows that are a whole number of words take one kernel for both results; other row lengths
 * take the two passes. */
bnn_status bnn_pack_sign_shift_abs_mean(const void* x, int x_dtype, int64_t rows, int64_t k,
                                        const void* bias, int bias_dtype, int64_t bias_len,
                                        double factor, uint32_t* x_packed, double* scale_out,
                                        void* workspace, size_t workspace_bytes, void* stream);
size_t bnn_pack_sign_shift_abs_mean_workspace_bytes(int64_t rows, int64_t k);

/* The same for NCHW activations (set_activation of BinaryConv2dCutlass): x_packed exactly as
 * bnn_pack_sign_nchw_shift, *scale_out = factor * mean|x| over all n*c*h*w elements; n >= 1.
 * Pixel planes whose size is a multiple of the 16-byte vector width take one kernel for both
 * results, others the two passes.
 *   workspace at least bnn_pack_sign_nchw_shift_abs_mean_workspace_bytes(x_dtype, n, c, h, w)
 *             bytes, 8-byte aligned. */
bnn_status bnn_pack_sign_nchw_shift_abs_mean(const void* x, int x_dtype, int64_t n, int64_t c,
                                             int64_t h, int64_t w, const void* bias, int bias_dtype,
                                             double factor, uint32_t* x_packed, double* scale_out,
                                             void* workspace, size_t workspace_bytes, void* stream);
size_t bnn_pack_sign_nchw_shift_abs_mean_workspace_bytes(int x_dtype, int64_t n, int64_t c,
                                                         int64_t h, int64_t w);

/* Weight pack (run once per layer, ahead of the forward).
 *   kernel_size == 0: linear weight [out_features, in_features] -> [out_features, ceil(in_features/32)].
 *   kernel_size >= 1: conv weight OIHW [out_features, in_features, k, k] -> [out_features, k, k, ceil(in_features/32)].
 *   w_dtype BNN_F32/F16/BF16; in_features >= 1 (bits past it 0); weight aligned to its element size. */
bnn_status bnn_w_pack(const void* weight, int w_dtype, int64_t out_features, int64_t in_features,
                      int kernel_size, uint32_t* w_packed, void* stream);

/* Binary linear forward: out[m][n] = scale_a * scale_w * sum_k sgn(x[m][k]) * sgn(W[n][k]).
 *   x         [m, k] in BNN_F32/F16/BF16 (packed here into the workspace), or
 *             [m, ceil(k/32)] BNN_U32_PACKED (already packed, bits past k 0; no workspace needed),
 *             or [m, ceil(k/8)] bytes BNN_U8_PACKED (8-bit containers, see bnn_dtype).
 *   w_packed  [n, ceil(k/32)] from bnn_w_pack(kernel_size = 0).
 *   out       [m, n] in out_dtype: BNN_F32/F16/BF16 (scaled) or BNN_I32 (raw accumulators).
 *   path      a bnn_path value.
 *   workspace device scratch of at least bnn_gemm_workspace_bytes(m, k, x_dtype) bytes
 *             (may be NULL when that is 0).
 * m == 0 or n == 0 is a no-op; k >= 1. */
bnn_status bnn_gemm(const void* x, int x_dtype, const uint32_t* w_packed, int64_t m, int64_t n,
                    int64_t k, double scale_a, double scale_w, int path, void* out, int out_dtype,
                    void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): bnn_gemm without a workspace argument. Float
 * activations are packed into a static device array of BNN_NOALLOC_SCRATCH_BYTES bytes that
 * the library holds on every device it runs on until the process ends; the call itself
 * allocates and frees nothing. Arguments, layouts, results and errors as bnn_gemm, plus:
 *   - m * ceil(k/32) * 4 > BNN_NOALLOC_SCRATCH_BYTES when x needs packing (float x, or 8-bit
 *     containers with k % 32 != 0) -> BNN_ERR_WORKSPACE, nothing enqueued; x already in words
 *     (BNN_U32_PACKED, or BNN_U8_PACKED with k % 32 == 0) needs no scratch and has no limit;
 *   - the array belongs to the current device, which must be the device of `stream`; its
 *     address is looked up on the first call on each device (BNN_ERR_HIP if that fails);
 *   - every call on a device shares that device's array and it keeps the last call's
 *     contents: calls that overlap on one device (other streams, other host threads) race.
 *     Calls on one stream are ordered and safe. */
#define BNN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
bnn_status bnn_gemm_noalloc(const void* x, int x_dtype, const uint32_t* w_packed, int64_t m,
                            int64_t n, int64_t k, double scale_a, double scale_w, int path,
                            void* out, int out_dtype, void* stream);

/* Binary conv2d forward (square kernel, symmetric stride/padding/dilation).
 *   x         NCHW [n, c, h, w] in BNN_F32/F16/BF16 (aligned to its element size, packed here into
 *             the workspace as bnn_pack_sign_nchw does), or [n, h, w, ceil(c/32)] BNN_U32_PACKED,
 *             or [n, h, w, ceil(c/8)] bytes BNN_U8_PACKED (8-bit containers, see bnn_dtype).
 *   w_packed  [out_channels, k, k, ceil(c/32)] from bnn_w_pack(kernel_size = k).
 *   out       NCHW [n, out_channels, Ho, Wo] in out_dtype (BNN_F32/F16/BF16/I32),
 *             Ho = floor((h + 2*padding - dilation*(k-1) - 1)/stride + 1), likewise Wo.
 *   Padded taps contribute 0 (they are not counted in the reduction).
 *   workspace at least bnn_conv2d_workspace_bytes(n, c, h, w, x_dtype) bytes.
 * Requires c >= 1, kernel_size >= 1, stride >= 1, dilation >= 1, padding >= 0, Ho, Wo >= 1.
 * n == 0 or out_channels == 0 is a no-op. */
bnn_status bnn_conv2d(const void* x, int x_dtype, int64_t n, int64_t c, int64_t h, int64_t w,
                      const uint32_t* w_packed, int64_t out_channels, double scale_a,
                      double scale_w, int kernel_size, int stride, int padding, int dilation,
                      int path, void* out, int out_dtype, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Binary conv2d forward, general geometry: a kernel_h x kernel_w kernel with stride, padding and
 * dilation given per axis (rows, then columns); each output extent follows the formula above along
 * its axis, Ho from (h, kernel_h, stride_h, pad_h, dil_h) and Wo from the column values. The layer
 * page's single ints are the square case, which bnn_conv2d passes here unchanged. Arguments, layouts
 * and errors otherwise as bnn_conv2d, with w_packed [out_channels, kernel_h, kernel_w, ceil(c/32)]
 * from bnn_w_pack_conv. BNN_PATH_XOR needs kernel_h * kernel_w <= 49; BNN_PATH_MFMA_FP4 needs
 * kernel_h * kernel_w * c <= 2^24; AUTO picks by that K as for bnn_conv2d. */
bnn_status bnn_conv2d_ex(const void* x, int x_dtype, int64_t n, int64_t c, int64_t h, int64_t w,
                         const uint32_t* w_packed, int64_t out_channels, double scale_a,
                         double scale_w, int kernel_h, int kernel_w, int stride_h, int stride_w,
                         int pad_h, int pad_w, int dil_h, int dil_w, int path, void* out,
                         int out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Conv weight pack for any kernel shape: OIHW [out_features, in_features, kernel_h, kernel_w] ->
 * [out_features, kernel_h, kernel_w, ceil(in_features/32)] (bits past in_features 0); weight
 * aligned to its element size. bnn_w_pack with kernel_size >= 1 is the square case. */
bnn_status bnn_w_pack_conv(const void* weight, int w_dtype, int64_t out_features,
                           int64_t in_features, int kernel_h, int kernel_w, uint32_t* w_packed,
                           void* stream);

/* W8A8 conv: the im2col + GEMM lowering with INT8 quantizers of the banghao.live blog post,
 * section 3 ("Add INT8-quantizer to im2col+gemm"), computed implicitly on the matrix cores.
 * The page does not define its quantizers; here they are per-tensor symmetric 8-bit with a
 * given amax > 0: step = (float)amax / 127 in fp32, code = clamp(rint(v / step), -127, 127)
 * (correctly rounded fp32 division, round half to even), NaN codes as 0. The page's
 * fake-quantized product is then step_x * step_w * sum(q_x * q_w), computed here as int32
 * sums scaled once in fp32 by (float)(step_x * step_w) and rounded to out_dtype (BNN_I32:
 * the raw sums). Padded taps contribute 0. Channel counts must be multiples of 16;
 * kernel_h * kernel_w * c <= 133144 (so |sum| < 2^31).
 *
 * Activation codes: x NCHW [n, c, h, w] (BNN_F32/F16/BF16) -> x_q NHWC int8 [n, h, w, c],
 * 16-byte aligned. */
bnn_status bnn_quant_i8_nhwc(const void* x, int x_dtype, int64_t n, int64_t c, int64_t h, int64_t w,
                             double amax, int8_t* x_q, void* stream);
/* Weight codes (once per layer): OIHW [out_channels, c, kernel_h, kernel_w] ->
 * w_q int8 [out_channels, kernel_h, kernel_w, c], 16-byte aligned. */
bnn_status bnn_quant_i8_weight(const void* weight, int w_dtype, int64_t out_channels, int64_t c,
                               int kernel_h, int kernel_w, double amax, int8_t* w_q, void* stream);
/* out NCHW [n, out_channels, Ho, Wo] = step_x * step_w * conv(x_q, w_q), geometry as
 * bnn_conv2d_ex; amax_x / amax_w are the amax values the codes were made with. */
bnn_status bnn_w8a8_conv2d(const int8_t* x_q, int64_t n, int64_t c, int64_t h, int64_t w,
                           const int8_t* w_q, int64_t out_channels, double amax_x, double amax_w,
                           int kernel_h, int kernel_w, int stride_h, int stride_w, int pad_h,
                           int pad_w, int dil_h, int dil_w, void* out, int out_dtype,
                           void* stream);

/* ---- Straight-through backward of the binarized linear layer ----
 * BinaryConv2dForward.backward on the qconv/binary/cutlass/layer page gives the steps for the
 * conv; the BinaryLinearForward page describes the linear layer's backward in the same terms
 * (signs and scales, clipped grad_input, grad_scale_a, no gradient for scale_w). These calls are
 * those steps with a 1x1 kernel:
 *   grad_in[m][k]  = (scale_w * sum_n g[m][n] * sign(W[n][k])) * mid(x[m][k])
 *   mid(v)         = 0 if the fp32 quotient v / scale_a is < -1 or > 1, else 1 (NaN -> 1)
 *   grad_scale_a   = sum over m, k of grad_in * sign(x), divided by sqrt(m * k)
 *   grad_w[n][k]   = scale_a * sum_m g[m][n] * sign(x[m][k])
 * with sign = torch.sign (0 for +-0, NaN for NaN), unlike the forward's x >= 0 rule.
 * g [m][n] (output gradient), W [n][k] (the float weight the layer keeps) and x [m][k] (the
 * layer's input) share one dtype, BNN_F16 or BNN_BF16; products are exact and sums fp32 (the
 * scale is applied once to the fp32 sum); grad_in and grad_w are fp32, grad_scale_a double
 * (summed in double). n and k must be multiples of 8; g, W and x 16-byte aligned. The int8
 * quantization of grad_w on the page is bnn_linear_grad_weight_i8 below.
 *
 * grad_input: m, k > 0 (the page divides by sqrt(m * k)); grad_in [m][k] and grad_scale_a
 * (one double) are device outputs; workspace: at least
 * bnn_linear_grad_input_workspace_bytes(m, k) bytes of device memory, 8-byte aligned, whose
 * contents are overwritten. */
size_t bnn_linear_grad_input_workspace_bytes(int64_t m, int64_t k);
bnn_status bnn_linear_grad_input(const void* grad_out, const void* weight, const void* x,
                                 int dtype, int64_t m, int64_t n, int64_t k, float scale_a,
                                 float scale_w, float* grad_in, double* grad_scale_a,
                                 void* workspace, size_t workspace_bytes, void* stream);
/* grad_weight: grad_w [n][k] fp32 device output; m = 0 writes zeros; n = 0 or k = 0 does
 * nothing. */
bnn_status bnn_linear_grad_weight(const void* grad_out, const void* x, int dtype, int64_t m,
                                  int64_t n, int64_t k, float scale_a, float* grad_w,
                                  void* stream);

/* grad_weight with the page's int8 step (grad_weight = nv_tensor_quant(grad_weight)[0] at the end of
 * BinaryConv2dForward.backward on the qconv/binary/cutlass/layer page). The quantizer is not on the
 * pages; it is the per-tensor symmetric one of the W8A8 calls with amax taken from the gradient:
 * amax = max |grad_w| over the fp32 gradient (NaN if any element is NaN), step = amax / 127 in fp32,
 * code = clamp(rint(grad_w / step), -127, 127) with ties to even, and a NaN quotient (every gradient
 * 0, a NaN amax, inf / inf) codes as 0. Outputs (device): grad_w [n][k] fp32 as bnn_linear_grad_weight
 * (16-byte aligned), grad_w_q [n][k] int8 (4-byte aligned), amax (one float; dequantized gradient =
 * code * amax / 127). workspace: at least bnn_linear_grad_weight_i8_workspace_bytes(n, k) bytes,
 * 4-byte aligned, overwritten. Shapes and dtypes as bnn_linear_grad_weight. */
size_t bnn_linear_grad_weight_i8_workspace_bytes(int64_t n, int64_t k);
bnn_status bnn_linear_grad_weight_i8(const void* grad_out, const void* x, int dtype, int64_t m,
                                     int64_t n, int64_t k, float scale_a, float* grad_w,
                                     int8_t* grad_w_q, float* amax, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* The int8 coder of bnn_linear_grad_weight_i8 on its own, for a gradient that was reduced
 * elsewhere first (e.g. summed over data-parallel ranks, whose amax is that of the sum): grad is
 * count fp32 values (count a multiple of 4, 16-byte aligned), codes count int8 (4-byte aligned),
 * amax one float, all device memory; workspace at least bnn_quant_grad_i8_workspace_bytes(count)
 * bytes, 4-byte aligned, overwritten. Same quantizer as bnn_linear_grad_weight_i8. */
size_t bnn_quant_grad_i8_workspace_bytes(int64_t count);
bnn_status bnn_quant_grad_i8(const float* grad, int64_t count, int8_t* codes, float* amax,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Workspace sizes (bytes) for the calls above; 0 when x is already packed. */
size_t bnn_gemm_workspace_bytes(int64_t m, int64_t k, int x_dtype);
size_t bnn_conv2d_workspace_bytes(int64_t n, int64_t c, int64_t h, int64_t w, int x_dtype);

/* Straight-through backward of the binarized conv (BinaryConv2dForward.backward on the
 * qconv/binary/cutlass/layer page): the page's conv2d_input with sign(W) * scale_w, the clip mask
 * of x / scale_a, grad_scale_a, and conv2d_weight with sign(x) * scale_a, whose int8 codes the
 * page takes last. sign is torch.sign (0 for +-0, NaN for NaN).
 *   grad_out [n, out_channels, Ho, Wo], weight [out_channels, c, kernel_h, kernel_w] (the float
 *   weight) and x [n, c, h, w] (the layer input) share one 16-bit dtype (BNN_F16 or BNN_BF16);
 *   Ho, Wo by the forward's formula from the per-axis stride / padding / dilation.
 *   n*Ho*Wo and c*kernel_h*kernel_w must be multiples of 8, every other size >= 1 (else
 *   BNN_ERR_SHAPE). weight 16-byte aligned, grad_out and x 2-byte aligned.
 *
 * grad_input: grad_in [n, c, h, w] fp32 = mid(x) * sum over (o, kh, kw) of grad_out at the output
 * pixel whose tap (kh, kw) reads that input element, times sign(W[o][c][kh][kw]) * scale_w; mid is
 * 0 where the fp32 quotient x / scale_a is below -1 or above 1, else 1. grad_scale_a (one double) =
 * sum(grad_in * sign(x)) / sqrt(n*c*h*w), summed in a fixed order (deterministic).
 *   workspace: bnn_conv2d_grad_input_workspace_bytes(...) bytes, 256-byte aligned. */
size_t bnn_conv2d_grad_input_workspace_bytes(int64_t n, int64_t c, int64_t h, int64_t w,
                                             int64_t out_channels, int kernel_h, int kernel_w,
                                             int stride_h, int stride_w, int pad_h, int pad_w,
                                             int dil_h, int dil_w);
bnn_status bnn_conv2d_grad_input(const void* grad_out, const void* weight, const void* x,
                                 int dtype, int64_t n, int64_t c, int64_t h, int64_t w,
                                 int64_t out_channels, int kernel_h, int kernel_w, int stride_h,
                                 int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                                 float scale_a, float scale_w, float* grad_in,
                                 double* grad_scale_a, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* grad_weight: grad_w [out_channels, c, kernel_h, kernel_w] fp32 (16-byte aligned) = scale_a *
 * sum over (b, oh, ow) of grad_out[b][o][oh][ow] * sign(x at tap (kh, kw) of that output pixel),
 * padded taps contributing 0. With grad_w_q and amax given (both or neither), also the int8 codes
 * the page takes (per-tensor symmetric: amax = max|grad_w|, code = clamp(rint(v / (amax / 127)),
 * +-127), a NaN quotient coding as 0), as bnn_quant_grad_i8 computes them.
 *   workspace: bnn_conv2d_grad_weight_workspace_bytes(...) bytes, 256-byte aligned. */
size_t bnn_conv2d_grad_weight_workspace_bytes(int64_t n, int64_t c, int64_t h, int64_t w,
                                              int64_t out_channels, int kernel_h, int kernel_w,
                                              int stride_h, int stride_w, int pad_h, int pad_w,
                                              int dil_h, int dil_w);
bnn_status bnn_conv2d_grad_weight(const void* grad_out, const void* x, int dtype, int64_t n,
                                  int64_t c, int64_t h, int64_t w, int64_t out_channels,
                                  int kernel_h, int kernel_w, int stride_h, int stride_w,
                                  int pad_h, int pad_w, int dil_h, int dil_w, float scale_a,
                                  float* grad_w, int8_t* grad_w_q, float* amax, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* The path that bnn_gemm / bnn_conv2d would take for a shape under BNN_PATH_AUTO (it depends only on
 * the reduction length K = k, or kernel_size^2 * c). */
int bnn_gemm_auto_path(int64_t m, int64_t n, int64_t k);
int bnn_conv2d_auto_path(int64_t n, int64_t c, int64_t h, int64_t w, int64_t out_channels,
                         int kernel_size, int stride, int padding, int dilation);

/* Path (BNN_PATH_XOR, BNN_PATH_MFMA or BNN_PATH_MFMA_FP4) taken by this thread's last successful
 * bnn_gemm / bnn_conv2d call; 0 before any such call. */
int bnn_last_path(void);

/* Static, human-readable text for a status code. */
const char* bnn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* BNN_H */
