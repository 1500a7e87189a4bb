// Host-side launchers of the libbnn kernels. Each returns the hipError_t of
// the launch; arguments are assumed validated by the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bnn_device.h"

namespace bnn {

// Row sign+pack: x [rows][k] -> words [rows][k/32], treated as one flat stream of words.
hipError_t launch_pack_rows(const void* x, int dtype, int64_t total_words, uint32_t* out,
                            hipStream_t stream);

// NCHW sign+pack: x [b][c][h][w] -> words [b][h][w][ceil(c/32)] (channel bits at or past c
// are 0). With a bias (element type
// bdtype), channel c is shifted by bias[c] before its sign is taken.
hipError_t launch_pack_nchw(const void* x, int dtype, int64_t b, int64_t c, int64_t h, int64_t w,
                            uint32_t* out, hipStream_t stream, const void* bias = nullptr,
                            int bdtype = -1);

// Shifted row sign+pack: bit = (x[r][col] + bias >= 0), bias[col] when percol, else bias[0].
// KW = k / 32 words per row.
hipError_t launch_pack_rows_shift(const void* x, int dtype, int64_t rows, int64_t KW,
                                  const void* bias, int bdtype, bool percol, uint32_t* out,
                                  hipStream_t stream);

// Row sign+pack (plain when bias is null, else shifted as above) for any row length k:
// words [rows][ceil(k/32)], bits at or past k are 0. Elements need only their natural alignment.
hipError_t launch_pack_rows_ragged(const void* x, int dtype, int64_t rows, int64_t k,
                                   const void* bias, int bdtype, bool percol, uint32_t* out,
                                   hipStream_t stream);

// factor * mean|x| over count elements into out[0] (double), through abs_mean_parts(count)
// double partial sums.
int abs_mean_parts(int64_t count);
hipError_t launch_abs_mean(const void* x, int dtype, int64_t count, double factor, double* partial,
                           double* out, hipStream_t stream);

// One-pass prologue: the shifted row pack (k = 32 * KW, 16-byte aligned x) that also leaves
// factor * mean|x| in scale_out[0], through pack_rows_shift_abs_parts(rows, KW) partial sums.
int64_t pack_rows_shift_abs_parts(int64_t rows, int64_t KW);
hipError_t launch_pack_rows_shift_abs(const void* x, int dtype, int64_t rows, int64_t KW,
                                      const void* bias, int bdtype, bool percol, uint32_t* out,
                                      double factor, double* partial, double* scale_out,
                                      hipStream_t stream);
// The same for the shifted NCHW pack, when pack_nchw_abs_fused (pixel planes a multiple of the
// 16-byte vector width, x 16-byte aligned); pack_nchw_abs_parts partial sums.
bool pack_nchw_abs_fused(int dtype, int64_t h, int64_t w, const void* x);
int64_t pack_nchw_abs_parts(int dtype, int64_t b, int64_t c, int64_t h, int64_t w);
hipError_t launch_pack_nchw_shift_abs(const void* x, int dtype, int64_t b, int64_t c, int64_t h,
                                      int64_t w, uint32_t* out, const void* bias, int bdtype,
                                      double factor, double* partial, double* scale_out,
                                      hipStream_t stream);

// OIHW conv weight pack: [o][c][kh][kw] -> [o][kh][kw][ceil(c/32)].
hipError_t launch_pack_conv_weight(const void* w, int dtype, int64_t o, int64_t c, int kh, int kw,
                                   uint32_t* out, hipStream_t stream);

// 8-bit sign containers [rows][ceil(bits/8)] bytes -> words [rows][ceil(bits/32)] (little-endian
// byte order, bits at or past `bits` cleared).
hipError_t launch_u8_to_words(const uint8_t* src, int64_t rows, int64_t bits, uint32_t* dst,
                              hipStream_t stream);

// XOR + popcount contraction on the vector ALUs.
hipError_t launch_xor(const Contraction& p, bool conv, int out_dtype, hipStream_t stream);

// int8 +-1 contraction on the matrix cores.
hipError_t launch_mfma(const Contraction& p, bool conv, int out_dtype, hipStream_t stream);

// fp4 (e2m1) +-1 contraction on the matrix cores; exact for a reduction length K <= 2^24
// (kMaxFp4K), checked by the caller.
constexpr int64_t kMaxFp4K = int64_t(1) << 24;
hipError_t launch_mfma_fp4(const Contraction& p, bool conv, int out_dtype, hipStream_t stream);

// W8A8 conv (int8 codes of per-tensor symmetric quantizers, int32 sums on the matrix cores).
// NCHW float -> NHWC int8 codes with step amax/127 (c % 16 == 0, 16-byte aligned out).
hipError_t launch_quant_nhwc(const void* x, int dtype, int64_t n, int64_t c, int64_t h, int64_t w,
                             float step, int8_t* out, hipStream_t stream);
// OIHW float -> [o][kh][kw][c] int8 codes.
hipError_t launch_quant_weight(const void* w, int dtype, int64_t o, int64_t c, int kh, int kw,
                               float step, int8_t* out, hipStream_t stream);
// Implicit-im2col int8 conv, out = alpha * sum q_x q_w (NCHW, out_dtype); c % 16 == 0.
hipError_t launch_w8a8_conv(const int8_t* xq, const int8_t* wq, void* out, int out_dtype,
                            int64_t n, int64_t c, int64_t h, int64_t w, int64_t o, int64_t ho,
                            int64_t wo, int kh, int kw, int sh, int sw, int ph, int pw, int dh,
                            int dw, float alpha, hipStream_t stream);

// Straight-through linear backward (bf = bfloat16 operands, else float16).
// grad_in [m][k] fp32, grad_scale_a one double, through bwd_grad_input_parts(m, k) doubles of part.
int64_t bwd_grad_input_parts(int64_t m, int64_t k);
hipError_t launch_linear_grad_input(const void* g, const void* w, const void* x, bool bf,
                                    int64_t m, int64_t n, int64_t k, float scale_a, float scale_w,
                                    float* grad_in, double* part, double* grad_scale_a,
                                    hipStream_t s);
// int8 codes of an fp32 gradient (count a multiple of 4, 16-byte aligned), amax to one device
// float, through bwd_grad_weight_i8_parts(n, k) floats of part.
int64_t bwd_grad_weight_i8_parts(int64_t n, int64_t k);
int64_t bwd_quant_grad_parts(int64_t count);
hipError_t launch_quant_grad(const float* grad_w, int64_t count, float* part, float* amax,
                             int8_t* codes, hipStream_t s);
// grad_w [n][k] fp32.
hipError_t launch_linear_grad_weight(const void* g, const void* x, bool bf, int64_t m, int64_t n,
                                     int64_t k, float scale_a, float* grad_w, hipStream_t s);

// Straight-through conv backward. geom = {B, C, H, W, O, KH, KW, SH, SW, PH, PW, DH, DW, Ho, Wo};
// g [B][O][Ho][Wo], W [O][C][KH][KW] and x [B][C][H][W] of one 16-bit dtype; B*Ho*Wo and C*KH*KW
// multiples of 8. grad_input scratch: gT [O][B*Ho*Wo] u16, wsign [O][C*KH*KW] u16, cols
// [C*KH*KW][B*Ho*Wo] fp32, conv_col2im_parts(B, C, H, W) doubles of part. grad_weight scratch: gT,
// xcol [B*Ho*Wo][C*KH*KW] u16 and, with conv_wgrad_splits(O, C*KH*KW, B*Ho*Wo) > 1, that many
// partial [O][C*KH*KW] fp32 results.
int64_t conv_col2im_parts(int64_t n, int64_t c, int64_t h, int64_t w);
int conv_wgrad_splits(int64_t o, int64_t j, int64_t pixels);
hipError_t launch_conv_grad_input(const void* g, const void* w, const void* x, bool bf,
                                  const int geom[15], float scale_a, float scale_w, float* grad_in,
                                  uint16_t* gT, uint16_t* wsign, float* cols, double* part,
                                  double* grad_scale_a, hipStream_t s);
hipError_t launch_conv_grad_weight(const void* g, const void* x, bool bf, const int geom[15],
                                   float scale_a, float* grad_w, uint16_t* gT, uint16_t* xcol,
                                   float* split_part, hipStream_t s);

}  // namespace bnn
