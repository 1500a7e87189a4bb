/*
 * CPU oracle for the binarized linear and conv2d forward pass.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it. It shares no code, header, table or constant with
 * the HIP library; it is plain, slow and meant to be checked by eye.
 *
 * What it computes, and where that is defined:
 *
 *  - The sign rule: a value maps to +1 when it is >= 0 and to -1 otherwise.
 *    The value is first widened exactly to float (fp16 and bf16 widen
 *    exactly), then compared with an IEEE compare, so -0 maps to +1, NaN to
 *    -1 (the compare is false), +-inf to +-1 and subnormals by their sign.
 *    (Rule taken from the method's statement that x >= 0 maps to +1; the
 *    bitorch-engine layer pages leave the sign step to their native kernel.)
 *
 *  - Bit packing: 32 sign bits per 32-bit word along the reduction axis,
 *    bit j of word q holding element 32q + j, bit value 1 for +1 and 0 for
 *    -1. (The layers pack weights once, ahead of the forward, with a native
 *    bit-packing kernel: BinaryConv2dCutlass.generate_quantized_weight on
 *    the qconv/binary/cutlass/layer page, BinaryLinearCuda.w_pack on the
 *    BinaryLinearCuda page. The word width 32 and the bit order are a
 *    reading taken here; the pages fix neither.) A reduction length that is
 *    not a whole number of words (the CUTLASS layer asserts that it is)
 *    leaves the missing bits of the last word 0: in both operands, so a
 *    XOR of the two sets no bit there, and the contraction itself still
 *    runs over the true length.
 *
 *  - Linear forward: acc[m][n] = sum_k sgn(x[m][k]) * sgn(W[n][k]), then
 *    y = acc * (scale_a * scale_w): the binary product multiplied by both
 *    scalar scales, with no bias (BinaryLinearForward.forward and .backward on
 *    the BinaryLinearForward page).
 *
 *  - Conv2d forward, lowered as im2col + GEMM exactly in the order of the
 *    banghao.live blog post, section 2 ("Implementation of im2col+gemm
 *    operation", MyConv2d.forward): output size
 *    Ho = floor((H + 2p - d(k-1) - 1)/s + 1), unfold into rows
 *    r = c*k*k + kh*k + kw and columns l = oh*Wo + ow, transpose to [L, R],
 *    multiply by the weight viewed as [O, C*k*k], reshape to [O, Ho, Wo].
 *    Signs are taken BEFORE the zero padding, so a padded tap contributes 0.
 *    The blog's unfold call omits the dilation although its output-size
 *    formula uses it; the unfold here applies the dilation (the conv forward
 *    on the qconv/binary/cutlass/layer page takes a dilation argument).
 *    The general form takes a KH x KW kernel and a stride, padding and
 *    dilation per axis (rows, columns), each output extent by the same
 *    formula along its axis; the layer's single ints are the square case.
 *    The scale product is the host-side product of the two scalar scales
 *    (BinaryConv2dForward.forward on the qconv/binary/cutlass/layer page).
 *
 *  - The activation prologue of both layers (set_activation of
 *    BinaryConv2dCutlass on the qconv/binary/cutlass/layer page and of
 *    BinaryLinearCuda on the BinaryLinearCuda page). The input is shifted by
 *    the learnable bias_a before its sign is taken: one value per input
 *    channel for the conv, broadcast over batch and pixels; the linear page
 *    calls its bias layer-wise without giving a shape, so the linear form
 *    takes either one value for the whole layer or one per input feature.
 *    The bit is the sign of x + b. The exact sum of two floats keeps its
 *    sign, and its zero-ness, when rounded to any IEEE format (a non-zero
 *    sum is a multiple of the smallest subnormal, so it never rounds to 0;
 *    overflow gives an infinity of the same sign), so the sign does not
 *    depend on the dtype the layer adds in; NaN operands and opposite
 *    infinities give NaN, hence -1. Here the sum is taken in double from
 *    the exactly widened operands.
 *    While scale_a is still zero the layer sets it to 2 * mean|x|
 *    (symmetric quantization) or 4 * mean|x|, over every element of the
 *    unshifted input: here the double sum of |x| in index order, divided by
 *    the element count, times the factor.
 *
 * Every accumulation is a sum of +-1 products; each partial sum is an
 * integer of magnitude at most K < 2^24, so float accumulation is exact in
 * any order (that is why the reductions may be vectorised).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

/* Element types of the oracle's inputs (its own numbering). */
#define ORACLE_F32 0
#define ORACLE_F16 1
#define ORACLE_BF16 2

/* IEEE 754 binary16 -> binary32, exact, written from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static float widen_f16(uint16_t h) {
  int sign = h >> 15;
  int e = (h >> 10) & 0x1f;
  int frac = h & 0x3ff;
  float v;
  if (e == 0)
    v = ldexpf((float)frac, -24);                 /* zero and subnormals: frac * 2^-24 */
  else if (e == 31)
    v = frac ? NAN : INFINITY;
  else
    v = ldexpf((float)(frac + 1024), e - 25);     /* (1 + frac/1024) * 2^(e-15) */
  return sign ? -v : v;
}

/* bfloat16 is the upper half of a binary32: widening appends 16 zero bits. */
static float widen_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

static float widen(const void *x, int dtype, int64_t i) {
  if (dtype == ORACLE_F32) return ((const float *)x)[i];
  if (dtype == ORACLE_F16) return widen_f16(((const uint16_t *)x)[i]);
  return widen_bf16(((const uint16_t *)x)[i]);
}

/* The sign rule: +1 for v >= 0, else -1. */
static float sgn(float v) { return v >= 0.0f ? 1.0f : -1.0f; }

int oracle_num_threads(void) { return omp_get_max_threads(); }

/* s[i] = sgn(widen(x[i])) for i < count. */
void oracle_sign(const void *x, int dtype, int64_t count, float *s) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; i++) s[i] = sgn(widen(x, dtype, i));
}

/* Row-major x[rows][k] -> words out[rows][ceil(k/32)]; bit j of word q is 1 iff 32q+j < k and
 * x[r][32q+j] >= 0 (a row that does not fill its last word leaves the missing bits 0). */
void oracle_pack_rows(const void *x, int dtype, int64_t rows, int64_t k, uint32_t *out) {
  int64_t kw = (k + 31) / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++)
    for (int64_t q = 0; q < kw; q++) {
      uint32_t word = 0;
      for (int j = 0; j < 32 && 32 * q + j < k; j++)
        if (sgn(widen(x, dtype, r * k + 32 * q + j)) > 0.0f) word |= (uint32_t)1 << j;
      out[r * kw + q] = word;
    }
}

/* NCHW x[b][c][h][w] -> words out[b][h][w][ceil(C/32)]; bit j of word q is 1 iff 32q+j < C and
 * x[b][32q+j][h][w] >= 0. */
void oracle_pack_nchw(const void *x, int dtype, int64_t B, int64_t C, int64_t H, int64_t W,
                      uint32_t *out) {
  int64_t cw = (C + 31) / 32;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < B; b++)
    for (int64_t ih = 0; ih < H; ih++)
      for (int64_t iw = 0; iw < W; iw++)
        for (int64_t q = 0; q < cw; q++) {
          uint32_t word = 0;
          for (int j = 0; j < 32 && 32 * q + j < C; j++) {
            int64_t idx = ((b * C + 32 * q + j) * H + ih) * W + iw;
            if (sgn(widen(x, dtype, idx)) > 0.0f) word |= (uint32_t)1 << j;
          }
          out[((b * H + ih) * W + iw) * cw + q] = word;
        }
}

/* OIHW weight w[o][c][i][j] of a KH x KW kernel -> words out[o][i][j][ceil(C/32)]; bit jj of word
 * q is 1 iff 32q+jj < C and w[o][32q+jj][i][j] >= 0. */
void oracle_pack_conv_weight2(const void *w, int dtype, int64_t O, int64_t C, int64_t KH,
                              int64_t KW, uint32_t *out) {
  int64_t cw = (C + 31) / 32;
#pragma omp parallel for schedule(static)
  for (int64_t o = 0; o < O; o++)
    for (int64_t i = 0; i < KH; i++)
      for (int64_t j = 0; j < KW; j++)
        for (int64_t q = 0; q < cw; q++) {
          uint32_t word = 0;
          for (int jj = 0; jj < 32 && 32 * q + jj < C; jj++) {
            int64_t idx = ((o * C + 32 * q + jj) * KH + i) * KW + j;
            if (sgn(widen(w, dtype, idx)) > 0.0f) word |= (uint32_t)1 << jj;
          }
          out[((o * KH + i) * KW + j) * cw + q] = word;
        }
}

/* Square kernels: oracle_pack_conv_weight2 with KH = KW = ks. */
void oracle_pack_conv_weight(const void *w, int dtype, int64_t O, int64_t C, int64_t ks,
                             uint32_t *out) {
  oracle_pack_conv_weight2(w, dtype, O, C, ks, ks, out);
}

/* 8-bit containers. The CUTLASS conv layer keeps its packed signs in uint8_t containers
 * (bits_binary_word = 8, BinaryConv2dCutlass.__init__ and _check_forward on the
 * qconv/binary/cutlass/layer page); the page does not print the bit order. Reading taken here:
 * the same order as the 32-bit words, bit j of byte b holding element 8b + j, so the four bytes
 * of a little-endian 32-bit word are four containers in row order. A row that does not fill its
 * last byte leaves the missing bits 0.
 *
 * Row-major x[rows][k] -> bytes out[rows][ceil(k/8)]. */
void oracle_pack_rows_u8(const void *x, int dtype, int64_t rows, int64_t k, uint8_t *out) {
  int64_t kb = (k + 7) / 8;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++)
    for (int64_t q = 0; q < kb; q++) {
      unsigned byte = 0;
      for (int j = 0; j < 8 && 8 * q + j < k; j++)
        if (sgn(widen(x, dtype, r * k + 8 * q + j)) > 0.0f) byte |= 1u << j;
      out[r * kb + q] = (uint8_t)byte;
    }
}

/* NCHW x[b][c][h][w] -> bytes out[b][h][w][ceil(C/8)]; bit j of byte q is 1 iff 8q+j < C and
 * x[b][8q+j][h][w] >= 0. */
void oracle_pack_nchw_u8(const void *x, int dtype, int64_t B, int64_t C, int64_t H, int64_t W,
                         uint8_t *out) {
  int64_t cb = (C + 7) / 8;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < B; b++)
    for (int64_t ih = 0; ih < H; ih++)
      for (int64_t iw = 0; iw < W; iw++)
        for (int64_t q = 0; q < cb; q++) {
          unsigned byte = 0;
          for (int j = 0; j < 8 && 8 * q + j < C; j++) {
            int64_t idx = ((b * C + 8 * q + j) * H + ih) * W + iw;
            if (sgn(widen(x, dtype, idx)) > 0.0f) byte |= 1u << j;
          }
          out[((b * H + ih) * W + iw) * cb + q] = (uint8_t)byte;
        }
}

/* OIHW weight w[o][c][i][j] of a KH x KW kernel -> bytes out[o][i][j][ceil(C/8)]; bit jj of byte
 * q is 1 iff 8q+jj < C and w[o][8q+jj][i][j] >= 0. */
void oracle_pack_conv_weight_u8(const void *w, int dtype, int64_t O, int64_t C, int64_t KH,
                                int64_t KW, uint8_t *out) {
  int64_t cb = (C + 7) / 8;
#pragma omp parallel for schedule(static)
  for (int64_t o = 0; o < O; o++)
    for (int64_t i = 0; i < KH; i++)
      for (int64_t j = 0; j < KW; j++)
        for (int64_t q = 0; q < cb; q++) {
          unsigned byte = 0;
          for (int jj = 0; jj < 8 && 8 * q + jj < C; jj++) {
            int64_t idx = ((o * C + 8 * q + jj) * KH + i) * KW + j;
            if (sgn(widen(w, dtype, idx)) > 0.0f) byte |= 1u << jj;
          }
          out[((o * KH + i) * KW + j) * cb + q] = (uint8_t)byte;
        }
}

/* Linear accumulators. acc[i][n] = sum_k sgn(x[m_i][k]) * sgn(W[n][k]) for the selected rows
 * m_i = rows[i] (all M rows in order when rows == NULL, nrows then ignored). Returns 0, or -1
 * when K is too long for the exact float accumulation or memory runs out. */
int oracle_linear_acc(const void *x, int xdt, const void *w, int wdt, int64_t M, int64_t N,
                      int64_t K, const int64_t *rows, int64_t nrows, int32_t *acc) {
  if (K >= (1 << 24)) return -1;
  if (!rows) nrows = M;
  float *sw = (float *)malloc(sizeof(float) * (size_t)(N * K));
  if (!sw) return -1;
  oracle_sign(w, wdt, N * K, sw);
  int fail = 0;
#pragma omp parallel
  {
    float *sx = (float *)malloc(sizeof(float) * (size_t)K);
    if (!sx) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; i++) {
      if (!sx) continue;
      int64_t m = rows ? rows[i] : i;
      for (int64_t k = 0; k < K; k++) sx[k] = sgn(widen(x, xdt, m * K + k));
      for (int64_t n = 0; n < N; n++) {
        const float *wr = sw + n * K;
        float s = 0.0f;
#pragma omp simd reduction(+ : s)
        for (int64_t k = 0; k < K; k++) s += sx[k] * wr[k];
        acc[i * N + n] = (int32_t)s;
      }
    }
    free(sx);
  }
  free(sw);
  return fail ? -1 : 0;
}

/* Output extent: floor((size + 2p - d(ks-1) - 1)/s + 1), with a true floor for negative numerators. */
int64_t oracle_conv_out_size(int64_t size, int64_t ks, int64_t s, int64_t p, int64_t d) {
  int64_t num = size + 2 * p - d * (ks - 1) - 1;
  int64_t q = num / s;
  if (num % s != 0 && num < 0) q -= 1;
  return q + 1;
}

/* Conv accumulators via zero-padded unfold + GEMM, for the selected images b_i = imgs[i]
 * (all B in order when imgs == NULL). acc[i][o][oh][ow]. A KH x KW kernel with stride
 * (sh, sw), zero padding (ph, pw) and dilation (dh, dw) along (rows, columns); each output
 * extent follows the same formula per axis. Returns 0, or -1 on a bad shape or when memory
 * runs out. */
int oracle_conv2d_acc2(const void *x, int xdt, const void *w, int wdt, int64_t B, int64_t C,
                       int64_t H, int64_t W, int64_t O, int64_t KH, int64_t KW, int64_t sh,
                       int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw,
                       const int64_t *imgs, int64_t nimgs, int32_t *acc) {
  int64_t Ho = oracle_conv_out_size(H, KH, sh, ph, dh);
  int64_t Wo = oracle_conv_out_size(W, KW, sw, pw, dw);
  if (Ho <= 0 || Wo <= 0 || sh < 1 || sw < 1 || dh < 1 || dw < 1 || ph < 0 || pw < 0 || KH < 1 ||
      KW < 1)
    return -1;
  int64_t R = C * KH * KW, L = Ho * Wo, Hp = H + 2 * ph, Wp = W + 2 * pw;
  if (R >= (1 << 24)) return -1;
  if (!imgs) nimgs = B;

  /* weight viewed as [O, C*KH*KW] over the OIHW order, signed */
  float *ws = (float *)malloc(sizeof(float) * (size_t)(O * R));
  float *xp = (float *)malloc(sizeof(float) * (size_t)(C * Hp * Wp));
  float *cols = (float *)malloc(sizeof(float) * (size_t)(L * R));
  if (!ws || !xp || !cols) {
    free(ws); free(xp); free(cols);
    return -1;
  }
  oracle_sign(w, wdt, O * R, ws);

  for (int64_t n = 0; n < nimgs; n++) {
    int64_t b = imgs ? imgs[n] : n;
    /* sign, then zero-pad by ph rows and pw columns on each side */
    memset(xp, 0, sizeof(float) * (size_t)(C * Hp * Wp));
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < C; c++)
      for (int64_t ih = 0; ih < H; ih++)
        for (int64_t iw = 0; iw < W; iw++)
          xp[(c * Hp + ih + ph) * Wp + iw + pw] = sgn(widen(x, xdt, ((b * C + c) * H + ih) * W + iw));
    /* unfold: kernel KH x KW, dilation (dh, dw), stride (sh, sw), stored transposed as cols[l][r] */
#pragma omp parallel for schedule(static)
    for (int64_t l = 0; l < L; l++) {
      int64_t oh = l / Wo, ow = l % Wo;
      for (int64_t c = 0; c < C; c++)
        for (int64_t i = 0; i < KH; i++)
          for (int64_t j = 0; j < KW; j++) {
            int64_t r = (c * KH + i) * KW + j;
            cols[l * R + r] = xp[(c * Hp + oh * sh + i * dh) * Wp + ow * sw + j * dw];
          }
    }
    /* [L, R] x [R, O] -> [L, O], written transposed as [O, Ho, Wo] */
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t o = 0; o < O; o++)
      for (int64_t l = 0; l < L; l++) {
        const float *wr = ws + o * R, *cr = cols + l * R;
        float sum = 0.0f;
#pragma omp simd reduction(+ : sum)
        for (int64_t r = 0; r < R; r++) sum += cr[r] * wr[r];
        acc[(n * O + o) * L + l] = (int32_t)sum;
      }
  }
  free(ws);
  free(xp);
  free(cols);
  return 0;
}

/* Square kernels, one stride / padding / dilation for both axes. */
int oracle_conv2d_acc(const void *x, int xdt, const void *w, int wdt, int64_t B, int64_t C,
                      int64_t H, int64_t W, int64_t O, int64_t ks, int64_t s, int64_t p, int64_t d,
                      const int64_t *imgs, int64_t nimgs, int32_t *acc) {
  return oracle_conv2d_acc2(x, xdt, w, wdt, B, C, H, W, O, ks, ks, s, s, p, p, d, d, imgs, nimgs,
                            acc);
}

/* Number of real (unpadded) reduction terms per output pixel, general form:
 * kv[oh][ow] = C * #{(i,j) : 0 <= oh*sh - ph + i*dh < H and 0 <= ow*sw - pw + j*dw < W}. */
int oracle_conv2d_kvalid2(int64_t C, int64_t H, int64_t W, int64_t KH, int64_t KW, int64_t sh,
                          int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw, int32_t *kv) {
  int64_t Ho = oracle_conv_out_size(H, KH, sh, ph, dh);
  int64_t Wo = oracle_conv_out_size(W, KW, sw, pw, dw);
  if (Ho <= 0 || Wo <= 0) return -1;
  for (int64_t oh = 0; oh < Ho; oh++)
    for (int64_t ow = 0; ow < Wo; ow++) {
      int64_t taps = 0;
      for (int64_t i = 0; i < KH; i++)
        for (int64_t j = 0; j < KW; j++) {
          int64_t ih = oh * sh - ph + i * dh, iw = ow * sw - pw + j * dw;
          if (ih >= 0 && ih < H && iw >= 0 && iw < W) taps++;
        }
      kv[oh * Wo + ow] = (int32_t)(C * taps);
    }
  return 0;
}

/* Square kernels. */
int oracle_conv2d_kvalid(int64_t C, int64_t H, int64_t W, int64_t ks, int64_t s, int64_t p,
                         int64_t d, int32_t *kv) {
  return oracle_conv2d_kvalid2(C, H, W, ks, ks, s, s, p, p, d, d, kv);
}

/* y[i] = acc[i] * (scale_a * scale_w), the product of the two scalar scales taken in double. */
void oracle_scale(const int32_t *acc, int64_t count, double scale_a, double scale_w, double *y) {
  double alpha = scale_a * scale_w;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; i++) y[i] = (double)acc[i] * alpha;
}

/* The shifted sign rule: +1 when x + b >= 0 (the sum taken in double), else -1. */
static float sgn_shift(float v, float b) {
  double sum = (double)v + (double)b;
  return sum >= 0.0 ? 1.0f : -1.0f;
}

/* Row-major x[rows][k] shifted by a bias, then packed as oracle_pack_rows does. The bias of
 * column kk is bias[kk] when blen == k and bias[0] for every column when blen == 1; bit j of
 * word q is 1 iff x[r][32q+j] + bias >= 0. */
void oracle_pack_rows_shift(const void *x, int dtype, int64_t rows, int64_t k, const void *bias,
                            int bdtype, int64_t blen, uint32_t *out) {
  int64_t kw = (k + 31) / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++)
    for (int64_t q = 0; q < kw; q++) {
      uint32_t word = 0;
      for (int j = 0; j < 32 && 32 * q + j < k; j++) {
        int64_t col = 32 * q + j;
        float b = widen(bias, bdtype, blen == 1 ? 0 : col);
        if (sgn_shift(widen(x, dtype, r * k + col), b) > 0.0f) word |= (uint32_t)1 << j;
      }
      out[r * kw + q] = word;
    }
}

/* NCHW x[b][c][h][w] shifted by bias[c], then packed as oracle_pack_nchw does: bit j of word
 * q of pixel (b, h, w) is 1 iff x[b][32q+j][h][w] + bias[32q+j] >= 0. */
void oracle_pack_nchw_shift(const void *x, int dtype, int64_t B, int64_t C, int64_t H, int64_t W,
                            const void *bias, int bdtype, uint32_t *out) {
  int64_t cw = (C + 31) / 32;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < B; b++)
    for (int64_t ih = 0; ih < H; ih++)
      for (int64_t iw = 0; iw < W; iw++)
        for (int64_t q = 0; q < cw; q++) {
          uint32_t word = 0;
          for (int j = 0; j < 32 && 32 * q + j < C; j++) {
            int64_t c = 32 * q + j;
            int64_t idx = ((b * C + c) * H + ih) * W + iw;
            if (sgn_shift(widen(x, dtype, idx), widen(bias, bdtype, c)) > 0.0f) word |= (uint32_t)1 << j;
          }
          out[((b * H + ih) * W + iw) * cw + q] = word;
        }
}

/* The lazily initialised activation scale: factor * mean|x| over count elements (factor 2 for
 * symmetric quantization, 4 otherwise), the sum of |x[i]| taken in double in index order. */
double oracle_abs_mean_scale(const void *x, int dtype, int64_t count, double factor) {
  double sum = 0.0;
  for (int64_t i = 0; i < count; i++) sum += fabs((double)widen(x, dtype, i));
  return factor * (sum / (double)count);
}

/* ---- W8A8 conv: the blog's im2col + GEMM with INT8 quantizers (section 3,
 * MyInitQuantConv2d: the unfolded input and the flattened weight each pass
 * through a quantizer before the mm). The quantizers are not defined on the
 * page; the reading taken here is per-tensor symmetric 8-bit with a given
 * amax: step s = amax / 127 (fp32), code q = clamp(rint(v / s), -127, 127)
 * with the division in fp32 and rint rounding half to even; NaN codes as 0.
 * The fake-quantized product then equals (s_x * s_w) * sum q_x * q_w, and
 * padded taps (zeros) code as 0. */

/* Step of the symmetric quantizer: amax / 127 in fp32. */
static float q_step(float amax) { return amax / 127.0f; }

static int8_t q_code(float v, float step) {
  if (v != v) return 0;
  float r = rintf(v / step);
  if (r > 127.0f) r = 127.0f;
  if (r < -127.0f) r = -127.0f;
  return (int8_t)r;
}

/* codes[i] = q(x[i]) for count elements, step amax / 127. */
void oracle_quant_i8(const void *x, int dtype, int64_t count, float amax, int8_t *codes) {
  float step = q_step(amax);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; i++) codes[i] = q_code(widen(x, dtype, i), step);
}

/* W8A8 conv accumulators acc[i][o][oh][ow] = sum over the unfolded reduction of
 * q(x) * q(w), by zero-padded unfold + GEMM as oracle_conv2d_acc2 (codes in place of signs),
 * summed in double (exact: |acc| < 127 * 127 * R < 2^53). Returns 0 or -1. */
int oracle_w8a8_conv2d_acc(const void *x, int xdt, const void *w, int wdt, int64_t B, int64_t C,
                           int64_t H, int64_t W, int64_t O, int64_t KH, int64_t KW, int64_t sh,
                           int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw,
                           float amax_x, float amax_w, const int64_t *imgs, int64_t nimgs,
                           int32_t *acc) {
  int64_t Ho = oracle_conv_out_size(H, KH, sh, ph, dh);
  int64_t Wo = oracle_conv_out_size(W, KW, sw, pw, dw);
  if (Ho <= 0 || Wo <= 0 || sh < 1 || sw < 1 || dh < 1 || dw < 1 || ph < 0 || pw < 0 || KH < 1 ||
      KW < 1)
    return -1;
  int64_t R = C * KH * KW, L = Ho * Wo, Hp = H + 2 * ph, Wp = W + 2 * pw;
  if (!imgs) nimgs = B;
  float step_x = q_step(amax_x), step_w = q_step(amax_w);
  double *wq = (double *)malloc(sizeof(double) * (size_t)(O * R));
  double *xp = (double *)malloc(sizeof(double) * (size_t)(C * Hp * Wp));
  double *cols = (double *)malloc(sizeof(double) * (size_t)(L * R));
  if (!wq || !xp || !cols) {
    free(wq); free(xp); free(cols);
    return -1;
  }
  for (int64_t i = 0; i < O * R; i++) wq[i] = (double)q_code(widen(w, wdt, i), step_w);
  for (int64_t n = 0; n < nimgs; n++) {
    int64_t b = imgs ? imgs[n] : n;
    /* quantize, then zero-pad (the unfold pads the input with zeros, whose code is 0) */
    memset(xp, 0, sizeof(double) * (size_t)(C * Hp * Wp));
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < C; c++)
      for (int64_t ih = 0; ih < H; ih++)
        for (int64_t iw = 0; iw < W; iw++)
          xp[(c * Hp + ih + ph) * Wp + iw + pw] =
              (double)q_code(widen(x, xdt, ((b * C + c) * H + ih) * W + iw), step_x);
#pragma omp parallel for schedule(static)
    for (int64_t l = 0; l < L; l++) {
      int64_t oh = l / Wo, ow = l % Wo;
      for (int64_t c = 0; c < C; c++)
        for (int64_t i = 0; i < KH; i++)
          for (int64_t j = 0; j < KW; j++)
            cols[l * R + (c * KH + i) * KW + j] = xp[(c * Hp + oh * sh + i * dh) * Wp + ow * sw + j * dw];
    }
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t o = 0; o < O; o++)
      for (int64_t l = 0; l < L; l++) {
        const double *wr = wq + o * R, *cr = cols + l * R;
        double sum = 0.0;
        for (int64_t r = 0; r < R; r++) sum += cr[r] * wr[r];
        acc[(n * O + o) * L + l] = (int32_t)sum;
      }
  }
  free(wq);
  free(xp);
  free(cols);
  return 0;
}

/* ---------------------------------------------------------------------------
 * Straight-through backward of the binarized linear layer.
 *
 * The BinaryLinearForward page describes its backward in words: the output
 * gradient meets the signed, scaled weights for grad_input and the signed,
 * scaled activations for grad_weight, grad_input is clipped, grad_scale_a is
 * returned and scale_w gets none. The qconv/binary/cutlass/layer page prints
 * the same steps for the conv (BinaryConv2dForward.backward). The linear form
 * here is that conv form with a 1x1 kernel on a 1x1 image (batch M, C = K
 * input features, O = N outputs), a reading taken here:
 *
 *   grad_in[m][k]  = (scale_w * sum_n g[m][n] * sign0(W[n][k])) * mid(x[m][k])
 *   mid(v)         = 0 if the fp32 quotient v / scale_a is < -1 or > 1, else 1
 *   grad_scale_a   = sum_{m,k} grad_in[m][k] * sign0(x[m][k]) / sqrt(M * K)
 *   grad_w[n][k]   = sum_m g[m][n] * (sign0(x[m][k]) * scale_a)
 *
 * sign0 is torch.sign as the backward uses it (unlike the forward's rule):
 * 0 for +-0, NaN for NaN, +-1 otherwise. The clip quotient is one IEEE fp32
 * division of the widened input by scale_a (a reading taken here: the page
 * divides in the layer's dtype); a NaN quotient fails both tests, so its mask
 * is 1, as the page's 1 - small - large gives. The mask multiplies (0 * inf
 * is NaN, as on the page). Sums are in double, products exact.
 * ------------------------------------------------------------------------- */
static double sign0(float v) {
  if (v != v) return NAN;
  return v > 0.0f ? 1.0 : (v < 0.0f ? -1.0 : 0.0);
}

static double clip_mid(float v, float scale_a) {
  float q = v / scale_a;
  double small = q < -1.0f ? 1.0 : 0.0, large = q > 1.0f ? 1.0 : 0.0;
  return 1.0 - small - large;
}

/* grad_in [M][K] and *grad_scale_a; g [M][N], W [N][K], x [M][K] in their dtypes. */
void oracle_linear_grad_input(const void *g, int gdt, const void *w, int wdt, const void *x, int xdt,
                              int64_t M, int64_t N, int64_t K, float scale_a, float scale_w,
                              double *grad_in, double *grad_scale_a) {
  double *ws = (double *)malloc(sizeof(double) * (size_t)(N * K));
  if (!ws) {
    *grad_scale_a = NAN;
    return;
  }
  for (int64_t i = 0; i < N * K; i++) ws[i] = sign0(widen(w, wdt, i)) * (double)scale_w;
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; m++) {
    double *row = grad_in + m * K;
    for (int64_t k = 0; k < K; k++) row[k] = 0.0;
    for (int64_t n = 0; n < N; n++) {
      double gv = (double)widen(g, gdt, m * N + n);
      const double *wr = ws + n * K;
      for (int64_t k = 0; k < K; k++) row[k] += gv * wr[k];
    }
    for (int64_t k = 0; k < K; k++) row[k] *= clip_mid(widen(x, xdt, m * K + k), scale_a);
  }
  free(ws);
  double total = 0.0;
  for (int64_t i = 0; i < M * K; i++) total += grad_in[i] * sign0(widen(x, xdt, i));
  *grad_scale_a = total / sqrt((double)M * (double)K);
}

/* grad_w [N][K]; g [M][N], x [M][K] in their dtypes. */
void oracle_linear_grad_weight(const void *g, int gdt, const void *x, int xdt, int64_t M, int64_t N,
                               int64_t K, float scale_a, double *grad_w) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; n++) {
    double *row = grad_w + n * K;
    for (int64_t k = 0; k < K; k++) row[k] = 0.0;
    for (int64_t m = 0; m < M; m++) {
      double gv = (double)widen(g, gdt, m * N + n);
      for (int64_t k = 0; k < K; k++) row[k] += gv * (sign0(widen(x, xdt, m * K + k)) * (double)scale_a);
    }
  }
}

/* int8 codes of grad_w, as the conv page's backward ends (grad_weight =
 * nv_tensor_quant(grad_weight)[0]). nv_tensor_quant is not on the pages; it is
 * read as the same per-tensor symmetric quantizer as the W8A8 conv, with amax
 * taken from the tensor itself: the gradient is held in fp32 (the value the
 * contraction produces), amax = max |v| (NaN if any v is NaN), step =
 * amax / 127 in fp32, code = clamp(rint(v / step), -127, 127), and a NaN
 * quotient (0 / 0 when every gradient is 0, a NaN amax, inf / inf) codes as 0. */
void oracle_quant_grad_i8(const double *grad_w, int64_t count, int8_t *codes, float *amax_out) {
  float amax = 0.0f;
  for (int64_t i = 0; i < count; i++) {
    float v = fabsf((float)grad_w[i]);
    if (v != v) {
      amax = v;
      break;
    }
    if (v > amax) amax = v;
  }
  *amax_out = amax;
  float step = amax / 127.0f;
  for (int64_t i = 0; i < count; i++) {
    float r = rintf((float)grad_w[i] / step);
    if (r != r) r = 0.0f;
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    codes[i] = (int8_t)r;
  }
}

/* Straight-through backward of the binarized conv, BinaryConv2dForward.backward on the
 * qconv/binary/cutlass/layer page, with a KH x KW kernel and a stride, padding and dilation per
 * axis (the forward's general form). Output gradient g [B][O][Ho][Wo], weight W [O][C][KH][KW],
 * input x [B][C][H][W]; a tap (oh, ow, i, j) reads input row oh*sh - ph + i*dh and column
 * ow*sw - pw + j*dw, and taps in the padding carry nothing (the page's gradient convolutions take
 * the same padding as the forward):
 *   grad_in[b][c][ih][iw] = (scale_w * sum of g[b][o][oh][ow] * sign0(W[o][c][i][j]) over the
 *                            taps that read (ih, iw)) * mid(x[b][c][ih][iw])
 *   grad_scale_a          = sum of grad_in * sign0(x) over every element / sqrt(B*C*H*W)
 *   grad_w[o][c][i][j]    = sum over b, oh, ow of g[b][o][oh][ow] * (sign0(x at the tap) * scale_a)
 * (torch.nn.grad.conv2d_input and conv2d_weight on the page), with sign0 and mid as for the
 * linear layer. Sums in double. Returns 0, or -1 for an empty output or a bad geometry. */
int oracle_conv2d_grad(const void *g, int gdt, const void *w, int wdt, const void *x, int xdt,
                       int64_t B, int64_t C, int64_t H, int64_t W, int64_t O, int64_t KH, int64_t KW,
                       int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw,
                       float scale_a, float scale_w, double *grad_in, double *grad_scale_a,
                       double *grad_w) {
  int64_t Ho = oracle_conv_out_size(H, KH, sh, ph, dh);
  int64_t Wo = oracle_conv_out_size(W, KW, sw, pw, dw);
  if (Ho <= 0 || Wo <= 0 || sh < 1 || sw < 1 || dh < 1 || dw < 1 || ph < 0 || pw < 0 || KH < 1 ||
      KW < 1 || B < 1 || C < 1)
    return -1;
  for (int64_t i = 0; i < B * C * H * W; i++) grad_in[i] = 0.0;
  for (int64_t i = 0; i < O * C * KH * KW; i++) grad_w[i] = 0.0;
  /* one input channel per thread: it owns grad_in[:, c] and grad_w[:, c] */
#pragma omp parallel for schedule(static)
  for (int64_t c = 0; c < C; c++)
    for (int64_t b = 0; b < B; b++)
      for (int64_t o = 0; o < O; o++)
        for (int64_t oh = 0; oh < Ho; oh++)
          for (int64_t ow = 0; ow < Wo; ow++) {
            double gv = (double)widen(g, gdt, ((b * O + o) * Ho + oh) * Wo + ow);
            for (int64_t i = 0; i < KH; i++)
              for (int64_t j = 0; j < KW; j++) {
                int64_t ih = oh * sh - ph + i * dh, iw = ow * sw - pw + j * dw;
                if (ih < 0 || ih >= H || iw < 0 || iw >= W) continue;
                int64_t xi = ((b * C + c) * H + ih) * W + iw, wi = ((o * C + c) * KH + i) * KW + j;
                grad_in[xi] += gv * (sign0(widen(w, wdt, wi)) * (double)scale_w);
                grad_w[wi] += gv * (sign0(widen(x, xdt, xi)) * (double)scale_a);
              }
          }
  double total = 0.0;
  for (int64_t i = 0; i < B * C * H * W; i++) {
    float v = widen(x, xdt, i);
    grad_in[i] *= clip_mid(v, scale_a);
    total += grad_in[i] * sign0(v);
  }
  *grad_scale_a = total / sqrt((double)(B * C * H * W));
  return 0;
}
