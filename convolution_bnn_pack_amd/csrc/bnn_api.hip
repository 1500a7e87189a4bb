// C ABI of libbnn: argument validation, output shapes, the scale product,
// per-shape path choice and kernel dispatch on the caller's stream.
//
// Every check runs before the first HIP call, so a rejected call enqueues
// nothing and leaves the outputs untouched (this also makes the checks
// testable on a host without a GPU).
#include <math.h>

#include <mutex>

#include "../../include/bnn.h"
#include "launch.h"

namespace bnn {
int xor_conv_max_taps();
}

namespace {

thread_local int g_last_path = 0;

bool float_dtype(int d) { return d == BNN_F32 || d == BNN_F16 || d == BNN_BF16; }
// Already-packed activations: 32-bit words, or the CUTLASS layer's 8-bit containers.
bool packed_dtype(int d) { return d == BNN_U32_PACKED || d == BNN_U8_PACKED; }
// 8-bit containers of a whole number of 32-bit words are those words byte for byte and are
// read in place; other lengths are repacked into the workspace.
bool u8_in_place(int x_dtype, int64_t bits) { return x_dtype == BNN_U8_PACKED && bits % 32 == 0; }
bool half_dtype(int d) { return d == BNN_F16 || d == BNN_BF16; }
bool out_dtype_ok(int d) { return float_dtype(d) || d == BNN_I32; }
int elem_bytes(int d) { return d == BNN_F32 ? 4 : 2; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// floor((size + 2p - d(k-1) - 1)/s + 1) with a true floor for negative numerators.
int64_t out_size(int64_t size, int64_t k, int64_t s, int64_t p, int64_t d) {
  const int64_t num = size + 2 * p - d * (k - 1) - 1;
  int64_t q = num / s;
  if (num % s != 0 && num < 0) q -= 1;
  return q + 1;
}

// The contraction's scale: the host product of the two scalar scales in
// double (as the layer forward computes it before calling the native
// kernel), rounded once to float for the fp32 epilogue.
float alpha_of(double scale_a, double scale_w) { return (float)(scale_a * scale_w); }

bnn_status hip_status(hipError_t e) { return e == hipSuccess ? BNN_OK : BNN_ERR_HIP; }

// Path choice. Measured over linear shapes from 64x256x512 to 16384x8192x8192
// and ResNet-style convs, the fp4 matrix-core path is the fastest everywhere,
// tiny layers included (its per-tile cost is lower than the VALU kernel's),
// and the int8 path runs within a few percent of it only on convs with 64
// channels. AUTO therefore takes fp4 whenever its fp32 sums are exact
// (K <= 2^24) and int8 beyond. The XOR path stays available on request: it is
// the pages' own formulation and an independent cross-check of the others.
int auto_path(int64_t k) { return k <= bnn::kMaxFp4K ? BNN_PATH_MFMA_FP4 : BNN_PATH_MFMA; }

bool int_fits(int64_t v) { return v >= 0 && v <= 0x7FFFFFFFLL; }

// Words holding n signs: the last one partly when n % 32 != 0 (its missing bits are 0).
int64_t words_of(int64_t n) { return (n + 31) / 32; }

// A reduction length the kernels can index: the contraction kernels count 32 signs per
// word in int, so 32 * words_of(n) must fit as well as n itself.
bool bits_fit(int64_t n) { return int_fits(n) && int_fits(32 * words_of(n)); }

// Row sign+pack of any row length: the 16-byte vector kernels when rows are whole words and
// the tensor is 16-byte aligned, the one-element-per-lane kernel otherwise.
hipError_t pack_rows_any(const void* x, int dtype, int64_t rows, int64_t k, const void* bias,
                         int bdtype, bool percol, uint32_t* out, hipStream_t s) {
  if (k % 32 == 0 && aligned(x, 16)) {
    if (!bias) return bnn::launch_pack_rows(x, dtype, rows * (k / 32), out, s);
    return bnn::launch_pack_rows_shift(x, dtype, rows, k / 32, bias, bdtype, percol, out, s);
  }
  return bnn::launch_pack_rows_ragged(x, dtype, rows, k, bias, bdtype, percol, out, s);
}

bool path_known(int path) {
  return path == BNN_PATH_AUTO || path == BNN_PATH_XOR || path == BNN_PATH_MFMA ||
         path == BNN_PATH_MFMA_FP4;
}

hipError_t run_path(int use, const bnn::Contraction& p, bool conv, int out_dtype, hipStream_t s) {
  switch (use) {
    case BNN_PATH_XOR: return bnn::launch_xor(p, conv, out_dtype, s);
    case BNN_PATH_MFMA_FP4: return bnn::launch_mfma_fp4(p, conv, out_dtype, s);
    default: return bnn::launch_mfma(p, conv, out_dtype, s);
  }
}

// Device memory of bnn_gemm_noalloc: the packed activations it would otherwise need a
// workspace for live in this file-scope array, which each device holds from the library's
// load until the process ends. Host code must never use the array's name as an address
// (on the host it is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, taken once per device with that device current and kept here.
constexpr size_t kScratchBytes = BNN_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint32_t scratch[kScratchBytes / sizeof(uint32_t)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch` (its address there), resolved on the first call on
// that device.
bnn_status scratch_of_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BNN_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BNN_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return BNN_OK;
}

// bnn_gemm's body. With use_scratch the packed activations go to the current device's
// `scratch` (at most kScratchBytes) instead of the caller's workspace.
bnn_status gemm_impl(const void* x, int x_dtype, const uint32_t* w_packed, int64_t m, int64_t n,
                     int64_t k, double scale_a, double scale_w, int path, void* out,
                     int out_dtype, void* workspace, size_t workspace_bytes, bool use_scratch,
                     void* stream);

}  // namespace

extern "C" {

const char* bnn_status_string(int s) {
  switch (s) {
    case BNN_OK: return "ok";
    case BNN_ERR_NULL: return "null pointer argument";
    case BNN_ERR_SHAPE: return "invalid shape (sizes, bias length, or empty conv output)";
    case BNN_ERR_DTYPE: return "dtype not allowed for this argument";
    case BNN_ERR_ALIGN: return "pointer not aligned as required";
    case BNN_ERR_WORKSPACE: return "workspace missing or too small";
    case BNN_ERR_PATH: return "unknown path or path cannot run this shape";
    case BNN_ERR_HIP: return "HIP runtime error on launch";
    default: return "unknown status";
  }
}

int bnn_last_path(void) { return g_last_path; }

size_t bnn_gemm_workspace_bytes(int64_t m, int64_t k, int x_dtype) {
  if (x_dtype == BNN_U32_PACKED || u8_in_place(x_dtype, k) || m <= 0 || k <= 0) return 0;
  return (size_t)m * (size_t)words_of(k) * 4u;
}

size_t bnn_conv2d_workspace_bytes(int64_t n, int64_t c, int64_t h, int64_t w, int x_dtype) {
  if (x_dtype == BNN_U32_PACKED || u8_in_place(x_dtype, c) || n <= 0 || c <= 0 || h <= 0 || w <= 0)
    return 0;
  return (size_t)n * (size_t)h * (size_t)w * (size_t)words_of(c) * 4u;
}

bnn_status bnn_u8_to_words(const uint8_t* src, int64_t rows, int64_t bits, uint32_t* dst,
                           void* stream) {
  if (rows < 0 || bits < 1 || !bits_fit(bits)) return BNN_ERR_SHAPE;
  if (!int_fits(rows) || !int_fits(words_of(bits)) || rows * words_of(bits) < 0) return BNN_ERR_SHAPE;
  if (rows == 0) return BNN_OK;
  if (!src || !dst) return BNN_ERR_NULL;
  if (!aligned(dst, 4)) return BNN_ERR_ALIGN;
  return hip_status(bnn::launch_u8_to_words(src, rows, bits, dst, static_cast<hipStream_t>(stream)));
}

int bnn_gemm_auto_path(int64_t m, int64_t n, int64_t k) {
  (void)m;
  (void)n;
  return auto_path(k);
}

int bnn_conv2d_auto_path(int64_t n, int64_t c, int64_t h, int64_t w, int64_t out_channels,
                         int kernel_size, int stride, int padding, int dilation) {
  (void)n;
  (void)h;
  (void)w;
  (void)out_channels;
  (void)stride;
  (void)padding;
  (void)dilation;
  return auto_path((int64_t)kernel_size * kernel_size * c);
}

bnn_status bnn_pack_sign(const void* x, int x_dtype, int64_t rows, int64_t k, uint32_t* x_packed,
                         void* stream) {
  if (!float_dtype(x_dtype)) return BNN_ERR_DTYPE;
  if (rows < 0 || k <= 0) return BNN_ERR_SHAPE;
  if (rows == 0) return BNN_OK;
  if (!x || !x_packed) return BNN_ERR_NULL;
  if (!aligned(x, elem_bytes(x_dtype)) || !aligned(x_packed, 4)) return BNN_ERR_ALIGN;
  return hip_status(pack_rows_any(x, x_dtype, rows, k, nullptr, 0, false, x_packed,
                                  static_cast<hipStream_t>(stream)));
}

bnn_status bnn_pack_sign_nchw(const void* x, int x_dtype, int64_t n, int64_t c, int64_t h,
                              int64_t w, uint32_t* x_packed, void* stream) {
  if (!float_dtype(x_dtype)) return BNN_ERR_DTYPE;
  if (n < 0 || c <= 0 || h <= 0 || w <= 0) return BNN_ERR_SHAPE;
  if (!int_fits(h * w) || !int_fits(n * words_of(c))) return BNN_ERR_SHAPE;
  if (n == 0) return BNN_OK;
  if (!x || !x_packed) return BNN_ERR_NULL;
  if (!aligned(x, elem_bytes(x_dtype)) || !aligned(x_packed, 4)) return BNN_ERR_ALIGN;
  return hip_status(bnn::launch_pack_nchw(x, x_dtype, n, c, h, w, x_packed,
                                          static_cast<hipStream_t>(stream)));
}

size_t bnn_abs_mean_workspace_bytes(int64_t count) {
  if (count <= 0) return 0;
  return (size_t)bnn::abs_mean_parts(count) * sizeof(double);
}

bnn_status bnn_pack_sign_shift(const void* x, int x_dtype, int64_t rows, int64_t k,
                               const void* bias, int bias_dtype, int64_t bias_len,
                               uint32_t* x_packed, void* stream) {
  if (!float_dtype(x_dtype) || !float_dtype(bias_dtype)) return BNN_ERR_DTYPE;
  if (rows < 0 || k <= 0) return BNN_ERR_SHAPE;
  if (bias_len != 1 && bias_len != k) return BNN_ERR_SHAPE;
  if (rows == 0) return BNN_OK;
  if (!x || !bias || !x_packed) return BNN_ERR_NULL;
  if (!aligned(x, elem_bytes(x_dtype)) || !aligned(x_packed, 4) ||
      !aligned(bias, elem_bytes(bias_dtype)))
    return BNN_ERR_ALIGN;
  return hip_status(pack_rows_any(x, x_dtype, rows, k, bias, bias_dtype, bias_len == k && k > 1,
                                  x_packed, static_cast<hipStream_t>(stream)));
}

bnn_status bnn_pack_sign_nchw_shift(const void* x, int x_dtype, int64_t n, int64_t c, int64_t h,
                                    int64_t w, const void* bias, int bias_dtype,
                                    uint32_t* x_packed, void* stream) {
  if (!float_dtype(x_dtype) || !float_dtype(bias_dtype)) return BNN_ERR_DTYPE;
  if (n < 0 || c <= 0 || h <= 0 || w <= 0) return BNN_ERR_SHAPE;
  if (!int_fits(h * w) || !int_fits(n * words_of(c))) return BNN_ERR_SHAPE;
  if (n == 0) return BNN_OK;
  if (!x || !bias || !x_packed) return BNN_ERR_NULL;
  if (!aligned(x, elem_bytes(x_dtype)) || !aligned(x_packed, 4) ||
      !aligned(bias, elem_bytes(bias_dtype)))
    return BNN_ERR_ALIGN;
  return hip_status(bnn::launch_pack_nchw(x, x_dtype, n, c, h, w, x_packed,
                                          static_cast<hipStream_t>(stream), bias, bias_dtype));
}

bnn_status bnn_abs_mean_scale(const void* x, int x_dtype, int64_t count, double factor,
                              double* scale_out, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (!float_dtype(x_dtype)) return BNN_ERR_DTYPE;
  if (count <= 0) return BNN_ERR_SHAPE;
  if (!x || !scale_out) return BNN_ERR_NULL;
  if (!aligned(x, 16) || !aligned(scale_out, 8)) return BNN_ERR_ALIGN;
  if (!workspace || workspace_bytes < bnn_abs_mean_workspace_bytes(count)) return BNN_ERR_WORKSPACE;
  if (!aligned(workspace, 8)) return BNN_ERR_ALIGN;
  return hip_status(bnn::launch_abs_mean(x, x_dtype, count, factor,
                                         static_cast<double*>(workspace), scale_out,
                                         static_cast<hipStream_t>(stream)));
}

size_t bnn_pack_sign_shift_abs_mean_workspace_bytes(int64_t rows, int64_t k) {
  if (rows <= 0 || k <= 0) return 0;
  const int64_t fused = k % 32 == 0 ? bnn::pack_rows_shift_abs_parts(rows, k / 32) : 0;
  const int64_t two = bnn::abs_mean_parts(rows * k);
  return (size_t)(fused > two ? fused : two) * sizeof(double);
}

bnn_status bnn_pack_sign_shift_abs_mean(const void* x, int x_dtype, int64_t rows, int64_t k,
                                        const void* bias, int bias_dtype, int64_t bias_len,
                                        double factor, uint32_t* x_packed, double* scale_out,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  if (!float_dtype(x_dtype) || !float_dtype(bias_dtype)) return BNN_ERR_DTYPE;
  if (rows <= 0 || k <= 0) return BNN_ERR_SHAPE;
  if (bias_len != 1 && bias_len != k) return BNN_ERR_SHAPE;
  if (!x || !bias || !x_packed || !scale_out) return BNN_ERR_NULL;
  if (!aligned(x, 16) || !aligned(x_packed, 4) || !aligned(bias, elem_bytes(bias_dtype)) ||
      !aligned(scale_out, 8))
    return BNN_ERR_ALIGN;
  if (!workspace || workspace_bytes < bnn_pack_sign_shift_abs_mean_workspace_bytes(rows, k))
    return BNN_ERR_WORKSPACE;
  if (!aligned(workspace, 8)) return BNN_ERR_ALIGN;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool percol = bias_len == k && k > 1;
  double* part = static_cast<double*>(workspace);
  if (k % 32 == 0)
    return hip_status(bnn::launch_pack_rows_shift_abs(x, x_dtype, rows, k / 32, bias, bias_dtype,
                                                      percol, x_packed, factor, part, scale_out, s));
  // rows that are not whole words: the two passes
  const hipError_t e = pack_rows_any(x, x_dtype, rows, k, bias, bias_dtype, percol, x_packed, s);
  if (e != hipSuccess) return BNN_ERR_HIP;
  return hip_status(bnn::launch_abs_mean(x, x_dtype, rows * k, factor, part, scale_out, s));
}

size_t bnn_pack_sign_nchw_shift_abs_mean_workspace_bytes(int x_dtype, int64_t n, int64_t c,
                                                         int64_t h, int64_t w) {
  if (!float_dtype(x_dtype) || n <= 0 || c <= 0 || h <= 0 || w <= 0) return 0;
  const int64_t fused = bnn::pack_nchw_abs_parts(x_dtype, n, c, h, w);
  const int64_t two = bnn::abs_mean_parts(n * c * h * w);
  return (size_t)(fused > two ? fused : two) * sizeof(double);
}

bnn_status bnn_pack_sign_nchw_shift_abs_mean(const void* x, int x_dtype, int64_t n, int64_t c,
                                             int64_t h, int64_t w, const void* bias, int bias_dtype,
                                             double factor, uint32_t* x_packed, double* scale_out,
                                             void* workspace, size_t workspace_bytes, void* stream) {
  if (!float_dtype(x_dtype) || !float_dtype(bias_dtype)) return BNN_ERR_DTYPE;
  if (n <= 0 || c <= 0 || h <= 0 || w <= 0) return BNN_ERR_SHAPE;
  if (!int_fits(h * w) || !int_fits(n * words_of(c)) || !int_fits(n * h * w)) return BNN_ERR_SHAPE;
  if (!x || !bias || !x_packed || !scale_out) return BNN_ERR_NULL;
  if (!aligned(x, 16) || !aligned(x_packed, 4) || !aligned(bias, elem_bytes(bias_dtype)) ||
      !aligned(scale_out, 8))
    return BNN_ERR_ALIGN;
  if (!workspace || workspace_bytes < bnn_pack_sign_nchw_shift_abs_mean_workspace_bytes(x_dtype, n, c, h, w))
    return BNN_ERR_WORKSPACE;
  if (!aligned(workspace, 8)) return BNN_ERR_ALIGN;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  double* part = static_cast<double*>(workspace);
  if (bnn::pack_nchw_abs_fused(x_dtype, h, w, x))
    return hip_status(bnn::launch_pack_nchw_shift_abs(x, x_dtype, n, c, h, w, x_packed, bias,
                                                      bias_dtype, factor, part, scale_out, s));
  // pixel planes that are not a multiple of the vector width: the two passes
  const hipError_t e = bnn::launch_pack_nchw(x, x_dtype, n, c, h, w, x_packed, s, bias, bias_dtype);
  if (e != hipSuccess) return BNN_ERR_HIP;
  return hip_status(bnn::launch_abs_mean(x, x_dtype, n * c * h * w, factor, part, scale_out, s));
}

bnn_status bnn_w_pack(const void* weight, int w_dtype, int64_t out_features, int64_t in_features,
                      int kernel_size, uint32_t* w_packed, void* stream) {
  if (!float_dtype(w_dtype)) return BNN_ERR_DTYPE;
  if (out_features < 0 || in_features <= 0 || kernel_size < 0) return BNN_ERR_SHAPE;
  if (out_features == 0) return BNN_OK;
  if (!weight || !w_packed) return BNN_ERR_NULL;
  if (!aligned(w_packed, 4)) return BNN_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kernel_size == 0) {
    if (!aligned(weight, elem_bytes(w_dtype))) return BNN_ERR_ALIGN;
    return hip_status(pack_rows_any(weight, w_dtype, out_features, in_features, nullptr, 0, false,
                                    w_packed, s));
  }
  return bnn_w_pack_conv(weight, w_dtype, out_features, in_features, kernel_size, kernel_size,
                         w_packed, stream);
}

bnn_status bnn_w_pack_conv(const void* weight, int w_dtype, int64_t out_features,
                           int64_t in_features, int kernel_h, int kernel_w, uint32_t* w_packed,
                           void* stream) {
  if (!float_dtype(w_dtype)) return BNN_ERR_DTYPE;
  if (out_features < 0 || in_features <= 0 || kernel_h < 1 || kernel_w < 1) return BNN_ERR_SHAPE;
  if (!int_fits((int64_t)kernel_h * kernel_w * words_of(in_features))) return BNN_ERR_SHAPE;
  if (out_features == 0) return BNN_OK;
  if (!weight || !w_packed) return BNN_ERR_NULL;
  if (!aligned(w_packed, 4) || !aligned(weight, elem_bytes(w_dtype))) return BNN_ERR_ALIGN;
  return hip_status(bnn::launch_pack_conv_weight(weight, w_dtype, out_features, in_features,
                                                 kernel_h, kernel_w,
                                                 static_cast<uint32_t*>(w_packed),
                                                 static_cast<hipStream_t>(stream)));
}

bnn_status bnn_gemm(const void* x, int x_dtype, const uint32_t* w_packed, int64_t m, int64_t n,
                    int64_t k, double scale_a, double scale_w, int path, void* out, int out_dtype,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return gemm_impl(x, x_dtype, w_packed, m, n, k, scale_a, scale_w, path, out, out_dtype,
                   workspace, workspace_bytes, false, stream);
}

bnn_status bnn_gemm_noalloc(const void* x, int x_dtype, const uint32_t* w_packed, int64_t m,
                            int64_t n, int64_t k, double scale_a, double scale_w, int path,
                            void* out, int out_dtype, void* stream) {
  return gemm_impl(x, x_dtype, w_packed, m, n, k, scale_a, scale_w, path, out, out_dtype, nullptr,
                   0, true, stream);
}

bnn_status bnn_conv2d_ex(const void* x, int x_dtype, int64_t n, int64_t c, int64_t h, int64_t w,
                         const uint32_t* w_packed, int64_t out_channels, double scale_a,
                         double scale_w, int kernel_h, int kernel_w, int stride_h, int stride_w,
                         int pad_h, int pad_w, int dil_h, int dil_w, int path, void* out,
                         int out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!(float_dtype(x_dtype) || packed_dtype(x_dtype)) || !out_dtype_ok(out_dtype))
    return BNN_ERR_DTYPE;
  if (n < 0 || out_channels < 0 || c <= 0 || h <= 0 || w <= 0) return BNN_ERR_SHAPE;
  if (kernel_h < 1 || kernel_w < 1 || stride_h < 1 || stride_w < 1 || dil_h < 1 || dil_w < 1 ||
      pad_h < 0 || pad_w < 0)
    return BNN_ERR_SHAPE;
  const int64_t ho = out_size(h, kernel_h, stride_h, pad_h, dil_h);
  const int64_t wo = out_size(w, kernel_w, stride_w, pad_w, dil_w);
  if (ho <= 0 || wo <= 0) return BNN_ERR_SHAPE;
  const int64_t taps = (int64_t)kernel_h * kernel_w;
  const int64_t kw_words = taps * words_of(c);
  if (!int_fits(n * ho * wo) || !int_fits(out_channels) || !int_fits(kw_words) ||
      !int_fits(n * h * w * words_of(c)) || !int_fits(h + 2 * (int64_t)pad_h) ||
      !int_fits(w + 2 * (int64_t)pad_w) || !int_fits(taps * c) || !bits_fit(c))
    return BNN_ERR_SHAPE;
  if (!path_known(path)) return BNN_ERR_PATH;
  if (path == BNN_PATH_XOR && taps > bnn::xor_conv_max_taps()) return BNN_ERR_PATH;
  if (path == BNN_PATH_MFMA_FP4 && taps * c > bnn::kMaxFp4K) return BNN_ERR_PATH;
  if (n == 0 || out_channels == 0) return BNN_OK;
  if (!x || !w_packed || !out) return BNN_ERR_NULL;
  const bool words_in = x_dtype == BNN_U32_PACKED || u8_in_place(x_dtype, c);
  // float x needs only its element alignment: unaligned tensors (a sliced batch) take the
  // element-wise NCHW pack
  const int x_align = words_in ? 4 : x_dtype == BNN_U8_PACKED ? 1 : elem_bytes(x_dtype);
  if (!aligned(x, x_align) || !aligned(w_packed, 4) || !aligned(out, 16)) return BNN_ERR_ALIGN;
  const size_t need = bnn_conv2d_workspace_bytes(n, c, h, w, x_dtype);
  if (need > 0 && (!workspace || workspace_bytes < need)) return BNN_ERR_WORKSPACE;
  if (need > 0 && !aligned(workspace, 4)) return BNN_ERR_ALIGN;

  const int use = path == BNN_PATH_AUTO ? auto_path(taps * c) : path;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint32_t* a = static_cast<const uint32_t*>(x);
  if (!words_in) {
    uint32_t* ws = static_cast<uint32_t*>(workspace);
    const hipError_t e =
        x_dtype == BNN_U8_PACKED
            ? bnn::launch_u8_to_words(static_cast<const uint8_t*>(x), n * h * w, c, ws, s)
            : bnn::launch_pack_nchw(x, x_dtype, n, c, h, w, ws, s);
    if (e != hipSuccess) return BNN_ERR_HIP;
    a = ws;
  }
  bnn::Contraction p{};
  p.a = a;
  p.w = w_packed;
  p.out = out;
  p.M = (int)(n * ho * wo);
  p.N = (int)out_channels;
  p.KW = (int)kw_words;
  p.KB = (int)c;
  p.alpha = alpha_of(scale_a, scale_w);
  p.H = (int)h;
  p.W = (int)w;
  p.CW = (int)words_of(c);
  p.Ho = (int)ho;
  p.Wo = (int)wo;
  p.KH = kernel_h;
  p.KWD = kernel_w;
  p.SH = stride_h;
  p.SW = stride_w;
  p.PH = pad_h;
  p.PW = pad_w;
  p.DH = dil_h;
  p.DW = dil_w;
  p.div_hw = bnn::FastDiv((uint32_t)(ho * wo));
  p.div_wo = bnn::FastDiv((uint32_t)wo);
  p.div_cw = bnn::FastDiv((uint32_t)p.CW);
  p.div_kwd = bnn::FastDiv((uint32_t)kernel_w);
  const hipError_t e = run_path(use, p, true, out_dtype, s);
  if (e != hipSuccess) return BNN_ERR_HIP;
  g_last_path = use;
  return BNN_OK;
}

bnn_status bnn_conv2d(const void* x, int x_dtype, int64_t n, int64_t c, int64_t h, int64_t w,
                      const uint32_t* w_packed, int64_t out_channels, double scale_a,
                      double scale_w, int kernel_size, int stride, int padding, int dilation,
                      int path, void* out, int out_dtype, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return bnn_conv2d_ex(x, x_dtype, n, c, h, w, w_packed, out_channels, scale_a, scale_w,
                       kernel_size, kernel_size, stride, stride, padding, padding, dilation,
                       dilation, path, out, out_dtype, workspace, workspace_bytes, stream);
}

// ---- W8A8 conv (the blog's im2col + GEMM with INT8 quantizers)

// Step of the per-tensor symmetric quantizer: amax / 127 in fp32.
static float w8a8_step(double amax) { return (float)amax / 127.0f; }
static bool amax_ok(double amax) { return amax > 0.0 && amax <= 3.0e38; }
// |acc| <= 127 * 127 * K must fit int32
static constexpr int64_t kMaxW8A8K = 0x7FFFFFFFLL / (127 * 127);

bnn_status bnn_quant_i8_nhwc(const void* x, int x_dtype, int64_t n, int64_t c, int64_t h, int64_t w,
                             double amax, int8_t* x_q, void* stream) {
  if (!float_dtype(x_dtype)) return BNN_ERR_DTYPE;
  if (n < 0 || c <= 0 || c % 16 != 0 || h <= 0 || w <= 0 || !amax_ok(amax)) return BNN_ERR_SHAPE;
  if (!int_fits(n * h * w) || !int_fits(c)) return BNN_ERR_SHAPE;
  if (n == 0) return BNN_OK;
  if (!x || !x_q) return BNN_ERR_NULL;
  if (!aligned(x, elem_bytes(x_dtype)) || !aligned(x_q, 16)) return BNN_ERR_ALIGN;
  return hip_status(bnn::launch_quant_nhwc(x, x_dtype, n, c, h, w, w8a8_step(amax), x_q,
                                           static_cast<hipStream_t>(stream)));
}

bnn_status bnn_quant_i8_weight(const void* weight, int w_dtype, int64_t out_channels, int64_t c,
                               int kernel_h, int kernel_w, double amax, int8_t* w_q, void* stream) {
  if (!float_dtype(w_dtype)) return BNN_ERR_DTYPE;
  if (out_channels < 0 || c <= 0 || c % 16 != 0 || kernel_h < 1 || kernel_w < 1 || !amax_ok(amax))
    return BNN_ERR_SHAPE;
  if (!int_fits((int64_t)kernel_h * kernel_w * c)) return BNN_ERR_SHAPE;
  if (out_channels == 0) return BNN_OK;
  if (!weight || !w_q) return BNN_ERR_NULL;
  if (!aligned(weight, elem_bytes(w_dtype)) || !aligned(w_q, 16)) return BNN_ERR_ALIGN;
  return hip_status(bnn::launch_quant_weight(weight, w_dtype, out_channels, c, kernel_h, kernel_w,
                                             w8a8_step(amax), w_q, static_cast<hipStream_t>(stream)));
}

bnn_status bnn_w8a8_conv2d(const int8_t* x_q, int64_t n, int64_t c, int64_t h, int64_t w,
                           const int8_t* w_q, int64_t out_channels, double amax_x, double amax_w,
                           int kernel_h, int kernel_w, int stride_h, int stride_w, int pad_h,
                           int pad_w, int dil_h, int dil_w, void* out, int out_dtype,
                           void* stream) {
  if (!out_dtype_ok(out_dtype)) return BNN_ERR_DTYPE;
  if (n < 0 || out_channels < 0 || c <= 0 || c % 16 != 0 || h <= 0 || w <= 0) return BNN_ERR_SHAPE;
  if (!amax_ok(amax_x) || !amax_ok(amax_w)) return BNN_ERR_SHAPE;
  if (kernel_h < 1 || kernel_w < 1 || stride_h < 1 || stride_w < 1 || dil_h < 1 || dil_w < 1 ||
      pad_h < 0 || pad_w < 0)
    return BNN_ERR_SHAPE;
  const int64_t ho = out_size(h, kernel_h, stride_h, pad_h, dil_h);
  const int64_t wo = out_size(w, kernel_w, stride_w, pad_w, dil_w);
  if (ho <= 0 || wo <= 0) return BNN_ERR_SHAPE;
  const int64_t k = (int64_t)kernel_h * kernel_w * c;
  if (k > kMaxW8A8K || !int_fits(n * ho * wo) || !int_fits(out_channels) || !int_fits(n * h * w * c))
    return BNN_ERR_SHAPE;
  if (n == 0 || out_channels == 0) return BNN_OK;
  if (!x_q || !w_q || !out) return BNN_ERR_NULL;
  if (!aligned(x_q, 16) || !aligned(w_q, 16) || !aligned(out, 16)) return BNN_ERR_ALIGN;
  // the output scale: the host product of the two fp32 steps, rounded once to float
  const float alpha = (float)((double)w8a8_step(amax_x) * (double)w8a8_step(amax_w));
  return hip_status(bnn::launch_w8a8_conv(x_q, w_q, out, out_dtype, n, c, h, w, out_channels, ho,
                                          wo, kernel_h, kernel_w, stride_h, stride_w, pad_h, pad_w,
                                          dil_h, dil_w, alpha, static_cast<hipStream_t>(stream)));
}

size_t bnn_linear_grad_input_workspace_bytes(int64_t m, int64_t k) {
  if (m <= 0 || k <= 0) return 0;
  return (size_t)bnn::bwd_grad_input_parts(m, k) * sizeof(double);
}

bnn_status bnn_linear_grad_input(const void* grad_out, const void* weight, const void* x,
                                 int dtype, int64_t m, int64_t n, int64_t k, float scale_a,
                                 float scale_w, float* grad_in, double* grad_scale_a,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  if (!half_dtype(dtype)) return BNN_ERR_DTYPE;
  if (m <= 0 || k <= 0 || n < 0 || n % 8 != 0 || k % 8 != 0) return BNN_ERR_SHAPE;
  if (!int_fits(m * k) || !int_fits(n * k) || !int_fits(m * n)) return BNN_ERR_SHAPE;
  if (!x || !grad_in || !grad_scale_a || (n > 0 && (!grad_out || !weight))) return BNN_ERR_NULL;
  if (!aligned(x, 2) || !aligned(grad_in, 4) || !aligned(grad_scale_a, 8)) return BNN_ERR_ALIGN;
  if (n > 0 && (!aligned(grad_out, 16) || !aligned(weight, 16))) return BNN_ERR_ALIGN;
  if (!workspace || workspace_bytes < bnn_linear_grad_input_workspace_bytes(m, k))
    return BNN_ERR_WORKSPACE;
  if (!aligned(workspace, 8)) return BNN_ERR_ALIGN;
  return hip_status(bnn::launch_linear_grad_input(
      grad_out, weight, x, dtype == BNN_BF16, m, n, k, scale_a, scale_w, grad_in,
      static_cast<double*>(workspace), grad_scale_a, static_cast<hipStream_t>(stream)));
}

bnn_status bnn_linear_grad_weight(const void* grad_out, const void* x, int dtype, int64_t m,
                                  int64_t n, int64_t k, float scale_a, float* grad_w,
                                  void* stream) {
  if (!half_dtype(dtype)) return BNN_ERR_DTYPE;
  if (m < 0 || n < 0 || k < 0 || n % 8 != 0 || k % 8 != 0) return BNN_ERR_SHAPE;
  if (!int_fits(m * k) || !int_fits(n * k) || !int_fits(m * n)) return BNN_ERR_SHAPE;
  if (n == 0 || k == 0) return BNN_OK;
  if (!grad_w || (m > 0 && (!grad_out || !x))) return BNN_ERR_NULL;
  if (!aligned(grad_w, 4)) return BNN_ERR_ALIGN;
  if (m > 0 && (!aligned(grad_out, 16) || !aligned(x, 16))) return BNN_ERR_ALIGN;
  return hip_status(bnn::launch_linear_grad_weight(grad_out, x, dtype == BNN_BF16, m, n, k,
                                                   scale_a, grad_w,
                                                   static_cast<hipStream_t>(stream)));
}

size_t bnn_linear_grad_weight_i8_workspace_bytes(int64_t n, int64_t k) {
  if (n <= 0 || k <= 0) return 0;
  return (size_t)bnn::bwd_grad_weight_i8_parts(n, k) * sizeof(float);
}

bnn_status bnn_linear_grad_weight_i8(const void* grad_out, const void* x, int dtype, int64_t m,
                                     int64_t n, int64_t k, float scale_a, float* grad_w,
                                     int8_t* grad_w_q, float* amax, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (!half_dtype(dtype)) return BNN_ERR_DTYPE;
  if (m < 0 || n < 0 || k < 0 || n % 8 != 0 || k % 8 != 0) return BNN_ERR_SHAPE;
  if (!int_fits(m * k) || !int_fits(n * k) || !int_fits(m * n)) return BNN_ERR_SHAPE;
  if (n == 0 || k == 0) return BNN_OK;
  if (!grad_w || !grad_w_q || !amax || (m > 0 && (!grad_out || !x))) return BNN_ERR_NULL;
  if (!aligned(grad_w, 16) || !aligned(grad_w_q, 4) || !aligned(amax, 4)) return BNN_ERR_ALIGN;
  if (m > 0 && (!aligned(grad_out, 16) || !aligned(x, 16))) return BNN_ERR_ALIGN;
  if (!workspace || workspace_bytes < bnn_linear_grad_weight_i8_workspace_bytes(n, k))
    return BNN_ERR_WORKSPACE;
  if (!aligned(workspace, 4)) return BNN_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e =
      bnn::launch_linear_grad_weight(grad_out, x, dtype == BNN_BF16, m, n, k, scale_a, grad_w, s);
  if (e != hipSuccess) return BNN_ERR_HIP;
  return hip_status(bnn::launch_quant_grad(grad_w, n * k, static_cast<float*>(workspace), amax,
                                           grad_w_q, s));
}

size_t bnn_quant_grad_i8_workspace_bytes(int64_t count) {
  if (count <= 0) return 0;
  return (size_t)bnn::bwd_quant_grad_parts(count) * sizeof(float);
}

bnn_status bnn_quant_grad_i8(const float* grad, int64_t count, int8_t* codes, float* amax,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (count < 0 || count % 4 != 0) return BNN_ERR_SHAPE;
  if (count == 0) return BNN_OK;
  if (!grad || !codes || !amax) return BNN_ERR_NULL;
  if (!aligned(grad, 16) || !aligned(codes, 4) || !aligned(amax, 4)) return BNN_ERR_ALIGN;
  if (!workspace || workspace_bytes < bnn_quant_grad_i8_workspace_bytes(count))
    return BNN_ERR_WORKSPACE;
  if (!aligned(workspace, 4)) return BNN_ERR_ALIGN;
  return hip_status(bnn::launch_quant_grad(grad, count, static_cast<float*>(workspace), amax,
                                           codes, static_cast<hipStream_t>(stream)));
}

// ---- conv backward (BinaryConv2dForward.backward)

}  // extern "C"

namespace {

// Geometry of the conv backward; BNN_OK when every size is usable: 16-bit dtype, positive sizes,
// a non-empty output, B*Ho*Wo and C*KH*KW multiples of 8 (16-byte operand loads), every count in
// int range.
struct ConvBwd {
  int geom[15];
  int64_t pixels, J, in_count;
};

bnn_status conv_bwd_geom(int64_t n, int64_t c, int64_t h, int64_t w, int64_t o, int kernel_h,
                         int kernel_w, int stride_h, int stride_w, int pad_h, int pad_w, int dil_h,
                         int dil_w, ConvBwd* q) {
  if (n < 1 || c < 1 || h < 1 || w < 1 || o < 1) return BNN_ERR_SHAPE;
  if (kernel_h < 1 || kernel_w < 1 || stride_h < 1 || stride_w < 1 || dil_h < 1 || dil_w < 1 ||
      pad_h < 0 || pad_w < 0)
    return BNN_ERR_SHAPE;
  const int64_t ho = out_size(h, kernel_h, stride_h, pad_h, dil_h);
  const int64_t wo = out_size(w, kernel_w, stride_w, pad_w, dil_w);
  if (ho <= 0 || wo <= 0) return BNN_ERR_SHAPE;
  const int64_t pixels = n * ho * wo, J = c * (int64_t)kernel_h * kernel_w;
  if (pixels % 8 != 0 || J % 8 != 0) return BNN_ERR_SHAPE;
  if (!int_fits(pixels) || !int_fits(J) || !int_fits(pixels * J) || !int_fits(o * pixels) ||
      !int_fits(n * c * h * w) || !int_fits(o * J) || !int_fits(h + 2 * (int64_t)pad_h) ||
      !int_fits(w + 2 * (int64_t)pad_w))
    return BNN_ERR_SHAPE;
  const int64_t vals[15] = {n, c, h, w, o, kernel_h, kernel_w, stride_h, stride_w, pad_h, pad_w,
                            dil_h, dil_w, ho, wo};
  for (int i = 0; i < 15; i++) q->geom[i] = (int)vals[i];
  q->pixels = pixels;
  q->J = J;
  q->in_count = n * c * h * w;
  return BNN_OK;
}

size_t round256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

extern "C" {

size_t bnn_conv2d_grad_input_workspace_bytes(int64_t n, int64_t c, int64_t h, int64_t w,
                                             int64_t out_channels, int kernel_h, int kernel_w,
                                             int stride_h, int stride_w, int pad_h, int pad_w,
                                             int dil_h, int dil_w) {
  ConvBwd q;
  if (conv_bwd_geom(n, c, h, w, out_channels, kernel_h, kernel_w, stride_h, stride_w, pad_h, pad_w,
                    dil_h, dil_w, &q) != BNN_OK)
    return 0;
  return round256((size_t)out_channels * q.pixels * 2) + round256((size_t)out_channels * q.J * 2) +
         round256((size_t)q.pixels * q.J * 4) +
         (size_t)bnn::conv_col2im_parts(n, c, h, w) * sizeof(double);
}

bnn_status bnn_conv2d_grad_input(const void* grad_out, const void* weight, const void* x,
                                 int dtype, int64_t n, int64_t c, int64_t h, int64_t w,
                                 int64_t out_channels, int kernel_h, int kernel_w, int stride_h,
                                 int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                                 float scale_a, float scale_w, float* grad_in,
                                 double* grad_scale_a, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (!half_dtype(dtype)) return BNN_ERR_DTYPE;
  ConvBwd q;
  const bnn_status st = conv_bwd_geom(n, c, h, w, out_channels, kernel_h, kernel_w, stride_h,
                                      stride_w, pad_h, pad_w, dil_h, dil_w, &q);
  if (st != BNN_OK) return st;
  if (!grad_out || !weight || !x || !grad_in || !grad_scale_a) return BNN_ERR_NULL;
  if (!aligned(grad_out, 2) || !aligned(weight, 16) || !aligned(x, 2) || !aligned(grad_in, 4) ||
      !aligned(grad_scale_a, 8))
    return BNN_ERR_ALIGN;
  const size_t need = bnn_conv2d_grad_input_workspace_bytes(n, c, h, w, out_channels, kernel_h,
                                                            kernel_w, stride_h, stride_w, pad_h,
                                                            pad_w, dil_h, dil_w);
  if (!workspace || workspace_bytes < need) return BNN_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return BNN_ERR_ALIGN;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint16_t* gT = reinterpret_cast<uint16_t*>(ws);
  uint8_t* at = ws + round256((size_t)out_channels * q.pixels * 2);
  uint16_t* wsign = reinterpret_cast<uint16_t*>(at);
  at += round256((size_t)out_channels * q.J * 2);
  float* cols = reinterpret_cast<float*>(at);
  double* part = reinterpret_cast<double*>(at + round256((size_t)q.pixels * q.J * 4));
  return hip_status(bnn::launch_conv_grad_input(grad_out, weight, x, dtype == BNN_BF16, q.geom,
                                                scale_a, scale_w, grad_in, gT, wsign, cols, part,
                                                grad_scale_a, static_cast<hipStream_t>(stream)));
}

size_t bnn_conv2d_grad_weight_workspace_bytes(int64_t n, int64_t c, int64_t h, int64_t w,
                                              int64_t out_channels, int kernel_h, int kernel_w,
                                              int stride_h, int stride_w, int pad_h, int pad_w,
                                              int dil_h, int dil_w) {
  ConvBwd q;
  if (conv_bwd_geom(n, c, h, w, out_channels, kernel_h, kernel_w, stride_h, stride_w, pad_h, pad_w,
                    dil_h, dil_w, &q) != BNN_OK)
    return 0;
  const int splits = bnn::conv_wgrad_splits(out_channels, q.J, q.pixels);
  return round256((size_t)out_channels * q.pixels * 2) + round256((size_t)q.pixels * q.J * 2) +
         (splits > 1 ? round256((size_t)splits * out_channels * q.J * 4) : 0) +
         (size_t)bnn::bwd_quant_grad_parts(out_channels * q.J) * sizeof(float);
}

bnn_status bnn_conv2d_grad_weight(const void* grad_out, const void* x, int dtype, int64_t n,
                                  int64_t c, int64_t h, int64_t w, int64_t out_channels,
                                  int kernel_h, int kernel_w, int stride_h, int stride_w,
                                  int pad_h, int pad_w, int dil_h, int dil_w, float scale_a,
                                  float* grad_w, int8_t* grad_w_q, float* amax, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (!half_dtype(dtype)) return BNN_ERR_DTYPE;
  ConvBwd q;
  const bnn_status st = conv_bwd_geom(n, c, h, w, out_channels, kernel_h, kernel_w, stride_h,
                                      stride_w, pad_h, pad_w, dil_h, dil_w, &q);
  if (st != BNN_OK) return st;
  if (!grad_out || !x || !grad_w) return BNN_ERR_NULL;
  if ((grad_w_q == nullptr) != (amax == nullptr)) return BNN_ERR_NULL;
  if (!aligned(grad_out, 2) || !aligned(x, 2) || !aligned(grad_w, 16)) return BNN_ERR_ALIGN;
  if (grad_w_q && (!aligned(grad_w_q, 4) || !aligned(amax, 4))) return BNN_ERR_ALIGN;
  const size_t need = bnn_conv2d_grad_weight_workspace_bytes(n, c, h, w, out_channels, kernel_h,
                                                             kernel_w, stride_h, stride_w, pad_h,
                                                             pad_w, dil_h, dil_w);
  if (!workspace || workspace_bytes < need) return BNN_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return BNN_ERR_ALIGN;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint16_t* gT = reinterpret_cast<uint16_t*>(ws);
  uint8_t* xc = ws + round256((size_t)out_channels * q.pixels * 2);
  const int splits = bnn::conv_wgrad_splits(out_channels, q.J, q.pixels);
  float* split_part = reinterpret_cast<float*>(xc + round256((size_t)q.pixels * q.J * 2));
  float* qpart = reinterpret_cast<float*>(
      reinterpret_cast<uint8_t*>(split_part) +
      (splits > 1 ? round256((size_t)splits * out_channels * q.J * 4) : 0));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = bnn::launch_conv_grad_weight(grad_out, x, dtype == BNN_BF16, q.geom, scale_a,
                                                    grad_w, gT, reinterpret_cast<uint16_t*>(xc),
                                                    split_part, s);
  if (e != hipSuccess) return BNN_ERR_HIP;
  if (!grad_w_q) return BNN_OK;
  return hip_status(bnn::launch_quant_grad(grad_w, out_channels * q.J, qpart, amax, grad_w_q, s));
}

}  // extern "C"

namespace {
bnn_status gemm_impl(const void* x, int x_dtype, const uint32_t* w_packed, int64_t m, int64_t n,
                     int64_t k, double scale_a, double scale_w, int path, void* out,
                     int out_dtype, void* workspace, size_t workspace_bytes, bool use_scratch,
                     void* stream) {
  if (!(float_dtype(x_dtype) || packed_dtype(x_dtype)) || !out_dtype_ok(out_dtype))
    return BNN_ERR_DTYPE;
  if (m < 0 || n < 0 || k < 1) return BNN_ERR_SHAPE;
  if (!int_fits(m) || !int_fits(n) || !bits_fit(k)) return BNN_ERR_SHAPE;
  if (!path_known(path)) return BNN_ERR_PATH;
  if (path == BNN_PATH_MFMA_FP4 && k > bnn::kMaxFp4K) return BNN_ERR_PATH;
  if (m == 0 || n == 0) return BNN_OK;
  if (!x || !w_packed || !out) return BNN_ERR_NULL;
  const bool words_in = x_dtype == BNN_U32_PACKED || u8_in_place(x_dtype, k);
  const int x_align = words_in ? 4 : x_dtype == BNN_U8_PACKED ? 1 : elem_bytes(x_dtype);
  if (!aligned(x, x_align) || !aligned(w_packed, 4) || !aligned(out, 16)) return BNN_ERR_ALIGN;
  const size_t need = bnn_gemm_workspace_bytes(m, k, x_dtype);
  if (use_scratch) {
    // every argument is checked by now; resolving the scratch address enqueues nothing
    if (need > kScratchBytes) return BNN_ERR_WORKSPACE;
    if (need > 0) {
      const bnn_status st = scratch_of_current_device(&workspace);
      if (st != BNN_OK) return st;
      workspace_bytes = kScratchBytes;
    }
  }
  if (need > 0 && (!workspace || workspace_bytes < need)) return BNN_ERR_WORKSPACE;
  if (need > 0 && !aligned(workspace, 4)) return BNN_ERR_ALIGN;

  const int use = path == BNN_PATH_AUTO ? auto_path(k) : path;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint32_t* a = static_cast<const uint32_t*>(x);
  if (!words_in) {
    uint32_t* ws = static_cast<uint32_t*>(workspace);
    const hipError_t e =
        x_dtype == BNN_U8_PACKED
            ? bnn::launch_u8_to_words(static_cast<const uint8_t*>(x), m, k, ws, s)
            : pack_rows_any(x, x_dtype, m, k, nullptr, 0, false, ws, s);
    if (e != hipSuccess) return BNN_ERR_HIP;
    a = ws;
  }
  bnn::Contraction p{};
  p.a = a;
  p.w = w_packed;
  p.out = out;
  p.M = (int)m;
  p.N = (int)n;
  p.KW = (int)words_of(k);
  p.KB = (int)k;
  p.alpha = alpha_of(scale_a, scale_w);
  const hipError_t e = run_path(use, p, false, out_dtype, s);
  if (e != hipSuccess) return BNN_ERR_HIP;
  g_last_path = use;
  return BNN_OK;
}

}  // namespace
