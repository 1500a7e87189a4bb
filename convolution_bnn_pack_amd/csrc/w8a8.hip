// W8A8 conv on the gfx950 matrix cores: the im2col + GEMM lowering with INT8 quantizers
// (banghao.live blog post, section 3, "Add INT8-quantizer to im2col+gemm"), computed
// implicitly.
//
// Quantizer (a reading: the page names input and weight quantizers without defining
// them): per-tensor symmetric 8-bit with a given amax, step = amax / 127 in fp32 and
// code = clamp(rint(v / step), -127, 127) with a correctly rounded fp32 division and
// round-half-to-even; NaN codes as 0. The fake-quantized product of the page equals
// step_x * step_w * sum(q_x * q_w), so the contraction runs on int8 codes with int32 sums
// and the epilogue scales once.
//
// Layouts: activations NHWC int8 [N][H][W][C] (a conv tap reads C contiguous codes),
// weights [O][KH][KW][C] int8, so reduction byte r = tap * C + c of a weight row is plain
// row-major. C must be a multiple of 16, so a 16-byte chunk of the reduction never leaves
// its tap; padded taps load zeros.
#include <type_traits>

#include "launch.h"

namespace bnn {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int8_t quant_code(float v, float step) {
  if (v != v) return 0;
  float r = rintf(v / step);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (int8_t)(int)r;
}

template <int DT>
__device__ __forceinline__ float load_f32(const void* base, int64_t i) {
  if constexpr (DT == kF32)
    return reinterpret_cast<const float*>(base)[i];
  else if constexpr (DT == kF16)
    return __half2float(reinterpret_cast<const __half*>(base)[i]);
  else
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(base)[i] << 16);
}

// NCHW float -> NHWC int8 codes. A 256-thread workgroup takes 64 pixels (of the flattened
// batch x plane axis) x 64 channels: threads read along pixels (coalesced per channel
// plane), codes meet in LDS as [pixel][channel], and each pixel's 64 channel codes leave
// as one contiguous run.
template <int DT>
__global__ __launch_bounds__(256) void quant_nhwc_kernel(const void* __restrict__ x,
                                                         int8_t* __restrict__ out, int C, int HW,
                                                         int P, float step) {
  __shared__ int8_t tile[64][64 + 4];
  const int p0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // pixel lane, channel group
  const int p = p0 + tx;
  // all 16 loads go out before any is used: addresses clamped into the tensor (the last pixel
  // or channel), the codes of clamped elements replaced by 0 afterwards (a load behind a
  // branch is waited for on the spot)
  const int pc = p < P ? p : P - 1;
  const int b = pc / HW, pix = pc - b * HW;
  float v[16];
#pragma unroll
  for (int k = 0; k < 16; k++) {
    const int c = c0 + ty + 4 * k;
    v[k] = load_f32<DT>(x, ((int64_t)b * C + (c < C ? c : C - 1)) * HW + pix);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < 16; k++) {
    const int cl = ty + 4 * k;
    tile[tx][cl] = (p < P && c0 + cl < C) ? quant_code(v[k], step) : 0;
  }
  __syncthreads();
  // write: thread -> (pixel row, 16-byte column); 64 pixels x 4 columns = 256 stores
  const int pr = threadIdx.x >> 2, col = (threadIdx.x & 3) * 16;
  const int pw = p0 + pr;
  if (pw < P) {
    int8_t* dst = out + (int64_t)pw * C + c0 + col;
    if (c0 + col + 16 <= C) {
      uint32_t v[4];
#pragma unroll
      for (int i = 0; i < 4; i++)
        v[i] = (uint32_t)(uint8_t)tile[pr][col + 4 * i] | ((uint32_t)(uint8_t)tile[pr][col + 4 * i + 1] << 8) |
               ((uint32_t)(uint8_t)tile[pr][col + 4 * i + 2] << 16) |
               ((uint32_t)(uint8_t)tile[pr][col + 4 * i + 3] << 24);
      *reinterpret_cast<uint4*>(dst) = make_uint4(v[0], v[1], v[2], v[3]);
    } else {
      for (int i = 0; i < 16 && c0 + col + i < C; i++) dst[i] = tile[pr][col + i];
    }
  }
}

// OIHW float -> [O][KH][KW][C] int8 codes, one thread per code (run once per layer).
template <int DT>
__global__ __launch_bounds__(256) void quant_weight_kernel(const void* __restrict__ w,
                                                           int8_t* __restrict__ out,
                                                           int64_t total, int C, int T,
                                                           float step) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int c = (int)(idx % C);
  const int64_t ot = idx / C;  // o * T + t
  const int t = (int)(ot % T);
  const int64_t o = ot / T;
  out[idx] = quant_code(load_f32<DT>(w, (o * C + c) * T + t), step);
}

// Implicit-im2col int8 contraction. Tile 128 output pixels x BN (128 or 256) output channels,
// eight waves in a 2 x 4 grid (two per SIMD), each a 64 x BN/4 sub-tile of 2 x BN/128 blocks of
// v_mfma_i32_32x32x32_i8. A stage is 128 reduction bytes (four MFMA k-steps): the A tile
// (pixels) and the W tile (channels) are loaded as 16-byte chunks into registers, written
// to one of two LDS buffers (rows padded to 144 bytes to spread the banks), and consumed
// after one barrier while the next stage's chunks are in flight. The MFMA computes
// D = A * W^T, so a lane's four consecutive accumulators are four consecutive pixels of
// one output channel (as in the binary conv tiles).
constexpr int kBM = 128, kSK = 128, kRow = kSK + 16;
constexpr int kThreads = 512, kWGM = 2, kWGN = 4;              // wave grid
constexpr int kWTM = kBM / kWGM;                               // wave sub-tile rows
constexpr int kFM = kWTM / 32;                                 // MFMA blocks per wave along pixels
constexpr int kCPR = kSK / 16;                                 // 16-byte chunks per row and stage
// Output channels per tile: BN = 256 (64 x 64 per wave, 2 x 2 blocks: 4 fragment reads per 4
// MFMAs) when the layer has more than 128 output channels, else 128 (64 x 32, 3 reads per 2).
// Loader split: every thread takes LPT consecutive chunks of one row of A (BM rows) and of W
// (BN rows) per stage.
template <int BN>
struct W8Tile {
  static constexpr int WTN = BN / kWGN, FN = WTN / 32;
  static constexpr int LPTA = kCPR * kBM / kThreads, TPRA = kCPR / LPTA;
  static constexpr int LPTW = kCPR * BN / kThreads, TPRW = kCPR / LPTW;
  static_assert(LPTA * TPRA == kCPR && TPRA * kBM == kThreads && LPTW * TPRW == kCPR &&
                    TPRW * BN == kThreads, "loader split");
};

struct W8A8Conv {
  const int8_t* a;  // NHWC codes
  const int8_t* w;  // [O][K] codes
  void* out;        // NCHW
  int M, N, K, C, H, W, Ho, Wo, KWD, SH, SW, PH, PW, DH, DW;
  float alpha;
  FastDiv div_c, div_kwd, div_hw, div_wo;  // by C, the kernel width, Ho*Wo and Wo
};

template <int OUT, int BN>
__global__ __launch_bounds__(kThreads) void w8a8_conv_kernel(W8A8Conv p) {
  using TL = W8Tile<BN>;
  constexpr int kBN = BN, kWTN = TL::WTN, kFN = TL::FN, LA = TL::LPTA, LW = TL::LPTW;
  __shared__ __attribute__((aligned(16))) int8_t lds[2][(kBM + kBN) * kRow];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % kWGM, wn = wave / kWGM;
  const int tiles_n = (p.N + kBN - 1) / kBN;
  const int m0 = (blockIdx.x / tiles_n) * kBM, n0 = (blockIdx.x % tiles_n) * kBN;

  // loaders: chunks ljA .. ljA + LA - 1 of A row lrowA, chunks ljW .. ljW + LW - 1 of W row lrowW
  const int lrowA = tid / TL::TPRA, ljA = (tid % TL::TPRA) * LA;
  const int lrowW = tid / TL::TPRW, ljW = (tid % TL::TPRW) * LW;
  const int am = m0 + lrowA, wnr = n0 + lrowW;
  const bool amok = am < p.M, wnok = wnr < p.N;
  // image and top-left input coordinate of this A row (row 0's for rows past M)
  const int hw = p.Ho * p.Wo;
  const int ab = p.div_hw.div(amok ? am : 0);
  const int ar = (amok ? am : 0) - ab * hw;
  const int aoh = p.div_wo.div(ar), aow = ar - aoh * p.Wo;
  const int aih = aoh * p.SH - p.PH, aiw = aow * p.SW - p.PW;
  const int8_t* wrow = p.w + (int64_t)(wnok ? wnr : 0) * p.K;
  // Every chunk is loaded unconditionally from an address clamped into the tensor (chunk 0 of
  // the pixel or weight row) and its validity kept beside it; the zeroing waits for the store
  // to LDS a stage later. A load behind a branch makes the compiler wait for all loads at the
  // next use (it can no longer count them), which would drain the prefetch every stage.
  auto load_stage = [&](int s, uint4 (&ra)[LA], uint4 (&rw)[LW], bool (&oa)[LA],
                        bool (&ow)[LW]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LA; i++) {
      const int r0 = s * kSK + 16 * (ljA + i);
      const bool kin = r0 < p.K;
      const int rk = kin ? r0 : 0;
      const int tap = p.div_c.div(rk), c = rk - tap * p.C;
      const int kh = p.div_kwd.div(tap), kw = tap - kh * p.KWD;
      const int ih = aih + kh * p.DH, iw = aiw + kw * p.DW;
      oa[i] = kin && amok && ih >= 0 && ih < p.H && iw >= 0 && iw < p.W;
      const int64_t aoff = oa[i] ? (((int64_t)ab * p.H + ih) * p.W + iw) * p.C + c : 0;
      ra[i] = *reinterpret_cast<const uint4*>(p.a + aoff);
    }
#pragma unroll
    for (int i = 0; i < LW; i++) {
      const int r0 = s * kSK + 16 * (ljW + i);
      const bool kin = r0 < p.K;
      ow[i] = kin && wnok;
      rw[i] = *reinterpret_cast<const uint4*>(wrow + (kin ? r0 : 0));
    }
  };
  auto store_stage = [&](int buf, const uint4 (&ra)[LA], const uint4 (&rw)[LW],
                         const bool (&oa)[LA], const bool (&ow)[LW]) __attribute__((always_inline)) {
    // masks rather than a select of whole vectors (which the compiler turns into a select of
    // addresses and a round trip through scratch memory)
#pragma unroll
    for (int i = 0; i < LA; i++) {
      const uint32_t ma = oa[i] ? ~0u : 0u;
      *reinterpret_cast<uint4*>(&lds[buf][lrowA * kRow + 16 * (ljA + i)]) =
          make_uint4(ra[i].x & ma, ra[i].y & ma, ra[i].z & ma, ra[i].w & ma);
    }
#pragma unroll
    for (int i = 0; i < LW; i++) {
      const uint32_t mw = ow[i] ? ~0u : 0u;
      *reinterpret_cast<uint4*>(&lds[buf][(kBM + lrowW) * kRow + 16 * (ljW + i)]) =
          make_uint4(rw[i].x & mw, rw[i].y & mw, rw[i].z & mw, rw[i].w & mw);
    }
  };

  v16i acc[kFN][kFM];
#pragma unroll
  for (int i = 0; i < kFN; i++)
#pragma unroll
    for (int j = 0; j < kFM; j++)
#pragma unroll
      for (int e = 0; e < 16; e++) acc[i][j][e] = 0;

  const int fr = lane & 31, half = lane >> 5;
  const int nstages = (p.K + kSK - 1) / kSK;
  // raw chunks two stages ahead: stage t is fetched into register set t % 2 two stages
  // before its MFMAs, and stored to LDS buffer t % 2 right after the MFMAs of stage t - 1
  uint4 ra[2][LA], rw[2][LW];
  bool oa[2][LA], ow[2][LW];
  auto compute = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < kSK / 32; kk++) {
      v4i fa[kFM], fw[kFN];
#pragma unroll
      for (int f = 0; f < kFM; f++)
        fa[f] = *reinterpret_cast<const v4i*>(&lds[buf][(wm * kWTM + f * 32 + fr) * kRow + 16 * (2 * kk + half)]);
#pragma unroll
      for (int f = 0; f < kFN; f++)
        fw[f] = *reinterpret_cast<const v4i*>(&lds[buf][(kBM + wn * kWTN + f * 32 + fr) * kRow + 16 * (2 * kk + half)]);
#pragma unroll
      for (int fn = 0; fn < kFN; fn++)
#pragma unroll
        for (int fm = 0; fm < kFM; fm++)
          acc[fn][fm] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[fm], fw[fn], acc[fn][fm], 0, 0, 0);
    }
  };
  // one stage: fetch stage s + 2 into set PH (stage s's set, already in LDS), run stage s from
  // buffer PH, store stage s + 1 (set PH ^ 1) into buffer PH ^ 1; PH = s % 2 at compile time
  auto stage = [&](auto phase, int s) __attribute__((always_inline)) {
    constexpr int PH = decltype(phase)::value;
    // past the last stage the loads fetch clamped, invalid chunks that are never stored
    load_stage(s + 2, ra[PH], rw[PH], oa[PH], ow[PH]);
    compute(PH);
    if (s + 1 < nstages) store_stage(PH ^ 1, ra[PH ^ 1], rw[PH ^ 1], oa[PH ^ 1], ow[PH ^ 1]);
    __syncthreads();
  };
  load_stage(0, ra[0], rw[0], oa[0], ow[0]);
  load_stage(1, ra[1], rw[1], oa[1], ow[1]);
  store_stage(0, ra[0], rw[0], oa[0], ow[0]);
  __syncthreads();
  int s = 0;
  for (; s + 2 <= nstages; s += 2) {
    stage(std::integral_constant<int, 0>{}, s);
    stage(std::integral_constant<int, 1>{}, s + 1);
  }
  if (s < nstages) stage(std::integral_constant<int, 0>{}, s);

  // epilogue: lane (fr, half) holds channel n = n0 + wn*kWTN + fn*32 + fr and, in e = 4g..4g+3,
  // the pixels m = m0 + wm*kWTM + fm*32 + 8g + 4*half + 0..3
#pragma unroll
  for (int fn = 0; fn < kFN; fn++) {
    const int n = n0 + wn * kWTN + fn * 32 + fr;
    if (n >= p.N) continue;
#pragma unroll
    for (int fm = 0; fm < kFM; fm++)
#pragma unroll
      for (int g = 0; g < 4; g++) {
        const int m = m0 + wm * kWTM + fm * 32 + 8 * g + 4 * half;
        if (m >= p.M) continue;
        const int b = p.div_hw.div(m), pix = m - b * hw;
        const int v0 = acc[fn][fm][4 * g], v1 = acc[fn][fm][4 * g + 1];
        const int v2 = acc[fn][fm][4 * g + 2], v3 = acc[fn][fm][4 * g + 3];
        if ((hw & 3) == 0) {
          store4<OUT>(p.out, ((int64_t)b * p.N + n) * hw + pix, v0, v1, v2, v3, p.alpha);
        } else {
          const int vals[4] = {v0, v1, v2, v3};
          int bi = b, pi = pix;
#pragma unroll
          for (int i = 0; i < 4; i++) {
            if (m + i >= p.M) break;
            store1<OUT>(p.out, ((int64_t)bi * p.N + n) * hw + pi, vals[i], p.alpha);
            if (++pi == hw) {
              pi = 0;
              ++bi;
            }
          }
        }
      }
  }
}

}  // namespace

hipError_t launch_quant_nhwc(const void* x, int dtype, int64_t n, int64_t c, int64_t h, int64_t w,
                             float step, int8_t* out, hipStream_t stream) {
  const int64_t P = n * h * w;
  if (P == 0 || c == 0) return hipSuccess;
  const dim3 grid((unsigned)((P + 63) / 64), (unsigned)((c + 63) / 64)), block(256);
  switch (dtype) {
    case kF32: hipLaunchKernelGGL(quant_nhwc_kernel<kF32>, grid, block, 0, stream, x, out, (int)c, (int)(h * w), (int)P, step); break;
    case kF16: hipLaunchKernelGGL(quant_nhwc_kernel<kF16>, grid, block, 0, stream, x, out, (int)c, (int)(h * w), (int)P, step); break;
    default: hipLaunchKernelGGL(quant_nhwc_kernel<kBF16>, grid, block, 0, stream, x, out, (int)c, (int)(h * w), (int)P, step); break;
  }
  return hipGetLastError();
}

hipError_t launch_quant_weight(const void* w, int dtype, int64_t o, int64_t c, int kh, int kw,
                               float step, int8_t* out, hipStream_t stream) {
  const int64_t total = o * kh * kw * c;
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
  const int T = kh * kw;
  switch (dtype) {
    case kF32: hipLaunchKernelGGL(quant_weight_kernel<kF32>, grid, block, 0, stream, w, out, total, (int)c, T, step); break;
    case kF16: hipLaunchKernelGGL(quant_weight_kernel<kF16>, grid, block, 0, stream, w, out, total, (int)c, T, step); break;
    default: hipLaunchKernelGGL(quant_weight_kernel<kBF16>, grid, block, 0, stream, w, out, total, (int)c, T, step); break;
  }
  return hipGetLastError();
}

template <int BN>
hipError_t launch_w8a8_t(const W8A8Conv& p, int out_dtype, hipStream_t stream) {
  const int64_t tiles = (int64_t)((p.M + kBM - 1) / kBM) * ((p.N + BN - 1) / BN);
  const dim3 grid((unsigned)tiles), block(kThreads);
  switch (out_dtype) {
    case kF32: hipLaunchKernelGGL((w8a8_conv_kernel<kF32, BN>), grid, block, 0, stream, p); break;
    case kF16: hipLaunchKernelGGL((w8a8_conv_kernel<kF16, BN>), grid, block, 0, stream, p); break;
    case kBF16: hipLaunchKernelGGL((w8a8_conv_kernel<kBF16, BN>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((w8a8_conv_kernel<kI32, BN>), grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_w8a8_conv(const int8_t* xq, const int8_t* wq, void* out, int out_dtype,
                            int64_t n, int64_t c, int64_t h, int64_t w, int64_t o, int64_t ho,
                            int64_t wo, int kh, int kw, int sh, int sw, int ph, int pw, int dh,
                            int dw, float alpha, hipStream_t stream) {
  W8A8Conv p{};
  p.a = xq;
  p.w = wq;
  p.out = out;
  p.M = (int)(n * ho * wo);
  p.N = (int)o;
  p.K = (int)(kh * kw * c);
  p.C = (int)c;
  p.H = (int)h;
  p.W = (int)w;
  p.Ho = (int)ho;
  p.Wo = (int)wo;
  p.KWD = kw;
  p.SH = sh;
  p.SW = sw;
  p.PH = ph;
  p.PW = pw;
  p.DH = dh;
  p.DW = dw;
  p.alpha = alpha;
  p.div_c = FastDiv((uint32_t)c);
  p.div_kwd = FastDiv((uint32_t)kw);
  p.div_hw = FastDiv((uint32_t)(ho * wo));
  p.div_wo = FastDiv((uint32_t)wo);
  if (p.M == 0 || p.N == 0) return hipSuccess;
  // 256-wide tiles when they fill at most one round of the 256 compute units (one workgroup
  // each: 108 KiB of LDS); with more tiles the 128-wide ones, two per compute unit, balance
  // better (measured on the 128 x 128 x 28 x 28 -> 256 layers: strided 20.0 -> 19.0 us with 256,
  // dilated 60.6 -> 66 us)
  const int64_t tiles256 = (int64_t)((p.M + kBM - 1) / kBM) * ((p.N + 255) / 256);
  return p.N > 128 && tiles256 <= 256 ? launch_w8a8_t<256>(p, out_dtype, stream)
                                      : launch_w8a8_t<128>(p, out_dtype, stream);
}

}  // namespace bnn
