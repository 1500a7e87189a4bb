// +-1-as-int8 binary contraction on the gfx950 matrix cores.
//
// The binary dot product is a dense contraction, so it can run on
// v_mfma_i32_32x32x32_i8 (32x32 output, 32-deep reduction, int32 sums).
// Signs stay bit-packed in HBM (one bit per element); a workgroup loads the
// packed words of its A and W tiles and expands each word in registers to
// 32 int8 values before storing them to LDS:
//
//   v_perm_b32 with selector bytes 8..11 replicates bits 15 and 31 of each of
//   its two sources into whole bytes (0x00 or 0xFF). With the sources w << 2d
//   and w << 2d+1 (d = 0..7) every bit of w lands in exactly one byte; OR-ing
//   0x01 turns 0xFF into -1 and 0x00 into +1. That maps a set bit (+1) to -1
//   and a clear bit to +1, i.e. both operands are negated, which leaves every
//   product unchanged. The byte order within a word is a fixed permutation
//   of its 32 reduction indices, the same for A and W, so the sums are the
//   binary dot products exactly. A padded conv tap expands to 0 bytes, so it
//   contributes 0 with no correction.
//
// Tiling: a 256-thread workgroup owns a 128 (rows of A) x 128 (rows of W)
// output tile and walks the reduction 4 words (128 signs) at a time. Each
// of its four waves computes a 64 x 64 sub-tile as 2 x 2 MFMA blocks. The
// MFMA computes D = W_tile * A_tile^T so that each lane's four consecutive
// accumulators are four consecutive output features of one row: linear
// outputs leave as 16-byte (f32) or 8-byte (f16/bf16) vector stores, conv
// outputs as lane-contiguous NCHW runs. LDS rows are 128 bytes; their 16-byte
// chunks are XOR-swizzled by (row >> 1) & 7 so the ds_read_b128 fragment
// reads of 16 consecutive rows hit distinct banks.
//
// Conv uses the same implicit im2col map as the XOR path (banghao.live blog
// post, section 2, lowered without materialising the column matrix).
#include "launch.h"

namespace bnn {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BKW = 4, ROWB = BKW * 32;  // bytes per LDS row

struct PixelCoord {
  int b, ihb, iwb;
};

__device__ __forceinline__ PixelCoord pixel_coord(const Contraction& p, int m) {
  const int hw = p.Ho * p.Wo;
  const int b = m / hw;
  const int r = m - b * hw;
  const int oh = r / p.Wo;
  const int ow = r - oh * p.Wo;
  return {b, oh * p.stride - p.pad, ow * p.stride - p.pad};
}

// Words q0..q0+3 of one tile row plus a validity flag per word (invalid: outside
// the matrix, past K, or a padded conv tap).
template <bool CONV, bool IS_A>
__device__ __forceinline__ void load_row4(const Contraction& p, int row, const PixelCoord& pc,
                                          int q0, uint32_t r[4], bool ok[4]) {
  if constexpr (!CONV || !IS_A) {
    const uint32_t* src = IS_A ? p.a : p.w;
    const int rows = IS_A ? p.M : p.N;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int q = q0 + i;
      ok[i] = row < rows && q < p.KW;
      r[i] = ok[i] ? src[(int64_t)row * p.KW + q] : 0u;
    }
  } else {
    int tap = q0 / p.CW;
    int cw = q0 - tap * p.CW;
    int kh = tap / p.ks;
    int kw = tap - kh * p.ks;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int q = q0 + i;
      const int ih = pc.ihb + kh * p.dil, iw = pc.iwb + kw * p.dil;
      ok[i] = row < p.M && q < p.KW && ih >= 0 && ih < p.H && iw >= 0 && iw < p.W;
      r[i] = ok[i] ? p.a[(((int64_t)pc.b * p.H + ih) * p.W + iw) * p.CW + cw] : 0u;
      if (++cw == p.CW) {
        cw = 0;
        if (++kw == p.ks) {
          kw = 0;
          ++kh;
        }
      }
    }
  }
}

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// Expand 4 packed words of one row to 128 int8 +-1 bytes (0 bytes for invalid
// words) and store them to the row's LDS line. Word i fills reduction chunk i
// (32 bytes = 16-byte halves 2i and 2i+1).
__device__ __forceinline__ void expand_store(uint8_t* line, int row, const uint32_t r[4],
                                             const bool ok[4]) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const uint32_t w = r[i];
    const uint32_t keep = ok[i] ? 0xFFFFFFFFu : 0u;
    const uint32_t ones = ok[i] ? 0x01010101u : 0u;
    uint32_t y[8];
#pragma unroll
    for (int d = 0; d < 8; d++) {
      const uint32_t m = __builtin_amdgcn_perm(w << (2 * d + 1), w << (2 * d), 0x0B0A0908u);
      y[d] = (m & keep) | ones;
    }
    *reinterpret_cast<uint4*>(line + 16 * swz(row, 2 * i)) = make_uint4(y[0], y[1], y[2], y[3]);
    *reinterpret_cast<uint4*>(line + 16 * swz(row, 2 * i + 1)) = make_uint4(y[4], y[5], y[6], y[7]);
  }
}

template <int OUT, bool CONV>
__global__ __launch_bounds__(256) void mfma_kernel(Contraction p) {
  __shared__ __attribute__((aligned(16))) uint8_t As[BM * ROWB];
  __shared__ __attribute__((aligned(16))) uint8_t Ws[BN * ROWB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int tiles_n = (p.N + BN - 1) / BN;
  const int m0 = (blockIdx.x / tiles_n) * BM;
  const int n0 = (blockIdx.x % tiles_n) * BN;

  // loader role: threads 0..127 expand A row tid, threads 128..255 W row tid-128
  const bool is_a = tid < BM;
  const int lrow = is_a ? tid : tid - BM;
  const int grow = is_a ? m0 + lrow : n0 + lrow;
  uint8_t* line = (is_a ? As : Ws) + lrow * ROWB;
  PixelCoord pc{0, 0, 0};
  if constexpr (CONV) {
    if (is_a && grow < p.M) pc = pixel_coord(p, grow);
  }

  uint32_t r[4];
  bool ok[4];
  if (is_a)
    load_row4<CONV, true>(p, grow, pc, 0, r, ok);
  else
    load_row4<CONV, false>(p, grow, pc, 0, r, ok);

  v16i acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int e = 0; e < 16; e++) acc[i][j][e] = 0;

  const int fr = lane & 31, half = lane >> 5;
  for (int kt = 0; kt < p.KW; kt += BKW) {
    __syncthreads();
    expand_store(line, lrow, r, ok);
    __syncthreads();
    if (kt + BKW < p.KW) {
      if (is_a)
        load_row4<CONV, true>(p, grow, pc, kt + BKW, r, ok);
      else
        load_row4<CONV, false>(p, grow, pc, kt + BKW, r, ok);
    }
#pragma unroll
    for (int kk = 0; kk < BKW; kk++) {
      v4i fa[2], fw[2];
#pragma unroll
      for (int f = 0; f < 2; f++) {
        const int ra = wm * 64 + f * 32 + fr;
        const int rw = wn * 64 + f * 32 + fr;
        fa[f] = *reinterpret_cast<const v4i*>(As + ra * ROWB + 16 * swz(ra, 2 * kk + half));
        fw[f] = *reinterpret_cast<const v4i*>(Ws + rw * ROWB + 16 * swz(rw, 2 * kk + half));
      }
#pragma unroll
      for (int fn = 0; fn < 2; fn++)
#pragma unroll
        for (int fm = 0; fm < 2; fm++)
          acc[fn][fm] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fw[fn], fa[fm], acc[fn][fm], 0, 0, 0);
    }
  }

  // epilogue: acc[fn][fm][e] is output (row m, feature n) with
  //   m = m0 + wm*64 + fm*32 + (lane & 31)
  //   n = n0 + wn*64 + fn*32 + 8*(e/4) + 4*(lane/32) + e%4
  const int hw = CONV ? p.Ho * p.Wo : 1;
#pragma unroll
  for (int fm = 0; fm < 2; fm++) {
    const int m = m0 + wm * 64 + fm * 32 + fr;
    if (m >= p.M) continue;
    int b = 0, pix = 0;
    if constexpr (CONV) {
      b = m / hw;
      pix = m - b * hw;
    }
#pragma unroll
    for (int fn = 0; fn < 2; fn++) {
#pragma unroll
      for (int g = 0; g < 4; g++) {
        const int n = n0 + wn * 64 + fn * 32 + 8 * g + 4 * half;
        const int a0 = acc[fn][fm][4 * g], a1 = acc[fn][fm][4 * g + 1];
        const int a2 = acc[fn][fm][4 * g + 2], a3 = acc[fn][fm][4 * g + 3];
        if constexpr (!CONV) {
          const int64_t base = (int64_t)m * p.N + n;
          if (n + 3 < p.N && (p.N & 3) == 0) {
            store4<OUT>(p.out, base, a0, a1, a2, a3, p.alpha);
          } else {
            const int av[4] = {a0, a1, a2, a3};
#pragma unroll
            for (int j = 0; j < 4; j++)
              if (n + j < p.N) store1<OUT>(p.out, base + j, av[j], p.alpha);
          }
        } else {
          const int av[4] = {a0, a1, a2, a3};
#pragma unroll
          for (int j = 0; j < 4; j++)
            if (n + j < p.N) store1<OUT>(p.out, ((int64_t)b * p.N + n + j) * hw + pix, av[j], p.alpha);
        }
      }
    }
  }
}

template <bool CONV>
hipError_t launch_mfma_t(const Contraction& p, int out_dtype, hipStream_t stream) {
  const int64_t tiles = (int64_t)((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  const dim3 grid((unsigned)tiles), block(256);
  switch (out_dtype) {
    case kF32: hipLaunchKernelGGL((mfma_kernel<kF32, CONV>), grid, block, 0, stream, p); break;
    case kF16: hipLaunchKernelGGL((mfma_kernel<kF16, CONV>), grid, block, 0, stream, p); break;
    case kBF16: hipLaunchKernelGGL((mfma_kernel<kBF16, CONV>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((mfma_kernel<kI32, CONV>), grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma(const Contraction& p, bool conv, int out_dtype, hipStream_t stream) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  return conv ? launch_mfma_t<true>(p, out_dtype, stream) : launch_mfma_t<false>(p, out_dtype, stream);
}

}  // namespace bnn
