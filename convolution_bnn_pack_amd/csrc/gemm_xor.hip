// XOR + popcount binary contraction on the vector ALUs (gfx950).
//
// dot(a, w) over K signs packed in words = K - 2 * sum_q popcount(a_q ^ w_q):
// one v_xor_b32 and one v_bcnt_u32_b32 (which also adds) per 32 MACs.
//
// Tiling: a 256-thread workgroup owns a 128 x 128 output tile and walks the
// reduction 8 words (256 signs) at a time through LDS, stored k-major so a
// thread reads its 8 row words and 8 column words with four ds_read_b128.
// Each thread accumulates an 8 x 8 micro-tile: per word 16 LDS dwords feed
// 128 VALU ops. The next tile's global words are fetched into registers
// while the current one is consumed.
//
// Conv (implicit im2col, the lowering of the banghao.live blog post,
// section 2, without materialising the column matrix): row m of A is output
// pixel (b, oh, ow) and reduction word q = tap * CW + cw reads activation
// word [b][oh*s - p + kh*d][ow*s - p + kw*d][cw]. A padded tap is loaded as
// the word 0, which adds popcount(w) for that tap; the epilogue subtracts it
// again (per-tap weight popcounts kept in LDS) and uses the pixel's real
// reduction length K_valid = C * (valid taps), so padded taps contribute
// exactly 0. A reduction length (K, or C per tap) that is not a whole number
// of words leaves zero bits at the top of the last word in both operands:
// their XOR adds nothing, and the true length enters only through K / C.
#include "launch.h"

namespace bnn {
namespace {

constexpr int BM = 128, BN = 128, BKW = 8, MAX_TAPS = 49;

struct PixelCoord {
  int b, ihb, iwb;  // image, top-left input coordinate of the receptive field
};

__device__ __forceinline__ PixelCoord pixel_coord(const Contraction& p, int m) {
  const int hw = p.Ho * p.Wo;
  const int b = p.div_hw.div(m);
  const int r = m - b * hw;
  const int oh = p.div_wo.div(r);
  const int ow = r - oh * p.Wo;
  return {b, oh * p.SH - p.PH, ow * p.SW - p.PW};
}

// Load 4 consecutive reduction words q0..q0+3 of A row m (0 outside the matrix or for padded taps).
template <bool CONV>
__device__ __forceinline__ void load_a4(const Contraction& p, int m, const PixelCoord& pc, int q0,
                                        uint32_t r[4]) {
  if constexpr (!CONV) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int q = q0 + i;
      r[i] = (m < p.M && q < p.KW) ? p.a[(int64_t)m * p.KW + q] : 0u;
    }
  } else {
    int tap = p.div_cw.div(q0);
    int cw = q0 - tap * p.CW;
    int kh = p.div_kwd.div(tap);
    int kw = tap - kh * p.KWD;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int q = q0 + i;
      const int ih = pc.ihb + kh * p.DH, iw = pc.iwb + kw * p.DW;
      const bool ok = m < p.M && q < p.KW && ih >= 0 && ih < p.H && iw >= 0 && iw < p.W;
      r[i] = ok ? p.a[(((int64_t)pc.b * p.H + ih) * p.W + iw) * p.CW + cw] : 0u;
      if (++cw == p.CW) {
        cw = 0;
        if (++kw == p.KWD) {
          kw = 0;
          ++kh;
        }
      }
    }
  }
}

__device__ __forceinline__ void load_w4(const Contraction& p, int n, int q0, uint32_t r[4]) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int q = q0 + i;
    r[i] = (n < p.N && q < p.KW) ? p.w[(int64_t)n * p.KW + q] : 0u;
  }
}

template <int OUT, bool CONV>
__global__ __launch_bounds__(256) void xor_kernel(Contraction p) {
  __shared__ uint32_t As[BKW][BM];
  __shared__ uint32_t Ws[BKW][BN];
  __shared__ int Ps[CONV ? MAX_TAPS : 1][BN];  // conv: per-tap popcount of each weight row

  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int tiles_n = (p.N + BN - 1) / BN;
  const int m0 = (blockIdx.x / tiles_n) * BM;
  const int n0 = (blockIdx.x % tiles_n) * BN;

  // loader role: row lr of the A and W tiles, words lq .. lq+3 of the k-tile
  const int lr = tid >> 1, lq = (tid & 1) * 4;
  const int am = m0 + lr, wn = n0 + lr;
  PixelCoord pc{0, 0, 0};
  if constexpr (CONV) {
    if (am < p.M) pc = pixel_coord(p, am);
    const int taps = p.KH * p.KWD;
    for (int i = tid; i < taps * BN; i += 256) {
      const int t = i / BN, nl = i - t * BN;
      const int n = n0 + nl;
      int s = 0;
      if (n < p.N)
        for (int cw = 0; cw < p.CW; cw++) s += __popc(p.w[(int64_t)n * p.KW + t * p.CW + cw]);
      Ps[t][nl] = s;
    }
  }

  uint32_t ra[4], rw[4];
  load_a4<CONV>(p, am, pc, lq, ra);
  load_w4(p, wn, lq, rw);

  int pop[8][8];
#pragma unroll
  for (int i = 0; i < 8; i++)
#pragma unroll
    for (int j = 0; j < 8; j++) pop[i][j] = 0;

  for (int kt = 0; kt < p.KW; kt += BKW) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; i++) {
      As[lq + i][lr] = ra[i];
      Ws[lq + i][lr] = rw[i];
    }
    __syncthreads();
    if (kt + BKW < p.KW) {
      load_a4<CONV>(p, am, pc, kt + BKW + lq, ra);
      load_w4(p, wn, kt + BKW + lq, rw);
    }
#pragma unroll
    for (int k = 0; k < BKW; k++) {
      const uint4 a0 = *reinterpret_cast<const uint4*>(&As[k][ty * 4]);
      const uint4 a1 = *reinterpret_cast<const uint4*>(&As[k][64 + ty * 4]);
      const uint4 w0 = *reinterpret_cast<const uint4*>(&Ws[k][tx * 4]);
      const uint4 w1 = *reinterpret_cast<const uint4*>(&Ws[k][64 + tx * 4]);
      const uint32_t av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      const uint32_t wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int i = 0; i < 8; i++)
#pragma unroll
        for (int j = 0; j < 8; j++) {
          pop[i][j] += __popc(av[i] ^ wv[j]);
          // An empty asm statement (no instruction) that takes and returns the accumulator in
          // a register: it keeps each word's count a v_bcnt_u32_b32 with the accumulator as
          // its addend. Left free, the compiler reassociates the unrolled sums into
          // v_bcnt pairs joined by v_add3_u32 (2.5 instead of 2 VALU operations per word pair).
          asm volatile("" : "+v"(pop[i][j]));
        }
    }
  }

  // epilogue
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int m = m0 + (i < 4 ? ty * 4 + i : 64 + ty * 4 + (i - 4));
    if (m >= p.M) continue;
    if constexpr (!CONV) {
      const int kbits = p.KB;
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const int n = n0 + h * 64 + tx * 4;
        int acc[4];
#pragma unroll
        for (int j = 0; j < 4; j++) acc[j] = kbits - 2 * pop[i][h * 4 + j];
        const int64_t base = (int64_t)m * p.N + n;
        if (n + 3 < p.N && (p.N & 3) == 0) {
          store4<OUT>(p.out, base, acc[0], acc[1], acc[2], acc[3], p.alpha);
        } else {
#pragma unroll
          for (int j = 0; j < 4; j++)
            if (n + j < p.N) store1<OUT>(p.out, base + j, acc[j], p.alpha);
        }
      }
    } else {
      const PixelCoord q = pixel_coord(p, m);
      int corr[8];
#pragma unroll
      for (int j = 0; j < 8; j++) corr[j] = 0;
      int valid_taps = 0;
      for (int kh = 0; kh < p.KH; kh++) {
        const int ih = q.ihb + kh * p.DH;
        const bool hok = ih >= 0 && ih < p.H;
        for (int kw = 0; kw < p.KWD; kw++) {
          const int iw = q.iwb + kw * p.DW;
          if (hok && iw >= 0 && iw < p.W) {
            valid_taps++;
          } else {
            const int t = kh * p.KWD + kw;
#pragma unroll
            for (int j = 0; j < 8; j++) corr[j] += Ps[t][j < 4 ? tx * 4 + j : 64 + tx * 4 + (j - 4)];
          }
        }
      }
      const int kvalid = p.KB * valid_taps;
      const int hw = p.Ho * p.Wo;
      const int pix = m - q.b * hw;
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const int n = n0 + (j < 4 ? tx * 4 + j : 64 + tx * 4 + (j - 4));
        if (n < p.N) {
          const int acc = kvalid - 2 * (pop[i][j] - corr[j]);
          store1<OUT>(p.out, ((int64_t)q.b * p.N + n) * hw + pix, acc, p.alpha);
        }
      }
    }
  }
}

template <bool CONV>
hipError_t launch_xor_t(const Contraction& p, int out_dtype, hipStream_t stream) {
  const int64_t tiles = (int64_t)((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  const dim3 grid((unsigned)tiles), block(256);
  switch (out_dtype) {
    case kF32: hipLaunchKernelGGL((xor_kernel<kF32, CONV>), grid, block, 0, stream, p); break;
    case kF16: hipLaunchKernelGGL((xor_kernel<kF16, CONV>), grid, block, 0, stream, p); break;
    case kBF16: hipLaunchKernelGGL((xor_kernel<kBF16, CONV>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((xor_kernel<kI32, CONV>), grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

}  // namespace

// Largest kernel tap count the conv epilogue's LDS table holds.
int xor_conv_max_taps() { return MAX_TAPS; }

hipError_t launch_xor(const Contraction& p, bool conv, int out_dtype, hipStream_t stream) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  return conv ? launch_xor_t<true>(p, out_dtype, stream) : launch_xor_t<false>(p, out_dtype, stream);
}

}  // namespace bnn
