// Sign + bit-pack kernels for gfx950.
//
// The rule (bitorch-engine binary layers: activations and weights are
// binarized and bit-packed along the reduction axis before the binary
// contraction; the packing kernel is the one BinaryLinearCuda.w_pack and
// BinaryConv2dCutlass.generate_quantized_weight call): element 32q + j of a
// row lands in bit j of word q, bit value 1 when the element is >= 0.
#include "launch.h"


namespace bnn {
namespace {

// DPP lane-permute controls (within each row of 16 lanes).
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror: lane i of each 8 <- lane 7-i

__device__ __forceinline__ uint32_t dpp_or(uint32_t v, int ctrl_sel) {
  int o;
  switch (ctrl_sel) {
    case 0: o = __builtin_amdgcn_mov_dpp((int)v, kDppQuadXor1, 0xF, 0xF, true); break;
    case 1: o = __builtin_amdgcn_mov_dpp((int)v, kDppQuadXor2, 0xF, 0xF, true); break;
    default: o = __builtin_amdgcn_mov_dpp((int)v, kDppHalfMirror, 0xF, 0xF, true); break;
  }
  return v | (uint32_t)o;
}

// ---- shifted sign (the layers' activation prologue) ----
//
// Before the sign is taken the layers add a learnable shift bias_a to the input
// (set_activation of BinaryConv2dCutlass / BinaryLinearCuda): one value per input
// channel for the conv, one value for the whole layer or one per input feature for
// the linear layer. The bit is the sign of x + b. Both operands are widened to fp32
// (exact for f16 and bf16) and added once in fp32. The rounded sum keeps the sign
// and the zero-ness of the exact sum: a non-zero exact sum of two fp32 values is a
// multiple of the smallest subnormal, so it never rounds to zero while subnormals
// are kept (the code objects of this library run with the fp32 denormal mode
// "preserve", the compiler's default), and overflow gives an infinity of the same
// sign. NaN operands and opposite infinities give NaN, which maps to -1 as in the
// plain sign rule; -0 + -0 = -0 counts as >= 0.

// Element e of a 16-byte vector, widened exactly to fp32.
template <int DT>
__device__ __forceinline__ float vec_elem(u32x4 v, int e) {
  if constexpr (DT == kF32) {
    return __uint_as_float(v[e]);
  } else {
    const uint32_t d = v[e >> 1];
    const uint32_t h = (e & 1) ? (d >> 16) : (d & 0xFFFFu);
    if constexpr (DT == kF16)
      return __half2float(__ushort_as_half((unsigned short)h));
    else
      return __uint_as_float(h << 16);
  }
}

// Element i of a typed array, widened exactly to fp32.
template <int DT>
__device__ __forceinline__ float elem_f32(const void* base, int64_t i) {
  if constexpr (DT == kF32)
    return reinterpret_cast<const float*>(base)[i];
  else if constexpr (DT == kF16)
    return __half2float(reinterpret_cast<const __half*>(base)[i]);
  else
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(base)[i] << 16);
}

// Shifted sign bits of the elements of a 16-byte vector, element e at bit e, with
// shift b[e] (PER) or b[0] for every element. The shift must not be -0 (the callers
// add +0 to it once, which turns -0 into +0 and leaves every other value alone), so
// the sum is never -0 and its sign bit alone decides, once a NaN sum is turned into
// -inf by max(s, -inf) (IEEE maxNum: the non-NaN operand; the kernels run in IEEE
// mode and a sum is never a signalling NaN). The sign bits are gathered with
// v_alignbit (acc << 1 | u >> 31), from the last element down, so bit e ends up as
// the sign of element e, and the word is complemented at the end: 1 for >= 0.
template <int DT, int EPL, bool PER>
__device__ __forceinline__ uint32_t vec_bits_shift(u32x4 v, const float* b) {
  uint32_t neg = 0;
#pragma unroll
  for (int e = EPL - 1; e >= 0; e--) {
    const float s = fmaxf(vec_elem<DT>(v, e) + b[PER ? e : 0], -__builtin_inff());
    neg = __builtin_amdgcn_alignbit(neg, __float_as_uint(s), 31);
  }
  return ~neg & ((EPL == 32) ? 0xFFFFFFFFu : ((1u << EPL) - 1u));
}

// Flat row pack. The packed output of a [rows][k] tensor with k % 32 == 0 is
// one contiguous stream of words, word i covering elements [32i, 32i+32).
//
// Each lane reads 16 bytes per load (4 f32 or 8 f16/bf16 elements), and the
// lanes of one load instruction read 1 KiB of consecutive bytes, so every
// load is fully coalesced. A word spans LPW adjacent lanes (8 for f32, 4 for
// 16-bit types); each lane shifts its bits into place and the group ORs them
// together with DPP lane swaps. One wave packs a chunk of 64 words with LPW
// loads per lane in flight; afterwards lane L keeps the word of load L % LPW,
// so the 64 lanes store 64 distinct words of one 256-byte span.
template <int DT>
__global__ __launch_bounds__(256) void pack_rows_kernel(const u32x4* __restrict__ x,
                                                        uint32_t* __restrict__ out,
                                                        int64_t total_words) {
  constexpr int EPL = (DT == kF32) ? 4 : 8;  // elements per 16-byte load
  constexpr int LPW = 32 / EPL;              // lanes per word
  constexpr int WPI = 64 / LPW;              // words per wave load instruction
  const int lane = threadIdx.x & 63;
  const int pos = lane % LPW;
  const int grp = lane / LPW;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  const int64_t nchunks = (total_words + 63) >> 6;

  for (int64_t ch = wave; ch < nchunks; ch += nwaves) {
    const int64_t wbase = ch << 6;
    u32x4 v[LPW];
#pragma unroll
    for (int j = 0; j < LPW; j++) {
      const int64_t word = wbase + j * WPI + grp;
      v[j] = (word < total_words) ? __builtin_nontemporal_load(&x[wbase * LPW + j * 64 + lane])
                                  : u32x4{0u, 0u, 0u, 0u};
    }
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < LPW; j++) {
      uint32_t part = vec_bits<DT>(v[j]) << (pos * EPL);
      part = dpp_or(part, 0);
      part = dpp_or(part, 1);
      if constexpr (LPW == 8) part = dpp_or(part, 2);
      mine = (pos == j) ? part : mine;
    }
    const int64_t myword = wbase + pos * WPI + grp;
    // packed words are written once: stream them past the caches (measured ~3 % faster)
    if (myword < total_words) __builtin_nontemporal_store(mine, out + myword);
  }
}

// Sum of v over a 256-thread workgroup (fixed order); the result is valid in thread 0.
__device__ __forceinline__ double block_sum_256(double v, double* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double t = 0.0;
  if (threadIdx.x == 0) t = (red[0] + red[1]) + (red[2] + red[3]);
  return t;
}

// Sum of the magnitudes of a 16-byte vector's elements, in double (a fixed pairwise tree).
template <int DT>
__device__ __forceinline__ double vec_abs_sum(u32x4 v) {
  constexpr int EPL = (DT == kF32) ? 4 : 8;
  double t[EPL];
#pragma unroll
  for (int e = 0; e < EPL; e++) t[e] = (double)fabsf(vec_elem<DT>(v, e));
#pragma unroll
  for (int w = EPL / 2; w >= 1; w /= 2)
#pragma unroll
    for (int e = 0; e < w; e++) t[e] = t[e] + t[e + w];
  return t[0];
}

// Row pack with the shift. Same lane layout as pack_rows_kernel, but a workgroup's
// waves stay on one 64-word column chunk (blockIdx.x) and walk down the rows
// (blockIdx.y, then the grid's row stride, two rows per step), so each lane loads the
// shift values of its elements once and keeps them in registers for every row it
// visits. PERCOL: one shift per column (bias[k]); otherwise bias[0] for every element.
// Loads use clamped addresses (always in bounds) so none sits behind a branch; words
// past the row end or rows past the last are simply not stored.
// ABS (the one-pass prologue): the same read also sums |x| (unshifted) in double, each
// vector by the fixed pairwise tree, each lane in its fixed order of rows, the clamped
// re-reads left out; the workgroup's sum goes to partial[blockIdx.y * gridDim.x +
// blockIdx.x]. The grid depends only on rows and KW, so the order of every addition does.
template <int DT, int BDT, bool PERCOL, bool ABS = false>
__global__ __launch_bounds__(256) void pack_rows_shift_kernel(const u32x4* __restrict__ x,
                                                              const void* __restrict__ bias,
                                                              uint32_t* __restrict__ out,
                                                              int64_t rows, int64_t KW,
                                                              double* __restrict__ partial = nullptr) {
  constexpr int EPL = (DT == kF32) ? 4 : 8;
  constexpr int LPW = 32 / EPL;
  constexpr int WPI = 64 / LPW;
  constexpr int NB = PERCOL ? EPL : 1;
  const int lane = threadIdx.x & 63;
  const int pos = lane % LPW;
  const int grp = lane / LPW;
  const int64_t q0 = (int64_t)blockIdx.x * 64;
  float bv[LPW][NB];
  int64_t qc[LPW];  // word of load j, clamped into the row
#pragma unroll
  for (int j = 0; j < LPW; j++) {
    const int64_t q = q0 + j * WPI + grp;
    qc[j] = q < KW ? q : KW - 1;
#pragma unroll
    for (int e = 0; e < NB; e++)
      bv[j][e] = elem_f32<BDT>(bias, PERCOL ? qc[j] * 32 + pos * EPL + e : 0) + 0.0f;
  }
  const int64_t myq = q0 + pos * WPI + grp;
  const int64_t step = (int64_t)gridDim.y * 4;
  double abs0 = 0.0, abs1 = 0.0;
  for (int64_t r = (int64_t)blockIdx.y * 4 + (threadIdx.x >> 6); r < rows; r += 2 * step) {
    const int64_t r1 = r + step < rows ? r + step : r;
    u32x4 v0[LPW], v1[LPW];
#pragma unroll
    for (int j = 0; j < LPW; j++) {
      v0[j] = __builtin_nontemporal_load(&x[(r * KW + qc[j]) * LPW + pos]);
      v1[j] = __builtin_nontemporal_load(&x[(r1 * KW + qc[j]) * LPW + pos]);
    }
    if constexpr (ABS) {
#pragma unroll
      for (int j = 0; j < LPW; j++) {
        if (q0 + j * WPI + grp < KW) {
          abs0 += vec_abs_sum<DT>(v0[j]);
          if (r + step < rows) abs1 += vec_abs_sum<DT>(v1[j]);
        }
      }
    }
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int j = 0; j < LPW; j++) {
      uint32_t a0 = vec_bits_shift<DT, EPL, PERCOL>(v0[j], bv[j]) << (pos * EPL);
      uint32_t a1 = vec_bits_shift<DT, EPL, PERCOL>(v1[j], bv[j]) << (pos * EPL);
      a0 = dpp_or(a0, 0);
      a1 = dpp_or(a1, 0);
      a0 = dpp_or(a0, 1);
      a1 = dpp_or(a1, 1);
      if constexpr (LPW == 8) {
        a0 = dpp_or(a0, 2);
        a1 = dpp_or(a1, 2);
      }
      w0 = (pos == j) ? a0 : w0;
      w1 = (pos == j) ? a1 : w1;
    }
    if (myq < KW) {
      __builtin_nontemporal_store(w0, out + r * KW + myq);
      if (r + step < rows) __builtin_nontemporal_store(w1, out + (r + step) * KW + myq);
    }
  }
  if constexpr (ABS) {
    __shared__ double red[4];
    const double t = block_sum_256(abs0 + abs1, red);
    if (threadIdx.x == 0) partial[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = t;
  }
}

// Row pack for rows that are not a whole number of words (k % 32 != 0), plain or shifted.
// Rows then start at arbitrary element offsets, so the 16-byte vector layout above does
// not apply: one wave packs 64 consecutive elements of one row per step, one element per
// lane (a coalesced 64-element load), and a ballot of the 64 sign bits gives two words,
// which lanes 0 and 1 store. Columns at or past k give 0 bits, so the last word of a row
// holds k % 32 signs and zeros above them. SHIFT: bit = (x + b >= 0) with b = bias[col]
// (PERCOL) or bias[0]; BDT is the shift's element type.
template <int DT, bool SHIFT, int BDT, bool PERCOL>
__global__ __launch_bounds__(256) void pack_rows_ragged_kernel(const void* __restrict__ x,
                                                               const void* __restrict__ bias,
                                                               uint32_t* __restrict__ out,
                                                               int64_t rows, int64_t k,
                                                               int64_t KW) {
  const int lane = threadIdx.x & 63;
  const int64_t chunks = (KW + 1) / 2;  // 64-element steps per row
  const int64_t total = rows * chunks;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  const float b0 = (SHIFT && !PERCOL) ? elem_f32<BDT>(bias, 0) + 0.0f : 0.0f;
  for (int64_t t = wave; t < total; t += nwaves) {
    const int64_t r = t / chunks, ch = t - r * chunks;
    const int64_t col = ch * 64 + lane;
    bool bit = false;
    if (col < k) {
      if constexpr (SHIFT) {
        const float b = PERCOL ? elem_f32<BDT>(bias, col) + 0.0f : b0;
        bit = elem_f32<DT>(x, r * k + col) + b >= 0.0f;
      } else {
        bit = elem_pos<DT>(x, r * k + col) != 0u;
      }
    }
    const uint64_t m = __ballot(bit);
    const int64_t q = ch * 2 + lane;
    if (lane < 2 && q < KW) out[r * KW + q] = (uint32_t)(lane == 0 ? m : (m >> 32));
  }
}

// NCHW pack along channels. Word (b, pixel, q) collects channel 32q + j of that pixel
// into bit j. A 256-thread workgroup packs 64*V consecutive pixels of one (b, q): lanes
// run along the contiguous pixel axis (V pixels each, one 16-byte load when the plane
// allows it, so each load instruction reads one channel plane contiguously), and wave w
// takes channels 8w .. 8w+7 of the word with its eight loads in flight at once. Each wave
// writes byte w of every pixel's word to LDS; the assembled words then leave in pixel order.
//
// BDT >= 0: the shifted form, channel c adding bias[c] (element type BDT) before the
// sign; the shift is uniform across a wave, so it is one scalar load per channel.
// The launcher uses this kernel with V = 1 (planes whose pixel count is not a multiple of
// the 16-byte vector width, or an unaligned tensor); pack_nchw_flat_kernel takes the rest.
template <int DT, int V, int BDT = -1>
__global__ __launch_bounds__(256) void pack_nchw_kernel(const void* __restrict__ x,
                                                        uint32_t* __restrict__ out, int64_t C,
                                                        int64_t HW, int64_t CW, int64_t nbq,
                                                        const void* __restrict__ bias = nullptr) {
  constexpr int ES = (DT == kF32) ? 4 : 2;
  constexpr int PIX = 64 * V;                     // pixels per workgroup
  __shared__ uint32_t words[PIX];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nchunks = (HW + PIX - 1) / PIX;
  for (int64_t bq = blockIdx.y; bq < nbq; bq += gridDim.y) {
    const int64_t b = bq / CW, q = bq - b * CW;
    const char* plane0 = reinterpret_cast<const char*>(x) + ((b * C + 32 * q + 8 * wave) * HW) * ES;
    // channels of this wave that exist (fewer than 8 only in the last word of a channel
    // count that is not a whole number of words: the missing channels give 0 bits)
    const int nch = (int)(C - (32 * q + 8 * wave) < 8 ? C - (32 * q + 8 * wave) : 8);
    float shift[8];
    if constexpr (BDT >= 0) {
#pragma unroll
      for (int c = 0; c < 8; c++) shift[c] = c < nch ? elem_f32<BDT>(bias, 32 * q + 8 * wave + c) + 0.0f : 0.0f;
    }
    for (int64_t ch = blockIdx.x; ch < nchunks; ch += gridDim.x) {
      const int64_t base = ch * PIX;
      const int64_t p0 = base + (int64_t)lane * V;
      uint32_t bits[8];
#pragma unroll
      for (int c = 0; c < 8; c++) {
        const char* src = plane0 + ((int64_t)c * HW + p0) * ES;
        if constexpr (V * ES == 16) {
          if (p0 < HW && c < nch) {
            const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
            if constexpr (BDT >= 0)
              bits[c] = vec_bits_shift<DT, V, false>(v, &shift[c]);
            else
              bits[c] = vec_bits<DT>(v);
          } else {
            bits[c] = 0u;
          }
        } else {
          uint32_t bb = 0;
#pragma unroll
          for (int v = 0; v < V; v++) {
            if (p0 + v < HW && c < nch) {
              if constexpr (BDT >= 0)
                bb |= (uint32_t)(elem_f32<DT>(src, v) + shift[c] >= 0.0f) << v;
              else
                bb |= elem_pos<DT>(src, v) << v;
            }
          }
          bits[c] = bb;
        }
      }
      uint8_t* wbytes = reinterpret_cast<uint8_t*>(words);
#pragma unroll
      for (int v = 0; v < V; v++) {
        uint32_t byte = 0;
#pragma unroll
        for (int c = 0; c < 8; c++) byte |= ((bits[c] >> v) & 1u) << c;
        wbytes[(lane * V + v) * 4 + wave] = (uint8_t)byte;
      }
      __syncthreads();
      for (int i = threadIdx.x; i < PIX; i += 256) {
        const int64_t pix = base + i;
        if (pix < HW) out[(b * HW + pix) * CW + q] = words[i];
      }
      __syncthreads();
    }
  }
}

// Sum of |x| in double (the lazy activation-scale init of the layers' set_activation:
// scale_a = factor * mean|x| over every element while scale_a is still zero).
// Every element is widened exactly to fp32, its magnitude converted exactly to
// double and added in double. Stage 1: each workgroup of a fixed-size grid adds a
// grid-strided share of the 16-byte vectors (workgroup 0 also the tail elements
// past the last whole vector), then the workgroup's sum goes to partial[blockIdx.x].
// Stage 2: one workgroup adds the partials in a fixed order and writes
// factor * (sum / count). The grid size depends only on count, so the result is
// the same on every run.

template <int DT>
__global__ __launch_bounds__(256) void abs_sum_kernel(const u32x4* __restrict__ x, int64_t nvec,
                                                      const void* __restrict__ tail,
                                                      int ntail, double* __restrict__ partial) {
  constexpr int U = 4;  // vectors in flight per thread
  __shared__ double red[4];
  double acc0 = 0.0, acc1 = 0.0;
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + (U - 1) * stride < nvec; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; u++) v[u] = __builtin_nontemporal_load(&x[i + u * stride]);
#pragma unroll
    for (int u = 0; u < U; u += 2) {
      acc0 += vec_abs_sum<DT>(v[u]);
      acc1 += vec_abs_sum<DT>(v[u + 1]);
    }
  }
  for (; i < nvec; i += stride) acc0 += vec_abs_sum<DT>(__builtin_nontemporal_load(&x[i]));
  double acc = acc0 + acc1;
  if (blockIdx.x == 0 && threadIdx.x < ntail) acc += (double)fabsf(elem_f32<DT>(tail, threadIdx.x));
  const double t = block_sum_256(acc, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = t;
}

__global__ __launch_bounds__(256) void abs_mean_final_kernel(const double* __restrict__ partial,
                                                             int nparts, double count,
                                                             double factor,
                                                             double* __restrict__ out) {
  __shared__ double red[4];
  // each thread adds partials threadIdx.x, +256, +512, ... in that order; sixteen of them are
  // loaded at once (clamped, unconditional loads; the ones past the end add +0, which leaves
  // the non-negative sum unchanged) so the loads' latency is paid once per sixteen, not each
  constexpr int U = 16;
  double acc = 0.0;
  for (int i0 = threadIdx.x; i0 < nparts; i0 += 256 * U) {
    double v[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int i = i0 + 256 * u;
      const double x = partial[i < nparts ? i : nparts - 1];
      v[u] = i < nparts ? x : 0.0;
    }
#pragma unroll
    for (int u = 0; u < U; u++) acc += v[u];
  }
  const double t = block_sum_256(acc, red);
  if (threadIdx.x == 0) out[0] = factor * (t / count);
}

// 8 x 8 bit transpose of a matrix held as two dwords, row r in byte r (lo: rows 0-3, hi:
// rows 4-7), bit c of a row = column c: afterwards byte c holds column c, bit r = row r.
// Three rounds swap ever larger off-diagonal blocks (1x1 inside 2x2, 2x2 inside 4x4, 4x4
// inside 8x8; the delta-swap method, see Warren, Hacker's Delight, section 7-3).
__device__ __forceinline__ void transpose8x8(uint32_t& lo, uint32_t& hi) {
  uint32_t t;
  t = (lo ^ (lo >> 7)) & 0x00AA00AAu;
  lo ^= t ^ (t << 7);
  t = (hi ^ (hi >> 7)) & 0x00AA00AAu;
  hi ^= t ^ (t << 7);
  t = (lo ^ (lo >> 14)) & 0x0000CCCCu;
  lo ^= t ^ (t << 14);
  t = (hi ^ (hi >> 14)) & 0x0000CCCCu;
  hi ^= t ^ (t << 14);
  t = (lo ^ (hi << 4)) & 0xF0F0F0F0u;
  lo ^= t;
  hi ^= t >> 4;
}

// NCHW pack over the flattened (image, pixel) axis, for planes whose pixel count is a
// multiple of the 16-byte vector width V (and a 16-byte aligned tensor): a workgroup packs
// word q of 64*V consecutive pixels of the whole batch, each lane's V pixels lying in one
// image, so no chunk is left partly empty at the end of an image plane (with 28x28 planes
// and 512-pixel chunks per image, a quarter of the lanes idled). Wave w loads channels
// 8w..8w+7 of the word (eight 16-byte loads in flight, each load instruction reading 1 KiB
// of one channel plane), an 8 x 8 bit transpose turns the channel bytes into pixel bytes,
// the four waves' bytes meet in LDS and the words leave in pixel order.
// ABS (the one-pass prologue): the same loads also give the sum of |x| in double (each vector
// by the fixed pairwise tree, the re-reads of missing channels and pixels left out), one
// partial per workgroup at partial[blockIdx.y * gridDim.x + blockIdx.x].
template <int DT, int V, int BDT, bool ABS = false>
__global__ __launch_bounds__(256) void pack_nchw_flat_kernel(const void* __restrict__ x,
                                                             uint32_t* __restrict__ out, int C,
                                                             int HW, int CW, int P,
                                                             const void* __restrict__ bias,
                                                             double* __restrict__ partial = nullptr) {
  constexpr int ES = (DT == kF32) ? 4 : 2;
  constexpr int PIX = 64 * V;
  static_assert(V * ES == 16, "one 16-byte vector per lane and channel");
  __shared__ uint32_t words[PIX];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nchunks = (P + PIX - 1) / PIX;
  double absacc = 0.0;
  for (int q = blockIdx.y; q < CW; q += gridDim.y) {
    const int c0 = 32 * q + 8 * wave;
    const int nch = C - c0 < 8 ? C - c0 : 8;  // fewer only in a last, partly filled word
    float shift[8];
    if constexpr (BDT >= 0) {
#pragma unroll
      for (int c = 0; c < 8; c++) shift[c] = elem_f32<BDT>(bias, c < nch ? c0 + c : 0) + 0.0f;
    }
    for (int ch = blockIdx.x; ch < nchunks; ch += gridDim.x) {
      // all eight loads go out before any is used (a load behind a branch would be waited
      // for on the spot); lanes past the end read pixel 0, missing channels (none, or fewer
      // than 8, exist in a last, partly filled word) re-read channel 0, and both give 0 bits
      const int f0 = ch * PIX + lane * V;
      const bool ok = f0 < P;
      const int fc = ok ? f0 : 0;
      const int b = fc / HW;
      const int pix = fc - b * HW;
      const char* img = reinterpret_cast<const char*>(x) + ((int64_t)b * C * HW + pix) * ES;
      u32x4 vin[8];
#pragma unroll
      for (int c = 0; c < 8; c++)
        vin[c] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(img + (int64_t)(c < nch ? c0 + c : 0) * HW * ES));
      // keep the scheduler from sinking each load to its use
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (ABS) {
#pragma unroll
        for (int c = 0; c < 8; c++)
          if (ok && c < nch) absacc += vec_abs_sum<DT>(vin[c]);
      }
      // byte c of (lo, hi) = the V pixel bits of channel c0 + c
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int c = 0; c < 8; c++) {
        uint32_t bb;
        if constexpr (BDT >= 0)
          bb = vec_bits_shift<DT, V, false>(vin[c], &shift[c]);
        else
          bb = vec_bits<DT>(vin[c]);
        bb = (ok && c < nch) ? bb : 0u;
        if (c < 4)
          lo |= bb << (8 * c);
        else
          hi |= bb << (8 * (c - 4));
      }
      transpose8x8(lo, hi);  // now byte v = the 8 channel bits of pixel v
      uint8_t* wbytes = reinterpret_cast<uint8_t*>(words);
#pragma unroll
      for (int v = 0; v < V; v++)
        wbytes[(lane * V + v) * 4 + wave] = (uint8_t)((v < 4 ? lo : hi) >> (8 * (v & 3)));
      __syncthreads();
#pragma unroll
      for (int i = threadIdx.x; i < PIX; i += 256) {
        const int f = ch * PIX + i;
        if (f < P) out[(int64_t)f * CW + q] = words[i];
      }
      __syncthreads();
    }
  }
  if constexpr (ABS) {
    __shared__ double red[4];
    const double t = block_sum_256(absacc, red);
    if (threadIdx.x == 0) partial[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = t;
  }
}

// OIHW weight pack: word (o, tap, q) collects w[o][32q + j][tap] into bit j (channels at or
// past C give 0 bits).
// Runs once per layer, off the forward path.
template <int DT>
__global__ __launch_bounds__(256) void pack_conv_weight_kernel(const void* __restrict__ w,
                                                               uint32_t* __restrict__ out,
                                                               int64_t total, int64_t C, int T,
                                                               int64_t CW) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int64_t q = idx % CW;
  const int64_t t = (idx / CW) % T;
  const int64_t o = idx / (CW * T);
  uint32_t word = 0;
  for (int j = 0; j < 32 && 32 * q + j < C; j++) word |= elem_pos<DT>(w, ((o * C + 32 * q + j) * T) + t) << j;
  out[idx] = word;
}

}  // namespace

hipError_t launch_pack_rows(const void* x, int dtype, int64_t total_words, uint32_t* out,
                            hipStream_t stream) {
  if (total_words <= 0) return hipSuccess;
  const int64_t chunks = (total_words + 63) / 64;
  const int64_t waves_per_block = 4;
  int64_t blocks = (chunks + waves_per_block - 1) / waves_per_block;
  if (blocks > 65536) blocks = 65536;
  const dim3 grid((unsigned)blocks), block(256);
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  switch (dtype) {
    case kF32: hipLaunchKernelGGL(pack_rows_kernel<kF32>, grid, block, 0, stream, xv, out, total_words); break;
    case kF16: hipLaunchKernelGGL(pack_rows_kernel<kF16>, grid, block, 0, stream, xv, out, total_words); break;
    default: hipLaunchKernelGGL(pack_rows_kernel<kBF16>, grid, block, 0, stream, xv, out, total_words); break;
  }
  return hipGetLastError();
}

namespace {

template <int DT, int V, int BDT>
void launch_nchw_t(dim3 grid, const void* x, uint32_t* out, int64_t c, int64_t HW, int64_t CW,
                   int64_t nbq, const void* bias, hipStream_t stream) {
  hipLaunchKernelGGL((pack_nchw_kernel<DT, V, BDT>), grid, dim3(256), 0, stream, x, out, c, HW, CW,
                     nbq, bias);
}

template <int DT, int V>
void launch_nchw_b(dim3 grid, const void* x, uint32_t* out, int64_t c, int64_t HW, int64_t CW,
                   int64_t nbq, const void* bias, int bdtype, hipStream_t stream) {
  switch (bdtype) {
    case kF32: launch_nchw_t<DT, V, kF32>(grid, x, out, c, HW, CW, nbq, bias, stream); break;
    case kF16: launch_nchw_t<DT, V, kF16>(grid, x, out, c, HW, CW, nbq, bias, stream); break;
    case kBF16: launch_nchw_t<DT, V, kBF16>(grid, x, out, c, HW, CW, nbq, bias, stream); break;
    default: launch_nchw_t<DT, V, -1>(grid, x, out, c, HW, CW, nbq, nullptr, stream); break;
  }
}

template <int DT, int V, int BDT>
void launch_nchw_flat_t(dim3 grid, const void* x, uint32_t* out, int64_t c, int64_t HW, int64_t CW,
                        int64_t P, const void* bias, double* partial, hipStream_t stream) {
  if (partial)
    hipLaunchKernelGGL((pack_nchw_flat_kernel<DT, V, BDT, true>), grid, dim3(256), 0, stream, x,
                       out, (int)c, (int)HW, (int)CW, (int)P, bias, partial);
  else
    hipLaunchKernelGGL((pack_nchw_flat_kernel<DT, V, BDT>), grid, dim3(256), 0, stream, x,
                       out, (int)c, (int)HW, (int)CW, (int)P, bias, nullptr);
}

template <int DT, int V>
void launch_nchw_flat_b(dim3 grid, const void* x, uint32_t* out, int64_t c, int64_t HW, int64_t CW,
                        int64_t P, const void* bias, int bdtype, double* partial, hipStream_t stream) {
  switch (bdtype) {
    case kF32: launch_nchw_flat_t<DT, V, kF32>(grid, x, out, c, HW, CW, P, bias, partial, stream); break;
    case kF16: launch_nchw_flat_t<DT, V, kF16>(grid, x, out, c, HW, CW, P, bias, partial, stream); break;
    case kBF16: launch_nchw_flat_t<DT, V, kBF16>(grid, x, out, c, HW, CW, P, bias, partial, stream); break;
    default: launch_nchw_flat_t<DT, V, -1>(grid, x, out, c, HW, CW, P, nullptr, partial, stream); break;
  }
}

// Grid of the flat NCHW pack: pixel chunks of 64 16-byte vectors by channel words.
dim3 nchw_flat_grid(int64_t P, int64_t CW, int V) {
  const int64_t fchunks = (P + 64 * V - 1) / (64 * V);
  return dim3((unsigned)(fchunks < 65535 ? fchunks : 65535), (unsigned)(CW < 65535 ? CW : 65535));
}

}  // namespace

hipError_t launch_pack_nchw(const void* x, int dtype, int64_t b, int64_t c, int64_t h, int64_t w,
                            uint32_t* out, hipStream_t stream, const void* bias, int bdtype) {
  const int64_t HW = h * w, CW = (c + 31) / 32;
  if (b * HW * CW == 0) return hipSuccess;
  const int es = dtype == kF32 ? 4 : 2;
  const int vfull = 16 / es;
  const bool vec = (HW % vfull) == 0 && (reinterpret_cast<uintptr_t>(x) % 16) == 0;
  const int V = vec ? vfull : 1;
  const int64_t nchunks = (HW + 64 * V - 1) / (64 * V);
  const int64_t nbq = b * CW;
  const dim3 grid((unsigned)(nchunks < 65535 ? nchunks : 65535), (unsigned)(nbq < 65535 ? nbq : 65535));
  if (!bias) bdtype = -1;
  if (vec) {
    // flattened pixel chunks (the sizes fit in int: the C ABI checks n*h*w*ceil(c/32))
    const int64_t P = b * HW;
    const dim3 fgrid = nchw_flat_grid(P, CW, V);
    switch (dtype) {
      case kF32: launch_nchw_flat_b<kF32, 4>(fgrid, x, out, c, HW, CW, P, bias, bdtype, nullptr, stream); break;
      case kF16: launch_nchw_flat_b<kF16, 8>(fgrid, x, out, c, HW, CW, P, bias, bdtype, nullptr, stream); break;
      default: launch_nchw_flat_b<kBF16, 8>(fgrid, x, out, c, HW, CW, P, bias, bdtype, nullptr, stream); break;
    }
  } else {
    switch (dtype) {
      case kF32: launch_nchw_b<kF32, 1>(grid, x, out, c, HW, CW, nbq, bias, bdtype, stream); break;
      case kF16: launch_nchw_b<kF16, 1>(grid, x, out, c, HW, CW, nbq, bias, bdtype, stream); break;
      default: launch_nchw_b<kBF16, 1>(grid, x, out, c, HW, CW, nbq, bias, bdtype, stream); break;
    }
  }
  return hipGetLastError();
}

namespace {

template <int DT, int BDT, bool ABS>
void launch_rows_shift_t(dim3 grid, const void* x, const void* bias, bool percol, uint32_t* out,
                         int64_t rows, int64_t KW, double* partial, hipStream_t stream) {
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  if (percol)
    hipLaunchKernelGGL((pack_rows_shift_kernel<DT, BDT, true, ABS>), grid, dim3(256), 0, stream, xv,
                       bias, out, rows, KW, partial);
  else
    hipLaunchKernelGGL((pack_rows_shift_kernel<DT, BDT, false, ABS>), grid, dim3(256), 0, stream, xv,
                       bias, out, rows, KW, partial);
}

template <int DT, bool ABS>
void launch_rows_shift_b(dim3 grid, const void* x, const void* bias, int bdtype, bool percol,
                         uint32_t* out, int64_t rows, int64_t KW, double* partial, hipStream_t stream) {
  switch (bdtype) {
    case kF32: launch_rows_shift_t<DT, kF32, ABS>(grid, x, bias, percol, out, rows, KW, partial, stream); break;
    case kF16: launch_rows_shift_t<DT, kF16, ABS>(grid, x, bias, percol, out, rows, KW, partial, stream); break;
    default: launch_rows_shift_t<DT, kBF16, ABS>(grid, x, bias, percol, out, rows, KW, partial, stream); break;
  }
}

// Grid of the shifted row pack: one column of workgroups per 64-word chunk, about 4096
// workgroups in all (16 waves per compute unit), each wave walking its rows.
dim3 rows_shift_grid(int64_t rows, int64_t KW) {
  const int64_t nchunk = (KW + 63) / 64;
  int64_t gy = (4096 + nchunk - 1) / nchunk;
  const int64_t row_groups = (rows + 3) / 4;
  if (gy > row_groups) gy = row_groups;
  if (gy > 65535) gy = 65535;
  if (gy < 1) gy = 1;
  return dim3((unsigned)nchunk, (unsigned)gy);
}

template <bool ABS>
hipError_t launch_rows_shift_any(const void* x, int dtype, int64_t rows, int64_t KW, const void* bias,
                                 int bdtype, bool percol, uint32_t* out, double* partial,
                                 hipStream_t stream) {
  const dim3 grid = rows_shift_grid(rows, KW);
  switch (dtype) {
    case kF32: launch_rows_shift_b<kF32, ABS>(grid, x, bias, bdtype, percol, out, rows, KW, partial, stream); break;
    case kF16: launch_rows_shift_b<kF16, ABS>(grid, x, bias, bdtype, percol, out, rows, KW, partial, stream); break;
    default: launch_rows_shift_b<kBF16, ABS>(grid, x, bias, bdtype, percol, out, rows, KW, partial, stream); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack_rows_shift(const void* x, int dtype, int64_t rows, int64_t KW,
                                  const void* bias, int bdtype, bool percol, uint32_t* out,
                                  hipStream_t stream) {
  if (rows <= 0 || KW <= 0) return hipSuccess;
  return launch_rows_shift_any<false>(x, dtype, rows, KW, bias, bdtype, percol, out, nullptr, stream);
}

int64_t pack_rows_shift_abs_parts(int64_t rows, int64_t KW) {
  if (rows <= 0 || KW <= 0) return 1;
  const dim3 g = rows_shift_grid(rows, KW);
  return (int64_t)g.x * g.y;
}

hipError_t launch_pack_rows_shift_abs(const void* x, int dtype, int64_t rows, int64_t KW,
                                      const void* bias, int bdtype, bool percol, uint32_t* out,
                                      double factor, double* partial, double* scale_out,
                                      hipStream_t stream) {
  hipError_t e = launch_rows_shift_any<true>(x, dtype, rows, KW, bias, bdtype, percol, out, partial,
                                             stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(abs_mean_final_kernel, dim3(1), dim3(256), 0, stream, partial,
                     (int)pack_rows_shift_abs_parts(rows, KW), (double)rows * KW * 32, factor,
                     scale_out);
  return hipGetLastError();
}

namespace {

template <int DT, bool SHIFT, int BDT, bool PERCOL>
void launch_ragged_t(dim3 grid, const void* x, const void* bias, uint32_t* out, int64_t rows,
                     int64_t k, int64_t KW, hipStream_t stream) {
  hipLaunchKernelGGL((pack_rows_ragged_kernel<DT, SHIFT, BDT, PERCOL>), grid, dim3(256), 0, stream,
                     x, bias, out, rows, k, KW);
}

template <int DT>
void launch_ragged_b(dim3 grid, const void* x, const void* bias, int bdtype, bool percol,
                     uint32_t* out, int64_t rows, int64_t k, int64_t KW, hipStream_t stream) {
  if (!bias) {
    launch_ragged_t<DT, false, kF32, false>(grid, x, nullptr, out, rows, k, KW, stream);
    return;
  }
  switch (bdtype) {
    case kF32:
      if (percol) launch_ragged_t<DT, true, kF32, true>(grid, x, bias, out, rows, k, KW, stream);
      else launch_ragged_t<DT, true, kF32, false>(grid, x, bias, out, rows, k, KW, stream);
      break;
    case kF16:
      if (percol) launch_ragged_t<DT, true, kF16, true>(grid, x, bias, out, rows, k, KW, stream);
      else launch_ragged_t<DT, true, kF16, false>(grid, x, bias, out, rows, k, KW, stream);
      break;
    default:
      if (percol) launch_ragged_t<DT, true, kBF16, true>(grid, x, bias, out, rows, k, KW, stream);
      else launch_ragged_t<DT, true, kBF16, false>(grid, x, bias, out, rows, k, KW, stream);
      break;
  }
}

}  // namespace

hipError_t launch_pack_rows_ragged(const void* x, int dtype, int64_t rows, int64_t k,
                                   const void* bias, int bdtype, bool percol, uint32_t* out,
                                   hipStream_t stream) {
  if (rows <= 0 || k <= 0) return hipSuccess;
  const int64_t KW = (k + 31) / 32;
  const int64_t waves = rows * ((KW + 1) / 2);
  int64_t blocks = (waves + 3) / 4;
  if (blocks > 16384) blocks = 16384;
  const dim3 grid((unsigned)blocks);
  switch (dtype) {
    case kF32: launch_ragged_b<kF32>(grid, x, bias, bdtype, percol, out, rows, k, KW, stream); break;
    case kF16: launch_ragged_b<kF16>(grid, x, bias, bdtype, percol, out, rows, k, KW, stream); break;
    default: launch_ragged_b<kBF16>(grid, x, bias, bdtype, percol, out, rows, k, KW, stream); break;
  }
  return hipGetLastError();
}

bool pack_nchw_abs_fused(int dtype, int64_t h, int64_t w, const void* x) {
  const int vfull = dtype == kF32 ? 4 : 8;
  return (h * w) % vfull == 0 && (reinterpret_cast<uintptr_t>(x) % 16) == 0;
}

int64_t pack_nchw_abs_parts(int dtype, int64_t b, int64_t c, int64_t h, int64_t w) {
  const int V = dtype == kF32 ? 4 : 8;
  const dim3 g = nchw_flat_grid(b * h * w, (c + 31) / 32, V);
  return (int64_t)g.x * g.y;
}

hipError_t launch_pack_nchw_shift_abs(const void* x, int dtype, int64_t b, int64_t c, int64_t h,
                                      int64_t w, uint32_t* out, const void* bias, int bdtype,
                                      double factor, double* partial, double* scale_out,
                                      hipStream_t stream) {
  const int64_t HW = h * w, CW = (c + 31) / 32, P = b * HW;
  const int V = dtype == kF32 ? 4 : 8;
  const dim3 fgrid = nchw_flat_grid(P, CW, V);
  switch (dtype) {
    case kF32: launch_nchw_flat_b<kF32, 4>(fgrid, x, out, c, HW, CW, P, bias, bdtype, partial, stream); break;
    case kF16: launch_nchw_flat_b<kF16, 8>(fgrid, x, out, c, HW, CW, P, bias, bdtype, partial, stream); break;
    default: launch_nchw_flat_b<kBF16, 8>(fgrid, x, out, c, HW, CW, P, bias, bdtype, partial, stream); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(abs_mean_final_kernel, dim3(1), dim3(256), 0, stream, partial,
                     (int)((int64_t)fgrid.x * fgrid.y), (double)(b * c * HW), factor, scale_out);
  return hipGetLastError();
}

int abs_mean_parts(int64_t count) {
  // one workgroup per 2048 elements, at most 1024 (a function of count alone, so the
  // order of the additions, hence the result, is the same on every run)
  int64_t parts = (count + 2047) / 2048;
  if (parts > 1024) parts = 1024;
  if (parts < 1) parts = 1;
  return (int)parts;
}

hipError_t launch_abs_mean(const void* x, int dtype, int64_t count, double factor, double* partial,
                           double* out, hipStream_t stream) {
  const int epl = dtype == kF32 ? 4 : 8;
  const int es = dtype == kF32 ? 4 : 2;
  const int64_t nvec = count / epl;
  const int ntail = (int)(count - nvec * epl);
  const void* tail = reinterpret_cast<const char*>(x) + nvec * epl * es;
  const int parts = abs_mean_parts(count);
  const dim3 grid((unsigned)parts), block(256);
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  switch (dtype) {
    case kF32: hipLaunchKernelGGL(abs_sum_kernel<kF32>, grid, block, 0, stream, xv, nvec, tail, ntail, partial); break;
    case kF16: hipLaunchKernelGGL(abs_sum_kernel<kF16>, grid, block, 0, stream, xv, nvec, tail, ntail, partial); break;
    default: hipLaunchKernelGGL(abs_sum_kernel<kBF16>, grid, block, 0, stream, xv, nvec, tail, ntail, partial); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(abs_mean_final_kernel, dim3(1), block, 0, stream, partial, parts, (double)count,
                     factor, out);
  return hipGetLastError();
}

hipError_t launch_pack_conv_weight(const void* w, int dtype, int64_t o, int64_t c, int kh, int kw,
                                   uint32_t* out, hipStream_t stream) {
  const int T = kh * kw;
  const int64_t CW = (c + 31) / 32;
  const int64_t total = o * T * CW;
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
  switch (dtype) {
    case kF32: hipLaunchKernelGGL(pack_conv_weight_kernel<kF32>, grid, block, 0, stream, w, out, total, c, T, CW); break;
    case kF16: hipLaunchKernelGGL(pack_conv_weight_kernel<kF16>, grid, block, 0, stream, w, out, total, c, T, CW); break;
    default: hipLaunchKernelGGL(pack_conv_weight_kernel<kBF16>, grid, block, 0, stream, w, out, total, c, T, CW); break;
  }
  return hipGetLastError();
}

namespace {

// 8-bit containers -> 32-bit words. Row r of src holds ceil(bits/8) bytes, bit j of byte q
// being sign 8q + j; row r of dst gets ceil(bits/32) words, word q = bytes 4q .. 4q + 3 in
// little-endian order (bytes past the row read as 0), and bits at or past `bits` in the last
// word are cleared, so a container whose unused high bits are not zero still gives words with
// the zero tail the contraction relies on. One thread per output word.
__global__ __launch_bounds__(256) void u8_to_words_kernel(const uint8_t* __restrict__ src,
                                                          uint32_t* __restrict__ dst,
                                                          int64_t total, int64_t nbytes,
                                                          int64_t nwords, uint32_t last_mask) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / nwords, q = i - r * nwords;
    const uint8_t* row = src + r * nbytes;
    uint32_t w = 0;
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const int64_t at = 4 * q + b;
      if (at < nbytes) w |= (uint32_t)row[at] << (8 * b);
    }
    if (q == nwords - 1) w &= last_mask;
    dst[i] = w;
  }
}

}  // namespace

hipError_t launch_u8_to_words(const uint8_t* src, int64_t rows, int64_t bits, uint32_t* dst,
                              hipStream_t stream) {
  const int64_t nbytes = (bits + 7) / 8, nwords = (bits + 31) / 32;
  const int64_t total = rows * nwords;
  if (total == 0) return hipSuccess;
  const uint32_t last_mask = bits % 32 == 0 ? 0xFFFFFFFFu : (1u << (bits % 32)) - 1u;
  const int64_t blocks = (total + 255) / 256;
  const dim3 grid((unsigned)(blocks < 65536 ? blocks : 65536)), block(256);
  hipLaunchKernelGGL(u8_to_words_kernel, grid, block, 0, stream, src, dst, total, nbytes, nwords,
                     last_mask);
  return hipGetLastError();
}

}  // namespace bnn
