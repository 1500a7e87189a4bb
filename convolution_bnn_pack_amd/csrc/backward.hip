// Straight-through backward of the binarized linear layer on the matrix cores.
//
// Both gradients are dense contractions of the 16-bit output gradient g with a
// matrix of signs (torch.sign: -1, 0, +1, NaN for NaN), so they run on the
// 32x32x16 bf16 / f16 MFMA with fp32 sums; every product is exact.
//   grad_input [M][K] = (scale_w * g[M][N] @ sign(W)[N][K]) * mid(x)
//   grad_weight[N][K] = scale_a * g^T[N][M] @ sign(x)[M][K]
// (BinaryConv2dForward.backward on the qconv/binary/cutlass/layer page, read
// with a 1x1 kernel, as the BinaryLinearForward page describes its backward.)
// mid is 0 where the fp32 quotient x / scale_a is below -1 or above 1 and 1
// elsewhere; the grad_input epilogue also forms each workgroup's double sum of
// grad_input * sign(x), and one more kernel reduces them into grad_scale_a.
//
// One kernel serves both: C[i][j] = scale * sum_r A(i, r) * sign(F[r][j]),
// where A is stored [I][R] (grad_input: g) or [R][I] (grad_weight: g read
// transposed) and F is [R][J] (W, or x). A 128x128 tile per workgroup of
// four waves (2x2, 64x64 each), 32-deep stages double-buffered in LDS with the
// reduction index innermost, so each lane's MFMA operand is one 16-byte read.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace bnn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#ifndef BWD_BK
#define BWD_BK 32
#endif
#ifndef BWD_BN
#define BWD_BN 128
#endif
constexpr int kBM = 128, kBN = BWD_BN, kBK = BWD_BK;
constexpr int kTJ = kBN / 64;    // 32-wide MFMA tiles per wave along j (each wave: 64 x kBN/2)
constexpr int kPitch = kBK + 8;  // u16 per LDS row: keeps rows 16-byte aligned, staggers banks
constexpr int kThreads = 256;

struct BwdArgs {
  const uint16_t* a;  // [I][R] or [R][I]
  const uint16_t* f;  // [R][J]; the operand is its sign
  const uint16_t* x;  // grad_input epilogue: x [I][J]
  float* out;         // [I][J]
  double* part;       // grad_input epilogue: one sum per workgroup
  int I, J, R;
  float scale;        // scale_w (grad_input) or scale_a (grad_weight)
  float scale_a;      // divisor of the clip test
  // split reduction: workgroup group s sums r in [s * rchunk, (s + 1) * rchunk) and writes its
  // partial result to out + s * out_split (rchunk = R: one group, the plain contraction)
  int rchunk = 0;
  int64_t out_split = 0;
};

// torch.sign of a 16-bit float, as bits of the same format.
template <bool BF>
__device__ inline uint32_t sign_bits(uint32_t v) {
  constexpr uint32_t inf = BF ? 0x7f80u : 0x7c00u, one = BF ? 0x3f80u : 0x3c00u,
                     nan = BF ? 0x7fc0u : 0x7e00u;
  const uint32_t a = v & 0x7fffu;
  return a == 0 ? 0u : (a > inf ? nan : ((v & 0x8000u) | one));
}

template <bool BF>
__device__ inline float widen16(uint16_t v) {
  if (BF) return __uint_as_float((uint32_t)v << 16);
  return (float)__ushort_as_half(v);
}

// 16-byte load from global memory. The pointers arrive inside a by-value argument struct, where
// the compiler no longer knows they are global and would issue flat loads, which it then waits on
// one by one; an explicit global pointer gives global loads that stay in flight.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ inline uint4 ldg16(const uint16_t* p) {
  const u32x4 v = *reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(
      reinterpret_cast<uintptr_t>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ inline uint16_t ldg2(const uint16_t* p) {
  return *reinterpret_cast<const __attribute__((address_space(1))) uint16_t*>(
      reinterpret_cast<uintptr_t>(p));
}

__device__ inline void stg4(float* p, float v) {
  *reinterpret_cast<__attribute__((address_space(1))) float*>(reinterpret_cast<uintptr_t>(p)) = v;
}

__device__ inline uint16_t u16_of(const uint4& v, int e) {
  const uint32_t w = e < 2 ? (e == 0 ? v.x : v.x >> 16) : e < 4 ? (e == 2 ? v.y : v.y >> 16)
                   : e < 6 ? (e == 4 ? v.z : v.z >> 16) : (e == 6 ? v.w : v.w >> 16);
  return (uint16_t)w;
}

template <bool BF>
__device__ inline void mfma(const uint16_t* pa, const uint16_t* pb, f32x16& acc) {
  if constexpr (BF) {
    const bf16x8 va = *reinterpret_cast<const bf16x8*>(pa);
    const bf16x8 vb = *reinterpret_cast<const bf16x8*>(pb);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, vb, acc, 0, 0, 0);
  } else {
    const f16x8 va = *reinterpret_cast<const f16x8*>(pa);
    const f16x8 vb = *reinterpret_cast<const f16x8*>(pb);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, vb, acc, 0, 0, 0);
  }
}

// AT: A stored [R][I]. GI: grad_input epilogue (clip mask, scale_a partial sums).
// Three waves per SIMD (at most 168 registers a lane): the grad_input epilogue would otherwise
// take the kernel to 177 and two waves, which leaves the LDS and barrier latency exposed.
#ifndef BWD_WAVES
#define BWD_WAVES 3
#endif
// SF: the sign is taken of F (false: F is used as it is, for a caller whose A already holds
// signs).
template <bool BF, bool AT, bool GI, bool SF = true>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(BWD_WAVES)))
void bwd_gemm_kernel(BwdArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kBM * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][kBN * kPitch];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_j = (p.J + kBN - 1) / kBN;
  const int tiles = ((p.I + kBM - 1) / kBM) * tiles_j;
  const int split = (int)blockIdx.x / tiles, tile = (int)blockIdx.x - split * tiles;
  const int i0 = (tile / tiles_j) * kBM, j0 = (tile % tiles_j) * kBN;
  // this workgroup's reduction range [r_lo, r_hi) and output slice
  const int r_lo = split * p.rchunk;
  const int r_hi = min(p.R, r_lo + p.rchunk);
  float* const out = p.out + split * p.out_split;
  const uint4 zero = make_uint4(0, 0, 0, 0);

  // Per stage: A [I][R] in 16-byte chunks (row, 8 consecutive r); A [R][I] and F [R][J] in
  // pairs of rows (2p, 2p + 1) of 8 consecutive columns, stored transposed as 32-bit pairs of
  // consecutive r so that the reduction index is innermost in LDS.
  constexpr int kRowChunks = kBK / 8;                       // A [I][R]: chunks per row
  constexpr int kNA = AT ? (kBK / 2) * (kBM / 8) / kThreads : kBM * kRowChunks / kThreads;
  constexpr int kNF = (kBK / 2) * (kBN / 8) / kThreads;     // F: row-pair chunks per thread
  static_assert(kNA >= 1 && kNF >= 1, "tile too small for the loader");
  // Transposed chunk c: its row pair and its 8-column chunk. Consecutive lanes take consecutive
  // row pairs, so a wave's 32-bit LDS stores (one LDS row per column) spread over the banks:
  // 2-way conflicts, where column-major lanes (rows 8 columns apart, 160 bytes) give 8-way.
  auto pair_of = [](int c) { return c % (kBK / 2); };
  auto col_of = [](int c) { return c / (kBK / 2); };
  uint4 ra[AT ? 2 * kNA : kNA], rf[2 * kNF];
  auto load = [&](int r0) {
    if constexpr (!AT) {
#pragma unroll
      for (int u = 0; u < kNA; u++) {
        const int c = tid + u * kThreads, row = c / kRowChunks, r = r0 + (c % kRowChunks) * 8;
        ra[u] = (i0 + row < p.I && r < r_hi) ? ldg16(p.a + (int64_t)(i0 + row) * p.R + r) : zero;
      }
    } else {
#pragma unroll
      for (int u = 0; u < kNA; u++) {
        const int c = tid + u * kThreads, i = i0 + col_of(c) * 8;
#pragma unroll
        for (int h = 0; h < 2; h++) {
          const int r = r0 + 2 * pair_of(c) + h;
          ra[2 * u + h] = (r < r_hi && i < p.I) ? ldg16(p.a + (int64_t)r * p.I + i) : zero;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kNF; u++) {
      const int c = tid + u * kThreads, j = j0 + col_of(c) * 8;
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const int r = r0 + 2 * pair_of(c) + h;
        rf[2 * u + h] = (r < r_hi && j < p.J) ? ldg16(p.f + (int64_t)r * p.J + j) : zero;
      }
    }
  };
  auto store = [&](int buf) {
    if constexpr (!AT) {
#pragma unroll
      for (int u = 0; u < kNA; u++) {
        const int c = tid + u * kThreads;
        *reinterpret_cast<uint4*>(&sA[buf][(c / kRowChunks) * kPitch + (c % kRowChunks) * 8]) = ra[u];
      }
    } else {
#pragma unroll
      for (int u = 0; u < kNA; u++) {
        const int c = tid + u * kThreads, rr = 2 * pair_of(c), ii = col_of(c) * 8;
#pragma unroll
        for (int e = 0; e < 8; e++)
          *reinterpret_cast<uint32_t*>(&sA[buf][(ii + e) * kPitch + rr]) =
              (uint32_t)u16_of(ra[2 * u], e) | ((uint32_t)u16_of(ra[2 * u + 1], e) << 16);
      }
    }
#pragma unroll
    for (int u = 0; u < kNF; u++) {
      const int c = tid + u * kThreads, rr = 2 * pair_of(c), jj = col_of(c) * 8;
#pragma unroll
      for (int e = 0; e < 8; e++)
        *reinterpret_cast<uint32_t*>(&sB[buf][(jj + e) * kPitch + rr]) =
            SF ? sign_bits<BF>(u16_of(rf[2 * u], e)) | (sign_bits<BF>(u16_of(rf[2 * u + 1], e)) << 16)
               : (uint32_t)u16_of(rf[2 * u], e) | ((uint32_t)u16_of(rf[2 * u + 1], e) << 16);
    }
  };

  f32x16 acc[2][kTJ];
#pragma unroll
  for (int a = 0; a < 2; a++)
#pragma unroll
    for (int b = 0; b < kTJ; b++)
#pragma unroll
      for (int v = 0; v < 16; v++) acc[a][b][v] = 0.0f;

  const int nk = r_hi > r_lo ? (r_hi - r_lo + kBK - 1) / kBK : 0;
  if (nk > 0) {
    load(r_lo);
    store(0);
  }
  __syncthreads();
  const int half = (lane >> 5) * 8, l32 = lane & 31;
  for (int kt = 0; kt < nk; kt++) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load(r_lo + (kt + 1) * kBK);
#pragma unroll
    for (int ks = 0; ks < kBK; ks += 16) {
#pragma unroll
      for (int ti = 0; ti < 2; ti++)
#pragma unroll
        for (int tj = 0; tj < kTJ; tj++)
          mfma<BF>(&sA[buf][(wm * 64 + ti * 32 + l32) * kPitch + ks + half],
                   &sB[buf][(wn * (kBN / 2) + tj * 32 + l32) * kPitch + ks + half], acc[ti][tj]);
    }
    if (kt + 1 < nk) store(buf ^ 1);
    __syncthreads();
  }

  // Lane (l32, half) of tile (ti, tj) holds column j = .. + l32 and rows 8g + half/2 + t.
  double part = 0.0;
#pragma unroll
  for (int ti = 0; ti < 2; ti++)
#pragma unroll
    for (int tj = 0; tj < kTJ; tj++) {
      const int j = j0 + wn * (kBN / 2) + tj * 32 + l32;
#pragma unroll
      for (int v = 0; v < 16; v++) {
        const int i = i0 + wm * 64 + ti * 32 + 8 * (v >> 2) + (half >> 1) + (v & 3);
        if (i >= p.I || j >= p.J) continue;
        const int64_t o = (int64_t)i * p.J + j;
        float val = acc[ti][tj][v] * p.scale;
        if constexpr (GI) {
          const float xv = widen16<BF>(ldg2(p.x + o));
          const float q = xv / p.scale_a;
          val *= 1.0f - (q < -1.0f ? 1.0f : 0.0f) - (q > 1.0f ? 1.0f : 0.0f);
          const double s = xv != xv ? (double)NAN : (xv > 0.0f ? 1.0 : (xv < 0.0f ? -1.0 : 0.0));
          part += (double)val * s;
        }
        stg4(out + o, val);
      }
    }
  if constexpr (GI) {
    __shared__ double red[kThreads];
    red[tid] = part;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
      if (tid < s) red[tid] += red[tid + s];
      __syncthreads();
    }
    if (tid == 0) p.part[blockIdx.x] = red[0];
  }
}

// grad_scale_a = (sum of the workgroup sums, in double) / sqrt(count).
__global__ __launch_bounds__(kThreads) void bwd_scale_a_kernel(const double* part, int n,
                                                                double count, double* out) {
  __shared__ double red[kThreads];
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += kThreads) s += part[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int h = kThreads / 2; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = red[0] / sqrt(count);
}

// ---- int8 codes of grad_w: amax = max |v| (NaN if any v is NaN), step = amax / 127, code =
// clamp(rint(v / step), -127, 127), a NaN quotient coding as 0 (the same symmetric quantizer as
// the W8A8 conv, its amax taken from the gradient itself).
constexpr int kAmaxParts = 1024;

__device__ inline float nan_max(float a, float b) { return a != a ? a : (b != b ? b : fmaxf(a, b)); }

__device__ inline float block_nan_max(float v, float* red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int h = kThreads / 2; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) red[threadIdx.x] = nan_max(red[threadIdx.x], red[threadIdx.x + h]);
    __syncthreads();
  }
  return red[0];
}

__device__ inline float abs_max4(const float4& q) {
  return nan_max(nan_max(fabsf(q.x), fabsf(q.y)), nan_max(fabsf(q.z), fabsf(q.w)));
}

__global__ __launch_bounds__(kThreads) void bwd_amax_kernel(const float4* v, int64_t n4, float* part) {
  __shared__ float red[kThreads];
  float m = 0.0f;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  // four independent 16-byte loads in flight per thread, then the remainder one at a time
  for (; i + 3 * stride < n4; i += 4 * stride) {
    const float4 q0 = v[i], q1 = v[i + stride], q2 = v[i + 2 * stride], q3 = v[i + 3 * stride];
    m = nan_max(m, nan_max(nan_max(abs_max4(q0), abs_max4(q1)), nan_max(abs_max4(q2), abs_max4(q3))));
  }
  for (; i < n4; i += stride) m = nan_max(m, abs_max4(v[i]));
  const float b = block_nan_max(m, red);
  if (threadIdx.x == 0) part[blockIdx.x] = b;
}

__global__ __launch_bounds__(kThreads) void bwd_amax_final_kernel(const float* part, int n, float* amax) {
  __shared__ float red[kThreads];
  float m = 0.0f;
  for (int i = threadIdx.x; i < n; i += kThreads) m = nan_max(m, part[i]);
  const float b = block_nan_max(m, red);
  if (threadIdx.x == 0) amax[0] = b;
}

__device__ inline int8_t grad_code(float v, float step) {
  float r = rintf(v / step);
  r = r != r ? 0.0f : fminf(fmaxf(r, -127.0f), 127.0f);
  return (int8_t)r;
}

__global__ __launch_bounds__(kThreads) void bwd_quant_kernel(const float4* v, int64_t n4, const float* amax,
                                                             char4* codes) {
  const float step = amax[0] / 127.0f;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += (int64_t)gridDim.x * kThreads) {
    const float4 q = v[i];
    codes[i] = make_char4(grad_code(q.x, step), grad_code(q.y, step), grad_code(q.z, step),
                          grad_code(q.w, step));
  }
}

int amax_parts(int64_t n4) {
  const int64_t blocks = (n4 + 4 * kThreads - 1) / (4 * kThreads);  // four vectors per thread
  return (int)(blocks < 1 ? 1 : (blocks > kAmaxParts ? kAmaxParts : blocks));
}

// A reduction of length R cut into at most `splits` chunks of whole kBK-stages: chunk length
// rchunk and the number of chunks used (asking again for `used` chunks gives the same plan).
struct SplitPlan {
  int rchunk, used;
};
SplitPlan split_plan(int64_t R, int splits) {
  if (R <= 0) return {1, 1};
  if (splits < 1) splits = 1;
  const int64_t stages = (R + kBK - 1) / kBK;
  const int64_t per = (stages + splits - 1) / splits;
  const int64_t chunk = per * kBK > R ? R : per * kBK;
  return {(int)chunk, (int)((R + chunk - 1) / chunk)};
}

// splits > 1 (no grad_input epilogue): the reduction range is cut as split_plan(R, splits) says,
// each chunk writing its partial contraction to out + s * I * J.
template <bool AT, bool GI, bool SF = true>
hipError_t launch_bwd(bool bf, BwdArgs a, hipStream_t s, int splits = 1) {
  const int64_t tiles = (int64_t)((a.I + kBM - 1) / kBM) * ((a.J + kBN - 1) / kBN);
  if (tiles == 0) return hipSuccess;
  const SplitPlan plan = split_plan(a.R, GI ? 1 : splits);
  a.rchunk = plan.rchunk;
  a.out_split = (int64_t)a.I * a.J;
  const dim3 grid((unsigned)(tiles * plan.used));
  if (bf)
    hipLaunchKernelGGL((bwd_gemm_kernel<true, AT, GI, SF>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_gemm_kernel<false, AT, GI, SF>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

// ---- Conv backward (BinaryConv2dForward.backward on the qconv/binary/cutlass/layer page): the
// page's conv2d_input and conv2d_weight, each lowered to the contraction above.
//   grad_input: colsT[c*T + t][pix] = scale_w * sum_o sign(W[o][c][t]) * g[b][o][pix] for every
//   output pixel pix = (b, oh, ow) and tap t = kh*KW + kw (sign(W) formed once, the columns
//   stored pixel-contiguous so the gather below reads them in runs), then each input element
//   gathers the columns whose tap lands on it (col2im), is multiplied by the clip mask, and adds
//   its grad_input * sign(x) to its workgroup's double sum.
//   grad_weight: GW[o][c*T + t] = scale_a * sum_pix g[b][o][pix] * sign(xcol[pix][c*T + t]),
//   xcol the unfolded input (0 where the tap falls in the padding), i.e. OIHW directly; the
//   pixel axis is long and the output small, so the contraction is split along the pixels and
//   the partial results are summed in a fixed order.
// g is first copied to [O][B*Ho*Wo] so both contractions read it as a plain matrix.

struct ConvGeom {
  int B, C, H, W, O, KH, KW, SH, SW, PH, PW, DH, DW, Ho, Wo;
};

// g NCHW [B][O][Ho*Wo] -> gT [O][B*Ho*Wo]: one contiguous run of Ho*Wo per (b, o), copied by a
// workgroup per run.
// VW-byte vectors (VW / 2 elements, hw a multiple of them): thread t copies vector t of the
// flattened (run, vector) space, so a wave moves 64 * VW consecutive bytes whatever the run length.
template <int VW>
__global__ __launch_bounds__(kThreads) void conv_g_transpose_kernel(const uint16_t* __restrict__ g,
                                                                   uint16_t* __restrict__ gT,
                                                                   int B, int O, int hw,
                                                                   FastDiv div_vpr, FastDiv div_o) {
  using V = std::conditional_t<VW == 16, uint4, std::conditional_t<VW == 8, uint2,
                               std::conditional_t<VW == 4, uint32_t, uint16_t>>>;
  constexpr int E = VW / 2;
  const int vpr = hw / E;
  const int64_t total = (int64_t)B * O * vpr;
  for (int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x; v < total;
       v += (int64_t)gridDim.x * kThreads) {
    // total < 2^31: the C ABI checks o * pixels
    const int run = div_vpr.div((int)v), within = (int)v - run * vpr;
    const int b = div_o.div(run), o = run - b * O;
    const V val = *reinterpret_cast<const V*>(g + (int64_t)run * hw + within * E);
    *reinterpret_cast<V*>(gT + ((int64_t)o * B + b) * hw + within * E) = val;
  }
}

// xcol[pix][c*T + t] = x[b][c][oh*SH - PH + kh*DH][ow*SW - PW + kw*DW], 0 outside the input. A
// thread fills 8 consecutive columns of one pixel with one 16-byte store (C*T is a multiple of
// 8), so a wave writes 1 KB of consecutive bytes; the gathered reads of x hit the caches.
__global__ __launch_bounds__(kThreads) void conv_im2col_kernel(const uint16_t* __restrict__ x,
                                                              uint16_t* __restrict__ xcol,
                                                              ConvGeom q, FastDiv div_t,
                                                              FastDiv div_kw) {
  const int T = q.KH * q.KW, hwo = q.Ho * q.Wo;
  const int64_t pixels = (int64_t)q.B * hwo;
  const int J = q.C * T, J8 = J / 8;
  const int64_t total = pixels * J8;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t pix = i / J8;
    const int j0 = (int)(i - pix * J8) * 8;
    const int b = (int)(pix / hwo), r = (int)(pix - (int64_t)b * hwo);
    const int oh = r / q.Wo, ow = r - oh * q.Wo;
    uint32_t v[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      uint32_t pair = 0;
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const int jj = j0 + e + h;
        const int c = div_t.div(jj), t = jj - c * T;
        const int kh = div_kw.div(t), kw = t - kh * q.KW;
        const int ih = oh * q.SH - q.PH + kh * q.DH, iw = ow * q.SW - q.PW + kw * q.DW;
        const bool in = ih >= 0 && ih < q.H && iw >= 0 && iw < q.W;
        const uint32_t val = in ? x[(((int64_t)b * q.C + c) * q.H + ih) * q.W + iw] : 0u;
        pair |= val << (16 * h);
      }
      v[e / 2] = pair;
    }
    *reinterpret_cast<uint4*>(xcol + pix * J + j0) = make_uint4(v[0], v[1], v[2], v[3]);
  }
}

// out[i] = torch.sign of the 16-bit w[i], as bits of the same format.
template <bool BF>
__global__ __launch_bounds__(kThreads) void sign16_kernel(const uint16_t* __restrict__ w,
                                                         uint16_t* __restrict__ out, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads)
    out[i] = (uint16_t)sign_bits<BF>(w[i]);
}

// grad_w[i] = sum over the splits s = 0, 1, ... of part[s][i], in that order.
__global__ __launch_bounds__(kThreads) void split_sum_kernel(const float* __restrict__ part,
                                                            float* __restrict__ out, int64_t n,
                                                            int splits) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads) {
    float v = 0.0f;
    for (int sp = 0; sp < splits; sp++) v += part[(int64_t)sp * n + i];
    out[i] = v;
  }
}

// The same unfolding, 32 pixels (consecutive rows of xcol) per workgroup through LDS, for column
// counts whose 32 rows fit in LDS. Gathered straight into 16-byte stores, each lane's 8 columns are
// 8 different channel planes or taps, so a load instruction touches 64 memory lines. Here the 32
// lanes of a half-wave take the 32 pixels of one column pair: consecutive output pixels of one row
// read neighbouring input elements, a line or two per instruction. Each pair goes to LDS as one
// dword (rows of RS = (J/2) | 1 dwords: an odd stride keeps the 32 rows in 32 banks); then the
// tile's 32 * J * 2 contiguous bytes of xcol leave as 16-byte stores. Column counts with
// RS > kIm2colMaxRS take the direct gather above.
constexpr int kIm2colPix = 32;
constexpr int kIm2colMaxRS = 640;  // 80 KiB of LDS: two workgroups per compute unit
__global__ __launch_bounds__(kThreads) void conv_im2col_tile_kernel(const uint16_t* __restrict__ x,
                                                                   uint16_t* __restrict__ xcol,
                                                                   ConvGeom q, FastDiv div_t,
                                                                   FastDiv div_kw, FastDiv div_hwo,
                                                                   FastDiv div_wo, FastDiv div_j8) {
  __shared__ uint32_t tile[kIm2colPix * kIm2colMaxRS];
  const int T = q.KH * q.KW, J = q.C * T, JP = J / 2, RS = JP | 1;
  const int hwo = q.Ho * q.Wo, pixels = q.B * hwo;
  const int ntiles = (pixels + kIm2colPix - 1) / kIm2colPix;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int p = lane & 31, sub = lane >> 5;
  for (int tl = blockIdx.x; tl < ntiles; tl += gridDim.x) {
    const int pix = tl * kIm2colPix + p;
    const bool pok = pix < pixels;
    const int b = div_hwo.div(pok ? pix : 0), r = (pok ? pix : 0) - b * hwo;
    const int oh = div_wo.div(r), ow = r - oh * q.Wo;
    const int ihb = oh * q.SH - q.PH, iwb = ow * q.SW - q.PW;
    const uint16_t* xb = x + (int64_t)b * q.C * q.H * q.W;
    // column pairs jp = 2 * wave + sub + 8 * i, kU pairs at a time: all 2 * kU loads go out
    // (clamped to element 0 where the tap falls outside, so none sits behind a branch) before
    // any is used
    constexpr int kU = 8;
    for (int jb = 2 * wave + sub; jb < JP; jb += 8 * kU) {
      uint32_t val[kU][2];
      bool in[kU][2];
#pragma unroll
      for (int u = 0; u < kU; u++)
#pragma unroll
        for (int h = 0; h < 2; h++) {
          const int jp = jb + 8 * u, j = 2 * jp + h;
          const int c = div_t.div(j), t = j - c * T;
          const int kh = div_kw.div(t), kw = t - kh * q.KW;
          const int ih = ihb + kh * q.DH, iw = iwb + kw * q.DW;
          in[u][h] = pok && jp < JP && ih >= 0 && ih < q.H && iw >= 0 && iw < q.W;
          val[u][h] = xb[in[u][h] ? ((int64_t)c * q.H + ih) * q.W + iw : 0];
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kU; u++) {
        const int jp = jb + 8 * u;
        if (jp < JP)
          tile[p * RS + jp] = (in[u][0] ? val[u][0] : 0u) | ((in[u][1] ? val[u][1] : 0u) << 16);
      }
    }
    __syncthreads();
    const int rows = pixels - tl * kIm2colPix < kIm2colPix ? pixels - tl * kIm2colPix : kIm2colPix;
    const int J8 = J / 8, nchunk = rows * J8;
    uint16_t* dst = xcol + (int64_t)tl * kIm2colPix * J;
    for (int k = threadIdx.x; k < nchunk; k += kThreads) {
      const int row = div_j8.div(k), cq = k - row * J8;
      const uint32_t* src = tile + row * RS + 4 * cq;
      *reinterpret_cast<uint4*>(dst + (int64_t)k * 8) = make_uint4(src[0], src[1], src[2], src[3]);
    }
    __syncthreads();
  }
}

// grad_in[b][c][ih][iw] = mid(x) * sum of colsT[c*T + t][(b, oh, ow)] over the taps t whose output
// pixel (oh, ow) = ((ih + PH - kh*DH) / SH, (iw + PW - kw*DW) / SW) exists (exact divisions, in
// range), in tap order; each workgroup writes its double sum of grad_in * sign(x) (a fixed grid,
// so the order of every sum is fixed).
// Divisions by launch-invariant sizes of the col2im gather (every index fits in int: the C ABI
// checks n*c*h*w and the column matrix's size).
struct Col2imDivs {
  FastDiv w, h, c, sh, sw, kw;
};

// SMALL: at most 9 taps (kh * kw <= 9), gathered with all loads in flight.
template <bool BF, bool SMALL>
__global__ __launch_bounds__(kThreads) void conv_col2im_kernel(const float* __restrict__ cols,
                                                              const uint16_t* __restrict__ x,
                                                              float* __restrict__ grad_in,
                                                              double* __restrict__ part, ConvGeom q,
                                                              Col2imDivs dv, float scale_a) {
  const int T = q.KH * q.KW;
  const int pixels = q.B * q.Ho * q.Wo;
  const int total = q.B * q.C * q.H * q.W;
  double sum = 0.0;
  for (int64_t ii = (int64_t)blockIdx.x * kThreads + threadIdx.x; ii < total;
       ii += (int64_t)gridDim.x * kThreads) {
    const int i = (int)ii;
    const int r1 = dv.w.div(i), iw = i - r1 * q.W;
    const int r2 = dv.h.div(r1), ih = r1 - r2 * q.H;
    const int b = dv.c.div(r2), c = r2 - b * q.C;
    const float* col_c = cols + (int64_t)c * T * pixels + b * q.Ho * q.Wo;
    float v = 0.0f;
    if constexpr (SMALL) {
      // up to 9 taps: every tap's column is loaded (clamped to the plane's first pixel where the
      // tap has no output pixel) before any is added, then the valid ones are added in tap
      // order (adding +0 for the others leaves v unchanged: v starts at +0 and is never -0)
      float tv[9];
      bool ok[9];
#pragma unroll
      for (int t = 0; t < 9; t++) {
        const int kh = t < T ? dv.kw.div(t) : 0, kw = t - kh * q.KW;
        const int nh = ih + q.PH - kh * q.DH, nw = iw + q.PW - kw * q.DW;
        const int oh = dv.sh.div(nh < 0 ? 0 : nh), ow = dv.sw.div(nw < 0 ? 0 : nw);
        ok[t] = t < T && nh >= 0 && nw >= 0 && oh * q.SH == nh && ow * q.SW == nw && oh < q.Ho &&
                ow < q.Wo;
        tv[t] = col_c[ok[t] ? (int64_t)t * pixels + oh * q.Wo + ow : 0];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 9; t++) v += ok[t] ? tv[t] : 0.0f;
    } else {
      for (int kh = 0; kh < q.KH; kh++) {
        const int nh = ih + q.PH - kh * q.DH;
        if (nh < 0) continue;
        const int oh = dv.sh.div(nh);
        if (oh * q.SH != nh || oh >= q.Ho) continue;
        for (int kw = 0; kw < q.KW; kw++) {
          const int nw = iw + q.PW - kw * q.DW;
          if (nw < 0) continue;
          const int ow = dv.sw.div(nw);
          if (ow * q.SW != nw || ow >= q.Wo) continue;
          v += col_c[(int64_t)(kh * q.KW + kw) * pixels + oh * q.Wo + ow];
        }
      }
    }
    const float xv = widen16<BF>(x[i]);
    const float qv = xv / scale_a;
    v *= 1.0f - (qv < -1.0f ? 1.0f : 0.0f) - (qv > 1.0f ? 1.0f : 0.0f);
    grad_in[i] = v;
    const double sg = xv != xv ? (double)NAN : (xv > 0.0f ? 1.0 : (xv < 0.0f ? -1.0 : 0.0));
    sum += (double)v * sg;
  }
  __shared__ double red[kThreads];
  red[threadIdx.x] = sum;
  __syncthreads();
  for (int h = kThreads / 2; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

constexpr int kCol2imBlocks = 2048;

int64_t grid_of(int64_t total, int64_t cap) {
  const int64_t b = (total + kThreads - 1) / kThreads;
  return b < 1 ? 1 : (b > cap ? cap : b);
}

}  // namespace

int64_t bwd_grad_input_parts(int64_t m, int64_t k) {
  return ((m + kBM - 1) / kBM) * ((k + kBN - 1) / kBN);
}

hipError_t launch_linear_grad_input(const void* g, const void* w, const void* x, bool bf,
                                    int64_t m, int64_t n, int64_t k, float scale_a, float scale_w,
                                    float* grad_in, double* part, double* grad_scale_a,
                                    hipStream_t s) {
  BwdArgs a{static_cast<const uint16_t*>(g), static_cast<const uint16_t*>(w),
            static_cast<const uint16_t*>(x), grad_in, part, (int)m, (int)k, (int)n, scale_w, scale_a};
  hipError_t e = launch_bwd<false, true>(bf, a, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_scale_a_kernel, dim3(1), dim3(kThreads), 0, s, part,
                     (int)bwd_grad_input_parts(m, k), (double)m * (double)k, grad_scale_a);
  return hipGetLastError();
}

int64_t bwd_grad_weight_i8_parts(int64_t n, int64_t k) { return amax_parts(n * k / 4); }

int64_t bwd_quant_grad_parts(int64_t count) { return amax_parts(count / 4); }

hipError_t launch_quant_grad(const float* grad_w, int64_t count, float* part, float* amax,
                             int8_t* codes, hipStream_t s) {
  const int64_t n4 = count / 4;
  const int parts = amax_parts(n4);
  hipLaunchKernelGGL(bwd_amax_kernel, dim3(parts), dim3(kThreads), 0, s,
                     reinterpret_cast<const float4*>(grad_w), n4, part);
  hipLaunchKernelGGL(bwd_amax_final_kernel, dim3(1), dim3(kThreads), 0, s, part, parts, amax);
  const int64_t qblocks = (n4 + 4 * kThreads - 1) / (4 * kThreads);
  hipLaunchKernelGGL(bwd_quant_kernel, dim3((unsigned)(qblocks < 1 ? 1 : (qblocks > 8192 ? 8192 : qblocks))),
                     dim3(kThreads), 0, s, reinterpret_cast<const float4*>(grad_w), n4, amax,
                     reinterpret_cast<char4*>(codes));
  return hipGetLastError();
}

hipError_t launch_linear_grad_weight(const void* g, const void* x, bool bf, int64_t m, int64_t n,
                                     int64_t k, float scale_a, float* grad_w, hipStream_t s) {
  BwdArgs a{static_cast<const uint16_t*>(g), static_cast<const uint16_t*>(x), nullptr, grad_w,
            nullptr, (int)n, (int)k, (int)m, scale_a, scale_a};
  return launch_bwd<true, false>(bf, a, s);
}

// ---- conv backward launchers

// g NCHW -> gT [O][B*Ho*Wo] with the widest vectors that the plane size and g's alignment allow
// (gT, in the workspace, is 256-byte aligned).
void launch_g_transpose(const uint16_t* g, uint16_t* gT, int B, int O, int hw, hipStream_t s) {
  const uintptr_t ga = reinterpret_cast<uintptr_t>(g);
  int e = 8;
  while (e > 1 && (hw % e != 0 || ga % (2 * e) != 0)) e /= 2;
  const int64_t total = (int64_t)B * O * (hw / e);
  const dim3 grid((unsigned)grid_of(total, 16384)), block(kThreads);
  const FastDiv dv((uint32_t)(hw / e)), dO((uint32_t)O);
  switch (e) {
    case 8: hipLaunchKernelGGL(conv_g_transpose_kernel<16>, grid, block, 0, s, g, gT, B, O, hw, dv, dO); break;
    case 4: hipLaunchKernelGGL(conv_g_transpose_kernel<8>, grid, block, 0, s, g, gT, B, O, hw, dv, dO); break;
    case 2: hipLaunchKernelGGL(conv_g_transpose_kernel<4>, grid, block, 0, s, g, gT, B, O, hw, dv, dO); break;
    default: hipLaunchKernelGGL(conv_g_transpose_kernel<2>, grid, block, 0, s, g, gT, B, O, hw, dv, dO); break;
  }
}

int64_t conv_col2im_parts(int64_t n, int64_t c, int64_t h, int64_t w) {
  return grid_of(n * c * h * w, kCol2imBlocks);
}

int conv_wgrad_splits(int64_t o, int64_t j, int64_t pixels) {
  const int64_t tiles = ((o + kBM - 1) / kBM) * ((j + kBN - 1) / kBN);
  int64_t sp = (512 + tiles - 1) / tiles;   // about two workgroups per compute unit
  // the number of chunks of whole stages launch_bwd actually makes of that request
  return split_plan(pixels, sp > 0x7fffffff ? 0x7fffffff : (int)sp).used;
}

hipError_t launch_conv_grad_input(const void* g, const void* w, const void* x, bool bf,
                                  const int geom[15], float scale_a, float scale_w, float* grad_in,
                                  uint16_t* gT, uint16_t* wsign, float* cols, double* part,
                                  double* grad_scale_a, hipStream_t s) {
  const ConvGeom q{geom[0], geom[1], geom[2], geom[3], geom[4], geom[5], geom[6], geom[7],
                   geom[8], geom[9], geom[10], geom[11], geom[12], geom[13], geom[14]};
  const int hwo = q.Ho * q.Wo, T = q.KH * q.KW, J = q.C * T;
  launch_g_transpose(static_cast<const uint16_t*>(g), gT, q.B, q.O, hwo, s);
  const int64_t nw = (int64_t)q.O * J;
  if (bf)
    hipLaunchKernelGGL(sign16_kernel<true>, dim3((unsigned)grid_of(nw, 4096)), dim3(kThreads), 0, s,
                       static_cast<const uint16_t*>(w), wsign, nw);
  else
    hipLaunchKernelGGL(sign16_kernel<false>, dim3((unsigned)grid_of(nw, 4096)), dim3(kThreads), 0, s,
                       static_cast<const uint16_t*>(w), wsign, nw);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // colsT [C*T][B*Ho*Wo] = scale_w * sign(W)^T @ gT: A = sign(W) stored [O][C*T], F = gT used as is
  BwdArgs a{wsign, gT, nullptr, cols, nullptr, J, q.B * hwo, q.O, scale_w, scale_a};
  e = launch_bwd<true, false, false>(bf, a, s);
  if (e != hipSuccess) return e;
  const int64_t total = (int64_t)q.B * q.C * q.H * q.W;
  const int parts = (int)grid_of(total, kCol2imBlocks);
  const Col2imDivs dv{FastDiv((uint32_t)q.W), FastDiv((uint32_t)q.H), FastDiv((uint32_t)q.C),
                      FastDiv((uint32_t)q.SH), FastDiv((uint32_t)q.SW), FastDiv((uint32_t)q.KW)};
  const uint16_t* xs = static_cast<const uint16_t*>(x);
  if (T <= 9) {
    if (bf)
      hipLaunchKernelGGL((conv_col2im_kernel<true, true>), dim3(parts), dim3(kThreads), 0, s, cols, xs,
                         grad_in, part, q, dv, scale_a);
    else
      hipLaunchKernelGGL((conv_col2im_kernel<false, true>), dim3(parts), dim3(kThreads), 0, s, cols, xs,
                         grad_in, part, q, dv, scale_a);
  } else {
    if (bf)
      hipLaunchKernelGGL((conv_col2im_kernel<true, false>), dim3(parts), dim3(kThreads), 0, s, cols, xs,
                         grad_in, part, q, dv, scale_a);
    else
      hipLaunchKernelGGL((conv_col2im_kernel<false, false>), dim3(parts), dim3(kThreads), 0, s, cols, xs,
                         grad_in, part, q, dv, scale_a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_scale_a_kernel, dim3(1), dim3(kThreads), 0, s, part, parts,
                     (double)total, grad_scale_a);
  return hipGetLastError();
}

hipError_t launch_conv_grad_weight(const void* g, const void* x, bool bf, const int geom[15],
                                   float scale_a, float* grad_w, uint16_t* gT, uint16_t* xcol,
                                   float* split_part, hipStream_t s) {
  const ConvGeom q{geom[0], geom[1], geom[2], geom[3], geom[4], geom[5], geom[6], geom[7],
                   geom[8], geom[9], geom[10], geom[11], geom[12], geom[13], geom[14]};
  const int hwo = q.Ho * q.Wo, T = q.KH * q.KW, J = q.C * T;
  launch_g_transpose(static_cast<const uint16_t*>(g), gT, q.B, q.O, hwo, s);
  if (((J / 2) | 1) <= kIm2colMaxRS) {
    const int64_t ntiles = ((int64_t)q.B * hwo + kIm2colPix - 1) / kIm2colPix;
    hipLaunchKernelGGL(conv_im2col_tile_kernel, dim3((unsigned)(ntiles < 65535 ? ntiles : 65535)),
                       dim3(kThreads), 0, s, static_cast<const uint16_t*>(x), xcol, q,
                       FastDiv((uint32_t)T), FastDiv((uint32_t)q.KW), FastDiv((uint32_t)hwo),
                       FastDiv((uint32_t)q.Wo), FastDiv((uint32_t)(J / 8)));
  } else {
    hipLaunchKernelGGL(conv_im2col_kernel, dim3((unsigned)grid_of((int64_t)q.B * hwo * (J / 8), 16384)),
                       dim3(kThreads), 0, s, static_cast<const uint16_t*>(x), xcol, q,
                       FastDiv((uint32_t)T), FastDiv((uint32_t)q.KW));
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // GW [O][C*T] = scale_a * gT @ sign(xcol), split along the pixels, then the splits summed
  const int splits = conv_wgrad_splits(q.O, J, (int64_t)q.B * hwo);
  BwdArgs a{gT, xcol, nullptr, splits > 1 ? split_part : grad_w, nullptr, q.O, J, q.B * hwo,
            scale_a, scale_a};
  e = launch_bwd<false, false>(bf, a, s, splits);
  if (e != hipSuccess || splits == 1) return e;
  const int64_t n = (int64_t)q.O * J;
  hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)grid_of(n, 4096)), dim3(kThreads), 0, s,
                     split_part, grad_w, n, splits);
  return hipGetLastError();
}

}  // namespace bnn
