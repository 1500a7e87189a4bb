// Device-side helpers shared by the libbnn kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

namespace bnn {

// Element / output type codes (numerically equal to include/bnn.h's bnn_dtype).
enum : int { kF32 = 0, kF16 = 1, kBF16 = 2, kI32 = 3, kPacked = 4, kPackedU8 = 5 };

// Sign bit of one element, from its raw IEEE bits: 1 when the value is >= 0
// (+0, -0, positive numbers, +inf), 0 otherwise (negative numbers, -inf, any
// NaN). Working on bits keeps the result independent of denormal modes.
__device__ __forceinline__ uint32_t pos_f32(uint32_t u) {
  return (uint32_t)(u <= 0x7F800000u) | (uint32_t)(u == 0x80000000u);
}
__device__ __forceinline__ uint32_t pos_f16(uint32_t h) {
  return (uint32_t)(h <= 0x7C00u) | (uint32_t)(h == 0x8000u);
}
__device__ __forceinline__ uint32_t pos_bf16(uint32_t b) {
  return (uint32_t)(b <= 0x7F80u) | (uint32_t)(b == 0x8000u);
}

// Sign bits of the two 16-bit elements in a dword (element 0 in the low half).
template <int DT>
__device__ __forceinline__ uint32_t pos2(uint32_t d) {
  if constexpr (DT == kF16)
    return pos_f16(d & 0xFFFFu) | (pos_f16(d >> 16) << 1);
  else
    return pos_bf16(d & 0xFFFFu) | (pos_bf16(d >> 16) << 1);
}

// Native 16-byte vector (usable with the nontemporal load builtin).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Sign bits of the elements in a 16-byte vector, element e at bit e
// (4 bits for f32, 8 bits for f16/bf16).
template <int DT>
__device__ __forceinline__ uint32_t vec_bits(u32x4 v) {
  if constexpr (DT == kF32) {
    return pos_f32(v.x) | (pos_f32(v.y) << 1) | (pos_f32(v.z) << 2) | (pos_f32(v.w) << 3);
  } else {
    return pos2<DT>(v.x) | (pos2<DT>(v.y) << 2) | (pos2<DT>(v.z) << 4) | (pos2<DT>(v.w) << 6);
  }
}

// Sign bit of one element read as raw bits from a typed array.
template <int DT>
__device__ __forceinline__ uint32_t elem_pos(const void* base, int64_t i) {
  if constexpr (DT == kF32)
    return pos_f32(reinterpret_cast<const uint32_t*>(base)[i]);
  else if constexpr (DT == kF16)
    return pos_f16(reinterpret_cast<const uint16_t*>(base)[i]);
  else
    return pos_bf16(reinterpret_cast<const uint16_t*>(base)[i]);
}

// Non-temporal 16-byte store, for output written once in whole 128-byte row segments:
// streaming such lines past the caches shortens the write-out at the end of a
// contraction (the whole output leaves at once). Scattered element stores (NCHW runs,
// ragged tails) stay ordinary stores, which the L2 merges into lines.
__device__ __forceinline__ void st_nt(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// One scaled output element: (float)acc * alpha rounded to the output type
// (round to nearest even), or the raw accumulator for kI32.
template <int OUT>
__device__ __forceinline__ void store1(void* out, int64_t idx, int acc, float alpha) {
  if constexpr (OUT == kF32) {
    reinterpret_cast<float*>(out)[idx] = (float)acc * alpha;
  } else if constexpr (OUT == kF16) {
    reinterpret_cast<__half*>(out)[idx] = __float2half_rn((float)acc * alpha);
  } else if constexpr (OUT == kBF16) {
    reinterpret_cast<__hip_bfloat16*>(out)[idx] = __float2bfloat16((float)acc * alpha);
  } else {
    reinterpret_cast<int*>(out)[idx] = acc;
  }
}

// Four consecutive output elements starting at idx (idx must be a multiple of 4).
template <int OUT>
__device__ __forceinline__ void store4(void* out, int64_t idx, int a0, int a1, int a2, int a3,
                                       float alpha) {
  if constexpr (OUT == kF32) {
    float4 v = make_float4((float)a0 * alpha, (float)a1 * alpha, (float)a2 * alpha,
                           (float)a3 * alpha);
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + idx) = v;
  } else if constexpr (OUT == kI32) {
    *reinterpret_cast<int4*>(reinterpret_cast<int*>(out) + idx) = make_int4(a0, a1, a2, a3);
  } else if constexpr (OUT == kF16) {
    __half h[4] = {__float2half_rn((float)a0 * alpha), __float2half_rn((float)a1 * alpha),
                   __float2half_rn((float)a2 * alpha), __float2half_rn((float)a3 * alpha)};
    *reinterpret_cast<uint2*>(reinterpret_cast<__half*>(out) + idx) =
        *reinterpret_cast<const uint2*>(h);
  } else {
    __hip_bfloat16 h[4] = {__float2bfloat16((float)a0 * alpha), __float2bfloat16((float)a1 * alpha),
                           __float2bfloat16((float)a2 * alpha), __float2bfloat16((float)a3 * alpha)};
    *reinterpret_cast<uint2*>(reinterpret_cast<__hip_bfloat16*>(out) + idx) =
        *reinterpret_cast<const uint2*>(h);
  }
}

// Output element type and a 4-element packed write (to LDS or memory) of scaled results.
template <int OUT> struct OutType;
template <> struct OutType<kF32> {
  using type = float;
  static __device__ __forceinline__ void put4(void* dst, int a0, int a1, int a2, int a3, float alpha) {
    *reinterpret_cast<float4*>(dst) = make_float4((float)a0 * alpha, (float)a1 * alpha,
                                                  (float)a2 * alpha, (float)a3 * alpha);
  }
};
template <> struct OutType<kI32> {
  using type = int;
  static __device__ __forceinline__ void put4(void* dst, int a0, int a1, int a2, int a3, float) {
    *reinterpret_cast<int4*>(dst) = make_int4(a0, a1, a2, a3);
  }
};
template <> struct OutType<kF16> {
  using type = __half;
  static __device__ __forceinline__ void put4(void* dst, int a0, int a1, int a2, int a3, float alpha) {
    __half h[4] = {__float2half_rn((float)a0 * alpha), __float2half_rn((float)a1 * alpha),
                   __float2half_rn((float)a2 * alpha), __float2half_rn((float)a3 * alpha)};
    *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(h);
  }
};
template <> struct OutType<kBF16> {
  using type = __hip_bfloat16;
  static __device__ __forceinline__ void put4(void* dst, int a0, int a1, int a2, int a3, float alpha) {
    __hip_bfloat16 h[4] = {__float2bfloat16((float)a0 * alpha), __float2bfloat16((float)a1 * alpha),
                           __float2bfloat16((float)a2 * alpha), __float2bfloat16((float)a3 * alpha)};
    *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(h);
  }
};

// Division of a non-negative int by a divisor fixed for the whole launch, without a division
// instruction: unsigned division by an invariant integer (Granlund and Montgomery, "Division by
// invariant integers using multiplication", 1994, figure 4.1). With l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, the quotient of any 0 <= n < 2^32 is
// (t + ((n - t) >> min(l, 1))) >> max(l - 1, 0) with t = the high word of m * n: a multiply
// and four cheap operations instead of the ~30-instruction integer division sequence.
struct FastDiv {
  uint32_t d = 1, m = 1, s1 = 0, s2 = 0;
  FastDiv() = default;
  explicit FastDiv(uint32_t div) : d(div) {
    uint32_t l = 0;
    while ((uint64_t(1) << l) < div) l++;
    m = (uint32_t)(((uint64_t(1) << 32) * ((uint64_t(1) << l) - div)) / div + 1);
    s1 = l > 0 ? 1 : 0;
    s2 = l > 0 ? l - 1 : 0;
  }
  __device__ __forceinline__ int div(int n) const {
    const uint32_t un = (uint32_t)n;
    const uint32_t t = __umulhi(m, un);
    return (int)((t + ((un - t) >> s1)) >> s2);
  }
};

// Shape of one contraction, shared by the GEMM and the implicit-im2col conv.
// Linear: A is packed activations [M][KW], W is packed weights [N][KW].
// Conv:   A is packed activations [B][H][W][CW] read through the implicit
//         im2col map; the reduction index q = tap * CW + cw with tap = kh*KWD + kw;
//         W is [N][KH][KWD][CW] = [N][KW]; M = B*Ho*Wo, output is NCHW.
// KB is the true number of signs per packed row (linear: K) or per tap (conv: C); when it is
// not a whole number of words, the last word of a row (of a tap) holds KB % 32 signs and
// zero bits above them in both operands.
struct Contraction {
  const uint32_t* a;
  const uint32_t* w;
  void* out;
  int M, N, KW;
  int KB;
  float alpha;
  // conv only
  // kernel KH x KWD, stride (SH, SW), padding (PH, PW), dilation (DH, DW) along (rows, columns)
  int H, W, CW, Ho, Wo, KH, KWD, SH, SW, PH, PW, DH, DW;
  // the same divisors for FastDiv: Ho * Wo, Wo, CW, KWD
  FastDiv div_hw, div_wo, div_cw, div_kwd;
  // matrix-core kernel: tiles along N of the launched tile shape (set by its launcher)
  FastDiv div_tn;
};

}  // namespace bnn
