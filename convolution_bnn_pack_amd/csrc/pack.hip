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

// NCHW pack along channels. Word (b, pixel, q) collects channel 32q + j of that pixel
// into bit j. A 256-thread workgroup packs 64*V consecutive pixels of one (b, q): lanes
// run along the contiguous pixel axis (V pixels each, one 16-byte load when the plane
// allows it, so each load instruction reads one channel plane contiguously), and wave w
// takes channels 8w .. 8w+7 of the word with its eight loads in flight at once. Each wave
// writes byte w of every pixel's word to LDS; the assembled words then leave in pixel order.
template <int DT, int V>
__global__ __launch_bounds__(256) void pack_nchw_kernel(const void* __restrict__ x,
                                                        uint32_t* __restrict__ out, int64_t C,
                                                        int64_t HW, int64_t CW, int64_t nbq) {
  constexpr int ES = (DT == kF32) ? 4 : 2;
  constexpr int PIX = 64 * V;                     // pixels per workgroup
  __shared__ uint32_t words[PIX];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nchunks = (HW + PIX - 1) / PIX;
  for (int64_t bq = blockIdx.y; bq < nbq; bq += gridDim.y) {
    const int64_t b = bq / CW, q = bq - b * CW;
    const char* plane0 = reinterpret_cast<const char*>(x) + ((b * C + 32 * q + 8 * wave) * HW) * ES;
    for (int64_t ch = blockIdx.x; ch < nchunks; ch += gridDim.x) {
      const int64_t base = ch * PIX;
      const int64_t p0 = base + (int64_t)lane * V;
      uint32_t bits[8];
#pragma unroll
      for (int c = 0; c < 8; c++) {
        const char* src = plane0 + ((int64_t)c * HW + p0) * ES;
        if constexpr (V * ES == 16) {
          bits[c] = (p0 < HW) ? vec_bits<DT>(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src))) : 0u;
        } else {
          uint32_t bb = 0;
#pragma unroll
          for (int v = 0; v < V; v++)
            if (p0 + v < HW) bb |= elem_pos<DT>(src, v) << v;
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

// OIHW weight pack: word (o, tap, q) collects w[o][32q + j][tap] into bit j.
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
  for (int j = 0; j < 32; j++) word |= elem_pos<DT>(w, ((o * C + 32 * q + j) * T) + t) << j;
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

hipError_t launch_pack_nchw(const void* x, int dtype, int64_t b, int64_t c, int64_t h, int64_t w,
                            uint32_t* out, hipStream_t stream) {
  const int64_t HW = h * w, CW = c / 32;
  if (b * HW * CW == 0) return hipSuccess;
  const int es = dtype == kF32 ? 4 : 2;
  const int vfull = 16 / es;
  const bool vec = (HW % vfull) == 0 && (reinterpret_cast<uintptr_t>(x) % 16) == 0;
  const int V = vec ? vfull : 1;
  const int64_t nchunks = (HW + 64 * V - 1) / (64 * V);
  const int64_t nbq = b * CW;
  const dim3 grid((unsigned)(nchunks < 65535 ? nchunks : 65535), (unsigned)(nbq < 65535 ? nbq : 65535)),
      block(256);
  if (vec) {
    switch (dtype) {
      case kF32: hipLaunchKernelGGL((pack_nchw_kernel<kF32, 4>), grid, block, 0, stream, x, out, c, HW, CW, nbq); break;
      case kF16: hipLaunchKernelGGL((pack_nchw_kernel<kF16, 8>), grid, block, 0, stream, x, out, c, HW, CW, nbq); break;
      default: hipLaunchKernelGGL((pack_nchw_kernel<kBF16, 8>), grid, block, 0, stream, x, out, c, HW, CW, nbq); break;
    }
  } else {
    switch (dtype) {
      case kF32: hipLaunchKernelGGL((pack_nchw_kernel<kF32, 1>), grid, block, 0, stream, x, out, c, HW, CW, nbq); break;
      case kF16: hipLaunchKernelGGL((pack_nchw_kernel<kF16, 1>), grid, block, 0, stream, x, out, c, HW, CW, nbq); break;
      default: hipLaunchKernelGGL((pack_nchw_kernel<kBF16, 1>), grid, block, 0, stream, x, out, c, HW, CW, nbq); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_pack_conv_weight(const void* w, int dtype, int64_t o, int64_t c, int ks,
                                   uint32_t* out, hipStream_t stream) {
  const int T = ks * ks;
  const int64_t CW = c / 32;
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

}  // namespace bnn
