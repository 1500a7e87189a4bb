// Binary contraction on the gfx950 matrix cores, with the signs expanded to
// int8 or to fp4 (e2m1) operands.
//
// The binary dot product is a dense contraction, so it runs on
// v_mfma_i32_32x32x32_i8 (32x32 output block, 32-deep reduction, int32
// sums) or on v_mfma_scale_f32_32x32x64_f8f6f4 with both operands fp4 and
// unit scales (64-deep reduction at twice the int8 rate, fp32 sums). Signs
// stay bit-packed in HBM; a workgroup loads the packed words of its A
// (activation) and W (weight) tiles and expands each word in registers before
// storing it to LDS.
//
// int8: dword d (d = 0..7) of a word's 32 expanded bytes holds bits d, d+8,
// d+16, d+24, one per byte:
//
//   t_d = (w >> d) & 0x01010101                   (bytes 0 / 1)
//   W bytes  w' = t_d = b
//   A bytes  a' = v_perm_b32(0, 0x000001FF, t_d)  (selector byte 0 or 1 picks
//            0xFF or 0x01, so a' = 2b - 1 = s), or a table of 0 for a padded
//            conv tap or a position past K (every byte 0).
//
// The byte order is a fixed permutation of the word's 32 reduction indices,
// the same for A and W, so the sums are unchanged. With b the packed bit (1
// for a +1 sign) and s = 2b - 1, the MFMA sum is sum a'w' = sum s_a b_w over
// the real terms, and since s_w = 2 b_w - 1 the binary dot product is
//   dot = sum s_a s_w = 2 * mfma - sum s_a = K_valid - 2 * popA + 2 * mfma,
// with popA the number of set bits among the row's real A words and K_valid
// = 32 * (number of real A words). Both are counted by the thread that loads
// the row, so padded taps need no per-weight correction. Expanding a word
// costs 15 VALU operations for W and 23 for A.
//
// fp4: a word expands to 16 bytes, nibble i of dword d (d = 0..3) holding bit
// 4i + d: W 0x2 (1.0) for a set bit, else 0x0; A 0x2 (+1.0) or 0xA (-1.0),
// and 0x0 throughout for an invalid word. The same sums and correction apply.
// Every product is 0 or +-1 and every partial sum an integer of magnitude at
// most K, exact in fp32 for K <= 2^24. A word costs 7 VALU operations for W
// and about 10 for A, and an MFMA k-step covers two words instead of one.
//
// Tiling: a workgroup of 2 x WGN waves owns a BM (rows of A) x BN (rows of W)
// output tile and walks the reduction KS words (32*KS signs) per stage
// through two LDS buffers (one barrier per stage): while the waves run the
// MFMAs of stage s from one buffer, they expand stage s+1 into the other and
// fetch stage s+PD from global memory (PD register sets of raw words). Each
// wave holds a (BM/2) x (BN/WGN) sub-tile of 32 x 32 MFMA blocks. For linear tiles
// the MFMA computes D = W_tile * A_tile^T, so each lane's four consecutive
// accumulators are four consecutive output features of one row (row segments staged
// through LDS, then 16-byte stores); for conv tiles D = A_tile * W_tile^T, four
// consecutive pixels of one feature, contiguous in the NCHW output. LDS rows are 128 bytes; the
// 16-byte chunks of a row are XOR-swizzled with a Gray code of the row index
// so the ds_read_b128 / ds_write_b128 of 8 or 16 consecutive rows hit
// distinct banks. Tiles are numbered so that each XCD (workgroups go
// round-robin to the 8 XCDs) receives a contiguous run of tiles sharing A rows.
//
// Conv is the im2col lowering of the banghao.live blog post, section 2,
// computed implicitly: A row m is output pixel (b, oh, ow) and reduction word
// q = tap * CW + cw reads activation word [b][oh*s - p + kh*d][ow*s - p + kw*d][cw].
#include <atomic>
#include <type_traits>
#include <utility>

#include "launch.h"

// Tuning knobs: m-tiles per band of the linear tile order (0 or 1: row-major tiles), and the
// fewest tiles a linear grid needs for the bands to apply.
#ifndef BNN_MFMA_GROUP_M
#define BNN_MFMA_GROUP_M 4
#endif
#ifndef BNN_MFMA_GROUP_MIN_TILES
#define BNN_MFMA_GROUP_MIN_TILES 1024
#endif

// Tuning knob: conv A words of the tiles that share a compute unit three ways addressed by a
// per-thread tap walk (1) or, like the other tiles, by dividing each stage's reduction index (0).
#ifndef BNN_CONV_INC
#define BNN_CONV_INC 1
#endif

// Tuning knob: a scheduling fence after every BNN_MFMA_SLOT_FENCE MFMA slots (0: none).
#ifndef BNN_MFMA_SLOT_FENCE
#define BNN_MFMA_SLOT_FENCE 4
#endif

// Tuning knob: fp4 convs with more tiles than resident workgroups run persistent workgroups.
#ifndef BNN_CONV_PERS
#define BNN_CONV_PERS 1
#endif

namespace bnn {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

// fp4 e2m1 format code of the scaled MFMA, and the E8M0 scale exponent of 1.0
constexpr int kFmtFp4 = 4;
constexpr int kScaleOne = 127;

template <int BM_, int BN_, int KS_, int PD_, int WGM_, int WGN_, bool F4_, int OCC_ = 1>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, KS = KS_;
  static constexpr bool F4 = F4_;                   // fp4 (e2m1) operands instead of int8
  static constexpr int OCC = OCC_;                  // waves per SIMD the registers must allow
  static constexpr int PD = PD_;                    // stages of raw words in flight (register sets)
  static constexpr int UNROLL = PD % 2 == 0 ? PD : 2 * PD;  // lcm(2, PD): LDS parity x register set
  static constexpr int WGM = WGM_, WGN = WGN_;      // wave grid: WGM waves along A rows, WGN along W rows
  static constexpr int THREADS = 64 * WGM * WGN;
  static constexpr int WTM = BM / WGM, WTN = BN / WGN;  // wave sub-tile
  static constexpr int FM = WTM / 32, FN = WTN / 32;    // MFMA blocks per wave
  static constexpr int CPW = F4 ? 1 : 2;            // 16-byte LDS chunks per expanded word
  static constexpr int UPW = 4 * CPW;               // expansion units (output dwords) per word
  static constexpr int ROWB = KS * 16 * CPW;        // LDS bytes per row per stage
  static constexpr int CHUNKS = ROWB / 16;
  static constexpr int KSTEPS = CHUNKS / 2;         // MFMA k-steps per stage (chunks 2kk, 2kk+1)
  static constexpr int BUF = (BM + BN) * ROWB;      // one LDS buffer: A rows, then W rows
  // loader split: every thread expands A_WPT consecutive words of one A row and W_WPT
  // consecutive words of one W row per stage
  static constexpr int A_WPT = BM * KS / THREADS, A_TPR = KS / A_WPT;
  static constexpr int W_WPT = BN * KS / THREADS, W_TPR = KS / W_WPT;
  static constexpr int SWZ_SHIFT = CHUNKS == 8 ? 0 : CHUNKS == 4 ? 1 : 2;
  static_assert(A_WPT >= 1 && KS % A_WPT == 0 && W_WPT >= 1 && KS % W_WPT == 0, "loader split");
};

// Physical 16-byte chunk of logical chunk c in LDS row r.
template <class T>
__device__ __forceinline__ int swz(int r, int c) {
  const int g = r >> T::SWZ_SHIFT;
  return c ^ ((g ^ (g >> 1)) & (T::CHUNKS - 1));
}

struct PixelCoord {
  int b, ihb, iwb;
};

__device__ __forceinline__ PixelCoord pixel_coord(const Contraction& p, int m) {
  const int hw = p.Ho * p.Wo;
  const int b = p.div_hw.div(m);
  const int r = m - b * hw;
  const int oh = p.div_wo.div(r);
  const int ow = r - oh * p.Wo;
  return {b, oh * p.SH - p.PH, ow * p.SW - p.PW};
}

__device__ __forceinline__ int clampi(int v, int hi) { return v < 0 ? 0 : (v > hi ? hi : v); }

// NW consecutive words as one 4/8/16-byte load (p must be NW*4-byte aligned).
template <int NW>
__device__ __forceinline__ void load_vec(const uint32_t* ptr, uint32_t r[NW]) {
  if constexpr (NW == 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(ptr);
    r[0] = v.x; r[1] = v.y; r[2] = v.z; r[3] = v.w;
  } else if constexpr (NW == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(ptr);
    r[0] = v.x; r[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < NW; i++) r[i] = ptr[i];
  }
}

// NW consecutive A words of row m (m < M known by `mok`) from word q0, raw; ok[i] is false
// past K or for a padded conv tap (the word must then be treated as 0). Addresses are
// clamped into the tensor so the loads are unconditional, and the validity select is
// applied only when the words are expanded a stage later: selecting on a loaded value
// here would make the wave wait for the load right away and defeat the prefetch.
// VEC: the NW words are contiguous and aligned (K, or C for conv, is a multiple of the
// stage width and q0 % NW == 0), so they arrive in one vector load instead of NW
// scattered dword loads -- each lane reads a different row, so fewer, wider requests
// matter.
template <int NW, bool CONV, bool VEC>
__device__ __forceinline__ void load_a(const Contraction& p, int m, bool mok, const PixelCoord& pc,
                                       int q0, uint32_t r[NW], bool ok[NW]) {
  if constexpr (CONV) {
    int tap = p.div_cw.div(q0);
    int cw = q0 - tap * p.CW;
    int kh = p.div_kwd.div(tap);
    int kw = tap - kh * p.KWD;
    if constexpr (VEC) {
      // the NW words share one tap
      const int ih = pc.ihb + kh * p.DH, iw = pc.iwb + kw * p.DW;
      const bool tok = mok && q0 < p.KW && ih >= 0 && ih < p.H && iw >= 0 && iw < p.W;
      const int cwc = q0 < p.KW ? cw : 0;
      load_vec<NW>(p.a + (((int64_t)pc.b * p.H + clampi(ih, p.H - 1)) * p.W + clampi(iw, p.W - 1)) * p.CW + cwc, r);
#pragma unroll
      for (int i = 0; i < NW; i++) ok[i] = tok;
    } else {
#pragma unroll
      for (int i = 0; i < NW; i++) {
        const int q = q0 + i;
        const int ih = pc.ihb + kh * p.DH, iw = pc.iwb + kw * p.DW;
        ok[i] = mok && q < p.KW && ih >= 0 && ih < p.H && iw >= 0 && iw < p.W;
        r[i] = p.a[(((int64_t)pc.b * p.H + clampi(ih, p.H - 1)) * p.W + clampi(iw, p.W - 1)) * p.CW + cw];
        if (++cw == p.CW) {
          cw = 0;
          if (++kw == p.KWD) {
            kw = 0;
            ++kh;
          }
        }
      }
    }
  } else {
    const int64_t rowoff = (int64_t)(mok ? m : 0) * p.KW;
    if constexpr (VEC) {
      load_vec<NW>(p.a + rowoff + (q0 < p.KW ? q0 : p.KW - NW), r);
#pragma unroll
      for (int i = 0; i < NW; i++) ok[i] = mok && q0 < p.KW;
    } else {
#pragma unroll
      for (int i = 0; i < NW; i++) {
        const int q = q0 + i;
        ok[i] = mok && q < p.KW;
        r[i] = p.a[rowoff + (q < p.KW ? q : p.KW - 1)];
      }
    }
  }
}

// NW consecutive W words of row n from word q0, raw; ok[i] false outside the matrix or past K.
template <int NW, bool VEC>
__device__ __forceinline__ void load_w(const Contraction& p, int n, int q0, uint32_t r[NW],
                                       bool ok[NW]) {
  const bool nok = n < p.N;
  const int64_t rowoff = (int64_t)(nok ? n : 0) * p.KW;
  if constexpr (VEC) {
    load_vec<NW>(p.w + rowoff + (q0 < p.KW ? q0 : p.KW - NW), r);
#pragma unroll
    for (int i = 0; i < NW; i++) ok[i] = nok && q0 < p.KW;
  } else {
#pragma unroll
    for (int i = 0; i < NW; i++) {
      const int q = q0 + i;
      ok[i] = nok && q < p.KW;
      r[i] = p.w[rowoff + (q < p.KW ? q : p.KW - 1)];
    }
  }
}

// Tile slot (the workgroup index, or slot + i * grid for a persistent workgroup) ->
// (m-tile, n-tile): contiguous runs of tiles per XCD (slot % 8); within a run, plain rows (n
// fastest) or, for linear grids of at least BNN_MFMA_GROUP_MIN_TILES tiles (four or more rounds),
// bands of BNN_MFMA_GROUP_M m-tiles walked m fastest, so the tiles an XCD runs at once share fewer
// operand panels in its L2 (smaller grids lose more to the band arithmetic than they save).
template <bool CONV>
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, const FastDiv& div_tn,
                                            int slot, int& tm, int& tn) {
  static_assert((BNN_MFMA_GROUP_M & (BNN_MFMA_GROUP_M - 1)) == 0, "bands of a power of two");
  const int total = tiles_m * tiles_n;
  int t = slot;
  if ((total & 7) == 0) t = (t & 7) * (total >> 3) + (t >> 3);
  if (!CONV && BNN_MFMA_GROUP_M > 1 && total >= BNN_MFMA_GROUP_MIN_TILES) {
    constexpr int G = BNN_MFMA_GROUP_M > 1 ? BNN_MFMA_GROUP_M : 1;
    constexpr int GS = G == 2 ? 1 : G == 4 ? 2 : G == 8 ? 3 : G == 16 ? 4 : 0;
    const int g = div_tn.div(t >> GS);  // band: t / (G * tiles_n)
    const int r = t - g * G * tiles_n;
    const int m0 = g * G;
    if (tiles_m - m0 >= G) {
      tn = r >> GS;
      tm = m0 + (r & (G - 1));
    } else {  // the last, partial band
      const int gm = tiles_m - m0;
      tn = r / gm;
      tm = m0 + (r - tn * gm);
    }
  } else {
    tm = div_tn.div(t);
    tn = t - tm * tiles_n;
  }
}

// One LDS fragment read (16 bytes per lane) of row r, reduction chunk c.
template <class T>
__device__ __forceinline__ v4i lds_frag(const uint8_t* buf, int r, int c) {
  return *reinterpret_cast<const v4i*>(buf + r * T::ROWB + 16 * swz<T>(r, c));
}

// Epilogue of the matrix-core kernel. For linear tiles acc[fn][fm][e] is output (row m,
// feature n) with
//   m = m0 + wm*WTM + fm*32 + (lane & 31)
//   n = n0 + wn*WTN + fn*32 + 8*(e/4) + 4*(lane/32) + e%4
// (conv tiles swap the roles of lane and e, see below), and the binary dot product is
// rowk(m - m0) + 2 * acc. Called by the WGM x WGN waves that
// hold accumulators (waves 0 .. WGM*WGN-1); the LDS buffers are free by then and serve as
// staging space.
template <class T, int OUT, bool CONV, class Acc, class RowK>
__device__ __forceinline__ void store_tile(const Contraction& p, const Acc (&acc)[T::FN][T::FM],
                                           RowK rowk, uint8_t* lds0, uint8_t* lds1, int m0,
                                           int n0, int wm, int wn) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 31, half = lane >> 5;
  auto acc_int = [&](int fn, int fm, int e) -> int { return (int)acc[fn][fm][e]; };
  if constexpr (CONV) {
    // NCHW. Conv tiles compute D = A * W^T, so lane (fr, half) holds feature
    // n = n0 + wn*WTN + fn*32 + fr and, in e = 4g .. 4g+3, the four consecutive pixels
    // m = m0 + wm*WTM + fm*32 + 8g + 4*half + 0..3: one 8- or 16-byte store each when the
    // output plane size is a multiple of 4 (the four pixels then share an image and the
    // address is aligned), element stores otherwise.
    const int hw = p.Ho * p.Wo;
    const bool quad = (hw & 3) == 0;
    // 16-bit outputs with planes a multiple of 8: lanes fr and fr + 32 (same feature) trade
    // halves of their pixel quads so each stores eight consecutive pixels (16 bytes) at once
    constexpr bool HALF16 = OUT == kF16 || OUT == kBF16;
    const bool oct = HALF16 && (hw & 7) == 0;
    // Everything that depends on the pixel but not on the feature is done once per tile
    // rather than once per feature block: the row bases rowk (K_valid - 2 popA of each of the
    // lane's 4 x 4 pixels per 32-pixel block) and the pixels' offsets in the output.
    // Floating-point outputs take the dot product as fma(2, acc, rowk) in fp32: both terms
    // are integers of magnitude at most K <= 2^24 and so is their sum, so it is exact, and
    // the result is the same as converting the integer sum.
    constexpr bool FDOT = OUT != kI32 && T::F4;
    using RK = std::conditional_t<FDOT, float, int>;
    RK rk[T::FM][16];
#pragma unroll
    for (int fm = 0; fm < T::FM; fm++)
#pragma unroll
      for (int e = 0; e < 16; e++) {
        const int v = rowk(wm * T::WTM + fm * 32 + 8 * (e >> 2) + 4 * half + (e & 3));
        rk[fm][e] = (RK)v;
      }
    auto dot = [&](int fn, int fm, int e) {
      if constexpr (FDOT)
        return __builtin_fmaf(2.0f, acc[fn][fm][e], rk[fm][e]);
      else
        return rk[fm][e] + 2 * acc_int(fn, fm, e);
    };
    auto scaled = [&](int fn, int fm, int e) -> float {
      if constexpr (FDOT)
        return dot(fn, fm, e) * p.alpha;
      else
        return (float)dot(fn, fm, e) * p.alpha;
    };
    auto bits16 = [&](float f) -> uint32_t {
      if constexpr (OUT == kF16) {
        const __half h = __float2half_rn(f);
        return *reinterpret_cast<const uint16_t*>(&h);
      } else {
        const __hip_bfloat16 h = __float2bfloat16(f);
        return *reinterpret_cast<const uint16_t*>(&h);
      }
    };
    const int64_t plane = (int64_t)p.N * hw;  // output elements per image
    using O = OutType<OUT>;
    typename O::type* const out = reinterpret_cast<typename O::type*>(p.out);
    // Staged write-out (planes a multiple of 4). Stored straight from the MFMA layout, each
    // store instruction would put 32 features x 8..32 bytes into 32 channel planes, a
    // fraction of a memory line each. Instead each wave turns one 32-feature block around in
    // its own 4 KiB of LDS (32 rows of 128 bytes, one per feature, holding PXS consecutive
    // pixels) and stores it back row-wise: LPC lanes per feature, 8 or 16 bytes each, so
    // an instruction writes whole 128-byte runs of 64 / LPC channel planes. Rows are
    // XOR-swizzled in 16-byte chunks (chunk k of row r at k ^ (r & 7)) to spread the
    // column-wise writes over the banks. `lds0` is a free buffer of T::BUF bytes.
    constexpr int ESZ = (int)sizeof(typename O::type);
    constexpr int PXS = 128 / ESZ < T::WTM ? 128 / ESZ : T::WTM;  // pixels per staged row
    constexpr int FMS = PXS / 32;                                 // MFMA blocks per row
    constexpr int NWAVES = T::WGM * T::WGN;
    constexpr bool STAGED = PXS * ESZ == 128 && NWAVES * 4096 <= T::BUF;
    if constexpr (STAGED) {
      if (quad) {
        const int pl = (ESZ == 2 && !oct) ? 4 : 16 / ESZ;  // pixels per lane store
        const int lpc = PXS / pl;                           // lanes per feature row
        const int cpi = 64 / lpc;                           // feature rows per instruction
        uint8_t* const st = lds0 + wave * 4096;
        auto at = [&](int r, int byte) { return st + r * 128 + (((byte >> 4) ^ (r & 7)) << 4) + (byte & 15); };
#pragma unroll
        for (int f0 = 0; f0 < T::FM; f0 += FMS) {
          // this lane's pixel run of the read-back, the same for every feature
          const int mrun = m0 + wm * T::WTM + f0 * 32 + (lane % lpc) * pl;
          const bool mok = mrun < p.M;
          const int b = p.div_hw.div(mok ? mrun : 0);
          typename O::type* const orun = out + (int64_t)b * plane + (mrun - b * hw);
          const int rbyte = (lane % lpc) * pl * ESZ;
#pragma unroll
          for (int fn = 0; fn < T::FN; fn++) {
#pragma unroll
            for (int ff = 0; ff < FMS; ff++)
#pragma unroll
              for (int g = 0; g < 4; g++) {
                const int fm = f0 + ff, e = 4 * g;
                uint8_t* const dst = at(fr, (ff * 32 + 8 * g + 4 * half) * ESZ);
                if constexpr (OUT == kI32) {
                  *reinterpret_cast<int4*>(dst) = make_int4(dot(fn, fm, e), dot(fn, fm, e + 1),
                                                            dot(fn, fm, e + 2), dot(fn, fm, e + 3));
                } else if constexpr (OUT == kF32) {
                  *reinterpret_cast<float4*>(dst) = make_float4(scaled(fn, fm, e), scaled(fn, fm, e + 1),
                                                                scaled(fn, fm, e + 2), scaled(fn, fm, e + 3));
                } else {
                  *reinterpret_cast<uint2*>(dst) =
                      make_uint2(bits16(scaled(fn, fm, e)) | (bits16(scaled(fn, fm, e + 1)) << 16),
                                 bits16(scaled(fn, fm, e + 2)) | (bits16(scaled(fn, fm, e + 3)) << 16));
                }
              }
            // the rows are private to this wave and its LDS accesses complete in order
            __builtin_amdgcn_wave_barrier();
            const int nb = n0 + wn * T::WTN + fn * 32;
            for (int i = 0; i < 32 / cpi; i++) {
              const int r = lane / lpc + cpi * i;
              const bool ok = mok && nb + r < p.N;
              typename O::type* const dst = orun + (int64_t)(nb + r) * hw;
              if (pl * ESZ == 16) {
                const uint4 v = *reinterpret_cast<const uint4*>(at(r, rbyte));
                if (ok) *reinterpret_cast<uint4*>(dst) = v;
              } else {
                const uint2 v = *reinterpret_cast<const uint2*>(at(r, rbyte));
                if (ok) *reinterpret_cast<uint2*>(dst) = v;
              }
            }
            __builtin_amdgcn_wave_barrier();
          }
        }
        return;
      }
    }
    if constexpr (HALF16) {
      if (oct) {
        // 16-pixel runs: pixels m0 + wm*WTM + fm*32 + 16j + 8*half + 0..7 leave from this lane
        int64_t off[T::FM][2];
        bool mok[T::FM][2];
#pragma unroll
        for (int fm = 0; fm < T::FM; fm++)
#pragma unroll
          for (int j = 0; j < 2; j++) {
            const int mg = m0 + wm * T::WTM + fm * 32 + 16 * j + 8 * half;
            mok[fm][j] = mg < p.M;
            const int b = p.div_hw.div(mok[fm][j] ? mg : 0);
            off[fm][j] = (int64_t)b * plane + (mg - b * hw);
          }
#pragma unroll
        for (int fn = 0; fn < T::FN; fn++) {
          const int n = n0 + wn * T::WTN + fn * 32 + fr;
          if (n >= p.N) continue;  // uniform over the lane pair fr, fr + 32
          typename O::type* const col = out + (int64_t)n * hw;
#pragma unroll
          for (int fm = 0; fm < T::FM; fm++)
#pragma unroll
            for (int j = 0; j < 2; j++) {
              // groups g = 2j (pixels +0..7) and 2j+1 (+8..15) of this 32-pixel block
              uint32_t q[2][2];
#pragma unroll
              for (int gg = 0; gg < 2; gg++) {
                const int g = 2 * j + gg;
                uint32_t h4[4];
#pragma unroll
                for (int i = 0; i < 4; i++) h4[i] = bits16(scaled(fn, fm, 4 * g + i));
                q[gg][0] = h4[0] | (h4[1] << 16);
                q[gg][1] = h4[2] | (h4[3] << 16);
              }
              const uint32_t s0 = half ? q[0][0] : q[1][0], s1 = half ? q[0][1] : q[1][1];
              const uint32_t r0 = (uint32_t)__shfl_xor((int)s0, 32), r1 = (uint32_t)__shfl_xor((int)s1, 32);
              if (mok[fm][j]) {
                const uint4 v = half ? make_uint4(r0, r1, q[1][0], q[1][1]) : make_uint4(q[0][0], q[0][1], r0, r1);
                *reinterpret_cast<uint4*>(col + off[fm][j]) = v;
              }
            }
        }
        return;
      }
    }
    if (quad) {
      int64_t off[T::FM][4];
      bool mok[T::FM][4];
#pragma unroll
      for (int fm = 0; fm < T::FM; fm++)
#pragma unroll
        for (int g = 0; g < 4; g++) {
          const int m = m0 + wm * T::WTM + fm * 32 + 8 * g + 4 * half;
          mok[fm][g] = m < p.M;
          const int b = p.div_hw.div(mok[fm][g] ? m : 0);
          off[fm][g] = (int64_t)b * plane + (m - b * hw);
        }
#pragma unroll
      for (int fn = 0; fn < T::FN; fn++) {
        const int n = n0 + wn * T::WTN + fn * 32 + fr;
        if (n >= p.N) continue;
        typename O::type* const col = out + (int64_t)n * hw;
#pragma unroll
        for (int fm = 0; fm < T::FM; fm++)
#pragma unroll
          for (int g = 0; g < 4; g++) {
            if (!mok[fm][g]) continue;
            typename O::type* const dst = col + off[fm][g];
            if constexpr (OUT == kI32) {
              *reinterpret_cast<int4*>(dst) = make_int4(dot(fn, fm, 4 * g), dot(fn, fm, 4 * g + 1),
                                                        dot(fn, fm, 4 * g + 2), dot(fn, fm, 4 * g + 3));
            } else if constexpr (OUT == kF32) {
              *reinterpret_cast<float4*>(dst) = make_float4(scaled(fn, fm, 4 * g), scaled(fn, fm, 4 * g + 1),
                                                            scaled(fn, fm, 4 * g + 2), scaled(fn, fm, 4 * g + 3));
            } else {
              const uint32_t lo = bits16(scaled(fn, fm, 4 * g)) | (bits16(scaled(fn, fm, 4 * g + 1)) << 16);
              const uint32_t hi = bits16(scaled(fn, fm, 4 * g + 2)) | (bits16(scaled(fn, fm, 4 * g + 3)) << 16);
              *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
            }
          }
      }
      return;
    }
    // planes of any size: element stores, each pixel's image found on its own
#pragma unroll
    for (int fn = 0; fn < T::FN; fn++) {
      const int n = n0 + wn * T::WTN + fn * 32 + fr;
      if (n >= p.N) continue;
#pragma unroll
      for (int fm = 0; fm < T::FM; fm++)
#pragma unroll
        for (int e = 0; e < 16; e++) {
          const int m = m0 + wm * T::WTM + fm * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
          if (m >= p.M) continue;
          const int b = p.div_hw.div(m);
          const int64_t idx = (int64_t)b * plane + (int64_t)n * hw + (m - b * hw);
          if constexpr (OUT == kI32)
            out[idx] = dot(fn, fm, e);
          else if constexpr (OUT == kF32)
            out[idx] = scaled(fn, fm, e);
          else
            reinterpret_cast<uint16_t*>(p.out)[idx] = (uint16_t)bits16(scaled(fn, fm, e));
        }
    }
  } else {
    // Row-major [M][N]: each lane's values are four features of one row, 32 rows per
    // half-wave, so storing them directly would scatter 8..16-byte pieces over 32 rows.
    // Instead each wave stages one 32-row band of its sub-tile in LDS (free after the
    // main loop; two waves' bands per buffer) and writes it back as whole contiguous row
    // segments, 16 bytes per lane.
    using O = OutType<OUT>;
    constexpr int WN = T::WTN;                          // columns of a wave's sub-tile
    constexpr int ROWS_B = WN * (int)sizeof(typename O::type) + 16;  // padded LDS row
    constexpr int NWAVES = T::WGM * T::WGN, HALFW = NWAVES / 2;
    static_assert(HALFW * 32 * ROWS_B <= T::BUF, "staging bands fit in the two LDS buffers");
    uint8_t* band = (wave < HALFW ? lds0 : lds1) + (wave % HALFW) * 32 * ROWS_B;
    constexpr int EPV = 16 / (int)sizeof(typename O::type);  // elements per 16-byte vector
    constexpr int VPR = WN / EPV;                            // vectors per band row
#pragma unroll
    for (int fm = 0; fm < T::FM; fm++) {
      const int base_k = rowk(wm * T::WTM + fm * 32 + fr);
      uint8_t* myrow = band + fr * ROWS_B;
#pragma unroll
      for (int fn = 0; fn < T::FN; fn++)
#pragma unroll
        for (int g = 0; g < 4; g++) {
          const int c = fn * 32 + 8 * g + 4 * half;
          O::put4(myrow + c * (int)sizeof(typename O::type), base_k + 2 * acc_int(fn, fm, 4 * g),
                  base_k + 2 * acc_int(fn, fm, 4 * g + 1), base_k + 2 * acc_int(fn, fm, 4 * g + 2),
                  base_k + 2 * acc_int(fn, fm, 4 * g + 3), p.alpha);
        }
      // the band is private to this wave and a wave's LDS accesses complete in order, so
      // no fence is needed (a memory fence here would also wait for the global stores)
      __builtin_amdgcn_wave_barrier();
      const int mrow0 = m0 + wm * T::WTM + fm * 32;
      const int ncol0 = n0 + wn * WN;
      constexpr int NV = 32 * VPR / 64;  // 16-byte vectors per lane for the band
      static_assert(NV >= 1 && (32 * VPR) % 64 == 0, "band splits evenly over the lanes");
      uint4 vals[NV];
#pragma unroll
      for (int t = 0; t < NV; t++) {
        const int v = lane + 64 * t;
        const int r = v / VPR, cv = v - r * VPR;
        vals[t] = *reinterpret_cast<const uint4*>(band + r * ROWS_B + cv * 16);
      }
      const bool full_rows = (p.N % EPV) == 0;
#pragma unroll
      for (int t = 0; t < NV; t++) {
        const int v = lane + 64 * t;
        const int r = v / VPR, cv = v - r * VPR;
        const int m = mrow0 + r, n = ncol0 + cv * EPV;
        if (m >= p.M) continue;
        typename O::type* dst = reinterpret_cast<typename O::type*>(p.out) + (int64_t)m * p.N + n;
        if (full_rows && n + EPV <= p.N) {
          st_nt(dst, u32x4{vals[t].x, vals[t].y, vals[t].z, vals[t].w});
        } else {
          const typename O::type* src = reinterpret_cast<const typename O::type*>(&vals[t]);
#pragma unroll
          for (int j = 0; j < EPV; j++)
            if (n + j < p.N) dst[j] = src[j];
        }
      }
      // the band is private to this wave and a wave's LDS accesses complete in order, so
      // no fence is needed (a memory fence here would also wait for the global stores)
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// PERS (conv): a persistent workgroup takes tiles slot, slot + grid, ... and streams their
// stages back to back: the loads and expansions run PD stages and one stage ahead across
// tile boundaries, and a tile's epilogue (direct NCHW stores) follows the barrier of its
// last stage while the next tile's first stage already sits in LDS. Row bases K_valid -
// 2*popA are kept per loader thread in LDS slots of two tile parities, so no LDS atomics
// or clearing are needed between tiles.
template <class T, int OUT, bool CONV, bool VEC, bool PERS>
__global__ __launch_bounds__(T::THREADS, T::OCC) void mfma_kernel(Contraction p) {
  static_assert(!PERS || CONV, "persistent tiles use the direct (unstaged) conv epilogue");
  // two distinct arrays (not one array indexed by stage parity) so the compiler can
  // tell the expansion's writes from the fragment reads
  __shared__ __attribute__((aligned(16))) uint8_t lds0[T::BUF];
  __shared__ __attribute__((aligned(16))) uint8_t lds1[T::BUF];
  // K_valid - 2 * popA per A row of the tile: one sum (atomics), or A_TPR partial sums
  // per row and tile parity (persistent)
  constexpr int RK_SLOTS = PERS ? 2 * T::BM * T::A_TPR : T::BM;
  __shared__ __attribute__((aligned(16))) int rowk[RK_SLOTS];

  constexpr int MPK = T::FN * T::FM;            // MFMAs per k-step
  constexpr int NM = MPK * T::KSTEPS;           // MFMAs per stage
  constexpr int RPK = T::FN + T::FM;            // fragment reads per k-step
  constexpr int NWORD = T::A_WPT + T::W_WPT;    // words this thread expands per stage
  constexpr int NU = NWORD * T::UPW;            // expansion units (one output dword each)

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave % T::WGM, wn = wave / T::WGM;
  const int tiles_m = (p.M + T::BM - 1) / T::BM, tiles_n = (p.N + T::BN - 1) / T::BN;
  const int total = tiles_m * tiles_n;
  // tiles of this workgroup: slots blockIdx.x + i * gridDim.x
  const int ntl = PERS ? (total - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x : 1;
  auto tile_origin = [&](int i, int& m0, int& n0) __attribute__((always_inline)) {
    int tm, tn;
    tile_coords<CONV>(tiles_m, tiles_n, p.div_tn, (int)blockIdx.x + i * (int)gridDim.x, tm, tn);
    m0 = tm * T::BM;
    n0 = tn * T::BN;
  };

  // loader roles
  const int a_row = tid / T::A_TPR, a_q = (tid % T::A_TPR) * T::A_WPT;
  const int w_row = tid / T::W_TPR, w_q = (tid % T::W_TPR) * T::W_WPT;
  int am = 0, wn_row = 0;
  bool amok = false;
  PixelCoord pc{0, 0, 0};
  // Conv tap walk (vector loads): this thread's next A load is word cw of tap (kh, kw) of its
  // pixel, at activation row ih = ihb + kh*DH, column iw = iwb + kw*DW and word offset
  // pix + toff + cw (pix: the pixel's (b, ihb, iwb) origin, toff: (kh*DH*W + kw*DW)*CW); each
  // load advances it by one stage (KS words) with additions only, instead of two invariant
  // divisions and three 64-bit products. Taken by the tiles sized for three workgroups per
  // compute unit, whose loop is bound by vector-ALU issue (the dilated 128x128x28x28 -> 256
  // layer: 33.3 -> 32.2 us); on the one-workgroup tiles it cost 1.5 %.
  constexpr bool INC = CONV && VEC && BNN_CONV_INC && T::OCC > 1;
  int tw_cw = 0, tw_kw = 0, tw_ih = 0, tw_iw = 0;
  int64_t tw_pix = 0, tw_toff = 0;
  // word offset steps of the walk: to the next kernel column, and from a row's last column to
  // the next row's first
  const int64_t tw_dcol = (int64_t)p.DW * p.CW;
  const int64_t tw_drow = ((int64_t)p.DH * p.W - (int64_t)(p.KWD - 1) * p.DW) * p.CW;
  auto loader_tile = [&](int i) __attribute__((always_inline)) {  // A row, pixel and W row of this thread in tile i
    int m0, n0;
    tile_origin(i, m0, n0);
    am = m0 + a_row;
    wn_row = n0 + w_row;
    amok = am < p.M;
    if constexpr (CONV) pc = pixel_coord(p, amok ? am : 0);
    if constexpr (INC) {
      const int tap = p.div_cw.div(a_q);
      tw_cw = a_q - tap * p.CW;
      const int kh = p.div_kwd.div(tap);
      tw_kw = tap - kh * p.KWD;
      tw_ih = pc.ihb + kh * p.DH;
      tw_iw = pc.iwb + tw_kw * p.DW;
      tw_toff = ((int64_t)kh * p.DH * p.W + (int64_t)tw_kw * p.DW) * p.CW;
      tw_pix = (((int64_t)pc.b * p.H + pc.ihb) * p.W + pc.iwb) * p.CW;
    }
  };
  loader_tile(0);
  if constexpr (!PERS)
    for (int i = tid; i < T::BM; i += T::THREADS) rowk[i] = 0;
  int rowk_part = 0;  // this thread's share of 32 * (real words) - 2 * popA

  // raw words of PD stages in flight; stage t lives in register set t % PD
  uint32_t ra[T::PD][T::A_WPT], rw[T::PD][T::W_WPT];
  bool oka[T::PD][T::A_WPT], okw[T::PD][T::W_WPT];
  auto load_words = [&](int set, int q0) __attribute__((always_inline)) {
    if constexpr (INC) {
      // q0 is always the walk's stage: loads go out stage by stage, and a new tile restarts
      // the walk in loader_tile; this thread's words start at q0 + a_q (past K in a short
      // last stage)
      const bool tok = amok && q0 + a_q < p.KW && (unsigned)tw_ih < (unsigned)p.H &&
                       (unsigned)tw_iw < (unsigned)p.W;
      load_vec<T::A_WPT>(p.a + (tok ? tw_pix + tw_toff + tw_cw : 0), ra[set]);
#pragma unroll
      for (int i = 0; i < T::A_WPT; i++) oka[set][i] = tok;
      tw_cw += T::KS;
      // (every step updates every field, by value selects: stores on only one side of a
      // branch would let the compiler select between the fields' addresses and keep them in
      // scratch memory)
      while (tw_cw >= p.CW) {
        tw_cw -= p.CW;
        const bool wrap = tw_kw + 1 == p.KWD;
        tw_kw = wrap ? 0 : tw_kw + 1;
        tw_iw = wrap ? pc.iwb : tw_iw + p.DW;
        tw_ih += wrap ? p.DH : 0;
        tw_toff += wrap ? tw_drow : tw_dcol;
      }
    } else {
      load_a<T::A_WPT, CONV, VEC>(p, am, amok, pc, q0 + a_q, ra[set], oka[set]);
    }
    load_w<T::W_WPT, VEC>(p, wn_row, q0 + w_q, rw[set], okw[set]);
  };
  // persistent stream position of the next loads: tile lt, stage ls
  const int nstages = (p.KW + T::KS - 1) / T::KS;
  int lt = 0, ls = 0;
  auto load_next = [&](int set) __attribute__((always_inline)) {
    // past the last tile: clamped, invalid words (q0 = K/32)
    load_words(set, lt < ntl ? ls * T::KS : p.KW);
    if (++ls == nstages) {
      ls = 0;
      if (++lt < ntl) loader_tile(lt);
    }
  };

  // expansion of stage words. int8: the source word, and for A words the byte table of
  // v_perm (0xFF for a 0 bit, 0x01 for a 1 bit; all 0 for an invalid word). fp4: W keeps
  // the word; A keeps its complement with an AND mask and an OR term (both 0 for an
  // invalid word).
  uint32_t src[NWORD], tab[T::A_WPT], tabo[T::A_WPT];
  int pt = 0, ps = 0;  // persistent stream position of the next prepare
  auto prepare = [&](int set) {
    if constexpr (PERS) {
      // the first stage of a new tile: the finished tile's row share goes to its LDS slot
      if (ps == 0 && pt > 0) {
        rowk[(((pt - 1) & 1) * T::BM + a_row) * T::A_TPR + a_q / T::A_WPT] = rowk_part;
        rowk_part = 0;
      }
      if (++ps == nstages) {
        ps = 0;
        ++pt;
      }
    }
#pragma unroll
    for (int i = 0; i < T::A_WPT; i++) {
      if constexpr (T::F4) {
        src[i] = ~ra[set][i];
        tab[i] = oka[set][i] ? 0x88888888u : 0u;
        tabo[i] = oka[set][i] ? 0x22222222u : 0u;
      } else {
        src[i] = ra[set][i];
        tab[i] = oka[set][i] ? 0x000001FFu : 0u;
      }
      rowk_part += oka[set][i] ? 32 - 2 * __popc(ra[set][i]) : 0;
    }
#pragma unroll
    for (int i = 0; i < T::W_WPT; i++) src[T::A_WPT + i] = okw[set][i] ? rw[set][i] : 0u;
  };
  uint32_t y[NU];
  auto expand_unit = [&](uint8_t* buf, int u) {
    const int wi = u / T::UPW, d = u % T::UPW;
    if constexpr (T::F4) {
      // nibble i of dword d is bit 4i + d: W 0x2 (1.0) or 0x0; A 0x2 (+1.0) or 0xA (-1.0)
      if (wi < T::A_WPT)
        y[u] = ((src[wi] << (3 - d)) & tab[wi]) | tabo[wi];
      else
        y[u] = (d == 0 ? src[wi] << 1 : src[wi] >> (d - 1)) & 0x22222222u;
    } else {
      // byte j of dword d is bit 8j + d: W 0 or 1; A -1 or +1
      const uint32_t t = (src[wi] >> d) & 0x01010101u;
      y[u] = wi < T::A_WPT ? __builtin_amdgcn_perm(0u, tab[wi], t) : t;
    }
    if ((d & 3) == 3) {
      const int lrow = wi < T::A_WPT ? a_row : T::BM + w_row;
      const int word = wi < T::A_WPT ? a_q + wi : w_q + (wi - T::A_WPT);
      uint8_t* line = buf + lrow * T::ROWB;
      *reinterpret_cast<uint4*>(line + 16 * swz<T>(lrow, T::CPW * word + (d >> 2))) =
          make_uint4(y[u - 3], y[u - 2], y[u - 1], y[u]);
    }
  };

  // int32 sums (int8 operands) or fp32 sums (fp4 operands; integers of magnitude at most
  // K <= 2^24, so every partial sum is exact)
  using Acc = std::conditional_t<T::F4, v16f, v16i>;
  Acc acc[T::FN][T::FM];
  auto clear_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < T::FN; i++)
#pragma unroll
      for (int j = 0; j < T::FM; j++)
#pragma unroll
        for (int e = 0; e < 16; e++) acc[i][j][e] = 0;
  };
  clear_acc();

  const int fr = lane & 31, half = lane >> 5;
  v4i fa[2][T::FM], fw[2][T::FN];
  auto read_frag = [&](const uint8_t* cur, int kk, int j) {
    const int fb = kk & 1;
    if (j < T::FM) {
      fa[fb][j] = lds_frag<T>(cur, wm * T::WTM + j * 32 + fr, 2 * kk + half);
    } else {
      const int f = j - T::FM;
      fw[fb][f] = lds_frag<T>(cur, T::BM + wn * T::WTN + f * 32 + fr, 2 * kk + half);
    }
  };

  // epilogue of the tile whose last stage just ended (persistent: tile ct)
  int ct = 0, cs = 0;
  // free: an LDS buffer (T::BUF bytes) that no wave reads or writes during the epilogue
  auto tile_epilogue = [&](int i, uint8_t* free) __attribute__((always_inline)) {
    int m0, n0;
    tile_origin(i, m0, n0);
    if constexpr (PERS) {
      const int* slots = rowk + (i & 1) * T::BM * T::A_TPR;
      store_tile<T, OUT, CONV>(
          p, acc,
          [&](int ml) {
            int v = 0;
#pragma unroll
            for (int j = 0; j < T::A_TPR; j++) v += slots[ml * T::A_TPR + j];
            return v;
          },
          free, nullptr, m0, n0, wm, wn);
    } else {
      store_tile<T, OUT, CONV>(p, acc, [&](int ml) { return rowk[ml]; }, free, lds1, m0, n0, wm, wn);
    }
  };

  // One MFMA of k-step fragments of parity par into acc[fn][fm].
  auto mfma = [&](int par, int fn, int fm) __attribute__((always_inline)) {
    if constexpr (T::F4) {
      // only the first four dwords of each operand carry fp4 data
      const v4i w4 = fw[par][fn], a4 = fa[par][fm];
      const v8i w8 = {w4[0], w4[1], w4[2], w4[3], 0, 0, 0, 0};
      const v8i a8 = {a4[0], a4[1], a4[2], a4[3], 0, 0, 0, 0};
      // linear: D = W * A^T (a lane holds four features of one row); conv: D = A * W^T (a
      // lane holds four pixels of one feature, contiguous in NCHW)
      if constexpr (CONV)
        acc[fn][fm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            a8, w8, acc[fn][fm], kFmtFp4, kFmtFp4, 0, kScaleOne, 0, kScaleOne);
      else
        acc[fn][fm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            w8, a8, acc[fn][fm], kFmtFp4, kFmtFp4, 0, kScaleOne, 0, kScaleOne);
    } else {
      if constexpr (CONV)
        acc[fn][fm] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[par][fm], fw[par][fn], acc[fn][fm],
                                                             0, 0, 0);
      else
        acc[fn][fm] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fw[par][fn], fa[par][fm], acc[fn][fm],
                                                             0, 0, 0);
    }
  };
  // XB (one tile per workgroup): the MFMAs of a stage's last k-step run at the start of the
  // next stage, after its barrier -- their fragments are already in registers -- so the
  // matrix cores have a k-step of work while the waves fetch the new stage's first fragments
  // (otherwise every wave leaves the barrier waiting on LDS reads at the same moment). Slot
  // group g = i / MPK of a stage then holds k-step g - 1 (g = 0: the previous stage's last),
  // and k-step g's fragments are read at group g's first slot. Before the first stage the
  // carried-over fragments are zero operands (they add exactly 0); after the last stage its
  // final k-step is drained before the epilogue.
  constexpr bool XB = !PERS;
  constexpr int LASTPAR = (T::KSTEPS - 1) & 1;
  static_assert(!XB || T::KSTEPS % 2 == 0, "carried k-step and k-step 0 use different fragment sets");
  // One stage: the MFMAs over the current LDS buffer, interleaved slot by slot with the
  // reads of the next k-step's fragments and the expansion of the next stage into the
  // other buffer; the global loads for stage s + PD go out first. Each slot is closed by
  // a scheduling barrier so the matrix core and the vector ALU stay busy together even
  // with one wave per SIMD. PH = s % UNROLL is a compile-time phase, which fixes the LDS
  // buffer parity and the register sets. Past the last stage the expansion writes
  // zero-contribution words into a buffer that is never read again, and the loads fetch
  // clamped, invalid words.
  auto stage = [&](auto phase, int s) {
    constexpr int PH = decltype(phase)::value;
    uint8_t* cur = (PH & 1) ? lds1 : lds0;
    uint8_t* nxt = (PH & 1) ? lds0 : lds1;
    if constexpr (PERS)
      load_next(PH % T::PD);
    else
      load_words(PH % T::PD, (s + T::PD) * T::KS);
#pragma unroll
    for (int j = 0; j < RPK; j++) read_frag(cur, 0, j);
    prepare((PH + 1) % T::PD);
#pragma unroll
    for (int i = 0; i < NM; i++) {
      const int g = i / MPK, j = i % MPK;
      const int fn = j / T::FM, fm = j % T::FM;
      if constexpr (XB) {
        mfma(g == 0 ? LASTPAR : (g - 1) & 1, fn, fm);
        // k-step g's fragments go out in group g's first slot, a group of MFMAs ahead of use
        if (g >= 1 && j == 0) {
#pragma unroll
          for (int f = 0; f < RPK; f++) read_frag(cur, g, f);
        }
      } else {
        mfma(g & 1, fn, fm);
        // the next k-step's RPK fragment reads all go out in its first slot, a whole k-step
        // of MFMAs ahead of their use
        if (g + 1 < T::KSTEPS && j == 0) {
#pragma unroll
          for (int f = 0; f < RPK; f++) read_frag(cur, g + 1, f);
        }
      }
#pragma unroll
      for (int u = i * NU / NM; u < (i + 1) * NU / NM; u++) expand_unit(nxt, u);
      if (BNN_MFMA_SLOT_FENCE > 0 && (i + 1) % (BNN_MFMA_SLOT_FENCE > 0 ? BNN_MFMA_SLOT_FENCE : 1) == 0)
        __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    if constexpr (PERS) {
      if (++cs == nstages) {
        // the finished stage's buffer is free until the next stage expands into it; the
        // barrier keeps that expansion off the rows other waves still stage through
        tile_epilogue(ct, cur);
        __syncthreads();
        clear_acc();
        cs = 0;
        ++ct;
      }
    }
  };

  // stages of this workgroup: one tile, or ntl tiles back to back
  const int nstream = PERS ? ntl * nstages : nstages;
#pragma unroll
  for (int t = 0; t < T::PD; t++) {
    if constexpr (PERS)
      load_next(t);
    else
      load_words(t, t * T::KS);  // clamped + invalid past K
  }
  prepare(0);
#pragma unroll
  for (int u = 0; u < NU; u++) expand_unit(lds0, u);
  if constexpr (XB) {
#pragma unroll
    for (int f = 0; f < T::FM; f++) fa[LASTPAR][f] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int f = 0; f < T::FN; f++) fw[LASTPAR][f] = v4i{0, 0, 0, 0};
  }
  __syncthreads();
  int s = 0;
  for (; s + T::UNROLL <= nstream; s += T::UNROLL) {
    stage(std::integral_constant<int, 0>{}, s);
    stage(std::integral_constant<int, 1>{}, s + 1);
    if constexpr (T::UNROLL > 2) {
      stage(std::integral_constant<int, 2>{}, s + 2);
      stage(std::integral_constant<int, 3>{}, s + 3);
    }
    if constexpr (T::UNROLL > 4) {
      stage(std::integral_constant<int, 4>{}, s + 4);
      stage(std::integral_constant<int, 5>{}, s + 5);
    }
  }
  if (s < nstream) stage(std::integral_constant<int, 0>{}, s);
  if (s + 1 < nstream) stage(std::integral_constant<int, 1>{}, s + 1);
  if constexpr (T::UNROLL > 2) {
    if (s + 2 < nstream) stage(std::integral_constant<int, 2>{}, s + 2);
    if (s + 3 < nstream) stage(std::integral_constant<int, 3>{}, s + 3);
  }
  if constexpr (T::UNROLL > 4) {
    if (s + 4 < nstream) stage(std::integral_constant<int, 4>{}, s + 4);
  }

  if constexpr (XB) {
    // drain: the last stage's final k-step
#pragma unroll
    for (int j = 0; j < MPK; j++) mfma(LASTPAR, j / T::FM, j % T::FM);
  }
  if constexpr (!PERS) {
    // rowk_part counted 32 signs per real A word; with a last word per row (linear) or per
    // tap (conv) that holds only KB % 32 signs, the row's K_valid is lower by
    // (32 * words - KB) per row or per real tap (the tail bits are 0 in A, so popA is right)
    const int short_bits = (CONV ? 32 * p.CW : 32 * p.KW) - p.KB;
    if (short_bits != 0 && a_q == 0 && amok) {
      int units = 1;
      if constexpr (CONV) {
        int nh = 0, nw = 0;
        for (int k = 0; k < p.KH; k++) {
          const int ih = pc.ihb + k * p.DH;
          nh += (ih >= 0 && ih < p.H);
        }
        for (int k = 0; k < p.KWD; k++) {
          const int iw = pc.iwb + k * p.DW;
          nw += (iw >= 0 && iw < p.W);
        }
        units = nh * nw;
      }
      rowk_part -= short_bits * units;
    }
    atomicAdd(&rowk[a_row], rowk_part);
    __syncthreads();
    tile_epilogue(0, lds0);
  }
}

// Workgroups of the persistent conv kernel for tile T that the current device holds at
// once (compute units x resident workgroups per unit), cached per device and kernel.
template <class T, int OUT, bool VEC>
int persistent_slots() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, mfma_kernel<T, OUT, true, VEC, true>,
                                                     T::THREADS, 0) != hipSuccess)
      return 0;
    v = cus * (per_cu > 0 ? per_cu : 1);
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

template <class T, int OUT, bool CONV, bool VEC>
hipError_t launch_tile_o(const Contraction& p0, hipStream_t stream) {
  Contraction p = p0;
  p.div_tn = FastDiv((uint32_t)((p.N + T::BN - 1) / T::BN));
  const int64_t tiles = (int64_t)((p.M + T::BM - 1) / T::BM) * ((p.N + T::BN - 1) / T::BN);
  const dim3 block(T::THREADS);
  if constexpr (CONV && T::F4 && T::THREADS == 512) {
    // (8-wave tiles only: the 4-wave conv tile runs three workgroups per compute unit instead,
    // so one's epilogue overlaps the others' loops)
    // more fp4 conv tiles than fit at once: one persistent workgroup per resident slot
    // streams its tiles back to back instead of running them in separate rounds (the
    // int8 256 x 256 conv tile would spill with the extra state). Channel counts that are
    // not a whole number of words take the one-tile-per-workgroup kernel, which corrects
    // K_valid for the short last word of each tap.
    const int slots = BNN_CONV_PERS && p.KB == 32 * p.CW ? persistent_slots<T, OUT, VEC>() : 0;
    if (slots > 0 && tiles > slots) {
      hipLaunchKernelGGL((mfma_kernel<T, OUT, CONV, VEC, true>), dim3((unsigned)slots), block, 0,
                         stream, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((mfma_kernel<T, OUT, CONV, VEC, false>), dim3((unsigned)tiles), block, 0,
                     stream, p);
  return hipGetLastError();
}

template <class T, bool CONV, bool VEC>
hipError_t launch_tile_v(const Contraction& p, int out_dtype, hipStream_t stream) {
  switch (out_dtype) {
    case kF32: return launch_tile_o<T, kF32, CONV, VEC>(p, stream);
    case kF16: return launch_tile_o<T, kF16, CONV, VEC>(p, stream);
    case kBF16: return launch_tile_o<T, kBF16, CONV, VEC>(p, stream);
    default: return launch_tile_o<T, kI32, CONV, VEC>(p, stream);
  }
}

// Vector loads need each thread's words of a stage to be contiguous, aligned and, for
// conv, within one tap: the per-thread word counts divide K/32 (linear) or C/32 and the
// weight row length (conv), and both operand bases are 16-byte aligned.
// TS: the tile used when vector loads are impossible (the fp4 256 x 256 tile would spill
// with the scalar loader's extra state).
template <class T, bool CONV, class TS = T>
hipError_t launch_tile(const Contraction& p, int out_dtype, hipStream_t stream) {
  const bool aligned = (reinterpret_cast<uintptr_t>(p.a) % 16) == 0 &&
                       (reinterpret_cast<uintptr_t>(p.w) % 16) == 0;
  const bool vec = aligned && (CONV ? p.CW : p.KW) % T::A_WPT == 0 && p.KW % T::W_WPT == 0;
  return vec ? launch_tile_v<T, CONV, true>(p, out_dtype, stream)
             : launch_tile_v<TS, CONV, false>(p, out_dtype, stream);
}

#ifndef BNN_MFMA_PD_L
#define BNN_MFMA_PD_L 2
#endif
#ifndef BNN_MFMA_PD_M
#define BNN_MFMA_PD_M 4
#endif
#ifndef BNN_MFMA_WAVES_N
#define BNN_MFMA_WAVES_N 4
#endif
// 2 x BNN_MFMA_WAVES_N waves per workgroup: with 4 along W there are two waves per SIMD,
// whose MFMA and expansion streams the hardware interleaves. A stage is 128 reductions
// (4 words) for int8 and 256 (8 words) for fp4: the same LDS row of 128 bytes and the
// same number of MFMAs per stage.
#ifndef BNN_MFMA_L_WAVES_N
#define BNN_MFMA_L_WAVES_N 4
#endif
#ifndef BNN_MFMA_PD_CF4
#define BNN_MFMA_PD_CF4 2
#endif
// fp4 conv tiles keep two prefetched stages (measured faster than four on the conv
// workloads, whose tiles have few stages, and spill-free) and stop at 128 x 256: with the
// implicit-im2col loaders' extra state a 256 x 256 tile no longer fits in 256 registers.
template <bool F4, bool CONV>
struct Tiles {
  static constexpr int KS = F4 ? 8 : 4;
  static constexpr int PD_M = F4 && CONV ? BNN_MFMA_PD_CF4 : BNN_MFMA_PD_M;
  using M = Tile<128, 256, KS, PD_M, 2, BNN_MFMA_WAVES_N, F4>;
  using L = std::conditional_t<F4 && CONV, M,
                               Tile<256, 256, KS, BNN_MFMA_PD_L, 2, BNN_MFMA_L_WAVES_N, F4>>;
  using S = Tile<128, 128, KS, PD_M, 2, BNN_MFMA_WAVES_N, F4>;
  // fp4 convs with two or more rounds of 128 x 256 tiles: 128 x 128 tiles of 2 x 2 waves (the
  // same 64 x 64 per wave), one tile per workgroup, stages of 4 words (32 KiB of LDS) and at most
  // 168 registers per lane so that three workgroups share a compute unit: on the dilated
  // 128 x 128 x 28 x 28 -> 256 layer 40.2 us with persistent 128 x 256 tiles, 37.5 with these
  // tiles at 8-word stages (two workgroups per compute unit), 34.0 at three (the strided layer,
  // one round of 128 x 256 tiles, stays on those: 13.7 against 14.3 us)
  using C2 = Tile<128, 128, F4 && CONV ? 4 : KS, PD_M, 2, 2, F4, F4 && CONV ? 3 : 1>;
  // fp4 layers whose 64 x 128 tiles fit in one round of workgroups: 64 x 128 tiles, 1 x 4
  // waves, twice the workgroups of 128 x 128 (the 32x256x14x14 stage-3 conv: 12.6 -> 10.7 us,
  // linear layers from 64x256x512 to 1024x2048x4096: 13-20 % faster; a 1536x2048x2048 layer,
  // whose 64 x 128 tiles would take two rounds, is faster on 128 x 128)
  using T64 = Tile<64, 128, KS, PD_M, 1, 4, F4>;
  // at most 64 output features (64-channel convs): 256 x 64 tiles, 4 x 2 waves, instead of
  // leaving three quarters of a 256-wide tile's W rows empty (fp4 only: an int8 stage of
  // 4 words has too few W words for 512 loader threads)
  using N64 = std::conditional_t<F4, Tile<256, 64, KS, PD_M, 4, 2, F4>, S>;
};

int64_t count_tiles(const Contraction& p, int bm, int bn) {
  return (int64_t)((p.M + bm - 1) / bm) * ((p.N + bn - 1) / bn);
}

// Largest tile that still gives every compute unit a workgroup; the smallest otherwise.
#ifndef BNN_MFMA_MIN_TILES
#define BNN_MFMA_MIN_TILES 256
#endif
#ifndef BNN_MFMA_MIN_TILES_CONV
#define BNN_MFMA_MIN_TILES_CONV 128
#endif
template <bool CONV, bool F4>
hipError_t launch_mfma_t(const Contraction& p, int out_dtype, hipStream_t stream) {
  constexpr int64_t kMinTiles = BNN_MFMA_MIN_TILES;  // one workgroup per compute unit
  using TS = Tiles<F4, CONV>;
#if defined(BNN_CONV_TILE)
  // tuning builds: one fixed fp4 conv tile (1: 128 x 256, 2: 128 x 128, 3: 64 x 128, 4: see below)
  if constexpr (CONV && F4) {
    if (BNN_CONV_TILE == 1) return launch_tile<typename TS::M, CONV>(p, out_dtype, stream);
    if (BNN_CONV_TILE == 2) return launch_tile<typename TS::S, CONV>(p, out_dtype, stream);
    if (BNN_CONV_TILE == 3) return launch_tile<typename TS::T64, CONV>(p, out_dtype, stream);
    if (BNN_CONV_TILE == 4) return launch_tile<typename TS::C2, CONV>(p, out_dtype, stream);
  }
#endif
  if (F4 && p.N <= 64 && count_tiles(p, 256, 64) >= kMinTiles)
    return launch_tile<typename TS::N64, CONV>(p, out_dtype, stream);
  if (CONV && F4 && count_tiles(p, 128, 256) >= 2 * kMinTiles)
    return launch_tile<typename TS::C2, CONV>(p, out_dtype, stream);
  if (count_tiles(p, 256, 256) >= kMinTiles)
    return launch_tile<typename TS::L, CONV, std::conditional_t<F4, typename TS::M, typename TS::L>>(
        p, out_dtype, stream);
  // conv outputs are written per element, so half a round of large tiles still beats two
  // rounds of small ones
  if (count_tiles(p, 128, 256) >= (CONV ? BNN_MFMA_MIN_TILES_CONV : kMinTiles))
    return launch_tile<typename TS::M, CONV>(p, out_dtype, stream);
  if (F4 && count_tiles(p, 64, 128) <= kMinTiles)
    return launch_tile<typename TS::T64, CONV>(p, out_dtype, stream);
  return launch_tile<typename TS::S, CONV>(p, out_dtype, stream);
}

}  // namespace

hipError_t launch_mfma(const Contraction& p, bool conv, int out_dtype, hipStream_t stream) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  return conv ? launch_mfma_t<true, false>(p, out_dtype, stream)
              : launch_mfma_t<false, false>(p, out_dtype, stream);
}

hipError_t launch_mfma_fp4(const Contraction& p, bool conv, int out_dtype, hipStream_t stream) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  return conv ? launch_mfma_t<true, true>(p, out_dtype, stream)
              : launch_mfma_t<false, true>(p, out_dtype, stream);
}

}  // namespace bnn
