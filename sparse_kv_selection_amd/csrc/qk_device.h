// Device-side helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

namespace qk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kEps = 1e-12f;          // lower clamp of every vector norm
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;

// bf16 is stored as raw 16-bit patterns; widening to fp32 is exact.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (lowered to v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  __bf16 h = static_cast<__bf16>(x);
  return __builtin_bit_cast(uint16_t, h);
}
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// two fp32 -> packed bf16 pair (one v_cvt_pk_bf16_f32), round to nearest even
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
// two fp32 -> packed fp16 pair, round to nearest even
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}
// packed fp16 pair -> two fp32 (exact)
__device__ __forceinline__ f32x2 unpack_f16x2(uint32_t w) {
  return __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p) { return *p; }
};
template <> struct Elem<uint16_t> {
  __device__ __forceinline__ static float load(const uint16_t* p) { return bf16_to_f32(*p); }
};

// Inclusive prefix sum over the 64 lanes of a wave in six DPP steps: shifts
// by 1, 2, 4 and 8 lanes inside each 16-lane row, then the end of row 0 (and
// of row 2) is added to row 1 (row 3), and the end of row 1 to rows 2 and 3.
// Lanes whose source lies outside the row keep the 0 they start from.  Every
// lane of the wave must be active.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  int v = static_cast<int>(x);
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return static_cast<uint32_t>(v);
}
// Sum over each aligned group of W consecutive lanes (W a power of two up to
// 64); every lane gets its group's sum.  Within 16 lanes the partners come
// from DPP (lane xor 1, xor 2, then the mirrored lane of the 8- and the
// 16-lane half, which after the earlier steps holds the other half's sum);
// wider groups add the gfx950 lane swaps (16-lane rows, then 32-lane halves),
// which stay in the vector unit (no LDS round trip).  Every lane of the wave
// must be active.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(x)));
}
// op(v, v of lane ^ X) for X = 16 or 32, op commutative: the swap hands every
// lane its own value and its partner's (in an order that depends on the lane).
template <int X, typename T, typename Op>
__device__ __forceinline__ T swap_op(T v, Op op) {
  static_assert(sizeof(T) == 4 && (X == 16 || X == 32), "32-bit values, xor 16 or 32");
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  if constexpr (X == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return op(__builtin_bit_cast(T, static_cast<uint32_t>(r[0])), __builtin_bit_cast(T, static_cast<uint32_t>(r[1])));
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return op(__builtin_bit_cast(T, static_cast<uint32_t>(r[0])), __builtin_bit_cast(T, static_cast<uint32_t>(r[1])));
  }
}
template <int W, typename T, typename Op>
__device__ __forceinline__ T group_reduce(T v, Op op) {
  auto step = [](T x, auto ctrl) {
    constexpr int C = decltype(ctrl)::value;
    if constexpr (__is_same(T, float)) return dpp_f<C>(x);
    else return static_cast<T>(dpp_i<C>(static_cast<int>(x)));
  };
  using q1 = std::integral_constant<int, 0xb1>;   // quad_perm [1,0,3,2]
  using q2 = std::integral_constant<int, 0x4e>;   // quad_perm [2,3,0,1]
  using hm = std::integral_constant<int, 0x141>;  // row_half_mirror
  using rm = std::integral_constant<int, 0x140>;  // row_mirror
  if constexpr (W >= 2) v = op(v, step(v, q1{}));
  if constexpr (W >= 4) v = op(v, step(v, q2{}));
  if constexpr (W >= 8) v = op(v, step(v, hm{}));
  if constexpr (W >= 16) v = op(v, step(v, rm{}));
  if constexpr (W >= 32) v = swap_op<16>(v, op);
  if constexpr (W >= 64) v = swap_op<32>(v, op);
  return v;
}
template <int W, typename T>
__device__ __forceinline__ T group_sum(T v) {
  return group_reduce<W>(v, [](T a, T b) { return a + b; });
}

// Value of lane 63 (for an inclusive scan: the wave total), uniform.
__device__ __forceinline__ uint32_t lane63(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 63));
}

// Histograms in LDS carry one padding word per 32 bins, so that the lanes of
// a crossing search, each reading a run of consecutive bins, hit different
// banks.  hpad(b) is the word of bin b.
__device__ __forceinline__ int hpad(int b) { return b + (b >> 5); }
__host__ __device__ constexpr int hist_words(int bins) { return bins + bins / 32; }

// Called by one whole wave: the bin b of counts h[hpad(0 .. 64 * PER)) with
// count(bins > b) < need <= count(bins >= b), for 1 <= need <= total;
// writes (*bin, *above = count(bins > b)) from the lane that holds it.  Each
// lane keeps its PER bins in registers: one batch of LDS reads, one wave scan
// and a register walk.
template <int PER>
__device__ void wave_crossing(const int* h, int need, int* bin, int* above) {
  const int lane = threadIdx.x & 63;
  const int top = 64 * PER - 1 - lane * PER;  // lane 0 holds the highest bins
  int c[PER];
  int sum = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    c[q] = h[hpad(top - q)];
    sum += c[q];
  }
  const int incl = static_cast<int>(wave_incl_scan(static_cast<uint32_t>(sum)));
  const int ex = incl - sum;
  if (ex < need && need <= incl) {
    int b = top, a = ex;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      if (a + c[q] >= need) { b = top - q; break; }
      a += c[q];
    }
    *bin = b;
    *above = a;
  }
}

// Order-preserving map of a float to uint32 (-0.0 maps like +0.0).
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Level-1 bins of order keys for top-k selection over scores (2048 bins),
// monotone in the key, so that every bin above the one holding the k-th
// largest score is selected whole.  Each sign gets 1024 bins: 64 per binade
// of |x| over [2^-8, 2^(1022/64 - 8)) (about 0.0039 to 250: cosine scores and
// dot products of unit-scale vectors), one bin for the smaller magnitudes
// next to zero and one for the larger ones (and NaN) at the end.  The top bits
// of the key alone would spend most bins on exponents that such scores never
// reach and put a tenth of a row into one bin.  The scoring pass can fill the
// histogram of its rows in these bins for the selection that follows it.
constexpr int kL1Bins = 2048;
constexpr int kL1Shift = 17;         // key bits below a bin: 23 - 6 mantissa bits
constexpr int kL1FineBase = 119 << 6;  // (exponent, top 6 mantissa bits) of 2^-8
__device__ __forceinline__ int l1_bin(uint32_t key) {
  const bool pos = key >= 0x80000000u;
  const uint32_t mag = pos ? (key & 0x7fffffffu) : (0x7fffffffu - key);  // bits of |x|
  const int v = static_cast<int>(mag >> kL1Shift) - kL1FineBase;
  const int i = v < 0 ? 0 : min(v + 1, 1023);
  return pos ? 1024 + i : 1023 - i;
}
// The keys of level-1 bin b: [*lo, *hi].
__device__ __forceinline__ void l1_bin_range(int b, uint32_t* lo, uint32_t* hi) {
  const bool pos = b >= 1024;
  const int i = pos ? b - 1024 : 1023 - b;
  const uint32_t mlo = i == 0 ? 0u : static_cast<uint32_t>(kL1FineBase + i - 1) << kL1Shift;
  const uint32_t mhi =
      i == 1023 ? 0x7fffffffu : (static_cast<uint32_t>(kL1FineBase + i) << kL1Shift) - 1u;
  *lo = pos ? (0x80000000u | mlo) : (0x7fffffffu - mhi);
  *hi = pos ? (0x80000000u | mhi) : (0x7fffffffu - mlo);
}

// OCP 8-bit floating point, E4M3: sign, 4 exponent bits (bias 7), 3 mantissa
// bits; exponent field 0 holds the subnormals m/8 * 2^-6.  Each value takes
// the nearest code, ties to the even code; magnitudes above 448 (the largest
// finite code) saturate to 448; the sign bit is copied, so values that round
// to zero keep it.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fminf(fabsf(x), 448.0f);
  uint32_t code;
  if (a < 0x1p-6f) {
    // below the smallest normal the codes are the multiples of 2^-9: adding
    // 2^14 (whose fp32 spacing is 2^-9) rounds to the nearest one, ties to
    // even; 2^-6 itself comes out as 8, the smallest normal code
    const float r = __fsub_rn(__fadd_rn(a, 0x1p14f), 0x1p14f);
    code = static_cast<uint32_t>(r * 512.0f);
  } else {
    // keep 3 of the 23 mantissa bits, rounding to nearest even (a carry moves
    // into the exponent), then rebias the exponent from 127 to 7
    const uint32_t b = __float_as_uint(a);
    const uint32_t r = b + 0x7ffffu + ((b >> 20) & 1u);
    code = (r >> 20) - (120u << 3);
  }
  return sign | code;
}

// 16 values as E4M3 codes, value e in byte e.
__device__ __forceinline__ u32x4 e4m3x16(const float* x) {
  u32x4 out;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    out[w] = e4m3_code(x[4 * w]) | (e4m3_code(x[4 * w + 1]) << 8) | (e4m3_code(x[4 * w + 2]) << 16) |
             (e4m3_code(x[4 * w + 3]) << 24);
  return out;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }
__device__ __forceinline__ float wave_max(float v) {
  return group_reduce<64>(v, [](float a, float b) { return fmaxf(a, b); });
}

// 16-byte global load through the vector path.
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D = A * B + C on a 32x32x16 bf16 matrix-core tile.
// A: lane l holds row (l % 32), k = 8 * (l / 32) + [0, 8).
// B: lane l holds column (l % 32), the same k slots.
// C/D: lane l holds column (l % 32), rows 8 * (r / 4) + 4 * (l / 32) + (r % 4), r < 16.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row (within a 32-row block) held in accumulator register r by lane half h.
__device__ __forceinline__ constexpr int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// XCD-aware block order: consecutive logical ids land on one XCD's L2.
__device__ __forceinline__ int xcd_swizzle(int lin, int n) {
  if ((n & 7) != 0) return lin;
  return (lin & 7) * (n >> 3) + (lin >> 3);
}

}  // namespace qk
