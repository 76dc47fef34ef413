// Matrix-core rate calibration (measurement only; computes nothing of the
// method).  Each of 256 workgroups of eight waves (the attention launch's
// shape: two waves per SIMD) runs `iters` tiles of the attention kernel's
// matrix work: 16 value products and 16 key products of 32x32x16 bf16, with
// the operands read from LDS in the attention kernel's swizzled layouts and six
// operands in flight, optionally followed by the tile's softmax vector work
// (maximum, exponentials, bf16 packing) that feeds the next value products.
// Operands are either near-constant or random bf16 values of magnitude about
// one: the rate the matrix cores sustain falls with the operands' switching
// activity, so the random form gives the ceiling for attention over real data.
#include <stdint.h>

#include "../../include/qk.h"
#include "qk_device.h"

namespace qk {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kD = 128;
constexpr int kRing = 6;

__device__ __forceinline__ bf16x8 read_tr_pair(const uint16_t* p) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 8 * kD));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// a bf16 bit pattern of magnitude in [0.5, 4) with a random sign and mantissa
__device__ __forceinline__ uint32_t rand_bf16(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return ((x >> 16) & 0x8000u) | ((126u + (x % 3u)) << 7) | (x & 0x7fu);
}

template <bool RANDOM, bool LDS, bool SOFT>
__global__ __launch_bounds__(512, 1) void calib_kernel(int iters, float* out) {
  __shared__ __attribute__((aligned(16))) uint16_t s[2 * 64 * kD];  // a K tile and a V tile
  const int tid = threadIdx.x, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  for (int i = tid; i < 2 * 64 * kD; i += 512)
    s[i] = static_cast<uint16_t>(RANDOM ? rand_bf16(static_cast<uint32_t>(i) * 2654435761u + blockIdx.x)
                                        : 0x3f80u + (i & 7));
  __syncthreads();
  // the attention kernel's read offsets (elements): K rows, transposed V reads
  int kofs[8], vofs[4];
  {
    const int fk = half ^ (col & 15);
    for (int st = 0; st < 8; ++st) kofs[st] = col * kD + 8 * ((2 * st) ^ fk);
    const int g = lane >> 4, jl = lane & 15, jj = jl >> 2;
    const int vr = 4 * (g >> 1) + jj;
    const int x = 2 * (g & 1) + ((jl & 3) >> 1);
    const int fv = 4 * (vr & 3);
    for (int db = 0; db < 4; ++db) vofs[db] = 64 * kD + vr * kD + 8 * ((4 * db + x) ^ fv) + 4 * (jl & 1);
  }
  f32x16 acc[4] = {};
  f32x16 S[2] = {};
  bf16x8 q[8], P[4];
  for (int i = 0; i < 8; ++i) {
    u32x4 w;
    for (int e = 0; e < 4; ++e)
      w[e] = RANDOM ? (rand_bf16(tid * 131u + i * 17u + e * 5u + blockIdx.x * 7919u) |
                       (rand_bf16(tid * 137u + i * 19u + e * 3u + blockIdx.x * 104729u) << 16))
                    : (0x3f803f80u + static_cast<uint32_t>(i + e));
    q[i] = as_bf16x8(w);
  }
  for (int i = 0; i < 4; ++i) P[i] = q[i];
  auto rd = [&](int i) __attribute__((always_inline)) {
    if (!LDS) return q[(i * 5) & 7];
    return i < 16 ? read_tr_pair(s + vofs[i & 3] + (i >> 2) * 16 * kD)
                  : as_bf16x8(*reinterpret_cast<const u32x4*>(s + kofs[(i - 16) >> 1] + ((i - 16) & 1) * 32 * kD));
  };
  float l = 0.f;
  for (int it = 0; it < iters; ++it) {
    bf16x8 ring[kRing];
#pragma unroll
    for (int i = 0; i < kRing; ++i) ring[i] = rd(i);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (i < 16) acc[i & 3] = mfma32(ring[i % kRing], P[i >> 2], acc[i & 3]);
      else S[i & 1] = mfma32(ring[i % kRing], q[(i - 16) >> 1], (i - 16) < 2 ? f32x16{} : S[i & 1]);
      if (i + kRing < 32) ring[i % kRing] = rd(i + kRing);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (SOFT) {
      float mx = S[0][0];
      for (int kb = 0; kb < 2; ++kb)
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kb][r]);
      for (int g16 = 0; g16 < 4; ++g16) {
        u32x4 w;
        for (int e = 0; e < 4; ++e) {
          const float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[g16 >> 1][8 * (g16 & 1) + 2 * e], 0.125f, -mx));
          const float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[g16 >> 1][8 * (g16 & 1) + 2 * e + 1], 0.125f, -mx));
          l += x0 + x1;
          w[e] = pack_bf16x2(x0, x1);
        }
        P[g16] = as_bf16x8(w);
      }
    } else {
      // keep the value products' operands dependent on the key products
      for (int g16 = 0; g16 < 4; ++g16) {
        u32x4 w;
        for (int e = 0; e < 4; ++e)
          w[e] = (__float_as_uint(S[g16 >> 1][8 * (g16 & 1) + 2 * e]) >> 16) |
                 (__float_as_uint(S[g16 >> 1][8 * (g16 & 1) + 2 * e + 1]) & 0xffff0000u);
        P[g16] = as_bf16x8(w);
      }
    }
  }
  float r = l;
  for (int e = 0; e < 16; ++e) r += acc[0][e] + acc[1][e] + acc[2][e] + acc[3][e] + S[0][e] + S[1][e];
  out[blockIdx.x * 512 + tid] = r;
}

}  // namespace
}  // namespace qk

extern "C" qk_status qk_calib_matrix_rate(int32_t mode, int32_t iters, float* out,
                                          qk_stream_t stream) {
  if (!out) return QK_ERR_NULL;
  if (iters < 1 || mode < 0 || mode > 7) return QK_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(out) & 3) != 0) return QK_ERR_ALIGN;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid(256), block(512);
#define QK_CALIB(R, L, S)                                                                    \
  if (mode == ((R) | ((L) << 1) | ((S) << 2))) {                                             \
    hipLaunchKernelGGL((qk::calib_kernel<R, L, S>), grid, block, 0, st, iters, out);         \
    return hipGetLastError() == hipSuccess ? QK_OK : QK_ERR_HIP;                             \
  }
  QK_CALIB(0, 0, 0) QK_CALIB(1, 0, 0) QK_CALIB(0, 1, 0) QK_CALIB(1, 1, 0)
  QK_CALIB(0, 1, 1) QK_CALIB(1, 1, 1) QK_CALIB(0, 0, 1) QK_CALIB(1, 0, 1)
#undef QK_CALIB
  return QK_ERR_SHAPE;
}
