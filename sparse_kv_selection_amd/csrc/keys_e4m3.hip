// Key storage for the 8-bit scoring pass: K rows as OCP E4M3 bytes.
//
// The attention co-design knowledge card ("Co-Designing AI Model Attention for
// Fast, Interactive Long-Context Inference", methods list) names FP8 KV
// caches among the measured prefill and decode kernels.  Here only the scoring
// pass reads 8-bit keys: it is bound by the bytes of K it streams, and E4M3
// halves them.  Attention keeps the bf16 rows.
//
// Encoding: e4m3_code (device header).  Callers convert the rows a chunk
// appends, once (qk_select can do it inside its scoring pass instead).
#include "qk_device.h"
#include "qk_internal.h"

namespace qk {
namespace {

// One thread per 16 consecutive elements of a row (d is a multiple of 16).
template <typename T>
__global__ __launch_bounds__(256) void keys_e4m3_kernel(const T* __restrict__ k,
                                                        uint8_t* __restrict__ k8, int bnkv,
                                                        int kv_cap, int d, int row0, int nrows) {
  const int per_row = d / 16;
  const long long total = static_cast<long long>(bnkv) * nrows * per_row;
  const long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int c = static_cast<int>(i % per_row);
  const long long rr = i / per_row;
  const int r = static_cast<int>(rr % nrows);
  const long long bj = rr / nrows;
  const size_t off = (static_cast<size_t>(bj) * kv_cap + row0 + r) * d + 16 * c;
  float x[16];
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 w = ld16(k + off + 8 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[8 * h + 2 * e] = bf16lo(w[e]);
        x[8 * h + 2 * e + 1] = bf16hi(w[e]);
      }
    }
  } else {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const f32x4 w = *reinterpret_cast<const f32x4*>(k + off + 4 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * h + e] = w[e];
    }
  }
  st16(k8 + off, e4m3x16(x));
}

}  // namespace

hipError_t launch_keys_e4m3(bool bf16, const void* k, uint8_t* k8, int bnkv, int kv_cap, int d,
                            int row0, int nrows, hipStream_t st) {
  const long long total = static_cast<long long>(bnkv) * nrows * (d / 16);
  if (total == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((total + 255) / 256)), block(256);
  if (bf16)
    hipLaunchKernelGGL(keys_e4m3_kernel<uint16_t>, grid, block, 0, st,
                       static_cast<const uint16_t*>(k), k8, bnkv, kv_cap, d, row0, nrows);
  else
    hipLaunchKernelGGL(keys_e4m3_kernel<float>, grid, block, 0, st, static_cast<const float*>(k),
                       k8, bnkv, kv_cap, d, row0, nrows);
  return hipGetLastError();
}

}  // namespace qk
