// Plain BF16 GEMV, y = W x with fp32 accumulation: the uncompressed reference
// the fused compressed matvec is measured against (the same machine, no
// decode; not part of the method).  Each wave streams one row with 16-byte
// loads, four chunks in flight, against the activations staged once per
// workgroup in LDS; a butterfly of lane shuffles sums the row.  Measured on
// MI355X over the Qwen3-4B layer set: 3.48 / 3.29 / 3.08 TB/s with 1 / 2 / 4
// rows per wave.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/nwc.h"

namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int kRowsPerWave = 1;
constexpr int64_t kMaxK = 24576;  // activations in LDS: 48 KiB

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ __forceinline__ float dot8(const uint4 &w, const uint4 &x, float acc) {
  acc = fmaf(bf16_lo(w.x), bf16_lo(x.x), acc);
  acc = fmaf(bf16_hi(w.x), bf16_hi(x.x), acc);
  acc = fmaf(bf16_lo(w.y), bf16_lo(x.y), acc);
  acc = fmaf(bf16_hi(w.y), bf16_hi(x.y), acc);
  acc = fmaf(bf16_lo(w.z), bf16_lo(x.z), acc);
  acc = fmaf(bf16_hi(w.z), bf16_hi(x.z), acc);
  acc = fmaf(bf16_lo(w.w), bf16_lo(x.w), acc);
  acc = fmaf(bf16_hi(w.w), bf16_hi(x.w), acc);
  return acc;
}

// k and ldw multiples of 8 (16-byte chunks); rows [r, r + kRowsPerWave) that
// exist are summed by one wave.
__global__ __launch_bounds__(kThreads) void bf16_gemv_kernel(const uint4 *__restrict__ w, int64_t n, int64_t k,
                                                             int64_t ldw, const uint4 *__restrict__ x,
                                                             float *__restrict__ y) {
  extern __shared__ uint4 s_x[];
  const int64_t kc = k / 8, ldc = ldw / 8;
  for (int64_t c = threadIdx.x; c < kc; c += kThreads) s_x[c] = x[c];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (kThreads / 64);
  for (int64_t r = ((int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)) * kRowsPerWave; r < n;
       r += waves * kRowsPerWave) {
    float acc[kRowsPerWave] = {};
    const uint4 *row[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) row[i] = w + (r + i < n ? r + i : r) * ldc;
    int64_t c = lane;
    for (; c + 192 < kc; c += 256) {
      uint4 v[kRowsPerWave][4];
#pragma unroll
      for (int i = 0; i < kRowsPerWave; ++i)
#pragma unroll
        for (int u = 0; u < 4; ++u) v[i][u] = row[i][c + 64 * u];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint4 xv = s_x[c + 64 * u];
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) acc[i] = dot8(v[i][u], xv, acc[i]);
      }
    }
    for (; c < kc; c += 64) {
      const uint4 xv = s_x[c];
#pragma unroll
      for (int i = 0; i < kRowsPerWave; ++i) acc[i] = dot8(row[i][c], xv, acc[i]);
    }
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      float a = acc[i];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) a += __shfl_xor(a, off, 64);
      if (lane == 0 && r + i < n) y[r + i] = a;
    }
  }
}

}  // namespace

extern "C" int nwc_bf16_gemv(const void *d_w, int64_t n, int64_t k, int64_t ldw, const void *d_x, float *d_y,
                             void *stream) {
  if (!d_w || !d_x || !d_y) return NWC_ERR_ARG;
  if (((uintptr_t)d_w | (uintptr_t)d_x) & 15 || (uintptr_t)d_y & 3) return NWC_ERR_ARG;
  if (n < 1 || k < 8 || k > kMaxK || k % 8 || ldw < k || ldw % 8 || n > ((int64_t)1 << 31)) return NWC_ERR_SHAPE;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return NWC_ERR_HIP;
  const int64_t rows_per_group = (kThreads / 64) * kRowsPerWave;
  const int64_t groups = (n + rows_per_group - 1) / rows_per_group;
  const int64_t grid = groups < (int64_t)cus * 8 ? groups : (int64_t)cus * 8;
  hipLaunchKernelGGL(bf16_gemv_kernel, dim3((unsigned)grid), dim3(kThreads), (size_t)(k / 8) * 16,
                     (hipStream_t)stream, (const uint4 *)d_w, n, k, ldw, (const uint4 *)d_x, d_y);
  return hipGetLastError() == hipSuccess ? NWC_OK : NWC_ERR_HIP;
}
